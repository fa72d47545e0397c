"""Host-side arithmetic pinned by the pages' worked examples (tests/golden/*.json, each cites its page).

These pin the block-count, row-stride and slot-flattening conventions that the generators and the
oracle both rely on, against numbers printed on the pages rather than against our own formulas.
"""
import numpy as np
import pytest

from conftest import golden
from workloads import F32, align_up_32, blocks_for_tokens


def test_block_counts_match_block_manager_examples():
    g = golden("block_counts.json")
    for tokens, blocks in g["tokens_to_blocks"]:
        assert blocks_for_tokens(tokens, g["block_size"]) == blocks


def test_sequence_split_example():
    g = golden("sequence_blocks.json")["split_example"]
    n, bs = g["num_tokens"], g["block_size"]
    nb = blocks_for_tokens(n, bs)
    assert nb == g["num_blocks"]
    counts = [min(bs, n - j * bs) for j in range(nb)]
    assert counts == g["block_token_counts"]
    assert counts[-1] == g["last_block_num_tokens"]


def test_append_opens_new_block_example():
    g = golden("sequence_blocks.json")["append_example"]
    bs, n = g["block_size"], g["length_after_append"]
    assert (blocks_for_tokens(n, bs) > blocks_for_tokens(n - 1, bs)) == g["opens_new_block"]
    assert (n % bs == 1) == g["opens_new_block"]


@pytest.mark.parametrize("bs", [1, 4, 16, 256])
def test_last_block_num_tokens_invariant(bs):
    """nano-vllm walkthrough, section 2 Sequence: last_block_num_tokens lies in [1, block_size] for n >= 1."""
    for n in range(1, 5 * bs + 3):
        nb = blocks_for_tokens(n, bs)
        last = n - (nb - 1) * bs
        assert 1 <= last <= bs
        assert (nb - 1) * bs < n <= nb * bs


def test_align_up_32_examples():
    for n, want in golden("align_and_pool.json")["align_up_32"]:
        assert align_up_32(n) == want


def test_cache_per_page_example():
    g = golden("align_and_pool.json")
    c = g["cache_per_page"]
    per_page = 2 * c["head_dim"] * c["num_kv_heads"] * c["page_size"] * c["dtype_bytes"] * c["num_layers"]
    assert per_page == c["bytes"]
    assert (20 * 1024 * 1024 * 1024) // per_page == g["pages_in_20GB"]


def test_kv_size_examples():
    g = golden("align_and_pool.json")
    m = g["kv_bytes_mha"]
    mha = 2 * m["layers"] * m["tokens"] * m["hidden"] * m["dtype_bytes"]
    assert mha / 1024 ** 3 == pytest.approx(m["gib"])
    q = g["kv_bytes_gqa"]
    gqa = 2 * q["layers"] * q["tokens"] * q["kv_heads"] * q["head_dim"] * q["dtype_bytes"]
    assert gqa / 1024 ** 3 == pytest.approx(q["gib"])
    assert gqa / 1e9 == pytest.approx(q["gb_decimal_approx"], abs=0.06)


def test_oracle_slot_flattening_matches_2d_index_example(orc):
    """A slot is row * STRIDE + pos with STRIDE = block_size: the page's (3, 4) example writes the
    ranges [(0,1,3), (2,0,2)] to flat rows [1, 2, 8, 9], i.e. block 0 offsets 1-2 and block 2 offsets 0-1."""
    g = golden("index_2d.json")
    rows, stride = g["rows"], g["stride"]
    slots = np.array(g["flat_indices"], dtype=np.int32)
    n = len(slots)
    key = np.arange(1, n + 1, dtype=np.float32).reshape(n, 1, 1)
    kc = np.zeros((rows, 1, stride, 1), np.float32)
    vc = np.zeros((rows, 1, stride, 1), np.float32)
    orc.store(F32, key, -key, kc, vc, slots)
    k = 0
    for row, begin, end in g["ranges"]:
        for pos in range(begin, end):
            assert kc[row, 0, pos, 0] == key[k, 0, 0]
            assert vc[row, 0, pos, 0] == -key[k, 0, 0]
            k += 1
    assert np.count_nonzero(kc) == n


def test_oracle_gather_follows_block_split_example(orc):
    """10 tokens at block size 4 occupy 4 + 4 + 2 rows of the three blocks in table order."""
    g = golden("sequence_blocks.json")["split_example"]
    n, bs = g["num_tokens"], g["block_size"]
    table = np.array([5, 0, 3, -1], dtype=np.int32)
    kc = np.full((6, 1, bs, 1), np.nan, np.float32)
    for b in range(6):
        kc[b, 0, :, 0] = 100 * b + np.arange(bs)
    ko, vo = orc.gather(F32, kc, kc.copy(), table, n)
    got = ko[:, 0, 0]
    want = []
    for j, cnt in enumerate(g["block_token_counts"]):
        want += [100 * table[j] + o for o in range(cnt)]
    assert got.tolist() == want
