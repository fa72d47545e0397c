"""paged_attention_prefill (store the chunk, then causal varlen attention on MFMA) versus the fp64 oracle.

Tolerance: |gpu - ref| <= 2e-2 + 1e-2 |ref| elementwise (bf16 inputs and outputs, fp32 accumulation,
softmax weights rounded to bf16 for the second product)."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import assert_close, assert_rel_norm, oracle_prefill_case, run_prefill_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pkv():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import paged_kv_cache_88_amd as m

    m.load_library()
    return m


def _case(seed, prefix, chunk, group, bs, causal=True, hkv=2):
    lk = [p + c for p, c in zip(prefix, chunk)]
    nb = sum(W.blocks_for_tokens(n, bs) for n in lk) + 5
    return W.make_prefill_case("pf", seed, W.BF16, prefix, chunk, hkv * group, hkv, 128, bs, nb, causal=causal)


@pytest.mark.parametrize("group", [1, 3, 4, 8])
@pytest.mark.parametrize("bs", [1, 16, 256])
def test_small_ragged(pkv, orc, group, bs):
    """Chunks shorter and longer than a tile, prefixes on and off block boundaries, a 1-token chunk."""
    c = _case(40 + group + bs, [0, 17, 256, 300, 5], [33, 1, 64, 130, 200], group, bs)
    got = run_prefill_case(pkv, c)
    assert_close(got, oracle_prefill_case(orc, c), W.BF16, f"prefill g{group} bs{bs}")


@pytest.mark.parametrize("bs", [2, 4, 8, 32, 64, 128])
def test_every_block_size(pkv, orc, bs):
    """The remaining block sizes: 64 and up gather a 64-key tile from one block, smaller ones row by row."""
    c = _case(60 + bs, [0, 63, 64, 129, 7], [65, 1, 64, 100, 190], 4, bs)
    got = run_prefill_case(pkv, c)
    assert_close(got, oracle_prefill_case(orc, c), W.BF16, f"prefill bs{bs}")


@pytest.mark.parametrize("group", [2, 5, 6, 7])
def test_remaining_groups(pkv, orc, group):
    """Head groupings whose rows do not fill the workgroup's 128 evenly."""
    c = _case(70 + group, [0, 40, 300], [97, 33, 150], group, 16)
    got = run_prefill_case(pkv, c)
    assert_close(got, oracle_prefill_case(orc, c), W.BF16, f"prefill g{group}")


@pytest.mark.parametrize("bs", [16, 64])
def test_block_table_past_64_blocks(pkv, orc, bs):
    """Cached prefixes spanning more than 64 blocks (block ids past the first 64 come from the table in
    memory, not from the lane-held slice): every row."""
    c = _case(80 + bs, [64 * bs + 77, 5], [70, 40], 4, bs)
    got = run_prefill_case(pkv, c)
    assert np.isfinite(got).all()
    assert_close(got, oracle_prefill_case(orc, c), W.BF16, f"long table bs{bs}")


@pytest.mark.parametrize("n", [64, 65, 130])
def test_many_sequences(pkv, orc, n):
    """Batches at and past the size the kernel ranks longest first (64 sequences): every row checked."""
    rng = np.random.default_rng(90 + n)
    prefix = rng.integers(0, 200, n).tolist()
    chunk = rng.integers(1, 80, n).tolist()
    c = _case(90 + n, prefix, chunk, 4, 16)
    got = run_prefill_case(pkv, c)
    assert_close(got, oracle_prefill_case(orc, c), W.BF16, f"{n} sequences")


@pytest.mark.parametrize("causal", [True, False])
def test_causal_and_full(pkv, orc, causal):
    c = _case(77, [0, 100, 513], [129, 64, 7], 4, 16, causal=causal)
    got = run_prefill_case(pkv, c)
    assert_close(got, oracle_prefill_case(orc, c), W.BF16, f"causal={causal}")


def test_empty_chunks_in_batch(pkv, orc):
    """Sequences with no new tokens contribute no rows; their neighbours are unaffected."""
    c = _case(5, [10, 40, 0, 7], [5, 0, 70, 0], 4, 16)
    got = run_prefill_case(pkv, c)
    assert_close(got, oracle_prefill_case(orc, c), W.BF16, "empty chunks")


def test_chunked_prefill_config(pkv, orc):
    """32 sequences, prefix U[0, 2048] + chunk U[64, 512], block 256, 32/8 heads: every row, head and dim
    against the oracle, plus the relative error norm."""
    c = W.chunked_prefill()
    got = run_prefill_case(pkv, c)
    assert np.isfinite(got).all()
    ref = oracle_prefill_case(orc, c)
    assert_close(got, ref, W.BF16, "chunked prefill config")
    assert_rel_norm(got, ref, what="chunked prefill config")


def test_prefill_last_row_matches_decode(pkv, orc):
    """The last chunk row of a causal prefill and a decode over the same Lk tokens agree (within
    tolerance; both against the oracle's decode)."""
    c = _case(9, [31, 200], [1, 17], 4, 16)
    got = run_prefill_case(pkv, c)
    last = c.cu_seqlens_q[1:] - 1
    kc, vc = c.pool.dense()
    orc.store(c.dtype, c.key, c.value, kc, vc, c.slot_mapping)
    lk = (c.prefix_lens + c.chunk_lens).astype(np.int32)
    ref = orc.decode(c.dtype, c.query[last], kc, vc, c.block_tables, lk, c.scale)
    assert_close(got[last], ref, W.BF16, "last row vs decode")


def test_prefill_rejects_fp32(pkv):
    kc = torch.zeros((4, 1, 16, 128), dtype=torch.float32, device="cuda")
    q = torch.zeros((3, 2, 128), dtype=torch.float32, device="cuda")
    cu = torch.tensor([0, 3], dtype=torch.int32, device="cuda")
    with pytest.raises(pkv.PagedKVError, match="EUNSUPPORTED"):
        pkv.paged_attention_prefill(torch.empty_like(q), q, kc, kc, torch.zeros((1, 1), dtype=torch.int32, device="cuda"),
                                    cu, cu, 3, 3, 0.1)
