"""The seeded generators: determinism, the stated shapes and distributions, valid metadata."""
import numpy as np
import pytest

import workloads as W


def _check_decode_metadata(c):
    bs = c.block_size
    nbs = [W.blocks_for_tokens(n, bs) for n in c.context_lens]
    assert c.block_table_stride % 32 == 0 and c.block_table_stride >= max(nbs)
    owned = np.concatenate([c.block_tables[i, :nb] for i, nb in enumerate(nbs)])
    assert len(np.unique(owned)) == len(owned), "block ownership must not overlap"
    assert owned.min() >= 0 and owned.max() < c.num_blocks
    for i, nb in enumerate(nbs):
        assert np.all(c.block_tables[i, nb:] == -1)
    live = c.slot_mapping[c.slot_mapping >= 0]
    assert len(np.unique(live)) == len(live)
    for i, n in enumerate(c.context_lens):
        s = int(c.slot_mapping[i])
        assert s // bs == c.block_tables[i, (n - 1) // bs] and s % bs == (n - 1) % bs
    assert sorted(c.pool.used_blocks.tolist()) == sorted(owned.tolist())


def test_tiny_config():
    c = W.tiny_decode()
    assert c.context_lens.tolist() == [300, 70, 200, 513]
    assert (c.num_heads, c.num_kv_heads, c.head_dim, c.block_size, c.num_blocks) == (8, 2, 64, 16, 128)
    assert c.dtype == W.F32 and c.scale == pytest.approx(1 / 8)
    assert sum(W.blocks_for_tokens(n, 16) for n in c.context_lens) == 70
    assert W.blocks_for_tokens(513, 16) == 33 and 513 - 32 * 16 == 1     # last block holds one token
    _check_decode_metadata(c)


def test_determinism_and_seed_dependence():
    a, b, c = W.tiny_decode(1), W.tiny_decode(1), W.tiny_decode(2)
    assert np.array_equal(a.block_tables, b.block_tables) and np.array_equal(a.query, b.query)
    assert np.array_equal(a.pool.key_blocks, b.pool.key_blocks, equal_nan=True)
    assert not np.array_equal(a.block_tables, c.block_tables)


def test_bulk_draws_are_deterministic():
    x = W._draw_values(np.random.default_rng(9), (64, 1 << 17), W.BF16)
    y = W._draw_values(np.random.default_rng(9), (64, 1 << 17), W.BF16)
    assert np.array_equal(x, y)
    f = W.bf16_bits_to_f32(x)
    assert abs(f.mean()) < 0.01 and abs(f.std() - 1) < 0.01


def test_nan_poison_positions():
    c = W.make_decode_case("t", 0, W.F32, [5, 8, 1], 2, 1, 4, 4, 10)
    kc, _ = c.pool.dense()
    for i, n in enumerate(c.context_lens):
        for t in range(W.blocks_for_tokens(n, 4) * 4):
            row = kc[c.block_tables[i, t // 4], 0, t % 4]
            assert np.isnan(row).all() == (t >= n - 1)


@pytest.mark.parametrize("n", [2, 3, 4])
def test_decode_configs_metadata(n):
    c = W.make_config(n)
    _check_decode_metadata(c)
    if n == 2:
        assert c.num_seqs == 64 and c.context_lens.min() >= 128 and c.context_lens.max() <= 4096
        assert (c.num_heads, c.num_kv_heads, c.block_size, c.num_blocks) == (32, 8, 256, 4096)
    if n == 3:
        assert c.num_seqs == 512 and c.context_lens.min() >= 16 and c.context_lens.max() <= 2048
        assert 250 <= np.median(c.context_lens) <= 350
        assert (c.num_heads, c.num_kv_heads, c.block_size, c.num_blocks) == (32, 8, 16, 80000)
    if n == 4:
        assert c.num_seqs == 16 and c.context_lens.min() >= 16384 and c.context_lens.max() <= 32768
        assert (c.num_heads, c.num_kv_heads, c.block_size, c.num_blocks) == (64, 8, 256, 2400)
    assert c.dtype == W.BF16 and c.head_dim == 128


def test_prefill_config():
    c = W.chunked_prefill()
    assert c.num_seqs == 32 and c.causal
    assert c.prefix_lens.min() >= 0 and c.prefix_lens.max() <= 2048
    assert c.chunk_lens.min() >= 64 and c.chunk_lens.max() <= 512
    assert np.array_equal(np.diff(c.cu_seqlens_q), c.chunk_lens)
    assert np.array_equal(np.diff(c.cu_seqlens_k), c.prefix_lens + c.chunk_lens)
    assert len(np.unique(c.slot_mapping)) == c.total_q
    bs = c.block_size
    for i in range(c.num_seqs):
        for j in (0, int(c.chunk_lens[i]) - 1):
            pos = int(c.prefix_lens[i]) + j
            s = int(c.slot_mapping[c.cu_seqlens_q[i] + j])
            assert s // bs == c.block_tables[i, pos // bs] and s % bs == pos % bs
