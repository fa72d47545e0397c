"""Planted dominant keys, with the oracle alone (no GPU).

At long contexts the bf16 tolerance |gpu - ref| <= 2e-2 + 1e-2 |ref| cannot see a missing tile when keys are
N(0, 1): outputs are about 1/sqrt(L). The GPU long-context tests therefore plant two equal dominant keys per
query head (``workloads.plant_dominant_keys``, positions from ``tests/needles.py``). These tests show, with the
oracle only, on the long-context decode shape (64 query / 8 kv heads, head_dim 128, block 256, contexts in
[16384, 32768]) that
* the oracle's output is then the mean of the two planted tokens' values (the rest weighs nothing);
* removing either planted token, or counting one of them twice, moves every head's output outside the
  tolerance, so a kernel that drops or repeats a tile holding one cannot pass.
"""
import copy

import numpy as np
import pytest

import needles as N
import workloads as W
from gpu_util import within_tol


def _long_case(seed=4, b=2):
    rng = np.random.default_rng(seed)
    lens = rng.integers(16384, 32768, size=b, endpoint=True).astype(np.int32)
    nb = int(sum(W.blocks_for_tokens(int(n), 256) for n in lens)) + 2
    return W.make_decode_case("needles", seed, W.BF16, lens, 64, 8, 128, 256, nb, rng=rng)


def _rows(case, i, kvh, t):
    """(K, V) storage rows of sequence i, kv head kvh, logical token t (the stored token for t = L - 1)."""
    if t == int(case.context_lens[i]) - 1:
        return case.key[i, kvh], case.value[i, kvh]
    k = int(np.flatnonzero(case.pool.used_blocks == case.block_tables[i, t // case.block_size])[0])
    return case.pool.key_blocks[k, kvh, t % case.block_size], case.pool.value_blocks[k, kvh, t % case.block_size]


def _set_rows(case, i, kvh, t, krow, vrow):
    ko, vo = _rows(case, i, kvh, t)
    ko[...] = krow
    vo[...] = vrow


def _decode(orc, case):
    kc, vc = case.pool.dense()
    orc.store(case.dtype, case.key, case.value, kc, vc, case.slot_mapping)
    return orc.decode(case.dtype, case.query, kc, vc, case.block_tables, case.context_lens, case.scale)


@pytest.fixture(scope="module")
def planted():
    plain = _long_case()
    case = copy.deepcopy(plain)
    pos = N.needle_positions(case, np.random.default_rng(7), workers=1024)
    W.plant_dominant_keys(case, pos)
    return plain, case, pos


@pytest.fixture(scope="module")
def reference(orc, planted):
    return _decode(orc, planted[1])


def test_planted_output_is_the_mean_of_the_planted_values(planted, reference):
    _, case, pos = planted
    g = case.num_heads // case.num_kv_heads
    for i in range(case.num_seqs):
        for h in range(case.num_heads):
            va, vb = (W.to_f32(_rows(case, i, h // g, t)[1], case.dtype).astype(np.float64) for t in pos[i][h])
            assert np.abs(reference[i, h] - (va + vb) / 2).max() <= 1e-9, (i, h)


@pytest.mark.parametrize("which", [0, 1])
def test_dropping_a_planted_token_leaves_the_tolerance(orc, planted, reference, which):
    """Planted token `which` of every head gets back its ordinary drawn key (an ordinary token's weight is
    below e^-36 of a planted one's, so this is the same as leaving it out): every (sequence, head) output then
    has elements outside the tolerance."""
    plain, case, pos = planted
    g = case.num_heads // case.num_kv_heads
    dropped = copy.deepcopy(case)
    for i in range(case.num_seqs):
        for h in range(case.num_heads):
            t = pos[i][h][which]
            k0, v0 = _rows(plain, i, h // g, t)
            _set_rows(dropped, i, h // g, t, k0, _rows(case, i, h // g, t)[1])
    moved = _decode(orc, dropped)
    bad = ~within_tol(moved, reference, W.BF16)
    assert bad.any(axis=-1).all(), f"{(~bad.any(axis=-1)).sum()} heads would not notice the drop"


def test_repeating_a_planted_token_leaves_the_tolerance(orc, planted, reference):
    """A copy of every head's first planted token (same key and value) at an unplanted position, as if a tile
    holding it were counted twice: output (2 v_a + v_b) / 3 instead of (v_a + v_b) / 2, outside the tolerance
    for every (sequence, head)."""
    _, case, pos = planted
    g = case.num_heads // case.num_kv_heads
    twice = copy.deepcopy(case)
    rng = np.random.default_rng(3)
    for i in range(case.num_seqs):
        L = int(case.context_lens[i])
        for kvh in range(case.num_kv_heads):
            used = {t for h in range(kvh * g, (kvh + 1) * g) for t in pos[i][h]}
            for h in range(kvh * g, (kvh + 1) * g):
                f = int(rng.integers(L - 1))
                while f in used:
                    f = int(rng.integers(L - 1))
                used.add(f)
                ka, va = _rows(case, i, kvh, pos[i][h][0])
                _set_rows(twice, i, kvh, f, ka.copy(), va.copy())
    moved = _decode(orc, twice)
    bad = ~within_tol(moved, reference, W.BF16)
    assert bad.any(axis=-1).all(), f"{(~bad.any(axis=-1)).sum()} heads would not notice the repeat"


def test_positions_cover_every_kind_of_boundary(planted):
    """The planted positions include sequence ends, tile, block and part first/last tokens, distinct within
    each kv head, two per head in different 32-token tiles."""
    _, case, pos = planted
    g = case.num_heads // case.num_kv_heads
    parts = N.plan_parts(case.context_lens, case.num_kv_heads, case.block_size, 1024)
    for i in range(case.num_seqs):
        L = int(case.context_lens[i])
        flat = [t for h in range(case.num_heads) for t in pos[i][h]]
        for kvh in range(case.num_kv_heads):
            mine = [t for h in range(kvh * g, (kvh + 1) * g) for t in pos[i][h]]
            assert len(set(mine)) == len(mine) == 2 * g
        for h in range(case.num_heads):
            a, b = pos[i][h]
            assert a // 32 != b // 32
        starts = {s for j, s, n in parts if j == i}
        assert {0, L - 1} & set(flat)
        assert any(t % 32 == 31 for t in flat) and any(t % 256 == 0 for t in flat)
        assert any(t % 256 == 255 for t in flat)
        assert (starts - {0}) & set(flat), "no part start planted"


@pytest.mark.parametrize("lens,hkv,bs,workers", [
    ([30011], 2, 256, 1024), ([16384, 32768, 20000], 8, 256, 1024), ([1, 0, 31, 32, 33, 5000], 8, 16, 2048),
    (list(range(1, 600, 7)), 8, 16, 2048), ([4000] * 16, 8, 16, 1024)])
def test_plan_parts_cover_each_sequence(lens, hkv, bs, workers):
    """The host restatement of the plan: each sequence's parts tile [0, L) in order, every part but the last is
    a whole number of 32-token tiles of one length, and a part's block-table slice fits 64 lanes."""
    parts = N.plan_parts(lens, hkv, bs, workers)
    for i, L in enumerate(lens):
        mine = [(s, n) for j, s, n in parts if j == i]
        if L == 0:
            assert not mine
            continue
        assert mine[0][0] == 0 and sum(n for _, n in mine) == L
        for (s0, n0), (s1, _) in zip(mine, mine[1:]):
            assert s1 == s0 + n0 and n0 % 32 == 0 and n0 == mine[0][1]
        for s, n in mine:
            assert (s + n - 1) // bs - s // bs + 1 <= 64
