"""Checks that pin the oracle to something other than itself.

Each check takes an ``oracle.Oracle`` and raises ``AssertionError`` on a mismatch. They are run against
the real oracle (tests/test_oracle_*.py) and against copies of ``oracle.c`` with planted mistakes
(tests/test_oracle_mutants.py), which must each fail at least one check.

What pins what:
* the pages' worked examples (slot flattening, block split) -- tests/test_golden_host.py;
* closed forms of softmax attention (one key; zero query; constant values; equal keys; two keys
  with a known score gap);
* ``torch.nn.functional.scaled_dot_product_attention`` in float64 on K/V gathered by numpy
  indexing from a pool laid out as ``[num_blocks, num_kv_heads, block_size, head_dim]``, with an
  explicit bottom-right causal mask for chunked prefill;
* invariants: permuting physical block ids, GQA versus MHA with repeated KV heads, decode versus the
  last row of causal prefill, chunk-split invariance;
* int8 cache quantization: exact cases (power-of-two scales), round-half-even ties, the half-step error
  bound, sign symmetry, placement by slot, and decode on an exactly quantized cache equal to decode on
  the float cache;
* fp8 (OCP float8 E4M3) cache quantization: the format's fixed points (zero, the smallest subnormal and
  normal, one, 448, the NaN patterns), its grid structure, encoding and decoding of every code against
  torch's own ``float8_e4m3fn`` conversion (round half to even, NaN past 464), the relative error bound,
  placement by slot, and decode on an exactly representable cache equal to decode on the float cache;
* int4 cache quantization: a hand-encoded row (its four bytes written out from the definition: offset-8
  codes, element 2j in the low nibble), exact cases, round-half-even ties, the half-step error bound, sign
  symmetry (u -> 16 - u), placement by slot, and decode on an exactly quantized cache equal to decode on
  the float cache.
"""
from __future__ import annotations

import math

import numpy as np
import torch

from workloads import F32, blocks_for_tokens


def _rand_pool(rng, nb, hkv, bs, d):
    kc = rng.standard_normal((nb, hkv, bs, d)).astype(np.float32)
    vc = rng.standard_normal((nb, hkv, bs, d)).astype(np.float32)
    return kc, vc


def _tables(rng, lens, bs, nb, stride=None):
    nbs = [blocks_for_tokens(n, bs) for n in lens]
    perm = rng.permutation(nb).astype(np.int32)
    stride = stride or max(max(nbs), 1)
    bt = np.full((len(lens), stride), -1, np.int32)
    off = 0
    for i, k in enumerate(nbs):
        bt[i, :k] = perm[off:off + k]
        off += k
    return bt


def numpy_gather(kc, bt_row, n):
    """Logical rows [0, n) of one table, by numpy indexing: [n, Hkv, D]."""
    bs = kc.shape[2]
    t = np.arange(n)
    return kc[bt_row[t // bs], :, t % bs, :].astype(np.float64)   # advanced axes first: [n, Hkv, D]


def sdpa64(q, k, v, scale, mask=None):
    """Library attention in float64. q [Hq, Lq, D], k/v [Hq, Lk, D]."""
    tq = torch.from_numpy(np.ascontiguousarray(q, np.float64))[None]
    tk = torch.from_numpy(np.ascontiguousarray(k, np.float64))[None]
    tv = torch.from_numpy(np.ascontiguousarray(v, np.float64))[None]
    am = None if mask is None else torch.from_numpy(mask)[None, None]
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=am, scale=scale)
    return o[0].numpy()


# ---- closed forms --------------------------------------------------------------------------------

def check_single_key(orc):
    """One cached token: the output is that token's value row, exactly."""
    rng = np.random.default_rng(11)
    kc, vc = _rand_pool(rng, 8, 2, 4, 8)
    bt = np.array([[5, -1]], np.int32)
    q = rng.standard_normal((1, 4, 8)).astype(np.float32)
    out = orc.decode(F32, q, kc, vc, bt, np.array([1], np.int32), 0.3)
    for h in range(4):
        assert np.array_equal(out[0, h], vc[5, h // 2, 0].astype(np.float64))


def check_zero_query(orc):
    """q = 0: every score ties, the output is the mean of the value rows."""
    rng = np.random.default_rng(12)
    kc, vc = _rand_pool(rng, 16, 2, 4, 8)
    lens = [7, 13]
    bt = _tables(rng, lens, 4, 16)
    q = np.zeros((2, 2, 8), np.float32)
    out = orc.decode(F32, q, kc, vc, bt, np.array(lens, np.int32), 1.0)
    for i, n in enumerate(lens):
        v = numpy_gather(vc, bt[i], n)
        for h in range(2):
            np.testing.assert_allclose(out[i, h], v[:, h].mean(axis=0), rtol=0, atol=1e-12)


def check_constant_values(orc):
    """All value rows equal c: the output is c whatever the scores."""
    rng = np.random.default_rng(13)
    kc, vc = _rand_pool(rng, 16, 1, 4, 8)
    c = rng.standard_normal(8).astype(np.float32)
    vc[:] = c
    bt = _tables(rng, [11], 4, 16)
    q = (3 * rng.standard_normal((1, 2, 8))).astype(np.float32)
    out = orc.decode(F32, q, kc, vc, bt, np.array([11], np.int32), 0.7)
    np.testing.assert_allclose(out[0], np.broadcast_to(c, (2, 8)), rtol=0, atol=1e-12)


def check_equal_keys(orc):
    """All key rows equal: every score ties, the output is the mean of the value rows."""
    rng = np.random.default_rng(14)
    kc, vc = _rand_pool(rng, 16, 2, 4, 8)
    kc[:] = rng.standard_normal(8).astype(np.float32)
    bt = _tables(rng, [9], 4, 16)
    q = rng.standard_normal((1, 4, 8)).astype(np.float32)
    out = orc.decode(F32, q, kc, vc, bt, np.array([9], np.int32), 0.5)
    v = numpy_gather(vc, bt[0], 9)
    for h in range(4):
        np.testing.assert_allclose(out[0, h], v[:, h // 2].mean(axis=0), rtol=0, atol=1e-12)


def check_two_keys_known_gap(orc):
    """Two keys whose scaled scores differ by g: weights are sigmoid(g) and 1 - sigmoid(g).
    q = e0, k0 = a e0, k1 = b e0 -> s0 - s1 = scale (a - b)."""
    d, scale, a, b = 8, 0.25, 3.0, -1.0
    kc = np.zeros((2, 1, 2, d), np.float32)
    vc = np.zeros((2, 1, 2, d), np.float32)
    kc[1, 0, 0, 0], kc[1, 0, 1, 0] = a, b           # logical tokens 0, 1 live in physical block 1
    vc[1, 0, 0, :] = 1.0
    vc[1, 0, 1, :] = -2.0
    q = np.zeros((1, 1, d), np.float32)
    q[0, 0, 0] = 1.0
    out = orc.decode(F32, q, kc, vc, np.array([[1]], np.int32), np.array([2], np.int32), scale)
    w0 = 1.0 / (1.0 + math.exp(-scale * (a - b)))
    np.testing.assert_allclose(out[0, 0], np.full(d, w0 * 1.0 + (1 - w0) * -2.0), rtol=0, atol=1e-12)


# ---- library routine -----------------------------------------------------------------------------

def check_decode_vs_sdpa(orc, hq=8, hkv=2, d=16, bs=4, lens=(1, 3, 4, 5, 9, 17), seed=21):
    rng = np.random.default_rng(seed)
    nb = sum(blocks_for_tokens(n, bs) for n in lens) + 3
    kc, vc = _rand_pool(rng, nb, hkv, bs, d)
    bt = _tables(rng, lens, bs, nb)
    q = rng.standard_normal((len(lens), hq, d)).astype(np.float32)
    scale = 1.0 / math.sqrt(d)
    out = orc.decode(F32, q, kc, vc, bt, np.array(lens, np.int32), scale)
    g = hq // hkv
    for i, n in enumerate(lens):
        k = numpy_gather(kc, bt[i], n).transpose(1, 0, 2).repeat(g, axis=0)
        v = numpy_gather(vc, bt[i], n).transpose(1, 0, 2).repeat(g, axis=0)
        ref = sdpa64(q[i][:, None, :].astype(np.float64), k, v, scale)[:, 0, :]
        np.testing.assert_allclose(out[i], ref, rtol=1e-12, atol=1e-12)


def _prefill_setup(rng, prefix, chunk, hq, hkv, d, bs, extra_blocks=2):
    lk = [p + c for p, c in zip(prefix, chunk)]
    nb = sum(blocks_for_tokens(n, bs) for n in lk) + extra_blocks
    kc, vc = _rand_pool(rng, nb, hkv, bs, d)
    bt = _tables(rng, lk, bs, nb)
    cu_q = np.concatenate([[0], np.cumsum(chunk)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    q = rng.standard_normal((int(cu_q[-1]), hq, d)).astype(np.float32)
    return kc, vc, bt, cu_q, cu_k, q


def check_prefill_vs_sdpa(orc, causal=True, seed=22):
    prefix, chunk = [0, 3, 5, 8], [4, 1, 6, 3]
    hq, hkv, d, bs = 4, 2, 8, 4
    rng = np.random.default_rng(seed)
    kc, vc, bt, cu_q, cu_k, q = _prefill_setup(rng, prefix, chunk, hq, hkv, d, bs)
    scale = 0.4
    out = orc.prefill(F32, q, kc, vc, bt, cu_q, cu_k, scale, causal=causal)
    g = hq // hkv
    for i, (p, c) in enumerate(zip(prefix, chunk)):
        lk = p + c
        k = numpy_gather(kc, bt[i], lk).transpose(1, 0, 2).repeat(g, axis=0)
        v = numpy_gather(vc, bt[i], lk).transpose(1, 0, 2).repeat(g, axis=0)
        qi = q[cu_q[i]:cu_q[i + 1]].transpose(1, 0, 2).astype(np.float64)
        mask = None
        if causal:
            mask = np.arange(lk)[None, :] <= (p + np.arange(c))[:, None]     # bottom-right aligned
        ref = sdpa64(qi, k, v, scale, mask).transpose(1, 0, 2)
        np.testing.assert_allclose(out[cu_q[i]:cu_q[i + 1]], ref, rtol=1e-12, atol=1e-12)


# ---- invariants ----------------------------------------------------------------------------------

def check_block_permutation_invariance(orc, seed=31):
    """Moving every physical block to a new id and rewriting the tables leaves outputs bit-identical."""
    rng = np.random.default_rng(seed)
    lens = [5, 12, 1, 16]
    bs, nb = 4, 20
    kc, vc = _rand_pool(rng, nb, 2, bs, 8)
    bt = _tables(rng, lens, bs, nb)
    q = rng.standard_normal((4, 4, 8)).astype(np.float32)
    cl = np.array(lens, np.int32)
    a = orc.decode(F32, q, kc, vc, bt, cl, 0.3)
    perm = rng.permutation(nb)
    kc2, vc2 = np.empty_like(kc), np.empty_like(vc)
    kc2[perm] = kc
    vc2[perm] = vc
    bt2 = np.where(bt >= 0, perm[np.maximum(bt, 0)], -1).astype(np.int32)
    b = orc.decode(F32, q, kc2, vc2, bt2, cl, 0.3)
    assert np.array_equal(a, b)
    # contiguous layout: identity table over a pool filled in logical order
    kc3 = np.zeros_like(kc)
    vc3 = np.zeros_like(vc)
    bt3 = np.full_like(bt, -1)
    nxt = 0
    for i, n in enumerate(lens):
        for j in range(blocks_for_tokens(n, bs)):
            kc3[nxt], vc3[nxt] = kc[bt[i, j]], vc[bt[i, j]]
            bt3[i, j] = nxt
            nxt += 1
    c = orc.decode(F32, q, kc3, vc3, bt3, cl, 0.3)
    assert np.array_equal(a, c)


def check_gqa_equals_repeated_mha(orc, seed=32):
    rng = np.random.default_rng(seed)
    lens = [6, 10]
    bs, nb, hkv, g, d = 4, 10, 2, 3, 8
    kc, vc = _rand_pool(rng, nb, hkv, bs, d)
    bt = _tables(rng, lens, bs, nb)
    q = rng.standard_normal((2, hkv * g, d)).astype(np.float32)
    cl = np.array(lens, np.int32)
    a = orc.decode(F32, q, kc, vc, bt, cl, 0.5)
    kr = np.ascontiguousarray(np.repeat(kc, g, axis=1))
    vr = np.ascontiguousarray(np.repeat(vc, g, axis=1))
    b = orc.decode(F32, q, kr, vr, bt, cl, 0.5)
    assert np.array_equal(a, b)


def check_decode_is_last_prefill_row(orc, seed=33):
    rng = np.random.default_rng(seed)
    prefix, chunk = [3, 0, 9], [2, 5, 1]
    kc, vc, bt, cu_q, cu_k, q = _prefill_setup(rng, prefix, chunk, 4, 2, 8, 4)
    out = orc.prefill(F32, q, kc, vc, bt, cu_q, cu_k, 0.6, causal=True)
    last = cu_q[1:] - 1
    lk = (cu_k[1:] - cu_k[:-1]).astype(np.int32)
    dec = orc.decode(F32, q[last], kc, vc, bt, lk, 0.6)
    assert np.array_equal(out[last], dec)


def check_chunk_split_invariance(orc, seed=34):
    """Prefill of (prefix P, chunk C) gives rows P..P+C-1 of one causal prefill over P + C tokens."""
    rng = np.random.default_rng(seed)
    p, c = 6, 5
    kc, vc, bt, _, _, _ = _prefill_setup(rng, [p], [c], 2, 1, 8, 4)
    q = rng.standard_normal((p + c, 2, 8)).astype(np.float32)
    whole = orc.prefill(F32, q, kc, vc, bt, np.array([0, p + c], np.int32), np.array([0, p + c], np.int32),
                        0.35, causal=True)
    part = orc.prefill(F32, q[p:], kc, vc, bt, np.array([0, c], np.int32), np.array([0, p + c], np.int32),
                       0.35, causal=True)
    assert np.array_equal(whole[p:], part)


def check_store_places_rows(orc, seed=41):
    """Store then read back by numpy indexing of the [NB, Hkv, bs, D] layout; untouched rows keep
    their sentinel; negative slots write nothing."""
    rng = np.random.default_rng(seed)
    nb, hkv, bs, d = 6, 3, 4, 5
    kc = np.full((nb, hkv, bs, d), -7.0, np.float32)
    vc = np.full((nb, hkv, bs, d), -9.0, np.float32)
    slots = np.array([0, 23, 5, -1, 14], np.int32)
    key = rng.standard_normal((5, hkv, d)).astype(np.float32)
    val = rng.standard_normal((5, hkv, d)).astype(np.float32)
    orc.store(F32, key, val, kc, vc, slots)
    touched = np.zeros((nb, bs), bool)
    for n, s in enumerate(slots):
        if s < 0:
            continue
        assert np.array_equal(kc[s // bs, :, s % bs, :], key[n])
        assert np.array_equal(vc[s // bs, :, s % bs, :], val[n])
        touched[s // bs, s % bs] = True
    assert np.all(kc.transpose(0, 2, 1, 3)[~touched] == -7.0)
    assert np.all(vc.transpose(0, 2, 1, 3)[~touched] == -9.0)


def check_gather_matches_numpy_indexing(orc, seed=42):
    """Gather of logical tokens equals numpy indexing of the [NB, Hkv, bs, D] pool (several KV heads,
    a ragged last block)."""
    rng = np.random.default_rng(seed)
    kc, vc = _rand_pool(rng, 9, 3, 4, 6)
    bt = _tables(rng, [14], 4, 9)
    ko, vo = orc.gather(F32, kc, vc, bt[0], 14)
    assert np.array_equal(ko.astype(np.float64), numpy_gather(kc, bt[0], 14))
    assert np.array_equal(vo.astype(np.float64), numpy_gather(vc, bt[0], 14))


def _sentinel_pool(nb, hkv, bs, d):
    """K holds 1, 2, 3, ... and V holds -1, -2, -3, ... in storage order: every element of the pool is
    distinct, so each block's contents name the block they came from. Small integers are exact in bf16."""
    n = nb * hkv * bs * d
    k = np.arange(1, n + 1, dtype=np.float32).reshape(nb, hkv, bs, d)
    return k, -k


def _copy_blocks_case(orc, dtype, pairs, holds, nb=5, hkv=2, bs=2, d=4):
    """Copy ``pairs`` in a sentinel pool; afterwards block b of both caches must hold what block holds[b]
    held before (worked out by hand from the pair list)."""
    from workloads import BF16, f32_to_bf16_bits

    k0, v0 = _sentinel_pool(nb, hkv, bs, d)
    if dtype == BF16:
        kc, vc = f32_to_bf16_bits(k0), f32_to_bf16_bits(v0)
    else:
        kc, vc = k0.copy(), v0.copy()
    before_k, before_v = kc.copy(), vc.copy()
    orc.copy_blocks(dtype, kc, vc, np.array(pairs, np.int32))
    for b, src in enumerate(holds):
        assert np.array_equal(kc[b], before_k[src]), f"K block {b} should hold old block {src}"
        assert np.array_equal(vc[b], before_v[src]), f"V block {b} should hold old block {src}"


def check_copy_blocks_worked_cases(orc):
    """Copy-on-write of whole blocks ("推理运行时", section Prefix cache 与 copy-on-write: a branch that
    writes into a shared block first gets a private copy of it). Pool of 5 blocks x 2 kv heads x 2 rows x
    4 dims with every element distinct.
    * pairs (3 -> 1), (0 -> 2): block 1 now holds old block 3 and block 2 old block 0; blocks 0, 3 and 4
      (the sources and the untouched neighbour of both destinations) keep their contents; both kv heads
      and both K and V move.
    * pairs (1 -> 0), (0 -> 2): block 0 is written by the first pair and read by the second; the copy
      reads every source before writing, so block 2 gets old block 0, not old block 1.
    Checked for float32 and for bf16 bit patterns (2-byte elements)."""
    from workloads import BF16

    for dt in (F32, BF16):
        _copy_blocks_case(orc, dt, [[3, 1], [0, 2]], [0, 3, 0, 3, 4])
        _copy_blocks_case(orc, dt, [[1, 0], [0, 2]], [1, 1, 0, 3, 4])
        _copy_blocks_case(orc, dt, [[4, 3]], [0, 1, 2, 4, 4])
    # one element written out: K of block 1, kv head 1, row 0, dim 2 after (3 -> 1) is old K[3, 1, 0, 2],
    # the element at flat index ((3 * 2 + 1) * 2 + 0) * 4 + 2 = 58, which holds 59
    k, v = _sentinel_pool(5, 2, 2, 4)
    orc.copy_blocks(F32, k, v, np.array([[3, 1]], np.int32))
    assert k[1, 1, 0, 2] == 59.0 and v[1, 1, 0, 2] == -59.0


def check_int8_power_of_two_scale(orc):
    """Rows whose largest magnitude is 127 * 2^-3 (a negative element) and whose other elements are integer
    multiples of 2^-3: scale = 2^-3 exactly, codes = the integers, dequantized values = the inputs."""
    k = np.array([[-127, 5, 0, 126, -3, 64, 1, -1], [100, -127, 7, 0, 0, 0, 2, 9]], np.int64)
    x = (k * 0.125).astype(np.float32)
    codes, scales = orc.quantize_int8(F32, x)
    assert np.array_equal(scales, np.full(2, 0.125, np.float32))
    assert np.array_equal(codes.astype(np.int64), k)
    assert np.array_equal(orc.dequantize_int8(codes, scales), x.astype(np.float64))


def check_int8_ties_to_even(orc):
    """scale 1 (absmax 127): halves round to the even integer (round-half-even), both signs."""
    x = np.array([[127.0, 0.5, 1.5, 2.5, 3.5, -0.5, -2.5, 126.5, -3.5, 0.0]], np.float32)
    codes, scales = orc.quantize_int8(F32, x)
    assert scales[0] == 1.0
    assert codes[0].tolist() == [127, 0, 2, 2, 4, 0, -2, 126, -4, 0]


def check_int8_zero_row_bound_and_symmetry(orc, seed=51):
    """A zero row gives scale 0 and codes 0. Random rows: |code * scale - x| <= scale / 2, the largest
    magnitude maps to +-127, and negating a row negates its codes with the same scale."""
    rng = np.random.default_rng(seed)
    z_codes, z_scales = orc.quantize_int8(F32, np.zeros((1, 16), np.float32))
    assert z_scales[0] == 0.0 and not z_codes.any()
    x = (rng.standard_normal((40, 64)) * rng.uniform(0.01, 100, (40, 1))).astype(np.float32)
    codes, scales = orc.quantize_int8(F32, x)
    err = np.abs(orc.dequantize_int8(codes, scales) - x.astype(np.float64))
    assert np.all(err <= scales[:, None].astype(np.float64) * (0.5 + 1e-6))
    i = np.argmax(np.abs(x), axis=1)
    assert np.array_equal(np.abs(codes[np.arange(40), i]).astype(np.int64), np.full(40, 127))
    n_codes, n_scales = orc.quantize_int8(F32, -x)
    assert np.array_equal(n_scales, scales) and np.array_equal(n_codes.astype(np.int64), -codes.astype(np.int64))


def check_int8_store_places_rows(orc, seed=52):
    """store_int8 puts each row's codes and scale at (s // bs, head, s % bs) of the [NB, Hkv, bs(, D)]
    arrays; untouched rows keep their sentinels; negative slots write nothing."""
    rng = np.random.default_rng(seed)
    nb, hkv, bs, d = 5, 2, 4, 8
    kc = np.full((nb, hkv, bs, d), 99, np.int8)
    vc = np.full((nb, hkv, bs, d), -99, np.int8)
    ks = np.full((nb, hkv, bs), -1.0, np.float32)
    vs = np.full((nb, hkv, bs), -2.0, np.float32)
    slots = np.array([3, 17, -1, 8, 19], np.int32)
    key = rng.standard_normal((5, hkv, d)).astype(np.float32)
    val = (3 * rng.standard_normal((5, hkv, d))).astype(np.float32)
    orc.store_int8(F32, key, val, kc, vc, ks, vs, slots)
    touched = np.zeros((nb, bs), bool)
    for n, s in enumerate(slots):
        if s < 0:
            continue
        for h in range(hkv):
            kq, ksc = orc.quantize_int8(F32, key[n, h][None])
            vq, vsc = orc.quantize_int8(F32, val[n, h][None])
            assert np.array_equal(kc[s // bs, h, s % bs], kq[0]) and ks[s // bs, h, s % bs] == ksc[0]
            assert np.array_equal(vc[s // bs, h, s % bs], vq[0]) and vs[s // bs, h, s % bs] == vsc[0]
        touched[s // bs, s % bs] = True
    assert np.all(kc.transpose(0, 2, 1, 3)[~touched] == 99) and np.all(vc.transpose(0, 2, 1, 3)[~touched] == -99)
    assert np.all(ks.transpose(0, 2, 1)[~touched] == -1.0) and np.all(vs.transpose(0, 2, 1)[~touched] == -2.0)


def check_int8_decode_exact_case_matches_float_decode(orc, seed=53):
    """When every row is an integer multiple of a power of two with absmax 127 times it, quantization
    is exact, so decode over the dequantized int8 cache ("f64") equals decode over the float cache."""
    rng = np.random.default_rng(seed)
    nb, hkv, bs, d = 8, 2, 4, 8
    ints = rng.integers(-127, 128, size=(nb, hkv, bs, d))
    ints[..., 0] = np.where(rng.random((nb, hkv, bs)) < 0.5, 127, -127)
    kf = (ints * 0.25).astype(np.float32)
    vf = (np.roll(ints, 1, axis=-1) * 0.5).astype(np.float32)
    kq, ks = orc.quantize_int8(F32, kf)
    vq, vs = orc.quantize_int8(F32, vf)
    bt = _tables(rng, [13, 5], bs, nb)
    q = rng.standard_normal((2, 4, d)).astype(np.float32)
    lens = np.array([13, 5], np.int32)
    ref = orc.decode(F32, q, kf, vf, bt, lens, 0.01)
    got = orc.decode("f64", q.astype(np.float64), orc.dequantize_int8(kq, ks), orc.dequantize_int8(vq, vs), bt, lens,
                     0.01)
    assert np.abs(got - ref).max() <= 1e-12 * max(1.0, np.abs(ref).max())


def check_e4m3_fixed_points_and_grid(orc):
    """Values the E4M3 format fixes: 0x00 = 0, 0x80 = -0, 0x01 = 2^-9 (smallest subnormal), 0x08 = 2^-6
    (smallest normal), 0x38 = 1, 0x40 = 2, 0x7e = 448 (largest finite), 0x7f and 0xff NaN. The non-negative
    finite codes increase; within the subnormals and the first binade the step is 2^-9; each further binade of
    8 codes doubles the one before; negative codes mirror positive ones."""
    v = [orc.e4m3_value(c) for c in range(256)]
    assert v[0x00] == 0.0 and not math.copysign(1.0, v[0x00]) < 0
    assert v[0x80] == 0.0 and math.copysign(1.0, v[0x80]) < 0
    assert v[0x01] == 2.0 ** -9 and v[0x08] == 2.0 ** -6 and v[0x38] == 1.0 and v[0x40] == 2.0 and v[0x7e] == 448.0
    assert math.isnan(v[0x7f]) and math.isnan(v[0xff])
    assert all(v[c + 1] > v[c] for c in range(0x7e))
    assert all(v[c + 1] - v[c] == 2.0 ** -9 for c in range(16))
    assert all(v[c + 8] == 2 * v[c] for c in range(8, 0x77))
    assert all(v[c | 0x80] == -v[c] for c in range(0x7f))


def check_e4m3_matches_torch(orc, seed=54):
    """Decoding of every code, and encoding of random floats (six decades, both signs), of every code's value,
    of every midpoint between neighbouring codes (ties), of points just off the midpoints, and of values
    around the top of the range, against torch's float8_e4m3fn conversion on the CPU."""
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    tv = codes.view(torch.float8_e4m3fn).double().numpy()
    ov = np.array([orc.e4m3_value(c) for c in range(256)])
    assert np.array_equal(np.isnan(tv), np.isnan(ov))
    fin = ~np.isnan(tv)
    assert np.array_equal(tv[fin], ov[fin]) and np.array_equal(np.signbit(tv[fin]), np.signbit(ov[fin]))
    rng = np.random.default_rng(seed)
    pos = np.array([orc.e4m3_value(c) for c in range(0x7f)])
    mids = (pos[:-1] + pos[1:]) / 2
    xs = np.concatenate([rng.standard_normal(4000) * 10.0 ** rng.uniform(-4, 2.6, 4000), pos, -pos, mids, -mids,
                         np.nextafter(mids, 0), np.nextafter(mids, 1e9), [448.0, 455.0, 463.99, 464.0, 464.01, 470.0,
                                                                          -464.0, -470.0, 1e-9, -1e-9, 0.0, -0.0]])
    xs = xs.astype(np.float32)
    want = torch.from_numpy(xs).to(torch.float8_e4m3fn).view(torch.uint8).numpy().astype(np.int64)
    got = np.array([orc.e4m3_encode(x) for x in xs], np.int64)
    assert np.array_equal(got, want)


def check_fp8_zero_row_bound_and_symmetry(orc, seed=55):
    """A zero row gives scale 0 and codes 0. Random rows: scale = max|x| / 448, the largest magnitude maps to
    +-448, |e4m3(code) * scale - x| <= 2^-4 |x| where x / scale is at least 2^-6 (normal codes) and
    <= 2^-10 scale below, and negating a row flips the sign bits with the same scale."""
    rng = np.random.default_rng(seed)
    z_codes, z_scales = orc.quantize_fp8(F32, np.zeros((1, 16), np.float32))
    assert z_scales[0] == 0.0 and not z_codes.any()
    x = (rng.standard_normal((40, 64)) * rng.uniform(0.01, 100, (40, 1))).astype(np.float32)
    x[3, :8] = 1e-4 * x[3, 8]                      # entries deep in the subnormal range of the row
    codes, scales = orc.quantize_fp8(F32, x)
    a = np.abs(x).max(axis=1)
    assert np.array_equal(scales, (a / np.float32(448.0)).astype(np.float32))
    deq = orc.dequantize_fp8(codes, scales)
    err = np.abs(deq - x.astype(np.float64))
    sc = scales[:, None].astype(np.float64)
    normal = np.abs(x) >= 2.0 ** -6 * sc
    assert np.all(err[normal] <= 2.0 ** -4 * np.abs(x.astype(np.float64))[normal] * (1 + 1e-6))
    assert np.all(err[~normal] <= 2.0 ** -10 * np.broadcast_to(sc, x.shape)[~normal] * (1 + 1e-6))
    i = np.argmax(np.abs(x), axis=1)
    assert np.array_equal(codes[np.arange(40), i] & 0x7f, np.full(40, 0x7e))
    n_codes, n_scales = orc.quantize_fp8(F32, -x)
    assert np.array_equal(n_scales, scales) and np.array_equal(n_codes, codes ^ 0x80)


def check_fp8_store_places_rows(orc, seed=56):
    """store_fp8 puts each row's codes and scale at (s // bs, head, s % bs) of the [NB, Hkv, bs(, D)]
    arrays; untouched rows keep their sentinels; negative slots write nothing."""
    rng = np.random.default_rng(seed)
    nb, hkv, bs, d = 5, 2, 4, 8
    kc = np.full((nb, hkv, bs, d), 99, np.uint8)
    vc = np.full((nb, hkv, bs, d), 199, np.uint8)
    ks = np.full((nb, hkv, bs), -1.0, np.float32)
    vs = np.full((nb, hkv, bs), -2.0, np.float32)
    slots = np.array([3, 17, -1, 8, 19], np.int32)
    key = rng.standard_normal((5, hkv, d)).astype(np.float32)
    val = (3 * rng.standard_normal((5, hkv, d))).astype(np.float32)
    orc.store_fp8(F32, key, val, kc, vc, ks, vs, slots)
    touched = np.zeros((nb, bs), bool)
    for n, s in enumerate(slots):
        if s < 0:
            continue
        for h in range(hkv):
            kq, ksc = orc.quantize_fp8(F32, key[n, h][None])
            vq, vsc = orc.quantize_fp8(F32, val[n, h][None])
            assert np.array_equal(kc[s // bs, h, s % bs], kq[0]) and ks[s // bs, h, s % bs] == ksc[0]
            assert np.array_equal(vc[s // bs, h, s % bs], vq[0]) and vs[s // bs, h, s % bs] == vsc[0]
        touched[s // bs, s % bs] = True
    assert np.all(kc.transpose(0, 2, 1, 3)[~touched] == 99) and np.all(vc.transpose(0, 2, 1, 3)[~touched] == 199)
    assert np.all(ks.transpose(0, 2, 1)[~touched] == -1.0) and np.all(vs.transpose(0, 2, 1)[~touched] == -2.0)


def check_fp8_decode_exact_case_matches_float_decode(orc, seed=57):
    """Rows whose elements are E4M3 values times a power of two, with one element at +-448 times it: the
    quantization is exact, so decode over the dequantized fp8 cache ("f64") equals decode over the float
    cache."""
    rng = np.random.default_rng(seed)
    nb, hkv, bs, d = 8, 2, 4, 8
    grid = np.array([orc.e4m3_value(c) for c in range(0x7f)])
    pick = grid[rng.integers(0, 0x7f, size=(nb, hkv, bs, d))] * np.where(rng.random((nb, hkv, bs, d)) < 0.5, 1, -1)
    pick[..., 0] = np.where(rng.random((nb, hkv, bs)) < 0.5, 448.0, -448.0)
    kf = (pick * 0.25).astype(np.float32)
    vf = (np.roll(pick, 1, axis=-1) * 2.0 ** -10).astype(np.float32)
    kq, ks = orc.quantize_fp8(F32, kf)
    vq, vs = orc.quantize_fp8(F32, vf)
    assert np.array_equal(orc.dequantize_fp8(kq, ks), kf.astype(np.float64))
    bt = _tables(rng, [13, 5], bs, nb)
    q = rng.standard_normal((2, 4, d)).astype(np.float32)
    lens = np.array([13, 5], np.int32)
    ref = orc.decode(F32, q, kf, vf, bt, lens, 0.01)
    got = orc.decode("f64", q.astype(np.float64), orc.dequantize_fp8(kq, ks), orc.dequantize_fp8(vq, vs), bt, lens,
                     0.01)
    assert np.abs(got - ref).max() <= 1e-12 * max(1.0, np.abs(ref).max())


def check_int4_hand_encoded_row(orc):
    """Row [3.5, -3.5, 0, 1, 0.25, -0.25, 1.5, 2]: absmax 3.5, scale 0.5; q = [7, -7, 0, 2, 0 (tie 0.5 to
    even), 0 (tie -0.5), 3, 4]; u = q + 8 = [15, 1, 8, 10, 8, 8, 11, 12]; bytes (low nibble first) 0x1f,
    0xa8, 0x88, 0xcb, worked by hand from the definition."""
    x = np.array([[3.5, -3.5, 0.0, 1.0, 0.25, -0.25, 1.5, 2.0]], np.float32)
    codes, scales = orc.quantize_int4(F32, x)
    assert scales.tolist() == [0.5]
    assert codes[0].tolist() == [0x1F, 0xA8, 0x88, 0xCB]
    assert orc.dequantize_int4(codes, scales)[0].tolist() == [3.5, -3.5, 0.0, 1.0, 0.0, 0.0, 1.5, 2.0]


def check_int4_power_of_two_scale(orc):
    """Rows whose largest magnitude is 7 * 2^-2 and whose elements are integer multiples of 2^-2:
    scale = 2^-2 exactly, q = the integers, dequantized values = the inputs."""
    k = np.array([[-7, 5, 0, 6, -3, 4, 1, -1, 2, -6], [7, -7, 3, 0, 0, 0, 2, -2, -5, 1]], np.int64)
    x = (k * 0.25).astype(np.float32)
    codes, scales = orc.quantize_int4(F32, x)
    assert np.array_equal(scales, np.full(2, 0.25, np.float32))
    lo, hi = (codes & 15).astype(np.int64) - 8, (codes >> 4).astype(np.int64) - 8
    assert np.array_equal(np.stack([lo, hi], axis=-1).reshape(2, -1), k)
    assert np.array_equal(orc.dequantize_int4(codes, scales), x.astype(np.float64))


def check_int4_ties_to_even(orc):
    """scale 1 (absmax 7): halves round to the even integer (round-half-even), both signs."""
    x = np.array([[7.0, 0.5, 1.5, 2.5, 3.5, -0.5, -2.5, 6.5, -3.5, 0.0]], np.float32)
    codes, scales = orc.quantize_int4(F32, x)
    assert scales[0] == 1.0
    q = np.stack([(codes[0] & 15).astype(int) - 8, (codes[0] >> 4).astype(int) - 8], axis=-1).reshape(-1)
    assert q.tolist() == [7, 0, 2, 2, 4, 0, -2, 6, -4, 0]


def check_int4_zero_row_bound_and_symmetry(orc, seed=58):
    """A zero row gives scale 0 and bytes 0x88 (q = 0). Random rows: |deq - x| <= scale / 2, the largest
    magnitude maps to +-7, and negating a row maps every code u to 16 - u with the same scale."""
    rng = np.random.default_rng(seed)
    z_codes, z_scales = orc.quantize_int4(F32, np.zeros((1, 16), np.float32))
    assert z_scales[0] == 0.0 and np.all(z_codes == 0x88)
    x = (rng.standard_normal((40, 64)) * rng.uniform(0.01, 100, (40, 1))).astype(np.float32)
    codes, scales = orc.quantize_int4(F32, x)
    deq = orc.dequantize_int4(codes, scales)
    assert np.all(np.abs(deq - x.astype(np.float64)) <= scales[:, None].astype(np.float64) * (0.5 + 1e-6))
    i = np.argmax(np.abs(x), axis=1)
    assert np.array_equal(np.abs(deq[np.arange(40), i]), 7 * scales.astype(np.float64))
    n_codes, n_scales = orc.quantize_int4(F32, -x)
    u = np.stack([codes & 15, codes >> 4], -1).astype(np.int64)
    nu = np.stack([n_codes & 15, n_codes >> 4], -1).astype(np.int64)
    assert np.array_equal(n_scales, scales) and np.array_equal(nu, 16 - u)


def check_int4_store_places_rows(orc, seed=59):
    """store_int4 puts each row's bytes and scale at (s // bs, head, s % bs) of the [NB, Hkv, bs(, D / 2)]
    arrays; untouched rows keep their sentinels; negative slots write nothing."""
    rng = np.random.default_rng(seed)
    nb, hkv, bs, d = 5, 2, 4, 8
    kc = np.full((nb, hkv, bs, d // 2), 0x55, np.uint8)
    vc = np.full((nb, hkv, bs, d // 2), 0xAA, np.uint8)
    ks = np.full((nb, hkv, bs), -1.0, np.float32)
    vs = np.full((nb, hkv, bs), -2.0, np.float32)
    slots = np.array([3, 17, -1, 8, 19], np.int32)
    key = rng.standard_normal((5, hkv, d)).astype(np.float32)
    val = (3 * rng.standard_normal((5, hkv, d))).astype(np.float32)
    orc.store_int4(F32, key, val, kc, vc, ks, vs, slots)
    touched = np.zeros((nb, bs), bool)
    for n, s in enumerate(slots):
        if s < 0:
            continue
        for h in range(hkv):
            kq, ksc = orc.quantize_int4(F32, key[n, h][None])
            vq, vsc = orc.quantize_int4(F32, val[n, h][None])
            assert np.array_equal(kc[s // bs, h, s % bs], kq[0]) and ks[s // bs, h, s % bs] == ksc[0]
            assert np.array_equal(vc[s // bs, h, s % bs], vq[0]) and vs[s // bs, h, s % bs] == vsc[0]
        touched[s // bs, s % bs] = True
    assert np.all(kc.transpose(0, 2, 1, 3)[~touched] == 0x55) and np.all(vc.transpose(0, 2, 1, 3)[~touched] == 0xAA)
    assert np.all(ks.transpose(0, 2, 1)[~touched] == -1.0) and np.all(vs.transpose(0, 2, 1)[~touched] == -2.0)


def check_int4_decode_exact_case_matches_float_decode(orc, seed=60):
    """When every row is an integer multiple of a power of two with absmax 7 times it, 4-bit quantization
    is exact, so decode over the dequantized int4 cache ("f64") equals decode over the float cache."""
    rng = np.random.default_rng(seed)
    nb, hkv, bs, d = 8, 2, 4, 8
    ints = rng.integers(-7, 8, size=(nb, hkv, bs, d))
    ints[..., 0] = np.where(rng.random((nb, hkv, bs)) < 0.5, 7, -7)
    kf = (ints * 0.25).astype(np.float32)
    vf = (np.roll(ints, 1, axis=-1) * 0.5).astype(np.float32)
    kq, ks = orc.quantize_int4(F32, kf)
    vq, vs = orc.quantize_int4(F32, vf)
    bt = _tables(rng, [13, 5], bs, nb)
    q = rng.standard_normal((2, 4, d)).astype(np.float32)
    lens = np.array([13, 5], np.int32)
    ref = orc.decode(F32, q, kf, vf, bt, lens, 0.01)
    got = orc.decode("f64", q.astype(np.float64), orc.dequantize_int4(kq, ks), orc.dequantize_int4(vq, vs), bt, lens,
                     0.01)
    assert np.abs(got - ref).max() <= 1e-12 * max(1.0, np.abs(ref).max())


ALL_CHECKS = [
    check_gather_matches_numpy_indexing,
    check_single_key,
    check_zero_query,
    check_constant_values,
    check_equal_keys,
    check_two_keys_known_gap,
    check_decode_vs_sdpa,
    check_prefill_vs_sdpa,
    check_block_permutation_invariance,
    check_gqa_equals_repeated_mha,
    check_decode_is_last_prefill_row,
    check_chunk_split_invariance,
    check_store_places_rows,
    check_copy_blocks_worked_cases,
    check_int8_power_of_two_scale,
    check_int8_ties_to_even,
    check_int8_zero_row_bound_and_symmetry,
    check_int8_store_places_rows,
    check_int8_decode_exact_case_matches_float_decode,
    check_e4m3_fixed_points_and_grid,
    check_e4m3_matches_torch,
    check_fp8_zero_row_bound_and_symmetry,
    check_fp8_store_places_rows,
    check_fp8_decode_exact_case_matches_float_decode,
    check_int4_hand_encoded_row,
    check_int4_power_of_two_scale,
    check_int4_ties_to_even,
    check_int4_zero_row_bound_and_symmetry,
    check_int4_store_places_rows,
    check_int4_decode_exact_case_matches_float_decode,
]
