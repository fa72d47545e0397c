"""Seeded synthetic inputs for the paged KV cache (shared by the oracle tests and the HIP path).

This module only *draws inputs*: context lengths, block tables, slots, Q/K/V values and the
physical pool contents. It holds none of the attention arithmetic and imports neither
``oracle`` nor ``paged_kv_cache_88_amd``.

The metadata it builds follows the pages' vocabulary:

* A request's tokens occupy fixed-size physical blocks; logical block ``j`` of a request maps
  to physical block ``block_tables[i, j]`` ("推理运行时" (wineandchord.com), section 分页 KV).
* A request with ``n`` tokens needs ``ceil(n / block_size)`` blocks ("LLM Infra 101 v0.5"
  (ifuryst.com), section KV Block Manager: 9/17/33 tokens at block size 16 need 1/2/3 blocks;
  nano-vllm walkthrough (lpnh.cn), section 2 Sequence, ``num_blocks``).
* A slot is the flat token-row index ``physical_block * block_size + offset`` (nano-vllm
  walkthrough, section 2 context, ``slot_mapping``; Mini-SGLang 源码解析（二）, section 6.8,
  row-major flattening ``row * STRIDE + pos``).
* Block-table rows are padded to a multiple of 32 int32 entries (Mini-SGLang 源码解析（二）,
  section 7.7) with the value -1, which is never read.

Physical cache layout: ``key_cache`` and ``value_cache`` are each
``[num_blocks, num_kv_heads, block_size, head_dim]``, so the rows of one (block, kv head)
are contiguous. Pool blocks that no request owns, and the positions of a request's last block
at or after its newest token, hold NaN: a kernel that reads beyond ``context_lens`` poisons its
output.

Random draws use ``numpy.random.default_rng(seed)`` in a fixed order:
lengths, pool permutation, query, new K, new V, pool contents.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

F32 = "f32"
BF16 = "bf16"

BF16_NAN = np.uint16(0x7FC0)


_THREADS = min(8, os.cpu_count() or 1)
_BULK = 1 << 22          # arrays above this many elements are drawn and rounded in parallel chunks


def _round_bf16(x: np.ndarray) -> np.ndarray:
    b = x.view(np.uint32)
    t = b >> np.uint32(16)
    t &= np.uint32(1)
    t += np.uint32(0x7FFF)
    t += b
    t >>= np.uint32(16)
    out = t.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = BF16_NAN
    return out


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even); return the 16-bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.size <= _BULK or x.ndim == 0:
        return _round_bf16(x)
    out = np.empty(x.shape, np.uint16)
    step = -(-x.shape[0] // (4 * _THREADS))

    def work(i):
        out[i * step:(i + 1) * step] = _round_bf16(x[i * step:(i + 1) * step])

    with ThreadPoolExecutor(_THREADS) as ex:
        list(ex.map(work, range(-(-x.shape[0] // step))))
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact upcast of bfloat16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def blocks_for_tokens(n: int, block_size: int) -> int:
    """Number of blocks that hold ``n`` tokens: ceil(n / block_size)."""
    return -(-int(n) // int(block_size))


def align_up_32(n: int) -> int:
    """Round ``n`` up to a multiple of 32 (block-table row stride, 128 bytes of int32)."""
    return (int(n) + 31) // 32 * 32


def _draw_values(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    """N(0, 1) values in storage form: float32 array, or uint16 bf16 bit patterns.

    Large arrays are split along the first axis into 16 chunks, each filled by a child generator
    spawned from ``rng`` (deterministic for a given seed and call order)."""
    v = np.empty(shape, np.float32)
    if v.size <= _BULK or v.shape[0] < 16:
        rng.standard_normal(dtype=np.float32, out=v)
    else:
        kids = rng.spawn(16)
        step = -(-v.shape[0] // 16)

        def work(i):
            if i * step < v.shape[0]:
                kids[i].standard_normal(dtype=np.float32, out=v[i * step:(i + 1) * step])

        with ThreadPoolExecutor(_THREADS) as ex:
            list(ex.map(work, range(16)))
    return v if dtype == F32 else f32_to_bf16_bits(v)


def storage_nan(dtype: str):
    return np.float32(np.nan) if dtype == F32 else BF16_NAN


def storage_np_dtype(dtype: str):
    return np.float32 if dtype == F32 else np.uint16


def to_f32(a: np.ndarray, dtype: str) -> np.ndarray:
    """Storage form -> float32 (exact for both dtypes)."""
    return np.asarray(a, dtype=np.float32) if dtype == F32 else bf16_bits_to_f32(a)


@dataclass
class Pool:
    """Physical K/V pool in compact form: only owned blocks carry values; the rest is NaN."""

    num_blocks: int
    num_kv_heads: int
    block_size: int
    head_dim: int
    dtype: str
    used_blocks: np.ndarray          # int32 [U] physical ids that carry values
    key_blocks: np.ndarray           # [U, Hkv, bs, D] storage dtype
    value_blocks: np.ndarray         # [U, Hkv, bs, D] storage dtype

    @property
    def block_shape(self):
        return (self.num_kv_heads, self.block_size, self.head_dim)

    def dense(self):
        """Full host pool arrays ``[NB, Hkv, bs, D]`` (NaN outside the owned blocks)."""
        shape = (self.num_blocks,) + self.block_shape
        kc = np.full(shape, storage_nan(self.dtype), dtype=storage_np_dtype(self.dtype))
        vc = np.full(shape, storage_nan(self.dtype), dtype=storage_np_dtype(self.dtype))
        kc[self.used_blocks] = self.key_blocks
        vc[self.used_blocks] = self.value_blocks
        return kc, vc


def cached_rows(pool: "Pool"):
    """Every row of the pool's owned blocks as store input: K and V ``[N, Hkv, D]`` (storage dtype) and
    the slot of each row (block * block_size + offset); rows not holding a cached token (NaN) get slot
    -1. Used to fill a cache of another element type through its own store call."""
    u, hkv, bs, d = pool.key_blocks.shape
    kr = pool.key_blocks.transpose(0, 2, 1, 3).reshape(u * bs, hkv, d)
    vr = pool.value_blocks.transpose(0, 2, 1, 3).reshape(u * bs, hkv, d)
    slots = (pool.used_blocks.astype(np.int64)[:, None] * bs + np.arange(bs)[None, :]).reshape(-1)
    as_f = (lambda a: bf16_bits_to_f32(a)) if pool.dtype == BF16 else (lambda a: np.asarray(a, np.float32))
    bad = np.isnan(as_f(kr)).any(axis=(1, 2)) | np.isnan(as_f(vr)).any(axis=(1, 2))
    return kr, vr, np.where(bad, -1, slots).astype(np.int32)


@dataclass
class DecodeCase:
    """One decode step: store one new token per sequence, then attend over ``context_lens``."""

    name: str
    seed: int
    dtype: str
    num_seqs: int
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    scale: float
    context_lens: np.ndarray         # int32 [B]; includes the token stored this step
    block_tables: np.ndarray         # int32 [B, stride], padded with -1
    slot_mapping: np.ndarray         # int32 [B]; slot of position context_lens - 1 (or -1 for L == 0)
    query: np.ndarray                # [B, Hq, D] storage dtype
    key: np.ndarray                  # [B, Hkv, D] new token's K (storage dtype)
    value: np.ndarray                # [B, Hkv, D]
    pool: Pool
    extra: dict = field(default_factory=dict)

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.num_seqs else 0

    @property
    def block_table_stride(self) -> int:
        return int(self.block_tables.shape[1])


@dataclass
class PrefillCase:
    """One chunked prefill step: store each sequence's new chunk, then causal attention of the chunk
    over its cached prefix plus the chunk."""

    name: str
    seed: int
    dtype: str
    num_seqs: int
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    scale: float
    causal: bool
    prefix_lens: np.ndarray          # int32 [B] cached tokens already in the pool
    chunk_lens: np.ndarray           # int32 [B] new tokens this step
    cu_seqlens_q: np.ndarray         # int32 [B+1] prefix sums of chunk_lens
    cu_seqlens_k: np.ndarray         # int32 [B+1] prefix sums of prefix_lens + chunk_lens
    block_tables: np.ndarray         # int32 [B, stride]
    slot_mapping: np.ndarray         # int32 [total_q]
    query: np.ndarray                # [total_q, Hq, D]
    key: np.ndarray                  # [total_q, Hkv, D]
    value: np.ndarray                # [total_q, Hkv, D]
    pool: Pool
    extra: dict = field(default_factory=dict)

    @property
    def total_q(self) -> int:
        return int(self.cu_seqlens_q[-1])

    @property
    def max_seqlen_q(self) -> int:
        return int(self.chunk_lens.max()) if self.num_seqs else 0

    @property
    def max_seqlen_k(self) -> int:
        return int((self.prefix_lens + self.chunk_lens).max()) if self.num_seqs else 0

    @property
    def block_table_stride(self) -> int:
        return int(self.block_tables.shape[1])


def _assign_blocks(rng, lens_total, block_size, num_blocks, stride_min=1):
    """Non-overlapping block ownership: permute the pool and slice it per sequence."""
    nbs = [blocks_for_tokens(n, block_size) for n in lens_total]
    need = int(sum(nbs))
    if need > num_blocks:
        raise ValueError(f"pool of {num_blocks} blocks cannot hold {need} blocks")
    perm = rng.permutation(num_blocks).astype(np.int32)
    stride = align_up_32(max(max(nbs, default=0), stride_min))
    bt = np.full((len(lens_total), stride), -1, dtype=np.int32)
    used = perm[:need]
    off = 0
    for i, nb in enumerate(nbs):
        bt[i, :nb] = perm[off:off + nb]
        off += nb
    return bt, used, nbs


def _fill_pool(rng, dtype, num_blocks, hkv, bs, d, used, bt, nbs, valid_tokens):
    """Random owned blocks; NaN at positions >= valid_tokens[i] inside sequence i's blocks."""
    u = len(used)
    kb = _draw_values(rng, (u, hkv, bs, d), dtype)
    vb = _draw_values(rng, (u, hkv, bs, d), dtype)
    nan = storage_nan(dtype)
    index_of = {int(b): k for k, b in enumerate(used)}
    for i, nb in enumerate(nbs):
        n_valid = int(valid_tokens[i])
        for j in range(nb):
            lo = j * bs
            if lo + bs <= n_valid:
                continue
            k = index_of[int(bt[i, j])]
            start = max(n_valid - lo, 0)
            kb[k, :, start:, :] = nan
            vb[k, :, start:, :] = nan
    return Pool(num_blocks, hkv, bs, d, dtype, used.astype(np.int32), kb, vb)


def _slot(bt_row, pos, bs) -> int:
    return int(bt_row[pos // bs]) * bs + pos % bs


def make_decode_case(name, seed, dtype, context_lens, num_heads, num_kv_heads, head_dim,
                     block_size, num_blocks, scale=None, rng=None):
    """Decode step over given lengths. Position ``L-1`` of each sequence is the new token: its slot is
    poisoned in the pool and the store writes it."""
    rng = np.random.default_rng(seed) if rng is None else rng
    lens = np.asarray(context_lens, dtype=np.int32)
    b = len(lens)
    bt, used, nbs = _assign_blocks(rng, lens, block_size, num_blocks)
    q = _draw_values(rng, (b, num_heads, head_dim), dtype)
    kn = _draw_values(rng, (b, num_kv_heads, head_dim), dtype)
    vn = _draw_values(rng, (b, num_kv_heads, head_dim), dtype)
    valid = np.maximum(lens - 1, 0)
    pool = _fill_pool(rng, dtype, num_blocks, num_kv_heads, block_size, head_dim, used, bt, nbs, valid)
    slots = np.array([_slot(bt[i], int(lens[i]) - 1, block_size) if lens[i] > 0 else -1
                      for i in range(b)], dtype=np.int32)
    scale = 1.0 / math.sqrt(head_dim) if scale is None else float(scale)
    return DecodeCase(name, seed, dtype, b, num_heads, num_kv_heads, head_dim, block_size,
                      num_blocks, scale, lens, bt, slots, q, kn, vn, pool)


def make_prefill_case(name, seed, dtype, prefix_lens, chunk_lens, num_heads, num_kv_heads, head_dim,
                      block_size, num_blocks, causal=True, scale=None, rng=None):
    """Chunked prefill step: the prefix is in the pool, the chunk's K/V are stored via slot_mapping."""
    rng = np.random.default_rng(seed) if rng is None else rng
    p = np.asarray(prefix_lens, dtype=np.int32)
    c = np.asarray(chunk_lens, dtype=np.int32)
    b = len(p)
    lk = p + c
    bt, used, nbs = _assign_blocks(rng, lk, block_size, num_blocks)
    total_q = int(c.sum())
    q = _draw_values(rng, (total_q, num_heads, head_dim), dtype)
    kn = _draw_values(rng, (total_q, num_kv_heads, head_dim), dtype)
    vn = _draw_values(rng, (total_q, num_kv_heads, head_dim), dtype)
    pool = _fill_pool(rng, dtype, num_blocks, num_kv_heads, block_size, head_dim, used, bt, nbs, p)
    cu_q = np.zeros(b + 1, dtype=np.int32)
    cu_k = np.zeros(b + 1, dtype=np.int32)
    cu_q[1:] = np.cumsum(c)
    cu_k[1:] = np.cumsum(lk)
    slots = np.empty(total_q, dtype=np.int32)
    for i in range(b):
        for j in range(int(c[i])):
            slots[cu_q[i] + j] = _slot(bt[i], int(p[i]) + j, block_size)
    scale = 1.0 / math.sqrt(head_dim) if scale is None else float(scale)
    return PrefillCase(name, seed, dtype, b, num_heads, num_kv_heads, head_dim, block_size,
                       num_blocks, scale, bool(causal), p, c, cu_q, cu_k, bt, slots, q, kn, vn, pool)


def plant_dominant_keys(case: DecodeCase, positions, gap: float = 36.0) -> DecodeCase:
    """Make chosen cached tokens dominate each query head's softmax (in place; returns the case).

    ``positions[i][h]`` lists the logical tokens of sequence ``i`` planted for query head ``h`` (kv head
    ``h // G``, G = Hq / Hkv); the positions of the heads of one kv head must be distinct. The head dims are
    split into G disjoint runs of D / G: head ``h`` keeps its drawn query values on run ``h % G`` and gets zeros
    elsewhere, and each planted token's key row (for kv head ``h // G``) is ``c * sign(q_h)`` on that run and
    zero elsewhere. So a planted key scores ``scale * c * sum|q_h|`` for its own head and exactly 0 for the other
    heads of its group, while an ordinary N(0, 1) key scores about N(0, (scale |q_h|)^2). ``c`` (rounded to
    bf16, the same for all of a head's planted keys, so their scores are equal) puts the planted score
    ``gap + 6 scale |q_h|`` above zero: every other token of the head then carries a weight below e^-gap
    relative to a planted one. All non-zero elements of a planted row have one magnitude, so an int8, fp8 or
    int4 cache represents the row exactly. Values are left as drawn.
    A position ``context_lens[i] - 1`` (the token stored this step) is planted in ``case.key``."""
    hq, hkv, d, bs = case.num_heads, case.num_kv_heads, case.head_dim, case.block_size
    g = hq // hkv
    run = d // g
    q = to_f32(case.query, case.dtype).astype(np.float64)
    blk_index = {int(b): k for k, b in enumerate(case.pool.used_blocks)}
    as_storage = (lambda a: f32_to_bf16_bits(np.asarray(a, np.float32))) if case.dtype == BF16 else \
        (lambda a: np.asarray(a, np.float32))
    for i, per_head in enumerate(positions):
        n = int(case.context_lens[i])
        taken = {}
        for h, pos in enumerate(per_head):
            if len(pos) == 0:
                continue
            lo, hi = (h % g) * run, (h % g + 1) * run
            qh = q[i, h].copy()
            qh[:lo] = 0.0
            qh[hi:] = 0.0
            sgn = np.where(qh[lo:hi] < 0, -1.0, 1.0)
            l1, l2 = np.abs(qh[lo:hi]).sum(), math.sqrt((qh[lo:hi] ** 2).sum())
            if l1 == 0.0:                                   # no usable query: give the head a unit entry
                qh[lo], l1, l2 = 1.0, 1.0, 1.0
            c32 = np.array([(gap + 6 * case.scale * l2) / (case.scale * l1)], np.float32)
            c = float(to_f32(as_storage(c32), case.dtype)[0])      # rounded to the storage dtype
            case.query[i, h] = as_storage(qh.astype(np.float32))
            row = np.zeros(d, np.float32)
            row[lo:hi] = c * sgn
            kvh = h // g
            for t in pos:
                t = int(t)
                if not 0 <= t < n:
                    raise ValueError(f"position {t} outside sequence {i} of {n} tokens")
                if taken.setdefault((kvh, t), h) != h:
                    raise ValueError(f"position {t} of sequence {i} planted for two heads of kv head {kvh}")
                if t == n - 1:
                    case.key[i, kvh] = as_storage(row)
                else:
                    k = blk_index[int(case.block_tables[i, t // bs])]
                    case.pool.key_blocks[k, kvh, t % bs] = as_storage(row)
    return case


# ---- the five workloads -------------------------------------------------------------------------

def lognormal_lengths(rng, n, median, sigma, lo, hi):
    """round(exp(ln(median) + sigma * z)) clipped to [lo, hi]."""
    z = rng.standard_normal(n)
    return np.clip(np.rint(np.exp(math.log(median) + sigma * z)), lo, hi).astype(np.int32)


def tiny_decode(seed: int = 1) -> DecodeCase:
    """4 sequences, lengths 300/70/200/513, block 16, 8 Q heads / 2 KV heads, head_dim 64, fp32,
    128-block pool."""
    return make_decode_case("tiny_decode_fp32", seed, F32, [300, 70, 200, 513], 8, 2, 64, 16, 128)


def qwen8b_decode(seed: int = 2) -> DecodeCase:
    """Batch 64, lengths U[128, 4096], block 256, 32/8 heads, head_dim 128, bf16, 4096-block pool."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(128, 4096, size=64, endpoint=True).astype(np.int32)
    return make_decode_case("decode_b64_u128_4096_bs256", seed, BF16, lens, 32, 8, 128, 256, 4096, rng=rng)


def short_context_decode(seed: int = 3, sigma: float = 1.0) -> DecodeCase:
    """Batch 512, lengths lognormal (median 300, sigma 1) clipped to [16, 2048], block 16, 32/8 heads,
    head_dim 128, bf16, 80000-block shuffled pool."""
    rng = np.random.default_rng(seed)
    lens = lognormal_lengths(rng, 512, 300.0, sigma, 16, 2048)
    c = make_decode_case("decode_b512_lognorm300_bs16", seed, BF16, lens, 32, 8, 128, 16, 80000, rng=rng)
    c.extra["sigma"] = sigma
    return c


def long_context_decode(seed: int = 4) -> DecodeCase:
    """Batch 16, lengths U[16384, 32768], block 256, 64/8 heads, head_dim 128, bf16, 2400-block pool."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(16384, 32768, size=16, endpoint=True).astype(np.int32)
    return make_decode_case("decode_b16_u16k_32k_bs256", seed, BF16, lens, 64, 8, 128, 256, 2400, rng=rng)


def chunked_prefill(seed: int = 5) -> PrefillCase:
    """32 sequences, cached prefix U[0, 2048] + chunk U[64, 512], causal, block 256, 32/8 heads,
    head_dim 128, bf16, 4096-block shuffled pool."""
    rng = np.random.default_rng(seed)
    p = rng.integers(0, 2048, size=32, endpoint=True).astype(np.int32)
    c = rng.integers(64, 512, size=32, endpoint=True).astype(np.int32)
    return make_prefill_case("prefill_b32_prefix2k_chunk512_bs256", seed, BF16, p, c, 32, 8, 128, 256,
                             4096, causal=True, rng=rng)


CONFIGS = {
    1: tiny_decode,
    2: qwen8b_decode,
    3: short_context_decode,
    4: long_context_decode,
    5: chunked_prefill,
}


def make_config(n: int, seed: int | None = None):
    fn = CONFIGS[n]
    return fn() if seed is None else fn(seed)
