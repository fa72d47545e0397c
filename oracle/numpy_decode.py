"""Decode attention over the paged cache in NumPy, float64 -- TEST INFRASTRUCTURE ONLY.

A second CPU statement of the decode, independent of ``oracle.c``: for sequence i with L_i cached tokens,
logical token t lives in row t % block_size of physical block block_tables[i, t // block_size] (the
block-table addressing of the nano-vllm walkthrough, section 2 context, and of "推理运行时", section 分页 KV).
The rows of the context are gathered through the table; the G query heads that share a KV head take their
scores from one matrix product with the gathered keys, s = scale q K^T; the output is the softmax of the
scores applied to the gathered values, sum_t exp(s_t - max s) v_t / sum_t exp(s_t - max s). A context of
length 0 gives zeros. Query head h reads KV head h // G.

The matrix products go through NumPy's BLAS, which is what ``bench.py``'s cpu_baseline leg times beside
the C oracle (with the BLAS thread count). Only ``tests/`` and that leg use this module; it imports nothing
from the HIP package. ``tests/test_oracle_numpy.py`` pins it to the C oracle (itself pinned to closed forms,
invariants and scaled_dot_product_attention).

Arrays use the storage conventions of the workloads: float32 arrays for fp32, uint16 bf16 bit patterns for
bf16; the pool is ``[num_blocks, num_kv_heads, block_size, head_dim]``.
"""
from __future__ import annotations

import numpy as np


def _f64(a, dtype: str) -> np.ndarray:
    """Storage form -> float64, exactly (a bf16 value is the top half of a float32)."""
    a = np.asarray(a)
    if dtype == "bf16":
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def decode(dtype, query, key_cache, value_cache, block_tables, context_lens, scale, seqs=None):
    """``[n, Hq, D]`` float64 outputs for the sequences ``seqs`` (all if None)."""
    q = _f64(query, dtype)
    b, hq, d = q.shape
    nb, hkv, bs, d2 = key_cache.shape
    if d2 != d or hq % hkv:
        raise ValueError("head_dim mismatch or num_heads not a multiple of num_kv_heads")
    g = hq // hkv
    bt = np.asarray(block_tables)
    lens = np.asarray(context_lens)
    sel = np.arange(b) if seqs is None else np.asarray(seqs)
    out = np.zeros((len(sel), hq, d), dtype=np.float64)
    for r, i in enumerate(sel):
        n = int(lens[i])
        if n <= 0:
            continue
        blocks = bt[i, : (n + bs - 1) // bs]
        # [Hkv, tokens, D]: the table's blocks in order, then the first n rows
        k = _f64(key_cache[blocks], dtype).transpose(1, 0, 2, 3).reshape(hkv, -1, d)[:, :n]
        v = _f64(value_cache[blocks], dtype).transpose(1, 0, 2, 3).reshape(hkv, -1, d)[:, :n]
        s = np.matmul(q[i].reshape(hkv, g, d), k.transpose(0, 2, 1)) * float(scale)    # [Hkv, G, n]
        w = np.exp(s - s.max(axis=-1, keepdims=True))
        o = np.matmul(w, v) / w.sum(axis=-1, keepdims=True)                             # [Hkv, G, D]
        out[r] = o.reshape(hq, d)
    return out
