"""Helpers for the GPU parity tests: move generated cases to the device, run the HIP path through
the binding, and compare with the oracle."""
from __future__ import annotations

import numpy as np
import torch

import workloads as W

BF16_ATOL, BF16_RTOL = 2e-2, 1e-2     # bf16 outputs vs the fp64 oracle: |gpu - ref| <= atol + rtol |ref|
F32_ATOL = 1e-5                        # fp32 outputs: max |gpu - ref| <= 1e-5


def tdtype(dtype):
    return torch.float32 if dtype == W.F32 else torch.bfloat16


def to_torch(a, dtype, device="cuda"):
    """Storage-form numpy array -> torch tensor on the device (bf16 bits reinterpreted)."""
    a = np.ascontiguousarray(a)
    if dtype == W.F32:
        return torch.from_numpy(a.astype(np.float32, copy=False)).to(device)
    return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)


def to_storage(t, dtype):
    """Device tensor -> storage-form numpy array (float32, or uint16 bf16 bits)."""
    t = t.detach().cpu().contiguous()
    if dtype == W.F32:
        return t.numpy()
    return t.view(torch.int16).numpy().view(np.uint16)


def device_pool(pool: W.Pool, device="cuda"):
    """Caches [NB, Hkv, bs, D] on the device: NaN everywhere, owned blocks filled."""
    shape = (pool.num_blocks,) + pool.block_shape
    td = tdtype(pool.dtype)
    kc = torch.full(shape, float("nan"), dtype=td, device=device)
    vc = torch.full(shape, float("nan"), dtype=td, device=device)
    idx = torch.from_numpy(pool.used_blocks.astype(np.int64)).to(device)
    kc.index_copy_(0, idx, to_torch(pool.key_blocks, pool.dtype, device))
    vc.index_copy_(0, idx, to_torch(pool.value_blocks, pool.dtype, device))
    return kc, vc


def i32(a, device="cuda"):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)


def within_tol(gpu, ref, dtype):
    """True where the GPU output is within the stated tolerance of the oracle."""
    gpu = np.asarray(gpu, np.float64)
    if dtype == W.F32:
        return np.abs(gpu - ref) <= F32_ATOL
    return np.abs(gpu - ref) <= BF16_ATOL + BF16_RTOL * np.abs(ref)


def assert_close(gpu, ref, dtype, what=""):
    ok = within_tol(gpu, ref, dtype)
    if not ok.all():
        bad = np.argwhere(~ok)
        i = tuple(bad[0])
        err = np.abs(np.asarray(gpu, np.float64) - ref)
        raise AssertionError(f"{what}: {len(bad)} of {ok.size} outside tolerance; first at {i}: gpu={gpu[i]} "
                             f"ref={ref[i]}; max abs err {err.max():.3g}")


def decode_workers(kind="bf16"):
    """Resident waves the decode plan sizes parts for on this GPU: 4 per compute unit for the matrix-core
    kernel over a bf16 cache, 8 over a quantized cache, and 8 (at most 2048) for the vector-ALU kernel."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    return {"bf16": 4 * cus, "q8": 8 * cus, "valu": min(8 * cus, 2048)}[kind]


def assert_rel_norm(got, ref, bound=1e-2, what=""):
    """||gpu - ref|| / ||ref|| <= bound over all elements: bf16 rounds each softmax weight and each output to
    8 significant bits (relative error <= 2^-9 each), which keeps the norm of the error within ~2^-8 of the
    norm of the output however small the elements are."""
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    r = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))
    assert r <= bound, f"{what}: relative error norm {r:.3g} > {bound}"


def run_decode_case(pkv, c: W.DecodeCase, store=True, device="cuda"):
    """Store the new token (HIP), then decode (HIP). Returns (out as float64 numpy, kc, vc)."""
    kc, vc = device_pool(c.pool, device)
    if store:
        pkv.kv_cache_store(to_torch(c.key, c.dtype), to_torch(c.value, c.dtype), kc, vc, i32(c.slot_mapping))
    q = to_torch(c.query, c.dtype)
    out = torch.empty_like(q)
    pkv.paged_attention_decode(out, q, kc, vc, i32(c.block_tables), i32(c.context_lens), c.max_context_len, c.scale)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), kc, vc


def oracle_decode_case(orc, c: W.DecodeCase, seqs=None):
    """Oracle store into host copies of the pool, then oracle decode (float64)."""
    kc, vc = c.pool.dense()
    orc.store(c.dtype, c.key, c.value, kc, vc, c.slot_mapping)
    return orc.decode(c.dtype, c.query, kc, vc, c.block_tables, c.context_lens, c.scale, seqs=seqs)


def run_prefill_case(pkv, c: W.PrefillCase, device="cuda"):
    """Store the chunk (HIP), then chunked prefill (HIP). Returns float64 numpy [total_q, Hq, D]."""
    kc, vc = device_pool(c.pool, device)
    pkv.kv_cache_store(to_torch(c.key, c.dtype), to_torch(c.value, c.dtype), kc, vc, i32(c.slot_mapping))
    q = to_torch(c.query, c.dtype)
    out = torch.full_like(q, float("nan"))
    pkv.paged_attention_prefill(out, q, kc, vc, i32(c.block_tables), i32(c.cu_seqlens_q), i32(c.cu_seqlens_k),
                                c.max_seqlen_q, c.max_seqlen_k, c.scale, causal=c.causal)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


def oracle_prefill_case(orc, c: W.PrefillCase, rows=None):
    kc, vc = c.pool.dense()
    orc.store(c.dtype, c.key, c.value, kc, vc, c.slot_mapping)
    return orc.prefill(c.dtype, c.query, kc, vc, c.block_tables, c.cu_seqlens_q, c.cu_seqlens_k, c.scale,
                       causal=c.causal, rows=rows)
