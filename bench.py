"""Benchmark of the paged KV cache decode step on one MI355X.

A step is one pass of the hot path over one batch: kv_cache_store of the batch's new token per
sequence, then paged_attention_decode over every sequence's context (the split-K reduce included
when a context spans several partitions), issued as one pkv_paged_decode_step call (the same step as
two calls is timed too). The default workload is batch 512 with context lengths
lognormal (median 300, sigma 1) clipped to [16, 2048], block size 16, 32 query / 8 KV heads,
head_dim 128, bf16, in a shuffled 80000-block pool.

Inputs are resident in HBM before timing. Each step reads a different copy of the pool (R copies,
R * step bytes >> the last-level cache), so K/V come from HBM, not from cache.

Prints one JSON line (rank 0): value = algorithmic bytes of the step / step time (GB/s, wall clock
over the timed steps), plus the roofline of the decode call measured with HIP events on the launch
stream (recorded around runs of ten back-to-back calls: each event costs the stream a few microseconds, so
recording them around every call would slow the calls it measures), and the CPU oracle's rate
on a bounded sample of the same workload. Secondary legs (not part of `value`): the same decode over
int8, fp8 (E4M3) and int4 caches (whole calls, and runs from one shared plan as a model's layers would make
them); the decode call on the other two decode workloads (batch 64 at block 256,
batch 16 at 16k-32k tokens); the chunked-prefill workload on MFMA (bf16, int8 and fp8 caches); and the
practical ceilings measured on the same GPU: the decode's read pattern (scrambled 4 KB and 64 KB chunks), the
matrix cores' rate for the prefill's MFMA instruction, and a bf16 GEMM.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, published
MFMA_BF16_PEAK = 2.5e15     # MI355X dense bf16 MFMA, published


def decode_bytes(c) -> int:
    """Algorithmic bytes of one decode call: K and V of every context token, q and out, the block-table
    entries used and context_lens."""
    e = 4 if c.dtype == "f32" else 2
    lens = c.context_lens.astype(np.int64)
    nb = -(-lens // c.block_size)
    return int(2 * lens.sum() * c.num_kv_heads * c.head_dim * e + 2 * c.num_seqs * c.num_heads * c.head_dim * e
               + 4 * nb.sum() + 4 * c.num_seqs)


def decode_bytes_q8(c) -> int:
    """Algorithmic bytes of one decode call over an 8-bit cache (int8 or fp8 codes): the one-byte codes of K
    and V of every context token, their fp32 row scales, q and out (bf16), the block-table entries used and
    context_lens."""
    lens = c.context_lens.astype(np.int64)
    nb = -(-lens // c.block_size)
    return int(2 * lens.sum() * c.num_kv_heads * (c.head_dim + 4) + 2 * c.num_seqs * c.num_heads * c.head_dim * 2
               + 4 * nb.sum() + 4 * c.num_seqs)


def decode_bytes_q4(c) -> int:
    """Algorithmic bytes of one decode call over an int4 cache: the half-byte codes of K and V of every
    context token, their fp32 row scales, q and out (bf16), the block-table entries used and context_lens."""
    lens = c.context_lens.astype(np.int64)
    nb = -(-lens // c.block_size)
    return int(2 * lens.sum() * c.num_kv_heads * (c.head_dim // 2 + 4) + 2 * c.num_seqs * c.num_heads * c.head_dim * 2
               + 4 * nb.sum() + 4 * c.num_seqs)


Q8_LEGS = {
    "int8": ("int8 codes + fp32 scale per (token, kv head) row", "kv_cache_store_int8", "paged_attention_decode_int8"),
    "fp8": ("float8 E4M3 codes + fp32 scale per (token, kv head) row", "kv_cache_store_fp8",
            "paged_attention_decode_fp8"),
    "int4": ("int4 codes (two per byte) + fp32 scale per (token, kv head) row", "kv_cache_store_int4",
             "paged_attention_decode_int4"),
}


def bench_q8(kind, pkv, torch, W, c, dev, copies, steps, warmup):
    """The same decode workload over a quantized cache (rows quantized by the library's store from the bf16
    values; pool copies rotated as in the main leg): average decode-call time from HIP events around runs of
    back-to-back calls."""
    what, store_name, decode_name = Q8_LEGS[kind]
    store, decode = getattr(pkv, store_name), getattr(pkv, decode_name)
    kr, vr, slots = W.cached_rows(c.pool)

    def tt(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    kr, vr, slots = tt(kr), tt(vr), torch.from_numpy(slots).to(dev)
    shape = (c.num_blocks, c.num_kv_heads, c.block_size, c.head_dim // 2 if kind == "int4" else c.head_dim)
    pools = []
    for _ in range(copies):
        kc = torch.zeros(shape, dtype=torch.int8 if kind == "int8" else torch.uint8, device=dev)
        vc = torch.zeros_like(kc)
        ks = torch.zeros(shape[:3], dtype=torch.float32, device=dev)
        vs = torch.zeros_like(ks)
        store(kr, vr, kc, vc, ks, vs, slots)
        store(tt(c.key), tt(c.value), kc, vc, ks, vs, torch.from_numpy(c.slot_mapping).to(dev))
        pools.append((kc, vc, ks, vs))
    q = tt(c.query)
    out = torch.empty_like(q)
    bt = torch.from_numpy(c.block_tables).to(dev)
    cl = torch.from_numpy(c.context_lens).to(dev)
    ws = torch.empty(pkv.decode_workspace_size(c.num_seqs, c.num_heads, c.num_kv_heads, c.head_dim, c.block_size,
                                               c.max_context_len), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    batch = 10                                # back-to-back calls between an event pair
    for k in range(warmup):
        kc, vc, ks, vs = pools[k % copies]
        decode(out, q, kc, vc, ks, vs, bt, cl, c.max_context_len, c.scale, workspace=ws, stream=stream)
    runs = []
    for b in range(0, steps, batch):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for k in range(b, min(steps, b + batch)):
            kc, vc, ks, vs = pools[k % copies]
            decode(out, q, kc, vc, ks, vs, bt, cl, c.max_context_len, c.scale, workspace=ws, stream=stream)
        e1.record(stream)
        runs.append((e0, e1, min(steps, b + batch) - b))
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(z) / n for a, z, n in runs]))
    finite = bool(torch.isfinite(out.float()).all().item())
    # the same decode as a model's layers run it: one plan per step, then one run per layer from it
    pkv.paged_attention_decode_plan(cl, c.max_context_len, c.num_heads, c.num_kv_heads, c.head_dim, c.block_size,
                                    ws, dtype=torch.bfloat16, cache=kind, stream=stream)
    run = getattr(pkv, decode_name + "_run")
    runs = []
    for b in range(0, steps, batch):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for k in range(b, min(steps, b + batch)):
            kc, vc, ks, vs = pools[k % copies]
            run(out, q, kc, vc, ks, vs, bt, c.max_context_len, c.scale, ws, stream=stream)
        e1.record(stream)
        runs.append((e0, e1, min(steps, b + batch) - b))
    torch.cuda.synchronize()
    run_ms = float(np.mean([a.elapsed_time(z) / n for a, z, n in runs]))
    nbytes = decode_bytes_q4(c) if kind == "int4" else decode_bytes_q8(c)
    return {"workload": c.name, "cache": what,
            "decode_ms": round(ms, 5), "algorithmic_bytes": nbytes,
            "achieved_gbs": round(nbytes / (ms * 1e-3) / 1e9, 2),
            "frac_of_hbm_peak": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "decode_tokens_per_s": round(c.num_seqs / (ms * 1e-3), 1),
            "per_layer_run": {"run_ms": round(run_ms, 5),
                              "frac_of_hbm_peak": round(nbytes / (run_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                              "what": "one paged_attention_decode_plan per step, then the "
                                      f"{decode_name}_run of each layer from it (the plan's kernel is outside)"},
            "outputs_finite": finite and bool(torch.isfinite(out.float()).all().item())}


def store_bytes(c) -> int:
    """Algorithmic bytes of one store call: read and write K and V rows of each new token, plus its slot."""
    e = 4 if c.dtype == "f32" else 2
    n = len(c.slot_mapping)
    return int(n * c.num_kv_heads * c.head_dim * e * 2 * 2 + 4 * n)


def measured_traffic(workload: str):
    """HBM bytes per decode call from the committed rocprofv3 counters (FETCH_SIZE and WRITE_SIZE, each
    scaled by the same counter on a copy of known size), or None when the counters were taken on other
    kernel sources than the ones built now, or on another workload."""
    import hashlib

    path = os.path.join(ROOT, "profiles", f"{workload}_counters.json")
    if not os.path.exists(path):
        return None
    with open(path, encoding="utf-8") as f:
        doc = json.load(f)
    h = hashlib.sha256()
    for src in doc["kernel_sources"]:
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    return doc["decode_call_traffic_bytes"] if h.hexdigest() == doc["kernel_sources_sha256"] else None


def cpu_baseline(c, target_s=12.0, single_s=3.0):
    """Time the oracle (float64) on bounded samples of the same workload: on all host cores, the decode of
    the whole batch repeated until about target_s seconds of CPU work (fewer sequences if one pass is
    already longer); on one core, a sample of about single_s seconds; and its NumPy statement (BLAS
    products, the BLAS thread count recorded) on a sample of about single_s seconds."""
    import oracle

    orc = oracle.default()
    cores = int(orc.max_threads())
    kc, vc = c.pool.dense()
    orc.store(c.dtype, c.key, c.value, kc, vc, c.slot_mapping)
    order = np.random.default_rng(0).permutation(c.num_seqs)
    e = 2 if c.dtype == "bf16" else 4

    def sample_bytes(sel, reps):
        lens = c.context_lens[sel].astype(np.int64)
        return reps * int(2 * lens.sum() * c.num_kv_heads * c.head_dim * e + 2 * len(sel) * c.num_heads * c.head_dim * e
                          + 4 * (-(-lens // c.block_size)).sum() + 4 * len(sel))

    def plan(threads, budget_s):
        probe = np.sort(order[:8]).astype(np.int32)
        t0 = time.perf_counter()
        orc.decode(c.dtype, c.query, kc, vc, c.block_tables, c.context_lens, c.scale, seqs=probe, nthreads=threads)
        per_token = (time.perf_counter() - t0) / max(1, int(c.context_lens[probe].sum()))
        if per_token * int(c.context_lens.sum()) >= budget_s:
            cum = np.cumsum(c.context_lens[order])
            k = max(8, min(c.num_seqs, int(np.searchsorted(cum, budget_s / per_token)) + 1))
            return np.sort(order[:k]).astype(np.int32), 1
        return None, max(1, int(round(budget_s / max(per_token * int(c.context_lens.sum()), 1e-9))))

    def run(threads, seqs, reps):
        t0 = time.perf_counter()
        for _ in range(reps):
            orc.decode(c.dtype, c.query, kc, vc, c.block_tables, c.context_lens, c.scale, seqs=seqs, nthreads=threads)
        return time.perf_counter() - t0

    seqs, reps = plan(cores, target_s)
    dt = run(cores, seqs, reps)
    sel = np.arange(c.num_seqs) if seqs is None else seqs
    nbytes = sample_bytes(sel, reps)
    seqs1, reps1 = plan(1, single_s)
    dt1 = run(1, seqs1, reps1)
    sel1 = np.arange(c.num_seqs) if seqs1 is None else seqs1
    nbytes1 = sample_bytes(sel1, reps1)
    orc.decode(c.dtype, c.query, kc, vc, c.block_tables, c.context_lens, c.scale, seqs=np.sort(order[:1]).astype(np.int32),
               nthreads=cores)                          # leave the oracle on all cores
    # the NumPy statement of the same decode (oracle/numpy_decode.py: gathered blocks, BLAS products), timed on
    # a sample of about single_s seconds, with the BLAS library's thread count
    from oracle import numpy_decode
    try:
        from threadpoolctl import threadpool_info
        blas = [x for x in threadpool_info() if x.get("user_api") == "blas"]
        blas_threads = int(sum(x.get("num_threads", 0) for x in blas)) or None
        blas_lib = blas[0].get("internal_api") if blas else None
    except ImportError:
        blas_threads, blas_lib = None, None
    probe = np.sort(order[:8]).astype(np.int32)
    t0 = time.perf_counter()
    numpy_decode.decode(c.dtype, c.query, kc, vc, c.block_tables, c.context_lens, c.scale, seqs=probe)
    per_seq = (time.perf_counter() - t0) / len(probe)
    kn = int(max(8, min(c.num_seqs, single_s / max(per_seq, 1e-9))))
    seln = np.sort(order[:kn]).astype(np.int32)
    t0 = time.perf_counter()
    numpy_decode.decode(c.dtype, c.query, kc, vc, c.block_tables, c.context_lens, c.scale, seqs=seln)
    dtn = time.perf_counter() - t0
    nbytesn = sample_bytes(seln, 1)
    numpy_leg = {"value": round(nbytesn / dtn / 1e9, 4), "unit": "GB/s", "blas_threads": blas_threads,
                 "blas": blas_lib,
                 "sample": f"decode of {kn} sequences ({int(c.context_lens[seln].sum())} context tokens), float64, "
                           f"{dtn:.2f} s"}
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"decode of {len(sel)} of {c.num_seqs} sequences ({int(c.context_lens[sel].sum())} context tokens) "
                      f"x {reps} passes, float64, {dt:.2f} s",
            "seconds": round(dt, 3), "decode_tokens_per_s": round(reps * len(sel) / dt, 3),
            "single_core": {"value": round(nbytes1 / dt1 / 1e9, 4), "unit": "GB/s", "cores": 1,
                            "sample": f"decode of {len(sel1)} sequences ({int(c.context_lens[sel1].sum())} context "
                                      f"tokens) x {reps1} passes, float64, {dt1:.2f} s"},
            "numpy": numpy_leg}


def bench_ceilings(pkv, torch, dev, reps=10):
    """Practical ceilings on this GPU, measured with HIP events on one stream around `reps` back-to-back launches:
    * the decode's read pattern (include/pagedkv_measure.h): a buffer read once as 4 KB chunks (the (block, kv
      head) slab at block size 16) and as 64 KB chunks (block size 256) in scrambled order; the best over 1 GiB
      and 8 GiB buffers and 4, 8 and 16 waves per compute unit (the rate moves by a few percent with the buffer's
      size and place; the best is the hardest bar);
    * the matrix cores' rate for v_mfma_f32_16x16x32_bf16 (the prefill's instruction) on register operands,
      best of 4 and 8 waves per compute unit;
    * a bf16 GEMM through torch.matmul (the vendor BLAS), 8192^3."""
    stream = torch.cuda.current_stream()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.zeros(4096 * cus * 8, dtype=torch.uint8, device=dev)

    def timed(launch):
        for _ in range(3):
            launch()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            launch()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    read = {}
    for gib in (1, 8):
        buf = torch.empty(gib << 30, dtype=torch.uint8, device=dev)
        buf.fill_(0x3c)
        for chunk in (4096, 65536):
            key = f"chunks_{chunk // 1024}k"
            for wpc in (4, 8, 16):
                nbytes = pkv.measure_read_chunks(buf, chunk, wpc, sink, stream=stream)
                ms = timed(lambda: pkv.measure_read_chunks(buf, chunk, wpc, sink, stream=stream))
                gbs = nbytes / (ms * 1e-3) / 1e9
                if key not in read or gbs > read[key]["gbs"]:
                    read[key] = {"gbs": round(gbs, 1), "buffer_gib": gib, "waves_per_cu": wpc, "ms": round(ms, 5),
                                 "bytes": nbytes, "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}
        del buf
        torch.cuda.empty_cache()
    mfma = None
    for wpc in (4, 8):
        fl = pkv.measure_mfma_rate(20000, wpc, sink, stream=stream)
        ms = timed(lambda: pkv.measure_mfma_rate(20000, wpc, sink, stream=stream))
        tf = fl / (ms * 1e-3) / 1e12
        if mfma is None or tf > mfma["tflops"]:
            mfma = {"tflops": round(tf, 1), "waves_per_cu": wpc, "frac_of_peak": round(tf * 1e12 / MFMA_BF16_PEAK, 4),
                    "instruction": "v_mfma_f32_16x16x32_bf16, 8 independent chains per wave, register operands"}
    n = 8192
    a = torch.randn((n, n), dtype=torch.bfloat16, device=dev)
    b = torch.randn((n, n), dtype=torch.bfloat16, device=dev)
    c = torch.empty((n, n), dtype=torch.bfloat16, device=dev)
    ms = timed(lambda: torch.matmul(a, b, out=c))
    gemm = {"tflops": round(2 * n ** 3 / (ms * 1e-3) / 1e12, 1), "shape": f"{n}x{n}x{n} bf16 torch.matmul",
            "frac_of_peak": round(2 * n ** 3 / (ms * 1e-3) / MFMA_BF16_PEAK, 4)}
    del a, b, c
    torch.cuda.empty_cache()
    return {"read_pattern": read, "mfma_16x16x32_bf16": mfma, "bf16_gemm": gemm}


def bench_decode_workload(pkv, torch, W, cfg, dev, steps, warmup):
    """The decode call alone on another decode workload (pool copies rotated so K/V come from HBM): HIP
    events around runs of back-to-back calls."""
    c = W.make_config(cfg)

    def tt(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    nbytes = decode_bytes(c)
    copies = max(2, min(8, int(np.ceil(2.0e9 / nbytes))))
    shape = (c.num_blocks,) + c.pool.block_shape
    idx = torch.from_numpy(c.pool.used_blocks.astype(np.int64)).to(dev)
    kb, vb = tt(c.pool.key_blocks), tt(c.pool.value_blocks)
    kn, vn, sm = tt(c.key), tt(c.value), torch.from_numpy(c.slot_mapping).to(dev)
    pools = []
    for _ in range(copies):
        kc = torch.full(shape, float("nan"), dtype=torch.bfloat16, device=dev)
        vc = torch.full(shape, float("nan"), dtype=torch.bfloat16, device=dev)
        kc.index_copy_(0, idx, kb)
        vc.index_copy_(0, idx, vb)
        pkv.kv_cache_store(kn, vn, kc, vc, sm)
        pools.append((kc, vc))
    del kb, vb
    q = tt(c.query)
    out = torch.empty_like(q)
    bt = torch.from_numpy(c.block_tables).to(dev)
    cl = torch.from_numpy(c.context_lens).to(dev)
    ws = torch.empty(pkv.decode_workspace_size(c.num_seqs, c.num_heads, c.num_kv_heads, c.head_dim, c.block_size,
                                               c.max_context_len), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    batch = 10                                # back-to-back calls between an event pair
    for k in range(warmup):
        kc, vc = pools[k % copies]
        pkv.paged_attention_decode(out, q, kc, vc, bt, cl, c.max_context_len, c.scale, workspace=ws, stream=stream)
    runs = []
    for b in range(0, steps, batch):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for k in range(b, min(steps, b + batch)):
            kc, vc = pools[k % copies]
            pkv.paged_attention_decode(out, q, kc, vc, bt, cl, c.max_context_len, c.scale, workspace=ws,
                                       stream=stream)
        e1.record(stream)
        runs.append((e0, e1, min(steps, b + batch) - b))
    torch.cuda.synchronize()
    ms = np.array([a.elapsed_time(z) / n for a, z, n in runs])
    gbs = nbytes / (ms.mean() * 1e-3) / 1e9
    res = {"workload": c.name, "num_seqs": c.num_seqs, "sum_context_tokens": int(c.context_lens.sum()),
           "block_size": c.block_size, "num_heads": c.num_heads, "num_kv_heads": c.num_kv_heads,
           "decode_ms": {"mean": round(float(ms.mean()), 5), "median": round(float(np.median(ms)), 5),
                         "p10": round(float(np.percentile(ms, 10)), 5), "p90": round(float(np.percentile(ms, 90)), 5)},
           "algorithmic_bytes": nbytes, "achieved_gbs": round(gbs, 1),
           "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
           "decode_tokens_per_s": round(c.num_seqs / (ms.mean() * 1e-3), 1), "pool_copies_rotated": copies,
           "outputs_finite": bool(torch.isfinite(out.float()).all().item())}
    del pools
    torch.cuda.empty_cache()
    return res


def prefill_flops(c) -> int:
    """Algorithmic flops of one causal chunked-prefill call: 2 flops per multiply-add of QK^T and of PV over
    the visible (query, key) pairs only; softmax not counted."""
    p = c.prefix_lens.astype(np.int64)
    q = c.chunk_lens.astype(np.int64)
    pairs = int((q * p + q * (q + 1) // 2).sum()) if c.causal else int((q * (p + q)).sum())
    return 4 * c.head_dim * c.num_heads * pairs


def bench_prefill(pkv, torch, dev, iters=20, copies=3):
    """Chunked prefill (32 sequences, prefix U[0, 2048] + chunk U[64, 512], block 256, 32/8 heads, bf16):
    store of the chunk then causal prefill, timed with HIP events on the launch stream. Successive calls read
    different copies of the pool (the K/V a call reads, ~0.3 GB, would otherwise partly stay in the last-level
    cache)."""
    import workloads as W

    c = W.chunked_prefill()

    def tt(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    shape = (c.num_blocks,) + c.pool.block_shape
    idx = torch.from_numpy(c.pool.used_blocks.astype(np.int64)).to(dev)
    kb, vb = tt(c.pool.key_blocks), tt(c.pool.value_blocks)
    pools = []
    for _ in range(copies):
        kc = torch.full(shape, float("nan"), dtype=torch.bfloat16, device=dev)
        vc = torch.full(shape, float("nan"), dtype=torch.bfloat16, device=dev)
        kc.index_copy_(0, idx, kb)
        vc.index_copy_(0, idx, vb)
        pools.append((kc, vc))
    del kb, vb
    q, kn, vn = tt(c.query), tt(c.key), tt(c.value)
    out = torch.empty_like(q)
    bt = torch.from_numpy(c.block_tables).to(dev)
    cq, ck = torch.from_numpy(c.cu_seqlens_q).to(dev), torch.from_numpy(c.cu_seqlens_k).to(dev)
    sm = torch.from_numpy(c.slot_mapping).to(dev)
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
    for k in range(iters + 3):
        e = ev[k - 3] if k >= 3 else None
        kc, vc = pools[k % copies]
        if e:
            e[0].record(stream)
        pkv.kv_cache_store(kn, vn, kc, vc, sm, stream=stream)
        if e:
            e[1].record(stream)
        pkv.paged_attention_prefill(out, q, kc, vc, bt, cq, ck, c.max_seqlen_q, c.max_seqlen_k, c.scale,
                                    causal=True, stream=stream)
        if e:
            e[2].record(stream)
    torch.cuda.synchronize()
    st_ms = float(np.mean([a.elapsed_time(b) for a, b, _ in ev]))
    pf_ms = float(np.mean([b.elapsed_time(d) for _, b, d in ev]))
    fl = prefill_flops(c)
    res = {"workload": c.name, "total_q": c.total_q, "prefill_ms": round(pf_ms, 5), "store_ms": round(st_ms, 5),
           "gflop": round(fl / 1e9, 2), "tflops": round(fl / (pf_ms * 1e-3) / 1e12, 2),
           "mfma_utilization": round(fl / (pf_ms * 1e-3) / MFMA_BF16_PEAK, 4), "peak_tflops": MFMA_BF16_PEAK / 1e12,
           "store_gbs": round(store_bytes(c) / (st_ms * 1e-3) / 1e9, 1), "pool_copies_rotated": copies,
           "outputs_finite": bool(torch.isfinite(out.float()).all().item())}
    del pools
    torch.cuda.empty_cache()
    # the same prefill over 8-bit caches (every cached row and the chunk quantized by the 8-bit store)
    kr, vr, slots = W.cached_rows(c.pool)
    for kind in ("int8", "fp8"):
        code = torch.int8 if kind == "int8" else torch.uint8
        store = pkv.kv_cache_store_int8 if kind == "int8" else pkv.kv_cache_store_fp8
        prefill = pkv.paged_attention_prefill_int8 if kind == "int8" else pkv.paged_attention_prefill_fp8
        qpools = []
        for _ in range(copies):
            kq = torch.zeros(shape, dtype=code, device=dev)
            vq = torch.zeros(shape, dtype=code, device=dev)
            ks = torch.zeros(shape[:3], dtype=torch.float32, device=dev)
            vs = torch.zeros(shape[:3], dtype=torch.float32, device=dev)
            store(tt(kr), tt(vr), kq, vq, ks, vs, torch.from_numpy(slots).to(dev), stream=stream)
            store(kn, vn, kq, vq, ks, vs, sm, stream=stream)
            qpools.append((kq, vq, ks, vs))
        ev8 = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
        for k in range(iters + 3):
            e = ev8[k - 3] if k >= 3 else None
            kq, vq, ks, vs = qpools[k % copies]
            if e:
                e[0].record(stream)
            prefill(out, q, kq, vq, ks, vs, bt, cq, ck, c.max_seqlen_q, c.max_seqlen_k, c.scale, causal=True,
                    stream=stream)
            if e:
                e[1].record(stream)
        torch.cuda.synchronize()
        ms8 = float(np.mean([a.elapsed_time(b) for a, b in ev8]))
        res[f"{kind}_cache"] = {"prefill_ms": round(ms8, 5), "tflops": round(fl / (ms8 * 1e-3) / 1e12, 2),
                                "mfma_utilization": round(fl / (ms8 * 1e-3) / MFMA_BF16_PEAK, 4),
                                "outputs_finite": bool(torch.isfinite(out.float()).all().item())}
        del kq, vq, ks, vs, qpools
        torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=3, choices=[1, 2, 3, 4], help="decode workload")
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--copies", type=int, default=0, help="pool copies rotated per step (0: auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true", help="skip the chunked-prefill leg")
    ap.add_argument("--no-int8", action="store_true", help="skip the quantized-cache (int8, fp8, int4) decode legs")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the read-pattern and MFMA ceiling legs")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="skip the decode legs of the other two decode workloads")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (use --gpus 1).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import paged_kv_cache_88_amd as pkv
    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    pkv.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    c = W.make_config(args.config, args.seed)
    td = torch.float32 if c.dtype == "f32" else torch.bfloat16

    def tt(a):
        a = np.ascontiguousarray(a)
        if c.dtype == "f32":
            return torch.from_numpy(a).to(dev)
        return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)

    step_bytes = decode_bytes(c) + store_bytes(c)
    copies = args.copies or max(2, min(8, int(np.ceil(2.0e9 / max(step_bytes, 1)))))
    shape = (c.num_blocks,) + c.pool.block_shape
    idx = torch.from_numpy(c.pool.used_blocks.astype(np.int64)).to(dev)
    kb, vb = tt(c.pool.key_blocks), tt(c.pool.value_blocks)
    pools = []
    for _ in range(copies):
        kc = torch.full(shape, float("nan"), dtype=td, device=dev)
        vc = torch.full(shape, float("nan"), dtype=td, device=dev)
        kc.index_copy_(0, idx, kb)
        vc.index_copy_(0, idx, vb)
        pools.append((kc, vc))
    del kb, vb
    q, kn, vn = tt(c.query), tt(c.key), tt(c.value)
    out = torch.empty_like(q)
    bt = torch.from_numpy(c.block_tables).to(dev)
    cl = torch.from_numpy(c.context_lens).to(dev)
    sm = torch.from_numpy(c.slot_mapping).to(dev)
    ws_n = pkv.decode_workspace_size(c.num_seqs, c.num_heads, c.num_kv_heads, c.head_dim, c.block_size,
                                     c.max_context_len)
    ws = torch.empty(max(ws_n, 256), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    # A recorded event costs the stream a few microseconds, so durations come from event pairs around runs of
    # back-to-back calls (BATCH calls per pair), never around single calls.
    BATCH = 10

    def step(k):
        kc, vc = pools[k % copies]
        pkv.kv_cache_store(kn, vn, kc, vc, sm, stream=stream)
        pkv.paged_attention_decode(out, q, kc, vc, bt, cl, c.max_context_len, c.scale, workspace=ws, stream=stream)

    def batched_ms(call, calls):
        """Average duration of call(k) over `calls` back-to-back calls: event pairs around runs of BATCH."""
        runs = []
        for b in range(0, calls, BATCH):
            n = min(BATCH, calls - b)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for k in range(b, b + n):
                call(k)
            e1.record(stream)
            runs.append((e0, e1, n))
        torch.cuda.synchronize()
        return np.array([a.elapsed_time(z) / n for a, z, n in runs])

    def one_call_step(k):
        kc, vc = pools[k % copies]
        pkv.paged_decode_step(kn, vn, sm, out, q, kc, vc, bt, cl, c.max_context_len, c.scale, workspace=ws,
                              stream=stream)

    # headline: the step as one call (store + decode, pkv_paged_decode_step), wall clock over the timed steps
    for k in range(args.warmup):
        one_call_step(k)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        one_call_step(k)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    value = step_bytes / (ms_per_step * 1e-3) / 1e9

    # the same step as two calls (kv_cache_store, then paged_attention_decode): wall clock
    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(k)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_two_calls = (t1 - t0) * 1e3 / args.steps

    # the decode call alone, back to back (pool copies rotated), for the roofline: events around runs of
    # BATCH calls; the call is plan + decode + reduce kernels
    def decode_call(k):
        kc, vc = pools[k % copies]
        pkv.paged_attention_decode(out, q, kc, vc, bt, cl, c.max_context_len, c.scale, workspace=ws, stream=stream)

    for k in range(args.warmup):
        decode_call(k)
    dec_ms = batched_ms(decode_call, args.steps)
    dec_avg_ms = float(dec_ms.mean())
    def dist(x):
        return {"mean": round(float(x.mean()), 5), "median": round(float(np.median(x)), 5),
                "p10": round(float(np.percentile(x, 10)), 5), "p90": round(float(np.percentile(x, 90)), 5)}
    achieved = decode_bytes(c) / (dec_avg_ms * 1e-3) / 1e9
    finite = bool(torch.isfinite(out.float()).all().item())
    # store alone, back to back
    def store_call(k):
        kc, vc = pools[k % copies]
        pkv.kv_cache_store(kn, vn, kc, vc, sm, stream=stream)

    store_ms = batched_ms(store_call, args.steps)
    # the same decode in two halves: one plan, then runs from it, as a model's layers would; plans back to
    # back are timed the same way
    def plan(k=0):
        pkv.paged_attention_decode_plan(cl, c.max_context_len, c.num_heads, c.num_kv_heads, c.head_dim,
                                        c.block_size, ws, dtype=td, stream=stream)

    def run_call(k):
        kc, vc = pools[k % copies]
        pkv.paged_attention_decode_run(out, q, kc, vc, bt, c.max_context_len, c.scale, ws, stream=stream)

    plan_ms = batched_ms(plan, 2 * BATCH)
    run_ms = batched_ms(run_call, args.steps)
    plan_run = {"plan_ms": round(float(plan_ms.mean()), 5), "run_ms": dist(run_ms),
                "what": "paged_attention_decode_plan, then paged_attention_decode_run per call from it "
                        f"(runs of {BATCH} back-to-back calls between event pairs)"}


    result = {
        "metric": "paged decode attention achieved HBM GB/s (% of peak) and decode tokens/s",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": c.dtype,
        "data": "synthetic",
        "config": {"workload": c.name, "num_seqs": c.num_seqs, "context_lens": "lognormal median 300 sigma 1 clip [16, 2048]"
                   if args.config == 3 else "see workloads", "sum_context_tokens": int(c.context_lens.sum()),
                   "max_context_len": c.max_context_len, "block_size": c.block_size, "num_heads": c.num_heads,
                   "num_kv_heads": c.num_kv_heads, "head_dim": c.head_dim, "num_blocks": c.num_blocks,
                   "seed": c.seed, "pool_copies_rotated": copies},
        "pct_of_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "decode_tokens_per_s": round(c.num_seqs / (ms_per_step * 1e-3), 1),
        "step_bytes": step_bytes,
        "step": "pkv_paged_decode_step: kv_cache_store of one token per sequence and paged_attention_decode in one "
                "call (the store shares a launch with the decode's plan)",
        "two_calls": {"ms_per_step": round(ms_two_calls, 5),
                      "value": round(step_bytes / (ms_two_calls * 1e-3) / 1e9, 2),
                      "what": "the same step as kv_cache_store then paged_attention_decode (wall clock)"},
        "plan_and_runs": plan_run,
        "timing_ms": {"decode_call": dist(dec_ms), "store": dist(store_ms),
                      "events": f"HIP events on the launch stream around runs of {BATCH} back-to-back calls "
                                f"({args.steps} calls, pool copies rotated); the distribution is over runs"},
        "roofline": {"bound": "hbm",
                     "kernel": "paged_attention_decode call (decode_plan_kernel + decode_mfma_kernel + decode_reduce_kernel)",
                     "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(c.name),
                     "avg_launch_ms": round(dec_avg_ms, 5), "algorithmic_bytes": decode_bytes(c)},
        "outputs_finite": finite,
        "gpu": torch.cuda.get_device_name(0),
        "torch": torch.__version__,
        "hip": torch.version.hip,
    }
    if c.dtype == "bf16" and c.head_dim == 128 and c.block_size >= 16 and not args.no_int8:
        pools = None
        for kind in ("int8", "fp8", "int4"):
            leg = bench_q8(kind, pkv, torch, W, c, dev, copies, args.steps, args.warmup)
            leg["speedup_vs_bf16_cache"] = round(dec_avg_ms / leg["decode_ms"], 3)
            result[f"{kind}_cache"] = leg
    pools = None
    torch.cuda.empty_cache()
    if not args.no_other_workloads:
        result["other_workloads"] = {
            W.CONFIGS[k].__name__: bench_decode_workload(pkv, torch, W, k, dev, max(args.steps, 20), args.warmup)
            for k in (2, 3, 4) if k != args.config}
    if not args.no_prefill:
        result["prefill"] = bench_prefill(pkv, torch, dev)
    if not args.no_ceilings:
        ceil = bench_ceilings(pkv, torch, dev)
        result["ceilings"] = ceil
        chunk = "chunks_4k" if c.block_size * c.head_dim * (2 if c.dtype == "bf16" else 4) <= 8192 else "chunks_64k"
        rc = ceil["read_pattern"][chunk]["gbs"]
        result["roofline"]["ceiling"] = {"measured_gbs": rc, "pattern": f"scrambled {chunk[7:]} chunks",
                                         "frac_of_ceiling": round(achieved / rc, 4)}
        for leg in result.get("other_workloads", {}).values():
            lc = "chunks_4k" if leg["block_size"] <= 16 else "chunks_64k"
            leg["frac_of_read_ceiling"] = round(leg["achieved_gbs"] / ceil["read_pattern"][lc]["gbs"], 4)
        if "prefill" in result:
            pf = result["prefill"]
            pf["frac_of_mfma_rate"] = round(pf["tflops"] / ceil["mfma_16x16x32_bf16"]["tflops"], 4)
            pf["frac_of_bf16_gemm"] = round(pf["tflops"] / ceil["bf16_gemm"]["tflops"], 4)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(c)
        result["cpu_baseline"]["host"] = platform.processor() or platform.machine()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
