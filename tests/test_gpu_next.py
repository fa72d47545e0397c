"""Beyond the core step: block copies (copy-on-write), prefix sharing through the host block manager,
mixed decode + chunked-prefill batches in one varlen call, and the decode step under HIP graph capture."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import assert_close, device_pool, i32, oracle_prefill_case, run_prefill_case, to_storage, to_torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pkv():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import paged_kv_cache_88_amd as m

    m.load_library()
    return m


@pytest.mark.parametrize("dtype,bs", [(W.BF16, 16), (W.F32, 256), (W.BF16, 1)])
def test_copy_blocks_bit_exact(pkv, orc, dtype, bs):
    rng = np.random.default_rng(3)
    nb, hkv, d = 40, 4, 128
    kc0 = W._draw_values(rng, (nb, hkv, bs, d), dtype)
    vc0 = W._draw_values(rng, (nb, hkv, bs, d), dtype)
    perm = rng.permutation(nb)
    pairs = np.stack([perm[:10], perm[10:20]], axis=1).astype(np.int32)
    kh, vh = kc0.copy(), vc0.copy()
    orc.copy_blocks(dtype, kh, vh, pairs)
    kc, vc = to_torch(kc0, dtype), to_torch(vc0, dtype)
    pkv.kv_cache_copy_blocks(kc, vc, i32(pairs))
    torch.cuda.synchronize()
    assert np.array_equal(to_storage(kc, dtype).view(np.uint8), kh.view(np.uint8))
    assert np.array_equal(to_storage(vc, dtype).view(np.uint8), vh.view(np.uint8))


def test_fork_copy_on_write_decode(pkv, orc):
    """Parent and forked child share blocks; both append one token; the child's write into the shared
    partial block goes to a copy made by kv_cache_copy_blocks. Both decodes match the oracle, and the
    parent's output is unaffected by the child."""
    dtype, bs, hq, hkv, d, nb = W.BF16, 16, 8, 2, 128, 64
    rng = np.random.default_rng(11)
    bm = pkv.BlockManager(nb, bs)
    L0 = 37                                           # last block partially filled
    bm.allocate(1, L0)
    bm.fork(1, 2)
    kc0 = W._draw_values(rng, (nb, hkv, bs, d), dtype)
    vc0 = W._draw_values(rng, (nb, hkv, bs, d), dtype)
    bm.append(1, 1)
    bm.append(2, 1)
    pairs = bm.take_copies()
    assert len(pairs) == 1
    slots = np.concatenate([bm.slot_mapping(1, L0, 1), bm.slot_mapping(2, L0, 1)])
    tables, lens = bm.build_tables([1, 2])
    knew = W._draw_values(rng, (2, hkv, d), dtype)
    vnew = W._draw_values(rng, (2, hkv, d), dtype)
    q = W._draw_values(rng, (2, hq, d), dtype)
    scale = 1 / np.sqrt(d)
    # oracle
    kh, vh = kc0.copy(), vc0.copy()
    orc.copy_blocks(dtype, kh, vh, pairs)
    orc.store(dtype, knew, vnew, kh, vh, slots)
    ref = orc.decode(dtype, q, kh, vh, tables, lens, scale)
    # GPU
    kc, vc = to_torch(kc0, dtype), to_torch(vc0, dtype)
    pkv.kv_cache_copy_blocks(kc, vc, i32(pairs))
    pkv.kv_cache_store(to_torch(knew, dtype), to_torch(vnew, dtype), kc, vc, i32(slots))
    out = torch.empty((2, hq, d), dtype=torch.bfloat16, device="cuda")
    pkv.paged_attention_decode(out, to_torch(q, dtype), kc, vc, i32(tables), i32(lens), int(lens.max()), scale)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    assert_close(got, ref, dtype, "fork + copy-on-write decode")
    # the first writer (the parent, which appended first) got the copy; the child kept the original block
    assert tables[0, -1 + int(lens[0] + 15) // 16] == pairs[0, 1] and tables[1, int(lens[1] - 1) // 16] == pairs[0, 0]
    # isolation: the child's token never reaches the parent's blocks (parent's decode without the child's store)
    kh2, vh2 = kc0.copy(), vc0.copy()
    orc.copy_blocks(dtype, kh2, vh2, pairs)
    orc.store(dtype, knew[:1], vnew[:1], kh2, vh2, slots[:1])
    alone = orc.decode(dtype, q[:1], kh2, vh2, tables[:1], lens[:1], scale)
    assert np.array_equal(alone, ref[:1])


def test_prefix_cache_shared_blocks_decode(pkv, orc):
    """Two requests whose prompts share two full blocks map them to the same physical blocks (prefix
    cache); decoding both over the shared pool matches decoding each over a private copy."""
    dtype, bs, hq, hkv, d, nb = W.BF16, 16, 8, 2, 128, 32
    rng = np.random.default_rng(12)
    common = rng.integers(0, 1000, 32).astype(np.int32)
    p1 = np.concatenate([common, rng.integers(0, 1000, 9).astype(np.int32)])
    p2 = np.concatenate([common, rng.integers(0, 1000, 20).astype(np.int32)])
    bm = pkv.BlockManager(nb, bs, prefix_caching=True)
    assert bm.allocate(1, len(p1), p1) == 0
    assert bm.allocate(2, len(p2), p2) == 32
    tables, lens = bm.build_tables([1, 2])
    assert (tables[0, :2] == tables[1, :2]).all()
    kc0 = W._draw_values(rng, (nb, hkv, bs, d), dtype)
    vc0 = W._draw_values(rng, (nb, hkv, bs, d), dtype)
    q = W._draw_values(rng, (2, hq, d), dtype)
    scale = 1 / np.sqrt(d)
    kc, vc = to_torch(kc0, dtype), to_torch(vc0, dtype)
    out = torch.empty((2, hq, d), dtype=torch.bfloat16, device="cuda")
    pkv.paged_attention_decode(out, to_torch(q, dtype), kc, vc, i32(tables), i32(lens), int(lens.max()), scale)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    # private copy for request 2: its shared blocks moved to unused ids
    used = set(tables[tables >= 0].tolist())
    spare = [b for b in range(nb) if b not in used][:2]
    kh, vh = kc0.copy(), vc0.copy()
    orc.copy_blocks(dtype, kh, vh, np.array([[tables[1, 0], spare[0]], [tables[1, 1], spare[1]]], np.int32))
    t2 = tables.copy()
    t2[1, :2] = spare
    ref = orc.decode(dtype, q, kh, vh, t2, lens, scale)
    assert_close(got, ref, dtype, "prefix-shared decode")


def test_mixed_decode_and_prefill_batch(pkv, orc):
    """One varlen call: decode rows (chunk of 1), a speculative-verify row group (chunk of 4) and prefill
    chunks, each over its own cached history ("推理运行时", section Prefill 与 decode 输入)."""
    prefix = [300, 17, 0, 1000, 40, 5]
    chunk = [1, 1, 200, 4, 1, 77]
    lk = [p + c for p, c in zip(prefix, chunk)]
    nb = sum(W.blocks_for_tokens(n, 16) for n in lk) + 3
    c = W.make_prefill_case("mixed", 31, W.BF16, prefix, chunk, 32, 8, 128, 16, nb)
    got = run_prefill_case(pkv, c)
    assert_close(got, oracle_prefill_case(orc, c), W.BF16, "mixed batch")


def test_decode_step_in_hip_graph(pkv, orc):
    """Store + decode captured once in a HIP graph and replayed with new inputs copied into the captured
    buffers (the plan kernel rebuilds the work list on device, no memset); every replay matches eager."""
    c = W.make_decode_case("graph", 5, W.BF16, [700, 33, 1300, 512, 9, 2047], 32, 8, 128, 16, 400)
    kc, vc = device_pool(c.pool)
    q = to_torch(c.query, c.dtype)
    kn, vn = to_torch(c.key, c.dtype), to_torch(c.value, c.dtype)
    bt, cl, sm = i32(c.block_tables), i32(c.context_lens), i32(c.slot_mapping)
    out = torch.empty_like(q)
    ws = torch.empty(pkv.decode_workspace_size(c.num_seqs, 32, 8, 128, 16, 2048), dtype=torch.uint8, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                       # warm up on the capture stream
        pkv.kv_cache_store(kn, vn, kc, vc, sm)
        pkv.paged_attention_decode(out, q, kc, vc, bt, cl, 2048, c.scale, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pkv.kv_cache_store(kn, vn, kc, vc, sm)
        pkv.paged_attention_decode(out, q, kc, vc, bt, cl, 2048, c.scale, workspace=ws)
    rng = np.random.default_rng(0)
    for rep in range(4):
        qn = W._draw_values(rng, q.shape, c.dtype)
        q.copy_(to_torch(qn, c.dtype))
        lens = np.minimum(c.context_lens, rng.integers(1, 2048, c.num_seqs)).astype(np.int32)
        lens[rep % c.num_seqs] = c.context_lens[rep % c.num_seqs]
        cl.copy_(i32(lens))
        g.replay()
        torch.cuda.synchronize()
        got = out.float().cpu().numpy().astype(np.float64)
        eager = torch.empty_like(out)
        pkv.paged_attention_decode(eager, q, kc, vc, bt, cl, 2048, c.scale, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep} differs from eager"
        kh, vh = c.pool.dense()
        orc.store(c.dtype, c.key, c.value, kh, vh, c.slot_mapping)
        ref = orc.decode(c.dtype, qn, kh, vh, c.block_tables, lens, c.scale)
        assert_close(got, ref, c.dtype, f"replay {rep}")


def _replays_match_eager(step, refresh, outs, reps=4, check=None):
    """Capture `step` once, then for each replay: refresh the captured inputs, replay, and compare every
    output with an eager run of `step` on the same inputs (bit for bit); `check(rep, outputs)` then compares
    the replayed outputs with the oracle."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                       # warm up on the capture stream
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(reps):
        refresh(rep)
        g.replay()
        torch.cuda.synchronize()
        replayed = [o.clone() for o in outs]
        step()
        torch.cuda.synchronize()
        for a, b in zip(replayed, outs):
            assert torch.isfinite(a.float()).all(), f"replay {rep}: non-finite output"
            assert torch.equal(a, b), f"replay {rep} differs from eager"
        if check is not None:
            check(rep, replayed)


def _f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def _quant_kind(kind):
    """Host and device helpers of one cache kind: (element dtype, row bytes factor, GPU store, oracle store,
    oracle dequantize)."""
    return {"int8": (torch.int8, 1, "kv_cache_store_int8", "store_int8", "dequantize_int8"),
            "fp8": (torch.uint8, 1, "kv_cache_store_fp8", "store_fp8", "dequantize_fp8"),
            "int4": (torch.uint8, 2, "kv_cache_store_int4", "store_int4", "dequantize_int4")}[kind]


class _QuantPool:
    """A quantized cache on the device and its host mirror, filled from a case's cached rows by the GPU store
    and the oracle's store; `extra` blocks past the case's pool are zero codes with zero scales."""

    def __init__(self, pkv, orc, kind, c, extra=0):
        ct, div, gstore, ostore, deq = _quant_kind(kind)
        self.kind, self.orc, self.dtype = kind, orc, c.dtype
        self.gstore, self.ostore, self.deq = getattr(pkv, gstore), getattr(orc, ostore), getattr(orc, deq)
        shape = (c.num_blocks + extra, c.num_kv_heads, c.block_size, c.head_dim // div)
        self.dev = [torch.zeros(shape, dtype=ct, device="cuda"), torch.zeros(shape, dtype=ct, device="cuda"),
                    torch.zeros(shape[:3], dtype=torch.float32, device="cuda"),
                    torch.zeros(shape[:3], dtype=torch.float32, device="cuda")]
        hct = np.int8 if ct == torch.int8 else np.uint8
        self.host = [np.zeros(shape, hct), np.zeros(shape, hct), np.zeros(shape[:3], np.float32),
                     np.zeros(shape[:3], np.float32)]
        kr, vr, slots = W.cached_rows(c.pool)
        self.store(kr, vr, slots)

    def store(self, k, v, slots, device=True):
        if device:
            self.gstore(to_torch(k, self.dtype), to_torch(v, self.dtype), *self.dev, i32(slots))
        self.ostore(self.dtype, k, v, *self.host, slots)

    def dequantized(self):
        return self.deq(self.host[0], self.host[2]), self.deq(self.host[1], self.host[3])

    def host_equals_device(self, blocks):
        return all(np.array_equal(d.cpu().numpy()[blocks].view(np.uint8), h[blocks].view(np.uint8))
                   for d, h in zip(self.dev, self.host))


@pytest.mark.parametrize("kind", ["fp8", "int4"])
def test_quantized_decode_step_in_hip_graph(pkv, orc, kind):
    """fp8 (or int4) store + decode captured once and replayed with new queries and context lengths: the plan
    kernel and the decode kernel's unit counter reset on the device, so every replay equals eager, and every
    replay matches the oracle over the dequantized cache."""
    c = W.make_decode_case("graph_fp8", 6, W.BF16, [700, 33, 1300, 512, 9, 2047], 32, 8, 128, 16, 400)
    pool = _QuantPool(pkv, orc, kind, c)
    store = getattr(pkv, f"kv_cache_store_{kind}")
    decode = getattr(pkv, f"paged_attention_decode_{kind}")
    kc, vc, ks, vs = pool.dev
    pool.store(c.key, c.value, c.slot_mapping, device=False)    # the captured step stores these every time
    q = to_torch(c.query, c.dtype)
    kn, vn = to_torch(c.key, c.dtype), to_torch(c.value, c.dtype)
    bt, cl, sm = i32(c.block_tables), i32(c.context_lens), i32(c.slot_mapping)
    out = torch.empty_like(q)
    ws = torch.empty(pkv.decode_workspace_size(c.num_seqs, 32, 8, 128, 16, 2048), dtype=torch.uint8, device="cuda")

    def step():
        store(kn, vn, kc, vc, ks, vs, sm)
        decode(out, q, kc, vc, ks, vs, bt, cl, 2048, c.scale, workspace=ws)

    rng = np.random.default_rng(1)
    state = {}

    def refresh(rep):
        state["q"] = W._draw_values(rng, q.shape, c.dtype)
        q.copy_(to_torch(state["q"], c.dtype))
        lens = np.minimum(c.context_lens, rng.integers(1, 2048, c.num_seqs)).astype(np.int32)
        lens[rep % c.num_seqs] = c.context_lens[rep % c.num_seqs]
        state["lens"] = lens
        cl.copy_(i32(lens))

    def check(rep, outs):
        fk, fv = pool.dequantized()
        qf = W.to_f32(state["q"], c.dtype).astype(np.float64)
        ref = orc.decode("f64", qf, fk, fv, c.block_tables, state["lens"], c.scale)
        assert_close(_f64(outs[0]), ref, W.BF16, f"{kind} replay {rep}")

    _replays_match_eager(step, refresh, [out], check=check)


@pytest.mark.parametrize("kind", ["bf16", "int8"])
def test_prefill_step_in_hip_graph(pkv, orc, kind):
    """Chunk store + chunked prefill captured once and replayed with new queries and chunk K/V: every replay
    equals eager and matches the oracle (bf16 cache, and an int8 cache)."""
    c = W.make_prefill_case("graph_pf", 7, W.BF16, [0, 300, 1000], [70, 129, 33], 32, 8, 128, 64, 64)
    q = to_torch(c.query, c.dtype)
    kn, vn = to_torch(c.key, c.dtype), to_torch(c.value, c.dtype)
    bt, cq, ck, sm = i32(c.block_tables), i32(c.cu_seqlens_q), i32(c.cu_seqlens_k), i32(c.slot_mapping)
    out = torch.empty_like(q)
    state = {}
    if kind == "bf16":
        kc, vc = device_pool(c.pool)
        hk, hv = c.pool.dense()

        def step():
            pkv.kv_cache_store(kn, vn, kc, vc, sm)
            pkv.paged_attention_prefill(out, q, kc, vc, bt, cq, ck, c.max_seqlen_q, c.max_seqlen_k, c.scale)

        def reference():
            orc.store(c.dtype, state["k"], state["v"], hk, hv, c.slot_mapping)
            return orc.prefill(c.dtype, state["q"], hk, hv, c.block_tables, c.cu_seqlens_q, c.cu_seqlens_k, c.scale)
    else:
        pool = _QuantPool(pkv, orc, "int8", c)
        kc, vc, ks, vs = pool.dev

        def step():
            pkv.kv_cache_store_int8(kn, vn, kc, vc, ks, vs, sm)
            pkv.paged_attention_prefill_int8(out, q, kc, vc, ks, vs, bt, cq, ck, c.max_seqlen_q, c.max_seqlen_k,
                                             c.scale)

        def reference():
            pool.store(state["k"], state["v"], c.slot_mapping, device=False)
            fk, fv = pool.dequantized()
            qf = W.to_f32(state["q"], c.dtype).astype(np.float64)
            return orc.prefill("f64", qf, fk, fv, c.block_tables, c.cu_seqlens_q, c.cu_seqlens_k, c.scale)

    rng = np.random.default_rng(2)

    def refresh(rep):
        for name, t in (("q", q), ("k", kn), ("v", vn)):
            state[name] = W._draw_values(rng, t.shape, c.dtype)
            t.copy_(to_torch(state[name], c.dtype))

    def check(rep, outs):
        assert_close(_f64(outs[0]), reference(), W.BF16, f"{kind} prefill replay {rep}")

    _replays_match_eager(step, refresh, [out], check=check)


@pytest.mark.parametrize("kind", ["bf16", "fp8"])
def test_graph_replay_with_dummy_block_padding(pkv, orc, kind):
    """Decode under a captured graph with dummy-request padding (Mini-SGLang 源码解析（二）, sections 7.5 and 7.6:
    a graph is captured per batch size and a smaller live batch is padded with dummy requests whose page-table
    rows point at one reserved extra page, so padding never touches a live page). Store + decode is captured
    at batch 8 over a pool of NB + 1 blocks, block NB being the dummy. Replays run 5, 7, 8 and 3 live
    sequences (new queries, new tokens, new lengths within their tables); each padding row has the dummy block
    as its whole table, context length 1 and its own slot in the dummy block. After each replay: live outputs
    match the oracle, padding outputs are finite, every live block equals the host mirror (which saw the live
    stores only) bit for bit, and the dummy block changed only in the padding rows' slots."""
    B, bs, hq, hkv, d = 8, 16, 32, 8, 128
    lens_full = [700, 33, 1300, 512, 9, 2047, 100, 64]
    nb = sum(W.blocks_for_tokens(n, bs) for n in lens_full) + 4
    c = W.make_decode_case("graph_pad", 12, W.BF16, lens_full, hq, hkv, d, bs, nb)
    dummy = nb
    if kind == "bf16":
        kc0, vc0 = device_pool(c.pool)
        pad = torch.zeros((1,) + tuple(kc0.shape[1:]), dtype=kc0.dtype, device="cuda")
        kc, vc = torch.cat([kc0, pad]), torch.cat([vc0, pad])
        del kc0, vc0
        hk, hv = c.pool.dense()
        hk = np.concatenate([hk, np.zeros((1,) + hk.shape[1:], hk.dtype)])
        hv = np.concatenate([hv, np.zeros((1,) + hv.shape[1:], hv.dtype)])
        devs, hosts = [kc, vc], [hk, hv]

        def host_store(k, v, slots):
            orc.store(c.dtype, k, v, hk, hv, slots)

        def host_decode(qh, bt, lens):
            return orc.decode(c.dtype, qh, hk, hv, bt, lens, c.scale)

        def step():
            pkv.kv_cache_store(kn, vn, kc, vc, sm)
            pkv.paged_attention_decode(out, q, kc, vc, bt_d, cl, 2048, c.scale, workspace=ws)
    else:
        pool = _QuantPool(pkv, orc, kind, c, extra=1)
        devs, hosts = pool.dev, pool.host
        kc, vc, ks, vs = pool.dev

        def host_store(k, v, slots):
            pool.store(k, v, slots, device=False)

        def host_decode(qh, bt, lens):
            fk, fv = pool.dequantized()
            return orc.decode("f64", W.to_f32(qh, c.dtype).astype(np.float64), fk, fv, bt, lens, c.scale)

        def step():
            pkv.kv_cache_store_fp8(kn, vn, kc, vc, ks, vs, sm)
            pkv.paged_attention_decode_fp8(out, q, kc, vc, ks, vs, bt_d, cl, 2048, c.scale, workspace=ws)

    q = to_torch(c.query, c.dtype)
    kn, vn = to_torch(c.key, c.dtype), to_torch(c.value, c.dtype)
    bt_d, cl, sm = i32(c.block_tables), i32(c.context_lens), i32(c.slot_mapping)
    out = torch.empty_like(q)
    ws = torch.empty(pkv.decode_workspace_size(B, hq, hkv, d, bs, 2048), dtype=torch.uint8, device="cuda")
    host_store(c.key, c.value, c.slot_mapping)          # the warm-up and capture run the step as set up
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    rng = np.random.default_rng(13)
    for rep, n_live in enumerate([5, 7, 8, 3]):
        before = [t[dummy].clone() for t in devs]
        qn = W._draw_values(rng, q.shape, c.dtype)
        kk = W._draw_values(rng, kn.shape, c.dtype)
        vv = W._draw_values(rng, vn.shape, c.dtype)
        lens = np.ones(B, np.int32)
        bt = np.full_like(c.block_tables, -1)
        slots = np.empty(B, np.int32)
        for i in range(B):
            if i < n_live:
                lens[i] = rng.integers(1, lens_full[i] + 1)
                bt[i] = c.block_tables[i]
                t = int(lens[i]) - 1
                slots[i] = int(bt[i, t // bs]) * bs + t % bs
            else:
                bt[i, 0] = dummy
                slots[i] = dummy * bs + (i - n_live)
        for dst, src in ((q, qn), (kn, kk), (vn, vv)):
            dst.copy_(to_torch(src, c.dtype))
        bt_d.copy_(i32(bt))
        cl.copy_(i32(lens))
        sm.copy_(i32(slots))
        g.replay()
        torch.cuda.synchronize()
        got = _f64(out)
        host_store(kk[:n_live], vv[:n_live], slots[:n_live])
        ref = host_decode(qn[:n_live], bt[:n_live], lens[:n_live])
        assert_close(got[:n_live], ref, W.BF16, f"{kind} replay {rep}: live rows")
        assert np.isfinite(got[n_live:]).all(), f"{kind} replay {rep}: padding output not finite"
        for dev, host in zip(devs, hosts):
            assert np.array_equal(dev[:nb].cpu().view(torch.uint8).numpy(), host[:nb].view(np.uint8)), \
                f"{kind} replay {rep}: a live block differs from its mirror"
        for dev, old in zip(devs, before):
            changed = (dev[dummy] != old).reshape(hkv, bs, -1).any(dim=(0, 2)) if dev.dim() == 4 else \
                (dev[dummy] != old).any(dim=0)
            rows = torch.nonzero(changed).flatten().tolist()
            assert all(r < B - n_live for r in rows), f"{kind} replay {rep}: dummy block changed at rows {rows}"
