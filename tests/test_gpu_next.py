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


def _replays_match_eager(step, refresh, outs, reps=4):
    """Capture `step` once, then for each replay: refresh the captured inputs, replay, and compare every
    output with an eager run of `step` on the same inputs (bit for bit)."""
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


@pytest.mark.parametrize("kind", ["fp8", "int4"])
def test_quantized_decode_step_in_hip_graph(pkv, kind):
    """fp8 (or int4) store + decode captured once and replayed with new queries and context lengths: the plan
    kernel and the decode kernel's unit counter reset on the device, so every replay equals eager."""
    c = W.make_decode_case("graph_fp8", 6, W.BF16, [700, 33, 1300, 512, 9, 2047], 32, 8, 128, 16, 400)
    kr, vr, slots = W.cached_rows(c.pool)
    store = getattr(pkv, f"kv_cache_store_{kind}")
    decode = getattr(pkv, f"paged_attention_decode_{kind}")
    shape = (c.num_blocks, c.num_kv_heads, c.block_size, c.head_dim // 2 if kind == "int4" else c.head_dim)
    kc = torch.zeros(shape, dtype=torch.uint8, device="cuda")
    vc = torch.zeros_like(kc)
    ks = torch.zeros(shape[:3], dtype=torch.float32, device="cuda")
    vs = torch.zeros_like(ks)
    store(to_torch(kr, c.dtype), to_torch(vr, c.dtype), kc, vc, ks, vs, i32(slots))
    q = to_torch(c.query, c.dtype)
    kn, vn = to_torch(c.key, c.dtype), to_torch(c.value, c.dtype)
    bt, cl, sm = i32(c.block_tables), i32(c.context_lens), i32(c.slot_mapping)
    out = torch.empty_like(q)
    ws = torch.empty(pkv.decode_workspace_size(c.num_seqs, 32, 8, 128, 16, 2048), dtype=torch.uint8, device="cuda")

    def step():
        store(kn, vn, kc, vc, ks, vs, sm)
        decode(out, q, kc, vc, ks, vs, bt, cl, 2048, c.scale, workspace=ws)

    rng = np.random.default_rng(1)

    def refresh(rep):
        q.copy_(to_torch(W._draw_values(rng, q.shape, c.dtype), c.dtype))
        lens = np.minimum(c.context_lens, rng.integers(1, 2048, c.num_seqs)).astype(np.int32)
        lens[rep % c.num_seqs] = c.context_lens[rep % c.num_seqs]
        cl.copy_(i32(lens))

    _replays_match_eager(step, refresh, [out])


@pytest.mark.parametrize("kind", ["bf16", "int8"])
def test_prefill_step_in_hip_graph(pkv, kind):
    """Chunk store + chunked prefill captured once and replayed with new queries and chunk K/V: every replay
    equals eager (bf16 cache, and an int8 cache)."""
    c = W.make_prefill_case("graph_pf", 7, W.BF16, [0, 300, 1000], [70, 129, 33], 32, 8, 128, 64, 64)
    q = to_torch(c.query, c.dtype)
    kn, vn = to_torch(c.key, c.dtype), to_torch(c.value, c.dtype)
    bt, cq, ck, sm = i32(c.block_tables), i32(c.cu_seqlens_q), i32(c.cu_seqlens_k), i32(c.slot_mapping)
    out = torch.empty_like(q)
    if kind == "bf16":
        kc, vc = device_pool(c.pool)

        def step():
            pkv.kv_cache_store(kn, vn, kc, vc, sm)
            pkv.paged_attention_prefill(out, q, kc, vc, bt, cq, ck, c.max_seqlen_q, c.max_seqlen_k, c.scale)
    else:
        kr, vr, slots = W.cached_rows(c.pool)
        shape = (c.num_blocks, c.num_kv_heads, c.block_size, c.head_dim)
        kc = torch.zeros(shape, dtype=torch.int8, device="cuda")
        vc = torch.zeros_like(kc)
        ks = torch.zeros(shape[:3], dtype=torch.float32, device="cuda")
        vs = torch.zeros_like(ks)
        pkv.kv_cache_store_int8(to_torch(kr, c.dtype), to_torch(vr, c.dtype), kc, vc, ks, vs, i32(slots))

        def step():
            pkv.kv_cache_store_int8(kn, vn, kc, vc, ks, vs, sm)
            pkv.paged_attention_prefill_int8(out, q, kc, vc, ks, vs, bt, cq, ck, c.max_seqlen_q, c.max_seqlen_k,
                                             c.scale)

    rng = np.random.default_rng(2)

    def refresh(rep):
        q.copy_(to_torch(W._draw_values(rng, q.shape, c.dtype), c.dtype))
        kn.copy_(to_torch(W._draw_values(rng, kn.shape, c.dtype), c.dtype))
        vn.copy_(to_torch(W._draw_values(rng, vn.shape, c.dtype), c.dtype))

    _replays_match_eager(step, refresh, [out])
