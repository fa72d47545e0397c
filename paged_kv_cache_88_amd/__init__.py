"""MI355X paged KV cache: Python binding of libpagedkv.so (see include/pagedkv.h).

This module only marshals arguments: it reads shapes from torch tensors, checks that they agree,
passes raw device pointers and the current HIP stream to the C ABI and turns a non-OK status into an
exception. Every step of the computation runs in the library's HIP kernels. There is no fallback:
if the library is missing or no GPU is present, calls raise.

Names match the C entry points without the ``pkv_`` prefix.
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpagedkv.so")

PKV_F32, PKV_BF16 = 0, 1
STATUS = {0: "PKV_OK", 1: "PKV_EINVAL", 2: "PKV_EUNSUPPORTED", 3: "PKV_EWORKSPACE", 4: "PKV_EHIP", 5: "PKV_ENOMEM"}

_lib = None


class PagedKVError(ValueError):
    """A non-OK status from the library; ``status`` holds its name."""

    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = STATUS.get(status, status)


def load_library(path: str = LIB_PATH):
    """Load libpagedkv.so (torch's HIP runtime must be loaded first: it is, by ``import torch``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    P, I32, I64, F, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    sig = {
        "pkv_kv_cache_store": [ctypes.c_int, P, P, P, P, P, I64, I32, I32, I32, I64, P],
        "pkv_kv_cache_gather": [ctypes.c_int, P, P, P, P, P, I32, I32, I32, I32, I64, P],
        "pkv_paged_attention_decode": [ctypes.c_int, P, P, P, P, P, I32, P, I32, I32, I32, I32, I32, I32, I64, F, P,
                                       SZ, P],
        "pkv_paged_decode_step": [ctypes.c_int, P, P, P, P, P, P, P, P, I32, P, I32, I32, I32, I32, I32, I32, I64, F,
                                  P, SZ, P],
        "pkv_paged_attention_decode_noalloc": [ctypes.c_int, P, P, P, P, P, I32, P, I32, I32, I32, I32, I32, I32,
                                               I64, F, P],
        "pkv_paged_attention_prefill": [ctypes.c_int, P, P, P, P, P, I32, P, P, I32, I32, I32, I32, I32, I32, I32,
                                        I64, F, I32, P],
        "pkv_kv_cache_store_int8": [ctypes.c_int, P, P, P, P, P, P, P, I64, I32, I32, I32, I64, P],
        "pkv_paged_attention_decode_int8": [ctypes.c_int, P, P, P, P, P, P, P, I32, P, I32, I32, I32, I32, I32, I32,
                                            I64, F, P, SZ, P],
        "pkv_kv_cache_store_fp8": [ctypes.c_int, P, P, P, P, P, P, P, I64, I32, I32, I32, I64, P],
        "pkv_paged_attention_decode_fp8": [ctypes.c_int, P, P, P, P, P, P, P, I32, P, I32, I32, I32, I32, I32, I32,
                                           I64, F, P, SZ, P],
        "pkv_paged_attention_decode_plan": [ctypes.c_int, I32, P, I32, I32, I32, I32, I32, I32, P, SZ, P],
        "pkv_paged_attention_decode_run": [ctypes.c_int, P, P, P, P, P, I32, I32, I32, I32, I32, I32, I32, I64, F, P,
                                           SZ, P],
        "pkv_paged_attention_decode_int8_run": [ctypes.c_int, P, P, P, P, P, P, P, I32, I32, I32, I32, I32, I32, I32,
                                                I64, F, P, SZ, P],
        "pkv_paged_attention_decode_fp8_run": [ctypes.c_int, P, P, P, P, P, P, P, I32, I32, I32, I32, I32, I32, I32,
                                               I64, F, P, SZ, P],
        "pkv_kv_cache_store_int4": [ctypes.c_int, P, P, P, P, P, P, P, I64, I32, I32, I32, I64, P],
        "pkv_paged_attention_decode_int4": [ctypes.c_int, P, P, P, P, P, P, P, I32, P, I32, I32, I32, I32, I32, I32,
                                            I64, F, P, SZ, P],
        "pkv_paged_attention_decode_int4_run": [ctypes.c_int, P, P, P, P, P, P, P, I32, I32, I32, I32, I32, I32, I32,
                                                I64, F, P, SZ, P],
        "pkv_paged_attention_prefill_int8": [ctypes.c_int, P, P, P, P, P, P, P, I32, P, P, I32, I32, I32, I32, I32,
                                             I32, I32, I64, F, I32, P],
        "pkv_paged_attention_prefill_fp8": [ctypes.c_int, P, P, P, P, P, P, P, I32, P, P, I32, I32, I32, I32, I32,
                                            I32, I32, I64, F, I32, P],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.pkv_kv_cache_copy_blocks.argtypes = [ctypes.c_int, P, P, P, I32, I32, I32, I32, I64, P]
    lib.pkv_kv_cache_copy_blocks.restype = ctypes.c_int
    H = ctypes.c_void_p
    lib.pkv_bm_create.argtypes = [I32, I32, I32, ctypes.POINTER(H)]
    lib.pkv_bm_destroy.argtypes = [H]
    lib.pkv_bm_destroy.restype = None
    lib.pkv_bm_allocate.argtypes = [H, I64, I32, P, ctypes.POINTER(I32)]
    lib.pkv_bm_append.argtypes = [H, I64, I32, P]
    lib.pkv_bm_fork.argtypes = [H, I64, I64]
    lib.pkv_bm_release.argtypes = [H, I64]
    lib.pkv_bm_block_table.argtypes = [H, I64, P, I32, ctypes.POINTER(I32), ctypes.POINTER(I64)]
    lib.pkv_bm_slot_mapping.argtypes = [H, I64, I64, I32, P]
    lib.pkv_bm_take_copies.argtypes = [H, P, I32, ctypes.POINTER(I32)]
    lib.pkv_bm_usage.argtypes = [H, ctypes.POINTER(BlockUsage)]
    for name in ("pkv_bm_create", "pkv_bm_allocate", "pkv_bm_append", "pkv_bm_fork", "pkv_bm_release",
                 "pkv_bm_block_table", "pkv_bm_slot_mapping", "pkv_bm_take_copies", "pkv_bm_usage"):
        getattr(lib, name).restype = ctypes.c_int
    lib.pkv_bm_last_error.restype = ctypes.c_char_p
    lib.pkv_measure_read_chunks.argtypes = [P, SZ, I32, I32, P, SZ, P]
    lib.pkv_measure_read_chunks.restype = ctypes.c_int
    lib.pkv_measure_read_chunks_bytes.argtypes = [SZ, I32]
    lib.pkv_measure_read_chunks_bytes.restype = I64
    lib.pkv_measure_mfma_rate.argtypes = [I32, I32, P, SZ, ctypes.POINTER(ctypes.c_double), P]
    lib.pkv_measure_mfma_rate.restype = ctypes.c_int
    lib.pkv_paged_attention_decode_status.argtypes = [P, P, P]
    lib.pkv_paged_attention_decode_status.restype = ctypes.c_int
    lib.pkv_paged_attention_decode_workspace_size.argtypes = [I32, I32, I32, I32, I32, I32]
    lib.pkv_paged_attention_decode_workspace_size.restype = SZ
    lib.pkv_last_error.restype = ctypes.c_char_p
    lib.pkv_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


class BlockUsage(ctypes.Structure):
    _fields_ = [("num_requests", ctypes.c_int64), ("allocated_tokens", ctypes.c_int64),
                ("reserved_tokens", ctypes.c_int64), ("internal_fragmentation_tokens", ctypes.c_int64),
                ("block_utilization", ctypes.c_double), ("used_blocks", ctypes.c_int64),
                ("free_blocks", ctypes.c_int64), ("max_request_tokens", ctypes.c_int64),
                ("contiguous_reserved_tokens", ctypes.c_int64), ("contiguous_fragmentation_tokens", ctypes.c_int64),
                ("contiguous_utilization", ctypes.c_double)]


def _check(rc: int):
    if rc != 0:
        raise PagedKVError(rc, load_library().pkv_last_error().decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return PKV_F32
    if t.dtype == torch.bfloat16:
        return PKV_BF16
    raise ValueError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _dev(*ts):
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("all tensors must be on the GPU")
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")


def _i32(*ts):
    for t in ts:
        if t.dtype != torch.int32:
            raise ValueError("index tensors must be int32")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def version() -> str:
    return load_library().pkv_version().decode()


def kv_cache_store(key, value, key_cache, value_cache, slot_mapping, stream=None):
    """Scatter ``key``/``value`` [N, Hkv, D] into ``key_cache``/``value_cache`` [NB, Hkv, bs, D] at the
    slots ``slot_mapping`` (int32 [N]; negative = skip)."""
    lib = load_library()
    _dev(key, value, key_cache, value_cache, slot_mapping)
    _i32(slot_mapping)
    nb, hkv, bs, d = key_cache.shape
    n = key.shape[0]
    if key.shape != (n, hkv, d) or value.shape != key.shape or value_cache.shape != key_cache.shape:
        raise ValueError("key/value must be [N, Hkv, D] and both caches [NB, Hkv, bs, D]")
    if slot_mapping.shape != (n,):
        raise ValueError("slot_mapping must have one entry per token")
    if not (key.dtype == value.dtype == key_cache.dtype == value_cache.dtype):
        raise ValueError("key, value and caches must share a dtype")
    _check(lib.pkv_kv_cache_store(_dtype_code(key), _ptr(key), _ptr(value), _ptr(key_cache), _ptr(value_cache),
                                  _ptr(slot_mapping), n, hkv, d, bs, nb, _stream(stream)))


def kv_cache_gather(key_out, value_out, key_cache, value_cache, block_table_row, length, stream=None):
    """Logical tokens [0, length) of one block table into ``key_out``/``value_out`` [length, Hkv, D]."""
    lib = load_library()
    _dev(key_out, value_out, key_cache, value_cache, block_table_row)
    _i32(block_table_row)
    nb, hkv, bs, d = key_cache.shape
    if key_out.shape != (length, hkv, d) or value_out.shape != key_out.shape:
        raise ValueError("outputs must be [length, Hkv, D]")
    if block_table_row.numel() * bs < length:
        raise ValueError("block_table_row too short for length")
    _check(lib.pkv_kv_cache_gather(_dtype_code(key_cache), _ptr(key_out), _ptr(value_out), _ptr(key_cache),
                                   _ptr(value_cache), _ptr(block_table_row), int(length), hkv, d, bs, nb,
                                   _stream(stream)))


def decode_workspace_size(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_context_len) -> int:
    return int(load_library().pkv_paged_attention_decode_workspace_size(num_seqs, num_heads, num_kv_heads, head_dim,
                                                                        block_size, max_context_len))


def paged_attention_decode(out, query, key_cache, value_cache, block_tables, context_lens, max_context_len, scale,
                           workspace=None, stream=None):
    """Decode attention: ``out``/``query`` [B, Hq, D]; ``block_tables`` int32 [B, stride];
    ``context_lens`` int32 [B]. ``workspace`` (uint8, device) is allocated here when None and needed."""
    lib = load_library()
    _dev(out, query, key_cache, value_cache, block_tables, context_lens, workspace)
    _i32(block_tables, context_lens)
    nb, hkv, bs, d = key_cache.shape
    b, hq, d2 = query.shape
    if d2 != d or out.shape != query.shape or value_cache.shape != key_cache.shape:
        raise ValueError("query/out must be [B, Hq, D] with the caches' D")
    if block_tables.dim() != 2 or block_tables.shape[0] != b or context_lens.shape != (b,):
        raise ValueError("block_tables must be [B, stride] and context_lens [B]")
    ws_need = decode_workspace_size(b, hq, hkv, d, bs, max_context_len)
    if workspace is None and ws_need > 0:
        workspace = torch.empty(ws_need, dtype=torch.uint8, device=query.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.pkv_paged_attention_decode(_dtype_code(query), _ptr(out), _ptr(query), _ptr(key_cache),
                                          _ptr(value_cache), _ptr(block_tables), block_tables.shape[1],
                                          _ptr(context_lens), b, int(max_context_len), hq, hkv, d, bs, nb, float(scale),
                                          _ptr(workspace), ws_bytes, _stream(stream)))


_CACHE_KINDS = {"elements": 0, "int8": 1, "fp8": 2, "int4": 3}


def paged_decode_step(key, value, slot_mapping, out, query, key_cache, value_cache, block_tables, context_lens,
                      max_context_len, scale, workspace=None, stream=None):
    """One decode step in one call: ``kv_cache_store(key, value, ..., slot_mapping)`` of each sequence's new token
    ``[B, Hkv, D]``, then ``paged_attention_decode`` (same results; the store shares a launch with the plan)."""
    lib = load_library()
    _dev(key, value, slot_mapping, out, query, key_cache, value_cache, block_tables, context_lens, workspace)
    _i32(slot_mapping, block_tables, context_lens)
    nb, hkv, bs, d = key_cache.shape
    b, hq, d2 = query.shape
    if d2 != d or out.shape != query.shape or value_cache.shape != key_cache.shape:
        raise ValueError("query/out must be [B, Hq, D] with the caches' D")
    if key.shape != (b, hkv, d) or value.shape != key.shape or slot_mapping.shape != (b,):
        raise ValueError("key/value must be [B, Hkv, D] and slot_mapping [B]")
    if key.dtype != query.dtype or key_cache.dtype != query.dtype:
        raise ValueError("key, value, caches and query must share one dtype")
    if block_tables.dim() != 2 or block_tables.shape[0] != b or context_lens.shape != (b,):
        raise ValueError("block_tables must be [B, stride] and context_lens [B]")
    ws_need = decode_workspace_size(b, hq, hkv, d, bs, max_context_len)
    if workspace is None and ws_need > 0:
        workspace = torch.empty(ws_need, dtype=torch.uint8, device=query.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.pkv_paged_decode_step(_dtype_code(query), _ptr(key), _ptr(value), _ptr(slot_mapping), _ptr(out),
                                     _ptr(query), _ptr(key_cache), _ptr(value_cache), _ptr(block_tables),
                                     block_tables.shape[1], _ptr(context_lens), b, int(max_context_len), hq, hkv, d, bs,
                                     nb, float(scale), _ptr(workspace), ws_bytes, _stream(stream)))
    return out


def paged_attention_decode_noalloc(out, query, key_cache, value_cache, block_tables, context_lens, max_context_len,
                                   scale, stream=None):
    """``paged_attention_decode`` without a workspace: the library's per-GPU scratch array stands in for it
    (nothing is allocated). Sizes past the scratch raise ``PagedKVError`` (PKV_EWORKSPACE); calls that may
    overlap on one GPU race on the shared array."""
    lib = load_library()
    _dev(out, query, key_cache, value_cache, block_tables, context_lens)
    _i32(block_tables, context_lens)
    b, hq, d = query.shape
    nb, hkv, bs, d2 = key_cache.shape
    if out.shape != query.shape or out.dtype != query.dtype or d2 != d or value_cache.shape != key_cache.shape:
        raise ValueError("shape mismatch between out, query and the caches")
    if block_tables.dim() != 2 or block_tables.shape[0] != b or context_lens.shape != (b,):
        raise ValueError("block_tables must be [B, stride] and context_lens [B]")
    _check(lib.pkv_paged_attention_decode_noalloc(_dtype_code(query), _ptr(out), _ptr(query), _ptr(key_cache),
                                                  _ptr(value_cache), _ptr(block_tables), block_tables.shape[1],
                                                  _ptr(context_lens), b, int(max_context_len), hq, hkv, d, bs, nb,
                                                  float(scale), _stream(stream)))
    return out


def paged_attention_decode_plan(context_lens, max_context_len, num_heads, num_kv_heads, head_dim, block_size,
                                workspace, dtype=torch.bfloat16, cache="elements", stream=None):
    """Build a decode work list from ``context_lens`` (int32 [B]) into ``workspace`` (uint8, device, at least
    ``decode_workspace_size(...)`` bytes), for later ``paged_attention_decode_run`` (``cache="elements"``, the
    query's ``dtype``) or ``paged_attention_decode_int8_run`` / ``_fp8_run`` (``cache="int8"`` / ``"fp8"``)."""
    lib = load_library()
    _dev(context_lens, workspace)
    _i32(context_lens)
    if cache not in _CACHE_KINDS:
        raise ValueError(f"cache must be one of {sorted(_CACHE_KINDS)}")
    code = {torch.float32: PKV_F32, torch.bfloat16: PKV_BF16}.get(dtype)
    if code is None:
        raise ValueError(f"unsupported dtype {dtype} (float32 or bfloat16)")
    b = context_lens.shape[0]
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib.pkv_paged_attention_decode_plan(code, _CACHE_KINDS[cache], _ptr(context_lens), b,
                                               int(max_context_len), int(num_heads), int(num_kv_heads),
                                               int(head_dim), int(block_size), _ptr(workspace), ws_bytes,
                                               _stream(stream)))


def paged_attention_decode_run(out, query, key_cache, value_cache, block_tables, max_context_len, scale, workspace,
                               stream=None):
    """``paged_attention_decode`` from a work list made by ``paged_attention_decode_plan`` (same batch,
    sizes and context lengths); ``context_lens`` is not read again."""
    lib = load_library()
    _dev(out, query, key_cache, value_cache, block_tables, workspace)
    _i32(block_tables)
    nb, hkv, bs, d = key_cache.shape
    b, hq, d2 = query.shape
    if d2 != d or out.shape != query.shape or value_cache.shape != key_cache.shape:
        raise ValueError("query/out must be [B, Hq, D] with the caches' D")
    if block_tables.dim() != 2 or block_tables.shape[0] != b:
        raise ValueError("block_tables must be [B, stride]")
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib.pkv_paged_attention_decode_run(_dtype_code(query), _ptr(out), _ptr(query), _ptr(key_cache),
                                              _ptr(value_cache), _ptr(block_tables), block_tables.shape[1], b,
                                              int(max_context_len), hq, hkv, d, bs, nb, float(scale), _ptr(workspace),
                                              ws_bytes, _stream(stream)))


_CODE_DTYPES = {"int8": (torch.int8,), "fp8": (torch.uint8, torch.float8_e4m3fn), "int4": (torch.uint8,)}


def paged_attention_decode_status(workspace, status=None, stream=None):
    """Enqueue a copy of ``workspace``'s run status into ``status`` (int32 [1] on the device; allocated when
    None) and return it: 0 when every run since the last plan matched that plan's sizes, 1 when a run found a
    plan for other sizes (and wrote nothing)."""
    _dev(workspace)
    if status is None:
        status = torch.empty(1, dtype=torch.int32, device=workspace.device)
    _dev(status)
    _check(load_library().pkv_paged_attention_decode_status(_ptr(workspace), _ptr(status), _stream(stream)))
    return status


def measure_read_chunks(buffer, chunk_bytes, waves_per_cu, sink, stream=None) -> int:
    """Enqueue one read of ``buffer`` (uint8, device) as scrambled chunks of ``chunk_bytes`` (the decode's
    access pattern, include/pagedkv_measure.h); returns the bytes it reads."""
    lib = load_library()
    _dev(buffer, sink)
    n = buffer.numel() * buffer.element_size()
    _check(lib.pkv_measure_read_chunks(_ptr(buffer), n, int(chunk_bytes), int(waves_per_cu), _ptr(sink),
                                       sink.numel() * sink.element_size(), _stream(stream)))
    return int(lib.pkv_measure_read_chunks_bytes(n, int(chunk_bytes)))


def measure_mfma_rate(iters, waves_per_cu, sink, stream=None) -> float:
    """Enqueue independent v_mfma_f32_16x16x32_bf16 chains on every wave (include/pagedkv_measure.h);
    returns the flops of the launch."""
    lib = load_library()
    _dev(sink)
    fl = ctypes.c_double(0.0)
    _check(lib.pkv_measure_mfma_rate(int(iters), int(waves_per_cu), _ptr(sink), sink.numel() * sink.element_size(),
                                     ctypes.byref(fl), _stream(stream)))
    return float(fl.value)


def _cache_dims(kind, key_cache):
    """(NB, Hkv, bs, head_dim) of a quantized cache: int4 rows hold two codes per byte."""
    nb, hkv, bs, last = key_cache.shape
    return nb, hkv, bs, 2 * last if kind == "int4" else last


def _store_q8(kind, key, value, key_cache, value_cache, key_scale, value_scale, slot_mapping, stream):
    lib = load_library()
    _dev(key, value, key_cache, value_cache, key_scale, value_scale, slot_mapping)
    _i32(slot_mapping)
    nb, hkv, bs, d = _cache_dims(kind, key_cache)
    n = key.shape[0]
    if key.shape != (n, hkv, d) or value.shape != key.shape or value_cache.shape != key_cache.shape:
        raise ValueError("key/value must be [N, Hkv, D] and both caches [NB, Hkv, bs, D] (D / 2 bytes for int4)")
    if key_scale.shape != (nb, hkv, bs) or value_scale.shape != (nb, hkv, bs):
        raise ValueError("scales must be [NB, Hkv, bs]")
    if key_cache.dtype not in _CODE_DTYPES[kind] or value_cache.dtype not in _CODE_DTYPES[kind]:
        raise ValueError(f"{kind} caches expected ({', '.join(str(t) for t in _CODE_DTYPES[kind])})")
    if key_scale.dtype != torch.float32 or value_scale.dtype != torch.float32:
        raise ValueError("float32 scales expected")
    if slot_mapping.shape != (n,) or key.dtype != value.dtype:
        raise ValueError("slot_mapping must have one entry per token; key and value share a dtype")
    fn = {"int8": lib.pkv_kv_cache_store_int8, "fp8": lib.pkv_kv_cache_store_fp8,
          "int4": lib.pkv_kv_cache_store_int4}[kind]
    _check(fn(_dtype_code(key), _ptr(key), _ptr(value), _ptr(key_cache), _ptr(value_cache), _ptr(key_scale),
              _ptr(value_scale), _ptr(slot_mapping), n, hkv, d, bs, nb, _stream(stream)))


def _decode_q8(kind, out, query, key_cache, value_cache, key_scale, value_scale, block_tables, context_lens,
               max_context_len, scale, workspace, stream):
    lib = load_library()
    _dev(out, query, key_cache, value_cache, key_scale, value_scale, block_tables, context_lens, workspace)
    _i32(block_tables, context_lens)
    nb, hkv, bs, d = _cache_dims(kind, key_cache)
    b, hq, d2 = query.shape
    if d2 != d or out.shape != query.shape or value_cache.shape != key_cache.shape:
        raise ValueError("query/out must be [B, Hq, D] with the caches' D")
    if key_scale.shape != (nb, hkv, bs) or value_scale.shape != (nb, hkv, bs):
        raise ValueError("scales must be [NB, Hkv, bs]")
    if key_cache.dtype not in _CODE_DTYPES[kind] or value_cache.dtype not in _CODE_DTYPES[kind] \
            or key_scale.dtype != torch.float32 or value_scale.dtype != torch.float32:
        raise ValueError(f"{kind} caches and float32 scales expected")
    if block_tables.dim() != 2 or block_tables.shape[0] != b or context_lens.shape != (b,):
        raise ValueError("block_tables must be [B, stride] and context_lens [B]")
    ws_need = decode_workspace_size(b, hq, hkv, d, bs, max_context_len)
    if workspace is None and ws_need > 0:
        workspace = torch.empty(ws_need, dtype=torch.uint8, device=query.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    fn = {"int8": lib.pkv_paged_attention_decode_int8, "fp8": lib.pkv_paged_attention_decode_fp8,
          "int4": lib.pkv_paged_attention_decode_int4}[kind]
    _check(fn(_dtype_code(query), _ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache), _ptr(key_scale),
              _ptr(value_scale), _ptr(block_tables), block_tables.shape[1], _ptr(context_lens), b,
              int(max_context_len), hq, hkv, d, bs, nb, float(scale), _ptr(workspace), ws_bytes, _stream(stream)))


def _decode_q8_run(kind, out, query, key_cache, value_cache, key_scale, value_scale, block_tables,
                   max_context_len, scale, workspace, stream):
    lib = load_library()
    _dev(out, query, key_cache, value_cache, key_scale, value_scale, block_tables, workspace)
    _i32(block_tables)
    nb, hkv, bs, d = _cache_dims(kind, key_cache)
    b, hq, d2 = query.shape
    if d2 != d or out.shape != query.shape or value_cache.shape != key_cache.shape:
        raise ValueError("query/out must be [B, Hq, D] with the caches' D")
    if key_scale.shape != (nb, hkv, bs) or value_scale.shape != (nb, hkv, bs):
        raise ValueError("scales must be [NB, Hkv, bs]")
    if key_cache.dtype not in _CODE_DTYPES[kind] or value_cache.dtype not in _CODE_DTYPES[kind] \
            or key_scale.dtype != torch.float32 or value_scale.dtype != torch.float32:
        raise ValueError(f"{kind} caches and float32 scales expected")
    if block_tables.dim() != 2 or block_tables.shape[0] != b:
        raise ValueError("block_tables must be [B, stride]")
    ws_bytes = workspace.numel() * workspace.element_size()
    fn = {"int8": lib.pkv_paged_attention_decode_int8_run, "fp8": lib.pkv_paged_attention_decode_fp8_run,
          "int4": lib.pkv_paged_attention_decode_int4_run}[kind]
    _check(fn(_dtype_code(query), _ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache), _ptr(key_scale),
              _ptr(value_scale), _ptr(block_tables), block_tables.shape[1], b, int(max_context_len), hq, hkv, d, bs,
              nb, float(scale), _ptr(workspace), ws_bytes, _stream(stream)))


def paged_attention_decode_int8_run(out, query, key_cache, value_cache, key_scale, value_scale, block_tables,
                                    max_context_len, scale, workspace, stream=None):
    """``paged_attention_decode_int8`` from a work list made by ``paged_attention_decode_plan(cache="int8")``."""
    _decode_q8_run("int8", out, query, key_cache, value_cache, key_scale, value_scale, block_tables,
                   max_context_len, scale, workspace, stream)


def paged_attention_decode_fp8_run(out, query, key_cache, value_cache, key_scale, value_scale, block_tables,
                                   max_context_len, scale, workspace, stream=None):
    """``paged_attention_decode_fp8`` from a work list made by ``paged_attention_decode_plan(cache="fp8")``."""
    _decode_q8_run("fp8", out, query, key_cache, value_cache, key_scale, value_scale, block_tables,
                   max_context_len, scale, workspace, stream)


def kv_cache_store_int8(key, value, key_cache, value_cache, key_scale, value_scale, slot_mapping, stream=None):
    """Quantize ``key``/``value`` [N, Hkv, D] (bf16 or fp32) row by row and scatter the int8 codes into
    ``key_cache``/``value_cache`` int8 [NB, Hkv, bs, D] and the fp32 row scales into ``key_scale``/
    ``value_scale`` [NB, Hkv, bs] at the slots ``slot_mapping`` (int32 [N]; negative = skip)."""
    _store_q8("int8", key, value, key_cache, value_cache, key_scale, value_scale, slot_mapping, stream)


def paged_attention_decode_int8(out, query, key_cache, value_cache, key_scale, value_scale, block_tables,
                                context_lens, max_context_len, scale, workspace=None, stream=None):
    """Decode attention over an int8 cache (codes [NB, Hkv, bs, D], fp32 scales [NB, Hkv, bs]); bf16
    ``out``/``query`` [B, Hq, D], D = 128, block size >= 16. Workspace as for ``paged_attention_decode``."""
    _decode_q8("int8", out, query, key_cache, value_cache, key_scale, value_scale, block_tables, context_lens,
               max_context_len, scale, workspace, stream)


def kv_cache_store_fp8(key, value, key_cache, value_cache, key_scale, value_scale, slot_mapping, stream=None):
    """``kv_cache_store_int8`` with OCP float8 E4M3 codes (scale max|x| / 448, round half to even); the caches
    hold the code bytes as uint8 (or torch.float8_e4m3fn) [NB, Hkv, bs, D]."""
    _store_q8("fp8", key, value, key_cache, value_cache, key_scale, value_scale, slot_mapping, stream)


def paged_attention_decode_fp8(out, query, key_cache, value_cache, key_scale, value_scale, block_tables,
                               context_lens, max_context_len, scale, workspace=None, stream=None):
    """Decode attention over an fp8 (E4M3) cache; otherwise as ``paged_attention_decode_int8``."""
    _decode_q8("fp8", out, query, key_cache, value_cache, key_scale, value_scale, block_tables, context_lens,
               max_context_len, scale, workspace, stream)


def kv_cache_store_int4(key, value, key_cache, value_cache, key_scale, value_scale, slot_mapping, stream=None):
    """``kv_cache_store_int8`` with 4-bit codes: scale max|x| / 7, q = round-half-even(x / scale) in [-7, 7],
    stored as q + 8, two per byte (element 2j in the low four bits of byte j); the caches are uint8
    [NB, Hkv, bs, D / 2]."""
    _store_q8("int4", key, value, key_cache, value_cache, key_scale, value_scale, slot_mapping, stream)


def paged_attention_decode_int4(out, query, key_cache, value_cache, key_scale, value_scale, block_tables,
                                context_lens, max_context_len, scale, workspace=None, stream=None):
    """Decode attention over an int4 cache (uint8 [NB, Hkv, bs, D / 2], fp32 scales [NB, Hkv, bs]); otherwise as
    ``paged_attention_decode_int8``."""
    _decode_q8("int4", out, query, key_cache, value_cache, key_scale, value_scale, block_tables, context_lens,
               max_context_len, scale, workspace, stream)


def paged_attention_decode_int4_run(out, query, key_cache, value_cache, key_scale, value_scale, block_tables,
                                    max_context_len, scale, workspace, stream=None):
    """``paged_attention_decode_int4`` from a work list made by ``paged_attention_decode_plan(cache="int4")``."""
    _decode_q8_run("int4", out, query, key_cache, value_cache, key_scale, value_scale, block_tables,
                   max_context_len, scale, workspace, stream)


def paged_attention_prefill(out, query, key_cache, value_cache, block_tables, cu_seqlens_q, cu_seqlens_k,
                            max_seqlen_q, max_seqlen_k, scale, causal=True, stream=None):
    """Varlen chunked prefill: ``out``/``query`` [total_q, Hq, D]; ``cu_seqlens_q/k`` int32 [B+1]."""
    lib = load_library()
    _dev(out, query, key_cache, value_cache, block_tables, cu_seqlens_q, cu_seqlens_k)
    _i32(block_tables, cu_seqlens_q, cu_seqlens_k)
    nb, hkv, bs, d = key_cache.shape
    tq, hq, d2 = query.shape
    b = cu_seqlens_q.shape[0] - 1
    if d2 != d or out.shape != query.shape or value_cache.shape != key_cache.shape:
        raise ValueError("query/out must be [total_q, Hq, D] with the caches' D")
    if cu_seqlens_k.shape != cu_seqlens_q.shape or b < 0 or block_tables.dim() != 2 or block_tables.shape[0] != b:
        raise ValueError("cu_seqlens_q/k must be [B+1] and block_tables [B, stride]")
    _check(lib.pkv_paged_attention_prefill(_dtype_code(query), _ptr(out), _ptr(query), _ptr(key_cache),
                                           _ptr(value_cache), _ptr(block_tables), block_tables.shape[1],
                                           _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), b, int(max_seqlen_q),
                                           int(max_seqlen_k), hq, hkv, d, bs, nb, float(scale), int(bool(causal)),
                                           _stream(stream)))


def _prefill_q8(kind, out, query, key_cache, value_cache, key_scale, value_scale, block_tables, cu_seqlens_q,
                cu_seqlens_k, max_seqlen_q, max_seqlen_k, scale, causal, stream):
    lib = load_library()
    _dev(out, query, key_cache, value_cache, key_scale, value_scale, block_tables, cu_seqlens_q, cu_seqlens_k)
    _i32(block_tables, cu_seqlens_q, cu_seqlens_k)
    nb, hkv, bs, d = key_cache.shape
    tq, hq, d2 = query.shape
    b = cu_seqlens_q.shape[0] - 1
    if d2 != d or out.shape != query.shape or value_cache.shape != key_cache.shape:
        raise ValueError("query/out must be [total_q, Hq, D] with the caches' D")
    if key_scale.shape != (nb, hkv, bs) or value_scale.shape != (nb, hkv, bs):
        raise ValueError("scales must be [NB, Hkv, bs]")
    if key_cache.dtype not in _CODE_DTYPES[kind] or value_cache.dtype not in _CODE_DTYPES[kind] \
            or key_scale.dtype != torch.float32 or value_scale.dtype != torch.float32:
        raise ValueError(f"{kind} caches and float32 scales expected")
    if cu_seqlens_k.shape != cu_seqlens_q.shape or b < 0 or block_tables.dim() != 2 or block_tables.shape[0] != b:
        raise ValueError("cu_seqlens_q/k must be [B+1] and block_tables [B, stride]")
    fn = lib.pkv_paged_attention_prefill_int8 if kind == "int8" else lib.pkv_paged_attention_prefill_fp8
    _check(fn(_dtype_code(query), _ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache), _ptr(key_scale),
              _ptr(value_scale), _ptr(block_tables), block_tables.shape[1], _ptr(cu_seqlens_q), _ptr(cu_seqlens_k),
              b, int(max_seqlen_q), int(max_seqlen_k), hq, hkv, d, bs, nb, float(scale), int(bool(causal)),
              _stream(stream)))


def paged_attention_prefill_int8(out, query, key_cache, value_cache, key_scale, value_scale, block_tables,
                                 cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, scale, causal=True,
                                 stream=None):
    """``paged_attention_prefill`` over an int8 cache (codes [NB, Hkv, bs, D], fp32 scales [NB, Hkv, bs]);
    bf16 ``out``/``query`` [total_q, Hq, D], D = 128. The chunk must be stored with ``kv_cache_store_int8``."""
    _prefill_q8("int8", out, query, key_cache, value_cache, key_scale, value_scale, block_tables, cu_seqlens_q,
                cu_seqlens_k, max_seqlen_q, max_seqlen_k, scale, causal, stream)


def paged_attention_prefill_fp8(out, query, key_cache, value_cache, key_scale, value_scale, block_tables,
                                cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, scale, causal=True,
                                stream=None):
    """``paged_attention_prefill_int8`` over an fp8 (E4M3) cache (code bytes as uint8 or torch.float8_e4m3fn)."""
    _prefill_q8("fp8", out, query, key_cache, value_cache, key_scale, value_scale, block_tables, cu_seqlens_q,
                cu_seqlens_k, max_seqlen_q, max_seqlen_k, scale, causal, stream)


def kv_cache_copy_blocks(key_cache, value_cache, pairs, stream=None):
    """Copy whole physical blocks of both caches: ``pairs`` is a device int32 tensor [n, 2] of (src, dst)."""
    lib = load_library()
    _dev(key_cache, value_cache, pairs)
    _i32(pairs)
    nb, hkv, bs, d = key_cache.shape
    if value_cache.shape != key_cache.shape or key_cache.dtype != value_cache.dtype:
        raise ValueError("both caches must be [NB, Hkv, bs, D] of one dtype")
    if pairs.dim() != 2 or pairs.shape[1] != 2:
        raise ValueError("pairs must be [n, 2]")
    _check(lib.pkv_kv_cache_copy_blocks(_dtype_code(key_cache), _ptr(key_cache), _ptr(value_cache), _ptr(pairs),
                                        pairs.shape[0], hkv, d, bs, nb, _stream(stream)))


class BlockManager:
    """Host KV block manager (the C++ one in libpagedkv.so): per-request block tables over a pool of
    ``total_blocks`` blocks of ``block_size`` tokens, with optional prefix caching and copy-on-write."""

    def __init__(self, total_blocks: int, block_size: int = 16, prefix_caching: bool = False):
        self._lib = load_library()
        h = ctypes.c_void_p()
        self._bm_check(self._lib.pkv_bm_create(total_blocks, block_size, int(prefix_caching), ctypes.byref(h)))
        self._h = h
        self.total_blocks, self.block_size, self.prefix_caching = total_blocks, block_size, prefix_caching

    def _bm_check(self, rc):
        if rc != 0:
            raise PagedKVError(rc, self._lib.pkv_bm_last_error().decode())

    def close(self):
        if getattr(self, "_h", None):
            self._lib.pkv_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    @staticmethod
    def _tok(token_ids):
        import numpy as np

        return None if token_ids is None else np.ascontiguousarray(token_ids, dtype=np.int32)

    def allocate(self, request_id: int, num_tokens: int, token_ids=None) -> int:
        """Blocks for a new request; returns the number of prompt tokens served from cached blocks."""
        tok = self._tok(token_ids)
        cached = ctypes.c_int32(0)
        self._bm_check(self._lib.pkv_bm_allocate(self._h, request_id, num_tokens,
                                                 None if tok is None else tok.ctypes.data_as(ctypes.c_void_p),
                                                 ctypes.byref(cached)))
        return cached.value

    def append(self, request_id: int, num_tokens: int = 1, token_ids=None):
        tok = self._tok(token_ids)
        self._bm_check(self._lib.pkv_bm_append(self._h, request_id, num_tokens,
                                               None if tok is None else tok.ctypes.data_as(ctypes.c_void_p)))

    def fork(self, parent_id: int, child_id: int):
        self._bm_check(self._lib.pkv_bm_fork(self._h, parent_id, child_id))

    def release(self, request_id: int):
        self._bm_check(self._lib.pkv_bm_release(self._h, request_id))

    def block_table(self, request_id: int):
        import numpy as np

        nb, nt = ctypes.c_int32(0), ctypes.c_int64(0)
        self._bm_check(self._lib.pkv_bm_block_table(self._h, request_id, None, 0, ctypes.byref(nb), ctypes.byref(nt)))
        out = np.empty(nb.value, dtype=np.int32)
        self._bm_check(self._lib.pkv_bm_block_table(self._h, request_id, out.ctypes.data_as(ctypes.c_void_p),
                                                    nb.value, ctypes.byref(nb), ctypes.byref(nt)))
        return out

    def num_tokens(self, request_id: int) -> int:
        nb, nt = ctypes.c_int32(0), ctypes.c_int64(0)
        self._bm_check(self._lib.pkv_bm_block_table(self._h, request_id, None, 0, ctypes.byref(nb), ctypes.byref(nt)))
        return nt.value

    def slot_mapping(self, request_id: int, first_position: int, count: int):
        import numpy as np

        out = np.empty(count, dtype=np.int32)
        self._bm_check(self._lib.pkv_bm_slot_mapping(self._h, request_id, first_position, count,
                                                     out.ctypes.data_as(ctypes.c_void_p)))
        return out

    def take_copies(self):
        """Pending copy-on-write pairs as an int32 array [n, 2] of (src, dst); empties the queue."""
        import numpy as np

        n = ctypes.c_int32(0)
        self._bm_check(self._lib.pkv_bm_take_copies(self._h, None, 0, ctypes.byref(n)))
        out = np.empty((n.value, 2), dtype=np.int32)
        if n.value:
            self._bm_check(self._lib.pkv_bm_take_copies(self._h, out.ctypes.data_as(ctypes.c_void_p), n.value,
                                                        ctypes.byref(n)))
        return out

    def usage(self) -> dict:
        u = BlockUsage()
        self._bm_check(self._lib.pkv_bm_usage(self._h, ctypes.byref(u)))
        return {name: getattr(u, name) for name, _ in BlockUsage._fields_}

    def build_tables(self, request_ids, stride: int | None = None):
        """Block tables [n, stride] (padded with -1; stride defaults to the longest table rounded up to a
        multiple of 32 entries) and the requests' token counts, as int32 numpy arrays."""
        import numpy as np

        tables = [self.block_table(r) for r in request_ids]
        lens = np.array([self.num_tokens(r) for r in request_ids], dtype=np.int32)
        longest = max((len(t) for t in tables), default=0)
        stride = stride or max(32, (longest + 31) // 32 * 32)
        out = np.full((len(tables), stride), -1, dtype=np.int32)
        for i, t in enumerate(tables):
            out[i, :len(t)] = t
        return out, lens
