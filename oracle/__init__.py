"""CPU oracle for the paged KV cache -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may import this
package. It shares no code with ``paged_kv_cache_88_amd`` and does not import it. The arithmetic lives
in ``oracle.c`` (float64, plain definitions); this file only builds and marshals.

Every function is pinned by ``tests/test_oracle_*.py`` against closed forms, invariants, brute force
on tiny inputs and ``torch.nn.functional.scaled_dot_product_attention`` in float64 (see each test's
docstring for the passage it follows).

Arrays use the storage conventions of ``workloads``: float32 arrays for fp32, uint16 bf16 bit
patterns for bf16; "f64" (float64 arrays) serves dequantized int8 caches.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

_DT = {"f32": 0, "bf16": 1, "f64": 3}


def build(force: bool = True, src: str = SRC, out: str = LIB) -> str:
    """Compile the oracle with gcc (-O2 -fopenmp, no fast-math: float64 in plain order)."""
    if force or not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(src):
        tmp = out + ".tmp"
        subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall", "-Wextra",
                        "-o", tmp, src, "-lm"], check=True)
        os.replace(tmp, out)
    return out


class OracleError(ValueError):
    pass


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype=None):
    return np.ascontiguousarray(a, dtype=dtype) if a is not None else None


def _store_dtype(dtype):
    return {"f32": np.float32, "bf16": np.uint16, "f64": np.float64}[dtype]


class Oracle:
    """The oracle's entry points bound to one compiled copy of ``oracle.c``."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        P, I32, I64, D = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        lib.orc_store.argtypes = [ctypes.c_int, P, P, P, P, P, I64, I32, I32, I32, I64]
        lib.orc_gather.argtypes = [ctypes.c_int, P, P, P, P, P, I32, I32, I32, I32, I64]
        lib.orc_copy_blocks.argtypes = [ctypes.c_int, P, P, P, I32, I32, I32, I32, I64]
        lib.orc_copy_blocks.restype = ctypes.c_int
        lib.orc_decode.argtypes = [ctypes.c_int, P, P, P, P, P, I32, P, I32, I32, I32, I32, I32, I64, D,
                                   P, I32, I32]
        lib.orc_prefill.argtypes = [ctypes.c_int, P, P, P, P, P, I32, P, P, I32, I32, I32, I32, I32, I64, D,
                                    I32, P, I32, I32]
        lib.orc_quantize_int8.argtypes = [ctypes.c_int, P, I64, I32, P, P]
        lib.orc_store_int8.argtypes = [ctypes.c_int, P, P, P, P, P, P, P, I64, I32, I32, I32, I64]
        lib.orc_dequantize_int8.argtypes = [P, P, I64, I32, P]
        lib.orc_e4m3_value.argtypes = [ctypes.c_int]
        lib.orc_e4m3_value.restype = ctypes.c_double
        lib.orc_e4m3_encode.argtypes = [ctypes.c_float]
        lib.orc_e4m3_encode.restype = ctypes.c_int
        lib.orc_quantize_fp8.argtypes = [ctypes.c_int, P, I64, I32, P, P]
        lib.orc_store_fp8.argtypes = [ctypes.c_int, P, P, P, P, P, P, P, I64, I32, I32, I32, I64]
        lib.orc_dequantize_fp8.argtypes = [P, P, I64, I32, P]
        lib.orc_quantize_int4.argtypes = [ctypes.c_int, P, I64, I32, P, P]
        lib.orc_store_int4.argtypes = [ctypes.c_int, P, P, P, P, P, P, P, I64, I32, I32, I32, I64]
        lib.orc_dequantize_int4.argtypes = [P, P, I64, I32, P]
        for f in (lib.orc_store, lib.orc_gather, lib.orc_decode, lib.orc_prefill, lib.orc_quantize_int8,
                  lib.orc_store_int8, lib.orc_dequantize_int8, lib.orc_quantize_fp8, lib.orc_store_fp8,
                  lib.orc_dequantize_fp8, lib.orc_quantize_int4, lib.orc_store_int4, lib.orc_dequantize_int4):
            f.restype = ctypes.c_int
        lib.orc_last_error.restype = ctypes.c_char_p
        lib.orc_max_threads.restype = ctypes.c_int
        self.lib = lib
        self.path = path

    def _check(self, rc):
        if rc != 0:
            raise OracleError(self.lib.orc_last_error().decode())

    def max_threads(self) -> int:
        return self.lib.orc_max_threads()

    def store(self, dtype, key, value, key_cache, value_cache, slot_mapping):
        """Scatter rows of key/value ``[N, Hkv, D]`` into the caches ``[NB, Hkv, bs, D]`` in place.

        Row ``n`` goes to slot ``slot_mapping[n]`` (block ``s // bs``, offset ``s % bs``); negative
        slots are skipped; an out-of-pool or repeated slot raises ``OracleError`` and writes nothing."""
        sd = _store_dtype(dtype)
        for a in (key_cache, value_cache):
            if a.dtype != sd or not a.flags.c_contiguous:
                raise TypeError("caches must be C-contiguous arrays of the storage dtype")
        key, value = _c(key, sd), _c(value, sd)
        sm = _c(slot_mapping, np.int32)
        nb, hkv, bs, d = key_cache.shape
        self._check(self.lib.orc_store(_DT[dtype], _ptr(key), _ptr(value), _ptr(key_cache), _ptr(value_cache),
                                       _ptr(sm), len(sm), hkv, d, bs, nb))

    def quantize_int8(self, dtype, rows):
        """int8 codes and float32 scales of rows ``[..., D]`` (one scale per row): scale = max|x| / 127,
        code = round-half-even(x / scale) clamped to [-127, 127], in float32; zero rows give scale 0."""
        sd = _store_dtype(dtype)
        r = _c(rows, sd)
        d = r.shape[-1]
        n = r.size // d
        codes = np.zeros(r.shape, dtype=np.int8)
        scales = np.zeros(r.shape[:-1], dtype=np.float32)
        self._check(self.lib.orc_quantize_int8(_DT[dtype], _ptr(r), n, d, _ptr(codes), _ptr(scales)))
        return codes, scales

    def store_int8(self, dtype, key, value, key_cache, value_cache, key_scale, value_scale, slot_mapping):
        """Quantize rows of key/value ``[N, Hkv, D]`` and scatter codes into the int8 caches
        ``[NB, Hkv, bs, D]`` and scales into ``[NB, Hkv, bs]`` float32, in place (slots as in ``store``)."""
        sd = _store_dtype(dtype)
        for a, t in ((key_cache, np.int8), (value_cache, np.int8), (key_scale, np.float32), (value_scale, np.float32)):
            if a.dtype != t or not a.flags.c_contiguous:
                raise TypeError("int8 caches and float32 scales must be C-contiguous")
        key, value = _c(key, sd), _c(value, sd)
        sm = _c(slot_mapping, np.int32)
        nb, hkv, bs, d = key_cache.shape
        if key_scale.shape != (nb, hkv, bs) or value_scale.shape != (nb, hkv, bs):
            raise ValueError("scale arrays must be [num_blocks, num_kv_heads, block_size]")
        self._check(self.lib.orc_store_int8(_DT[dtype], _ptr(key), _ptr(value), _ptr(key_cache), _ptr(value_cache),
                                            _ptr(key_scale), _ptr(value_scale), _ptr(sm), len(sm), hkv, d, bs, nb))

    def dequantize_int8(self, codes, scales):
        """float64 values code * scale (exact) of int8 rows ``[..., D]`` with scales ``[...]``."""
        c, sc = _c(codes, np.int8), _c(scales, np.float32)
        d = c.shape[-1]
        if sc.shape != c.shape[:-1]:
            raise ValueError("one scale per row")
        out = np.empty(c.shape, dtype=np.float64)
        self._check(self.lib.orc_dequantize_int8(_ptr(c), _ptr(sc), c.size // d, d, _ptr(out)))
        return out

    def e4m3_value(self, code: int) -> float:
        """Value of an OCP float8 E4M3 code (NaN for 0x7f and 0xff)."""
        return self.lib.orc_e4m3_value(int(code))

    def e4m3_encode(self, v: float) -> int:
        """E4M3 code of the finite value nearest to float32 ``v`` (ties to an even mantissa)."""
        return self.lib.orc_e4m3_encode(float(np.float32(v)))

    def quantize_fp8(self, dtype, rows):
        """E4M3 codes (uint8) and float32 scales of rows ``[..., D]`` (one scale per row): scale = max|x| / 448,
        code = e4m3(x / scale) rounded half to even, in float32; zero rows give scale 0."""
        sd = _store_dtype(dtype)
        r = _c(rows, sd)
        d = r.shape[-1]
        n = r.size // d
        codes = np.zeros(r.shape, dtype=np.uint8)
        scales = np.zeros(r.shape[:-1], dtype=np.float32)
        self._check(self.lib.orc_quantize_fp8(_DT[dtype], _ptr(r), n, d, _ptr(codes), _ptr(scales)))
        return codes, scales

    def store_fp8(self, dtype, key, value, key_cache, value_cache, key_scale, value_scale, slot_mapping):
        """Quantize rows of key/value ``[N, Hkv, D]`` to E4M3 and scatter codes into the fp8 caches
        ``[NB, Hkv, bs, D]`` (uint8) and scales into ``[NB, Hkv, bs]`` float32, in place (slots as in ``store``)."""
        sd = _store_dtype(dtype)
        for a, t in ((key_cache, np.uint8), (value_cache, np.uint8), (key_scale, np.float32), (value_scale, np.float32)):
            if a.dtype != t or not a.flags.c_contiguous:
                raise TypeError("fp8 caches (uint8) and float32 scales must be C-contiguous")
        key, value = _c(key, sd), _c(value, sd)
        sm = _c(slot_mapping, np.int32)
        nb, hkv, bs, d = key_cache.shape
        if key_scale.shape != (nb, hkv, bs) or value_scale.shape != (nb, hkv, bs):
            raise ValueError("scale arrays must be [num_blocks, num_kv_heads, block_size]")
        self._check(self.lib.orc_store_fp8(_DT[dtype], _ptr(key), _ptr(value), _ptr(key_cache), _ptr(value_cache),
                                           _ptr(key_scale), _ptr(value_scale), _ptr(sm), len(sm), hkv, d, bs, nb))

    def dequantize_fp8(self, codes, scales):
        """float64 values e4m3(code) * scale (exact) of fp8 rows ``[..., D]`` with scales ``[...]``."""
        c, sc = _c(codes, np.uint8), _c(scales, np.float32)
        d = c.shape[-1]
        if sc.shape != c.shape[:-1]:
            raise ValueError("one scale per row")
        out = np.empty(c.shape, dtype=np.float64)
        self._check(self.lib.orc_dequantize_fp8(_ptr(c), _ptr(sc), c.size // d, d, _ptr(out)))
        return out

    def quantize_int4(self, dtype, rows):
        """4-bit codes and float32 scales of rows ``[..., D]`` (D even; one scale per row): scale = max|x| / 7,
        q = round-half-even(x / scale) clamped to [-7, 7], in float32, stored as u = q + 8 two per byte (element
        2j in the low four bits of byte j): codes ``[..., D / 2]`` uint8; zero rows give scale 0 and u = 8."""
        sd = _store_dtype(dtype)
        r = _c(rows, sd)
        d = r.shape[-1]
        n = r.size // d
        codes = np.zeros(r.shape[:-1] + (d // 2,), dtype=np.uint8)
        scales = np.zeros(r.shape[:-1], dtype=np.float32)
        self._check(self.lib.orc_quantize_int4(_DT[dtype], _ptr(r), n, d, _ptr(codes), _ptr(scales)))
        return codes, scales

    def store_int4(self, dtype, key, value, key_cache, value_cache, key_scale, value_scale, slot_mapping):
        """Quantize rows of key/value ``[N, Hkv, D]`` to 4-bit codes and scatter them into the int4 caches
        ``[NB, Hkv, bs, D / 2]`` (uint8) and scales into ``[NB, Hkv, bs]`` float32, in place (slots as in
        ``store``)."""
        sd = _store_dtype(dtype)
        for a, t in ((key_cache, np.uint8), (value_cache, np.uint8), (key_scale, np.float32), (value_scale, np.float32)):
            if a.dtype != t or not a.flags.c_contiguous:
                raise TypeError("int4 caches (uint8) and float32 scales must be C-contiguous")
        key, value = _c(key, sd), _c(value, sd)
        sm = _c(slot_mapping, np.int32)
        nb, hkv, bs, half = key_cache.shape
        if key.shape[-1] != 2 * half:
            raise ValueError("int4 cache rows hold head_dim / 2 bytes")
        if key_scale.shape != (nb, hkv, bs) or value_scale.shape != (nb, hkv, bs):
            raise ValueError("scale arrays must be [num_blocks, num_kv_heads, block_size]")
        self._check(self.lib.orc_store_int4(_DT[dtype], _ptr(key), _ptr(value), _ptr(key_cache), _ptr(value_cache),
                                            _ptr(key_scale), _ptr(value_scale), _ptr(sm), len(sm), hkv, 2 * half, bs,
                                            nb))

    def dequantize_int4(self, codes, scales):
        """float64 values (u - 8) * scale (exact) of int4 rows ``[..., D / 2]`` bytes with scales ``[...]``:
        returns ``[..., D]``."""
        c, sc = _c(codes, np.uint8), _c(scales, np.float32)
        half = c.shape[-1]
        if sc.shape != c.shape[:-1]:
            raise ValueError("one scale per row")
        out = np.empty(c.shape[:-1] + (2 * half,), dtype=np.float64)
        self._check(self.lib.orc_dequantize_int4(_ptr(c), _ptr(sc), c.size // half, 2 * half, _ptr(out)))
        return out

    def copy_blocks(self, dtype, key_cache, value_cache, pairs):
        """In place: block pairs[k, 1] of both caches becomes a copy of block pairs[k, 0]."""
        sd = _store_dtype(dtype)
        for a in (key_cache, value_cache):
            if a.dtype != sd or not a.flags.c_contiguous:
                raise TypeError("caches must be C-contiguous arrays of the storage dtype")
        pr = _c(pairs, np.int32).reshape(-1, 2)
        nb, hkv, bs, d = key_cache.shape
        self._check(self.lib.orc_copy_blocks(_DT[dtype], _ptr(key_cache), _ptr(value_cache), _ptr(pr), len(pr), hkv, d,
                                             bs, nb))

    def gather(self, dtype, key_cache, value_cache, block_table_row, length):
        """Logical tokens ``[0, length)`` of one block table as contiguous ``[length, Hkv, D]`` K and V."""
        sd = _store_dtype(dtype)
        kc, vc = _c(key_cache, sd), _c(value_cache, sd)
        nb, hkv, bs, d = kc.shape
        ko = np.empty((length, hkv, d), dtype=sd)
        vo = np.empty((length, hkv, d), dtype=sd)
        bt = _c(block_table_row, np.int32)
        self._check(self.lib.orc_gather(_DT[dtype], _ptr(ko), _ptr(vo), _ptr(kc), _ptr(vc), _ptr(bt), int(length),
                                        hkv, d, bs, nb))
        return ko, vo

    def decode(self, dtype, query, key_cache, value_cache, block_tables, context_lens, scale, seqs=None,
               nthreads=0):
        """Decode attention in float64: ``[n, Hq, D]`` for the sequences ``seqs`` (all if None)."""
        sd = _store_dtype(dtype)
        q, kc, vc = _c(query, sd), _c(key_cache, sd), _c(value_cache, sd)
        bt, cl = _c(block_tables, np.int32), _c(context_lens, np.int32)
        b, hq, d = q.shape
        nb, hkv, bs, d2 = kc.shape
        if d2 != d:
            raise ValueError("head_dim mismatch")
        sub = None if seqs is None else _c(seqs, np.int32)
        n = b if sub is None else len(sub)
        out = np.zeros((n, hq, d), dtype=np.float64)
        self._check(self.lib.orc_decode(_DT[dtype], _ptr(out), _ptr(q), _ptr(kc), _ptr(vc), _ptr(bt), bt.shape[1],
                                        _ptr(cl), b, hq, hkv, d, bs, nb, float(scale), _ptr(sub), n,
                                        int(nthreads)))
        return out

    def prefill(self, dtype, query, key_cache, value_cache, block_tables, cu_seqlens_q, cu_seqlens_k, scale,
                causal=True, rows=None, nthreads=0):
        """Varlen prefill attention in float64: ``[n, Hq, D]`` for the query rows ``rows`` (all if None)."""
        sd = _store_dtype(dtype)
        q, kc, vc = _c(query, sd), _c(key_cache, sd), _c(value_cache, sd)
        bt = _c(block_tables, np.int32)
        cq, ck = _c(cu_seqlens_q, np.int32), _c(cu_seqlens_k, np.int32)
        tq, hq, d = q.shape
        nb, hkv, bs, d2 = kc.shape
        if d2 != d:
            raise ValueError("head_dim mismatch")
        if len(cq) != len(ck) or len(cq) < 1:
            raise ValueError("cu_seqlens_q and cu_seqlens_k must both have num_seqs + 1 entries")
        if int(cq[-1]) != tq:
            raise ValueError("cu_seqlens_q[-1] must equal the number of query rows")
        sub = None if rows is None else _c(rows, np.int32)
        n = tq if sub is None else len(sub)
        out = np.zeros((n, hq, d), dtype=np.float64)
        self._check(self.lib.orc_prefill(_DT[dtype], _ptr(out), _ptr(q), _ptr(kc), _ptr(vc), _ptr(bt),
                                         bt.shape[1], _ptr(cq), _ptr(ck), len(cq) - 1, hq, hkv, d, bs, nb,
                                         float(scale), int(bool(causal)), _ptr(sub), n, int(nthreads)))
        return out


_default = None


def default() -> Oracle:
    global _default
    if _default is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build(force=True)
        _default = Oracle(LIB)
    return _default


def max_threads() -> int:
    return default().max_threads()


def store(*a, **k):
    return default().store(*a, **k)


def gather(*a, **k):
    return default().gather(*a, **k)


def copy_blocks(*a, **k):
    return default().copy_blocks(*a, **k)


def decode(*a, **k):
    return default().decode(*a, **k)


def prefill(*a, **k):
    return default().prefill(*a, **k)


def quantize_int8(*a, **k):
    return default().quantize_int8(*a, **k)


def store_int8(*a, **k):
    return default().store_int8(*a, **k)


def dequantize_int8(*a, **k):
    return default().dequantize_int8(*a, **k)


def e4m3_value(*a, **k):
    return default().e4m3_value(*a, **k)


def e4m3_encode(*a, **k):
    return default().e4m3_encode(*a, **k)


def quantize_fp8(*a, **k):
    return default().quantize_fp8(*a, **k)


def store_fp8(*a, **k):
    return default().store_fp8(*a, **k)


def dequantize_fp8(*a, **k):
    return default().dequantize_fp8(*a, **k)


def quantize_int4(*a, **k):
    return default().quantize_int4(*a, **k)


def store_int4(*a, **k):
    return default().store_int4(*a, **k)


def dequantize_int4(*a, **k):
    return default().dequantize_int4(*a, **k)
