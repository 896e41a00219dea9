"""The oracle: a plain, slow FP64 CPU implementation of the verify attention.

TEST INFRASTRUCTURE ONLY. Only tests/, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of bench.py may import this package. The product path
(the HIP library and its Python binding under paged_fp8_split_amd/) never
imports, links or calls anything here, and this package imports nothing from
the product path: the two share no code.

``oracle.c`` holds the arithmetic (see its header for the passages of the
pages it follows); this module only compiles it with gcc and marshals numpy
arrays through ctypes.

Pins (tests/test_oracle_pins.py and tests/golden/) tie it to things other
than itself: torch's float8_e4m3fn / float16 decoders over every byte and bit
pattern, torch's scaled-dot-product attention in float64 on dense gathered
inputs, closed-form special cases (single visible key, uniform scores, a
dominating key, exact FP16 midpoints), and invariances (partition size, page
relocation, tail sentinels, scale by powers of two, causal masking).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")
CFLAGS = ["-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared", "-std=c11"]

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so (gcc, -O2, no fast-math)."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + f".tmp{os.getpid()}"
        subprocess.run(["gcc", *CFLAGS, "-o", tmp, SRC, "-lm"], check=True)
        os.replace(tmp, LIB)
    return LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        build(force=True)
    lib = ctypes.CDLL(LIB)
    c = ctypes
    P = c.c_void_p
    lib.oracle_e4m3_value.restype = c.c_double
    lib.oracle_e4m3_value.argtypes = [c.c_uint32]
    lib.oracle_fp16_value.restype = c.c_double
    lib.oracle_fp16_value.argtypes = [c.c_uint32]
    lib.oracle_e4m3_table.restype = None
    lib.oracle_e4m3_table.argtypes = [P]
    lib.oracle_e5m2_value.restype = c.c_double
    lib.oracle_e5m2_value.argtypes = [c.c_uint32]
    lib.oracle_kv_table.restype = c.c_int
    lib.oracle_kv_table.argtypes = [c.c_int32, P]
    lib.oracle_visible_keys.restype = c.c_int64
    lib.oracle_visible_keys.argtypes = [c.c_int64, c.c_int32, c.c_int32]
    lib.oracle_max_threads.restype = c.c_int32
    lib.oracle_max_threads.argtypes = []
    lib.oracle_verify.restype = c.c_int
    lib.oracle_verify.argtypes = [c.c_int32] * 9 + [c.c_int64] * 3 + [P] * 9 + [c.c_double, P, c.c_int32, c.c_int32]
    lib.oracle_e4m3_encode.restype = c.c_uint32
    lib.oracle_e4m3_encode.argtypes = [c.c_float]
    lib.oracle_e5m2_encode.restype = c.c_uint32
    lib.oracle_e5m2_encode.argtypes = [c.c_float]
    lib.oracle_quantize_fp16.restype = c.c_uint32
    lib.oracle_quantize_fp16.argtypes = [c.c_uint32, c.c_float, c.c_int32]
    lib.oracle_fp16_rne.restype = c.c_uint32
    lib.oracle_fp16_rne.argtypes = [c.c_double]
    lib.oracle_dequant.restype = c.c_int
    lib.oracle_dequant.argtypes = [c.c_int32] * 6 + [c.c_int64] * 3 + [P] * 5 + [c.c_int32]
    lib.oracle_kv_append.restype = c.c_int
    lib.oracle_kv_append.argtypes = [c.c_int32] * 7 + [c.c_int64] * 3 + [P] * 8 + [c.c_int32]
    _lib = lib
    return lib


KV_FORMATS = {"e4m3": 0, "e5m2": 1}


def _fmt(name: str) -> int:
    try:
        return KV_FORMATS[name]
    except KeyError:
        raise ValueError(f"unknown KV format {name!r}") from None


def kv_table(kv_format: str = "e4m3") -> np.ndarray:
    """Decoded value of every byte 0..255 of a KV format (float64)."""
    out = np.empty(256, dtype=np.float64)
    if _load().oracle_kv_table(_fmt(kv_format), out.ctypes.data) != 0:
        raise ValueError(kv_format)
    return out


def e5m2_table() -> np.ndarray:
    """Decoded value of every E5M2 byte 0..255 (float64; +-inf and NaN codes included)."""
    return np.array([_load().oracle_e5m2_value(b) for b in range(256)], dtype=np.float64)


def e4m3_table() -> np.ndarray:
    """Decoded value of every E4M3 byte 0..255 (float64; NaN for 0x7F/0xFF)."""
    out = np.empty(256, dtype=np.float64)
    _load().oracle_e4m3_table(out.ctypes.data)
    return out


def fp16_value(bits: int) -> float:
    return _load().oracle_fp16_value(int(bits) & 0xFFFF)


def visible_keys(live_len: int, q: int, row: int) -> int:
    return int(_load().oracle_visible_keys(int(live_len), int(q), int(row)))


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def _ptr(a: np.ndarray):
    return a.ctypes.data


def verify(w, *, partition_tokens: Optional[int] = None, unit_mask: Optional[np.ndarray] = None,
           threads: int = 0, sm_scale: Optional[float] = None) -> np.ndarray:
    """FP64 verify attention of workload ``w`` -> float64 [B, q, Hq, D].

    partition_tokens: partition size T (default: the workload's, 64); 0 means
    one partition per row (the unsplit softmax).
    unit_mask: optional bool/uint8 [B, Hq]; only those (request, query head)
    units are computed, the others are NaN.
    """
    T = w.partition_tokens if partition_tokens is None else int(partition_tokens)
    qb = np.ascontiguousarray(w.q_fp16).view(np.uint16)
    kp = np.ascontiguousarray(w.k_pool, dtype=np.uint8)
    vp = np.ascontiguousarray(w.v_pool, dtype=np.uint8)
    ks = np.ascontiguousarray(w.k_scale, dtype=np.float32)
    vs = np.ascontiguousarray(w.v_scale, dtype=np.float32)
    bt = np.ascontiguousarray(w.block_table, dtype=np.int32)
    ll = np.ascontiguousarray(w.live_len, dtype=np.int32)
    hm = np.ascontiguousarray(w.head_map, dtype=np.int32)
    out = np.full((w.batch, w.q, w.num_q_heads, w.head_dim), np.nan, dtype=np.float64)
    mask = None
    if unit_mask is not None:
        mask = np.ascontiguousarray(np.asarray(unit_mask).reshape(w.batch, w.num_q_heads), dtype=np.uint8)
    rc = _load().oracle_verify(
        w.batch, w.q, w.num_q_heads, w.num_kv_heads, w.head_dim, w.page_size, w.max_pages_per_row,
        w.num_pool_pages, T, w.page_stride, w.token_stride, w.head_stride,
        _ptr(qb), _ptr(kp), _ptr(vp), _ptr(ks), _ptr(vs), _ptr(bt), _ptr(ll), _ptr(hm),
        _ptr(mask) if mask is not None else None,
        float(w.sm_scale if sm_scale is None else sm_scale), _ptr(out), int(threads),
        _fmt(getattr(w, "kv_format", "e4m3")))
    if rc != 0:
        raise RuntimeError(f"oracle_verify failed with code {rc}")
    return out


def e4m3_encode(values) -> np.ndarray:
    """E4M3FN code (uint8) of each FP32 value: nearest, ties to even,
    saturating at +-448, NaN -> 0x7F."""
    lib = _load()
    v = np.asarray(values, dtype=np.float32).ravel()
    return np.array([lib.oracle_e4m3_encode(float(x)) for x in v], dtype=np.uint8).reshape(np.shape(values))


def e5m2_encode(values) -> np.ndarray:
    """E5M2 code (uint8) of each FP32 value: nearest, ties to even,
    saturating at +-57344, NaN -> 0x7F."""
    lib = _load()
    v = np.asarray(values, dtype=np.float32).ravel()
    return np.array([lib.oracle_e5m2_encode(float(x)) for x in v], dtype=np.uint8).reshape(np.shape(values))


def quantize_fp16(bits, scale: float, kv_format: str = "e4m3") -> np.ndarray:
    """Code of (float)x / scale in ``kv_format`` for FP16 bit patterns ``bits``."""
    lib = _load()
    f = _fmt(kv_format)
    b = np.asarray(bits, dtype=np.uint16).ravel()
    s = float(np.float32(scale))
    return np.array([lib.oracle_quantize_fp16(int(x), s, f) for x in b], dtype=np.uint8).reshape(np.shape(bits))


def kv_append(w, k_new_fp16: np.ndarray, v_new_fp16: np.ndarray, k_scale=None, v_scale=None):
    """Store the draft tokens' FP16 K/V [B, q, Hkv, D] of workload ``w`` into
    copies of its pools; returns (k_pool, v_pool) as new uint8 arrays."""
    kp = np.array(w.k_pool, dtype=np.uint8, copy=True)
    vp = np.array(w.v_pool, dtype=np.uint8, copy=True)
    kn = np.ascontiguousarray(k_new_fp16, dtype=np.float16).view(np.uint16)
    vn = np.ascontiguousarray(v_new_fp16, dtype=np.float16).view(np.uint16)
    assert kn.shape == (w.batch, w.q, w.num_kv_heads, w.head_dim) and vn.shape == kn.shape
    ks = np.ascontiguousarray(w.k_scale if k_scale is None else k_scale, dtype=np.float32)
    vs = np.ascontiguousarray(w.v_scale if v_scale is None else v_scale, dtype=np.float32)
    bt = np.ascontiguousarray(w.block_table, dtype=np.int32)
    ll = np.ascontiguousarray(w.live_len, dtype=np.int32)
    rc = _load().oracle_kv_append(
        w.batch, w.q, w.num_kv_heads, w.head_dim, w.page_size, w.max_pages_per_row, w.num_pool_pages,
        w.page_stride, w.token_stride, w.head_stride, _ptr(kn), _ptr(vn), _ptr(ks), _ptr(vs), _ptr(bt), _ptr(ll),
        _ptr(kp), _ptr(vp), _fmt(getattr(w, "kv_format", "e4m3")))
    if rc != 0:
        raise RuntimeError(f"oracle_kv_append failed with code {rc}")
    return kp, vp


def fp16_rne(values) -> np.ndarray:
    """IEEE binary16 bits (uint16) of each float64 value, rounded to nearest even."""
    lib = _load()
    v = np.asarray(values, dtype=np.float64).ravel()
    return np.array([lib.oracle_fp16_rne(float(x)) for x in v], dtype=np.uint16).reshape(np.shape(values))


def dequant(w, pool: Optional[np.ndarray] = None, scale: Optional[np.ndarray] = None) -> np.ndarray:
    """Paged FP8 -> FP16 bridge of workload ``w``'s pool (K by default):
    float16 [B, capacity, Hkv, D], dec(byte) * scale rounded once, with dec
    the decoder of the workload's KV format; +0.0 beyond each live length.
    scale None means 1."""
    p = np.ascontiguousarray(w.k_pool if pool is None else pool, dtype=np.uint8)
    sc = None if scale is None else np.ascontiguousarray(scale, dtype=np.float32)
    bt = np.ascontiguousarray(w.block_table, dtype=np.int32)
    ll = np.ascontiguousarray(w.live_len, dtype=np.int32)
    out = np.empty((w.batch, w.capacity, w.num_kv_heads, w.head_dim), dtype=np.uint16)
    rc = _load().oracle_dequant(w.batch, w.num_kv_heads, w.head_dim, w.page_size, w.max_pages_per_row,
                                w.num_pool_pages, w.page_stride, w.token_stride, w.head_stride, _ptr(p),
                                _ptr(sc) if sc is not None else None, _ptr(bt), _ptr(ll), _ptr(out),
                                _fmt(getattr(w, "kv_format", "e4m3")))
    if rc != 0:
        raise RuntimeError(f"oracle_dequant failed with code {rc}")
    return out.view(np.float16)
