"""CPU oracle for int4 (and int8) group-affine KV quantisation and decode
attention.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product library and its Python
binding never do. The arithmetic lives in ``kvq_oracle.c`` (plain C, float64
attention); this module builds it with gcc and marshals numpy arrays.

Every function says which passage it follows; the page-level citations and the
readings taken where the pages are silent are in the header of
``kvq_oracle.c``.
"""

from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kvq_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-pthread"]

_lib = None


def build(force: bool = True) -> str:
    """Compile kvq_oracle.c into liboracle.so with gcc (strict IEEE flags)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    build(force=False)
    lib = C.CDLL(_LIB)
    u16p, u32p, f32p, f64p, u8p = (C.POINTER(C.c_uint16), C.POINTER(C.c_uint32), C.POINTER(C.c_float),
                                   C.POINTER(C.c_double), C.POINTER(C.c_uint8))
    lib.oracle_f16_to_f64_n.restype = None
    lib.oracle_f16_to_f64_n.argtypes = [u16p, C.c_int64, f64p]
    lib.oracle_f16_round_n.restype = None
    lib.oracle_f16_round_n.argtypes = [f32p, C.c_int64, C.c_int, u16p]
    lib.oracle_quantize_group.restype = None
    lib.oracle_quantize_group.argtypes = [f32p, C.c_int, u16p, u16p, u8p]
    lib.oracle_quantize_group_bits.restype = None
    lib.oracle_quantize_group_bits.argtypes = [f32p, C.c_int, C.c_int, u16p, u16p, u8p]
    lib.oracle_pack_row_bits.argtypes = [u8p, C.c_int, C.c_int, u32p]
    lib.oracle_unpack_row_bits.argtypes = [u32p, C.c_int, C.c_int, u8p]
    lib.oracle_quantize_rows.restype = C.c_int
    lib.oracle_quantize_rows.argtypes = [f32p, C.c_int64, C.c_int, C.c_int, C.c_int, u32p, u16p, u16p]
    lib.oracle_dequantize_rows.restype = None
    lib.oracle_dequantize_rows.argtypes = [u32p, u16p, u16p, C.c_int64, C.c_int, C.c_int, C.c_int, f64p]
    cache_args = [u32p, u32p, u16p, u16p, u16p, u16p, C.c_int, C.c_int, C.c_int, C.c_int, C.c_int, C.c_int64,
                  C.c_int64, f64p, C.c_int, C.c_double]
    lib.oracle_sdpa.restype = C.c_int
    lib.oracle_sdpa.argtypes = cache_args + [f64p, C.c_int]
    lib.oracle_sdpa_partials.restype = C.c_int
    lib.oracle_sdpa_partials.argtypes = cache_args + [C.c_int64, f64p, f64p, f64p, C.c_int]
    lib.oracle_hadamard_rows.restype = C.c_int
    lib.oracle_hadamard_rows.argtypes = [f64p, C.c_int64, C.c_int, f64p]
    lib.oracle_combine_partials.restype = None
    lib.oracle_combine_partials.argtypes = [f64p, f64p, f64p, C.c_int64, C.c_int64, C.c_int, f64p]
    _lib = lib
    return lib


def _p(a: np.ndarray, ct):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(C.POINTER(ct))


def default_threads() -> int:
    return max(1, min(64, os.cpu_count() or 1))


# ------------------------------------------------------------------- fp16

def f16_to_f64(bits) -> np.ndarray:
    """Value of fp16 bit patterns, decoded from the binary16 definition."""
    lib = _load()
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.zeros(b.shape, dtype=np.float64)
    lib.oracle_f16_to_f64_n(_p(b, C.c_uint16), b.size, _p(out, C.c_double))
    return out


def _f16_round(mode, x) -> np.ndarray:
    lib = _load()
    a = np.ascontiguousarray(x, dtype=np.float32)
    out = np.zeros(a.shape, dtype=np.uint16)
    lib.oracle_f16_round_n(_p(a, C.c_float), a.size, mode, _p(out, C.c_uint16))
    return out


def f16_rn(x):
    """fp32 -> fp16 bits, round to nearest even."""
    return _f16_round(0, x)


def f16_rd(x):
    """fp32 -> largest fp16 not above x (bits)."""
    return _f16_round(1, x)


def f16_ru(x):
    """fp32 -> smallest fp16 not below x (bits)."""
    return _f16_round(2, x)


# -------------------------------------------------------------- quantiser

BITS = (4, 8)


def _check_bits(bits):
    if bits not in BITS:
        raise ValueError("bits must be 4 or 8, got %r" % (bits,))
    return 32 // bits  # codes per word


def quantize_group(x: np.ndarray, bits: int = 4):
    """One group -> (codes uint8[G], scale bits, bias bits). Group-affine
    quantisation with a scale and a bias per group ("Background: Why
    TurboQuant Fails on Gemma 4"; the README's lesson on asymmetric int4):
    codes 0..15 for bits=4, 0..255 for the 8-bit variant (the Gemma page's
    "What I Tried" table lists int8 KV; the blog's driver takes 4 or 8 KV
    bits)."""
    lib = _load()
    _check_bits(bits)
    x = np.ascontiguousarray(x, dtype=np.float32).ravel()
    codes = np.zeros(x.size, dtype=np.uint8)
    s = C.c_uint16()
    b = C.c_uint16()
    lib.oracle_quantize_group_bits(_p(x, C.c_float), x.size, bits, C.byref(s), C.byref(b), _p(codes, C.c_uint8))
    return codes, int(s.value), int(b.value)


def pack_row(codes: np.ndarray, bits: int = 4) -> np.ndarray:
    """Codes of one row -> uint32 words, 32/bits per word, lowest field first
    ("What I Built Instead": masks 0xF, 0xF0, 0xF00, 0xF000; bytes for the
    8-bit variant)."""
    lib = _load()
    P = _check_bits(bits)
    c = np.ascontiguousarray(codes, dtype=np.uint8).ravel()
    w = np.zeros(c.size // P, dtype=np.uint32)
    lib.oracle_pack_row_bits(_p(c, C.c_uint8), c.size, bits, _p(w, C.c_uint32))
    return w


def unpack_row(words: np.ndarray, bits: int = 4) -> np.ndarray:
    lib = _load()
    P = _check_bits(bits)
    w = np.ascontiguousarray(words, dtype=np.uint32).ravel()
    c = np.zeros(w.size * P, dtype=np.uint8)
    lib.oracle_unpack_row_bits(_p(w, C.c_uint32), c.size, bits, _p(c, C.c_uint8))
    return c


def quantize_rows(x: np.ndarray, group: int = 64, bits: int = 4):
    """x[..., D] (fp16 or fp32; widened exactly to fp32) -> (words uint32[...,
    D*bits/32], scale uint16[..., D/G], bias uint16[..., D/G])."""
    lib = _load()
    P = _check_bits(bits)
    x32 = np.ascontiguousarray(x, dtype=np.float32)
    D = x32.shape[-1]
    rows = x32.size // D
    lead = x32.shape[:-1]
    words = np.zeros(lead + (D // P,), dtype=np.uint32)
    scale = np.zeros(lead + (D // group,), dtype=np.uint16)
    bias = np.zeros(lead + (D // group,), dtype=np.uint16)
    rc = lib.oracle_quantize_rows(_p(x32, C.c_float), rows, D, group, bits, _p(words, C.c_uint32),
                                  _p(scale, C.c_uint16), _p(bias, C.c_uint16))
    if rc != 0:
        raise ValueError("oracle_quantize_rows: bad shape D=%d G=%d" % (D, group))
    return words, scale, bias


def dequantize_rows(words: np.ndarray, scale: np.ndarray, bias: np.ndarray, group: int = 64,
                    bits: int = 4) -> np.ndarray:
    """Packed rows -> float64 values code * scale + bias (exact in float64)."""
    lib = _load()
    P = _check_bits(bits)
    w = np.ascontiguousarray(words, dtype=np.uint32)
    s = np.ascontiguousarray(scale, dtype=np.uint16)
    b = np.ascontiguousarray(bias, dtype=np.uint16)
    D = w.shape[-1] * P
    rows = w.size // w.shape[-1]
    out = np.zeros(w.shape[:-1] + (D,), dtype=np.float64)
    lib.oracle_dequantize_rows(_p(w, C.c_uint32), _p(s, C.c_uint16), _p(b, C.c_uint16), rows, D, group, bits,
                               _p(out, C.c_double))
    return out


class Cache:
    """Host copy of one layer's quantised cache in the oracle's layout:
    words [B][Hkv][cap][D*bits/32]; scale/bias [B][Hkv][cap][D/G] (fp16
    bits)."""

    def __init__(self, B, Hkv, D, cap, group=64, bits=4):
        P = _check_bits(bits)
        self.B, self.Hkv, self.D, self.cap, self.G, self.bits = B, Hkv, D, cap, group, bits
        self.k_q = np.zeros((B, Hkv, cap, D // P), dtype=np.uint32)
        self.v_q = np.zeros_like(self.k_q)
        self.k_scale = np.zeros((B, Hkv, cap, D // group), dtype=np.uint16)
        self.k_bias = np.zeros_like(self.k_scale)
        self.v_scale = np.zeros_like(self.k_scale)
        self.v_bias = np.zeros_like(self.k_scale)

    def append(self, k: np.ndarray, v: np.ndarray, length: int):
        """Quantise k, v [B][Hkv][n][D] into rows [length, length + n)."""
        n = k.shape[2]
        assert length + n <= self.cap
        for src, wq, sc, bi in ((k, self.k_q, self.k_scale, self.k_bias), (v, self.v_q, self.v_scale, self.v_bias)):
            w, s, b = quantize_rows(src, self.G, self.bits)
            wq[:, :, length:length + n] = w
            sc[:, :, length:length + n] = s
            bi[:, :, length:length + n] = b

    def append_rotated(self, k: np.ndarray, v: np.ndarray, length: int):
        """Hadamard-rotated append (TurboQuant explainer blog, "TurboQuant"
        section and step "1. Vector Rotation"): each fp16 row x is rotated to
        fl32(hadamard(x)) and that fp32 row is quantised into rows
        [length, length + n). fp16 inputs only: their rotation sums are exact,
        so the fp32 values, and with them the codes, are fixed."""
        k, v = np.asarray(k), np.asarray(v)
        if k.dtype != np.float16 or v.dtype != np.float16:
            raise TypeError("append_rotated takes fp16 rows")
        self.append(hadamard(k).astype(np.float32), hadamard(v).astype(np.float32), length)

    def _args(self):
        return (_p(self.k_q, C.c_uint32), _p(self.v_q, C.c_uint32), _p(self.k_scale, C.c_uint16),
                _p(self.k_bias, C.c_uint16), _p(self.v_scale, C.c_uint16), _p(self.v_bias, C.c_uint16),
                self.B, self.Hkv, self.D, self.G, self.bits, self.cap)


def sdpa(cache: Cache, skv: int, q: np.ndarray, alpha: float, nthreads: int | None = None) -> np.ndarray:
    """Exact decode attention over rows [0, skv) of the cache, float64.

    q[B][Hq][D] (fp16/fp32, widened exactly). Scores alpha * q . k^, exact
    two-pass softmax, weighted sum of v^ (README kernel paragraph; GQA with
    query head h on KV head h / (Hq/Hkv))."""
    lib = _load()
    q64 = np.ascontiguousarray(q, dtype=np.float64)
    B, Hq, D = q64.shape
    out = np.zeros((B, Hq, D), dtype=np.float64)
    rc = lib.oracle_sdpa(*cache._args(), skv, _p(q64, C.c_double), Hq, float(alpha), _p(out, C.c_double),
                         nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle_sdpa failed (%d)" % rc)
    return out


def sdpa_partials(cache: Cache, skv: int, q: np.ndarray, alpha: float, chunk: int, nthreads: int | None = None):
    """Split-K partials per chunk (README split-K paragraph): (m, l, acc) with
    m[B][Hq][C], l[B][Hq][C], acc[B][Hq][C][D], all float64."""
    lib = _load()
    q64 = np.ascontiguousarray(q, dtype=np.float64)
    B, Hq, D = q64.shape
    nc = (skv + chunk - 1) // chunk
    m = np.zeros((B, Hq, nc))
    l = np.zeros((B, Hq, nc))
    acc = np.zeros((B, Hq, nc, D))
    rc = lib.oracle_sdpa_partials(*cache._args(), skv, _p(q64, C.c_double), Hq, float(alpha), chunk,
                                  _p(m, C.c_double), _p(l, C.c_double), _p(acc, C.c_double),
                                  nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle_sdpa_partials failed (%d)" % rc)
    return m, l, acc


def sdpa_prefill(cache: Cache, q_start: int, q: np.ndarray, alpha: float, nthreads: int | None = None) -> np.ndarray:
    """Prefill-side attention over the quantised cache, float64 (the README's
    hybrid paragraph routes Sq > 1 to a separate attention; here it reads the
    same quantised cache): q[B][Hq][Sq][D] holds the queries of positions
    q_start .. q_start + Sq - 1, whose K/V rows are already cache rows
    [q_start, q_start + Sq); query i attends to rows [0, q_start + i]
    (causal). Each position is the decode attention (sdpa) over its own
    prefix, taken one position at a time."""
    q64 = np.asarray(q, dtype=np.float64)
    B, Hq, Sq, D = q64.shape
    out = np.zeros((B, Hq, Sq, D), dtype=np.float64)
    for i in range(Sq):
        out[:, :, i] = sdpa(cache, q_start + i + 1, np.ascontiguousarray(q64[:, :, i]), alpha, nthreads)
    return out


def hadamard(x: np.ndarray) -> np.ndarray:
    """Normalised Hadamard rotation of the last axis (a power of two), in
    float64: y = H_n x / sqrt(n) with H_n in Sylvester order (the TurboQuant
    explainer blog's worked example). Its own inverse."""
    lib = _load()
    x64 = np.ascontiguousarray(x, dtype=np.float64)
    n = x64.shape[-1]
    out = np.zeros_like(x64)
    if lib.oracle_hadamard_rows(_p(x64, C.c_double), x64.size // n, n, _p(out, C.c_double)) != 0:
        raise ValueError("hadamard: length %d is not a power of two" % n)
    return out


def sdpa_rotated(cache: Cache, skv: int, q: np.ndarray, alpha: float, nthreads: int | None = None) -> np.ndarray:
    """Attention over a Hadamard-rotated cache (rows appended with
    Cache.append_rotated): the query is rotated the same way, so its scores
    against rotated keys equal those against the original keys, and the
    output, a combination of rotated value rows, is rotated back (the
    rotation is its own inverse). float64 throughout."""
    return hadamard(sdpa(cache, skv, hadamard(q), alpha, nthreads))


def combine_partials(m: np.ndarray, l: np.ndarray, acc: np.ndarray) -> np.ndarray:
    """Reduce split-K partials to the attention output (float64)."""
    lib = _load()
    m = np.ascontiguousarray(m, dtype=np.float64)
    l = np.ascontiguousarray(l, dtype=np.float64)
    acc = np.ascontiguousarray(acc, dtype=np.float64)
    nc, D = acc.shape[-2], acc.shape[-1]
    heads = m.size // nc
    out = np.zeros(m.shape[:-1] + (D,), dtype=np.float64)
    lib.oracle_combine_partials(_p(m, C.c_double), _p(l, C.c_double), _p(acc, C.c_double), heads, nc, D,
                                _p(out, C.c_double))
    return out
