"""CPU oracle for the scaled FP8 (OCP E4M3) GEMM -- test infrastructure only.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never does, and
shares no code with it: this is a plain, slow, exact restatement of what the
pages compute, used to check the HIP kernels.

What it computes (pages: "Triton FP8 GEMM via CUTLASS naming", kernel section
and parameter list -- e4m3fn inputs within +-448, FP32 accumulator,
acc*scale_a*scale_b, output dequantised to FP32 or BF16; "FP8 GEMM in JAX with
Triton for Blackwell", parameter paragraph -- 32x32 block scales -- and MoE
paragraph -- grouped GEMM over experts):

* ``e4m3_table``       -- decode of all 256 codes (a typed-out table in C).
* ``quantize_*``       -- amax, scale = fl32(amax/448) (1 for an all-zero
                          group), codes = RNE-saturating E4M3 of fl32(x/scale).
* ``gemm_rows`` / ``gemm_sampled`` -- exact sum_k a*b (FP64 is exact here),
                          scaled by sa*sb and rounded once to FP32 or BF16.
* ``gemm_blockscaled_rows`` -- per-32-K-block exact partials, scaled by
                          s_a*s_b and summed in FP64, rounded once.
* ``grouped_gemm_rows`` -- the per-tensor GEMM applied per expert group.
* ``quantize_blocked_t`` / ``gemm_blockscaled_rows_t`` -- block scales of
                          32x32 or 64x64 tiles (the Blackwell page's
                          granularity and its coarser fallback).
* ``quantize_blocked_e8m0`` / ``gemm_blockscaled_e8m0_rows`` -- 32x32 tile
                          scales as powers of two (OCP MX shared exponents,
                          E8M0 bytes).
* ``prune_2of4`` / ``compress_2of4`` -- 2:4 magnitude pruning of the weights
                          along K and the compressed (values, 2-bit
                          positions) form the sparse matrix cores take; the
                          GEMM itself is ``gemm_rows`` on the pruned codes.
* ``e5m2_table``, ``quantize_*_fmt``, ``gemm_rows_fmt`` -- the same for OCP
                          E5M2 operands (scale = fl32(amax/57344)) and mixed
                          E4M3 x E5M2 pairs, summed exactly in 128-bit
                          integers, rounded once to FP32, BF16 or FP16
                          ("FP8 GEMM in JAX with Triton for Blackwell":
                          opening section, kernel sketch's float16 store).

The C core lives in ``oracle.c`` and is compiled to ``liboracle.so`` with gcc
(``build()``); every function there cites the passage it follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

F32, BF16, F16 = 0, 1, 2  # output kinds
E4M3, E5M2 = 0, 1        # operand formats


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so (plain gcc, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-Wall",
                               "-shared", "-fPIC", _SRC, "-o", tmp])
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i64, i32, f32 = ctypes.c_int64, ctypes.c_int32, ctypes.c_float
        L.orc_e4m3_decode.restype = ctypes.c_double
        L.orc_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.orc_e4m3_table.argtypes = [P]
        L.orc_e4m3_rne_sat.restype = ctypes.c_uint8
        L.orc_e4m3_rne_sat.argtypes = [f32]
        L.orc_amax.restype = f32
        L.orc_amax.argtypes = [P, i64]
        L.orc_scale_from_amax.restype = f32
        L.orc_scale_from_amax.argtypes = [f32]
        L.orc_quantize_with_scale.argtypes = [P, i64, f32, P]
        L.orc_quantize_pertensor.argtypes = [P, i64, P, P, P]
        L.orc_quantize_blocked.argtypes = [P, i64, i64, P, P]
        L.orc_quantize_grouped.argtypes = [P, i64, i64, P, i32, P, P, P]
        L.orc_round_scaled.restype = ctypes.c_uint32
        L.orc_round_scaled.argtypes = [i64, f32, f32, ctypes.c_int]
        L.orc_round_f64.restype = ctypes.c_uint32
        L.orc_round_f64.argtypes = [ctypes.c_double, ctypes.c_int]
        L.orc_gemm_dot_i64.argtypes = [P, P, i64, i64, i64, P]
        L.orc_gemm_rows_f64.argtypes = [P, P, i64, i64, P, i64, P, P]
        L.orc_gemm_rows.argtypes = [P, P, f32, f32, i64, i64, P, i64, ctypes.c_int, P, P, P, P]
        L.orc_gemm_sampled.argtypes = [P, P, f32, f32, i64, i64, P, P, i64, ctypes.c_int, P, P, P]
        L.orc_gemm_blockscaled_rows.argtypes = [P, P, P, P, i64, i64, P, i64, ctypes.c_int, P, P, P, P]
        L.orc_e5m2_decode.restype = ctypes.c_double
        L.orc_e5m2_decode.argtypes = [ctypes.c_uint8]
        L.orc_e5m2_table.argtypes = [P]
        L.orc_e5m2_rne_sat.restype = ctypes.c_uint8
        L.orc_e5m2_rne_sat.argtypes = [f32]
        L.orc_scale_from_amax_fmt.restype = f32
        L.orc_scale_from_amax_fmt.argtypes = [f32, ctypes.c_int]
        L.orc_quantize_with_scale_fmt.argtypes = [P, i64, f32, ctypes.c_int, P]
        L.orc_quantize_pertensor_fmt.argtypes = [P, i64, ctypes.c_int, P, P, P]
        L.orc_quantize_grouped_fmt.argtypes = [P, i64, P, i32, ctypes.c_int, P, P, P]
        L.orc_round_ieee_f64.restype = ctypes.c_uint32
        L.orc_round_ieee_f64.argtypes = [ctypes.c_double, ctypes.c_int]
        L.orc_gemm_rows_fmt.restype = ctypes.c_int
        L.orc_gemm_rows_fmt.argtypes = [P, P, ctypes.c_int, ctypes.c_int, f32, f32, i64, i64, P, i64, ctypes.c_int,
                                        P, P, P]
        L.orc_quantize_blocked_t.argtypes = [P, i64, i64, ctypes.c_int, P, P]
        L.orc_gemm_blockscaled_rows_t.argtypes = [P, P, P, P, i64, i64, ctypes.c_int, P, i64, ctypes.c_int, P, P, P]
        L.orc_e8m0_exponent.restype = ctypes.c_int
        L.orc_e8m0_exponent.argtypes = [f32]
        L.orc_quantize_blocked_e8m0.argtypes = [P, i64, i64, P, P]
        L.orc_gemm_blockscaled_e8m0_rows.argtypes = [P, P, P, P, i64, i64, P, i64, ctypes.c_int, P, P, P]
        L.orc_prune_2of4.argtypes = [P, i64, i64, P]
        L.orc_compress_2of4.argtypes = [P, i64, i64, P, P]
        L.orc_num_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def _p(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def num_threads() -> int:
    return int(lib().orc_num_threads())


# --------------------------------------------------------------------------
# E4M3 codes
# --------------------------------------------------------------------------
def e4m3_table() -> np.ndarray:
    """float64[256]: the value of every E4M3 code (NaN for 0x7F and 0xFF)."""
    out = np.zeros(256, dtype=np.float64)
    lib().orc_e4m3_table(_p(out))
    return out


def decode(q: np.ndarray) -> np.ndarray:
    return e4m3_table()[np.asarray(q, dtype=np.uint8)]


def e4m3_rne_sat(v: float) -> int:
    """One binary32 value to its RNE-saturating E4M3 code."""
    return int(lib().orc_e4m3_rne_sat(ctypes.c_float(v)))


def convert(x: np.ndarray) -> np.ndarray:
    """Elementwise RNE-saturating FP32 -> E4M3 codes (scale 1)."""
    x = _c(x, np.float32)
    q = np.empty(x.shape, dtype=np.uint8)
    lib().orc_quantize_with_scale(_p(x), x.size, ctypes.c_float(1.0), _p(q))
    return q


# --------------------------------------------------------------------------
# Quantization
# --------------------------------------------------------------------------
def amax(x: np.ndarray) -> np.float32:
    x = _c(x, np.float32)
    return np.float32(lib().orc_amax(_p(x), x.size))


def scale_from_amax(a: float) -> np.float32:
    return np.float32(lib().orc_scale_from_amax(ctypes.c_float(a)))


def quantize_with_scale(x: np.ndarray, scale: float) -> np.ndarray:
    x = _c(x, np.float32)
    q = np.empty(x.shape, dtype=np.uint8)
    lib().orc_quantize_with_scale(_p(x), x.size, ctypes.c_float(scale), _p(q))
    return q


def quantize_pertensor(x: np.ndarray):
    """Returns (codes uint8 same shape, scale float32, amax float32)."""
    x = _c(x, np.float32)
    q = np.empty(x.shape, dtype=np.uint8)
    s = np.zeros(1, np.float32)
    a = np.zeros(1, np.float32)
    lib().orc_quantize_pertensor(_p(x), x.size, _p(q), _p(s), _p(a))
    return q, s[0], a[0]


def quantize_blocked(x: np.ndarray):
    """32x32 tiles; returns (codes, tile scales float32[rows/32, cols/32])."""
    x = _c(x, np.float32)
    rows, cols = x.shape
    assert rows % 32 == 0 and cols % 32 == 0
    q = np.empty(x.shape, dtype=np.uint8)
    ts = np.empty((rows // 32, cols // 32), dtype=np.float32)
    lib().orc_quantize_blocked(_p(x), rows, cols, _p(q), _p(ts))
    return q, ts


def quantize_grouped(x: np.ndarray, offsets: np.ndarray):
    """Row groups [off[g], off[g+1]); returns (codes, scales[G], amax[G])."""
    x = _c(x, np.float32)
    rows, cols = x.shape
    off = _c(offsets, np.int32)
    G = off.size - 1
    q = np.zeros(x.shape, dtype=np.uint8)
    s = np.empty(G, np.float32)
    a = np.empty(G, np.float32)
    lib().orc_quantize_grouped(_p(x), rows, cols, _p(off), G, _p(q), _p(s), _p(a))
    return q, s, a


# --------------------------------------------------------------------------
# Rounding
# --------------------------------------------------------------------------
def round_scaled(d: int, sa: float, sb: float, kind: int) -> int:
    """Bits of sa*sb*d*2^-18 rounded once (kind F32 -> uint32 bits, BF16 -> uint16 bits)."""
    return int(lib().orc_round_scaled(int(d), ctypes.c_float(sa), ctypes.c_float(sb), kind))


def round_f64(x: float, kind: int) -> int:
    return int(lib().orc_round_f64(float(x), kind))


# --------------------------------------------------------------------------
# GEMMs
# --------------------------------------------------------------------------
def gemm_dot_i64(qa: np.ndarray, qb: np.ndarray) -> np.ndarray:
    """Exact sum_k a*b in units of 2^-18 by the naive integer triple loop."""
    qa = _c(qa, np.uint8)
    qb = _c(qb, np.uint8)
    M, K = qa.shape
    K2, N = qb.shape
    assert K == K2
    D = np.empty((M, N), dtype=np.int64)
    lib().orc_gemm_dot_i64(_p(qa), _p(qb), M, N, K, _p(D))
    return D


def gemm_rows_f64(qa, qb, rows=None):
    """Exact (sum_k a*b, sum_k |a*b|) in FP64 for the selected rows of A."""
    qa = _c(qa, np.uint8)
    qb = _c(qb, np.uint8)
    M, K = qa.shape
    N = qb.shape[1]
    rows = np.arange(M, dtype=np.int64) if rows is None else _c(rows, np.int64)
    dot = np.empty((rows.size, N), np.float64)
    sab = np.empty((rows.size, N), np.float64)
    lib().orc_gemm_rows_f64(_p(qa), _p(qb), N, K, _p(rows), rows.size, _p(dot), _p(sab))
    return dot, sab


def gemm_rows(qa, qb, sa, sb, kind, rows=None):
    """Per-tensor scaled GEMM on the selected rows of A.

    Returns (bits, exact, sumabs): bits are the once-rounded outputs (uint32
    FP32 bits or uint16 BF16 bits), exact is sa*sb*sum_k a*b in FP64 and
    sumabs is sum_k |a*b| (unscaled).  kind: F32 or BF16 (FP16 output:
    gemm_rows_fmt)."""
    if kind not in (F32, BF16):
        raise ValueError("gemm_rows rounds to FP32 or BF16 only (kind %r); use gemm_rows_fmt for FP16" % (kind,))
    qa = _c(qa, np.uint8)
    qb = _c(qb, np.uint8)
    M, K = qa.shape
    N = qb.shape[1]
    rows = np.arange(M, dtype=np.int64) if rows is None else _c(rows, np.int64)
    nr = rows.size
    exact = np.empty((nr, N), np.float64)
    sab = np.empty((nr, N), np.float64)
    o32 = np.empty((nr, N), np.uint32) if kind == F32 else np.empty(1, np.uint32)
    o16 = np.empty((nr, N), np.uint16) if kind == BF16 else np.empty(1, np.uint16)
    lib().orc_gemm_rows(_p(qa), _p(qb), ctypes.c_float(sa), ctypes.c_float(sb), N, K, _p(rows), nr,
                        kind, _p(o32), _p(o16), _p(exact), _p(sab))
    return (o32 if kind == F32 else o16), exact, sab


def gemm_sampled(qa, qb, sa, sb, kind, ii, jj):
    """Entries C[ii[s], jj[s]] one by one: (bits uint32, exact f64, sumabs f64)."""
    qa = _c(qa, np.uint8)
    qb = _c(qb, np.uint8)
    K = qa.shape[1]
    N = qb.shape[1]
    ii = _c(ii, np.int64)
    jj = _c(jj, np.int64)
    n = ii.size
    bits = np.empty(n, np.uint32)
    exact = np.empty(n, np.float64)
    sab = np.empty(n, np.float64)
    lib().orc_gemm_sampled(_p(qa), _p(qb), ctypes.c_float(sa), ctypes.c_float(sb), N, K, _p(ii), _p(jj), n,
                           kind, _p(bits), _p(exact), _p(sab))
    return bits, exact, sab


def gemm_blockscaled_rows(qa, qb, s_a, s_b, kind, rows=None):
    """Block-scaled GEMM (32x32 tile scales) on the selected rows of A.

    Returns (bits, fp64 sum, scaled sumabs).  kind: F32 or BF16."""
    if kind not in (F32, BF16):
        raise ValueError("gemm_blockscaled_rows rounds to FP32 or BF16 only (kind %r)" % (kind,))
    qa = _c(qa, np.uint8)
    qb = _c(qb, np.uint8)
    s_a = _c(s_a, np.float32)
    s_b = _c(s_b, np.float32)
    M, K = qa.shape
    N = qb.shape[1]
    assert M % 32 == 0 and N % 32 == 0 and K % 32 == 0
    assert s_a.shape == (M // 32, K // 32) and s_b.shape == (K // 32, N // 32)
    rows = np.arange(M, dtype=np.int64) if rows is None else _c(rows, np.int64)
    nr = rows.size
    exact = np.empty((nr, N), np.float64)
    sab = np.empty((nr, N), np.float64)
    o32 = np.empty((nr, N), np.uint32) if kind == F32 else np.empty(1, np.uint32)
    o16 = np.empty((nr, N), np.uint16) if kind == BF16 else np.empty(1, np.uint16)
    lib().orc_gemm_blockscaled_rows(_p(qa), _p(qb), _p(s_a), _p(s_b), N, K, _p(rows), nr, kind,
                                    _p(o32), _p(o16), _p(exact), _p(sab))
    return (o32 if kind == F32 else o16), exact, sab


def grouped_gemm_rows(qx, qw, offsets, scale_x, scale_w, kind, rows=None):
    """MoE grouped GEMM: rows [off[e], off[e+1]) of X times W[e], scaled by
    scale_x[e]*scale_w[e] (the per-tensor GEMM applied per expert group).

    qx is T x K, qw is E x K x N.  Returns (bits, exact, sumabs) for the
    selected rows (default: all T rows)."""
    qx = _c(qx, np.uint8)
    qw = _c(qw, np.uint8)
    off = np.asarray(offsets, dtype=np.int64)
    T, K = qx.shape
    E, K2, N = qw.shape
    assert K == K2 and off.size == E + 1
    rows = np.arange(T, dtype=np.int64) if rows is None else _c(rows, np.int64)
    nr = rows.size
    dt = np.uint32 if kind == F32 else np.uint16
    bits = np.zeros((nr, N), dt)
    exact = np.zeros((nr, N), np.float64)
    sab = np.zeros((nr, N), np.float64)
    expert = np.searchsorted(off, rows, side="right") - 1
    for e in range(E):
        sel = np.nonzero(expert == e)[0]
        if sel.size == 0:
            continue
        b, x, s = gemm_rows(qx, qw[e], scale_x[e], scale_w[e], kind, rows=rows[sel])
        bits[sel] = b
        exact[sel] = x
        sab[sel] = s
    return bits, exact, sab


# --------------------------------------------------------------------------
# Operand formats (E4M3, E5M2) and FP16 output
# ("FP8 GEMM in JAX with Triton for Blackwell": both FP8 formats on the matrix
# cores; its kernel sketch stores the accumulator as float16)
# --------------------------------------------------------------------------
FMT_MAX = {E4M3: 448.0, E5M2: 57344.0}


def e5m2_table() -> np.ndarray:
    """float64[256]: the value of every E5M2 code (+-Inf for 0x7C/0xFC, NaN for 0x7D-0x7F, 0xFD-0xFF)."""
    out = np.zeros(256, dtype=np.float64)
    lib().orc_e5m2_table(_p(out))
    return out


def table(fmt: int) -> np.ndarray:
    return e5m2_table() if fmt == E5M2 else e4m3_table()


def e5m2_rne_sat(v: float) -> int:
    return int(lib().orc_e5m2_rne_sat(ctypes.c_float(v)))


def convert_fmt(x: np.ndarray, fmt: int) -> np.ndarray:
    """Elementwise RNE-saturating FP32 -> codes of the format (scale 1)."""
    x = _c(x, np.float32)
    q = np.empty(x.shape, dtype=np.uint8)
    lib().orc_quantize_with_scale_fmt(_p(x), x.size, ctypes.c_float(1.0), fmt, _p(q))
    return q


def scale_from_amax_fmt(a: float, fmt: int) -> np.float32:
    return np.float32(lib().orc_scale_from_amax_fmt(ctypes.c_float(a), fmt))


def quantize_pertensor_fmt(x: np.ndarray, fmt: int):
    """Returns (codes, scale, amax) with scale = fl32(amax / format max)."""
    x = _c(x, np.float32)
    q = np.empty(x.shape, dtype=np.uint8)
    s = np.zeros(1, np.float32)
    a = np.zeros(1, np.float32)
    lib().orc_quantize_pertensor_fmt(_p(x), x.size, fmt, _p(q), _p(s), _p(a))
    return q, s[0], a[0]


def quantize_grouped_fmt(x: np.ndarray, offsets: np.ndarray, fmt: int):
    x = _c(x, np.float32)
    rows, cols = x.shape
    off = _c(offsets, np.int32)
    G = off.size - 1
    q = np.zeros(x.shape, dtype=np.uint8)
    s = np.empty(G, np.float32)
    a = np.empty(G, np.float32)
    lib().orc_quantize_grouped_fmt(_p(x), cols, _p(off), G, fmt, _p(q), _p(s), _p(a))
    return q, s, a


def round_ieee_f64(x: float, kind: int) -> int:
    """A double rounded once to FP32 / BF16 / FP16 bits (kind F32 / BF16 / F16)."""
    return int(lib().orc_round_ieee_f64(float(x), kind))


def gemm_rows_fmt(qa, qb, fa, fb, sa, sb, kind, rows=None):
    """Per-tensor scaled GEMM with operand formats fa, fb on the selected rows.

    Returns (bits, exact, sumabs): bits uint32 (FP32) or uint16 (BF16, FP16),
    rounded once from the exact 128-bit sum; exact = sa*sb*sum_k a*b in FP64;
    sumabs = sum_k |a*b| (unscaled)."""
    qa = _c(qa, np.uint8)
    qb = _c(qb, np.uint8)
    M, K = qa.shape
    N = qb.shape[1]
    assert qb.shape[0] == K
    rows = np.arange(M, dtype=np.int64) if rows is None else _c(rows, np.int64)
    nr = rows.size
    out = np.empty((nr, N), np.uint32)
    exact = np.empty((nr, N), np.float64)
    sab = np.empty((nr, N), np.float64)
    st = lib().orc_gemm_rows_fmt(_p(qa), _p(qb), fa, fb, ctypes.c_float(sa), ctypes.c_float(sb), N, K, _p(rows),
                                 nr, kind, _p(out), _p(exact), _p(sab))
    if st != 0:
        raise OverflowError("sum too large for the oracle's 128-bit scaled product")
    return (out if kind == F32 else out.astype(np.uint16)), exact, sab


# --------------------------------------------------------------------------
# Block-scale granularity T = 32 or 64 ("FP8 GEMM in JAX with Triton for
# Blackwell": 32x32 blocks in the parameter paragraph, 64x64 as the coarser
# granularity of the monitoring paragraph)
# --------------------------------------------------------------------------
def quantize_blocked_t(x: np.ndarray, T: int):
    """T x T tiles; returns (codes, tile scales float32[rows/T, cols/T])."""
    x = _c(x, np.float32)
    rows, cols = x.shape
    assert rows % T == 0 and cols % T == 0
    q = np.empty(x.shape, dtype=np.uint8)
    ts = np.empty((rows // T, cols // T), dtype=np.float32)
    lib().orc_quantize_blocked_t(_p(x), rows, cols, T, _p(q), _p(ts))
    return q, ts


def gemm_blockscaled_rows_t(qa, qb, s_a, s_b, T, kind, rows=None):
    """Block-scaled GEMM with T-deep K blocks and T x T scale tiles on the
    selected rows: (bits uint32 (FP32) / uint16 (BF16, FP16), FP64 sum,
    scaled sumabs)."""
    qa = _c(qa, np.uint8)
    qb = _c(qb, np.uint8)
    s_a = _c(s_a, np.float32)
    s_b = _c(s_b, np.float32)
    M, K = qa.shape
    N = qb.shape[1]
    assert M % T == 0 and N % T == 0 and K % T == 0
    assert s_a.shape == (M // T, K // T) and s_b.shape == (K // T, N // T)
    rows = np.arange(M, dtype=np.int64) if rows is None else _c(rows, np.int64)
    nr = rows.size
    out = np.empty((nr, N), np.uint32)
    exact = np.empty((nr, N), np.float64)
    sab = np.empty((nr, N), np.float64)
    lib().orc_gemm_blockscaled_rows_t(_p(qa), _p(qb), _p(s_a), _p(s_b), N, K, T, _p(rows), nr, kind, _p(out),
                                      _p(exact), _p(sab))
    return (out if kind == F32 else out.astype(np.uint16)), exact, sab


# --------------------------------------------------------------------------
# 32x32 block scales as powers of two (E8M0 bytes): the Blackwell page's
# 32x32 microscaling with OCP MX shared exponents
# --------------------------------------------------------------------------
def e8m0_exponent(amax: float) -> int:
    """Shared exponent floor(log2(amax)) - 8, clamped to [-127, 127]; 0 for amax 0."""
    return int(lib().orc_e8m0_exponent(ctypes.c_float(amax)))


def quantize_blocked_e8m0(x: np.ndarray):
    """32x32 tiles; returns (codes, E8M0 bytes uint8[rows/32, cols/32])."""
    x = _c(x, np.float32)
    rows, cols = x.shape
    assert rows % 32 == 0 and cols % 32 == 0
    q = np.empty(x.shape, dtype=np.uint8)
    sc = np.empty((rows // 32, cols // 32), dtype=np.uint8)
    lib().orc_quantize_blocked_e8m0(_p(x), rows, cols, _p(q), _p(sc))
    return q, sc


def gemm_blockscaled_e8m0_rows(qa, qb, s_a, s_b, kind, rows=None):
    """GEMM with E8M0 32x32 tile scales on the selected rows: (bits, FP64 sum, scaled sumabs)."""
    qa = _c(qa, np.uint8)
    qb = _c(qb, np.uint8)
    s_a = _c(s_a, np.uint8)
    s_b = _c(s_b, np.uint8)
    M, K = qa.shape
    N = qb.shape[1]
    assert M % 32 == 0 and N % 32 == 0 and K % 32 == 0
    assert s_a.shape == (M // 32, K // 32) and s_b.shape == (K // 32, N // 32)
    rows = np.arange(M, dtype=np.int64) if rows is None else _c(rows, np.int64)
    nr = rows.size
    out = np.empty((nr, N), np.uint32)
    exact = np.empty((nr, N), np.float64)
    sab = np.empty((nr, N), np.float64)
    lib().orc_gemm_blockscaled_e8m0_rows(_p(qa), _p(qb), _p(s_a), _p(s_b), N, K, _p(rows), nr, kind, _p(out),
                                         _p(exact), _p(sab))
    return (out if kind == F32 else out.astype(np.uint16)), exact, sab


# --------------------------------------------------------------------------
# 2:4 structured sparsity of the weights ("FP8 GEMM in JAX with Triton for
# Blackwell", opening section: sparsity support, ~2x at 50% sparsity)
# --------------------------------------------------------------------------
def prune_2of4(w: np.ndarray) -> np.ndarray:
    """Keep the two largest-|w| entries (ties: lower k) of every group of 4 consecutive K of each column."""
    w = _c(w, np.float32)
    K, N = w.shape
    assert K % 4 == 0
    out = np.empty_like(w)
    lib().orc_prune_2of4(_p(w), K, N, _p(out))
    return out


def compress_2of4(q: np.ndarray):
    """2:4-sparse codes (K x N, K % 32 == 0) -> (vals uint8[K/2, N], idx uint32[K/32, N])."""
    q = _c(q, np.uint8)
    K, N = q.shape
    assert K % 32 == 0
    vals = np.empty((K // 2, N), np.uint8)
    idx = np.empty((K // 32, N), np.uint32)
    lib().orc_compress_2of4(_p(q), K, N, _p(vals), _p(idx))
    return vals, idx
