"""CPU oracle for weight-only NVFP4 projection GEMV -- test infrastructure only.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP library and its Python binding
never do; the two share no code.

The arithmetic lives in ``nvfp4_oracle.c`` (plain C, fp32 quantizer, fp64
projection).  This module only builds it with gcc and marshals numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nvfp4_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-fPIC", "-shared", "-Wall", "-Wextra"]

_lib = None


def build(force: bool = True) -> str:
    """Compile ``liboracle.so`` with gcc; returns its path."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *_CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build()
    lib = ctypes.CDLL(_LIB)
    c_u8p = ctypes.POINTER(ctypes.c_uint8)
    c_f32p = ctypes.POINTER(ctypes.c_float)
    c_f64p = ctypes.POINTER(ctypes.c_double)
    c_u16p = ctypes.POINTER(ctypes.c_uint16)
    c_i64p = ctypes.POINTER(ctypes.c_int64)
    i64 = ctypes.c_int64
    lib.nvo_e2m1_value.argtypes = [ctypes.c_uint]
    lib.nvo_e2m1_value.restype = ctypes.c_double
    lib.nvo_e2m1_encode.argtypes = [ctypes.c_float]
    lib.nvo_e2m1_encode.restype = ctypes.c_uint
    lib.nvo_e4m3_value.argtypes = [ctypes.c_uint]
    lib.nvo_e4m3_value.restype = ctypes.c_float
    lib.nvo_e4m3_encode.argtypes = [ctypes.c_float]
    lib.nvo_e4m3_encode.restype = ctypes.c_uint
    lib.nvo_bf16_value.argtypes = [ctypes.c_uint16]
    lib.nvo_bf16_value.restype = ctypes.c_double
    lib.nvo_bf16_from_double.argtypes = [ctypes.c_double]
    lib.nvo_bf16_from_double.restype = ctypes.c_uint16
    lib.nvo_quantize.argtypes = [c_f32p, i64, i64, c_u8p, c_u8p, c_f32p]
    lib.nvo_quantize.restype = ctypes.c_int
    lib.nvo_dequant.argtypes = [c_u8p, c_u8p, ctypes.c_float, i64, i64, c_f32p]
    lib.nvo_dequant.restype = None
    lib.nvo_gemv.argtypes = [c_u8p, c_u8p, ctypes.c_float, i64, i64, c_u16p, ctypes.c_int,
                             c_i64p, i64, c_f64p, c_f64p, c_u16p]
    lib.nvo_gemv.restype = ctypes.c_int
    lib.nvo_gemv_f32seq.argtypes = [c_u8p, c_u8p, ctypes.c_float, i64, i64, c_u16p, ctypes.c_int,
                                    c_i64p, i64, c_f32p, c_u16p]
    lib.nvo_gemv_f32seq.restype = ctypes.c_int
    lib.nvo_gemv_dual_silu.argtypes = [c_u8p, c_u8p, ctypes.c_float, c_u8p, c_u8p, ctypes.c_float,
                                       i64, i64, c_u16p, ctypes.c_int, c_i64p, i64,
                                       c_f64p, c_f64p, c_f64p, c_f64p, c_f64p, c_u16p]
    lib.nvo_gemv_dual_silu.restype = ctypes.c_int
    lib.nvo_set_num_threads.argtypes = [ctypes.c_int]
    lib.nvo_set_num_threads.restype = None
    lib.nvo_dense_gemv.argtypes = [c_u16p, i64, i64, c_u16p, ctypes.c_int, c_i64p, i64, c_f64p, c_f64p, c_u16p]
    lib.nvo_dense_gemv.restype = None
    lib.nvo_residual_rmsnorm.argtypes = [c_u16p, c_u16p, c_u16p, i64, ctypes.c_int, ctypes.c_double, ctypes.c_int,
                                         c_u16p, c_u16p, c_f64p]
    lib.nvo_residual_rmsnorm.restype = None
    lib.nvo_e8m0_value.argtypes = [ctypes.c_uint]
    lib.nvo_e8m0_value.restype = ctypes.c_double
    lib.nvo_mx_quantize.argtypes = [c_f32p, i64, i64, c_u8p, c_u8p]
    lib.nvo_mx_quantize.restype = ctypes.c_int
    lib.nvo_mx_dequant.argtypes = [c_u8p, c_u8p, i64, i64, c_f64p]
    lib.nvo_mx_dequant.restype = None
    lib.nvo_mx_gemv.argtypes = [c_u8p, c_u8p, i64, i64, c_u16p, ctypes.c_int, c_i64p, i64, c_f64p, c_f64p, c_u16p]
    lib.nvo_mx_gemv.restype = None
    c_i8p = ctypes.POINTER(ctypes.c_int8)
    lib.nvo_f16_value.argtypes = [ctypes.c_uint16]
    lib.nvo_f16_value.restype = ctypes.c_double
    lib.nvo_w8_quantize.argtypes = [c_f32p, i64, i64, c_i8p, c_u16p]
    lib.nvo_w8_quantize.restype = ctypes.c_int
    lib.nvo_w8_dequant.argtypes = [c_i8p, c_u16p, i64, i64, c_f64p]
    lib.nvo_w8_dequant.restype = None
    lib.nvo_w8_gemv.argtypes = [c_i8p, c_u16p, i64, i64, c_u16p, ctypes.c_int, c_i64p, i64, c_f64p, c_f64p, c_u16p]
    lib.nvo_w8_gemv.restype = None
    lib.nvo_num_threads.argtypes = []
    lib.nvo_num_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a, ctype):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ---- scalar codecs -------------------------------------------------------

def e2m1_value(code: int) -> float:
    return _load().nvo_e2m1_value(int(code))


def e2m1_encode(v: float) -> int:
    return int(_load().nvo_e2m1_encode(float(v)))


def e4m3_value(byte: int) -> float:
    return float(_load().nvo_e4m3_value(int(byte)))


def e4m3_encode(v: float) -> int:
    return int(_load().nvo_e4m3_encode(float(v)))


def bf16_value(bits: int) -> float:
    return float(_load().nvo_bf16_value(int(bits)))


def bf16_from_double(v: float) -> int:
    return int(_load().nvo_bf16_from_double(float(v)))


# ---- array API -------------------------------------------------------------

def quantize(W):
    """W float32 [n, k] -> (codes uint8 [n, k/2], scales uint8 [n, k/16], s_g float32)."""
    W = _c(W, np.float32)
    n, k = W.shape
    codes = np.zeros((n, k // 2), np.uint8)
    scales = np.zeros((n, max(k // 16, 1)), np.uint8)
    sg = np.zeros(1, np.float32)
    rc = _load().nvo_quantize(_ptr(W, ctypes.c_float), n, k, _ptr(codes, ctypes.c_uint8),
                              _ptr(scales, ctypes.c_uint8), _ptr(sg, ctypes.c_float))
    if rc == -1:
        raise ValueError("oracle quantize: k must be a positive multiple of 16")
    if rc == -2:
        raise ValueError("oracle quantize: non-finite weight")
    return codes, scales, np.float32(sg[0])


def dequant(codes, scales, s_g):
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    n = codes.shape[0]
    k = codes.shape[1] * 2
    D = np.zeros((n, k), np.float32)
    _load().nvo_dequant(_ptr(codes, ctypes.c_uint8), _ptr(scales, ctypes.c_uint8),
                        float(s_g), n, k, _ptr(D, ctypes.c_float))
    return D


def _sel(sel, n):
    if sel is None:
        return None, n
    sel = _c(sel, np.int64)
    if sel.size and (sel.min() < 0 or sel.max() >= n):
        raise IndexError("selected output feature out of range")
    return sel, sel.size


def gemv(codes, scales, s_g, x_bf16, sel=None):
    """Projection in fp64.  x_bf16: uint16 [rows, k] (bf16 bit patterns).

    Returns (y fp64 [rows, nsel], sum|D*x| fp64 [rows, nsel], y_bf16 uint16 [rows, nsel]).
    """
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    x = _c(x_bf16, np.uint16)
    n = codes.shape[0]
    k = codes.shape[1] * 2
    rows = x.shape[0]
    if x.shape[1] != k or not 1 <= rows <= 64:
        raise ValueError("x must be [rows<=64, k]")
    sel, nsel = _sel(sel, n)
    y = np.zeros((rows, nsel), np.float64)
    a = np.zeros((rows, nsel), np.float64)
    yb = np.zeros((rows, nsel), np.uint16)
    st = _load().nvo_gemv(_ptr(codes, ctypes.c_uint8), _ptr(scales, ctypes.c_uint8), float(s_g), n, k,
                          _ptr(x, ctypes.c_uint16), rows, _ptr(sel, ctypes.c_int64), nsel,
                          _ptr(y, ctypes.c_double), _ptr(a, ctypes.c_double), _ptr(yb, ctypes.c_uint16))
    if st:
        raise ValueError("nvo_gemv refused the arguments")
    return y, a, yb


def gemv_f32seq(codes, scales, s_g, x_bf16, sel=None):
    """Projection as the plain fp32 definition: D = dequant in fp32, then
    y32 = sum_k D*x with one fp32 rounding per multiply and per add, ascending
    k from +0.0.  Returns (y32 float32 [rows, nsel], y_bf16 uint16 [rows, nsel])."""
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    x = _c(x_bf16, np.uint16)
    n = codes.shape[0]
    k = codes.shape[1] * 2
    rows = x.shape[0]
    if x.shape[1] != k or not 1 <= rows <= 64:
        raise ValueError("x must be [rows<=64, k]")
    sel, nsel = _sel(sel, n)
    y = np.zeros((rows, nsel), np.float32)
    yb = np.zeros((rows, nsel), np.uint16)
    st = _load().nvo_gemv_f32seq(_ptr(codes, ctypes.c_uint8), _ptr(scales, ctypes.c_uint8), float(s_g), n, k,
                                 _ptr(x, ctypes.c_uint16), rows, _ptr(sel, ctypes.c_int64), nsel,
                                 _ptr(y, ctypes.c_float), _ptr(yb, ctypes.c_uint16))
    if st:
        raise ValueError("nvo_gemv_f32seq refused the arguments")
    return y, yb


def gemv_dual_silu(gate, up, x_bf16, sel=None):
    """gate/up: (codes, scales, s_g) triples.  Returns dict of fp64 arrays
    o, g, u, abs_g, abs_u [rows, nsel] and o_bf16 uint16."""
    gc, gs, gg = _c(gate[0], np.uint8), _c(gate[1], np.uint8), float(gate[2])
    uc, us, ug = _c(up[0], np.uint8), _c(up[1], np.uint8), float(up[2])
    x = _c(x_bf16, np.uint16)
    n = gc.shape[0]
    k = gc.shape[1] * 2
    if uc.shape != gc.shape:
        raise ValueError("gate and up must have the same shape")
    rows = x.shape[0]
    if x.shape[1] != k or not 1 <= rows <= 64:
        raise ValueError("x must be [rows<=64, k]")
    sel, nsel = _sel(sel, n)
    out = {name: np.zeros((rows, nsel), np.float64) for name in ("o", "g", "u", "abs_g", "abs_u")}
    ob = np.zeros((rows, nsel), np.uint16)
    f64 = ctypes.c_double
    st = _load().nvo_gemv_dual_silu(_ptr(gc, ctypes.c_uint8), _ptr(gs, ctypes.c_uint8), gg,
                               _ptr(uc, ctypes.c_uint8), _ptr(us, ctypes.c_uint8), ug,
                               n, k, _ptr(x, ctypes.c_uint16), rows, _ptr(sel, ctypes.c_int64), nsel,
                               _ptr(out["o"], f64), _ptr(out["g"], f64), _ptr(out["u"], f64),
                               _ptr(out["abs_g"], f64), _ptr(out["abs_u"], f64),
                               _ptr(ob, ctypes.c_uint16))
    if st:
        raise ValueError("nvo_gemv_dual_silu refused the arguments")
    out["o_bf16"] = ob
    return out


def num_threads() -> int:
    return int(_load().nvo_num_threads())


def set_num_threads(n: int) -> None:
    """Threads the oracle's projections use (OpenMP over output features; the
    results do not depend on it)."""
    _load().nvo_set_num_threads(int(n))


def dense_gemv(W_bf16, x_bf16, sel=None):
    """Dense bf16 projection in fp64.  W_bf16: uint16 [n, k], x_bf16: uint16
    [rows, k] (bf16 bit patterns).  Returns (y fp64 [rows, nsel], sum|W*x| fp64
    [rows, nsel], y_bf16 uint16 [rows, nsel])."""
    W = _c(W_bf16, np.uint16)
    x = _c(x_bf16, np.uint16)
    n, k = W.shape
    rows = x.shape[0]
    if x.ndim != 2 or x.shape[1] != k or rows < 1:
        raise ValueError("x must be [rows, k]")
    sel, nsel = _sel(sel, n)
    y = np.zeros((rows, nsel), np.float64)
    a = np.zeros((rows, nsel), np.float64)
    yb = np.zeros((rows, nsel), np.uint16)
    _load().nvo_dense_gemv(_ptr(W, ctypes.c_uint16), n, k, _ptr(x, ctypes.c_uint16), rows,
                           _ptr(sel, ctypes.c_int64), nsel, _ptr(y, ctypes.c_double), _ptr(a, ctypes.c_double),
                           _ptr(yb, ctypes.c_uint16))
    return y, a, yb


def residual_rmsnorm(r_bf16, h_bf16, w_bf16, eps, gemma_offset=False):
    """Residual add + RMSNorm per row in fp64 over bf16 inputs.  r, h: uint16
    [rows, k]; w: uint16 [k].  Returns (r_out uint16 [rows, k], x uint16
    [rows, k], inv_rms fp64 [rows])."""
    r = _c(r_bf16, np.uint16)
    h = _c(h_bf16, np.uint16)
    w = _c(w_bf16, np.uint16)
    rows, k = r.shape
    if h.shape != r.shape or w.shape != (k,):
        raise ValueError("r, h must be [rows, k] and w [k]")
    ro = np.zeros((rows, k), np.uint16)
    xo = np.zeros((rows, k), np.uint16)
    inv = np.zeros(rows, np.float64)
    _load().nvo_residual_rmsnorm(_ptr(r, ctypes.c_uint16), _ptr(h, ctypes.c_uint16), _ptr(w, ctypes.c_uint16), k,
                                 rows, float(eps), int(bool(gemma_offset)), _ptr(ro, ctypes.c_uint16),
                                 _ptr(xo, ctypes.c_uint16), _ptr(inv, ctypes.c_double))
    return ro, xo, inv


# ---- MXFP4 (E2M1 codes + one E8M0 scale per 32 k) ---------------------------

def e8m0_value(byte: int) -> float:
    return float(_load().nvo_e8m0_value(int(byte)))


def mx_quantize(W):
    """W float32 [n, k] (k % 32 == 0) -> (codes uint8 [n, k/2], scales uint8 [n, k/32])."""
    W = _c(W, np.float32)
    n, k = W.shape
    codes = np.zeros((n, k // 2), np.uint8)
    scales = np.zeros((n, k // 32), np.uint8)
    st = _load().nvo_mx_quantize(_ptr(W, ctypes.c_float), n, k, _ptr(codes, ctypes.c_uint8),
                                 _ptr(scales, ctypes.c_uint8))
    if st != 0:
        raise ValueError("mx_quantize: k must be a multiple of 32 and W finite (status %d)" % st)
    return codes, scales


def mx_dequant(codes, scales):
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    n, k = codes.shape[0], codes.shape[1] * 2
    out = np.zeros((n, k), np.float64)
    _load().nvo_mx_dequant(_ptr(codes, ctypes.c_uint8), _ptr(scales, ctypes.c_uint8), n, k,
                           _ptr(out, ctypes.c_double))
    return out


def mx_gemv(codes, scales, x_bf16, sel=None):
    """MXFP4 projection in fp64: (y [rows, nsel], sum|D*x| [rows, nsel], y_bf16)."""
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    x = _c(x_bf16, np.uint16)
    n, k = codes.shape[0], codes.shape[1] * 2
    rows = x.shape[0]
    if x.shape[1] != k or scales.shape != (n, k // 32):
        raise ValueError("x must be [rows, k] and scales [n, k/32]")
    sel, nsel = _sel(sel, n)
    y = np.zeros((rows, nsel), np.float64)
    a = np.zeros((rows, nsel), np.float64)
    yb = np.zeros((rows, nsel), np.uint16)
    _load().nvo_mx_gemv(_ptr(codes, ctypes.c_uint8), _ptr(scales, ctypes.c_uint8), n, k, _ptr(x, ctypes.c_uint16),
                        rows, _ptr(sel, ctypes.c_int64), nsel, _ptr(y, ctypes.c_double), _ptr(a, ctypes.c_double),
                        _ptr(yb, ctypes.c_uint16))
    return y, a, yb


# ---- W8G32_F16S (int8 codes + one fp16 scale per 32 k) ---------------------

def f16_value(bits: int) -> float:
    return float(_load().nvo_f16_value(int(bits)))


def w8_quantize(W):
    """W float32 [n, k] (k % 32 == 0) -> (codes int8 [n, k], scales uint16 fp16 bits [n, k/32])."""
    W = _c(W, np.float32)
    n, k = W.shape
    codes = np.zeros((n, k), np.int8)
    scales = np.zeros((n, k // 32), np.uint16)
    st = _load().nvo_w8_quantize(_ptr(W, ctypes.c_float), n, k, _ptr(codes, ctypes.c_int8),
                                 _ptr(scales, ctypes.c_uint16))
    if st != 0:
        raise ValueError("w8_quantize: k must be a multiple of 32 and W finite (status %d)" % st)
    return codes, scales


def w8_dequant(codes, scales):
    codes = _c(codes, np.int8)
    scales = _c(scales, np.uint16)
    n, k = codes.shape
    out = np.zeros((n, k), np.float64)
    _load().nvo_w8_dequant(_ptr(codes, ctypes.c_int8), _ptr(scales, ctypes.c_uint16), n, k,
                           _ptr(out, ctypes.c_double))
    return out


def w8_gemv(codes, scales, x_bf16, sel=None):
    """W8G32_F16S projection in fp64: (y [rows, nsel], sum|D*x| [rows, nsel], y_bf16)."""
    codes = _c(codes, np.int8)
    scales = _c(scales, np.uint16)
    x = _c(x_bf16, np.uint16)
    n, k = codes.shape
    rows = x.shape[0]
    if x.shape[1] != k or scales.shape != (n, k // 32):
        raise ValueError("x must be [rows, k] and scales [n, k/32]")
    sel, nsel = _sel(sel, n)
    y = np.zeros((rows, nsel), np.float64)
    a = np.zeros((rows, nsel), np.float64)
    yb = np.zeros((rows, nsel), np.uint16)
    _load().nvo_w8_gemv(_ptr(codes, ctypes.c_int8), _ptr(scales, ctypes.c_uint16), n, k, _ptr(x, ctypes.c_uint16),
                        rows, _ptr(sel, ctypes.c_int64), nsel, _ptr(y, ctypes.c_double), _ptr(a, ctypes.c_double),
                        _ptr(yb, ctypes.c_uint16))
    return y, a, yb
