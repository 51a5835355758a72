"""CPU oracle for the W4A16 group-affine product -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It wraps ``liboracle.so`` (built from
``oracle.c`` by ``__graft_entry__.build()``) with ctypes and numpy; every
number it returns comes from that plain C code, which shares nothing with the
HIP library.  See ``oracle.c`` for what is computed and which passages of the
pages each step follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# Tests may point this at a deliberately broken build to show the pins catch it.
LIB_PATH = os.environ.get("W4A16_ORACLE_LIB", os.path.join(_HERE, "liboracle.so"))
SRC_PATH = os.path.join(_HERE, "oracle.c")

# No contraction, no fast-math: the C source's fmaf and fp64 sums are what run.
CFLAGS = ["-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math"]


def build(verbose: bool = False) -> str:
    """Compile oracle.c into liboracle.so with gcc (always recompiles)."""
    cmd = ["gcc", *CFLAGS, "-o", LIB_PATH, SRC_PATH, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    return LIB_PATH


_lib = None
_u16p = ctypes.POINTER(ctypes.c_uint16)
_u32p = ctypes.POINTER(ctypes.c_uint32)
_u8p = ctypes.POINTER(ctypes.c_uint8)
_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)
_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_i64 = ctypes.c_int64


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        L.orc_bf16_to_f32.restype = ctypes.c_float
        L.orc_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.orc_f64_to_bf16.restype = ctypes.c_uint16
        L.orc_f64_to_bf16.argtypes = [ctypes.c_double]
        L.orc_round_bf16.restype = None
        L.orc_round_bf16.argtypes = [_f64p, _i64, _u16p]
        L.orc_pack8.restype = ctypes.c_uint32
        L.orc_pack8.argtypes = [_u8p]
        L.orc_unpack.restype = ctypes.c_int
        L.orc_unpack.argtypes = [ctypes.c_uint32, ctypes.c_int]
        L.orc_pack_rows.restype = ctypes.c_int
        L.orc_pack_rows.argtypes = [_u8p, _i64, _i64, _u32p]
        L.orc_unpack_rows.restype = ctypes.c_int
        L.orc_unpack_rows.argtypes = [_u32p, _i64, _i64, _u8p]
        L.orc_dequant.restype = ctypes.c_float
        L.orc_dequant.argtypes = [ctypes.c_uint16, ctypes.c_uint16, ctypes.c_int]
        L.orc_dequant_rows.restype = ctypes.c_int
        L.orc_dequant_rows.argtypes = [_u32p, _u16p, _u16p, _i64, _i64, _i64, _i32p, _i64, _f32p]
        L.orc_qmm.restype = ctypes.c_int
        L.orc_qmm.argtypes = [_u16p, _u32p, _u16p, _u16p, _i64, _i64, _i64, _i64, _i32p, _i64,
                              _f64p, _f64p]
        L.orc_qmm_id.restype = ctypes.c_int
        L.orc_qmm_id.argtypes = [_u16p, ctypes.c_int, _u32p, _u16p, _u16p, _i32p, _i64, _i64, _i64,
                                 _i64, _i64, _i64, _f64p, _f64p]
        L.orc_argmax.restype = ctypes.c_int
        L.orc_argmax.argtypes = [_f64p, _i64, _i64p, _f64p]
        L.orc_geglu.restype = ctypes.c_int
        L.orc_geglu.argtypes = [_f64p, _f64p, _i64, _f64p]
        _lib = L
    return _lib


def _ptr(a: np.ndarray, t):
    return a.ctypes.data_as(t)


def _c(a: np.ndarray, dtype) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    return np.ascontiguousarray(a)


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (rc={rc})")


# ---- scalar helpers ----------------------------------------------------------

def bf16_to_f32(bits) -> np.ndarray:
    """bf16 bit patterns -> float32 values (elementwise through the C oracle)."""
    b = np.asarray(bits, dtype=np.uint16)
    f = lib().orc_bf16_to_f32
    return np.array([f(int(v)) for v in b.ravel()], dtype=np.float32).reshape(b.shape)


def f64_to_bf16(y) -> np.ndarray:
    """Round fp64 values to bf16 bits (nearest-even, one rounding)."""
    y = np.ascontiguousarray(np.asarray(y, dtype=np.float64))
    out = np.empty(y.shape, dtype=np.uint16)
    lib().orc_round_bf16(_ptr(y, _f64p), y.size, _ptr(out, _u16p))
    return out


def pack8(codes) -> int:
    c = np.ascontiguousarray(np.asarray(codes, dtype=np.uint8))
    assert c.size == 8
    return int(lib().orc_pack8(_ptr(c, _u8p)))


def unpack(word: int, i: int) -> int:
    return int(lib().orc_unpack(ctypes.c_uint32(word), i))


def pack_rows(codes: np.ndarray) -> np.ndarray:
    c = _c(codes, np.uint8)
    N, K = c.shape
    qw = np.empty((N, K // 8), dtype=np.uint32)
    _check(lib().orc_pack_rows(_ptr(c, _u8p), N, K, _ptr(qw, _u32p)), "pack_rows")
    return qw


def unpack_rows(qw: np.ndarray, K: int) -> np.ndarray:
    q = _c(qw, np.uint32)
    N = q.shape[0]
    codes = np.empty((N, K), dtype=np.uint8)
    _check(lib().orc_unpack_rows(_ptr(q, _u32p), N, K, _ptr(codes, _u8p)), "unpack_rows")
    return codes


def dequant(s_bits: int, b_bits: int, q: int) -> np.float32:
    return np.float32(lib().orc_dequant(s_bits, b_bits, q))


def dequant_rows(qw, scales, biases, K: int, group: int = 64, rows=None) -> np.ndarray:
    q = _c(qw, np.uint32)
    s = _c(scales, np.uint16)
    b = _c(biases, np.uint16)
    N = q.shape[0]
    if rows is None:
        R, rp = N, None
    else:
        r = _c(np.asarray(rows, dtype=np.int32), np.int32)
        R, rp = r.size, _ptr(r, _i32p)
    out = np.empty((R, K), dtype=np.float32)
    _check(lib().orc_dequant_rows(_ptr(q, _u32p), _ptr(s, _u16p), _ptr(b, _u16p), N, K, group,
                                  rp, R, _ptr(out, _f32p)), "dequant_rows")
    return out


def qmm(x, qw, scales, biases, group: int = 64, rows=None):
    """Return (y64, absy) with shape [M, R]: fp64 sums and sum of |x*w|."""
    xx = _c(x, np.uint16)
    if xx.ndim == 1:
        xx = xx[None, :]
    M, K = xx.shape
    q = _c(qw, np.uint32)
    s = _c(scales, np.uint16)
    b = _c(biases, np.uint16)
    N = q.shape[0]
    if rows is None:
        R, rp, keep = N, None, None
    else:
        keep = _c(np.asarray(rows, dtype=np.int32), np.int32)
        R, rp = keep.size, _ptr(keep, _i32p)
    y = np.empty((M, R), dtype=np.float64)
    a = np.empty((M, R), dtype=np.float64)
    _check(lib().orc_qmm(_ptr(xx, _u16p), _ptr(q, _u32p), _ptr(s, _u16p), _ptr(b, _u16p), M, N, K,
                         group, rp, R, _ptr(y, _f64p), _ptr(a, _f64p)), "qmm")
    return y, a


def qmm_id(x, qw, scales, biases, ids, x_per_slot: bool = False, group: int = 64):
    """Routed product: returns (y64, absy) with shape [M, top_k, N]."""
    xx = _c(x, np.uint16)
    q = _c(qw, np.uint32)
    s = _c(scales, np.uint16)
    b = _c(biases, np.uint16)
    i = _c(ids, np.int32)
    M, top_k = i.shape
    E, N = q.shape[0], q.shape[1]
    K = xx.shape[-1]
    y = np.empty((M, top_k, N), dtype=np.float64)
    a = np.empty((M, top_k, N), dtype=np.float64)
    _check(lib().orc_qmm_id(_ptr(xx, _u16p), int(bool(x_per_slot)), _ptr(q, _u32p), _ptr(s, _u16p),
                            _ptr(b, _u16p), _ptr(i, _i32p), M, top_k, E, N, K, group,
                            _ptr(y, _f64p), _ptr(a, _f64p)), "qmm_id")
    return y, a


def argmax(y) -> tuple[int, float]:
    """(index, top-2 gap) of a 1-D fp64 vector; ties keep the lowest index."""
    v = np.ascontiguousarray(np.asarray(y, dtype=np.float64))
    best = ctypes.c_int64(0)
    gap = ctypes.c_double(0.0)
    _check(lib().orc_argmax(_ptr(v, _f64p), v.size, ctypes.byref(best), ctypes.byref(gap)), "argmax")
    return int(best.value), float(gap.value)


def geglu_values(gate, up) -> np.ndarray:
    """h = GELU(gate) * up elementwise in fp64 (exact GELU: g * Phi(g))."""
    g = _c(np.asarray(gate, dtype=np.float64), np.float64)
    u = _c(np.broadcast_to(np.asarray(up, dtype=np.float64), g.shape), np.float64)
    h = np.empty_like(g)
    _check(lib().orc_geglu(_ptr(g, _f64p), _ptr(u, _f64p), g.size, _ptr(h, _f64p)), "geglu")
    return h


def geglu(x, qw, scales, biases, I: int, group: int = 64, cols=None):
    """Gated MLP activation on a fused [2I, K] gate+up matrix (gate rows 0..I-1,
    up rows I..2I-1): h[m, j] = GELU(gate[m, j]) * up[m, j] for j in cols (all
    I when None).  Returns (h, gate, gate_abs, up, up_abs), each [M, len(cols)]:
    the fp64 sums of the two products and their sum |x w| error scales."""
    js = np.arange(I, dtype=np.int32) if cols is None else np.asarray(cols, dtype=np.int32)
    g, ga = qmm(x, qw, scales, biases, group, rows=js)
    u, ua = qmm(x, qw, scales, biases, group, rows=js + I)
    return geglu_values(g, u), g, ga, u, ua
