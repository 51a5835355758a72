"""Python binding of the W4A16 decode library (libw4a16.so, gfx950).

The functions carry the C-ABI names of include/w4a16.h and only marshal
arguments: torch tensors become device pointers and the current HIP stream;
every step of the computation runs in the library's kernels.  If the library
is not built, importing works but every call raises.

Tensor conventions (all on the same GPU, contiguous):
  x, scales, biases, bf16 outputs : torch.bfloat16
  qw                              : torch.int32 (the uint32 words, bit for bit)
  ids, argmax, rows               : torch.int32
  fp32 outputs                    : torch.float32
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# W4A16_LIB: another build of the same library (the sanitizer test loads a
# host-only build instrumented with ASan/UBSan through it)
LIB_PATH = os.environ.get("W4A16_LIB", os.path.join(_HERE, "libw4a16.so"))

OUT_BF16 = 0
OUT_F32 = 1
GROUP = 64
MAX_M = 8
MAX_PREFILL_M = 65536   # W4A16_MAX_PREFILL_M
MAX_GROUP = 8           # W4A16_MAX_GROUP
MAX_N = 1 << 30         # W4A16_MAX_N
MAX_K = 1 << 24         # W4A16_MAX_K

STATUS = {0: "OK", 1: "ERR_NULL", 2: "ERR_SHAPE", 3: "ERR_UNSUPPORTED", 4: "ERR_ALIGN",
          5: "ERR_WORKSPACE", 6: "ERR_HIP", 7: "ERR_SCRATCH"}
NOALLOC_SCRATCH_BYTES = 1 << 20   # W4A16_NOALLOC_SCRATCH_BYTES

EXPORTS = ("w4a16_matmul", "w4a16_matmul_geglu", "w4a16_matmul_prefill", "w4a16_matmul_grouped", "w4a16_matmul_id", "w4a16_lmhead_argmax_workspace_bytes",
           "w4a16_lmhead_argmax", "w4a16_lmhead_argmax_noalloc", "w4a16_dequant", "w4a16_gather_rows", "w4a16_pack", "w4a16_status_str",
           "w4a16_abi_version", "w4a16_schedule_name")


class Matrix(ctypes.Structure):
    """w4a16_matrix_t: one matrix of a grouped product."""
    _fields_ = [("qw", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("biases", ctypes.c_void_p),
                ("y", ctypes.c_void_p), ("N", ctypes.c_int)]


class W4A16Error(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)} ({_status_str(status)})")


_lib = None
_vp = ctypes.c_void_p
_int = ctypes.c_int
_size = ctypes.c_size_t


def lib() -> ctypes.CDLL:
    """Load libw4a16.so; raises if it is not built (there is no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        L.w4a16_matmul.restype = _int
        L.w4a16_matmul.argtypes = [_vp, _vp, _vp, _vp, _vp, _int, _int, _int, _int, _int, _vp]
        L.w4a16_matmul_geglu.restype = _int
        L.w4a16_matmul_geglu.argtypes = [_vp, _vp, _vp, _vp, _vp, _int, _int, _int, _int, _int, _vp]
        L.w4a16_matmul_prefill.restype = _int
        L.w4a16_matmul_prefill.argtypes = [_vp, _vp, _vp, _vp, _vp, _int, _int, _int, _int, _int, _vp]
        L.w4a16_matmul_grouped.restype = _int
        L.w4a16_matmul_grouped.argtypes = [_vp, ctypes.POINTER(Matrix), _int, _int, _int, _int, _int, _vp]
        L.w4a16_matmul_id.restype = _int
        L.w4a16_matmul_id.argtypes = [_vp, ctypes.c_int64, _vp, _vp, _vp, _vp, _vp, _int, _int, _int, _int, _int,
                                      _int, _int, _vp]
        L.w4a16_lmhead_argmax_workspace_bytes.restype = _size
        L.w4a16_lmhead_argmax_workspace_bytes.argtypes = [_int, _int, _int, _int]
        L.w4a16_lmhead_argmax.restype = _int
        L.w4a16_lmhead_argmax.argtypes = [_vp, _vp, _vp, _vp, _vp, _int, _vp, _vp, _size, _int, _int,
                                          _int, _int, _vp]
        L.w4a16_lmhead_argmax_noalloc.restype = _int
        L.w4a16_lmhead_argmax_noalloc.argtypes = [_vp, _vp, _vp, _vp, _vp, _int, _vp, _int, _int, _int, _int, _vp]
        L.w4a16_dequant.restype = _int
        L.w4a16_dequant.argtypes = [_vp, _vp, _vp, _vp, _int, _vp, _int, _int, _int, _vp]
        L.w4a16_gather_rows.restype = _int
        L.w4a16_gather_rows.argtypes = [_vp, _vp, _vp, _vp, _int, _vp, _int, _int, _int, _vp]
        L.w4a16_pack.restype = _int
        L.w4a16_pack.argtypes = [_vp, _vp, _int, _int, _vp]
        L.w4a16_status_str.restype = ctypes.c_char_p
        L.w4a16_status_str.argtypes = [_int]
        L.w4a16_abi_version.restype = _int
        L.w4a16_abi_version.argtypes = []
        L.w4a16_schedule_name.restype = ctypes.c_char_p
        L.w4a16_schedule_name.argtypes = [_int, _int, _int, _int]
        _lib = L
    return _lib


def _status_str(s: int) -> str:
    try:
        return lib().w4a16_status_str(s).decode()
    except Exception:
        return "?"


def _check(status: int, what: str) -> None:
    if status != 0:
        raise W4A16Error(status, what)


def _ptr(t):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _on_device(*ts, contiguous=True) -> None:
    """Every tensor on the same GPU (and contiguous unless told otherwise);
    checked after the shapes, before any pointer reaches the library."""
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("tensors must be on the GPU")
        if contiguous and not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"tensors must be on one device ({dev} and {t.device})")


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _out_code(t) -> int:
    if t.dtype == torch.bfloat16:
        return OUT_BF16
    if t.dtype == torch.float32:
        return OUT_F32
    raise TypeError("outputs are torch.bfloat16 or torch.float32")


def _dtype(t, want, name):
    if t.dtype != want:
        raise TypeError(f"{name} must be {want}, got {t.dtype}")


def _shape(t, want, name):
    if tuple(t.shape) != tuple(want):
        raise ValueError(f"{name} must have shape {list(want)}, got {list(t.shape)}")


def _activations(x, name="x"):
    _dtype(x, torch.bfloat16, name)
    if x.dim() != 2:
        raise ValueError(f"{name} must be 2-D [M, K], got {list(x.shape)}")
    return x.shape


def _weights(qw, scales, biases, N, K, group, lead=()):
    """qw int32 [*lead, N, K/8]; scales, biases bf16 [*lead, N, K/group]."""
    _dtype(qw, torch.int32, "qw")
    _dtype(scales, torch.bfloat16, "scales")
    _dtype(biases, torch.bfloat16, "biases")
    if group <= 0 or K % group != 0:
        raise ValueError(f"K = {K} is not a multiple of the group {group}")
    _shape(qw, (*lead, N, K // 8), "qw")
    _shape(scales, (*lead, N, K // group), "scales")
    _shape(biases, (*lead, N, K // group), "biases")


# ---- C-ABI entry points ---------------------------------------------------------

def w4a16_matmul(x, qw, scales, biases, y, group: int = GROUP, stream=None) -> None:
    """y[M,N] = x[M,K] . W^T  (W = packed qw [N,K/8] with bf16 scales/biases [N,K/group])."""
    M, K = _activations(x)
    _dtype(qw, torch.int32, "qw")
    N = qw.shape[0] if qw.dim() == 2 else -1
    _weights(qw, scales, biases, N, K, group)
    code = _out_code(y)
    _shape(y, (M, N), "y")
    _on_device(x, qw, scales, biases, y)
    _check(lib().w4a16_matmul(_ptr(x), _ptr(qw), _ptr(scales), _ptr(biases), _ptr(y), code,
                              M, N, K, group, _stream(stream)), "w4a16_matmul")


def w4a16_matmul_geglu(x, qw, scales, biases, h, group: int = GROUP, stream=None) -> None:
    """h[M,I] = GELU(x . Wg^T) * (x . Wu^T) for a fused gate+up matrix qw [2I, K/8]
    (gate rows first), exact GELU g * Phi(g)."""
    M, K = _activations(x)
    _dtype(qw, torch.int32, "qw")
    if qw.dim() != 2 or qw.shape[0] % 2:
        raise ValueError("a fused gate+up matrix is 2-D with an even number of rows")
    I = qw.shape[0] // 2
    _weights(qw, scales, biases, 2 * I, K, group)
    code = _out_code(h)
    _shape(h, (M, I), "h")
    _on_device(x, qw, scales, biases, h)
    _check(lib().w4a16_matmul_geglu(_ptr(x), _ptr(qw), _ptr(scales), _ptr(biases), _ptr(h), code,
                                    M, I, K, group, _stream(stream)), "w4a16_matmul_geglu")


def w4a16_matmul_prefill(x, qw, scales, biases, y, group: int = GROUP, stream=None) -> None:
    """y[M,N] = x[M,K] . W^T for prefill-sized M (matrix cores; not bitwise equal to w4a16_matmul).

    Up to 16 rows: the decode kernels on chunks of 8 rows (their bound and
    results).  Small grids: bounded on sum |w x|.  The LDS-tiled form (M > 64
    and at least 96 output tiles of 128 x 128, or M > 40 and 160..255 of
    64 x 128) uses the rearranged per-group sums
    and is bounded on sum |s x (q - 8)| + |(b + 8 s) x|, which is weaker where
    the dequantized weights cancel."""
    M, K = _activations(x)
    _dtype(qw, torch.int32, "qw")
    N = qw.shape[0] if qw.dim() == 2 else -1
    _weights(qw, scales, biases, N, K, group)
    code = _out_code(y)
    _shape(y, (M, N), "y")
    _on_device(x, qw, scales, biases, y)
    _check(lib().w4a16_matmul_prefill(_ptr(x), _ptr(qw), _ptr(scales), _ptr(biases), _ptr(y), code,
                                      M, N, K, group, _stream(stream)), "w4a16_matmul_prefill")


def w4a16_matmul_grouped(x, mats, group: int = GROUP, stream=None) -> None:
    """mats: sequence of (qw, scales, biases, y) sharing K and x; y_i[M,N_i] = x . W_i^T."""
    M, K = _activations(x)
    if len(mats) > MAX_GROUP:
        raise ValueError(f"at most {MAX_GROUP} matrices per grouped call")
    arr = (Matrix * max(1, len(mats)))()
    code = None
    for i, (qw, s, b, y) in enumerate(mats):
        _dtype(qw, torch.int32, f"mats[{i}].qw")
        N = qw.shape[0] if qw.dim() == 2 else -1
        _weights(qw, s, b, N, K, group)
        c = _out_code(y)
        if code is not None and c != code:
            raise TypeError("all outputs of a grouped product share one dtype")
        code = c
        _shape(y, (M, N), f"mats[{i}].y")
    _on_device(x, *(t for m in mats for t in m))
    for i, (qw, s, b, y) in enumerate(mats):
        arr[i] = Matrix(_ptr(qw), _ptr(s), _ptr(b), _ptr(y), qw.shape[0])
    _check(lib().w4a16_matmul_grouped(_ptr(x), arr, len(mats), OUT_BF16 if code is None else code, M, K, group,
                                      _stream(stream)), "w4a16_matmul_grouped")


def w4a16_matmul_id(x, qw, scales, biases, ids, y, group: int = GROUP, stream=None) -> None:
    """y[M,top_k,N]: slot (m,j) uses expert ids[m,j] of the stack qw [E,N,K/8].

    x [M, K] is shared by a token's slots (x_slot_stride 0); x [M, top_k, K]
    gives one row per slot (x_slot_stride = x.stride(1), so a row-padded view
    of a larger buffer works as well as a contiguous tensor)."""
    _dtype(x, torch.bfloat16, "x")
    _dtype(ids, torch.int32, "ids")
    if ids.dim() != 2:
        raise ValueError(f"ids must be 2-D [M, top_k], got {list(ids.shape)}")
    M, top_k = ids.shape
    _dtype(qw, torch.int32, "qw")
    if qw.dim() != 3:
        raise ValueError(f"qw must be 3-D [E, N, K/8], got {list(qw.shape)}")
    E, N = qw.shape[0], qw.shape[1]
    K = x.shape[-1]
    if x.dim() == 2:
        _shape(x, (M, K), "x")
        stride = 0
    elif x.dim() == 3:
        _shape(x, (M, top_k, K), "x")
        if x.stride(2) != 1 or x.stride(0) != top_k * x.stride(1) or x.stride(1) < K:
            raise ValueError("a per-slot x must have unit stride along K, rows at least K apart, "
                             "and tokens top_k rows apart")
        stride = x.stride(1)
    else:
        raise ValueError(f"x must be [M, K] or [M, top_k, K], got {list(x.shape)}")
    _weights(qw, scales, biases, N, K, group, lead=(E,))
    code = _out_code(y)
    _shape(y, (M, top_k, N), "y")
    _on_device(x, contiguous=(stride == 0))
    _on_device(qw, scales, biases, ids, y)
    if x.device != qw.device:
        raise ValueError("tensors must be on one device")
    _check(lib().w4a16_matmul_id(_ptr(x), stride, _ptr(qw), _ptr(scales), _ptr(biases),
                                 _ptr(ids), _ptr(y), code, M, top_k, E, N, K, group,
                                 _stream(stream)), "w4a16_matmul_id")


def w4a16_lmhead_argmax_workspace_bytes(M: int, N: int, K: int, group: int = GROUP) -> int:
    return int(lib().w4a16_lmhead_argmax_workspace_bytes(M, N, K, group))


def w4a16_lmhead_argmax(x, qw, scales, biases, logits, argmax, workspace, group: int = GROUP,
                        stream=None, out_dtype=None) -> None:
    """argmax[M] (int32) of x . W^T, optional logits [M,N]; workspace: a uint8 device tensor."""
    M, K = _activations(x)
    _dtype(qw, torch.int32, "qw")
    N = qw.shape[0] if qw.dim() == 2 else -1
    _weights(qw, scales, biases, N, K, group)
    _dtype(argmax, torch.int32, "argmax")
    _shape(argmax, (M,), "argmax")
    if logits is not None:
        code = _out_code(logits)
        _shape(logits, (M, N), "logits")
    else:
        code = OUT_BF16 if out_dtype is None else out_dtype
    _dtype(workspace, torch.uint8, "workspace")
    _on_device(x, qw, scales, biases, logits, argmax, workspace)
    _check(lib().w4a16_lmhead_argmax(_ptr(x), _ptr(qw), _ptr(scales), _ptr(biases), _ptr(logits), code,
                                     _ptr(argmax), _ptr(workspace), workspace.numel(),
                                     M, N, K, group, _stream(stream)), "w4a16_lmhead_argmax")


def w4a16_lmhead_argmax_noalloc(x, qw, scales, biases, logits, argmax, group: int = GROUP, stream=None,
                                out_dtype=None) -> None:
    """w4a16_lmhead_argmax with the library's built-in scratch instead of a
    workspace: allocates nothing (calls overlapping on one GPU race)."""
    M, K = _activations(x)
    _dtype(qw, torch.int32, "qw")
    N = qw.shape[0] if qw.dim() == 2 else -1
    _weights(qw, scales, biases, N, K, group)
    _dtype(argmax, torch.int32, "argmax")
    _shape(argmax, (M,), "argmax")
    if logits is not None:
        code = _out_code(logits)
        _shape(logits, (M, N), "logits")
    else:
        code = OUT_BF16 if out_dtype is None else out_dtype
    _on_device(x, qw, scales, biases, logits, argmax)
    _check(lib().w4a16_lmhead_argmax_noalloc(_ptr(x), _ptr(qw), _ptr(scales), _ptr(biases), _ptr(logits), code,
                                             _ptr(argmax), M, N, K, group, _stream(stream)),
           "w4a16_lmhead_argmax_noalloc")


def _rows(rows, name="rows"):
    _dtype(rows, torch.int32, name)
    if rows.dim() != 1:
        raise ValueError(f"{name} must be 1-D, got {list(rows.shape)}")
    return rows.numel()


def w4a16_dequant(qw, scales, biases, out, rows=None, group: int = GROUP, stream=None) -> None:
    """out[R,K] (fp32) = dequantized rows (rows=None: all N rows)."""
    _dtype(qw, torch.int32, "qw")
    if qw.dim() != 2:
        raise ValueError(f"qw must be 2-D [N, K/8], got {list(qw.shape)}")
    N, K = qw.shape[0], qw.shape[1] * 8
    _weights(qw, scales, biases, N, K, group)
    R = _rows(rows) if rows is not None else N
    _dtype(out, torch.float32, "out")
    _shape(out, (R, K), "out")
    _on_device(qw, scales, biases, rows, out)
    _check(lib().w4a16_dequant(_ptr(qw), _ptr(scales), _ptr(biases), _ptr(rows), R, _ptr(out), N, K, group,
                               _stream(stream)), "w4a16_dequant")


def w4a16_gather_rows(qw, scales, biases, rows, out, group: int = GROUP, stream=None) -> None:
    """out[R,K] (bf16) = rows[R] of the packed table, dequantized and rounded to bf16."""
    _dtype(qw, torch.int32, "qw")
    if qw.dim() != 2:
        raise ValueError(f"qw must be 2-D [N, K/8], got {list(qw.shape)}")
    N, K = qw.shape[0], qw.shape[1] * 8
    _weights(qw, scales, biases, N, K, group)
    R = _rows(rows)
    _dtype(out, torch.bfloat16, "out")
    _shape(out, (R, K), "out")
    _on_device(qw, scales, biases, rows, out)
    _check(lib().w4a16_gather_rows(_ptr(qw), _ptr(scales), _ptr(biases), _ptr(rows), R, _ptr(out), N, K,
                                   group, _stream(stream)), "w4a16_gather_rows")


def w4a16_pack(codes, qw, stream=None) -> None:
    """codes uint8 [N,K] -> qw int32 [N,K/8] (first code in the lowest nibble)."""
    _dtype(codes, torch.uint8, "codes")
    _dtype(qw, torch.int32, "qw")
    if codes.dim() != 2 or codes.shape[1] % 8:
        raise ValueError(f"codes must be 2-D [N, K] with K a multiple of 8, got {list(codes.shape)}")
    N, K = codes.shape
    _shape(qw, (N, K // 8), "qw")
    _on_device(codes, qw)
    _check(lib().w4a16_pack(_ptr(codes), _ptr(qw), N, K, _stream(stream)), "w4a16_pack")


def w4a16_status_str(status: int) -> str:
    return _status_str(status)


def w4a16_abi_version() -> int:
    return int(lib().w4a16_abi_version())


def w4a16_schedule_name(M: int, N: int, K: int, group: int = GROUP) -> str:
    return lib().w4a16_schedule_name(M, N, K, group).decode()


# ---- allocating conveniences (torch allocates; the library computes) ------------

def matmul(x, qw, scales, biases, out_dtype=torch.bfloat16, group: int = GROUP, stream=None):
    y = torch.empty((x.shape[0], qw.shape[0]), dtype=out_dtype, device=x.device)
    w4a16_matmul(x, qw, scales, biases, y, group=group, stream=stream)
    return y


def matmul_prefill(x, qw, scales, biases, out_dtype=torch.bfloat16, group: int = GROUP, stream=None):
    y = torch.empty((x.shape[0], qw.shape[0]), dtype=out_dtype, device=x.device)
    w4a16_matmul_prefill(x, qw, scales, biases, y, group=group, stream=stream)
    return y


def matmul_id(x, qw, scales, biases, ids, out_dtype=torch.bfloat16, group: int = GROUP, stream=None):
    y = torch.empty((ids.shape[0], ids.shape[1], qw.shape[1]), dtype=out_dtype, device=x.device)
    w4a16_matmul_id(x, qw, scales, biases, ids, y, group=group, stream=stream)
    return y


def lmhead_argmax(x, qw, scales, biases, want_logits=True, out_dtype=torch.bfloat16, group: int = GROUP,
                  stream=None):
    M, K = x.shape
    N = qw.shape[0]
    ws = torch.empty(max(1, w4a16_lmhead_argmax_workspace_bytes(M, N, K, group)), dtype=torch.uint8, device=x.device)
    am = torch.empty(M, dtype=torch.int32, device=x.device)
    logits = torch.empty((M, N), dtype=out_dtype, device=x.device) if want_logits else None
    w4a16_lmhead_argmax(x, qw, scales, biases, logits, am, ws, group=group, stream=stream,
                        out_dtype=OUT_F32 if out_dtype == torch.float32 else OUT_BF16)
    return am, logits


def dequant(qw, scales, biases, rows=None, group: int = GROUP, stream=None):
    R = rows.numel() if rows is not None else qw.shape[0]
    out = torch.empty((R, qw.shape[1] * 8), dtype=torch.float32, device=qw.device)
    w4a16_dequant(qw, scales, biases, out, rows=rows, group=group, stream=stream)
    return out


def gather_rows(qw, scales, biases, rows, group: int = GROUP, stream=None):
    out = torch.empty((rows.numel(), qw.shape[1] * 8), dtype=torch.bfloat16, device=qw.device)
    w4a16_gather_rows(qw, scales, biases, rows, out, group=group, stream=stream)
    return out


def pack(codes, stream=None):
    qw = torch.empty((codes.shape[0], codes.shape[1] // 8), dtype=torch.int32, device=codes.device)
    w4a16_pack(codes, qw, stream=stream)
    return qw
