"""Thin Python binding of libfp8sg.so (the C ABI in include/fp8sg.h).

Argument marshalling only: every function checks that its torch tensors are
what the C call will read or write (on the GPU, contiguous, of the expected
dtype and at least as large as the sizes passed imply), hands their device
pointers to the C entry point of the same name and raises ``Fp8Error`` on a
non-zero status.  All arithmetic runs in the library's HIP kernels.  There is
no fallback: if the library is missing the import fails loudly.

Workspaces.  The amax-producing calls take ``workspace``: a device buffer of
``WORKSPACE_BYTES`` from :func:`workspace` (allocated by torch, prepared by
``fp8_workspace_init``).  Left as ``None``, a fresh workspace is taken from
torch's allocator for that one call, on the call's stream, which costs one
small fill kernel; callers that time or capture the path pass their own.
"""
from __future__ import annotations

import ctypes
import os

import torch

E4M3 = 0
E5M2 = 1
SCALE_TENSOR = 0
SCALE_BLOCK_1x128 = 1
SCALE_BLOCK_128x128 = 2
SCALE_MX_1x32 = 3

# FP8_WORKSPACE_BYTES of include/fp8sg.h
WORKSPACE_BYTES = 295552

STATUS = {0: "FP8_OK", 1: "FP8_ERR_NULL", 2: "FP8_ERR_SHAPE", 3: "FP8_ERR_ALIGN",
          4: "FP8_ERR_UNSUPPORTED", 5: "FP8_ERR_HIP"}

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfp8sg.so")


class Fp8Error(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} returned {STATUS.get(status, status)}")
        self.status = status


class Operand(ctypes.Structure):
    """fp8_operand_t: FP8 data [rows][K], format, scaling and scale_inv."""
    _fields_ = [("data", ctypes.c_void_p), ("fmt", ctypes.c_int32),
                ("scaling", ctypes.c_int32), ("scale_inv", ctypes.c_void_p)]


_lib = None


def lib():
    """Load libfp8sg.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m scaled_fp8_gemm_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        sig = {
            "fp8_workspace_init": [vp, i32, vp],
            "fp8_amax": [vp, i64, i64, i32, vp, vp, vp, vp, vp],
            "fp8_quantize_tensor": [vp, i64, i64, i32, vp, vp, vp, vp, vp, vp],
            "fp8_amax_f32": [vp, i64, i64, i32, vp, vp, vp, vp, vp],
            "fp8_quantize_tensor_current": [vp, i64, i64, i32, vp, vp, vp, vp, vp, vp, vp],
            "fp8_quantize_tensor_current_noalloc": [vp, i64, i64, i32, vp, vp, vp, vp, vp, vp],
            "fp8_quantize_pair_current": [vp, i64, i64, i32, vp, vp, vp, vp,
                                          vp, i64, i64, i32, vp, vp, vp, vp, vp, vp],
            "fp8_quantize_tensor_f32": [vp, i64, i64, i32, vp, vp, vp, vp, vp, vp],
            "fp8_amax_history_update": [vp, i32, i64, vp, i32, vp, vp, vp],
            "fp8_quantize_block": [vp, i64, i64, i32, i32, i32, vp, vp, vp],
            "fp8_quantize_mx": [vp, i64, i64, i32, vp, vp, vp],
            "fp8_quantize_block_t": [vp, i64, i64, i32, i32, vp, vp, vp, vp, vp],
            "fp8_quantize_mx_t": [vp, i64, i64, i32, vp, vp, vp, vp, vp],
            "fp8_gemm_fprop": [vp, vp, i64, i64, i64, vp, vp],
            "fp8_gemm_dgrad": [vp, vp, i64, i64, i64, vp, vp],
            "fp8_gemm_wgrad": [vp, vp, i64, i64, i64, vp, vp],
            "fp8_gemm_wgrad_f32": [vp, vp, i64, i64, i64, vp, i32, vp],
            "fp8_gemm_fprop_fused": [vp, vp, i64, i64, i64, vp, i32, vp, vp, vp, vp, vp],
            "fp8_convert_f32": [vp, i64, i32, vp, vp],
        }
        for name, args in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        L.fp8_status_string.argtypes = [ctypes.c_int]
        L.fp8_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


# ------------------------------------------------------------ marshalling
_BF16 = (torch.bfloat16, torch.int16)
_F32 = (torch.float32,)
_U8 = (torch.uint8,)


def _t(x, name, dtypes, numel, optional=False):
    """Check a tensor argument; returns its device pointer (None if absent)."""
    if x is None:
        if optional or numel == 0:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(x, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not x.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if not x.is_contiguous():
        raise ValueError(f"{name} must be contiguous (row-major)")
    if x.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {x.dtype}, expected one of {dtypes}")
    if x.numel() < numel:
        raise ValueError(f"{name} holds {x.numel()} elements, the call touches {numel}")
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _check(name: str, status: int):
    if status != 0:
        raise Fp8Error(name, status)


def _rc(x: torch.Tensor, name="x"):
    if not isinstance(x, torch.Tensor) or x.dim() != 2:
        raise ValueError(f"{name} must be a 2-D tensor")
    return x.shape[0], x.shape[1]


def workspace(device=None, wait_polls: int = 0, stream=None) -> torch.Tensor:
    """A device workspace for the amax-producing calls, prepared on `stream`
    by fp8_workspace_init (wait_polls: the one-launch wait's bound, 0 =
    default).  Calls that may run at the same time need different ones."""
    dev = torch.device("cuda") if device is None else torch.device(device)
    ws = torch.empty(WORKSPACE_BYTES, dtype=torch.uint8, device=dev)
    fp8_workspace_init(ws, wait_polls, stream)
    return ws


def fp8_workspace_init(ws, wait_polls=0, stream=None):
    _check("fp8_workspace_init",
           lib().fp8_workspace_init(_t(ws, "workspace", _U8, WORKSPACE_BYTES), int(wait_polls),
                                    _stream(stream)))


class _Ws:
    """The call's workspace: the caller's, or a fresh one kept alive until
    the call's stream has passed it."""

    def __init__(self, ws, stream):
        if ws is not None:
            self.ptr = _t(ws, "workspace", _U8, WORKSPACE_BYTES)
            return
        s = stream if isinstance(stream, torch.cuda.Stream) else None
        if stream is not None and s is None:
            raise ValueError("pass a workspace when the stream is a raw handle")
        self.t = workspace(stream=stream)
        if s is not None:
            self.t.record_stream(s)
        self.ptr = self.t.data_ptr()


# ------------------------------------------------------------ quantise
def fp8_amax(x, fmt, amax, scale=None, scale_inv=None, stream=None, workspace=None):
    rows, cols = _rc(x)
    ws = _Ws(workspace, stream)
    _check("fp8_amax", lib().fp8_amax(_t(x, "x", _BF16, rows * cols), rows, cols, fmt,
                                      _t(amax, "amax", _F32, 1), _t(scale, "scale", _F32, 1, True),
                                      _t(scale_inv, "scale_inv", _F32, 1, True), ws.ptr,
                                      _stream(stream)))


def fp8_quantize_tensor(x, fmt, scale, q, qT=None, amax_out=None, stream=None, workspace=None):
    rows, cols = _rc(x)
    n = rows * cols
    ws = _Ws(workspace, stream) if amax_out is not None else None
    _check("fp8_quantize_tensor",
           lib().fp8_quantize_tensor(_t(x, "x", _BF16, n), rows, cols, fmt,
                                     _t(scale, "scale", _F32, 1), _t(q, "q", _U8, n),
                                     _t(qT, "qT", _U8, n, True),
                                     _t(amax_out, "amax_out", _F32, 1, True),
                                     ws.ptr if ws else None, _stream(stream)))


def fp8_quantize_tensor_current(x, fmt, q, qT, amax, scale, scale_inv, stream=None,
                                workspace=None):
    rows, cols = _rc(x)
    n = rows * cols
    ws = _Ws(workspace, stream)
    _check("fp8_quantize_tensor_current",
           lib().fp8_quantize_tensor_current(_t(x, "x", _BF16, n), rows, cols, fmt,
                                             _t(q, "q", _U8, n), _t(qT, "qT", _U8, n, True),
                                             _t(amax, "amax", _F32, 1),
                                             _t(scale, "scale", _F32, 1, True),
                                             _t(scale_inv, "scale_inv", _F32, 1), ws.ptr,
                                             _stream(stream)))


def fp8_quantize_tensor_current_noalloc(x, fmt, q, qT, amax, scale, scale_inv, stream=None):
    """fp8_quantize_tensor_current through the library's static scratch: no
    workspace, nothing allocated (calls that overlap on one GPU race)."""
    rows, cols = _rc(x)
    n = rows * cols
    _check("fp8_quantize_tensor_current_noalloc",
           lib().fp8_quantize_tensor_current_noalloc(
               _t(x, "x", _BF16, n), rows, cols, fmt, _t(q, "q", _U8, n),
               _t(qT, "qT", _U8, n, True), _t(amax, "amax", _F32, 1),
               _t(scale, "scale", _F32, 1, True), _t(scale_inv, "scale_inv", _F32, 1),
               _stream(stream)))


def fp8_quantize_pair_current(a, fmt_a, qa, amax_a, scale_a, scale_inv_a,
                              b, fmt_b, qb, amax_b, scale_b, scale_inv_b, stream=None,
                              workspace=None):
    ra, ca = _rc(a, "a")
    rb, cb = _rc(b, "b")
    ws = _Ws(workspace, stream)
    _check("fp8_quantize_pair_current",
           lib().fp8_quantize_pair_current(
               _t(a, "a", _BF16, ra * ca), ra, ca, fmt_a, _t(qa, "qa", _U8, ra * ca),
               _t(amax_a, "amax_a", _F32, 1), _t(scale_a, "scale_a", _F32, 1, True),
               _t(scale_inv_a, "scale_inv_a", _F32, 1),
               _t(b, "b", _BF16, rb * cb), rb, cb, fmt_b, _t(qb, "qb", _U8, rb * cb),
               _t(amax_b, "amax_b", _F32, 1), _t(scale_b, "scale_b", _F32, 1, True),
               _t(scale_inv_b, "scale_inv_b", _F32, 1), ws.ptr, _stream(stream)))


def fp8_amax_f32(x, fmt, amax, scale=None, scale_inv=None, stream=None, workspace=None):
    rows, cols = _rc(x)
    ws = _Ws(workspace, stream)
    _check("fp8_amax_f32",
           lib().fp8_amax_f32(_t(x, "x", _F32, rows * cols), rows, cols, fmt,
                              _t(amax, "amax", _F32, 1), _t(scale, "scale", _F32, 1, True),
                              _t(scale_inv, "scale_inv", _F32, 1, True), ws.ptr,
                              _stream(stream)))


def fp8_quantize_tensor_f32(x, fmt, scale, q, qT=None, amax_out=None, stream=None,
                            workspace=None):
    rows, cols = _rc(x)
    n = rows * cols
    ws = _Ws(workspace, stream) if amax_out is not None else None
    _check("fp8_quantize_tensor_f32",
           lib().fp8_quantize_tensor_f32(_t(x, "x", _F32, n), rows, cols, fmt,
                                         _t(scale, "scale", _F32, 1), _t(q, "q", _U8, n),
                                         _t(qT, "qT", _U8, n, True),
                                         _t(amax_out, "amax_out", _F32, 1, True),
                                         ws.ptr if ws else None, _stream(stream)))


def fp8_amax_history_update(history, step, amax, fmt, scale, scale_inv, stream=None):
    _check("fp8_amax_history_update",
           lib().fp8_amax_history_update(_t(history, "history", _F32, 1), history.numel(),
                                         int(step), _t(amax, "amax", _F32, 1), fmt,
                                         _t(scale, "scale", _F32, 1),
                                         _t(scale_inv, "scale_inv", _F32, 1), _stream(stream)))


def _blocks(n, b):
    return (n + b - 1) // b


def fp8_quantize_block(x, fmt, block_rows, block_cols, q, scale_inv, stream=None):
    rows, cols = _rc(x)
    n = rows * cols
    ns = _blocks(rows, max(block_rows, 1)) * _blocks(cols, max(block_cols, 1))
    _check("fp8_quantize_block",
           lib().fp8_quantize_block(_t(x, "x", _BF16, n), rows, cols, fmt, block_rows, block_cols,
                                    _t(q, "q", _U8, n), _t(scale_inv, "scale_inv", _F32, ns),
                                    _stream(stream)))


def fp8_quantize_mx(x, fmt, q, scale_e8m0, stream=None):
    rows, cols = _rc(x)
    n = rows * cols
    _check("fp8_quantize_mx",
           lib().fp8_quantize_mx(_t(x, "x", _BF16, n), rows, cols, fmt, _t(q, "q", _U8, n),
                                 _t(scale_e8m0, "scale_e8m0", _U8, rows * _blocks(cols, 32)),
                                 _stream(stream)))


def fp8_quantize_block_t(x, fmt, block_rows, q, scale_inv, qT, scale_inv_T, stream=None):
    rows, cols = _rc(x)
    n = rows * cols
    br = max(block_rows, 1)
    ns = _blocks(rows, br) * _blocks(cols, 128)
    nsT = (cols if br == 1 else _blocks(cols, 128)) * _blocks(rows, 128)
    _check("fp8_quantize_block_t",
           lib().fp8_quantize_block_t(_t(x, "x", _BF16, n), rows, cols, fmt, block_rows,
                                      _t(q, "q", _U8, n, True),
                                      _t(scale_inv, "scale_inv", _F32, ns, True),
                                      _t(qT, "qT", _U8, n),
                                      _t(scale_inv_T, "scale_inv_T", _F32, nsT),
                                      _stream(stream)))


def fp8_quantize_mx_t(x, fmt, q, scale_e8m0, qT, scale_e8m0_T, stream=None):
    rows, cols = _rc(x)
    n = rows * cols
    _check("fp8_quantize_mx_t",
           lib().fp8_quantize_mx_t(_t(x, "x", _BF16, n), rows, cols, fmt,
                                   _t(q, "q", _U8, n, True),
                                   _t(scale_e8m0, "scale_e8m0", _U8, rows * _blocks(cols, 32),
                                      True),
                                   _t(qT, "qT", _U8, n),
                                   _t(scale_e8m0_T, "scale_e8m0_T", _U8,
                                      cols * _blocks(rows, 32)),
                                   _stream(stream)))


# ------------------------------------------------------------ GEMMs
def operand(data, fmt, scaling, scale_inv) -> Operand:
    """The operand holds the two tensors as well as their addresses, so that
    temporaries passed here stay allocated until the GEMM call has been
    enqueued (after that, torch's stream-ordered reuse is safe).  Sizes are
    checked by the GEMM call, which knows the operand's rows and contraction."""
    o = Operand(None if data is None else data.data_ptr(), fmt, scaling,
                None if scale_inv is None else scale_inv.data_ptr())
    o._tensors = (data, scale_inv)
    return o


def _check_operand(o: Operand, name, rows, kc):
    data, sc = o._tensors
    _t(data, f"{name}.data", _U8, rows * kc)
    if o.scaling == SCALE_TENSOR:
        _t(sc, f"{name}.scale_inv", _F32, 1 if rows * kc else 0)
    elif o.scaling == SCALE_BLOCK_1x128:
        _t(sc, f"{name}.scale_inv", _F32, rows * _blocks(kc, 128))
    elif o.scaling == SCALE_BLOCK_128x128:
        _t(sc, f"{name}.scale_inv", _F32, _blocks(rows, 128) * _blocks(kc, 128))
    elif o.scaling == SCALE_MX_1x32:
        _t(sc, f"{name}.scale_inv", _U8, rows * _blocks(kc, 32))


def _gemm_args(a, b, rows_a, rows_b, kc, c, c_dtypes, c_name):
    _check_operand(a, "a", rows_a, kc)
    _check_operand(b, "b", rows_b, kc)
    return _t(c, c_name, c_dtypes, rows_a * rows_b)


def fp8_gemm_fprop(x: Operand, w: Operand, M, N, K, y, stream=None):
    yp = _gemm_args(x, w, M, N, K, y, _BF16, "y")
    _check("fp8_gemm_fprop", lib().fp8_gemm_fprop(ctypes.byref(x), ctypes.byref(w), M, N, K,
                                                  yp, _stream(stream)))


def fp8_gemm_dgrad(dy: Operand, wT: Operand, M, N, K, dx, stream=None):
    dxp = _gemm_args(dy, wT, M, K, N, dx, _BF16, "dx")
    _check("fp8_gemm_dgrad", lib().fp8_gemm_dgrad(ctypes.byref(dy), ctypes.byref(wT), M, N, K,
                                                  dxp, _stream(stream)))


def fp8_gemm_wgrad(dyT: Operand, xT: Operand, M, N, K, dw, stream=None):
    dwp = _gemm_args(dyT, xT, N, K, M, dw, _BF16, "dw")
    _check("fp8_gemm_wgrad", lib().fp8_gemm_wgrad(ctypes.byref(dyT), ctypes.byref(xT), M, N, K,
                                                  dwp, _stream(stream)))


def fp8_gemm_fprop_fused(x: Operand, w: Operand, M, N, K, y, y_fmt, y_scale, y_q, y_amax,
                         stream=None, workspace=None):
    _check_operand(x, "x", M, K)
    _check_operand(w, "w", N, K)
    yp = _t(y, "y", _BF16, M * N, True)
    ws = _Ws(workspace, stream) if y_amax is not None else None
    _check("fp8_gemm_fprop_fused",
           lib().fp8_gemm_fprop_fused(ctypes.byref(x), ctypes.byref(w), M, N, K, yp, y_fmt,
                                      _t(y_scale, "y_scale", _F32, 1, True),
                                      _t(y_q, "y_q", _U8, M * N, True),
                                      _t(y_amax, "y_amax", _F32, 1, True),
                                      ws.ptr if ws else None, _stream(stream)))


def fp8_gemm_wgrad_f32(dyT: Operand, xT: Operand, M, N, K, dw, accumulate=False, stream=None):
    dwp = _gemm_args(dyT, xT, N, K, M, dw, _F32, "dw")
    _check("fp8_gemm_wgrad_f32",
           lib().fp8_gemm_wgrad_f32(ctypes.byref(dyT), ctypes.byref(xT), M, N, K, dwp,
                                    1 if accumulate else 0, _stream(stream)))


def fp8_convert_f32(x, fmt, q, stream=None):
    n = x.numel()
    _check("fp8_convert_f32", lib().fp8_convert_f32(_t(x, "x", _F32, n), n, fmt,
                                                    _t(q, "q", _U8, n), _stream(stream)))


def fp8_status_string(status: int) -> str:
    return lib().fp8_status_string(status).decode()
