"""Thin Python binding of libfp8sg.so (the C ABI in include/fp8sg.h).

Argument marshalling only: every function hands device pointers of torch
tensors to the C entry point of the same name and raises ``Fp8Error`` on a
non-zero status.  All arithmetic runs in the library's HIP kernels.  There is
no fallback: if the library is missing the import fails loudly.
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
_EXPORTS = ["fp8_amax", "fp8_quantize_tensor", "fp8_quantize_tensor_current",
            "fp8_quantize_pair_current", "fp8_amax_f32",
            "fp8_quantize_tensor_f32",
            "fp8_amax_history_update", "fp8_quantize_block",
            "fp8_quantize_mx", "fp8_quantize_block_t", "fp8_quantize_mx_t", "fp8_gemm_fprop",
            "fp8_gemm_dgrad", "fp8_gemm_wgrad", "fp8_gemm_fprop_fused", "fp8_gemm_wgrad_f32",
            "fp8_convert_f32",
            "fp8_status_string"]


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
            "fp8_amax": [vp, i64, i64, i32, vp, vp, vp, vp],
            "fp8_quantize_tensor": [vp, i64, i64, i32, vp, vp, vp, vp, vp],
            "fp8_amax_f32": [vp, i64, i64, i32, vp, vp, vp, vp],
            "fp8_quantize_tensor_current": [vp, i64, i64, i32, vp, vp, vp, vp, vp, vp],
            "fp8_quantize_pair_current": [vp, i64, i64, i32, vp, vp, vp, vp,
                                          vp, i64, i64, i32, vp, vp, vp, vp, vp],
            "fp8_quantize_tensor_f32": [vp, i64, i64, i32, vp, vp, vp, vp, vp],
            "fp8_amax_history_update": [vp, i32, i64, vp, i32, vp, vp, vp],
            "fp8_quantize_block": [vp, i64, i64, i32, i32, i32, vp, vp, vp],
            "fp8_quantize_mx": [vp, i64, i64, i32, vp, vp, vp],
            "fp8_quantize_block_t": [vp, i64, i64, i32, i32, vp, vp, vp, vp, vp],
            "fp8_quantize_mx_t": [vp, i64, i64, i32, vp, vp, vp, vp, vp],
            "fp8_gemm_fprop": [vp, vp, i64, i64, i64, vp, vp],
            "fp8_gemm_dgrad": [vp, vp, i64, i64, i64, vp, vp],
            "fp8_gemm_wgrad": [vp, vp, i64, i64, i64, vp, vp],
            "fp8_gemm_wgrad_f32": [vp, vp, i64, i64, i64, vp, i32, vp],
            "fp8_gemm_fprop_fused": [vp, vp, i64, i64, i64, vp, i32, vp, vp, vp, vp],
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


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _check(name: str, status: int):
    if status != 0:
        raise Fp8Error(name, status)


def _rc(x: torch.Tensor):
    assert x.dim() == 2, "2-D tensors expected"
    return x.shape[0], x.shape[1]


def fp8_amax(x, fmt, amax, scale=None, scale_inv=None, stream=None):
    rows, cols = _rc(x)
    _check("fp8_amax", lib().fp8_amax(_ptr(x), rows, cols, fmt, _ptr(amax), _ptr(scale),
                                      _ptr(scale_inv), _stream(stream)))


def fp8_quantize_tensor(x, fmt, scale, q, qT=None, amax_out=None, stream=None):
    rows, cols = _rc(x)
    _check("fp8_quantize_tensor",
           lib().fp8_quantize_tensor(_ptr(x), rows, cols, fmt, _ptr(scale), _ptr(q), _ptr(qT),
                                     _ptr(amax_out), _stream(stream)))


def fp8_quantize_tensor_current(x, fmt, q, qT, amax, scale, scale_inv, stream=None):
    rows, cols = _rc(x)
    _check("fp8_quantize_tensor_current",
           lib().fp8_quantize_tensor_current(_ptr(x), rows, cols, fmt, _ptr(q), _ptr(qT),
                                             _ptr(amax), _ptr(scale), _ptr(scale_inv),
                                             _stream(stream)))


def fp8_quantize_pair_current(a, fmt_a, qa, amax_a, scale_a, scale_inv_a,
                              b, fmt_b, qb, amax_b, scale_b, scale_inv_b, stream=None):
    ra, ca = _rc(a)
    rb, cb = _rc(b)
    _check("fp8_quantize_pair_current",
           lib().fp8_quantize_pair_current(_ptr(a), ra, ca, fmt_a, _ptr(qa), _ptr(amax_a),
                                           _ptr(scale_a), _ptr(scale_inv_a),
                                           _ptr(b), rb, cb, fmt_b, _ptr(qb), _ptr(amax_b),
                                           _ptr(scale_b), _ptr(scale_inv_b), _stream(stream)))


def fp8_amax_f32(x, fmt, amax, scale=None, scale_inv=None, stream=None):
    rows, cols = _rc(x)
    _check("fp8_amax_f32", lib().fp8_amax_f32(_ptr(x), rows, cols, fmt, _ptr(amax), _ptr(scale),
                                              _ptr(scale_inv), _stream(stream)))


def fp8_quantize_tensor_f32(x, fmt, scale, q, qT=None, amax_out=None, stream=None):
    rows, cols = _rc(x)
    _check("fp8_quantize_tensor_f32",
           lib().fp8_quantize_tensor_f32(_ptr(x), rows, cols, fmt, _ptr(scale), _ptr(q), _ptr(qT),
                                         _ptr(amax_out), _stream(stream)))


def fp8_amax_history_update(history, step, amax, fmt, scale, scale_inv, stream=None):
    _check("fp8_amax_history_update",
           lib().fp8_amax_history_update(_ptr(history), history.numel(), int(step), _ptr(amax),
                                         fmt, _ptr(scale), _ptr(scale_inv), _stream(stream)))


def fp8_quantize_block(x, fmt, block_rows, block_cols, q, scale_inv, stream=None):
    rows, cols = _rc(x)
    _check("fp8_quantize_block",
           lib().fp8_quantize_block(_ptr(x), rows, cols, fmt, block_rows, block_cols, _ptr(q),
                                    _ptr(scale_inv), _stream(stream)))


def fp8_quantize_mx(x, fmt, q, scale_e8m0, stream=None):
    rows, cols = _rc(x)
    _check("fp8_quantize_mx", lib().fp8_quantize_mx(_ptr(x), rows, cols, fmt, _ptr(q),
                                                    _ptr(scale_e8m0), _stream(stream)))


def fp8_quantize_block_t(x, fmt, block_rows, q, scale_inv, qT, scale_inv_T, stream=None):
    rows, cols = _rc(x)
    _check("fp8_quantize_block_t",
           lib().fp8_quantize_block_t(_ptr(x), rows, cols, fmt, block_rows, _ptr(q),
                                      _ptr(scale_inv), _ptr(qT), _ptr(scale_inv_T),
                                      _stream(stream)))


def fp8_quantize_mx_t(x, fmt, q, scale_e8m0, qT, scale_e8m0_T, stream=None):
    rows, cols = _rc(x)
    _check("fp8_quantize_mx_t",
           lib().fp8_quantize_mx_t(_ptr(x), rows, cols, fmt, _ptr(q), _ptr(scale_e8m0), _ptr(qT),
                                   _ptr(scale_e8m0_T), _stream(stream)))


def operand(data, fmt, scaling, scale_inv) -> Operand:
    """The operand holds the two tensors as well as their addresses, so that
    temporaries passed here stay allocated until the GEMM call has been
    enqueued (after that, torch's stream-ordered reuse is safe)."""
    o = Operand(_ptr(data), fmt, scaling, _ptr(scale_inv))
    o._tensors = (data, scale_inv)
    return o


def fp8_gemm_fprop(x: Operand, w: Operand, M, N, K, y, stream=None):
    _check("fp8_gemm_fprop", lib().fp8_gemm_fprop(ctypes.byref(x), ctypes.byref(w), M, N, K,
                                                  _ptr(y), _stream(stream)))


def fp8_gemm_dgrad(dy: Operand, wT: Operand, M, N, K, dx, stream=None):
    _check("fp8_gemm_dgrad", lib().fp8_gemm_dgrad(ctypes.byref(dy), ctypes.byref(wT), M, N, K,
                                                  _ptr(dx), _stream(stream)))


def fp8_gemm_wgrad(dyT: Operand, xT: Operand, M, N, K, dw, stream=None):
    _check("fp8_gemm_wgrad", lib().fp8_gemm_wgrad(ctypes.byref(dyT), ctypes.byref(xT), M, N, K,
                                                  _ptr(dw), _stream(stream)))


def fp8_gemm_fprop_fused(x: Operand, w: Operand, M, N, K, y, y_fmt, y_scale, y_q, y_amax,
                         stream=None):
    _check("fp8_gemm_fprop_fused",
           lib().fp8_gemm_fprop_fused(ctypes.byref(x), ctypes.byref(w), M, N, K, _ptr(y), y_fmt,
                                      _ptr(y_scale), _ptr(y_q), _ptr(y_amax), _stream(stream)))


def fp8_gemm_wgrad_f32(dyT: Operand, xT: Operand, M, N, K, dw, accumulate=False, stream=None):
    _check("fp8_gemm_wgrad_f32",
           lib().fp8_gemm_wgrad_f32(ctypes.byref(dyT), ctypes.byref(xT), M, N, K, _ptr(dw),
                                    1 if accumulate else 0, _stream(stream)))


def fp8_convert_f32(x, fmt, q, stream=None):
    _check("fp8_convert_f32", lib().fp8_convert_f32(_ptr(x), x.numel(), fmt, _ptr(q),
                                                    _stream(stream)))


def fp8_status_string(status: int) -> str:
    return lib().fp8_status_string(status).decode()
