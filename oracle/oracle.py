"""Python face of the CPU oracle (``fp8_oracle.c``) plus whole-matrix GEMMs.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg import this module.  It never imports the product
package and the product package never imports it.

Element-wise work (codec, amax, scale rules, casts, history, blockwise and MX
casts, single GEMM outputs) runs in the C file.  The whole-matrix GEMMs here
decode both FP8 operands exactly to float64 and use numpy's float64 matmul as
the contraction step; the scale algebra around it is the definition written
out (see ``fp8_oracle.c`` for the cited passages):

* tensor scaling:  C = (sa * sb) * (A . B^T)
* block scaling:   C = sum_b  Sa_b (x) Sb_b  *  (A_b . B_b^T)   (128-wide K blocks)
* MX scaling:      C = (A * 2^ea) . (B * 2^eb)^T                (32-wide K blocks)
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

E4M3 = 0
E5M2 = 1
FMAX = {E4M3: 448.0, E5M2: 57344.0}
SCALE_TENSOR, SCALE_BLOCK, SCALE_MX = 0, 1, 2

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fp8_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call([
            "gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
            "-shared", "-fPIC", "-std=c11", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        u8p = ctypes.POINTER(ctypes.c_uint8)
        L.oracle_fp8_decode.restype = ctypes.c_double
        L.oracle_fp8_decode.argtypes = [ctypes.c_uint8, ctypes.c_int]
        L.oracle_fp8_encode.restype = ctypes.c_uint8
        L.oracle_fp8_encode.argtypes = [ctypes.c_float, ctypes.c_int]
        L.oracle_bf16_to_f32.restype = ctypes.c_float
        L.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.oracle_f64_to_bf16.restype = ctypes.c_uint16
        L.oracle_f64_to_bf16.argtypes = [ctypes.c_double]
        L.oracle_amax.restype = ctypes.c_float
        L.oracle_amax.argtypes = [ctypes.c_void_p, ctypes.c_int64]
        L.oracle_scale_from_amax.restype = None
        L.oracle_scale_from_amax.argtypes = [ctypes.c_float, ctypes.c_int,
                                             ctypes.c_void_p, ctypes.c_void_p]
        L.oracle_quantize_tensor.restype = None
        L.oracle_quantize_tensor.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                             ctypes.c_int, ctypes.c_float, ctypes.c_void_p,
                                             ctypes.c_void_p, ctypes.c_void_p]
        L.oracle_amax_f32.restype = ctypes.c_float
        L.oracle_amax_f32.argtypes = [ctypes.c_void_p, ctypes.c_int64]
        L.oracle_quantize_tensor_f32.restype = None
        L.oracle_quantize_tensor_f32.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                                 ctypes.c_int, ctypes.c_float, ctypes.c_void_p,
                                                 ctypes.c_void_p, ctypes.c_void_p]
        L.oracle_amax_history_update.restype = None
        L.oracle_amax_history_update.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                                 ctypes.c_float, ctypes.c_int,
                                                 ctypes.c_void_p, ctypes.c_void_p]
        L.oracle_quantize_block.restype = None
        L.oracle_quantize_block.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                            ctypes.c_int, ctypes.c_int32, ctypes.c_int32,
                                            ctypes.c_void_p, ctypes.c_void_p]
        L.oracle_mx_exponent.restype = ctypes.c_int
        L.oracle_mx_exponent.argtypes = [ctypes.c_float, ctypes.c_int]
        L.oracle_quantize_mx.restype = None
        L.oracle_quantize_mx.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                         ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
        L.oracle_gemm_entries.restype = None
        L.oracle_gemm_entries.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
            ctypes.c_int, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32,
            ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p]
        L.oracle_f64_to_bf16_array.restype = None
        L.oracle_f64_to_bf16_array.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
        L.oracle_fp8_encode_array.restype = None
        L.oracle_fp8_encode_array.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                              ctypes.c_void_p]
        L.oracle_fp8_encode_bits_range.restype = None
        L.oracle_fp8_encode_bits_range.argtypes = [ctypes.c_uint64, ctypes.c_uint64,
                                                   ctypes.c_int, ctypes.c_void_p]
        del u8p
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _u16(x) -> np.ndarray:
    x = np.ascontiguousarray(x)
    assert x.dtype == np.uint16, "BF16 tensors are passed as their uint16 bit patterns"
    return x


# ------------------------------------------------------------------ codec
def decode(code: int, fmt: int) -> float:
    return lib().oracle_fp8_decode(int(code) & 0xFF, fmt)


def decode_table(fmt: int) -> np.ndarray:
    """Exact float64 value of all 256 codes (index = code)."""
    return np.array([decode(c, fmt) for c in range(256)], dtype=np.float64)


def encode(f, fmt: int) -> np.ndarray:
    f = np.ascontiguousarray(np.asarray(f, dtype=np.float32))
    out = np.empty(f.shape, dtype=np.uint8)
    lib().oracle_fp8_encode_array(_p(f), f.size, fmt, _p(out))
    return out


def encode_bits_range(lo: int, hi: int, fmt: int) -> np.ndarray:
    out = np.empty(hi - lo, dtype=np.uint8)
    lib().oracle_fp8_encode_bits_range(lo, hi, fmt, _p(out))
    return out


def bf16_to_f32(b) -> np.ndarray:
    b = np.asarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def f64_to_bf16(v) -> np.ndarray:
    v = np.ascontiguousarray(np.asarray(v, dtype=np.float64))
    out = np.empty(v.shape, dtype=np.uint16)
    lib().oracle_f64_to_bf16_array(_p(v), v.size, _p(out))
    return out


# ----------------------------------------------------------- quantisation
def amax(x) -> float:
    x = _u16(x)
    return float(lib().oracle_amax(_p(x), x.size))


def scale_from_amax(a: float, fmt: int):
    s = np.zeros(1, np.float32)
    si = np.zeros(1, np.float32)
    lib().oracle_scale_from_amax(float(a), fmt, _p(s), _p(si))
    return np.float32(s[0]), np.float32(si[0])


def quantize_tensor(x, fmt: int, scale, transposed: bool = False, want_amax: bool = False):
    """Returns (q[R,C], qT[C,R] or None, amax or None)."""
    x = _u16(x)
    R, C = x.shape
    q = np.empty((R, C), np.uint8)
    qT = np.empty((C, R), np.uint8) if transposed else None
    am = np.zeros(1, np.float32)
    lib().oracle_quantize_tensor(_p(x), R, C, fmt, float(np.float32(scale)), _p(q),
                                 _p(qT) if qT is not None else None,
                                 _p(am) if want_amax else None)
    return q, qT, (np.float32(am[0]) if want_amax else None)


def amax_f32(x) -> float:
    """amax of an FP32 array (FP32 master weight)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return float(np.float32(lib().oracle_amax_f32(_p(x), x.size)))


def quantize_tensor_f32(x, fmt: int, scale, transposed: bool = False, want_amax: bool = False):
    """Per-tensor cast of an FP32 array; returns (q, qT or None, amax or None)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    R, C = x.shape
    q = np.empty((R, C), np.uint8)
    qT = np.empty((C, R), np.uint8) if transposed else None
    am = np.zeros(1, np.float32)
    lib().oracle_quantize_tensor_f32(_p(x), R, C, fmt, float(np.float32(scale)), _p(q),
                                     _p(qT) if qT is not None else None,
                                     _p(am) if want_amax else None)
    return q, qT, (np.float32(am[0]) if want_amax else None)


def amax_history_update(hist: np.ndarray, step: int, a: float, fmt: int):
    """Updates ``hist`` (float32[H]) in place; returns (scale, scale_inv) for step+1."""
    assert hist.dtype == np.float32 and hist.flags["C_CONTIGUOUS"]
    s = np.zeros(1, np.float32)
    si = np.zeros(1, np.float32)
    lib().oracle_amax_history_update(_p(hist), hist.size, int(step), float(a), fmt,
                                     _p(s), _p(si))
    return np.float32(s[0]), np.float32(si[0])


def quantize_block(x, fmt: int, block_rows: int, block_cols: int = 128):
    x = _u16(x)
    R, C = x.shape
    assert C % block_cols == 0 and R % block_rows == 0
    q = np.empty((R, C), np.uint8)
    si = np.empty((R // block_rows, C // block_cols), np.float32)
    lib().oracle_quantize_block(_p(x), R, C, fmt, block_rows, block_cols, _p(q), _p(si))
    return q, si


def mx_exponent(a: float, fmt: int) -> int:
    return int(lib().oracle_mx_exponent(float(a), fmt))


def quantize_mx(x, fmt: int = E4M3):
    x = _u16(x)
    R, C = x.shape
    assert C % 32 == 0
    q = np.empty((R, C), np.uint8)
    e = np.empty((R, C // 32), np.uint8)
    lib().oracle_quantize_mx(_p(x), R, C, fmt, _p(q), _p(e))
    return q, e


# ------------------------------------------------------------------ GEMMs
def gemm_entries(A, B, fmt_a, fmt_b, mode, sa, sb, ii, jj, block_rows_a=1, block_rows_b=1):
    """C[ii[t], jj[t]] one by one (FP64), its sum of |terms|, and its BF16 bits."""
    A = np.ascontiguousarray(A, dtype=np.uint8)
    B = np.ascontiguousarray(B, dtype=np.uint8)
    assert A.shape[1] == B.shape[1]
    K = A.shape[1]
    ii = np.ascontiguousarray(ii, dtype=np.int64)
    jj = np.ascontiguousarray(jj, dtype=np.int64)
    assert ii.shape == jj.shape
    assert ii.size == 0 or (ii.min() >= 0 and ii.max() < A.shape[0] and jj.min() >= 0
                            and jj.max() < B.shape[0])
    if mode == SCALE_MX:
        sa = np.ascontiguousarray(sa, dtype=np.uint8)
        sb = np.ascontiguousarray(sb, dtype=np.uint8)
    else:
        sa = np.ascontiguousarray(sa, dtype=np.float32)
        sb = np.ascontiguousarray(sb, dtype=np.float32)
    n = ii.size
    out = np.empty(n, np.float64)
    absd = np.empty(n, np.float64)
    bf = np.empty(n, np.uint16)
    lib().oracle_gemm_entries(_p(A), _p(B), K, fmt_a, fmt_b, mode, _p(sa), block_rows_a,
                              _p(sb), block_rows_b, n, _p(ii), _p(jj), _p(out), _p(absd),
                              _p(bf))
    return out, absd, bf


def _dec(A, fmt):
    return decode_table(fmt)[np.asarray(A, dtype=np.uint8)]


def gemm_full(A, B, fmt_a, fmt_b, mode, sa, sb, block_rows_a=1, block_rows_b=1):
    """Whole C = A . B^T (both K-contiguous) in FP64; returns (C, sum|terms|, BF16 bits)."""
    A = np.asarray(A, dtype=np.uint8)
    B = np.asarray(B, dtype=np.uint8)
    K = A.shape[1]
    Ad, Bd = _dec(A, fmt_a), _dec(B, fmt_b)
    if mode == SCALE_TENSOR:
        s = float(np.float32(np.asarray(sa).reshape(-1)[0])) * float(
            np.float32(np.asarray(sb).reshape(-1)[0]))
        C = (Ad @ Bd.T) * s
        Cabs = (np.abs(Ad) @ np.abs(Bd).T) * abs(s)
    elif mode == SCALE_BLOCK:
        sa = np.asarray(sa, dtype=np.float64)
        sb = np.asarray(sb, dtype=np.float64)
        Sa = np.repeat(sa, block_rows_a, axis=0)[: A.shape[0]]     # [Ra, K/128]
        Sb = np.repeat(sb, block_rows_b, axis=0)[: B.shape[0]]     # [Rb, K/128]
        C = np.zeros((A.shape[0], B.shape[0]))
        Cabs = np.zeros_like(C)
        for b in range(K // 128):
            sl = slice(b * 128, (b + 1) * 128)
            s = np.outer(Sa[:, b], Sb[:, b])
            C += s * (Ad[:, sl] @ Bd[:, sl].T)
            Cabs += np.abs(s) * (np.abs(Ad[:, sl]) @ np.abs(Bd[:, sl]).T)
    elif mode == SCALE_MX:
        def mult(e):
            e = np.asarray(e, dtype=np.int64)
            m = np.ldexp(1.0, (e - 127).astype(np.int32)).astype(np.float64)
            m[e == 0xFF] = np.nan
            return np.repeat(m, 32, axis=1)
        Ad = Ad * mult(sa)
        Bd = Bd * mult(sb)
        C = Ad @ Bd.T
        Cabs = np.abs(Ad) @ np.abs(Bd).T
    else:
        raise ValueError(mode)
    return C, Cabs, f64_to_bf16(C)
