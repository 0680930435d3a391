"""Pins of the oracle's FP8 / BF16 codec against what the formats fix.

The FP8 guide page (section "format choice: E4M3 and E5M2") fixes the bit
splits 1/4/3 and 1/5/2; the OCP 8-bit formats fix the biases, the E4M3FN
special values and the largest finite values 448 and 57344.  These tests
check enumerated facts of all 256 codes, round trips, ordering, midpoint
behaviour, saturation, and a second encoder with a different algorithm
(nearest value by search over the decoded table).
"""
import ctypes
import math
import os
import subprocess
from fractions import Fraction

import numpy as np
import pytest

E4M3, E5M2 = 0, 1


def test_e4m3_code_census(orc):
    t = orc.decode_table(E4M3)
    nan = np.isnan(t)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.isinf(t).sum() == 0
    fin = t[~nan]
    assert fin.size == 254
    assert np.unique(fin).size == 253           # +0 and -0 compare equal
    assert fin.max() == 448.0 and fin.min() == -448.0
    pos = fin[fin > 0]
    assert pos.min() == 2.0 ** -9               # smallest subnormal
    assert t[0x08] == 2.0 ** -6                 # smallest normal
    assert t[0x38] == 1.0                       # exponent field 7 = bias
    assert t[0x39] == 1.125 and t[0x3F] == 1.875
    assert t[0xC0] == -2.0
    assert t[0x7E] == 448.0 and t[0x77] == 240.0
    assert math.copysign(1.0, t[0x80]) == -1.0 and t[0x80] == 0.0


def test_e5m2_code_census(orc):
    t = orc.decode_table(E5M2)
    nan = np.isnan(t)
    assert nan.sum() == 6
    assert np.isinf(t).sum() == 2 and t[0x7C] == np.inf and t[0xFC] == -np.inf
    fin = t[np.isfinite(t)]
    assert fin.size == 248
    assert fin.max() == 57344.0
    pos = fin[fin > 0]
    assert pos.min() == 2.0 ** -16
    assert t[0x04] == 2.0 ** -14
    assert t[0x3C] == 1.0 and t[0x3D] == 1.25
    assert t[0x7B] == 57344.0


def _exact_value(code, ebits, mbits, bias):
    """Exact rational value of a finite code straight from its bit fields."""
    s = -1 if code >> 7 else 1
    e = (code >> mbits) & ((1 << ebits) - 1)
    m = code & ((1 << mbits) - 1)
    if e == 0:
        return s * Fraction(m, 1 << mbits) * Fraction(2) ** (1 - bias)
    return s * (1 + Fraction(m, 1 << mbits)) * Fraction(2) ** (e - bias)


@pytest.mark.parametrize("fmt,ebits,mbits,bias", [(E4M3, 4, 3, 7), (E5M2, 5, 2, 15)])
def test_decode_matches_bit_fields(orc, fmt, ebits, mbits, bias):
    t = orc.decode_table(fmt)
    for c in range(256):
        if np.isfinite(t[c]):
            assert Fraction(t[c]) == _exact_value(c, ebits, mbits, bias), hex(c)


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_round_trip_and_order(orc, fmt):
    t = orc.decode_table(fmt)
    codes = [c for c in range(256) if not np.isnan(t[c]) and not np.isinf(t[c])]
    back = orc.encode(t[codes].astype(np.float32), fmt)
    assert list(back) == codes                   # includes -0 -> 0x80
    top = 0x7E if fmt == E4M3 else 0x7B
    pos = t[: top + 1]
    assert np.all(np.diff(pos) > 0)              # positive codes strictly increasing
    assert np.all(t[0x80: 0x80 + top + 1] == -pos)


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_midpoints_round_to_even(orc, fmt):
    t = orc.decode_table(fmt)
    top = 0x7E if fmt == E4M3 else 0x7B
    for c in range(top):
        lo, hi = t[c], t[c + 1]
        mid = np.float32((lo + hi) / 2)
        assert float(mid) == (lo + hi) / 2       # every midpoint is an FP32 number
        even = c if c % 2 == 0 else c + 1
        for sgn, off in ((1, 0), (-1, 0x80)):
            m = np.float32(sgn * mid)
            assert orc.encode([m], fmt)[0] == even + off
            up = np.nextafter(np.float32(sgn * mid), np.float32(sgn * np.inf))
            dn = np.nextafter(np.float32(sgn * mid), np.float32(0))
            assert orc.encode([up], fmt)[0] == c + 1 + off
            assert orc.encode([dn], fmt)[0] == c + off


@pytest.mark.parametrize("fmt,fmax,maxc", [(E4M3, 448.0, 0x7E), (E5M2, 57344.0, 0x7B)])
def test_saturation_and_specials(orc, fmt, fmax, maxc):
    big = [fmax * (1 + 2 ** -20), np.inf, 1e30, 3.0e38, fmax * 1.06, fmax * 1.5]
    assert list(orc.encode(np.array(big, np.float32), fmt)) == [maxc] * len(big)
    assert list(orc.encode(-np.array(big, np.float32), fmt)) == [0x80 | maxc] * len(big)
    # NaN (any sign or payload) -> the format's canonical NaN code
    nan_code = 0xFF if fmt == E4M3 else 0xFE
    nans = np.array([0x7FC00000, 0xFFC00000, 0x7F800001, 0xFFFFFFFF], np.uint32).view(np.float32)
    assert list(orc.encode(nans, fmt)) == [nan_code] * 4
    assert np.isnan(orc.decode_table(fmt)[nan_code])
    assert orc.encode([np.float32(0.0)], fmt)[0] == 0x00
    assert orc.encode([np.float32(-0.0)], fmt)[0] == 0x80
    # FP32 subnormals and values below half the smallest FP8 subnormal -> signed zero
    tiny = np.array([1e-45, 1e-40, 2.0 ** -40], np.float32)
    assert list(orc.encode(tiny, fmt)) == [0, 0, 0]
    assert list(orc.encode(-tiny, fmt)) == [0x80] * 3


def _nearest_codec(fmt, orc):
    """Second encoder: nearest finite magnitude by search, ties to even code."""
    t = orc.decode_table(fmt)
    top = 0x7E if fmt == E4M3 else 0x7B
    vals = t[: top + 1]
    codes = np.arange(top + 1, dtype=np.int64)

    def enc(f):
        f = np.asarray(f, np.float32)
        with np.errstate(invalid="ignore"):
            a = np.abs(f.astype(np.float64))
        hi = np.clip(np.searchsorted(vals, a, side="right"), 1, top)
        lo = hi - 1
        dl = a - vals[lo]
        dh = vals[hi] - a
        pick = np.where(dl < dh, codes[lo], np.where(dh < dl, codes[hi],
                                                     np.where(codes[lo] % 2 == 0, codes[lo],
                                                              codes[hi])))
        pick = np.where(a >= vals[top], top, pick)
        pick = np.where(np.signbit(f), pick | 0x80, pick)
        pick = np.where(np.isnan(f), 0xFF if fmt == E4M3 else 0xFE, pick)
        return pick.astype(np.uint8)
    return enc


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_structured_fp32_cross_check(orc, fmt):
    """Every FP32 exponent and sign, the top 12 mantissa bits exhaustively,
    and low-bit patterns that sit on and beside every rounding boundary."""
    hi12 = np.arange(4096, dtype=np.uint32) << 11
    low = np.array([0, 1, 0x3FF, 0x400, 0x401, 0x7FF], np.uint32)
    mant = (hi12[:, None] | low[None, :]).reshape(-1)
    exps = np.arange(256, dtype=np.uint32) << 23
    u = (exps[:, None] | mant[None, :]).reshape(-1)
    u = np.concatenate([u, u | 0x80000000])
    rng = np.random.Generator(np.random.PCG64(7))
    u = np.concatenate([u, rng.integers(0, 2 ** 32, size=1 << 22, dtype=np.uint64).astype(
        np.uint32)])
    f = u.view(np.float32)
    got = orc.encode(f, fmt)
    want = _nearest_codec(fmt, orc)(f)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, (hex(int(u[bad[0]])), got[bad[0]], want[bad[0]])


@pytest.mark.slow
@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_all_fp32_patterns_cross_check(orc, fmt, tmp_path):
    """All 2^32 FP32 inputs: oracle encoder vs the independent nearest search."""
    src = os.path.join(os.path.dirname(__file__), "pins", "fp8_nearest_sweep.c")
    so = str(tmp_path / "sweep.so")
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-o", so, src, "-lm"])
    sw = ctypes.CDLL(so)
    sw.fp8_sweep.restype = ctypes.c_int64
    sw.fp8_sweep.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int, ctypes.c_void_p,
                             ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    t = orc.decode_table(fmt)
    top = 0x7E if fmt == E4M3 else 0x7B
    vals = np.ascontiguousarray(t[: top + 1])
    codes = np.arange(top + 1, dtype=np.uint8)
    first = np.zeros(1, np.uint64)
    fn = ctypes.cast(orc.lib().oracle_fp8_encode, ctypes.c_void_p)
    bad = sw.fp8_sweep(0, 1 << 32, fmt, vals.ctypes.data, codes.ctypes.data, top + 1,
                       fn, first.ctypes.data)
    assert bad == 0, hex(int(first[0]))


def test_bf16_rounding(orc):
    # FP32 inputs: the single RNE FP32 -> BF16 step of torch is a library routine.
    import torch
    rng = np.random.Generator(np.random.PCG64(11))
    u = rng.integers(0, 2 ** 32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    f = u.view(np.float32)
    f = f[np.isfinite(f)]
    got = orc.f64_to_bf16(f.astype(np.float64))
    want = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want)
    # FP64 inputs beyond FP32: exact rational rounding with ties to even.
    for v in [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -40, -(1.0 + 2 ** -8 - 2 ** -50),
              3.3895313892515355e38, 3.4e38, 1e-39, 2.0 ** -134, 2.0 ** -133 * 1.5]:
        b = int(orc.f64_to_bf16([v])[0])
        # nearest BF16 value to v by exact search around an FP32 anchor, ties to even
        x = Fraction(v)
        f32 = np.float32(v)
        anchor = int(np.array([f32]).view(np.uint32)[0] >> 16)
        best = None
        for cb in range(max(anchor - 2, 0), min(anchor + 3, 0xFFFF)):
            val = np.array([cb << 16], np.uint32).view(np.float32)[0]
            if not np.isfinite(val):
                continue
            d = abs(Fraction(float(val)) - x)
            key = (d, cb & 1)
            if best is None or key < best[0]:
                best = (key, cb)
        if abs(v) > 3.3961e38:
            assert b & 0x7FFF == 0x7F80
        else:
            assert b == best[1], (v, hex(b), hex(best[1]))
    assert orc.f64_to_bf16([np.nan])[0] == 0x7FC0
    assert orc.f64_to_bf16([np.inf])[0] == 0x7F80
    assert orc.f64_to_bf16([-np.inf])[0] == 0xFF80
