"""Pins of the oracle's scaled FP8 GEMMs.

The pages fix the data flow (search-result snippet on the forward pass: FP8
inputs, accumulation, BF16 output; guide section "code changes": the three
GEMMs of a layer take quantised inputs and keep BF16 outputs).  Exact
arithmetic and textbook linear algebra fix the rest:

* exact rational dot products on tiny shapes (E4M3 x E4M3 sums are exact in
  FP64, so the oracle must equal them; other formats within FP64's bound);
* W = c * I reduces the GEMM to a dequantise;
* MX with every scale byte 127 (x1) equals the unscaled GEMM;
* blockwise with uniform block scales equals per-tensor scaling;
* fprop / dgrad / wgrad through transposed quantised copies equal
  Y = X W, dX = dY W^T and dW = X^T dY of the logical [K x N] weight.
"""
from fractions import Fraction

import numpy as np
import pytest

E4M3, E5M2 = 0, 1
TENSOR, BLOCK, MX = 0, 1, 2


def rand_codes(shape, fmt, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    c = rng.integers(0, 256, size=shape, dtype=np.int64).astype(np.uint8)
    bad = (c & 0x7F) == 0x7F if fmt == E4M3 else (c & 0x7C) == 0x7C
    c[bad] = 0x30                                      # replace NaN / inf codes
    return c


def frac_dot(a_codes, b_codes, ta, tb):
    return sum(Fraction(ta[x]) * Fraction(tb[y]) for x, y in zip(a_codes, b_codes))


def all_entries(R, C):
    ii, jj = np.meshgrid(np.arange(R), np.arange(C), indexing="ij")
    return ii.reshape(-1), jj.reshape(-1)


def test_tiny_exact_e4m3(orc):
    ta = orc.decode_table(E4M3)
    A = rand_codes((7, 256), E4M3, 1)
    B = rand_codes((5, 256), E4M3, 2)
    ii, jj = all_entries(7, 5)
    one = np.ones(1, np.float32)
    val, absd, bf = orc.gemm_entries(A, B, E4M3, E4M3, TENSOR, one, one, ii, jj)
    for t, (i, j) in enumerate(zip(ii, jj)):
        exact = frac_dot(A[i], B[j], ta, ta)
        assert Fraction(val[t]) == exact                 # FP64 sum is exact here
        assert bf[t] == orc.f64_to_bf16([float(exact)])[0]
        assert Fraction(absd[t]) == sum(abs(Fraction(ta[x]) * Fraction(ta[y]))
                                        for x, y in zip(A[i], B[j]))


@pytest.mark.parametrize("fa,fb", [(E5M2, E4M3), (E4M3, E5M2), (E5M2, E5M2)])
def test_tiny_mixed_formats_within_fp64_bound(orc, fa, fb):
    ta, tb = orc.decode_table(fa), orc.decode_table(fb)
    A = rand_codes((6, 192), fa, 3)
    B = rand_codes((4, 192), fb, 4)
    sa = np.array([0.37], np.float32)
    sb = np.array([1.9], np.float32)
    ii, jj = all_entries(6, 4)
    val, absd, _ = orc.gemm_entries(A, B, fa, fb, TENSOR, sa, sb, ii, jj)
    s = Fraction(float(sa[0])) * Fraction(float(sb[0]))
    for t, (i, j) in enumerate(zip(ii, jj)):
        exact = s * frac_dot(A[i], B[j], ta, tb)
        bound = Fraction(192 + 2) * Fraction(2) ** -53 * Fraction(absd[t]) * 2
        assert abs(Fraction(val[t]) - exact) <= bound


def test_identity_weight_is_dequantise(orc):
    t = orc.decode_table(E4M3)
    K = 128
    A = rand_codes((9, K), E4M3, 5)
    c_code = 0x40                                       # 2.0
    W = np.zeros((K, K), np.uint8)
    W[np.arange(K), np.arange(K)] = c_code
    sa = np.array([0.5], np.float32)
    sb = np.array([0.25], np.float32)
    C, _, bf = orc.gemm_full(A, W, E4M3, E4M3, TENSOR, sa, sb)
    want = t[A] * 2.0 * 0.5 * 0.25
    assert np.array_equal(C, want)


def test_mx_neutral_scales_equal_plain(orc):
    A = rand_codes((12, 256), E4M3, 6)
    B = rand_codes((10, 256), E4M3, 7)
    ea = np.full((12, 8), 127, np.uint8)
    eb = np.full((10, 8), 127, np.uint8)
    one = np.ones(1, np.float32)
    Cm, _, bm = orc.gemm_full(A, B, E4M3, E4M3, MX, ea, eb)
    Ct, _, bt = orc.gemm_full(A, B, E4M3, E4M3, TENSOR, one, one)
    assert np.array_equal(Cm, Ct) and np.array_equal(bm, bt)
    # a power-of-two block scale multiplies exactly that block's contribution
    ea2 = ea.copy()
    ea2[3, 2] = 130                                     # x8 on row 3, k in [64, 96)
    Cm2, _, _ = orc.gemm_full(A, B, E4M3, E4M3, MX, ea2, eb)
    ta = orc.decode_table(E4M3)
    extra = 7.0 * (ta[A[3, 64:96]] @ ta[B[:, 64:96]].T)
    assert np.allclose(Cm2[3] - Cm[3], extra, rtol=0, atol=1e-9)
    assert np.array_equal(np.delete(Cm2, 3, 0), np.delete(Cm, 3, 0))


def test_mx_entries_exact_rational(orc):
    ta = orc.decode_table(E4M3)
    A = rand_codes((3, 96), E4M3, 8)
    B = rand_codes((2, 96), E4M3, 9)
    rng = np.random.Generator(np.random.PCG64(10))
    ea = rng.integers(120, 135, size=(3, 3)).astype(np.uint8)
    eb = rng.integers(120, 135, size=(2, 3)).astype(np.uint8)
    ii, jj = all_entries(3, 2)
    val, _, _ = orc.gemm_entries(A, B, E4M3, E4M3, MX, ea, eb, ii, jj)
    for t, (i, j) in enumerate(zip(ii, jj)):
        exact = sum(Fraction(ta[A[i, k]]) * Fraction(2) ** (int(ea[i, k // 32]) - 127) *
                    Fraction(ta[B[j, k]]) * Fraction(2) ** (int(eb[j, k // 32]) - 127)
                    for k in range(96))
        assert Fraction(val[t]) == exact


@pytest.mark.parametrize("brb", [128, 1])
def test_block_exact_and_uniform_reduction(orc, brb):
    ta = orc.decode_table(E4M3)
    K = 256
    A = rand_codes((4, K), E4M3, 11)
    B = rand_codes((256, K), E4M3, 12)
    rng = np.random.Generator(np.random.PCG64(13))
    sa = rng.uniform(0.01, 2, size=(4, 2)).astype(np.float32)
    sb = rng.uniform(0.01, 2, size=(256 // brb, 2)).astype(np.float32)
    ii = np.array([0, 1, 2, 3, 3, 0])
    jj = np.array([0, 127, 128, 255, 5, 200])
    val, _, _ = orc.gemm_entries(A, B, E4M3, E4M3, BLOCK, sa, sb, ii, jj, 1, brb)
    for t, (i, j) in enumerate(zip(ii, jj)):
        exact = sum(Fraction(float(sa[i, b])) * Fraction(float(sb[j // brb, b])) *
                    frac_dot(A[i, b * 128:(b + 1) * 128], B[j, b * 128:(b + 1) * 128], ta, ta)
                    for b in range(2))
        assert abs(Fraction(val[t]) - exact) <= abs(exact) * Fraction(2) ** -50
    Cb, _, _ = orc.gemm_full(A, B, E4M3, E4M3, BLOCK, sa, sb, 1, brb)
    vb, _, _ = orc.gemm_entries(A, B, E4M3, E4M3, BLOCK, sa, sb, *all_entries(4, 256), 1, brb)
    assert np.allclose(Cb.reshape(-1), vb, rtol=1e-14, atol=0)
    # uniform tiles reduce to per-tensor scaling
    ua = np.full((4, 2), 0.75, np.float32)
    ub = np.full((256 // brb, 2), 0.125, np.float32)
    Cu, _, _ = orc.gemm_full(A, B, E4M3, E4M3, BLOCK, ua, ub, 1, brb)
    Ct, _, _ = orc.gemm_full(A, B, E4M3, E4M3, TENSOR, np.float32([0.75]), np.float32([0.125]))
    assert np.allclose(Cu, Ct, rtol=1e-14, atol=0)


def test_layer_gemms_textbook_algebra(orc):
    """fprop, dgrad and wgrad through the oracle's transposed quantised copies
    equal the textbook products of the dequantised logical matrices."""
    from tests.test_oracle_quant import rand_bf16
    M, K, N = 24, 64, 40
    X = rand_bf16((M, K), 21, 1.0)
    Wst = rand_bf16((N, K), 22, 0.02)                   # stored [N, K] = logical W^T
    G = rand_bf16((M, N), 23, 1e-3)
    sx, six = orc.scale_from_amax(orc.amax(X), E4M3)
    sw, siw = orc.scale_from_amax(orc.amax(Wst), E4M3)
    sg, sig = orc.scale_from_amax(orc.amax(G), E5M2)
    Xq, XqT, _ = orc.quantize_tensor(X, E4M3, sx, transposed=True)
    Wq, WqT, _ = orc.quantize_tensor(Wst, E4M3, sw, transposed=True)
    Gq, GqT, _ = orc.quantize_tensor(G, E5M2, sg, transposed=True)
    t4, t5 = orc.decode_table(E4M3), orc.decode_table(E5M2)
    Xd = t4[Xq] * float(six)
    Wlog = (t4[Wq] * float(siw)).T                      # logical [K, N]
    Gd = t5[Gq] * float(sig)
    f32 = lambda v: np.array([v], np.float32)
    Y, _, _ = orc.gemm_full(Xq, Wq, E4M3, E4M3, TENSOR, f32(six), f32(siw))
    dX, _, _ = orc.gemm_full(Gq, WqT, E5M2, E4M3, TENSOR, f32(sig), f32(siw))
    dW, _, _ = orc.gemm_full(GqT, XqT, E5M2, E4M3, TENSOR, f32(sig), f32(six))
    assert np.allclose(Y, Xd @ Wlog, rtol=1e-12, atol=1e-300)
    assert np.allclose(dX, Gd @ Wlog.T, rtol=1e-12, atol=1e-300)
    assert np.allclose(dW.T, Xd.T @ Gd, rtol=1e-12, atol=1e-300)   # dW stored [N, K]
    assert Y.shape == (M, N) and dX.shape == (M, K) and dW.shape == (N, K)
