"""Bit-exact parity of the GEMM epilogue's FP32 -> BF16 rounding.

The fp8+bf8 search-result snippet on the forward pass has the output cast
back to BF16 after the FP32 accumulation; the rounding taken is round to
nearest, ties to even.  The element-wise GEMM bound of tests/gpu_helpers.py
allows about one BF16 ulp either way, so it cannot tell that rounding from
truncation or from rounding half away from zero.  Two tests close that gap:

* exact sums: operands whose every product and partial sum is exact in FP32
  (small integers, power-of-two scales, products on the MFMA's summation
  grid), so the FP32 accumulator equals the oracle's FP64 value r exactly and
  the BF16 output must equal RNE(r) bit for bit.  The sums are steered into
  binades where a BF16 ulp is 2, 4 or 8, so a large share of them are exact
  ties or lie a quarter ulp from one; the test first shows, on the CPU, that
  its expected codes differ from truncation and from half-away rounding in
  many places, so a kernel rounding either way would fail it;
* same accumulator, two stores: on random operands, the BF16 output of a
  GEMM equals the oracle's RNE rounding of the FP32 output of the same GEMM
  (same kernel, same operands, only the epilogue's store mode differs).

Every store path is covered: the LDS-staged whole-row stores (N % 8 == 0),
the per-fragment 8-byte stores (N % 4 == 0), the scalar stores (N odd), the
fused epilogue (next-layer FP8 copy and amax), and the MXFP8 kernel for a
contraction that is not a multiple of 128.
"""
import numpy as np
import pytest
import torch

from tests.gpu_helpers import DEV, bits16, dev_f32, dev_u8
from tests.test_gpu_gemm import rand_codes

E4M3, E5M2 = 0, 1
TENSOR, B1, B128, MX = 0, 1, 2, 3


@pytest.fixture(scope="module")
def F():
    from scaled_fp8_gemm_amd import fp8sg
    fp8sg.lib()
    return fp8sg


# ---------------------------------------------------------------- CPU side
def round_bf16_variants(r: np.ndarray):
    """BF16 codes of FP32-exact values r under three roundings: nearest-even,
    truncation toward zero and nearest with ties away from zero (integer
    operations on the FP32 bits; r must be finite and exact in FP32)."""
    f = np.asarray(r, np.float64).astype(np.float32)
    assert np.array_equal(f.astype(np.float64), np.asarray(r, np.float64)), "not exact in FP32"
    b = f.view(np.uint32).astype(np.uint64)
    rne = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)
    trunc = (b >> 16).astype(np.uint16)
    away = ((b + 0x8000) >> 16).astype(np.uint16)
    return rne, trunc, away


def exact_sum_operands(R, C, Kc, seed):
    """E4M3 codes A[R][Kc], B[C][Kc] of small integers whose dot products are
    integers steered into [256, 2048): the first four contraction columns
    carry a bias of c_i * 256 (c_i in 0..4, sign per row), the rest random
    integers in [-3, 3].  Every product is an integer of magnitude <= 256,
    so it lies on the MFMA's summation grid (2^(E-13) <= 2^-5) and every
    partial sum is an integer below 2^24: exact in FP32."""
    from oracle import oracle as orc
    rng = np.random.Generator(np.random.PCG64(seed))
    a = rng.integers(-3, 4, size=(R, Kc)).astype(np.float32)
    b = rng.integers(-3, 4, size=(C, Kc)).astype(np.float32)
    cnt = rng.integers(0, 5, size=R)
    sign = np.where(rng.random(R) < 0.5, -1.0, 1.0)
    a[:, :4] = 0
    b[:, :4] = 16
    for t in range(4):
        a[:, t] = np.where(cnt > t, 16 * sign, 0)
    return orc.encode(a, E4M3), orc.encode(b, E4M3)


def expected_bits(orc, A, B, mode, sa, sb, bra=1, brb=1):
    mode_o = {0: orc.SCALE_TENSOR, 1: orc.SCALE_BLOCK, 2: orc.SCALE_MX}[mode]
    r, _, _ = orc.gemm_full(A, B, E4M3, E4M3, mode_o, sa, sb, bra, brb)
    return r, orc.f64_to_bf16(r)


def test_exact_sum_operands_separate_the_roundings(orc):
    """CPU only in effect: the expected codes of the exact-sum operands are
    RNE of values that are exact in FP32, and they differ from truncation and
    from half-away rounding often enough that either rounding fails the GPU
    tests below."""
    A, B = exact_sum_operands(300, 264, 256, 1)
    one = np.float32([1.0])
    r, want = expected_bits(orc, A, B, 0, one, one)
    rne, trunc, away = round_bf16_variants(r)
    assert np.array_equal(want, rne)
    n = r.size
    ties = np.count_nonzero(np.asarray(r, np.float32).view(np.uint32) & 0xFFFF == 0x8000)
    assert ties > 0.05 * n, ties
    assert np.count_nonzero(want != trunc) > 0.2 * n
    assert np.count_nonzero(want != away) > 0.02 * n


# ---------------------------------------------------------------- GPU side
def _call(F, entry, A, B, sca, scb, sa, sb, R, C, Kc, out_dtype=torch.bfloat16):
    """C[R][C] = A[R][Kc] . B[C][Kc]^T through one of the GEMM entry points
    (each maps its own M / N / K onto rows and contraction)."""
    sad = dev_u8(sa) if sca == MX else dev_f32(sa)
    sbd = dev_u8(sb) if scb == MX else dev_f32(sb)
    oa = F.operand(dev_u8(A), E4M3, sca, sad)
    ob = F.operand(dev_u8(B), E4M3, scb, sbd)
    out = torch.full((R, C), float("nan"), dtype=out_dtype, device=DEV)
    if entry == "fprop":            # y[M][N], contraction K
        F.fp8_gemm_fprop(oa, ob, R, C, Kc, out)
    elif entry == "dgrad":          # dx[M][K], contraction N
        F.fp8_gemm_dgrad(oa, ob, R, Kc, C, out)
    elif entry == "wgrad":          # dw[N][K], contraction M
        F.fp8_gemm_wgrad(oa, ob, Kc, R, C, out)
    elif entry == "wgrad_f32":
        F.fp8_gemm_wgrad_f32(oa, ob, Kc, R, C, out, accumulate=False)
    else:                           # fused: BF16 y plus its FP8 copy and amax
        am = torch.empty(1, dtype=torch.float32, device=DEV)
        ys = torch.ones(1, dtype=torch.float32, device=DEV)
        yq = torch.empty((R, C), dtype=torch.uint8, device=DEV)
        F.fp8_gemm_fprop_fused(oa, ob, R, C, Kc, out, E4M3, ys, yq, am)
    torch.cuda.synchronize()
    return out


def _scales(scaling, R, C, Kc, rng):
    """Power-of-two scales (exact products) of the scaling family:
    (scaling of A, of B, scales of A, of B, oracle mode, rows per A scale,
    rows per B scale)."""
    if scaling == "tensor":
        return TENSOR, TENSOR, np.float32([0.125]), np.float32([2.0]), 0, 1, 1
    if scaling == "block":
        sa = np.ldexp(1.0, rng.integers(-2, 2, size=(R, Kc // 128))).astype(np.float32)
        sb = np.ldexp(1.0, rng.integers(-2, 2, size=(C // 128, Kc // 128))).astype(np.float32)
        return B1, B128, sa, sb, 1, 1, 128
    ea = rng.integers(126, 129, size=(R, Kc // 32)).astype(np.uint8)
    eb = rng.integers(126, 129, size=(C, Kc // 32)).astype(np.uint8)
    return MX, MX, ea, eb, 2, 1, 1


@pytest.mark.gpu
@pytest.mark.parametrize("entry", ["fprop", "dgrad", "wgrad", "fused"])
@pytest.mark.parametrize("scaling,R,C,Kc", [
    ("tensor", 300, 272, 256),     # LDS-staged whole-row stores, ragged tiles
    ("tensor", 300, 260, 256),     # 8-byte fragment stores (C % 8 == 4)
    ("tensor", 299, 261, 128),     # scalar stores (C odd)
    ("block", 300, 384, 256),      # 1x128 x 128x128 block scales
    ("mx", 300, 272, 256),         # block-scaled MFMA
    ("mx", 300, 260, 160),         # MX kernel for a contraction % 128 != 0
    ("mx", 300, 272, 160),         # the same, whole 16-column groups (fused)
])
def test_exact_sums_round_to_nearest_even(F, orc, entry, scaling, R, C, Kc):
    if entry == "fused" and C % 16:
        pytest.skip("the fused epilogue needs N % 16 == 0")
    rng = np.random.Generator(np.random.PCG64(R * 7 + C + Kc))
    A, B = exact_sum_operands(R, C, Kc, R + 3 * C + Kc)
    sca, scb, sa, sb, mode, bra, brb = _scales(scaling, R, C, Kc, rng)
    r, want = expected_bits(orc, A, B, mode, sa, sb, bra, brb)
    rne, trunc, _ = round_bf16_variants(r)        # r is exact in FP32 by construction
    assert np.array_equal(want, rne)
    assert np.count_nonzero(want != trunc) > 0.1 * r.size
    print(f"epilogue exact sums: {entry} {scaling} {R}x{C}x{Kc}", flush=True)
    g = bits16(_call(F, entry, A, B, sca, scb, sa, sb, R, C, Kc))
    bad = np.argwhere(g != want)
    assert bad.size == 0, (f"{entry} {scaling} {R}x{C}x{Kc}: {len(bad)} outputs not RNE; first "
                           f"{tuple(bad[0])}: gpu 0x{int(g[tuple(bad[0])]):04x} want "
                           f"0x{int(want[tuple(bad[0])]):04x} (exact {r[tuple(bad[0])]})")
    if entry == "wgrad":
        # the FP32 store of the same accumulator is the exact sum itself
        o32 = _call(F, "wgrad_f32", A, B, sca, scb, sa, sb, R, C, Kc, torch.float32)
        assert np.array_equal(o32.cpu().numpy().astype(np.float64), r)


@pytest.mark.gpu
@pytest.mark.parametrize("scaling,R,C,Kc", [
    ("tensor", 600, 520, 384),     # LDS-staged stores (C % 8 == 0)
    ("tensor", 300, 268, 256),     # fragment stores
    ("tensor", 257, 131, 128),     # scalar stores
    ("block", 512, 384, 384),
    ("mx", 520, 264, 512),
    ("mx", 300, 261, 352),         # MX kernel for a contraction % 128 != 0, C odd
])
def test_bf16_output_is_rne_of_fp32_output(F, orc, scaling, R, C, Kc):
    """Random full-range operands: wgrad's BF16 output equals the oracle's
    RNE rounding of wgrad_f32's output for the same operands, element by
    element (the FP32 accumulator is the kernel's; only the store differs)."""
    A = rand_codes((R, Kc), E4M3, 91 + R)
    B = rand_codes((C, Kc), E4M3, 92 + C)
    rng = np.random.Generator(np.random.PCG64(93))
    if scaling == "tensor":
        sca, scb, sa, sb = TENSOR, TENSOR, np.float32([0.0371]), np.float32([1.9e-3])
    elif scaling == "block":
        sca, scb = B1, B1
        sa = (10.0 ** rng.uniform(-3, 1, size=(R, Kc // 128))).astype(np.float32)
        sb = (10.0 ** rng.uniform(-3, 1, size=(C, Kc // 128))).astype(np.float32)
    else:
        sca, scb = MX, MX
        sa = rng.integers(115, 135, size=(R, Kc // 32)).astype(np.uint8)
        sb = rng.integers(115, 135, size=(C, Kc // 32)).astype(np.uint8)
    sad = dev_u8(sa) if sca == MX else dev_f32(sa)
    sbd = dev_u8(sb) if scb == MX else dev_f32(sb)
    oa = F.operand(dev_u8(A), E4M3, sca, sad)
    ob = F.operand(dev_u8(B), E4M3, scb, sbd)
    yb = torch.full((R, C), float("nan"), dtype=torch.bfloat16, device=DEV)
    yf = torch.full((R, C), float("nan"), dtype=torch.float32, device=DEV)
    # wgrad contracts over M: dyT[N][M] . xT[K][M]^T -> dw[N][K]
    F.fp8_gemm_wgrad(oa, ob, Kc, R, C, yb)
    F.fp8_gemm_wgrad_f32(oa, ob, Kc, R, C, yf, accumulate=False)
    torch.cuda.synchronize()
    f = yf.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(f))
    want = orc.f64_to_bf16(f)
    g = bits16(yb)
    bad = np.argwhere(g != want)
    assert bad.size == 0, (f"{scaling} {R}x{C}x{Kc}: {len(bad)} BF16 outputs are not the RNE "
                           f"of the FP32 output; first {tuple(bad[0])}: bf16 "
                           f"0x{int(g[tuple(bad[0])]):04x}, fp32 {f[tuple(bad[0])]!r}")
    # the comparison separates the roundings: most FP32 values are not BF16
    _, trunc, _ = round_bf16_variants(f)
    assert np.count_nonzero(want != trunc) > 0.2 * f.size
