"""GPU parity of the scaled FP8 GEMMs at sizes that span several 256x256
tiles and ragged edges: every output element against the oracle, within the
MFMA error bound derived in tests/gpu_helpers.py.  Random-code operands span
the whole FP8 range (the worst case for the MFMA's aligned sum); the layer
test uses quantised Gaussian data and also holds the 2-ulp typical bar."""
import numpy as np
import pytest
import torch

from tests.gpu_helpers import (DEV, bits16, bytes8, check_gemm, check_gemm_f32, dev_bf16,
                                dev_f32, dev_u8, f32)
from tests.test_gpu_quant import rand_bits

pytestmark = pytest.mark.gpu

E4M3, E5M2 = 0, 1
TENSOR, B1, B128, MX = 0, 1, 2, 3


@pytest.fixture(scope="module")
def F():
    from scaled_fp8_gemm_amd import fp8sg
    fp8sg.lib()
    return fp8sg


def rand_codes(shape, fmt, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    c = rng.integers(0, 256, size=shape, dtype=np.int64).astype(np.uint8)
    bad = (c & 0x7F) == 0x7F if fmt == E4M3 else (c & 0x7C) == 0x7C
    c[bad] = 0x38 if fmt == E4M3 else 0x3C
    return c


def run_gemm(F, which, A, B, fa, fb, sca, scb, sa, sb, M, N, K):
    """Call fprop / dgrad / wgrad on host arrays; returns output BF16 bits."""
    Ad, Bd = dev_u8(A), dev_u8(B)
    sad = dev_u8(sa) if sca == MX else dev_f32(sa)
    sbd = dev_u8(sb) if scb == MX else dev_f32(sb)
    oa = F.operand(Ad, fa, sca, sad)
    ob = F.operand(Bd, fb, scb, sbd)
    shape = {"fprop": (M, N), "dgrad": (M, K), "wgrad": (N, K)}[which]
    out = torch.full(shape, float("nan"), dtype=torch.bfloat16, device=DEV)
    getattr(F, f"fp8_gemm_{which}")(oa, ob, M, N, K, out)
    torch.cuda.synchronize()
    return bits16(out)


# K <= 4096 spreads the next step's loads over four fragment columns; K =
# 4224 (33 steps) takes the other schedule, with ragged row and column tiles
@pytest.mark.parametrize("M,N,K", [(256, 256, 256), (600, 520, 400), (17, 33, 16), (1, 1, 128),
                                   (513, 257, 1024), (300, 700, 2048), (300, 520, 4224)])
@pytest.mark.parametrize("fa,fb", [(E4M3, E4M3), (E5M2, E4M3), (E4M3, E5M2), (E5M2, E5M2)])
def test_tensor_scaled(F, orc, M, N, K, fa, fb):
    A = rand_codes((M, K), fa, M + K)
    B = rand_codes((N, K), fb, N + 3 * K)
    sa = np.array([0.031], np.float32)
    sb = np.array([1.7e-3], np.float32)
    g = run_gemm(F, "fprop", A, B, fa, fb, TENSOR, TENSOR, sa, sb, M, N, K)
    check_gemm(orc, g, A, B, fa, fb, 0, sa, sb, label=f"tensor {M}x{N}x{K} fmt {fa}{fb}")


def test_empty_and_zero_k(F, orc):
    one = np.ones(1, np.float32)
    g = run_gemm(F, "fprop", np.zeros((0, 16), np.uint8), np.zeros((32, 16), np.uint8),
                 E4M3, E4M3, TENSOR, TENSOR, one, one, 0, 32, 16)
    assert g.size == 0
    g = run_gemm(F, "fprop", np.zeros((16, 0), np.uint8), np.zeros((48, 0), np.uint8),
                 E4M3, E4M3, TENSOR, TENSOR, one, one, 16, 48, 0)
    assert np.all(g == 0)


@pytest.mark.parametrize("sca,scb", [(B1, B128), (B1, B1), (B128, B1), (B128, B128)])
@pytest.mark.parametrize("M,N,K", [(640, 512, 384), (256, 384, 1024), (128, 128, 128)])
def test_block_scaled(F, orc, sca, scb, M, N, K):
    A = rand_codes((M, K), E4M3, 5 + M)
    B = rand_codes((N, K), E4M3, 6 + N)
    rng = np.random.Generator(np.random.PCG64(M * N))
    bra = 1 if sca == B1 else 128
    brb = 1 if scb == B1 else 128
    sa = (10.0 ** rng.uniform(-4, 1, size=(M // bra, K // 128))).astype(np.float32)
    sb = (10.0 ** rng.uniform(-4, 1, size=(N // brb, K // 128))).astype(np.float32)
    g = run_gemm(F, "fprop", A, B, E4M3, E4M3, sca, scb, sa, sb, M, N, K)
    check_gemm(orc, g, A, B, E4M3, E4M3, 1, sa, sb, bra, brb, label=f"block {sca}{scb} {M}x{N}x{K}")


# (300, 700, 1664): 13 steps, so the last chunk of four steps' scales is
# partial, with ragged row and column tiles on both operands
@pytest.mark.parametrize("M,N,K", [(600, 520, 352), (256, 256, 256), (40, 1000, 4096),
                                   (300, 700, 1664)])
@pytest.mark.parametrize("fa,fb", [(E4M3, E4M3), (E5M2, E4M3), (E4M3, E5M2)])
def test_mx_scaled(F, orc, M, N, K, fa, fb):
    A = rand_codes((M, K), fa, 7 + K)
    B = rand_codes((N, K), fb, 8 + K)
    rng = np.random.Generator(np.random.PCG64(M + N + K))
    ea = rng.integers(110, 140, size=(M, K // 32)).astype(np.uint8)
    eb = rng.integers(110, 140, size=(N, K // 32)).astype(np.uint8)
    g = run_gemm(F, "fprop", A, B, fa, fb, MX, MX, ea, eb, M, N, K)
    check_gemm(orc, g, A, B, fa, fb, 2, ea, eb, label=f"mx {M}x{N}x{K} fmt {fa}{fb}")


@pytest.mark.parametrize("K", [128, 256, 1024, 1536])
def test_mx_nan_scale_and_distinct_block_scales(F, orc, K):
    """Every 32-block has its own scale; a NaN scale (0xFF) poisons its row,
    over one, two, eight and twelve 128-K steps (the E8M0 bytes move through
    LDS in chunks of four steps)."""
    M, N = 64, 48
    A = rand_codes((M, K), E4M3, 1)
    B = rand_codes((N, K), E4M3, 2)
    ea = (117 + (np.arange(M * (K // 32)) % 20)).astype(np.uint8).reshape(M, K // 32)
    eb = (127 - (np.arange(N * (K // 32)) % 13)).astype(np.uint8).reshape(N, K // 32)
    ea[5, 3] = 0xFF
    g = run_gemm(F, "fprop", A, B, E4M3, E4M3, MX, MX, ea, eb, M, N, K)
    C, _, _ = orc.gemm_full(A, B, E4M3, E4M3, orc.SCALE_MX, ea, eb)
    assert np.all(np.isnan(C[5]))
    check_gemm(orc, g, A, B, E4M3, E4M3, 2, ea, eb, label="mx distinct scales")


@pytest.mark.parametrize("M,K,N", [(272, 384, 400), (512, 256, 768)])
def test_layer_three_gemms(F, orc, M, K, N):
    """Quantise X, W, dY on the GPU (per-tensor current scaling, transposed
    copies), run fprop / dgrad / wgrad, compare each with the oracle."""
    x = rand_bits((M, K), 1, 1.0)
    w = rand_bits((N, K), 2, 0.02)
    gr = rand_bits((M, N), 3, 1e-3)
    out = {}
    for name, t, fmt in (("x", x, E4M3), ("w", w, E4M3), ("g", gr, E5M2)):
        td = dev_bf16(t)
        R, C = t.shape
        am, s, si = (torch.empty(1, dtype=torch.float32, device=DEV) for _ in range(3))
        F.fp8_amax(td, fmt, am, s, si)
        q = torch.empty((R, C), dtype=torch.uint8, device=DEV)
        qT = torch.empty((C, R), dtype=torch.uint8, device=DEV)
        F.fp8_quantize_tensor(td, fmt, s, q, qT)
        out[name] = (q, qT, si, fmt)
        ws, wsi = orc.scale_from_amax(orc.amax(t), fmt)
        wq, wqT, _ = orc.quantize_tensor(t, fmt, ws, transposed=True)
        assert np.array_equal(bytes8(q), wq) and np.array_equal(bytes8(qT), wqT)
        assert f32(si)[0] == wsi
    (xq, xqT, xsi, _), (wq, wqT, wsi, _), (gq, gqT, gsi, _) = out["x"], out["w"], out["g"]
    T = TENSOR
    y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    F.fp8_gemm_fprop(F.operand(xq, E4M3, T, xsi), F.operand(wq, E4M3, T, wsi), M, N, K, y)
    dx = torch.empty((M, K), dtype=torch.bfloat16, device=DEV)
    F.fp8_gemm_dgrad(F.operand(gq, E5M2, T, gsi), F.operand(wqT, E4M3, T, wsi), M, N, K, dx)
    dw = torch.empty((N, K), dtype=torch.bfloat16, device=DEV)
    F.fp8_gemm_wgrad(F.operand(gqT, E5M2, T, gsi), F.operand(xqT, E4M3, T, xsi), M, N, K, dw)
    torch.cuda.synchronize()
    sx, sw, sg = f32(xsi), f32(wsi), f32(gsi)
    check_gemm(orc, bits16(y), bytes8(xq), bytes8(wq), E4M3, E4M3, 0, sx, sw, label="fprop",
               realistic=True)
    check_gemm(orc, bits16(dx), bytes8(gq), bytes8(wqT), E5M2, E4M3, 0, sg, sw, label="dgrad",
               realistic=True)
    check_gemm(orc, bits16(dw), bytes8(gqT), bytes8(xqT), E5M2, E4M3, 0, sg, sx, label="wgrad",
               realistic=True)


@pytest.mark.parametrize("M,K,N", [(256, 384, 512), (384, 256, 640)])
def test_layer_three_gemms_blockwise(F, orc, M, K, N):
    """Blockwise training step: X and G in 1x128 tiles (row-wise copies along
    their contraction, column-wise transposed copies for wgrad), W in 128x128
    blocks (and W^T for dgrad), all E4M3; fprop (1x128 x 128x128), dgrad
    (1x128 x 128x128), wgrad (1x128 x 1x128) against the oracle."""
    x = rand_bits((M, K), 31, 1.0)
    w = rand_bits((N, K), 32, 0.02)
    gr = rand_bits((M, N), 33, 1e-3)
    q = {}
    for name, t, br in (("x", x, 1), ("w", w, 128), ("g", gr, 1)):
        R, C = t.shape
        qd = torch.empty((R, C), dtype=torch.uint8, device=DEV)
        sd = torch.empty((R // br, C // 128), dtype=torch.float32, device=DEV)
        qTd = torch.empty((C, R), dtype=torch.uint8, device=DEV)
        sTd = torch.empty((C, R // 128) if br == 1 else (C // 128, R // 128), dtype=torch.float32,
                          device=DEV)
        F.fp8_quantize_block_t(dev_bf16(t), E4M3, br, qd, sd, qTd, sTd)
        q[name] = (qd, sd, qTd, sTd)
    (xq, xs, xqT, xsT), (wq, ws, wqT, wsT), (gq, gs, gqT, gsT) = q["x"], q["w"], q["g"]
    y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    F.fp8_gemm_fprop(F.operand(xq, E4M3, B1, xs), F.operand(wq, E4M3, B128, ws), M, N, K, y)
    dx = torch.empty((M, K), dtype=torch.bfloat16, device=DEV)
    F.fp8_gemm_dgrad(F.operand(gq, E4M3, B1, gs), F.operand(wqT, E4M3, B128, wsT), M, N, K, dx)
    dw = torch.empty((N, K), dtype=torch.bfloat16, device=DEV)
    F.fp8_gemm_wgrad(F.operand(gqT, E4M3, B1, gsT), F.operand(xqT, E4M3, B1, xsT), M, N, K, dw)
    torch.cuda.synchronize()
    h = lambda d: bytes8(d)
    check_gemm(orc, bits16(y), h(xq), h(wq), E4M3, E4M3, 1, f32(xs), f32(ws), 1, 128,
               label="block fprop", realistic=True)
    check_gemm(orc, bits16(dx), h(gq), h(wqT), E4M3, E4M3, 1, f32(gs), f32(wsT), 1, 128,
               label="block dgrad", realistic=True)
    check_gemm(orc, bits16(dw), h(gqT), h(xqT), E4M3, E4M3, 1, f32(gsT), f32(xsT), 1, 1,
               label="block wgrad", realistic=True)


@pytest.mark.parametrize("M,K,N", [(256, 384, 512), (320, 256, 384)])
def test_layer_three_gemms_mx(F, orc, M, K, N):
    """MXFP8 training step: 1x32 E8M0 blocks along each GEMM's contraction --
    row-wise copies for fprop / dgrad's left operand, column-wise transposed
    copies (32-token or 32-feature blocks) for W^T, G^T and X^T."""
    x = rand_bits((M, K), 41, 1.0)
    w = rand_bits((N, K), 42, 0.006)
    gr = rand_bits((M, N), 43, 1e-3)
    q = {}
    for name, t in (("x", x), ("w", w), ("g", gr)):
        R, C = t.shape
        qd = torch.empty((R, C), dtype=torch.uint8, device=DEV)
        ed = torch.empty((R, C // 32), dtype=torch.uint8, device=DEV)
        qTd = torch.empty((C, R), dtype=torch.uint8, device=DEV)
        eTd = torch.empty((C, R // 32), dtype=torch.uint8, device=DEV)
        F.fp8_quantize_mx_t(dev_bf16(t), E4M3, qd, ed, qTd, eTd)
        q[name] = (qd, ed, qTd, eTd)
    (xq, xe, xqT, xeT), (wq, we, wqT, weT), (gq, ge, gqT, geT) = q["x"], q["w"], q["g"]
    y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    F.fp8_gemm_fprop(F.operand(xq, E4M3, MX, xe), F.operand(wq, E4M3, MX, we), M, N, K, y)
    dx = torch.empty((M, K), dtype=torch.bfloat16, device=DEV)
    F.fp8_gemm_dgrad(F.operand(gq, E4M3, MX, ge), F.operand(wqT, E4M3, MX, weT), M, N, K, dx)
    dw = torch.empty((N, K), dtype=torch.bfloat16, device=DEV)
    F.fp8_gemm_wgrad(F.operand(gqT, E4M3, MX, geT), F.operand(xqT, E4M3, MX, xeT), M, N, K, dw)
    torch.cuda.synchronize()
    h = bytes8
    check_gemm(orc, bits16(y), h(xq), h(wq), E4M3, E4M3, 2, h(xe), h(we), label="mx fprop",
               realistic=True)
    check_gemm(orc, bits16(dx), h(gq), h(wqT), E4M3, E4M3, 2, h(ge), h(weT), label="mx dgrad",
               realistic=True)
    check_gemm(orc, bits16(dw), h(gqT), h(xqT), E4M3, E4M3, 2, h(geT), h(xeT), label="mx wgrad",
               realistic=True)


# wgrad's output dw[N][K]: K = 90 exercises the scalar (N % 4 != 0) store path
@pytest.mark.parametrize("scaling", ["tensor", "block", "mx", "mx_k32"])
@pytest.mark.parametrize("M,N,K", [(256, 384, 512), (384, 72, 90)])
def test_wgrad_f32_store_and_accumulate(F, orc, scaling, M, N, K):
    """FP32 wgrad: stored, then accumulated onto a previous FP32 gradient."""
    if scaling == "block" and M % 128:
        pytest.skip("1x128 blocks need a contraction that is a multiple of 128")
    if scaling == "mx_k32":
        M = 352                                   # MX contraction % 128 != 0
    fa, fb = (E5M2, E4M3) if scaling == "tensor" else (E4M3, E4M3)
    A = rand_codes((N, M), fa, 61)                # dy^T
    B = rand_codes((K, M), fb, 62)                # x^T
    rng = np.random.Generator(np.random.PCG64(63))
    if scaling == "tensor":
        sca = scb = TENSOR
        sa, sb = np.float32([0.37]), np.float32([1.75])
        mode, bra, brb = 0, 1, 1
    elif scaling == "block":
        sca = scb = B1
        sa = (rng.random((N, M // 128)) + 0.5).astype(np.float32)
        sb = (rng.random((K, M // 128)) + 0.5).astype(np.float32)
        mode, bra, brb = 1, 1, 1
    else:
        sca = scb = MX
        sa = rng.integers(120, 134, size=(N, M // 32)).astype(np.uint8)
        sb = rng.integers(120, 134, size=(K, M // 32)).astype(np.uint8)
        mode, bra, brb = 2, 1, 1
    Ad, Bd = dev_u8(A), dev_u8(B)
    sad = dev_u8(sa) if sca == MX else dev_f32(sa)
    sbd = dev_u8(sb) if scb == MX else dev_f32(sb)
    oa, ob = F.operand(Ad, fa, sca, sad), F.operand(Bd, fb, scb, sbd)
    dw = torch.full((N, K), float("nan"), dtype=torch.float32, device=DEV)
    F.fp8_gemm_wgrad_f32(oa, ob, M, N, K, dw, accumulate=False)
    torch.cuda.synchronize()
    g1 = dw.cpu().numpy().copy()
    check_gemm_f32(orc, g1, A, B, fa, fb, mode, sa, sb, bra, brb, label=f"{scaling} store")
    old = (rng.standard_normal((N, K)) * np.abs(g1).max()).astype(np.float32)
    dw.copy_(torch.from_numpy(old))
    F.fp8_gemm_wgrad_f32(oa, ob, M, N, K, dw, accumulate=True)
    torch.cuda.synchronize()
    g2 = dw.cpu().numpy()
    check_gemm_f32(orc, g2, A, B, fa, fb, mode, sa, sb, bra, brb, old=old,
                   label=f"{scaling} accumulate")
    # store then accumulate agree with one FP32 add of the stored result
    assert np.array_equal(g2, (old + g1).astype(np.float32))


@pytest.mark.parametrize("scaling", ["tensor", "block", "mx", "mx_k32"])
@pytest.mark.parametrize("yfmt", [E4M3, E5M2])
def test_fprop_fused_next_layer_quantise(F, orc, scaling, yfmt):
    """The fused epilogue writes exactly what fp8_quantize_tensor and fp8_amax
    (pinned oracle) give for the BF16 output, with and without storing it."""
    M, N, K = 600, 528, 384 if scaling != "mx_k32" else 352
    rng = np.random.Generator(np.random.PCG64(51))
    A, B = rand_codes((M, K), E4M3, 52), rand_codes((N, K), E4M3, 53)
    if scaling == "tensor":
        sca = scb = TENSOR
        sa, sb = np.float32([0.013]), np.float32([0.021])
    elif scaling == "block":
        sca, scb = B1, B128
        M, N = 640, 512
        A, B = rand_codes((M, K), E4M3, 52), rand_codes((N, K), E4M3, 53)
        sa = (rng.random((M, K // 128)) * 0.02 + 0.005).astype(np.float32)
        sb = (rng.random((N // 128, K // 128)) * 0.02 + 0.005).astype(np.float32)
    else:
        sca = scb = MX
        sa = rng.integers(118, 124, size=(M, K // 32)).astype(np.uint8)
        sb = rng.integers(118, 124, size=(N, K // 32)).astype(np.uint8)
        sa[7, 1] = 0xFF                                  # NaN scale: row 7 of y is NaN
    Ad, Bd = dev_u8(A), dev_u8(B)
    sad = dev_u8(sa) if sca == MX else dev_f32(sa)
    sbd = dev_u8(sb) if scb == MX else dev_f32(sb)
    oa, ob = F.operand(Ad, E4M3, sca, sad), F.operand(Bd, E4M3, scb, sbd)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    F.fp8_gemm_fprop(oa, ob, M, N, K, y)
    yf = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    yq = torch.empty((M, N), dtype=torch.uint8, device=DEV)
    yq2 = torch.empty((M, N), dtype=torch.uint8, device=DEV)
    am = torch.empty(1, dtype=torch.float32, device=DEV)
    ys = torch.tensor([0.75 if yfmt == E4M3 else 3.0], dtype=torch.float32, device=DEV)
    F.fp8_gemm_fprop_fused(oa, ob, M, N, K, yf, yfmt, ys, yq, am)
    F.fp8_gemm_fprop_fused(oa, ob, M, N, K, None, yfmt, ys, yq2, None)   # FP8 only
    torch.cuda.synchronize()
    yb = bits16(y)
    assert np.array_equal(bits16(yf), yb)
    wq, _, wam = orc.quantize_tensor(yb, yfmt, f32(ys)[0], want_amax=True)
    assert np.array_equal(bytes8(yq), wq) and np.array_equal(bytes8(yq2), wq)
    assert f32(am)[0].view(np.uint32) == np.float32(wam).view(np.uint32)
    if scaling.startswith("mx"):
        assert np.isnan(f32(am)[0])
    else:
        mode = {"tensor": 0, "block": 1}[scaling]
        check_gemm(orc, yb, A, B, E4M3, E4M3, mode, sa, sb, 1, 128 if scaling == "block" else 1,
                   label=f"fused {scaling}")


def test_gemm_at_the_contraction_limit(F, orc):
    """Maximum size: K = 2^23, the largest contraction the GEMM accepts (a
    256-row operand tile then spans 2^31 bytes, the edge of the kernels'
    32-bit buffer offsets).  One 256 x 256 tile of random E4M3 codes of
    magnitude 0.5 .. 7.5 (a quantised tensor's spread; full-range codes would
    let the instruction's truncation reach 1 % over 65536 steps); sampled
    outputs, including all four corners, against the oracle's FP64 values:
    the MFMA error bound, max-relative <= 1e-2 and p99 <= 2 BF16 ulp."""
    from tests.gpu_helpers import compare, entries_reference
    M = N = 256
    K = 1 << 23
    rng = np.random.Generator(np.random.PCG64(223))

    def codes(rows):
        c = rng.integers(0, 256, size=(rows, K), dtype=np.uint8)
        # random sign and mantissa, exponent field 6 .. 9 (no NaN codes)
        return (c & 0x87) | ((((c >> 3) & 3) + 6) << 3).astype(np.uint8)

    A, B = codes(M), codes(N)
    sa, sb = np.float32([0.5]), np.float32([0.25])
    y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    F.fp8_gemm_fprop(F.operand(dev_u8(A), E4M3, TENSOR, dev_f32(sa)),
                     F.operand(dev_u8(B), E4M3, TENSOR, dev_f32(sb)), M, N, K, y)
    torch.cuda.synchronize()
    ii = np.concatenate([[0, 0, M - 1, M - 1], rng.integers(0, M, 28)]).astype(np.int64)
    jj = np.concatenate([[0, N - 1, 0, N - 1], rng.integers(0, N, 28)]).astype(np.int64)
    val, absd, T, S = entries_reference(orc, A, B, E4M3, E4M3, 0, sa, sb, ii, jj, chunk=4)
    compare(orc, bits16(y)[ii, jj], val, absd, T, S, label="K = 2^23", realistic=True)


def test_gemm_output_beyond_2_31_elements(F, orc):
    """Maximum size: Y of 65792 x 32768 = 2^31 + 2^23 elements (4.3 GB of
    BF16), K = 128, so output offsets pass 2^31.  Sampled outputs (the last
    rows included) against the oracle within the MFMA bound; then the fused
    epilogue at the same size: its BF16 output equals the plain call's bit for
    bit, and its FP8 copy and amax equal the oracle's cast and amax of that
    output."""
    from tests.gpu_helpers import compare, entries_reference
    M, N, K = 65792, 32768, 128
    rng = np.random.Generator(np.random.PCG64(231))

    def codes(rows):
        c = rng.integers(0, 256, size=(rows, K), dtype=np.uint8)
        return (c & 0x87) | ((((c >> 3) & 3) + 6) << 3).astype(np.uint8)

    A, B = codes(M), codes(N)
    sa, sb = np.float32([0.5]), np.float32([0.25])
    oa = F.operand(dev_u8(A), E4M3, TENSOR, dev_f32(sa))
    ob = F.operand(dev_u8(B), E4M3, TENSOR, dev_f32(sb))
    y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    F.fp8_gemm_fprop(oa, ob, M, N, K, y)
    ii = np.concatenate([np.full(64, M - 1), rng.integers(M - 256, M, 64),
                         rng.integers(0, M, 128)]).astype(np.int64)
    jj = np.concatenate([rng.integers(0, N, 64), np.full(64, N - 1),
                         rng.integers(0, N, 128)]).astype(np.int64)
    g = bits16(y[torch.from_numpy(ii).to(DEV), torch.from_numpy(jj).to(DEV)])
    val, absd, T, S = entries_reference(orc, A, B, E4M3, E4M3, 0, sa, sb, ii, jj)
    compare(orc, g, val, absd, T, S, label="Y > 2^31 elements", realistic=True)

    yf = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    yq = torch.empty((M, N), dtype=torch.uint8, device=DEV)
    am = torch.empty(1, dtype=torch.float32, device=DEV)
    ys = torch.tensor([0.01], dtype=torch.float32, device=DEV)
    F.fp8_gemm_fprop_fused(oa, ob, M, N, K, yf, E4M3, ys, yq, am)
    torch.cuda.synchronize()
    assert bool(torch.equal(yf.view(torch.int16), y.view(torch.int16)))
    del yf
    yb = bits16(y)
    del y
    wq, _, wam = orc.quantize_tensor(yb, E4M3, f32(ys)[0], want_amax=True)
    assert f32(am)[0].view(np.uint32) == np.float32(wam).view(np.uint32)
    assert np.array_equal(bytes8(yq), wq)
