"""GPU parity at the five workloads' full sizes, in the launch configuration
the benchmark times (the same C-ABI calls, shapes and recipes):

* quantisation (FP8 bytes, transposed copies, scales, amax, E8M0 bytes,
  delayed-scaling history) is compared bit for bit on whole tensors;
* GEMM outputs are compared on sampled elements -- whole first and last rows
  and columns plus random positions -- which the oracle computes one by one,
  within the MFMA error bound of tests/gpu_helpers.py and the 2-ulp typical bar.

Inputs are the seeded synthetic tensors of scaled_fp8_gemm_amd.gen, drawn on
the GPU and copied to the host for the oracle.
"""
import numpy as np
import pytest
import torch

from scaled_fp8_gemm_amd import gen
from tests.gpu_helpers import DEV, bits16, bytes8, compare, entries_reference, f32

pytestmark = pytest.mark.gpu

E4M3, E5M2 = 0, 1
T, B1, B128, MX = 0, 1, 2, 3


@pytest.fixture(scope="module")
def F():
    from scaled_fp8_gemm_amd import fp8sg
    fp8sg.lib()
    return fp8sg


def sample_entries(R, C, seed, n_random=3000):
    rng = np.random.Generator(np.random.PCG64(seed))
    ii = [np.zeros(C, np.int64), np.full(C, R - 1), np.arange(R), np.arange(R)]
    jj = [np.arange(C), np.arange(C), np.zeros(R, np.int64), np.full(R, C - 1)]
    ii.append(rng.integers(0, R, n_random))
    jj.append(rng.integers(0, C, n_random))
    ii, jj = np.concatenate(ii), np.concatenate(jj)
    # keep the sample bounded: subsample the edge rows/cols of very wide outputs
    if ii.size > 20000:
        keep = rng.choice(ii.size, 20000, replace=False)
        ii, jj = ii[keep], jj[keep]
    return ii, jj


def check_gemm_sampled(orc, out, A, B, fa, fb, mode, sa, sb, label, bra=1, brb=1, seed=0):
    R, C = out.shape
    ii, jj = sample_entries(R, C, seed)
    g = bits16(out)[ii, jj]
    val, absd, Tb, S = entries_reference(orc, A, B, fa, fb, mode, sa, sb, ii, jj, bra, brb)
    return compare(orc, g, val, absd, Tb, S, label, realistic=True)


def empty(shape, dt):
    return torch.empty(shape, dtype=dt, device=DEV)


def quant_tensor_current(F, orc, t, fmt, label):
    """GPU amax + scale + cast of one tensor, checked bit-exactly; returns
    (q device, scale_inv device, host bytes, host scale_inv)."""
    R, C = t.shape
    am, s, si = empty(1, torch.float32), empty(1, torch.float32), empty(1, torch.float32)
    F.fp8_amax(t, fmt, am, s, si)
    q = empty((R, C), torch.uint8)
    F.fp8_quantize_tensor(t, fmt, s, q)
    tb = bits16(t)
    wa = orc.amax(tb)
    ws, wsi = orc.scale_from_amax(wa, fmt)
    assert f32(am)[0].view(np.uint32) == np.float32(wa).view(np.uint32), f"{label} amax"
    assert f32(s)[0] == ws and f32(si)[0] == wsi, f"{label} scale"
    wq, _, _ = orc.quantize_tensor(tb, fmt, ws)
    qh = bytes8(q)
    assert np.array_equal(qh, wq), f"{label} bytes"
    return q, si, qh, f32(si)


def quant_tensor_current_one_call(F, orc, t, fmt, label):
    """fp8_quantize_tensor_current (the benchmark's call), checked bit-exactly."""
    R, C = t.shape
    am, s, si = empty(1, torch.float32), empty(1, torch.float32), empty(1, torch.float32)
    q = empty((R, C), torch.uint8)
    F.fp8_quantize_tensor_current(t, fmt, q, None, am, s, si)
    tb = bits16(t)
    wa = orc.amax(tb)
    ws, wsi = orc.scale_from_amax(wa, fmt)
    assert f32(am)[0].view(np.uint32) == np.float32(wa).view(np.uint32), f"{label} amax"
    assert f32(s)[0] == ws and f32(si)[0] == wsi, f"{label} scale"
    wq, _, _ = orc.quantize_tensor(tb, fmt, ws)
    qh = bytes8(q)
    assert np.array_equal(qh, wq), f"{label} bytes"
    return q, si, qh, f32(si)


def quant_pair_current(F, orc, x, w, fmt, label):
    """fp8_quantize_pair_current of X and W (the benchmark's call), each
    checked bit-exactly; returns the quant_tensor_current tuple per tensor."""
    outs = [(empty(t.shape, torch.uint8),) + tuple(empty(1, torch.float32) for _ in range(3))
            for t in (x, w)]
    F.fp8_quantize_pair_current(x, fmt, *outs[0], w, fmt, *outs[1])
    res = []
    for t, (q, am, s, si), name in zip((x, w), outs, ("X", "W")):
        tb = bits16(t)
        wa = orc.amax(tb)
        ws, wsi = orc.scale_from_amax(wa, fmt)
        assert f32(am)[0].view(np.uint32) == np.float32(wa).view(np.uint32), f"{label} {name} amax"
        assert f32(s)[0] == ws and f32(si)[0] == wsi, f"{label} {name} scale"
        wq, _, _ = orc.quantize_tensor(tb, fmt, ws)
        qh = bytes8(q)
        assert np.array_equal(qh, wq), f"{label} {name} bytes"
        res.append((q, si, qh, f32(si)))
    return res


# tiny case: the two-call sequence; LLaMA2-7B up-projection: X and W in one
# launch (the call the benchmark times), and the one-call current scaling of
# each tensor
@pytest.mark.parametrize("key,calls", [("c1", "two"), ("c2", "pair"), ("c2", "one")])
def test_per_tensor_current_fprop(F, orc, key, calls):
    cfg = gen.CONFIGS[key]
    x = gen.make_x(cfg, DEV)
    w = gen.make_w(cfg, DEV)
    if calls == "pair":
        (xq, xsi, xh, xs), (wq, wsi, wh, ws) = quant_pair_current(F, orc, x, w, E4M3, key)
    else:
        quant = quant_tensor_current if calls == "two" else quant_tensor_current_one_call
        xq, xsi, xh, xs = quant(F, orc, x, E4M3, f"{key} X")
        wq, wsi, wh, ws = quant(F, orc, w, E4M3, f"{key} W")
    y = empty((cfg.M, cfg.N), torch.bfloat16)
    F.fp8_gemm_fprop(F.operand(xq, E4M3, T, xsi), F.operand(wq, E4M3, T, wsi),
                     cfg.M, cfg.N, cfg.K, y)
    torch.cuda.synchronize()
    check_gemm_sampled(orc, y, xh, wh, E4M3, E4M3, 0, xs, ws, f"{key} fprop", seed=1)


def test_blockwise_qkv_fprop(F, orc):
    cfg = gen.CONFIGS["c3"]
    x = gen.make_x(cfg, DEV)
    w = gen.make_w(cfg, DEV)
    M, K, N = cfg.M, cfg.K, cfg.N
    xq, xsi = empty((M, K), torch.uint8), empty((M, K // 128), torch.float32)
    wq, wsi = empty((N, K), torch.uint8), empty((N // 128, K // 128), torch.float32)
    F.fp8_quantize_block(x, E4M3, 1, 128, xq, xsi)
    F.fp8_quantize_block(w, E4M3, 128, 128, wq, wsi)
    y = empty((M, N), torch.bfloat16)
    F.fp8_gemm_fprop(F.operand(xq, E4M3, B1, xsi), F.operand(wq, E4M3, B128, wsi), M, N, K, y)
    torch.cuda.synchronize()
    oxq, oxsi = orc.quantize_block(bits16(x), E4M3, 1, 128)
    owq, owsi = orc.quantize_block(bits16(w), E4M3, 128, 128)
    assert np.array_equal(bytes8(xq), oxq) and np.array_equal(f32(xsi).view(np.uint32),
                                                              oxsi.view(np.uint32))
    assert np.array_equal(bytes8(wq), owq) and np.array_equal(f32(wsi).view(np.uint32),
                                                              owsi.view(np.uint32))
    check_gemm_sampled(orc, y, oxq, owq, E4M3, E4M3, 1, oxsi, owsi, "c3 fprop", 1, 128, seed=3)


def test_mxfp8_gpt175b_share(F, orc):
    cfg = gen.CONFIGS["c5"]
    x = gen.make_x(cfg, DEV)
    w = gen.make_w(cfg, DEV)
    M, K, N = cfg.M, cfg.K, cfg.N
    xq, xe = empty((M, K), torch.uint8), empty((M, K // 32), torch.uint8)
    wq, we = empty((N, K), torch.uint8), empty((N, K // 32), torch.uint8)
    F.fp8_quantize_mx(x, E4M3, xq, xe)
    F.fp8_quantize_mx(w, E4M3, wq, we)
    y = empty((M, N), torch.bfloat16)
    F.fp8_gemm_fprop(F.operand(xq, E4M3, MX, xe), F.operand(wq, E4M3, MX, we), M, N, K, y)
    torch.cuda.synchronize()
    del x
    oxq, oxe = orc.quantize_mx(bits16(gen.make_x(cfg, DEV)), E4M3)
    assert np.array_equal(bytes8(xq), oxq) and np.array_equal(bytes8(xe), oxe)
    wb = bits16(w)
    del w
    owq, owe = orc.quantize_mx(wb, E4M3)
    del wb
    assert np.array_equal(bytes8(we), owe)
    assert np.array_equal(bytes8(wq), owq)
    check_gemm_sampled(orc, y, oxq, owq, E4M3, E4M3, 2, oxe, owe, "c5 fprop", seed=5)


def test_delayed_training_step_16(F, orc):
    """The LLaMA2-13B-width training step over 16 seeded steps: delayed
    scaling with a 16-step history per tensor role, fused amax, transposed
    copies, fprop / dgrad / wgrad.  Every step's bytes, amax, history and
    scales are bit-exact; GEMMs are sampled at the first, a middle and the
    last step."""
    cfg = gen.CONFIGS["c4"]
    M, K, N = cfg.M, cfg.K, cfg.N
    H = 16
    w = gen.make_w(cfg, DEV)
    wb = bits16(w)
    roles = {"x": E4M3, "w": E4M3, "g": E5M2}
    hist_d = {r: torch.zeros(H, dtype=torch.float32, device=DEV) for r in roles}
    sc_d = {r: torch.ones(1, dtype=torch.float32, device=DEV) for r in roles}
    sci_d = {r: torch.ones(1, dtype=torch.float32, device=DEV) for r in roles}
    hist_h = {r: np.zeros(H, np.float32) for r in roles}
    sc_h = {r: np.float32(1.0) for r in roles}
    sci_h = {r: np.float32(1.0) for r in roles}
    shapes = {"x": (M, K), "w": (N, K), "g": (M, N)}
    q = {r: empty(shapes[r], torch.uint8) for r in roles}
    qT = {r: empty(shapes[r][::-1], torch.uint8) for r in roles}
    am = {r: empty(1, torch.float32) for r in roles}
    y, dx, dw = empty((M, N), torch.bfloat16), empty((M, K), torch.bfloat16), \
        empty((N, K), torch.bfloat16)
    for t in range(cfg.steps):
        src = {"x": gen.make_x(cfg, DEV, step=t), "w": w, "g": gen.make_g(cfg, DEV, step=t)}
        for r, fmt in roles.items():
            F.fp8_quantize_tensor(src[r], fmt, sc_d[r], q[r], qT[r], am[r])
        F.fp8_gemm_fprop(F.operand(q["x"], E4M3, T, sci_d["x"]),
                         F.operand(q["w"], E4M3, T, sci_d["w"]), M, N, K, y)
        F.fp8_gemm_dgrad(F.operand(q["g"], E5M2, T, sci_d["g"]),
                         F.operand(qT["w"], E4M3, T, sci_d["w"]), M, N, K, dx)
        F.fp8_gemm_wgrad(F.operand(qT["g"], E5M2, T, sci_d["g"]),
                         F.operand(qT["x"], E4M3, T, sci_d["x"]), M, N, K, dw)
        for r, fmt in roles.items():
            F.fp8_amax_history_update(hist_d[r], t, am[r], fmt, sc_d[r], sci_d[r])
        torch.cuda.synchronize()
        host = {}
        for r, fmt in roles.items():
            xb = wb if r == "w" else bits16(src[r])
            wq, wqT, wam = orc.quantize_tensor(xb, fmt, sc_h[r], transposed=True, want_amax=True)
            assert np.array_equal(bytes8(q[r]), wq), f"step {t} {r} bytes"
            assert np.array_equal(bytes8(qT[r]), wqT), f"step {t} {r} transposed bytes"
            assert f32(am[r])[0].view(np.uint32) == np.float32(wam).view(np.uint32), \
                f"step {t} {r} amax"
            host[r] = (wq, wqT, sci_h[r])
            sc_h[r], sci_h[r] = orc.amax_history_update(hist_h[r], t, wam, fmt)
            assert np.array_equal(f32(hist_d[r]).view(np.uint32), hist_h[r].view(np.uint32))
            assert f32(sc_d[r])[0] == sc_h[r] and f32(sci_d[r])[0] == sci_h[r], \
                f"step {t} {r} next scale"
        if t in (0, 8, cfg.steps - 1):
            s = {r: np.float32([host[r][2]]) for r in roles}
            check_gemm_sampled(orc, y, host["x"][0], host["w"][0], E4M3, E4M3, 0, s["x"], s["w"],
                               f"step {t} fprop", seed=t)
            check_gemm_sampled(orc, dx, host["g"][0], host["w"][1], E5M2, E4M3, 0, s["g"],
                               s["w"], f"step {t} dgrad", seed=t + 100)
            check_gemm_sampled(orc, dw, host["g"][1], host["x"][1], E5M2, E4M3, 0, s["g"],
                               s["x"], f"step {t} wgrad", seed=t + 200)


def test_blockwise_training_step_qkv(F, orc):
    """The blockwise recipe's training step at the QKV shape: X and G in 1x128
    tiles with column-wise transposed copies (128-token tiles) for wgrad, W in
    128x128 blocks with W^T for dgrad; every byte and scale bit-exact, GEMM
    entries sampled."""
    cfg = gen.CONFIGS["c3"]
    M, K, N = cfg.M, cfg.K, cfg.N
    out = {}
    for name, make, br in (("x", gen.make_x, 1), ("w", gen.make_w, 128), ("g", gen.make_g, 1)):
        t = make(cfg, DEV)
        R, C = t.shape
        q, qT = empty((R, C), torch.uint8), empty((C, R), torch.uint8)
        s = empty((R // br, C // 128), torch.float32)
        sT = empty((C, R // 128) if br == 1 else (C // 128, R // 128), torch.float32)
        F.fp8_quantize_block_t(t, E4M3, br, q, s, qT, sT)
        torch.cuda.synchronize()
        tb = bits16(t)
        del t
        wq, ws = orc.quantize_block(tb, E4M3, br, 128)
        if br == 1:
            wqT, wsT = orc.quantize_block(np.ascontiguousarray(tb.T), E4M3, 1, 128)
        else:
            wqT, wsT = np.ascontiguousarray(wq.T), np.ascontiguousarray(ws.T)
        del tb
        for got, want, what in ((q, wq, "q"), (qT, wqT, "qT")):
            assert np.array_equal(bytes8(got), want), f"{name} {what}"
        for got, want, what in ((s, ws, "scale_inv"), (sT, wsT, "scale_inv_T")):
            assert np.array_equal(f32(got).view(np.uint32), want.view(np.uint32)), f"{name} {what}"
        out[name] = (q, s, qT, sT, wq, ws, wqT, wsT)
    x, w, g = out["x"], out["w"], out["g"]
    y, dx, dw = empty((M, N), torch.bfloat16), empty((M, K), torch.bfloat16), \
        empty((N, K), torch.bfloat16)
    F.fp8_gemm_fprop(F.operand(x[0], E4M3, B1, x[1]), F.operand(w[0], E4M3, B128, w[1]),
                     M, N, K, y)
    F.fp8_gemm_dgrad(F.operand(g[0], E4M3, B1, g[1]), F.operand(w[2], E4M3, B128, w[3]),
                     M, N, K, dx)
    F.fp8_gemm_wgrad(F.operand(g[2], E4M3, B1, g[3]), F.operand(x[2], E4M3, B1, x[3]),
                     M, N, K, dw)
    torch.cuda.synchronize()
    check_gemm_sampled(orc, y, x[4], w[4], E4M3, E4M3, 1, x[5], w[5], "block fprop", 1, 128,
                       seed=11)
    check_gemm_sampled(orc, dx, g[4], w[6], E4M3, E4M3, 1, g[5], w[7], "block dgrad", 1, 128,
                       seed=12)
    check_gemm_sampled(orc, dw, g[6], x[6], E4M3, E4M3, 1, g[7], x[7], "block wgrad", 1, 1,
                       seed=13)


def test_mx_training_step_gpt175b_share(F, orc):
    """The MXFP8 training step at one GPU's share of the GPT-175B MLP: 1x32
    E8M0 blocks along each GEMM's contraction (row-wise copies and
    column-wise transposed copies); bytes and scale bytes bit-exact, GEMM
    entries sampled."""
    cfg = gen.CONFIGS["c5"]
    M, K, N = cfg.M, cfg.K, cfg.N
    out = {}
    for name, make in (("x", gen.make_x), ("w", gen.make_w), ("g", gen.make_g)):
        t = make(cfg, DEV)
        R, C = t.shape
        q, qT = empty((R, C), torch.uint8), empty((C, R), torch.uint8)
        e, eT = empty((R, C // 32), torch.uint8), empty((C, R // 32), torch.uint8)
        F.fp8_quantize_mx_t(t, E4M3, q, e, qT, eT)
        torch.cuda.synchronize()
        tb = bits16(t)
        del t
        wq, we = orc.quantize_mx(tb, E4M3)
        assert np.array_equal(bytes8(e), we) and np.array_equal(bytes8(q), wq), name
        tbT = np.ascontiguousarray(tb.T)
        del tb
        wqT, weT = orc.quantize_mx(tbT, E4M3)
        del tbT
        assert np.array_equal(bytes8(eT), weT) and np.array_equal(bytes8(qT), wqT), f"{name} T"
        out[name] = (q, e, qT, eT, wq, we, wqT, weT)
        torch.cuda.empty_cache()
    x, w, g = out["x"], out["w"], out["g"]
    y, dx, dw = empty((M, N), torch.bfloat16), empty((M, K), torch.bfloat16), \
        empty((N, K), torch.bfloat16)
    F.fp8_gemm_fprop(F.operand(x[0], E4M3, MX, x[1]), F.operand(w[0], E4M3, MX, w[1]),
                     M, N, K, y)
    F.fp8_gemm_dgrad(F.operand(g[0], E4M3, MX, g[1]), F.operand(w[2], E4M3, MX, w[3]),
                     M, N, K, dx)
    F.fp8_gemm_wgrad(F.operand(g[2], E4M3, MX, g[3]), F.operand(x[2], E4M3, MX, x[3]),
                     M, N, K, dw)
    torch.cuda.synchronize()
    check_gemm_sampled(orc, y, x[4], w[4], E4M3, E4M3, 2, x[5], w[5], "mx fprop", seed=21)
    check_gemm_sampled(orc, dx, g[4], w[6], E4M3, E4M3, 2, g[5], w[7], "mx dgrad", seed=22)
    check_gemm_sampled(orc, dw, g[6], x[6], E4M3, E4M3, 2, g[7], x[7], "mx wgrad", seed=23)
