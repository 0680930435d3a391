"""Determinism and resume of the hot path at the workloads' full sizes.

* Determinism: the same inputs through the same calls give the same bytes --
  FP8 codes, scales, E8M0 bytes, amax and the BF16 GEMM outputs -- on every
  run (the path has no atomics whose order reaches a result: maxima are
  order-independent and each GEMM output element is summed by one lane in a
  fixed order).
* Resume: delayed scaling keeps its state in the amax history and the scale
  pair of each tensor role (Colossal-AI FP8 story, scaling paragraph: the
  scale comes from a window of past values; FP8 quantisation training
  guide, section "three scaling algorithms": a buffer of past maxima).
  Copying that state to the host after 8 steps, rebuilding the device
  buffers from the copy and running 8 more steps gives bit for bit what 16
  uninterrupted steps give.
"""
import numpy as np
import pytest
import torch

from scaled_fp8_gemm_amd import gen
from tests.gpu_helpers import DEV

pytestmark = pytest.mark.gpu

E4M3, E5M2 = 0, 1
T, B1, B128, MX = 0, 1, 2, 3


@pytest.fixture(scope="module")
def F():
    from scaled_fp8_gemm_amd import fp8sg
    fp8sg.lib()
    return fp8sg


def empty(shape, dt):
    return torch.empty(shape, dtype=dt, device=DEV)


def same(a: torch.Tensor, b: torch.Tensor) -> bool:
    """Bitwise equality (NaN payloads included)."""
    if a.dtype in (torch.bfloat16, torch.float16):
        a, b = a.view(torch.int16), b.view(torch.int16)
    elif a.dtype == torch.float32:
        a, b = a.view(torch.int32), b.view(torch.int32)
    return a.shape == b.shape and bool(torch.equal(a, b))


def run_c2(F, x, w):
    cfg = gen.CONFIGS["c2"]
    M, K, N = cfg.M, cfg.K, cfg.N
    o = {"xq": empty((M, K), torch.uint8), "wq": empty((N, K), torch.uint8),
         "y": empty((M, N), torch.bfloat16)}
    for k in ("xa", "xs", "xsi", "wa", "ws", "wsi"):
        o[k] = empty(1, torch.float32)
    F.fp8_quantize_pair_current(x, E4M3, o["xq"], o["xa"], o["xs"], o["xsi"],
                                w, E4M3, o["wq"], o["wa"], o["ws"], o["wsi"])
    F.fp8_gemm_fprop(F.operand(o["xq"], E4M3, T, o["xsi"]), F.operand(o["wq"], E4M3, T, o["wsi"]),
                     M, N, K, o["y"])
    torch.cuda.synchronize()
    return o


def run_c3(F, x, w):
    cfg = gen.CONFIGS["c3"]
    M, K, N = cfg.M, cfg.K, cfg.N
    o = {"xq": empty((M, K), torch.uint8), "xs": empty((M, K // 128), torch.float32),
         "wq": empty((N, K), torch.uint8), "ws": empty((N // 128, K // 128), torch.float32),
         "y": empty((M, N), torch.bfloat16)}
    F.fp8_quantize_block(x, E4M3, 1, 128, o["xq"], o["xs"])
    F.fp8_quantize_block(w, E4M3, 128, 128, o["wq"], o["ws"])
    F.fp8_gemm_fprop(F.operand(o["xq"], E4M3, B1, o["xs"]), F.operand(o["wq"], E4M3, B128, o["ws"]),
                     M, N, K, o["y"])
    torch.cuda.synchronize()
    return o


def run_c5(F, x, w):
    cfg = gen.CONFIGS["c5"]
    M, K, N = cfg.M, cfg.K, cfg.N
    o = {"xq": empty((M, K), torch.uint8), "xe": empty((M, K // 32), torch.uint8),
         "wq": empty((N, K), torch.uint8), "we": empty((N, K // 32), torch.uint8),
         "y": empty((M, N), torch.bfloat16)}
    F.fp8_quantize_mx(x, E4M3, o["xq"], o["xe"])
    F.fp8_quantize_mx(w, E4M3, o["wq"], o["we"])
    F.fp8_gemm_fprop(F.operand(o["xq"], E4M3, MX, o["xe"]), F.operand(o["wq"], E4M3, MX, o["we"]),
                     M, N, K, o["y"])
    torch.cuda.synchronize()
    return o


@pytest.mark.parametrize("key,run", [("c2", run_c2), ("c3", run_c3), ("c5", run_c5)])
def test_same_inputs_same_bytes(F, key, run):
    cfg = gen.CONFIGS[key]
    print(f"determinism {key}", flush=True)
    x = gen.make_x(cfg, DEV)
    w = gen.make_w(cfg, DEV)
    a = run(F, x, w)
    b = run(F, x, w)
    for k in a:
        assert same(a[k], b[k]), f"{key}: {k} differs between two runs"
    del a, b
    torch.cuda.empty_cache()


class Delayed:
    """Device state and buffers of the LLaMA2-13B-width delayed-scaling
    training step (16-step history per tensor role)."""

    ROLES = {"x": E4M3, "w": E4M3, "g": E5M2}

    def __init__(self, state=None):
        cfg = gen.CONFIGS["c4"]
        self.cfg = cfg
        M, K, N = cfg.M, cfg.K, cfg.N
        if state is None:
            self.hist = {r: torch.zeros(16, dtype=torch.float32, device=DEV) for r in self.ROLES}
            self.sc = {r: torch.ones(1, dtype=torch.float32, device=DEV) for r in self.ROLES}
            self.sci = {r: torch.ones(1, dtype=torch.float32, device=DEV) for r in self.ROLES}
        else:   # rebuilt from host copies
            self.hist = {r: torch.from_numpy(state["hist"][r].copy()).to(DEV) for r in self.ROLES}
            self.sc = {r: torch.from_numpy(state["sc"][r].copy()).to(DEV) for r in self.ROLES}
            self.sci = {r: torch.from_numpy(state["sci"][r].copy()).to(DEV) for r in self.ROLES}
        shapes = {"x": (M, K), "w": (N, K), "g": (M, N)}
        self.q = {r: empty(shapes[r], torch.uint8) for r in self.ROLES}
        self.qT = {r: empty(shapes[r][::-1], torch.uint8) for r in self.ROLES}
        self.am = {r: empty(1, torch.float32) for r in self.ROLES}
        self.y, self.dx, self.dw = (empty((M, N), torch.bfloat16), empty((M, K), torch.bfloat16),
                                    empty((N, K), torch.bfloat16))

    def host_state(self):
        return {"hist": {r: self.hist[r].cpu().numpy().copy() for r in self.ROLES},
                "sc": {r: self.sc[r].cpu().numpy().copy() for r in self.ROLES},
                "sci": {r: self.sci[r].cpu().numpy().copy() for r in self.ROLES}}

    def step(self, F, t, w):
        cfg = self.cfg
        M, K, N = cfg.M, cfg.K, cfg.N
        src = {"x": gen.make_x(cfg, DEV, step=t), "w": w, "g": gen.make_g(cfg, DEV, step=t)}
        for r, fmt in self.ROLES.items():
            F.fp8_quantize_tensor(src[r], fmt, self.sc[r], self.q[r], self.qT[r], self.am[r])
        F.fp8_gemm_fprop(F.operand(self.q["x"], E4M3, T, self.sci["x"]),
                         F.operand(self.q["w"], E4M3, T, self.sci["w"]), M, N, K, self.y)
        F.fp8_gemm_dgrad(F.operand(self.q["g"], E5M2, T, self.sci["g"]),
                         F.operand(self.qT["w"], E4M3, T, self.sci["w"]), M, N, K, self.dx)
        F.fp8_gemm_wgrad(F.operand(self.qT["g"], E5M2, T, self.sci["g"]),
                         F.operand(self.qT["x"], E4M3, T, self.sci["x"]), M, N, K, self.dw)
        for r, fmt in self.ROLES.items():
            F.fp8_amax_history_update(self.hist[r], t, self.am[r], fmt, self.sc[r], self.sci[r])
        torch.cuda.synchronize()
        # per-step record: amax, history and the next scale pair of each role
        return {f"{k}.{r}": getattr(self, k)[r].cpu().numpy().view(np.uint32).copy()
                for k in ("am", "hist", "sc", "sci") for r in self.ROLES}


def test_delayed_resume_after_8_steps_equals_16_straight(F):
    cfg = gen.CONFIGS["c4"]
    w = gen.make_w(cfg, DEV)
    print("resume: 16 straight steps", flush=True)
    straight = Delayed()
    rec_a = [straight.step(F, t, w) for t in range(16)]
    final_a = {"q": straight.q, "qT": straight.qT, "y": straight.y, "dx": straight.dx,
               "dw": straight.dw}

    print("resume: 8 steps, host copy, rebuild, 8 steps", flush=True)
    first = Delayed()
    rec_b = [first.step(F, t, w) for t in range(8)]
    state = first.host_state()
    del first
    torch.cuda.empty_cache()
    resumed = Delayed(state)
    rec_b += [resumed.step(F, t, w) for t in range(8, 16)]

    for t in range(16):
        for k in rec_a[t]:
            assert np.array_equal(rec_a[t][k], rec_b[t][k]), f"step {t}: {k} differs after resume"
    for k in ("q", "qT"):
        for r in Delayed.ROLES:
            assert same(final_a[k][r], getattr(resumed, k)[r]), f"step 15: {k}.{r} differs"
    for k in ("y", "dx", "dw"):
        assert same(final_a[k], getattr(resumed, k)), f"step 15: {k} differs"
    # the history really carried state: the scales after step 15 are not the
    # initial ones and the resumed run's first step used a recorded scale
    assert not np.array_equal(rec_a[15]["sc.x"], np.float32([1.0]).view(np.uint32))
    assert np.array_equal(state["sc"]["x"].view(np.uint32), rec_a[7]["sc.x"])
