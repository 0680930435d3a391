"""A whole per-tensor current-scaling step (one-launch amax+cast of X and W,
one launch per tensor or both in one, then fprop) captured in a HIP graph and
replayed.  The one-launch cast keeps a
generation number and counters in the per-stream workspace between calls, so
replays must leave them consistent: every replay's FP8 bytes, scales and BF16
output equal the eager step's bit for bit, with unrelated eager work on the
same stream between replays.  The stream is used eagerly before the capture,
so the library's workspace for it exists and nothing allocates while
capturing."""
import numpy as np
import pytest
import torch

from scaled_fp8_gemm_amd import gen
from tests.gpu_helpers import DEV, bytes8, f32

pytestmark = pytest.mark.gpu

E4M3 = 0


@pytest.fixture(scope="module")
def F():
    from scaled_fp8_gemm_amd import fp8sg
    fp8sg.lib()
    return fp8sg


@pytest.mark.parametrize("calls", ["one", "pair"])
def test_graph_replay_current_scaling_step(F, calls):
    cfg = gen.CONFIGS["c2"]
    M, K, N = 1024, cfg.K, 2048
    x = gen.make_x(cfg, DEV, M=M)
    w = gen.make_w(cfg, DEV, N=N)
    other = gen.make_x(cfg, DEV, step=1, M=512)   # eager work between replays

    def buffers():
        return dict(xq=torch.empty((M, K), dtype=torch.uint8, device=DEV),
                    wq=torch.empty((N, K), dtype=torch.uint8, device=DEV),
                    y=torch.empty((M, N), dtype=torch.bfloat16, device=DEV),
                    **{k: torch.empty(1, device=DEV) for k in ("xa", "xs", "xsi", "wa", "ws", "wsi")})

    def step(b):
        if calls == "pair":
            F.fp8_quantize_pair_current(x, E4M3, b["xq"], b["xa"], b["xs"], b["xsi"],
                                        w, E4M3, b["wq"], b["wa"], b["ws"], b["wsi"])
        else:
            F.fp8_quantize_tensor_current(x, E4M3, b["xq"], None, b["xa"], b["xs"], b["xsi"])
            F.fp8_quantize_tensor_current(w, E4M3, b["wq"], None, b["wa"], b["ws"], b["wsi"])
        F.fp8_gemm_fprop(F.operand(b["xq"], E4M3, F.SCALE_TENSOR, b["xsi"]),
                         F.operand(b["wq"], E4M3, F.SCALE_TENSOR, b["wsi"]), M, N, K, b["y"])

    def snapshot(b):
        return {k: (bytes8(v) if v.dtype == torch.uint8 else
                    v.view(torch.int16).cpu().numpy() if v.dtype == torch.bfloat16 else f32(v))
                for k, v in b.items()}

    s = torch.cuda.Stream()
    eager, cap = buffers(), buffers()
    oq = torch.empty((512, K), dtype=torch.uint8, device=DEV)
    oa, os_, osi = (torch.empty(1, device=DEV) for _ in range(3))
    with torch.cuda.stream(s):
        step(eager)                       # first use of the stream: its workspace
        step(cap)
    torch.cuda.synchronize()
    want = snapshot(eager)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step(cap)
    for rep in range(4):
        with torch.cuda.stream(s):
            for v in cap.values():
                v.zero_()
            g.replay()
            F.fp8_quantize_tensor_current(other, E4M3, oq, None, oa, os_, osi)
        torch.cuda.synchronize()
        got = snapshot(cap)
        for k in want:
            assert np.array_equal(got[k], want[k]), f"replay {rep}: {k}"
