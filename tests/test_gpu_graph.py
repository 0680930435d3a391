"""Per-tensor current-scaling steps (one-launch amax+cast of X and W, one
launch per tensor or both in one, then fprop) captured in HIP graphs and
replayed.  The one-launch cast keeps a generation number and counters in the
caller's workspace between calls, so replays must leave them consistent:
every replay's FP8 bytes, scales and BF16 output equal the eager step's bit
for bit, with unrelated eager work between replays.

* a stream's very first current-scaling call, with a workspace prepared
  inside the capture, is captured and replayed (nothing is allocated or
  cleared by the library outside the graph);
* two graphs captured on one stream with workspaces of their own replay
  concurrently on two other streams;
* two graphs that share one workspace replay one after the other on
  different streams.
"""
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


def _inputs(M, N, step=0):
    cfg = gen.CONFIGS["c2"]
    return gen.make_x(cfg, DEV, step=step, M=M), gen.make_w(cfg, DEV, N=N)


def _buffers(M, N, K):
    return dict(xq=torch.empty((M, K), dtype=torch.uint8, device=DEV),
                wq=torch.empty((N, K), dtype=torch.uint8, device=DEV),
                y=torch.empty((M, N), dtype=torch.bfloat16, device=DEV),
                **{k: torch.empty(1, device=DEV) for k in ("xa", "xs", "xsi", "wa", "ws", "wsi")})


def _step(F, calls, x, w, b, ws):
    M, K = x.shape
    N = w.shape[0]
    if calls == "pair":
        F.fp8_quantize_pair_current(x, E4M3, b["xq"], b["xa"], b["xs"], b["xsi"],
                                    w, E4M3, b["wq"], b["wa"], b["ws"], b["wsi"], workspace=ws)
    else:
        F.fp8_quantize_tensor_current(x, E4M3, b["xq"], None, b["xa"], b["xs"], b["xsi"],
                                      workspace=ws)
        F.fp8_quantize_tensor_current(w, E4M3, b["wq"], None, b["wa"], b["ws"], b["wsi"],
                                      workspace=ws)
    F.fp8_gemm_fprop(F.operand(b["xq"], E4M3, F.SCALE_TENSOR, b["xsi"]),
                     F.operand(b["wq"], E4M3, F.SCALE_TENSOR, b["wsi"]), M, N, K, b["y"])


def _snapshot(b):
    return {k: (bytes8(v) if v.dtype == torch.uint8 else
                v.view(torch.int16).cpu().numpy() if v.dtype == torch.bfloat16 else f32(v))
            for k, v in b.items()}


def _assert_same(got, want, label):
    for k in want:
        assert np.array_equal(got[k], want[k]), f"{label}: {k}"


@pytest.mark.parametrize("calls", ["one", "pair"])
def test_graph_replay_current_scaling_step(F, calls):
    """The stream's first call is the captured one; its workspace is made
    and prepared (fp8_workspace_init, a kernel) inside the capture too."""
    M, K, N = 1024, gen.CONFIGS["c2"].K, 2048
    x, w = _inputs(M, N)
    other = gen.make_x(gen.CONFIGS["c2"], DEV, step=1, M=512)   # eager work between replays
    eager = _buffers(M, N, K)
    _step(F, calls, x, w, eager, F.workspace())
    torch.cuda.synchronize()
    want = _snapshot(eager)

    s = torch.cuda.Stream()
    cap = _buffers(M, N, K)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        ws_cap = torch.empty(F.WORKSPACE_BYTES, dtype=torch.uint8, device=DEV)
        F.fp8_workspace_init(ws_cap)
        _step(F, calls, x, w, cap, ws_cap)
    oq = torch.empty((512, K), dtype=torch.uint8, device=DEV)
    oa, os_, osi = (torch.empty(1, device=DEV) for _ in range(3))
    ws_other = F.workspace()
    for rep in range(4):
        with torch.cuda.stream(s):
            for v in cap.values():
                v.zero_()
            g.replay()
            F.fp8_quantize_tensor_current(other, E4M3, oq, None, oa, os_, osi, workspace=ws_other)
        torch.cuda.synchronize()
        _assert_same(_snapshot(cap), want, f"replay {rep}")


def test_two_graphs_replayed_concurrently_on_other_streams(F):
    """Two graphs captured on one stream, each with its own workspace, are
    replayed at the same time on two different streams (not the capture
    stream), several times."""
    K = gen.CONFIGS["c2"].K
    cases = [(1024, 2048, 0), (768, 1536, 3)]
    wants, caps, graphs = [], [], []
    for M, N, step in cases:
        x, w = _inputs(M, N, step)
        b = _buffers(M, N, K)
        _step(F, "pair", x, w, b, F.workspace())
        torch.cuda.synchronize()
        wants.append(_snapshot(b))
        caps.append((x, w, _buffers(M, N, K), F.workspace()))
    torch.cuda.synchronize()
    cs = torch.cuda.Stream()
    for x, w, b, ws in caps:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cs):
            _step(F, "pair", x, w, b, ws)
        graphs.append(g)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for rep in range(3):
        for _, _, b, _ in caps:
            for v in b.values():
                v.zero_()
        torch.cuda.synchronize()
        with torch.cuda.stream(s1):
            graphs[0].replay()
        with torch.cuda.stream(s2):
            graphs[1].replay()
        torch.cuda.synchronize()
        for i in range(2):
            _assert_same(_snapshot(caps[i][2]), wants[i], f"graph {i} replay {rep}")


def test_two_graphs_sharing_a_workspace_replayed_in_turn(F):
    """Two graphs that share one workspace, replayed one after the other on
    different streams: the workspace each leaves behind is ready for the
    other."""
    K = gen.CONFIGS["c2"].K
    ws = F.workspace()
    cases = [(1024, 2048, 0), (512, 1024, 5)]
    wants, caps, graphs = [], [], []
    for M, N, step in cases:
        x, w = _inputs(M, N, step)
        b = _buffers(M, N, K)
        _step(F, "one", x, w, b, ws)
        torch.cuda.synchronize()
        wants.append(_snapshot(b))
        caps.append((x, w, _buffers(M, N, K)))
    cs = torch.cuda.Stream()
    for x, w, b in caps:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cs):
            _step(F, "one", x, w, b, ws)
        graphs.append(g)
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for rep in range(4):
        for i in (0, 1):
            with torch.cuda.stream(streams[(i + rep) % 2]):
                graphs[i].replay()
            torch.cuda.synchronize()
            _assert_same(_snapshot(caps[i][2]), wants[i], f"graph {i} replay {rep}")
