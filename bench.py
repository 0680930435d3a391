"""Benchmark of the FP8 scaled-GEMM hot path on one MI355X.

One step = one pass of the path over one batch of synthetic input for the
chosen workload (default: the LLaMA2-7B MLP up-projection fprop,
X[4096x4096] . W[4096x11008], per-tensor current scaling, E4M3):
    amax(X) -> scale pair, amax(W) -> scale pair,
    cast X, cast W (E4M3), FP8 GEMM with FP32 accumulation -> BF16 Y.
Inputs are resident in HBM before the timed region.  W is re-quantised from
its BF16 copy every step (training keeps a BF16 master and an FP8 copy).

Prints one JSON line: throughput = 2MNK / (time per step) in TFLOP/s, with
the GEMM's roofline (its average duration from HIP events recorded around
each GEMM launch on the launch stream) and the CPU oracle timed on a bounded
sample of the same workload as a baseline.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--workload c2|c3|c4|c5]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "FP8 scaled-GEMM TFLOP/s incl. quantise, % of MI355X FP8 MFMA peak"
PEAK_FP8_TFLOPS = 5000.0        # MI355X dense FP8 MFMA (published)
PEAK_HBM_GBS = 8000.0           # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="c2", choices=["c2", "c3", "c4", "c5"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    return ap.parse_args()


class Path:
    """Device buffers and the launch sequence of one hot-path step."""

    def __init__(self, key, dev):
        import torch
        from scaled_fp8_gemm_amd import fp8sg as F
        from scaled_fp8_gemm_amd import gen
        self.F, self.torch, self.key = F, torch, key
        cfg = gen.CONFIGS[key]
        self.cfg = cfg
        M, K, N = cfg.M, cfg.K, cfg.N
        self.M, self.K, self.N = M, K, N
        e = lambda shape, dt: torch.empty(shape, dtype=dt, device=dev)
        self.x = gen.make_x(cfg, dev)
        self.w = gen.make_w(cfg, dev)
        self.xq, self.wq = e((M, K), torch.uint8), e((N, K), torch.uint8)
        self.y = e((M, N), torch.bfloat16)
        f1 = lambda: e(1, torch.float32)
        if cfg.recipe == "tensor":
            self.xa, self.xs, self.xsi = f1(), f1(), f1()
            self.wa, self.ws, self.wsi = f1(), f1(), f1()
            self.flops = 2.0 * M * N * K
        elif cfg.recipe == "block":
            self.xsi = e((M, K // 128), torch.float32)
            self.wsi = e((N // 128, K // 128), torch.float32)
            self.flops = 2.0 * M * N * K
        elif cfg.recipe == "mx":
            self.xe = e((M, K // 32), torch.uint8)
            self.we = e((N, K // 32), torch.uint8)
            self.flops = 2.0 * M * N * K
        else:  # delayed: one training step (fprop, dgrad, wgrad)
            self.g = gen.make_g(cfg, dev)
            self.xqT, self.wqT = e((K, M), torch.uint8), e((K, N), torch.uint8)
            self.gq, self.gqT = e((M, N), torch.uint8), e((N, M), torch.uint8)
            self.dx, self.dw = e((M, K), torch.bfloat16), e((N, K), torch.bfloat16)
            self.hist = {r: torch.zeros(16, dtype=torch.float32, device=dev) for r in "xwg"}
            self.sc = {r: torch.ones(1, dtype=torch.float32, device=dev) for r in "xwg"}
            self.sci = {r: torch.ones(1, dtype=torch.float32, device=dev) for r in "xwg"}
            self.am = {r: f1() for r in "xwg"}
            self.flops = 3 * 2.0 * M * N * K
            self.t = 0
        self.gemm_events = []

    def step(self, record=False):
        F, torch = self.F, self.torch
        M, K, N = self.M, self.K, self.N
        rec = self.gemm_events if record else None
        r = self.cfg.recipe
        if r == "tensor":
            F.fp8_amax(self.x, F.E4M3, self.xa, self.xs, self.xsi)
            F.fp8_amax(self.w, F.E4M3, self.wa, self.ws, self.wsi)
            F.fp8_quantize_tensor(self.x, F.E4M3, self.xs, self.xq)
            F.fp8_quantize_tensor(self.w, F.E4M3, self.ws, self.wq)
            self._gemm(rec, F.fp8_gemm_fprop,
                       F.operand(self.xq, F.E4M3, F.SCALE_TENSOR, self.xsi),
                       F.operand(self.wq, F.E4M3, F.SCALE_TENSOR, self.wsi), M, N, K, self.y)
        elif r == "block":
            F.fp8_quantize_block(self.x, F.E4M3, 1, 128, self.xq, self.xsi)
            F.fp8_quantize_block(self.w, F.E4M3, 128, 128, self.wq, self.wsi)
            self._gemm(rec, F.fp8_gemm_fprop,
                       F.operand(self.xq, F.E4M3, F.SCALE_BLOCK_1x128, self.xsi),
                       F.operand(self.wq, F.E4M3, F.SCALE_BLOCK_128x128, self.wsi),
                       M, N, K, self.y)
        elif r == "mx":
            F.fp8_quantize_mx(self.x, F.E4M3, self.xq, self.xe)
            F.fp8_quantize_mx(self.w, F.E4M3, self.wq, self.we)
            self._gemm(rec, F.fp8_gemm_fprop,
                       F.operand(self.xq, F.E4M3, F.SCALE_MX_1x32, self.xe),
                       F.operand(self.wq, F.E4M3, F.SCALE_MX_1x32, self.we), M, N, K, self.y)
        else:
            T = F.SCALE_TENSOR
            F.fp8_quantize_tensor(self.x, F.E4M3, self.sc["x"], self.xq, self.xqT, self.am["x"])
            F.fp8_quantize_tensor(self.w, F.E4M3, self.sc["w"], self.wq, self.wqT, self.am["w"])
            F.fp8_quantize_tensor(self.g, F.E5M2, self.sc["g"], self.gq, self.gqT, self.am["g"])
            self._gemm(rec, F.fp8_gemm_fprop, F.operand(self.xq, F.E4M3, T, self.sci["x"]),
                       F.operand(self.wq, F.E4M3, T, self.sci["w"]), M, N, K, self.y)
            self._gemm(rec, F.fp8_gemm_dgrad, F.operand(self.gq, F.E5M2, T, self.sci["g"]),
                       F.operand(self.wqT, F.E4M3, T, self.sci["w"]), M, N, K, self.dx)
            self._gemm(rec, F.fp8_gemm_wgrad, F.operand(self.gqT, F.E5M2, T, self.sci["g"]),
                       F.operand(self.xqT, F.E4M3, T, self.sci["x"]), M, N, K, self.dw)
            for role, fmt in (("x", F.E4M3), ("w", F.E4M3), ("g", F.E5M2)):
                F.fp8_amax_history_update(self.hist[role], self.t, self.am[role], fmt,
                                          self.sc[role], self.sci[role])
            self.t += 1

    def _gemm(self, rec, fn, a, b, M, N, K, out):
        if rec is None:
            fn(a, b, M, N, K, out)
            return
        e0 = self.torch.cuda.Event(enable_timing=True)
        e1 = self.torch.cuda.Event(enable_timing=True)
        e0.record()
        fn(a, b, M, N, K, out)
        e1.record()
        rec.append((e0, e1))


def cpu_baseline(key):
    """The oracle as it stands, on a bounded sample of the same workload:
    amax, scale and cast of the whole X and W (C oracle, OpenMP), and the
    GEMM for a sample of output rows (numpy FP64 matmul of the decoded
    operands); the step time is extrapolated to all rows."""
    import numpy as np
    import torch
    from oracle import oracle as orc
    from scaled_fp8_gemm_amd import gen
    cfg = gen.CONFIGS[key]
    M, K, N = cfg.M, cfg.K, cfg.N
    x = gen.make_x(cfg, "cpu").view(torch.int16).numpy().view(np.uint16)
    w = gen.make_w(cfg, "cpu").view(torch.int16).numpy().view(np.uint16)
    orc.lib()
    rows = 256
    t0 = time.perf_counter()
    sx, six = orc.scale_from_amax(orc.amax(x), orc.E4M3)
    sw, siw = orc.scale_from_amax(orc.amax(w), orc.E4M3)
    xq, _, _ = orc.quantize_tensor(x, orc.E4M3, sx)
    wq, _, _ = orc.quantize_tensor(w, orc.E4M3, sw)
    t1 = time.perf_counter()
    orc.gemm_full(xq[:rows], wq, orc.E4M3, orc.E4M3, orc.SCALE_TENSOR,
                  np.float32([six]), np.float32([siw]))
    t2 = time.perf_counter()
    t_step = (t1 - t0) + (t2 - t1) * (M / rows)
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": round(2.0 * M * N * K / t_step / 1e12, 6), "unit": "TFLOP/s",
            "cores": cores, "kind": "oracle",
            "sample": (f"amax+scale+E4M3 cast of all of X[{M}x{K}] and W[{N}x{K}] "
                       f"({t1 - t0:.2f} s) + FP64 GEMM of {rows} of {M} output rows "
                       f"({t2 - t1:.2f} s), extrapolated to the full step "
                       f"({t_step:.1f} s)")}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus must be 1 "
                                   "(the multi-GPU sharding is described, not built)"}))
        sys.exit(2)
    import torch
    dev = torch.device("cuda:0")
    p = Path(args.workload, dev)
    for _ in range(args.warmup):
        p.step()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        p.step(record=True)
    stop.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    ms = total_ms / args.steps
    tflops = p.flops / (ms * 1e-3) / 1e12
    gemm_ms = [a.elapsed_time(b) for a, b in p.gemm_events]
    gemm_avg_ms = sum(gemm_ms) / len(gemm_ms)
    flops_per_launch = 2.0 * p.M * p.N * p.K
    achieved = flops_per_launch / (gemm_avg_ms * 1e-3) / 1e12
    cfg = p.cfg
    recipe = {"tensor": "per-tensor current scaling, E4M3 x E4M3",
              "block": "blockwise 1x128 (X) / 128x128 (W), E4M3",
              "delayed": "delayed scaling H=16, fprop+dgrad+wgrad, E4M3 / E5M2 grads",
              "mx": "MXFP8 1x32 E8M0, E4M3"}[cfg.recipe]
    out = {
        "metric": METRIC,
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "pct_of_peak": round(100.0 * tflops / PEAK_FP8_TFLOPS, 2),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8",
        "data": "synthetic",
        "config": {"workload": cfg.name, "M": cfg.M, "K": cfg.K, "N": cfg.N, "recipe": recipe},
        "roofline": {"bound": "mfma", "kernel": "k_gemm (FP8 MFMA GEMM)",
                     "achieved": round(achieved, 3), "peak": PEAK_FP8_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP8_TFLOPS, 4),
                     "avg_ms": round(gemm_avg_ms, 5), "traffic": None},
    }
    if not args.no_cpu_baseline and args.workload in ("c2",):
        out["cpu_baseline"] = cpu_baseline(args.workload)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
