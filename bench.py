"""Benchmark of the FP8 scaled-GEMM hot path on one MI355X.

One step = one pass of the path over one batch of synthetic input for the
chosen workload.  The default is the largest workload, one GPU's share of a
GPT-175B MLP under MXFP8: X[4096x12288] . W[12288x49152] (W stored
[49152x12288]), 1x32 blocks with E8M0 scales, E4M3 elements:
    MX cast of X, MX cast of W, then the block-scaled FP8 GEMM with FP32
    accumulation -> BF16 Y.
Inputs are resident in HBM before the timed region.  W is re-quantised from
its BF16 copy every step (training keeps a BF16 master and an FP8 copy).

Prints one JSON line: throughput = 2MNK / (time per step) in TFLOP/s, with
the GEMM's roofline (its average duration from HIP events recorded around
each GEMM launch on the launch stream), the algorithmic GB/s of every
quantise pass (events around each call), and the CPU oracle timed on a
bounded sample of the same workload as a baseline.  `roofline.traffic` is the
GEMM's HBM bytes per launch from the rocprofv3 FETCH_SIZE / WRITE_SIZE summary
kept under profiles/, scaled by the same counters' reading for a plain copy of
known size; it is null when that summary is missing or was taken from another
version of the GEMM source.  Unless --no-subconfigs, the line also carries
`subconfigs`: the same measurement (fewer fields) for the other workloads --
the LLaMA2-7B up-projection (per-tensor current scaling), the QKV projection
(blockwise), the LLaMA2-13B-width training step under delayed scaling and the
same step under per-tensor current scaling -- and `delayed_vs_current`, the
step-time gap between those two recipes.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--workload c2|c3|c4|c5|...]
    python bench.py --copy-calibration      # the plain copy the counters are scaled by
"""
from __future__ import annotations

import argparse
import hashlib
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
    ap.add_argument("--workload", default="c5", choices=list(SLUG))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-subconfigs", action="store_true",
                    help="time only the chosen workload")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 512 MiB device copy (counter calibration)")
    return ap.parse_args()


COPY_BYTES = 512 << 20
# file-name slug of each workload (profiles/ summaries are named by kernel + slug)
# (c3-step / c5-step: the blockwise and MXFP8 training steps -- fprop, dgrad,
# wgrad with column-wise transposed copies -- at the QKV and GPT-175B shapes)
# (c4-current: the LLaMA2-13B-width training step under per-tensor current
# scaling instead of delayed scaling, for the recipes' efficiency gap)
SLUG = {"c2": "llama7b_upproj_4096x4096x11008", "c3": "qkv_block_8192x4096x12288",
        "c4": "llama13b_step_8192x5120x13824", "c5": "gpt175b_mlp_mx_4096x12288x49152",
        "c3-step": "qkv_block_step_8192x4096x12288",
        "c5-step": "gpt175b_mlp_mx_step_4096x12288x49152",
        "c4-current": "llama13b_step_current_8192x5120x13824"}
# sources of the GEMM kernel the traffic counters describe
GEMM_SOURCES = [os.path.join(ROOT, "scaled_fp8_gemm_amd", "csrc", f)
                for f in ("gemm.hip", "gemm_common.h", "fp8_device.h")]


def gemm_source_sha256():
    h = hashlib.sha256()
    for path in GEMM_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def copy_calibration():
    """A plain device-to-device copy of COPY_BYTES, five times: FETCH_SIZE and
    WRITE_SIZE of this kernel give the counters' bytes per true byte."""
    import torch
    src = torch.empty(COPY_BYTES // 4, dtype=torch.int32, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "launches": 5}), flush=True)


def traffic_per_launch(workload):
    """HBM bytes per GEMM launch from the committed counter summary, or None.

    The summary (profiles/k_gemm8_<slug>_traffic.txt) holds key = value
    lines: gemm_source_sha256, fetch_kib, write_kib (per GEMM dispatch) and
    copy_fetch_kib, copy_write_kib (per copy of COPY_BYTES)."""
    path = os.path.join(ROOT, "profiles", f"k_gemm8_{SLUG[workload]}_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.lstrip().startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("gemm_source_sha256") != gemm_source_sha256():
        return None
    fetch_factor = float(kv["copy_fetch_kib"]) * 1024 / COPY_BYTES
    write_factor = float(kv["copy_write_kib"]) * 1024 / COPY_BYTES
    return (float(kv["fetch_kib"]) * 1024 / fetch_factor
            + float(kv["write_kib"]) * 1024 / write_factor)


class Path:
    """Device buffers and the launch sequence of one hot-path step."""

    def __init__(self, key, dev):
        import torch
        from scaled_fp8_gemm_amd import fp8sg as F
        from scaled_fp8_gemm_amd import gen
        self.F, self.torch, self.key = F, torch, key
        cfg = gen.CONFIGS[key.split("-")[0]]
        self.cfg = cfg
        # the recipe of one step: the config's own, its training step, or
        # (c4-current) the delayed step's shapes under current scaling
        if key == "c4-current":
            self.kind = "current-step"
        else:
            self.kind = cfg.recipe if "-" not in key else {"block": "block-step",
                                                           "mx": "mx-step"}[cfg.recipe]
        # workspace of the amax-producing calls (one stream, calls in order)
        self.wspace = F.workspace(dev)
        M, K, N = cfg.M, cfg.K, cfg.N
        self.M, self.K, self.N = M, K, N
        e = lambda shape, dt: torch.empty(shape, dtype=dt, device=dev)
        self.x = gen.make_x(cfg, dev)
        self.w = gen.make_w(cfg, dev)
        self.xq, self.wq = e((M, K), torch.uint8), e((N, K), torch.uint8)
        self.y = e((M, N), torch.bfloat16)
        f1 = lambda: e(1, torch.float32)
        if self.kind in ("block-step", "mx-step"):
            self.g = gen.make_g(cfg, dev)
            self.xqT, self.wqT = e((K, M), torch.uint8), e((K, N), torch.uint8)
            self.gq, self.gqT = e((M, N), torch.uint8), e((N, M), torch.uint8)
            self.dx, self.dw = e((M, K), torch.bfloat16), e((N, K), torch.bfloat16)
            self.flops = 3 * 2.0 * M * N * K
            if self.kind == "block-step":
                f32 = torch.float32
                self.xs, self.xsT = e((M, K // 128), f32), e((K, M // 128), f32)
                self.ws, self.wsT = e((N // 128, K // 128), f32), e((K // 128, N // 128), f32)
                self.gs, self.gsT = e((M, N // 128), f32), e((N, M // 128), f32)
            else:
                u8 = torch.uint8
                self.xs, self.xsT = e((M, K // 32), u8), e((K, M // 32), u8)
                self.ws, self.wsT = e((N, K // 32), u8), e((K, N // 32), u8)
                self.gs, self.gsT = e((M, N // 32), u8), e((N, M // 32), u8)
        elif cfg.recipe == "tensor":
            self.xa, self.xs, self.xsi = f1(), f1(), f1()
            self.wa, self.ws_, self.wsi = f1(), f1(), f1()
            self.flops = 2.0 * M * N * K
        elif cfg.recipe == "block":
            self.xsi = e((M, K // 128), torch.float32)
            self.wsi = e((N // 128, K // 128), torch.float32)
            self.flops = 2.0 * M * N * K
        elif cfg.recipe == "mx":
            self.xe = e((M, K // 32), torch.uint8)
            self.we = e((N, K // 32), torch.uint8)
            self.flops = 2.0 * M * N * K
        elif self.kind == "current-step":
            self.g = gen.make_g(cfg, dev)
            self.xqT, self.wqT = e((K, M), torch.uint8), e((K, N), torch.uint8)
            self.gq, self.gqT = e((M, N), torch.uint8), e((N, M), torch.uint8)
            self.dx, self.dw = e((M, K), torch.bfloat16), e((N, K), torch.bfloat16)
            self.am = {r: f1() for r in "xwg"}
            self.sc = {r: f1() for r in "xwg"}
            self.sci = {r: f1() for r in "xwg"}
            self.flops = 3 * 2.0 * M * N * K
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
        # label -> (kind, algorithmic bytes or FLOP per call, [(start, end) events])
        self.calls = {}

    def step(self, record=None):
        """One pass of the path.  record: None (no events), "gemm" (events
        around the GEMM launches only) or "all" (events around every call)."""
        F = self.F
        M, K, N = self.M, self.K, self.N
        c = lambda label, kind, work, fn, *a: self._call(record, label, kind, work, fn, *a)
        gemm = 2.0 * M * N * K
        r = self.kind
        if r in ("block-step", "mx-step"):
            blk = r == "block-step"
            E4 = F.E4M3
            if blk:
                sx, sw = F.SCALE_BLOCK_1x128, F.SCALE_BLOCK_128x128
                qt = lambda label, t, br, *out: c(
                    label, "hbm", 4 * t.numel() + 8 * t.numel() // (128 * br),
                    F.fp8_quantize_block_t, t, E4, br, *out)
                qt("block_t X", self.x, 1, self.xq, self.xs, self.xqT, self.xsT)
                qt("block_t W", self.w, 128, self.wq, self.ws, self.wqT, self.wsT)
                qt("block_t G", self.g, 1, self.gq, self.gs, self.gqT, self.gsT)
            else:
                sx = sw = F.SCALE_MX_1x32
                qt = lambda label, t, *out: c(label, "hbm", 4 * t.numel() + 2 * t.numel() // 32,
                                              F.fp8_quantize_mx_t, t, E4, *out)
                qt("mx_t X", self.x, self.xq, self.xs, self.xqT, self.xsT)
                qt("mx_t W", self.w, self.wq, self.ws, self.wqT, self.wsT)
                qt("mx_t G", self.g, self.gq, self.gs, self.gqT, self.gsT)
            sg = sx
            c("gemm fprop", "mfma", gemm, F.fp8_gemm_fprop, F.operand(self.xq, E4, sx, self.xs),
              F.operand(self.wq, E4, sw, self.ws), M, N, K, self.y)
            c("gemm dgrad", "mfma", gemm, F.fp8_gemm_dgrad, F.operand(self.gq, E4, sg, self.gs),
              F.operand(self.wqT, E4, sw, self.wsT), M, N, K, self.dx)
            c("gemm wgrad", "mfma", gemm, F.fp8_gemm_wgrad, F.operand(self.gqT, E4, sg, self.gsT),
              F.operand(self.xqT, E4, sx, self.xsT), M, N, K, self.dw)
        elif r == "tensor":
            # current scaling of both operands in one launch: each tensor's amax
            # from a grid-wide maximum of its own, then its cast, reading each
            # BF16 tensor once and writing its FP8 copy (3 B/element, the least
            # any pass can move)
            c("amax+cast X and W", "hbm", 3 * (M * K + N * K), F.fp8_quantize_pair_current,
              self.x, F.E4M3, self.xq, self.xa, self.xs, self.xsi,
              self.w, F.E4M3, self.wq, self.wa, self.ws_, self.wsi, None, self.wspace)
            c("gemm fprop", "mfma", gemm, F.fp8_gemm_fprop,
              F.operand(self.xq, F.E4M3, F.SCALE_TENSOR, self.xsi),
              F.operand(self.wq, F.E4M3, F.SCALE_TENSOR, self.wsi), M, N, K, self.y)
        elif r == "block":
            c("block 1x128 X", "hbm", 3 * M * K + 4 * M * K // 128, F.fp8_quantize_block,
              self.x, F.E4M3, 1, 128, self.xq, self.xsi)
            c("block 128x128 W", "hbm", 3 * N * K + 4 * N * K // 16384, F.fp8_quantize_block,
              self.w, F.E4M3, 128, 128, self.wq, self.wsi)
            c("gemm fprop", "mfma", gemm, F.fp8_gemm_fprop,
              F.operand(self.xq, F.E4M3, F.SCALE_BLOCK_1x128, self.xsi),
              F.operand(self.wq, F.E4M3, F.SCALE_BLOCK_128x128, self.wsi), M, N, K, self.y)
        elif r == "mx":
            c("mx X", "hbm", 3 * M * K + M * K // 32, F.fp8_quantize_mx,
              self.x, F.E4M3, self.xq, self.xe)
            c("mx W", "hbm", 3 * N * K + N * K // 32, F.fp8_quantize_mx,
              self.w, F.E4M3, self.wq, self.we)
            c("gemm fprop", "mfma", gemm, F.fp8_gemm_fprop,
              F.operand(self.xq, F.E4M3, F.SCALE_MX_1x32, self.xe),
              F.operand(self.wq, F.E4M3, F.SCALE_MX_1x32, self.we), M, N, K, self.y)
        elif r == "current-step":
            # current scaling with transposed copies: an amax pass, then the
            # cast + transposed copy, per tensor (2 + 4 bytes per element)
            T = F.SCALE_TENSOR
            for role, t, q, qT, fmt, n in (("X", self.x, self.xq, self.xqT, F.E4M3, M * K),
                                           ("W", self.w, self.wq, self.wqT, F.E4M3, N * K),
                                           ("G", self.g, self.gq, self.gqT, F.E5M2, M * N)):
                k = role.lower()
                c(f"amax, cast+T {role}", "hbm", 6 * n, F.fp8_quantize_tensor_current,
                  t, fmt, q, qT, self.am[k], self.sc[k], self.sci[k], None, self.wspace)
            self._gemms_tensor(c, gemm)
        else:
            T = F.SCALE_TENSOR
            c("cast+T+amax X", "hbm", 4 * M * K, F.fp8_quantize_tensor,
              self.x, F.E4M3, self.sc["x"], self.xq, self.xqT, self.am["x"], None, self.wspace)
            c("cast+T+amax W", "hbm", 4 * N * K, F.fp8_quantize_tensor,
              self.w, F.E4M3, self.sc["w"], self.wq, self.wqT, self.am["w"], None, self.wspace)
            c("cast+T+amax G", "hbm", 4 * M * N, F.fp8_quantize_tensor,
              self.g, F.E5M2, self.sc["g"], self.gq, self.gqT, self.am["g"], None, self.wspace)
            self._gemms_tensor(c, gemm)
            for role, fmt in (("x", F.E4M3), ("w", F.E4M3), ("g", F.E5M2)):
                c(f"history {role.upper()}", "hbm", 2 * 16 * 4, F.fp8_amax_history_update,
                  self.hist[role], self.t, self.am[role], fmt, self.sc[role], self.sci[role])
            self.t += 1

    def _gemms_tensor(self, c, gemm):
        """fprop, dgrad and wgrad of the per-tensor-scaled training step."""
        F, T = self.F, self.F.SCALE_TENSOR
        M, K, N = self.M, self.K, self.N
        c("gemm fprop", "mfma", gemm, F.fp8_gemm_fprop,
          F.operand(self.xq, F.E4M3, T, self.sci["x"]),
          F.operand(self.wq, F.E4M3, T, self.sci["w"]), M, N, K, self.y)
        c("gemm dgrad", "mfma", gemm, F.fp8_gemm_dgrad,
          F.operand(self.gq, F.E5M2, T, self.sci["g"]),
          F.operand(self.wqT, F.E4M3, T, self.sci["w"]), M, N, K, self.dx)
        c("gemm wgrad", "mfma", gemm, F.fp8_gemm_wgrad,
          F.operand(self.gqT, F.E5M2, T, self.sci["g"]),
          F.operand(self.xqT, F.E4M3, T, self.sci["x"]), M, N, K, self.dw)

    def _call(self, record, label, kind, work, fn, *args):
        if record is None or (record == "gemm" and kind != "mfma"):
            fn(*args)
            return
        e0 = self.torch.cuda.Event(enable_timing=True)
        e1 = self.torch.cuda.Event(enable_timing=True)
        e0.record()
        fn(*args)
        e1.record()
        self.calls.setdefault(label, (kind, work, []))[2].append((e0, e1))

    def summary(self, kinds=("mfma", "hbm")):
        """Per call: average duration (ms) and achieved rate."""
        out = {}
        for label, (kind, work, evs) in self.calls.items():
            if kind not in kinds:
                continue
            ms = sum(a.elapsed_time(b) for a, b in evs) / len(evs)
            if kind == "mfma":
                out[label] = {"avg_ms": round(ms, 5), "TFLOP/s": round(work / ms / 1e9, 2),
                              "frac_fp8_peak": round(work / ms / 1e9 / PEAK_FP8_TFLOPS, 4)}
            else:
                gbs = work / ms / 1e6
                out[label] = {"avg_ms": round(ms, 5), "bytes": int(work), "GB/s": round(gbs, 1),
                              "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)}
        return out


def cpu_model():
    """The host CPU's model name (first processor in /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(key, dev):
    """The oracle as it stands, on the host cores, repeated until about 10 s
    of CPU work (at least one step, at most 20).  Inputs are the same seeded
    tensors, drawn on the GPU and copied to the host.

    c2 (LLaMA2-7B up-projection): whole steps -- amax, scale and E4M3 cast of
    all of X and W (C oracle, OpenMP), then the FP64 GEMM of every output
    (numpy matmul of the decoded operands).
    c5 (GPT-175B MLP share, MXFP8): the MX cast of all of X and W (C oracle),
    then the FP64 GEMM of a 512 x 4096 block of outputs (rows 0..511, columns
    0..4095, the whole contraction), scaled to the full 4096 x 49152 output
    by its FLOP count; the time of a whole step is the cast time plus that
    scaled GEMM time."""
    import numpy as np
    import torch
    from oracle import oracle as orc
    from scaled_fp8_gemm_amd import gen
    cfg = gen.CONFIGS[key]
    M, K, N = cfg.M, cfg.K, cfg.N
    u16 = lambda t: t.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    x = u16(gen.make_x(cfg, dev))
    w = u16(gen.make_w(cfg, dev))
    orc.lib()
    t_quant = t_gemm = 0.0
    steps = 0
    gm, gn = (M, N) if key == "c2" else (512, 4096)     # GEMM block the oracle computes
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        if key == "c2":
            sx, six = orc.scale_from_amax(orc.amax(x), orc.E4M3)
            sw, siw = orc.scale_from_amax(orc.amax(w), orc.E4M3)
            xq, _, _ = orc.quantize_tensor(x, orc.E4M3, sx)
            wq, _, _ = orc.quantize_tensor(w, orc.E4M3, sw)
            t1 = time.perf_counter()
            orc.gemm_full(xq, wq, orc.E4M3, orc.E4M3, orc.SCALE_TENSOR,
                          np.float32([six]), np.float32([siw]))
        else:
            xq, xe = orc.quantize_mx(x, orc.E4M3)
            wq, we = orc.quantize_mx(w, orc.E4M3)
            t1 = time.perf_counter()
            orc.gemm_full(xq[:gm], wq[:gn], orc.E4M3, orc.E4M3, orc.SCALE_MX, xe[:gm], we[:gn])
        t2 = time.perf_counter()
        t_quant += t1 - t0
        t_gemm += t2 - t1
        steps += 1
        if t2 - t_start >= 10.0 or steps >= 20:
            break
    scale = (M * N) / (gm * gn)
    t_step = (t_quant + t_gemm * scale) / steps
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    if key == "c2":
        sample = (f"{steps} whole step(s): amax+scale+E4M3 cast of all of X[{M}x{K}] and "
                  f"W[{N}x{K}] ({t_quant / steps:.2f} s per step) + FP64 GEMM of all "
                  f"{M}x{N} outputs ({t_gemm / steps:.2f} s per step); "
                  f"{t_quant + t_gemm:.1f} s in total")
    else:
        sample = (f"{steps} step(s): MX 1x32 cast of all of X[{M}x{K}] and W[{N}x{K}] "
                  f"({t_quant / steps:.2f} s per step) + FP64 GEMM of a {gm}x{gn} block of "
                  f"the {M}x{N} output over the whole K ({t_gemm / steps:.2f} s per step, "
                  f"scaled x{scale:g} by FLOP count); {t_quant + t_gemm:.1f} s in total")
    return {"value": round(2.0 * M * N * K / t_step / 1e12, 6), "unit": "TFLOP/s",
            "cores": cores, "kind": "oracle", "cpu_model": cpu_model(), "sample": sample}


RECIPE = {"tensor": "per-tensor current scaling, E4M3 x E4M3",
          "block": "blockwise 1x128 (X) / 128x128 (W), E4M3",
          "delayed": "delayed scaling H=16, fprop+dgrad+wgrad, E4M3 / E5M2 grads",
          "current-step": "per-tensor current scaling (amax pass, then cast with transposed "
                          "copy), fprop+dgrad+wgrad, E4M3 / E5M2 grads",
          "mx": "MXFP8 1x32 E8M0, E4M3",
          "block-step": "blockwise training step: X, G 1x128 (+ column-wise 128-token "
                        "tiles for wgrad), W 128x128 (+ W^T), fprop+dgrad+wgrad, E4M3",
          "mx-step": "MXFP8 training step: 1x32 E8M0 blocks along each GEMM's "
                     "contraction (row- and column-wise copies), fprop+dgrad+wgrad, E4M3"}
KERNEL = {"tensor": "k_gemm8<tensor> (FP8 MFMA 16x16x128, 8 waves, 256x256 tile)",
          "block": "k_gemm8<block> (FP8 MFMA, per-128-K promotion on VALU)",
          "delayed": "k_gemm8<tensor> (fprop, dgrad, wgrad launches)",
          "current-step": "k_gemm8<tensor> (fprop, dgrad, wgrad launches)",
          "mx": "k_gemm8<mx> (block-scaled MFMA 16x16x128, E8M0 operands)",
          "block-step": "k_gemm8<block> (fprop, dgrad, wgrad launches)",
          "mx-step": "k_gemm8<mx> (fprop, dgrad, wgrad launches)"}


def measure(key, steps, warmup, dev):
    """Warm-up, then `steps` timed steps of workload `key`; returns the
    step's throughput, the GEMM roofline and per-call rates."""
    import torch
    p = Path(key, dev)
    # Warm-up steps run exactly as the timed ones (same event recording), so
    # one-time costs (first event records on a stream) land before the clock
    # starts; their events are discarded.
    for _ in range(warmup):
        p.step(record="gemm")
    torch.cuda.synchronize()
    p.calls = {}
    # Timed region: whole steps; events bracket the GEMM launches only (the
    # roofline kernel), on the launch stream.
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        p.step(record="gemm")
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / steps
    tflops = p.flops / (ms * 1e-3) / 1e12
    gemm_calls = p.summary(kinds=("mfma",))
    gemm_avg_ms = sum(v["avg_ms"] for v in gemm_calls.values()) / len(gemm_calls)
    flops_per_launch = 2.0 * p.M * p.N * p.K
    achieved = flops_per_launch / (gemm_avg_ms * 1e-3) / 1e12
    # Attribution pass (not part of the timed region): events around every
    # call give each quantise pass its own duration and GB/s.
    p.calls = {}
    for _ in range(min(steps, 20)):
        p.step(record="all")
    torch.cuda.synchronize()
    cfg = p.cfg
    res = {
        "value": round(tflops, 3),
        "pct_of_peak": round(100.0 * tflops / PEAK_FP8_TFLOPS, 2),
        "ms_per_step": round(ms, 5),
        "config": {"workload": (cfg.name if p.kind == cfg.recipe else
                                f"{cfg.name.split(',')[0]}, training step"
                                + (", per-tensor current scaling"
                                   if p.kind == "current-step" else "")),
                   "M": cfg.M, "K": cfg.K, "N": cfg.N, "recipe": RECIPE[p.kind]},
        "roofline": {"bound": "mfma", "kernel": KERNEL[p.kind],
                     "achieved": round(achieved, 3), "peak": PEAK_FP8_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP8_TFLOPS, 4),
                     "avg_ms": round(gemm_avg_ms, 5), "flop_per_launch": flops_per_launch,
                     "traffic": traffic_per_launch(key)},
        "calls": p.summary(),
    }
    del p
    torch.cuda.empty_cache()
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the library runs on one GPU; --gpus must be 1 "
                                   "(how the path would shard is described, not implemented)"}))
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    import torch
    dev = torch.device("cuda:0")
    head = measure(args.workload, args.steps, args.warmup, dev)
    out = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "TFLOP/s",
        "pct_of_peak": head["pct_of_peak"],
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8",
        "data": "synthetic",
        "config": head["config"],
        "roofline": head["roofline"],
        "calls": head["calls"],
        "calls_note": "per-call events from a separate pass after the timed region",
    }
    if not args.no_subconfigs:
        subs = {}
        for key in ("c2", "c3", "c4", "c4-current"):
            if key != args.workload:
                subs[key] = measure(key, args.steps, args.warmup, dev)
        if args.workload in ("c4", "c4-current"):
            subs[args.workload] = head
        out["subconfigs"] = {k: v for k, v in subs.items() if k != args.workload}
        if "c4" in subs and "c4-current" in subs:
            d, c = subs["c4"]["ms_per_step"], subs["c4-current"]["ms_per_step"]
            out["delayed_vs_current"] = {
                "workload": "LLaMA2-13B-width training step 8192x5120x13824 "
                            "(three quantise passes with transposed copies, three GEMMs)",
                "delayed_ms_per_step": d, "current_ms_per_step": c,
                "current_slower_pct": round(100.0 * (c / d - 1.0), 2)}
    if not args.no_cpu_baseline and args.workload in ("c2", "c5"):
        out["cpu_baseline"] = cpu_baseline(args.workload, dev)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
