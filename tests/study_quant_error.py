"""Quantisation error of the scaling recipes on the QKV workload's tensors.

The FP8 training guide (section "blockwise scaling") states that blockwise
scaling lowers the quantisation error against per-tensor scaling.  This script
measures it with the oracle only (no GPU): the relative L2 error
||x - dequant(quant(x))|| / ||x|| in FP64, for the seeded synthetic X[8192x4096]
and W[12288x4096] (Student-t(3) values with per-channel magnitudes spread over
five decades), under per-tensor current scaling, blockwise scaling (1x128
tiles for X, 128x128 blocks for W) and MXFP8 (1x32 blocks, E8M0 scales), all
E4M3.  A reported figure, not a test: run ``python -m tests.study_quant_error``
(add ``--rows N`` for a quicker run on the first N rows).
"""
from __future__ import annotations

import argparse

import numpy as np
import torch

from oracle import oracle
from scaled_fp8_gemm_amd import gen


def rel_err(x: np.ndarray, deq: np.ndarray) -> float:
    return float(np.linalg.norm(x - deq) / np.linalg.norm(x))


def study(bits: np.ndarray, block_rows: int) -> dict:
    fmt = oracle.E4M3
    x = oracle.bf16_to_f32(bits).astype(np.float64)
    table = oracle.decode_table(fmt).astype(np.float64)
    out = {}
    a = oracle.amax(bits)
    s, si = oracle.scale_from_amax(a, fmt)
    q, _, _ = oracle.quantize_tensor(bits, fmt, s)
    out["per-tensor current"] = rel_err(x, table[q] * float(si))
    q, sib = oracle.quantize_block(bits, fmt, block_rows, 128)
    sc = np.repeat(np.repeat(sib.astype(np.float64), block_rows, axis=0), 128, axis=1)
    out[f"blockwise {block_rows}x128"] = rel_err(x, table[q] * sc)
    q, e = oracle.quantize_mx(bits, fmt)
    sc = np.repeat(np.exp2(e.astype(np.float64) - 127.0), 32, axis=1)
    out["MXFP8 1x32"] = rel_err(x, table[q] * sc)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--rows", type=int, default=0, help="first N rows only (multiple of 128)")
    args = ap.parse_args()
    oracle.build()
    cfg = gen.CONFIGS["c3"]
    for name, t, br in (("X", gen.make_x(cfg), 1), ("W", gen.make_w(cfg), 128)):
        bits = t.contiguous().view(torch.int16).numpy().view(np.uint16)
        if args.rows:
            bits = bits[: args.rows]
        res = study(np.ascontiguousarray(bits), br)
        base = res["per-tensor current"]
        print(f"{name} {bits.shape[0]}x{bits.shape[1]}: " + "; ".join(
            f"{k} {v:.4e} ({(v / base - 1) * 100:+.0f} %)" for k, v in res.items()), flush=True)


if __name__ == "__main__":
    main()
