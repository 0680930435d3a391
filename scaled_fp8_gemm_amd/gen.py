"""Seeded synthetic inputs for the FP8 scaled-GEMM workloads.

This module holds no FP8 arithmetic: it only draws BF16 tensors.  Tests,
the benchmark and the smoke check hand the same bytes to the HIP path and to
the CPU oracle.

Recipe (counter-based, so any element can be drawn independently and on any
device):

* ``splitmix64(seed + (i + 1) * 0x9E3779B97F4A7C15)`` gives 64 random bits for
  counter ``i`` (Steele, Lea and Flood's SplitMix64 finaliser, 2014);
* a uniform is ``((bits >> 11) + 0.5) * 2**-53``, in (0, 1);
* a normal is Box-Muller, ``sqrt(-2 ln u1) * cos(2 pi u2)``, with u1 and u2
  from counters ``2i`` and ``2i + 1`` of the tensor's stream;
* a Student-t with 3 degrees of freedom is ``Z0 / sqrt((Z1^2 + Z2^2 + Z3^2) / 3)``
  from four independent normal streams;
* draws are made in float64, rounded to float32 and then to bfloat16 (both
  round-to-nearest-even);
* each tensor's seed is ``splitmix64(BASE_SEED ^ fnv1a64("<config>/<tensor>/<step>"))``.

The workload table (shapes and distributions of the five measured workloads)
is ``CONFIGS``.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

BASE_SEED = 20261202
GAMMA = 0x9E3779B97F4A7C15
_M64 = (1 << 64) - 1


def _i64(c: int) -> int:
    """uint64 constant as the int64 with the same bits."""
    c &= _M64
    return c - (1 << 64) if c >= (1 << 63) else c


def _srl(z: torch.Tensor, s: int) -> torch.Tensor:
    """Logical right shift of int64 bit patterns."""
    return (z >> s) & ((1 << (64 - s)) - 1)


def splitmix64_t(z: torch.Tensor) -> torch.Tensor:
    """SplitMix64 finaliser on int64 tensors (two's-complement wrap-around)."""
    z = (z ^ _srl(z, 30)) * _i64(0xBF58476D1CE4E5B9)
    z = (z ^ _srl(z, 27)) * _i64(0x94D049BB133111EB)
    return z ^ _srl(z, 31)


def splitmix64_int(x: int) -> int:
    """Python-int SplitMix64 finaliser (used for seeds and by the tests)."""
    z = x & _M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _M64
    return z ^ (z >> 31)


def fnv1a64(s: str) -> int:
    h = 0xCBF29CE484222325
    for b in s.encode():
        h = ((h ^ b) * 0x100000001B3) & _M64
    return h


def seed_for(config: str, tensor: str, step: int = 0) -> int:
    return splitmix64_int(BASE_SEED ^ fnv1a64(f"{config}/{tensor}/{step}"))


def bits(seed: int, start: int, n: int, device) -> torch.Tensor:
    """Random 64-bit words (int64 bit patterns) for counters start .. start+n-1."""
    idx = torch.arange(start + 1, start + n + 1, dtype=torch.int64, device=device)
    z = _i64(seed) + idx * _i64(GAMMA)
    return splitmix64_t(z)


def uniform(seed: int, start: int, n: int, device) -> torch.Tensor:
    b = _srl(bits(seed, start, n, device), 11)
    return (b.to(torch.float64) + 0.5) * (2.0 ** -53)


def normal(seed: int, start: int, n: int, device) -> torch.Tensor:
    """n standard normals (float64) for element indices start .. start+n-1."""
    u = uniform(seed, 2 * start, 2 * n, device).view(n, 2)
    return torch.sqrt(-2.0 * torch.log(u[:, 0])) * torch.cos((2.0 * math.pi) * u[:, 1])


def _to_bf16(v: torch.Tensor) -> torch.Tensor:
    return v.to(torch.float32).to(torch.bfloat16)


_CHUNK = 1 << 24


def normal_bf16(shape, std: float, seed: int, device="cpu") -> torch.Tensor:
    n = int(np.prod(shape))
    out = torch.empty(n, dtype=torch.bfloat16, device=device)
    for s in range(0, n, _CHUNK):
        m = min(_CHUNK, n - s)
        out[s:s + m] = _to_bf16(normal(seed, s, m, device) * std)
    return out.view(*shape)


def student_t3_bf16(shape, scale: float, seed: int, row_mag=None, col_mag=None,
                    device="cpu") -> torch.Tensor:
    """scale * mag * t3, with optional per-row or per-column magnitudes (float64)."""
    R, C = shape
    n = R * C
    seeds = [splitmix64_int(seed ^ (j + 1)) for j in range(4)]
    out = torch.empty(n, dtype=torch.bfloat16, device=device)
    for s in range(0, n, _CHUNK):
        m = min(_CHUNK, n - s)
        z0 = normal(seeds[0], s, m, device)
        chi = sum(normal(seeds[j], s, m, device) ** 2 for j in (1, 2, 3))
        t = z0 / torch.sqrt(chi / 3.0)
        idx = torch.arange(s, s + m, device=device)
        if row_mag is not None:
            t = t * row_mag.to(device)[idx // C]
        if col_mag is not None:
            t = t * col_mag.to(device)[idx % C]
        out[s:s + m] = _to_bf16(t * scale)
    return out.view(R, C)


def log_uniform(seed: int, n: int, lo_exp: float, hi_exp: float, device="cpu") -> torch.Tensor:
    """10**U(lo_exp, hi_exp), float64."""
    u = uniform(seed, 0, n, device)
    return torch.pow(10.0, lo_exp + (hi_exp - lo_exp) * u)


def outlier_positions(seed: int, total: int, count: int) -> np.ndarray:
    """`count` distinct flat positions in [0, total), uniformly chosen (seeded)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return np.sort(rng.choice(total, size=count, replace=False))


# --------------------------------------------------------------- workloads
@dataclasses.dataclass(frozen=True)
class Config:
    key: str
    name: str
    M: int          # tokens
    K: int          # input features (contraction of fprop)
    N: int          # output features
    recipe: str     # "tensor" | "block" | "delayed" | "mx"
    steps: int = 1


CONFIGS = {
    "c1": Config("c1", "tiny per-tensor current scaling 256x256x256", 256, 256, 256, "tensor"),
    "c2": Config("c2", "LLaMA2-7B MLP up-projection fprop 4096x4096x11008, per-tensor current",
                 4096, 4096, 11008, "tensor"),
    "c3": Config("c3", "QKV projection fprop 8192x4096x12288, blockwise 1x128 / 128x128",
                 8192, 4096, 12288, "block"),
    "c4": Config("c4", "LLaMA2-13B-width linear training step 8192x5120x13824, delayed H=16",
                 8192, 5120, 13824, "delayed", steps=16),
    "c5": Config("c5", "GPT-175B MLP one-GPU share 4096x12288x49152, MXFP8 1x32",
                 4096, 12288, 49152, "mx"),
}


def make_x(cfg: Config, device="cpu", step: int = 0, M=None, K=None) -> torch.Tensor:
    """Activation X[M, K] for a workload (shape overridable for scaled-down tests)."""
    M = cfg.M if M is None else M
    K = cfg.K if K is None else K
    if cfg.recipe == "block":
        mag = log_uniform(seed_for(cfg.key, "X.mag"), K, -3.0, 2.0)
        return student_t3_bf16((M, K), 0.02, seed_for(cfg.key, "X"), col_mag=mag, device=device)
    x = normal_bf16((M, K), 1.0, seed_for(cfg.key, "X", step), device)
    if cfg.key == "c2":
        # 0.1% of the entries (round(0.001*M*K) distinct positions) scaled x50,
        # applied to the float draw before BF16 rounding.
        cnt = int(round(0.001 * M * K))
        pos = outlier_positions(seed_for(cfg.key, "X.outliers"), M * K, cnt)
        p = torch.from_numpy(pos).to(device)
        vals = _gather_normals(seed_for(cfg.key, "X", step), pos, device)
        x.view(-1)[p] = _to_bf16(vals * 50.0)
    return x


def _gather_normals(seed: int, pos: np.ndarray, device) -> torch.Tensor:
    """Normals of the stream `seed` at arbitrary element indices `pos`."""
    p = torch.from_numpy(pos.astype(np.int64)).to(device)
    b1 = _srl(splitmix64_t(_i64(seed) + (2 * p + 1) * _i64(GAMMA)), 11)
    b2 = _srl(splitmix64_t(_i64(seed) + (2 * p + 2) * _i64(GAMMA)), 11)
    u1 = (b1.to(torch.float64) + 0.5) * (2.0 ** -53)
    u2 = (b2.to(torch.float64) + 0.5) * (2.0 ** -53)
    return torch.sqrt(-2.0 * torch.log(u1)) * torch.cos((2.0 * math.pi) * u2)


W_STD = {"c1": 0.02, "c2": 0.02, "c4": 0.02, "c5": 0.006}


def make_w(cfg: Config, device="cpu", N=None, K=None) -> torch.Tensor:
    """Weight stored [N, K] (K-contiguous), i.e. the transpose of the logical [K, N]."""
    N = cfg.N if N is None else N
    K = cfg.K if K is None else K
    if cfg.recipe == "block":
        mag = log_uniform(seed_for(cfg.key, "W.mag"), N, -3.0, 2.0)
        return student_t3_bf16((N, K), 0.02, seed_for(cfg.key, "W"), row_mag=mag, device=device)
    return normal_bf16((N, K), W_STD[cfg.key], seed_for(cfg.key, "W"), device)


def make_g(cfg: Config, device="cpu", step: int = 0, M=None, N=None) -> torch.Tensor:
    """Output gradient dY[M, N] ~ N(0, 1e-3), for the training steps of every
    recipe (fresh per step)."""
    M = cfg.M if M is None else M
    N = cfg.N if N is None else N
    return normal_bf16((M, N), 1e-3, seed_for(cfg.key, "G", step), device)
