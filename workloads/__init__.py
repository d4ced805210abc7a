"""Seeded synthetic inputs for the W4A8 / W4FP8 GEMM workloads.

This module only draws random numbers and describes shapes.  It performs
none of the quantisation or GEMM arithmetic; both the CPU oracle and the
HIP path receive the float32 arrays it returns.

Distributions (LiquidGEMM, Pith review of arXiv 2509.01229, "The reading"
and the referee summary name LLaMA2-7B/70B linear layers as the workload;
FireQ, arXiv 2505.20839, abstract, motivates activation outlier channels):

* weights  W[N][K] ~ Normal(mean 0, std 0.02), float32;
* activations X[M][K] ~ Normal(0, 1), float32, with round(1 % of K)
  distinct K-channels (the same channels for every token) multiplied by 20.

Seeds: numpy PCG64 via ``default_rng(1000*cfg + t)`` with t = 1 for W
(plus 10 per further (N, K) pair of the same config),
t = 2 for X and t = 3 for the outlier channel set; a sweep over M draws X
from ``1000*cfg + 100 + M`` so every M has its own reproducible tokens.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

W_STD = 0.02
OUTLIER_FRAC = 0.01
OUTLIER_SCALE = 20.0


@dataclass(frozen=True)
class Shape:
    """One GEMM: Y[M][N] = X[M][K] . W[N][K]^T with K-groups of ``group``."""
    M: int
    N: int
    K: int
    group: int = 64
    name: str = ""


@dataclass(frozen=True)
class Config:
    cfg: int
    name: str
    shapes: tuple = field(default_factory=tuple)
    fp8: bool = False


def _sweep(cfg, name, Ms, NK, group):
    out = []
    for (N, K, tag) in NK:
        for M in Ms:
            out.append(Shape(M, N, K, group, f"{name}:{tag}:M{M}"))
    return tuple(out)


# Workload ids (they also select the seeds below).
TINY = 0               # one small GEMM the oracle finishes at once
LLAMA7B_DECODE = 1     # Llama-2-7B attention projections, 1-16 tokens
LLAMA7B_PREFILL = 2    # Llama-2-7B MLP, 2048 tokens
LLAMA70B_SWEEP = 3     # Llama-2-70B MLP, 1 .. 4096 tokens
FP8_VARIANT = 4        # INT4 x FP8, 2048 x 8192 x 8192

# Workloads: the Llama-2 linear-layer shapes (7B: hidden 4096, MLP 11008;
# 70B: hidden 8192, MLP 28672) at decode and prefill token counts.
CONFIGS = {
    TINY: Config(TINY, "tiny", (Shape(16, 256, 512, 64, "tiny:M16"),)),
    LLAMA7B_DECODE: Config(LLAMA7B_DECODE, "llama2-7b attn-proj decode",
                           _sweep(LLAMA7B_DECODE, "7b-attn", (1, 4, 16),
                                  ((4096, 4096, "qkvo"),), 64)),
    LLAMA7B_PREFILL: Config(LLAMA7B_PREFILL, "llama2-7b mlp prefill",
                            _sweep(LLAMA7B_PREFILL, "7b-mlp", (2048,),
                                   ((11008, 4096, "upgate"), (4096, 11008, "down")), 64)),
    LLAMA70B_SWEEP: Config(LLAMA70B_SWEEP, "llama2-70b linear sweep",
                           _sweep(LLAMA70B_SWEEP, "70b", (1, 16, 128, 1024, 4096),
                                  ((28672, 8192, "upgate"), (8192, 28672, "down")), 128)),
    FP8_VARIANT: Config(FP8_VARIANT, "int4-fp8 variant",
                        (Shape(2048, 8192, 8192, 0, "fp8:M2048"),), fp8=True),
}


def seed_w(cfg: int, pair: int = 0) -> int:
    """Weight seed; ``pair`` numbers the distinct (N, K) pairs of a config."""
    return 1000 * cfg + 1 + 10 * pair


def seed_x(cfg: int, M: int | None = None) -> int:
    return 1000 * cfg + 2 if M is None else 1000 * cfg + 100 + M


def seed_outliers(cfg: int) -> int:
    return 1000 * cfg + 3


def gen_weights(N: int, K: int, seed: int) -> np.ndarray:
    """float32 [N][K] ~ Normal(0, 0.02)."""
    rng = np.random.default_rng(seed)
    w = rng.standard_normal((N, K), dtype=np.float32)
    w *= np.float32(W_STD)
    return w


def outlier_channels(K: int, seed: int, frac: float = OUTLIER_FRAC) -> np.ndarray:
    """round(frac*K) distinct channel indices from a seeded permutation."""
    n_out = int(round(frac * K))
    rng = np.random.default_rng(seed)
    return np.sort(rng.permutation(K)[:n_out]).astype(np.int64)


def gen_activations(M: int, K: int, seed: int, outlier_seed: int,
                    frac: float = OUTLIER_FRAC,
                    scale: float = OUTLIER_SCALE) -> np.ndarray:
    """float32 [M][K] ~ Normal(0, 1) with the outlier channels times ``scale``."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K), dtype=np.float32)
    ch = outlier_channels(K, outlier_seed, frac)
    if len(ch):
        x[:, ch] *= np.float32(scale)
    return x


def nk_pairs(cfg: int):
    """Distinct (N, K) pairs of a config, in table order."""
    out = []
    for sh in CONFIGS[cfg].shapes:
        if (sh.N, sh.K) not in out:
            out.append((sh.N, sh.K))
    return out


def inputs_for(cfg: int, shape: Shape, sweep_x: bool = True):
    """(W, X) float32 arrays for one shape of a config, with the seeds above."""
    pair = nk_pairs(cfg).index((shape.N, shape.K)) if cfg in CONFIGS else 0
    w = gen_weights(shape.N, shape.K, seed_w(cfg, pair))
    x = gen_activations(shape.M, shape.K,
                        seed_x(cfg, shape.M if sweep_x else None),
                        seed_outliers(cfg))
    return w, x
