"""Seeded synthetic workloads for the W4A8 linear and MoE-expert path.

This module only draws numbers: it holds no quantization, GEMM or combine
arithmetic, so the CPU oracle and the HIP path can both consume its output
without sharing any of the method's code.  Every tensor is drawn from
``numpy.random.Generator(PCG64(seed))``; activations are drawn in float32 and
rounded once to bfloat16, and that bfloat16 tensor is the single input handed
to both sides.

The shapes follow the workloads the source pages discuss: a single Linear with
outlier channels, a decode-shape fused gate/up projection, a prefill-shape
projection pair, and two MoE expert layers (a 64-expert top-6 layer with
skewed routing and a 256-expert top-8 decode step).  The pages use no public
dataset for this path; these generators stand in for real activations and
trained weights, which are not available.

The router (softmax over logits, top-k, weights not renormalised) lives here
because the library receives ``topk_ids``/``topk_w`` as inputs: the pages keep
the router in FP16/BF16 outside the quantized path ("Kimi 2.7 MoE: 4-bit
storage to INT8", section 4.1).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def to_bf16(x: np.ndarray) -> torch.Tensor:
    """float32 numpy array -> CPU bfloat16 tensor (round-to-nearest-even)."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)


def bf16_values(t: torch.Tensor) -> np.ndarray:
    """CPU bfloat16 tensor -> float32 numpy array holding the same values exactly."""
    return t.to(torch.float32).numpy()


# --------------------------------------------------------------------------------------
# configurations
# --------------------------------------------------------------------------------------
@dataclass(frozen=True)
class DenseConfig:
    name: str
    M: int
    K: int
    N: int
    group_size: int
    asymmetric: bool
    seed: int
    outlier_cols: int = 0          # number of activation channels scaled up
    outlier_scale: float = 1.0
    w_std: float = 0.02
    x_dist: str = "normal"          # "normal" | "student_t3"


@dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int                # tokens
    H: int                # hidden size (gate/up K, down N)
    I: int                # expert intermediate size (gate/up N = 2I, down K)
    E: int                # experts
    topk: int
    group_size: int
    asymmetric: bool
    seed: int
    zipf_s: float = 0.0   # expert bias -s*ln(rank); 0 disables the skew
    x_dist: str = "normal"
    w_std: float = 0.02


# Single Linear with 4 outlier channels x20.
C1 = DenseConfig("linear_m16_k1024_n1024_sym_g128", 16, 1024, 1024, 128, False, 101,
                 outlier_cols=4, outlier_scale=20.0)
# Decode-shape fused gate/up projection; M in {1, 8, 32}; 0.1% outlier channels x50.
C2_M = (1, 8, 32)
C2 = DenseConfig("decode_k4096_n14336_sym_g128", 32, 4096, 14336, 128, False, 102,
                 outlier_cols=4, outlier_scale=50.0)
# Prefill-shape projection pair (batch 4 x seq 1024), asymmetric uint4 weights.
C3_UP = DenseConfig("prefill_m4096_k4096_n14336_asym_g128", 4096, 4096, 14336, 128, True, 103)
C3_DOWN = DenseConfig("prefill_m4096_k14336_n4096_asym_g128", 4096, 14336, 4096, 128, True, 1103)
# MoE expert layer: T=512, E=64, top-6, Zipf(1.1) expert skew.
C4 = MoEConfig("moe_t512_e64_top6_h4096_i1408_sym_g128", 512, 4096, 1408, 64, 6, 128, False, 104,
               zipf_s=1.1)
# Large MoE decode step on one GPU: T=64, E=256, top-8, asymmetric g64, heavy-tailed acts.
C5 = MoEConfig("moe_t64_e256_top8_h7168_i2048_asym_g64", 64, 7168, 2048, 256, 8, 64, True, 105,
               x_dist="student_t3")


def with_decode_m(cfg: DenseConfig, M: int) -> DenseConfig:
    return DenseConfig(cfg.name.replace("decode", f"decode_m{M}"), M, cfg.K, cfg.N, cfg.group_size,
                       cfg.asymmetric, cfg.seed, cfg.outlier_cols, cfg.outlier_scale, cfg.w_std,
                       cfg.x_dist)


# --------------------------------------------------------------------------------------
# dense inputs
# --------------------------------------------------------------------------------------
def draw_activations(g: np.random.Generator, M: int, K: int, dist: str = "normal",
                     outlier_cols: int = 0, outlier_scale: float = 1.0) -> np.ndarray:
    if dist == "normal":
        x = g.standard_normal((M, K), dtype=np.float32)
    elif dist == "student_t3":
        x = g.standard_t(3.0, size=(M, K)).astype(np.float32)
    else:
        raise ValueError(dist)
    if outlier_cols:
        cols = g.choice(K, size=outlier_cols, replace=False)
        x[:, cols] *= np.float32(outlier_scale)
    return x


def draw_weights(g: np.random.Generator, K: int, N: int, std: float = 0.02) -> np.ndarray:
    return (g.standard_normal((K, N), dtype=np.float32) * np.float32(std)).astype(np.float32)


def dense_inputs(cfg: DenseConfig, M: int | None = None):
    """Returns (X bf16 CPU tensor [M,K], W float32 numpy [K,N])."""
    M = cfg.M if M is None else M
    g = rng(cfg.seed)
    W = draw_weights(g, cfg.K, cfg.N, cfg.w_std)
    x = draw_activations(rng(cfg.seed + 7919), M, cfg.K, cfg.x_dist, cfg.outlier_cols,
                         cfg.outlier_scale)
    return to_bf16(x), W


def random_activations(seed: int, M: int, K: int, dist: str = "normal", outlier_cols: int = 0,
                       outlier_scale: float = 1.0) -> torch.Tensor:
    return to_bf16(draw_activations(rng(seed), M, K, dist, outlier_cols, outlier_scale))


def random_weights(seed: int, K: int, N: int, std: float = 0.02) -> np.ndarray:
    return draw_weights(rng(seed), K, N, std)


# --------------------------------------------------------------------------------------
# MoE inputs
# --------------------------------------------------------------------------------------
def route(logits: np.ndarray, topk: int):
    """Router: softmax over experts in float32, top-k by probability (ties -> lower expert id),
    returned weights are the selected probabilities, not renormalised."""
    z = logits.astype(np.float32)
    z = z - z.max(axis=1, keepdims=True)
    p = np.exp(z)
    p = (p / p.sum(axis=1, keepdims=True)).astype(np.float32)
    # stable sort on -p keeps the lower id first among equal probabilities
    order = np.argsort(-p, axis=1, kind="stable")[:, :topk]
    ids = order.astype(np.int32)
    w = np.take_along_axis(p, order, axis=1).astype(np.float32)
    return ids, w


def moe_routing(cfg: MoEConfig, T: int | None = None):
    T = cfg.T if T is None else T
    g = rng(cfg.seed)
    logits = g.standard_normal((T, cfg.E), dtype=np.float32)
    if cfg.zipf_s:
        ranks = g.permutation(cfg.E) + 1
        logits = logits + (-cfg.zipf_s * np.log(ranks)).astype(np.float32)[None, :]
    return route(logits, cfg.topk)


def moe_activations(cfg: MoEConfig, T: int | None = None) -> torch.Tensor:
    T = cfg.T if T is None else T
    return random_activations(cfg.seed + 31337, T, cfg.H, cfg.x_dist)


def expert_weights(cfg: MoEConfig, e: int):
    """Float32 weights of expert e: (W_gu [H, 2I], W_d [I, H]); gate = first I columns."""
    g = rng(cfg.seed * 100003 + e)
    W_gu = draw_weights(g, cfg.H, 2 * cfg.I, cfg.w_std)
    W_d = draw_weights(g, cfg.I, cfg.H, cfg.w_std)
    return W_gu, W_d


def random_codes(seed: int, K: int, N: int, group_size: int, asymmetric: bool):
    """Random but well-formed quantized weights (codes, scales, zeros) for timing runs whose
    float weights would not fit the host: codes uniform over the format's range, scales
    ~|N(0, 0.02)|/7, zero-points uniform in [4, 11]."""
    g = rng(seed)
    G = K // group_size
    if asymmetric:
        codes = g.integers(0, 16, size=(K, N), dtype=np.int8)
        zeros = g.integers(4, 12, size=(G, N), dtype=np.uint8)
    else:
        codes = g.integers(-7, 8, size=(K, N), dtype=np.int8)
        zeros = None
    scales = (np.abs(g.standard_normal((G, N), dtype=np.float32)) * np.float32(0.02 / 7)
              + np.float32(1e-4)).astype(np.float32)
    return codes, scales, zeros
