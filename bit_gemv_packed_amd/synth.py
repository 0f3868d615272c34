"""Seeded synthetic inputs for the sign-GEMV path.

This module only draws numbers; it holds none of the method's arithmetic
(no signs, scales, packing or products).  Both the HIP path and the CPU
oracle consume what it returns, so the two sides always see the same inputs.

The pages measure on LLaMA-2/3.1 and Qwen3 projection matrices (FluxBin Sec. 4,
App. D and E.4; BiLoCo "Result two").  Those weights are not available, so
every input here is a seeded draw of the same shape:

* W ~ N(0, 0.02) float32, [M][N];
* x drawn as [B][N] float32 (so batch 1 is a prefix of batch 16) and handed
  out as [N][B]; stored as bf16 (round-to-nearest-even) except in the tiny
  fp32 workload;
* outlier channels: round(0.005 N) channels, chosen by a seeded permutation,
  scaled by 20 before the bf16 rounding;
* heavy-tailed activations: standard Student-t with 3 degrees of freedom;
* low-rank factors: u, v Bernoulli(1/2) signs, alpha_r drawn per workload and
  stored as fp16; the rank is padded to a multiple of 32 with alpha_r = 0 and
  u = v = +1;
* calibration activations for the protected-row statistic: 128 vectors from
  the workload's own x distribution.

Random streams: numpy.random.default_rng([workload, part, stream]) with
stream 0 = W, 1 = x, 2 = u/v/alpha_r, 3 = outlier channels, 4 = calibration.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np

W_STD = 0.02


@dataclasses.dataclass(frozen=True)
class Shape:
    name: str
    M: int
    N: int


@dataclasses.dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    shapes: List[Shape]
    K: int
    colscale: bool
    x_dtype: str                 # "f32" or "bf16"
    x_dist: str                  # "normal" or "student_t3"
    outlier_frac: float = 0.0
    outlier_gain: float = 20.0
    rank: int = 0                # low-rank rank before padding
    alpha_r_dist: str = ""       # "uniform_0_0.01" or "abs_normal_0.005"
    salient_frac: float = 0.0
    batches: tuple = (1,)


WORKLOADS = {
    1: Workload(1, "tiny_256x256_k1_r8", [Shape("w", 256, 256)], K=1, colscale=False,
                x_dtype="f32", x_dist="normal", rank=8, alpha_r_dist="uniform_0_0.01"),
    2: Workload(2, "llama7b_proj_4096x4096_k2_colscale", [Shape("w", 4096, 4096)], K=2,
                colscale=True, x_dtype="bf16", x_dist="normal"),
    3: Workload(3, "proj_5120x5120_k3_r512_outliers", [Shape("w", 5120, 5120)], K=3,
                colscale=False, x_dtype="bf16", x_dist="normal", outlier_frac=0.005,
                rank=512, alpha_r_dist="abs_normal_0.005"),
    4: Workload(4, "llama3_8b_layer_7gemv_k2",
                [Shape("q", 4096, 4096), Shape("k", 1024, 4096), Shape("v", 1024, 4096),
                 Shape("o", 4096, 4096), Shape("gate", 14336, 4096), Shape("up", 14336, 4096),
                 Shape("down", 4096, 14336)],
                K=2, colscale=False, x_dtype="bf16", x_dist="normal", batches=(1, 4, 16)),
    5: Workload(5, "mlp_13b_70b_k2_r512_salient1pct",
                [Shape("up13b", 13824, 5120), Shape("down13b", 5120, 13824),
                 Shape("up70b", 28672, 8192)],
                K=2, colscale=False, x_dtype="bf16", x_dist="student_t3", rank=512,
                alpha_r_dist="abs_normal_0.005", salient_frac=0.01, batches=(1, 16)),
}


def rng(wid: int, part: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([wid, part, stream])


def padded_rank(r: int) -> int:
    return (r + 31) // 32 * 32


def n_outliers(N: int, frac: float) -> int:
    return int(np.floor(frac * N + 0.5))


def n_salient(M: int, frac: float) -> int:
    return int(np.floor(frac * M + 0.5))


def weights(wid: int, part: int, M: int, N: int) -> np.ndarray:
    """W ~ N(0, 0.02), float32 [M][N]."""
    g = rng(wid, part, 0)
    return g.standard_normal((M, N), dtype=np.float32) * np.float32(W_STD)


def _to_bf16_values(a: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest-even) and return the values as float32."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).float().numpy()


def _draw_x(w: Workload, part: int, N: int, B: int, stream: int) -> np.ndarray:
    g = rng(w.wid, part, stream)
    if w.x_dist == "normal":
        x = g.standard_normal((B, N), dtype=np.float32)
    elif w.x_dist == "student_t3":
        x = g.standard_t(3, size=(B, N)).astype(np.float32)
    else:
        raise ValueError(w.x_dist)
    if w.outlier_frac > 0:
        nout = n_outliers(N, w.outlier_frac)
        ch = rng(w.wid, part, 3).permutation(N)[:nout]
        x[:, ch] *= np.float32(w.outlier_gain)
    return x


def activations(w: Workload, part: int, N: int, B: int) -> np.ndarray:
    """x as float32 values [N][B], already rounded to the workload's storage
    dtype (bf16 values are exact in float32)."""
    x = _draw_x(w, part, N, B, 1)
    if w.x_dtype == "bf16":
        x = _to_bf16_values(x)
    return np.ascontiguousarray(x.T)


def calibration(w: Workload, part: int, N: int, S: int = 128) -> np.ndarray:
    """S calibration activation vectors [S][N] (float32 values of the storage dtype)."""
    x = _draw_x(w, part, N, S, 4)
    if w.x_dtype == "bf16":
        x = _to_bf16_values(x)
    return x


@dataclasses.dataclass
class LowRank:
    r: int                 # padded rank
    u: np.ndarray          # float32 +-1 [M][r]
    v: np.ndarray          # float32 +-1 [r][N]
    alpha_r_f16: np.ndarray  # uint16 fp16 bits [r]


def low_rank(w: Workload, part: int, M: int, N: int) -> Optional[LowRank]:
    if w.rank <= 0:
        return None
    r0, r = w.rank, padded_rank(w.rank)
    g = rng(w.wid, part, 2)
    u = np.ones((M, r), np.float32)
    v = np.ones((r, N), np.float32)
    u[:, :r0] = np.where(g.integers(0, 2, size=(M, r0)) == 1, 1.0, -1.0)
    v[:r0, :] = np.where(g.integers(0, 2, size=(r0, N)) == 1, 1.0, -1.0)
    a = np.zeros((r,), np.float32)
    if w.alpha_r_dist == "uniform_0_0.01":
        a[:r0] = g.uniform(0.0, 0.01, size=r0).astype(np.float32)
    elif w.alpha_r_dist == "abs_normal_0.005":
        a[:r0] = np.abs(g.standard_normal(r0).astype(np.float32) * np.float32(0.005))
    else:
        raise ValueError(w.alpha_r_dist)
    return LowRank(r=r, u=u, v=v, alpha_r_f16=a.astype(np.float16).view(np.uint16))


def random_bits(seed: int, K: int, M: int, N: int) -> np.ndarray:
    """Uniform random logical sign words [K][M][ceil(N/32)], padding bits clear."""
    g = np.random.default_rng([9001, seed])
    nd = (N + 31) // 32
    b = g.integers(0, 2**32, size=(K, M, nd), dtype=np.uint64).astype(np.uint32)
    if N % 32:
        b[..., -1] &= np.uint32((1 << (N % 32)) - 1)
    return b


def random_scales(seed: int, K: int, M: int, N: int, colscale: bool):
    """alpha float32 [K][M] ~ |N(0.016, 0.004)|, colscale fp16 bits [K][N] ~ U(0.5, 1.5) or None."""
    g = np.random.default_rng([9002, seed])
    alpha = np.abs(g.normal(0.016, 0.004, size=(K, M))).astype(np.float32)
    cs = None
    if colscale:
        cs = g.uniform(0.5, 1.5, size=(K, N)).astype(np.float32).astype(np.float16).view(np.uint16)
    return alpha, cs


def random_x(seed: int, N: int, B: int, dtype: str = "bf16", dist: str = "normal") -> np.ndarray:
    """x float32 values [N][B] rounded to dtype ("f32", "bf16", "f16")."""
    g = np.random.default_rng([9003, seed])
    if dist == "normal":
        x = g.standard_normal((B, N), dtype=np.float32)
    elif dist == "student_t3":
        x = g.standard_t(3, size=(B, N)).astype(np.float32)
    else:
        raise ValueError(dist)
    if dtype == "bf16":
        x = _to_bf16_values(x)
    elif dtype == "f16":
        x = x.astype(np.float16).astype(np.float32)
    return np.ascontiguousarray(x.T)
