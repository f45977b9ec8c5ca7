"""Seeded synthetic inputs for exact Lloyd k-means (tests and benchmark).

This module only draws random inputs; it holds none of the method's
arithmetic (no distances, no argmin, no means), so both the GPU path's tests
and the oracle consume exactly the same bytes from it.

The pages benchmark FP16 data with d = 128 over sweeps of N, K and batch B
(7minutos.es article on Flash-KMeans, section "Punto de referencia";
tilnote.io overview, benchmark conditions) and an FP32, d = 128 pinned-host,
chunked large-tensor sweep (tilnote.io overview, last paragraph before the
conclusion).  They name no dataset for the method, so seeded Gaussian mixtures
of the same shapes stand in for those workloads.

All draws use torch's CPU generator (Mersenne Twister, seeded),
so the bytes do not depend on a GPU being present.  16-bit outputs are
rounded from fp32 with torch's CPU conversion (round to nearest, ties to even).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

__all__ = ["Workload", "CONFIGS", "make", "make_streamed", "integer_problem", "init_indices"]


@dataclasses.dataclass(frozen=True)
class Workload:
    """One benchmark configuration (full size)."""
    name: str
    B: int
    N: int
    K: int
    d: int
    dtype: str          # 'f32' | 'f16' | 'bf16'
    iters: int
    mean_std: float     # means ~ N(0, mean_std^2 I)
    sigma: float        # per-coordinate noise around the mean
    weights: str        # 'equal-exact' | 'uniform' | 'zipf1.2'
    unit: bool          # normalise means and points to unit length
    init: str           # 'first' | 'sample'
    seed: int
    init_seed: int


# The five workloads (sizes, distributions, iteration counts).  Where a
# workload's definition leaves a value open (the noise level and init of the
# last three, the per-coordinate noise of the unit-vector one) the value here
# is a reading: the one the other workloads use.
CONFIGS = {
    1: Workload("gmm32_n4096_k32_d128_f32", 1, 4096, 32, 128, "f32", 10, 2.0, 1.0,
                "equal-exact", False, "first", 1001, 2001),
    2: Workload("gmm1024_b32_n65536_k1024_d128_f16", 32, 65536, 1024, 128, "f16", 25, 1.0, 0.3,
                "uniform", False, "sample", 1002, 2002),
    3: Workload("zipf4096_n1m_k4096_d128_f16", 1, 1 << 20, 4096, 128, "f16", 20, 1.0, 0.3,
                "zipf1.2", False, "sample", 1003, 2003),
    4: Workload("unit65536_n1m_k65536_d1024_bf16", 1, 1 << 20, 65536, 1024, "bf16", 10, 1.0, 0.1,
                "uniform", True, "sample", 1004, 2004),
    5: Workload("gmm4096_n128m_k4096_d128_f32_host", 1, 1 << 27, 4096, 128, "f32", 5, 1.0, 0.5,
                "uniform", False, "sample", 1005, 2005),
}

_TORCH_DTYPE = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def _component_ids(w: Workload, B: int, N: int, K: int, g: torch.Generator) -> torch.Tensor:
    if w.weights == "equal-exact":
        # exactly N/K points per component, in a seeded random order
        base = torch.arange(N, dtype=torch.int64) % K
        return torch.stack([base[torch.randperm(N, generator=g)] for _ in range(B)])
    if w.weights == "uniform":
        return torch.randint(0, K, (B, N), generator=g, dtype=torch.int64)
    if w.weights == "zipf1.2":
        # weights proportional to j^-1.2, j = 1..K; inverse-CDF sampling
        j = torch.arange(1, K + 1, dtype=torch.float64)
        p = j.pow(-1.2)
        cdf = torch.cumsum(p / p.sum(), 0)
        cdf[-1] = 1.0
        u = torch.rand((B, N), generator=g, dtype=torch.float64)
        return torch.searchsorted(cdf, u).clamp_(max=K - 1)
    raise ValueError(w.weights)


def make(cfg: int | Workload, N: int | None = None, B: int | None = None,
         K: int | None = None, d: int | None = None, dtype: str | None = None,
         seed: int | None = None):
    """Seeded (X, C0) for a workload, optionally shrunk.

    Returns X as a CPU torch tensor (B, N, d) in the workload dtype and C0 as
    fp32 (B, K, d): the initial centroids, which are points of X (so the
    16-bit value converts to fp32 exactly and back).
    """
    w = CONFIGS[cfg] if isinstance(cfg, int) else cfg
    B = w.B if B is None else B
    N = w.N if N is None else N
    K = w.K if K is None else K
    d = w.d if d is None else d
    dtype = w.dtype if dtype is None else dtype
    seed = w.seed if seed is None else seed
    g = torch.Generator().manual_seed(seed)
    means = torch.randn((B, K, d), generator=g, dtype=torch.float32) * w.mean_std
    if w.unit:
        means = means / means.norm(dim=-1, keepdim=True)
    z = _component_ids(w, B, N, K, g)
    X = torch.randn((B, N, d), generator=g, dtype=torch.float32)
    X.mul_(w.sigma)
    X.add_(torch.gather(means, 1, z.unsqueeze(-1).expand(B, N, d)))
    if w.unit:
        X.div_(X.norm(dim=-1, keepdim=True))
    X = X.to(_TORCH_DTYPE[dtype])
    idx = init_indices(w, B, N, K, seed=w.init_seed if seed == w.seed else seed + 1000)
    C0 = torch.gather(X, 1, idx.unsqueeze(-1).expand(B, K, d)).to(torch.float32)
    return X, C0


def make_streamed(cfg: int | Workload, N: int | None = None, piece: int = 1 << 22,
                  log=None, pin: bool = True):
    """Seeded (X_host, C0) for a single-problem workload too large to build
    at once: X_host (1, N, d) is allocated in host memory (pinned unless
    pin=False) and filled
    piece by piece (piece j draws its component ids and noise from a
    generator seeded with seed * 1000003 + j), so peak extra memory is one
    piece.  Same distribution as make(); a different random stream.
    C0 = the init points (fp32)."""
    w = CONFIGS[cfg] if isinstance(cfg, int) else cfg
    N = w.N if N is None else N
    K, d = w.K, w.d
    assert w.B == 1 and w.weights == "uniform" and not w.unit
    g = torch.Generator().manual_seed(w.seed)
    means = torch.randn((K, d), generator=g, dtype=torch.float32) * w.mean_std
    X = torch.empty((1, N, d), dtype=_TORCH_DTYPE[w.dtype], pin_memory=pin)
    for j, i0 in enumerate(range(0, N, piece)):
        n = min(piece, N - i0)
        gj = torch.Generator().manual_seed(w.seed * 1000003 + j)
        z = torch.randint(0, K, (n,), generator=gj, dtype=torch.int64)
        x = torch.randn((n, d), generator=gj, dtype=torch.float32)
        x.mul_(w.sigma).add_(means[z])
        X[0, i0:i0 + n].copy_(x)
        if log and j % 8 == 0:
            log(f"[synth] {i0 + n} of {N} points")
    gi = torch.Generator().manual_seed(w.init_seed)
    idx = torch.randperm(N, generator=gi)[:K]
    C0 = X[0, idx].to(torch.float32).unsqueeze(0).contiguous()
    return X, C0


def init_indices(w: Workload, B: int, N: int, K: int, seed: int) -> torch.Tensor:
    """K initial point indices per problem: the first K points, or K indices
    drawn without replacement (seeded)."""
    if w.init == "first" or K > N:
        if K > N:
            # more centroids than points: cycle through the points
            return (torch.arange(K, dtype=torch.int64) % N).expand(B, K).contiguous()
        return torch.arange(K, dtype=torch.int64).expand(B, K).contiguous()
    g = torch.Generator().manual_seed(seed)
    return torch.stack([torch.randperm(N, generator=g)[:K] for _ in range(B)])


def integer_problem(B: int, N: int, K: int, d: int, lo: int = -3, hi: int = 3,
                    seed: int = 0, planted_ties: bool = True):
    """Small integer-valued problem (X, C) as int64 arrays.

    Coordinates are integers in [lo, hi]; with planted_ties some centroids are
    duplicated (so several centroids sit at exactly equal distance from every
    point) and some points sit exactly midway between two centroids.  Such
    inputs are exact in fp16, bf16 and fp32, and all sums of products of
    d <= 3 coordinates stay far below 2^11, so any fp32 accumulation of them
    is exact.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    X = rng.integers(lo, hi + 1, size=(B, N, d), dtype=np.int64)
    C = rng.integers(lo, hi + 1, size=(B, K, d), dtype=np.int64)
    if planted_ties and K >= 3:
        for b in range(B):
            # duplicate a centroid at a higher index: exact ties everywhere
            src, dst = rng.choice(K, size=2, replace=False)
            lo_i, hi_i = min(src, dst), max(src, dst)
            C[b, hi_i] = C[b, lo_i]
            # a point exactly midway between two centroids two units apart
            if N >= 2:
                c0 = C[b, 0].copy()
                C[b, 1] = c0
                C[b, 1, 0] = c0[0] + 2
                X[b, N - 1] = c0
                X[b, N - 1, 0] = c0[0] + 1
    return X, C


def zipf_top_share(K: int, s: float = 1.2) -> float:
    """Expected fraction of points in the heaviest Zipf component (for logs)."""
    return 1.0 / sum(j ** (-s) for j in range(1, K + 1))


def nbytes(w: Workload) -> int:
    return w.B * w.N * w.d * (4 if w.dtype == "f32" else 2)


def describe(w: Workload) -> str:
    return (f"B={w.B}, N={w.N}, K={w.K}, d={w.d} {w.dtype}; {w.weights} mixture, "
            f"means~N(0,{w.mean_std**2:g}I){' unit' if w.unit else ''}, sigma={w.sigma}; "
            f"init={w.init}; {w.iters} iterations")
