"""User-facing k-means API over the C ABI: a batched function in the shape
of the package's ``batch_kmeans_Euclid`` (the tilnote.io overview of
Flash-KMeans, section on where it is useful: batched Euclidean k-means on GPU
tensors) and a small scikit-learn-like ``KMeans`` estimator (fit / predict /
fit_predict; the 7minutos.es article, section "Usándolo", says the interface
mirrors faiss and scikit-learn on a batched (B, N, d) tensor).

Everything numeric runs in the library's kernels (fk_lloyd, fk_assign);
this module only picks the initial centroids, allocates outputs with torch
and reshapes.  Inputs must already live on the GPU.

Conventions: labels are 0-based int32; centroids are returned in fp32 (the
library carries them in fp32 and assigns with their round-to-nearest-even
copy in the input dtype); ``tol`` is the library's stopping rule: stop after
the first iteration whose largest squared centroid move is <= tol (0 runs
exactly ``max_iter`` iterations without a host synchronisation per
iteration).
"""
from __future__ import annotations

import torch

from . import fk_assign, fk_lloyd, fk_sort_labels

__all__ = ["batch_kmeans_euclid", "KMeans", "initial_centroids"]


def _as_batched(X: torch.Tensor) -> tuple[torch.Tensor, bool]:
    if not isinstance(X, torch.Tensor):
        raise TypeError("X must be a torch tensor")
    if X.device.type != "cuda":
        raise ValueError("X must be on the GPU")
    if X.dtype not in (torch.float32, torch.float16, torch.bfloat16):
        raise ValueError("X must be float32, float16 or bfloat16")
    if X.dim() == 2:
        return X.unsqueeze(0).contiguous(), True
    if X.dim() != 3:
        raise ValueError("X must be (N, d) or (B, N, d)")
    return X.contiguous(), False


def initial_centroids(X: torch.Tensor, n_clusters: int, init="sample", seed: int = 0) -> torch.Tensor:
    """Initial fp32 centroids (B, K, d) for batched X (B, N, d).

    init: "sample" -- K distinct points per problem drawn with a seeded
    generator (with K > N, every point then repeats cyclically); "first" --
    the first K points; or a tensor (K, d) / (B, K, d) of centroids."""
    B, N, d = X.shape
    K = int(n_clusters)
    if K < 1:
        raise ValueError("n_clusters must be >= 1")
    if isinstance(init, torch.Tensor):
        C = init.to(device=X.device, dtype=torch.float32)
        if C.dim() == 2 and tuple(C.shape) == (K, d):
            C = C.unsqueeze(0).expand(B, K, d)
        if tuple(C.shape) != (B, K, d):
            raise ValueError(f"init centroids must be ({K}, {d}) or ({B}, {K}, {d})")
        return C.contiguous().clone()
    if init == "first" or K > N:
        idx = (torch.arange(K) % N).expand(B, K)
    elif init == "sample":
        g = torch.Generator().manual_seed(int(seed))
        idx = torch.stack([torch.randperm(N, generator=g)[:K] for _ in range(B)])
    else:
        raise ValueError(f"unknown init {init!r}")
    idx = idx.to(X.device)
    rows = torch.gather(X, 1, idx.unsqueeze(-1).expand(B, K, d))
    return rows.to(torch.float32).contiguous()


def batch_kmeans_euclid(X: torch.Tensor, n_clusters: int, max_iter: int = 100, tol: float = 0.0,
                        init="sample", seed: int = 0, deterministic: bool = False, stream=None):
    """Exact Lloyd k-means on each of the B problems of X (B, N, d).

    deterministic: the library's FK_DETERMINISTIC mode (bit-identical results
    on every run).  Returns (labels (B, N) int32 of the last
    assignment, centroids (B, K, d) fp32 after the last update, number of
    iterations run)."""
    Xb, _ = _as_batched(X)
    if max_iter < 1:
        raise ValueError("max_iter must be >= 1")
    if tol < 0:
        raise ValueError("tol must be >= 0")
    B, N, d = Xb.shape
    C = initial_centroids(Xb, n_clusters, init, seed)
    labels = torch.empty((B, N), dtype=torch.int32, device=Xb.device)
    counts = torch.empty((B, C.shape[1]), dtype=torch.int32, device=Xb.device)
    n = fk_lloyd(Xb, C, labels, counts, int(max_iter), float(tol), want_n_iter=tol > 0,
                 stream=stream, deterministic=deterministic)
    return labels, C, (n if tol > 0 else int(max_iter))


class KMeans:
    """Exact Lloyd k-means, scikit-learn style, on GPU tensors.

    After fit: ``cluster_centers_`` (K, d) fp32 (or (B, K, d) for batched
    input), ``labels_`` and ``inertia_`` of the assignment to those final
    centroids (sum of squared distances, per problem for batched input),
    ``counts_`` (points per centroid of that assignment) and ``n_iter_``."""

    def __init__(self, n_clusters: int = 8, max_iter: int = 300, tol: float = 1e-4,
                 init="sample", seed: int = 0, deterministic: bool = False):
        self.deterministic = bool(deterministic)
        self.n_clusters = int(n_clusters)
        self.max_iter = int(max_iter)
        self.tol = float(tol)
        self.init = init
        self.seed = int(seed)

    def fit(self, X: torch.Tensor) -> "KMeans":
        Xb, single = _as_batched(X)
        _, C, n = batch_kmeans_euclid(Xb, self.n_clusters, self.max_iter, self.tol, self.init,
                                      self.seed, self.deterministic)
        self._single = single
        self._C = C
        self.n_iter_ = n
        labels, dist = self._assign(Xb)
        B, N, d = Xb.shape
        K = self.n_clusters
        counts = torch.empty((B, K), dtype=torch.int32, device=Xb.device)
        offsets = torch.empty((B, K + 1), dtype=torch.int32, device=Xb.device)
        order = torch.empty((B, N), dtype=torch.int32, device=Xb.device)
        fk_sort_labels(labels, K, counts, offsets, order, d=d, dtype=Xb.dtype)
        self.counts_ = self._squeeze(counts)
        self.labels_ = self._squeeze(labels)
        inertia = dist.cpu().double().sum(dim=1)   # reported in fp64, summed on the host
        self.inertia_ = float(inertia[0]) if single else inertia
        self.cluster_centers_ = self._squeeze(C)
        return self

    def predict(self, X: torch.Tensor) -> torch.Tensor:
        if not hasattr(self, "_C"):
            raise RuntimeError("fit first")
        Xb, single = _as_batched(X)
        if Xb.shape[0] != self._C.shape[0] or Xb.shape[2] != self._C.shape[2]:
            raise ValueError("X must have the batch and dimension of the fitted data")
        labels, _ = self._assign(Xb)
        return labels[0] if single else labels

    def fit_predict(self, X: torch.Tensor) -> torch.Tensor:
        return self.fit(X).labels_

    def _assign(self, Xb: torch.Tensor):
        B, N, _ = Xb.shape
        Cq = self._C.to(Xb.dtype).contiguous()
        labels = torch.empty((B, N), dtype=torch.int32, device=Xb.device)
        dist = torch.empty((B, N), dtype=torch.float32, device=Xb.device)
        fk_assign(Xb, Cq, labels, dist)
        return labels, dist

    def _squeeze(self, t: torch.Tensor) -> torch.Tensor:
        return t[0] if self._single else t
