"""Comparison of the HIP path with the fp64 oracle (element by element).

Tolerances (stated by the benchmark definition of the method):
  * labels and counts: bit-exact, except points whose best and second-best
    oracle distances differ by less than TAU relative, (d2 - d1) / d2 < TAU,
    with TAU = 1e-4 for fp32 inputs and 1e-2 for fp16/bf16 inputs.  An
    excluded point must still receive a near-optimal centroid: its oracle
    distance to the chosen centroid is at most d1 * (1 + TAU).
  * centroids: per centroid row, max_j |c_gpu - c_ref| <= CTOL * max_j |c_ref|,
    CTOL = 1e-4 for fp32 inputs and 2e-3 for fp16/bf16 inputs, comparing the
    fp32 centroid before its rounding to the input dtype.
  * empty clusters keep the previous centroid bit for bit; the low-precision
    copy equals the round-to-nearest-even of the fp32 centroid bit for bit.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle

TAU = {"f32": 1e-4, "f16": 1e-2, "bf16": 1e-2}
CTOL = {"f32": 1e-4, "f16": 2e-3, "bf16": 2e-3}
FMT = {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16"}
TORCH = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def to_storage(t: torch.Tensor) -> np.ndarray:
    """CPU numpy view of a tensor's stored bits (16-bit floats as uint16)."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.float32:
        return t.numpy()
    if t.dtype in (torch.float16, torch.bfloat16):
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def check_labels(gpu_labels: torch.Tensor, X: torch.Tensor, Cq: torch.Tensor,
                 rows: np.ndarray | None = None, min_dist: torch.Tensor | None = None,
                 keep_oracle_labels: bool = False) -> dict:
    """GPU labels (B, N) against the oracle's assignment of X to Cq (the
    centroids exactly as the GPU read them).  With rows, only those flattened
    point ids are checked.  The returned counts: n checked points, near_ties
    (points excluded from the bit-exact rule by the gap test) and
    excluded_diff (excluded points whose GPU label differs from the
    oracle's); with keep_oracle_labels also the oracle's labels."""
    fmt = FMT[X.dtype]
    tau = TAU[fmt]
    Xs, Cs = to_storage(X), to_storage(Cq)
    lab, d1, d2 = oracle.assign(Xs, Cs, fmt_x=fmt, fmt_c=fmt, rows=rows)
    g = gpu_labels.cpu().numpy()
    g = g.reshape(-1)[rows] if rows is not None else g.reshape(-1)
    lab, d1, d2 = lab.reshape(-1), d1.reshape(-1), d2.reshape(-1)
    pts = rows if rows is not None else np.arange(lab.size)
    K = Cq.shape[1]
    assert g.min() >= 0 and g.max() < K, "GPU label out of range"
    with np.errstate(divide="ignore", invalid="ignore"):
        gap = np.where(d2 > 0, (d2 - d1) / d2, 0.0)
    strict = gap >= tau
    bad = np.flatnonzero(strict & (g != lab))
    assert bad.size == 0, (f"{bad.size} labels differ outside near-ties, e.g. point {pts[bad[0]]}: "
                           f"gpu {g[bad[0]]} oracle {lab[bad[0]]} gap {gap[bad[0]]:.3g}")
    excl = np.flatnonzero(~strict & (g != lab))
    if excl.size:
        dg = oracle.pair_dist(Xs, Cs, pts[excl], g[excl], fmt_x=fmt, fmt_c=fmt)
        worst = np.max(dg / np.maximum(d1[excl], 1e-300) - 1.0)
        assert np.all(dg <= d1[excl] * (1 + tau) + 1e-300), f"excluded label not near-optimal ({worst})"
    if min_dist is not None:
        md = min_dist.cpu().numpy().reshape(-1)
        md = md[rows] if rows is not None else md
        dg = oracle.pair_dist(Xs, Cs, pts, g, fmt_x=fmt, fmt_c=fmt)
        xx = oracle.pair_dist(Xs, np.zeros_like(Cs[:, :1]), pts, np.zeros(pts.size, np.int32),
                              fmt_x=fmt, fmt_c=fmt)
        cc = oracle.decode(Cs, fmt)
        cn = (cc ** 2).sum(-1).reshape(-1)
        Kc = Cq.shape[1]
        N = X.shape[1]
        scale = xx + cn[(pts // N) * Kc + g]
        assert np.all(np.abs(md - dg) <= 1e-5 * scale + 1e-6), "min_dist off"
    out = {"n": int(lab.size), "near_ties": int((~strict).sum()), "excluded_diff": int(excl.size)}
    if keep_oracle_labels:
        out["oracle_labels"] = lab
    return out


def check_update(X: torch.Tensor, labels: torch.Tensor, C_prev: torch.Tensor,
                 C_next: torch.Tensor, counts: torch.Tensor,
                 C_lowp: torch.Tensor | None = None) -> dict:
    """GPU update from GPU labels against the oracle's update from the same
    labels: counts bit-exact, centroids within CTOL, empties unchanged,
    low-precision copy = RNE(fp32 centroid)."""
    fmt = FMT[X.dtype]
    Xs = to_storage(X)
    lab = labels.cpu().numpy().astype(np.int32)
    Cp = C_prev.cpu().numpy()
    ocnt, oC, _ = oracle.update(Xs, lab, Cp, fmt_x=fmt, fmt_c="f32")
    gcnt = counts.cpu().numpy()
    assert np.array_equal(gcnt, ocnt), f"counts differ at {np.argwhere(gcnt != ocnt)[:5]}"
    gC = C_next.cpu().numpy().astype(np.float64)
    err = np.abs(gC - oC).max(-1)
    ref = np.abs(oC).max(-1)
    tol = CTOL[fmt]
    badrows = np.argwhere(err > tol * np.maximum(ref, 1e-30))
    assert badrows.size == 0, (f"{len(badrows)} centroid rows beyond tolerance, e.g. {badrows[0]}: "
                               f"err {err[tuple(badrows[0])]:.3g} ref {ref[tuple(badrows[0])]:.3g}")
    empty = ocnt == 0
    assert np.array_equal(C_next.cpu().numpy()[empty], Cp[empty]), "empty cluster moved"
    if C_lowp is not None and fmt != "f32":
        rne = oracle.encode_rne(C_next.cpu().numpy(), fmt)
        assert np.array_equal(to_storage(C_lowp), rne), "low-precision copy is not RNE"
    rel = float((err / np.maximum(ref, 1e-30)).max()) if err.size else 0.0
    return {"max_rel_row_err": rel, "empty": int(empty.sum())}
