"""Pins for the fp64 oracle: checks against facts fixed by the pages and by
mathematics, never against the oracle's own formulas.

Each ``pin_*`` takes an ``oracle.Oracle`` and raises AssertionError when the
oracle disagrees with the pinned fact.  ``test_oracle_pins.py`` runs them on
the in-tree oracle; ``test_oracle_mutants.py`` runs them on deliberately broken
builds and requires every break to be caught by at least one pin.

What pins what:
  * stored-float decoders  -- numpy's float16 and the bf16 = top-16-bits-of-fp32
    layout (library routine / format definition);
  * RNE encoders           -- numpy float16 and torch bfloat16 conversions;
  * distances              -- the expansion |x-c|^2 = |x|^2 + |c|^2 - 2 x.c
    (papernotes.org notes on Flash-KMeans, 关键设计 1) with a rounding bound;
  * assignment, ties, means -- exhaustive exact integer / rational arithmetic;
  * assignment             -- scipy.cluster.vq.vq (library routine), and the
    d = 1 nearest-centre closed form (sorted midpoints);
  * update                 -- K = 1 gives the sample mean; counts = bincount;
    centroids = member means; empty clusters unchanged;
  * iteration              -- planted partition reaches its known fixed point;
    the Lloyd objective never increases (textbook property).
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import torch

import synth

EPS64 = np.finfo(np.float64).eps


# --------------------------------------------------------------------------
# stored-float decoding and RNE encoding
# --------------------------------------------------------------------------
def pin_decode_f16(orc):
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = orc.decode(bits, "f16")
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan), "f16 NaN set differs"
    assert np.array_equal(got[~nan], ref[~nan]), "f16 decode differs from numpy"
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan])), "f16 sign of zero"


def pin_decode_bf16(orc):
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = orc.decode(bits, "bf16")
    # bf16 is by definition the upper half of an IEEE binary32 pattern
    ref = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan), "bf16 NaN set differs"
    assert np.array_equal(got[~nan], ref[~nan]), "bf16 decode differs from bit layout"


def _fp32_probes(seed=7, n=200_000):
    rng = np.random.Generator(np.random.PCG64(seed))
    pats = rng.integers(0, 1 << 32, size=n, dtype=np.uint64).astype(np.uint32)
    vals = pats.view(np.float32)
    vals = vals[np.isfinite(vals)]
    # values near the fp16 range: normals, subnormals, overflow threshold
    mid = rng.uniform(-7e4, 7e4, size=n).astype(np.float32)
    small = (rng.uniform(-1, 1, size=n) * 2.0 ** rng.integers(-30, -10, size=n)).astype(np.float32)
    # exact ties for fp16: odd multiples of half a unit in the last place
    k = rng.integers(1 << 10, 1 << 11, size=n)
    e = rng.integers(-14, 15, size=n).astype(np.float64)
    tie16 = ((k + 0.5) * 2.0 ** (e - 10)).astype(np.float32)
    # exact ties for bf16: low 16 bits exactly 0x8000
    hi = rng.integers(0, 1 << 16, size=n, dtype=np.uint64).astype(np.uint32)
    tieb = ((hi << 16) | 0x8000).astype(np.uint32).view(np.float32)
    tieb = tieb[np.isfinite(tieb)]
    edge = np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, 65536.0, 2.0 ** -24, 2.0 ** -25,
                     1.5 * 2.0 ** -25, 2.0 ** -14, 3.0e38, -3.0e38, np.inf, -np.inf],
                    dtype=np.float32)
    return np.concatenate([vals, mid, small, tie16, tieb, edge]).astype(np.float32)


def pin_encode_f16(orc):
    v = _fp32_probes()
    got = orc.encode_rne(v, "f16")
    ref = v.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref), f"f16 RNE differs on {np.sum(got != ref)} values"


def pin_encode_bf16(orc):
    v = _fp32_probes(seed=8)
    got = orc.encode_rne(v, "bf16")
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref), f"bf16 RNE differs on {np.sum(got != ref)} values"


# --------------------------------------------------------------------------
# assignment
# --------------------------------------------------------------------------
def pin_distance_expansion(orc):
    """|x-c|^2 = |x|^2 + |c|^2 - 2 x.c, with fp64 rounding bound."""
    rng = np.random.Generator(np.random.PCG64(11))
    B, N, K, d = 3, 257, 37, 19
    X = rng.normal(size=(B, N, d)) * 3.0
    C = rng.normal(size=(B, K, d)) * 3.0 + 0.5
    labels, d1, d2 = orc.assign(X, C)
    xx = (X ** 2).sum(-1)[:, :, None]
    cc = (C ** 2).sum(-1)[:, None, :]
    D = xx + cc - 2.0 * np.matmul(X, C.transpose(0, 2, 1))
    bound = 8.0 * d * EPS64 * (xx + cc).max(-1)
    Ds = np.sort(D, axis=-1)
    assert np.all(np.abs(d1 - Ds[..., 0]) <= bound * 2), "d1 is not the minimum distance"
    assert np.all(np.abs(d2 - Ds[..., 1]) <= bound * 2), "d2 is not the second minimum"
    chosen = np.take_along_axis(D, labels[..., None].astype(np.int64), -1)[..., 0]
    assert np.all(np.abs(chosen - d1) <= bound * 2), "label does not attain d1"
    # sampled pair distances follow the same identity
    rng2 = np.random.Generator(np.random.PCG64(12))
    pts = rng2.integers(0, B * N, size=500)
    cen = rng2.integers(0, K, size=500).astype(np.int32)
    pd = orc.pair_dist(X, C, pts, cen)
    ref = D.reshape(B * N, K)[pts, cen]
    assert np.all(np.abs(pd - ref) <= 2 * bound.reshape(-1)[pts]), "pair distance differs"
    # small integers: every quantity is exact, so the identity holds exactly
    Xi, Ci = synth.integer_problem(2, 40, 7, 3, seed=3)
    Xi, Ci = Xi.astype(np.float64), Ci.astype(np.float64)
    _, e1, e2 = orc.assign(Xi, Ci)
    Di = (Xi ** 2).sum(-1)[:, :, None] + (Ci ** 2).sum(-1)[:, None, :] \
        - 2.0 * np.matmul(Xi, Ci.transpose(0, 2, 1))
    Dis = np.sort(Di, axis=-1)
    assert np.array_equal(e1, Dis[..., 0]) and np.array_equal(e2, Dis[..., 1])


def _exact_assign(X, C):
    """Exhaustive integer arithmetic: (labels, d1, d2) with lowest-index ties."""
    B, N, _ = X.shape
    K = C.shape[1]
    lab = np.zeros((B, N), np.int64)
    m1 = np.zeros((B, N), object)
    m2 = np.zeros((B, N), object)
    for b in range(B):
        for i in range(N):
            dists = [sum((int(X[b, i, j]) - int(C[b, k, j])) ** 2 for j in range(X.shape[2]))
                     for k in range(K)]
            best = min(dists)
            lab[b, i] = dists.index(best)          # first (lowest) index attaining it
            rest = sorted(dists)
            m1[b, i] = best
            m2[b, i] = rest[1] if K > 1 else float("inf")
    return lab, m1, m2


def _exact_update(X, lab, Cprev):
    """Counts and correctly rounded fp64 means via exact rationals."""
    B, N, d = X.shape
    K = Cprev.shape[1]
    counts = np.zeros((B, K), np.int64)
    means = np.array(Cprev, dtype=np.float64, copy=True)
    for b in range(B):
        for k in range(K):
            members = [i for i in range(N) if lab[b, i] == k]
            counts[b, k] = len(members)
            if members:
                for j in range(d):
                    s = sum(Fraction(int(X[b, i, j])) for i in members)
                    means[b, k, j] = float(s / len(members))
    return counts, means


def pin_exact_tiny_integers(orc):
    """Brute force with exact arithmetic on many tiny integer problems with
    planted exact ties, in every stored dtype."""
    rng = np.random.Generator(np.random.PCG64(5))
    for case in range(80):
        B = int(rng.integers(1, 3))
        N = int(rng.integers(1, 13))
        K = int(rng.integers(1, 5))
        d = int(rng.integers(1, 4))
        X, C = synth.integer_problem(B, N, K, d, seed=100 + case)
        lab, m1, m2 = _exact_assign(X, C)
        for fmt, npdt in (("f64", np.float64), ("f32", np.float32), ("f16", np.float16)):
            labels, d1, d2 = orc.assign(X.astype(npdt), C.astype(npdt), fmt_x=fmt, fmt_c=fmt)
            assert np.array_equal(labels, lab), f"labels differ (case {case}, {fmt})"
            assert np.array_equal(d1, m1.astype(np.float64)), f"d1 differs (case {case})"
            assert np.array_equal(d2, m2.astype(np.float64)), f"d2 differs (case {case})"
        Cprev = C.astype(np.float64) + 0.25     # distinguishable from any mean
        counts, means = _exact_update(X, lab, Cprev)
        got_c, got_m, bad = orc.update(X.astype(np.float64), lab.astype(np.int32), Cprev)
        assert bad == 0
        assert np.array_equal(got_c, counts), f"counts differ (case {case})"
        assert np.array_equal(got_m, means), f"means differ (case {case})"


def pin_scipy_vq(orc):
    """Assignment agrees with scipy.cluster.vq.vq on tie-free data."""
    from scipy.cluster.vq import vq
    rng = np.random.Generator(np.random.PCG64(21))
    B, N, K, d = 2, 500, 40, 9
    X = rng.normal(size=(B, N, d))
    C = rng.normal(size=(B, K, d))
    labels, d1, d2 = orc.assign(X, C)
    for b in range(B):
        code, dist = vq(X[b], C[b])
        gap = (d2[b] - d1[b]) / d2[b]
        ok = gap > 1e-9
        assert np.array_equal(labels[b][ok], code[ok]), "labels differ from scipy vq"
        assert np.allclose(d1[b], dist ** 2, rtol=1e-10, atol=1e-12)


def pin_d1_closed_form(orc):
    """d = 1: the nearest centre is found by thresholding at midpoints of the
    sorted distinct centre values; an exact midpoint goes to the lower index."""
    rng = np.random.Generator(np.random.PCG64(31))
    K, N = 13, 400
    c = rng.integers(-20, 21, size=K).astype(np.float64)
    c[7] = c[2]                                   # duplicate value: lower index must win
    x = rng.integers(-45, 46, size=N) / 2.0       # half-integers: hits midpoints exactly
    labels, _, _ = orc.assign(x.reshape(1, N, 1), c.reshape(1, K, 1))
    vals = np.unique(c)
    first_idx = np.array([np.flatnonzero(c == v).min() for v in vals])
    mids = (vals[:-1] + vals[1:]) / 2.0
    pos = np.searchsorted(mids, x, side="left")   # region of x
    exp = first_idx[pos]
    on_mid = np.isin(x, mids)
    j = np.searchsorted(mids, x[on_mid])
    exp[on_mid] = np.minimum(first_idx[j], first_idx[j + 1])
    assert np.array_equal(labels[0], exp), "d=1 closed form differs"


def pin_self_assignment(orc):
    rng = np.random.Generator(np.random.PCG64(41))
    B, N, K, d = 2, 300, 25, 6
    X = rng.normal(size=(B, N, d))
    rows = np.stack([rng.choice(N, K, replace=False) for _ in range(B)])
    C = np.stack([X[b, rows[b]] for b in range(B)])
    labels, d1, _ = orc.assign(X, C)
    for b in range(B):
        assert np.array_equal(labels[b, rows[b]], np.arange(K)), "a centroid row not self-assigned"
        assert np.all(d1[b, rows[b]] == 0.0)


# --------------------------------------------------------------------------
# update
# --------------------------------------------------------------------------
def pin_k1_mean(orc):
    rng = np.random.Generator(np.random.PCG64(51))
    X = rng.normal(size=(3, 1000, 8)) + 4.0
    C = rng.normal(size=(3, 1, 8))
    labels, _, _ = orc.assign(X, C)
    assert np.all(labels == 0)
    counts, Cn, _ = orc.update(X, labels, C)
    assert np.all(counts == 1000)
    assert np.allclose(Cn[:, 0], X.mean(axis=1), rtol=1e-13, atol=1e-13)


def pin_counts_and_member_means(orc):
    rng = np.random.Generator(np.random.PCG64(61))
    B, N, K, d = 2, 900, 30, 5
    X = rng.normal(size=(B, N, d)).astype(np.float32)
    lab = rng.integers(0, K - 3, size=(B, N)).astype(np.int32)   # last 3 clusters empty
    Cprev = rng.normal(size=(B, K, d)).astype(np.float32)
    counts, Cn, bad = orc.update(X, lab, Cprev)
    assert bad == 0
    for b in range(B):
        assert np.array_equal(counts[b], np.bincount(lab[b], minlength=K))
        for k in range(K):
            m = lab[b] == k
            if m.any():
                assert np.allclose(Cn[b, k], X[b][m].astype(np.float64).mean(0),
                                   rtol=1e-13, atol=1e-13)
            else:
                assert np.array_equal(Cn[b, k], Cprev[b, k].astype(np.float64)), "empty moved"


def pin_empty_keeps_previous(orc):
    rng = np.random.Generator(np.random.PCG64(71))
    X = rng.normal(size=(1, 200, 4))
    C = rng.normal(size=(1, 5, 4))
    C[0, 3] = 1e6                                   # nobody is near centroid 3
    labels, _, _ = orc.assign(X, C)
    counts, Cn, _ = orc.update(X, labels, C)
    assert counts[0, 3] == 0 and counts.sum() == 200
    assert np.array_equal(Cn[0, 3], C[0, 3])


# --------------------------------------------------------------------------
# iteration
# --------------------------------------------------------------------------
def _planted(seed=81, K=6, d=5, N=600):
    rng = np.random.Generator(np.random.PCG64(seed))
    mu = rng.normal(size=(K, d)) * 100.0
    z = rng.integers(0, K, size=N)
    z[:K] = np.arange(K)            # every component present
    rng.shuffle(z)
    X = mu[z] + rng.normal(size=(N, d))
    return X, z


def pin_planted_partition(orc):
    """Well separated components, one initial centroid inside each: after one
    iteration the labels are the components, the centroids their sample means,
    and a second iteration changes nothing."""
    X, z = _planted()
    K = int(z.max()) + 1
    first = np.array([np.flatnonzero(z == k)[0] for k in range(K)])
    order = np.argsort(first)                    # init = first point of each component, in order
    init_rows = first[order]
    C0 = X[init_rows][None]
    comp_of_centroid = z[init_rows]
    labels, _, _ = orc.assign(X[None], C0)
    assert np.array_equal(comp_of_centroid[labels[0]], z), "planted labels not recovered"
    counts, C1, _ = orc.update(X[None], labels, C0)
    assert np.array_equal(counts[0], np.bincount(z, minlength=K)[comp_of_centroid])
    for k in range(K):
        assert np.allclose(C1[0, k], X[z == comp_of_centroid[k]].mean(0), rtol=1e-13, atol=1e-11)
    labels2, _, _ = orc.assign(X[None], C1)
    counts2, C2, _ = orc.update(X[None], labels2, C1)
    assert np.array_equal(labels2, labels) and np.array_equal(C2, C1), "not a fixed point"


def pin_objective_nonincreasing(orc):
    X, C0 = synth.make(1, N=2048, K=16, d=12)
    X = X.numpy()
    C0 = C0.numpy().astype(np.float64)
    _, labels, counts, obj = orc.lloyd(X, C0, 8)
    assert np.all(obj[1:] <= obj[:-1] * (1 + 1e-12)), f"objective increased: {obj}"
    assert counts.sum() == 2048
    assert np.array_equal(counts[0], np.bincount(labels[0], minlength=16))


def pin_lloyd_is_assign_then_update(orc):
    rng = np.random.Generator(np.random.PCG64(91))
    X = rng.normal(size=(2, 300, 4))
    C0 = rng.normal(size=(2, 9, 4))
    CT, labT, cntT, _ = orc.lloyd(X, C0, 3)
    C = C0
    for _ in range(3):
        lab, _, _ = orc.assign(X, C)
        cnt, C, _ = orc.update(X, lab, C)
    assert np.array_equal(labT, lab) and np.array_equal(cntT, cnt) and np.array_equal(CT, C)


def pin_rows_subset(orc):
    rng = np.random.Generator(np.random.PCG64(95))
    X = rng.normal(size=(3, 400, 7)).astype(np.float32)
    C = rng.normal(size=(3, 20, 7)).astype(np.float32)
    full, f1, f2 = orc.assign(X, C)
    rows = rng.choice(3 * 400, 150, replace=False)
    sub, s1, s2 = orc.assign(X, C, rows=rows)
    assert np.array_equal(sub, full.reshape(-1)[rows])
    assert np.array_equal(s1, f1.reshape(-1)[rows]) and np.array_equal(s2, f2.reshape(-1)[rows])


ALL_PINS = [
    pin_decode_f16, pin_decode_bf16, pin_encode_f16, pin_encode_bf16,
    pin_distance_expansion, pin_exact_tiny_integers, pin_scipy_vq, pin_d1_closed_form,
    pin_self_assignment, pin_k1_mean, pin_counts_and_member_means, pin_empty_keeps_previous,
    pin_planted_partition, pin_objective_nonincreasing, pin_lloyd_is_assign_then_update,
    pin_rows_subset,
]
