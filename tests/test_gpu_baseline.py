"""The unfused baselines (include/fk_baseline.h) on the GPU: the materialised
score matrix + argmin must give exactly the fused assign's labels (same fp32
scores, same tie rule) and pass the oracle; the scatter-atomic update must
give the oracle's counts exactly and its centroids within tolerance."""
import numpy as np
import pytest
import torch

import exact_lloyd_means_amd as fk
import oracle
import synth
from parity import TORCH, check_labels, check_update, to_storage

pytestmark = pytest.mark.gpu

# (B, N, K, d): several tiles with ragged tails, K below one tile, d not a
# multiple of 8 (element loads), K not a multiple of 4 (scalar score stores)
SHAPES = [(2, 3000, 300, 128), (1, 1000, 20, 64), (2, 777, 130, 40), (1, 513, 37, 256),
          (3, 64, 1, 16)]


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"


def random_case(B, N, K, d, dt):
    g = torch.Generator().manual_seed(B * 1000003 + N * 1009 + K * 31 + d)
    X = torch.randn((B, N, d), generator=g).to(TORCH[dt]).cuda()
    C = (torch.randn((B, K, d), generator=g) * 1.2).to(TORCH[dt]).cuda()
    return X, C


def materialised(X, C):
    B, N, _ = X.shape
    K = C.shape[1]
    bias = torch.empty((B, K), dtype=torch.float32, device="cuda")
    fk.fk_centroid_bias(C, bias)
    D = torch.full((B, N, K), float("nan"), dtype=torch.float32, device="cuda")
    fk.fk_baseline_scores(X, C, bias, D)
    lab = torch.empty((B, N), dtype=torch.int32, device="cuda")
    fk.fk_baseline_argmin(D, lab)
    torch.cuda.synchronize()
    return D, lab, bias


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_materialised_assign(dt, shape):
    B, N, K, d = shape
    X, C = random_case(B, N, K, d, dt)
    D, lab, bias = materialised(X, C)
    # every score written, each within fp32 accumulation error of the exact
    # x.c - |c|^2/2 of the stored values (d roundings of at most 2^-24 of the
    # magnitude sum, counted twice for the bias)
    assert not torch.isnan(D).any(), "score matrix not fully written"
    xs = oracle.decode(to_storage(X), dt)
    cs = oracle.decode(to_storage(C), dt)
    exact = np.einsum("bnd,bkd->bnk", xs, cs) - 0.5 * (cs ** 2).sum(-1)[:, None, :]
    scale = np.abs(xs).sum(-1)[:, :, None] * np.abs(cs).max(-1)[:, None, :] + \
        (cs ** 2).sum(-1)[:, None, :]
    assert np.all(np.abs(D.cpu().numpy() - exact) <= 2 * d * 2.0 ** -24 * scale + 1e-6)
    # the labels: those of the fused kernel on the same scores, bit for bit
    fused = torch.empty_like(lab)
    fk.fk_assign_with_bias(X, C, bias, fused)
    torch.cuda.synchronize()
    assert torch.equal(lab, fused)
    check_labels(lab, X, C)


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_materialised_integer_ties(dt):
    """Exact ties (duplicated centroids, midway points): lowest index."""
    Xi, Ci = synth.integer_problem(2, 700, 50, 3, seed=11)
    X = torch.from_numpy(Xi).to(TORCH[dt]).cuda()
    C = torch.from_numpy(Ci).to(TORCH[dt]).cuda()
    _, lab, _ = materialised(X, C)
    ref, _, _ = oracle.assign(to_storage(X), to_storage(C), fmt_x=dt, fmt_c=dt)
    assert np.array_equal(lab.cpu().numpy().reshape(-1), np.asarray(ref).reshape(-1))


def test_materialised_rejects_fp32():
    X = torch.randn((1, 64, 16)).cuda()
    C = torch.randn((1, 8, 16)).cuda()
    bias = torch.zeros((1, 8), device="cuda")
    D = torch.empty((1, 64, 8), device="cuda")
    with pytest.raises(fk.FKError):
        fk.fk_baseline_scores(X, C, bias, D)


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("shape", [(2, 3000, 300, 128), (1, 5000, 7, 40), (2, 100, 400, 33)],
                         ids=lambda s: "x".join(map(str, s)))
def test_scatter_update(dt, shape):
    B, N, K, d = shape
    X, C0 = random_case(B, N, K, d, dt)
    rng = np.random.Generator(np.random.PCG64(N + K))
    # a skewed label mix: half the points on one centroid, empties included
    lab_np = rng.integers(0, K, size=(B, N)).astype(np.int32)
    lab_np[:, : N // 2] = K // 3
    labels = torch.from_numpy(lab_np).cuda()
    C_prev = C0.float().contiguous()
    C_next = torch.empty_like(C_prev)
    low = torch.empty((B, K, d), dtype=X.dtype, device="cuda") if dt != "f32" else None
    counts = torch.empty((B, K), dtype=torch.int32, device="cuda")
    sums = torch.full((B, K, d), 7.0, device="cuda")   # cleared by the call
    fk.fk_baseline_update_scatter(X, labels, C_prev, C_next, low, counts, sums)
    torch.cuda.synchronize()
    check_update(X, labels, C_prev, C_next, counts, C_lowp=low)
    assert int(sums.abs().max()) == 0, "sums not left zero"
    # the fused update from the same labels: identical counts, close centroids
    c2 = torch.empty_like(counts)
    n2 = torch.empty_like(C_next)
    fk.fk_update(X, labels, C_prev, n2, None, c2)
    torch.cuda.synchronize()
    assert torch.equal(counts, c2)


def test_scatter_update_in_place_and_bad_labels():
    X, C0 = random_case(1, 2000, 50, 64, "f16")
    labels = torch.randint(0, 50, (1, 2000), dtype=torch.int32).cuda()
    labels[0, :10] = -1
    labels[0, 10:20] = 50
    C = C0.float().contiguous()
    C_prev = C.clone()
    counts = torch.empty((1, 50), dtype=torch.int32, device="cuda")
    sums = torch.empty((1, 50, 64), device="cuda")
    fk.fk_baseline_update_scatter(X, labels, C, C, None, counts, sums)
    torch.cuda.synchronize()
    assert int(counts.sum()) == 1980
    cnt_ref = np.bincount(labels[0, 20:].cpu().numpy(), minlength=50)
    assert np.array_equal(counts[0].cpu().numpy(), cnt_ref)
    # the 20 skipped points are left out of the oracle's update as well
    sub = X[:, 20:].contiguous()
    check_update(sub, labels[:, 20:].contiguous(), C_prev, C, counts)
