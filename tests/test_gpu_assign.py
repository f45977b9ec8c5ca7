"""Fused assign (fk_assign) against the fp64 oracle on the GPU."""
import numpy as np
import pytest
import torch

import exact_lloyd_means_amd as fk
import oracle
import synth
from parity import TORCH, check_labels, to_storage

pytestmark = pytest.mark.gpu

DT = ["f32", "f16", "bf16"]


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    torch.cuda.init()


def run_assign(X, C, with_dist=True):
    B, N, _ = X.shape
    labels = torch.empty((B, N), dtype=torch.int32, device="cuda")
    md = torch.empty((B, N), dtype=torch.float32, device="cuda") if with_dist else None
    fk.fk_assign(X, C, labels, md)
    torch.cuda.synchronize()
    return labels, md


def int_case(B, N, K, d, dt, seed):
    Xi, Ci = synth.integer_problem(B, N, K, d, seed=seed)
    X = torch.from_numpy(Xi).to(TORCH[dt]).cuda()
    C = torch.from_numpy(Ci).to(TORCH[dt]).cuda()
    return Xi, Ci, X, C


@pytest.mark.parametrize("dt", DT)
def test_golden_tie_case(dt):
    import test_golden
    g = test_golden.load_golden()
    X = torch.tensor(g["X"], dtype=TORCH[dt], device="cuda")
    C = torch.tensor(g["C"], dtype=TORCH[dt], device="cuda")
    labels, md = run_assign(X, C)
    assert labels.cpu().numpy().tolist() == g["labels"].tolist()
    assert np.array_equal(md.cpu().numpy().astype(np.float64), g["d1"])


SHAPES_INT = [(1, 1, 1, 1), (2, 37, 5, 3), (3, 300, 70, 2), (1, 1000, 33, 3), (2, 129, 1, 1),
              (1, 5, 9, 2), (2, 700, 64, 16), (1, 513, 100, 127), (2, 300, 40, 128),
              (1, 257, 65, 129), (1, 200, 50, 256), (1, 300, 300, 1024), (1, 100, 40, 600)]


@pytest.mark.parametrize("dt", DT)
@pytest.mark.parametrize("shape", SHAPES_INT, ids=lambda s: "x".join(map(str, s)))
def test_integer_ties_exact(dt, shape):
    """Integer inputs: every product and partial sum is exact in fp32, so the
    GPU must reproduce the lowest-index tie rule bit for bit (no exclusions)."""
    B, N, K, d = shape
    Xi, Ci, X, C = int_case(B, N, K, d, dt, seed=hash(shape) % 1000)
    labels, md = run_assign(X, C)
    lab, d1, _ = oracle.assign(Xi.astype(np.float64), Ci.astype(np.float64))
    assert np.array_equal(labels.cpu().numpy(), lab)
    assert np.array_equal(md.cpu().numpy().astype(np.float64), d1)


@pytest.mark.parametrize("dt", DT)
@pytest.mark.parametrize("B,N,K,d", [(2, 3000, 64, 16), (1, 2000, 100, 128), (1, 1500, 1000, 64),
                                     (1, 700, 45, 256), (1, 500, 300, 1024)])
def test_duplicate_centroids_take_the_lowest_copy(dt, B, N, K, d):
    """Centroid k repeats centroid k mod 7, so copies tie exactly (same values,
    same score) inside a tile, across tiles and in the overlapping last tile:
    the lowest index rule puts every label below 7, whatever the rounding of
    the scores.  Zero points (score = bias alone) are included."""
    g = torch.Generator().manual_seed(B * 7 + N + K + d)
    X = torch.randn((B, N, d), generator=g)
    X[:, :5] = 0.0
    base = torch.randn((B, 7, d), generator=g)
    C = base[:, torch.arange(K) % 7]
    X, C = X.to(TORCH[dt]).cuda(), C.to(TORCH[dt]).contiguous().cuda()
    labels, md = run_assign(X, C)
    lab = labels.cpu()
    assert int(lab.min()) >= 0 and int(lab.max()) < 7
    # and the copy chosen is the nearest of the 7 distinct centroids
    check_labels(labels, X, C[:, :7].contiguous())


CFG_SHRUNK = {1: dict(), 2: dict(B=2, N=8192), 3: dict(N=16384), 4: dict(N=3000, K=1100)}


@pytest.mark.parametrize("cfg", sorted(CFG_SHRUNK))
def test_config_inputs(cfg):
    X, C0 = synth.make(cfg, **CFG_SHRUNK[cfg])
    X = X.cuda()
    Cq = C0.to(X.dtype).cuda()
    labels, md = run_assign(X, Cq)
    stats = check_labels(labels, X, Cq, min_dist=md)
    print(cfg, stats)


EDGE = [(1, 1, 1, 1), (1, 31, 2, 2), (2, 33, 31, 3), (1, 257, 33, 8), (3, 1000, 100, 17),
        (1, 300, 64, 64), (1, 129, 100, 127), (2, 500, 97, 128), (1, 250, 130, 129),
        (1, 200, 70, 200), (1, 130, 40, 256), (1, 100, 35, 300), (1, 70, 33, 512),
        # row strides of 8 or 4 bytes (rows loaded in 8- or 4-byte units)
        (1, 300, 70, 98), (2, 200, 90, 100), (1, 120, 260, 258), (1, 300, 64, 20),
        (2, 100, 40, 6), (1, 250, 130, 228), (1, 250, 130, 250), (2, 300, 97, 196),
        # rows longer than the register-resident limit: split-d kernel
        (1, 300, 70, 513), (2, 257, 300, 1024), (1, 100, 40, 1000), (1, 64, 33, 1100),
        (1, 150, 300, 516),
        (1, 600, 520, 640)]


@pytest.mark.parametrize("dt", DT)
@pytest.mark.parametrize("shape", EDGE, ids=lambda s: "x".join(map(str, s)))
def test_edge_shapes_random(dt, shape):
    B, N, K, d = shape
    g = torch.Generator().manual_seed(B * 1000003 + N * 1009 + K * 31 + d)
    X = torch.randn((B, N, d), generator=g).to(TORCH[dt]).cuda()
    C = (torch.randn((B, K, d), generator=g) * 1.2).to(TORCH[dt]).cuda()
    labels, md = run_assign(X, C)
    check_labels(labels, X, C, min_dist=md)


def test_K_larger_than_N_and_one_centroid():
    X = torch.randn((2, 50, 40)).half().cuda()
    C = torch.randn((2, 300, 40)).half().cuda()
    labels, md = run_assign(X, C)
    check_labels(labels, X, C, min_dist=md)
    C1 = torch.randn((2, 1, 40)).half().cuda()
    labels, _ = run_assign(X, C1)
    assert int(labels.abs().sum()) == 0


def test_bit_reproducible():
    X, C0 = synth.make(2, B=2, N=4096)
    X = X.cuda()
    C = C0.half().cuda()
    a, ma = run_assign(X, C)
    b, mb = run_assign(X, C)
    assert torch.equal(a, b) and torch.equal(ma, mb)


def test_misaligned_view_rejected():
    X = torch.randn((1, 65, 8)).half().cuda()
    C = torch.randn((1, 4, 8)).half().cuda()
    Xv = X.view(-1)[1:1 + 64 * 8].view(1, 64, 8)   # 2-byte offset
    labels = torch.empty((1, 64), dtype=torch.int32, device="cuda")
    with pytest.raises(fk.FKError):
        fk.fk_assign(Xv, C, labels)


@pytest.mark.parametrize("dt", DT)
def test_assign_with_bias_matches_assign(dt):
    X, C0 = synth.make(2, B=2, N=3000, K=300, dtype=dt)
    X = X.cuda()
    C = C0.to(X.dtype).cuda()
    a, ma = run_assign(X, C)
    bias = torch.empty((2, 300), dtype=torch.float32, device="cuda")
    fk.fk_centroid_bias(C, bias)
    lab = torch.empty_like(a)
    md = torch.empty_like(ma)
    fk.fk_assign_with_bias(X, C, bias, lab, md)
    torch.cuda.synchronize()
    assert torch.equal(a, lab) and torch.equal(ma, md)
    # the bias is -|c|^2/2 of the stored values
    cc = oracle.decode(to_storage(C), dt).astype(np.float64)
    ref = -0.5 * (cc ** 2).sum(-1)
    assert np.allclose(bias.cpu().numpy(), ref, rtol=1e-6, atol=1e-6)


@pytest.mark.parametrize("dt", DT)
@pytest.mark.parametrize("shape", [(2, 700, 90, 128), (1, 600, 300, 1024), (1, 300, 20, 40)],
                         ids=lambda s: "x".join(map(str, s)))
def test_nonfinite_points_leave_the_others_alone(dt, shape):
    """Labels of points with NaN or infinite coordinates are undefined, but
    they stay in [0, K) and every finite point still gets its oracle label
    (each point's running minimum is its own; resident, split-d and
    element-load kernels)."""
    B, N, K, d = shape
    g = torch.Generator().manual_seed(N + K + d)
    X = torch.randn((B, N, d), generator=g)
    C = torch.randn((B, K, d), generator=g) * 1.2
    bad = torch.zeros((B, N), dtype=torch.bool)
    bad[:, 3::17] = True
    X[:, 3::17, 5] = float("nan")
    X[:, 10::17] = float("inf")
    bad[:, 10::17] = True
    X[:, 12::17, 0] = float("-inf")
    bad[:, 12::17] = True
    X = X.to(TORCH[dt]).cuda()
    C = C.to(TORCH[dt]).cuda()
    labels, _ = run_assign(X, C)
    lab = labels.cpu()
    assert int(lab.min()) >= 0 and int(lab.max()) < K
    rows = np.flatnonzero(~bad.reshape(-1).numpy())
    check_labels(labels, X, C, rows=rows)
