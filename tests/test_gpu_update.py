"""Sort-inverse update (fk_sort_labels, fk_update) against the oracle on the GPU."""
import numpy as np
import pytest
import torch

import exact_lloyd_means_amd as fk
import oracle
from parity import TORCH, check_update

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"


def sort_labels(labels, K):
    B, N = labels.shape
    counts = torch.empty((B, K), dtype=torch.int32, device="cuda")
    offsets = torch.empty((B, K + 1), dtype=torch.int32, device="cuda")
    sidx = torch.empty((B, N), dtype=torch.int32, device="cuda")
    fk.fk_sort_labels(labels, K, counts, offsets, sidx)
    torch.cuda.synchronize()
    return counts.cpu().numpy(), offsets.cpu().numpy(), sidx.cpu().numpy()


def check_sort(lab, K, counts, offsets, sidx):
    B = lab.shape[0]
    for b in range(B):
        ref = np.bincount(lab[b], minlength=K)
        assert np.array_equal(counts[b], ref)
        assert offsets[b, 0] == 0 and np.array_equal(offsets[b, 1:], np.cumsum(ref))
    assert oracle.argsort_valid(lab, sidx, K)


@pytest.mark.parametrize("B,N,K", [(1, 1, 1), (3, 10000, 777), (2, 4097, 1024), (1, 5000, 9000),
                                   (1, 70000, 65536), (2, 100, 16384), (1, 3000, 16385)])
def test_sort_uniform(B, N, K):
    g = torch.Generator().manual_seed(N + K)
    lab = torch.randint(0, K, (B, N), generator=g, dtype=torch.int32)
    c, o, s = sort_labels(lab.cuda(), K)
    check_sort(lab.numpy(), K, c, o, s)


@pytest.mark.parametrize("B,N,K", [(1, 300001, 700), (3, 300001, 4096), (1, 262145, 5000),
                                   (2, 4096 * 64, 3)])
def test_sort_many_tiles(B, N, K):
    """64 or more sort tiles per problem (the wide column pass), a ragged
    last tile, tile counts that are not a multiple of the 8 XCDs (padding
    workgroups of the per-XCD tile runs), both tiled scatters (K <= 4096 and
    above): the argsort must equal numpy's stable argsort exactly."""
    g = torch.Generator().manual_seed(N + K + B)
    j = torch.arange(1, K + 1, dtype=torch.float64)
    p = j.pow(-1.2)
    lab = torch.multinomial(p / p.sum(), B * N, replacement=True, generator=g).int().view(B, N)
    c, o, s = sort_labels(lab.cuda(), K)
    check_sort(lab.numpy(), K, c, o, s)
    for b in range(B):
        assert np.array_equal(s[b], np.argsort(lab[b].numpy(), kind="stable"))


def test_sort_skewed_and_constant():
    g = torch.Generator().manual_seed(5)
    K = 4096
    j = torch.arange(1, K + 1, dtype=torch.float64)
    p = j.pow(-1.2)
    lab = torch.multinomial(p / p.sum(), 200000, replacement=True, generator=g).int().view(1, -1)
    c, o, s = sort_labels(lab.cuda(), K)
    check_sort(lab.numpy(), K, c, o, s)
    lab0 = torch.zeros((2, 50000), dtype=torch.int32)
    c, o, s = sort_labels(lab0.cuda(), 10)
    check_sort(lab0.numpy(), 10, c, o, s)


def run_update(X, labels, C_prev, want_lowp=True):
    B, N, d = X.shape
    K = C_prev.shape[1]
    C_next = torch.empty_like(C_prev)
    lowp = torch.empty((B, K, d), dtype=X.dtype, device="cuda") if (
        want_lowp and X.dtype != torch.float32) else None
    counts = torch.empty((B, K), dtype=torch.int32, device="cuda")
    fk.fk_update(X, labels, C_prev, C_next, lowp, counts)
    torch.cuda.synchronize()
    return C_next, lowp, counts


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("B,N,K,d", [(1, 1, 1, 1), (2, 5000, 100, 128), (1, 3000, 700, 3),
                                     (3, 2000, 50, 129), (1, 1000, 20, 1024), (1, 4097, 64, 100),
                                     (2, 100, 300, 64), (1, 300001, 3000, 16)])
def test_update_vs_oracle(dt, B, N, K, d):
    g = torch.Generator().manual_seed(B + N + K + d)
    X = torch.randn((B, N, d), generator=g).to(TORCH[dt]).cuda()
    # leave a few clusters empty
    lab = torch.randint(0, max(1, K - 3), (B, N), generator=g, dtype=torch.int32).cuda()
    C_prev = torch.randn((B, K, d), generator=g).cuda()
    C_next, lowp, counts = run_update(X, lab, C_prev)
    check_update(X, lab, C_prev, C_next, counts, lowp)


def test_update_in_place_alias():
    X = torch.randn((1, 3000, 64)).half().cuda()
    lab = torch.randint(0, 40, (1, 3000), dtype=torch.int32).cuda()
    C = torch.randn((1, 50, 64)).cuda()
    C0 = C.clone()
    counts = torch.empty((1, 50), dtype=torch.int32, device="cuda")
    fk.fk_update(X, lab, C, C, None, counts)
    torch.cuda.synchronize()
    check_update(X, lab, C0, C, counts)


def test_update_single_hot_cluster():
    """Every point in one cluster: the whole sorted range is one segment."""
    X = torch.randn((1, 200000, 128)).half().cuda()
    lab = torch.zeros((1, 200000), dtype=torch.int32).cuda()
    C_prev = torch.randn((1, 8, 128)).cuda()
    C_next, lowp, counts = run_update(X, lab, C_prev)
    check_update(X, lab, C_prev, C_next, counts, lowp)


def test_update_out_of_range_labels_skipped():
    B, N, K, d = 2, 3000, 30, 16
    X = torch.randn((B, N, d)).cuda()
    lab = torch.randint(0, K, (B, N), dtype=torch.int32)
    lab[0, ::7] = -1
    lab[1, ::11] = K
    C_prev = torch.randn((B, K, d)).cuda()
    p = fk.problem(B, N, K, d, torch.float32)
    ws = fk.workspace(p)
    C_next = torch.empty_like(C_prev)
    counts = torch.empty((B, K), dtype=torch.int32, device="cuda")
    fk.fk_update(X, lab.cuda(), C_prev, C_next, None, counts, ws=ws)
    n_bad = fk.fk_error_count(p, ws)
    assert n_bad == int((lab < 0).sum() + (lab >= K).sum())
    check_update(X, lab, C_prev, C_next, counts)


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("shape", [(2, 3000, 300, 128), (1, 5000, 40, 40), (2, 900, 500, 1000)],
                         ids=lambda s: "x".join(map(str, s)))
def test_update_bias_matches_centroid_bias(dt, shape):
    """fk_update_bias: the same update as fk_update, and a next-assignment
    bias bit-identical to fk_centroid_bias of the new (rounded) centroids,
    for single-piece, multi-piece and empty segments."""
    import synth
    B, N, K, d = shape
    X, _ = synth.make(2, B=B, N=N, K=K, d=d, dtype=dt)
    X = X.cuda()
    g = torch.Generator().manual_seed(N + d)
    lab = torch.randint(0, K, (B, N), generator=g, dtype=torch.int32)
    lab[:, : N // 3] = 1                  # a long segment; most labels unused when K > N
    labels = lab.cuda()
    C = torch.randn((B, K, d), generator=g).cuda()
    Cn = torch.empty_like(C)
    low = torch.empty((B, K, d), dtype=X.dtype, device="cuda") if dt != "f32" else None
    counts = torch.empty((B, K), dtype=torch.int32, device="cuda")
    bias = torch.empty((B, K), dtype=torch.float32, device="cuda")
    fk.fk_update_bias(X, labels, C, Cn, low, counts, bias)
    Cn2 = torch.empty_like(C)
    counts2 = torch.empty_like(counts)
    fk.fk_update(X, labels, C, Cn2, None, counts2)
    ref = torch.empty_like(bias)
    fk.fk_centroid_bias(low if low is not None else Cn, ref)
    torch.cuda.synchronize()
    assert torch.equal(counts, counts2)
    assert torch.equal(bias, ref)
    check_update(X, labels, C, Cn, counts, C_lowp=low)
