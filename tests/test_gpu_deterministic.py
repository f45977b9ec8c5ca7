"""Run-to-run reproducibility on the GPU: the argsort is stable (points of a
label in increasing index order), the update of segments of at most 256
points is reproducible by default, and FK_DETERMINISTIC makes every update
and Lloyd run bit-identical (long segments added in piece order)."""
import numpy as np
import pytest
import torch

import exact_lloyd_means_amd as fk
import synth
from parity import TORCH, check_update

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"


@pytest.mark.parametrize("K", [1, 7, 1000, 4096, 16000, 16001, 65536, 70000])
def test_argsort_is_stable(K):
    """Tiled counting sort up to K = 16000, radix passes above (two for
    K <= 65536, three beyond)."""
    B, N = 2, 3 * 4096 + 1234          # several sort tiles and a ragged tail
    rng = np.random.Generator(np.random.PCG64(K))
    lab = rng.integers(0, K, size=(B, N)).astype(np.int32)
    lab[0, : N // 3] = K // 2          # one long run
    lab[1, ::97] = -1                   # skipped labels
    lab[1, 5::89] = K
    labels = torch.from_numpy(lab).cuda()
    counts = torch.empty((B, K), dtype=torch.int32, device="cuda")
    offsets = torch.empty((B, K + 1), dtype=torch.int32, device="cuda")
    sidx = torch.empty((B, N), dtype=torch.int32, device="cuda")
    fk.fk_sort_labels(labels, K, counts, offsets, sidx)
    torch.cuda.synchronize()
    for b in range(B):
        valid = np.flatnonzero((lab[b] >= 0) & (lab[b] < K))
        ref = valid[np.argsort(lab[b][valid], kind="stable")]
        assert np.array_equal(sidx[b, : ref.size].cpu().numpy(), ref)
        assert int(offsets[b, K]) == ref.size


def skewed_case(B, N, K, d, dt, seed):
    g = torch.Generator().manual_seed(seed)
    X = torch.randn((B, N, d), generator=g).to(TORCH[dt]).cuda()
    C = torch.randn((B, K, d), generator=g).float().cuda()
    rng = np.random.Generator(np.random.PCG64(seed))
    lab = rng.integers(0, K, size=(B, N)).astype(np.int32)
    lab[:, : N // 2] = 3               # a segment of N/2 points: many pieces
    lab[:, N // 2: N // 2 + 700] = K - 1
    return X, C, torch.from_numpy(lab).cuda()


def run_update(X, C, labels, deterministic):
    B, K, d = C.shape
    Cn = torch.empty_like(C)
    low = torch.empty((B, K, d), dtype=X.dtype, device="cuda") if X.dtype != torch.float32 else None
    counts = torch.empty((B, K), dtype=torch.int32, device="cuda")
    fk.fk_update(X, labels, C, Cn, low, counts, deterministic=deterministic)
    torch.cuda.synchronize()
    return Cn, low, counts


def test_short_segments_reproducible_by_default():
    X, _ = synth.make(2, B=2, N=3000, K=64)
    X = X.cuda()
    C = torch.randn((2, 64, X.shape[2])).cuda()
    labels = torch.randint(0, 64, (2, 3000), dtype=torch.int32).cuda()
    a = run_update(X, C, labels, False)
    b = run_update(X, C, labels, False)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("shape", [(2, 20000, 50, 128), (1, 9000, 300, 40), (3, 5000, 16, 1024)],
                         ids=lambda s: "x".join(map(str, s)))
def test_deterministic_update(dt, shape):
    B, N, K, d = shape
    X, C, labels = skewed_case(B, N, K, d, dt, seed=N + d)
    runs = [run_update(X, C, labels, True) for _ in range(3)]
    for r in runs[1:]:
        assert torch.equal(r[0], runs[0][0]) and torch.equal(r[2], runs[0][2])
        if r[1] is not None:
            assert torch.equal(r[1], runs[0][1])
    check_update(X, labels, C, runs[0][0], runs[0][2], C_lowp=runs[0][1])
    # same counts and close centroids as the default (atomic) mode
    ref = run_update(X, C, labels, False)
    assert torch.equal(ref[2], runs[0][2])
    assert torch.allclose(ref[0], runs[0][0], rtol=1e-5, atol=1e-6)


def test_deterministic_lloyd_bit_identical():
    X, C0 = synth.make(3, N=60000, K=256)      # Zipf cluster sizes: long segments
    X = X.cuda()
    out = []
    for _ in range(2):
        C = C0.cuda().clone()
        labels = torch.empty((1, 60000), dtype=torch.int32, device="cuda")
        counts = torch.empty((1, 256), dtype=torch.int32, device="cuda")
        fk.fk_lloyd(X, C, labels, counts, 4, deterministic=True)
        torch.cuda.synchronize()
        out.append((C, labels, counts))
    assert int(out[0][2].max()) > 256
    assert torch.equal(out[0][0], out[1][0]) and torch.equal(out[0][1], out[1][1])


def test_deterministic_api():
    X, _ = synth.make(2, B=2, N=5000, K=32)
    X = X.cuda()
    a = fk.batch_kmeans_euclid(X, 32, max_iter=5, deterministic=True)
    b = fk.batch_kmeans_euclid(X, 32, max_iter=5, deterministic=True)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_deterministic_update_large_K(dt):
    """K above the tiled sort (radix argsort), long and empty segments."""
    X, C, labels = skewed_case(2, 30000, 20000, 64, dt, seed=7)
    runs = [run_update(X, C, labels, True) for _ in range(2)]
    assert torch.equal(runs[0][0], runs[1][0]) and torch.equal(runs[0][2], runs[1][2])
    check_update(X, labels, C, runs[0][0], runs[0][2], C_lowp=runs[0][1])
