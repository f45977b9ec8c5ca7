"""The user-facing API on the GPU: it marshals to the same kernels as the C
ABI (bit-identical results) and its reported statistics are those of the
final centroids."""
import numpy as np
import pytest
import torch

import exact_lloyd_means_amd as fk
import oracle
import synth
from parity import check_labels, to_storage

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"


@pytest.mark.parametrize("dt", ["f32", "f16"])
def test_batch_function_matches_c_abi(dt):
    X, _ = synth.make(2, B=2, N=3000, K=64, dtype=dt)
    X = X.cuda()
    labels, C, n = fk.batch_kmeans_euclid(X, 64, max_iter=4, init="sample", seed=3)
    assert n == 4
    C0 = fk.initial_centroids(X, 64, "sample", seed=3)
    lab2 = torch.empty_like(labels)
    cnt = torch.empty((2, 64), dtype=torch.int32, device="cuda")
    fk.fk_lloyd(X, C0, lab2, cnt, 4)
    torch.cuda.synchronize()
    # same kernels: same labels; centroid low bits may differ between runs
    # outside the deterministic mode
    assert torch.equal(labels, lab2)
    assert torch.allclose(C, C0, rtol=1e-6, atol=1e-6)


def test_kmeans_estimator_statistics():
    X, _ = synth.make(1, N=4000, K=16)       # well separated mixture, fp32
    X2 = X[0].cuda()
    km = fk.KMeans(16, max_iter=50, tol=1e-6, init="sample", seed=1).fit(X2)
    assert km.cluster_centers_.shape == (16, X2.shape[1])
    assert 1 <= km.n_iter_ < 50                # converged before the limit
    # labels_ and inertia_ belong to the final centroids
    Cq = km.cluster_centers_.unsqueeze(0)
    check_labels(km.labels_.unsqueeze(0), X2.unsqueeze(0), Cq)
    lab = km.labels_.cpu().numpy().astype(np.int32)
    d = oracle.pair_dist(to_storage(X2.unsqueeze(0)), to_storage(Cq), np.arange(lab.size),
                         lab, fmt_x="f32", fmt_c="f32")
    assert abs(km.inertia_ - d.sum()) <= 1e-4 * d.sum()
    assert np.array_equal(km.counts_.cpu().numpy(), np.bincount(lab, minlength=16))
    # predict = the assignment to the final centroids
    assert torch.equal(km.predict(X2), km.labels_)
    Xn = torch.randn_like(X2)
    ref = torch.empty((1, Xn.shape[0]), dtype=torch.int32, device="cuda")
    fk.fk_assign(Xn.unsqueeze(0), Cq.contiguous(), ref)
    torch.cuda.synchronize()
    assert torch.equal(km.predict(Xn), ref[0])


def test_kmeans_batched_bf16():
    X, _ = synth.make(2, B=3, N=2048, K=32, dtype="bf16")
    X = X.cuda()
    km = fk.KMeans(32, max_iter=3, tol=0.0).fit(X)
    assert km.n_iter_ == 3
    assert km.labels_.shape == (3, 2048) and km.cluster_centers_.shape == (3, 32, X.shape[2])
    assert km.inertia_.shape == (3,)
    assert int(km.counts_.sum()) == 3 * 2048
    check_labels(km.labels_, X, km.cluster_centers_.to(torch.bfloat16))
