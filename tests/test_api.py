"""Host-side behaviour of the user-facing API (exact_lloyd_means_amd.api):
argument checks and the choice of initial centroids, on CPU tensors."""
import pytest
import torch

from exact_lloyd_means_amd import KMeans, batch_kmeans_euclid, initial_centroids


def test_inputs_must_be_on_the_gpu():
    X = torch.randn(100, 8)
    with pytest.raises(ValueError, match="GPU"):
        KMeans(4).fit(X)
    with pytest.raises(ValueError, match="GPU"):
        batch_kmeans_euclid(X.unsqueeze(0), 4)


def test_predict_before_fit():
    with pytest.raises(RuntimeError):
        KMeans(4).predict(torch.randn(10, 8))


def test_initial_centroids_first_and_cycle():
    X = torch.arange(2 * 5 * 3, dtype=torch.float32).reshape(2, 5, 3)
    C = initial_centroids(X, 3, "first")
    assert torch.equal(C, X[:, :3])
    C = initial_centroids(X, 7, "sample")          # K > N: points repeat cyclically
    assert torch.equal(C, X[:, [0, 1, 2, 3, 4, 0, 1]])


def test_initial_centroids_sample_is_seeded_and_distinct():
    X = torch.randn(3, 50, 4)
    a = initial_centroids(X, 10, "sample", seed=5)
    b = initial_centroids(X, 10, "sample", seed=5)
    c = initial_centroids(X, 10, "sample", seed=6)
    assert torch.equal(a, b) and not torch.equal(a, c)
    for bb in range(3):
        rows = {tuple(r.tolist()) for r in a[bb]}
        assert len(rows) == 10
        assert all(any(torch.equal(r, x) for x in X[bb]) for r in a[bb])


def test_initial_centroids_given():
    X = torch.randn(2, 20, 4, dtype=torch.float16)
    C0 = torch.randn(6, 4)
    C = initial_centroids(X, 6, C0)
    assert C.shape == (2, 6, 4) and C.dtype == torch.float32
    assert torch.equal(C[0], C0) and torch.equal(C[1], C0)
    with pytest.raises(ValueError):
        initial_centroids(X, 6, torch.randn(5, 4))
    with pytest.raises(ValueError):
        initial_centroids(X, 6, "kmeans++")
