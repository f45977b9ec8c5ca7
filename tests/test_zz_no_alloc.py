"""fk_update_bias_noalloc (the library's static per-device scratch, nothing
allocated) against fk_update_bias (the caller's workspace) on the same
inputs, through the C ABI.

Two calls in a row, the second on a smaller problem, so the second runs on
scratch that still holds the first call's contents: a region the update
fails to clear shows up as a difference.  With the deterministic flag both
entry points run the same kernels in a fixed order, so every output is
compared bit for bit.  Without it, segments longer than 256 points add
their pieces with atomics in timing order: counts stay bit-exact and the
centroids agree within the update's fp32 tolerance (one rounding per
added piece), and the bias is checked against the centroids written.
"""
import pytest
import torch

import exact_lloyd_means_amd as fk
import synth
from parity import CTOL

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"


def inputs(cfg, N=None, B=None, K=None, d=None, dtype=None, seed=None):
    """Seeded points and initial centroids of a workload (optionally shrunk)
    and the labels the fused assignment gives them."""
    X_cpu, C0 = synth.make(cfg, N=N, B=B, K=K, d=d, dtype=dtype, seed=seed)
    X = X_cpu.cuda()
    C = C0.cuda()
    Cq = C.to(X.dtype).contiguous() if X.dtype != torch.float32 else C.clone()
    bias = torch.empty(C.shape[:2], dtype=torch.float32, device="cuda")
    fk.fk_centroid_bias(Cq, bias)
    labels = torch.empty(X.shape[:2], dtype=torch.int32, device="cuda")
    fk.fk_assign_with_bias(X, Cq, bias, labels)
    return X, C, labels


def outputs(X, C):
    B, K, d = C.shape
    lowp = torch.full((B, K, d), float("nan"), dtype=X.dtype, device="cuda") \
        if X.dtype != torch.float32 else None
    return dict(C_next=torch.full_like(C, float("nan")), lowp=lowp,
                counts=torch.full((B, K), -7, dtype=torch.int32, device="cuda"),
                bias=torch.full((B, K), float("nan"), dtype=torch.float32, device="cuda"))


def run_pair(X, C, labels, deterministic, stream=None):
    """The same update through both entry points; returns (workspace, noalloc)."""
    ref, got = outputs(X, C), outputs(X, C)
    fk.fk_update_bias(X, labels, C, ref["C_next"], ref["lowp"], ref["counts"], ref["bias"],
                      deterministic=deterministic)
    torch.cuda.synchronize()
    fk.fk_update_bias_noalloc(X, labels, C, got["C_next"], got["lowp"], got["counts"],
                              got["bias"], stream=stream, deterministic=deterministic)
    torch.cuda.synchronize()
    return ref, got


def assert_same(ref, got, exact, fmt):
    assert torch.equal(ref["counts"], got["counts"]), "counts differ"
    if exact:
        assert torch.equal(ref["C_next"], got["C_next"]), "centroids differ"
        if ref["lowp"] is not None:
            assert torch.equal(ref["lowp"], got["lowp"]), "low-precision centroids differ"
        assert torch.equal(ref["bias"], got["bias"]), "bias differs"
        return
    a, b = ref["C_next"].double(), got["C_next"].double()
    err = (a - b).abs().amax(-1)
    scale = a.abs().amax(-1).clamp_min(1e-30)
    assert bool((err <= CTOL[fmt] * scale).all()), float((err / scale).max())
    # the bias written is that of the centroids written
    src = got["lowp"] if got["lowp"] is not None else got["C_next"]
    chk = torch.empty_like(got["bias"])
    fk.fk_centroid_bias(src, chk)
    torch.cuda.synchronize()
    assert torch.equal(chk, got["bias"]), "bias is not that of the written centroids"


@pytest.mark.timeout(300)
def test_noalloc_matches_workspace_entry_point():
    # call 1: the B=32, N=65536, K=1024, d=128 fp16 mixture workload at its
    # full size, deterministic: bit for bit
    X, C, labels = inputs(2)
    print("[noalloc] call 1: B=32 N=65536 K=1024 d=128 f16, deterministic", flush=True)
    ref, got = run_pair(X, C, labels, deterministic=True)
    assert_same(ref, got, exact=True, fmt="f16")
    assert int(got["counts"].sum()) == X.shape[0] * X.shape[1]
    # call 2: smaller, ragged, bf16, on a side stream; every segment is under
    # 256 points (about 43 per label), so no atomics: bit for bit
    del X, C, labels, ref, got
    X, C, labels = inputs(2, B=2, N=3000, K=70, d=96, dtype="bf16", seed=77)
    print("[noalloc] call 2: B=2 N=3000 K=70 d=96 bf16, side stream", flush=True)
    side = torch.cuda.Stream()
    ref, got = run_pair(X, C, labels, deterministic=False, stream=side)
    assert_same(ref, got, exact=True, fmt="bf16")


@pytest.mark.timeout(300)
def test_noalloc_default_flags_within_tolerance():
    # the default (atomic) path at full size, then a smaller Zipf problem
    # whose head clusters exceed 256 points
    X, C, labels = inputs(2)
    print("[noalloc] B=32 N=65536 K=1024 d=128 f16, default flags", flush=True)
    ref, got = run_pair(X, C, labels, deterministic=False)
    assert_same(ref, got, exact=False, fmt="f16")
    del X, C, labels, ref, got
    X, C, labels = inputs(3, N=200_000, K=512, seed=91)
    print("[noalloc] Zipf N=200000 K=512 d=128 f16, default flags", flush=True)
    ref, got = run_pair(X, C, labels, deterministic=False)
    assert_same(ref, got, exact=False, fmt="f16")


def test_noalloc_rejects_problems_beyond_the_scratch():
    X = torch.empty((1, 1 << 24, 128), dtype=torch.float16, device="cuda")
    C = torch.zeros((1, 4096, 128), dtype=torch.float32, device="cuda")
    labels = torch.zeros((1, 1 << 24), dtype=torch.int32, device="cuda")
    counts = torch.full((1, 4096), -7, dtype=torch.int32, device="cuda")
    bias = torch.empty((1, 4096), dtype=torch.float32, device="cuda")
    with pytest.raises(RuntimeError, match="static scratch"):
        fk.fk_update_bias_noalloc(X, labels, C, C, None, counts, bias)
    torch.cuda.synchronize()
    assert bool((counts == -7).all()), "a rejected call wrote its outputs"
