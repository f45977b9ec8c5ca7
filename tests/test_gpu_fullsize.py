"""Full-size workloads in exactly the launch sequence the benchmark times
(fused assign with the current bias -> in-place update writing the next
low-precision centroids and their bias), checked against the fp64 oracle:
labels on a
seeded random sample of points (the oracle computes them one by one), counts
and centroids of the update on every point."""
import numpy as np
import pytest
import torch

import exact_lloyd_means_amd as fk
import synth
from parity import check_labels, check_update

pytestmark = pytest.mark.gpu

# points whose labels the oracle recomputes, per workload
SAMPLE = {2: 8192, 3: 4096, 4: 384}
ITERS = {2: 2, 3: 2, 4: 1}


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"


@pytest.mark.parametrize("cfg", [2, 3, 4])
def test_full_size_lockstep(cfg):
    w = synth.CONFIGS[cfg]
    print(f"[fullsize] {w.name}: generating", flush=True)
    X_cpu, C0 = synth.make(cfg)
    X = X_cpu.cuda()
    B, N, d = X.shape
    K = C0.shape[1]
    C = C0.cuda()
    Cq = C.to(X.dtype).contiguous() if w.dtype != "f32" else C.clone()
    bias = torch.empty((B, K), dtype=torch.float32, device="cuda")
    labels = torch.empty((B, N), dtype=torch.int32, device="cuda")
    counts = torch.empty((B, K), dtype=torch.int32, device="cuda")
    ws = fk.workspace(fk.problem(B, N, K, d, X.dtype))
    rng = np.random.Generator(np.random.PCG64(500 + cfg))
    fk.fk_centroid_bias(Cq, bias)
    for it in range(ITERS[cfg]):
        C_prev = C.clone()
        Cq_used = Cq.clone()
        fk.fk_assign_with_bias(X, Cq, bias, labels)
        fk.fk_update_bias(X, labels, C, C, Cq if w.dtype != "f32" else None, counts, bias, ws=ws)
        torch.cuda.synchronize()
        rows = rng.choice(B * N, size=SAMPLE[cfg], replace=False)
        print(f"[fullsize] {w.name} iteration {it}: checking", flush=True)
        st = check_labels(labels, X_cpu, Cq_used, rows=rows)
        su = check_update(X_cpu, labels, C_prev, C, counts,
                          C_lowp=Cq if w.dtype != "f32" else None)
        assert int(counts.sum()) == B * N
        print(f"[fullsize] {w.name} iteration {it}: {st} {su}", flush=True)
        if w.dtype == "f32":
            Cq = C.clone()
        # the bias written by the update is that of the centroids now in Cq
        ref = torch.empty_like(bias)
        fk.fk_centroid_bias(Cq, ref)
        torch.cuda.synchronize()
        assert torch.equal(bias, ref)


def test_streamed_full_chunk_lockstep():
    """The pinned-host workload in the benchmark's streamed launch shape
    (chunks of 2^24 points, copy stream overlapped with compute), at N = 2^25:
    one iteration checked against the oracle (labels on a sample, counts and
    centroids of the update on every point)."""
    w = synth.CONFIGS[5]
    N, chunk = 1 << 25, 1 << 24
    print(f"[fullsize] {w.name} N={N}: generating", flush=True)
    X_host, C0 = synth.make_streamed(w, N=N)
    C = C0.cuda()
    C_prev = C.clone()
    labels = torch.empty((1, N), dtype=torch.int32, device="cuda")
    counts = torch.empty((1, w.K), dtype=torch.int32, device="cuda")
    copy = torch.cuda.Stream()
    fk.fk_lloyd_streamed(X_host, C, labels, counts, 1, chunk, copy_stream=copy)
    torch.cuda.synchronize()
    rows = np.random.Generator(np.random.PCG64(505)).choice(N, size=2048, replace=False)
    print(f"[fullsize] {w.name}: checking", flush=True)
    st = check_labels(labels, X_host, C_prev, rows=rows)
    su = check_update(X_host, labels, C_prev, C, counts)
    assert int(counts.sum()) == N
    print(f"[fullsize] {w.name}: {st} {su}", flush=True)
