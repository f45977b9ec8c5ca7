"""Lloyd iterations on the GPU against the oracle: lock-step per iteration
(assign and update checked on exactly what the GPU consumed), the fused
fk_lloyd loop, and the free-running fp32 trajectory of the small workload."""
import numpy as np
import pytest
import torch

import exact_lloyd_means_amd as fk
import oracle
import synth
from parity import CTOL, FMT, check_labels, check_update, to_storage

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"


LOCKSTEP = {1: (dict(), 10), 2: (dict(B=2, N=8192), 4), 3: (dict(N=32768), 3)}


@pytest.mark.parametrize("cfg", sorted(LOCKSTEP))
def test_lockstep(cfg):
    kw, T = LOCKSTEP[cfg]
    X, C0 = synth.make(cfg, **kw)
    X = X.cuda()
    B, N, d = X.shape
    K = C0.shape[1]
    C = C0.cuda()
    Cq = C.to(X.dtype)            # the init is a set of points: exact in the input dtype
    ws = fk.workspace(fk.problem(B, N, K, d, X.dtype))
    labels = torch.empty((B, N), dtype=torch.int32, device="cuda")
    counts = torch.empty((B, K), dtype=torch.int32, device="cuda")
    for t in range(T):
        fk.fk_assign(X, Cq, labels, ws=ws)
        torch.cuda.synchronize()
        check_labels(labels, X, Cq)
        C_next = torch.empty_like(C)
        lowp = torch.empty_like(Cq) if X.dtype != torch.float32 else None
        fk.fk_update(X, labels, C, C_next, lowp, counts, ws=ws)
        torch.cuda.synchronize()
        check_update(X, labels, C, C_next, counts, lowp)
        C = C_next
        Cq = lowp if lowp is not None else C_next


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_fused_loop_lockstep_oracle(dt):
    """The 16-bit fk_lloyd loop against the oracle, one iteration per call:
    each call rounds the fp32 centroids it is given to the input dtype
    (nearest, ties to even), assigns and updates.  The labels must be the
    oracle's assignment to the oracle's own RNE rounding of those centroids
    (so a copy rounded any other way shows up as label differences), and
    counts and centroids the oracle's update from those labels.  Then
    fk_lloyd(T) in one call -- where every assignment after the first reads
    the rounded copy and bias written by the previous update -- must reach
    the same state bit for bit (FK_DETERMINISTIC on both sides)."""
    X, C0 = synth.make(2, B=2, N=8192, dtype=dt)
    T = 4
    Xg = X.cuda()
    B, N, d = X.shape
    K = C0.shape[1]
    labels = torch.empty((B, N), dtype=torch.int32, device="cuda")
    counts = torch.empty((B, K), dtype=torch.int32, device="cuda")
    ws = fk.workspace(fk.problem(B, N, K, d, X.dtype, deterministic=True))
    C = C0.cuda().clone()
    for t in range(T):
        C_t = C.clone()
        fk.fk_lloyd(Xg, C, labels, counts, max_iters=1, ws=ws, deterministic=True)
        torch.cuda.synchronize()
        rne = oracle.encode_rne(C_t.cpu().numpy(), dt)
        Cq_t = torch.from_numpy(rne.view(np.int16)).view(X.dtype)
        st = check_labels(labels, X, Cq_t)
        su = check_update(X, labels, C_t, C, counts)
        print(f"[lloyd {dt}] iteration {t}: labels {st} update {su}", flush=True)
    C2 = C0.cuda().clone()
    lab2 = torch.empty_like(labels)
    cnt2 = torch.empty_like(counts)
    fk.fk_lloyd(Xg, C2, lab2, cnt2, max_iters=T, ws=ws, deterministic=True)
    torch.cuda.synchronize()
    assert torch.equal(lab2, labels)
    assert torch.equal(cnt2, counts)
    assert torch.equal(C2, C)


def test_free_run_small_fp32():
    """Well separated fp32 mixture, 10 iterations: the GPU trajectory follows
    the fp64 free-running oracle (labels identical, centroids within 1e-4)."""
    X, C0 = synth.make(1)
    T = synth.CONFIGS[1].iters
    Xg = X.cuda()
    B, N, d = X.shape
    K = C0.shape[1]
    C = C0.cuda().clone()
    labels = torch.empty((B, N), dtype=torch.int32, device="cuda")
    counts = torch.empty((B, K), dtype=torch.int32, device="cuda")
    n = fk.fk_lloyd(Xg, C, labels, counts, max_iters=T, want_n_iter=True)
    assert n == T
    oC, olab, ocnt, obj = oracle.lloyd(X.numpy(), C0.numpy().astype(np.float64), T)
    assert np.array_equal(labels.cpu().numpy(), olab)
    assert np.array_equal(counts.cpu().numpy(), ocnt)
    err = np.abs(C.cpu().numpy() - oC).max(-1)
    ref = np.abs(oC).max(-1)
    assert np.all(err <= CTOL["f32"] * ref)
    assert np.all(obj[1:] <= obj[:-1] * (1 + 1e-12))


def test_tol_stops_early():
    X, C0 = synth.make(1)
    Xg = X.cuda()
    C = C0.cuda().clone()
    labels = torch.empty((1, X.shape[1]), dtype=torch.int32, device="cuda")
    counts = torch.empty((1, C0.shape[1]), dtype=torch.int32, device="cuda")
    n = fk.fk_lloyd(Xg, C, labels, counts, max_iters=50, tol=1e-10, want_n_iter=True)
    assert 1 <= n < 50
