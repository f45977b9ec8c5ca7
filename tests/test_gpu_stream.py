"""Streamed Lloyd (fk_lloyd_streamed): pinned host X copied to the GPU in
chunks on a copy stream, overlapped with assign/update on the compute stream.
Checked in lock-step against the oracle and against the resident path."""
import numpy as np
import pytest
import torch

import exact_lloyd_means_amd as fk
import synth
from parity import check_labels, check_update

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"


def pinned(X):
    return X.contiguous().pin_memory()


def run_streamed(Xh, C, iters, chunk):
    B, N, _ = Xh.shape
    K = C.shape[1]
    labels = torch.empty((B, N), dtype=torch.int32, device="cuda")
    counts = torch.empty((B, K), dtype=torch.int32, device="cuda")
    copy = torch.cuda.Stream()
    fk.fk_lloyd_streamed(Xh, C, labels, counts, iters, chunk, copy_stream=copy)
    torch.cuda.synchronize()
    return labels, counts


@pytest.mark.parametrize("cfg,kw,chunk,iters", [
    (5, dict(N=1 << 18), 1 << 16, 3),          # the out-of-core workload, shrunk
    (1, dict(), 1000, 4),                      # ragged chunks
    (2, dict(B=2, N=6000, K=300), 2048, 2),    # fp16, several problems
])
def test_streamed_lockstep(cfg, kw, chunk, iters):
    X, C0 = synth.make(cfg, **kw)
    Xh = pinned(X)
    Xg = X.cuda()
    C = C0.cuda()
    for _ in range(iters):
        C_prev = C.clone()
        Cq = C_prev.to(X.dtype)
        labels, counts = run_streamed(Xh, C, 1, chunk)
        check_labels(labels, Xg, Cq)
        # C was updated in place from C_prev with these labels
        check_update(Xg, labels, C_prev, C, counts)


def test_streamed_deterministic():
    """FK_DETERMINISTIC on the streamed path: bit-identical reruns, and one
    iteration still matches the oracle (Zipf sizes: long segments)."""
    X, C0 = synth.make(3, N=40000, K=128)
    Xh = pinned(X)
    outs = []
    for _ in range(2):
        C = C0.cuda().clone()
        labels = torch.empty((1, 40000), dtype=torch.int32, device="cuda")
        counts = torch.empty((1, 128), dtype=torch.int32, device="cuda")
        fk.fk_lloyd_streamed(Xh, C, labels, counts, 1, 9000, copy_stream=torch.cuda.Stream(),
                             deterministic=True)
        torch.cuda.synchronize()
        outs.append((C, labels, counts))
    assert int(outs[0][2].max()) > 256
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    Xg = X.cuda()
    check_labels(outs[0][1], Xg, C0.cuda().to(X.dtype))
    check_update(Xg, outs[0][1], C0.cuda(), outs[0][0], outs[0][2])


def test_streamed_matches_resident():
    X, C0 = synth.make(1)
    Xh = pinned(X)
    C1 = C0.cuda().clone()
    l1, c1 = run_streamed(Xh, C1, 5, 777)
    C2 = C0.cuda().clone()
    l2 = torch.empty_like(l1)
    c2 = torch.empty_like(c1)
    fk.fk_lloyd(X.cuda(), C2, l2, c2, max_iters=5)
    torch.cuda.synchronize()
    assert torch.equal(l1, l2) and torch.equal(c1, c2)
    assert (C1 - C2).abs().max().item() <= 1e-4 * C2.abs().max().item()


def test_streamed_single_stream_and_bf16():
    X, C0 = synth.make(2, B=1, N=5000, K=100, dtype="bf16")
    Xh = pinned(X)
    C = C0.cuda()
    B, N, _ = X.shape
    labels = torch.empty((B, N), dtype=torch.int32, device="cuda")
    counts = torch.empty((B, 100), dtype=torch.int32, device="cuda")
    C_prev = C.clone()
    fk.fk_lloyd_streamed(Xh, C, labels, counts, 1, 1024)   # copy and compute on one stream
    torch.cuda.synchronize()
    check_labels(labels, X.cuda(), C_prev.to(X.dtype))
    check_update(X.cuda(), labels, C_prev, C, counts)


def test_streamed_rejects_pageable_host_memory():
    X, C0 = synth.make(1)
    C = C0.cuda()
    labels = torch.empty((1, X.shape[1]), dtype=torch.int32, device="cuda")
    counts = torch.empty((1, C0.shape[1]), dtype=torch.int32, device="cuda")
    p = fk.problem(1, X.shape[1], C0.shape[1], X.shape[2], X.dtype)
    ws = fk.workspace(p, "cuda", 1024)
    import ctypes
    st = fk.lib.fk_lloyd_streamed(ctypes.byref(p), ctypes.c_void_p(X.data_ptr()), 1024,
                                  ctypes.c_void_p(C.data_ptr()), ctypes.c_void_p(labels.data_ptr()),
                                  ctypes.c_void_p(counts.data_ptr()), 1,
                                  ctypes.c_void_p(ws.data_ptr()), ws.numel(), None, None)
    assert st == fk.FK_EINVAL
    assert b"pinned" in fk.lib.fk_last_error()
