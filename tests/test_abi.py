"""The C ABI without a GPU: the library loads, exports every function the
header declares, and rejects bad arguments with the documented status before
touching the device (fake device addresses are never dereferenced)."""
import ctypes
import glob
import os
import re

import pytest

import exact_lloyd_means_amd as fk

INCLUDE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
HEADER = os.path.join(INCLUDE, "fk.h")

FAKE = 0x10000          # 16-byte aligned, never dereferenced
FAKE_MISALIGNED = 0x10004


def declared_functions():
    names = set()
    for path in sorted(glob.glob(os.path.join(INCLUDE, "*.h"))):
        text = re.sub(r"/\*.*?\*/", "", open(path).read(), flags=re.S)
        names |= set(re.findall(r"\b(fk_[a-z_0-9]+)\s*\(", text))
    return sorted(names)


def test_header_symbols_exported():
    names = declared_functions()
    assert "fk_assign" in names and "fk_update" in names and "fk_lloyd" in names
    assert "fk_baseline_scores" in names and "fk_baseline_update_scatter" in names
    for name in names:
        assert hasattr(fk.lib, name), f"{name} declared in include/ but not exported"


def test_abi_version_matches_header():
    m = re.search(r"#define FK_ABI_VERSION (\d+)", open(HEADER).read())
    assert fk.abi_version() == int(m.group(1))


def test_status_strings():
    for code in (0, -1, -2, -3, -4, -5):
        assert fk.lib.fk_status_str(code)
    assert b"unknown" in fk.lib.fk_status_str(42)


def P(B=2, N=100, K=10, d=16, dtype=fk.FK_F16, flags=0):
    return fk.Problem(B, N, K, d, dtype, flags)


def ws_size(p):
    return fk.workspace_size(p)


def call_assign(p, X=FAKE, C=FAKE, labels=FAKE, md=None, ws=FAKE, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = ws_size(p) if p.B > 0 and p.N > 0 and p.K > 0 and p.d > 0 else 0
    return fk.lib.fk_assign(ctypes.byref(p) if p is not None else None, X, C, labels, md, ws,
                            ws_bytes, None)


@pytest.mark.parametrize("field", ["B", "N", "K", "d"])
def test_sizes_below_one_rejected(field):
    p = P()
    setattr(p, field, 0)
    assert call_assign(p) == fk.FK_EINVAL
    assert b"sizes" in fk.lib.fk_last_error()


def test_null_problem_rejected():
    assert fk.lib.fk_assign(None, FAKE, FAKE, FAKE, None, FAKE, 1 << 20, None) == fk.FK_EINVAL


def test_unknown_dtype_rejected():
    assert call_assign(P(dtype=7), ws_bytes=1 << 30) == fk.FK_EUNSUPPORTED


def test_deterministic_workspace_is_larger():
    p = P(flags=fk.FK_DETERMINISTIC)
    n = ctypes.c_size_t(0)
    for chunk in (0, 64):
        assert fk.lib.fk_workspace_size(ctypes.byref(p), chunk, ctypes.byref(n)) == fk.FK_OK
        assert n.value > fk.workspace_size(P(), chunk)


def test_unknown_flags_rejected():
    assert call_assign(P(flags=2), ws_bytes=1 << 30) == fk.FK_EINVAL
    assert b"flag" in fk.lib.fk_last_error()
    assert call_assign(P(flags=fk.FK_DETERMINISTIC), ws_bytes=0) == fk.FK_EWORKSPACE


@pytest.mark.parametrize("which", ["X", "C", "labels"])
def test_null_and_misaligned_pointers(which):
    p = P()
    assert call_assign(p, **{which: None}) == fk.FK_EINVAL
    assert call_assign(p, **{which: FAKE_MISALIGNED}) == fk.FK_EINVAL
    assert b"aligned" in fk.lib.fk_last_error()


def test_workspace_checks():
    p = P()
    assert call_assign(p, ws=None) == fk.FK_EWORKSPACE
    assert call_assign(p, ws_bytes=ws_size(p) - 1) == fk.FK_EWORKSPACE
    assert b"needs" in fk.lib.fk_last_error()


def test_too_large_sizes():
    assert call_assign(P(N=1 << 31), ws_bytes=0) == fk.FK_EUNSUPPORTED
    assert call_assign(P(d=65537), ws_bytes=0) == fk.FK_EUNSUPPORTED


def test_update_and_lloyd_validation():
    p = P()
    n = ws_size(p)
    lib = fk.lib
    # C_next missing
    assert lib.fk_update(ctypes.byref(p), FAKE, FAKE, FAKE, None, None, FAKE, FAKE, n,
                         None) == fk.FK_EINVAL
    # workspace too small
    assert lib.fk_update(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, n - 256,
                         None) == fk.FK_EWORKSPACE
    # max_iters < 1, negative tol
    assert lib.fk_lloyd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, 0, 0.0, None, FAKE, n,
                        None) == fk.FK_EINVAL
    assert lib.fk_lloyd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, 3, -1.0, None, FAKE, n,
                        None) == fk.FK_EINVAL
    # sort: offsets missing
    assert lib.fk_sort_labels(ctypes.byref(p), FAKE, FAKE, None, FAKE, FAKE, n,
                              None) == fk.FK_EINVAL
    # error count: host pointer missing
    assert lib.fk_error_count(ctypes.byref(p), FAKE, n, None, None) == fk.FK_EINVAL
    # update with bias: bias_next required
    assert lib.fk_update_bias(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, None, FAKE, None, FAKE, n,
                              None) == fk.FK_EINVAL


def test_baseline_validation():
    lib = fk.lib
    p = P()
    ok = dict(X=FAKE, C=FAKE, bias=FAKE, D=FAKE)
    # scores: 16-bit and d <= 256 only, every pointer required and aligned
    assert lib.fk_baseline_scores(ctypes.byref(P(dtype=fk.FK_F32)), *ok.values(),
                                  None) == fk.FK_EUNSUPPORTED
    assert lib.fk_baseline_scores(ctypes.byref(P(d=257)), *ok.values(), None) == fk.FK_EUNSUPPORTED
    for name in ok:
        args = dict(ok, **{name: None})
        assert lib.fk_baseline_scores(ctypes.byref(p), *args.values(), None) == fk.FK_EINVAL
        args = dict(ok, **{name: FAKE_MISALIGNED})
        assert lib.fk_baseline_scores(ctypes.byref(p), *args.values(), None) == fk.FK_EINVAL
    assert lib.fk_baseline_argmin(ctypes.byref(p), None, FAKE, None) == fk.FK_EINVAL
    assert lib.fk_baseline_argmin(ctypes.byref(P(K=0)), FAKE, FAKE, None) == fk.FK_EINVAL
    # scatter update: sums required; fp32 low copy must not alias C_next
    assert lib.fk_baseline_update_scatter(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, None, FAKE,
                                          None, None) == fk.FK_EINVAL
    q = P(dtype=fk.FK_F32)
    assert lib.fk_baseline_update_scatter(ctypes.byref(q), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                          FAKE, None) == fk.FK_EINVAL
    assert b"differ" in lib.fk_last_error()


def test_assign_variant_validation():
    lib = fk.lib

    def call(p, np_=4, waves=8, grid=0):
        return lib.fk_assign_variant(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, np_, waves, grid,
                                     None)
    assert call(P(d=128, K=64, dtype=fk.FK_F32)) == fk.FK_EUNSUPPORTED
    assert call(P(d=100, K=64)) == fk.FK_EUNSUPPORTED
    assert call(P(d=128, K=16)) == fk.FK_EUNSUPPORTED
    assert call(P(d=128, K=64), np_=3) == fk.FK_EINVAL
    assert call(P(d=128, K=64), waves=6) == fk.FK_EINVAL
    assert call(P(d=128, K=64), grid=-1) == fk.FK_EINVAL


def test_workspace_has_no_NK_term():
    """Workspace grows with B*N, B*K*d and B*K only (no distance matrix)."""
    def size(B, N, K, d):
        return fk.workspace_size(fk.problem(B, N, K, d, fk.FK_F16))
    base = size(1, 1 << 16, 1 << 12, 128)
    # doubling N adds at most three int32 per point (sorted index, sort table
    # bounded by 4N, run labels), not K values per point
    assert size(1, 1 << 17, 1 << 12, 128) - base <= 12 * (1 << 16) + 4096
    # large N and K together stay far below N*K
    big = size(1, 1 << 20, 1 << 16, 128)
    assert big < (1 << 20) * (1 << 16) // 64
    # config sizes
    assert size(32, 65536, 1024, 128) < 64 << 20


def test_last_error_is_per_call():
    p = P()
    call_assign(p, ws=None)
    first = fk.lib.fk_last_error()
    assert first
    ok = fk.lib.fk_workspace_size(ctypes.byref(p), 0, ctypes.byref(ctypes.c_size_t()))
    assert ok == fk.FK_OK


def test_workspace_bytes_matches_size():
    for p in (P(), P(flags=fk.FK_DETERMINISTIC), P(B=3, N=5000, K=700, d=129, dtype=fk.FK_F32)):
        assert fk.lib.fk_workspace_bytes(ctypes.byref(p), 0) == ws_size(p)
        assert fk.lib.fk_workspace_bytes(ctypes.byref(p), 64) == fk.workspace_size(p, 64)


def test_workspace_bytes_zero_on_error():
    p = P(K=0)
    assert fk.lib.fk_workspace_bytes(ctypes.byref(p), 0) == 0
    assert b"sizes" in fk.lib.fk_last_error()
    assert fk.lib.fk_workspace_bytes(ctypes.byref(P()), -1) == 0


def noalloc_limit():
    m = re.search(r"#define FK_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", open(HEADER).read())
    return int(m.group(1)) << int(m.group(2))


def call_noalloc(p, X=FAKE, labels=FAKE, C_prev=FAKE, C_next=FAKE, lowp=None, counts=FAKE,
                 bias=FAKE):
    return fk.lib.fk_update_bias_noalloc(ctypes.byref(p), X, labels, C_prev, C_next, lowp,
                                         counts, bias, None)


def test_noalloc_scratch_holds_the_mixture_workloads():
    limit = noalloc_limit()
    assert limit == 64 << 20
    for det in (0, fk.FK_DETERMINISTIC):
        assert ws_size(P(32, 65536, 1024, 128, fk.FK_F16, det)) <= limit
        assert ws_size(P(1, 1 << 20, 4096, 128, fk.FK_F16, det)) <= limit


def test_noalloc_rejects_problems_beyond_the_scratch():
    # checked before the scratch is looked up, so no GPU is needed
    p = P(1, 1 << 24, 4096, 128)
    assert ws_size(p) > noalloc_limit()
    assert call_noalloc(p) == fk.FK_EUNSUPPORTED
    assert b"static scratch" in fk.lib.fk_last_error()


@pytest.mark.parametrize("which", ["X", "labels", "C_prev", "C_next", "counts", "bias"])
def test_noalloc_null_and_misaligned_pointers(which):
    assert call_noalloc(P(), **{which: None}) == fk.FK_EINVAL
    assert call_noalloc(P(), **{which: FAKE_MISALIGNED}) == fk.FK_EINVAL


def test_noalloc_validation():
    assert call_noalloc(P(d=2048)) == fk.FK_EUNSUPPORTED
    assert call_noalloc(P(dtype=fk.FK_F32), C_next=FAKE, lowp=FAKE) == fk.FK_EINVAL
    assert call_noalloc(P(flags=4)) == fk.FK_EINVAL
