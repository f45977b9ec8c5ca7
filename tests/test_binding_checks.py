"""The Python binding rejects tensors of the wrong dtype, shape or device
before anything reaches libfk (CPU only: every call here raises in the
binding, so no kernel is launched and no device memory is touched)."""
import pytest
import torch

import exact_lloyd_means_amd as fk

B, N, K, d = 2, 64, 8, 16


def good(dtype=torch.float16):
    return dict(
        X=torch.zeros(B, N, d, dtype=dtype),
        Cq=torch.zeros(B, K, d, dtype=dtype),
        C=torch.zeros(B, K, d, dtype=torch.float32),
        labels=torch.zeros(B, N, dtype=torch.int32),
        counts=torch.zeros(B, K, dtype=torch.int32),
        bias=torch.zeros(B, K, dtype=torch.float32),
        md=torch.zeros(B, N, dtype=torch.float32),
    )


def test_correct_cpu_tensors_are_rejected_only_for_their_device():
    t = good()
    with pytest.raises(ValueError, match="on the GPU"):
        fk.fk_assign_with_bias(t["X"], t["Cq"], t["bias"], t["labels"])
    with pytest.raises(ValueError, match="on the GPU"):
        fk.fk_update(t["X"], t["labels"], t["C"], t["C"], t["Cq"], t["counts"])
    with pytest.raises(ValueError, match="on the GPU"):
        fk.fk_lloyd(t["X"], t["C"], t["labels"], t["counts"], 1)


@pytest.mark.parametrize("which,bad,match", [
    ("labels", torch.zeros(B, N, dtype=torch.int64), "labels must be torch.int32"),
    ("labels", torch.zeros(B, N + 1, dtype=torch.int32), r"labels must have shape \(2, 64\)"),
    ("Cq", torch.zeros(B, K, d, dtype=torch.bfloat16), "C must be torch.float16"),
    ("Cq", torch.zeros(B, K, d + 1, dtype=torch.float16), "C must have shape"),
    ("bias", torch.zeros(B, K, dtype=torch.float16), "bias must be torch.float32"),
    ("bias", torch.zeros(B, K + 1, dtype=torch.float32), "bias must have shape"),
    ("md", torch.zeros(B, N, dtype=torch.float64), "min_dist must be torch.float32"),
])
def test_assign_rejects(which, bad, match):
    t = good()
    t[which] = bad
    with pytest.raises(ValueError, match=match):
        fk.fk_assign_with_bias(t["X"], t["Cq"], t["bias"], t["labels"], t["md"])


def test_assign_rejects_integer_points():
    t = good()
    with pytest.raises(ValueError, match="X must be float32, float16 or bfloat16"):
        fk.fk_assign_with_bias(t["X"].to(torch.int16), t["Cq"], t["bias"], t["labels"])


@pytest.mark.parametrize("which,bad,match", [
    ("C_prev", torch.zeros(B, K, d, dtype=torch.float16), "C_prev must be torch.float32"),
    ("C_next", torch.zeros(B, K, d, dtype=torch.float16), "C_next must be torch.float32"),
    ("C_next", torch.zeros(B, K - 1, d, dtype=torch.float32), "C_next must have shape"),
    ("lowp", torch.zeros(B, K, d, dtype=torch.float32), "C_next_lowp must be torch.float16"),
    ("counts", torch.zeros(B, K, dtype=torch.int64), "counts must be torch.int32"),
    ("counts", torch.zeros(B, 2 * K, dtype=torch.int32), "counts must have shape"),
    ("labels", torch.zeros(B * N, dtype=torch.int32), "labels must have shape"),
    ("bias_next", torch.zeros(B, K, dtype=torch.float64), "bias_next must be torch.float32"),
])
def test_update_rejects(which, bad, match):
    t = good()
    args = dict(C_prev=t["C"], C_next=t["C"].clone(), lowp=t["Cq"], counts=t["counts"],
                labels=t["labels"], bias_next=t["bias"])
    args[which] = bad
    with pytest.raises(ValueError, match=match):
        fk.fk_update_bias(t["X"], args["labels"], args["C_prev"], args["C_next"], args["lowp"],
                          args["counts"], args["bias_next"])


def test_update_rejects_non_contiguous():
    t = good()
    C_next = torch.zeros(B, d, K, dtype=torch.float32).transpose(1, 2)
    with pytest.raises(ValueError, match="contiguous"):
        fk.fk_update(t["X"], t["labels"], t["C"], C_next, t["Cq"], t["counts"])


def test_lloyd_rejects_16bit_centroids():
    t = good()
    with pytest.raises(ValueError, match="C must be torch.float32"):
        fk.fk_lloyd(t["X"], t["Cq"], t["labels"], t["counts"], 1)


def test_workspace_must_be_bytes():
    t = good()
    with pytest.raises(ValueError, match="ws must be a 1-D uint8 tensor"):
        fk._want_ws(torch.zeros(16, dtype=torch.int32), t["X"].device)


@pytest.mark.parametrize("which,bad,match", [
    ("counts", torch.zeros(B, K + 1, dtype=torch.int32), "counts must have shape"),
    ("offsets", torch.zeros(B, K, dtype=torch.int32), "offsets must have shape"),
    ("sorted_idx", torch.zeros(B, N, dtype=torch.int64), "sorted_idx must be torch.int32"),
])
def test_sort_rejects(which, bad, match):
    t = good()
    args = dict(counts=t["counts"], offsets=torch.zeros(B, K + 1, dtype=torch.int32),
                sorted_idx=torch.zeros(B, N, dtype=torch.int32))
    args[which] = bad
    with pytest.raises(ValueError, match=match):
        fk.fk_sort_labels(t["labels"], K, args["counts"], args["offsets"], args["sorted_idx"])


def test_centroid_bias_rejects_wrong_bias():
    t = good()
    with pytest.raises(ValueError, match="bias must have shape"):
        fk.fk_centroid_bias(t["Cq"], torch.zeros(B, K, 1, dtype=torch.float32))


def test_baselines_reject():
    t = good()
    with pytest.raises(ValueError, match="D must have shape"):
        fk.fk_baseline_scores(t["X"], t["Cq"], t["bias"], torch.zeros(B, N, K + 1))
    with pytest.raises(ValueError, match="labels must be torch.int32"):
        fk.fk_baseline_argmin(torch.zeros(B, N, K), torch.zeros(B, N, dtype=torch.int64))


def test_noalloc_rejects_before_the_library():
    t = good()
    with pytest.raises(ValueError, match="bias_next must have shape"):
        fk.fk_update_bias_noalloc(t["X"], t["labels"], t["C"], t["C"].clone(), t["Cq"],
                                  t["counts"], torch.zeros(B, K + 1, dtype=torch.float32))
    with pytest.raises(ValueError, match="on the GPU"):
        fk.fk_update_bias_noalloc(t["X"], t["labels"], t["C"], t["C"].clone(), t["Cq"],
                                  t["counts"], t["bias"])
