"""Every shape of the fp16 assign kernel (include/fk_tune.h) gives the
library's labels bit for bit, and those labels pass the oracle."""
import pytest
import torch

import exact_lloyd_means_amd as fk
from parity import check_labels

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"


@pytest.mark.parametrize("d", [64, 128, 256])
def test_all_shapes_agree(d):
    B, N, K = 2, 5000, 300
    g = torch.Generator().manual_seed(d)
    X = torch.randn((B, N, d), generator=g).half().cuda()
    C = torch.randn((B, K, d), generator=g).half().cuda()
    bias = torch.empty((B, K), dtype=torch.float32, device="cuda")
    fk.fk_centroid_bias(C, bias)
    ref = torch.empty((B, N), dtype=torch.int32, device="cuda")
    fk.fk_assign_with_bias(X, C, bias, ref)
    lab = torch.empty_like(ref)
    for np_ in (1, 2, 4, 8):
        for waves in (2, 4, 8):
            for grid in (0, 7):
                lab.fill_(-1)
                fk.fk_assign_variant(X, C, bias, lab, np_, waves, grid)
                torch.cuda.synchronize()
                assert torch.equal(lab, ref), (np_, waves, grid)
    check_labels(ref, X, C)
