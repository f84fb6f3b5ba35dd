"""GPU router (softmax + top-k) against the oracle through the C ABI."""
import numpy as np
import pytest
import torch

from oracle import qma_oracle as O
from quantized_moe_align_amd import qma

pytestmark = pytest.mark.gpu


def run(lg, topk, weights=True):
    T, E = lg.shape
    d = torch.from_numpy(np.ascontiguousarray(lg, np.float32)).cuda()
    ids = torch.full((max(T, 1), topk), -7, dtype=torch.int32, device="cuda")
    w = torch.full((max(T, 1), topk), -1.0, dtype=torch.float32, device="cuda") if weights else None
    qma.qma_router_topk(d, T, E, topk, ids, w)
    torch.cuda.synchronize()
    return ids.cpu().numpy()[:T], (w.cpu().numpy()[:T] if weights else None)


@pytest.mark.parametrize("T,E,topk", [(1, 8, 2), (64, 8, 2), (257, 48, 1), (256, 384, 8),
                                      (130, 1000, 16), (33, 1024, 16), (5, 16, 16)])
def test_router_matches_oracle(gpu, T, E, topk):
    rng = np.random.default_rng(T * 7 + E)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    ids, w = run(lg, topk)
    rid, rw = O.router_topk(lg, topk)
    assert np.array_equal(ids, rid)
    np.testing.assert_allclose(w, rw, rtol=2e-6, atol=1e-9)


def test_router_ties_and_extremes(gpu):
    rng = np.random.default_rng(3)
    lg = rng.integers(-2, 3, (300, 40)).astype(np.float32)   # many equal logits
    lg[0] = 0.0                                              # all equal
    lg[1, :] = -1000.0
    lg[1, 17] = 1000.0
    ids, w = run(lg, 6)
    rid, rw = O.router_topk(lg, 6)
    assert np.array_equal(ids, rid)
    np.testing.assert_allclose(w, rw, rtol=2e-6, atol=1e-12)
    assert list(ids[0]) == [0, 1, 2, 3, 4, 5]


def test_router_without_weights_and_empty(gpu):
    lg = np.random.default_rng(4).standard_normal((10, 48)).astype(np.float32)
    ids, _ = run(lg, 8, weights=False)
    assert np.array_equal(ids, O.router_topk(lg, 8)[0])
    ids0, _ = run(np.zeros((0, 48), np.float32), 8)
    assert ids0.shape == (0, 8)


def test_router_rejects_bad_sizes(gpu):
    d = torch.zeros((4, 8), dtype=torch.float32, device="cuda")
    ids = torch.zeros((4, 8), dtype=torch.int32, device="cuda")
    for E, k in ((8, 9), (8, 0), (2000, 4), (32, 17)):
        with pytest.raises(qma.QmaError):
            qma.qma_router_topk(d, 4, E, k, ids)
