"""Pins of the oracle's router (softmax + top-k), independent of its code:
the defining order property by brute force, argmax for k = 1, closed
forms and the softmax weight identities."""
import itertools

import numpy as np
import pytest

from oracle import qma_oracle as O


def test_order_property_brute_force():
    # every logit row over {-1, 0, 1} for E <= 4 (ties everywhere), every k
    for E in range(1, 5):
        for row in itertools.product((-1.0, 0.0, 1.0), repeat=E):
            lg = np.array([row], dtype=np.float32)
            for k in range(1, E + 1):
                ids, w = O.router_topk(lg, k)
                chosen = list(ids[0])
                assert len(set(chosen)) == k
                rest = [f for f in range(E) if f not in chosen]
                for e in chosen:                      # every chosen beats every other
                    for f in rest:
                        assert row[e] > row[f] or (row[e] == row[f] and e < f)
                for a, b in zip(chosen, chosen[1:]):  # listed best first
                    assert row[a] > row[b] or (row[a] == row[b] and a < b)


def test_top1_is_argmax():
    rng = np.random.default_rng(0)
    lg = rng.integers(-3, 4, (200, 9)).astype(np.float32)   # many ties
    ids, _ = O.router_topk(lg, 1)
    assert np.array_equal(ids[:, 0], np.argmax(lg, axis=1))


def test_equal_logits_closed_form():
    ids, w = O.router_topk(np.zeros((3, 8), np.float32), 3)
    assert np.array_equal(ids, np.tile([0, 1, 2], (3, 1)))
    assert np.allclose(w, 1.0 / 8, rtol=0, atol=1e-15)


def test_weights_are_full_softmax():
    rng = np.random.default_rng(1)
    lg = rng.standard_normal((50, 12)).astype(np.float32)
    ids, w = O.router_topk(lg, 12)                 # k = E: all experts
    assert np.allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    ids4, w4 = O.router_topk(lg, 4)
    l64 = lg.astype(np.float64)
    for t in range(50):                            # ratios are exp of logit gaps
        a, b = ids4[t, 0], ids4[t, 3]
        assert w4[t, 0] / w4[t, 3] == pytest.approx(np.exp(l64[t, a] - l64[t, b]), rel=1e-12)
    assert np.all(w4.sum(axis=1) < 1.0)            # not renormalised over k


def test_extreme_logits_do_not_overflow():
    lg = np.array([[1000.0, 0.0, -1000.0, 999.0]], np.float32)
    ids, w = O.router_topk(lg, 2)
    assert list(ids[0]) == [0, 3]
    assert w[0, 0] == pytest.approx(1 / (1 + np.exp(-1.0)), rel=1e-12)
    assert np.isfinite(w).all()
