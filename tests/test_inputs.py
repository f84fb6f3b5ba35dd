"""The seeded generator: determinism, independence of tensors, shapes and the
workload structure (counts, masks, padding)."""
import numpy as np
import pytest

from quantized_moe_align_amd import inputs


def test_deterministic_and_independent_streams():
    a = inputs.make("tiny", seed=1)
    b = inputs.make("tiny", seed=1)
    c = inputs.make("tiny", seed=2)
    for k in a.arrays:
        assert np.array_equal(a[k], b[k])
    assert not np.array_equal(a["a"], c["a"])
    # the weights do not depend on whether the router or activations changed
    d = inputs.make_router_workload("x", 1, 8, 64, 2, 256, 128)
    e = inputs.make_router_workload("x", 1, 8, 32, 2, 256, 128)
    assert np.array_equal(d["w13"], e["w13"]) and np.array_equal(d["s2"], e["s2"])


def test_tiny_shapes():
    w = inputs.make("tiny", seed=0)
    assert w["a"].shape == (64, 256) and w["a"].dtype == np.uint16
    assert w["topk_ids"].shape == (64, 2)
    assert w["w13"].shape == (8, 256, 32) and w["w13"].dtype == np.int32
    assert w["s13"].shape == (8, 256, 8)
    assert w["w2"].shape == (8, 256, 16) and w["s2"].shape == (8, 256, 4)
    # top-2 picks two distinct experts per token
    assert np.all(w["topk_ids"][:, 0] != w["topk_ids"][:, 1])


def test_decode_counts_and_prefill_zipf():
    w = inputs.make("ep8_decode", seed=0, weights=False)
    counts = np.bincount(w["topk_ids"][:, 0], minlength=48)
    assert counts.min() >= 9 and counts.max() <= 15 and w.T == counts.sum()
    p = inputs.make("ep8_prefill", seed=0, weights=False)
    c = np.bincount(p["topk_ids"][:, 0], minlength=48)
    assert c.sum() == 8192 and c.max() > 1000 and (c >= 80).sum() > 10
    s = inputs.span_counts(0, 48, 8192)
    assert s.sum() == 8192 and 15 <= s.min() and s.max() <= 650


def test_grouped_layouts():
    c = inputs.make_contiguous("c", 0, 3, 0, 64, 32, counts=[5, 0, 130])
    m = c["m_indices"]
    assert m.size == 128 + 256
    assert np.all(m[:5] == 0) and np.all(m[5:128] == -1)
    assert np.all(m[128:258] == 2) and np.all(m[258:] == -1)
    mk = inputs.make("masked", seed=0, weights=False)
    assert mk["a"].shape == (48, 64, 7168) and np.all(mk["masked_m"] == 32)


def test_scales_are_positive_bf16():
    w = inputs.make("tiny", seed=0)
    s = w["s13"]
    assert np.all((s & 0x8000) == 0)                  # |N(0, 0.02)|


def test_mid_and_ep128_shares():
    m = inputs.make("ep8_mid", seed=0, weights=False)
    c = np.bincount(m["topk_ids"][:, 0], minlength=48)
    assert m.E == 48 and c.min() >= 40 and c.max() <= 56 and m.T == c.sum()
    assert (33 <= c).all() and (c < 80).all()          # between decode and large-M
    e = inputs.make("ep128_decode", seed=0, weights=False)
    c3 = np.bincount(e["topk_ids"][:, 0], minlength=3)
    assert e.E == 3 and c3.min() >= 9 and c3.max() <= 15
