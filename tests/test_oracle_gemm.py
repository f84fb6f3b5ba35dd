"""Pins for the oracle's expert GEMMs, activation and combine.

Checked against exact integer arithmetic (pure Python loops), identity
weights, a dense-matmul special case (torch float64), an independent
float64 triple loop, and SciPy's logistic function.
"""
import struct

import numpy as np
import pytest
import scipy.special
import torch

from oracle import qma_oracle as O
from quantized_moe_align_amd import inputs


def _bf16_bits(values):
    return torch.tensor(np.asarray(values, dtype=np.float64)).to(
        torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)


def _int_problem(rng, E, T, topk, K, N):
    """Activations in {-2..2}, scales 2^j, random q: exact in every format."""
    a_int = rng.integers(-2, 3, (T, K))
    q = rng.integers(0, 16, (E, N, K))
    j = rng.integers(-3, 3, (E, N, K // 32))
    ids = rng.integers(-1, E, (T, topk))
    return a_int, q, j, ids


def test_indexed_integer_exact_vs_python_ints():
    rng = np.random.default_rng(5)
    E, T, topk, K, N = 3, 5, 2, 64, 6
    a_int, q, j, ids = _int_problem(rng, E, T, topk, K, N)
    out = O.moe_gemm_by_slot(_bf16_bits(a_int), topk, ids, O.pack_uint4(q),
                             _bf16_bits(2.0 ** j))
    from fractions import Fraction
    for s in range(T * topk):
        e = int(ids.flat[s])
        for n in range(N):
            if e < 0:
                assert np.isnan(out[s, n])
                continue
            acc = Fraction(0)
            for k in range(K):
                acc += int(a_int[s // topk, k]) * (int(q[e, n, k]) - 8) * \
                    Fraction(2) ** int(j[e, n, k // 32])
            assert out[s, n] == float(acc), (s, n)


def test_identity_weights_reduce_to_gather():
    rng = np.random.default_rng(6)
    E, T, topk, K, N = 4, 7, 3, 64, 32
    q = np.full((E, N, K), 8)
    for n in range(N):
        q[:, n, n] = 9                                   # W = [I | 0]
    a = inputs.bf16_normal(rng, (T, K))
    ids = rng.integers(0, E, (T, topk))
    out = O.moe_gemm_by_slot(a, topk, ids, O.pack_uint4(q),
                             np.full((E, N, K // 32), 0x3F80, np.uint16))
    A = O.bf16_to_f64(a)
    for s in range(T * topk):
        assert np.array_equal(out[s], A[s // topk, :N])


def test_single_expert_is_dense_matmul():
    rng = np.random.default_rng(7)
    T, K, N = 9, 96, 40
    w_int = rng.integers(-8, 8, (N, K))
    sc = 2.0 ** rng.integers(-6, -2, (N, K // 32)) * rng.choice([1.0, 1.5, 1.25], (N, K // 32))
    a = inputs.bf16_normal(rng, (T, K))
    out = O.moe_gemm_by_slot(a, 1, np.zeros(T, dtype=np.int32),
                             O.pack_uint4(w_int[None] + 8), _bf16_bits(sc)[None])
    W = torch.tensor(w_int, dtype=torch.float64) * torch.tensor(
        np.repeat(sc, 32, axis=1))
    ref = torch.tensor(O.bf16_to_f64(a)) @ W.T
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-12, atol=1e-12)


def _f(bits):
    return struct.unpack(">f", int(bits).to_bytes(2, "big") + b"\0\0")[0]


def test_random_vs_float64_triple_loop():
    rng = np.random.default_rng(8)
    E, T, topk, K, N = 2, 3, 2, 32, 8
    a = inputs.bf16_normal(rng, (T, K))
    w = inputs.random_words(rng, (E, N, K // 8))
    s = inputs.bf16_normal(rng, (E, N, K // 32), 0.02, absolute=True)
    ids = np.array([[0, 1], [1, 1], [1, 0]])
    out = O.moe_gemm_by_slot(a, topk, ids, w, s)
    wu = w.view(np.uint32)
    for slot in range(T * topk):
        e = ids.flat[slot]
        for n in range(N):
            acc = 0.0
            for k in range(K):
                qv = (int(wu[e, n, k // 8]) >> (4 * (k % 8))) & 15
                acc += _f(a[slot // topk, k]) * (qv - 8) * _f(s[e, n, k // 32])
            assert abs(out[slot, n] - acc) <= 1e-12 * (1 + abs(acc))


def test_topk_weights_and_cols_subset():
    rng = np.random.default_rng(9)
    wl = inputs.make("tiny", seed=3)
    ids = wl["topk_ids"]
    full = O.moe_gemm_by_slot(wl["a"], wl.topk, ids, wl["w13"], wl["s13"])
    cols = np.array([0, 5, 17, 255])
    sub = O.moe_gemm_by_slot(wl["a"], wl.topk, ids, wl["w13"], wl["s13"], cols=cols)
    assert np.array_equal(full[:, cols], sub)
    tw = rng.random(ids.size).astype(np.float32)
    scaled = O.moe_gemm_by_slot(wl["a"], wl.topk, ids, wl["w13"], wl["s13"],
                                topk_weights=tw)
    np.testing.assert_allclose(scaled, full * tw[:, None].astype(np.float64),
                               rtol=1e-15)


def test_buffers_form_equals_slot_form_with_overallocation():
    wl = inputs.make("tiny", seed=4)
    for B in (16, 32):
        cap, _ = O.align_sizes(wl.T, wl.topk, wl.E, B)
        s, e, ntp = O.moe_align(wl["topk_ids"], wl.E, B, cap + 37)
        a = O.indexed_gemm_from_buffers(wl["a"], wl.topk, wl["w13"], wl["s13"],
                                        s, e, ntp, B, wl.T * wl.topk)
        b = O.moe_gemm_by_slot(wl["a"], wl.topk, wl["topk_ids"], wl["w13"], wl["s13"])
        assert np.array_equal(a, b, equal_nan=True)


def test_grouped_contiguous_and_masked_vs_python_ints():
    rng = np.random.default_rng(10)
    E, K, N = 3, 64, 5
    q = rng.integers(0, 16, (E, N, K))
    j = rng.integers(-2, 2, (E, N, K // 32))
    w, s = O.pack_uint4(q), _bf16_bits(2.0 ** j)
    m_idx = np.array([2, 2, -1, 0, 0, 0, -1, 1])
    a_int = rng.integers(-2, 3, (m_idx.size, K))
    out = O.grouped_contiguous(_bf16_bits(a_int), m_idx, w, s)
    for r, e in enumerate(m_idx):
        for n in range(N):
            if e < 0:
                assert np.isnan(out[r, n])
            else:
                ref = sum(int(a_int[r, k]) * (int(q[e, n, k]) - 8) * 2.0 ** int(j[e, n, k // 32])
                          for k in range(K))
                assert out[r, n] == ref
    budget = 4
    masked_m = np.array([1, 4, 0])
    a3 = rng.integers(-2, 3, (E, budget, K))
    out3 = O.grouped_masked(_bf16_bits(a3), masked_m, w, s)
    for e in range(E):
        for r in range(budget):
            for n in range(N):
                if r >= masked_m[e]:
                    assert np.isnan(out3[e, r, n])
                else:
                    ref = sum(int(a3[e, r, k]) * (int(q[e, n, k]) - 8) * 2.0 ** int(j[e, n, k // 32])
                              for k in range(K))
                    assert out3[e, r, n] == ref


def test_permutation_equivariance():
    wl = inputs.make("tiny", seed=11)
    perm = np.random.default_rng(0).permutation(wl.T)
    base = O.moe_gemm_by_slot(wl["a"], wl.topk, wl["topk_ids"], wl["w13"], wl["s13"])
    p = O.moe_gemm_by_slot(wl["a"][perm], wl.topk, wl["topk_ids"][perm],
                           wl["w13"], wl["s13"])
    slot_perm = (perm[:, None] * wl.topk + np.arange(wl.topk)).reshape(-1)
    assert np.array_equal(p, base[slot_perm])


def test_silu_and_mul_vs_scipy_expit_and_identities():
    rng = np.random.default_rng(12)
    g = rng.standard_normal(1000) * 6
    u = rng.standard_normal(1000)
    x = np.concatenate([_bf16_bits(g), _bf16_bits(u)])[None]
    out = O.silu_and_mul(x)[0]
    gb, ub = O.bf16_to_f64(_bf16_bits(g)), O.bf16_to_f64(_bf16_bits(u))
    np.testing.assert_allclose(out, gb * scipy.special.expit(gb) * ub,
                               rtol=1e-14, atol=1e-300)
    # silu(g) - silu(-g) = g, with up = 1
    ones = _bf16_bits(np.ones(1000))
    pos = O.silu_and_mul(np.concatenate([_bf16_bits(g), ones])[None])[0]
    neg = O.silu_and_mul(np.concatenate([_bf16_bits(-g), ones])[None])[0]
    np.testing.assert_allclose(pos - neg, gb, rtol=1e-13, atol=1e-13)
    # gate half first: gate 1, up 2 -> 2*sigmoid(1); swapped halves give silu(2)
    two = O.silu_and_mul(_bf16_bits([[1.0, 2.0]]))
    assert abs(two[0, 0] - 2 * scipy.special.expit(1.0)) < 1e-15


def test_combine_weighted_sum():
    rng = np.random.default_rng(13)
    T, topk, N = 4, 3, 5
    c2 = rng.standard_normal((T * topk, N))
    w = rng.random((T, topk))
    out = O.moe_combine(c2, w, topk)
    for t in range(T):
        ref = sum(w[t, k] * c2[t * topk + k] for k in range(topk))
        np.testing.assert_allclose(out[t], ref, rtol=1e-14)
