"""Helpers shared by the GPU parity tests (tolerance checks, input variants).

The tolerance is the stated bar for the GEMM outputs, applied per expert:
|gpu - ref| <= 2e-2 * max_e |ref| + 1e-3 over the expert's valid rows.
"""
import numpy as np
import torch

from oracle import qma_oracle as O
from quantized_moe_align_amd import inputs
from quantized_moe_align_amd.moe import to_device, to_host

RTOL, ATOL = 2e-2, 1e-3


def assert_per_expert(gpu_bits, ref, row_expert, what=""):
    """gpu_bits: bf16 bits [rows, n]; ref: float64 [rows, n] (NaN = undefined);
    row_expert: expert of each row (-1 = undefined row, skipped)."""
    g = O.bf16_to_f64(gpu_bits)
    row_expert = np.asarray(row_expert).reshape(-1)
    assert g.shape == ref.shape, (g.shape, ref.shape)
    worst = 0.0
    for e in np.unique(row_expert[row_expert >= 0]):
        rows = row_expert == e
        r = ref[rows]
        assert not np.isnan(r).any(), f"{what}: oracle undefined on expert {e}"
        gg = g[rows]
        assert np.isfinite(gg).all(), f"{what}: non-finite GPU output for expert {e}"
        bound = RTOL * np.abs(r).max() + ATOL
        err = np.abs(gg - r).max()
        worst = max(worst, err / bound)
        assert err <= bound, f"{what}: expert {e} max err {err:.3e} > bound {bound:.3e}"
    return worst


def bf16_pow2(rng, shape, lo=-3, hi=2):
    j = rng.integers(lo, hi + 1, shape)
    return ((127 + j) << 7).astype(np.uint16)


def bf16_small_ints(rng, shape, lo=-2, hi=2):
    v = rng.integers(lo, hi + 1, shape).astype(np.float32)
    return inputs.f32_to_bf16_bits(v)


def rne(ref):
    return O.f64_to_bf16(ref)


def slot_experts(topk_ids, E):
    ids = np.asarray(topk_ids).reshape(-1).astype(np.int64)
    return np.where((ids >= 0) & (ids < E), ids, -1)
