"""silu_and_mul and the top-k combine on the GPU against the oracle.

silu_and_mul computes in fp32 and rounds once to bf16. The bar is one bf16
ulp from the float64 result, because fp32 rounding error can move a value
that lies within a few fp32 ulps of a bf16 tie to the neighbouring bf16.
Outputs in the subnormal range may also be flushed to zero.
"""
import numpy as np
import pytest
import torch

from oracle import qma_oracle as O
from quantized_moe_align_amd import inputs, qma
from quantized_moe_align_amd.moe import empty_bf16, to_device, to_host

pytestmark = pytest.mark.gpu


def run_silu(x_bits):
    R, I2 = x_bits.shape
    x = to_device(x_bits)
    y = empty_bf16(R, I2 // 2)
    qma.qma_silu_and_mul(x, y, R, I2 // 2)
    torch.cuda.synchronize()
    return to_host(y, bf16=True)


def assert_within_one_ulp(got_bits, ref):
    ref_bits = O.f64_to_bf16(ref)
    g = O.bf16_to_f64(got_bits)
    nan = np.isnan(ref)
    assert np.all(np.isnan(g[nan]))
    ok = ~nan
    gb = got_bits[ok].astype(np.int64)
    rb = ref_bits[ok].astype(np.int64)
    # signed-magnitude bit patterns -> ordered integers
    to_ord = lambda b: np.where(b & 0x8000, -(b & 0x7FFF), b & 0x7FFF)
    diff = np.abs(to_ord(gb) - to_ord(rb))
    tiny = np.abs(ref[ok]) < 2.0 ** -126
    bad = (diff > 1) & ~(tiny & (g[ok] == 0))
    assert not bad.any(), (np.nonzero(bad)[0][:5], gb[bad][:5], rb[bad][:5])
    return int(diff.max()) if diff.size else 0


def test_exhaustive_gate_with_unit_up(gpu):
    gates = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ones = np.full_like(gates, 0x3F80)
    x = np.stack([gates, ones], axis=1)                       # I = 1 (scalar path)
    got = run_silu(x)[:, 0]
    ref = O.silu_and_mul(x)[:, 0]
    assert_within_one_ulp(got, ref)


def test_exhaustive_up_with_fixed_gates(gpu):
    ups = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    for gate in (0.5, -3.0, 10.0, -0.0078125):
        gb = inputs.f32_to_bf16_bits(np.array([gate], np.float32))[0]
        x = np.stack([np.full_like(ups, gb), ups], axis=1)
        got = run_silu(x)[:, 0]
        ref = O.silu_and_mul(x)[:, 0]
        assert_within_one_ulp(got, ref)


@pytest.mark.parametrize("R,I", [(576, 2048), (37, 128), (5, 24), (3, 7)])
def test_vector_and_scalar_paths(gpu, R, I):
    rng = np.random.default_rng(R + I)
    x = inputs.bf16_normal(rng, (R, 2 * I), std=3.0)
    got = run_silu(x)
    assert_within_one_ulp(got.reshape(-1), O.silu_and_mul(x).reshape(-1))


def test_combine(gpu):
    rng = np.random.default_rng(7)
    T, topk, N, E = 33, 4, 96, 6
    c2 = inputs.bf16_normal(rng, (T * topk, N))
    w = rng.random((T, topk)).astype(np.float32)
    ids = rng.integers(-1, E, (T, topk)).astype(np.int32)
    out = empty_bf16(T, N)
    qma.qma_moe_combine(to_device(c2), torch.from_numpy(w).cuda(), to_device(ids), E, T, topk,
                        N, out)
    torch.cuda.synchronize()
    got = O.bf16_to_f64(to_host(out, bf16=True))
    c2m = O.bf16_to_f64(c2).copy()
    c2m[ids.reshape(-1) < 0] = 0.0
    ref = O.moe_combine(c2m, w, topk)
    # fp32 fused multiply-adds over <= 4 terms, then one bf16 rounding
    assert np.all(np.abs(got - ref) <= 2.0 ** -7 * np.abs(ref) + 1e-6)
