"""Pins for the oracle's bf16 conversions and the packed uint4 format.

These are CPU-only (-m "not gpu"). They check the oracle against library
conversions, closed forms and exhaustive enumeration, not against itself.
"""
import struct

import numpy as np
import pytest
import torch

from oracle import qma_oracle as O


def _bf16_bits_by_struct(bits):
    # Independent decode: a bf16 is the high half of a big-endian float32.
    return struct.unpack(">f", int(bits).to_bytes(2, "big") + b"\0\0")[0]


def test_bf16_decode_all_patterns_vs_struct():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = O.bf16_to_f64(bits)
    for b in list(range(0, 1 << 16, 97)) + [0x7F80, 0xFF80, 0x0001, 0x8001]:
        ref = _bf16_bits_by_struct(b)
        assert (np.isnan(ref) and np.isnan(got[b])) or got[b] == ref, hex(b)


def test_bf16_roundtrip_every_pattern():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    back = O.f64_to_bf16(O.bf16_to_f64(bits))
    nan = np.isnan(O.bf16_to_f64(bits))
    assert np.array_equal(back[~nan], bits[~nan])
    assert np.all(back[nan] == 0x7FC0)


def test_bf16_rounding_vs_torch_library():
    rng = np.random.default_rng(1)
    x32 = np.concatenate([
        (rng.standard_normal(200000) * 10.0 ** rng.integers(
            -40, 39, 200000)).astype(np.float32),
        # exact ties: low 16 bits 0x8000, both parities of the kept LSB
        (rng.integers(0, 1 << 31, 5000, dtype=np.int64).astype(np.uint32)
         & 0xFFFF0000 | 0x8000).view(np.float32),
    ])
    x32 = x32[np.isfinite(x32)]
    got = O.f64_to_bf16(x32.astype(np.float64))
    ref = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy()
    assert np.array_equal(got, ref.astype(np.uint16))


def test_bf16_rounding_of_float64_is_nearest_exactly():
    # torch rounds float64 -> bf16 through float32 (two roundings); the
    # oracle rounds once. Check nearest-with-ties-to-even with exact fractions.
    from fractions import Fraction
    rng = np.random.default_rng(4)
    x = np.concatenate([rng.standard_normal(3000) * 10.0 ** rng.integers(-30, 30, 3000),
                        [9.18551480857184e+29]])
    got = O.f64_to_bf16(x)
    for xi, b in zip(x, got):
        v = Fraction(float(xi))
        cand = [int(b) - 1, int(b), int(b) + 1]
        d = [abs(Fraction(_bf16_bits_by_struct(c & 0xFFFF)) - v) for c in cand]
        assert d[1] <= d[0] and d[1] <= d[2]
        if d[1] in (d[0], d[2]):
            assert int(b) % 2 == 0


@pytest.mark.parametrize("x,bits", [
    (1.0, 0x3F80), (-2.0, 0xC000), (1 + 2 ** -8, 0x3F80),     # tie -> even
    (1 + 3 * 2 ** -8, 0x3F82), (1 + 2 ** -8 + 2 ** -20, 0x3F81),
    (0.0, 0x0000), (-0.0, 0x8000), (float("inf"), 0x7F80),
    (3.4e38, 0x7F80), (2.0 ** -133, 0x0001), (2.0 ** -134, 0x0000),
])
def test_bf16_rounding_closed_forms(x, bits):
    assert int(O.f64_to_bf16(np.array([x]))[0]) == bits


def test_unpack_closed_forms():
    w = np.array([0x76543210, 0xFEDCBA98 - (1 << 32), 0x00000000, -1],
                 dtype=np.int64).astype(np.int32)
    q = O.unpack_uint4(w)
    assert q[:8].tolist() == list(range(8))
    assert q[8:16].tolist() == list(range(8, 16))
    assert q[16:24].tolist() == [0] * 8
    assert q[24:32].tolist() == [15] * 8


def test_unpack_every_value_every_position():
    for j in range(8):
        for v in range(16):
            w = np.array([(v << (4 * j)) & 0xFFFFFFFF], dtype=np.uint32).view(np.int32)
            q = O.unpack_uint4(w)
            expect = [0] * 8
            expect[j] = v
            assert q.tolist() == expect, (j, v)


def test_pack_unpack_inverse():
    rng = np.random.default_rng(2)
    w = rng.integers(0, 1 << 32, (5, 7, 12), dtype=np.uint64).astype(
        np.uint32).view(np.int32)
    assert np.array_equal(O.pack_uint4(O.unpack_uint4(w)), w)
    q = rng.integers(0, 16, (3, 64)).astype(np.uint8)
    assert np.array_equal(O.unpack_uint4(O.pack_uint4(q)), q)


def test_dequant_zero_point_and_scale_groups():
    N, K = 3, 96
    # 0x88888888: every q = 8 -> weight exactly 0 whatever the scale
    w8 = np.full((N, K // 8), 0x88888888 - (1 << 32), dtype=np.int64).astype(np.int32)
    s = np.full((N, K // 32), 0x3F80, dtype=np.uint16)          # 1.0
    assert np.all(O.dequant(w8, s) == 0.0)
    # q = 9 everywhere, scale of group g = g + 1 (exact in bf16):
    # W[n, k] = (9 - 8) * (k // 32 + 1)
    w9 = np.full((N, K // 8), 0x99999999 - (1 << 32), dtype=np.int64).astype(np.int32)
    sg = np.stack([torch.tensor([float(g + 1) for g in range(K // 32)]).to(
        torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)] * N)
    W = O.dequant(w9, sg)
    assert np.array_equal(W, np.tile(np.arange(K) // 32 + 1.0, (N, 1)))
    # q = 0 -> -8 * scale (sign of the zero point)
    w0 = np.zeros((N, K // 8), dtype=np.int32)
    assert np.all(O.dequant(w0, s) == -8.0)


def test_dequant_matches_independent_nibble_walk():
    rng = np.random.default_rng(3)
    N, K = 4, 64
    w = rng.integers(0, 1 << 32, (N, K // 8), dtype=np.uint64).astype(np.uint32)
    s = (rng.integers(0x3C00, 0x4100, (N, K // 32))).astype(np.uint16)
    W = O.dequant(w.view(np.int32), s)
    for n in range(N):
        for k in range(K):
            q = (int(w[n, k // 8]) >> (4 * (k % 8))) & 15
            sc = _bf16_bits_by_struct(s[n, k // 32])
            assert W[n, k] == (q - 8) * sc
