"""Seeded synthetic inputs for the W4A16 MoE expert GEMM pair.

This module is shared by the HIP path's callers (tests, bench) and by the
oracle's callers. It produces raw bit patterns only -- bf16 as uint16, packed
uint4 as int32 words, routing as int32 -- and holds none of the GEMM path's
arithmetic: no unpacking, dequantisation, routing alignment, GEMM or
activation. The one computation beyond sampling is on the input side: the
router-routed workloads (tiny, tp8) pick each token's experts as the top-k of
seeded N(0,1) logits, standing in for the router upstream of the path. That
choice orders logits the way the library's router kernel does (descending,
lower expert index on ties), but the kernel is checked against the oracle's
router, never against this generator.

Every tensor of a workload draws from its own child of one
``numpy.random.SeedSequence`` (PCG64), keyed by the tensor's name, so adding or
changing one tensor never shifts the bits of another. Both sides of a parity
check consume the same bits, as the [announce] page's per-layer measurement
section has both kernels run on the same routing sample.

Workloads (shapes of one EP8 or TP8 rank's share of a Kimi K2.x MoE layer:
hidden 7168, intermediate 2048, 384 experts, top-8):

* ``tiny``        8 experts, top-2, 64 tokens, K=256, I=128.
* ``ep8_decode``  48 local experts, per-expert counts U{9..15}, topk=1
                  (each dispatched (token, expert) pair is one row).
* ``tp8``         384 experts, 256 tokens, top-8, I/8=256.
* ``ep8_prefill`` 48 experts, 8192 rows, expert choice Zipf(1.1) over a
                  seeded permutation of the experts.
* ``ep8_prefill_span`` the same row total with counts spanning ~590..20.
* ``contiguous``  48 experts x 128 rows, grouped_contiguous layout.
* ``masked``      48 experts, 64-row budget, 32 valid rows each.
* ``ep16_decode`` 24 local experts, counts U{9..15} (EP16 rank share).
* ``ep32_decode`` 12 local experts, counts U{9..15} (EP32 rank share).
* ``ep8_mid``     48 local experts, counts U{40..56}: the 33..79 rows per
                  expert between decode and the large-M threshold.
* ``ep128_decode`` 3 local experts, counts U{9..15} (an EP128 rank share:
                  so few tiles that the split-K gate turns on).
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field
from typing import Dict, Optional

import numpy as np

HIDDEN = 7168
INTER = 2048


def _child(seed: int, name: str) -> np.random.Generator:
    key = int.from_bytes(hashlib.sha256(name.encode()).digest()[:8], "little")
    ss = np.random.SeedSequence(entropy=seed, spawn_key=(key,))
    return np.random.Generator(np.random.PCG64(ss))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even) and return the bits.

    Used to turn sampled normals into bf16 inputs; NaN is not produced here.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    bias = 0x7FFF + ((u >> 16) & 1)
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_normal(rng: np.random.Generator, shape, std: float = 1.0,
                absolute: bool = False) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32) * np.float32(std)
    if absolute:
        x = np.abs(x)
    return f32_to_bf16_bits(x)


def random_words(rng: np.random.Generator, shape) -> np.ndarray:
    """Uniform 32-bit words as int32: eight i.i.d. uniform uint4 values each."""
    return rng.integers(0, 1 << 32, size=shape, dtype=np.uint64).astype(
        np.uint32).view(np.int32)


@dataclass
class Workload:
    """One workload's inputs, as raw bit patterns (host numpy arrays)."""
    name: str
    kind: str                      # "indexed" | "contiguous" | "masked"
    E: int
    K: int                         # hidden (gate_up K, down N)
    I: int                         # intermediate (gate_up N = 2I, down K)
    T: int = 0                     # tokens (indexed)
    topk: int = 1
    arrays: Dict[str, np.ndarray] = field(default_factory=dict)
    meta: Dict[str, object] = field(default_factory=dict)

    def __getitem__(self, k):
        return self.arrays[k]


def _router_topk(rng: np.random.Generator, T: int, E: int, topk: int):
    """Routing input for router-routed workloads: each token's experts are
    the top-k of seeded N(0,1) logits, by descending logit with ties to the
    lower expert index (a stable sort); the weights are the softmax
    probabilities of the chosen experts over all E, not renormalised."""
    logits = rng.standard_normal(size=(T, E), dtype=np.float32).astype(np.float64)
    order = np.argsort(-logits, axis=1, kind="stable")[:, :topk]
    z = np.exp(logits - logits.max(axis=1, keepdims=True))
    p = z / z.sum(axis=1, keepdims=True)
    w = np.take_along_axis(p, order, axis=1).astype(np.float32)
    return order.astype(np.int32), w


def _weights(rng_w, rng_s, E: int, N: int, K: int):
    qweight = random_words(rng_w, (E, N, K // 8))
    scales = bf16_normal(rng_s, (E, N, K // 32), std=0.02, absolute=True)
    return qweight, scales


def _with_weights(wl: Workload, seed: int, weights: bool):
    if not weights:
        return wl
    E, K, I = wl.E, wl.K, wl.I
    wl.arrays["w13"], wl.arrays["s13"] = _weights(
        _child(seed, "w13"), _child(seed, "s13"), E, 2 * I, K)
    wl.arrays["w2"], wl.arrays["s2"] = _weights(
        _child(seed, "w2"), _child(seed, "s2"), E, K, I)
    return wl


def _indexed_from_ids(name, seed, E, K, I, ids, topk, topk_w, weights, meta):
    T = ids.shape[0]
    wl = Workload(name=name, kind="indexed", E=E, K=K, I=I, T=T, topk=topk,
                  meta=dict(meta))
    wl.arrays["topk_ids"] = np.ascontiguousarray(ids, dtype=np.int32)
    wl.arrays["topk_weights"] = np.ascontiguousarray(topk_w, dtype=np.float32)
    wl.arrays["a"] = bf16_normal(_child(seed, "a"), (T, K))
    return _with_weights(wl, seed, weights)


def _shuffled_multiset(rng, counts):
    ids = np.repeat(np.arange(len(counts), dtype=np.int32), counts)
    rng.shuffle(ids)
    return ids


def make_router_workload(name, seed, E, T, topk, K, I, weights=True):
    ids, w = _router_topk(_child(seed, "router"), T, E, topk)
    return _indexed_from_ids(name, seed, E, K, I, ids, topk, w, weights,
                             {"routing": "softmax(N(0,1)) top-%d" % topk})


def make_count_workload(name, seed, counts, K, I, weights=True, meta=None):
    """topk=1 workload whose per-expert row counts are exactly ``counts``."""
    counts = np.asarray(counts, dtype=np.int64)
    ids = _shuffled_multiset(_child(seed, "shuffle"), counts)[:, None]
    w = np.ones_like(ids, dtype=np.float32)
    m = {"counts": counts.tolist()}
    if meta:
        m.update(meta)
    return _indexed_from_ids(name, seed, len(counts), K, I, ids, 1, w, weights, m)


def uniform_counts(seed, E, lo=9, hi=15):
    return _child(seed, "counts").integers(lo, hi + 1, size=E)


def zipf_ids(seed, E, R, s=1.1):
    """R i.i.d. expert choices with P(rank r) proportional to r^-s over a
    seeded permutation of the experts (truncated Zipf)."""
    r = np.arange(1, E + 1, dtype=np.float64)
    p = r ** -s
    p /= p.sum()
    perm = _child(seed, "perm").permutation(E)
    ranks = _child(seed, "choice").choice(E, size=R, p=p)
    return perm[ranks].astype(np.int32)


def span_counts(seed, E, R, hi=600.0, ratio=30.0):
    """Geometric counts from ``hi`` down to hi/ratio, rescaled to sum R with
    largest-remainder rounding, then assigned to a seeded permutation."""
    c = hi * ratio ** (-(np.arange(E) / (E - 1)))
    c = c * (R / c.sum())
    base = np.floor(c).astype(np.int64)
    rem = R - base.sum()
    base[np.argsort(-(c - base), kind="stable")[:rem]] += 1
    out = np.empty(E, dtype=np.int64)
    out[_child(seed, "perm").permutation(E)] = base
    return out


def make_contiguous(name, seed, E, rows_per_expert, K, I, pad_to=128,
                    counts=None, weights=True):
    """grouped_contiguous input: each expert's rows contiguous and padded to a
    multiple of ``pad_to`` rows; padding rows have m_indices = -1."""
    if counts is None:
        counts = np.full(E, rows_per_expert, dtype=np.int64)
    counts = np.asarray(counts, dtype=np.int64)
    padded = ((counts + pad_to - 1) // pad_to) * pad_to
    M = int(padded.sum())
    m_idx = np.full(M, -1, dtype=np.int32)
    off = 0
    for e in range(E):
        m_idx[off:off + counts[e]] = e
        off += int(padded[e])
    wl = Workload(name=name, kind="contiguous", E=E, K=K, I=I,
                  meta={"counts": counts.tolist(), "M": M})
    wl.arrays["m_indices"] = m_idx
    wl.arrays["a"] = bf16_normal(_child(seed, "a"), (M, K))
    return _with_weights(wl, seed, weights)


def make_masked(name, seed, E, budget, valid, K, I, expected_m=None,
                masked_m=None, weights=True):
    """grouped_masked input: A [E, budget, K]; rows r < masked_m[e] are valid."""
    if masked_m is None:
        masked_m = np.full(E, valid, dtype=np.int32)
    masked_m = np.asarray(masked_m, dtype=np.int32)
    wl = Workload(name=name, kind="masked", E=E, K=K, I=I,
                  meta={"budget": budget,
                        "expected_m": int(expected_m if expected_m is not None
                                          else valid)})
    wl.arrays["masked_m"] = masked_m
    wl.arrays["a"] = bf16_normal(_child(seed, "a"), (E, budget, K))
    return _with_weights(wl, seed, weights)


WORKLOADS = ("tiny", "ep8_decode", "tp8", "ep8_prefill", "ep8_prefill_span",
             "contiguous", "masked", "ep16_decode", "ep32_decode", "ep8_mid",
             "ep128_decode")


def make(name: str, seed: int = 0, weights: bool = True,
         K: Optional[int] = None, I: Optional[int] = None) -> Workload:
    """Build one named workload. ``K``/``I`` override hidden/intermediate for
    reduced-size runs of the same structure."""
    K = HIDDEN if K is None else K
    I = INTER if I is None else I
    if name == "tiny":
        return make_router_workload(name, seed, 8, 64, 2,
                                    256 if K == HIDDEN else K,
                                    128 if I == INTER else I, weights)
    if name == "ep8_decode":
        return make_count_workload(name, seed, uniform_counts(seed, 48), K, I,
                                   weights, {"routing": "U{9..15} per expert"})
    if name == "ep16_decode":
        return make_count_workload(name, seed, uniform_counts(seed, 24), K, I,
                                   weights, {"routing": "U{9..15} per expert"})
    if name == "ep32_decode":
        return make_count_workload(name, seed, uniform_counts(seed, 12), K, I,
                                   weights, {"routing": "U{9..15} per expert"})
    if name == "ep8_mid":
        return make_count_workload(name, seed, uniform_counts(seed, 48, 40, 56), K, I,
                                   weights, {"routing": "U{40..56} per expert"})
    if name == "ep128_decode":
        return make_count_workload(name, seed, uniform_counts(seed, 3), K, I,
                                   weights, {"routing": "U{9..15} per expert"})
    if name == "tp8":
        return make_router_workload(name, seed, 384, 256, 8, K,
                                    256 if I == INTER else I, weights)
    if name == "ep8_prefill":
        ids = zipf_ids(seed, 48, 8192)[:, None]
        w = np.ones_like(ids, dtype=np.float32)
        return _indexed_from_ids(name, seed, 48, K, I, ids, 1, w, weights,
                                 {"routing": "Zipf(1.1) over 48 experts"})
    if name == "ep8_prefill_span":
        return make_count_workload(name, seed, span_counts(seed, 48, 8192), K,
                                   I, weights, {"routing": "geometric 600..20"})
    if name == "contiguous":
        return make_contiguous(name, seed, 48, 128, K, I, weights=weights)
    if name == "masked":
        return make_masked(name, seed, 48, 64, 32, K, I, weights=weights)
    raise KeyError(name)
