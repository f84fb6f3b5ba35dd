"""CPU oracle for the W4A16 MoE expert GEMM pair (gate_up, activation, down).

TEST INFRASTRUCTURE. Only the tests, the smoke check and the CPU-baseline
leg of the benchmark may import this module. The library's product path never
calls it, and this module imports nothing from the HIP side.

It is written to be read against the pages, not to be fast. Floating point is
float64. Each function names the passage it follows. The pages are cited as:

* [release] "vLLM and Novita AI release Chord: a fast INT4 MoE kernel for
  Kimi K2.x" (agentlenshq.com, Japanese);
* [announce] "vLLM announces that the Humming backend can run Novita's
  open-source Chord kernel" (arex-research.com, Chinese).

Readings of points the pages leave open:

* zero point 8: w = (q - 8) * scale;
* nibble k % 8 of a packed int32 word sits at bits 4*(k % 8) .. +3;
* sentinel slot id = T*topk;
* ascending slot order inside an expert's segment;
* expert id -1 means "not on this rank" and is skipped;
* SiLU is the gate activation: the first I columns are the gate, the last I
  the up projection.

Every function here is pinned by the CPU tests: brute force, closed forms,
invariants and library special cases.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

ZERO_POINT = 8
GROUP = 32


# --------------------------------------------------------------------------
# bf16 <-> float64  (BF16 activations and scales: [release] TL;DR;
# [announce] integration section: uint4 weights with group-32 BF16 scales)
# --------------------------------------------------------------------------

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64. A bf16 is the top half of a float32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to bf16 (nearest, ties to even); return the bits.

    bf16 carries 8 significant bits and float32's exponent range. A finite x
    is rounded to the multiple of its quantum 2^(e-8) (x = m*2^e with
    0.5 <= |m| < 1). Below the normal range the quantum is fixed at
    2^-133. Values that round past the largest finite bf16 become infinity.
    NaN becomes the quiet NaN 0x7FC0.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    nan = np.isnan(x)
    fin = np.isfinite(x)
    _, e = np.frexp(np.where(fin, x, 1.0))
    quantum_exp = np.maximum(e - 8, -133)
    q = np.ldexp(1.0, quantum_exp)
    r = np.rint(np.where(fin, x, 0.0) / q) * q          # rint: ties to even
    over = fin & (np.abs(r) >= 2.0 ** 128)
    with np.errstate(over="ignore"):
        r32 = r.astype(np.float32)
    bits = (r32.view(np.uint32) >> 16).astype(np.uint16)
    out[...] = bits
    inf_bits = np.where(np.signbit(x), 0xFF80, 0x7F80).astype(np.uint16)
    out[over | np.isinf(x)] = inf_bits[over | np.isinf(x)]
    out[nan] = 0x7FC0
    return out


# --------------------------------------------------------------------------
# Packed uint4 format  ([announce] integration section: compressed-tensors
# pack-quantized INT4 group-32 checkpoints; [release] TL;DR: INT4 weights)
# --------------------------------------------------------------------------

def unpack_uint4(qweight: np.ndarray) -> np.ndarray:
    """int32 words [..., K/8] -> uint4 values [..., K] (as uint8).

    Element k is nibble k % 8 of word k // 8, at bits 4*(k % 8) .. +3.
    """
    w = np.asarray(qweight).astype(np.int64) & 0xFFFFFFFF
    shifts = 4 * np.arange(8, dtype=np.int64)
    q = (w[..., :, None] >> shifts) & 0xF
    return q.reshape(*w.shape[:-1], w.shape[-1] * 8).astype(np.uint8)


def pack_uint4(q: np.ndarray) -> np.ndarray:
    """uint4 values [..., K] -> int32 words [..., K/8] (inverse of unpack)."""
    q = np.asarray(q).astype(np.int64)
    assert q.shape[-1] % 8 == 0 and q.min() >= 0 and q.max() <= 15
    g = q.reshape(*q.shape[:-1], q.shape[-1] // 8, 8)
    w = np.zeros(g.shape[:-1], dtype=np.int64)
    for j in range(8):
        w |= g[..., j] << (4 * j)
    return w.astype(np.uint32).view(np.int32)


def dequant(qweight: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """W[..., n, k] = (q[..., n, k] - 8) * scale[..., n, k // 32], in float64.

    The product of a 4-bit integer and a bf16 scale is exact in float64.
    """
    q = unpack_uint4(qweight).astype(np.float64)
    s = bf16_to_f64(scales)
    K = q.shape[-1]
    assert s.shape[-1] * GROUP == K
    return (q - ZERO_POINT) * np.repeat(s, GROUP, axis=-1)


# --------------------------------------------------------------------------
# moe_align  ([announce] scheduling section: the indexed path consumes the
# sorted_ids / expert_ids / num_tokens_padded tensors of vLLM's block-aligned
# routing; [release] runtime considerations: those buffers are
# over-allocated)
# --------------------------------------------------------------------------

def align_sizes(T: int, topk: int, E: int, block_m: int):
    """Capacity that always suffices: sum_e ceil(c_e/B)*B <= R + E*(B-1)."""
    R = T * topk
    cap = R + E * (block_m - 1)
    return cap, (cap + block_m - 1) // block_m


def moe_align(topk_ids: np.ndarray, E: int, block_m: int,
              sorted_cap: Optional[int] = None):
    """Stable counting sort of the routed slots by expert, padded per expert.

    Slot i = t*topk + k holds expert topk_ids[t, k]. For each expert e in
    order, its slots are listed in ascending order. The list is padded with
    the sentinel R = T*topk up to a multiple of block_m. An expert with no
    slots gets no block. expert_ids names the expert of each block. Entries
    past num_tokens_padded hold the sentinel (sorted_ids) or -1
    (expert_ids). Slots whose id is outside [0, E) are left out.
    """
    ids = np.asarray(topk_ids, dtype=np.int64).reshape(-1)
    R = ids.size
    if sorted_cap is None:
        sorted_cap = R + E * (block_m - 1)
    blocks_cap = (sorted_cap + block_m - 1) // block_m
    sorted_ids = np.full(sorted_cap, R, dtype=np.int32)
    expert_ids = np.full(blocks_cap, -1, dtype=np.int32)
    pos = 0
    for e in range(E):
        slots = [i for i in range(R) if ids[i] == e]        # ascending
        if not slots:
            continue
        padded = -(-len(slots) // block_m) * block_m
        assert pos + padded <= sorted_cap, "sorted_cap too small"
        sorted_ids[pos:pos + len(slots)] = slots
        expert_ids[pos // block_m:(pos + padded) // block_m] = e
        pos += padded
    return sorted_ids, expert_ids, np.int32(pos)


def moe_align_fast(topk_ids: np.ndarray, E: int, block_m: int,
                   sorted_cap: Optional[int] = None):
    """The same result as :func:`moe_align`, vectorised for large inputs
    (a stable argsort by expert takes the place of the per-expert scan)."""
    ids = np.asarray(topk_ids, dtype=np.int64).reshape(-1)
    R = ids.size
    if sorted_cap is None:
        sorted_cap = R + E * (block_m - 1)
    blocks_cap = (sorted_cap + block_m - 1) // block_m
    valid = (ids >= 0) & (ids < E)
    counts = np.bincount(ids[valid], minlength=E)
    padded = -(-counts // block_m) * block_m
    starts = np.concatenate([[0], np.cumsum(padded)[:-1]])
    order = np.argsort(np.where(valid, ids, E), kind="stable")[:valid.sum()]
    sorted_ids = np.full(sorted_cap, R, dtype=np.int32)
    ranks = np.arange(order.size) - np.repeat(
        np.concatenate([[0], np.cumsum(counts)[:-1]]), counts)
    ntp = int(padded.sum())
    assert ntp <= sorted_cap, "sorted_cap too small"
    sorted_ids[np.repeat(starts, counts) + ranks] = order
    expert_ids = np.full(blocks_cap, -1, dtype=np.int32)
    expert_ids[:ntp // block_m] = np.repeat(np.arange(E), padded // block_m)
    return sorted_ids, expert_ids, np.int32(ntp)


# --------------------------------------------------------------------------
# Expert GEMMs  ([announce] measurement section: a layer is the gate/up GEMM
# and the down GEMM; [release] TL;DR: W4A16, INT4 weights, BF16 activations)
# --------------------------------------------------------------------------

def _rows_dot(a_rows: np.ndarray, qweight_e: np.ndarray, scales_e: np.ndarray,
              cols: Optional[np.ndarray]) -> np.ndarray:
    """a_rows [m, K] (float64) times dequantised W_e[cols]^T -> [m, |cols|]."""
    if cols is not None:
        qweight_e = qweight_e[cols]
        scales_e = scales_e[cols]
    return a_rows @ dequant(qweight_e, scales_e).T


def moe_gemm_by_slot(a_bits: np.ndarray, a_row_div: int, slot_expert: np.ndarray,
                     qweight: np.ndarray, scales: np.ndarray,
                     cols: Optional[Sequence[int]] = None,
                     topk_weights: Optional[np.ndarray] = None) -> np.ndarray:
    """C[s, n] = sum_k A[s // a_row_div, k] * W[e(s)][n, k] for every slot s.

    e(s) = slot_expert[s]. Slots with e(s) outside [0, E) are undefined and
    hold NaN. gate_up reads token row s // topk; down reads row s. When
    topk_weights is given, row s is scaled by topk_weights.flat[s].
    """
    A = bf16_to_f64(a_bits)
    se = np.asarray(slot_expert, dtype=np.int64).reshape(-1)
    E, N = qweight.shape[0], qweight.shape[1]
    cols_a = None if cols is None else np.asarray(cols, dtype=np.int64)
    out = np.full((se.size, N if cols_a is None else cols_a.size), np.nan)
    for e in range(E):
        slots = np.nonzero(se == e)[0]
        if slots.size == 0:
            continue
        out[slots] = _rows_dot(A[slots // a_row_div], qweight[e], scales[e],
                               cols_a)
    if topk_weights is not None:
        out *= np.asarray(topk_weights, dtype=np.float64).reshape(-1)[:, None]
    return out


def indexed_gemm_from_buffers(a_bits, a_row_div, qweight, scales, sorted_ids,
                              expert_ids, num_tokens_padded, block_m,
                              num_slots, cols=None, topk_weights=None):
    """What the indexed GEMM computes from the routing buffers.

    For every block b < num_tokens_padded / block_m, with expert
    e = expert_ids[b], and every row s = sorted_ids[b*block_m + i] with
    s < num_slots: C[s] = A[s // a_row_div] . W_e^T. Rows of C that no block
    names are NaN (the GPU leaves them untouched).
    """
    slot_expert = np.full(num_slots, -1, dtype=np.int64)
    nb = int(num_tokens_padded) // block_m
    for b in range(nb):
        e = int(expert_ids[b])
        for s in sorted_ids[b * block_m:(b + 1) * block_m]:
            if s < num_slots:
                slot_expert[s] = e
    return moe_gemm_by_slot(a_bits, a_row_div, slot_expert, qweight, scales,
                            cols, topk_weights)


def grouped_contiguous(a_bits, m_indices, qweight, scales, cols=None):
    """C[r] = A[r] . W[m_indices[r]]^T for rows with m_indices[r] >= 0
    ([release] grouped SM90 techniques: contiguous prefill pads each expert
    to 128 rows). Padding rows (-1) are NaN."""
    return moe_gemm_by_slot(a_bits, 1, m_indices, qweight, scales, cols)


def grouped_masked(a_bits, masked_m, qweight, scales, cols=None):
    """C[e, r] = A[e, r] . W[e]^T for r < masked_m[e] ([release] grouped SM90
    techniques: masked decode keeps a fixed row budget per expert). Other
    rows are NaN. a_bits is [E, budget, K]; the result is [E, budget, N]."""
    E, budget, K = a_bits.shape
    slot_expert = np.full((E, budget), -1, dtype=np.int64)
    for e in range(E):
        slot_expert[e, :int(masked_m[e])] = e
    out = moe_gemm_by_slot(a_bits.reshape(E * budget, K), 1,
                           slot_expert.reshape(-1), qweight, scales, cols)
    return out.reshape(E, budget, -1)


# --------------------------------------------------------------------------
# Activation between the GEMMs ([announce] measurement section names an
# "activation" between gate/up and down; the reading is SiLU-gated)
# --------------------------------------------------------------------------

def silu_and_mul(x_bits: np.ndarray) -> np.ndarray:
    """x [R, 2I] bf16 -> silu(x[:, :I]) * x[:, I:] in float64."""
    x = bf16_to_f64(x_bits)
    I = x.shape[-1] // 2
    g, u = x[..., :I], x[..., I:]
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g)) * u


# --------------------------------------------------------------------------
# Combine over top-k (the step after down; the pages exclude it from the
# kernel timing)
# --------------------------------------------------------------------------

def moe_combine(c2: np.ndarray, topk_weights: np.ndarray, topk: int):
    """out[t] = sum_k w[t, k] * C2[t*topk + k]."""
    T = c2.shape[0] // topk
    w = np.asarray(topk_weights, dtype=np.float64).reshape(T, topk)
    return (c2.reshape(T, topk, -1) * w[:, :, None]).sum(axis=1)


def router_topk(logits, topk: int):
    """Router of the MoE layer, the step before moe_align (the pages' decode
    and prefill scenarios route each token to its top-k experts). Reading
    adopted: weights are the softmax over all E experts, not renormalised
    over the chosen k; the k experts are those with the largest logits
    (softmax is monotone, so this is the largest-probability choice without
    rounding ties), equal logits going to the lower expert index.

    logits: [T, E] float32. Returns (topk_ids [T, topk] int32,
    topk_weights [T, topk] float64), ids in descending order of logit."""
    lg = np.asarray(logits, dtype=np.float64)
    T, E = lg.shape
    ids = np.empty((T, topk), dtype=np.int32)
    w = np.empty((T, topk), dtype=np.float64)
    for t in range(T):
        row = lg[t]
        m = row.max()
        ex = np.exp(row - m)
        p = ex / ex.sum()
        # descending logit, lower index first on equal logits
        order = sorted(range(E), key=lambda e: (-row[e], e))[:topk]
        ids[t] = order
        w[t] = p[order]
    return ids, w

