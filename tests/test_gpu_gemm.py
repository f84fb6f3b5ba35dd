"""Expert GEMMs on the GPU against the oracle, at sizes the oracle finishes in
seconds (several tiles, ragged tails, every kernel instance), through the C
ABI: random inputs within the per-expert tolerance, integer-exact inputs
bit-for-bit, and the method's invariants and edge cases."""
import numpy as np
import pytest
import torch

from oracle import qma_oracle as O
from quantized_moe_align_amd import inputs, qma
from quantized_moe_align_amd.moe import (ExpertWeights, IndexedMoE, empty_bf16, to_device,
                                         to_host, workspace_for)
from gpu_common import assert_per_expert, bf16_pow2, bf16_small_ints, rne, slot_experts

pytestmark = pytest.mark.gpu

SENT = 0x5A5A  # pattern pre-filled into outputs to detect untouched rows


def weights(rng, E, N, K, integer=False):
    w = inputs.random_words(rng, (E, N, K // 8))
    s = bf16_pow2(rng, (E, N, K // 32)) if integer else \
        inputs.bf16_normal(rng, (E, N, K // 32), 0.02, absolute=True)
    return w, s


def apply_override(plan, override):
    """Set plan fields; an override that gives no schedule runs semi-static
    (the shapes it sets need not take the planner's schedule)."""
    if override:
        plan.schedule = qma.SCHEDULE_SEMI_STATIC
    for k, v in (override or {}).items():
        setattr(plan, k, v)


def indexed(a_bits, a_row_div, ids, w, s, *, T=None, topk=None, force_bm=0, override=None,
            extra_cap=0, junk_tail=False, topk_w=None, pre=None, flags=0):
    """Run moe_align + one indexed GEMM through the ABI; return output bits
    ([R, N], or [R, N / 2] for a layer with the activation fused)."""
    E, N, K8 = w.shape
    ids = np.asarray(ids, np.int32)
    T = ids.shape[0] if T is None else T
    topk = ids.shape[1] if topk is None else topk
    R = T * topk
    W = ExpertWeights(w, s, flags=flags)
    if W.fused:
        N //= 2
    plan = qma.qma_plan_indexed(W.layer, T, topk, force_bm)
    apply_override(plan, override)
    B = plan.block_m
    cap = qma.qma_align_sizes(T, topk, E, B)[0] + extra_cap
    sorted_ids = torch.empty(cap, dtype=torch.int32, device="cuda")
    expert_ids = torch.empty(-(-cap // B), dtype=torch.int32, device="cuda")
    ntp = torch.empty(1, dtype=torch.int32, device="cuda")
    d_ids = to_device(ids)
    qma.qma_moe_align(d_ids, T, topk, E, B, sorted_ids, expert_ids, ntp, cap)
    if junk_tail:
        torch.cuda.synchronize()
        n = int(ntp.item())
        sorted_ids[n:] = 0                 # looks like a real slot
        expert_ids[n // B:] = E - 1        # looks like a real expert
    a = to_device(a_bits)
    c = torch.full((R, N), SENT, dtype=torch.int16, device="cuda") if pre is None else pre
    ws = workspace_for(plan)
    tw = None if topk_w is None else torch.from_numpy(np.ascontiguousarray(topk_w, np.float32)).cuda()
    qma.qma_indexed_gemm(W.layer, plan, a, a_bits.shape[0], a_row_div, W.packed, sorted_ids,
                         expert_ids, ntp, cap, R, tw, c, ws, 0 if ws is None else ws.numel())
    torch.cuda.synchronize()
    return to_host(c, bf16=True), plan


SHAPES = [  # (E, T, topk, K, N)
    (8, 64, 2, 256, 256),        # tiny gate_up
    (8, 128, 1, 128, 256),       # tiny down (K = I = 128, one chunk)
    (6, 100, 3, 512, 384),       # ragged: N % 128 != 0, tails in every expert
    (5, 37, 4, 1024, 160),       # 16-wide column tail (N = 10 tiles)
]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("force_bm", [0, 16, 32, 64])
def test_indexed_random_within_tolerance(gpu, shape, force_bm):
    E, T, topk, K, N = shape
    rng = np.random.default_rng(hash((shape, force_bm)) % 2**32)
    w, s = weights(rng, E, N, K)
    a = inputs.bf16_normal(rng, (T, K))
    ids = rng.integers(0, E, (T, topk)).astype(np.int32)
    got, plan = indexed(a, topk, ids, w, s, force_bm=force_bm)
    ref = O.moe_gemm_by_slot(a, topk, ids, w, s)
    assert_per_expert(got, ref, slot_experts(ids, E), f"{shape} bm={plan.block_m}")


# (force_bm, ntw, waves_k); 0 = planner. waves_k 1 with 2 or 4 column tiles
# per wave is the shared-row kernel, the rest the per-wave-row kernel.
KERNEL_INSTANCES = [(0, 0, 0), (16, 1, 4), (16, 1, 1), (16, 2, 1), (16, 4, 2), (16, 4, 4), (16, 4, 1),
                    (32, 2, 4), (32, 2, 2), (32, 1, 1), (32, 4, 1), (32, 2, 1), (64, 2, 1),
                    (64, 1, 1), (64, 1, 2), (64, 1, 4)]


def _fits(shape, inst):
    _, ntw, wk = inst
    return not ntw or shape[4] % (ntw * 16 * (4 // wk)) == 0


@pytest.mark.parametrize("shape,force_bm,ntw,wk",
                         [(sh,) + inst for sh in SHAPES for inst in KERNEL_INSTANCES
                          if _fits(sh, inst)])
def test_indexed_integer_exact_bitwise(gpu, shape, force_bm, ntw, wk):
    E, T, topk, K, N = shape
    block_n = ntw * 16 * (4 // wk) if ntw else 0
    rng = np.random.default_rng(7 + E + T)
    w, s = weights(rng, E, N, K, integer=True)
    a = bf16_small_ints(rng, (T, K))
    ids = rng.integers(-1, E, (T, topk)).astype(np.int32)
    got, _ = indexed(a, topk, ids, w, s, force_bm=force_bm,
                     override={"block_n": block_n, "waves_k": wk, "split_k": 1}
                     if block_n else None)
    ref = O.moe_gemm_by_slot(a, topk, ids, w, s)
    valid = slot_experts(ids, E) >= 0
    assert np.array_equal(got[valid], rne(ref[valid]))
    assert np.all(got[~valid] == SENT)           # rows of slots not on this rank untouched


# (force_bm, plan edits): shared-row kernel at 32 and 64 rows, and the
# per-wave-row kernel (waves splitting K)
SPLIT_FAMILIES = [(0, {}), (64, {}), (16, {"block_n": 64, "waves_k": 4})]


@pytest.mark.parametrize("split", [2, 3, 4])
@pytest.mark.parametrize("family", range(len(SPLIT_FAMILIES)))
def test_split_k_matches_unsplit(gpu, split, family):
    force_bm, edits = SPLIT_FAMILIES[family]
    E, T, topk, K, N = 3, 40, 2, 2048, 256
    rng = np.random.default_rng(split)
    w, s = weights(rng, E, N, K, integer=True)
    a = bf16_small_ints(rng, (T, K))
    ids = rng.integers(0, E, (T, topk)).astype(np.int32)
    base, p0 = indexed(a, topk, ids, w, s, force_bm=force_bm, override=dict(edits) or None)
    got, p1 = indexed(a, topk, ids, w, s, force_bm=force_bm, override={**edits, "split_k": split})
    assert p1.split_k == split and qma.qma_workspace_bytes(p1) > 0
    assert np.array_equal(base, got)
    assert np.array_equal(got, rne(O.moe_gemm_by_slot(a, topk, ids, w, s)))
    # random inputs: same bar as the unsplit kernel
    w2, s2 = weights(rng, E, N, K)
    a2 = inputs.bf16_normal(rng, (T, K))
    tw = rng.random(T * topk).astype(np.float32)
    got2, _ = indexed(a2, topk, ids, w2, s2, topk_w=tw, force_bm=force_bm,
                      override={**edits, "split_k": split})
    assert_per_expert(got2, O.moe_gemm_by_slot(a2, topk, ids, w2, s2, topk_weights=tw),
                      slot_experts(ids, E))


def test_overallocated_buffers_with_junk_tail(gpu):
    E, T, topk, K, N = 6, 50, 2, 512, 128
    rng = np.random.default_rng(11)
    w, s = weights(rng, E, N, K, integer=True)
    a = bf16_small_ints(rng, (T, K))
    ids = rng.integers(0, E, (T, topk)).astype(np.int32)
    base, _ = indexed(a, topk, ids, w, s)
    got, _ = indexed(a, topk, ids, w, s, extra_cap=200, junk_tail=True)
    assert np.array_equal(base, got)


def test_identity_weights_gather_exactly(gpu):
    # W = [I | 0]: the GEMM is a pure gather. With integer activations every
    # sum is exact, so the output equals the gathered rows bit for bit; with
    # random activations it is within the tolerance (the zero-point fold
    # sums x*(128+q) and -136*x in fp32).
    E, T, topk, K, N = 4, 30, 3, 256, 128
    rng = np.random.default_rng(12)
    q = np.full((E, N, K), 8)
    for n in range(N):
        q[:, n, n] = 9
    w = O.pack_uint4(q)
    s = np.full((E, N, K // 32), 0x3F80, np.uint16)
    ids = rng.integers(0, E, (T, topk)).astype(np.int32)
    slots = np.arange(T * topk)
    a = bf16_small_ints(rng, (T, K), -100, 100)
    got, _ = indexed(a, topk, ids, w, s)
    assert np.array_equal(got, a[slots // topk, :N])
    a2 = inputs.bf16_normal(rng, (T, K))
    got2, _ = indexed(a2, topk, ids, w, s)
    assert_per_expert(got2, O.bf16_to_f64(a2[slots // topk, :N]), slot_experts(ids, E))


def test_nan_poisoned_unused_data_is_never_read(gpu):
    E, T, topk, K, N = 8, 40, 2, 256, 128
    rng = np.random.default_rng(13)
    w, s = weights(rng, E, N, K)
    a = inputs.bf16_normal(rng, (T, K))
    ids = rng.integers(0, 5, (T, topk)).astype(np.int32)     # experts 5..7 get no tokens
    ids[3] = -1                                               # token 3 is not on this rank
    s_poison = s.copy()
    s_poison[5:] = 0x7FC0
    a_poison = a.copy()
    a_poison[3] = 0x7FC0
    got, _ = indexed(a_poison, topk, ids, w, s_poison)
    ref = O.moe_gemm_by_slot(a, topk, ids, w, s)
    assert_per_expert(got, ref, slot_experts(ids, E))


def test_topk_weights_in_epilogue(gpu):
    E, T, topk, K, N = 4, 20, 2, 256, 128
    rng = np.random.default_rng(14)
    w, s = weights(rng, E, N, K)
    a = inputs.bf16_normal(rng, (T * topk, K))
    ids = rng.integers(0, E, (T, topk)).astype(np.int32)
    tw = rng.random(T * topk).astype(np.float32)
    got, _ = indexed(a, 1, ids, w, s, topk_w=tw)             # down-style: row = slot
    ref = O.moe_gemm_by_slot(a, 1, ids, w, s, topk_weights=tw)
    assert_per_expert(got, ref, slot_experts(ids, E))


def test_permutation_equivariance_bitwise(gpu):
    E, T, topk, K, N = 6, 48, 2, 512, 128
    rng = np.random.default_rng(15)
    w, s = weights(rng, E, N, K)
    a = inputs.bf16_normal(rng, (T, K))
    ids = rng.integers(0, E, (T, topk)).astype(np.int32)
    perm = rng.permutation(T)
    base, _ = indexed(a, topk, ids, w, s)
    got, _ = indexed(a[perm], topk, ids[perm], w, s)
    slot_perm = (perm[:, None] * topk + np.arange(topk)).reshape(-1)
    assert np.array_equal(got, base[slot_perm])


# ---- grouped paths -------------------------------------------------------

def contiguous(a_bits, m_idx, w, s, override=None, flags=0):
    E, N, K8 = w.shape
    W = ExpertWeights(w, s, qma.PATH_GROUPED_CONTIGUOUS, flags=flags)
    if W.fused:
        N //= 2
    M = m_idx.size
    plan = qma.qma_plan_grouped(W.layer, M, 0)
    apply_override(plan, override)
    c = torch.full((M, N), SENT, dtype=torch.int16, device="cuda")
    ws = workspace_for(plan)
    qma.qma_grouped_contiguous_gemm(W.layer, plan, to_device(a_bits), to_device(m_idx), M,
                                    W.packed, c, ws, 0 if ws is None else ws.numel())
    torch.cuda.synchronize()
    return to_host(c, bf16=True)


def masked(a_bits, masked_m, expected_m, w, s, override=None, flags=0):
    E, N, K8 = w.shape
    Eb, Mb, K = a_bits.shape
    W = ExpertWeights(w, s, qma.PATH_GROUPED_MASKED, flags=flags)
    if W.fused:
        N //= 2
    plan = qma.qma_plan_grouped(W.layer, Mb, expected_m)
    apply_override(plan, override)
    c = torch.full((E, Mb, N), SENT, dtype=torch.int16, device="cuda")
    ws = workspace_for(plan)
    qma.qma_grouped_masked_gemm(W.layer, plan, to_device(a_bits), to_device(masked_m), Mb,
                                expected_m, W.packed, c, ws, 0 if ws is None else ws.numel())
    torch.cuda.synchronize()
    return to_host(c, bf16=True)


@pytest.mark.parametrize("integer", [False, True])
def test_contiguous(gpu, integer):
    E, K, N = 8, 512, 256
    rng = np.random.default_rng(20 + integer)
    wl = inputs.make_contiguous("c", 3, E, 0, K, N // 2,
                                counts=[130, 0, 7, 128, 1, 40, 70, 100], weights=False)
    m_idx = wl["m_indices"]
    w, s = weights(rng, E, N, K, integer)
    a = bf16_small_ints(rng, (m_idx.size, K)) if integer else wl["a"]
    a_poison = a.copy()
    a_poison[m_idx < 0] = 0x7FC0                             # padding rows are never read
    for override in (None, {"kernel": 1, "block_m": 16, "block_n": 64, "waves_k": 4},
                     {"kernel": 1, "block_m": 32, "block_n": 64, "waves_k": 2},
                     {"kernel": 1, "block_m": 64, "block_n": 128, "waves_k": 1},
                     {"kernel": qma.KERNEL_LARGE_M, "split_k": 2},
                     {"kernel": qma.KERNEL_LARGE_M, "split_k": 1}):
        got = contiguous(a_poison, m_idx, w, s, override)
        ref = O.grouped_contiguous(a, m_idx, w, s)
        valid = m_idx >= 0
        if integer:
            assert np.array_equal(got[valid], rne(ref[valid]))
        else:
            assert_per_expert(got, np.where(valid[:, None], ref, np.nan), m_idx, "contiguous")
        assert np.all(got[~valid] == SENT)


@pytest.mark.parametrize("integer", [False, True])
def test_masked(gpu, integer):
    E, Mb, K, N = 6, 64, 512, 256
    rng = np.random.default_rng(30 + integer)
    masked_m = np.array([32, 0, 64, 1, 17, 33], np.int32)
    w, s = weights(rng, E, N, K, integer)
    a = bf16_small_ints(rng, (E, Mb, K)) if integer else inputs.bf16_normal(rng, (E, Mb, K))
    a_poison = a.copy()
    for e in range(E):
        a_poison[e, masked_m[e]:] = 0x7FC0                   # rows past masked_m unread
    for expected in (32, 16, 64):
        got = masked(a_poison, masked_m, expected, w, s)
        ref = O.grouped_masked(a, masked_m, w, s)
        row_e = np.array([[e if r < masked_m[e] else -1 for r in range(Mb)] for e in range(E)])
        valid = row_e >= 0
        if integer:
            assert np.array_equal(got[valid], rne(ref[valid]))
        else:
            assert_per_expert(got.reshape(E * Mb, N), ref.reshape(E * Mb, N),
                              row_e.reshape(-1), f"masked expected={expected}")
        assert np.all(got[~valid] == SENT)


def test_indexed_equals_contiguous_on_same_rows(gpu):
    # The same rows through the indexed and the contiguous routing give the
    # same bits when the same kernel runs them (the per-element arithmetic
    # does not depend on where a row sits in its tile).
    E, K, N = 4, 512, 256
    rng = np.random.default_rng(40)
    counts = [20, 3, 0, 45]
    wl = inputs.make_contiguous("c", 4, E, 0, K, N // 2, counts=counts, weights=False)
    m_idx = wl["m_indices"]
    w, s = weights(rng, E, N, K)
    ids = np.where(m_idx >= 0, m_idx, -1).astype(np.int32)[:, None]
    valid = m_idx >= 0
    small = {"kernel": 1, "block_m": 16, "block_n": 64, "waves_k": 4, "split_k": 1}
    got_c = contiguous(wl["a"], m_idx, w, s, small)
    got_i, _ = indexed(wl["a"], 1, ids, w, s, force_bm=16, override=small)
    assert_per_expert(got_c, O.grouped_contiguous(wl["a"], m_idx, w, s), m_idx)
    assert np.array_equal(got_c[valid], got_i[valid])
    got_cl = contiguous(wl["a"], m_idx, w, s, {"split_k": 1})          # large-M
    got_il, pl = indexed(wl["a"], 1, ids, w, s, force_bm=128, override={"split_k": 1})
    assert pl.kernel in qma.LARGE_M_KERNELS
    assert_per_expert(got_cl, O.grouped_contiguous(wl["a"], m_idx, w, s), m_idx)
    assert np.array_equal(got_cl[valid], got_il[valid])


LARGE_SHAPES = [  # (E, T, topk, K, N): >= 80 rows per expert
    (3, 300, 1, 512, 512),
    (2, 200, 2, 1024, 256),
    (4, 130, 3, 256, 768),
]


# expert row counts on both sides of every 32-row group boundary of a 128-row
# tile: the large-M kernel computes only the groups that hold tokens, so a
# tile ending an expert's rows runs with 1, 2, 3 or 4 groups
HALF_TILE_COUNTS = [1, 31, 32, 33, 63, 64, 65, 95, 96, 97, 127, 128, 129, 191, 192, 193,
                    0, 256, 287]


# the two large-M kernels: (kernel, split_k)
LM_VARIANTS = [(qma.KERNEL_LARGE_M, 1), (qma.KERNEL_LARGE_M, 2), (qma.KERNEL_LARGE_M_PC, 1)]
LM_IDS = ["large_m", "large_m_split2", "large_m_pc"]


@pytest.mark.parametrize("kernel,split", LM_VARIANTS, ids=LM_IDS)
def test_large_m_half_tiles_bitwise(gpu, kernel, split):
    E, K, N = len(HALF_TILE_COUNTS), 512, 256
    rng = np.random.default_rng(70 + split)
    w, s = weights(rng, E, N, K, integer=True)
    ids = np.repeat(np.arange(E, dtype=np.int32), HALF_TILE_COUNTS)
    ids = rng.permutation(ids)[:, None]
    a = bf16_small_ints(rng, (ids.shape[0], K))
    got, plan = indexed(a, 1, ids, w, s, force_bm=128,
                        override={"kernel": kernel, "split_k": split})
    assert plan.kernel == kernel and plan.split_k == split
    ref = O.moe_gemm_by_slot(a, 1, ids, w, s)
    assert np.array_equal(got, rne(ref))


@pytest.mark.parametrize("kernel", [qma.KERNEL_LARGE_M, qma.KERNEL_LARGE_M_PC],
                         ids=["large_m", "large_m_pc"])
def test_large_m_several_rounds_per_xcd_bitwise(gpu, kernel):
    # 45 tiles dealt to the 8 XCDs (5 or 6 each) x 16 column blocks: each
    # XCD's list spans more than one round of its workgroup slots (several
    # items per persistent workgroup), and the ragged experts' last tiles are
    # partly filled
    K, N = 256, 4096
    counts = [2200, 1300, 900, 700, 33, 3]
    E = len(counts)
    rng = np.random.default_rng(91)
    w, s = weights(rng, E, N, K, integer=True)
    ids = rng.permutation(np.repeat(np.arange(E, dtype=np.int32), counts))[:, None]
    a = bf16_small_ints(rng, (ids.shape[0], K))
    got, plan = indexed(a, 1, ids, w, s, force_bm=128, override={"split_k": 1, "kernel": kernel})
    assert plan.kernel == kernel and plan.block_n == 256
    ref = O.moe_gemm_by_slot(a, 1, ids, w, s)
    assert np.array_equal(got, rne(ref))


@pytest.mark.parametrize("kernel,split", LM_VARIANTS, ids=LM_IDS)
def test_large_m_masked_half_tiles_bitwise(gpu, kernel, split):
    E, Mb, K, N = 11, 256, 256, 256
    rng = np.random.default_rng(80 + split)
    masked_m = np.array([0, 1, 31, 33, 64, 65, 96, 97, 129, 161, 256], np.int32)
    w, s = weights(rng, E, N, K, integer=True)
    a = bf16_small_ints(rng, (E, Mb, K))
    large = {"kernel": kernel, "block_m": 128, "block_n": 256, "waves_k": 1,
             "split_k": split}
    got = masked(a, masked_m, 128, w, s, large)
    ref = O.grouped_masked(a, masked_m, w, s)
    for e in range(E):
        m = masked_m[e]
        assert np.array_equal(got[e, :m], rne(ref[e, :m])), e
        assert np.all(got[e, m:] == SENT), e


@pytest.mark.parametrize("shape", LARGE_SHAPES)
def test_large_m_integer_exact_bitwise(gpu, shape):
    E, T, topk, K, N = shape
    rng = np.random.default_rng(50 + E)
    w, s = weights(rng, E, N, K, integer=True)
    a = bf16_small_ints(rng, (T, K))
    ids = rng.integers(-1, E, (T, topk)).astype(np.int32)
    planned, plan = indexed(a, topk, ids, w, s)
    assert plan.kernel == qma.KERNEL_LARGE_M and plan.block_m == 128
    got, _ = indexed(a, topk, ids, w, s,
                     override={"kernel": qma.KERNEL_LARGE_M_PC, "split_k": 1})
    ref = O.moe_gemm_by_slot(a, topk, ids, w, s)
    valid = slot_experts(ids, E) >= 0
    assert np.array_equal(got[valid], rne(ref[valid]))
    assert np.all(got[~valid] == SENT)
    assert np.array_equal(planned, got)
    split, _ = indexed(a, topk, ids, w, s, override={"split_k": 2, "kernel": qma.KERNEL_LARGE_M})
    assert np.array_equal(split, got)
    one, _ = indexed(a, topk, ids, w, s, override={"kernel": qma.KERNEL_LARGE_M, "split_k": 1})
    assert np.array_equal(one, got)


@pytest.mark.parametrize("shape", LARGE_SHAPES)
def test_large_m_random_within_tolerance(gpu, shape):
    E, T, topk, K, N = shape
    rng = np.random.default_rng(60 + E)
    w, s = weights(rng, E, N, K)
    a = inputs.bf16_normal(rng, (T, K))
    ids = rng.integers(0, E, (T, topk)).astype(np.int32)
    tw = rng.random(T * topk).astype(np.float32)
    got, plan = indexed(a, topk, ids, w, s, topk_w=tw,
                        override={"kernel": qma.KERNEL_LARGE_M_PC, "split_k": 1})
    ref = O.moe_gemm_by_slot(a, topk, ids, w, s, topk_weights=tw)
    assert_per_expert(got, ref, slot_experts(ids, E), f"large-M {shape}")
    # the two large-M kernels sum the same products in the same K order
    old, _ = indexed(a, topk, ids, w, s, topk_w=tw,
                     override={"kernel": qma.KERNEL_LARGE_M, "split_k": 1})
    assert np.array_equal(old, got)


def test_large_m_nan_poisoned_padding(gpu):
    E, T, topk, K, N = 4, 300, 1, 512, 256
    rng = np.random.default_rng(70)
    w, s = weights(rng, E, N, K)
    a = inputs.bf16_normal(rng, (T, K))
    ids = rng.integers(0, 3, (T, topk)).astype(np.int32)   # expert 3: no tokens
    ids[:7] = -1                                             # rows not on this rank
    s_p = s.copy(); s_p[3] = 0x7FC0
    a_p = a.copy(); a_p[:7] = 0x7FC0
    got, plan = indexed(a_p, topk, ids, w, s_p, force_bm=128)
    assert plan.kernel in qma.LARGE_M_KERNELS
    assert_per_expert(got, O.moe_gemm_by_slot(a, topk, ids, w, s), slot_experts(ids, E))


# ---- the chained layer and graph capture ---------------------------------

def _tiny_moe(seed=0):
    wl = inputs.make("tiny", seed=seed)
    w13 = ExpertWeights(wl["w13"], wl["s13"])
    w2 = ExpertWeights(wl["w2"], wl["s2"])
    moe = IndexedMoE(w13, w2, wl.T, wl.topk)
    return wl, moe


def test_tiny_layer_chain(gpu):
    wl, moe = _tiny_moe()
    a = to_device(wl["a"])
    ids = to_device(wl["topk_ids"])
    moe.forward(a, ids)
    torch.cuda.synchronize()
    se = slot_experts(wl["topk_ids"], wl.E)
    c1 = to_host(moe.c1, bf16=True)
    h = to_host(moe.h, bf16=True)
    c2 = to_host(moe.c2, bf16=True)
    assert_per_expert(c1, O.moe_gemm_by_slot(wl["a"], wl.topk, wl["topk_ids"], wl["w13"],
                                             wl["s13"]), se, "gate_up")
    assert_per_expert(c2, O.moe_gemm_by_slot(h, 1, wl["topk_ids"], wl["w2"], wl["s2"]), se,
                      "down (GPU's own activation as input)")
    # fully chained: the oracle rounds C1 and H to bf16 where the GPU does
    c1_ref = rne(O.moe_gemm_by_slot(wl["a"], wl.topk, wl["topk_ids"], wl["w13"], wl["s13"]))
    h_ref = rne(O.silu_and_mul(c1_ref))
    assert_per_expert(c2, O.moe_gemm_by_slot(h_ref, 1, wl["topk_ids"], wl["w2"], wl["s2"]),
                      se, "down (chained)")


def test_graph_capture_replays_match_eager(gpu):
    wl, moe = _tiny_moe(seed=1)
    a = to_device(wl["a"])
    ids = to_device(wl["topk_ids"])
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        moe.forward(a, ids)                      # warm up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    eager = to_host(moe.c2, bf16=True).copy()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe.forward(a, ids)
    for i in range(4):
        moe.c2.fill_(0)
        moe.routing.sorted_ids.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(to_host(moe.c2, bf16=True), eager), f"replay {i}"


def test_graph_capture_fused_gang(gpu):
    # the default decode step's pieces in one graph: gate_up with the
    # activation fused and both GEMMs on the gang schedule (dynamic LDS,
    # persistent groups), replayed against the eager result
    wl = inputs.make("tiny", seed=3)
    moe = IndexedMoE(ExpertWeights(wl["w13"], wl["s13"], flags=qma.LAYER_FUSE_SILU_MUL),
                     ExpertWeights(wl["w2"], wl["s2"]), wl.T, wl.topk)
    assert moe.set_schedule(qma.SCHEDULE_GANG) == (True, True)
    a = to_device(wl["a"])
    ids = to_device(wl["topk_ids"])
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        moe.forward(a, ids)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    eager = to_host(moe.c2, bf16=True).copy()
    h_eager = to_host(moe.h, bf16=True).copy()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe.forward(a, ids)
    for i in range(4):
        moe.c2.fill_(0)
        moe.h.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(to_host(moe.h, bf16=True), h_eager), f"replay {i} h"
        assert np.array_equal(to_host(moe.c2, bf16=True), eager), f"replay {i}"


def test_graph_capture_large_m_split_k(gpu):
    # the large-M kernel with split-K (fp32 partials in the workspace, then
    # the reduce kernel) for both projections, captured and replayed
    E, T, K, I = 3, 300, 512, 256
    rng = np.random.default_rng(77)
    w13, s13 = weights(rng, E, 2 * I, K)
    w2, s2 = weights(rng, E, K, I)
    moe = IndexedMoE(ExpertWeights(w13, s13), ExpertWeights(w2, s2), T, 1, force_block_m=128)
    assert moe.plan13.kernel in qma.LARGE_M_KERNELS and moe.plan2.kernel in qma.LARGE_M_KERNELS
    moe.plan13.kernel = moe.plan2.kernel = qma.KERNEL_LARGE_M
    moe.plan13.split_k = 2
    moe.plan2.split_k = 2
    moe.ws13 = workspace_for(moe.plan13)
    moe.ws2 = workspace_for(moe.plan2)
    a = to_device(inputs.bf16_normal(rng, (T, K)))
    ids = to_device(rng.integers(0, E, (T, 1)).astype(np.int32))
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        moe.forward(a, ids)
    torch.cuda.current_stream().wait_stream(st)
    torch.cuda.synchronize()
    eager = to_host(moe.c2, bf16=True).copy()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe.forward(a, ids)
    for i in range(3):
        moe.c2.fill_(0)
        moe.c1.fill_(0)
        moe.ws13.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(to_host(moe.c2, bf16=True), eager), f"replay {i}"


@pytest.mark.parametrize("kind", ["contiguous", "masked", "masked_dynamic"])
def test_graph_capture_grouped(gpu, kind):
    # grouped paths captured and replayed; the masked replay after new
    # device-side row counts must match an eager run with those counts
    from quantized_moe_align_amd.moe import GroupedMoE
    E, K, I = 4, 256, 128
    rng = np.random.default_rng(88)
    path = qma.PATH_GROUPED_CONTIGUOUS if kind == "contiguous" else qma.PATH_GROUPED_MASKED
    w13, s13 = weights(rng, E, 2 * I, K)
    w2, s2 = weights(rng, E, K, I)
    W13, W2 = ExpertWeights(w13, s13, path), ExpertWeights(w2, s2, path)
    if kind == "contiguous":
        m_idx = np.repeat(np.arange(E, dtype=np.int32), 128)
        m_idx[100:128] = -1
        moe = GroupedMoE(W13, W2, m_idx.size)
        a = to_device(inputs.bf16_normal(rng, (m_idx.size, K)))
        index = to_device(m_idx)
        counts2 = None
    else:
        moe = GroupedMoE(W13, W2, 64, 32)
        if kind == "masked_dynamic":
            assert moe.set_schedule(qma.SCHEDULE_DYNAMIC) == (True, True)
        a = to_device(inputs.bf16_normal(rng, (E, 64, K)))
        index = to_device(np.array([32, 7, 0, 64], np.int32))
        counts2 = np.array([5, 64, 33, 0], np.int32)
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        moe.forward(a, index)
    torch.cuda.current_stream().wait_stream(st)
    torch.cuda.synchronize()
    eager = to_host(moe.c2, bf16=True).copy()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe.forward(a, index)
    for i in range(3):
        moe.c2.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = to_host(moe.c2, bf16=True)
        if counts2 is None:                     # padding rows are never written
            valid = m_idx >= 0
            assert np.array_equal(got[valid], eager[valid]), f"replay {i}"
        else:
            rows = to_host(index)
            for e in range(E):
                assert np.array_equal(got.reshape(E, 64, K)[e, :rows[e]],
                                      eager.reshape(E, 64, K)[e, :rows[e]]), (i, e)
    if counts2 is not None:
        index.copy_(torch.from_numpy(counts2))
        moe.c2.fill_(0)
        moe.forward(a, index)
        torch.cuda.synchronize()
        eager2 = to_host(moe.c2, bf16=True).copy()
        moe.c2.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = to_host(moe.c2, bf16=True).reshape(E, 64, K)
        for e in range(E):
            assert np.array_equal(got[e, :counts2[e]],
                                  eager2.reshape(E, 64, K)[e, :counts2[e]]), e


# Streaming small-M (one workgroup walks several column blocks of its
# expert): (E, T, topk, K, N, block_n, n_stream). 7 or 14 column blocks, so
# some streams end on a partial group.
STREAM_CASES = [
    (5, 40, 2, 256, 1792, 256, 3),
    (5, 40, 2, 256, 1792, 256, 7),
    (3, 30, 1, 128, 1792, 128, 4),
    (4, 24, 3, 384, 512, 128, 2),
]


def _stream_override(block_n, n_stream):
    return {"kernel": qma.KERNEL_SMALL_M, "block_m": 16, "block_n": block_n, "waves_k": 1,
            "split_k": 1, "n_stream": n_stream}


@pytest.mark.parametrize("case", STREAM_CASES)
def test_stream_integer_exact_bitwise(gpu, case):
    E, T, topk, K, N, bn, ns = case
    rng = np.random.default_rng(80 + ns)
    w, s = weights(rng, E, N, K, integer=True)
    a = bf16_small_ints(rng, (T, K))
    ids = rng.integers(-1, E, (T, topk)).astype(np.int32)
    got, plan = indexed(a, topk, ids, w, s, force_bm=16, override=_stream_override(bn, ns))
    assert plan.n_stream == ns
    ref = O.moe_gemm_by_slot(a, topk, ids, w, s)
    valid = slot_experts(ids, E) >= 0
    assert np.array_equal(got[valid], rne(ref[valid]))
    assert np.all(got[~valid] == SENT)
    one, _ = indexed(a, topk, ids, w, s, force_bm=16, override=_stream_override(bn, 1))
    assert np.array_equal(one, got)


def test_stream_random_topk_weights_and_grouped(gpu):
    E, T, topk, K, N = 6, 50, 2, 256, 1024
    rng = np.random.default_rng(90)
    w, s = weights(rng, E, N, K)
    a = inputs.bf16_normal(rng, (T, K))
    ids = rng.integers(0, E, (T, topk)).astype(np.int32)
    tw = rng.random(T * topk).astype(np.float32)
    got, _ = indexed(a, topk, ids, w, s, force_bm=16, topk_w=tw, override=_stream_override(256, 3))
    ref = O.moe_gemm_by_slot(a, topk, ids, w, s, topk_weights=tw)
    assert_per_expert(got, ref, slot_experts(ids, E), "stream indexed")
    # contiguous and masked routing through the streaming kernel
    wl = inputs.make_contiguous("c", 5, E, 0, K, N // 2, counts=[20, 0, 7, 16, 1, 33],
                                weights=False)
    m_idx = wl["m_indices"]
    got_c = contiguous(wl["a"], m_idx, w, s, _stream_override(256, 2))
    assert_per_expert(got_c, O.grouped_contiguous(wl["a"], m_idx, w, s), m_idx, "stream contiguous")
    Mb = 32
    masked_m = np.array([16, 0, 32, 1, 9, 17], np.int32)
    am = inputs.bf16_normal(rng, (E, Mb, K))
    got_m = masked(am, masked_m, 16, w, s, _stream_override(128, 4))
    ref_m = O.grouped_masked(am, masked_m, w, s)
    row_e = np.array([[e if r < masked_m[e] else -1 for r in range(Mb)] for e in range(E)])
    assert_per_expert(got_m.reshape(E * Mb, N), ref_m.reshape(E * Mb, N), row_e.reshape(-1),
                      "stream masked")
    assert np.all(got_m[row_e < 0] == SENT)


# Dynamic schedule (a persistent grid taking (tile, column block) items from
# a work counter) against the semi-static grid: same kernel body, so the
# outputs must agree bit for bit, and with integer-exact inputs both equal
# the oracle.
@pytest.mark.parametrize("bm,bn", [(16, 128), (16, 256), (32, 256), (32, 128)])
def test_dynamic_schedule_matches_semi_static(gpu, bm, bn):
    E, T, topk, K, N = 7, 90, 2, 512, 768 if bn == 256 else 640
    if N % bn:
        N = bn * 3
    rng = np.random.default_rng(100 + bm + bn)
    w, s = weights(rng, E, N, K, integer=True)
    a = bf16_small_ints(rng, (T, K))
    ids = rng.integers(-1, E, (T, topk)).astype(np.int32)
    ov = {"kernel": qma.KERNEL_SMALL_M, "block_m": bm, "block_n": bn, "waves_k": 1,
          "split_k": 1, "n_stream": 1}
    static, _ = indexed(a, topk, ids, w, s, force_bm=bm, override=ov)
    dyn, plan = indexed(a, topk, ids, w, s, force_bm=bm,
                        override=dict(ov, schedule=qma.SCHEDULE_DYNAMIC))
    assert plan.schedule == qma.SCHEDULE_DYNAMIC
    assert np.array_equal(dyn, static)
    ref = O.moe_gemm_by_slot(a, topk, ids, w, s)
    valid = slot_experts(ids, E) >= 0
    assert np.array_equal(dyn[valid], rne(ref[valid]))
    assert np.all(dyn[~valid] == SENT)


def test_dynamic_schedule_grouped(gpu):
    E, K, N = 5, 512, 512
    rng = np.random.default_rng(110)
    w, s = weights(rng, E, N, K)
    wl = inputs.make_contiguous("c", 6, E, 0, K, N // 2, counts=[20, 0, 7, 16, 33],
                                weights=False)
    m_idx = wl["m_indices"]
    ov = {"kernel": qma.KERNEL_SMALL_M, "block_m": 16, "block_n": 128, "waves_k": 1,
          "split_k": 1, "n_stream": 1}
    got = contiguous(wl["a"], m_idx, w, s, dict(ov, schedule=qma.SCHEDULE_DYNAMIC))
    assert np.array_equal(got, contiguous(wl["a"], m_idx, w, s, ov))
    Mb = 64
    masked_m = np.array([32, 0, 64, 1, 17], np.int32)
    am = inputs.bf16_normal(rng, (E, Mb, K))
    ovm = dict(ov, block_m=32, block_n=256)
    got_m = masked(am, masked_m, 32, w, s, dict(ovm, schedule=qma.SCHEDULE_DYNAMIC))
    assert np.array_equal(got_m, masked(am, masked_m, 32, w, s, ovm))
    ref_m = O.grouped_masked(am, masked_m, w, s)
    row_e = np.array([[e if r < masked_m[e] else -1 for r in range(Mb)] for e in range(E)])
    assert_per_expert(got_m.reshape(E * Mb, N), ref_m.reshape(E * Mb, N), row_e.reshape(-1),
                      "dynamic masked")


# Gang schedule (one workgroup of three lock-step groups per CU, each group on
# its own item, looping over rounds of items) against the semi-static grid:
# the same kernel body, so bit for bit the same outputs, and with
# integer-exact inputs both equal the oracle. The shapes give more items than
# one round of 3 x 256 groups (so groups loop), ragged expert counts, slots
# routed off the rank, and split-K with its reduction.
GANG_CASES = [(16, 128, 1), (16, 256, 1), (32, 256, 1), (32, 128, 1), (64, 128, 1),
              (16, 256, 2), (32, 128, 3), (64, 128, 2)]


@pytest.mark.parametrize("bm,bn,split", GANG_CASES)
def test_gang_schedule_matches_semi_static(gpu, bm, bn, split):
    E, T, topk, K, N = 37, 700, 2, 512, 2048
    rng = np.random.default_rng(300 + bm + bn + split)
    w, s = weights(rng, E, N, K, integer=True)
    a = bf16_small_ints(rng, (T, K))
    ids = rng.integers(-1, E, (T, topk)).astype(np.int32)
    ids[ids == 5] = 6                             # one expert with no rows
    ov = {"kernel": qma.KERNEL_SMALL_M, "block_m": bm, "block_n": bn, "waves_k": 1,
          "split_k": split, "n_stream": 1}
    static, _ = indexed(a, topk, ids, w, s, force_bm=bm, override=ov)
    gang, plan = indexed(a, topk, ids, w, s, force_bm=bm, junk_tail=(bm == 32),
                         override=dict(ov, schedule=qma.SCHEDULE_GANG))
    assert plan.schedule == qma.SCHEDULE_GANG
    assert np.array_equal(gang, static)
    ref = O.moe_gemm_by_slot(a, topk, ids, w, s)
    valid = slot_experts(ids, E) >= 0
    assert np.array_equal(gang[valid], rne(ref[valid]))
    assert np.all(gang[~valid] == SENT)


def test_gang_schedule_grouped(gpu):
    E, K, N = 23, 512, 1536
    rng = np.random.default_rng(320)
    w, s = weights(rng, E, N, K)
    counts = [int(c) for c in rng.integers(0, 90, E)]
    counts[3] = 0
    wl = inputs.make_contiguous("c", 6, E, 0, K, N // 2, counts=counts, weights=False)
    m_idx = wl["m_indices"]
    ov = {"kernel": qma.KERNEL_SMALL_M, "block_m": 16, "block_n": 128, "waves_k": 1,
          "split_k": 1, "n_stream": 1}
    got = contiguous(wl["a"], m_idx, w, s, dict(ov, schedule=qma.SCHEDULE_GANG))
    assert np.array_equal(got, contiguous(wl["a"], m_idx, w, s, ov))
    assert_per_expert(got, O.grouped_contiguous(wl["a"], m_idx, w, s), m_idx, "gang contiguous")
    Mb = 64
    masked_m = rng.integers(0, Mb + 1, E).astype(np.int32)
    masked_m[:3] = (0, 1, Mb)
    am = inputs.bf16_normal(rng, (E, Mb, K))
    for ovm in (dict(ov, block_m=32, block_n=256), dict(ov, block_m=64, split_k=2)):
        got_m = masked(am, masked_m, 32, w, s, dict(ovm, schedule=qma.SCHEDULE_GANG))
        assert np.array_equal(got_m, masked(am, masked_m, 32, w, s, ovm))
        ref_m = O.grouped_masked(am, masked_m, w, s)
        row_e = np.array([[e if r < masked_m[e] else -1 for r in range(Mb)] for e in range(E)])
        assert_per_expert(got_m.reshape(E * Mb, N), ref_m.reshape(E * Mb, N),
                          row_e.reshape(-1), "gang masked")
        assert np.all(got_m[row_e < 0] == SENT)


# Stream-K gang schedule (one workgroup per CU holding a contiguous share of
# the items, its groups splitting the share's K chunks evenly, pieces of an
# item cut in K added in LDS in K order): with integer-exact inputs every
# partial sum is exact, so the output equals the semi-static grid's and the
# oracle's bit for bit, and with the activation fused the activation kernel
# on that output. The shapes give many items per CU with ragged expert
# counts and slots routed off the rank, fewer items than CUs (items cut
# over three or four groups), an EP8-down-like share, and a K of 9 chunks.
SK_CASES = [  # (E, T, topk, K, N, block_m, block_n)
    (37, 700, 2, 1024, 2048, 16, 128),
    (37, 700, 2, 1024, 2048, 16, 256),
    (37, 400, 2, 1024, 2048, 32, 128),
    (37, 400, 2, 1024, 2048, 32, 256),
    (5, 60, 2, 2048, 512, 16, 128),
    (48, 280, 2, 2048, 7168, 16, 128),
    (3, 9, 1, 1152, 256, 16, 128),
]


@pytest.mark.parametrize("case", SK_CASES)
def test_stream_k_matches_semi_static(gpu, case):
    E, T, topk, K, N, bm, bn = case
    print(f"stream-K case {case}", flush=True)
    rng = np.random.default_rng(400 + sum(case))
    w, s = weights(rng, E, N, K, integer=True)
    a = bf16_small_ints(rng, (T, K))
    ids = rng.integers(-1, E, (T, topk)).astype(np.int32)
    if E > 2:
        ids[ids == 2] = 1                            # one expert with no rows
    ov = {"kernel": qma.KERNEL_SMALL_M, "block_m": bm, "block_n": bn, "waves_k": 1,
          "split_k": 1, "n_stream": 1}
    static, _ = indexed(a, topk, ids, w, s, force_bm=bm, override=ov)
    got, plan = indexed(a, topk, ids, w, s, force_bm=bm, junk_tail=True,
                        override=dict(ov, schedule=qma.SCHEDULE_STREAM_K))
    assert plan.schedule == qma.SCHEDULE_STREAM_K
    assert np.array_equal(got, static)
    ref = O.moe_gemm_by_slot(a, topk, ids, w, s)
    valid = slot_experts(ids, E) >= 0
    assert np.array_equal(got[valid], rne(ref[valid]))
    assert np.all(got[~valid] == SENT)
    h, _ = indexed(a, topk, ids, w, s, force_bm=bm, flags=qma.LAYER_FUSE_SILU_MUL,
                   override=dict(ov, schedule=qma.SCHEDULE_STREAM_K))
    h_ref = silu_of(static)
    assert np.array_equal(h[valid], h_ref[valid])
    assert np.all(h[~valid] == SENT)


def test_stream_k_random_within_tolerance(gpu):
    # random inputs: the cut points change only the fp32 summation order
    E, T, topk, K, N = 24, 300, 2, 2048, 1536
    rng = np.random.default_rng(420)
    w, s = weights(rng, E, N, K)
    a = inputs.bf16_normal(rng, (T, K))
    ids = rng.integers(0, E, (T, topk)).astype(np.int32)
    tw = rng.random((T, topk)).astype(np.float32)
    ov = {"kernel": qma.KERNEL_SMALL_M, "block_m": 16, "block_n": 128, "waves_k": 1,
          "split_k": 1, "n_stream": 1, "schedule": qma.SCHEDULE_STREAM_K}
    got, _ = indexed(a, topk, ids, w, s, force_bm=16, override=ov, topk_w=tw)
    ref = O.moe_gemm_by_slot(a, topk, ids, w, s, topk_weights=tw)
    assert_per_expert(got, ref, slot_experts(ids, E), "stream-K random")


def test_stream_k_with_nothing_routed(gpu):
    E, T, topk, K, N = 6, 50, 2, 1024, 512
    rng = np.random.default_rng(430)
    w, s = weights(rng, E, N, K)
    a = inputs.bf16_normal(rng, (T, K))
    ids = np.full((T, topk), -1, np.int32)
    got, plan = indexed(a, topk, ids, w, s, force_bm=16,
                        override={"block_n": 128, "waves_k": 1, "split_k": 1, "n_stream": 1,
                                  "schedule": qma.SCHEDULE_STREAM_K})
    assert plan.schedule == qma.SCHEDULE_STREAM_K
    assert np.all(got == SENT)


# Few token tiles are folded into column-block groups dealt to the XCDs
# separately (the fold follows the plan's tile estimate, est_tiles / column
# blocks). Folding moves work between workgroups only: every fold gives the
# unfolded output bit for bit, on every kernel family that deals tiles that
# way, and the oracle with integer-exact inputs.
FOLD_PLANS = [
    {"block_n": 128, "waves_k": 1, "split_k": 1, "n_stream": 1},
    {"block_n": 128, "waves_k": 1, "split_k": 1, "n_stream": 1, "schedule": qma.SCHEDULE_GANG},
    {"block_n": 256, "waves_k": 1, "split_k": 2, "n_stream": 1},
    {"block_n": 64, "waves_k": 4, "split_k": 1, "n_stream": 1},
    {"block_n": 128, "waves_k": 2, "split_k": 1, "n_stream": 1},
    {"block_n": 128, "waves_k": 1, "split_k": 1, "n_stream": 2},
]


@pytest.mark.parametrize("plan_i", range(len(FOLD_PLANS)))
def test_xcd_fold_bitwise(gpu, plan_i):
    E, T, topk, N = 5, 60, 2, 2048
    ov = FOLD_PLANS[plan_i]
    K = 256 if ov["n_stream"] > 1 else 1024
    rng = np.random.default_rng(360 + plan_i)
    w, s = weights(rng, E, N, K, integer=True)
    a = bf16_small_ints(rng, (T, K))
    ids = rng.integers(-1, E, (T, topk)).astype(np.int32)
    nb = N // ov["block_n"]
    outs = []
    for tiles_est in (1 << 12, 3, 12, 1):        # fold 1, then 8, 2 and 8
        got, plan = indexed(a, topk, ids, w, s, force_bm=16,
                            override=dict(ov, kernel=qma.KERNEL_SMALL_M, block_m=16,
                                          est_tiles=tiles_est * nb))
        outs.append(got)
    for got in outs[1:]:
        assert np.array_equal(got, outs[0])
    ref = O.moe_gemm_by_slot(a, topk, ids, w, s)
    valid = slot_experts(ids, E) >= 0
    assert np.array_equal(outs[0][valid], rne(ref[valid]))
    assert np.all(outs[0][~valid] == SENT)


def test_gang_schedule_with_nothing_routed(gpu):
    E, T, topk, K, N = 6, 50, 2, 1024, 512
    rng = np.random.default_rng(330)
    w, s = weights(rng, E, N, K)
    a = inputs.bf16_normal(rng, (T, K))
    ids = np.full((T, topk), -1, np.int32)
    got, plan = indexed(a, topk, ids, w, s, force_bm=16,
                        override={"block_n": 128, "waves_k": 1, "split_k": 1, "n_stream": 1,
                                  "schedule": qma.SCHEDULE_GANG})
    assert plan.schedule == qma.SCHEDULE_GANG
    assert np.all(got == SENT)


# Gate_up with the activation fused: h = silu(gate) * up from the GEMM's own
# epilogue (or split-K reduction) equals the activation kernel applied to the
# unfused output, bit for bit, on every kernel family a gate_up plan can take.
def silu_of(c_bits):
    """The library's activation kernel on an unfused gate_up output."""
    R, N = c_bits.shape
    x = to_device(c_bits)
    h = torch.empty((R, N // 2), dtype=torch.int16, device="cuda")
    qma.qma_silu_and_mul(x, h, R, N // 2)
    torch.cuda.synchronize()
    return to_host(h, bf16=True)


FUSED_PLANS = [
    ({"block_m": 16, "block_n": 128, "waves_k": 1}, 1024),
    ({"block_m": 16, "block_n": 256, "waves_k": 1, "schedule": qma.SCHEDULE_GANG}, 1024),
    ({"block_m": 32, "block_n": 256, "waves_k": 1, "schedule": qma.SCHEDULE_DYNAMIC}, 1024),
    ({"block_m": 64, "block_n": 128, "waves_k": 1}, 1024),
    ({"block_m": 16, "block_n": 128, "waves_k": 2}, 1024),
    ({"block_m": 16, "block_n": 64, "waves_k": 4}, 1024),
    ({"block_m": 16, "block_n": 128, "waves_k": 1, "split_k": 3}, 1024),
    ({"block_m": 16, "block_n": 64, "waves_k": 4, "split_k": 2}, 1024),
    ({"block_m": 16, "block_n": 256, "waves_k": 1, "n_stream": 3}, 256),
    ({"kernel": qma.KERNEL_LARGE_M, "block_m": 128, "block_n": 256}, 512),
    ({"kernel": qma.KERNEL_LARGE_M, "block_m": 128, "block_n": 256, "split_k": 2}, 512),
]


@pytest.mark.parametrize("case", range(len(FUSED_PLANS)))
def test_fused_activation_matches_unfused(gpu, case):
    ov, K = FUSED_PLANS[case]
    ov = dict({"kernel": qma.KERNEL_SMALL_M, "split_k": 1, "n_stream": 1}, **ov)
    large = ov["kernel"] == qma.KERNEL_LARGE_M
    E, T, topk, N = 6, 420 if large else 150, 2, 1536
    rng = np.random.default_rng(380 + case)
    w, s = weights(rng, E, N, K)
    a = inputs.bf16_normal(rng, (T, K))
    ids = rng.integers(-1, E, (T, topk)).astype(np.int32)
    tw = rng.random(T * topk).astype(np.float32)
    bm = ov["block_m"]
    plain, _ = indexed(a, topk, ids, w, s, force_bm=bm, override=ov)
    fused, plan = indexed(a, topk, ids, w, s, force_bm=bm, override=ov,
                          flags=qma.LAYER_FUSE_SILU_MUL)
    assert plan.kernel == ov["kernel"] and plan.split_k == ov["split_k"]
    valid = slot_experts(ids, E) >= 0
    ref = silu_of(plain)
    assert np.array_equal(fused[valid], ref[valid])
    assert np.all(fused[~valid] == SENT)
    # and the oracle's activation of the same gate_up output, within one bf16 ulp
    h64 = O.silu_and_mul(plain[valid])
    ulp = np.abs(O.bf16_to_f64(rne(h64)) * 2.0 ** -7) + 2.0 ** -126
    assert np.all(np.abs(O.bf16_to_f64(fused[valid]) - h64) <= ulp)


def test_fused_activation_grouped(gpu):
    E, K, N = 5, 512, 1024
    rng = np.random.default_rng(395)
    w, s = weights(rng, E, N, K)
    wl = inputs.make_contiguous("c", 6, E, 0, K, N // 2, counts=[200, 0, 70, 128, 33],
                                weights=False)
    m_idx = wl["m_indices"]
    got = contiguous(wl["a"], m_idx, w, s, flags=qma.LAYER_FUSE_SILU_MUL)
    ref = silu_of(contiguous(wl["a"], m_idx, w, s))
    assert np.array_equal(got[m_idx >= 0], ref[m_idx >= 0])
    Mb = 64
    masked_m = np.array([32, 0, 64, 1, 17], np.int32)
    am = inputs.bf16_normal(rng, (E, Mb, K))
    got_m = masked(am, masked_m, 32, w, s, flags=qma.LAYER_FUSE_SILU_MUL)
    plain_m = masked(am, masked_m, 32, w, s)
    ref_m = silu_of(plain_m.reshape(E * Mb, N)).reshape(E, Mb, N // 2)
    row_e = np.array([[r < masked_m[e] for r in range(Mb)] for e in range(E)])
    assert np.array_equal(got_m[row_e], ref_m[row_e])
    assert np.all(got_m[~row_e] == SENT)


# ---- degenerate routing: nothing to compute --------------------------------

@pytest.mark.parametrize("force_bm", [16, 32, 64, 128])
def test_indexed_no_routed_slot_writes_nothing(gpu, force_bm):
    # every slot routed off this rank (-1): moe_align pads nothing, every
    # GEMM workgroup exits, and the output keeps its pre-filled pattern
    E, T, topk, K, N = 4, 40, 2, 256, 256
    rng = np.random.default_rng(200 + force_bm)
    w, s = weights(rng, E, N, K)
    a = inputs.bf16_normal(rng, (T, K))
    ids = np.full((T, topk), -1, np.int32)
    got, plan = indexed(a, topk, ids, w, s, force_bm=force_bm)
    assert plan.block_m == force_bm
    assert np.all(got == SENT)


def test_grouped_with_no_valid_rows_writes_nothing(gpu):
    E, K, N = 3, 256, 256
    rng = np.random.default_rng(210)
    w, s = weights(rng, E, N, K)
    m_idx = np.full(2 * 128, -1, np.int32)                 # two padding-only blocks
    a = inputs.bf16_normal(rng, (m_idx.size, K))
    for override in (None, {"kernel": 1, "block_m": 16, "block_n": 64, "waves_k": 4}):
        assert np.all(contiguous(a, m_idx, w, s, override) == SENT)
    a3 = inputs.bf16_normal(rng, (E, 64, K))
    got = masked(a3, np.zeros(E, np.int32), 32, w, s)
    assert np.all(got == SENT)


# ---- pipeline depth: bit-identical output --------------------------------
# The number of K chunks in flight only changes when loads are issued, not
# the order in which each output's products are summed, so every depth must
# give the same bits ([announce] scheduling section and [release] indexed
# techniques: the pipelined main loop keeps the output bit-identical).
DEPTH_PLANS = [  # small-M overrides that reach gemm_small_m_kernel<1, 4, WK, D>
    {"block_n": 128, "waves_k": 2, "split_k": 1},
    {"block_n": 64, "waves_k": 4, "split_k": 1},
    {"block_n": 128, "waves_k": 2, "split_k": 2},
]


@pytest.mark.parametrize("plan_i", range(len(DEPTH_PLANS)))
@pytest.mark.parametrize("integer", [True, False])
def test_pipeline_depth_bit_identical(gpu, plan_i, integer):
    E, T, topk, K, N = 5, 60, 2, 2048, 512
    rng = np.random.default_rng(300 + plan_i + 10 * integer)
    w, s = weights(rng, E, N, K, integer)
    a = bf16_small_ints(rng, (T, K)) if integer else inputs.bf16_normal(rng, (T, K))
    ids = rng.integers(-1, E, (T, topk)).astype(np.int32)
    base = dict(DEPTH_PLANS[plan_i], kernel=qma.KERNEL_SMALL_M, block_m=16, n_stream=1)
    outs = []
    for depth in (256, 384):
        got, plan = indexed(a, topk, ids, w, s, force_bm=16, override=dict(base, k_depth=depth))
        assert plan.k_depth == depth
        outs.append(got)
    assert np.array_equal(outs[0], outs[1])
    ref = O.moe_gemm_by_slot(a, topk, ids, w, s)
    valid = slot_experts(ids, E) >= 0
    if integer:
        assert np.array_equal(outs[0][valid], rne(ref[valid]))
    else:
        assert_per_expert(outs[0], ref, slot_experts(ids, E), "depth")
    assert np.all(outs[0][~valid] == SENT)


# Randomized shapes (seeded): on each, every schedule and layout variant a
# plan can take (the planner's own plan, the gang schedule, folds of the
# column blocks over the XCDs, split-K, the activation fused) agrees bit for
# bit with the semi-static, unsplit, unfused run of the same tile size, and
# that run with the oracle (integer-exact inputs).
def _variant_run(W, plan, a_bits, ids, T, topk, out_cols):
    E, B = W.E, plan.block_m
    cap = qma.qma_align_sizes(T, topk, E, B)[0]
    sorted_ids = torch.empty(cap, dtype=torch.int32, device="cuda")
    expert_ids = torch.empty(-(-cap // B), dtype=torch.int32, device="cuda")
    ntp = torch.empty(1, dtype=torch.int32, device="cuda")
    qma.qma_moe_align(to_device(ids), T, topk, E, B, sorted_ids, expert_ids, ntp, cap)
    R = T * topk
    c = torch.full((R, out_cols), SENT, dtype=torch.int16, device="cuda")
    ws = workspace_for(plan)
    qma.qma_indexed_gemm(W.layer, plan, to_device(a_bits), T, topk, W.packed, sorted_ids,
                         expert_ids, ntp, cap, R, None, c, ws, 0 if ws is None else ws.numel())
    torch.cuda.synchronize()
    return to_host(c, bf16=True)


@pytest.mark.parametrize("case", range(12))
def test_randomized_plan_variants_bitwise(gpu, case):
    rng = np.random.default_rng(900 + case)
    E, topk, T = int(rng.integers(1, 40)), int(rng.integers(1, 4)), int(rng.integers(1, 300))
    K = int(rng.choice([256, 512, 1024, 2048]))
    N = int(rng.choice([256, 512, 768, 1024, 1536, 2048]))
    w, s = weights(rng, E, N, K, integer=True)
    a = bf16_small_ints(rng, (T, K))
    ids = rng.integers(-1, E, (T, topk)).astype(np.int32)
    plain = ExpertWeights(w, s)
    fused = ExpertWeights(w, s, flags=qma.LAYER_FUSE_SILU_MUL)
    base = qma.qma_plan_indexed(plain.layer, T, topk, 0)
    bm = base.block_m
    ref_plan = qma.qma_plan_indexed(plain.layer, T, topk, bm)
    ref_plan.schedule = qma.SCHEDULE_SEMI_STATIC
    if ref_plan.kernel == qma.KERNEL_SMALL_M:
        ref_plan.split_k = 1
    ref = _variant_run(plain, ref_plan, a, ids, T, topk, N)
    valid = slot_experts(ids, E) >= 0
    assert np.array_equal(ref[valid], rne(O.moe_gemm_by_slot(a, topk, ids, w, s)[valid]))
    h_ref = silu_of(ref)
    variants = [{}]
    if base.kernel == qma.KERNEL_SMALL_M:
        nb = N // base.block_n
        variants += [{"est_tiles": nb}, {"est_tiles": 3 * nb}, {"split_k": 2, "n_stream": 1}]
        if base.waves_k == 1 and base.n_stream == 1 and base.block_n in (128, 256) and bm <= 32:
            variants.append({"schedule": qma.SCHEDULE_GANG})
            if K >= 1024:
                variants.append({"schedule": qma.SCHEDULE_STREAM_K})
    for ov in variants:
        for W, want, cols in ((plain, ref, N), (fused, h_ref, N // 2)):
            plan = qma.qma_plan_indexed(W.layer, T, topk, bm)
            for k, v in ov.items():
                setattr(plan, k, v)
            got = _variant_run(W, plan, a, ids, T, topk, cols)
            assert np.array_equal(got[valid], want[valid]), (ov, W.fused, plan.as_dict())
            assert np.all(got[~valid] == SENT), (ov, W.fused)
