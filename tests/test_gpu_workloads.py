"""Full-size workloads through the same calls the benchmark times, checked
against the oracle stage by stage, each stage on the GPU's own input to it
(gate_up, the activation, down), plus a fully chained sample.

* decode-shaped workloads (EP8/EP16/EP32/EP128 decode, the 33..79-row EP8
  share, TP8, masked): every output element of both GEMMs and the activation;
* prefill-shaped workloads (EP8 prefill, its span-matched variant,
  contiguous): every row, and 16 columns of every 256-column block, so that
  every (row tile, expert, column block) workgroup of the launch is checked.

Routing buffers are validated in full."""
import numpy as np
import pytest
import torch

from oracle import qma_oracle as O
from quantized_moe_align_amd import inputs, qma
from quantized_moe_align_amd.moe import ExpertWeights, GroupedMoE, IndexedMoE, to_device, to_host
from gpu_common import assert_per_expert, rne, slot_experts

pytestmark = pytest.mark.gpu

N_CHAIN = 12
PREFILL = {"ep8_prefill", "ep8_prefill_span", "contiguous"}


def _sampled(rng, slot_expert, n_slots):
    valid = np.nonzero(slot_expert >= 0)[0]
    # at least one slot from every expert that has rows, then random ones
    firsts = [valid[slot_expert[valid] == e][0] for e in np.unique(slot_expert[valid])]
    extra = rng.choice(valid, size=min(n_slots, valid.size), replace=False)
    return np.unique(np.concatenate([firsts, extra]))


def _only(slot_expert, slots):
    m = np.full_like(slot_expert, -1)
    m[slots] = slot_expert[slots]
    return m


def _block_cols(rng, N, per_block=16, block=256):
    """per_block random columns from every block of 256 (or the whole of a
    narrower N), sorted."""
    if N <= block:
        return np.arange(N)
    return np.sort(np.concatenate([b + rng.choice(block, per_block, replace=False)
                                   for b in range(0, N, block)]))


def check_stages(a_bits, a_row_div, slot_expert, c1, h, c2, w13, s13, w2, s2, rng, what,
                 full=True):
    N1, N2 = w13.shape[1], w2.shape[1]
    slots = np.nonzero(slot_expert >= 0)[0]
    if full:
        cols1, cols2 = np.arange(N1), np.arange(N2)
    else:
        cols1, cols2 = _block_cols(rng, N1), _block_cols(rng, N2)
    se = _only(slot_expert, slots)
    ref1 = O.moe_gemm_by_slot(a_bits, a_row_div, se, w13, s13, cols=cols1)
    assert_per_expert(c1[slots][:, cols1], ref1[slots], se[slots], f"{what} gate_up")
    # activation on the GPU's own gate_up output, within one bf16 ulp
    ref_h = O.silu_and_mul(c1[slots])
    gh = O.bf16_to_f64(h[slots])
    ulp = np.abs(O.bf16_to_f64(rne(ref_h)) * 2.0 ** -7) + 2.0 ** -126
    assert np.all(np.abs(gh - ref_h) <= ulp), f"{what} silu_and_mul"
    ref2 = O.moe_gemm_by_slot(h, 1, se, w2, s2, cols=cols2)
    assert_per_expert(c2[slots][:, cols2], ref2[slots], se[slots], f"{what} down")
    # chained: oracle gate_up rows rounded to bf16, oracle activation, oracle down
    cs = _sampled(rng, slot_expert, N_CHAIN)[:N_CHAIN]
    sc = _only(slot_expert, cs)
    c1_ref = O.moe_gemm_by_slot(a_bits, a_row_div, sc, w13, s13)
    h_ref = np.zeros(h.shape, np.uint16)
    h_ref[cs] = rne(O.silu_and_mul(rne(c1_ref[cs])))
    ref_chain = O.moe_gemm_by_slot(h_ref, 1, sc, w2, s2, cols=cols2)
    assert_per_expert(c2[cs][:, cols2], ref_chain[cs], sc[cs], f"{what} chained")


@pytest.mark.parametrize("name", ["ep8_decode", "tp8", "ep8_prefill", "ep16_decode", "ep32_decode",
                                  "ep8_prefill_span", "ep8_mid", "ep128_decode"])
def test_indexed_workload(gpu, name):
    wl = inputs.make(name, seed=0)
    rng = np.random.default_rng(1)
    moe = IndexedMoE(ExpertWeights(wl["w13"], wl["s13"]), ExpertWeights(wl["w2"], wl["s2"]),
                     wl.T, wl.topk)
    a = to_device(wl["a"])
    ids = to_device(wl["topk_ids"])
    moe.forward(a, ids)
    torch.cuda.synchronize()
    r = moe.routing
    qma.qma_validate_routing(ids, wl.T, wl.topk, wl.E, r.block_m, r.sorted_ids, r.expert_ids,
                             r.ntp, r.cap)
    c1, h, c2 = (to_host(t, bf16=True) for t in (moe.c1, moe.h, moe.c2))
    check_stages(wl["a"], wl.topk, slot_experts(wl["topk_ids"], wl.E), c1, h, c2, wl["w13"],
                 wl["s13"], wl["w2"], wl["s2"], rng, name, full=name not in PREFILL)


@pytest.mark.parametrize("name", ["contiguous", "masked"])
def test_grouped_workload(gpu, name):
    wl = inputs.make(name, seed=0)
    rng = np.random.default_rng(2)
    path = qma.PATH_GROUPED_CONTIGUOUS if name == "contiguous" else qma.PATH_GROUPED_MASKED
    w13 = ExpertWeights(wl["w13"], wl["s13"], path)
    w2 = ExpertWeights(wl["w2"], wl["s2"], path)
    if name == "contiguous":
        index = wl["m_indices"]
        moe = GroupedMoE(w13, w2, index.size)
        row_e = index.astype(np.int64)
        a_rows = wl["a"]
    else:
        index = wl["masked_m"]
        budget = wl.meta["budget"]
        moe = GroupedMoE(w13, w2, budget, wl.meta["expected_m"])
        row_e = np.array([[e if r < index[e] else -1 for r in range(budget)]
                          for e in range(wl.E)]).reshape(-1)
        a_rows = wl["a"].reshape(-1, wl.K)
    moe.forward(to_device(wl["a"]), to_device(index))
    torch.cuda.synchronize()
    c1, h, c2 = (to_host(t, bf16=True) for t in (moe.c1, moe.h, moe.c2))
    check_stages(a_rows, 1, row_e, c1, h, c2, wl["w13"], wl["s13"], wl["w2"], wl["s2"], rng,
                 name, full=name not in PREFILL)


@pytest.mark.parametrize("name", ["ep8_decode", "tp8", "ep128_decode", "ep32_decode", "ep8_prefill",
                                  "contiguous", "masked"])
def test_fused_activation_full_size(gpu, name):
    """gate_up with the activation fused (the benchmark's default step) gives
    the unfused gate_up + activation kernel's h bit for bit, and the same
    down output, at the workload's full size and with the planner's plans."""
    wl = inputs.make(name, seed=0)
    outs = {}
    for flags in (0, qma.LAYER_FUSE_SILU_MUL):
        if wl.kind == "indexed":
            moe = IndexedMoE(ExpertWeights(wl["w13"], wl["s13"], flags=flags),
                             ExpertWeights(wl["w2"], wl["s2"]), wl.T, wl.topk)
            moe.forward(to_device(wl["a"]), to_device(wl["topk_ids"]))
            valid = slot_experts(wl["topk_ids"], wl.E) >= 0
        else:
            path = (qma.PATH_GROUPED_CONTIGUOUS if wl.kind == "contiguous"
                    else qma.PATH_GROUPED_MASKED)
            w13 = ExpertWeights(wl["w13"], wl["s13"], path, flags=flags)
            w2 = ExpertWeights(wl["w2"], wl["s2"], path)
            if wl.kind == "contiguous":
                index = wl["m_indices"]
                moe = GroupedMoE(w13, w2, index.size)
                valid = index >= 0
            else:
                index = wl["masked_m"]
                budget = wl.meta["budget"]
                moe = GroupedMoE(w13, w2, budget, wl.meta["expected_m"])
                valid = np.array([[r < index[e] for r in range(budget)]
                                  for e in range(wl.E)]).reshape(-1)
            moe.forward(to_device(wl["a"]), to_device(index))
        torch.cuda.synchronize()
        assert moe.fused == bool(flags)
        outs[flags] = (to_host(moe.h, bf16=True)[valid], to_host(moe.c2, bf16=True)[valid])
        del moe
    assert np.array_equal(outs[0][0], outs[qma.LAYER_FUSE_SILU_MUL][0]), f"{name} h"
    assert np.array_equal(outs[0][1], outs[qma.LAYER_FUSE_SILU_MUL][1]), f"{name} down"
