"""qma_indexed_gemm_scratch (the indexed GEMM for callers that cannot
allocate) against qma_indexed_gemm with a caller-allocated workspace, through
the C ABI: two calls in a row per plan family, the second with a smaller
input, each bit-identical to the workspace call (same kernels, same order)
and within the per-expert tolerance of the oracle."""
import numpy as np
import pytest
import torch

from oracle import qma_oracle as O
from quantized_moe_align_amd import inputs, qma
from quantized_moe_align_amd.moe import ExpertWeights, to_device, to_host, workspace_for
from gpu_common import assert_per_expert, slot_experts

pytestmark = pytest.mark.gpu

SENT = 0x5A5A


def _call(rng, E, T, topk, K, N, force_bm=0, override=None):
    w = inputs.random_words(rng, (E, N, K // 8))
    s = inputs.bf16_normal(rng, (E, N, K // 32), 0.02, absolute=True)
    a = inputs.bf16_normal(rng, (T, K))
    ids = rng.integers(0, E, (T, topk)).astype(np.int32)
    W = ExpertWeights(w, s)
    plan = qma.qma_plan_indexed(W.layer, T, topk, force_bm)
    if override:
        plan.schedule = qma.SCHEDULE_SEMI_STATIC   # unless the override names one
    for k, v in (override or {}).items():
        setattr(plan, k, v)
    B = plan.block_m
    cap = qma.qma_align_sizes(T, topk, E, B)[0]
    sorted_ids = torch.empty(cap, dtype=torch.int32, device="cuda")
    expert_ids = torch.empty(-(-cap // B), dtype=torch.int32, device="cuda")
    ntp = torch.empty(1, dtype=torch.int32, device="cuda")
    qma.qma_moe_align(to_device(ids), T, topk, E, B, sorted_ids, expert_ids, ntp, cap)
    d_a = to_device(a)
    R = T * topk
    ws = workspace_for(plan)
    assert ws is not None, "the plan must use a workspace for this test to mean anything"
    c_ws = torch.full((R, N), SENT, dtype=torch.int16, device="cuda")
    qma.qma_indexed_gemm(W.layer, plan, d_a, T, topk, W.packed, sorted_ids, expert_ids, ntp,
                         cap, R, None, c_ws, ws, ws.numel())
    c_sc = torch.full((R, N), SENT, dtype=torch.int16, device="cuda")
    qma.qma_indexed_gemm_scratch(W.layer, plan, d_a, T, topk, W.packed, sorted_ids, expert_ids,
                                 ntp, cap, R, None, c_sc)
    torch.cuda.synchronize()
    got_ws, got_sc = to_host(c_ws, bf16=True), to_host(c_sc, bf16=True)
    assert np.array_equal(got_sc, got_ws)
    assert_per_expert(got_sc, O.moe_gemm_by_slot(a, topk, ids, w, s), slot_experts(ids, E),
                      "scratch")
    return plan


# (first call, second call with a smaller input) per plan family
FAMILIES = {
    "small_m_split": ((3, 40, 2, 2048, 1024, 16, {"split_k": 4, "block_n": 64, "waves_k": 4}),
                      (1, 12, 1, 1024, 512, 16, {"split_k": 2, "block_n": 64, "waves_k": 4})),
    "planner_split": ((1, 12, 1, 4096, 4096, 0, None), (1, 5, 1, 4096, 2048, 0, None)),
    "dynamic": ((5, 60, 2, 1024, 768, 16, {"block_n": 256, "waves_k": 1, "split_k": 1,
                                           "n_stream": 1, "schedule": 1}),
                (2, 9, 1, 512, 512, 16, {"block_n": 128, "waves_k": 1, "split_k": 1,
                                         "n_stream": 1, "schedule": 1})),
    "large_m_split": ((2, 300, 1, 1024, 512, 128, {"split_k": 4, "kernel": 2}),
                      (1, 90, 1, 512, 256, 128, {"split_k": 2, "kernel": 2})),
}


@pytest.mark.parametrize("family", sorted(FAMILIES))
def test_scratch_matches_workspace_twice(gpu, family):
    rng = np.random.default_rng(sorted(FAMILIES).index(family) + 500)
    for args in FAMILIES[family]:
        plan = _call(rng, *args[:5], force_bm=args[5], override=args[6])
        if family.endswith("split"):
            assert plan.split_k > 1
        if family == "dynamic":
            assert plan.schedule == qma.SCHEDULE_DYNAMIC


def test_scratch_rejects_plans_beyond_its_size(gpu):
    lay = qma.qma_layer_create(1, 4096, 2048)
    try:
        plan = qma.qma_plan_indexed(lay, 12, 1, 16)
        plan.split_k = 8
        plan.block_n, plan.waves_k = 64, 4
        fake = 1 << 20                     # rejected on the host; never dereferenced
        rows = 300000                      # 8 splits x 300000 rows x 4096 x 4 B > 32 MiB
        with pytest.raises(qma.QmaError) as ei:
            qma.qma_indexed_gemm_scratch(lay, plan, fake, rows, 1, fake, fake, fake, fake,
                                         rows + 15, rows, None, fake)
        assert ei.value.status == qma.QMA_ERR_WORKSPACE and "scratch" in ei.value.detail
    finally:
        qma.qma_layer_destroy(lay)
