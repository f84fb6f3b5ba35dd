"""Device-side orchestration of the MoE expert GEMM pair over libqma.

PyTorch only allocates device memory and supplies the stream; every step of
the path (moe_align, prepack, gate_up, silu_and_mul, down, combine) is a
libqma call. Host numpy arrays hold raw bit patterns: bf16 as uint16,
packed uint4 as int32.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from . import qma


def to_device(x: np.ndarray, device="cuda") -> torch.Tensor:
    """Copy a host bit-pattern array to the device (uint16 -> int16 view)."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        x = x.view(np.int16)
    elif x.dtype == np.uint32:
        x = x.view(np.int32)
    return torch.from_numpy(x).to(device)


def to_host(t: torch.Tensor, bf16: bool = False) -> np.ndarray:
    a = t.detach().cpu().numpy()
    return a.view(np.uint16) if bf16 else a


def empty_bf16(*shape, device="cuda") -> torch.Tensor:
    return torch.empty(shape, dtype=torch.int16, device=device)


class ExpertWeights:
    """One projection's experts: the layer handle and its prepacked weights."""

    def __init__(self, qweight: np.ndarray, scales: np.ndarray, path: int = qma.PATH_INDEXED,
                 device="cuda", stream=None, flags: int = 0):
        E, N, K8 = qweight.shape
        self.E, self.N, self.K = E, N, K8 * 8
        self.path, self.flags = path, flags
        self.fused = bool(flags & qma.LAYER_FUSE_SILU_MUL)
        self.layer = qma.qma_layer_create(E, N, self.K, path, flags=flags)
        nbytes = qma.qma_packed_weight_bytes(self.layer)
        self.packed = torch.empty(nbytes, dtype=torch.uint8, device=device)
        qw = to_device(qweight, device)
        sc = to_device(scales, device)
        qma.qma_prepack(self.layer, qw, sc, self.packed, stream)
        torch.cuda.current_stream().synchronize()
        del qw, sc

    def with_path(self, path: int) -> "ExpertWeights":
        """The same prepacked weights under a layer handle of another routing
        family (one packed layout serves every family, so nothing is packed
        again)."""
        other = ExpertWeights.__new__(ExpertWeights)
        other.E, other.N, other.K, other.path = self.E, self.N, self.K, path
        other.flags, other.fused = self.flags, self.fused
        other.layer = qma.qma_layer_create(self.E, self.N, self.K, path, flags=self.flags)
        if qma.qma_packed_weight_bytes(other.layer) != self.packed.numel():
            raise ValueError("packed sizes differ between paths")
        other.packed = self.packed
        return other

    @property
    def info(self):
        return qma.qma_layer_info(self.layer)

    def __del__(self):
        lay = getattr(self, "layer", None)
        if lay is not None and qma._lib is not None:
            qma.qma_layer_destroy(lay)
            self.layer = None


def workspace_for(plan: qma.Plan, device="cuda") -> Optional[torch.Tensor]:
    n = qma.qma_workspace_bytes(plan)
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None


def schedule_applies(plan: qma.Plan, schedule: int = qma.SCHEDULE_DYNAMIC) -> bool:
    """Whether a plan can take `schedule`: semi-static always; dynamic for
    16/32-row small-M tiles with one K partition, no split-K and no
    column-block streaming; gang for the shared-row small-M instances (one K
    partition per workgroup, 128 or 256 columns, 16/32/64-row tiles, with
    or without split-K, no streaming); stream-K for the 16/32-row shared-row
    instances of an indexed layer without split-K (the call may still refuse
    a sorted capacity that gives a group three token tiles)."""
    if schedule == qma.SCHEDULE_SEMI_STATIC:
        return True
    shared = (plan.kernel == qma.KERNEL_SMALL_M and plan.waves_k == 1 and plan.n_stream == 1
              and plan.block_n in (128, 256))
    if schedule == qma.SCHEDULE_DYNAMIC:
        return shared and plan.split_k == 1 and plan.block_m in (16, 32)
    if schedule == qma.SCHEDULE_GANG:
        return shared and (plan.block_m, plan.block_n) in ((16, 128), (16, 256), (32, 128),
                                                           (32, 256), (64, 128))
    if schedule == qma.SCHEDULE_STREAM_K:
        return (shared and plan.path == qma.PATH_INDEXED and plan.split_k == 1
                and plan.block_m in (16, 32) and plan.k >= 8 * 128)
    return False


@dataclass
class Routing:
    sorted_ids: torch.Tensor
    expert_ids: torch.Tensor
    ntp: torch.Tensor
    cap: int
    block_m: int


class IndexedMoE:
    """gate_up -> silu_and_mul -> down over the indexed path for one batch
    shape (T tokens, top-k). Buffers are allocated once, so forward() only
    enqueues kernels and can be captured in a hipGraph. With a fused gate_up
    layer (ExpertWeights(..., flags=LAYER_FUSE_SILU_MUL)) gate_up writes the
    activation h itself and act() enqueues nothing."""

    def __init__(self, w13: ExpertWeights, w2: ExpertWeights, T: int, topk: int,
                 force_block_m: int = 0, extra_cap: int = 0, device="cuda"):
        self.w13, self.w2, self.T, self.topk = w13, w2, T, topk
        self.E = w13.E
        self.I = w13.N // 2
        self.K = w13.K
        self.plan13 = qma.qma_plan_indexed(w13.layer, T, topk, force_block_m)
        self.plan2 = qma.qma_plan_indexed(w2.layer, T, topk, self.plan13.block_m)
        bm = self.plan13.block_m
        cap, blocks = qma.qma_align_sizes(T, topk, self.E, bm)
        cap += extra_cap
        blocks = -(-cap // bm)
        R = T * topk
        dev = device
        self.routing = Routing(torch.empty(cap, dtype=torch.int32, device=dev),
                               torch.empty(blocks, dtype=torch.int32, device=dev),
                               torch.empty(1, dtype=torch.int32, device=dev), cap, bm)
        self.fused = w13.fused
        self.c1 = None if self.fused else empty_bf16(max(R, 1), 2 * self.I, device=dev)
        self.h = empty_bf16(max(R, 1), self.I, device=dev)
        self.c2 = empty_bf16(max(R, 1), self.K, device=dev)
        self.ws13 = workspace_for(self.plan13, dev)
        self.ws2 = workspace_for(self.plan2, dev)
        self._dev = dev

    def align(self, topk_ids: torch.Tensor, stream=None):
        r = self.routing
        qma.qma_moe_align(topk_ids, self.T, self.topk, self.E, r.block_m, r.sorted_ids,
                          r.expert_ids, r.ntp, r.cap, stream)

    def set_schedule(self, schedule: int) -> tuple:
        """Switch both GEMMs to `schedule` where their plan accepts it;
        returns which of (gate_up, down) changed."""
        done = []
        for name in ("13", "2"):
            plan = getattr(self, "plan" + name)
            ok = schedule_applies(plan, schedule)
            if ok:
                plan.schedule = schedule
                setattr(self, "ws" + name, workspace_for(plan, self._dev))
            done.append(ok)
        return tuple(done)

    def gate_up(self, a: torch.Tensor, stream=None):
        r = self.routing
        qma.qma_indexed_gemm(self.w13.layer, self.plan13, a, self.T, self.topk,
                             self.w13.packed, r.sorted_ids, r.expert_ids, r.ntp, r.cap,
                             self.T * self.topk, None, self.h if self.fused else self.c1,
                             self.ws13, 0 if self.ws13 is None else self.ws13.numel(), stream)

    def act(self, stream=None):
        if not self.fused:
            qma.qma_silu_and_mul(self.c1, self.h, self.T * self.topk, self.I, stream)

    def down(self, topk_weights: Optional[torch.Tensor] = None, stream=None):
        r = self.routing
        R = self.T * self.topk
        qma.qma_indexed_gemm(self.w2.layer, self.plan2, self.h, R, 1, self.w2.packed,
                             r.sorted_ids, r.expert_ids, r.ntp, r.cap, R, topk_weights,
                             self.c2, self.ws2, 0 if self.ws2 is None else self.ws2.numel(),
                             stream)

    def forward(self, a, topk_ids, topk_weights=None, stream=None):
        self.align(topk_ids, stream)
        self.gate_up(a, stream)
        self.act(stream)
        self.down(topk_weights, stream)
        return self.c2


class GroupedMoE:
    """gate_up -> silu_and_mul -> down over a grouped path (contiguous rows
    with m_indices, or masked [E, budget, K] with masked_m)."""

    def __init__(self, w13: ExpertWeights, w2: ExpertWeights, rows_or_budget: int,
                 expected_m: int = 0, device="cuda"):
        assert w13.path == w2.path
        self.w13, self.w2 = w13, w2
        self.masked = w13.path == qma.PATH_GROUPED_MASKED
        self.E, self.I, self.K = w13.E, w13.N // 2, w13.K
        self.rows_or_budget, self.expected_m = rows_or_budget, expected_m
        self.plan13 = qma.qma_plan_grouped(w13.layer, rows_or_budget, expected_m)
        self.plan2 = qma.qma_plan_grouped(w2.layer, rows_or_budget, expected_m)
        rows = rows_or_budget * (self.E if self.masked else 1)
        self.rows = rows
        self.fused = w13.fused
        self.c1 = None if self.fused else empty_bf16(max(rows, 1), 2 * self.I, device=device)
        self.h = empty_bf16(max(rows, 1), self.I, device=device)
        self.c2 = empty_bf16(max(rows, 1), self.K, device=device)
        self.ws13 = workspace_for(self.plan13, device)
        self.ws2 = workspace_for(self.plan2, device)
        self._dev = device

    def _gemm(self, w, plan, a, c, ws, index, stream):
        wsb = 0 if ws is None else ws.numel()
        if self.masked:
            qma.qma_grouped_masked_gemm(w.layer, plan, a, index, self.rows_or_budget,
                                        self.expected_m, w.packed, c, ws, wsb, stream)
        else:
            qma.qma_grouped_contiguous_gemm(w.layer, plan, a, index, self.rows, w.packed, c,
                                            ws, wsb, stream)

    def set_schedule(self, schedule: int) -> tuple:
        """Switch both GEMMs to `schedule` where their plan accepts it;
        returns which of (gate_up, down) changed."""
        done = []
        for name in ("13", "2"):
            plan = getattr(self, "plan" + name)
            ok = schedule_applies(plan, schedule)
            if ok:
                plan.schedule = schedule
                setattr(self, "ws" + name, workspace_for(plan, self._dev))
            done.append(ok)
        return tuple(done)

    def gate_up(self, a, index, stream=None):
        self._gemm(self.w13, self.plan13, a, self.h if self.fused else self.c1, self.ws13, index,
                   stream)

    def act(self, stream=None):
        if not self.fused:
            qma.qma_silu_and_mul(self.c1, self.h, self.rows, self.I, stream)

    def down(self, index, stream=None):
        self._gemm(self.w2, self.plan2, self.h, self.c2, self.ws2, index, stream)

    def forward(self, a, index, stream=None):
        self.gate_up(a, index, stream)
        self.act(stream)
        self.down(index, stream)
        return self.c2
