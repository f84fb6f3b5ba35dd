#!/usr/bin/env python3
"""Benchmark of the W4A16 MoE expert GEMM pair on one MI355X.

One step is one pass of the whole hot path over one batch. On the indexed
path that is moe_align, gate_up, silu_and_mul and down; on the grouped
paths it is gate_up, silu_and_mul and down. Inputs are resident in HBM
before timing starts. W warm-up steps run untimed (continued until the step
has run back to back for --settle-ms, so that the clocks have left their
idle ramp), then exactly K steps run back to back between device
synchronisations: that wall time is ms_per_step. K further steps with HIP
event pairs around every stage, on the launching stream, time each kernel.
The per-layer gate_up+down time (the pages' kernel-level metric, which
leaves out routing and activation) is reported next to the whole-step time.

`value` is the whole step's effective throughput: algorithmic HBM bytes
(decode shapes, GB/s) or algorithmic flops (prefill shapes, TFLOP/s)
divided by ms_per_step. The roofline object covers the gate_up GEMM
launch. The oracle's CPU time on a bounded sample of the same workload is
reported as `cpu_baseline`.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("gate_up+down µs/layer; effective HBM GB/s (decode) and TFLOP/s (prefill)")
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
HBM_BOUND = {"ep8_decode", "tp8", "masked", "ep16_decode", "ep32_decode", "tiny"}

DESCRIPTIONS = {
    "ep8_decode": "indexed EP8 decode share: 48 experts x U{9..15} rows, hidden 7168, "
                  "intermediate 2048, W4A16 g32",
    "tp8": "indexed TP8 share: 384 experts, 256 tokens top-8, hidden 7168, I/8 256",
    "ep8_prefill": "indexed EP8 prefill share: 48 experts, 8192 rows Zipf(1.1), hidden 7168, "
                   "intermediate 2048",
    "ep8_prefill_span": "indexed EP8 prefill share, counts 590..20 geometric, 8192 rows",
    "contiguous": "grouped_contiguous: 48 experts x 128 rows, hidden 7168, intermediate 2048",
    "masked": "grouped_masked: 48 experts, budget 64, 32 valid rows, hidden 7168, "
              "intermediate 2048",
    "ep16_decode": "indexed EP16 decode share: 24 experts x U{9..15} rows",
    "ep32_decode": "indexed EP32 decode share: 12 experts x U{9..15} rows",
    "tiny": "tiny: 8 experts, 64 tokens top-2, K 256, I 128",
}


def algorithmic_work(wl):
    """Bytes each GEMM must move and flops it must do: packed weights and
    scales of experts that have rows (0.5625 B per weight), distinct
    activation rows read once, output rows written once; 2*rows*N*K flops
    over valid rows only."""
    import numpy as np
    K, I, E = wl.K, wl.I, wl.E
    if wl.kind == "indexed":
        ids = wl["topk_ids"]
        valid = (ids >= 0) & (ids < E)
        counts = np.bincount(ids[valid], minlength=E)
        rows = int(valid.sum())
        a_rows = int(valid.any(axis=1).sum())
    elif wl.kind == "contiguous":
        m = wl["m_indices"]
        counts = np.bincount(m[m >= 0], minlength=E)
        rows = a_rows = int((m >= 0).sum())
    else:
        counts = np.asarray(wl["masked_m"])
        rows = a_rows = int(counts.sum())
    ne = int((counts > 0).sum())
    w13 = ne * 2 * I * K * 9 // 16
    w2 = ne * K * I * 9 // 16
    gu_bytes = w13 + a_rows * K * 2 + rows * 2 * I * 2
    dn_bytes = w2 + rows * I * 2 + rows * K * 2
    return {"rows": rows, "experts_with_rows": ne,
            "gate_up_bytes": gu_bytes, "down_bytes": dn_bytes,
            "gate_up_flops": 2 * rows * 2 * I * K, "down_flops": 2 * rows * K * I}


def kernel_src_hash():
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "quantized_moe_align_amd", "csrc", "*"))):
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(workload):
    """HBM traffic of the gate_up launch from a committed rocprofv3 --pmc
    summary, if it was taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", f"pmc_gate_up_{workload}.md")
    if not os.path.exists(path):
        return None
    m = re.search(r"qma-traffic: (\{.*\})", open(path).read())
    if not m:
        return None
    d = json.loads(m.group(1))
    if d.get("src_sha") != kernel_src_hash():
        return None
    return d.get("bytes_per_launch")


def cpu_baseline(wl, budget_s):
    """The oracle as it stands, timed on the host on whole experts of the
    same workload (gate_up, activation and down per expert) until about
    budget_s of CPU work; the rate is scaled to the metric's unit."""
    import numpy as np
    from oracle import qma_oracle as O
    try:
        from threadpoolctl import threadpool_info
        pools = threadpool_info()
        threads = max([t.get("num_threads", 1) for t in pools] + [1])
        blas = ", ".join(sorted({f"{t.get('internal_api')} {t.get('version')}" for t in pools
                                 if t.get("user_api") == "blas"})) or "unknown"
    except Exception:                                     # pragma: no cover
        threads, blas = 1, "unknown"
    E, K, I = wl.E, wl.K, wl.I
    if wl.kind == "indexed":
        se = np.where((wl["topk_ids"] >= 0) & (wl["topk_ids"] < E), wl["topk_ids"], -1)
        se = se.reshape(-1)
        a, div = wl["a"], wl.topk
    elif wl.kind == "contiguous":
        se, a, div = wl["m_indices"].astype(np.int64), wl["a"], 1
    else:
        mm = wl["masked_m"]
        budget = wl.meta["budget"]
        se = np.array([[e if r < mm[e] else -1 for r in range(budget)] for e in range(E)])
        se, a, div = se.reshape(-1), wl["a"].reshape(-1, K), 1
    done_bytes = done_flops = 0
    t_total = 0.0
    experts = []
    for e in range(E):
        rows = np.nonzero(se == e)[0]
        if rows.size == 0:
            continue
        only = np.full_like(se, -1)
        only[rows] = e
        t0 = time.perf_counter()
        c1 = O.moe_gemm_by_slot(a, div, only, wl["w13"], wl["s13"])
        h = O.f64_to_bf16(O.silu_and_mul(O.f64_to_bf16(c1[rows])))
        hh = np.zeros((se.size, I), np.uint16)
        hh[rows] = h
        O.moe_gemm_by_slot(hh, 1, only, wl["w2"], wl["s2"])
        t_total += time.perf_counter() - t0
        n = rows.size
        done_bytes += (2 * I * K + K * I) * 9 // 16 + n * (K * 2 + 2 * I * 2 + I * 2 + K * 2)
        done_flops += 2 * n * 2 * I * K + 2 * n * K * I
        experts.append(e)
        if t_total >= budget_s:
            break
    return t_total, done_bytes, done_flops, threads, experts, blas


def host_cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:                                       # pragma: no cover
        pass
    return "unknown"


def practical_roofs(torch, dev):
    """What plain reference work reaches on this GPU, next to the vendor
    peaks: a 1 GiB device copy (torch's copy kernel; read + write bytes), a
    16-row bf16 product against a 1 GiB bf16 weight matrix (weight read
    bytes; the decode-shaped read roof) and a dense 8192^3 bf16 matmul, the
    last two through the vendor GEMM library via torch. All are measured
    after the timed region, back to back with a settle, and serve as context
    only; none is on the product path."""
    import time as _t

    def run(fn, n):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        t0 = _t.perf_counter()
        while _t.perf_counter() - t0 < 0.2:
            fn()
            torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / n                  # s per call

    nbytes = 1 << 30
    src = torch.empty(nbytes // 4, dtype=torch.int32, device=dev).fill_(1)
    dst = torch.empty_like(src)
    t_copy = run(lambda: dst.copy_(src), 20)
    del src, dst
    # read-bound: 16 bf16 token rows against a 1 GiB bf16 weight matrix
    # (the vendor GEMM library's skinny product reads the matrix once)
    kk, nn = 16384, 32768
    wg = torch.empty(nn, kk, dtype=torch.bfloat16, device=dev).fill_(0.5)
    xg = torch.randn(16, kk, device=dev).to(torch.bfloat16)
    t_read = run(lambda: torch.nn.functional.linear(xg, wg), 20)
    del wg, xg
    n = 8192
    a = torch.randn(n, n, device=dev).to(torch.bfloat16).contiguous()
    b = torch.randn(n, n, device=dev).to(torch.bfloat16).contiguous()
    t_mm = run(lambda: torch.mm(a, b), 10)
    del a, b
    return {"copy_GBps": round(2 * nbytes / t_copy / 1e9, 1),
            "gemv16_read_GBps": round(kk * nn * 2 / t_read / 1e9, 1),
            "dense_bf16_gemm_TFLOPs": round(2 * n ** 3 / t_mm / 1e12, 1),
            "note": "1 GiB device copy (read + write); 16 bf16 rows x 1 GiB bf16 weights "
                    "(weight reads); dense 8192^3 bf16 matmul; all via torch"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="ep8_decode", choices=sorted(DESCRIPTIONS))
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of oracle CPU work for cpu_baseline (0 = skip)")
    ap.add_argument("--schedule", default="semi_static", choices=("semi_static", "dynamic"),
                    help="how small-M GEMMs hand out (tile, column block) work; dynamic "
                         "applies where the plan accepts it (16/32-row tiles, one K "
                         "partition)")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="after the run, copy a buffer of this many bytes 3 times (a "
                         "plain copy kernel of known size, to calibrate rocprofv3 "
                         "FETCH_SIZE / WRITE_SIZE)")
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="continue the untimed warm-up until the step has run back to "
                         "back for this long (clock ramp from idle)")
    ap.add_argument("--no-roofs", dest="roofs", action="store_false",
                    help="skip the practical-roof measurements (device copy, dense bf16 GEMM)")
    ap.add_argument("--idle-gap-ms", type=float, default=0.0,
                    help="idle the GPU this long before each timed step (untimed), to "
                         "compare isolated launches with the sustained back-to-back "
                         "default; ms_per_step is then the sum of the stage medians")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU: the expert GEMM "
                          "pair is one rank's share and has no cross-GPU step; "
                          f"--gpus {args.gpus} is not supported"}))
        sys.exit(2)

    import numpy as np
    import torch
    from quantized_moe_align_amd import inputs, qma
    from quantized_moe_align_amd.moe import (ExpertWeights, GroupedMoE, IndexedMoE, to_device)

    qma.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = inputs.make(args.workload, seed=args.seed)
    work = algorithmic_work(wl)

    if wl.kind == "indexed":
        w13 = ExpertWeights(wl["w13"], wl["s13"])
        w2 = ExpertWeights(wl["w2"], wl["s2"])
        moe = IndexedMoE(w13, w2, wl.T, wl.topk)
        a = to_device(wl["a"])
        ids = to_device(wl["topk_ids"])
        stages = [("moe_align", lambda: moe.align(ids)), ("gate_up", lambda: moe.gate_up(a)),
                  ("silu_and_mul", moe.act), ("down", lambda: moe.down())]
    else:
        path = (qma.PATH_GROUPED_CONTIGUOUS if wl.kind == "contiguous"
                else qma.PATH_GROUPED_MASKED)
        w13 = ExpertWeights(wl["w13"], wl["s13"], path)
        w2 = ExpertWeights(wl["w2"], wl["s2"], path)
        if wl.kind == "contiguous":
            index = to_device(wl["m_indices"])
            moe = GroupedMoE(w13, w2, wl["m_indices"].size)
        else:
            index = to_device(wl["masked_m"])
            moe = GroupedMoE(w13, w2, wl.meta["budget"], wl.meta["expected_m"])
        a = to_device(wl["a"])
        stages = [("gate_up", lambda: moe.gate_up(a, index)), ("silu_and_mul", moe.act),
                  ("down", lambda: moe.down(index))]
    sched_applied = (False, False)
    if args.schedule == "dynamic":
        sched_applied = moe.set_schedule(qma.SCHEDULE_DYNAMIC)
    stream = torch.cuda.current_stream()

    # Warm-up: W steps, continued (untimed) until the GPU has run the step
    # back-to-back for at least --settle-ms. From idle, the clocks take some
    # tens of ms to reach their sustained level; steps timed inside that
    # ramp measure the power state, not the kernels.
    t_w = time.perf_counter()
    n_warm = 0
    while n_warm < args.warmup or (time.perf_counter() - t_w) * 1e3 < args.settle_ms:
        for _ in range(10 if n_warm >= args.warmup else 1):
            for _, fn in stages:
                fn()
            n_warm += 1
        if n_warm >= args.warmup:
            torch.cuda.synchronize()
    torch.cuda.synchronize()

    def timed_steps(per_stage: bool):
        """K steps between device synchronisations; with per_stage, an event
        pair around every stage (each record adds a few us of launch gap)."""
        pairs = [(name, torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                 for _ in range(args.steps) for name, _ in stages] if per_stage else []
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        i = 0
        for _ in range(args.steps):
            if args.idle_gap_ms > 0:
                torch.cuda.synchronize()
                time.sleep(args.idle_gap_ms * 1e-3)
            for name, fn in stages:
                if per_stage:
                    pairs[i][1].record(stream)
                fn()
                if per_stage:
                    pairs[i][2].record(stream)
                i += 1
        torch.cuda.synchronize()
        return time.perf_counter() - t0, pairs

    # The timed region: exactly K steps, launched back to back.
    wall, _ = timed_steps(per_stage=False)
    ms_per_step = wall / args.steps * 1e3
    # Per-kernel times: K more steps with events around every stage.
    _, pairs = timed_steps(per_stage=True)
    ev = {name: [] for name, _ in stages}
    for name, e0, e1 in pairs:
        ev[name].append(e0.elapsed_time(e1) * 1e3)          # us
    us = {k: float(np.mean(v)) for k, v in ev.items()}
    med = {k: float(np.median(v)) for k, v in ev.items()}
    if args.idle_gap_ms > 0:
        ms_per_step = sum(med.values()) * 1e-3

    hbm = args.workload in HBM_BOUND
    total_bytes = work["gate_up_bytes"] + work["down_bytes"]
    total_flops = work["gate_up_flops"] + work["down_flops"]
    if hbm:
        value = total_bytes / (ms_per_step * 1e-3) / 1e9
        unit = "GB/s"
        achieved = work["gate_up_bytes"] / (us["gate_up"] * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4)}
    else:
        value = total_flops / (ms_per_step * 1e-3) / 1e12
        unit = "TFLOP/s"
        achieved = work["gate_up_flops"] / (us["gate_up"] * 1e-6) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4)}
    roof["traffic"] = read_traffic(args.workload)
    roof["kernel"] = "gate_up GEMM (" + ("small-M" if moe.plan13.kernel == 1 else "large-M") + ")"

    cpu = None
    if args.cpu_budget > 0:
        t_cpu, b_cpu, f_cpu, threads, experts, blas = cpu_baseline(wl, args.cpu_budget)
        cpu = {"value": round((b_cpu / t_cpu / 1e9) if hbm else (f_cpu / t_cpu / 1e12), 4),
               "unit": unit, "cores": threads, "kind": "oracle",
               "host": {"cpu": host_cpu_model(), "nproc": os.cpu_count(), "blas": blas},
               "sample": f"experts {experts[0]}..{experts[-1]} ({len(experts)} of "
                         f"{work['experts_with_rows']}) of the same workload: gate_up, "
                         f"activation and down per expert in float64, {t_cpu:.1f} s"}

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": unit, "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "warmup_settle_ms": args.settle_ms,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": DESCRIPTIONS[args.workload], "name": args.workload,
                   "rows": work["rows"], "weights": "uint4 group-32 bf16 scales, zero point 8",
                   "parallelism": "one EP/TP rank's share on one GPU",
                   "schedule": {"gate_up": "dynamic" if sched_applied[0] else "semi_static",
                                "down": "dynamic" if sched_applied[1] else "semi_static"},
                   **({"idle_gap_ms": args.idle_gap_ms} if args.idle_gap_ms > 0 else {})},
        "us_per_layer_gate_up_down": round(us["gate_up"] + us["down"], 2),
        "kernel_us_mean": {k: round(v, 2) for k, v in us.items()},
        "kernel_us_median": {k: round(v, 2) for k, v in med.items()},
        "kernel_us_p10_p90": {k: [round(float(np.percentile(v, 10)), 2),
                                  round(float(np.percentile(v, 90)), 2)] for k, v in ev.items()},
        "gemm_pair_effective": {"GB/s": round(total_bytes / ((us["gate_up"] + us["down"]) * 1e-6)
                                              / 1e9, 1),
                                "TFLOP/s": round(total_flops / ((us["gate_up"] + us["down"])
                                                                * 1e-6) / 1e12, 2)},
        "algorithmic": work,
        "plan": {"gate_up": moe.plan13.as_dict(), "down": moe.plan2.as_dict()},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    if args.roofs:
        out["practical_roofs"] = practical_roofs(torch, dev)
    if args.copy_bytes > 0:
        src = torch.empty(args.copy_bytes // 4, dtype=torch.int32, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_calibration_bytes"] = args.copy_bytes
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
