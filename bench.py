#!/usr/bin/env python3
"""Benchmark of the W4A16 MoE expert GEMM pair on one MI355X.

One step is one pass of the whole hot path over one batch. On the indexed
path that is moe_align, gate_up, the activation silu(gate) * up, and down;
on the grouped paths it is gate_up, the activation and down. By default the
activation runs in gate_up's epilogue (a gate_up layer made with the fused
flag); --activation separate runs it as its own kernel (silu_and_mul)
between the GEMMs. Inputs are resident in HBM before timing starts.

The headline workload (--workload, default the EP8 decode share) gives
`value`: W warm-up steps run untimed (continued until the step has run back
to back for --settle-ms, so that the clocks have left their idle ramp), then
exactly K steps run back to back between device synchronisations; that wall
time is ms_per_step. K further steps with HIP event pairs around every stage,
on the launching stream, time each kernel. `value` is the whole step's
effective throughput: algorithmic HBM bytes (decode shapes, GB/s) or
algorithmic flops (prefill shapes, TFLOP/s) divided by ms_per_step. The
roofline object covers the headline workload's gate_up GEMM launch.

The `configs` object repeats the measurement for every workload of the
pages' scenarios (tiny, EP8 decode, TP8, EP8 prefill, grouped contiguous,
grouped masked) in the same run: per-kernel event times, the gate_up+down
pair time (the pages' per-layer kernel metric, which leaves out routing and
the activation), the pair's rate, roofline fractions per GEMM and for the
pair, and HBM traffic from the committed rocprofv3 summaries. With flushing
on (the default), each stage is also timed cold: a 512 MiB device read
before every timed call evicts the L2s and the MALL. (A write would leave
up to the MALL's size of dirty lines, whose write-back then competes with
the timed kernel's reads.)

The oracle's CPU time on a bounded sample of the headline workload is
reported as `cpu_baseline` (float64, as the oracle stands), with fp32
timings next to it: per-expert dequantisation included, and matmuls alone on
cached fp32 weights.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import re
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("gate_up+down µs/layer; effective HBM GB/s (decode) and TFLOP/s (prefill)")
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
HBM_BOUND = {"ep8_decode", "tp8", "masked", "ep16_decode", "ep32_decode", "tiny", "ep8_mid",
             "ep128_decode"}
# the pages' six measured scenarios map onto the first six workloads; the last two
# cover the 33..79 rows-per-expert regime and a share where split-K turns on
DEFAULT_CONFIGS = ("tiny", "ep8_decode", "tp8", "ep8_prefill", "contiguous", "masked", "ep8_mid",
                   "ep128_decode")
FLUSH_BYTES = 512 << 20

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
    "ep8_mid": "indexed EP8 share between decode and prefill: 48 experts x U{40..56} rows",
    "ep128_decode": "indexed EP128 decode share: 3 experts x U{9..15} rows (split-K on)",
    "tiny": "tiny: 8 experts, 64 tokens top-2, K 256, I 128",
}


def algorithmic_work(wl, fused=False):
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
    # gate_up writes h [rows, I] with the activation fused, else [rows, 2I]
    gu_bytes = w13 + a_rows * K * 2 + rows * (1 if fused else 2) * I * 2
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
    """HBM traffic per launch of the gate_up and down GEMMs from the committed
    rocprofv3 --pmc summary, if it was taken on the current kernel sources:
    {"gate_up": bytes or None, "down": bytes or None}."""
    out = {"gate_up": None, "down": None}
    path = os.path.join(ROOT, "profiles", f"pmc_gate_up_{workload}.md")
    if not os.path.exists(path):
        return out
    m = re.search(r"qma-traffic: (\{.*\})", open(path).read())
    if not m:
        return out
    d = json.loads(m.group(1))
    if d.get("src_sha") != kernel_src_hash():
        return out
    out["gate_up"] = d.get("bytes_per_launch")
    out["down"] = d.get("down_bytes_per_launch")
    return out


# --------------------------------------------------------------------------
# CPU baseline (the oracle, plus plain fp32 NumPy next to it)
# --------------------------------------------------------------------------

def _blas_info():
    try:
        from threadpoolctl import threadpool_info
        pools = threadpool_info()
        threads = max([t.get("num_threads", 1) for t in pools] + [1])
        blas = ", ".join(sorted({f"{t.get('internal_api')} {t.get('version')}" for t in pools
                                 if t.get("user_api") == "blas"})) or "unknown"
    except Exception:                                     # pragma: no cover
        threads, blas = 1, "unknown"
    return threads, blas


def _slot_experts(wl):
    import numpy as np
    E, K = wl.E, wl.K
    if wl.kind == "indexed":
        se = np.where((wl["topk_ids"] >= 0) & (wl["topk_ids"] < E), wl["topk_ids"], -1)
        return se.reshape(-1), wl["a"], wl.topk
    if wl.kind == "contiguous":
        return wl["m_indices"].astype(np.int64), wl["a"], 1
    mm = wl["masked_m"]
    budget = wl.meta["budget"]
    se = np.array([[e if r < mm[e] else -1 for r in range(budget)] for e in range(E)])
    return se.reshape(-1), wl["a"].reshape(-1, K), 1


def _expert_bytes_flops(wl, n):
    K, I = wl.K, wl.I
    b = (2 * I * K + K * I) * 9 // 16 + n * (K * 2 + 2 * I * 2 + I * 2 + K * 2)
    f = 2 * n * 2 * I * K + 2 * n * K * I
    return b, f


def cpu_oracle(wl, budget_s):
    """The oracle as it stands, timed on the host on whole experts of the
    same workload (gate_up, activation and down per expert) until about
    budget_s of CPU work."""
    import numpy as np
    from oracle import qma_oracle as O
    se, a, div = _slot_experts(wl)
    I = wl.I
    done_bytes = done_flops = 0
    t_total = 0.0
    experts = []
    for e in range(wl.E):
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
        b, f = _expert_bytes_flops(wl, rows.size)
        done_bytes += b
        done_flops += f
        experts.append(e)
        if t_total >= budget_s:
            break
    return t_total, done_bytes, done_flops, experts


def cpu_fp32(wl, n_experts, reps=3):
    """Plain fp32 NumPy on the host over the first n_experts experts with
    rows: gate_up, SiLU-gated activation and down per expert, (i) with the
    expert's weights dequantised to fp32 inside the timed region, (ii) with
    them dequantised beforehand (matmuls alone). 1 warm-up + `reps` timed
    repetitions each; median seconds per repetition."""
    import numpy as np
    from oracle import qma_oracle as O
    se, a, div = _slot_experts(wl)
    I = wl.I
    a32 = O.bf16_to_f64(a).astype(np.float32)
    jobs = []
    for e in range(wl.E):
        rows = np.nonzero(se == e)[0]
        if rows.size:
            jobs.append((e, rows))
        if len(jobs) == n_experts:
            break

    def deq32(qw, sc):
        q = O.unpack_uint4(qw).astype(np.float32) - np.float32(8)
        s = O.bf16_to_f64(sc).astype(np.float32)
        return q * np.repeat(s, 32, axis=-1)

    def layer(x, w13, w2):
        c1 = x @ w13.T
        g, u = c1[:, :I], c1[:, I:]
        h = g / (np.float32(1) + np.exp(-g)) * u
        return h @ w2.T

    def with_deq():
        for e, rows in jobs:
            layer(a32[rows // div], deq32(wl["w13"][e], wl["s13"][e]),
                  deq32(wl["w2"][e], wl["s2"][e]))

    cached = {e: (deq32(wl["w13"][e], wl["s13"][e]), deq32(wl["w2"][e], wl["s2"][e]))
              for e, _ in jobs}

    def matmul_only():
        for e, rows in jobs:
            layer(a32[rows // div], *cached[e])

    def timed(fn):
        fn()
        ts = []
        for _ in range(reps):
            t0 = time.perf_counter()
            fn()
            ts.append(time.perf_counter() - t0)
        return float(np.median(ts))

    t_deq = timed(with_deq)
    t_mm = timed(matmul_only)
    b = f = 0
    for _, rows in jobs:
        bb, ff = _expert_bytes_flops(wl, rows.size)
        b += bb
        f += ff
    return t_deq, t_mm, b, f, [e for e, _ in jobs]


def host_cpu():
    info = {"nproc": os.cpu_count()}
    try:
        fields = {}
        for line in open("/proc/cpuinfo"):
            k, _, v = line.partition(":")
            k = k.strip()
            if k in ("model name", "cpu family", "model", "stepping", "vendor_id") and k not in fields:
                fields[k] = v.strip()
        info["model_name"] = fields.get("model name", "unknown")
        info["vendor"] = fields.get("vendor_id")
        info["family_model_stepping"] = "%s/%s/%s" % (fields.get("cpu family"), fields.get("model"),
                                                      fields.get("stepping"))
    except OSError:                                       # pragma: no cover
        info["model_name"] = "unknown"
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            k, _, v = line.partition(":")
            if k.strip() in ("Model name", "BIOS Model name", "Socket(s)", "Core(s) per socket",
                             "Thread(s) per core"):
                info["lscpu " + k.strip()] = v.strip()
    except Exception:                                     # pragma: no cover
        pass
    return info


# --------------------------------------------------------------------------
# GPU side
# --------------------------------------------------------------------------

def practical_roofs(torch, dev):
    """What plain reference work reaches on this GPU, next to the vendor
    peaks: a 1 GiB device copy (torch's copy kernel; read + write bytes), a
    16-row bf16 product against a 1 GiB bf16 weight matrix (weight read
    bytes; the decode-shaped read roof) and a dense 8192^3 bf16 matmul, the
    last two through the vendor GEMM library via torch. All are measured
    after the timed region, back to back with a settle, and serve as context
    only; none is on the product path."""
    def run(fn, n):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < 0.2:
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


class WeightCache:
    """Host arrays and prepacked device weights per (E, K, I, seed): the EP8
    decode, EP8 prefill, contiguous and masked workloads share one EP8 weight
    set (same shapes, same seed), generated and packed once."""

    def __init__(self):
        self.host = {}
        self.dev = {}

    def attach(self, wl, seed):
        from quantized_moe_align_amd import inputs
        key = (wl.E, wl.K, wl.I, seed)
        if key not in self.host:
            full = inputs._with_weights(inputs.Workload(wl.name, wl.kind, wl.E, wl.K, wl.I),
                                        seed, True)
            self.host[key] = {k: full[k] for k in ("w13", "s13", "w2", "s2")}
        wl.arrays.update(self.host[key])
        return key

    def packed(self, key, path, fused=False):
        from quantized_moe_align_amd import qma
        from quantized_moe_align_amd.moe import ExpertWeights
        dkey = (key, fused)
        if dkey not in self.dev:
            h = self.host[key]
            flags = qma.LAYER_FUSE_SILU_MUL if fused else 0
            self.dev[dkey] = {qma.PATH_INDEXED: (ExpertWeights(h["w13"], h["s13"], flags=flags),
                                                 ExpertWeights(h["w2"], h["s2"]))}
        d = self.dev[dkey]
        if path not in d:
            base13, base2 = d[qma.PATH_INDEXED]
            d[path] = (base13.with_path(path), base2.with_path(path))
        return d[path]


def build_runner(name, seed, cache, schedule, overrides, fused=True):
    """Inputs on the device and the step's stages for one workload."""
    import torch
    from quantized_moe_align_amd import inputs, qma
    from quantized_moe_align_amd.moe import GroupedMoE, IndexedMoE, to_device, workspace_for

    wl = inputs.make(name, seed=seed, weights=False)
    key = cache.attach(wl, seed)
    work = algorithmic_work(wl, fused)
    if wl.kind == "indexed":
        w13, w2 = cache.packed(key, qma.PATH_INDEXED, fused)
        moe = IndexedMoE(w13, w2, wl.T, wl.topk)
        a = to_device(wl["a"])
        ids = to_device(wl["topk_ids"])
        stages = [("moe_align", lambda: moe.align(ids)), ("gate_up", lambda: moe.gate_up(a)),
                  ("silu_and_mul", moe.act), ("down", lambda: moe.down())]
        if fused:
            del stages[2]
    else:
        path = (qma.PATH_GROUPED_CONTIGUOUS if wl.kind == "contiguous"
                else qma.PATH_GROUPED_MASKED)
        w13, w2 = cache.packed(key, path, fused)
        if wl.kind == "contiguous":
            index = to_device(wl["m_indices"])
            moe = GroupedMoE(w13, w2, wl["m_indices"].size)
        else:
            index = to_device(wl["masked_m"])
            moe = GroupedMoE(w13, w2, wl.meta["budget"], wl.meta["expected_m"])
        a = to_device(wl["a"])
        stages = [("gate_up", lambda: moe.gate_up(a, index)), ("silu_and_mul", moe.act),
                  ("down", lambda: moe.down(index))]
        if fused:
            del stages[1]
    applied = (False, False)
    if schedule != "planner":
        applied = moe.set_schedule({"semi_static": qma.SCHEDULE_SEMI_STATIC,
                                    "dynamic": qma.SCHEDULE_DYNAMIC,
                                    "gang": qma.SCHEDULE_GANG,
                                    "stream_k": qma.SCHEDULE_STREAM_K}[schedule])
    for which, ov in (("13", overrides.get("gate_up")), ("2", overrides.get("down"))):
        if ov:
            plan = getattr(moe, "plan" + which)
            for k, v in ov.items():
                setattr(plan, k, v)
            setattr(moe, "ws" + which, workspace_for(plan))
    torch.cuda.synchronize()
    return {"name": name, "wl": wl, "work": work, "moe": moe, "stages": stages,
            "schedule": applied}


def measure(r, steps, warmup, settle_ms, idle_gap_ms=0.0, flush=None):
    """ms_per_step over K back-to-back steps, per-stage event times over K
    more steps, and (with a flush buffer) per-stage times with a 512 MiB
    device read before every timed call."""
    import numpy as np
    import torch
    stages = r["stages"]
    stream = torch.cuda.current_stream()
    t_w = time.perf_counter()
    n_warm = 0
    while n_warm < warmup or (time.perf_counter() - t_w) * 1e3 < settle_ms:
        for _ in range(10 if n_warm >= warmup else 1):
            for _, fn in stages:
                fn()
            n_warm += 1
        if n_warm >= warmup:
            torch.cuda.synchronize()
    torch.cuda.synchronize()

    def timed_steps(per_stage, flush_buf=None):
        pairs = [(name, torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                 for _ in range(steps) for name, _ in stages] if per_stage else []
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        i = 0
        for s in range(steps):
            if idle_gap_ms > 0:
                torch.cuda.synchronize()
                time.sleep(idle_gap_ms * 1e-3)
            for name, fn in stages:
                if flush_buf is not None:
                    flush_buf.max()          # reads 512 MiB: evicts with clean lines
                if per_stage:
                    pairs[i][1].record(stream)
                fn()
                if per_stage:
                    pairs[i][2].record(stream)
                i += 1
        torch.cuda.synchronize()
        return time.perf_counter() - t0, pairs

    # the timed region: exactly K steps, launched back to back
    wall, _ = timed_steps(per_stage=False)
    out = {"ms_per_step": wall / steps * 1e3}

    def collect(pairs):
        ev = {name: [] for name, _ in stages}
        for name, e0, e1 in pairs:
            ev[name].append(e0.elapsed_time(e1) * 1e3)       # us
        return ev

    _, pairs = timed_steps(per_stage=True)
    out["ev"] = collect(pairs)
    if flush is not None:
        _, fpairs = timed_steps(per_stage=True, flush_buf=flush)
        out["ev_flushed"] = collect(fpairs)
    if idle_gap_ms > 0:
        out["ms_per_step"] = sum(float(np.median(v)) for v in out["ev"].values()) * 1e-3
    return out


def pair_report(name, work, ev, traffic):
    """gate_up, down and pair times with rates and roofline fractions."""
    import numpy as np
    hbm = name in HBM_BOUND
    mean = {k: float(np.mean(v)) for k, v in ev.items()}
    med = {k: float(np.median(v)) for k, v in ev.items()}
    gu, dn = mean["gate_up"], mean["down"]
    rep = {"us_mean": {k: round(v, 2) for k, v in mean.items()},
           "us_median": {k: round(v, 2) for k, v in med.items()},
           "pair_us": round(gu + dn, 2), "pair_us_median": round(med["gate_up"] + med["down"], 2)}
    if hbm:
        def rate(b, us):
            return b / (us * 1e-6) / 1e9
        rg, rd = rate(work["gate_up_bytes"], gu), rate(work["down_bytes"], dn)
        rp = rate(work["gate_up_bytes"] + work["down_bytes"], gu + dn)
        rep.update({"bound": "hbm", "unit": "GB/s", "pair_rate": round(rp, 1),
                    "gate_up_rate": round(rg, 1), "down_rate": round(rd, 1),
                    "frac": {"gate_up": round(rg / HBM_PEAK_GBS, 4),
                             "down": round(rd / HBM_PEAK_GBS, 4),
                             "pair": round(rp / HBM_PEAK_GBS, 4)}})
    else:
        def rate(f, us):
            return f / (us * 1e-6) / 1e12
        rg, rd = rate(work["gate_up_flops"], gu), rate(work["down_flops"], dn)
        rp = rate(work["gate_up_flops"] + work["down_flops"], gu + dn)
        rep.update({"bound": "mfma", "unit": "TFLOP/s", "pair_rate": round(rp, 2),
                    "gate_up_rate": round(rg, 2), "down_rate": round(rd, 2),
                    "frac": {"gate_up": round(rg / MFMA_BF16_PEAK_TFLOPS, 4),
                             "down": round(rd / MFMA_BF16_PEAK_TFLOPS, 4),
                             "pair": round(rp / MFMA_BF16_PEAK_TFLOPS, 4)}})
    if traffic is not None:
        rep["traffic_bytes"] = traffic
        rep["traffic_over_algorithmic"] = {
            k: (round(traffic[k] / work[k + "_bytes"], 3) if traffic.get(k) else None)
            for k in ("gate_up", "down")}
    return rep


def plan_brief(plan):
    d = plan.as_dict()
    return {k: d[k] for k in ("kernel", "block_m", "block_n", "split_k", "k_depth", "waves_k",
                              "n_stream", "schedule")}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="ep8_decode", choices=sorted(DESCRIPTIONS),
                    help="the headline workload that gives `value` and `roofline`")
    ap.add_argument("--configs", default="default",
                    help="workloads measured into the `configs` object: 'default' (the "
                         "pages' scenarios: %s), 'none', or a comma-separated list"
                         % ", ".join(DEFAULT_CONFIGS))
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-budget", type=float, default=10.0,
                    help="seconds of oracle CPU work for cpu_baseline (0 = skip the CPU legs)")
    ap.add_argument("--cpu-fp32-experts", type=int, default=4,
                    help="experts in the fp32 NumPy legs of cpu_baseline")
    ap.add_argument("--activation", default="fused", choices=("fused", "separate"),
                    help="silu(gate) * up in gate_up's epilogue (fused, the default) or as its "
                         "own kernel between the GEMMs (separate)")
    ap.add_argument("--schedule", default="planner",
                    choices=("planner", "semi_static", "dynamic", "gang", "stream_k"),
                    help="how small-M GEMMs hand out (tile, column block) work: the "
                         "planner's choice, or one schedule forced where the plan accepts "
                         "it (dynamic: 16/32-row tiles, one K partition; gang: the "
                         "shared-row instances; stream_k: their 16/32-row indexed plans "
                         "without split-K)")
    ap.add_argument("--override-gate-up", default="",
                    help="JSON object of plan fields to set on the headline workload's "
                         "gate_up plan before timing (A/B runs, e.g. '{\"split_k\": 1}')")
    ap.add_argument("--override-down", default="", help="the same for the down plan")
    ap.add_argument("--no-flush", dest="flush", action="store_false",
                    help="skip the cold timings (a 512 MiB device read before each call)")
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
    if args.configs == "default":
        configs = list(DEFAULT_CONFIGS)
    elif args.configs == "none":
        configs = []
    else:
        configs = [c for c in args.configs.split(",") if c]
        for c in configs:
            if c not in DESCRIPTIONS:
                ap.error(f"unknown config {c}")
    overrides = {"gate_up": json.loads(args.override_gate_up) if args.override_gate_up else {},
                 "down": json.loads(args.override_down) if args.override_down else {}}

    import numpy as np
    import torch
    from quantized_moe_align_amd import qma

    qma.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cache = WeightCache()
    flush = (torch.ones(FLUSH_BYTES // 4, dtype=torch.int32, device=dev)
             if args.flush and configs else None)

    # headline workload
    fused = args.activation == "fused"
    r = build_runner(args.workload, args.seed, cache, args.schedule, overrides, fused)
    m = measure(r, args.steps, args.warmup, args.settle_ms, args.idle_gap_ms)
    work, moe, ev = r["work"], r["moe"], m["ev"]
    ms_per_step = m["ms_per_step"]
    us = {k: float(np.mean(v)) for k, v in ev.items()}
    med = {k: float(np.median(v)) for k, v in ev.items()}
    hbm = args.workload in HBM_BOUND
    total_bytes = work["gate_up_bytes"] + work["down_bytes"]
    total_flops = work["gate_up_flops"] + work["down_flops"]
    traffic = read_traffic(args.workload)
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
    roof["traffic"] = traffic["gate_up"]
    roof["kernel"] = "gate_up GEMM (" + ("small-M" if moe.plan13.kernel == 1 else "large-M") + ")"
    sched = {"gate_up": qma.SCHEDULE_NAMES.get(moe.plan13.schedule, "?"),
             "down": qma.SCHEDULE_NAMES.get(moe.plan2.schedule, "?")}
    headline_plan = {"gate_up": moe.plan13.as_dict(), "down": moe.plan2.as_dict()}
    wl_main = r["wl"]
    del r, moe

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": unit, "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "warmup_settle_ms": args.settle_ms,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": DESCRIPTIONS[args.workload], "name": args.workload,
                   "rows": work["rows"], "weights": "uint4 group-32 bf16 scales, zero point 8",
                   "parallelism": "one EP/TP rank's share on one GPU",
                   "schedule": sched,
                   "activation": "fused into gate_up" if fused else "separate kernel",
                   **({"plan_overrides": overrides} if any(overrides.values()) else {}),
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
        "plan": headline_plan,
        "roofline": roof,
        "kernel_src_sha": kernel_src_hash(),
    }

    # every scenario of the pages, measured in the same run
    if configs:
        cfg_out = {}
        for name in configs:
            rc = build_runner(name, args.seed, cache, "planner", {}, fused)
            mc = measure(rc, args.steps, args.warmup, min(args.settle_ms, 150.0), flush=flush)
            rep = pair_report(name, rc["work"], mc["ev"], read_traffic(name))
            rep["ms_per_step"] = round(mc["ms_per_step"], 4)
            rep["workload"] = DESCRIPTIONS[name]
            rep["plan"] = {"gate_up": plan_brief(rc["moe"].plan13),
                           "down": plan_brief(rc["moe"].plan2)}
            if "ev_flushed" in mc:
                f = pair_report(name, rc["work"], mc["ev_flushed"], None)
                rep["flushed"] = {k: f[k] for k in ("us_mean", "pair_us", "pair_rate", "frac")}
            cfg_out[name] = rep
            del rc
            torch.cuda.synchronize()
        out["configs"] = cfg_out

    if args.cpu_budget > 0:
        threads, blas = _blas_info()
        t_cpu, b_cpu, f_cpu, experts = cpu_oracle(wl_main, args.cpu_budget)
        t_deq, t_mm, b32, f32, ex32 = cpu_fp32(wl_main, args.cpu_fp32_experts)

        def rate(b, f, t):
            return round((b / t / 1e9) if hbm else (f / t / 1e12), 4)
        out["cpu_baseline"] = {
            "value": rate(b_cpu, f_cpu, t_cpu), "unit": unit, "cores": threads, "kind": "oracle",
            "host": {**host_cpu(), "blas": blas},
            "sample": f"experts {experts[0]}..{experts[-1]} ({len(experts)} of "
                      f"{work['experts_with_rows']}) of the same workload: gate_up, activation "
                      f"and down per expert in float64 (the oracle), {t_cpu:.1f} s",
            "fp32": {"with_dequant": rate(b32, f32, t_deq), "matmul_only": rate(b32, f32, t_mm),
                     "unit": unit,
                     "sample": f"experts {ex32[0]}..{ex32[-1]} ({len(ex32)}), NumPy fp32 "
                               f"gate_up, SiLU-gated activation and down; median of 3 after "
                               f"1 warm-up: {t_deq:.2f} s with per-expert dequantisation, "
                               f"{t_mm:.3f} s on cached fp32 weights"}}
    else:
        out["cpu_baseline"] = None
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
