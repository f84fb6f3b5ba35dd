"""bench.py contract on the host: one-GPU refusal, workload coverage, and the
committed rocprofv3 traffic summaries it reads."""
import glob
import importlib.util
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def test_every_workload_has_a_bench_description():
    from quantized_moe_align_amd import inputs
    bench = _bench()
    assert set(inputs.WORKLOADS) <= set(bench.DESCRIPTIONS)
    assert bench.HBM_BOUND <= set(bench.DESCRIPTIONS)


def test_traffic_summaries_parse():
    files = sorted(glob.glob(os.path.join(ROOT, "profiles", "pmc_gate_up_*.md")))
    assert files
    for f in files:
        lines = [l for l in open(f) if l.startswith("qma-traffic: ")]
        assert len(lines) == 1, f
        d = json.loads(lines[0][len("qma-traffic: "):])
        assert d["workload"] in os.path.basename(f)
        assert d["bytes_per_launch"] > 0 and d["read_factor"] > 0 and d["write_factor"] > 0
        assert len(d["src_sha"]) == 16


def test_algorithmic_work_per_expert_and_per_row():
    # W4-g32 costs N*K*9/16 bytes of packed weights and scales per expert and
    # GEMM; 2*N*K flops per routed row and GEMM. At the EP8 shapes (hidden
    # 7168, intermediate 2048) that is 16,515,072 + 8,257,536 bytes per expert
    # and 88,080,384 flops per row; at the TP8 share (intermediate 256)
    # 2,064,384 + 1,032,192 bytes and 11,010,048 flops.
    from quantized_moe_align_amd import inputs
    bench = _bench()
    for name, gu_e, dn_e, fl_row in (("ep8_decode", 16515072, 8257536, 88080384),
                                     ("tp8", 2064384, 1032192, 11010048),
                                     ("masked", 16515072, 8257536, 88080384)):
        wl = inputs.make(name, seed=0, weights=False)
        w = bench.algorithmic_work(wl)
        K, I, ne, rows = wl.K, wl.I, w["experts_with_rows"], w["rows"]
        a_rows = rows if name != "tp8" else wl.T
        assert w["gate_up_bytes"] == ne * gu_e + a_rows * K * 2 + rows * 2 * I * 2, name
        assert w["down_bytes"] == ne * dn_e + rows * I * 2 + rows * K * 2, name
        assert w["gate_up_flops"] + w["down_flops"] == rows * fl_row, name
