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
