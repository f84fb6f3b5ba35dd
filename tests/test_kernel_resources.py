"""Register budget of every compiled GEMM instance (CPU: hipcc cross-compiles).

The kernel file is compiled for gfx950 with the library's own device flags
and the compiler's per-kernel resource remarks. Every kernel the planner or
an edited plan can launch must run without scratch: a spilled VGPR turns
into a private-memory round trip inside the K loop. The shared-row small-M
instances must also fit the workgroups per compute unit they are built for
(four: at most 128 VGPRs and a quarter of the LDS; three for the 32-row,
4-tile instance), the gang instances one workgroup of three groups, and the
stream-K instances one workgroup of four (three at 256 columns) groups.
"""
import os
import re
import shutil
import subprocess

import pytest

from quantized_moe_align_amd import build

KERNELS = os.path.join(build.HERE, "csrc", "qma_kernels.hip")


def _remarks(tmp_path):
    hipcc = build.hipcc()
    out = tmp_path / "k.o"
    cmd = [hipcc, f"--offload-arch={build.ARCH}", "-O3", "-std=c++17", "-fPIC",
           *build.DEVICE_FLAGS, "-I", os.path.join(build.ROOT, "include"),
           "--cuda-device-only", "-c", KERNELS, "-o", str(out),
           "-Rpass-analysis=kernel-resource-usage"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    kernels, cur = {}, None
    for line in res.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            cur = kernels.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+([^:\[]+?)(?: \[bytes/[a-z]+\]| \[waves/SIMD\])?: (\d+)", line)
        if m and cur is not None:
            cur[m.group(1).strip()] = int(m.group(2))
    return kernels


@pytest.fixture(scope="module")
def resources(tmp_path_factory):
    if not (shutil.which("hipcc") or os.path.exists("/opt/rocm/bin/hipcc")):
        pytest.skip("hipcc not available")
    return _remarks(tmp_path_factory.mktemp("ru"))


def test_every_kernel_reports(resources):
    names = " ".join(resources)
    for k in ("gemm_small_m_xs_kernel", "gemm_small_m_xs_dyn_kernel",
              "gemm_small_m_xs_gang_kernel", "gemm_small_m_sk_kernel", "gemm_small_m_kernel",
              "gemm_small_m_stream_kernel", "gemm_large_m_kernel", "gemm_large_m_pc_kernel",
              "splitk_reduce_kernel", "moe_align_kernel"):
        assert k in names, k
    for name, r in resources.items():
        assert "ScratchSize" in r and "VGPRs" in r, name


def test_no_kernel_uses_scratch(resources):
    bad = {n: (r.get("VGPRs"), r.get("VGPRs Spill"), r["ScratchSize"])
           for n, r in resources.items() if r["ScratchSize"] or r.get("VGPRs Spill", 0)}
    assert not bad, bad


def test_shared_row_instances_fit_their_occupancy(resources):
    # four workgroups per CU, three for the 32-row 4-tile instance
    xs = {n: r for n, r in resources.items() if "gemm_small_m_xs_kernel" in n}
    assert len(xs) == 5, sorted(xs)            # (1,2) (1,4) (2,2) (2,4) (4,2)
    for n, r in xs.items():
        per_cu = 3 if "ILi2ELi4E" in n else 4
        assert r["VGPRs"] <= 512 // per_cu // 8 * 8, (n, r["VGPRs"])
        assert r["LDS Size"] <= 160 * 1024 // per_cu, (n, r["LDS Size"])


def test_gang_instances_fit_one_workgroup_per_cu(resources):
    # three four-wave groups per workgroup: three waves per SIMD, so at most
    # 512 // 3 VGPRs rounded down to the allocation granule, and the groups'
    # LDS within one CU's 160 KiB
    gang = {n: r for n, r in resources.items() if "gemm_small_m_xs_gang_kernel" in n}
    assert len(gang) == 5, sorted(gang)
    for n, r in gang.items():
        assert r["VGPRs"] <= 512 // 3 // 8 * 8, (n, r["VGPRs"])
        assert r["LDS Size"] <= 160 * 1024, (n, r["LDS Size"])


def test_stream_k_instances_fit_one_workgroup_per_cu(resources):
    # four four-wave groups for the 128-column instances (at most 128 VGPRs),
    # three for the 256-column ones; the groups' LDS within one CU's 160 KiB
    sk = {n: r for n, r in resources.items() if "gemm_small_m_sk_kernel" in n}
    assert len(sk) == 4, sorted(sk)
    for n, r in sk.items():
        groups = 3 if "Li4ELi3EE" in n else 4
        assert r["VGPRs"] <= 512 // groups // 8 * 8, (n, r["VGPRs"])
        assert r["LDS Size"] <= 160 * 1024, (n, r["LDS Size"])

