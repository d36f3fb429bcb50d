"""Resource invariants of the decode-sized expert kernels (CPU only).

The GEMV and fused down+combine kernels hide memory latency with the loads
of several waves in flight, so their speed rests on how many waves fit on a
SIMD; the fused down+combine keeps several batches of rows in flight per
wave, which costs registers, and its 8-wave blocks must still fit two waves
per SIMD.  This test builds ffn_gemv.hip for gfx950 with the
compiler's resource-usage remarks and checks that no kernel spills to
scratch and that the kernels keep the occupancy the launches are sized for.
"""
import os
import re
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "routed_expert_mxfp4_amd", "csrc", "ffn_gemv.hip")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.fixture(scope="module")
def resources():
    hipcc = HIPCC if os.path.exists(HIPCC) else shutil.which("hipcc")
    if hipcc is None:
        pytest.skip("hipcc not available")
    with tempfile.TemporaryDirectory() as td:
        cmd = [hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature",
               "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"),
               "--cuda-device-only", "-c", "-o", os.path.join(td, "x.o"), SRC,
               "-Rpass-analysis=kernel-resource-usage"]
        err = subprocess.run(cmd, check=True, capture_output=True, text=True).stderr
    out, cur = {}, None
    for line in err.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            cur = m.group(1)
            out[cur] = {}
            continue
        if cur is None:
            continue
        for key, pat in (("vgpr", r"VGPRs: (\d+)"), ("agpr", r"AGPRs: (\d+)"),
                         ("scratch", r"ScratchSize \[bytes/lane\]: (\d+)"),
                         ("occupancy", r"Occupancy \[waves/SIMD\]: (\d+)")):
            m = re.search(pat, line)
            if m:
                out[cur][key] = int(m.group(1))
    return out


def _of(res, pattern):
    found = {k: v for k, v in res.items() if re.search(pattern, k)}
    assert found, "no kernel matches %s" % pattern
    return found


def test_no_kernel_spills(resources):
    assert resources
    for name, r in resources.items():
        assert r.get("scratch", 0) == 0, name


def test_fused_down_combine_8_wave_blocks_fit(resources):
    # 8-wave blocks (two waves per SIMD, at most 256 registers per lane);
    # the one-MX-block-per-lane variants with their ring of three batches
    # stay at three waves per SIMD
    for name, r in _of(resources, r"down_combine_split_kernelILi\d+ELi\d+ELi4ELi\dELi8E").items():
        assert r["occupancy"] >= 2, (name, r)
    for name, r in _of(resources, r"down_combine_split_kernelILi1ELi\d+ELi4ELi3ELi8E").items():
        assert r["occupancy"] >= 3, (name, r)


def test_decode_gate_up_two_blocks_per_cu(resources):
    # one-token gate/up: 4-wave blocks, two resident per CU at least
    for name, r in _of(resources, r"gate_up_mfma_token_kernel").items():
        assert r["occupancy"] >= 2, (name, r)


def test_one_row_down_gemv_keeps_four_waves(resources):
    # the few-token down GEMV over one-MX-block-per-lane rows (f <= 2048)
    # streams at four waves per SIMD; both variants (one row at a time,
    # several rows through LDS) keep that
    for name, r in _of(resources, r"down_rows_kernelILi1E").items():
        assert r["occupancy"] >= 4, (name, r)
