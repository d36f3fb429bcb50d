"""Code-generation invariants of the scaled-MFMA expert GEMM (CPU only).

The GEMM moves every operand global -> LDS with inline-asm buffer loads that
write LDS directly, waited for by an explicit vmcnt(0) and a barrier at the
top of each K step; the compiler sees none of them.  That is only correct if
the kernels' MFMA loops hold no vector-memory load into registers (whose
wait the compiler would place on its own), and the design relies on two
waves per SIMD (no scratch, at most 256 registers).  This test builds the
kernel source to gfx950 assembly with hipcc and checks the MFMA loops (one
per tile height, two for 16-row tiles) and the resource use.
"""
import os
import re
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "routed_expert_mxfp4_amd", "csrc", "ffn_mfma.hip")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _regs(tok):
    m = re.match(r"v\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def _kernels(asm):
    out, cur = {}, None
    for line in asm.splitlines():
        m = re.match(r"^(_Z\S*ffn_mfma_kernel\S*):", line)
        if m:
            cur = m.group(1)
            out[cur] = []
            continue
        if cur and line.startswith(".Lfunc_end"):
            cur = None
            continue
        if cur:
            out[cur].append(line)
    return out


def _loops(lines):
    """Every loop holding MFMAs, as (blocks, all blocks) -- one per tile
    height the kernel dispatches to (two for 16-row tiles)."""
    blocks, cur = [], None
    for line in lines:
        m = re.match(r"^(\.LBB\d+_\d+):(.*)$", line)
        if m:
            cur = [m.group(1), m.group(2), []]
            blocks.append(cur)
            continue
        if cur is not None:
            cur[2].append(line.strip())
    loops = []
    for hb in [b for b in blocks if "Loop Header" in b[1]]:
        h = hb[0].replace(".LBB", "BB")
        lp = [b for b in blocks if b is hb or re.search(r"Header=%s\b" % h, b[1])]
        if any(x.startswith("v_mfma") for b in lp for x in b[2]):
            loops.append(lp)
    return loops, blocks


@pytest.fixture(scope="module")
def gemm_asm():
    if not os.path.exists(HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("hipcc not available")
    hipcc = HIPCC if os.path.exists(HIPCC) else shutil.which("hipcc")
    with tempfile.TemporaryDirectory() as td:
        out = os.path.join(td, "ffn_mfma.s")
        cmd = [hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature",
               "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"),
               "--cuda-device-only", "-S", "-o", out, SRC]
        subprocess.run(cmd, check=True, capture_output=True)
        return open(out).read()


@pytest.fixture(scope="module")
def gemm_resources():
    if not os.path.exists(HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("hipcc not available")
    hipcc = HIPCC if os.path.exists(HIPCC) else shutil.which("hipcc")
    with tempfile.TemporaryDirectory() as td:
        cmd = [hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature",
               "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"),
               "--cuda-device-only", "-c", "-o", os.path.join(td, "x.o"), SRC,
               "-Rpass-analysis=kernel-resource-usage"]
        err = subprocess.run(cmd, check=True, capture_output=True, text=True).stderr
    out, cur = {}, None
    for line in err.splitlines():
        m = re.search(r"Function Name: (\S*ffn_mfma_kernel\S*)", line)
        if m:
            cur = m.group(1)
            out[cur] = {}
            continue
        if cur is None:
            continue
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m:
            out[cur]["scratch"] = int(m.group(1))
        m = re.search(r"Occupancy \[waves/SIMD\]: (\d+)", line)
        if m:
            out[cur]["occupancy"] = int(m.group(1))
            cur = None
    assert len(out) == 4, out
    return out


# <gate/up?, one term (activation-MX mode)?>
KERNELS = ["ILb1ELb0E", "ILb1ELb1E", "ILb0ELb0E", "ILb0ELb1E"]
KERNEL_IDS = ["gate_up", "gate_up_single", "down", "down_single"]


def test_all_gemm_kernels_present(gemm_asm):
    assert len(_kernels(gemm_asm)) == 4


@pytest.mark.parametrize("which", KERNELS, ids=KERNEL_IDS)
def test_mfma_loops_load_only_into_lds(gemm_asm, which):
    (lines,) = [v for k, v in _kernels(gemm_asm).items() if which in k]
    loops, _ = _loops(lines)
    # one per tile height, two for 16-row tiles (super-steps on the
    # canonical store, the one-step deep ring otherwise)
    assert len(loops) == 5, "expected five MFMA loops, found %d" % len(loops)
    for lp in loops:
        body = [x for b in lp for x in b[2]]
        assert sum(x.startswith("v_mfma_scale") for x in body) > 0
        loads = [x for x in body if re.match(r"(buffer|global|flat)_load", x)]
        assert loads and all(x.rstrip().endswith(" lds") for x in loads), loads[:5]
        assert not [x for x in body if x.startswith("scratch_")]
        # the step's wait: every load of the wave, then the barrier
        i = next(i for i, x in enumerate(body) if x.startswith("s_barrier"))
        assert any("vmcnt(0)" in x for x in body[:i]), body[:i]


def test_two_waves_per_simd(gemm_resources):
    for name, res in gemm_resources.items():
        assert res["scratch"] == 0, name
        assert res["occupancy"] >= 2, (name, res)


def test_fp6_conversions_do_not_overlap_their_sources(gemm_asm):
    """The gfx950 scaled FP6 pack/unpack instructions write their first
    result registers before reading all of their sources: a destination
    that overlaps a source register corrupts elements.  Every such
    instruction in the file (the activation split kernels and the gate/up
    epilogue) must have disjoint destination and source registers."""
    seen = 0
    for line in gemm_asm.splitlines():
        m = re.match(r"\s*(v_cvt_scalef32_\S+)\s+(.*)$", line)
        if not m:
            continue
        ops = [o.strip() for o in m.group(2).split(";")[0].split(",")]
        dst = _regs(ops[0])
        for src in ops[1:]:
            assert not (dst & _regs(src)), line.strip()
        seen += 1
    assert seen >= 6, "conversion instructions not found"
