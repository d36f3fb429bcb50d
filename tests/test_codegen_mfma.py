"""Code-generation invariants of the scaled-MFMA expert GEMM (CPU only).

The GEMM's weight and activation loads are inline asm, waited for by one
explicit vmcnt per K step, so the compiler does not know when their
destination registers are written.  That is only correct if (1) the main
loop never copies a vector register (a copy could read a register whose load
is still in flight) and (2) after the loop no instruction writes a register
that an in-flight load targets before the final vmcnt(0).  This test builds
the kernel source to gfx950 assembly with hipcc and checks both on the
kernels' main loop (the loop that holds the MFMAs).
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
    height the kernel dispatches to."""
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
        lp = [b for b in blocks if b is hb or ("Header=" + h) in b[1]]
        if any(x.startswith("v_mfma") for b in lp for x in b[2]):
            loops.append(lp)
    return loops, blocks


def _analyse_all(lines):
    loops, blocks = _loops(lines)
    assert len(loops) == 4, "expected one MFMA loop per tile height, found %d" % len(loops)
    return [_analyse_loop(lp, blocks) for lp in loops]


def _analyse_loop(loop, blocks):
    names = {b[0] for b in loop}
    body = [x for b in loop for x in b[2]]
    copies = [x for x in body if re.match(r"(v_mov_b32|v_accvgpr_\w+|scratch_\w+)\b", x)]
    dests = set()
    for x in body:
        if x.startswith("buffer_load"):
            dests |= _regs(x.split()[1].rstrip(","))
    exits = set()
    for b in loop:
        for x in b[2]:
            m = re.match(r"s_cbranch_\w+\s+(\.LBB\d+_\d+)|s_branch\s+(\.LBB\d+_\d+)", x)
            if m:
                t = m.group(1) or m.group(2)
                if t not in names:
                    exits.add(t)
    order = [b[0] for b in blocks]
    clobbers = []
    for t in exits:
        done = False
        for b in blocks[order.index(t):]:
            for x in b[2]:
                if "s_waitcnt vmcnt(0)" in x:
                    done = True
                    break
                m = re.match(r"(v_\w+)\s+(v\[\d+:\d+\]|v\d+)", x)
                if m and _regs(m.group(2)) & dests:
                    clobbers.append(x)
            if done:
                break
        assert done, "no vmcnt(0) on the loop exit path"
    return body, copies, dests, clobbers


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


# <gate/up?, one term (activation-MX mode)?>
KERNELS = ["ILb1ELb0E", "ILb1ELb1E", "ILb0ELb0E", "ILb0ELb1E"]
KERNEL_IDS = ["gate_up", "gate_up_single", "down", "down_single"]


def test_all_gemm_kernels_present(gemm_asm):
    assert len(_kernels(gemm_asm)) == 4


@pytest.mark.parametrize("which", KERNELS, ids=KERNEL_IDS)
def test_main_loops_have_no_register_copies(gemm_asm, which):
    (lines,) = [v for k, v in _kernels(gemm_asm).items() if which in k]
    for body, copies, dests, _ in _analyse_all(lines):
        assert sum(x.startswith("v_mfma") for x in body) > 0
        assert len(dests) >= 128, "weight ring registers not found"
        assert copies == [], copies[:5]


@pytest.mark.parametrize("which", KERNELS, ids=KERNEL_IDS)
def test_in_flight_registers_untouched_until_drained(gemm_asm, which):
    (lines,) = [v for k, v in _kernels(gemm_asm).items() if which in k]
    for _, _, _, clobbers in _analyse_all(lines):
        assert clobbers == [], clobbers[:5]


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
