"""Code-generation invariants of filtered routing (CPU only).

The certified interval of the routing filter assumes that the bf16 MFMA
logits are built from sums of at most 64 products: each 64-wide K stage is
two chained MFMAs, the first from a zero accumulator, and the stage sums are
added in fp32 on the vector ALU.  A compiler that folded those adds back
into the accumulator chain would silently widen the error past the bound.
This test builds route_filter.hip to gfx950 assembly and checks, in the
filter GEMM, that every MFMA either starts from the literal 0 or continues a
chain that a zero-start MFMA began (chains of exactly two), and that the
stage sums meet on v_add_f32.  It also checks that the selection and refine
kernels keep spills out of their loops.
"""
import os
import re
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "routed_expert_mxfp4_amd", "csrc", "route_filter.hip")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.fixture(scope="module")
def asm():
    if not (os.path.exists(HIPCC) or shutil.which("hipcc")):
        pytest.skip("hipcc not available")
    with tempfile.TemporaryDirectory() as td:
        out = os.path.join(td, "rf.s")
        cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature",
               "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"),
               "--cuda-device-only", "-S", SRC, "-o", out]
        r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
        assert r.returncode == 0, r.stderr[-2000:]
        return open(out).read()


def _kernel(asm, pattern):
    out = {}
    cur = None
    for line in asm.splitlines():
        m = re.match(r"^(_Z\S*" + pattern + r"\S*):", line)
        if m:
            cur = m.group(1)
            out[cur] = []
            continue
        if cur and line.startswith(".Lfunc_end"):
            cur = None
            continue
        if cur:
            out[cur].append(line.strip())
    return out


def test_filter_gemm_stage_chains(asm):
    ks = _kernel(asm, "filter_gemm_kernel")
    assert len(ks) == 1
    lines = next(iter(ks.values()))
    chain = {}
    zero_start = chained = 0
    for x in lines:
        if not x.startswith("v_mfma"):
            continue
        ops = [o.strip() for o in x.split(None, 1)[1].split(",")]
        dst, c = ops[0], ops[3]
        if c == "0":
            chain[dst] = 1
            zero_start += 1
        else:
            assert chain.get(c) == 1, "MFMA accumulates onto %s, not a fresh stage start: %s" % (c, x)
            chain[c] = 0                       # consumed: may not be extended again
            chain[dst] = 2
            chained += 1
    assert zero_start > 0 and zero_start == chained, (zero_start, chained)
    n_add = sum(1 for x in lines if x.startswith("v_add_f32"))
    assert n_add >= 4 * zero_start, n_add
    assert not any(x.startswith("v_pk_add_f32") for x in lines)


def _resource(asm, name, what):
    m = re.search(r"\.set " + re.escape(name) + r"\." + what + r", (\d+)", asm)
    assert m, (name, what)
    return int(m.group(1))


def _loop_lines(lines):
    """Instructions of the basic blocks that belong to a loop."""
    out, inloop = [], False
    for x in lines:
        if re.match(r"^(\.LBB\d+_\d+:|; %bb\.\d+:)", x):
            inloop = "Loop" in x
            continue
        if inloop:
            out.append(x)
    return out


def test_route_filter_kernels_do_not_spill(asm):
    sel = _kernel(asm, "select_cand_kernel")
    ref = _kernel(asm, "refine_topk_kernel")
    assert len(sel) == 3 and len(ref) == 3, (list(sel), list(ref))
    for name in list(sel) + [k for k in ref if "ILi14E" not in k]:
        assert _resource(asm, name, "private_seg_size") == 0, name
    # the 14-chunk refine (d = 7168) is held to four waves per SIMD; the few
    # bytes it may then spill stay out of its loops
    big = [k for k in ref if "ILi14E" in k]
    assert len(big) == 1
    assert _resource(asm, big[0], "num_vgpr") + _resource(asm, big[0], "num_agpr") <= 128
    assert _resource(asm, big[0], "private_seg_size") <= 16
    body = _loop_lines(ref[big[0]])
    assert any(x.startswith("v_fma_f64") for x in body)
    assert not any(x.startswith("scratch_") for x in body)
