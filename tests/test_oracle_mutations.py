"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake in a copy of the oracle's C source (on the CPU,
in a temporary directory), builds it, and runs the pin tests against that
build in a subprocess: at least one pin must fail.
"""
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "moe_oracle.c")

# (name, exact text in the source, replacement)
MUTATIONS = [
    ("nibble order swapped",
     "(col & 1) ? (byte >> 4) : (byte & 0x0Fu)",
     "(col & 1) ? (byte & 0x0Fu) : (byte >> 4)"),
    ("E2M1 subnormal value",
     "(e == 0) ? 0.5 * (double)m", "(e == 0) ? 1.0 * (double)m"),
    ("E8M0 bias off by one",
     "ldexp(1.0, (int)(code & 0xFFu) - 127)", "ldexp(1.0, (int)(code & 0xFFu) - 126)"),
    ("scale block index",
     "(size_t)(col / 32)]", "(size_t)(col / 16) % (size_t)(K / 32)]"),
    ("gate and up swapped",
     "g = g + xv[kk] * orc_mxfp4_weight(gu_codes, gu_scales, d, n, kk);",
     "g = g + xv[kk] * orc_mxfp4_weight(gu_codes, gu_scales, d, f + n, kk);"),
    ("silu sign",
     "return z / (1.0 + exp(-z));", "return z / (1.0 + exp(z));"),
    ("router operand transposed",
     "router_w[(size_t)e * d + kk]", "router_w[(size_t)(e % T) * d + kk]"),
    ("router bias dropped",
     "(bias ? (double)bias[e] : 0.0)", "0.0"),
    ("router tree pairs wrong",
     "part[c] = part[c] + part[c + width];\n            double l = part[0]",
     "part[c] = part[c] + part[(c + 2 * width) % 64];\n            double l = part[0]"),
    ("router single running sum",
     "for (int width = 1; width < 64; width *= 2)\n                for",
     "for (int c = 1; c < 64; ++c) part[0] = part[0] + part[c];\n            for (int width = 64; width < 64; width *= 2)\n                for"),
    ("RMSNorm tree pairs wrong",
     "part[c] = part[c] + part[c + width];\n        double ms",
     "part[c] = part[c] + part[(c + 2 * width) % 64];\n        double ms"),
    ("top-k ties to higher index",
     "if (best < 0 || l[e] > l[best])", "if (best < 0 || l[e] >= l[best])"),
    ("softmax denominator misses a slot",
     "for (int j = 0; j < k; ++j)\n            denom +=",
     "for (int j = 1; j < k; ++j)\n            denom +="),
    ("permutation not stable",
     "for (int t = 0; t < T; ++t) {\n            for (int j = 0; j < k; ++j) {\n                int32_t r = t * k + j;",
     "for (int t = T - 1; t >= 0; --t) {\n            for (int j = 0; j < k; ++j) {\n                int32_t r = t * k + j;"),
    ("combine drops last slot",
     "for (int j = 0; j < k; ++j)\n            s = s + w[j] * o[(size_t)j * d + m];",
     "for (int j = 0; j + 1 < k; ++j)\n            s = s + w[j] * o[(size_t)j * d + m];"),
    ("bf16 rounding truncates",
     "double r = nearbyint(a / q) * q;", "double r = floor(a / q) * q;"),
    ("bf16 subnormal spacing",
     "qexp = -133;", "qexp = -126;"),
    ("MX shared exponent off by one",
     "X = (fe - 1) - F.emax;", "X = fe - F.emax;"),
    ("MX no saturation",
     "if (a >= F->maxval) {\n        v = F->maxval;\n    } else {",
     "{"),
    ("MX ties away from zero",
     "v = nearbyint(a / q) * q;", "v = round(a / q) * q;"),
    ("activation-MX mode: x not rounded",
     "    if (act)\n        orc_mx_round(ORC_FMT_E2M3, d, xv);", ""),
    ("activation-MX mode: h not rounded",
     "    if (act)\n        orc_mx_round(ORC_FMT_E2M3, f, h);", ""),
    ("FP8 block scale column index",
     "(size_t)(K / 128) + (size_t)(col / 128)]",
     "(size_t)(K / 128) + (size_t)(col / 64) % (size_t)(K / 128)]"),
    ("FP8 block scale row index",
     "scales[(size_t)(row / 128) * (size_t)(K / 128)",
     "scales[(size_t)((row / 64) % 2) * (size_t)(K / 128)"),
    ("FP8 expert gate and up swapped",
     "u = u + xv * orc_fp8_weight(gu_codes, gu_scales, d, f + n, kk);",
     "u = u + xv * orc_fp8_weight(gu_codes, gu_scales, d, n, kk);"),
    ("RMSNorm eps outside the square root",
     "double den = sqrt(ms + (double)eps);", "double den = sqrt(ms) + (double)eps;"),
    ("RMSNorm sum instead of mean",
     "double ms = part[0] / (double)d;", "double ms = part[0];"),
    ("RMSNorm gamma dropped",
     "double v = (orc_bf16_value(xr[i]) / den) * orc_bf16_value(gamma[i]);",
     "double v = (orc_bf16_value(xr[i]) / den);"),
    ("shared expert gate and up swapped",
     "g = g + xv * orc_bf16_value(sgu[(size_t)n * d + kk]);",
     "g = g + xv * orc_bf16_value(sgu[(size_t)(fs + n) * d + kk]);"),
    ("residual dropped",
     "double v = orc_bf16_value(x[i]) + y[i] + s[m];", "double v = y[i] + s[m];"),
    ("block routes the raw input",
     "layer_forward_impl(T, d, E, k, f, 0, xn_out, router_w",
     "layer_forward_impl(T, d, E, k, f, 0, x, router_w"),
]


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_mistake(name, old, new, tmp_path):
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation anchor not found exactly once: " + name
    mutated = tmp_path / "moe_oracle.c"
    mutated.write_text(src.replace(old, new))
    hdr = os.path.join(ROOT, "oracle", "moe_oracle.h")
    (tmp_path / "moe_oracle.h").write_text(open(hdr).read())
    so = tmp_path / "libmut.so"
    subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fopenmp", "-std=c11",
                           "-shared", "-fPIC", "-o", str(so), str(mutated), "-lm"])
    env = dict(os.environ, MOE_ORACLE_LIB=str(so))
    files = ["test_oracle_formats.py", "test_oracle_router.py", "test_oracle_ffn.py",
             "test_oracle_mx.py", "test_oracle_tail.py", "test_oracle_fp8.py"]
    # every pin file runs; the one aimed at the mutated function goes first,
    # so that -x stops early (a speed-up only: any failing pin counts)
    for key, f in (("FP8", "test_oracle_fp8.py"), ("RMSNorm", "test_oracle_tail.py"),
                   ("residual", "test_oracle_tail.py"), ("shared", "test_oracle_tail.py"),
                   ("block", "test_oracle_tail.py"), ("MX", "test_oracle_mx.py")):
        if key in name:
            files.remove(f)
            files.insert(0, f)
            break
    pins = [os.path.join(ROOT, "tests", f) for f in files]
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider"] + pins,
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, "no pin caught: " + name + "\n" + r.stdout[-2000:]
