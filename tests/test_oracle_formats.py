"""Pins for the oracle's scalar formats, byte layout and bf16 rounding.

Each check compares the oracle against something other than itself: the
OCP table of E2M1 values, closed forms, torch's own bf16 conversion, an
exhaustive brute-force nearest search, and byte counts printed on the pages.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from routed_expert_mxfp4_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _e2m1_table():
    vals = {}
    with open(os.path.join(GOLDEN, "e2m1_ocp.txt")) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            c, v = line.split()
            vals[int(c, 16)] = float(v)
    return vals


def test_e2m1_all_codes_match_ocp_table():
    table = _e2m1_table()
    assert len(table) == 16
    for code, v in table.items():
        got = oracle.e2m1_value(code)
        assert got == v, (code, got, v)
    # code 8 is negative zero: numerically zero
    assert oracle.e2m1_value(8) == 0.0


def test_e8m0_all_codes_closed_form():
    for s in range(255):
        assert oracle.e8m0_value(s) == math.ldexp(1.0, s - 127)
    assert math.isnan(oracle.e8m0_value(255))
    # code 0 is 2^-127: subnormal in fp32 but exact in fp64
    assert oracle.e8m0_value(0) == 2.0 ** -127


def test_mxfp4_weight_all_code_scale_pairs():
    # every (code, scale) pair through the packed layout, both nibbles
    table = _e2m1_table()
    K = 64
    for s in range(0, 255, 1):
        codes = np.zeros((1, K // 2), np.uint8)
        for i in range(16):
            codes[0, i] = (i << 4) | ((15 - i) & 0xF)   # odd col = high nibble
        scales = np.array([[s, (s + 1) % 255]], np.uint8)
        for col in range(32):
            code = (codes[0, col // 2] >> 4) if col & 1 else (codes[0, col // 2] & 0xF)
            want = table[int(code)] * math.ldexp(1.0, s - 127)
            assert oracle.mxfp4_weight(codes, scales, K, 0, col) == want


def test_bf16_value_exhaustive_vs_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.bf16_array_to_f64(bits)
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()


def _bf16_sorted_positive():
    bits = np.arange(0, 0x7F81, dtype=np.uint32)          # +0 .. +inf
    vals = (bits << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    return bits.astype(np.uint16), vals


def _brute_round_bf16(v):
    """Nearest bf16 to v, ties to even, by search over all positive bf16."""
    bits, vals = _bf16_sorted_positive()
    a = abs(v)
    sign = 0x8000 if math.copysign(1.0, v) < 0 else 0
    max_finite = vals[-2]
    # overflow: at or beyond max + half an ulp rounds to infinity
    half_ulp_top = Fraction(vals[-2]) + (Fraction(vals[-2]) - Fraction(vals[-3])) / 2
    if Fraction(a) >= half_ulp_top:
        return sign | 0x7F80
    i = int(np.searchsorted(vals[:-1], a))
    if i < len(vals) - 1 and vals[i] == a:
        return sign | int(bits[i])
    lo, hi = i - 1, i
    if hi == len(vals) - 1:          # above the largest finite, below overflow
        return sign | int(bits[lo])
    dlo = Fraction(a) - Fraction(vals[lo])
    dhi = Fraction(vals[hi]) - Fraction(a)
    if dlo < dhi:
        return sign | int(bits[lo])
    if dhi < dlo:
        return sign | int(bits[hi])
    return sign | int(bits[lo] if bits[lo] % 2 == 0 else bits[hi])


def test_round_to_bf16_brute_force():
    rng = np.random.default_rng(123)
    cases = list(rng.standard_normal(300) * 10.0 ** rng.integers(-40, 38, 300))
    # exact ties between two bf16 neighbours (tie to even both ways)
    for b in (0x3F80, 0x3F81, 0x4049, 0x0001, 0x0080, 0x7F7E):
        lo = float(np.uint32(b << 16).view(np.float32))
        hi = float(np.uint32((b + 1) << 16).view(np.float32))
        cases += [(lo + hi) / 2, -(lo + hi) / 2, np.nextafter((lo + hi) / 2, 0),
                  np.nextafter((lo + hi) / 2, 1e300)]
    # subnormal range, the smallest subnormal and values below half of it
    cases += [2.0 ** -133, 2.0 ** -134, 2.0 ** -134 * 1.0000001, 3 * 2.0 ** -135,
              2.0 ** -126 * 0.75, 1e-45, 1e-300, 3.3895313892515355e38,
              3.39e38, 3.4e38, 1.0 + 2.0 ** -9, 1.0 + 2.0 ** -9 + 2.0 ** -40,
              2.0 ** 128 - 2.0 ** 119, np.nextafter(2.0 ** 128 - 2.0 ** 119, 0)]
    for v in cases:
        v = float(v)
        assert oracle.round_to_bf16(v) == _brute_round_bf16(v), v


def test_round_to_bf16_matches_torch_on_fp32_inputs():
    # for inputs already representable in fp32 there is no double rounding,
    # so torch's fp32 -> bf16 conversion (RNE) is an independent reference
    rng = np.random.default_rng(7)
    f32 = rng.integers(0, 2 ** 32, 20000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    f32 = f32[np.isfinite(f32)]
    ref = torch.from_numpy(f32.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    for v, r in zip(f32[:4000], ref[:4000]):
        assert oracle.round_to_bf16(float(v)) == int(r)


def test_expert_byte_count_matches_pages():
    g = json.load(open(os.path.join(GOLDEN, "page_byte_counts.json")))
    per_expert = g["canonical_expert_store_bytes"] // g["routed_experts"]
    assert per_expert * g["routed_experts"] == g["canonical_expert_store_bytes"]
    assert g["routed_experts"] == g["routed_layers"] * g["experts_per_layer"]
    cfg = synth.CONFIGS[1]
    assert cfg.expert_bytes == per_expert == 17547264
    # decoded slot printed as 16.734 MiB
    assert round(per_expert / 2 ** 20, 3) == g["decoded_slot_mib"]
    # cache sizes: slots x layers x expert bytes
    assert round(32 * 92 * per_expert / 2 ** 30, 2) == g["cache_32_slots_gib"]
    assert round(30 * 92 * per_expert / 2 ** 30, 3) == g["cache_30_slots_gib"]
    # the generator's tensors add up to the same bytes
    sizes = synth.expert_sizes(cfg)
    assert sum(a * b for a, b in sizes.values()) == per_expert
    # one expert's 2*3*d*f is the page's "~66 MFLOPs"; d = 7168 is "7KB/hop"
    assert round(2 * 3 * cfg.d * cfg.f / 1e6) == g["mflops_per_token_claim"]
    assert round(cfg.d / 1024) == g["hop_kb"]
