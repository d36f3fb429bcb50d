"""Pins for the oracle's OCP MX conversion model (E4M3 / E2M3 / E2M1).

References: the element grids enumerated from the format definitions (sign,
exponent and mantissa fields), a brute-force nearest-grid-point search with
ties to even, the shared-exponent rule computed with math.frexp, and exact
rational arithmetic for the two-term split.  Inputs cover every bf16 value.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle

FORMATS = {
    # fmt: (ebits, mbits, bias, emax, maxval)
    oracle.FMT_E4M3: (4, 3, 7, 8, 448.0),
    oracle.FMT_E2M3: (2, 3, 1, 2, 7.5),
    oracle.FMT_E2M1: (2, 1, 1, 2, 6.0),
}


def _grid(fmt):
    """Every finite non-negative code of the format and its value, from the
    field definitions (independent of the oracle's decoder)."""
    eb, mb, bias, _, maxval = FORMATS[fmt]
    out = []
    for e in range(1 << eb):
        for m in range(1 << mb):
            if e == 0:
                v = m / (1 << mb) * 2.0 ** (1 - bias)
            else:
                v = (1 + m / (1 << mb)) * 2.0 ** (e - bias)
            if v <= maxval:
                out.append(((e << mb) | m, v))
    return out


@pytest.mark.parametrize("fmt", list(FORMATS))
def test_elem_value_matches_field_definition(fmt):
    eb, mb, *_ = FORMATS[fmt]
    for code, v in _grid(fmt):
        assert oracle.elem_value(fmt, code) == v
        assert oracle.elem_value(fmt, code | (1 << (eb + mb))) == -v


def _brute_nearest_codes(fmt, r):
    """Nearest grid code to each r (ties: even code), saturating, by a
    distance search over the whole grid (numpy, vectorised)."""
    eb, mb, _, _, maxval = FORMATS[fmt]
    grid = _grid(fmt)
    gc = np.array([c for c, _ in grid])
    gv = np.array([v for _, v in grid])
    a = np.abs(r)
    D = np.abs(a[:, None] - gv[None, :])
    mins = D.min(axis=1)
    cand = D == mins[:, None]
    # among equally near candidates prefer the even code
    score = np.where(cand, np.where(gc[None, :] % 2 == 0, 2, 1), 0)
    pick = gc[np.argmax(score, axis=1)]
    top = gc[np.argmax(gv)]
    pick = np.where(a >= maxval, top, pick)
    sign = np.where(np.signbit(r), 1 << (eb + mb), 0)
    return (sign | pick).astype(np.uint8)


def _all_bf16_finite():
    bits = np.arange(65536, dtype=np.uint32)
    v = (bits << 16).astype(np.uint32).view(np.float32)
    return v[np.isfinite(v)]


@pytest.mark.parametrize("fmt", list(FORMATS))
def test_scale_rule_every_bf16_amax(fmt):
    emax = FORMATS[fmt][3]
    for v in _all_bf16_finite():
        blk = np.zeros(32)
        blk[5] = v
        sc, codes = oracle.mx_quantize_block(fmt, blk)
        if v == 0:
            assert sc == 0
            continue
        m, e = math.frexp(abs(float(v)))
        X = min(max(e - 1 - emax, -127), 127)
        assert sc == X + 127, v


@pytest.mark.parametrize("fmt", list(FORMATS))
def test_elements_are_nearest_grid_points_every_bf16(fmt):
    # every finite bf16 value of magnitude <= the block maximum, for several
    # block maxima (the maximum sets the shared exponent)
    vals = _all_bf16_finite().astype(np.float64)
    emax = FORMATS[fmt][3]
    for anchor in [1.0, 448.0, 7.5, 2.0 ** -20, 3.0e4, 6.0]:
        sel = vals[np.abs(vals) <= anchor]
        m, e = math.frexp(anchor)
        X = min(max(e - 1 - emax, -127), 127)
        want = _brute_nearest_codes(fmt, np.ldexp(sel, -X))
        got = np.empty(sel.size, np.uint8)
        for i0 in range(0, sel.size, 31):
            chunk = sel[i0:i0 + 31]
            blk = np.zeros(32)
            blk[0] = anchor
            blk[1:1 + chunk.size] = chunk
            sc, codes = oracle.mx_quantize_block(fmt, blk)
            assert sc == X + 127
            got[i0:i0 + chunk.size] = codes[1:1 + chunk.size]
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, (anchor, sel[bad[:5]], got[bad[:5]], want[bad[:5]])


@pytest.mark.parametrize("fmt", [oracle.FMT_E4M3, oracle.FMT_E2M3])
def test_saturation(fmt):
    maxval = FORMATS[fmt][4]
    emax = FORMATS[fmt][3]
    # amax just below the next power of two: v / 2^X lies in [2^emax, 2^(emax+1))
    # and everything above maxval saturates to maxval
    blk = np.array([2.0 ** (emax + 1) * (1 - 2.0 ** -8)] + [0.0] * 31)
    sc, codes = oracle.mx_quantize_block(fmt, blk)
    assert sc == 127
    assert oracle.elem_value(fmt, codes[0]) == maxval


@pytest.mark.parametrize("fmt", [oracle.FMT_E4M3, oracle.FMT_E2M3])
def test_two_term_split_is_exact_residual(fmt):
    rng = np.random.default_rng(17 + fmt)
    x = (rng.standard_normal((6, 64)) * np.exp(rng.standard_normal((6, 64)) * 2)).astype(np.float32)
    x[0, :32] = 0.0                                  # all-zero block
    hs, hc, ls, lc = oracle.mx_split_rows(fmt, x)
    assert hs[0, 0] == 0 and (hc[0, :32] & 0x7F == 0).all()
    for r in range(x.shape[0]):
        for b in range(2):
            blk = x[r, 32 * b:32 * b + 32].astype(np.float64)
            s_hi = Fraction(2) ** (int(hs[r, b]) - 127)
            s_lo = Fraction(2) ** (int(ls[r, b]) - 127)
            hi = [Fraction(oracle.elem_value(fmt, c)) * s_hi for c in hc[r, 32 * b:32 * b + 32]]
            # the residual is formed exactly and is itself MX-quantised
            res = np.array([float(Fraction(float(v)) - h) for v, h in zip(blk, hi)])
            sc, codes = oracle.mx_quantize_block(fmt, res)
            assert sc == ls[r, b]
            np.testing.assert_array_equal(codes, lc[r, 32 * b:32 * b + 32])
            lo = [Fraction(oracle.elem_value(fmt, c)) * s_lo for c in codes]
            # two terms reconstruct to within half a quantum of the residual grid
            amax_res = max(abs(v) for v in res)
            for v, h, l in zip(blk, hi, lo):
                err = abs(Fraction(float(v)) - h - l)
                assert err <= Fraction(amax_res) / 8 + Fraction(0)
