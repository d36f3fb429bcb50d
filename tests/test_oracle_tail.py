"""Pins of the oracle's MoE tail: the RMSNorm before the router, the shared
expert and the residual add of the pre-norm block (CPU only).

* RMSNorm: against an exact evaluation (rational sum of squares, 80-digit
  square root and quotient, exact nearest-even choice on the bf16 grid), on
  rows whose scale runs from where eps dominates to where it vanishes; plus
  the exact scale invariance at eps = 0 and a constant row.
* Shared expert: against the dense SwiGLU MLP written with numpy matmuls.
* Block: the special cases that isolate each term -- all-zero routed experts
  and no shared expert give exactly the residual; zero routed experts leave
  the residual plus the shared expert; the routed part and the routing are
  those of the routed layer on the normalised input.
"""
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest

import oracle


def _bf16_bits_to_f64(b):
    return (np.asarray(b, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


def _f64_to_bf16_bits(v):
    """Round fp64 -> bf16 through fp32 (only used on values that are exactly
    representable in fp32, e.g. draws)."""
    return (np.asarray(v, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _rand_bf16(rng, shape, scale=1.0):
    v = (rng.standard_normal(shape) * scale).astype(np.float32)
    # round to nearest even bf16 via the fp32 bits
    u = v.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def _exact_bf16_of(v: Decimal):
    """Nearest bf16 (ties to even) of a high-precision value, with the
    distance of the value from the nearest tie point (in quanta)."""
    if v == 0:
        return 0, Decimal(1)
    sign = 0x8000 if v < 0 else 0
    a = abs(v)
    e = 0
    # a in [2^e, 2^(e+1))
    while Decimal(2) ** e > a:
        e -= 1
    while Decimal(2) ** (e + 1) <= a:
        e += 1
    qexp = max(e - 7, -133)
    r = a / (Decimal(2) ** qexp)
    n = int(r)                       # floor for positive r
    frac = r - n
    tie_dist = abs(frac - Decimal("0.5"))
    if frac > Decimal("0.5") or (frac == Decimal("0.5") and n % 2 == 1):
        n += 1
    val = Fraction(n) * Fraction(2) ** qexp
    bits = np.array([float(val)], dtype=np.float32).view(np.uint32)[0] >> 16
    return sign | int(bits), tie_dist


def _exact_rmsnorm_row(xb, gb, eps):
    getcontext().prec = 80
    xs = [Fraction(float(v)) for v in _bf16_bits_to_f64(xb)]
    gs = [Decimal(float(v)) for v in _bf16_bits_to_f64(gb)]
    d = len(xs)
    ms = sum(v * v for v in xs) / d + Fraction(float(np.float32(eps)))
    den = (Decimal(ms.numerator) / Decimal(ms.denominator)).sqrt()
    out, ties = [], []
    for xv, g in zip(xs, gs):
        val = (Decimal(xv.numerator) / Decimal(xv.denominator)) / den * g
        b, t = _exact_bf16_of(val)
        out.append(b)
        ties.append(t)
    return np.array(out, dtype=np.uint16), np.array([float(t) for t in ties])


def test_rmsnorm_matches_exact_evaluation():
    rng = np.random.default_rng(11)
    d = 128
    scales = [1e-5, 3e-4, 1e-3, 3e-3, 1e-2, 1.0, 37.0]
    x = np.concatenate([_rand_bf16(rng, (1, d), s) for s in scales])
    gamma = _rand_bf16(rng, (d,), 0.3)
    gamma = _f64_to_bf16_bits(1.0 + _bf16_bits_to_f64(gamma))
    eps = 1e-6
    xn = oracle.rmsnorm(x, gamma, eps)
    checked = 0
    for t in range(x.shape[0]):
        ref, tie = _exact_rmsnorm_row(x[t], gamma, eps)
        ok = tie > 1e-9          # not within rounding noise of a tie point
        assert (xn[t][ok] == ref[ok]).all(), "row %d (scale %g)" % (t, scales[t])
        checked += int(ok.sum())
    assert checked >= 0.99 * x.size


def test_rmsnorm_scale_invariant_without_eps():
    rng = np.random.default_rng(12)
    x = _rand_bf16(rng, (3, 192))
    gamma = _rand_bf16(rng, (192,))
    xn = oracle.rmsnorm(x, gamma, 0.0)
    for j in (-20, -3, 5, 30):
        xs = _f64_to_bf16_bits(_bf16_bits_to_f64(x) * 2.0 ** j)   # exact
        assert (oracle.rmsnorm(xs, gamma, 0.0) == xn).all(), j


def test_rmsnorm_constant_row():
    # x_i = c, gamma = 1: xn_i = c / sqrt(c^2 + eps)
    d = 64
    one = np.full(d, 0x3F80, dtype=np.uint16)
    for c, eps, expect in ((2.0, 1e-6, 1.0), (-0.5, 1e-6, -1.0), (1e-3, 3e-6, 0.5)):
        x = _f64_to_bf16_bits(np.full((1, d), c))
        xn = oracle.rmsnorm(x, one, eps)
        assert (_bf16_bits_to_f64(xn) == expect).all(), (c, eps)


def _dense_swiglu(xn_f64, sgu, sdn):
    fs = sgu.shape[0] // 2
    W = _bf16_bits_to_f64(sgu)
    D = _bf16_bits_to_f64(sdn)
    gu = W @ xn_f64
    g, u = gu[:fs], gu[fs:]
    h = g / (1.0 + np.exp(-g)) * u
    return D @ h


def test_shared_expert_is_the_dense_swiglu_mlp():
    rng = np.random.default_rng(13)
    d, fs = 96, 48
    xn = _rand_bf16(rng, (d,))
    sgu = _rand_bf16(rng, (2 * fs, d), 0.5)
    sdn = _rand_bf16(rng, (d, fs), 0.5)
    _, o = oracle.shared_expert_row(xn, sgu, sdn)
    ref = _dense_swiglu(_bf16_bits_to_f64(xn), sgu, sdn)
    assert np.abs(o - ref).max() <= 1e-12 * np.abs(ref).max()


def _small_block(rng, T=5, d=128, E=8, k=2, f=64, fs=32, zero_experts=False):
    x = _rand_bf16(rng, (T, d))
    gamma = _f64_to_bf16_bits(1.0 + 0.1 * rng.standard_normal(d))
    rw = _rand_bf16(rng, (E, d), 0.05)
    if zero_experts:
        gu_c = np.zeros((E, 2 * f, d // 2), np.uint8)
        dn_c = np.zeros((E, d, f // 2), np.uint8)
    else:
        gu_c = rng.integers(0, 256, (E, 2 * f, d // 2), dtype=np.uint8)
        dn_c = rng.integers(0, 256, (E, d, f // 2), dtype=np.uint8)
    gu_s = rng.integers(123, 128, (E, 2 * f, d // 32), dtype=np.uint8)
    dn_s = rng.integers(123, 128, (E, d, f // 32), dtype=np.uint8)
    sgu = _rand_bf16(rng, (2 * fs, d), 0.3)
    sdn = _rand_bf16(rng, (d, fs), 0.3)
    return dict(x=x, gamma=gamma, rw=rw, gu_c=gu_c, gu_s=gu_s, dn_c=dn_c, dn_s=dn_s,
                sgu=sgu, sdn=sdn, k=k)


def _run_block(b, shared=True, eps=1e-6):
    return oracle.block_forward(b["x"], b["gamma"], eps, b["rw"], None, b["gu_c"], b["gu_s"],
                                b["dn_c"], b["dn_s"], b["sgu"] if shared else None,
                                b["sdn"] if shared else None, b["k"], n_threads=2)


def test_block_residual_only():
    b = _small_block(np.random.default_rng(14), zero_experts=True)
    r = _run_block(b, shared=False)
    assert (r["out"] == b["x"]).all()
    assert (r["out64"] == _bf16_bits_to_f64(b["x"])).all()


def test_block_residual_plus_shared_expert():
    b = _small_block(np.random.default_rng(15), zero_experts=True)
    r = _run_block(b)
    assert (r["xn"] == oracle.rmsnorm(b["x"], b["gamma"], 1e-6)).all()
    xf = _bf16_bits_to_f64(b["x"])
    for t in range(b["x"].shape[0]):
        s = _dense_swiglu(_bf16_bits_to_f64(r["xn"][t]), b["sgu"], b["sdn"])
        assert np.abs(r["out64"][t] - xf[t] - s).max() <= 1e-12 * np.abs(s).max()
    # one rounding, straight from fp64
    assert all(int(r["out"].flat[i]) == oracle.round_to_bf16(float(r["out64"].flat[i]))
               for i in range(0, r["out"].size, 7))


def test_block_routes_the_normalised_input():
    b = _small_block(np.random.default_rng(16))
    r = _run_block(b, shared=False)
    lay = oracle.layer_forward(r["xn"], b["rw"], None, b["gu_c"], b["gu_s"], b["dn_c"],
                               b["dn_s"], b["k"], n_threads=2)
    assert (r["topk_ids"] == lay["topk_ids"]).all()
    assert (r["logits"] == lay["logits"]).all()
    xf = _bf16_bits_to_f64(b["x"])
    y = lay["y64"]
    assert np.abs(r["out64"] - xf - y).max() <= 1e-12 * np.abs(y).max()
    # and not the raw input: the routing of x itself differs on these rows
    raw = oracle.router_logits(b["x"], b["rw"])
    assert not (raw == r["logits"]).all()
