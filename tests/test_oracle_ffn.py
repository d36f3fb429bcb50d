"""Pins for the oracle's expert FFN, combine and whole-layer composition.

References: a numpy float64 dense SwiGLU MLP whose weights are dequantised
from the OCP E2M1 table (not through the oracle's decoder), an 80-bit
long-double evaluation, exact zero and power-of-two identities, and a row
pick for one-hot combine weights.
"""
import math
import os

import numpy as np
import pytest
import scipy.special

import oracle
from routed_expert_mxfp4_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _table():
    t = np.zeros(16)
    for line in open(os.path.join(GOLDEN, "e2m1_ocp.txt")):
        line = line.strip()
        if line and not line.startswith("#"):
            c, v = line.split()
            t[int(c, 16)] = float(v)
    return t


def _dequant_np(codes, scales, dtype=np.float64):
    """[R][K/2] codes + [R][K/32] scales -> [R][K] using the OCP table."""
    tab = _table().astype(dtype)
    lo = codes & 0xF
    hi = codes >> 4
    R, half = codes.shape
    vals = np.empty((R, 2 * half), dtype)
    vals[:, 0::2] = tab[lo]
    vals[:, 1::2] = tab[hi]
    sc = np.ldexp(np.ones_like(scales, dtype=np.float64), scales.astype(np.int64) - 127).astype(dtype)
    return vals * np.repeat(sc, 32, axis=1)


def _bf16_to_f64(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _small_cfg(E=1, k=1, d=128, f=64, T=4, seed=0):
    return synth.Config(99, "test", T, d, E, k, f, seed=seed)


def _dense_swiglu(xv, gu, dn, f):
    g = xv @ gu[:f].T
    u = xv @ gu[f:].T
    h = g / (1.0 + np.exp(-g)) * u
    return h, h @ dn.T


def test_single_expert_is_dense_swiglu_mlp():
    cfg = _small_cfg(d=256, f=128, T=3)
    W = {k: v.numpy() for k, v in synth.gen_experts(cfg).items()}
    x = synth.as_u16(synth.gen_x(cfg))
    gu = _dequant_np(W["gu_codes"][0], W["gu_scales"][0])
    dn = _dequant_np(W["dn_codes"][0], W["dn_scales"][0])
    href, oref = _dense_swiglu(_bf16_to_f64(x), gu, dn, cfg.f)
    for t in range(cfg.T):
        h, o = oracle.expert_row(x[t], W["gu_codes"][0], W["gu_scales"][0],
                                 W["dn_codes"][0], W["dn_scales"][0], cfg.d, cfg.f)
        np.testing.assert_allclose(h, href[t], rtol=1e-12, atol=1e-12 * np.abs(href).max())
        np.testing.assert_allclose(o, oref[t], rtol=1e-12, atol=1e-12 * np.abs(oref).max())
    # the whole layer with E = k = 1 is the dense MLP (weight 1)
    res = oracle.layer_forward(x, synth.as_u16(synth.gen_router_w(cfg)), None,
                               W["gu_codes"], W["gu_scales"], W["dn_codes"],
                               W["dn_scales"], k=1, n_threads=1)
    assert (res["topk_ids"] == 0).all() and (res["topk_w"] == 1.0).all()
    np.testing.assert_allclose(res["y64"], oref, rtol=1e-12, atol=1e-12 * np.abs(oref).max())


def test_expert_row_vs_long_double():
    cfg = _small_cfg(d=128, f=64, T=1, seed=3)
    W = {k: v.numpy() for k, v in synth.gen_experts(cfg).items()}
    x = synth.as_u16(synth.gen_x(cfg))[0]
    L = np.longdouble
    gu = _dequant_np(W["gu_codes"][0], W["gu_scales"][0], dtype=L)
    dn = _dequant_np(W["dn_codes"][0], W["dn_scales"][0], dtype=L)
    xv = _bf16_to_f64(x).astype(L)
    g = np.array([sum(xv[i] * gu[n, i] for i in range(cfg.d)) for n in range(cfg.f)], L)
    u = np.array([sum(xv[i] * gu[cfg.f + n, i] for i in range(cfg.d)) for n in range(cfg.f)], L)
    h = g / (L(1) + np.exp(-g)) * u
    o = np.array([sum(h[n] * dn[m, n] for n in range(cfg.f)) for m in range(cfg.d)], L)
    h64, o64 = oracle.expert_row(x, W["gu_codes"][0], W["gu_scales"][0],
                                 W["dn_codes"][0], W["dn_scales"][0], cfg.d, cfg.f)
    assert np.max(np.abs(h64 - h.astype(np.float64))) <= 1e-12 * float(np.max(np.abs(h)))
    assert np.max(np.abs(o64 - o.astype(np.float64))) <= 1e-12 * float(np.max(np.abs(o)))


def test_all_zero_expert_gives_exact_zero():
    cfg = _small_cfg(d=128, f=64, T=2)
    W = {k: v.numpy().copy() for k, v in synth.gen_experts(cfg).items()}
    rng = np.random.default_rng(0)
    # every nibble is +0 (code 0) or -0 (code 8)
    for name in ("gu_codes", "dn_codes"):
        lo = rng.choice([0, 8], W[name].shape)
        hi = rng.choice([0, 8], W[name].shape)
        W[name] = (lo | (hi << 4)).astype(np.uint8)
    x = synth.as_u16(synth.gen_x(cfg))
    for t in range(cfg.T):
        h, o = oracle.expert_row(x[t], W["gu_codes"][0], W["gu_scales"][0],
                                 W["dn_codes"][0], W["dn_scales"][0], cfg.d, cfg.f)
        assert (h == 0).all() and (o == 0).all()


def test_scale_code_plus_one_doubles_exactly():
    cfg = _small_cfg(d=128, f=64, T=2, seed=5)
    W = {k: v.numpy().copy() for k, v in synth.gen_experts(cfg).items()}
    x = synth.as_u16(synth.gen_x(cfg))
    base = [oracle.expert_row(x[t], W["gu_codes"][0], W["gu_scales"][0],
                              W["dn_codes"][0], W["dn_scales"][0], cfg.d, cfg.f)
            for t in range(cfg.T)]
    dn2 = W["dn_scales"][0] + 1
    up2 = W["gu_scales"][0].copy()
    up2[cfg.f:] += 1                       # the up half only
    for t in range(cfg.T):
        _, o = oracle.expert_row(x[t], W["gu_codes"][0], W["gu_scales"][0],
                                 W["dn_codes"][0], dn2, cfg.d, cfg.f)
        assert (o == 2 * base[t][1]).all()
        h, o = oracle.expert_row(x[t], W["gu_codes"][0], up2,
                                 W["dn_codes"][0], W["dn_scales"][0], cfg.d, cfg.f)
        assert (h == 2 * base[t][0]).all() and (o == 2 * base[t][1]).all()


def test_combine_one_hot_is_row_pick_and_weighted_sum():
    rng = np.random.default_rng(3)
    o = rng.standard_normal((4, 64)) * 100
    for j in range(4):
        w = np.zeros(4)
        w[j] = 1.0
        y64, yb = oracle.combine_token(w, o)
        assert (y64 == o[j]).all()
        assert all(yb[m] == oracle.round_to_bf16(o[j, m]) for m in range(64))
    w = scipy.special.softmax(rng.standard_normal(4))
    y64, _ = oracle.combine_token(w, o)
    np.testing.assert_allclose(y64, w @ o, rtol=1e-13, atol=1e-12)


def test_tiny_layer_matches_independent_numpy_pipeline():
    cfg = synth.CONFIGS[0]
    L = synth.gen_layer(cfg)
    x, wr = synth.as_u16(L["x"]), synth.as_u16(L["router_w"])
    W = {k: L[k].numpy() for k in ("gu_codes", "gu_scales", "dn_codes", "dn_scales")}
    res = oracle.layer_forward(x, wr, None, W["gu_codes"], W["gu_scales"],
                               W["dn_codes"], W["dn_scales"], k=cfg.k, n_threads=2)
    # routing: numpy fp64 logits are within fp32 rounding of the oracle's
    xv, wv = _bf16_to_f64(x), _bf16_to_f64(wr)
    lg = xv @ wv.T
    assert np.max(np.abs(res["logits"] - lg)) <= 2.0 ** -22 * np.max(np.abs(lg))
    ids = res["topk_ids"]
    for t in range(cfg.T):
        ref = sorted(range(cfg.E), key=lambda e: (-float(res["logits"][t, e]), e))[:cfg.k]
        assert list(ids[t]) == ref
    y = np.zeros((cfg.T, cfg.d))
    for t in range(cfg.T):
        sel = res["logits"][t, ids[t]].astype(np.float64)
        w = scipy.special.softmax(sel)
        np.testing.assert_allclose(res["topk_w"][t], w, rtol=1e-14)
        for j, e in enumerate(ids[t]):
            gu = _dequant_np(W["gu_codes"][e], W["gu_scales"][e])
            dn = _dequant_np(W["dn_codes"][e], W["dn_scales"][e])
            _, o = _dense_swiglu(xv[t:t + 1], gu, dn, cfg.f)
            y[t] += w[j] * o[0]
    np.testing.assert_allclose(res["y64"], y, rtol=1e-12, atol=1e-12 * np.abs(y).max())
    yb = np.array([[oracle.round_to_bf16(v) for v in row] for row in res["y64"]], np.uint16)
    np.testing.assert_array_equal(res["y"], yb)


def test_activation_mx_mode_hand_example():
    """The activation-MX mode on a layer small enough to do by hand (one
    expert, d = f = 32, weights 0 or 1.0, E8M0 scale 2^0).
    x = (1.1015625, 0.30078125, 0, ...) (bf16 of 1.1 and 0.3).  Its block
    amax gives X = floor(log2 1.10) - 2 = -2, so x / 2^X = (4.40625,
    1.203125) rounds on the E2M3 grid to (4.5, 1.25): x' = (1.125, 0.3125).
    Gate rows 0, 1 pick x'0, x'1 and up rows 0, 1 pick x'1, x'0, so
    h0 = silu(1.125) * 0.3125 = 0.265400 and h1 = silu(0.3125) * 1.125 =
    0.203026.  Their block gives X = -2 - 2 = -4: h / 2^X = (4.2464,
    3.2484) round to (4.0, 3.25), h' = (0.25, 0.203125).  The down row 0
    sums h'0 + h'1 = 0.453125, and k = 1 makes y0 = o0 exactly (every other
    output is 0).  Without the rounding of x the result is 0.4375, without
    that of h 0.468426; the plain mode gives silu(1.1015625) * 0.30078125 +
    silu(0.30078125) * 1.1015625."""
    d = f = 32
    x = np.zeros((1, d), dtype=np.uint16)
    x[0, 0], x[0, 1] = 0x3F8D, 0x3E9A               # bf16 1.1015625, 0.30078125
    gu_codes = np.zeros((1, 2 * f, d // 2), dtype=np.uint8)
    gu_codes[0, 0, 0] = 0x02                         # gate row 0: element 0 = 1.0
    gu_codes[0, 1, 0] = 0x20                         # gate row 1: element 1 = 1.0
    gu_codes[0, f + 0, 0] = 0x20                     # up row 0: element 1
    gu_codes[0, f + 1, 0] = 0x02                     # up row 1: element 0
    gu_scales = np.full((1, 2 * f, d // 32), 127, dtype=np.uint8)
    dn_codes = np.zeros((1, d, f // 2), dtype=np.uint8)
    dn_codes[0, 0, 0] = 0x22                         # down row 0: elements 0, 1
    dn_scales = np.full((1, d, f // 32), 127, dtype=np.uint8)
    wr = np.zeros((1, d), dtype=np.uint16)
    args = (x, wr, None, gu_codes, gu_scales, dn_codes, dn_scales)
    amx = oracle.layer_forward(*args, k=1, act=1)
    assert amx["y64"][0, 0] == 0.453125
    assert (amx["y64"][0, 1:] == 0.0).all()
    plain = oracle.layer_forward(*args, k=1)
    sl = lambda z: z / (1.0 + math.exp(-z))
    x0, x1 = 1.1015625, 0.30078125
    assert abs(plain["y64"][0, 0] - (sl(x0) * x1 + sl(x1) * x0)) <= 1e-15
    # the rounding helper on its own: the x block above
    v = np.zeros(32)
    v[0], v[1] = x0, x1
    r = oracle.mx_round(oracle.FMT_E2M3, v)
    assert r[0] == 1.125 and r[1] == 0.3125 and (r[2:] == 0).all()
