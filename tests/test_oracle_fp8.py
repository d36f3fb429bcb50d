"""Pins of the oracle's FP8 expert variant (E4M3FN codes, fp32 scale per
128 x 128 block; CPU only).

* E4M3FN codes: the format's edge values printed in the OCP 8-bit floating
  point and MX specifications (tests/golden/e4m3fn_ocp.txt); every finite
  code is also pinned by the field definition in test_oracle_mx.py.
* The block-scaled weight and the FP8 expert: against the dense SwiGLU MLP
  in numpy, with the scale blocks spread over the matrix by np.kron (so a
  wrong block index, a transposed block grid or a gate/up swap fails).
* Power-of-two scaling is exact: doubling one expert's down scales doubles
  its output bit for bit; all-zero codes give exactly zero.
* The FP8 layer: routing identical to the MXFP4 layer's (same router), the
  combine of the FP8 expert rows.
"""
import math
import os

import numpy as np

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_e4m3fn_edge_values_from_the_specification():
    for line in open(os.path.join(ROOT, "tests", "golden", "e4m3fn_ocp.txt")):
        if line.startswith("#") or not line.strip():
            continue
        code, val = line.split()
        got = oracle.elem_value(oracle.FMT_E4M3, int(code, 16))
        if val == "nan":
            assert math.isnan(got), code
        else:
            assert got == float(val) and math.copysign(1, got) == math.copysign(1, float(val)), code


def _rand_fp8(rng, shape):
    b = rng.integers(0, 256, shape, dtype=np.uint8)
    return np.where((b & 0x7F) == 0x7F, b - 1, b).astype(np.uint8)


def _table():
    return np.array([oracle.elem_value(oracle.FMT_E4M3, c) for c in range(256)])


def _dense(codes, scales):
    """[rows][K] fp64: decoded codes times their 128 x 128 block's scale."""
    return _table()[codes] * np.kron(scales.astype(np.float64), np.ones((128, 128)))


def _bf16(rng, shape):
    v = rng.standard_normal(shape).astype(np.float32)
    u = v.view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _bf16_f64(b):
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _expert(rng, d, f):
    gu = _rand_fp8(rng, (2 * f, d))
    dn = _rand_fp8(rng, (d, f))
    gs = rng.uniform(2 ** -9, 2 ** -7, (2 * f // 128, d // 128)).astype(np.float32)
    ds = rng.uniform(2 ** -9, 2 ** -7, (d // 128, f // 128)).astype(np.float32)
    return gu, gs, dn, ds


def test_fp8_weight_block_scale_indexing():
    rng = np.random.default_rng(21)
    codes = _rand_fp8(rng, (256, 384))
    scales = rng.uniform(0.5, 2.0, (2, 3)).astype(np.float32)
    W = _dense(codes, scales)
    for r, c in [(0, 0), (127, 127), (128, 127), (127, 128), (255, 383), (200, 300), (5, 260)]:
        assert oracle.fp8_weight(codes, scales, 384, r, c) == W[r, c], (r, c)


def test_fp8_expert_is_the_dense_swiglu_mlp():
    rng = np.random.default_rng(22)
    d, f = 256, 256
    gu, gs, dn, ds = _expert(rng, d, f)
    x = _bf16(rng, d)
    h, o = oracle.expert_row_fp8(x, gu, gs, dn, ds, d, f)
    Wgu, Wdn = _dense(gu, gs), _dense(dn, ds)
    gu_v = Wgu @ _bf16_f64(x)
    g, u = gu_v[:f], gu_v[f:]
    h_ref = g / (1.0 + np.exp(-g)) * u
    o_ref = Wdn @ h_ref
    assert np.abs(h - h_ref).max() <= 1e-12 * np.abs(h_ref).max()
    assert np.abs(o - o_ref).max() <= 1e-12 * np.abs(o_ref).max()


def test_fp8_power_of_two_scale_and_zero_codes_are_exact():
    rng = np.random.default_rng(23)
    d, f = 128, 128
    gu, gs, dn, ds = _expert(rng, d, f)
    x = _bf16(rng, d)
    _, o = oracle.expert_row_fp8(x, gu, gs, dn, ds, d, f)
    _, o2 = oracle.expert_row_fp8(x, gu, gs, dn, ds * np.float32(2), d, f)
    assert (o2 == 2 * o).all()
    _, oz = oracle.expert_row_fp8(x, np.zeros_like(gu), gs, dn, ds, d, f)
    assert (oz == 0).all()


def test_fp8_layer_routes_like_the_layer_and_combines_its_rows():
    rng = np.random.default_rng(24)
    T, d, E, k, f = 3, 128, 6, 2, 128
    x = _bf16(rng, (T, d))
    rw = _bf16(rng, (E, d))
    ex = [_expert(rng, d, f) for _ in range(E)]
    gu = np.stack([e[0] for e in ex]); gs = np.stack([e[1] for e in ex])
    dn = np.stack([e[2] for e in ex]); ds = np.stack([e[3] for e in ex])
    r = oracle.layer_forward_fp8(x, rw, None, gu, gs, dn, ds, k, n_threads=2)
    ids, w = oracle.topk_softmax(oracle.router_logits(x, rw), k)
    assert (r["topk_ids"] == ids).all() and (r["topk_w"] == w).all()
    for t in range(T):
        o = np.stack([oracle.expert_row_fp8(x[t], gu[e], gs[e], dn[e], ds[e], d, f)[1]
                      for e in ids[t]])
        y, yb = oracle.combine_token(w[t], o)
        assert (r["y64"][t] == y).all() and (r["y"][t] == yb).all()
