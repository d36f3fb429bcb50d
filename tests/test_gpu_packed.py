"""The operand-order (packed) MXFP4 store (include/moe_packed.h) on the GPU.

* moe_prepack_experts is the byte permutation the header states, checked
  against a numpy construction from the scaled MFMA's B-operand layout
  (lane l = r + 16 g: row r of a 16-row tile, K elements 32 g .. 32 g + 31
  of the 128-element step; scales: 16 bytes per row per 4 K steps).
* moe_layer_forward_packed gives the same bits as moe_layer_forward on the
  canonical store (whose parity with the oracle the other GPU tests pin),
  in both activation modes, on ragged shapes and at the skewed-prefill
  size; and the same output as the oracle on a small case.
"""
import numpy as np
import pytest
import torch

import oracle
from routed_expert_mxfp4_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from routed_expert_mxfp4_amd import moe
    moe.lib()
    return torch.device("cuda:0")


def _moe():
    from routed_expert_mxfp4_amd import moe
    return moe


def _np_pack_codes(c, K):
    """[E][rows][K/2] -> packed bytes, from the operand layout."""
    E, rows, _ = c.shape
    S = K // 128
    # [E][t][r][s][g][16]: row 16 t + r, step s, K block g of the step
    v = c.reshape(E, rows // 16, 16, S, 4, 16)
    # packed order: [E][t][s][g][r][16] (lane l = r + 16 g)
    return np.ascontiguousarray(v.transpose(0, 1, 3, 4, 2, 5)).reshape(-1)


def _np_pack_scales(sc, K):
    E, rows, _ = sc.shape
    G = K // 512
    v = sc.reshape(E, rows // 16, 16, G, 16)          # [E][t][r][q][16]
    return np.ascontiguousarray(v.transpose(0, 1, 3, 2, 4)).reshape(-1)


def test_prepack_is_the_stated_permutation(dev):
    moe = _moe()
    cfg = synth.Config(400, "case", 1, 1024, 5, 2, 512, seed=40)
    W = synth.gen_experts(cfg)
    P = moe.moe_prepack_experts({n: v.to(dev) for n, v in W.items()}, cfg.d, cfg.f)
    torch.cuda.synchronize()
    Wn = {n: v.numpy() for n, v in W.items()}
    np.testing.assert_array_equal(P["gu_codes"].cpu().numpy().reshape(-1),
                                  _np_pack_codes(Wn["gu_codes"], cfg.d))
    np.testing.assert_array_equal(P["dn_codes"].cpu().numpy().reshape(-1),
                                  _np_pack_codes(Wn["dn_codes"], cfg.f))
    np.testing.assert_array_equal(P["gu_scales"].cpu().numpy().reshape(-1),
                                  _np_pack_scales(Wn["gu_scales"], cfg.d))
    np.testing.assert_array_equal(P["dn_scales"].cpu().numpy().reshape(-1),
                                  _np_pack_scales(Wn["dn_scales"], cfg.f))


CASES = [
    # (T, d, E, k, f, seed, act)
    (128, 512, 16, 2, 512, 41, 0),       # the smallest prefill call
    (300, 1024, 24, 4, 512, 42, 0),      # filtered routing, ragged groups
    (200, 512, 9, 3, 1024, 43, 1),       # activation-MX mode (one pass)
]


@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_packed_layer_equals_canonical_bit_for_bit(dev, case):
    moe = _moe()
    T, d, E, k, f, seed, act = case
    cfg = synth.Config(400 + seed, "case", T, d, E, k, f, seed=seed)
    L = synth.gen_layer(cfg, device=dev)
    ex = {n: L[n] for n in ("gu_codes", "gu_scales", "dn_codes", "dn_scales")}
    P = moe.moe_prepack_experts(ex, d, f)
    y0, i0, w0 = moe.moe_layer_forward(L["x"], L["router_w"], ex, k, return_routing=True, act=act)
    y1, i1, w1 = moe.moe_layer_forward_packed(L["x"], L["router_w"], P, k, return_routing=True,
                                              act=act)
    torch.cuda.synchronize()
    assert torch.equal(i0, i1) and torch.equal(w0, w1)
    assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))
    if case == CASES[0]:
        ref = oracle.layer_forward(synth.as_u16(L["x"]), synth.as_u16(L["router_w"]), None,
                                   *[ex[n].cpu().numpy() for n in ("gu_codes", "gu_scales",
                                                                   "dn_codes", "dn_scales")], k)
        err = np.abs(y1.float().cpu().numpy().astype(np.float64) - ref["y64"]).max()
        assert err <= 1e-2 * np.abs(ref["y64"]).max()


def test_packed_skewed_prefill_full_size_equals_canonical(dev):
    moe = _moe()
    cfg = synth.CONFIGS[3]
    ex = synth.gen_experts(cfg, device=dev)
    P = moe.moe_prepack_experts(ex, cfg.d, cfg.f)
    x = synth.gen_x(cfg).to(dev)
    wr = synth.gen_router_w(cfg).to(dev)
    b = synth.gen_bias(cfg).to(dev)
    y0 = moe.moe_layer_forward(x, wr, ex, cfg.k, router_bias=b)
    y1 = moe.moe_layer_forward_packed(x, wr, P, cfg.k, router_bias=b)
    torch.cuda.synchronize()
    assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))
    del ex, P
    torch.cuda.empty_cache()
