"""E8M0 scale codes at the ends of their range, on every expert path.

The workloads draw scale codes 123..127 only.  OCP MX E8M0 code c means
2^(c - 127) for c <= 254, so code 0 is 2^-127 (a subnormal in fp32), and code
255 is NaN.  These cases put such codes into small layers on each path the
library takes:

  one token (top-k and grouping inside the gate/up GEMV, fused down+combine;
  at f = 128 and at the K3 width f = 1536),
  few tokens (one-launch top-k + grouping, grouped GEMV, fused down+combine),
  more tokens (grouped GEMVs, separate combine),
  the scaled-MFMA GEMMs on the canonical store and on the packed store,
  and moe_expert_ffn's rows on the GEMV and MFMA paths.

* Down scale codes 0..4 with the usual gate/up scales: every output is
  around 1e-34, still normal in fp32 and bf16, and must match the oracle
  within 1e-2 max|oracle| (a flush to zero anywhere fails that).
* Code 255 in a few down blocks of one expert: exactly the output columns
  of those rows are NaN for the tokens that use the expert, as in the
  oracle; everything else is finite and within tolerance.
* Code 255 in one gate row's block: that expert's h is NaN in one column,
  so every output of every token that uses it is NaN, as in the oracle.

The activation-MX mode is not covered here: its rounding of a NaN block is
not defined by the conversion model.
"""
import numpy as np
import pytest
import torch

import oracle
from routed_expert_mxfp4_amd import synth

from test_gpu_parity import _small_cfg, dev  # noqa: F401

pytestmark = pytest.mark.gpu

TOL = 1e-2

PATHS = [
    # (name, T, d, E, k, f, seed, packed)
    ("one_token", 1, 256, 16, 4, 128, 301, False),
    ("one_token_f1536", 1, 512, 16, 4, 1536, 306, False),
    ("few_tokens", 3, 256, 16, 4, 128, 302, False),
    ("grouped_gemv", 20, 256, 16, 4, 128, 303, False),
    ("mfma", 160, 512, 8, 2, 256, 304, False),
    ("mfma_packed", 160, 512, 8, 2, 512, 305, True),
]


def _moe():
    from routed_expert_mxfp4_amd import moe
    return moe


def _compare(gpu, ref, what):
    """NaN exactly where the oracle has NaN; the rest within tolerance."""
    gpu = np.asarray(gpu, dtype=np.float64)
    nan_g, nan_o = np.isnan(gpu), np.isnan(ref)
    assert (nan_g == nan_o).all(), "%s: NaN at %d places, oracle at %d (%d differ)" % (
        what, nan_g.sum(), nan_o.sum(), (nan_g != nan_o).sum())
    fin = ~nan_o
    if fin.any():
        err = np.abs(gpu[fin] - ref[fin]).max()
        scale = np.abs(ref[fin]).max()
        assert err <= TOL * scale, "%s: max err %.4g > %.0e * %.4g" % (what, err, TOL, scale)
        return err, scale
    return 0.0, 0.0


def _layer(case, variant):
    name, T, d, E, k, f, seed, packed = case
    cfg = _small_cfg(T, d, E, k, f, seed)
    L = synth.gen_layer(cfg)
    x16, wr16 = synth.as_u16(L["x"]), synth.as_u16(L["router_w"])
    ids0, _ = oracle.topk_softmax(oracle.router_logits(x16[:1], wr16), k)
    e = int(ids0[0, 0])                       # an expert token 0 uses
    if variant == "down_codes_0_4":
        L["dn_scales"] = L["dn_scales"] - synth.SCALE_CODE_LO        # codes 0..4
    elif variant == "down_nan":
        L["dn_scales"] = L["dn_scales"].clone()
        for m, b in ((3, 0), (d // 2 + 1, f // 32 - 1), (d - 1, 0)):
            L["dn_scales"][e, m, b] = 255
    elif variant == "gate_nan":
        L["gu_scales"] = L["gu_scales"].clone()
        L["gu_scales"][e, f // 2, d // 64] = 255
    else:
        raise ValueError(variant)
    return cfg, L, e


VARIANTS = ["down_codes_0_4", "down_nan", "gate_nan"]


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("case", PATHS, ids=[c[0] for c in PATHS])
def test_edge_scale_codes_layer(dev, case, variant):
    moe = _moe()
    print("path", case[0], "variant", variant, flush=True)
    cfg, L, e = _layer(case, variant)
    W = {n: L[n].numpy() for n in ("gu_codes", "gu_scales", "dn_codes", "dn_scales")}
    ref = oracle.layer_forward(synth.as_u16(L["x"]), synth.as_u16(L["router_w"]), None,
                               W["gu_codes"], W["gu_scales"], W["dn_codes"], W["dn_scales"],
                               cfg.k)
    ex = {n: L[n].to(dev).contiguous() for n in W}
    x, wr = L["x"].to(dev), L["router_w"].to(dev)
    if case[7]:
        ex = moe.moe_prepack_experts(ex, cfg.d, cfg.f)
        y, ids, w = moe.moe_layer_forward_packed(x, wr, ex, cfg.k, return_routing=True)
    else:
        y, ids, w = moe.moe_layer_forward(x, wr, ex, cfg.k, return_routing=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ids.cpu().numpy(), ref["topk_ids"])
    y64 = ref["y64"]
    users = (ref["topk_ids"] == e).any(1)
    if variant == "down_codes_0_4":
        assert np.abs(y64).max() < 1e-30 and np.abs(y64).max() > 1e-37
    elif variant == "down_nan":
        assert np.isnan(y64[users]).any() and not np.isnan(y64[~users]).any()
    else:
        assert np.isnan(y64[users]).all() and not np.isnan(y64[~users]).any()
    err, scale = _compare(y.float().cpu().numpy(), y64, "%s/%s y" % (case[0], variant))
    print("max err %.3g of max|oracle| %.3g" % (err, scale))


FFN_PATHS = [c for c in PATHS if c[0] in ("grouped_gemv", "mfma")]


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("case", FFN_PATHS, ids=[c[0] for c in FFN_PATHS])
def test_edge_scale_codes_expert_rows(dev, case, variant):
    moe = _moe()
    cfg, L, e = _layer(case, variant)
    x16, wr16 = synth.as_u16(L["x"]), synth.as_u16(L["router_w"])
    ids_o, _ = oracle.topk_softmax(oracle.router_logits(x16, wr16), cfg.k)
    _, off_o, sr_o, _ = oracle.permute(ids_o, cfg.E)
    W = {n: L[n].numpy() for n in ("gu_codes", "gu_scales", "dn_codes", "dn_scales")}
    o = np.zeros((cfg.T * cfg.k, cfg.d))
    for p, r in enumerate(sr_o):
        t, j = divmod(int(r), cfg.k)
        ee = ids_o[t, j]
        o[p] = oracle.expert_row(x16[t], W["gu_codes"][ee], W["gu_scales"][ee],
                                 W["dn_codes"][ee], W["dn_scales"][ee], cfg.d, cfg.f)[1]
    ex = {n: L[n].to(dev).contiguous() for n in W}
    rows = moe.moe_expert_ffn(L["x"].to(dev), ex, torch.from_numpy(off_o).to(dev),
                              torch.from_numpy(sr_o).to(dev), cfg.k)
    torch.cuda.synchronize()
    _compare(rows.float().cpu().numpy(), o, "%s/%s rows_out" % (case[0], variant))
