"""GPU parity of the activation-MX mode (moe_dims.act = MOE_ACT_MX_E2M3).

In this mode x and h are each rounded to one MX E2M3 term per 32 elements
before their products; the oracle's layer_forward(act=1) defines the
result.  Every expert path is covered: the scaled-MFMA prefill path (one
matrix pass), the one-token fused top-k + gate/up kernel, the fused
down + combine of small T and the grouped GEMVs.  Routing is the plain
mode's, bit for bit; outputs within max|gpu - oracle| <= 1e-2 max|oracle|.
The mode's distance from the W4A16 result is printed (a few % of max|y|).
"""
import numpy as np
import pytest
import torch

import oracle
from routed_expert_mxfp4_amd import synth

from test_gpu_parity import (W_TOL, _bf16_to_f64, _close, _dev_experts, _np_experts,  # noqa: F401
                             _small_cfg, dev)

pytestmark = pytest.mark.gpu

AMX_CASES = [
    # (T, d, E, k, f, seed)
    (200, 512, 16, 4, 256, 91),      # scaled-MFMA path, ragged tiles
    (160, 1536, 12, 2, 512, 92),     # MFMA, longer K
    (1, 512, 64, 8, 96, 93),         # one token: top-k inside the gate/up kernel
    (3, 256, 40, 5, 64, 94),         # fused down + combine
    (20, 512, 70, 3, 128, 95),       # grouped GEMVs, rows_out + combine
    (64, 512, 8, 4, 128, 96),        # ~32 rows per expert on the GEMVs: four-row passes
]


def _moe():
    from routed_expert_mxfp4_amd import moe
    return moe


@pytest.mark.parametrize("case", AMX_CASES, ids=[str(c) for c in AMX_CASES])
def test_activation_mx_layer(dev, case):
    moe = _moe()
    T, d, E, k, f, seed = case
    print("case", case, flush=True)
    cfg = _small_cfg(T, d, E, k, f, seed)
    L = synth.gen_layer(cfg)
    x16, wr16 = synth.as_u16(L["x"]), synth.as_u16(L["router_w"])
    W = _np_experts(L)
    args = (x16, wr16, None, W["gu_codes"], W["gu_scales"], W["dn_codes"], W["dn_scales"])
    ref = oracle.layer_forward(*args, k=k, act=1)
    plain = oracle.layer_forward(*args, k=k)
    np.testing.assert_array_equal(ref["topk_ids"], plain["topk_ids"])
    ex = _dev_experts(L, dev)
    y, ids, w = moe.moe_layer_forward(L["x"].to(dev), L["router_w"].to(dev), ex, k,
                                      return_routing=True, act=moe.ACT_MX_E2M3)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ids.cpu().numpy(), ref["topk_ids"])
    assert np.abs(w.cpu().numpy() - ref["topk_w"]).max() <= W_TOL
    _close(_bf16_to_f64(y), ref["y64"], "activation-MX y")
    scale = np.abs(plain["y64"]).max()
    print("activation-MX vs W4A16: max|dy| / max|y| = %.4f"
          % (np.abs(ref["y64"] - plain["y64"]).max() / scale))


@pytest.mark.parametrize("case", [AMX_CASES[0], AMX_CASES[4]], ids=["mfma", "gemv"])
def test_activation_mx_expert_ffn_entry(dev, case):
    moe = _moe()
    T, d, E, k, f, seed = case
    cfg = _small_cfg(T, d, E, k, f, seed)
    L = synth.gen_layer(cfg)
    x16, wr16 = synth.as_u16(L["x"]), synth.as_u16(L["router_w"])
    W = _np_experts(L)
    ids_o, _ = oracle.topk_softmax(oracle.router_logits(x16, wr16), k)
    _, _, sr_o, _ = oracle.permute(ids_o, E)
    o = np.zeros((T * k, d))
    for r in range(T * k):
        t, e = r // k, int(ids_o.flat[r])
        o[r] = oracle.expert_row(x16[t], W["gu_codes"][e], W["gu_scales"][e], W["dn_codes"][e],
                                 W["dn_scales"][e], d, f, act=1)[1]
    ids_t = torch.from_numpy(ids_o).to(dev)
    counts, offsets, sr, rp = moe.moe_permute(ids_t, E)
    rows_out = moe.moe_expert_ffn(L["x"].to(dev), _dev_experts(L, dev), offsets, sr, k,
                                  act=moe.ACT_MX_E2M3)
    torch.cuda.synchronize()
    _close(_bf16_to_f64(rows_out), o[sr_o], "activation-MX rows_out")
