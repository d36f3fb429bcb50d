"""The Python binding's buffers on a side stream, and workspace growth.

* Every wrapper makes its temporaries (workspace, outputs, dtype copies) on
  the stream it launches on.  The layer run on a side stream, with
  allocations churning on the default stream meanwhile, must give the same
  bits as the layer run on the default stream.
* The layer workspace is not monotonic in T: in the activation-MX mode the
  expert path changes at 128 tokens.  A Layer first used at 128 tokens (the
  MFMA path) and then at 127 (the GEMV path, whose fp32 h is larger) must
  grow its workspace instead of refusing the call.
"""
import pytest
import torch

from routed_expert_mxfp4_amd import synth

from test_gpu_parity import _small_cfg, dev  # noqa: F401

pytestmark = pytest.mark.gpu


def _moe():
    from routed_expert_mxfp4_amd import moe
    return moe


def test_layer_on_side_stream(dev):
    moe = _moe()
    cfg = _small_cfg(40, 512, 64, 8, 128, 401)
    L = synth.gen_layer(cfg)
    x, wr = L["x"].to(dev), L["router_w"].to(dev)
    bias = torch.linspace(-0.3, 0.3, cfg.E, dtype=torch.float64).to(dev)  # wrapper casts it
    ex = {n: L[n].to(dev) for n in ("gu_codes", "gu_scales", "dn_codes", "dn_scales")}
    y0, ids0, w0 = moe.moe_layer_forward(x, wr, ex, cfg.k, router_bias=bias,
                                         return_routing=True)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(4):
        outs.append(moe.moe_layer_forward(x, wr, ex, cfg.k, router_bias=bias,
                                          return_routing=True, stream=side))
        # allocations on the default stream while the side stream's work runs
        junk = [torch.full((1 << 18,), 0x5A, dtype=torch.uint8, device=dev) for _ in range(8)]
        del junk
    layer = moe.Layer(ex, wr, cfg.k, bias.float(), T=1)
    y_l = layer.forward(x, stream=side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for y, ids, w in outs:
        assert torch.equal(y, y0) and torch.equal(ids, ids0) and torch.equal(w, w0)
    assert torch.equal(y_l, y0)


def test_layer_workspace_grows_by_bytes(dev):
    # The activation-MX mode switches from the GEMVs (fp32 h of every row)
    # to the scaled-MFMA path at 128 tokens, so 127 tokens need more
    # workspace than 128: a Layer reserved for 128 must grow for 127.
    moe = _moe()
    act = moe.ACT_MX_E2M3
    cfg = _small_cfg(128, 512, 16, 4, 256, 402)
    big_t, small_t = 128, 127
    n_big = moe.moe_workspace_bytes(moe.dims_of(big_t, cfg.d, cfg.E, cfg.k, cfg.f, act),
                                    moe.ENTRY_LAYER_FORWARD)
    n_small = moe.moe_workspace_bytes(moe.dims_of(small_t, cfg.d, cfg.E, cfg.k, cfg.f, act),
                                      moe.ENTRY_LAYER_FORWARD)
    assert n_small > n_big, "shape no longer exercises a smaller workspace at larger T"
    L = synth.gen_layer(cfg)
    x, wr = L["x"].to(dev), L["router_w"].to(dev)
    ex = {n: L[n].to(dev) for n in ("gu_codes", "gu_scales", "dn_codes", "dn_scales")}
    layer = moe.Layer(ex, wr, cfg.k, None, T=big_t, act=act)
    layer.forward(x)
    y = layer.forward(x[:small_t].contiguous())
    y_ref = moe.moe_layer_forward(x[:small_t].contiguous(), wr, ex, cfg.k, act=act)
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref)
