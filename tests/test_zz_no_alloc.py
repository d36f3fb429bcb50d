"""moe_layer_forward_noalloc against moe_layer_forward.

The no-allocation entry point runs the same kernels on the library's static
scratch array instead of a caller workspace, so its outputs must be the
workspace entry point's bits exactly.  Each case makes two calls in a row
through the C ABI, the second on a smaller input (the array keeps the first
call's contents), and compares both with moe_layer_forward; a call beyond
the array's size is refused without touching the outputs.
"""
import pytest
import torch

from routed_expert_mxfp4_amd import synth

from test_gpu_parity import _small_cfg, dev  # noqa: F401

pytestmark = pytest.mark.gpu


def _moe():
    from routed_expert_mxfp4_amd import moe
    return moe


CASES = [
    # (name, T first, T second, d, E, k, f, seed): the second call is smaller
    ("few_tokens", 8, 3, 256, 16, 2, 128, 501),       # topk+grouping in one block, fused down
    ("one_token", 12, 1, 256, 64, 8, 96, 502),        # then the one-token fused path
    ("mfma", 200, 130, 512, 16, 4, 256, 503),         # scaled-MFMA expert path both times
    ("mfma_then_gemv", 160, 40, 512, 16, 4, 256, 504),
    ("filtered_routing", 300, 257, 512, 64, 6, 256, 505),
    ("wide_one_token", 4, 1, 4608, 24, 16, 1536, 506),   # one token on 96-pair gate/up blocks
]


def _ref(moe, x, wr, ex, k, bias):
    return moe.moe_layer_forward(x, wr, ex, k, router_bias=bias, return_routing=True)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_noalloc_matches_workspace_entry(dev, case):
    moe = _moe()
    name, t1, t2, d, E, k, f, seed = case
    print("case", case, flush=True)
    cfg = _small_cfg(t1, d, E, k, f, seed)
    L = synth.gen_layer(cfg)
    x, wr = L["x"].to(dev), L["router_w"].to(dev)
    bias = torch.linspace(-0.2, 0.2, E, dtype=torch.float32).to(dev)
    ex = {n: L[n].to(dev) for n in ("gu_codes", "gu_scales", "dn_codes", "dn_scales")}
    for T in (t1, t2):
        xs = x[:T].contiguous()
        y = torch.empty((T, d), dtype=torch.bfloat16, device=dev)
        ids = torch.empty((T, k), dtype=torch.int32, device=dev)
        w = torch.empty((T, k), dtype=torch.float32, device=dev)
        moe.moe_layer_forward_noalloc(xs, wr, ex, k, router_bias=bias, y=y, topk_ids=ids,
                                      topk_w=w)
        y_r, ids_r, w_r = _ref(moe, xs, wr, ex, k, bias)
        torch.cuda.synchronize()
        assert torch.equal(ids, ids_r), (name, T)
        assert torch.equal(w, w_r), (name, T)
        assert torch.equal(y, y_r), (name, T)


def test_noalloc_refuses_oversize_and_leaves_outputs(dev):
    moe = _moe()
    T, d, E, k, f = 300, 7168, 896, 16, 1536       # needs more than the static scratch
    dims = moe.dims_of(T, d, E, k, f)
    assert moe.moe_workspace_bytes(dims, moe.ENTRY_LAYER_FORWARD) > moe.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((T, d), dtype=torch.bfloat16, device=dev)
    wr = torch.zeros((E, d), dtype=torch.bfloat16, device=dev)
    tiny = torch.zeros((1, 2 * f), dtype=torch.uint8, device=dev)     # never read
    ex = {"gu_codes": tiny, "gu_scales": tiny, "dn_codes": tiny, "dn_scales": tiny}
    y = torch.full((T, d), 3.0, dtype=torch.bfloat16, device=dev)
    with pytest.raises(moe.MoeError) as err:
        moe.moe_layer_forward_noalloc(x, wr, ex, k, y=y)
    assert err.value.status == moe.MOE_ERR_SCRATCH
    torch.cuda.synchronize()
    assert (y.float() == 3.0).all()
