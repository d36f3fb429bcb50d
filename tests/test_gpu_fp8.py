"""GPU parity of the FP8 expert variant (include/moe_fp8.h) against the CPU
oracle.

Bar: routing ids bit-exact, weights within 1e-5; rows_out and y within
max|gpu - oracle| <= 1e-2 * max|oracle|.  Exact checks, on the GEMVs (few
tokens) and on the matrix-core GEMMs (from 128 tokens): doubling an
expert's down scales doubles its rows bit for bit; all-zero codes give
exactly zero; two runs are identical.  Full size (d = 7168, E = 896, top-16,
f = 1536): decode and skewed prefill on sampled tokens.
"""
import concurrent.futures as cf
import os

import numpy as np
import pytest
import torch

import oracle
from routed_expert_mxfp4_amd import synth

pytestmark = pytest.mark.gpu

TOL = 1e-2
W_TOL = 1e-5


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from routed_expert_mxfp4_amd import moe
    moe.lib()              # raises if the HIP library is missing: no fallback
    return torch.device("cuda:0")


def _moe():
    from routed_expert_mxfp4_amd import moe
    return moe


def _bf16_to_f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def _close(gpu, ref, what):
    err = float(np.max(np.abs(gpu - ref)))
    scale = float(np.max(np.abs(ref)))
    assert err <= TOL * scale, "%s: max err %.4g > %.0e * %.4g" % (what, err, TOL, scale)


def _np(W):
    return {n: v.cpu().numpy() for n, v in W.items()}


def _case(T, d, E, k, f, seed):
    cfg = synth.Config(300 + seed, "case", T, d, E, k, f, seed=seed, wfmt="fp8")
    x = synth.gen_x(cfg)
    wr = synth.gen_router_w(cfg)
    W = synth.gen_experts_fp8(cfg)
    return cfg, x, wr, W


CASES = [
    # (T, d, E, k, f, seed)
    (1, 256, 16, 2, 128, 0),          # one token: top-k inside gate/up, fused down + combine
    (1, 512, 64, 8, 256, 6),          # one token, two scale blocks along f
    (3, 384, 40, 5, 256, 5),          # fused down + combine for three tokens
    (4, 256, 16, 16, 128, 7),         # four tokens, top-16 (the widest fused down + combine)
    (8, 256, 16, 2, 128, 1),          # fused top-k + grouping (T <= 16)
    (5, 384, 40, 5, 256, 2),          # three scale blocks along d, two along f
    (20, 256, 24, 3, 128, 3),         # separate top-k and permute
    (300, 256, 24, 4, 128, 4),        # filtered routing; matrix-core GEMMs (T >= 128)
    # matrix-core GEMMs: a partial down column block (d = 384: 256 + 128),
    # ragged row tiles, three gate/up column blocks, experts over 128 rows
    (160, 384, 8, 2, 256, 10),
    (400, 256, 4, 2, 384, 11),
    (130, 512, 64, 3, 128, 12),       # many experts with a handful of rows, some with none
]


@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_fp8_layer_small(dev, case):
    moe = _moe()
    T, d, E, k, f, seed = case
    print("fp8 case", case, flush=True)
    cfg, x, wr, W = _case(*case)
    y, ids, w = moe.moe_layer_forward_fp8(x.to(dev), wr.to(dev),
                                          {n: v.to(dev) for n, v in W.items()}, k,
                                          return_routing=True)
    torch.cuda.synchronize()
    Wn = _np(W)
    ref = oracle.layer_forward_fp8(synth.as_u16(x), synth.as_u16(wr), None, Wn["gu_codes"],
                                   Wn["gu_scales"], Wn["dn_codes"], Wn["dn_scales"], k)
    np.testing.assert_array_equal(ids.cpu().numpy(), ref["topk_ids"])
    assert np.abs(w.cpu().numpy() - ref["topk_w"]).max() <= W_TOL
    _close(_bf16_to_f64(y), ref["y64"], "y")


@pytest.mark.parametrize("T", [12, 160], ids=["gemv", "mfma"])
def test_fp8_expert_ffn_entry_and_exact_scaling(dev, T):
    moe = _moe()
    d, E, k, f = 256, 8, 3, 256
    cfg, x, wr, W = _case(T, d, E, k, f, 9)
    Wd = {n: v.to(dev) for n, v in W.items()}
    ids, _ = moe.moe_route(x.to(dev), wr.to(dev), k)
    counts, offsets, sorted_rows, row_pos = moe.moe_permute(ids, E)
    rows = moe.moe_expert_ffn_fp8(x.to(dev), Wd, offsets, sorted_rows, k)
    torch.cuda.synchronize()
    Wn = _np(W)
    xs = synth.as_u16(x)
    srt, off = sorted_rows.cpu().numpy(), offsets.cpu().numpy()
    for e in range(E):
        for p in range(off[e], off[e + 1]):
            t = srt[p] // k
            _, o = oracle.expert_row_fp8(xs[t], Wn["gu_codes"][e], Wn["gu_scales"][e],
                                         Wn["dn_codes"][e], Wn["dn_scales"][e], d, f)
            _close(_bf16_to_f64(rows[p]), o, "row %d" % p)
    # doubling expert e's down scales doubles its rows exactly; zero codes give 0
    e = int(ids[0, 0])
    Wd2 = dict(Wd)
    Wd2["dn_scales"] = Wd["dn_scales"].clone()
    Wd2["dn_scales"][e] *= 2
    Wd2["gu_codes"] = Wd["gu_codes"].clone()
    z = int(ids[1, 0]) if int(ids[1, 0]) != e else int(ids[1, 1])
    Wd2["gu_codes"][z] = 0
    rows2 = moe.moe_expert_ffn_fp8(x.to(dev), Wd2, offsets, sorted_rows, k)
    torch.cuda.synchronize()
    seg = slice(off[e], off[e + 1])
    assert torch.equal(rows2[seg].float(), 2 * rows[seg].float())
    assert (rows2[off[z]:off[z + 1]].float() == 0).all()
    rows3 = moe.moe_expert_ffn_fp8(x.to(dev), Wd, offsets, sorted_rows, k)
    torch.cuda.synchronize()
    assert torch.equal(rows3.view(torch.int16), rows.view(torch.int16))


_FULL = {}


def _full_parity(dev, cfg, tokens):
    moe = _moe()
    if cfg.index not in _FULL:
        _FULL.clear()
        torch.cuda.empty_cache()
        _FULL[cfg.index] = synth.gen_experts_fp8(cfg, device=dev)
    ex = _FULL[cfg.index]
    x_cpu = synth.gen_x(cfg)
    wr_cpu = synth.gen_router_w(cfg)
    bias = synth.gen_bias(cfg)
    y, ids, w = moe.moe_layer_forward_fp8(x_cpu.to(dev), wr_cpu.to(dev), ex, cfg.k,
                                          router_bias=None if bias is None else bias.to(dev),
                                          return_routing=True)
    torch.cuda.synchronize()
    sel = synth.as_u16(x_cpu)[tokens]
    lg = oracle.router_logits(sel, synth.as_u16(wr_cpu), None if bias is None else bias.numpy())
    ids_o, w_o = oracle.topk_softmax(lg, cfg.k)
    np.testing.assert_array_equal(ids.cpu().numpy()[tokens], ids_o)
    assert np.abs(w.cpu().numpy()[tokens] - w_o).max() <= W_TOL
    need = sorted(set(ids_o.ravel().tolist()))
    Wn = _np(synth.gen_experts_fp8(cfg, experts=need))
    remap = {e: i for i, e in enumerate(need)}

    def row(ij):
        i, j = ij
        r = remap[int(ids_o[i, j])]
        return oracle.expert_row_fp8(sel[i], Wn["gu_codes"][r], Wn["gu_scales"][r],
                                     Wn["dn_codes"][r], Wn["dn_scales"][r], cfg.d, cfg.f)[1]

    jobs = [(i, j) for i in range(len(tokens)) for j in range(cfg.k)]
    with cf.ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as pool:
        outs = list(pool.map(row, jobs))
    yg = _bf16_to_f64(y)
    for i, t in enumerate(tokens):
        y_o, _ = oracle.combine_token(w_o[i], np.stack(outs[i * cfg.k:(i + 1) * cfg.k]))
        _close(yg[t], y_o, "token %d" % t)


def test_fp8_decode_full_size(dev):
    _full_parity(dev, synth.CONFIGS[7], [0])


def test_fp8_prefill_full_size(dev):
    _full_parity(dev, synth.CONFIGS[8], [0, 4095])
    _FULL.clear()
    torch.cuda.empty_cache()
