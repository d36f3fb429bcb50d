"""Full-size parity of routing and grouping: every token of every workload.

* One-token decode (d = 7168, 896 experts, top-16): all 1000 seeded tokens
  go through moe_layer_forward one at a time; every token's expert ids must
  equal the oracle's and every weight must be within 1e-5 of it.  Layer
  outputs of 16 tokens spread over the 1000 are checked against the oracle.
* Batched decode (64 tokens): five of the seeded batches in full, ids and
  weights; every token's 17 largest canonical logits are distinct (the
  workload is tie-free, so the 16/17 boundary is never decided by index).
* Skewed (4096 tokens) and long (32768 tokens) prefill: the routing that the
  layer uses for many tokens (bf16 MFMA filter + certified intervals +
  canonical refinement) equals the canonical routing over ALL tokens, ids
  and weights bit for bit.  The canonical logits equal the oracle's bit for
  bit on a stratified sample of at least 256 tokens that holds tokens of the
  hottest and of the coldest expert.  moe_permute on the GPU's own ids
  equals the oracle's grouping bit for bit (counts, offsets, sorted rows,
  inverse).
* The skewed workload's load: max / mean rows per expert equals what the
  oracle's routing gives (tests/golden/zipf_beta.json, in [9.5, 10.5]).

Expected values come from the oracle only; inputs from the seeded generator.
"""
import concurrent.futures as cf
import json
import os

import numpy as np
import pytest
import torch

import oracle
from routed_expert_mxfp4_amd import synth

from test_gpu_parity import W_TOL, _FULL, _close, dev, full_experts  # noqa: F401

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
THREADS = max(1, min(16, os.cpu_count() or 1))


def _moe():
    from routed_expert_mxfp4_amd import moe
    return moe


def _pool_map(fn, items):
    with cf.ThreadPoolExecutor(max_workers=THREADS) as pool:
        return list(pool.map(fn, items))


def _oracle_logits(x16, wr16, bias):
    """Canonical logits of the given token rows (the oracle's C code releases
    the GIL, so token chunks run in parallel threads)."""
    b = None if bias is None else bias.numpy()
    chunks = [c for c in np.array_split(np.arange(x16.shape[0]), THREADS) if c.size]
    parts = _pool_map(lambda idx: oracle.router_logits(x16[idx], wr16, b), chunks)
    return np.concatenate(parts)


def _check_routing(ids_g, w_g, ids_o, w_o, what):
    bad = np.nonzero((ids_g != ids_o).any(1))[0]
    assert bad.size == 0, "%s: ids differ at %d tokens, first %s" % (what, bad.size, bad[:8])
    assert np.abs(w_g.astype(np.float64) - w_o).max() <= W_TOL, what
    assert np.abs(w_g.astype(np.float64).sum(1) - 1.0).max() <= 1e-6, what


def _oracle_y(x16_rows, ids_rows, w_rows, ex, cfg):
    """Oracle layer output of a few tokens, on the expert bytes read back from
    the device copy of the seeded store."""
    need = sorted(set(int(e) for e in ids_rows.ravel()))
    W = {n: ex[n][need].cpu().numpy() for n in ("gu_codes", "gu_scales", "dn_codes", "dn_scales")}
    at = {e: i for i, e in enumerate(need)}
    jobs = [(i, j) for i in range(ids_rows.shape[0]) for j in range(cfg.k)]

    def row(ij):
        i, j = ij
        r = at[int(ids_rows[i, j])]
        return oracle.expert_row(x16_rows[i], W["gu_codes"][r], W["gu_scales"][r],
                                 W["dn_codes"][r], W["dn_scales"][r], cfg.d, cfg.f)[1]

    outs = _pool_map(row, jobs)
    ys = []
    for i in range(ids_rows.shape[0]):
        o = np.stack(outs[i * cfg.k:(i + 1) * cfg.k])
        ys.append(oracle.combine_token(w_rows[i], o)[0])
    return np.stack(ys)


def test_decode_all_tokens(dev, full_experts):
    moe = _moe()
    cfg = synth.CONFIGS[1]
    ex = full_experts(1)
    n = cfg.batches
    wr = synth.gen_router_w(cfg)
    xs = torch.cat([synth.gen_x(cfg, b) for b in range(n)])           # [1000][d]
    layer = moe.Layer(ex, wr.to(dev), cfg.k, None, T=1)
    xd = xs.to(dev)
    ids = torch.empty((n, cfg.k), dtype=torch.int32, device=dev)
    w = torch.empty((n, cfg.k), dtype=torch.float32, device=dev)
    y = torch.empty((n, cfg.d), dtype=torch.bfloat16, device=dev)
    for b in range(n):
        layer.forward(xd[b:b + 1], y=y[b:b + 1], topk_ids=ids[b:b + 1], topk_w=w[b:b + 1])
    torch.cuda.synchronize()
    print("decode: %d tokens routed on the GPU" % n, flush=True)
    x16, wr16 = synth.as_u16(xs), synth.as_u16(wr)
    lg = _oracle_logits(x16, wr16, None)
    ids_o, w_o = oracle.topk_softmax(lg, cfg.k)
    ids_g, w_g = ids.cpu().numpy(), w.cpu().numpy()
    _check_routing(ids_g, w_g, ids_o, w_o, "decode routing, all tokens")
    sample = np.linspace(0, n - 1, 16).astype(int)
    y_o = _oracle_y(x16[sample], ids_o[sample], w_o[sample], ex, cfg)
    yg = y.float().cpu().numpy().astype(np.float64)
    for i, t in enumerate(sample):
        _close(yg[t], y_o[i], "decode token %d" % t)


def test_batched_decode_five_batches(dev, full_experts):
    moe = _moe()
    cfg = synth.CONFIGS[2]
    ex = full_experts(2)
    wr = synth.gen_router_w(cfg)
    wr16 = synth.as_u16(wr)
    layer = moe.Layer(ex, wr.to(dev), cfg.k, None, T=cfg.T)
    for batch in (0, 1, 17, 33, 49):
        x = synth.gen_x(cfg, batch)
        ids = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device=dev)
        w = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device=dev)
        y = layer.forward(x.to(dev), topk_ids=ids, topk_w=w)
        torch.cuda.synchronize()
        print("batched decode: batch", batch, flush=True)
        x16 = synth.as_u16(x)
        lg = _oracle_logits(x16, wr16, None)
        # the workload is tie-free at the selection boundary and inside it
        top17 = -np.sort(-lg, axis=1)[:, :cfg.k + 1]
        assert (np.diff(top17, axis=1) < 0).all(), "batch %d: tied canonical logits" % batch
        ids_o, w_o = oracle.topk_softmax(lg, cfg.k)
        _check_routing(ids.cpu().numpy(), w.cpu().numpy(), ids_o, w_o, "batch %d" % batch)
        if batch == 17:
            tok = np.array([5, 40])
            y_o = _oracle_y(x16[tok], ids_o[tok], w_o[tok], ex, cfg)
            yg = y.float().cpu().numpy().astype(np.float64)
            for i, t in enumerate(tok):
                _close(yg[t], y_o[i], "batch 17 token %d" % t)


def _stratified(ids, E, n_random, seed):
    """Tokens of the hottest expert (64), of the coldest (all, up to 64) and
    n_random others drawn with a seeded generator, sorted and unique."""
    counts = np.bincount(ids.ravel(), minlength=E)
    hot, cold = int(np.argmax(counts)), int(np.argmin(np.where(counts > 0, counts, 1 << 30)))
    hot_t = np.nonzero((ids == hot).any(1))[0][:64]
    cold_t = np.nonzero((ids == cold).any(1))[0][:64]
    rnd = np.random.default_rng(seed).choice(ids.shape[0], size=n_random, replace=False)
    sel = np.unique(np.concatenate([hot_t, cold_t, rnd]))
    return sel, hot, cold


@pytest.mark.parametrize("index", [3, 4])
def test_prefill_routing_and_grouping_all_tokens(dev, index):
    moe = _moe()
    cfg = synth.CONFIGS[index]
    print("workload", cfg.name, flush=True)
    x, wr, bias = synth.gen_x(cfg), synth.gen_router_w(cfg), synth.gen_bias(cfg)
    xd, wd = x.to(dev), wr.to(dev)
    bd = None if bias is None else bias.to(dev)
    ids_f, w_f = moe.moe_route(xd, wd, cfg.k, router_bias=bd)                  # filtered
    ids_c, w_c, lg = moe.moe_route(xd, wd, cfg.k, router_bias=bd, want_logits=True)
    torch.cuda.synchronize()
    ids_f, w_f = ids_f.cpu().numpy(), w_f.cpu().numpy()
    ids_c, w_c = ids_c.cpu().numpy(), w_c.cpu().numpy()
    bad = np.nonzero((ids_f != ids_c).any(1))[0]
    assert bad.size == 0, "filtered != canonical ids at %d tokens: %s" % (bad.size, bad[:8])
    assert (w_f.view(np.uint32) == w_c.view(np.uint32)).all(), "weights not bit-identical"
    print("filtered == canonical over %d tokens" % cfg.T, flush=True)
    # the canonical logits against the oracle on a stratified sample
    sel, hot, cold = _stratified(ids_c, cfg.E, 200, seed=index)
    assert sel.size >= 256
    lg_o = _oracle_logits(synth.as_u16(x)[sel], synth.as_u16(wr), bias)
    lg_g = lg.cpu().numpy()[sel]
    assert (lg_g.view(np.uint32) == lg_o.view(np.uint32)).all(), "canonical logits differ"
    ids_o, w_o = oracle.topk_softmax(lg_o, cfg.k)
    _check_routing(ids_c[sel], w_c[sel], ids_o, w_o, "stratified sample")
    print("oracle logits on %d tokens (hot expert %d, cold %d)" % (sel.size, hot, cold),
          flush=True)
    # grouping of the GPU's own ids
    counts, offsets, sr, rp = moe.moe_permute(torch.from_numpy(ids_f).to(dev), cfg.E)
    torch.cuda.synchronize()
    c_o, off_o, sr_o, rp_o = oracle.permute(ids_f, cfg.E)
    np.testing.assert_array_equal(counts.cpu().numpy(), c_o)
    np.testing.assert_array_equal(offsets.cpu().numpy(), off_o)
    np.testing.assert_array_equal(sr.cpu().numpy(), sr_o)
    np.testing.assert_array_equal(rp.cpu().numpy(), rp_o)
    mean = cfg.T * cfg.k / cfg.E
    print("rows per expert: max %d, min %d, max/mean %.3f" % (c_o.max(), c_o.min(),
                                                               c_o.max() / mean), flush=True)
    if index == 3:
        rec = json.load(open(os.path.join(GOLDEN, "zipf_beta.json")))
        assert rec["beta"] == cfg.zipf_beta
        assert int(c_o.max()) == rec["max_rows"] and int(c_o.min()) == rec["min_rows"]
        assert 9.5 <= c_o.max() / mean <= 10.5
        assert (c_o > 0).all()
