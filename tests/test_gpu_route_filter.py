"""GPU parity of routing for many tokens (T >= 256 without logits output).

That path never materialises all canonical logits: bf16 MFMA logits and
certified error intervals pick the candidates, whose canonical logits are
then computed exactly.  Its top-k ids and softmax weights must therefore be
bit-identical to those of the canonical path (moe_route asked for its
logits computes all of them) and match the oracle's routing.  Covered:
random rows at several shapes, exact ties from duplicated router rows (lower
index first), a block of identical router rows that puts 41 or 71 tied
experts into the candidate lists (ranking at up to 64 candidates, then the
fallback), all-equal logits (more candidates than the filter keeps: every
expert is refined), rows holding subnormal or huge values (no finite
interval: every expert is refined), and the Zipf router bias.
"""
import numpy as np
import pytest
import torch

import oracle
from routed_expert_mxfp4_amd import synth

from test_gpu_parity import W_TOL, _small_cfg, dev  # noqa: F401

pytestmark = pytest.mark.gpu


def _moe():
    from routed_expert_mxfp4_amd import moe
    return moe


def _both_paths(dev, x, wr, k, bias=None):
    moe = _moe()
    xd, wd = x.to(dev), wr.to(dev)
    bd = None if bias is None else bias.to(dev)
    ids_c, w_c, logits = moe.moe_route(xd, wd, k, router_bias=bd, want_logits=True)
    ids_f, w_f = moe.moe_route(xd, wd, k, router_bias=bd)
    torch.cuda.synchronize()
    return (ids_c.cpu().numpy(), w_c.cpu().numpy(), logits.cpu().numpy(),
            ids_f.cpu().numpy(), w_f.cpu().numpy())


def _check(dev, x, wr, k, bias=None, oracle_check=True):
    ids_c, w_c, lg, ids_f, w_f = _both_paths(dev, x, wr, k, bias)
    np.testing.assert_array_equal(ids_f, ids_c)
    np.testing.assert_array_equal(w_f.view(np.uint32), w_c.view(np.uint32))
    if oracle_check:
        lg_o = oracle.router_logits(synth.as_u16(x), synth.as_u16(wr),
                                    None if bias is None else bias.numpy())
        assert (lg.view(np.uint32) == lg_o.view(np.uint32)).all()
        ids_o, w_o = oracle.topk_softmax(lg_o, k)
        np.testing.assert_array_equal(ids_f, ids_o)
        assert np.abs(w_f - w_o).max() <= W_TOL
    return ids_f


ROUTE_CASES = [
    # (T, d, E, k, seed)
    (256, 512, 64, 6, 81),           # smallest T of the filtered path
    (300, 1024, 256, 16, 82),        # ragged 128-token GEMM tiles
    (257, 192, 40, 5, 83),           # chunk length 3, E not a multiple of 64
    (320, 7168, 896, 16, 84),        # the layer's router shape (register-resident chunks)
    (272, 4096, 256, 8, 89),         # the second routing shape (64-element chunks in registers)
    (260, 64, 1000, 32, 85),         # k = 32, E near the limit, chunk length 1
]


@pytest.mark.parametrize("case", ROUTE_CASES, ids=[str(c) for c in ROUTE_CASES])
def test_filtered_routing_matches_canonical(dev, case):
    T, d, E, k, seed = case
    print("case", case, flush=True)
    cfg = _small_cfg(T, d, E, k, 64, seed)
    _check(dev, synth.gen_x(cfg), synth.gen_router_w(cfg), k)


def test_filtered_routing_exact_ties(dev):
    cfg = _small_cfg(288, 512, 128, 8, 64, 86)
    x = synth.gen_x(cfg)
    wr = synth.gen_router_w(cfg).clone()
    # duplicate the rows of experts that many tokens rank highly
    lg = oracle.router_logits(synth.as_u16(x), synth.as_u16(wr))
    top = np.bincount(np.argsort(-lg, axis=1)[:, :4].ravel(), minlength=cfg.E).argsort()[::-1][:6]
    for j, e in enumerate(top):
        wr[(e + 17 + j) % cfg.E] = wr[e]
    bias = torch.zeros(cfg.E, dtype=torch.float32)
    ids = _check(dev, x, wr, cfg.k, bias)
    # at least one token saw a tie between two selected experts
    ties = sum(len(set(lg_row)) < len(lg_row) for lg_row in
               oracle.router_logits(synth.as_u16(x), synth.as_u16(wr))[np.arange(cfg.T)[:, None], ids])
    assert ties > 0


def test_filtered_routing_all_equal_logits(dev):
    cfg = _small_cfg(256, 256, 96, 6, 64, 87)
    x = synth.gen_x(cfg)
    wr = torch.zeros((cfg.E, cfg.d), dtype=torch.bfloat16)
    ids = _check(dev, x, wr, cfg.k)
    np.testing.assert_array_equal(ids, np.tile(np.arange(cfg.k, dtype=np.int32), (cfg.T, 1)))


def test_filtered_routing_subnormal_and_huge_rows(dev):
    cfg = _small_cfg(256, 256, 64, 4, 64, 88)
    x = synth.gen_x(cfg).clone()
    xb = x.view(torch.int16)
    xb[3, 7] = 1                                     # a bf16 subnormal
    x[5] = x[5] * 1e30                                # huge but finite logits
    wr = synth.gen_router_w(cfg)
    _check(dev, x, wr, cfg.k)


def test_filtered_routing_zipf_bias(dev):
    cfg = synth.CONFIGS[3]
    small = _small_cfg(256, cfg.d, cfg.E, cfg.k, 64, 3)
    x = synth.gen_x(small)
    wr = synth.gen_router_w(cfg)
    bias = synth.gen_bias(cfg)
    _check(dev, x, wr, cfg.k, bias)


@pytest.mark.parametrize("copies", [40, 70])
def test_filtered_routing_many_tied_candidates(dev, copies):
    # expert 5's router row copied into `copies` others: for every token
    # where it ranks high, all copies tie with it, so a token's candidate
    # list holds them all (40: ranked within the 64-entry list; 70: more
    # than it holds, so every expert is refined for that token)
    cfg = _small_cfg(256, 512, 128, 16, 64, 90 + copies)
    x = synth.gen_x(cfg)
    wr = synth.gen_router_w(cfg).clone()
    for j in range(copies):
        wr[(5 + 1 + 3 * j) % cfg.E] = wr[5]
    ids = _check(dev, x, wr, cfg.k)
    lg = oracle.router_logits(synth.as_u16(x), synth.as_u16(wr))
    tied = (lg[:, 5:6] == lg).sum(axis=1)
    # the copies really tie, and some token takes several of them
    assert tied.min() >= copies + 1
    assert (np.isin(ids, [5] + [(5 + 1 + 3 * j) % cfg.E for j in range(copies)]).sum(axis=1) >= 2).any()
