"""GPU parity of the MoE tail (include/moe_tail.h) against the CPU oracle.

Bar: xn (the RMSNorm output) and the routing ids bit-exact; routing weights
within 1e-5; the block output within max|gpu - oracle| <= 1e-2 *
max|oracle|.  The paths: few tokens (T <= 8: shared expert GEMVs, the
residual add in their down pass) and many (shared expert on the library
GEMM, the residual add in the combine pass), each with the routed layer's
GEMV or scaled-MFMA experts, with and without a shared expert.
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


def _u16(t):
    return synth.as_u16(t)


def _bf16_to_f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def _close(gpu, ref, what):
    err = float(np.max(np.abs(gpu - ref)))
    scale = float(np.max(np.abs(ref)))
    assert err <= TOL * scale, "%s: max err %.4g > %.0e * %.4g" % (what, err, TOL, scale)
    return err, scale


def _bits_to_bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)


@pytest.mark.parametrize("T,d,eps", [(33, 64, 1e-6), (7, 192, 0.0), (65, 7168, 1e-6),
                                     (3, 4096, 1e-5)])
def test_rmsnorm_bit_exact(dev, T, d, eps):
    moe = _moe()
    g = torch.Generator().manual_seed(T * 1000 + d)
    scales = torch.logspace(-5, 3, T, dtype=torch.float64).view(T, 1)
    x = (torch.randn(T, d, generator=g, dtype=torch.float64) * scales).to(torch.bfloat16)
    gamma = (1.0 + 0.3 * torch.randn(d, generator=g)).to(torch.bfloat16)
    if eps > 0:
        x[0] = 0.0                                   # an all-zero row: xn = 0
    xn = moe.moe_rmsnorm(x.to(dev), gamma.to(dev), eps)
    torch.cuda.synchronize()
    ref = oracle.rmsnorm(_u16(x), _u16(gamma), eps)
    np.testing.assert_array_equal(_u16(xn), ref)


def test_rmsnorm_subnormal_and_overflowing_outputs(dev):
    moe = _moe()
    d = 128
    g = torch.Generator().manual_seed(5)
    x = torch.randn(4, d, generator=g).to(torch.bfloat16)
    # gamma spans bf16 subnormals (down to 2^-133) and values near the top of
    # the range, so xn hits the subnormal rounding and the overflow to inf
    ex = torch.linspace(-133, 127, d).round()
    gamma = (torch.pow(2.0, ex.double()) * (1 + 0.5 * torch.rand(d, generator=g).double()))
    gamma = gamma.to(torch.float32).to(torch.bfloat16)
    # the last inputs, |x| = 4 against gamma ~ 2^127: |xn| >= 2^128 -> +-inf
    x[:, -4:] = 4.0
    x[1, -4:] = -4.0
    xn = moe.moe_rmsnorm(x.to(dev), gamma.to(dev), 1e-6)
    torch.cuda.synchronize()
    ref = oracle.rmsnorm(_u16(x), _u16(gamma), 1e-6)
    got = _u16(xn)
    np.testing.assert_array_equal(got, ref)
    assert ((ref & 0x7F80) == 0).any() and ((ref & 0x7FFF) == 0x7F80).any()


def _small(T, d, E, k, f, fs, seed, zero_experts=False, bias=False):
    cfg = synth.Config(200 + seed, "case", T, d, E, k, f, seed=seed)
    L = synth.gen_layer(cfg)
    if zero_experts:
        for n in ("gu_codes", "dn_codes"):
            L[n].zero_()
    if bias:
        L["bias"] = (0.05 * torch.randn(E, generator=torch.Generator().manual_seed(seed)))
    tail = synth.gen_tail(cfg, fs=fs) if fs else dict(synth.gen_tail(cfg, fs=32),
                                                        shared_gu=None, shared_dn=None)
    return cfg, L, tail


def _gpu_block(dev, cfg, L, tail, act=0):
    moe = _moe()
    ex = {n: L[n].to(dev) for n in ("gu_codes", "gu_scales", "dn_codes", "dn_scales")}
    td = {"gamma": tail["gamma"].to(dev), "eps": tail["eps"],
          "shared_gu": None if tail["shared_gu"] is None else tail["shared_gu"].to(dev),
          "shared_dn": None if tail["shared_dn"] is None else tail["shared_dn"].to(dev)}
    bias = None if L["bias"] is None else L["bias"].to(dev)
    out, ids, w = moe.moe_block_forward(L["x"].to(dev), L["router_w"].to(dev), ex, cfg.k, td,
                                        router_bias=bias, return_routing=True, act=act)
    torch.cuda.synchronize()
    return out, ids, w


def _oracle_block(cfg, L, tail):
    sgu = None if tail["shared_gu"] is None else _u16(tail["shared_gu"])
    sdn = None if tail["shared_dn"] is None else _u16(tail["shared_dn"])
    return oracle.block_forward(_u16(L["x"]), _u16(tail["gamma"]), tail["eps"],
                                _u16(L["router_w"]),
                                None if L["bias"] is None else L["bias"].numpy(),
                                L["gu_codes"].numpy(), L["gu_scales"].numpy(),
                                L["dn_codes"].numpy(), L["dn_scales"].numpy(), sgu, sdn, cfg.k)


BLOCK_CASES = [
    # (T, d, E, k, f, fs, seed): the path is set by T (and d, f for MFMA)
    (1, 256, 16, 2, 128, 128, 0),     # one token: fused top-k gate/up, shared GEMVs
    (8, 256, 16, 2, 128, 128, 1),     # the tiny workload's shape
    (5, 192, 40, 5, 64, 96, 2),       # odd chunk length, unfused routed down
    (3, 256, 16, 2, 128, 0, 3),       # no shared expert, few tokens
    (20, 256, 24, 3, 128, 64, 4),     # many tokens: shared GEMMs, combine adds
    (40, 256, 24, 3, 128, 0, 5),      # no shared expert, many tokens
    (200, 512, 16, 2, 256, 256, 6),   # scaled-MFMA routed experts (T >= 128)
    (300, 512, 24, 4, 256, 160, 7),   # filtered routing (T >= 256), ragged fs
    (20, 256, 24, 3, 128, 96, 8),     # shared down GEMM's K = 96: a half K step
    (12, 192, 40, 5, 64, 96, 9),      # d = 192: a half N tile in the down GEMM
    (520, 1024, 32, 4, 256, 320, 10), # five row tiles (the last ragged), five gate tiles
]


@pytest.mark.parametrize("case", BLOCK_CASES, ids=[str(c) for c in BLOCK_CASES])
def test_block_small(dev, case):
    T, d, E, k, f, fs, seed = case
    print("block case", case, flush=True)
    cfg, L, tail = _small(T, d, E, k, f, fs, seed, bias=(seed % 2 == 1))
    out, ids, w = _gpu_block(dev, cfg, L, tail)
    ref = _oracle_block(cfg, L, tail)
    np.testing.assert_array_equal(ids.cpu().numpy(), ref["topk_ids"])
    assert np.abs(w.cpu().numpy() - ref["topk_w"]).max() <= W_TOL
    _close(_bf16_to_f64(out), ref["out64"], "block out")


@pytest.mark.parametrize("T", [9, 333])
def test_block_shared_expert_at_the_model_shape(dev, T):
    """Routed experts all zero, so out = x + shared(xn): the shared expert's
    two matrix-core GEMMs at d = 7168, fs = 1536 (ragged row tiles) against
    the oracle's fp64 shared expert."""
    cfg, L, tail = _small(T, 7168, 8, 2, 256, 1536, 60 + T, zero_experts=True)
    out, _, _ = _gpu_block(dev, cfg, L, tail)
    ref = _oracle_block(cfg, L, tail)
    err, scale = _close(_bf16_to_f64(out), ref["out64"], "block out")
    print("T=%d: max err %.3g of max|out| %.3g" % (T, err, scale))


@pytest.mark.parametrize("T", [2, 6, 20, 150])
def test_block_residual_exact(dev, T):
    """All-zero routed experts and a zero shared expert: out == x bit for bit
    (the residual passes through both epilogues unchanged)."""
    cfg, L, tail = _small(T, 512, 16, 2, 256, 64, 30 + T, zero_experts=True)
    tail["shared_dn"] = torch.zeros_like(tail["shared_dn"])
    out, _, _ = _gpu_block(dev, cfg, L, tail)
    assert torch.equal(out.cpu().view(torch.int16), L["x"].view(torch.int16))


@pytest.mark.parametrize("T", [4, 24])
def test_block_residual_visible(dev, T):
    """A residual far larger than the expert terms: the output must carry it
    (the tolerance alone would not see a dropped residual at the usual
    magnitudes)."""
    cfg, L, tail = _small(T, 256, 16, 2, 128, 64, 40 + T)
    for n in ("gu_scales", "dn_scales"):
        L[n].fill_(100)                           # expert weights scaled by 2^-27
    tail["shared_dn"] = (tail["shared_dn"].float() * 2.0 ** -20).to(torch.bfloat16)
    L["x"] = (L["x"].float() * 1e4).to(torch.bfloat16)
    out, _, _ = _gpu_block(dev, cfg, L, tail)
    ref = _oracle_block(cfg, L, tail)
    _close(_bf16_to_f64(out), ref["out64"], "block out")
    xf = _bf16_to_f64(L["x"])
    assert np.abs(ref["out64"] - xf).max() < 1e-3 * np.abs(xf).max()   # x dominates


def test_block_deterministic(dev):
    cfg, L, tail = _small(20, 256, 24, 3, 128, 64, 50)
    a, _, _ = _gpu_block(dev, cfg, L, tail)
    b, _, _ = _gpu_block(dev, cfg, L, tail)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


# ---- full sizes: sampled tokens against the oracle's steps ------------------------
_FULL = {}


@pytest.fixture(scope="module")
def full_experts(dev):
    def get(index):
        if index not in _FULL:
            _FULL.clear()
            torch.cuda.empty_cache()
            _FULL[index] = synth.gen_experts(synth.CONFIGS[index], device=dev)
        return _FULL[index]
    yield get
    _FULL.clear()


def _block_parity_full(dev, cfg, batch, tokens, ex):
    """The block at full size on the GPU; for the sampled tokens the oracle's
    steps in the block's order (RMSNorm, routing of xn, the selected experts
    and the combine, the shared expert, the residual)."""
    moe = _moe()
    x_cpu = synth.gen_x(cfg, batch)
    wr_cpu = synth.gen_router_w(cfg)
    bias = synth.gen_bias(cfg)
    tail = synth.gen_tail(cfg)
    td = {"gamma": tail["gamma"].to(dev), "eps": tail["eps"],
          "shared_gu": tail["shared_gu"].to(dev), "shared_dn": tail["shared_dn"].to(dev)}
    out, ids, w = moe.moe_block_forward(x_cpu.to(dev), wr_cpu.to(dev), ex, cfg.k, td,
                                        router_bias=None if bias is None else bias.to(dev),
                                        return_routing=True)
    torch.cuda.synchronize()
    x16 = _u16(x_cpu)[tokens]
    xn = oracle.rmsnorm(x16, _u16(tail["gamma"]), tail["eps"])
    lg = oracle.router_logits(xn, _u16(wr_cpu), None if bias is None else bias.numpy())
    ids_o, w_o = oracle.topk_softmax(lg, cfg.k)
    np.testing.assert_array_equal(ids.cpu().numpy()[tokens], ids_o)
    assert np.abs(w.cpu().numpy()[tokens] - w_o).max() <= W_TOL
    need = sorted(set(ids_o.ravel().tolist()))
    Wn = {n: v.numpy() for n, v in synth.gen_experts(cfg, experts=need).items()}
    remap = {e: i for i, e in enumerate(need)}
    sgu, sdn = _u16(tail["shared_gu"]), _u16(tail["shared_dn"])

    def row(ij):
        i, j = ij
        if j == cfg.k:
            return oracle.shared_expert_row(xn[i], sgu, sdn)[1]
        r = remap[int(ids_o[i, j])]
        return oracle.expert_row(xn[i], Wn["gu_codes"][r], Wn["gu_scales"][r],
                                 Wn["dn_codes"][r], Wn["dn_scales"][r], cfg.d, cfg.f)[1]

    jobs = [(i, j) for i in range(len(tokens)) for j in range(cfg.k + 1)]
    with cf.ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as pool:
        outs = list(pool.map(row, jobs))
    og = _bf16_to_f64(out)
    for i, t in enumerate(tokens):
        rows = outs[i * (cfg.k + 1):(i + 1) * (cfg.k + 1)]
        y_o, _ = oracle.combine_token(w_o[i], np.stack(rows[:cfg.k]))
        ref = oracle.bf16_array_to_f64(x16[i]) + y_o + rows[cfg.k]
        _close(og[t], ref, "token %d" % t)


def test_block_decode_full_size(dev, full_experts):
    cfg = synth.CONFIGS[1]
    ex = full_experts(1)
    for batch in (0, 999):
        print("block decode token", batch, flush=True)
        _block_parity_full(dev, cfg, batch, [0], ex)


def test_block_batched_decode_full_size(dev, full_experts):
    cfg = synth.CONFIGS[2]
    ex = full_experts(2)
    _block_parity_full(dev, cfg, 0, [0, 63], ex)


def test_block_prefill_full_size(dev, full_experts):
    cfg = synth.CONFIGS[3]
    ex = full_experts(3)
    _block_parity_full(dev, cfg, 0, [0, 2047, 4095], ex)
