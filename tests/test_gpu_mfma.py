"""GPU parity of the scaled-MFMA (prefill) expert path.

* The activation split (two-term MX E2M3 codes and E8M0 scales) must equal
  the oracle's OCP MX conversion model bit for bit.
* The layer on shapes that take the MFMA path (T >= 128, d a multiple of
  512, f of 256) must match the oracle within max|gpu - oracle| <= 1e-2 max|oracle|,
  with routing and grouping bit-exact; ragged tiles and experts spanning
  several 128-row tiles are covered.
* The skewed 4096-token and the 32768-token workloads at full size: routing
  of sampled tokens bit-exact, their outputs within tolerance.
"""
import numpy as np
import pytest
import torch

import oracle
from routed_expert_mxfp4_amd import synth

from test_gpu_parity import (_FULL, _bf16_to_f64, _close, _decode_parity, _dev_experts,
                             _np_experts, _oracle_o_rows, _small_cfg, dev, full_experts)  # noqa: F401

pytestmark = pytest.mark.gpu


def _moe():
    from routed_expert_mxfp4_amd import moe
    return moe


def _unpack(q, K):
    """GPU split layout -> per-element codes [R][K] and scales [R][K/32]
    (hi, lo).  Per row and 128-element step: block g at 48 g holds
    [hi 0..15][lo 0..15][hi 16..23][lo 16..23] of the two 24-byte code
    streams, then the scales (hi, lo) per block at 192 + 2 g."""
    R = q.shape[0]
    nst = K // 128
    st = q.reshape(R, nst, 208)
    blk = st[:, :, :192].reshape(R, nst, 4, 48)
    hi = np.concatenate([blk[..., 0:16], blk[..., 32:40]], axis=-1)      # [R][st][g][24]
    lo = np.concatenate([blk[..., 16:32], blk[..., 40:48]], axis=-1)
    assert (st[:, :, 200:] == 0).all()

    def codes(b):
        bits = np.unpackbits(b, axis=-1, bitorder="little").reshape(R, nst, 4, 32, 6)
        return (bits * (1 << np.arange(6))).sum(-1).astype(np.uint8).reshape(R, K)
    sc = st[:, :, 192:200].reshape(R, nst, 4, 2)
    return (sc[..., 0].reshape(R, K // 32), codes(hi), sc[..., 1].reshape(R, K // 32), codes(lo))


def _split_inputs():
    rng = np.random.default_rng(77)
    R, K = 24, 512
    v = rng.standard_normal((R, K)) * np.exp(rng.standard_normal((R, K)) * 3)
    v[0, :32] = 0.0                                   # all-zero block
    v[1, :32] = -0.0                                  # negative zeros
    v[2, :64] = rng.standard_normal(64) * 1e-40       # fp32 subnormals
    v[3, :32] = 1e30 * rng.standard_normal(32)        # large
    # exact E2M3 midpoints relative to the block scale (ties to even)
    grid = np.array([0, 1, 2, 3, 4, 5, 6, 7]) / 8.0
    mids = (grid[:-1] + grid[1:]) / 2
    v[4, :32] = np.concatenate([[7.5], mids, -mids, mids * 2 + 0, np.full(32 - 1 - 21, 0.3)])[:32]
    v[5, :32] = np.linspace(-7.9, 7.9, 32)            # saturation above 7.5
    return v.astype(np.float32)


def test_activation_split_bit_exact_fp32(dev):
    moe = _moe()
    v = _split_inputs()
    q = moe.diag_mx_split_e2m3(torch.from_numpy(v).to(dev))
    torch.cuda.synchronize()
    hs, hc, ls, lc = _unpack(q.cpu().numpy(), v.shape[1])
    ohs, ohc, ols, olc = oracle.mx_split_rows(oracle.FMT_E2M3, v)
    np.testing.assert_array_equal(hs, ohs)
    np.testing.assert_array_equal(ls, ols)
    np.testing.assert_array_equal(hc, ohc)
    np.testing.assert_array_equal(lc, olc)


def test_activation_split_bit_exact_bf16_workload_rows(dev):
    moe = _moe()
    cfg = synth.CONFIGS[4]
    x = synth.gen_x(cfg, tokens=range(16))
    q = moe.diag_mx_split_e2m3(x.to(dev))
    torch.cuda.synchronize()
    hs, hc, ls, lc = _unpack(q.cpu().numpy(), cfg.d)
    ohs, ohc, ols, olc = oracle.mx_split_rows(oracle.FMT_E2M3, x.float().numpy())
    np.testing.assert_array_equal(hs, ohs)
    np.testing.assert_array_equal(hc, ohc)
    np.testing.assert_array_equal(ls, ols)
    np.testing.assert_array_equal(lc, olc)


def _exhaustive_blocks():
    """Every finite bf16 value, placed in 32-element blocks under a set of
    block maxima.  For each anchor M, the values v with |v| <= M (both signs,
    +-0 and the subnormals included) fill 31 lanes of each block and M takes
    the remaining lane (its position cycling over the 32), so the block's
    shared exponent is floor(log2 M) - 2 (clamped at -127) while every value
    is quantised under it; the residual term gets its own exponent.  Rows
    of 128 elements (4 blocks), zero blocks pad the last row."""
    bits = np.arange(1 << 16, dtype=np.uint32)
    finite = bits[(bits & 0x7F80) != 0x7F80]
    vals = (finite << 16).view(np.float32)
    anchors = [np.float32(v) for v in (
        (np.uint32(0x7F7F) << 16).view(np.float32),      # largest finite bf16
        2.0 ** 100, 2.0 ** 20, 448.0, 7.5, 1.0, 0.75, 1.5 * 2.0 ** -20, 2.0 ** -100,
        2.0 ** -124, 2.0 ** -125, 2.0 ** -126, 2.0 ** -130, 2.0 ** -133)]
    blocks = []
    for M in anchors:
        v = vals[np.abs(vals) <= M]
        nb = -(-v.size // 31)
        v = np.concatenate([v, np.zeros(nb * 31 - v.size, np.float32)]).reshape(nb, 31)
        pos = np.arange(nb) % 32
        blk = np.zeros((nb, 32), np.float32)
        for b in range(nb):
            blk[b] = np.insert(v[b], pos[b], M)
        blocks.append(blk)
    allb = np.concatenate(blocks)
    pad = (-allb.shape[0]) % 4
    allb = np.concatenate([allb, np.zeros((pad, 32), np.float32)])
    return allb.reshape(-1, 128)


def test_activation_split_exhaustive_bf16_values(dev):
    moe = _moe()
    v = _exhaustive_blocks()
    print("exhaustive split: %d blocks" % (v.size // 32), flush=True)
    ohs, ohc, ols, olc = oracle.mx_split_rows(oracle.FMT_E2M3, v)
    for kind in ("bf16", "fp32"):
        t = torch.from_numpy(v)
        t = t.to(torch.bfloat16) if kind == "bf16" else t
        assert torch.equal(t.float(), torch.from_numpy(v))          # exact in bf16
        q = moe.diag_mx_split_e2m3(t.to(dev))
        torch.cuda.synchronize()
        hs, hc, ls, lc = _unpack(q.cpu().numpy(), v.shape[1])
        for got, want, what in ((hs, ohs, "hi scales"), (hc, ohc, "hi codes"),
                                (ls, ols, "lo scales"), (lc, olc, "lo codes")):
            bad = np.argwhere(got != want)
            assert bad.size == 0, "%s input, %s differ at %d places, first %s" % (
                kind, what, len(bad), bad[:4].tolist())


MFMA_CASES = [
    # (T, d, E, k, f, seed); the MFMA path takes d % 512 == 0, f % 256 == 0
    (200, 512, 16, 4, 256, 71),      # ragged tiles
    (400, 512, 8, 4, 256, 72),       # ~200 rows per expert: two 128-row tiles each
    (300, 1024, 40, 6, 256, 73),     # 8 K steps of gate/up (loop tail after 3 x 2)
    (128, 512, 64, 2, 768, 74),      # 6 K steps of down, three n-blocks; one-row experts
    (160, 1536, 12, 2, 512, 76),     # 12 / 4 K steps, three down n-blocks
]


@pytest.mark.parametrize("case", MFMA_CASES, ids=[str(c) for c in MFMA_CASES])
def test_mfma_path_small(dev, case):
    moe = _moe()
    T, d, E, k, f, seed = case
    cfg = _small_cfg(T, d, E, k, f, seed)
    print("case", case, flush=True)
    L = synth.gen_layer(cfg)
    x16, wr16 = synth.as_u16(L["x"]), synth.as_u16(L["router_w"])
    W = _np_experts(L)
    lg = oracle.router_logits(x16, wr16)
    ids_o, w_o = oracle.topk_softmax(lg, k)
    counts_o, offsets_o, sr_o, rp_o = oracle.permute(ids_o, E)
    o_rows = _oracle_o_rows(x16, ids_o, W, d, f)
    y_o = np.einsum("tj,tjd->td", w_o, o_rows)
    x, wr = L["x"].to(dev), L["router_w"].to(dev)
    ex = _dev_experts(L, dev)
    ids, w = moe.moe_route(x, wr, k)
    counts, offsets, sr, rp = moe.moe_permute(ids, E)
    rows_out = moe.moe_expert_ffn(x, ex, offsets, sr, k)
    y2, ids2, w2 = moe.moe_layer_forward(x, wr, ex, k, return_routing=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ids.cpu().numpy(), ids_o)
    np.testing.assert_array_equal(sr.cpu().numpy(), sr_o)
    np.testing.assert_array_equal(ids2.cpu().numpy(), ids_o)
    o_sorted = o_rows.reshape(T * k, d)[sr_o]
    _close(_bf16_to_f64(rows_out), o_sorted, "rows_out")
    _close(_bf16_to_f64(y2), y_o, "layer_forward y")


def _skewed_case(T, d, E, k, f, seed):
    """A layer whose router bias makes a few experts hot and many cold, so
    that one call holds experts on both sides of the GEMV / MFMA crossover."""
    cfg = _small_cfg(T, d, E, k, f, seed)
    L = synth.gen_layer(cfg)
    bias = torch.zeros(E, dtype=torch.float32)
    bias[:4] = 0.3                       # hot experts
    bias[E // 2:] = -0.6                 # cold experts: a few rows or none
    return cfg, L, bias


def test_mixed_path_in_one_call(dev):
    """Experts with at most the crossover's rows take the GEMVs, the others
    the MFMA tiles, in the same call; both match the oracle."""
    moe = _moe()
    T, d, E, k, f = 160, 512, 32, 4, 256
    cfg, L, bias = _skewed_case(T, d, E, k, f, 91)
    x16, wr16 = synth.as_u16(L["x"]), synth.as_u16(L["router_w"])
    W = _np_experts(L)
    lg = oracle.router_logits(x16, wr16, bias.numpy())
    ids_o, w_o = oracle.topk_softmax(lg, k)
    counts = np.bincount(ids_o.ravel(), minlength=E)
    R = moe.diag_gemv_max_rows()
    assert R >= 1
    assert ((counts >= 1) & (counts <= R)).any() and (counts > R).any(), counts
    o_rows = _oracle_o_rows(x16, ids_o, W, d, f)
    y_o = np.einsum("tj,tjd->td", w_o, o_rows)
    x, wr, bd = L["x"].to(dev), L["router_w"].to(dev), bias.to(dev)
    ex = _dev_experts(L, dev)
    launched = {}
    for kname in ("gemv_gate_up", "gate_up_mfma", "gemv_down", "down_mfma"):
        moe.diag_time_kernel(kname, capacity=4)
        y, ids, w = moe.moe_layer_forward(x, wr, ex, k, router_bias=bd, return_routing=True)
        torch.cuda.synchronize()
        launched[kname] = moe.diag_kernel_time()[1]
    moe.diag_time_kernel(None, 0)
    assert all(n == 1 for n in launched.values()), launched
    np.testing.assert_array_equal(ids.cpu().numpy(), ids_o)
    _close(_bf16_to_f64(y), y_o, "mixed layer y")
    ids2, w2 = moe.moe_route(x, wr, k, router_bias=bd)
    counts_d, offsets, sr, rp = moe.moe_permute(ids2, E)
    rows_out = moe.moe_expert_ffn(x, ex, offsets, sr, k)
    torch.cuda.synchronize()
    _, _, sr_o, _ = oracle.permute(ids_o, E)
    _close(_bf16_to_f64(rows_out), o_rows.reshape(T * k, d)[sr_o], "mixed rows_out")


@pytest.mark.parametrize("override", [0, 1, 16, None])
def test_crossover_override(dev, override):
    """Every crossover setting (all MFMA tiles, GEMVs for one-row experts,
    GEMVs up to 16 rows, the built-in one) gives the oracle's result; T = 48
    takes the MFMA tiles only through the per-expert choice."""
    moe = _moe()
    T, d, E, k, f = 48, 512, 32, 4, 256
    cfg, L, bias = _skewed_case(T, d, E, k, f, 92)
    x16, wr16 = synth.as_u16(L["x"]), synth.as_u16(L["router_w"])
    W = _np_experts(L)
    lg = oracle.router_logits(x16, wr16, bias.numpy())
    ids_o, w_o = oracle.topk_softmax(lg, k)
    y_o = np.einsum("tj,tjd->td", w_o, _oracle_o_rows(x16, ids_o, W, d, f))
    moe.diag_set_gemv_max_rows(override)
    try:
        y = moe.moe_layer_forward(L["x"].to(dev), L["router_w"].to(dev), _dev_experts(L, dev), k,
                                  router_bias=bias.to(dev))
        torch.cuda.synchronize()
    finally:
        moe.diag_set_gemv_max_rows(None)
    _close(_bf16_to_f64(y), y_o, "override %s" % override)


def test_tile_heights_at_their_edges(dev):
    """Experts with 16, 17, 32, 33, 64, 65, 128 and 129 rows: tiles of 1, 2,
    2, 4, 4, 8, 8 and 8 + 1 m-tiles of 16 rows (the smallest height that
    holds a tile's rows), against the oracle row by row."""
    moe = _moe()
    n_e = [16, 17, 32, 33, 64, 65, 128, 129]
    E, k, d, f = len(n_e), 1, 512, 256
    T = sum(n_e)
    cfg = _small_cfg(T, d, E, k, f, 93)
    L = synth.gen_layer(cfg)
    # token t goes to the expert whose row range holds t (one slot per token)
    ids_np = np.repeat(np.arange(E, dtype=np.int32), n_e).reshape(T, 1)
    ids_np = ids_np[np.random.default_rng(93).permutation(T)]
    _, off_o, sr_o, _ = oracle.permute(ids_np, E)
    x16 = synth.as_u16(L["x"])
    W = _np_experts(L)
    o = np.zeros((T, d))
    for p, r in enumerate(sr_o):
        e = ids_np[r, 0]
        o[p] = oracle.expert_row(x16[r], W["gu_codes"][e], W["gu_scales"][e], W["dn_codes"][e],
                                 W["dn_scales"][e], d, f)[1]
    moe.diag_set_gemv_max_rows(0)                  # every expert on MFMA tiles
    try:
        counts, offsets, sr, rp = moe.moe_permute(torch.from_numpy(ids_np).to(dev), E)
        rows = moe.moe_expert_ffn(L["x"].to(dev), _dev_experts(L, dev), offsets, sr, k)
        torch.cuda.synchronize()
    finally:
        moe.diag_set_gemv_max_rows(None)
    np.testing.assert_array_equal(counts.cpu().numpy(), n_e)
    got = _bf16_to_f64(rows)
    for e in range(E):
        lo, hi = off_o[e], off_o[e + 1]
        _close(got[lo:hi], o[lo:hi], "expert with %d rows" % n_e[e])


def test_mfma_path_deterministic(dev):
    moe = _moe()
    cfg = _small_cfg(256, 512, 12, 3, 256, 75)
    L = synth.gen_layer(cfg)
    x, wr, ex = L["x"].to(dev), L["router_w"].to(dev), _dev_experts(L, dev)
    a = moe.moe_layer_forward(x, wr, ex, cfg.k)
    b = moe.moe_layer_forward(x, wr, ex, cfg.k)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def _layer_routing_is_the_router_entrys(dev, cfg, ids):
    """The routing the layer used (every token) equals moe_route's."""
    moe = _moe()
    bias = synth.gen_bias(cfg)
    ids_r, _ = moe.moe_route(synth.gen_x(cfg).to(dev), synth.gen_router_w(cfg).to(dev), cfg.k,
                             router_bias=None if bias is None else bias.to(dev))
    torch.cuda.synchronize()
    assert torch.equal(ids.cpu(), ids_r.cpu())


def test_skewed_prefill_full_size(dev, full_experts):
    cfg = synth.CONFIGS[3]
    full_experts(3)
    ids = _decode_parity(dev, cfg, 0, [0, 1777, 4095])
    _layer_routing_is_the_router_entrys(dev, cfg, ids)
    # the Zipf bias concentrates load: the hottest expert at about ten times
    # the mean (beta bisected for [9.5, 10.5] on the oracle's routing)
    counts = torch.bincount(ids.flatten().long(), minlength=cfg.E).cpu().numpy()
    ratio = counts.max() / (cfg.T * cfg.k / cfg.E)
    print("max/mean expert load", ratio)
    assert 9.5 <= ratio <= 10.5
    assert (counts > 0).all()


def test_long_prefill_full_size(dev, full_experts):
    cfg = synth.CONFIGS[4]
    full_experts(4)
    ids = _decode_parity(dev, cfg, 0, [0, 12345, 32767])
    _layer_routing_is_the_router_entrys(dev, cfg, ids)


def test_second_shape_prefill_full_size(dev, full_experts):
    # 256 experts, top-8, d = 4096, f = 2048, 4096 tokens
    cfg = synth.CONFIGS[6]
    full_experts(6)
    _decode_parity(dev, cfg, 0, [0, 2048, 4095])
