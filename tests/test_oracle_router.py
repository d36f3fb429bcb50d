"""Pins for the oracle's router, top-k selection, softmax and permutation.

References used here are independent of the oracle: exact rational dot
products, Python's stable ``sorted``, scipy's softmax, and hand-derived
values for the summation-order example.
"""
from fractions import Fraction

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from routed_expert_mxfp4_amd import synth


def _bf16_bits(a):
    t = torch.tensor(np.asarray(a, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _bf16_val(bits):
    return torch.from_numpy(np.asarray(bits, np.uint16).view(np.int16).copy()).view(
        torch.bfloat16).to(torch.float64).numpy()


def test_router_exact_on_dyadic_inputs():
    # small dyadic inputs: every partial sum is exact in fp64 and the result
    # is exact in fp32, so the logit must equal the exact rational dot product
    rng = np.random.default_rng(1)
    T, d, E = 3, 128, 5                       # T != E catches a transposed operand
    x = rng.integers(-16, 17, (T, d)) / 8.0
    w = rng.integers(-16, 17, (E, d)) / 64.0
    b = rng.integers(-64, 65, E) / 32.0
    xb, wb = _bf16_bits(x), _bf16_bits(w)
    got = oracle.router_logits(xb, wb, b.astype(np.float32))
    for t in range(T):
        for e in range(E):
            exact = sum(Fraction(float(x[t, i])) * Fraction(float(w[e, i]))
                        for i in range(d)) + Fraction(float(b[e]))
            assert Fraction(float(got[t, e])) == exact


def test_router_close_to_exact_on_gaussian_inputs():
    cfg = synth.CONFIGS[0]
    x = synth.gen_x(cfg)
    w = synth.gen_router_w(cfg)
    xb, wb = synth.as_u16(x), synth.as_u16(w)
    got = oracle.router_logits(xb, wb)
    xv, wv = _bf16_val(xb), _bf16_val(wb)
    n_equal = 0
    for t in range(cfg.T):
        for e in range(cfg.E):
            exact = sum(Fraction(float(xv[t, i])) * Fraction(float(wv[e, i]))
                        for i in range(cfg.d))
            rn = np.float32(float(exact))     # within 1 ulp of RN32(exact)
            diff = abs(float(got[t, e]) - float(rn))
            assert diff <= float(np.spacing(np.float32(abs(rn)))), (t, e)
            n_equal += int(got[t, e] == rn)
    # fp64 accumulation error is ~1e-16 relative: nearly always RN32(exact)
    assert n_equal >= cfg.T * cfg.E - 2


def test_router_summation_order_chunks_then_pairwise_tree():
    # d = 128 -> 64 chunks of 2.  Chunk 0 holds 2^60 and 1, chunk 1 holds
    # -2^60 and 1.  In fp64, 2^60 + 1 rounds to 2^60 and -2^60 + 1 rounds to
    # -2^60, so the chunk sums cancel in the tree and the canonical logit is
    # exactly the bias.  (A single running sum would give 1, the exact sum 2.)
    d = 128
    x = np.zeros((1, d), np.float32)
    w = np.zeros((1, d), np.float32)
    x[0, 0], w[0, 0] = 2.0 ** 30, 2.0 ** 30
    x[0, 1], w[0, 1] = 1.0, 1.0
    x[0, 2], w[0, 2] = -(2.0 ** 30), 2.0 ** 30
    x[0, 3], w[0, 3] = 1.0, 1.0
    got = oracle.router_logits(_bf16_bits(x), _bf16_bits(w), np.array([0.25], np.float32))
    assert got[0, 0] == np.float32(0.25)
    # the tree pairs chunk 0 with chunk 1 before anything else: put the
    # cancelling pair in chunks 0 and 2 instead, with chunk 1 holding 2^-1.
    # Level 1: (2^60 + 2^-1) rounds to 2^60, (-2^60 + 0) = -2^60; level 2
    # cancels them: the 2^-1 is lost.
    x = np.zeros((1, d), np.float32)
    w = np.zeros((1, d), np.float32)
    x[0, 0], w[0, 0] = 2.0 ** 30, 2.0 ** 30
    x[0, 2], w[0, 2] = 0.5, 1.0
    x[0, 4], w[0, 4] = -(2.0 ** 30), 2.0 ** 30
    got = oracle.router_logits(_bf16_bits(x), _bf16_bits(w))
    assert got[0, 0] == 0.0
    # pairwise versus running sum over the chunk sums: chunk sums 2^60, 0,
    # 128, 128, -2^60.  The tree forms 128 + 128 = 256 first, and 2^60 + 256
    # is exact, so the logit is 256.  A running sum adds 128 to 2^60 twice;
    # each is a tie that rounds back to 2^60 (even), giving 0.
    x = np.zeros((1, d), np.float32)
    w = np.zeros((1, d), np.float32)
    x[0, 0], w[0, 0] = 2.0 ** 30, 2.0 ** 30
    x[0, 4], w[0, 4] = 16.0, 8.0
    x[0, 6], w[0, 6] = 16.0, 8.0
    x[0, 8], w[0, 8] = -(2.0 ** 30), 2.0 ** 30
    got = oracle.router_logits(_bf16_bits(x), _bf16_bits(w))
    assert got[0, 0] == 256.0


def _ref_topk(logits, k):
    T, E = logits.shape
    ids = np.array([sorted(range(E), key=lambda e: (-float(logits[t, e]), e))[:k]
                    for t in range(T)], np.int32)
    return ids


@pytest.mark.parametrize("E,k", [(16, 2), (896, 16), (7, 7), (64, 1)])
def test_topk_matches_stable_sort_with_forced_ties(E, k):
    rng = np.random.default_rng(E * 100 + k)
    T = 40
    # few distinct values -> many exact ties, which must resolve to lower e
    logits = rng.integers(-3, 4, (T, E)).astype(np.float32) * np.float32(0.75)
    ids, w = oracle.topk_softmax(logits, k)
    np.testing.assert_array_equal(ids, _ref_topk(logits, k))
    sel = np.take_along_axis(logits.astype(np.float64), ids.astype(np.int64), 1)
    np.testing.assert_allclose(w, scipy.special.softmax(sel, axis=1), rtol=1e-14, atol=0)
    np.testing.assert_allclose(w.sum(1), 1.0, rtol=0, atol=1e-15)


def test_topk_with_duplicated_router_rows_picks_lower_index():
    # duplicated router rows give exactly equal canonical logits
    cfg = synth.CONFIGS[0]
    x = synth.as_u16(synth.gen_x(cfg))
    w = synth.as_u16(synth.gen_router_w(cfg)).copy()
    w[9] = w[3]
    w[12] = w[3]
    logits = oracle.router_logits(x, w)
    assert (logits[:, 3] == logits[:, 9]).all() and (logits[:, 3] == logits[:, 12]).all()
    ids, _ = oracle.topk_softmax(logits, cfg.E)
    for t in range(cfg.T):
        row = list(ids[t])
        assert row.index(3) < row.index(9) < row.index(12)
    np.testing.assert_array_equal(ids, _ref_topk(logits, cfg.E))


def test_topk_k_equals_E_is_full_softmax():
    rng = np.random.default_rng(5)
    logits = (rng.standard_normal((10, 16)) * 3).astype(np.float32)
    ids, w = oracle.topk_softmax(logits, 16)
    full = scipy.special.softmax(logits.astype(np.float64), axis=1)
    np.testing.assert_allclose(w, np.take_along_axis(full, ids.astype(np.int64), 1),
                               rtol=1e-14)


def _permute_checks(ids, E):
    T, k = ids.shape
    counts, offsets, sorted_rows, row_pos = oracle.permute(ids, E)
    ref = sorted(range(T * k), key=lambda r: (int(ids.flat[r]), r))
    np.testing.assert_array_equal(sorted_rows, np.array(ref, np.int32))
    assert counts.sum() == T * k
    np.testing.assert_array_equal(counts, np.bincount(ids.ravel(), minlength=E))
    assert offsets[0] == 0 and offsets[E] == T * k
    np.testing.assert_array_equal(np.diff(offsets), counts)
    assert sorted(sorted_rows.tolist()) == list(range(T * k))
    np.testing.assert_array_equal(row_pos[sorted_rows], np.arange(T * k))
    # each token appears exactly k times, once per selected expert
    tok = sorted_rows // k
    np.testing.assert_array_equal(np.bincount(tok, minlength=T), np.full(T, k))
    for e in range(E):
        seg = sorted_rows[offsets[e]:offsets[e + 1]]
        assert (np.diff(seg) > 0).all()
        assert (ids.ravel()[seg] == e).all()


def test_permute_matches_stable_sort_and_invariants():
    rng = np.random.default_rng(11)
    for T, E, k in [(8, 16, 2), (33, 40, 5), (1, 896, 16), (100, 7, 7)]:
        ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
        _permute_checks(ids, E)


def test_permute_empty_and_single_expert():
    counts, offsets, sr, rp = oracle.permute(np.zeros((0, 3), np.int32), 5)
    assert counts.sum() == 0 and (offsets == 0).all() and sr.size == 0
    ids = np.zeros((6, 1), np.int32)
    _permute_checks(ids, 1)


def test_c2_workload_is_tie_free_among_top17():
    # the batched-decode workload is stated to have distinct router logits
    cfg = synth.CONFIGS[2]
    x = synth.as_u16(synth.gen_x(cfg, tokens=range(8)))
    w = synth.as_u16(synth.gen_router_w(cfg))
    logits = oracle.router_logits(x, w)
    for t in range(x.shape[0]):
        top = np.sort(logits[t])[::-1][:17]
        assert len(set(top.tolist())) == 17
