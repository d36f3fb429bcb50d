"""CPU oracle of one routed MoE FFN layer with MXFP4 experts (fp64, plain C).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The GPU library never imports,
links or calls anything here, and this package imports nothing from it.

The arithmetic lives in ``moe_oracle.c`` (see its header comment for the
passages of the pages each step follows); this module only marshals numpy
arrays through ctypes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
# An alternative build (the mutation test points this at deliberately
# broken copies of the oracle to show that the pins catch them).
_LIB_OVERRIDE = os.environ.get("MOE_ORACLE_LIB")
_lib = None

FMT_E4M3, FMT_E2M3, FMT_E2M1 = 0, 1, 2


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call([
            "gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
            "-std=c11", "-Wall", "-Wextra", "-shared", "-fPIC", "-o", tmp,
            _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            L = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            if not os.path.exists(_LIB_PATH) or (
                    os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
                build(force=True)
            L = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        i = ctypes.c_int
        L.orc_bf16_value.restype = ctypes.c_double
        L.orc_bf16_value.argtypes = [ctypes.c_uint16]
        L.orc_e2m1_value.restype = ctypes.c_double
        L.orc_e2m1_value.argtypes = [ctypes.c_uint]
        L.orc_e8m0_value.restype = ctypes.c_double
        L.orc_e8m0_value.argtypes = [ctypes.c_uint]
        L.orc_round_to_bf16.restype = ctypes.c_uint16
        L.orc_round_to_bf16.argtypes = [ctypes.c_double]
        L.orc_mxfp4_weight.restype = ctypes.c_double
        L.orc_mxfp4_weight.argtypes = [P, P, i, i, i]
        L.orc_router_logits.restype = None
        L.orc_router_logits.argtypes = [i, i, i, P, P, P, P]
        L.orc_topk_softmax.restype = None
        L.orc_topk_softmax.argtypes = [i, i, i, P, P, P]
        L.orc_permute.restype = None
        L.orc_permute.argtypes = [i, i, i, P, P, P, P, P]
        L.orc_expert_row.restype = None
        L.orc_expert_row.argtypes = [i, i, P, P, P, P, P, P, P]
        L.orc_combine_token.restype = None
        L.orc_combine_token.argtypes = [i, i, P, P, P, P]
        L.orc_layer_forward.restype = ctypes.c_int
        L.orc_layer_forward.argtypes = [i, i, i, i, i] + [P] * 12 + [i]
        L.orc_layer_forward_act.restype = ctypes.c_int
        L.orc_layer_forward_act.argtypes = [i, i, i, i, i, i] + [P] * 12 + [i]
        L.orc_expert_row_act.restype = None
        L.orc_expert_row_act.argtypes = [i, i, i, P, P, P, P, P, P, P]
        L.orc_mx_round.restype = None
        L.orc_mx_round.argtypes = [i, i, P]
        L.orc_elem_value.restype = ctypes.c_double
        L.orc_elem_value.argtypes = [i, ctypes.c_uint]
        L.orc_mx_quantize_block.restype = None
        L.orc_mx_quantize_block.argtypes = [i, P, P, P]
        L.orc_mx_split_block.restype = None
        L.orc_mx_split_block.argtypes = [i, P, P, P, P, P]
        L.orc_fp8_weight.restype = ctypes.c_double
        L.orc_fp8_weight.argtypes = [P, P, i, i, i]
        L.orc_expert_row_fp8.restype = None
        L.orc_expert_row_fp8.argtypes = [i, i, P, P, P, P, P, P, P]
        L.orc_layer_forward_fp8.restype = ctypes.c_int
        L.orc_layer_forward_fp8.argtypes = [i, i, i, i, i] + [P] * 12 + [i]
        L.orc_rmsnorm.restype = None
        L.orc_rmsnorm.argtypes = [i, i, P, P, ctypes.c_float, P]
        L.orc_shared_expert_row.restype = None
        L.orc_shared_expert_row.argtypes = [i, i, P, P, P, P, P]
        L.orc_block_forward.restype = ctypes.c_int
        L.orc_block_forward.argtypes = ([i] * 6 + [P, P, ctypes.c_float] + [P] * 14 + [i])
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


# ---- scalar formats ---------------------------------------------------------
def bf16_value(bits: int) -> float:
    return lib().orc_bf16_value(int(bits))


def e2m1_value(code: int) -> float:
    return lib().orc_e2m1_value(int(code))


def e8m0_value(code: int) -> float:
    return lib().orc_e8m0_value(int(code))


def round_to_bf16(v: float) -> int:
    return int(lib().orc_round_to_bf16(float(v)))


def bf16_array_to_f64(a: np.ndarray) -> np.ndarray:
    out = np.empty(a.shape, dtype=np.float64)
    flat = np.ascontiguousarray(a, dtype=np.uint16).ravel()
    L = lib()
    o = out.ravel()
    for i in range(flat.size):
        o[i] = L.orc_bf16_value(int(flat[i]))
    return out


def mxfp4_weight(codes: np.ndarray, scales: np.ndarray, K: int, row: int,
                 col: int) -> float:
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    return lib().orc_mxfp4_weight(_p(codes), _p(scales), K, row, col)


def dequant_matrix(codes: np.ndarray, scales: np.ndarray, rows: int,
                   K: int) -> np.ndarray:
    """[rows][K] fp64 matrix, element by element through the oracle."""
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    L = lib()
    out = np.empty((rows, K), dtype=np.float64)
    pc, ps = _p(codes), _p(scales)
    for r in range(rows):
        for c in range(K):
            out[r, c] = L.orc_mxfp4_weight(pc, ps, K, r, c)
    return out


# ---- router -----------------------------------------------------------------
def router_logits(x, router_w, bias=None):
    x = _c(x, np.uint16)
    router_w = _c(router_w, np.uint16)
    T, d = x.shape
    E = router_w.shape[0]
    assert router_w.shape[1] == d and d % 64 == 0
    b = None if bias is None else _c(bias, np.float32)
    out = np.empty((T, E), dtype=np.float32)
    lib().orc_router_logits(T, d, E, _p(x), _p(router_w), _p(b), _p(out))
    return out


def topk_softmax(logits, k):
    logits = _c(logits, np.float32)
    T, E = logits.shape
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    lib().orc_topk_softmax(T, E, k, _p(logits), _p(ids), _p(w))
    return ids, w


def permute(topk_ids, E):
    topk_ids = _c(topk_ids, np.int32)
    T, k = topk_ids.shape
    counts = np.empty(E, dtype=np.int32)
    offsets = np.empty(E + 1, dtype=np.int32)
    sorted_rows = np.empty(T * k, dtype=np.int32)
    row_pos = np.empty(T * k, dtype=np.int32)
    lib().orc_permute(T, E, k, _p(topk_ids), _p(counts), _p(offsets),
                      _p(sorted_rows), _p(row_pos))
    return counts, offsets, sorted_rows, row_pos


# ---- expert FFN / combine -----------------------------------------------------
def expert_row(x_row, gu_codes, gu_scales, dn_codes, dn_scales, d, f, act=0):
    """One expert on one token row.  Weight arrays are that expert's own
    [2f][d/2], [2f][d/32], [d][f/2], [d][f/32] slices.  Returns (h, o).
    act = 1: the activation-MX mode (x and h rounded to one MX E2M3 term per
    32 elements before their products; h is returned rounded)."""
    x_row = _c(x_row, np.uint16)
    args = [_c(a, np.uint8) for a in (gu_codes, gu_scales, dn_codes, dn_scales)]
    h = np.empty(f, dtype=np.float64)
    o = np.empty(d, dtype=np.float64)
    if act:
        lib().orc_expert_row_act(d, f, int(act), _p(x_row), *[_p(a) for a in args], _p(h),
                                 _p(o))
    else:
        lib().orc_expert_row(d, f, _p(x_row), *[_p(a) for a in args], _p(h), _p(o))
    return h, o


def mx_round(fmt, v):
    """Each 32-element block of the fp64 vector v rounded to one MX term."""
    v = np.array(v, dtype=np.float64, copy=True)
    assert v.ndim == 1 and v.size % 32 == 0
    lib().orc_mx_round(int(fmt), int(v.size), _p(v))
    return v


def combine_token(w, o):
    w = _c(w, np.float64)
    o = _c(o, np.float64)
    k, d = o.shape
    y64 = np.empty(d, dtype=np.float64)
    yb = np.empty(d, dtype=np.uint16)
    lib().orc_combine_token(d, k, _p(w), _p(o), _p(y64), _p(yb))
    return y64, yb


def layer_forward(x, router_w, bias, gu_codes, gu_scales, dn_codes, dn_scales,
                  k, n_threads=0, act=0):
    """Whole layer on full weight arrays [E][...].  Returns a dict.  act = 1:
    expert rows in the activation-MX mode (the router sees x as given)."""
    x = _c(x, np.uint16)
    router_w = _c(router_w, np.uint16)
    T, d = x.shape
    E = router_w.shape[0]
    f = gu_codes.shape[1] // 2
    b = None if bias is None else _c(bias, np.float32)
    ws = [_c(a, np.uint8) for a in (gu_codes, gu_scales, dn_codes, dn_scales)]
    logits = np.empty((T, E), dtype=np.float32)
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    y64 = np.empty((T, d), dtype=np.float64)
    yb = np.empty((T, d), dtype=np.uint16)
    if act:
        rc = lib().orc_layer_forward_act(T, d, E, k, f, int(act), _p(x), _p(router_w), _p(b),
                                         *[_p(a) for a in ws], _p(logits), _p(ids),
                                         _p(w), _p(y64), _p(yb), int(n_threads))
    else:
        rc = lib().orc_layer_forward(T, d, E, k, f, _p(x), _p(router_w), _p(b),
                                     *[_p(a) for a in ws], _p(logits), _p(ids),
                                     _p(w), _p(y64), _p(yb), int(n_threads))
    if rc != 0:
        raise MemoryError("oracle layer_forward: allocation failed")
    return {"logits": logits, "topk_ids": ids, "topk_w": w, "y64": y64,
            "y": yb}


# ---- FP8 experts (E4M3FN, fp32 scale per 128 x 128 block) ---------------------
def fp8_weight(codes, scales, K, row, col):
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.float32)
    return lib().orc_fp8_weight(_p(codes), _p(scales), int(K), int(row), int(col))


def expert_row_fp8(x_row, gu_codes, gu_scales, dn_codes, dn_scales, d, f):
    """One FP8 expert on one token row: returns (h, o) in fp64."""
    args = [_c(x_row, np.uint16), _c(gu_codes, np.uint8), _c(gu_scales, np.float32),
            _c(dn_codes, np.uint8), _c(dn_scales, np.float32)]
    h = np.empty(f, dtype=np.float64)
    o = np.empty(d, dtype=np.float64)
    lib().orc_expert_row_fp8(int(d), int(f), *[_p(a) for a in args], _p(h), _p(o))
    return h, o


def layer_forward_fp8(x, router_w, bias, gu_codes, gu_scales, dn_codes, dn_scales, k,
                      n_threads=0):
    """The layer with FP8 experts (full arrays [E][...])."""
    x = _c(x, np.uint16)
    router_w = _c(router_w, np.uint16)
    T, d = x.shape
    E = router_w.shape[0]
    f = gu_codes.shape[1] // 2
    b = None if bias is None else _c(bias, np.float32)
    ws = [_c(gu_codes, np.uint8), _c(gu_scales, np.float32), _c(dn_codes, np.uint8),
          _c(dn_scales, np.float32)]
    logits = np.empty((T, E), dtype=np.float32)
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    y64 = np.empty((T, d), dtype=np.float64)
    yb = np.empty((T, d), dtype=np.uint16)
    rc = lib().orc_layer_forward_fp8(T, d, E, k, f, _p(x), _p(router_w), _p(b),
                                     *[_p(a) for a in ws], _p(logits), _p(ids), _p(w), _p(y64),
                                     _p(yb), int(n_threads))
    if rc != 0:
        raise MemoryError("oracle layer_forward_fp8: allocation failed")
    return {"logits": logits, "topk_ids": ids, "topk_w": w, "y64": y64, "y": yb}


# ---- MoE tail ---------------------------------------------------------------------
def rmsnorm(x, gamma, eps):
    """xn (bf16 bits [T][d]) = RMSNorm(x) * gamma, canonical fp64 (see the C source)."""
    x = _c(x, np.uint16)
    gamma = _c(gamma, np.uint16)
    T, d = x.shape
    xn = np.empty((T, d), dtype=np.uint16)
    lib().orc_rmsnorm(T, d, _p(x), _p(gamma), float(eps), _p(xn))
    return xn


def shared_expert_row(xn_row, sgu, sdn):
    """The shared expert on one normalised row: returns (h, o) in fp64."""
    xn_row = _c(xn_row, np.uint16)
    sgu = _c(sgu, np.uint16)
    sdn = _c(sdn, np.uint16)
    d = xn_row.size
    fs = sgu.shape[0] // 2
    h = np.empty(fs, dtype=np.float64)
    o = np.empty(d, dtype=np.float64)
    lib().orc_shared_expert_row(d, fs, _p(xn_row), _p(sgu), _p(sdn), _p(h), _p(o))
    return h, o


def block_forward(x, gamma, eps, router_w, bias, gu_codes, gu_scales, dn_codes, dn_scales,
                  sgu, sdn, k, n_threads=0):
    """out = x + routed(xn) + shared(xn), xn = RMSNorm(x) * gamma (sgu None: no
    shared expert).  Returns a dict with xn, logits, topk_ids, topk_w, out64, out."""
    x = _c(x, np.uint16)
    gamma = _c(gamma, np.uint16)
    router_w = _c(router_w, np.uint16)
    T, d = x.shape
    E = router_w.shape[0]
    f = gu_codes.shape[1] // 2
    b = None if bias is None else _c(bias, np.float32)
    ws = [_c(a, np.uint8) for a in (gu_codes, gu_scales, dn_codes, dn_scales)]
    if sgu is None:
        fs, sgu_a, sdn_a = 0, None, None
    else:
        sgu_a, sdn_a = _c(sgu, np.uint16), _c(sdn, np.uint16)
        fs = sgu_a.shape[0] // 2
    xn = np.empty((T, d), dtype=np.uint16)
    logits = np.empty((T, E), dtype=np.float32)
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    out64 = np.empty((T, d), dtype=np.float64)
    out = np.empty((T, d), dtype=np.uint16)
    rc = lib().orc_block_forward(T, d, E, k, f, fs, _p(x), _p(gamma), float(eps),
                                 _p(router_w), _p(b), *[_p(a) for a in ws], _p(sgu_a),
                                 _p(sdn_a), _p(xn), _p(logits), _p(ids), _p(w), _p(out64),
                                 _p(out), int(n_threads))
    if rc != 0:
        raise MemoryError("oracle block_forward: allocation failed")
    return {"xn": xn, "logits": logits, "topk_ids": ids, "topk_w": w, "out64": out64,
            "out": out}


# ---- MX conversion model --------------------------------------------------------
def elem_value(fmt, code):
    return lib().orc_elem_value(int(fmt), int(code))


def mx_quantize_block(fmt, v):
    v = _c(v, np.float64)
    assert v.size == 32
    sc = np.zeros(1, dtype=np.uint8)
    codes = np.zeros(32, dtype=np.uint8)
    lib().orc_mx_quantize_block(int(fmt), _p(v), _p(sc), _p(codes))
    return int(sc[0]), codes


def mx_split_rows(fmt, v):
    """Split every 32-element block of each row of an fp32 [R][K] array.
    Returns hi_scales [R][K/32], hi_codes [R][K], lo_scales, lo_codes."""
    v = _c(v, np.float32)
    R, K = v.shape
    assert K % 32 == 0
    hs = np.zeros((R, K // 32), dtype=np.uint8)
    hc = np.zeros((R, K), dtype=np.uint8)
    ls = np.zeros((R, K // 32), dtype=np.uint8)
    lc = np.zeros((R, K), dtype=np.uint8)
    L = lib()
    for r in range(R):
        for b in range(K // 32):
            blk = np.ascontiguousarray(v[r, 32 * b:32 * b + 32])
            t_hs = np.zeros(1, np.uint8)
            t_ls = np.zeros(1, np.uint8)
            t_hc = np.zeros(32, np.uint8)
            t_lc = np.zeros(32, np.uint8)
            L.orc_mx_split_block(int(fmt), _p(blk), _p(t_hs), _p(t_hc),
                                 _p(t_ls), _p(t_lc))
            hs[r, b] = t_hs[0]
            ls[r, b] = t_ls[0]
            hc[r, 32 * b:32 * b + 32] = t_hc
            lc[r, 32 * b:32 * b + 32] = t_lc
    return hs, hc, ls, lc
