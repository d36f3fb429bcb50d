"""CPU-side checks of the C ABI library: it loads, exports every symbol that
include/moe.h declares, sizes workspaces, and refuses bad arguments on the
host before any launch (no GPU is touched: every call here fails validation
or has T = 0)."""
import ctypes
import glob
import os
import re

import pytest

from routed_expert_mxfp4_amd import build as hipbuild
from routed_expert_mxfp4_amd import moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(hipbuild.LIB_PATH):
        hipbuild.build()
    return moe.lib()


def _declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        src = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src))
    return sorted(names)


def test_exports_every_declared_symbol(L):
    declared = _declared_functions()
    assert set(declared) == set(moe.EXPORTS), declared
    for name in declared:
        assert hasattr(L, name), name
    assert L.moe_abi_version() == 3


def test_build_entry_checks_the_headers_abi_version(L):
    # __graft_entry__.build() compares the built library with include/moe.h
    import __graft_entry__
    assert __graft_entry__.header_abi_version() == L.moe_abi_version()


def test_status_strings(L):
    for s in range(8):
        txt = moe.status_str(s)
        assert txt and "unknown" not in txt
    assert "unknown" in moe.status_str(99)


def _dims(T=8, d=256, E=16, k=2, f=128, act=0):
    return moe.dims_of(T, d, E, k, f, act)


def test_workspace_sizes(L):
    for entry in range(5):
        n = moe.moe_workspace_bytes(_dims(), entry)
        assert 0 <= n < 1 << 40
    # the big prefill shape fits comfortably in one GPU's HBM
    big = moe.moe_workspace_bytes(_dims(32768, 7168, 896, 16, 1536), moe.ENTRY_LAYER_FORWARD)
    assert big < 16 * 2 ** 30
    assert L.moe_workspace_bytes(ctypes.byref(_dims()), 17) == moe.SIZE_MAX
    with pytest.raises(moe.MoeError):
        moe.moe_workspace_bytes(_dims(d=100), 0)
    # the activation-MX mode's GEMV path adds a rounded copy of x
    plain = moe.moe_workspace_bytes(_dims(), moe.ENTRY_EXPERT_FFN)
    amx = moe.moe_workspace_bytes(_dims(act=moe.ACT_MX_E2M3), moe.ENTRY_EXPERT_FFN)
    assert amx >= plain + 8 * 256 * 2


@pytest.mark.parametrize("bad", [dict(d=100), dict(d=0), dict(f=48), dict(E=0), dict(E=2000),
                                 dict(k=0), dict(k=17, E=16), dict(k=33, E=64), dict(T=-1),
                                 dict(T=1 << 27, k=16), dict(d=65536), dict(act=2),
                                 dict(act=-1)])
def test_bad_shapes_refused(L, bad):
    dims = _dims(**bad)
    P = ctypes.c_void_p(0x1000)
    ex = moe.Experts(0x1000, 0x1000, 0x1000, 0x1000)
    st = L.moe_layer_forward(ctypes.byref(dims), P, P, None, ctypes.byref(ex), P, None, None,
                             P, 1 << 40, None)
    assert st == moe.MOE_ERR_SHAPE
    st = L.moe_route(ctypes.byref(dims), P, P, None, P, P, P, None, 0, None)
    assert st == moe.MOE_ERR_SHAPE


def test_null_and_alignment_refused(L):
    dims = _dims()
    A = ctypes.c_void_p(0x10000)
    M = ctypes.c_void_p(0x10008)          # 8-byte aligned only
    ex = moe.Experts(0x10000, 0x10000, 0x10000, 0x10000)
    exm = moe.Experts(0x10000, 0x10008, 0x10000, 0x10000)
    exn = moe.Experts(0x10000, None, 0x10000, 0x10000)
    big = 1 << 40
    f = L.moe_layer_forward
    assert f(None, A, A, None, ctypes.byref(ex), A, None, None, A, big, None) == moe.MOE_ERR_NULL
    assert f(ctypes.byref(dims), None, A, None, ctypes.byref(ex), A, None, None, A, big, None) == moe.MOE_ERR_NULL
    assert f(ctypes.byref(dims), A, A, None, None, A, None, None, A, big, None) == moe.MOE_ERR_NULL
    assert f(ctypes.byref(dims), A, A, None, ctypes.byref(exn), A, None, None, A, big, None) == moe.MOE_ERR_NULL
    assert f(ctypes.byref(dims), M, A, None, ctypes.byref(ex), A, None, None, A, big, None) == moe.MOE_ERR_ALIGN
    assert f(ctypes.byref(dims), A, A, None, ctypes.byref(exm), A, None, None, A, big, None) == moe.MOE_ERR_ALIGN
    assert f(ctypes.byref(dims), A, A, None, ctypes.byref(ex), A, None, None, None, big, None) == moe.MOE_ERR_NULL
    assert f(ctypes.byref(dims), A, A, None, ctypes.byref(ex), A, None, None, M, big, None) == moe.MOE_ERR_ALIGN
    need = moe.moe_workspace_bytes(dims, moe.ENTRY_LAYER_FORWARD)
    assert f(ctypes.byref(dims), A, A, None, ctypes.byref(ex), A, None, None, A, need - 1, None) == moe.MOE_ERR_WORKSPACE
    # route: logits buffer or workspace required
    r = L.moe_route
    assert r(ctypes.byref(dims), A, A, None, None, A, A, None, 0, None) == moe.MOE_ERR_NULL
    assert r(ctypes.byref(dims), A, A, None, None, A, A, A, 1, None) == moe.MOE_ERR_WORKSPACE
    assert r(ctypes.byref(dims), A, A, None, A, None, A, None, 0, None) == moe.MOE_ERR_NULL
    # permute / ffn / combine
    p = L.moe_permute
    assert p(ctypes.byref(dims), None, A, A, A, A, None, 0, None) == moe.MOE_ERR_NULL
    big_dims = _dims(T=4096, d=7168, E=896, k=16, f=1536)
    assert p(ctypes.byref(big_dims), A, A, A, A, A, None, 0, None) == moe.MOE_ERR_NULL
    assert p(ctypes.byref(big_dims), A, A, A, A, A, A, 16, None) == moe.MOE_ERR_WORKSPACE
    e = L.moe_expert_ffn
    assert e(ctypes.byref(dims), A, ctypes.byref(ex), A, A, A, None, 0, None) == moe.MOE_ERR_NULL
    assert e(ctypes.byref(dims), A, ctypes.byref(ex), A, A, M, A, big, None) == moe.MOE_ERR_ALIGN
    assert e(ctypes.byref(dims), A, ctypes.byref(ex), A, A, A, A, 16, None) == moe.MOE_ERR_WORKSPACE
    c = L.moe_combine
    assert c(ctypes.byref(dims), A, A, A, None, None) == moe.MOE_ERR_NULL
    assert c(ctypes.byref(dims), M, A, A, A, None) == moe.MOE_ERR_ALIGN


def test_zero_tokens_is_a_no_op(L):
    dims = _dims(T=0)
    ex = moe.Experts(0x10000, 0x10000, 0x10000, 0x10000)
    # nothing is validated beyond the dims and nothing is launched
    assert L.moe_layer_forward(ctypes.byref(dims), None, None, None, ctypes.byref(ex), None,
                               None, None, None, 0, None) == moe.MOE_OK
    assert L.moe_permute(ctypes.byref(dims), None, None, None, None, None, None, 0, None) == moe.MOE_OK
    assert L.moe_combine(ctypes.byref(dims), None, None, None, None, None) == moe.MOE_OK


def test_noalloc_refuses_before_any_launch(L):
    A = ctypes.c_void_p(0x10000)
    M = ctypes.c_void_p(0x10008)
    ex = moe.Experts(0x10000, 0x10000, 0x10000, 0x10000)
    f = L.moe_layer_forward_noalloc
    # the K3 shape: the largest token count whose layer scratch fits, and the next
    need = [moe.moe_workspace_bytes(_dims(T=t, d=7168, E=896, k=16, f=1536),
                                    moe.ENTRY_LAYER_FORWARD) for t in range(1, 400)]
    limit = max(t for t, n in zip(range(1, 400), need) if n <= moe.NOALLOC_SCRATCH_BYTES)
    assert limit >= 128 and all(n <= moe.NOALLOC_SCRATCH_BYTES for n in need[:limit])
    over = _dims(T=limit + 1, d=7168, E=896, k=16, f=1536)
    assert f(ctypes.byref(over), A, A, None, ctypes.byref(ex), A, None, None, None) == moe.MOE_ERR_SCRATCH
    big = _dims(T=32768, d=7168, E=896, k=16, f=1536)
    assert f(ctypes.byref(big), A, A, None, ctypes.byref(ex), A, None, None, None) == moe.MOE_ERR_SCRATCH
    dims = _dims()
    assert f(None, A, A, None, ctypes.byref(ex), A, None, None, None) == moe.MOE_ERR_NULL
    assert f(ctypes.byref(dims), None, A, None, ctypes.byref(ex), A, None, None, None) == moe.MOE_ERR_NULL
    assert f(ctypes.byref(dims), A, A, None, None, A, None, None, None) == moe.MOE_ERR_NULL
    assert f(ctypes.byref(dims), A, A, None, ctypes.byref(ex), M, None, None, None) == moe.MOE_ERR_ALIGN
    assert f(ctypes.byref(_dims(d=100)), A, A, None, ctypes.byref(ex), A, None, None, None) == moe.MOE_ERR_SHAPE
    assert f(ctypes.byref(_dims(T=0)), None, None, None, ctypes.byref(ex), None, None, None,
             None) == moe.MOE_OK
    assert "MOE_NOALLOC_SCRATCH_BYTES" in moe.status_str(moe.MOE_ERR_SCRATCH)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(moe, "_lib", None)
    monkeypatch.setattr(moe, "LIB_PATH", str(tmp_path / "nope.so"))
    with pytest.raises(RuntimeError, match="not built"):
        moe.lib()


def test_tail_entries_refuse_bad_arguments(L):
    dims = _dims()
    A = ctypes.c_void_p(0x10000)
    M = ctypes.c_void_p(0x10008)
    B = ctypes.c_void_p(0x20000)          # an output that does not alias x
    ex = moe.Experts(0x10000, 0x10000, 0x10000, 0x10000)
    tw = moe.TailWeights(0x10000, 1e-6, 64, 0x10000, 0x10000)
    big = 1 << 40
    ws = L.moe_block_workspace_bytes
    assert ws(ctypes.byref(dims), ctypes.byref(tw)) not in (0, moe.SIZE_MAX)
    assert ws(ctypes.byref(dims), None) == moe.SIZE_MAX
    for bad in (moe.TailWeights(0x10000, 1e-6, 48, 0x10000, 0x10000),      # fs % 32
                moe.TailWeights(0x10000, -1.0, 64, 0x10000, 0x10000),      # eps < 0
                moe.TailWeights(0x10000, float("nan"), 64, 0x10000, 0x10000),
                moe.TailWeights(0x10000, 1e-6, 16384 + 32, 0x10000, 0x10000)):
        assert ws(ctypes.byref(dims), ctypes.byref(bad)) == moe.SIZE_MAX
    # no shared expert is valid and needs no shared pointers
    none = moe.TailWeights(0x10000, 1e-6, 0, None, None)
    assert ws(ctypes.byref(dims), ctypes.byref(none)) != moe.SIZE_MAX
    f = L.moe_block_forward
    need = ws(ctypes.byref(dims), ctypes.byref(tw))
    call = lambda x, t, rw, e, out, w, n: f(ctypes.byref(dims), x, t, rw, None, e, out, None, None,
                                            w, n, None)
    assert call(None, ctypes.byref(tw), A, ctypes.byref(ex), B, A, big) == moe.MOE_ERR_NULL
    assert call(A, None, A, ctypes.byref(ex), B, A, big) == moe.MOE_ERR_NULL
    assert call(A, ctypes.byref(tw), A, ctypes.byref(ex), None, A, big) == moe.MOE_ERR_NULL
    nog = moe.TailWeights(None, 1e-6, 64, 0x10000, 0x10000)
    assert call(A, ctypes.byref(nog), A, ctypes.byref(ex), B, A, big) == moe.MOE_ERR_NULL
    nos = moe.TailWeights(0x10000, 1e-6, 64, None, 0x10000)
    assert call(A, ctypes.byref(nos), A, ctypes.byref(ex), B, A, big) == moe.MOE_ERR_NULL
    mis = moe.TailWeights(0x10000, 1e-6, 64, 0x10008, 0x10000)
    assert call(A, ctypes.byref(mis), A, ctypes.byref(ex), B, A, big) == moe.MOE_ERR_ALIGN
    assert call(M, ctypes.byref(tw), A, ctypes.byref(ex), B, A, big) == moe.MOE_ERR_ALIGN
    assert call(A, ctypes.byref(tw), A, ctypes.byref(ex), B, A, need - 1) == moe.MOE_ERR_WORKSPACE
    assert call(A, ctypes.byref(tw), A, ctypes.byref(ex), B, None, big) == moe.MOE_ERR_NULL
    # the output may not overwrite the residual input
    assert call(A, ctypes.byref(tw), A, ctypes.byref(ex), A, A, big) == moe.MOE_ERR_UNSUPPORTED
    r = L.moe_rmsnorm
    assert r(ctypes.byref(dims), None, A, 1e-6, A, None) == moe.MOE_ERR_NULL
    assert r(ctypes.byref(dims), A, M, 1e-6, A, None) == moe.MOE_ERR_ALIGN
    assert r(ctypes.byref(dims), A, A, -1.0, A, None) == moe.MOE_ERR_SHAPE
    zero = _dims(T=0)
    assert r(ctypes.byref(zero), None, None, 1e-6, None, None) == moe.MOE_OK
    assert f(ctypes.byref(zero), None, ctypes.byref(tw), None, None, ctypes.byref(ex), None,
             None, None, None, 0, None) == moe.MOE_OK


def test_fp8_entries_refuse_bad_arguments(L):
    A = ctypes.c_void_p(0x10000)
    M = ctypes.c_void_p(0x10008)
    big = 1 << 40
    dims = _dims(d=256, f=128)
    ex = moe.Fp8Experts(0x10000, 0x10000, 0x10000, 0x10000)
    exm = moe.Fp8Experts(0x10000, 0x10004, 0x10000, 0x10000)
    exn = moe.Fp8Experts(0x10000, 0x10000, None, 0x10000)
    w = L.moe_fp8_workspace_bytes
    assert w(ctypes.byref(dims), moe.ENTRY_LAYER_FORWARD) not in (0, moe.SIZE_MAX)
    assert w(ctypes.byref(dims), moe.ENTRY_EXPERT_FFN) not in (0, moe.SIZE_MAX)
    assert w(ctypes.byref(dims), moe.ENTRY_ROUTE) == moe.SIZE_MAX
    bad = _dims(d=192, f=128)                     # d % 128 != 0
    assert w(ctypes.byref(bad), moe.ENTRY_LAYER_FORWARD) == moe.SIZE_MAX
    f = L.moe_layer_forward_fp8
    assert f(ctypes.byref(bad), A, A, None, ctypes.byref(ex), A, None, None, A, big, None) == moe.MOE_ERR_SHAPE
    amx = _dims(d=256, f=128, act=1)
    assert f(ctypes.byref(amx), A, A, None, ctypes.byref(ex), A, None, None, A, big, None) == moe.MOE_ERR_UNSUPPORTED
    assert f(ctypes.byref(dims), A, A, None, None, A, None, None, A, big, None) == moe.MOE_ERR_NULL
    assert f(ctypes.byref(dims), A, A, None, ctypes.byref(exn), A, None, None, A, big, None) == moe.MOE_ERR_NULL
    assert f(ctypes.byref(dims), A, A, None, ctypes.byref(exm), A, None, None, A, big, None) == moe.MOE_ERR_ALIGN
    assert f(ctypes.byref(dims), M, A, None, ctypes.byref(ex), A, None, None, A, big, None) == moe.MOE_ERR_ALIGN
    need = w(ctypes.byref(dims), moe.ENTRY_LAYER_FORWARD)
    assert f(ctypes.byref(dims), A, A, None, ctypes.byref(ex), A, None, None, A, need - 1, None) == moe.MOE_ERR_WORKSPACE
    e = L.moe_expert_ffn_fp8
    assert e(ctypes.byref(dims), A, ctypes.byref(ex), A, A, None, A, big, None) == moe.MOE_ERR_NULL
    need = w(ctypes.byref(dims), moe.ENTRY_EXPERT_FFN)
    assert e(ctypes.byref(dims), A, ctypes.byref(ex), A, A, A, A, need - 1, None) == moe.MOE_ERR_WORKSPACE
    zero = _dims(T=0, d=256, f=128)
    assert f(ctypes.byref(zero), None, None, None, ctypes.byref(ex), None, None, None, None, 0, None) == moe.MOE_OK


def test_packed_entries_refuse_bad_arguments(L):
    A = ctypes.c_void_p(0x10000)
    big = 1 << 40
    ex = moe.Experts(0x10000, 0x10000, 0x10000, 0x10000)
    exo = moe.Experts(0x100000000, 0x200000000, 0x300000000, 0x400000000)
    dims = _dims(T=256, d=512, E=16, k=2, f=512)
    p = L.moe_prepack_experts
    assert p(ctypes.byref(_dims(d=256, f=128)), ctypes.byref(ex), ctypes.byref(exo), None) == moe.MOE_ERR_UNSUPPORTED
    assert p(ctypes.byref(dims), ctypes.byref(ex), None, None) == moe.MOE_ERR_NULL
    # destination overlapping the source
    assert p(ctypes.byref(dims), ctypes.byref(ex), ctypes.byref(ex), None) == moe.MOE_ERR_UNSUPPORTED
    f = L.moe_layer_forward_packed
    small = _dims(T=64, d=512, E=16, k=2, f=512)          # below the prefill path
    assert f(ctypes.byref(small), A, A, None, ctypes.byref(ex), A, None, None, A, big, None) == moe.MOE_ERR_UNSUPPORTED
    odd = _dims(T=256, d=512, E=16, k=2, f=256)           # f % 512 != 0
    assert f(ctypes.byref(odd), A, A, None, ctypes.byref(ex), A, None, None, A, big, None) == moe.MOE_ERR_UNSUPPORTED
    assert f(ctypes.byref(dims), None, A, None, ctypes.byref(ex), A, None, None, A, big, None) == moe.MOE_ERR_NULL
    need = moe.moe_workspace_bytes(dims, moe.ENTRY_LAYER_FORWARD)
    assert f(ctypes.byref(dims), A, A, None, ctypes.byref(ex), A, None, None, A, need - 1, None) == moe.MOE_ERR_WORKSPACE
    zero = _dims(T=0, d=512, f=512)
    assert f(ctypes.byref(zero), None, None, None, None, None, None, None, None, 0, None) == moe.MOE_OK
