"""Thin Python binding of the C ABI in ``include/moe.h``,
``include/moe_tail.h``, ``include/moe_fp8.h`` and ``include/moe_packed.h``.

Argument marshalling only: every step of the layer runs in the HIP kernels
of ``libmoe_mxfp4.so``.  Torch supplies device memory (outputs and
workspace) and the current stream.  There is no fallback: if the compiled
library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

from .build import LIB_PATH

MOE_OK, MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_ALIGN = 0, 1, 2, 3
MOE_ERR_WORKSPACE, MOE_ERR_UNSUPPORTED, MOE_ERR_DEVICE, MOE_ERR_SCRATCH = 4, 5, 6, 7
NOALLOC_SCRATCH_BYTES = 64 << 20      # MOE_NOALLOC_SCRATCH_BYTES (include/moe.h)
ENTRY_ROUTE, ENTRY_PERMUTE, ENTRY_EXPERT_FFN, ENTRY_COMBINE, ENTRY_LAYER_FORWARD = range(5)
SIZE_MAX = (1 << 64) - 1


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s: %s" % (where, status_str(status)))


class Dims(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("d", ctypes.c_int32), ("E", ctypes.c_int32),
                ("k", ctypes.c_int32), ("f", ctypes.c_int32), ("act", ctypes.c_int32)]


ACT_BF16, ACT_MX_E2M3 = 0, 1          # MOE_ACT_* (include/moe.h)


class Experts(ctypes.Structure):
    _fields_ = [("gu_codes", ctypes.c_void_p), ("gu_scales", ctypes.c_void_p),
                ("dn_codes", ctypes.c_void_p), ("dn_scales", ctypes.c_void_p)]


class Fp8Experts(ctypes.Structure):
    _fields_ = [("gu_codes", ctypes.c_void_p), ("gu_scales", ctypes.c_void_p),
                ("dn_codes", ctypes.c_void_p), ("dn_scales", ctypes.c_void_p)]


class TailWeights(ctypes.Structure):
    _fields_ = [("norm_w", ctypes.c_void_p), ("eps", ctypes.c_float), ("fs", ctypes.c_int32),
                ("shared_gu", ctypes.c_void_p), ("shared_dn", ctypes.c_void_p)]


EXPORTS = ("moe_abi_version", "moe_status_str", "moe_workspace_bytes", "moe_route",
           "moe_permute", "moe_expert_ffn", "moe_combine", "moe_layer_forward",
           "moe_diag_time_kernel", "moe_diag_kernel_time", "moe_diag_mx_split_e2m3",
           "moe_block_workspace_bytes", "moe_rmsnorm", "moe_block_forward",
           "moe_fp8_workspace_bytes", "moe_expert_ffn_fp8", "moe_layer_forward_fp8",
           "moe_prepack_experts", "moe_layer_forward_packed", "moe_diag_kernel_times",
           "moe_layer_forward_noalloc", "moe_diag_set_gemv_max_rows",
           "moe_diag_gemv_max_rows", "moe_diag_stream_read", "moe_diag_mfma_rate",
           "moe_diag_time_kernel_every")

_lib = None


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                "libmoe_mxfp4.so is not built (run `python -m routed_expert_mxfp4_amd.build`); "
                "there is no fallback path")
        L = ctypes.CDLL(LIB_PATH)
        P, S, I = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
        DP = ctypes.POINTER(Dims)
        EP = ctypes.POINTER(Experts)
        L.moe_abi_version.restype = I
        L.moe_abi_version.argtypes = []
        L.moe_status_str.restype = ctypes.c_char_p
        L.moe_status_str.argtypes = [I]
        L.moe_workspace_bytes.restype = S
        L.moe_workspace_bytes.argtypes = [DP, I]
        L.moe_route.restype = I
        L.moe_route.argtypes = [DP, P, P, P, P, P, P, P, S, P]
        L.moe_permute.restype = I
        L.moe_permute.argtypes = [DP, P, P, P, P, P, P, S, P]
        L.moe_expert_ffn.restype = I
        L.moe_expert_ffn.argtypes = [DP, P, EP, P, P, P, P, S, P]
        L.moe_combine.restype = I
        L.moe_combine.argtypes = [DP, P, P, P, P, P]
        L.moe_layer_forward.restype = I
        L.moe_layer_forward.argtypes = [DP, P, P, P, EP, P, P, P, P, S, P]
        L.moe_layer_forward_noalloc.restype = I
        L.moe_layer_forward_noalloc.argtypes = [DP, P, P, P, EP, P, P, P, P]
        FP = ctypes.POINTER(Fp8Experts)
        L.moe_fp8_workspace_bytes.restype = S
        L.moe_fp8_workspace_bytes.argtypes = [DP, I]
        L.moe_expert_ffn_fp8.restype = I
        L.moe_expert_ffn_fp8.argtypes = [DP, P, FP, P, P, P, P, S, P]
        L.moe_layer_forward_fp8.restype = I
        L.moe_layer_forward_fp8.argtypes = [DP, P, P, P, FP, P, P, P, P, S, P]
        L.moe_prepack_experts.restype = I
        L.moe_prepack_experts.argtypes = [DP, EP, EP, P]
        L.moe_layer_forward_packed.restype = I
        L.moe_layer_forward_packed.argtypes = [DP, P, P, P, EP, P, P, P, P, S, P]
        TP = ctypes.POINTER(TailWeights)
        L.moe_block_workspace_bytes.restype = S
        L.moe_block_workspace_bytes.argtypes = [DP, TP]
        L.moe_rmsnorm.restype = I
        L.moe_rmsnorm.argtypes = [DP, P, P, ctypes.c_float, P, P]
        L.moe_block_forward.restype = I
        L.moe_block_forward.argtypes = [DP, P, TP, P, P, EP, P, P, P, P, S, P]
        L.moe_diag_time_kernel.restype = I
        L.moe_diag_time_kernel.argtypes = [ctypes.c_char_p, I]
        L.moe_diag_time_kernel_every.restype = I
        L.moe_diag_time_kernel_every.argtypes = [ctypes.c_char_p, I, I]
        L.moe_diag_mx_split_e2m3.restype = I
        L.moe_diag_mx_split_e2m3.argtypes = [P, I, I, I, P, P]
        L.moe_diag_kernel_times.restype = I
        L.moe_diag_kernel_times.argtypes = [ctypes.POINTER(ctypes.c_double), I,
                                            ctypes.POINTER(ctypes.c_longlong)]
        L.moe_diag_set_gemv_max_rows.restype = I
        L.moe_diag_set_gemv_max_rows.argtypes = [I]
        L.moe_diag_gemv_max_rows.restype = I
        L.moe_diag_gemv_max_rows.argtypes = []
        L.moe_diag_stream_read.restype = I
        L.moe_diag_stream_read.argtypes = [P, S, P, I, P]
        L.moe_diag_mfma_rate.restype = I
        L.moe_diag_mfma_rate.argtypes = [I, I, I, P, P]
        L.moe_diag_kernel_time.restype = I
        L.moe_diag_kernel_time.argtypes = [ctypes.POINTER(ctypes.c_double),
                                           ctypes.POINTER(ctypes.c_longlong)]
        _lib = L
    return _lib


def diag_time_kernel(kernel, capacity: int = 4096, every: int = 1):
    """Time every launch (or one launch in ``every``) of one named kernel
    with HIP events (None stops)."""
    name = None if kernel is None else kernel.encode()
    if lib().moe_diag_time_kernel_every(name, int(capacity), int(every)) != 0:
        raise RuntimeError("moe_diag_time_kernel_every failed")


def diag_kernel_time():
    """(total ms, launches) recorded since the last call; synchronise first."""
    ms = ctypes.c_double(0.0)
    n = ctypes.c_longlong(0)
    if lib().moe_diag_kernel_time(ctypes.byref(ms), ctypes.byref(n)) != 0:
        raise RuntimeError("moe_diag_kernel_time failed")
    return ms.value, n.value


def diag_kernel_times(cap: int):
    """Per-launch times (ms, launch order) recorded since the last call;
    synchronise first."""
    buf = (ctypes.c_double * max(cap, 1))()
    n = ctypes.c_longlong(0)
    if lib().moe_diag_kernel_times(buf, int(cap), ctypes.byref(n)) != 0:
        raise RuntimeError("moe_diag_kernel_times failed")
    return [buf[i] for i in range(min(cap, n.value))]


def diag_set_gemv_max_rows(rows):
    """Override the per-expert crossover (experts with at most ``rows`` rows
    take the GEMVs in a scaled-MFMA call); None restores the built-in one."""
    if lib().moe_diag_set_gemv_max_rows(-1 if rows is None else int(rows)) != 0:
        raise ValueError("gemv_max_rows must be 0..16 or None")


def diag_gemv_max_rows() -> int:
    return int(lib().moe_diag_gemv_max_rows())


MFMA_RATE_KINDS = {"fp6xfp4": 0, "fp8xfp4": 1, "fp4xfp4": 2, "fp8xfp8": 3, "bf16": 4,
                   "fp6xfp4_32x32x64": 5, "fp4xfp4_32x32x64": 6}
MFMA_RATE_FLOPS = {0: 2 * 16 * 16 * 128, 1: 2 * 16 * 16 * 128, 2: 2 * 16 * 16 * 128,
                   3: 2 * 16 * 16 * 128, 4: 2 * 32 * 32 * 16, 5: 2 * 32 * 32 * 64,
                   6: 2 * 32 * 32 * 64}


def diag_stream_read(src, nbytes: int, out, blocks: int, stream=None):
    """One streaming-read launch over the first ``nbytes`` bytes of the device
    tensor ``src``; ``out`` (int32, >= blocks elements) takes a checksum per
    block."""
    import torch
    if nbytes > src.numel() * src.element_size() or out.numel() < blocks:
        raise ValueError("buffer too small")
    with torch.cuda.stream(_on(stream)) as _:
        s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        if lib().moe_diag_stream_read(ctypes.c_void_p(src.data_ptr()), int(nbytes),
                                      ctypes.c_void_p(out.data_ptr()), int(blocks), s) != 0:
            raise RuntimeError("moe_diag_stream_read failed")


def diag_mfma_rate(kind: str, blocks: int, iters: int, out, stream=None):
    """One launch issuing blocks * 4 waves * iters * 4 matrix instructions of
    the given kind; ``out`` (float32, >= 4 blocks elements) takes one sum per
    wave.  Returns the launch's flops."""
    import torch
    k = MFMA_RATE_KINDS[kind]
    if out.numel() < 4 * blocks:
        raise ValueError("out too small")
    with torch.cuda.stream(_on(stream)) as _:
        s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        if lib().moe_diag_mfma_rate(k, int(blocks), int(iters), ctypes.c_void_p(out.data_ptr()),
                                    s) != 0:
            raise RuntimeError("moe_diag_mfma_rate failed")
    return float(blocks) * 4 * iters * 4 * MFMA_RATE_FLOPS[k]


def diag_mx_split_e2m3(rows_tensor, stream=None):
    """Two-term MX E2M3 split of a [rows][K] bf16 or fp32 device tensor (the
    scaled-MFMA path's activation staging).  Returns uint8 [rows][K/128*208]
    in the library's split layout (codes of both terms, then their scales,
    per 128-element step)."""
    t = rows_tensor.contiguous()
    R, K = t.shape
    out = torch.empty((R, K // 128 * 208), dtype=torch.uint8, device=t.device)
    is_bf16 = 1 if t.dtype == torch.bfloat16 else 0
    if not is_bf16:
        assert t.dtype == torch.float32
    rc = lib().moe_diag_mx_split_e2m3(_ptr(t), is_bf16, R, K, _ptr(out), _stream(stream))
    if rc != 0:
        raise RuntimeError("moe_diag_mx_split_e2m3 failed")
    return out


def status_str(status: int) -> str:
    return lib().moe_status_str(int(status)).decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _on(stream):
    """The stream a call runs on (the current one if None).  Wrappers make
    their temporaries (workspace, outputs, dtype or layout copies) inside
    ``torch.cuda.stream(_on(stream))``, so the caching allocator ties those
    blocks to the stream whose kernels use them: a block freed when the
    wrapper returns is not handed to another stream's work while the
    queued kernels still read or write it."""
    return torch.cuda.current_stream() if stream is None else stream


def _keep(t, stream):
    """A long-lived buffer (a Layer's workspace) used on ``stream``: mark it
    in use there, so that freeing it later waits for that stream's work."""
    if t is not None and stream is not None and stream != torch.cuda.current_stream(t.device):
        t.record_stream(stream)


def _check(status: int, where: str):
    if status != MOE_OK:
        raise MoeError(status, where)


def dims_of(T, d, E, k, f, act=ACT_BF16) -> Dims:
    return Dims(int(T), int(d), int(E), int(k), int(f), int(act))


def experts_of(w: dict) -> Experts:
    return Experts(w["gu_codes"].data_ptr(), w["gu_scales"].data_ptr(),
                   w["dn_codes"].data_ptr(), w["dn_scales"].data_ptr())


def moe_workspace_bytes(dims: Dims, entry: int) -> int:
    n = lib().moe_workspace_bytes(ctypes.byref(dims), int(entry))
    if n == SIZE_MAX:
        raise MoeError(MOE_ERR_SHAPE, "moe_workspace_bytes")
    return n


def workspace(dims: Dims, entry: int, device) -> torch.Tensor:
    n = moe_workspace_bytes(dims, entry)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def _bits16(t: torch.Tensor) -> torch.Tensor:
    assert t.dtype in (torch.bfloat16, torch.int16, torch.uint16), t.dtype
    return t.contiguous()


def moe_route(x, router_w, k, router_bias=None, want_logits=False, ws=None, stream=None):
    """Router + top-k + softmax.  Returns (topk_ids int32 [T][k],
    topk_w fp32 [T][k]) and, if ``want_logits``, the fp32 [T][E] logits."""
    s = _on(stream)
    with torch.cuda.stream(s):
        x, router_w = _bits16(x), _bits16(router_w)
        T, d = x.shape
        E = router_w.shape[0]
        dims = dims_of(T, d, E, k, 32)
        dev = x.device
        ids = torch.empty((T, k), dtype=torch.int32, device=dev)
        w = torch.empty((T, k), dtype=torch.float32, device=dev)
        logits = torch.empty((T, E), dtype=torch.float32, device=dev) if want_logits else None
        if ws is None and not want_logits:
            ws = workspace(dims, ENTRY_ROUTE, dev)
        bias = None if router_bias is None else router_bias.contiguous().float()
        st = lib().moe_route(ctypes.byref(dims), _ptr(x), _ptr(router_w), _ptr(bias),
                             _ptr(logits), _ptr(ids), _ptr(w), _ptr(ws),
                             0 if ws is None else ws.numel(), _stream(s))
    _check(st, "moe_route")
    return (ids, w, logits) if want_logits else (ids, w)


def moe_permute(topk_ids, E, ws=None, stream=None):
    """Group rows by expert.  Returns (counts [E], offsets [E+1],
    sorted_rows [T*k], row_pos [T*k]), all int32."""
    s = _on(stream)
    with torch.cuda.stream(s):
        topk_ids = topk_ids.contiguous()
        T, k = topk_ids.shape
        dims = dims_of(T, 64, E, k, 32)
        dev = topk_ids.device
        counts = torch.empty(E, dtype=torch.int32, device=dev)
        offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
        sorted_rows = torch.empty(T * k, dtype=torch.int32, device=dev)
        row_pos = torch.empty(T * k, dtype=torch.int32, device=dev)
        if ws is None:
            ws = workspace(dims, ENTRY_PERMUTE, dev)
        st = lib().moe_permute(ctypes.byref(dims), _ptr(topk_ids), _ptr(counts), _ptr(offsets),
                               _ptr(sorted_rows), _ptr(row_pos), _ptr(ws), ws.numel(),
                               _stream(s))
    _check(st, "moe_permute")
    return counts, offsets, sorted_rows, row_pos


def moe_expert_ffn(x, experts: dict, offsets, sorted_rows, k, ws=None, stream=None,
                   act=ACT_BF16):
    """Expert FFN over grouped rows.  Returns rows_out bf16 [T*k][d].
    act: ACT_BF16, or ACT_MX_E2M3 for the activation-MX mode."""
    s = _on(stream)
    with torch.cuda.stream(s):
        x = _bits16(x)
        T, d = x.shape
        E, two_f = experts["gu_codes"].shape[:2]
        dims = dims_of(T, d, E, k, two_f // 2, act)
        rows_out = torch.empty((T * k, d), dtype=torch.bfloat16, device=x.device)
        if ws is None:
            ws = workspace(dims, ENTRY_EXPERT_FFN, x.device)
        offsets, sorted_rows = offsets.contiguous(), sorted_rows.contiguous()
        ex = experts_of(experts)
        st = lib().moe_expert_ffn(ctypes.byref(dims), _ptr(x), ctypes.byref(ex), _ptr(offsets),
                                  _ptr(sorted_rows), _ptr(rows_out), _ptr(ws), ws.numel(),
                                  _stream(s))
    _check(st, "moe_expert_ffn")
    return rows_out


def moe_combine(rows_out, row_pos, topk_w, stream=None):
    """Weighted combine.  Returns y bf16 [T][d]."""
    s = _on(stream)
    with torch.cuda.stream(s):
        rows_out = _bits16(rows_out)
        T, k = topk_w.shape
        d = rows_out.shape[1]
        dims = dims_of(T, d, max(k, 1), k, 32)
        y = torch.empty((T, d), dtype=torch.bfloat16, device=rows_out.device)
        row_pos, topk_w = row_pos.contiguous(), topk_w.contiguous()
        st = lib().moe_combine(ctypes.byref(dims), _ptr(rows_out), _ptr(row_pos),
                               _ptr(topk_w), _ptr(y), _stream(s))
    _check(st, "moe_combine")
    return y


class _Reusable:
    """A workspace kept across calls, grown when a call needs more bytes
    (the byte count is not monotonic in T: the expert path changes with
    it)."""

    _ws = None

    def _ensure_ws(self, nbytes: int, device):
        if nbytes == SIZE_MAX:
            raise MoeError(MOE_ERR_SHAPE, type(self).__name__ + " workspace")
        if self._ws is None or self._ws.numel() < nbytes:
            self._ws = None
            self._ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        return self._ws


class Layer(_Reusable):
    """Holds device pointers, dims and a reusable workspace for repeated
    ``moe_layer_forward`` calls (the benchmark's hot loop)."""

    _entry = "moe_layer_forward"

    def __init__(self, experts: dict, router_w, k, router_bias=None, T=1, act=ACT_BF16):
        self.act = int(act)
        self.experts = experts
        self.router_w = _bits16(router_w)
        self.bias = None if router_bias is None else router_bias.contiguous().float()
        self.E, self.d = self.router_w.shape
        self.f = experts["gu_codes"].shape[1] // 2
        self.k = k
        self._ex = experts_of(experts)
        self.reserve(T)

    def _dims(self, T):
        return dims_of(T, self.d, self.E, self.k, self.f, self.act)

    def _ws_bytes(self, dims):
        return lib().moe_workspace_bytes(ctypes.byref(dims), ENTRY_LAYER_FORWARD)

    def reserve(self, T):
        """Make the workspace large enough for a call with T tokens."""
        return self._ensure_ws(self._ws_bytes(self._dims(T)), self.router_w.device)

    def forward(self, x, y=None, topk_ids=None, topk_w=None, stream=None):
        s = _on(stream)
        with torch.cuda.stream(s):
            x = _bits16(x)
            T = x.shape[0]
            dims = self._dims(T)
            ws = self.reserve(T)
            _keep(ws, s)
            if y is None:
                y = torch.empty((T, self.d), dtype=torch.bfloat16, device=x.device)
            st = getattr(lib(), self._entry)(
                ctypes.byref(dims), _ptr(x), _ptr(self.router_w), _ptr(self.bias),
                ctypes.byref(self._ex), _ptr(y), _ptr(topk_ids), _ptr(topk_w), _ptr(ws),
                ws.numel(), _stream(s))
        _check(st, self._entry)
        return y


def _routing_outputs(T, k, device, want):
    if not want:
        return None, None
    return (torch.empty((T, k), dtype=torch.int32, device=device),
            torch.empty((T, k), dtype=torch.float32, device=device))


def moe_layer_forward(x, router_w, experts: dict, k, router_bias=None, return_routing=False,
                      stream=None, act=ACT_BF16):
    """The whole layer.  Returns y bf16 [T][d] (and topk_ids, topk_w).
    act: ACT_BF16, or ACT_MX_E2M3 for the activation-MX mode."""
    s = _on(stream)
    with torch.cuda.stream(s):
        x = _bits16(x)
        T = x.shape[0]
        layer = Layer(experts, router_w, k, router_bias, T=T, act=act)
        ids, w = _routing_outputs(T, k, x.device, return_routing)
        y = layer.forward(x, topk_ids=ids, topk_w=w, stream=s)
    return (y, ids, w) if return_routing else y


def moe_layer_forward_noalloc(x, router_w, experts: dict, k, router_bias=None, y=None,
                              topk_ids=None, topk_w=None, stream=None):
    """The layer on the library's static scratch (no workspace, no device
    allocation inside the call).  Outputs are the caller's: pass y (bf16
    [T][d]) and, if wanted, topk_ids / topk_w to allocate nothing at all."""
    s = _on(stream)
    with torch.cuda.stream(s):
        x, router_w = _bits16(x), _bits16(router_w)
        T, d = x.shape
        E = router_w.shape[0]
        f = experts["gu_codes"].shape[1] // 2
        if y is None:
            y = torch.empty((T, d), dtype=torch.bfloat16, device=x.device)
        bias = None if router_bias is None else router_bias.contiguous().float()
        dims = dims_of(T, d, E, k, f)
        ex = experts_of(experts)
        st = lib().moe_layer_forward_noalloc(ctypes.byref(dims), _ptr(x), _ptr(router_w),
                                             _ptr(bias), ctypes.byref(ex), _ptr(y),
                                             _ptr(topk_ids), _ptr(topk_w), _stream(s))
    _check(st, "moe_layer_forward_noalloc")
    return y


# ---- MoE tail (include/moe_tail.h) ------------------------------------------------
def tail_of(tail: dict) -> TailWeights:
    """tail: {"gamma": bf16 [d], "eps": float, "shared_gu": bf16 [2fs][d] or None,
    "shared_dn": bf16 [d][fs] or None}."""
    sgu, sdn = tail.get("shared_gu"), tail.get("shared_dn")
    fs = 0 if sgu is None else sgu.shape[0] // 2
    return TailWeights(tail["gamma"].data_ptr(), float(tail["eps"]), int(fs),
                       None if sgu is None else sgu.data_ptr(),
                       None if sdn is None else sdn.data_ptr())


def moe_rmsnorm(x, gamma, eps, stream=None):
    """xn bf16 [T][d] = RMSNorm(x) * gamma (canonical fp64 order, bit-exact)."""
    s = _on(stream)
    with torch.cuda.stream(s):
        x, gamma = _bits16(x), _bits16(gamma)
        T, d = x.shape
        dims = dims_of(T, d, 1, 1, 32)
        xn = torch.empty((T, d), dtype=torch.bfloat16, device=x.device)
        st = lib().moe_rmsnorm(ctypes.byref(dims), _ptr(x), _ptr(gamma), float(eps),
                               _ptr(xn), _stream(s))
    _check(st, "moe_rmsnorm")
    return xn


class Block(_Reusable):
    """Device pointers, dims and a reusable workspace for repeated
    ``moe_block_forward`` calls: out = x + routed(xn) + shared(xn),
    xn = RMSNorm(x) * gamma."""

    def __init__(self, experts: dict, router_w, k, tail: dict, router_bias=None, T=1,
                 act=ACT_BF16):
        self.act = int(act)
        self.experts = experts
        self.tail = tail
        self.router_w = _bits16(router_w)
        self.bias = None if router_bias is None else router_bias.contiguous().float()
        self.E, self.d = self.router_w.shape
        self.f = experts["gu_codes"].shape[1] // 2
        self.k = k
        self._ex = experts_of(experts)
        self._tw = tail_of(tail)
        self.reserve(T)

    def reserve(self, T):
        """Make the workspace large enough for a call with T tokens."""
        dims = dims_of(T, self.d, self.E, self.k, self.f, self.act)
        n = lib().moe_block_workspace_bytes(ctypes.byref(dims), ctypes.byref(self._tw))
        return self._ensure_ws(n, self.router_w.device)

    def forward(self, x, out=None, topk_ids=None, topk_w=None, stream=None):
        s = _on(stream)
        with torch.cuda.stream(s):
            x = _bits16(x)
            T = x.shape[0]
            ws = self.reserve(T)
            _keep(ws, s)
            if out is None:
                out = torch.empty((T, self.d), dtype=torch.bfloat16, device=x.device)
            dims = dims_of(T, self.d, self.E, self.k, self.f, self.act)
            st = lib().moe_block_forward(ctypes.byref(dims), _ptr(x), ctypes.byref(self._tw),
                                         _ptr(self.router_w), _ptr(self.bias),
                                         ctypes.byref(self._ex), _ptr(out), _ptr(topk_ids),
                                         _ptr(topk_w), _ptr(ws), ws.numel(), _stream(s))
        _check(st, "moe_block_forward")
        return out


def moe_block_forward(x, router_w, experts: dict, k, tail: dict, router_bias=None,
                      return_routing=False, stream=None, act=ACT_BF16):
    """The pre-norm MoE block.  Returns out bf16 [T][d] (and topk_ids, topk_w)."""
    s = _on(stream)
    with torch.cuda.stream(s):
        x = _bits16(x)
        T = x.shape[0]
        blk = Block(experts, router_w, k, tail, router_bias, T=T, act=act)
        ids, w = _routing_outputs(T, k, x.device, return_routing)
        out = blk.forward(x, topk_ids=ids, topk_w=w, stream=s)
    return (out, ids, w) if return_routing else out


# ---- FP8 experts (include/moe_fp8.h) ----------------------------------------------
def fp8_experts_of(w: dict) -> Fp8Experts:
    return Fp8Experts(w["gu_codes"].data_ptr(), w["gu_scales"].data_ptr(),
                      w["dn_codes"].data_ptr(), w["dn_scales"].data_ptr())


def fp8_workspace(dims: Dims, entry: int, device) -> torch.Tensor:
    n = lib().moe_fp8_workspace_bytes(ctypes.byref(dims), int(entry))
    if n == SIZE_MAX:
        raise MoeError(MOE_ERR_SHAPE, "moe_fp8_workspace_bytes")
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def moe_expert_ffn_fp8(x, experts: dict, offsets, sorted_rows, k, ws=None, stream=None):
    """Expert FFN over grouped rows with FP8 experts.  Returns rows_out bf16
    [T*k][d]."""
    s = _on(stream)
    with torch.cuda.stream(s):
        x = _bits16(x)
        T, d = x.shape
        E, two_f = experts["gu_codes"].shape[:2]
        dims = dims_of(T, d, E, k, two_f // 2)
        rows_out = torch.empty((T * k, d), dtype=torch.bfloat16, device=x.device)
        if ws is None:
            ws = fp8_workspace(dims, ENTRY_EXPERT_FFN, x.device)
        offsets, sorted_rows = offsets.contiguous(), sorted_rows.contiguous()
        ex = fp8_experts_of(experts)
        st = lib().moe_expert_ffn_fp8(ctypes.byref(dims), _ptr(x), ctypes.byref(ex),
                                      _ptr(offsets), _ptr(sorted_rows), _ptr(rows_out),
                                      _ptr(ws), ws.numel(), _stream(s))
    _check(st, "moe_expert_ffn_fp8")
    return rows_out


class Fp8Layer(Layer):
    """Reusable workspace and pointers for repeated moe_layer_forward_fp8 calls."""

    _entry = "moe_layer_forward_fp8"

    def __init__(self, experts: dict, router_w, k, router_bias=None, T=1):
        super().__init__(experts, router_w, k, router_bias, T=T)
        self._ex = fp8_experts_of(experts)

    def _ws_bytes(self, dims):
        return lib().moe_fp8_workspace_bytes(ctypes.byref(dims), ENTRY_LAYER_FORWARD)


def moe_layer_forward_fp8(x, router_w, experts: dict, k, router_bias=None,
                          return_routing=False, stream=None):
    """The layer with FP8 experts.  Returns y bf16 [T][d] (and topk_ids, topk_w)."""
    s = _on(stream)
    with torch.cuda.stream(s):
        x = _bits16(x)
        T = x.shape[0]
        layer = Fp8Layer(experts, router_w, k, router_bias, T=T)
        ids, w = _routing_outputs(T, k, x.device, return_routing)
        y = layer.forward(x, topk_ids=ids, topk_w=w, stream=s)
    return (y, ids, w) if return_routing else y


# ---- operand-order (packed) expert store (include/moe_packed.h) ---------------------
def moe_prepack_experts(experts: dict, d: int, f: int, stream=None) -> dict:
    """The packed layout of an MXFP4 store (new tensors of the same shapes)."""
    s = _on(stream)
    with torch.cuda.stream(s):
        E = experts["gu_codes"].shape[0]
        dims = dims_of(1, d, E, 1, f)
        out = {n: torch.empty_like(v) for n, v in experts.items()
               if n in ("gu_codes", "gu_scales", "dn_codes", "dn_scales")}
        src, dst = experts_of(experts), experts_of(out)
        st = lib().moe_prepack_experts(ctypes.byref(dims), ctypes.byref(src), ctypes.byref(dst),
                                       _stream(s))
    _check(st, "moe_prepack_experts")
    return out


class PackedLayer(Layer):
    """moe_layer_forward_packed with a reusable workspace (prefill-sized T)."""

    _entry = "moe_layer_forward_packed"


def moe_layer_forward_packed(x, router_w, packed: dict, k, router_bias=None,
                             return_routing=False, stream=None, act=ACT_BF16):
    """The layer on a packed store (T >= 128).  Returns y (and topk_ids, topk_w)."""
    s = _on(stream)
    with torch.cuda.stream(s):
        x = _bits16(x)
        T = x.shape[0]
        layer = PackedLayer(packed, router_w, k, router_bias, T=T, act=act)
        ids, w = _routing_outputs(T, k, x.device, return_routing)
        y = layer.forward(x, topk_ids=ids, topk_w=w, stream=s)
    return (y, ids, w) if return_routing else y
