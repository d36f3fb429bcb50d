// moe_abi.cpp -- the C ABI of include/moe.h: host-side validation, workspace
// planning and dispatch of the gfx950 kernels onto the caller's stream.
//
// Every entry point validates all arguments before launching anything
// (a refused request leaves the outputs untouched), never allocates, never
// synchronises the host with the device, and never lets a C++ exception out.
#include "../../include/moe.h"
#include "../../include/moe_diag.h"
#include "../../include/moe_fp8.h"
#include "../../include/moe_packed.h"
#include "../../include/moe_tail.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "moe_internal.hpp"

namespace {

using moe::ExpertArgs;

constexpr int64_t kRowsLimit = (int64_t)1 << 31;
constexpr int kFuseMaxT = 4;          // small T: fused down + combine

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
size_t al256(size_t v) { return (v + 255) & ~(size_t)255; }

moe_status check_dims(const moe_dims *dm) {
    if (!dm) return MOE_ERR_NULL;
    const moe_dims &D = *dm;
    if (D.T < 0 || D.d <= 0 || D.E <= 0 || D.k <= 0 || D.f <= 0) return MOE_ERR_SHAPE;
    if (D.d % 64 != 0 || D.d > 32768) return MOE_ERR_SHAPE;
    if (D.f % 32 != 0 || D.f > 16384) return MOE_ERR_SHAPE;
    if (D.E > moe::kMaxExperts) return MOE_ERR_SHAPE;
    if (D.k > D.E || D.k > moe::kMaxTopK) return MOE_ERR_SHAPE;
    if ((int64_t)D.T * D.k >= kRowsLimit) return MOE_ERR_SHAPE;
    if (D.act != MOE_ACT_BF16 && D.act != MOE_ACT_MX_E2M3) return MOE_ERR_SHAPE;
    return MOE_OK;
}

moe_status check_experts(const moe_mxfp4_experts *w) {
    if (!w) return MOE_ERR_NULL;
    if (!w->gu_codes || !w->gu_scales || !w->dn_codes || !w->dn_scales) return MOE_ERR_NULL;
    if (!aligned16(w->gu_codes) || !aligned16(w->gu_scales) || !aligned16(w->dn_codes) ||
        !aligned16(w->dn_scales))
        return MOE_ERR_ALIGN;
    return MOE_OK;
}

moe_status device_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_DEVICE; }

// ---- workspace layouts ------------------------------------------------------
// Route: logits (the canonical ones, or the filter's approximations) and
// the row norms and candidate lists of the filtered path.
struct RouteWs {
    size_t logits, nx, nw, cand, ncand, total;
};
RouteWs route_ws(const moe_dims &D) {
    RouteWs w;
    size_t p = 0;
    w.logits = p; p += al256((size_t)D.T * D.E * 4);
    w.nx = p; p += al256((size_t)D.T * 4);
    w.nw = p; p += al256((size_t)D.E * 4);
    w.cand = p; p += al256((size_t)D.T * moe::kRouteCandMax * 4);
    w.ncand = p; p += al256((size_t)D.T * 4);
    w.total = p;
    return w;
}

// ---- expert path ---------------------------------------------------------------
// The diagnostic override of the per-expert crossover (-1: the built-in one).
std::atomic<int> g_gemv_max_override{-1};

// Rows at or below which an expert of a scaled-MFMA call takes the grouped
// GEMVs (0: every expert on MFMA tiles).  -1 where there is no per-expert
// choice: the activation-MX mode (whose GEMVs would need a rounded copy of
// x), the packed store (the GEMVs read the canonical one) and shapes the
// small-expert GEMVs do not serve.
int ffn_gemv_max(const moe_dims &D, bool packed) {
    if (packed || D.act != MOE_ACT_BF16 || !moe::gemv_small_ok(D.d, D.f)) return -1;
    const int o = g_gemv_max_override.load(std::memory_order_relaxed);
    return o >= 0 ? o : moe::kGemvMaxRows;
}

// Whether a call takes the scaled-MFMA expert path (with its small experts
// on the GEMVs), else the GEMV path for every expert.  The choice is per
// expert, by its rows: with the crossover R the call goes to the mixed path
// as soon as some expert could have more than R rows (T > R).  Without a
// per-expert choice, from kMfmaMinT tokens on.  A few tokens keep the fused
// down + combine.
bool use_mfma(const moe_dims &D, bool packed) {
    if (!moe::mfma_shape_ok(D.T, D.d, D.k, D.f) || D.T <= kFuseMaxT) return false;
    const int R = ffn_gemv_max(D, packed);
    return R < 0 ? D.T >= moe::kMfmaMinT : D.T > R;
}

struct FfnWs {
    size_t plan, h, mfma, xr, total;
};
FfnWs ffn_ws(const moe_dims &D, bool packed = false) {
    FfnWs w;
    w.plan = 0;
    w.h = al256((size_t)(D.E + 1) * 4);
    w.mfma = w.h;
    w.xr = w.h;
    // the fp32 h of the GEMV path (and, in the activation-MX mode, the
    // rounded copy of x); the MFMA path keeps h split in its own ws, and the
    // mixed path its small experts' compact fp32 h
    if (use_mfma(D, packed)) {
        w.total = w.mfma + al256(moe::mixed_ws_bytes(D.T, D.d, D.E, D.k, D.f,
                                                     std::max(0, ffn_gemv_max(D, packed))));
    } else {
        w.xr = w.h + al256((size_t)D.T * D.k * D.f * 4);
        w.total = w.xr + (D.act ? al256((size_t)D.T * D.d * 2) : 0);
    }
    return w;
}

struct LayerWs {
    size_t route, ids, tw, counts, offsets, sorted_rows, row_pos, perm, ffn, rows_out, total;
};
LayerWs layer_ws(const moe_dims &D, bool packed = false) {
    const size_t rows = (size_t)D.T * D.k;
    LayerWs w;
    size_t p = 0;
    w.route = p; p += route_ws(D).total;
    w.ids = p; p += al256(rows * 4);
    w.tw = p; p += al256(rows * 4);
    w.counts = p; p += al256((size_t)D.E * 4);
    w.offsets = p; p += al256((size_t)(D.E + 1) * 4);
    w.sorted_rows = p; p += al256(rows * 4);
    w.row_pos = p; p += al256(rows * 4);
    w.perm = p; p += al256(moe::permute_ws_bytes(D.T, D.E));
    w.ffn = p; p += al256(ffn_ws(D, packed).total);
    w.rows_out = p;
    if (D.T > kFuseMaxT) p += al256(rows * D.d * 2);
    w.total = p;
    return w;
}

// ---- diagnostics: HIP events around the launches of one named kernel ------
struct Diag {
    std::mutex mu;
    std::atomic<bool> active{false};
    std::string name;
    std::vector<hipEvent_t> ev;       // [2 * capacity]: start, stop pairs
    int used = 0;
    int every = 1;                    // time one launch in `every`
    long long seen = 0;               // launches of the named kernel so far
};
Diag g_diag;

// FP8 experts: the grouped GEMVs for few tokens, the bf16 matrix-core GEMMs
// from kMfmaMinT tokens on.  FFN: the plan, then h [T*k][f] (fp32 on the
// GEMV path, bf16 on the GEMM path), then the GEMMs' row-tile list.  Layer:
// the routed layer's routing and grouping scratch, that, and rows_out
// [T*k][d] bf16.
struct Fp8FfnWs {
    size_t plan, h, tiles, total;
};
Fp8FfnWs fp8_ffn_ws(const moe_dims &D) {
    Fp8FfnWs w;
    w.plan = 0;
    w.h = al256((size_t)(D.E + 1) * 4);
    w.tiles = w.h + al256((size_t)D.T * D.k * D.f * 4);
    w.total = w.tiles;
    if (moe::fp8_mfma_ok(D.T, D.d, D.E, D.k, D.f))
        w.total += al256(moe::fp8_mfma_tiles_bytes(D.T, D.E, D.k));
    return w;
}
struct Fp8LayerWs {
    size_t route, ids, tw, counts, offsets, sorted_rows, row_pos, perm, ffn, rows_out, total;
};
Fp8LayerWs fp8_layer_ws(const moe_dims &D) {
    const size_t rows = (size_t)D.T * D.k;
    Fp8LayerWs w;
    size_t p = 0;
    w.route = p; p += route_ws(D).total;
    w.ids = p; p += al256(rows * 4);
    w.tw = p; p += al256(rows * 4);
    w.counts = p; p += al256((size_t)D.E * 4);
    w.offsets = p; p += al256((size_t)(D.E + 1) * 4);
    w.sorted_rows = p; p += al256(rows * 4);
    w.row_pos = p; p += al256(rows * 4);
    w.perm = p; p += al256(moe::permute_ws_bytes(D.T, D.E));
    w.ffn = p; p += fp8_ffn_ws(D).total;
    w.rows_out = p; p += al256(rows * D.d * 2);
    w.total = p;
    return w;
}

moe_status check_fp8(const moe_dims &D, const moe_fp8_experts *w) {
    if (D.d % 128 != 0 || D.f % 128 != 0) return MOE_ERR_SHAPE;
    if (D.act != MOE_ACT_BF16) return MOE_ERR_UNSUPPORTED;
    if (!w) return MOE_ERR_NULL;
    if (!w->gu_codes || !w->gu_scales || !w->dn_codes || !w->dn_scales) return MOE_ERR_NULL;
    if (!aligned16(w->gu_codes) || !aligned16(w->gu_scales) || !aligned16(w->dn_codes) ||
        !aligned16(w->dn_scales))
        return MOE_ERR_ALIGN;
    return MOE_OK;
}

// Pre-norm block: the routed layer's scratch, then xn; few tokens: the
// routed output y and the shared expert's fp32 h; many tokens: the shared
// expert's bf16 h and its down output (fp32).
struct BlockWs {
    size_t layer, xn, yr, hs, hb, sx, total;
};
BlockWs block_ws(const moe_dims &D, int fs) {
    BlockWs w;
    const size_t T = (size_t)D.T, d = (size_t)D.d;
    size_t p = 0;
    w.layer = p; p += layer_ws(D).total;
    w.xn = p; p += al256(T * d * 2);
    w.yr = w.hs = w.hb = w.sx = p;
    if (D.T <= moe::kSharedGemvMaxT) {
        w.yr = p; p += al256(T * d * 2);
        w.hs = p; p += al256(T * (size_t)fs * 4);
    } else if (fs > 0) {
        w.hb = p; p += al256(T * (size_t)fs * 2);
        w.sx = p; p += al256(T * d * 4);
    }
    w.total = p;
    return w;
}

moe_status check_tail(const moe_tail_weights *tw) {
    if (!tw) return MOE_ERR_NULL;
    if (!tw->norm_w) return MOE_ERR_NULL;
    if (!std::isfinite(tw->eps) || tw->eps < 0.f) return MOE_ERR_SHAPE;
    if (tw->fs < 0 || tw->fs > 16384 || tw->fs % 32 != 0) return MOE_ERR_SHAPE;
    if (tw->fs > 0 && (!tw->shared_gu || !tw->shared_dn)) return MOE_ERR_NULL;
    if (!aligned16(tw->norm_w)) return MOE_ERR_ALIGN;
    if (tw->fs > 0 && (!aligned16(tw->shared_gu) || !aligned16(tw->shared_dn)))
        return MOE_ERR_ALIGN;
    return MOE_OK;
}

template <typename Fn>
moe_status guarded(Fn fn) {
    try {
        return fn();
    } catch (...) {
        return MOE_ERR_DEVICE;
    }
}

}  // namespace

namespace moe {
// Records a start event before and a stop event after the launches in the
// scope's lifetime when that kernel name is being timed.
DiagScope::DiagScope(const char *kernel, hipStream_t s) : s_(s) {
    if (!g_diag.active.load(std::memory_order_acquire)) return;
    std::lock_guard<std::mutex> lk(g_diag.mu);
    if (g_diag.name != kernel) return;
    if (g_diag.seen++ % g_diag.every != 0) return;
    if (2 * (g_diag.used + 1) > (int)g_diag.ev.size()) return;
    hipEvent_t start = g_diag.ev[2 * g_diag.used];
    stop_ = g_diag.ev[2 * g_diag.used + 1];
    ++g_diag.used;
    (void)hipEventRecord(start, s_);
}
DiagScope::~DiagScope() {
    if (stop_) (void)hipEventRecord(stop_, s_);
}
void diag_launch_events(const char *kernel, hipEvent_t *start, hipEvent_t *stop) {
    *start = *stop = nullptr;
    if (!g_diag.active.load(std::memory_order_acquire)) return;
    std::lock_guard<std::mutex> lk(g_diag.mu);
    if (g_diag.name != kernel) return;
    if (g_diag.seen++ % g_diag.every != 0) return;
    if (2 * (g_diag.used + 1) > (int)g_diag.ev.size()) return;
    *start = g_diag.ev[2 * g_diag.used];
    *stop = g_diag.ev[2 * g_diag.used + 1];
    ++g_diag.used;
}
}  // namespace moe

using moe::DiagScope;

namespace {

// The routed layer (steps 1-5 of moe.h) on validated arguments, its scratch
// at base (layout layer_ws).  resid / extra (nullable, only with
// D.T > kFuseMaxT): the pre-norm block's residual (bf16 [T][d]) and
// shared-expert output (fp32 [T][d]) added in the combine pass.
hipError_t run_layer(const moe_dims &D, const uint16_t *x, const uint16_t *router_w,
                     const float *router_bias, const moe_mxfp4_experts &experts, uint16_t *y,
                     int32_t *topk_ids_out, float *topk_w_out, char *base, hipStream_t s,
                     const uint16_t *resid, const float *extra, bool packed = false) {
    const LayerWs L = layer_ws(D, packed);
    const RouteWs RW = route_ws(D);
    float *logits = reinterpret_cast<float *>(base + L.route + RW.logits);
    int32_t *ids = topk_ids_out ? topk_ids_out : reinterpret_cast<int32_t *>(base + L.ids);
    float *tw = topk_w_out ? topk_w_out : reinterpret_cast<float *>(base + L.tw);
    int32_t *counts = reinterpret_cast<int32_t *>(base + L.counts);
    int32_t *offsets = reinterpret_cast<int32_t *>(base + L.offsets);
    int32_t *sorted_rows = reinterpret_cast<int32_t *>(base + L.sorted_rows);
    int32_t *row_pos = reinterpret_cast<int32_t *>(base + L.row_pos);
    void *perm_ws = base + L.perm;
    const FfnWs F = ffn_ws(D, packed);
    int32_t *plan = reinterpret_cast<int32_t *>(base + L.ffn + F.plan);
    float *h = reinterpret_cast<float *>(base + L.ffn + F.h);
    uint16_t *rows_out = reinterpret_cast<uint16_t *>(base + L.rows_out);
    const ExpertArgs W{experts.gu_codes, experts.gu_scales, experts.dn_codes,
                       experts.dn_scales};

    hipError_t e;
    const bool filtered = moe::route_filter_ok(D.T, D.d, D.E);
    // one token: top-k and grouping run inside the gate/up pass
    const bool token_fused =
        !filtered && moe::gate_up_token_fusable(D.T, D.d, D.E, D.k, D.f);
    if (filtered) {
        e = moe::launch_route_filtered(x, router_w, router_bias, logits,
                                       reinterpret_cast<float *>(base + L.route + RW.nx),
                                       reinterpret_cast<float *>(base + L.route + RW.nw),
                                       reinterpret_cast<int32_t *>(base + L.route + RW.cand),
                                       reinterpret_cast<int32_t *>(base + L.route + RW.ncand),
                                       ids, tw, D.T, D.d, D.E, D.k, s);
    } else {
        e = moe::launch_router_logits(x, router_w, router_bias, logits, D.T, D.d, D.E, s);
    }
    if (filtered) {
        if (e == hipSuccess) {
            DiagScope t("permute", s);
            e = moe::launch_permute(ids, counts, offsets, sorted_rows, row_pos, plan, D.T,
                                    D.E, D.k, perm_ws, s);
        }
    } else if (token_fused) {
    } else if (moe::topk_permute_fusable(D.T, D.E, D.k)) {
        if (e == hipSuccess) {
            e = moe::launch_topk_permute_small(logits, ids, tw, counts, offsets, sorted_rows,
                                               row_pos, plan, D.T, D.E, D.k, s);
        }
    } else {
        if (e == hipSuccess) {
            e = moe::launch_topk_softmax(logits, ids, tw, D.T, D.E, D.k, s);
        }
        if (e == hipSuccess) {
            DiagScope t("permute", s);
            e = moe::launch_permute(ids, counts, offsets, sorted_rows, row_pos, plan, D.T,
                                    D.E, D.k, perm_ws, s);
        }
    }
    if (use_mfma(D, packed)) {
        if (e == hipSuccess) {
            DiagScope t("mfma_ffn", s);
            e = moe::launch_mfma_ffn(x, W, offsets, sorted_rows, plan, rows_out,
                                     base + L.ffn + F.mfma, D.T, D.d, D.E, D.k, D.f,
                                     D.act == MOE_ACT_MX_E2M3, s, packed,
                                     std::max(0, ffn_gemv_max(D, packed)));
        }
        if (e == hipSuccess) {
            e = moe::launch_combine(rows_out, row_pos, tw, y, D.T, D.d, D.k, s, resid, extra);
        }
        return e;
    }
    // activation-MX mode on the GEMV path: x rounded into a copy (the
    // router above saw it as given), h in place
    const uint16_t *xa = x;
    if (D.act == MOE_ACT_MX_E2M3 && e == hipSuccess) {
        uint16_t *xr = reinterpret_cast<uint16_t *>(base + L.ffn + F.xr);
        e = moe::launch_mx_round_bf16(x, D.T, D.d, xr, s);
        xa = xr;
    }
    // bf16 mode, few tokens: h goes from gate/up to the fused down + combine
    // as bf16 (the prefill path's two-term split of h carries the same
    // precision); the activation-MX mode rounds an fp32 h in place
    const bool hb = D.act == MOE_ACT_BF16 && D.T <= kFuseMaxT &&
                    moe::gemv_bf16_h_ok(D.T, D.d, D.f);
    if (e == hipSuccess) {
        e = token_fused ? moe::launch_gate_up_token(logits, xa, W, ids, tw, counts, offsets,
                                                    sorted_rows, row_pos, plan, h, D.d, D.E,
                                                    D.k, D.f, s, hb)
                        : moe::launch_gemv_gate_up(xa, W, offsets, sorted_rows, plan, h, D.T,
                                                   D.d, D.E, D.k, D.f, s, hb);
    }
    if (D.act == MOE_ACT_MX_E2M3 && e == hipSuccess)
        e = moe::launch_mx_round_f32(h, D.T * D.k, D.f, h, s);
    if (D.T <= kFuseMaxT) {
        if (e == hipSuccess) {
            e = moe::launch_down_combine(h, W, ids, tw, row_pos, y, D.T, D.d, D.E, D.k, D.f, s,
                                         hb);
        }
    } else {
        if (e == hipSuccess) {
            e = moe::launch_gemv_down(h, W, offsets, plan, rows_out, D.T, D.d, D.E, D.k, D.f,
                                      s);
        }
        if (e == hipSuccess) {
            e = moe::launch_combine(rows_out, row_pos, tw, y, D.T, D.d, D.k, s, resid, extra);
        }
    }
    return e;
}

}  // namespace

// ---- static scratch of moe_layer_forward_noalloc ------------------------------
// One array per device, in the code object's data (not an allocation).  Host
// code never passes `scratch` itself to a kernel or a copy: on the host the
// name is only a stand-in for the symbol.  Its address on a device comes
// from hipGetSymbolAddress with that device current, once per device.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch` (looked up on first use).
moe_status scratch_for_current_device(hipStream_t s, void **ptr) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return MOE_ERR_DEVICE;
    if (dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
    if (s) {
        hipDevice_t sd = -1;
        if (hipStreamGetDevice(s, &sd) != hipSuccess) return MOE_ERR_DEVICE;
        if ((int)sd != dev) return MOE_ERR_UNSUPPORTED;
    }
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
            return MOE_ERR_DEVICE;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return MOE_OK;
}

}  // namespace


extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char *moe_status_str(int status) {
    switch (status) {
    case MOE_OK: return "MOE_OK: success";
    case MOE_ERR_NULL: return "MOE_ERR_NULL: a required pointer is NULL";
    case MOE_ERR_SHAPE: return "MOE_ERR_SHAPE: dims outside the supported limits";
    case MOE_ERR_ALIGN: return "MOE_ERR_ALIGN: a pointer is not 16-byte aligned";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace smaller than moe_workspace_bytes()";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: valid request this library does not serve";
    case MOE_ERR_DEVICE: return "MOE_ERR_DEVICE: HIP reported an error while launching";
    case MOE_ERR_SCRATCH:
        return "MOE_ERR_SCRATCH: the call needs more scratch than MOE_NOALLOC_SCRATCH_BYTES";
    default: return "unknown moe_status";
    }
}

size_t moe_workspace_bytes(const moe_dims *dims, int entry) {
    if (check_dims(dims) != MOE_OK) return (size_t)-1;
    const moe_dims &D = *dims;
    switch (entry) {
    case MOE_ENTRY_ROUTE: return route_ws(D).total;
    case MOE_ENTRY_PERMUTE: return moe::permute_ws_bytes(D.T, D.E);
    case MOE_ENTRY_EXPERT_FFN: return ffn_ws(D).total;
    case MOE_ENTRY_COMBINE: return 0;
    case MOE_ENTRY_LAYER_FORWARD: return layer_ws(D).total;
    default: return (size_t)-1;
    }
}

moe_status moe_route(const moe_dims *dims, const uint16_t *x, const uint16_t *router_w,
                     const float *router_bias, float *logits_out, int32_t *topk_ids,
                     float *topk_w, void *ws, size_t ws_bytes, void *hip_stream) {
    return guarded([&]() -> moe_status {
        moe_status st = check_dims(dims);
        if (st != MOE_OK) return st;
        const moe_dims &D = *dims;
        if (D.T == 0) return MOE_OK;
        if (!x || !router_w || !topk_ids || !topk_w) return MOE_ERR_NULL;
        if (!aligned16(x) || !aligned16(router_w)) return MOE_ERR_ALIGN;
        hipStream_t s = static_cast<hipStream_t>(hip_stream);
        hipError_t e;
        if (!logits_out && moe::route_filter_ok(D.T, D.d, D.E)) {
            if (!ws) return MOE_ERR_NULL;
            if (!aligned16(ws)) return MOE_ERR_ALIGN;
            const RouteWs R = route_ws(D);
            if (ws_bytes < R.total) return MOE_ERR_WORKSPACE;
            char *base = static_cast<char *>(ws);
            e = moe::launch_route_filtered(x, router_w, router_bias,
                                           reinterpret_cast<float *>(base + R.logits),
                                           reinterpret_cast<float *>(base + R.nx),
                                           reinterpret_cast<float *>(base + R.nw),
                                           reinterpret_cast<int32_t *>(base + R.cand),
                                           reinterpret_cast<int32_t *>(base + R.ncand), topk_ids,
                                           topk_w, D.T, D.d, D.E, D.k, s);
            return device_status(e);
        }
        float *logits = logits_out;
        if (!logits) {
            if (!ws) return MOE_ERR_NULL;
            if (!aligned16(ws)) return MOE_ERR_ALIGN;
            if (ws_bytes < route_ws(D).total) return MOE_ERR_WORKSPACE;
            logits = reinterpret_cast<float *>(static_cast<char *>(ws) + route_ws(D).logits);
        }
        {
            e = moe::launch_router_logits(x, router_w, router_bias, logits, D.T, D.d, D.E, s);
        }
        if (e == hipSuccess) {
            e = moe::launch_topk_softmax(logits, topk_ids, topk_w, D.T, D.E, D.k, s);
        }
        return device_status(e);
    });
}

moe_status moe_permute(const moe_dims *dims, const int32_t *topk_ids, int32_t *counts,
                       int32_t *offsets, int32_t *sorted_rows, int32_t *row_pos, void *ws,
                       size_t ws_bytes, void *hip_stream) {
    return guarded([&]() -> moe_status {
        moe_status st = check_dims(dims);
        if (st != MOE_OK) return st;
        const moe_dims &D = *dims;
        if (D.T == 0) return MOE_OK;
        if (!topk_ids || !counts || !offsets || !sorted_rows || !row_pos) return MOE_ERR_NULL;
        const size_t need = moe::permute_ws_bytes(D.T, D.E);
        if (need) {
            if (!ws) return MOE_ERR_NULL;
            if (!aligned16(ws)) return MOE_ERR_ALIGN;
            if (ws_bytes < need) return MOE_ERR_WORKSPACE;
        }
        hipStream_t s = static_cast<hipStream_t>(hip_stream);
        DiagScope t("permute", s);
        return device_status(moe::launch_permute(topk_ids, counts, offsets, sorted_rows, row_pos,
                                                 nullptr, D.T, D.E, D.k, ws, s));
    });
}

moe_status moe_expert_ffn(const moe_dims *dims, const uint16_t *x,
                          const moe_mxfp4_experts *experts, const int32_t *offsets,
                          const int32_t *sorted_rows, uint16_t *rows_out, void *ws,
                          size_t ws_bytes, void *hip_stream) {
    return guarded([&]() -> moe_status {
        moe_status st = check_dims(dims);
        if (st != MOE_OK) return st;
        const moe_dims &D = *dims;
        if (D.T == 0) return MOE_OK;
        if (!x || !offsets || !sorted_rows || !rows_out) return MOE_ERR_NULL;
        if ((st = check_experts(experts)) != MOE_OK) return st;
        if (!aligned16(x) || !aligned16(rows_out)) return MOE_ERR_ALIGN;
        const FfnWs L = ffn_ws(D);
        if (!ws) return MOE_ERR_NULL;
        if (!aligned16(ws)) return MOE_ERR_ALIGN;
        if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
        char *base = static_cast<char *>(ws);
        int32_t *plan = reinterpret_cast<int32_t *>(base + L.plan);
        float *h = reinterpret_cast<float *>(base + L.h);
        const ExpertArgs W{experts->gu_codes, experts->gu_scales, experts->dn_codes,
                           experts->dn_scales};
        hipStream_t s = static_cast<hipStream_t>(hip_stream);
        hipError_t e;
        {
            DiagScope t("plan", s);
            e = moe::launch_plan(offsets, plan, D.E, s);
        }
        if (use_mfma(D, false)) {
            if (e == hipSuccess) {
                DiagScope t("mfma_ffn", s);
                e = moe::launch_mfma_ffn(x, W, offsets, sorted_rows, plan, rows_out,
                                         base + L.mfma, D.T, D.d, D.E, D.k, D.f,
                                         D.act == MOE_ACT_MX_E2M3, s, false,
                                         std::max(0, ffn_gemv_max(D, false)));
            }
            return device_status(e);
        }
        // activation-MX mode on the GEMV path: x rounded into a copy, h in place
        const uint16_t *xa = x;
        if (D.act == MOE_ACT_MX_E2M3 && e == hipSuccess) {
            uint16_t *xr = reinterpret_cast<uint16_t *>(base + L.xr);
            e = moe::launch_mx_round_bf16(x, D.T, D.d, xr, s);
            xa = xr;
        }
        if (e == hipSuccess) {
            e = moe::launch_gemv_gate_up(xa, W, offsets, sorted_rows, plan, h, D.T, D.d, D.E,
                                         D.k, D.f, s);
        }
        if (D.act == MOE_ACT_MX_E2M3 && e == hipSuccess)
            e = moe::launch_mx_round_f32(h, D.T * D.k, D.f, h, s);
        if (e == hipSuccess) {
            e = moe::launch_gemv_down(h, W, offsets, plan, rows_out, D.T, D.d, D.E, D.k, D.f, s);
        }
        return device_status(e);
    });
}

moe_status moe_combine(const moe_dims *dims, const uint16_t *rows_out, const int32_t *row_pos,
                       const float *topk_w, uint16_t *y, void *hip_stream) {
    return guarded([&]() -> moe_status {
        moe_status st = check_dims(dims);
        if (st != MOE_OK) return st;
        const moe_dims &D = *dims;
        if (D.T == 0) return MOE_OK;
        if (!rows_out || !row_pos || !topk_w || !y) return MOE_ERR_NULL;
        if (!aligned16(rows_out) || !aligned16(y)) return MOE_ERR_ALIGN;
        hipStream_t s = static_cast<hipStream_t>(hip_stream);
        return device_status(moe::launch_combine(rows_out, row_pos, topk_w, y, D.T, D.d, D.k, s));
    });
}

moe_status moe_layer_forward(const moe_dims *dims, const uint16_t *x, const uint16_t *router_w,
                             const float *router_bias, const moe_mxfp4_experts *experts,
                             uint16_t *y, int32_t *topk_ids_out, float *topk_w_out, void *ws,
                             size_t ws_bytes, void *hip_stream) {
    return guarded([&]() -> moe_status {
        moe_status st = check_dims(dims);
        if (st != MOE_OK) return st;
        const moe_dims &D = *dims;
        if (D.T == 0) return MOE_OK;
        if (!x || !router_w || !y) return MOE_ERR_NULL;
        if ((st = check_experts(experts)) != MOE_OK) return st;
        if (!aligned16(x) || !aligned16(router_w) || !aligned16(y)) return MOE_ERR_ALIGN;
        const LayerWs L = layer_ws(D);
        if (!ws) return MOE_ERR_NULL;
        if (!aligned16(ws)) return MOE_ERR_ALIGN;
        if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
        return device_status(run_layer(D, x, router_w, router_bias, *experts, y, topk_ids_out,
                                       topk_w_out, static_cast<char *>(ws),
                                       static_cast<hipStream_t>(hip_stream), nullptr, nullptr));
    });
}

moe_status moe_layer_forward_noalloc(const moe_dims *dims, const uint16_t *x,
                                     const uint16_t *router_w, const float *router_bias,
                                     const moe_mxfp4_experts *experts, uint16_t *y,
                                     int32_t *topk_ids_out, float *topk_w_out,
                                     void *hip_stream) {
    return guarded([&]() -> moe_status {
        moe_status st = check_dims(dims);
        if (st != MOE_OK) return st;
        const moe_dims &D = *dims;
        if (D.T == 0) return MOE_OK;
        if (!x || !router_w || !y) return MOE_ERR_NULL;
        if ((st = check_experts(experts)) != MOE_OK) return st;
        if (!aligned16(x) || !aligned16(router_w) || !aligned16(y)) return MOE_ERR_ALIGN;
        if (layer_ws(D).total > MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_SCRATCH;
        hipStream_t s = static_cast<hipStream_t>(hip_stream);
        void *ws = nullptr;
        if ((st = scratch_for_current_device(s, &ws)) != MOE_OK) return st;
        return device_status(run_layer(D, x, router_w, router_bias, *experts, y, topk_ids_out,
                                       topk_w_out, static_cast<char *>(ws), s, nullptr,
                                       nullptr));
    });
}

moe_status moe_prepack_experts(const moe_dims *dims, const moe_mxfp4_experts *src,
                               const moe_mxfp4_experts *dst, void *hip_stream) {
    return guarded([&]() -> moe_status {
        moe_status st = check_dims(dims);
        if (st != MOE_OK) return st;
        const moe_dims &D = *dims;
        if ((st = check_experts(src)) != MOE_OK) return st;
        if ((st = check_experts(dst)) != MOE_OK) return st;
        if (!moe::prepack_ok(D.d, D.f)) return MOE_ERR_UNSUPPORTED;
        // no overlap between any source array and any destination array
        const size_t E = (size_t)D.E, d = (size_t)D.d, f = (size_t)D.f;
        const void *sp[4] = {src->gu_codes, src->gu_scales, src->dn_codes, src->dn_scales};
        const void *dp[4] = {dst->gu_codes, dst->gu_scales, dst->dn_codes, dst->dn_scales};
        const size_t nb[4] = {E * 2 * f * (d / 2), E * 2 * f * (d / 32), E * d * (f / 2),
                              E * d * (f / 32)};
        for (int i = 0; i < 4; ++i)
            for (int j = 0; j < 4; ++j) {
                const uintptr_t a0 = (uintptr_t)sp[i], a1 = a0 + nb[i];
                const uintptr_t b0 = (uintptr_t)dp[j], b1 = b0 + nb[j];
                if (a0 < b1 && b0 < a1) return MOE_ERR_UNSUPPORTED;
            }
        const ExpertArgs S{src->gu_codes, src->gu_scales, src->dn_codes, src->dn_scales};
        const ExpertArgs Dd{dst->gu_codes, dst->gu_scales, dst->dn_codes, dst->dn_scales};
        return device_status(moe::launch_prepack(S, Dd, D.E, D.d, D.f,
                                                 static_cast<hipStream_t>(hip_stream)));
    });
}

moe_status moe_layer_forward_packed(const moe_dims *dims, const uint16_t *x,
                                    const uint16_t *router_w, const float *router_bias,
                                    const moe_mxfp4_experts *packed, uint16_t *y,
                                    int32_t *topk_ids_out, float *topk_w_out, void *ws,
                                    size_t ws_bytes, void *hip_stream) {
    return guarded([&]() -> moe_status {
        moe_status st = check_dims(dims);
        if (st != MOE_OK) return st;
        const moe_dims &D = *dims;
        if (D.T == 0) return MOE_OK;
        if (!moe::prepack_ok(D.d, D.f) || !use_mfma(D, true)) return MOE_ERR_UNSUPPORTED;
        if (!x || !router_w || !y) return MOE_ERR_NULL;
        if ((st = check_experts(packed)) != MOE_OK) return st;
        if (!aligned16(x) || !aligned16(router_w) || !aligned16(y)) return MOE_ERR_ALIGN;
        // the documented size (moe_workspace_bytes for the canonical store),
        // which covers the packed call's own layout
        if (!ws) return MOE_ERR_NULL;
        if (!aligned16(ws)) return MOE_ERR_ALIGN;
        if (ws_bytes < layer_ws(D).total || ws_bytes < layer_ws(D, true).total)
            return MOE_ERR_WORKSPACE;
        return device_status(run_layer(D, x, router_w, router_bias, *packed, y, topk_ids_out,
                                       topk_w_out, static_cast<char *>(ws),
                                       static_cast<hipStream_t>(hip_stream), nullptr, nullptr,
                                       true));
    });
}

size_t moe_fp8_workspace_bytes(const moe_dims *dims, int entry) {
    if (check_dims(dims) != MOE_OK) return (size_t)-1;
    if (dims->d % 128 != 0 || dims->f % 128 != 0) return (size_t)-1;
    if (entry == MOE_ENTRY_EXPERT_FFN) return fp8_ffn_ws(*dims).total;
    if (entry == MOE_ENTRY_LAYER_FORWARD) return fp8_layer_ws(*dims).total;
    return (size_t)-1;
}

moe_status moe_expert_ffn_fp8(const moe_dims *dims, const uint16_t *x,
                              const moe_fp8_experts *experts, const int32_t *offsets,
                              const int32_t *sorted_rows, uint16_t *rows_out, void *ws,
                              size_t ws_bytes, void *hip_stream) {
    return guarded([&]() -> moe_status {
        moe_status st = check_dims(dims);
        if (st != MOE_OK) return st;
        const moe_dims &D = *dims;
        if ((st = check_fp8(D, experts)) != MOE_OK) return st;
        if (D.T == 0) return MOE_OK;
        if (!x || !offsets || !sorted_rows || !rows_out) return MOE_ERR_NULL;
        if (!aligned16(x) || !aligned16(rows_out)) return MOE_ERR_ALIGN;
        const Fp8FfnWs F = fp8_ffn_ws(D);
        if (!ws) return MOE_ERR_NULL;
        if (!aligned16(ws)) return MOE_ERR_ALIGN;
        if (ws_bytes < F.total) return MOE_ERR_WORKSPACE;
        char *base = static_cast<char *>(ws);
        int32_t *plan = reinterpret_cast<int32_t *>(base + F.plan);
        float *h = reinterpret_cast<float *>(base + F.h);
        const moe::Fp8Args W{experts->gu_codes, experts->gu_scales, experts->dn_codes,
                             experts->dn_scales};
        hipStream_t s = static_cast<hipStream_t>(hip_stream);
        if (moe::fp8_mfma_ok(D.T, D.d, D.E, D.k, D.f))
            return device_status(moe::launch_fp8_mfma_ffn(
                x, W, offsets, sorted_rows, reinterpret_cast<int32_t *>(base + F.tiles),
                reinterpret_cast<uint16_t *>(h), rows_out, D.T, D.d, D.E, D.k, D.f, s));
        hipError_t e = moe::launch_plan(offsets, plan, D.E, s);
        if (e == hipSuccess)
            e = moe::launch_fp8_gate_up(x, W, offsets, sorted_rows, plan, h, D.T, D.d, D.E, D.k,
                                        D.f, s);
        if (e == hipSuccess)
            e = moe::launch_fp8_down(h, W, offsets, plan, rows_out, D.T, D.d, D.E, D.k, D.f, s);
        return device_status(e);
    });
}

moe_status moe_layer_forward_fp8(const moe_dims *dims, const uint16_t *x,
                                 const uint16_t *router_w, const float *router_bias,
                                 const moe_fp8_experts *experts, uint16_t *y,
                                 int32_t *topk_ids_out, float *topk_w_out, void *ws,
                                 size_t ws_bytes, void *hip_stream) {
    return guarded([&]() -> moe_status {
        moe_status st = check_dims(dims);
        if (st != MOE_OK) return st;
        const moe_dims &D = *dims;
        if ((st = check_fp8(D, experts)) != MOE_OK) return st;
        if (D.T == 0) return MOE_OK;
        if (!x || !router_w || !y) return MOE_ERR_NULL;
        if (!aligned16(x) || !aligned16(router_w) || !aligned16(y)) return MOE_ERR_ALIGN;
        const Fp8LayerWs L = fp8_layer_ws(D);
        if (!ws) return MOE_ERR_NULL;
        if (!aligned16(ws)) return MOE_ERR_ALIGN;
        if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
        char *base = static_cast<char *>(ws);
        const RouteWs RW = route_ws(D);
        float *logits = reinterpret_cast<float *>(base + L.route + RW.logits);
        int32_t *ids = topk_ids_out ? topk_ids_out : reinterpret_cast<int32_t *>(base + L.ids);
        float *tw = topk_w_out ? topk_w_out : reinterpret_cast<float *>(base + L.tw);
        int32_t *counts = reinterpret_cast<int32_t *>(base + L.counts);
        int32_t *offsets = reinterpret_cast<int32_t *>(base + L.offsets);
        int32_t *sorted_rows = reinterpret_cast<int32_t *>(base + L.sorted_rows);
        int32_t *row_pos = reinterpret_cast<int32_t *>(base + L.row_pos);
        const Fp8FfnWs F = fp8_ffn_ws(D);
        int32_t *plan = reinterpret_cast<int32_t *>(base + L.ffn + F.plan);
        float *h = reinterpret_cast<float *>(base + L.ffn + F.h);
        uint16_t *rows_out = reinterpret_cast<uint16_t *>(base + L.rows_out);
        const moe::Fp8Args W{experts->gu_codes, experts->gu_scales, experts->dn_codes,
                             experts->dn_scales};
        hipStream_t s = static_cast<hipStream_t>(hip_stream);
        hipError_t e;
        const bool mfma = moe::fp8_mfma_ok(D.T, D.d, D.E, D.k, D.f);
        // one token: top-k and grouping inside the gate/up pass
        const bool token_fused = !mfma && !moe::route_filter_ok(D.T, D.d, D.E) &&
                                 moe::fp8_gate_up_token_fusable(D.T, D.d, D.E, D.k, D.f);
        // few tokens: down and combine in one pass
        const bool dc_fused = !mfma && moe::fp8_down_combine_ok(D.T, D.d, D.k, D.f);
        // routing and grouping as in the MXFP4 layer (the plan is written too)
        if (token_fused) {
            e = moe::launch_router_logits(x, router_w, router_bias, logits, D.T, D.d, D.E, s);
            if (e == hipSuccess)
                e = moe::launch_fp8_gate_up_token(logits, x, W, ids, tw, counts, offsets,
                                                  sorted_rows, row_pos, plan, h, D.d, D.E, D.k,
                                                  D.f, s);
        } else if (moe::route_filter_ok(D.T, D.d, D.E)) {
            e = moe::launch_route_filtered(x, router_w, router_bias, logits,
                                           reinterpret_cast<float *>(base + L.route + RW.nx),
                                           reinterpret_cast<float *>(base + L.route + RW.nw),
                                           reinterpret_cast<int32_t *>(base + L.route + RW.cand),
                                           reinterpret_cast<int32_t *>(base + L.route + RW.ncand),
                                           ids, tw, D.T, D.d, D.E, D.k, s);
            if (e == hipSuccess)
                e = moe::launch_permute(ids, counts, offsets, sorted_rows, row_pos, plan, D.T,
                                        D.E, D.k, base + L.perm, s);
        } else {
            e = moe::launch_router_logits(x, router_w, router_bias, logits, D.T, D.d, D.E, s);
            if (e == hipSuccess) {
                if (moe::topk_permute_fusable(D.T, D.E, D.k)) {
                    e = moe::launch_topk_permute_small(logits, ids, tw, counts, offsets,
                                                       sorted_rows, row_pos, plan, D.T, D.E, D.k,
                                                       s);
                } else {
                    e = moe::launch_topk_softmax(logits, ids, tw, D.T, D.E, D.k, s);
                    if (e == hipSuccess)
                        e = moe::launch_permute(ids, counts, offsets, sorted_rows, row_pos, plan,
                                                D.T, D.E, D.k, base + L.perm, s);
                }
            }
        }
        if (mfma) {
            if (e == hipSuccess)
                e = moe::launch_fp8_mfma_ffn(x, W, offsets, sorted_rows,
                                             reinterpret_cast<int32_t *>(base + L.ffn + F.tiles),
                                             reinterpret_cast<uint16_t *>(h), rows_out, D.T, D.d,
                                             D.E, D.k, D.f, s);
        } else {
            if (e == hipSuccess && !token_fused)
                e = moe::launch_fp8_gate_up(x, W, offsets, sorted_rows, plan, h, D.T, D.d, D.E,
                                            D.k, D.f, s);
            if (dc_fused) {
                if (e == hipSuccess)
                    e = moe::launch_fp8_down_combine(h, W, ids, tw, row_pos, y, D.T, D.d, D.E,
                                                     D.k, D.f, s);
                return device_status(e);
            }
            if (e == hipSuccess)
                e = moe::launch_fp8_down(h, W, offsets, plan, rows_out, D.T, D.d, D.E, D.k, D.f,
                                         s);
        }
        if (e == hipSuccess)
            e = moe::launch_combine(rows_out, row_pos, tw, y, D.T, D.d, D.k, s);
        return device_status(e);
    });
}

size_t moe_block_workspace_bytes(const moe_dims *dims, const moe_tail_weights *tail) {
    if (check_dims(dims) != MOE_OK || check_tail(tail) != MOE_OK) return (size_t)-1;
    return block_ws(*dims, tail->fs).total;
}

moe_status moe_rmsnorm(const moe_dims *dims, const uint16_t *x, const uint16_t *gamma,
                       float eps, uint16_t *xn, void *hip_stream) {
    return guarded([&]() -> moe_status {
        moe_status st = check_dims(dims);
        if (st != MOE_OK) return st;
        const moe_dims &D = *dims;
        if (!std::isfinite(eps) || eps < 0.f) return MOE_ERR_SHAPE;
        if (D.T == 0) return MOE_OK;
        if (!x || !gamma || !xn) return MOE_ERR_NULL;
        if (!aligned16(x) || !aligned16(gamma) || !aligned16(xn)) return MOE_ERR_ALIGN;
        return device_status(moe::launch_rmsnorm(x, gamma, eps, xn, D.T, D.d,
                                                 static_cast<hipStream_t>(hip_stream)));
    });
}

moe_status moe_block_forward(const moe_dims *dims, const uint16_t *x,
                             const moe_tail_weights *tail, const uint16_t *router_w,
                             const float *router_bias, const moe_mxfp4_experts *experts,
                             uint16_t *out, int32_t *topk_ids_out, float *topk_w_out, void *ws,
                             size_t ws_bytes, void *hip_stream) {
    return guarded([&]() -> moe_status {
        moe_status st = check_dims(dims);
        if (st != MOE_OK) return st;
        if ((st = check_tail(tail)) != MOE_OK) return st;
        const moe_dims &D = *dims;
        if (D.T == 0) return MOE_OK;
        if (!x || !router_w || !out) return MOE_ERR_NULL;
        if ((st = check_experts(experts)) != MOE_OK) return st;
        if (!aligned16(x) || !aligned16(router_w) || !aligned16(out)) return MOE_ERR_ALIGN;
        if (x == out) return MOE_ERR_UNSUPPORTED;
        const int fs = tail->fs;
        const BlockWs B = block_ws(D, fs);
        if (!ws) return MOE_ERR_NULL;
        if (!aligned16(ws)) return MOE_ERR_ALIGN;
        if (ws_bytes < B.total) return MOE_ERR_WORKSPACE;
        char *base = static_cast<char *>(ws);
        hipStream_t s = static_cast<hipStream_t>(hip_stream);
        uint16_t *xn = reinterpret_cast<uint16_t *>(base + B.xn);
        hipError_t e = moe::launch_rmsnorm(x, tail->norm_w, tail->eps, xn, D.T, D.d, s);
        if (D.T <= moe::kSharedGemvMaxT) {
            // few tokens: the routed output first, then the shared expert's
            // GEMVs, whose down pass adds x and y
            uint16_t *yr = reinterpret_cast<uint16_t *>(base + B.yr);
            if (e == hipSuccess)
                e = run_layer(D, xn, router_w, router_bias, *experts, yr, topk_ids_out,
                              topk_w_out, base + B.layer, s, nullptr, nullptr);
            if (e == hipSuccess)
                e = moe::launch_shared_gemv(xn, tail->shared_gu, tail->shared_dn, x, yr,
                                            reinterpret_cast<float *>(base + B.hs), out, D.T,
                                            D.d, fs, s);
            return device_status(e);
        }
        // many tokens: the shared expert's two GEMMs (SwiGLU fused into the
        // first), then the routed layer, whose combine pass adds x and the
        // shared output
        float *sx = nullptr;
        if (fs > 0) {
            uint16_t *hb = reinterpret_cast<uint16_t *>(base + B.hb);
            sx = reinterpret_cast<float *>(base + B.sx);
            if (e == hipSuccess)
                e = moe::launch_shared_gate_up_gemm(xn, tail->shared_gu, hb, D.T, D.d, fs, s);
            if (e == hipSuccess)
                e = moe::launch_shared_down_gemm(hb, tail->shared_dn, sx, D.T, D.d, fs, s);
        }
        if (e == hipSuccess)
            e = run_layer(D, xn, router_w, router_bias, *experts, out, topk_ids_out, topk_w_out,
                          base + B.layer, s, x, sx);
        return device_status(e);
    });
}

int moe_diag_mx_split_e2m3(const void *in, int in_is_bf16, int rows, int K, uint8_t *out,
                           void *hip_stream) {
    try {
        if (!in || !out || rows < 0 || K <= 0 || K % 128 != 0) return -1;
        if ((((uintptr_t)in | (uintptr_t)out) & 15u) != 0) return -1;
        if ((double)rows * (K / 128) * 208.0 >= 4294967296.0) return -1;
        hipStream_t st = static_cast<hipStream_t>(hip_stream);
        hipError_t e = in_is_bf16
                           ? moe::launch_mx_split_bf16(static_cast<const uint16_t *>(in), rows, K, out, st)
                           : moe::launch_mx_split_f32(static_cast<const float *>(in), rows, K, out, st);
        return e == hipSuccess ? 0 : -1;
    } catch (...) {
        return -1;
    }
}

int moe_diag_stream_read(const void *src, size_t bytes, uint32_t *out, int blocks,
                         void *hip_stream) {
    try {
        return moe::launch_stream_read(src, bytes, out, blocks,
                                       static_cast<hipStream_t>(hip_stream)) == hipSuccess
                   ? 0
                   : -1;
    } catch (...) {
        return -1;
    }
}

int moe_diag_mfma_rate(int kind, int blocks, int iters, float *out, void *hip_stream) {
    try {
        return moe::launch_mfma_rate(kind, blocks, iters, out,
                                     static_cast<hipStream_t>(hip_stream)) == hipSuccess
                   ? 0
                   : -1;
    } catch (...) {
        return -1;
    }
}

int moe_diag_set_gemv_max_rows(int rows) {
    if (rows < -1 || rows > moe::kGemvMaxRowsCap) return -1;
    g_gemv_max_override.store(rows, std::memory_order_relaxed);
    return 0;
}

int moe_diag_gemv_max_rows(void) {
    const int o = g_gemv_max_override.load(std::memory_order_relaxed);
    return o >= 0 ? o : moe::kGemvMaxRows;
}

int moe_diag_time_kernel(const char *kernel, int capacity) {
    return moe_diag_time_kernel_every(kernel, capacity, 1);
}

int moe_diag_time_kernel_every(const char *kernel, int capacity, int every) {
    try {
        if (capacity < 0 || every < 1) return -1;
        std::lock_guard<std::mutex> lk(g_diag.mu);
        g_diag.active.store(false, std::memory_order_release);
        g_diag.used = 0;
        g_diag.every = every;
        g_diag.seen = 0;
        g_diag.name = kernel ? kernel : "";
        while ((int)g_diag.ev.size() < 2 * capacity) {
            hipEvent_t ev;
            // timing only (read after the caller synchronises the device):
            // no system-scope fence, whose cache writeback and invalidate
            // would add to every timed launch
            if (hipEventCreateWithFlags(&ev, hipEventDisableSystemFence) != hipSuccess) return -1;
            g_diag.ev.push_back(ev);
        }
        g_diag.active.store(!g_diag.name.empty() && capacity > 0, std::memory_order_release);
        return 0;
    } catch (...) {
        return -1;
    }
}

int moe_diag_kernel_time(double *total_ms, long long *launches) {
    try {
        std::lock_guard<std::mutex> lk(g_diag.mu);
        double sum = 0.0;
        int rc = 0;
        for (int i = 0; i < g_diag.used; ++i) {
            float ms = 0.f;
            if (hipEventElapsedTime(&ms, g_diag.ev[2 * i], g_diag.ev[2 * i + 1]) != hipSuccess)
                rc = -1;
            sum += ms;
        }
        if (total_ms) *total_ms = sum;
        if (launches) *launches = g_diag.used;
        g_diag.used = 0;
        return rc;
    } catch (...) {
        return -1;
    }
}

int moe_diag_kernel_times(double *ms_out, int cap, long long *launches) {
    try {
        if (cap < 0 || (cap > 0 && !ms_out)) return -1;
        std::lock_guard<std::mutex> lk(g_diag.mu);
        int rc = 0;
        for (int i = 0; i < g_diag.used && i < cap; ++i) {
            float ms = 0.f;
            if (hipEventElapsedTime(&ms, g_diag.ev[2 * i], g_diag.ev[2 * i + 1]) != hipSuccess)
                rc = -1;
            ms_out[i] = ms;
        }
        if (launches) *launches = g_diag.used;
        g_diag.used = 0;
        return rc;
    } catch (...) {
        return -1;
    }
}

}  // extern "C"
