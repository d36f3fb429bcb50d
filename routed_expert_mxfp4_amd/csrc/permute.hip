// permute.hip -- group the T*k (token, slot) rows by expert (gfx950).
//
// The plan is built from routing alone, before any expert weight is read
// (the "payload-free plan" of layer-major prefill: Moonshine README, "How
// the engine works").  Rows r = t*k + j are ordered by (expert, token,
// slot): a stable counting sort, bit-exact integer work with no order-
// dependent atomics.
//
// Because the k experts of one token are distinct, the tokens that chose
// expert e inside a tile of 64 tokens form a 64-bit mask; the rank of token
// t among them is a popcount of the mask below bit t.  Tiles of 64 tokens
// are grouped into blocks of kSub tiles; block-level counts are scanned over
// blocks (per expert) and over experts (offsets).
#include "moe_internal.hpp"
#include "select_dev.hpp"

namespace moe {
namespace {

constexpr int kSub = 4;                    // 64-token tiles per block
constexpr int kTokBlk = 64 * kSub;         // tokens per block

// Exclusive scan of one int per thread over a block of 1024 threads.
__device__ int block_exclusive_scan(int v, int *tmp /* >= 16 ints */, int *total) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    int inc = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        int u = __shfl_up(inc, o, 64);
        if (lane >= o) inc += u;
    }
    if (lane == 63) tmp[wid] = inc;
    __syncthreads();
    if (wid == 0) {
        int w = lane < 16 ? tmp[lane] : 0;
        int wi = w;
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) {
            int u = __shfl_up(wi, o, 64);
            if (lane >= o) wi += u;
        }
        if (lane < 16) tmp[16 + lane] = wi - w;      // exclusive wave offsets
        if (lane == 15) tmp[32] = wi;
    }
    __syncthreads();
    int res = tmp[16 + wid] + inc - v;
    *total = tmp[32];
    __syncthreads();
    return res;
}

__device__ __forceinline__ int valid_id(int e, int E) { return (unsigned)e < (unsigned)E; }

// ---------------------------------------------------------------------------
// T <= kTokBlk: one block of 1024 threads does everything.
// ---------------------------------------------------------------------------
// mask: LDS u64 [kSub][E]; off_s: LDS int [E]; tmp: LDS int [48].
__device__ void permute_block(const int32_t *ids, unsigned long long *mask, int *off_s,
                              int *tmp, int32_t *__restrict__ counts,
                              int32_t *__restrict__ offsets, int32_t *__restrict__ sorted_rows,
                              int32_t *__restrict__ row_pos, int32_t *__restrict__ plan, int T,
                              int E, int k) {
    const int tid = threadIdx.x;
    const int nrows = T * k;
    for (int i = tid; i < kSub * E; i += 1024) mask[i] = 0ull;
    __syncthreads();
    for (int r = tid; r < nrows; r += 1024) {
        const int t = r / k, e = ids[r];
        if (valid_id(e, E)) atomicOr(&mask[(t >> 6) * E + e], 1ull << (t & 63));
    }
    __syncthreads();
    int c = 0;
    if (tid < E)
        for (int sb = 0; sb < kSub; ++sb) c += __popcll(mask[sb * E + tid]);
    int total;
    const int off = block_exclusive_scan(tid < E ? c : 0, tmp, &total);
    if (tid < E) {
        off_s[tid] = off;
        counts[tid] = c;
        offsets[tid] = off;
    }
    if (tid == 0) offsets[E] = total;
    if (plan) {
        int act_total;
        const int a = block_exclusive_scan(tid < E && c > 0 ? 1 : 0, tmp, &act_total);
        if (tid < E && c > 0) plan[1 + a] = tid;
        if (tid == 0) plan[0] = act_total;
    }
    __syncthreads();
    for (int r = tid; r < nrows; r += 1024) {
        const int t = r / k, e = ids[r];
        if (!valid_id(e, E)) continue;
        const int sb = t >> 6, tl = t & 63;
        int pos = off_s[e];
        for (int s2 = 0; s2 < sb; ++s2) pos += __popcll(mask[s2 * E + e]);
        pos += __popcll(mask[sb * E + e] & ((1ull << tl) - 1ull));
        sorted_rows[pos] = r;
        row_pos[r] = pos;
    }
}

__global__ __launch_bounds__(1024) void permute_single_kernel(
    const int32_t *__restrict__ ids, int32_t *__restrict__ counts,
    int32_t *__restrict__ offsets, int32_t *__restrict__ sorted_rows,
    int32_t *__restrict__ row_pos, int32_t *__restrict__ plan, int T, int E, int k) {
    extern __shared__ unsigned long long smem_u64[];
    unsigned long long *mask = smem_u64;                         // [kSub][E]
    int *off_s = reinterpret_cast<int *>(mask + kSub * E);       // [E]
    __shared__ int tmp[48];
    permute_block(ids, mask, off_s, tmp, counts, offsets, sorted_rows, row_pos, plan, T, E, k);
}

// T <= 16: top-k + softmax (one wave per token) and the grouping in one block.
template <int PL>
__global__ __launch_bounds__(1024) void topk_permute_small_kernel(
    const float *__restrict__ logits, int32_t *__restrict__ ids, float *__restrict__ tw,
    int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
    int32_t *__restrict__ sorted_rows, int32_t *__restrict__ row_pos,
    int32_t *__restrict__ plan, int T, int E, int k) {
    extern __shared__ unsigned long long smem_u64[];
    unsigned long long *mask = smem_u64;                         // [kSub][E]
    int *off_s = reinterpret_cast<int *>(mask + kSub * E);       // [E]
    int *ids_s = off_s + E;                                      // [16 * k]
    __shared__ int tmp[48];
    __shared__ __align__(16) uint32_t tsc[16][kTopkScratch];
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    if (wid < T) {
        int e;
        float wt;
        wave_topk_softmax<PL>(logits + (size_t)wid * E, E, k, tsc[wid], &e, &wt);
        if (lane < k) {
            ids[(size_t)wid * k + lane] = e;
            tw[(size_t)wid * k + lane] = wt;
            ids_s[wid * k + lane] = e;
        }
    }
    __syncthreads();
    permute_block(ids_s, mask, off_s, tmp, counts, offsets, sorted_rows, row_pos, plan, T, E, k);
}

// T * k <= 256: top-k + softmax (wave t for token t), then the grouping with
// three barriers.  Each row's key (expert << 8 | row) is distinct, so its
// position in (expert, token, slot) order is the number of smaller keys;
// offsets[e] is the lower bound of e << 8 in the sorted keys; the plan lists
// the experts that start a run of the sorted keys.
constexpr int kTinyRows = 256;

template <int PL>
__global__ __launch_bounds__(1024) void topk_permute_tiny_kernel(
    const float *__restrict__ logits, int32_t *__restrict__ ids, float *__restrict__ tw,
    int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
    int32_t *__restrict__ sorted_rows, int32_t *__restrict__ row_pos,
    int32_t *__restrict__ plan, int T, int E, int k) {
    __shared__ uint32_t key[kTinyRows];
    __shared__ uint32_t skey[kTinyRows];
    __shared__ int wcnt[16];
    __shared__ __align__(16) uint32_t tsc[16][kTopkScratch];
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int R = T * k;
    if (wid < T) {
        int e;
        float wt;
        wave_topk_softmax<PL>(logits + (size_t)wid * E, E, k, tsc[wid], &e, &wt);
        if (lane < k) {
            const int r = wid * k + lane;
            ids[r] = e;
            tw[r] = wt;
            key[r] = ((uint32_t)min(max(e, 0), E - 1) << 8) | (uint32_t)r;
        }
    }
    __syncthreads();
    if (tid < R) {
        const uint32_t kv = key[tid];
        int pos = 0;
        for (int i = 0; i < R; ++i) pos += key[i] < kv ? 1 : 0;
        skey[pos] = kv;
        sorted_rows[pos] = tid;
        row_pos[tid] = pos;
    }
    __syncthreads();
    for (int e = tid; e <= E; e += 1024) {
        int lo = 0, hi = R;
        const uint32_t t0 = (uint32_t)e << 8;
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (skey[mid] < t0) lo = mid + 1;
            else hi = mid;
        }
        offsets[e] = lo;
        if (e < E) {
            int lo2 = lo, hi2 = R;
            const uint32_t t1 = (uint32_t)(e + 1) << 8;
            while (lo2 < hi2) {
                const int mid = (lo2 + hi2) >> 1;
                if (skey[mid] < t1) lo2 = mid + 1;
                else hi2 = mid;
            }
            counts[e] = lo2 - lo;
        }
    }
    if (plan) {
        const bool start = tid < R && (tid == 0 || (skey[tid] >> 8) != (skey[tid - 1] >> 8));
        const unsigned long long m = __ballot(start);
        if (lane == 0) wcnt[wid] = (int)__popcll(m);
        __syncthreads();
        int base = 0;
        for (int w = 0; w < wid; ++w) base += wcnt[w];
        if (start) plan[1 + base + (int)__popcll(m & ((1ull << lane) - 1ull))] = (int)(skey[tid] >> 8);
        if (tid == 0) {
            int tot = 0;
            for (int w = 0; w < 16; ++w) tot += wcnt[w];
            plan[0] = tot;
        }
    }
}

// ---------------------------------------------------------------------------
// General T: count -> scan over blocks -> scan over experts -> scatter.
// ---------------------------------------------------------------------------
// masks   u64 [nb][kSub][E]   tokens of each 64-token tile that chose e
// blkcnt  int [E][nb]         rows of expert e in block b
// blkpre  int [E][nb]         exclusive prefix of blkcnt over b
// totals  int [E]
__global__ __launch_bounds__(256) void permute_count_kernel(
    const int32_t *__restrict__ ids, unsigned long long *__restrict__ masks,
    int32_t *__restrict__ blkcnt, int T, int E, int k, int nb) {
    extern __shared__ unsigned long long smem_u64[];
    unsigned long long *mask = smem_u64;                         // [kSub][E]
    const int b = blockIdx.x, tid = threadIdx.x;
    for (int i = tid; i < kSub * E; i += 256) mask[i] = 0ull;
    __syncthreads();
    const int t0 = b * kTokBlk;
    const int t1 = min(T, t0 + kTokBlk);
    for (int r = t0 * k + tid; r < t1 * k; r += 256) {
        int t = r / k, e = ids[r];
        if (valid_id(e, E)) atomicOr(&mask[((t - t0) >> 6) * E + e], 1ull << (t & 63));
    }
    __syncthreads();
    for (int e = tid; e < E; e += 256) {
        int c = 0;
        for (int sb = 0; sb < kSub; ++sb) {
            unsigned long long m = mask[sb * E + e];
            masks[((size_t)b * kSub + sb) * E + e] = m;
            c += __popcll(m);
        }
        blkcnt[(size_t)e * nb + b] = c;
    }
}

// One wave per expert: exclusive scan of blkcnt[e][0..nb).
__global__ __launch_bounds__(64) void permute_scan_blocks_kernel(
    const int32_t *__restrict__ blkcnt, int32_t *__restrict__ blkpre,
    int32_t *__restrict__ totals, int E, int nb) {
    const int e = blockIdx.x, lane = threadIdx.x;
    const int32_t *src = blkcnt + (size_t)e * nb;
    int32_t *dst = blkpre + (size_t)e * nb;
    int carry = 0;
    for (int b0 = 0; b0 < nb; b0 += 64) {
        int v = b0 + lane < nb ? src[b0 + lane] : 0;
        int inc = v;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            int u = __shfl_up(inc, o, 64);
            if (lane >= o) inc += u;
        }
        if (b0 + lane < nb) dst[b0 + lane] = carry + inc - v;
        carry += __shfl(inc, 63, 64);
    }
    if (lane == 0) totals[e] = carry;
}

__global__ __launch_bounds__(1024) void permute_scan_experts_kernel(
    const int32_t *__restrict__ totals, int32_t *__restrict__ counts,
    int32_t *__restrict__ offsets, int32_t *__restrict__ plan, int E) {
    __shared__ int tmp[48];
    const int tid = threadIdx.x;
    int c = tid < E ? totals[tid] : 0;
    int total;
    int off = block_exclusive_scan(c, tmp, &total);
    if (tid < E) {
        counts[tid] = c;
        offsets[tid] = off;
    }
    if (tid == 0) offsets[E] = total;
    if (plan) {
        int act_total;
        int a = block_exclusive_scan(tid < E && c > 0 ? 1 : 0, tmp, &act_total);
        if (tid < E && c > 0) plan[1 + a] = tid;
        if (tid == 0) plan[0] = act_total;
    }
}

__global__ __launch_bounds__(256) void permute_scatter_kernel(
    const int32_t *__restrict__ ids, const unsigned long long *__restrict__ masks,
    const int32_t *__restrict__ blkpre, const int32_t *__restrict__ offsets,
    int32_t *__restrict__ sorted_rows, int32_t *__restrict__ row_pos, int T, int E, int k,
    int nb) {
    const long long r = (long long)blockIdx.x * 256 + threadIdx.x;
    if (r >= (long long)T * k) return;
    const int t = (int)(r / k), e = ids[r];
    if (!valid_id(e, E)) return;
    const int b = t / kTokBlk, sb = (t % kTokBlk) >> 6, tl = t & 63;
    int pos = offsets[e] + blkpre[(size_t)e * nb + b];
    const unsigned long long *mb = masks + (size_t)b * kSub * E + e;
    for (int s2 = 0; s2 < sb; ++s2) pos += __popcll(mb[(size_t)s2 * E]);
    pos += __popcll(mb[(size_t)sb * E] & ((1ull << tl) - 1ull));
    sorted_rows[pos] = (int32_t)r;
    row_pos[r] = pos;
}

// Active-expert list from offsets: plan[0] = count, plan[1..] = ids (ascending).
__global__ __launch_bounds__(1024) void plan_kernel(const int32_t *__restrict__ offsets,
                                                    int32_t *__restrict__ plan, int E) {
    __shared__ int tmp[48];
    const int tid = threadIdx.x;
    int c = tid < E ? offsets[tid + 1] - offsets[tid] : 0;
    int act_total;
    int a = block_exclusive_scan(c > 0 ? 1 : 0, tmp, &act_total);
    if (tid < E && c > 0) plan[1 + a] = tid;
    if (tid == 0) plan[0] = act_total;
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

}  // namespace

size_t permute_ws_bytes(int T, int E) {
    if (T <= kTokBlk) return 0;
    const size_t nb = (size_t)(T + kTokBlk - 1) / kTokBlk;
    return align256(nb * kSub * E * 8) + 2 * align256(nb * E * 4) + align256((size_t)E * 4);
}

hipError_t launch_permute(const int32_t *ids, int32_t *counts, int32_t *offsets,
                          int32_t *sorted_rows, int32_t *row_pos, int32_t *plan, int T,
                          int E, int k, void *ws, hipStream_t s) {
    if (T <= kTokBlk) {
        size_t lds = (size_t)kSub * E * 8 + (size_t)E * 4;
        permute_single_kernel<<<1, 1024, lds, s>>>(ids, counts, offsets, sorted_rows, row_pos,
                                                   plan, T, E, k);
        return hipGetLastError();
    }
    const int nb = (T + kTokBlk - 1) / kTokBlk;
    char *p = static_cast<char *>(ws);
    auto *masks = reinterpret_cast<unsigned long long *>(p);
    p += align256((size_t)nb * kSub * E * 8);
    auto *blkcnt = reinterpret_cast<int32_t *>(p);
    p += align256((size_t)nb * E * 4);
    auto *blkpre = reinterpret_cast<int32_t *>(p);
    p += align256((size_t)nb * E * 4);
    auto *totals = reinterpret_cast<int32_t *>(p);
    permute_count_kernel<<<nb, 256, (size_t)kSub * E * 8, s>>>(ids, masks, blkcnt, T, E, k, nb);
    permute_scan_blocks_kernel<<<E, 64, 0, s>>>(blkcnt, blkpre, totals, E, nb);
    permute_scan_experts_kernel<<<1, 1024, 0, s>>>(totals, counts, offsets, plan, E);
    const long long rows = (long long)T * k;
    permute_scatter_kernel<<<(unsigned)((rows + 255) / 256), 256, 0, s>>>(
        ids, masks, blkpre, offsets, sorted_rows, row_pos, T, E, k, nb);
    return hipGetLastError();
}

bool topk_permute_fusable(int T, int E, int k) { return T <= 16 && E <= 1024 && k <= 32; }

hipError_t launch_topk_permute_small(const float *logits, int32_t *ids, float *tw,
                                     int32_t *counts, int32_t *offsets, int32_t *sorted_rows,
                                     int32_t *row_pos, int32_t *plan, int T, int E, int k,
                                     hipStream_t s) {
    const size_t lds = (size_t)kSub * E * 8 + (size_t)E * 4 + (size_t)16 * k * 4;
    const int pl = (E + 63) / 64;
    if (T * k <= kTinyRows) {
        if (pl <= 4)
            (void)timed_launch("topk_permute", topk_permute_tiny_kernel<4>, dim3(1), dim3(1024), 0, s, logits, ids, tw, counts, offsets,
                                                          sorted_rows, row_pos, plan, T, E, k);
        else if (pl <= 8)
            (void)timed_launch("topk_permute", topk_permute_tiny_kernel<8>, dim3(1), dim3(1024), 0, s, logits, ids, tw, counts, offsets,
                                                          sorted_rows, row_pos, plan, T, E, k);
        else
            (void)timed_launch("topk_permute", topk_permute_tiny_kernel<16>, dim3(1), dim3(1024), 0, s, logits, ids, tw, counts, offsets,
                                                           sorted_rows, row_pos, plan, T, E, k);
        return hipGetLastError();
    }
    if (pl <= 4)
        (void)timed_launch("topk_permute", topk_permute_small_kernel<4>, dim3(1), dim3(1024), lds, s, logits, ids, tw, counts, offsets,
                                                          sorted_rows, row_pos, plan, T, E, k);
    else if (pl <= 8)
        (void)timed_launch("topk_permute", topk_permute_small_kernel<8>, dim3(1), dim3(1024), lds, s, logits, ids, tw, counts, offsets,
                                                          sorted_rows, row_pos, plan, T, E, k);
    else
        (void)timed_launch("topk_permute", topk_permute_small_kernel<16>, dim3(1), dim3(1024), lds, s, logits, ids, tw, counts, offsets,
                                                           sorted_rows, row_pos, plan, T, E, k);
    return hipGetLastError();
}

hipError_t launch_plan(const int32_t *offsets, int32_t *plan, int E, hipStream_t s) {
    plan_kernel<<<1, 1024, 0, s>>>(offsets, plan, E);
    return hipGetLastError();
}

}  // namespace moe
