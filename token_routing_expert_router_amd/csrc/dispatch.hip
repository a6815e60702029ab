// Dispatch: the plan (per-expert counts, offsets, a stable slot per (token, expert)
// pair) and the copy of each token into its slots, plus the copy's transpose for the
// backward. [EFA] = Perplexity, "Enabling trillion-parameter models on AWS EFA"
// (2025). Section "Dispatch and combine": per-expert token counts are accumulated
// atomically in the shared memory of one block, and their cumulative sum gives the
// offsets that pack tokens into contiguous per-destination send buffers. Section
// "Send and receive buffers": each sender's rows at a destination are one
// contiguous chunk (one write per peer); a destination receives at most
// N*T*max(R, E/N) rows.
//
// Plan kernels (deterministic, no order-dependent atomics):
//   k_plan_count  one workgroup per 256-token block of one source: every pair sets
//                 bit (t mod 256) of its expert's 256-bit mask in LDS (atomic OR,
//                 whose result does not depend on the order); popcounts are the
//                 block's per-expert counts.
//   k_plan_scan   one workgroup: per-source counts, expert offsets, chunk offsets
//                 per destination, and the first row of every (block, expert).
//   k_plan_slots  rebuilds the masks; a pair's rank inside its expert is the
//                 popcount of the mask bits below its token, so tokens keep their
//                 order inside every expert.
//   k_row_fill    marks rows no pair uses with -1 in row_pair.
// Copy kernel: one wavefront per token reads the row once with 16-byte loads and
// writes it to each of its k rows (coalesced 1 KiB per wavefront instruction).
#include "common.h"

namespace moe {
namespace {

constexpr int kPlanBlock = 256;                 // tokens per plan block
constexpr int kMaskWords = kPlanBlock / 64;     // 64-bit words per expert mask
constexpr int kScanThreads = 1024;
constexpr int kScanLdsInts = 16384;             // 64 KiB of LDS for the scan

struct PlanGeom {
    int T, k, E, n_src, n_dst, Ts, bps, B, epr;
    int64_t cap;
};

PlanGeom make_geom(int64_t T, int32_t E, int32_t k, const moe_layout_t *lay) {
    PlanGeom g;
    g.T = int(T);
    g.k = k;
    g.E = E;
    g.n_src = lay ? lay->n_src : 1;
    g.n_dst = lay ? lay->n_dst : 1;
    g.cap = lay ? lay->cap_rows_per_dst : T * k;
    g.Ts = g.T / g.n_src;
    g.bps = int(cdiv(g.Ts, kPlanBlock));
    g.B = g.n_src * g.bps;
    g.epr = E / g.n_dst;
    return g;
}

// Workspace: [0,256) status flag; blk_flags [B]; blk_counts [B][E]; blk_base [B][E].
// The flag is overwritten (never accumulated across calls), so nothing needs clearing.
size_t ws_bytes_for(const PlanGeom &g) {
    return 256 + align256(size_t(g.B) * sizeof(int)) + 2 * align256(size_t(g.B) * g.E * sizeof(int));
}

__device__ __forceinline__ void build_masks(unsigned long long *masks, const int *idx,
                                            int t_begin, int n, int k, int E, int *flag) {
    for (int i = threadIdx.x; i < E * kMaskWords; i += blockDim.x) masks[i] = 0ull;
    __syncthreads();
    const int t = threadIdx.x;
    if (t < n) {
        for (int j = 0; j < k; ++j) {
            const int e = idx[size_t(t_begin + t) * k + j];
            if (e < 0 || e >= E) {
                atomicOr(flag, kFlagBadIndex);
                continue;
            }
            const unsigned long long bit = 1ull << (t & 63);
            const unsigned long long old = atomicOr(&masks[e * kMaskWords + (t >> 6)], bit);
            if (old & bit) atomicOr(flag, kFlagBadIndex);   // expert listed twice
        }
    }
    __syncthreads();
}

__global__ __launch_bounds__(kPlanBlock) void k_plan_count(const int *__restrict__ idx, PlanGeom g,
                                                          int *__restrict__ blk_counts,
                                                          int *__restrict__ blk_flags) {
    extern __shared__ unsigned long long masks[];
    __shared__ int bflag;
    const int b = blockIdx.x;
    const int s = b / g.bps, tb = (b % g.bps) * kPlanBlock;
    const int n = min(kPlanBlock, g.Ts - tb);
    if (threadIdx.x == 0) bflag = 0;
    build_masks(masks, idx, s * g.Ts + tb, n, g.k, g.E, &bflag);
    if (threadIdx.x == 0) blk_flags[b] = bflag;
    for (int e = threadIdx.x; e < g.E; e += blockDim.x) {
        int c = 0;
#pragma unroll
        for (int w = 0; w < kMaskWords; ++w) c += __popcll(masks[e * kMaskWords + w]);
        blk_counts[size_t(b) * g.E + e] = c;
    }
}

__global__ __launch_bounds__(kScanThreads) void k_plan_scan(
    const int *__restrict__ blk_counts, const int *__restrict__ blk_flags, PlanGeom g,
    int *__restrict__ counts, int *__restrict__ expert_off, int *__restrict__ chunk_off,
    int *__restrict__ blk_base, int *__restrict__ flag) {
    extern __shared__ int lds[];
    __shared__ int sflag;
    const int E = g.E, ns = g.n_src, nd = g.n_dst, epr = g.epr;
    int *cnt = lds;                      // [ns][E]: counts, then rows before e in its chunk
    int *tot = cnt + ns * E;             // [E]: per-expert totals, then their scan
    int *chk = tot + E;                  // [ns][nd]: chunk sizes, then chunk offsets
    const int tid = threadIdx.x;
    if (tid == 0) sflag = 0;
    __syncthreads();
    for (int b = tid; b < g.B; b += kScanThreads)
        if (blk_flags[b]) atomicOr(&sflag, blk_flags[b]);

    // per-source counts
    for (int se = tid; se < ns * E; se += kScanThreads) {
        const int s = se / E, e = se % E;
        int c = 0;
        for (int bb = 0; bb < g.bps; ++bb) c += blk_counts[size_t(s * g.bps + bb) * E + e];
        cnt[se] = c;
        counts[se] = c;
    }
    __syncthreads();
    // per-expert totals
    for (int e = tid; e < E; e += kScanThreads) {
        int c = 0;
        for (int s = 0; s < ns; ++s) c += cnt[s * E + e];
        tot[e] = c;
    }
    __syncthreads();
    // rows before expert e inside (source s -> destination r), and chunk sizes
    for (int sr = tid; sr < ns * nd; sr += kScanThreads) {
        const int s = sr / nd, r = sr % nd;
        int run = 0;
        for (int e = r * epr; e < (r + 1) * epr; ++e) {
            const int c = cnt[s * E + e];
            cnt[s * E + e] = run;
            run += c;
        }
        chk[s * nd + r] = run;
    }
    __syncthreads();
    // chunk offsets inside every destination, in sender order
    for (int r = tid; r < nd; r += kScanThreads) {
        int run = 0;
        for (int s = 0; s < ns; ++s) {
            const int c = chk[s * nd + r];
            chk[s * nd + r] = run;
            chunk_off[r * (ns + 1) + s] = run;
            run += c;
        }
        chunk_off[r * (ns + 1) + ns] = run;
        if (int64_t(run) > g.cap) atomicOr(&sflag, kFlagCapacity);
    }
    // exclusive scan of the per-expert totals (E <= 1024: one value per thread)
    {
        int v = (tid < E) ? tot[tid] : 0;
        const int own = v;
        __syncthreads();
        for (int off = 1; off < kScanThreads; off <<= 1) {
            if (tid < E) tot[tid] = v;
            __syncthreads();
            if (tid >= off && tid < E) v += tot[tid - off];
            __syncthreads();
        }
        if (tid < E) expert_off[tid] = v - own;
        if (tid == E - 1) expert_off[E] = v;
    }
    __syncthreads();
    if (tid == 0) *flag = sflag;      // overwrites the previous call's flag
    // first row of every (block, expert)
    for (int se = tid; se < ns * E; se += kScanThreads) {
        const int s = se / E, e = se % E, r = e / epr;
        int run = int(int64_t(r) * g.cap) + chk[s * nd + r] + cnt[se];
        for (int bb = 0; bb < g.bps; ++bb) {
            const size_t b = size_t(s * g.bps + bb) * E + e;
            blk_base[b] = run;
            run += blk_counts[b];
        }
    }
}

__global__ __launch_bounds__(kPlanBlock) void k_plan_slots(const int *__restrict__ idx, PlanGeom g,
                                                          const int *__restrict__ blk_base,
                                                          int *__restrict__ pair_slot,
                                                          int *__restrict__ row_pair,
                                                          int *__restrict__ flag) {
    extern __shared__ unsigned long long masks[];
    const int b = blockIdx.x;
    const int s = b / g.bps, tb = (b % g.bps) * kPlanBlock;
    const int n = min(kPlanBlock, g.Ts - tb);
    const int t_begin = s * g.Ts + tb;
    build_masks(masks, idx, t_begin, n, g.k, g.E, flag);
    const int t = threadIdx.x;
    if (t >= n) return;
    const int tg = t_begin + t;
    for (int j = 0; j < g.k; ++j) {
        const int e = idx[size_t(tg) * g.k + j];
        int slot = -1;
        if (e >= 0 && e < g.E) {
            const unsigned long long *m = masks + e * kMaskWords;
            int rank = 0;
            for (int w = 0; w < (t >> 6); ++w) rank += __popcll(m[w]);
            rank += __popcll(m[t >> 6] & ((1ull << (t & 63)) - 1ull));
            const int row = blk_base[size_t(b) * g.E + e] + rank;
            const int r = e / g.epr;
            if (int64_t(row) - int64_t(r) * g.cap < g.cap) {
                slot = row;
                row_pair[row] = tg * g.k + j;
            } else {
                atomicOr(flag, kFlagCapacity);
            }
        }
        pair_slot[size_t(tg) * g.k + j] = slot;
    }
}

__global__ void k_row_fill(PlanGeom g, const int *__restrict__ chunk_off, int *__restrict__ row_pair) {
    const int64_t total = int64_t(g.n_dst) * g.cap;
    for (int64_t row = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; row < total;
         row += int64_t(gridDim.x) * blockDim.x) {
        const int r = int(row / g.cap);
        const int64_t in_r = row - int64_t(r) * g.cap;
        if (in_r >= chunk_off[r * (g.n_src + 1) + g.n_src]) row_pair[row] = -1;
    }
}

// x_disp[pair_slot[t,j]] = x[t]: one wavefront per token, 16-byte chunks.
__global__ __launch_bounds__(256) void k_dispatch_rows(const uint4 *__restrict__ x,
                                                       const int *__restrict__ pair_slot, int T,
                                                       int k, int rc, int64_t rows_total,
                                                       uint4 *__restrict__ x_disp) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave0 = __builtin_amdgcn_readfirstlane((blockIdx.x * blockDim.x + threadIdx.x) / kWave);
    const int nwaves = gridDim.x * blockDim.x / kWave;
    for (int t = wave0; t < T; t += nwaves) {
        const int *ps = pair_slot + size_t(t) * k;
        const uint4 *src = x + size_t(t) * rc;
        int c = lane;
        for (; c + 3 * kWave < rc; c += 4 * kWave) {
            const uint4 v0 = src[c], v1 = src[c + kWave], v2 = src[c + 2 * kWave],
                        v3 = src[c + 3 * kWave];
            for (int j = 0; j < k; ++j) {
                const int s = ps[j];
                if (s < 0 || s >= rows_total) continue;
                uint4 *dst = x_disp + size_t(s) * rc;
                dst[c] = v0;
                dst[c + kWave] = v1;
                dst[c + 2 * kWave] = v2;
                dst[c + 3 * kWave] = v3;
            }
        }
        for (; c < rc; c += kWave) {
            const uint4 v = src[c];
            for (int j = 0; j < k; ++j) {
                const int s = ps[j];
                if (s < 0 || s >= rows_total) continue;
                x_disp[size_t(s) * rc + c] = v;
            }
        }
    }
}

// dx[t] = sum_j dx_disp[pair_slot[t,j]] + sum_j dl[t,j] * w_router[idx[t,j]]
template <int DT>
__global__ __launch_bounds__(256) void k_dispatch_bwd(const uint4 *__restrict__ dx_disp,
                                                      const int *__restrict__ pair_slot,
                                                      const int *__restrict__ topk_idx,
                                                      const float *__restrict__ dl,
                                                      const uint4 *__restrict__ w_router, int T,
                                                      int k, int E, int rc, int64_t rows_total,
                                                      uint4 *__restrict__ dx) {
    constexpr int VN = Vec<DT>::N;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave0 = __builtin_amdgcn_readfirstlane((blockIdx.x * blockDim.x + threadIdx.x) / kWave);
    const int nwaves = gridDim.x * blockDim.x / kWave;
    for (int t = wave0; t < T; t += nwaves) {
        const int *ps = pair_slot + size_t(t) * k;
        for (int c = lane; c < rc; c += kWave) {
            float acc[VN];
#pragma unroll
            for (int i = 0; i < VN; ++i) acc[i] = 0.0f;
            for (int j = 0; j < k; ++j) {
                const int s = ps[j];
                if (s < 0 || s >= rows_total) continue;
                float f[VN];
                Vec<DT>::unpack(dx_disp[size_t(s) * rc + c], f);
#pragma unroll
                for (int i = 0; i < VN; ++i) acc[i] += f[i];
            }
            if (dl != nullptr) {
                for (int j = 0; j < k; ++j) {
                    const int e = topk_idx[size_t(t) * k + j];
                    if (e < 0 || e >= E) continue;
                    const float g = dl[size_t(t) * k + j];
                    float f[VN];
                    Vec<DT>::unpack(w_router[size_t(e) * rc + c], f);
#pragma unroll
                    for (int i = 0; i < VN; ++i) acc[i] = __builtin_fmaf(g, f[i], acc[i]);
                }
            }
            dx[size_t(t) * rc + c] = Vec<DT>::pack(acc);
        }
    }
}

int copy_grid(int64_t T) { return int(std::min<int64_t>(cdiv(T, 4), 8192)); }

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" size_t moe_dispatch_workspace_size(int64_t T, int32_t E, int32_t k,
                                              const moe_layout_t *layout) {
    if (T < 0 || E <= 0 || k <= 0) return 0;
    if (layout && (layout->n_src <= 0 || layout->n_dst <= 0 || T % layout->n_src)) return 0;
    return ws_bytes_for(make_geom(T, E, k, layout));
}

extern "C" moe_status_t moe_dispatch(const void *x, const int32_t *topk_idx, int64_t T,
                                     int64_t d, int32_t E, int32_t k, moe_dtype_t dtype,
                                     const moe_layout_t *layout, int32_t *counts,
                                     int32_t *expert_off, int32_t *chunk_off, int32_t *pair_slot,
                                     int32_t *row_pair, void *x_disp, void *ws, size_t ws_bytes,
                                     void *stream) {
    if (!valid_dtype(dtype) || T < 0 || d <= 0 || E <= 0 || k <= 0) return MOE_ERR_INVALID_ARG;
    if (k > E) return MOE_ERR_SHAPE;
    if (layout && (layout->n_src <= 0 || layout->n_dst <= 0 || layout->cap_rows_per_dst < 0))
        return MOE_ERR_INVALID_ARG;
    const int n_src = layout ? layout->n_src : 1, n_dst = layout ? layout->n_dst : 1;
    if (T % n_src != 0 || E % n_dst != 0) return MOE_ERR_SHAPE;
    if (E > 1024 || T * k >= (int64_t(1) << 31)) return MOE_ERR_UNSUPPORTED;
    const PlanGeom g = make_geom(T, E, k, layout);
    // tight form of the receive bound: a token sends at most min(k, E/N) rows to one
    // destination, so a destination receives at most n_src * Ts * min(k, E/N) rows
    const int64_t need = int64_t(n_src) * g.Ts * std::min<int64_t>(k, g.epr);
    if (g.cap < need) return MOE_ERR_CAPACITY;
    if (int64_t(n_dst) * g.cap >= (int64_t(1) << 31)) return MOE_ERR_UNSUPPORTED;
    const size_t lds_scan = size_t(n_src * E + E + n_src * n_dst) * sizeof(int);
    if (lds_scan > size_t(kScanLdsInts) * sizeof(int)) return MOE_ERR_UNSUPPORTED;
    if (T == 0) return MOE_OK;
    if (!topk_idx || !counts || !expert_off || !chunk_off || !pair_slot || !row_pair || !ws)
        return MOE_ERR_INVALID_ARG;
    if ((x == nullptr) != (x_disp == nullptr)) return MOE_ERR_INVALID_ARG;
    if (ws_bytes < ws_bytes_for(g)) return MOE_ERR_CAPACITY;
    if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return MOE_ERR_ALIGN;
    const int64_t rowb = d * elt_size(dtype);
    if (x && (rowb % 16 != 0 || !aligned16(x) || !aligned16(x_disp))) return MOE_ERR_ALIGN;

    const hipStream_t st = as_stream(stream);
    char *wsb = static_cast<char *>(ws);
    int *flag = reinterpret_cast<int *>(wsb);
    int *blk_flags = reinterpret_cast<int *>(wsb + 256);
    int *blk_counts = reinterpret_cast<int *>(wsb + 256 + align256(size_t(g.B) * sizeof(int)));
    int *blk_base = blk_counts + align256(size_t(g.B) * E * sizeof(int)) / sizeof(int);
    const size_t lds_mask = size_t(E) * kMaskWords * sizeof(unsigned long long);

    hipLaunchKernelGGL(k_plan_count, dim3(g.B), dim3(kPlanBlock), lds_mask, st, topk_idx, g,
                       blk_counts, blk_flags);
    hipLaunchKernelGGL(k_plan_scan, dim3(1), dim3(kScanThreads), lds_scan, st, blk_counts,
                       blk_flags, g, counts, expert_off, chunk_off, blk_base, flag);
    hipLaunchKernelGGL(k_plan_slots, dim3(g.B), dim3(kPlanBlock), lds_mask, st, topk_idx, g,
                       blk_base, pair_slot, row_pair, flag);
    {
        const int64_t rows = int64_t(n_dst) * g.cap;
        const int grid = int(std::min<int64_t>(cdiv(rows, 256), 4096));
        hipLaunchKernelGGL(k_row_fill, dim3(grid), dim3(256), 0, st, g, chunk_off, row_pair);
    }
    if (x) {
        hipLaunchKernelGGL(k_dispatch_rows, dim3(copy_grid(T)), dim3(256), 0, st,
                           static_cast<const uint4 *>(x), pair_slot, int(T), k, int(rowb / 16),
                           int64_t(n_dst) * g.cap, static_cast<uint4 *>(x_disp));
    }
    return launch_status();
}

extern "C" moe_status_t moe_dispatch_status(const void *ws, void *stream) {
    if (!ws) return MOE_ERR_INVALID_ARG;
    int flag = 0;
    if (hipStreamSynchronize(as_stream(stream)) != hipSuccess) return MOE_ERR_HIP;
    if (hipMemcpy(&flag, ws, sizeof(int), hipMemcpyDeviceToHost) != hipSuccess) return MOE_ERR_HIP;
    if (flag & kFlagBadIndex) return MOE_ERR_BAD_INDEX;
    if (flag & kFlagCapacity) return MOE_ERR_CAPACITY;
    return MOE_OK;
}

extern "C" moe_status_t moe_dispatch_bwd(const void *dx_disp, const int32_t *pair_slot,
                                         const int32_t *topk_idx, const float *dlogits_sel,
                                         const void *w_router, int64_t T, int32_t k, int64_t d,
                                         int32_t E, int64_t rows_total, moe_dtype_t dtype,
                                         void *dx, void *stream) {
    if (!valid_dtype(dtype) || T < 0 || d <= 0 || k <= 0 || rows_total < 0)
        return MOE_ERR_INVALID_ARG;
    if (T == 0) return MOE_OK;
    if (!dx_disp || !pair_slot || !dx) return MOE_ERR_INVALID_ARG;
    if (dlogits_sel && (!topk_idx || !w_router || E <= 0)) return MOE_ERR_INVALID_ARG;
    const int64_t rowb = d * elt_size(dtype);
    if (rowb % 16 != 0 || !aligned16(dx_disp) || !aligned16(dx) ||
        (w_router && !aligned16(w_router)))
        return MOE_ERR_ALIGN;
    const hipStream_t st = as_stream(stream);
    if (dtype == MOE_BF16)
        hipLaunchKernelGGL(k_dispatch_bwd<MOE_BF16>, dim3(copy_grid(T)), dim3(256), 0, st,
                           static_cast<const uint4 *>(dx_disp), pair_slot, topk_idx, dlogits_sel,
                           static_cast<const uint4 *>(w_router), int(T), k, E, int(rowb / 16),
                           rows_total, static_cast<uint4 *>(dx));
    else
        hipLaunchKernelGGL(k_dispatch_bwd<MOE_F32>, dim3(copy_grid(T)), dim3(256), 0, st,
                           static_cast<const uint4 *>(dx_disp), pair_slot, topk_idx, dlogits_sel,
                           static_cast<const uint4 *>(w_router), int(T), k, E, int(rowb / 16),
                           rows_total, static_cast<uint4 *>(dx));
    return launch_status();
}
