// Receive side of the emulated expert-parallel layout: one destination's region of the
// rank-major dispatch buffer reordered so that each of its local experts' rows are
// contiguous (the order its grouped GEMM needs), and the reverse move of the expert
// outputs back into the region for the return trip. [EFA] = Perplexity, "Enabling
// trillion-parameter models on AWS EFA" (2025): the receiver moves the tokens into the
// tensor handed to the grouped GEMM (Dispatch and combine); each sender's rows form one
// contiguous chunk of the destination's region (Send and receive buffers).
#include "common.h"

#include <algorithm>

namespace moe {
namespace {

constexpr int kRecvMaxPairs = 8192;      // local experts x senders held in LDS
constexpr int kRecvThreads = 1024;

// One workgroup. c[le][s] = counts[s][r*epr + le]. Local row of (le, s, i):
// local_off[le] + sum_{s' < s} c[le][s'] + i; its region row:
// chunk_off[r][s] + sum_{le' < le} c[le'][s] + i.
// LDS (dynamic): c [np] (then its prefix over s), cp [np] (prefix over le), rs [epr+1]
// (row sums, then their exclusive prefix = local_off). Every prefix is taken with
// independent loads in flight, never as one thread's chain of dependent LDS reads.
__global__ __launch_bounds__(kRecvThreads) void k_ep_recv_plan(const int *__restrict__ counts,
                                                               const int *__restrict__ chunk_off,
                                                               int n_src, int E, int epr, int r,
                                                               int cap, int *__restrict__ local_off,
                                                               int *__restrict__ row_src) {
    extern __shared__ int lds_plan[];
    const int np = epr * n_src;
    int *c = lds_plan;
    int *cp = c + np;
    int *rs = cp + np;
    __shared__ int scan_tmp[kRecvThreads];
    const int tid = threadIdx.x;
    for (int p = tid; p < np; p += blockDim.x) {
        const int le = p / n_src, s = p % n_src;
        c[p] = counts[size_t(s) * E + size_t(r) * epr + le];
    }
    __syncthreads();
    // cp[le][s] = sum_{le' < le} c[le'][s]: one thread per sender, eight loads in flight
    for (int s = tid; s < n_src; s += blockDim.x) {
        int run = 0, le = 0;
        for (; le + 8 <= epr; le += 8) {
            int w[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) w[u] = c[(le + u) * n_src + s];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                cp[(le + u) * n_src + s] = run;
                run += w[u];
            }
        }
        for (; le < epr; ++le) {
            const int w = c[le * n_src + s];
            cp[le * n_src + s] = run;
            run += w;
        }
    }
    __syncthreads();   // every read of c above is done before it is rewritten in place
    // row sums, and c[le][s] -> sum_{s' < s} c[le][s'] in place: one thread per expert
    for (int le = tid; le < epr; le += blockDim.x) {
        int *row = c + le * n_src;
        int run = 0, s = 0;
        for (; s + 8 <= n_src; s += 8) {
            int w[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) w[u] = row[s + u];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                row[s + u] = run;
                run += w[u];
            }
        }
        for (; s < n_src; ++s) {
            const int w = row[s];
            row[s] = run;
            run += w;
        }
        rs[le] = run;
    }
    __syncthreads();
    // local_off = exclusive prefix of the row sums (epr <= 1024: one per thread)
    int v = tid < epr ? rs[tid] : 0;
    const int mine = v;
    for (int off = 1; off < kRecvThreads; off <<= 1) {
        scan_tmp[tid] = v;
        __syncthreads();
        if (tid >= off) v += scan_tmp[tid - off];
        __syncthreads();
    }
    if (tid < epr) rs[tid] = v - mine;
    if (tid == kRecvThreads - 1) rs[epr] = v;        // inclusive total
    __syncthreads();
    const int live = rs[epr];
    for (int le = tid; le <= epr; le += blockDim.x) local_off[le] = rs[le];
    for (int p = tid; p < np; p += blockDim.x) {
        const int le = p / n_src, s = p % n_src;
        const int reg = chunk_off[size_t(r) * (n_src + 1) + s] + cp[p];
        const int loc = rs[le] + c[p];
        const int end = (s + 1 < n_src) ? c[p + 1] : rs[le + 1] - rs[le];
        const int n = end - c[p];
        for (int i = 0; i < n; ++i) {
            // an over-capacity plan (flagged by the dispatch) is cut at cap, never
            // written or read past it
            if (loc + i >= cap) break;
            row_src[loc + i] = (reg + i < cap) ? reg + i : -1;
        }
    }
    for (int j = live + tid; j < cap; j += blockDim.x) row_src[j] = -1;
}

// Row moves, one wavefront per row with 16-byte lanes. GATHER: dst[j] = src[row_src[j]];
// otherwise dst[row_src[j]] = src[j]; rows whose row_src is -1 are skipped.
template <bool GATHER>
__global__ __launch_bounds__(256) void k_ep_rows(const uint4 *__restrict__ src,
                                                 const int *__restrict__ row_src, int cap, int rc,
                                                 uint4 *__restrict__ dst) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wpb = blockDim.x / kWave;
    const int w0 = blockIdx.x * wpb + threadIdx.x / kWave;
    for (int j = w0; j < cap; j += gridDim.x * wpb) {
        const int q = row_src[j];
        if (q < 0 || q >= cap) continue;
        const uint4 *s = src + size_t(GATHER ? q : j) * rc;
        uint4 *o = dst + size_t(GATHER ? j : q) * rc;
        int ch = lane;
        for (; ch + 3 * kWave < rc; ch += 4 * kWave) {
            const uint4 v0 = s[ch], v1 = s[ch + kWave], v2 = s[ch + 2 * kWave], v3 = s[ch + 3 * kWave];
            o[ch] = v0;
            o[ch + kWave] = v1;
            o[ch + 2 * kWave] = v2;
            o[ch + 3 * kWave] = v3;
        }
        for (; ch < rc; ch += kWave) o[ch] = s[ch];
    }
}

// Gather with dequantization of the block-scaled fp8 payload: x_local[j] =
// bf16(decode(code) * scale) of region row row_src[j] (row j itself when row_src is
// null). A lane holds 8 codes (8 bytes) of a row; 16 lanes share one 128-element block.
__global__ __launch_bounds__(256) void k_ep_rows_fp8(const uint2 *__restrict__ q,
                                                     const float *__restrict__ qs,
                                                     const int *__restrict__ row_src, int cap,
                                                     int rc, uint4 *__restrict__ dst) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wpb = blockDim.x / kWave;
    const int w0 = blockIdx.x * wpb + threadIdx.x / kWave;
    const int nb = rc / 16;
    for (int j = w0; j < cap; j += gridDim.x * wpb) {
        const int src = row_src ? row_src[j] : j;
        if (src < 0 || src >= cap) continue;
        const uint2 *qr = q + size_t(src) * rc;
        const float *sr = qs + size_t(src) * nb;
        uint4 *o = dst + size_t(j) * rc;
        for (int c = lane; c < rc; c += kWave) {
            const uint2 w = qr[c];
            const float sc = sr[c / 16];
            float f[8];
            f[0] = __builtin_amdgcn_cvt_f32_fp8(int(w.x), 0) * sc;
            f[1] = __builtin_amdgcn_cvt_f32_fp8(int(w.x), 1) * sc;
            f[2] = __builtin_amdgcn_cvt_f32_fp8(int(w.x), 2) * sc;
            f[3] = __builtin_amdgcn_cvt_f32_fp8(int(w.x), 3) * sc;
            f[4] = __builtin_amdgcn_cvt_f32_fp8(int(w.y), 0) * sc;
            f[5] = __builtin_amdgcn_cvt_f32_fp8(int(w.y), 1) * sc;
            f[6] = __builtin_amdgcn_cvt_f32_fp8(int(w.y), 2) * sc;
            f[7] = __builtin_amdgcn_cvt_f32_fp8(int(w.y), 3) * sc;
            o[c] = Vec<MOE_BF16>::pack(f);
        }
    }
}

moe_status_t check_rows(const void *a, const void *row_src, int64_t cap, int64_t d,
                        moe_dtype_t dtype, const void *b) {
    if (!valid_dtype(dtype) || cap < 0 || d <= 0) return MOE_ERR_INVALID_ARG;
    if (cap >= (int64_t(1) << 31)) return MOE_ERR_UNSUPPORTED;
    if (cap == 0) return MOE_OK;
    if (!a || !row_src || !b) return MOE_ERR_INVALID_ARG;
    if ((d * elt_size(dtype)) % 16 != 0 || !aligned16(a) || !aligned16(b)) return MOE_ERR_ALIGN;
    return MOE_OK;
}

template <bool GATHER>
moe_status_t launch_rows(const void *src, const int32_t *row_src, int64_t cap, int64_t d,
                         moe_dtype_t dtype, void *dst, void *stream) {
    const moe_status_t c = check_rows(src, row_src, cap, d, dtype, dst);
    if (c != MOE_OK || cap == 0) return c;
    const int rc = int(d * elt_size(dtype) / 16);
    // four rows per workgroup, at most 2048 workgroups; each wavefront strides on
    const int g = int(std::min<int64_t>(cdiv(cap, 4), 2048));
    hipLaunchKernelGGL(k_ep_rows<GATHER>, dim3(g), dim3(256), 0, as_stream(stream),
                       static_cast<const uint4 *>(src), row_src, int(cap), rc,
                       static_cast<uint4 *>(dst));
    return launch_status();
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" moe_status_t moe_ep_recv_plan(const int32_t *counts, const int32_t *chunk_off,
                                         int32_t n_src, int32_t n_dst, int32_t E, int32_t r,
                                         int64_t cap, int32_t *local_off, int32_t *row_src,
                                         void *stream) {
    if (n_src <= 0 || n_dst <= 0 || E <= 0 || cap < 0) return MOE_ERR_INVALID_ARG;
    if (E % n_dst != 0 || r < 0 || r >= n_dst) return MOE_ERR_SHAPE;
    const int epr = E / n_dst;
    if (epr > 1024 || int64_t(epr) * n_src > kRecvMaxPairs || cap >= (int64_t(1) << 31))
        return MOE_ERR_UNSUPPORTED;
    if (!counts || !chunk_off || !local_off || (cap > 0 && !row_src)) return MOE_ERR_INVALID_ARG;
    const int lds = (2 * epr * n_src + epr + 1) * int(sizeof(int));
    if (!lds_limit_once<&k_ep_recv_plan>(2 * kRecvMaxPairs * 4 + 1025 * 4)) return MOE_ERR_HIP;
    hipLaunchKernelGGL(k_ep_recv_plan, dim3(1), dim3(kRecvThreads), lds, as_stream(stream), counts,
                       chunk_off, n_src, E, epr, r, int(cap), local_off, row_src);
    return launch_status();
}

extern "C" moe_status_t moe_ep_recv_gather(const void *x_region, const int32_t *row_src,
                                           int64_t cap, int64_t d, moe_dtype_t dtype,
                                           void *x_local, void *stream) {
    return launch_rows<true>(x_region, row_src, cap, d, dtype, x_local, stream);
}

extern "C" moe_status_t moe_ep_recv_gather_fp8(const uint8_t *q_region, const float *scale_region,
                                               const int32_t *row_src, int64_t cap, int64_t d,
                                               void *x_local, void *stream) {
    if (cap < 0 || d <= 0) return MOE_ERR_INVALID_ARG;
    if (cap >= (int64_t(1) << 31)) return MOE_ERR_UNSUPPORTED;
    if (cap == 0) return MOE_OK;
    if (!q_region || !scale_region || !x_local) return MOE_ERR_INVALID_ARG;
    if (d % 128 != 0) return MOE_ERR_UNSUPPORTED;
    if ((reinterpret_cast<uintptr_t>(q_region) & 7u) != 0 || !aligned16(scale_region) ||
        !aligned16(x_local))
        return MOE_ERR_ALIGN;
    const int rc = int(d / 8);
    const int g = int(std::min<int64_t>(cdiv(cap, 4), 2048));
    hipLaunchKernelGGL(k_ep_rows_fp8, dim3(g), dim3(256), 0, as_stream(stream),
                       reinterpret_cast<const uint2 *>(q_region), scale_region, row_src, int(cap),
                       rc, static_cast<uint4 *>(x_local));
    return launch_status();
}

extern "C" moe_status_t moe_ep_recv_scatter(const void *y_local, const int32_t *row_src,
                                            int64_t cap, int64_t d, moe_dtype_t dtype,
                                            void *y_region, void *stream) {
    return launch_rows<false>(y_local, row_src, cap, d, dtype, y_region, stream);
}
