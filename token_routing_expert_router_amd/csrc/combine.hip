// Combine: each token's expert outputs come back and are averaged with the gate
// weights, y[t] = sum_j w[t,j] * y_disp[pair_slot[t,j]]. [EFA] = Perplexity,
// "Enabling trillion-parameter models on AWS EFA" (2025): the combine kernel is the
// dual of dispatch and computes the weighted average of the returned tokens
// (Introduction); it reuses the routing information dispatch produced and
// accumulates from the receive buffers into the output tensor (Dispatch and combine);
// accumulation happens at the receiver only (Dispatch/combine latency).
//
// One wavefront per token; lane c owns 16-byte column chunks c, c+64, ...; the k
// gathered rows are independent 16-byte loads (eight in flight together), summed in
// float32 in j order and rounded once; lane j holds pair j's slot and gate. The backward is the transpose: a scatter of
// w*dy into the k rows, and a dot product per (t, j) for the gate gradient.
#include "common.h"

namespace moe {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// NT: the gathered rows are read with the non-temporal cache policy (see combine_impl)
template <int DT, bool NT>
__global__ __launch_bounds__(256) void k_combine(const uint4 *__restrict__ y_disp,
                                                 const int *__restrict__ pair_slot,
                                                 const float *__restrict__ topk_w, int T, int k,
                                                 int rc, int64_t rows_total,
                                                 const uint4 *__restrict__ residual,
                                                 uint4 *__restrict__ y) {
    constexpr int VN = Vec<DT>::N;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave0 = __builtin_amdgcn_readfirstlane((blockIdx.x * blockDim.x + threadIdx.x) / kWave);
    const int nwaves = gridDim.x * blockDim.x / kWave;
    for (int t = wave0; t < T; t += nwaves) {
        // lane j < k holds pair j's slot and gate; the row loop reads them by lane
        const int my_s = lane < k ? pair_slot[size_t(t) * k + lane] : -1;
        const float my_g = lane < k ? topk_w[size_t(t) * k + lane] : 0.0f;
        for (int c = lane; c < rc; c += kWave) {
            float acc[VN];
            if (residual) {
                Vec<DT>::unpack(residual[size_t(t) * rc + c], acc);   // the sum starts here
            } else {
#pragma unroll
                for (int i = 0; i < VN; ++i) acc[i] = 0.0f;
            }
            // eight rows' loads in flight together, then their terms in j order
            for (int j0 = 0; j0 < k; j0 += 8) {
                uint4 v[8];
                bool ok[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int sj = __builtin_amdgcn_readlane(my_s, min(j0 + u, kWave - 1));
                    ok[u] = j0 + u < k && sj >= 0 && sj < rows_total;   // uniform
                    v[u] = make_uint4(0u, 0u, 0u, 0u);
                    if (ok[u]) {
                        if (NT)
                            v[u] = __builtin_bit_cast(uint4, __builtin_nontemporal_load(
                                reinterpret_cast<const u32x4 *>(y_disp) + size_t(sj) * rc + c));
                        else
                            v[u] = y_disp[size_t(sj) * rc + c];
                    }
                }
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    if (!ok[u]) continue;
                    const float g = __builtin_bit_cast(
                        float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_g), j0 + u));
                    float f[VN];
                    Vec<DT>::unpack(v[u], f);
#pragma unroll
                    for (int i = 0; i < VN; ++i) acc[i] = __builtin_fmaf(g, f[i], acc[i]);
                }
            }
            y[size_t(t) * rc + c] = Vec<DT>::pack(acc);
        }
    }
}

// dy_disp[pair_slot[t,j]] = w[t,j] * dy[t];  dtopk_w[t,j] = <dy[t], y_disp[pair_slot[t,j]]>
// For k <= 8 one pass over the row serves all pairs (the dy chunk and the k gathered
// chunks in flight together, a partial dot product per pair in registers); above that,
// one pass per pair, the token's dy row staying in cache between passes. Both sum each
// dot product in the same per-lane order and butterfly, so they agree bit for bit.
template <int DT>
__global__ __launch_bounds__(256) void k_combine_bwd(const uint4 *__restrict__ dy,
                                                     const uint4 *__restrict__ y_disp,
                                                     const int *__restrict__ pair_slot,
                                                     const float *__restrict__ topk_w, int T,
                                                     int k, int rc, int64_t rows_total,
                                                     uint4 *__restrict__ dy_disp,
                                                     float *__restrict__ dtopk_w) {
    constexpr int VN = Vec<DT>::N;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave0 = __builtin_amdgcn_readfirstlane((blockIdx.x * blockDim.x + threadIdx.x) / kWave);
    const int nwaves = gridDim.x * blockDim.x / kWave;
    for (int t = wave0; t < T; t += nwaves) {
        if (k <= 8) {
            // one pass over the row for all k pairs: the dy chunk and the k gathered chunks
            // in flight together; per pair the same per-lane order over c and the same
            // butterfly as the pass-per-pair form below
            const int my_s = lane < k ? pair_slot[size_t(t) * k + lane] : -1;
            const float my_w = lane < k ? topk_w[size_t(t) * k + lane] : 0.0f;
            float dot[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) dot[u] = 0.0f;
            for (int c = lane; c < rc; c += kWave) {
                const uint4 gv = dy[size_t(t) * rc + c];
                uint4 v[8];
                bool ok[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int su = __builtin_amdgcn_readlane(my_s, u);
                    ok[u] = u < k && su >= 0 && su < rows_total;   // uniform
                    v[u] = make_uint4(0u, 0u, 0u, 0u);
                    if (ok[u]) v[u] = y_disp[size_t(su) * rc + c];
                }
                float g[VN];
                Vec<DT>::unpack(gv, g);
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    if (!ok[u]) continue;
                    const int su = __builtin_amdgcn_readlane(my_s, u);
                    const float w = __builtin_bit_cast(
                        float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_w), u));
                    float f[VN], o[VN];
                    Vec<DT>::unpack(v[u], f);
#pragma unroll
                    for (int i = 0; i < VN; ++i) {
                        dot[u] = __builtin_fmaf(g[i], f[i], dot[u]);
                        o[i] = w * g[i];
                    }
                    dy_disp[size_t(su) * rc + c] = Vec<DT>::pack(o);
                }
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                if (u >= k) break;
                float dv = dot[u];
#pragma unroll
                for (int off = kWave / 2; off > 0; off >>= 1) dv += __shfl_xor(dv, off, kWave);
                if (lane == 0) dtopk_w[size_t(t) * k + u] = dv;
            }
            continue;
        }
        for (int j = 0; j < k; ++j) {
            const int s = pair_slot[size_t(t) * k + j];
            const bool ok = s >= 0 && s < rows_total;
            const float w = topk_w[size_t(t) * k + j];
            float dot = 0.0f;
            if (ok) {
                for (int c = lane; c < rc; c += kWave) {
                    float g[VN], f[VN], o[VN];
                    Vec<DT>::unpack(dy[size_t(t) * rc + c], g);
                    Vec<DT>::unpack(y_disp[size_t(s) * rc + c], f);
#pragma unroll
                    for (int i = 0; i < VN; ++i) {
                        dot = __builtin_fmaf(g[i], f[i], dot);
                        o[i] = w * g[i];
                    }
                    dy_disp[size_t(s) * rc + c] = Vec<DT>::pack(o);
                }
            }
#pragma unroll
            for (int off = kWave / 2; off > 0; off >>= 1) dot += __shfl_xor(dot, off, kWave);
            if (lane == 0) dtopk_w[size_t(t) * k + j] = dot;
        }
    }
}

// Partial combine at the destinations of the rank-major layout: for every token t and
// every destination r holding rows of t (rows [r*cap, (r+1)*cap)), the gate-weighted
// sum of t's rows at r, float32 fused multiply-adds in j order, one rounding:
// partial[r*T + t] (rows of tokens without rows at r are not written). Lane j < k of
// the token's wavefront holds slot j and its destination; the wavefront's set of
// destinations is a 64-bit mask (n_dst <= 64).
__device__ __forceinline__ uint64_t wave_or64(uint64_t v) {
    uint32_t lo = uint32_t(v), hi = uint32_t(v >> 32);
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        lo |= __shfl_xor(lo, off, kWave);
        hi |= __shfl_xor(hi, off, kWave);
    }
    return (uint64_t(hi) << 32) | lo;
}

template <int DT, bool NT>
__global__ __launch_bounds__(256) void k_combine_partial(const uint4 *__restrict__ y_disp,
                                                         const int *__restrict__ pair_slot,
                                                         const float *__restrict__ topk_w, int T,
                                                         int k, int rc, int n_dst, int cap,
                                                         uint4 *__restrict__ partial) {
    constexpr int VN = Vec<DT>::N;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave0 = __builtin_amdgcn_readfirstlane((blockIdx.x * blockDim.x + threadIdx.x) / kWave);
    const int nwaves = gridDim.x * blockDim.x / kWave;
    const int rows_total = n_dst * cap;
    for (int t = wave0; t < T; t += nwaves) {
        const int my_s = lane < k ? pair_slot[size_t(t) * k + lane] : -1;
        const bool ok = my_s >= 0 && my_s < rows_total;
        const int my_r = ok ? my_s / cap : -1;
        const float my_g = lane < k ? topk_w[size_t(t) * k + lane] : 0.0f;
        uint64_t dm = wave_or64(ok ? (uint64_t(1) << my_r) : 0);
        while (dm) {
            const int r = __builtin_ctzll(dm);
            dm &= dm - 1;
            // the pairs at r, j ascending (lanes whose destination is r)
            const uint64_t at_r = __ballot(ok && my_r == r);
            for (int c = lane; c < rc; c += kWave) {
                float acc[VN];
#pragma unroll
                for (int i = 0; i < VN; ++i) acc[i] = 0.0f;
                // eight of those rows' loads in flight together, then their terms in j order
                uint64_t pend = at_r;
                while (pend) {
                    uint4 v[8];
                    int jj[8];
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        jj[u] = pend ? __builtin_ctzll(pend) : -1;
                        if (pend) pend &= pend - 1;
                        v[u] = make_uint4(0u, 0u, 0u, 0u);
                        if (jj[u] >= 0) {
                            const size_t o = size_t(__builtin_amdgcn_readlane(my_s, jj[u])) * rc + c;
                            if (NT)
                                v[u] = __builtin_bit_cast(uint4, __builtin_nontemporal_load(
                                    reinterpret_cast<const u32x4 *>(y_disp) + o));
                            else
                                v[u] = y_disp[o];
                        }
                    }
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        if (jj[u] < 0) continue;
                        const float g = __builtin_bit_cast(
                            float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_g), jj[u]));
                        float f[VN];
                        Vec<DT>::unpack(v[u], f);
#pragma unroll
                        for (int i = 0; i < VN; ++i) acc[i] = __builtin_fmaf(g, f[i], acc[i]);
                    }
                }
                partial[(size_t(r) * T + t) * rc + c] = Vec<DT>::pack(acc);
            }
        }
    }
}

// The sources' side: y[t] = sum over the destinations r holding rows of t, in ascending
// r, of partial[r*T + t] (float32 additions, one rounding).
template <int DT>
__global__ __launch_bounds__(256) void k_combine_partials(const uint4 *__restrict__ partial,
                                                          const int *__restrict__ pair_slot,
                                                          int T, int k, int rc, int n_dst,
                                                          int cap, uint4 *__restrict__ y) {
    constexpr int VN = Vec<DT>::N;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave0 = __builtin_amdgcn_readfirstlane((blockIdx.x * blockDim.x + threadIdx.x) / kWave);
    const int nwaves = gridDim.x * blockDim.x / kWave;
    const int rows_total = n_dst * cap;
    for (int t = wave0; t < T; t += nwaves) {
        const int my_s = lane < k ? pair_slot[size_t(t) * k + lane] : -1;
        const bool ok = my_s >= 0 && my_s < rows_total;
        const uint64_t dm0 = wave_or64(ok ? (uint64_t(1) << (my_s / cap)) : 0);
        for (int c = lane; c < rc; c += kWave) {
            float acc[VN];
#pragma unroll
            for (int i = 0; i < VN; ++i) acc[i] = 0.0f;
            // destinations ascending, four partial rows' loads in flight together
            uint64_t dm = dm0;
            while (dm) {
                uint4 v[4];
                bool use[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    use[u] = dm != 0;
                    v[u] = make_uint4(0u, 0u, 0u, 0u);
                    if (use[u]) {
                        const int r = __builtin_ctzll(dm);
                        dm &= dm - 1;
                        v[u] = partial[(size_t(r) * T + t) * rc + c];
                    }
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    if (!use[u]) continue;
                    float f[VN];
                    Vec<DT>::unpack(v[u], f);
#pragma unroll
                    for (int i = 0; i < VN; ++i) acc[i] += f[i];
                }
            }
            y[size_t(t) * rc + c] = Vec<DT>::pack(acc);
        }
    }
}

int row_grid(int64_t T) { return int(std::min<int64_t>(cdiv(T, 4), 8192)); }

}  // namespace
}  // namespace moe

using namespace moe;

namespace {
moe_status_t combine_impl(const void *y_disp, const int32_t *pair_slot, const float *topk_w,
                          int64_t T, int32_t k, int64_t d, int64_t rows_total, moe_dtype_t dtype,
                          const void *residual, void *y, void *stream) {
    if (!valid_dtype(dtype) || T < 0 || d <= 0 || k <= 0 || rows_total < 0)
        return MOE_ERR_INVALID_ARG;
    if (T > (int64_t(1) << 31) / 64 || k > kWave) return MOE_ERR_UNSUPPORTED;
    if (T == 0) return MOE_OK;
    if (!y_disp || !pair_slot || !topk_w || !y) return MOE_ERR_INVALID_ARG;
    const int64_t rowb = d * elt_size(dtype);
    if (rowb % 16 != 0 || !aligned16(y_disp) || !aligned16(y) || (residual && !aligned16(residual)))
        return MOE_ERR_ALIGN;
    const hipStream_t st = as_stream(stream);
    // Gathered rows that outgrow the 256 MB Infinity Cache are read non-temporally: they
    // arrive from HBM either way, and the hint keeps them from evicting lines that are
    // still of use (measured on the 384-expert layer, 0.94 GB of rows: 222 -> 200 us;
    // the 32-source EP combine, 470 MB: 138 -> 104 us).
    // Smaller ones are mostly still in the cache from the kernel that wrote them, where
    // the hint slows the reads (100 MB: 22.7 -> 24.7 us).
    const bool nt = size_t(T) * k * rowb > (size_t(256) << 20);
#define MOE_COMBINE_LAUNCH(DTV, NTV)                                                         \
    hipLaunchKernelGGL((k_combine<DTV, NTV>), dim3(row_grid(T)), dim3(256), 0, st,             \
                       static_cast<const uint4 *>(y_disp), pair_slot, topk_w, int(T), k,        \
                       int(rowb / 16), rows_total, static_cast<const uint4 *>(residual),        \
                       static_cast<uint4 *>(y))
    if (dtype == MOE_BF16) {
        if (nt) MOE_COMBINE_LAUNCH(MOE_BF16, true);
        else MOE_COMBINE_LAUNCH(MOE_BF16, false);
    } else {
        if (nt) MOE_COMBINE_LAUNCH(MOE_F32, true);
        else MOE_COMBINE_LAUNCH(MOE_F32, false);
    }
#undef MOE_COMBINE_LAUNCH
    return launch_status();
}
}  // namespace

extern "C" moe_status_t moe_combine(const void *y_disp, const int32_t *pair_slot,
                                    const float *topk_w, int64_t T, int32_t k, int64_t d,
                                    int64_t rows_total, moe_dtype_t dtype, void *y, void *stream) {
    return combine_impl(y_disp, pair_slot, topk_w, T, k, d, rows_total, dtype, nullptr, y, stream);
}

extern "C" moe_status_t moe_combine_add(const void *y_disp, const int32_t *pair_slot,
                                        const float *topk_w, int64_t T, int32_t k, int64_t d,
                                        int64_t rows_total, moe_dtype_t dtype, const void *residual,
                                        void *y, void *stream) {
    if (!residual) return MOE_ERR_INVALID_ARG;
    return combine_impl(y_disp, pair_slot, topk_w, T, k, d, rows_total, dtype, residual, y, stream);
}

extern "C" moe_status_t moe_combine_bwd(const void *dy, const void *y_disp,
                                        const int32_t *pair_slot, const float *topk_w, int64_t T,
                                        int32_t k, int64_t d, int64_t rows_total,
                                        moe_dtype_t dtype, void *dy_disp, float *dtopk_w,
                                        void *stream) {
    if (!valid_dtype(dtype) || T < 0 || d <= 0 || k <= 0 || rows_total < 0)
        return MOE_ERR_INVALID_ARG;
    if (k > 32 || T > (int64_t(1) << 31) / 64) return MOE_ERR_UNSUPPORTED;
    if (T == 0) return MOE_OK;
    if (!dy || !y_disp || !pair_slot || !topk_w || !dy_disp || !dtopk_w) return MOE_ERR_INVALID_ARG;
    const int64_t rowb = d * elt_size(dtype);
    if (rowb % 16 != 0 || !aligned16(dy) || !aligned16(y_disp) || !aligned16(dy_disp))
        return MOE_ERR_ALIGN;
    const hipStream_t st = as_stream(stream);
    if (dtype == MOE_BF16)
        hipLaunchKernelGGL(k_combine_bwd<MOE_BF16>, dim3(row_grid(T)), dim3(256), 0, st,
                           static_cast<const uint4 *>(dy), static_cast<const uint4 *>(y_disp),
                           pair_slot, topk_w, int(T), k, int(rowb / 16), rows_total,
                           static_cast<uint4 *>(dy_disp), dtopk_w);
    else
        hipLaunchKernelGGL(k_combine_bwd<MOE_F32>, dim3(row_grid(T)), dim3(256), 0, st,
                           static_cast<const uint4 *>(dy), static_cast<const uint4 *>(y_disp),
                           pair_slot, topk_w, int(T), k, int(rowb / 16), rows_total,
                           static_cast<uint4 *>(dy_disp), dtopk_w);
    return launch_status();
}

namespace {
moe_status_t check_partial(const void *a, const int32_t *pair_slot, int64_t T, int32_t k,
                           int64_t d, int32_t n_dst, int64_t cap, moe_dtype_t dtype, const void *b) {
    if (!valid_dtype(dtype) || T < 0 || d <= 0 || k <= 0 || n_dst <= 0 || cap <= 0)
        return MOE_ERR_INVALID_ARG;
    if (n_dst > 64 || k > 64 || int64_t(n_dst) * cap >= (int64_t(1) << 31) ||
        int64_t(n_dst) * T >= (int64_t(1) << 31))
        return MOE_ERR_UNSUPPORTED;
    if (T == 0) return MOE_OK;
    if (!a || !pair_slot || !b) return MOE_ERR_INVALID_ARG;
    if ((d * elt_size(dtype)) % 16 != 0 || !aligned16(a) || !aligned16(b)) return MOE_ERR_ALIGN;
    return MOE_OK;
}
}  // namespace

extern "C" moe_status_t moe_combine_partial(const void *y_disp, const int32_t *pair_slot,
                                            const float *topk_w, int64_t T, int32_t k, int64_t d,
                                            int32_t n_dst, int64_t cap, moe_dtype_t dtype,
                                            void *partial, void *stream) {
    const moe_status_t c = check_partial(y_disp, pair_slot, T, k, d, n_dst, cap, dtype, partial);
    if (c != MOE_OK || T == 0) return c;
    if (!topk_w) return MOE_ERR_INVALID_ARG;
    const int rc = int(d * elt_size(dtype) / 16);
    const hipStream_t st = as_stream(stream);
    // the gathered rows' cache policy as in the combine
    const bool nt = size_t(T) * k * rc * 16 > (size_t(256) << 20);
#define MOE_PARTIAL_LAUNCH(DTV, NTV)                                                          \
    hipLaunchKernelGGL((k_combine_partial<DTV, NTV>), dim3(row_grid(T)), dim3(256), 0, st,      \
                       static_cast<const uint4 *>(y_disp), pair_slot, topk_w, int(T), k, rc,     \
                       n_dst, int(cap), static_cast<uint4 *>(partial))
    if (dtype == MOE_BF16) {
        if (nt) MOE_PARTIAL_LAUNCH(MOE_BF16, true);
        else MOE_PARTIAL_LAUNCH(MOE_BF16, false);
    } else {
        if (nt) MOE_PARTIAL_LAUNCH(MOE_F32, true);
        else MOE_PARTIAL_LAUNCH(MOE_F32, false);
    }
#undef MOE_PARTIAL_LAUNCH
    return launch_status();
}

extern "C" moe_status_t moe_combine_partials(const void *partial, const int32_t *pair_slot,
                                             int64_t T, int32_t k, int64_t d, int32_t n_dst,
                                             int64_t cap, moe_dtype_t dtype, void *y, void *stream) {
    const moe_status_t c = check_partial(partial, pair_slot, T, k, d, n_dst, cap, dtype, y);
    if (c != MOE_OK || T == 0) return c;
    const int rc = int(d * elt_size(dtype) / 16);
    const hipStream_t st = as_stream(stream);
    if (dtype == MOE_BF16)
        hipLaunchKernelGGL(k_combine_partials<MOE_BF16>, dim3(row_grid(T)), dim3(256), 0, st,
                           static_cast<const uint4 *>(partial), pair_slot, int(T), k, rc, n_dst,
                           int(cap), static_cast<uint4 *>(y));
    else
        hipLaunchKernelGGL(k_combine_partials<MOE_F32>, dim3(row_grid(T)), dim3(256), 0, st,
                           static_cast<const uint4 *>(partial), pair_slot, int(T), k, rc, n_dst,
                           int(cap), static_cast<uint4 *>(y));
    return launch_status();
}
