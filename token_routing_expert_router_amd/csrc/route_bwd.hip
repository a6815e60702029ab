// Backward of the router: the softmax-over-top-k Jacobian and the router weights'
// gradient. With g the k gates of a token and dg their upstream gradient,
//   dl_j = g_j (dg_j - sum_i g_i dg_i)          (selected logits; others get none:
//                                                the top-k choice is piecewise constant)
//   dWr[e,:] = sum over pairs (t, j) routed to e of dl[t,j] * x[t,:]
// The second sum runs over expert e's rows of the expert-major plan, i.e. over its
// tokens, in one fixed order (eight interleaved float32 partial sums, see below).
#include "common.h"

#include <algorithm>

namespace moe {
namespace {

__global__ void k_route_bwd_sel(const float *__restrict__ g, const float *__restrict__ dg, int T,
                                int k, float *__restrict__ dl) {
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= T) return;
    const float *gt = g + size_t(t) * k;
    const float *dgt = dg + size_t(t) * k;
    float s = 0.0f;
    for (int j = 0; j < k; ++j) s = __builtin_fmaf(gt[j], dgt[j], s);
    for (int j = 0; j < k; ++j) dl[size_t(t) * k + j] = gt[j] * (dgt[j] - s);
}

// dw = 0 (the router gradient of an empty batch: there is no plan to read).
__global__ __launch_bounds__(256) void k_zero_f32(float4 *__restrict__ p, int64_t n4) {
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n4;
         i += int64_t(gridDim.x) * blockDim.x)
        p[i] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
}

// One workgroup per (expert, 32 16-byte chunks of the row). Its 256 threads are 8 row
// groups x 32 chunks: group g sums the expert's rows r0 + g, r0 + g + 8, ... in
// ascending order, and the 8 partial sums are then added in group order. The order is
// fixed, so the result is bitwise reproducible.
constexpr int kRbGroups = 8, kRbChunks = 32;
template <int DT>
__global__ __launch_bounds__(256) void k_route_bwd_w(const uint4 *__restrict__ x,
                                                     const float *__restrict__ dl,
                                                     const int *__restrict__ expert_off,
                                                     const int *__restrict__ row_pair, int k,
                                                     int rc, float *__restrict__ dw) {
    constexpr int VN = Vec<DT>::N;
    __shared__ float part[kRbGroups][kRbChunks][VN + 1];
    const int e = blockIdx.x;
    const int lc = threadIdx.x % kRbChunks, g = threadIdx.x / kRbChunks;
    const int c = blockIdx.y * kRbChunks + lc;
    const bool live = c < rc;
    const int r0 = expert_off[e], r1 = expert_off[e + 1];
    float acc[VN];
#pragma unroll
    for (int i = 0; i < VN; ++i) acc[i] = 0.0f;
    int r = r0 + g;
    // four rows of this group in flight per step
    for (; r + 3 * kRbGroups < r1; r += 4 * kRbGroups) {
        int p[4];
        float w[4];
        uint4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) p[u] = row_pair[r + u * kRbGroups];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int q = p[u] < 0 ? 0 : p[u];
            w[u] = p[u] < 0 ? 0.0f : dl[q];
            v[u] = live ? x[size_t(q / k) * rc + c] : uint4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (p[u] < 0) continue;
            float f[VN];
            Vec<DT>::unpack(v[u], f);
#pragma unroll
            for (int i = 0; i < VN; ++i) acc[i] = __builtin_fmaf(w[u], f[i], acc[i]);
        }
    }
    for (; r < r1; r += kRbGroups) {
        const int p = row_pair[r];
        if (p < 0 || !live) continue;
        float f[VN];
        Vec<DT>::unpack(x[size_t(p / k) * rc + c], f);
        const float w = dl[p];
#pragma unroll
        for (int i = 0; i < VN; ++i) acc[i] = __builtin_fmaf(w, f[i], acc[i]);
    }
#pragma unroll
    for (int i = 0; i < VN; ++i) part[g][lc][i] = acc[i];
    __syncthreads();
    if (g != 0 || !live) return;
#pragma unroll
    for (int i = 0; i < VN; ++i) acc[i] = part[0][lc][i];
    for (int h = 1; h < kRbGroups; ++h)
#pragma unroll
        for (int i = 0; i < VN; ++i) acc[i] += part[h][lc][i];
    float4 *out = reinterpret_cast<float4 *>(dw + size_t(e) * rc * VN + size_t(c) * VN);
#pragma unroll
    for (int i = 0; i < VN; i += 4) out[i / 4] = make_float4(acc[i], acc[i + 1], acc[i + 2], acc[i + 3]);
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" moe_status_t moe_route_bwd(const void *x, const int32_t *topk_idx, const float *topk_w,
                                      const float *dtopk_w, const int32_t *expert_off,
                                      const int32_t *row_pair, int64_t T, int64_t d, int32_t E,
                                      int32_t k, moe_dtype_t dtype, float *dlogits_sel,
                                      float *dw_router, void *stream) {
    if (!valid_dtype(dtype) || T < 0 || d <= 0 || E <= 0 || k <= 0) return MOE_ERR_INVALID_ARG;
    if (k > E) return MOE_ERR_SHAPE;
    if (E > 65535 || T * k >= (int64_t(1) << 31) || d > (int64_t(1) << 24)) return MOE_ERR_UNSUPPORTED;
    const int64_t rowb = d * elt_size(dtype);
    const hipStream_t st = as_stream(stream);
    if (T == 0) {
        // an empty batch: dw_router = 0, and nothing of the plan or x is read
        if (!dw_router) return MOE_ERR_INVALID_ARG;
        if (rowb % 16 != 0 || !aligned16(dw_router)) return MOE_ERR_ALIGN;
        const int64_t n4 = int64_t(E) * d / 4;      // d * 4 bytes % 16 == 0 by the check above
        hipLaunchKernelGGL(k_zero_f32, dim3(unsigned(std::min<int64_t>(cdiv(n4, 256), 4096))),
                           dim3(256), 0, st, reinterpret_cast<float4 *>(dw_router), n4);
        return launch_status();
    }
    if (!x || !topk_idx || !topk_w || !dtopk_w || !expert_off || !row_pair || !dlogits_sel ||
        !dw_router)
        return MOE_ERR_INVALID_ARG;
    if (rowb % 16 != 0 || !aligned16(x) || !aligned16(dw_router)) return MOE_ERR_ALIGN;
    hipLaunchKernelGGL(k_route_bwd_sel, dim3(unsigned(cdiv(T, 256))), dim3(256), 0, st, topk_w,
                       dtopk_w, int(T), k, dlogits_sel);
    const int rc = int(rowb / 16);
    const dim3 grid(unsigned(E), unsigned(cdiv(rc, kRbChunks)));
    if (dtype == MOE_BF16)
        hipLaunchKernelGGL(k_route_bwd_w<MOE_BF16>, grid, dim3(256), 0, st,
                           static_cast<const uint4 *>(x), dlogits_sel, expert_off, row_pair, k, rc,
                           dw_router);
    else
        hipLaunchKernelGGL(k_route_bwd_w<MOE_F32>, grid, dim3(256), 0, st,
                           static_cast<const uint4 *>(x), dlogits_sel, expert_off, row_pair, k, rc,
                           dw_router);
    return launch_status();
}
