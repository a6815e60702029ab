// Router: logits in the canonical float32 order, top-k selection by wavefront
// shuffles, softmax gates. [EFA] = Perplexity, "Enabling trillion-parameter models
// on AWS EFA" (2025): a small linear routing layer picks the experts of each token
// (Introduction); each token goes to R of E experts (Send and receive buffers).
//
// Logits: acc = fmaf(x[t,i], w[e,i], acc) for i = 0..d-1 from +0, float32. The
// integer routing decision depends on these bits, so the order is fixed; that keeps
// the contraction on the vector ALU (matrix cores accumulate in their own order).
// The kernel is an LDS-tiled register-blocked product: a workgroup owns TT tokens and
// all (padded) experts, each thread TM tokens x TE experts whose accumulation chains
// each run over i in order. Top-k then runs on the logits tile held in LDS.
#include "common.h"

namespace moe {
namespace {

constexpr int kRouteBK = 32;      // input elements per LDS stage
constexpr int kRouteThreads = 256;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <int DT, int TM, int TE>
__global__ __launch_bounds__(kRouteThreads) void k_router_topk(
    const void *__restrict__ xv, const void *__restrict__ wv, int T, int d, int E, int k,
    int full_softmax, float *__restrict__ logits, int *__restrict__ topk_idx,
    float *__restrict__ topk_w) {
    constexpr int TT = 8 * TM;            // tokens per workgroup
    constexpr int EP = 32 * TE;           // experts, padded to the thread grid
    constexpr int BK = kRouteBK;
    constexpr int SX = TT + 4;            // LDS row stride of the x tile (k-major)
    constexpr int SW = EP + 2;            // LDS row stride of the w tile (k-major)
    constexpr int SL = EP + 1;            // LDS row stride of the logits tile
    constexpr int VN = Vec<DT>::N;        // elements per 16-byte chunk
    constexpr int CH = BK / VN;           // chunks per tile row
    constexpr int NV = (EP + kWave - 1) / kWave;
    constexpr int NXC = (TT * CH + kRouteThreads - 1) / kRouteThreads;   // x chunks per thread
    constexpr int NWC = (EP * CH + kRouteThreads - 1) / kRouteThreads;   // w chunks per thread
    static_assert(TT * SL <= BK * SW, "logits tile must fit in the w staging area");
    static_assert(NV <= 32, "experts per lane");

    __shared__ __align__(16) float xs[BK * SX];
    __shared__ __align__(16) float wsm[BK * SW];

    const int tid = threadIdx.x;
    const int eg = tid & 31;              // expert group: experts eg, eg+32, ...
    const int tg = tid >> 5;              // token group: tokens tg*TM .. tg*TM+TM-1
    const int t0 = blockIdx.x * TT;
    const int esz = (DT == MOE_BF16) ? 2 : 4;
    const size_t rowb = size_t(d) * esz;
    const char *xb = static_cast<const char *>(xv);
    const char *wb = static_cast<const char *>(wv);

    float acc[TM][TE];
#pragma unroll
    for (int m = 0; m < TM; ++m)
#pragma unroll
        for (int q = 0; q < TE; ++q) acc[m][q] = 0.0f;

    // Next stage's chunks are fetched into registers while the current stage is
    // consumed from LDS (elements past T, E or d read as zero; they never reach an
    // output: padded experts and tokens are dropped, and the last stage stops at d).
    u32x4 rx[NXC], rw[NWC];
    auto fetch = [&](int k0) {
#pragma unroll
        for (int j = 0; j < NXC; ++j) {
            const int c = tid + j * kRouteThreads;
            const int r = c / CH, kk = k0 + (c % CH) * VN;
            rx[j] = (c < TT * CH && t0 + r < T && kk < d)
                        ? *reinterpret_cast<const u32x4 *>(xb + size_t(t0 + r) * rowb + size_t(kk) * esz)
                        : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int j = 0; j < NWC; ++j) {
            const int c = tid + j * kRouteThreads;
            const int e = c / CH, kk = k0 + (c % CH) * VN;
            rw[j] = (c < EP * CH && e < E && kk < d)
                        ? *reinterpret_cast<const u32x4 *>(wb + size_t(e) * rowb + size_t(kk) * esz)
                        : u32x4{0u, 0u, 0u, 0u};
        }
    };
    auto stage = [&]() {
#pragma unroll
        for (int j = 0; j < NXC; ++j) {
            const int c = tid + j * kRouteThreads;
            if (c < TT * CH) {
                const int r = c / CH, kc = c % CH;
                float f[VN];
                Vec<DT>::unpack(make_uint4(rx[j].x, rx[j].y, rx[j].z, rx[j].w), f);
#pragma unroll
                for (int i = 0; i < VN; ++i) xs[(kc * VN + i) * SX + r] = f[i];
            }
        }
#pragma unroll
        for (int j = 0; j < NWC; ++j) {
            const int c = tid + j * kRouteThreads;
            if (c < EP * CH) {
                const int e = c / CH, kc = c % CH;
                float f[VN];
                Vec<DT>::unpack(make_uint4(rw[j].x, rw[j].y, rw[j].z, rw[j].w), f);
#pragma unroll
                for (int i = 0; i < VN; ++i) wsm[(kc * VN + i) * SW + e] = f[i];
            }
        }
    };

    fetch(0);
    stage();
    __syncthreads();
    for (int k0 = 0; k0 < d; k0 += BK) {
        const bool more = k0 + BK < d;
        if (more) fetch(k0 + BK);
        auto step = [&](int kk) {
            float xr[TM], wr[TE];
#pragma unroll
            for (int m = 0; m < TM; ++m) xr[m] = xs[kk * SX + tg * TM + m];
#pragma unroll
            for (int q = 0; q < TE; ++q) wr[q] = wsm[kk * SW + q * 32 + eg];
#pragma unroll
            for (int m = 0; m < TM; ++m)
#pragma unroll
                for (int q = 0; q < TE; ++q) acc[m][q] = __builtin_fmaf(xr[m], wr[q], acc[m][q]);
        };
        if (k0 + BK <= d) {
#pragma unroll 8
            for (int kk = 0; kk < BK; ++kk) step(kk);
        } else {
            // last, partial stage: the chain stops exactly at i = d-1
            for (int kk = 0; kk < d - k0; ++kk) step(kk);
        }
        __syncthreads();
        if (more) {
            stage();
            __syncthreads();
        }
    }

    // logits tile -> LDS (reusing the w staging area)
    float *lg = wsm;
#pragma unroll
    for (int m = 0; m < TM; ++m)
#pragma unroll
        for (int q = 0; q < TE; ++q) lg[(tg * TM + m) * SL + q * 32 + eg] = acc[m][q];
    __syncthreads();

    if (logits != nullptr) {
        for (int c = tid; c < TT * E; c += kRouteThreads) {
            const int r = c / E, e = c % E;
            if (t0 + r < T) logits[size_t(t0 + r) * E + e] = lg[r * SL + e];
        }
    }

    // top-k: one wavefront per token. Lane l holds experts l, l+64, ...
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    for (int r = wave; r < TT; r += kRouteThreads / kWave) {
        const int t = t0 + r;
        if (t >= T) break;
        float v[NV];
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int e = lane + i * kWave;
            v[i] = (e < E) ? lg[r * SL + e] : 0.0f;
        }
        uint32_t taken = 0;
        int my_idx = 0;
        float my_v = 0.0f;
        for (int j = 0; j < k; ++j) {
            float bv = 0.0f;
            int bi = 0x7fffffff;           // "none"
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                const int e = lane + i * kWave;
                // ascending e and strict '>' keep the lower id on ties
                if (e < E && !((taken >> i) & 1u) && (bi == 0x7fffffff || v[i] > bv)) {
                    bv = v[i];
                    bi = e;
                }
            }
#pragma unroll
            for (int off = kWave / 2; off > 0; off >>= 1) {
                const float ov = __shfl_xor(bv, off, kWave);
                const int oi = __shfl_xor(bi, off, kWave);
                if (oi != 0x7fffffff &&
                    (bi == 0x7fffffff || ov > bv || (ov == bv && oi < bi))) {
                    bv = ov;
                    bi = oi;
                }
            }
            if (lane == j) {
                my_idx = bi;
                my_v = bv;
            }
            if ((bi & (kWave - 1)) == lane) taken |= 1u << (bi / kWave);
        }
        const float vmax = __shfl(my_v, 0, kWave);   // the first pick is the largest
        float z, s;
        if (!full_softmax) {
            z = (lane < k) ? expf(my_v - vmax) : 0.0f;
            s = z;
        } else {
            z = (lane < k) ? expf(my_v - vmax) : 0.0f;
            s = 0.0f;
#pragma unroll
            for (int i = 0; i < NV; ++i)
                if (lane + i * kWave < E) s += expf(v[i] - vmax);
        }
#pragma unroll
        for (int off = kWave / 2; off > 0; off >>= 1) s += __shfl_xor(s, off, kWave);
        if (lane < k) {
            topk_idx[size_t(t) * k + lane] = my_idx;
            topk_w[size_t(t) * k + lane] = z / s;
        }
    }
}

template <int DT, int TM>
moe_status_t launch_route_tm(const void *x, const void *w, int T, int d, int E, int k, int full,
                             float *logits, int *idx, float *gw, hipStream_t st) {
    const int te = int(cdiv(E, 32));
    const dim3 grid(unsigned(cdiv(T, 8 * TM)));
#define MOE_ROUTE_CASE(TEV)                                                                 \
    if (te <= TEV) {                                                                        \
        hipLaunchKernelGGL((k_router_topk<DT, TM, TEV>), grid, dim3(kRouteThreads), 0, st, x, \
                           w, T, d, E, k, full, logits, idx, gw);                           \
        return launch_status();                                                             \
    }
    MOE_ROUTE_CASE(1)
    MOE_ROUTE_CASE(2)
    MOE_ROUTE_CASE(4)
    MOE_ROUTE_CASE(8)
    MOE_ROUTE_CASE(12)
    MOE_ROUTE_CASE(16)
#undef MOE_ROUTE_CASE
    return MOE_ERR_UNSUPPORTED;
}

template <int DT>
moe_status_t launch_route(const void *x, const void *w, int T, int d, int E, int k, int full,
                          float *logits, int *idx, float *gw, hipStream_t st) {
    // 32 tokens per workgroup once that still gives one workgroup per CU, else 16
    if (cdiv(T, 32) >= 256) return launch_route_tm<DT, 4>(x, w, T, d, E, k, full, logits, idx, gw, st);
    return launch_route_tm<DT, 2>(x, w, T, d, E, k, full, logits, idx, gw, st);
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" moe_status_t moe_route(const void *x, const void *w_router, int64_t T, int64_t d,
                                  int32_t E, int32_t k, moe_dtype_t dtype, int32_t flags,
                                  float *logits, int32_t *topk_idx, float *topk_w, void *stream) {
    if (!valid_dtype(dtype) || (flags != MOE_ROUTE_RENORM && flags != MOE_ROUTE_FULL_SOFTMAX))
        return MOE_ERR_INVALID_ARG;
    if (T < 0 || d <= 0 || E <= 0 || k <= 0) return MOE_ERR_INVALID_ARG;
    if (k > E) return MOE_ERR_SHAPE;
    if (k > 32 || E > 512 || T > (int64_t(1) << 31) / 64 || d > (int64_t(1) << 30))
        return MOE_ERR_UNSUPPORTED;
    if (T == 0) return MOE_OK;
    if (!x || !w_router || !topk_idx || !topk_w) return MOE_ERR_INVALID_ARG;
    if ((d * elt_size(dtype)) % 16 != 0 || !aligned16(x) || !aligned16(w_router))
        return MOE_ERR_ALIGN;
    const hipStream_t st = as_stream(stream);
    if (dtype == MOE_BF16)
        return launch_route<MOE_BF16>(x, w_router, int(T), int(d), E, k, flags, logits, topk_idx,
                                      topk_w, st);
    return launch_route<MOE_F32>(x, w_router, int(T), int(d), E, k, flags, logits, topk_idx,
                                 topk_w, st);
}
