// Router: logits in the canonical float32 order, top-k selection by wavefront
// shuffles, softmax gates. [EFA] = Perplexity, "Enabling trillion-parameter models
// on AWS EFA" (2025): a small linear routing layer picks the experts of each token
// (Introduction); each token goes to R of E experts (Send and receive buffers).
//
// Logits: acc = fmaf(x[t,i], w[e,i], acc) for i = 0..d-1 from +0, float32. The
// integer routing decision depends on these bits, so the order is fixed: every
// output is one chain of d dependent multiply-adds, never split or reassociated.
//
// bf16 path (matrix cores): a product of two bf16 values is exact in float32 (8-bit
// significands), so one float32 outer-product step D = C + a*b of
// v_mfma_f32_4x4x1_16b_f32 (sixteen 4x4 blocks, one product per output) rounds
// exactly as fmaf(a, b, C) does. Chaining those steps over i = 0..d-1 gives the
// canonical logits bit for bit, with the multiply-adds on the matrix cores at twice
// the vector-ALU rate. Up to 64 experts, 16-token x 16-expert chains on the 4x4x1
// form, four per workgroup (one per SIMD); above 64, 16-token x 64-expert chains on
// v_mfma_f32_16x16x1_4b_f32 (the same single-rounding step, four times the products
// per operand byte), 32 tokens per workgroup.
// float32 path (vector ALU): products are not exact there, so the chains run as
// v_fma_f32 in an LDS-tiled register-blocked kernel: a workgroup owns TT tokens and all
// (padded) experts, each thread TM tokens x TE experts.
// Both paths then run top-k on the workgroup's logits tile in LDS.
#include "common.h"

#include <algorithm>
#include <mutex>

namespace moe {
namespace {

constexpr int kRouteBK = 32;      // input elements per LDS stage
constexpr int kRouteThreads = 256;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Top-k and gates of the workgroup's rows of the logits tile lg[rows][SL] (LDS), one
// wavefront per row; lane l holds experts l, l+64, ... (NV candidates per lane).
template <int NV>
__device__ __forceinline__ void topk_rows(const float *lg, int SL, int rows, int t0, int T, int E,
                                          int k, int full_softmax, int *__restrict__ topk_idx,
                                          float *__restrict__ topk_w, int wave, int lane,
                                          int nwaves) {
    for (int r = wave; r < rows; r += nwaves) {
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

    topk_rows<NV>(lg, SL, TT, t0, T, E, k, full_softmax, topk_idx, topk_w, tid / kWave,
              tid & (kWave - 1), kRouteThreads / kWave);
}

// ---------------------------------------------------------------- bf16 matrix-core path
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kRouteTT = 16;          // tokens per workgroup of the matrix-core path

// Chain c of wave v covers tokens t0..t0+15 and experts e = 16*(NCH*v + c) .. +15.
// MFMA 4x4x1_16b lane layout (block b = l >> 2): lane l supplies operand A of block b,
// row l & 3, and operand B of block b, column l & 3; result register q of lane l is
// block b, row q, column l & 3. Blocks are laid out as 4 token groups x 4 expert groups
// (b = 4 * (l >> 4) + ((l >> 2) & 3)), so lane l feeds token t0 + 4*(l >> 4) + (l & 3)
// and expert e + (l & 15), and ends holding the logits of tokens t0 + 4*(l >> 4) + q
// for expert e + (l & 15).
// Operands are staged in LDS as float32, BK elements of every row per stage (each
// value widened once per workgroup: a vector-ALU op costs the matrix pipe about as
// much as a step), and read 4 steps at a time; the raw bf16 rows of the next four
// stages are in flight in registers meanwhile. Elements past the row end stage as
// zeros: adding the product +0 leaves an accumulator unchanged (it is never -0: it
// starts at +0 and round-to-nearest-even turns exact cancellation into +0), so every
// chain is exactly the d-step chain.
template <int NCH, int NV, int BK, int CPTW>
__global__ __launch_bounds__(512) void k_router_mfma(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ w, int T, int d, int E, int k,
    int full_softmax, float *__restrict__ logits, int *__restrict__ topk_idx,
    float *__restrict__ topk_w) {
    constexpr int XP = BK + 4;                        // LDS row pitch (floats)
    constexpr int CPR = BK / 8;                       // 16-byte chunks per row and stage
    constexpr int PF = 4;                             // stages of raw rows in flight
    constexpr int NL = 1 + CPTW;                      // loads per thread and stage
    extern __shared__ __align__(16) float smem[];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int nthreads = int(blockDim.x);
    const int nwaves = nthreads / kWave;
    const int ep = 16 * NCH * nwaves;                 // padded experts of the workgroup
    const int rows = kRouteTT + ep;                   // staged rows: tokens, then experts
    const int stage_floats = rows * XP;
    const int t0 = blockIdx.x * kRouteTT;

    // Chunk = 8 elements of one row. Load 0 of a thread is token chunk tid % (16*CPR)
    // (staged by threads < 16*CPR only); loads 1.. are expert chunks tid + j*nthreads
    // (the host makes ep*CPR == CPTW*nthreads). Buffer loads: per-chunk row offset in
    // the lane, stage offset uniform; a read past a row end lands in the next row (or
    // reads zeros past the buffer) and is zeroed when staged.
    const int xc = tid % (kRouteTT * CPR);
    const bool xown = tid < kRouteTT * CPR;
    const int64_t xrem = (int64_t(T) - t0) * d * 2;   // bytes from the tile's first row on
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(x + size_t(t0) * d), 0, int(xrem < 0x7fffffff ? xrem : 0x7fffffff), 0x00020000);
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(w), 0, int(int64_t(E) * d * 2), 0x00020000);
    uint32_t voff[NL];
    int lofs[NL], coff[NL];
    {
        const int r = xc / CPR;
        coff[0] = 8 * (xc % CPR);
        voff[0] = uint32_t((min(t0 + r, T - 1) - t0) * d + coff[0]) * 2u;
        lofs[0] = r * XP + coff[0];
    }
#pragma unroll
    for (int j = 0; j < CPTW; ++j) {
        const int c = tid + j * nthreads;
        const int r = c / CPR;
        coff[1 + j] = 8 * (c % CPR);
        voff[1 + j] = uint32_t(min(r, E - 1) * d + coff[1 + j]) * 2u;
        lofs[1 + j] = (kRouteTT + r) * XP + coff[1 + j];
    }
    uint4 raw[PF][NL];
    auto fetch = [&](int sidx, uint4 (&dst)[NL]) {
        const int so = sidx * BK * 2;
        dst[0] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, voff[0], so, 0));
#pragma unroll
        for (int j = 1; j < NL; ++j)
            dst[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rw, voff[j], so, 0));
    };
    auto cvt_store = [&](float *buf, int lo, uint4 u) {
        float4 *dst = reinterpret_cast<float4 *>(buf + lo);
        dst[0] = make_float4(bf16_lo(u.x), bf16_hi(u.x), bf16_lo(u.y), bf16_hi(u.y));
        dst[1] = make_float4(bf16_lo(u.z), bf16_hi(u.z), bf16_lo(u.w), bf16_hi(u.w));
    };
    auto stage = [&](int sidx, const uint4 (&v)[NL], float *buf) {
        const uint4 z = make_uint4(0u, 0u, 0u, 0u);
        if ((sidx + 1) * BK <= d) {                    // the whole stage is inside the rows
            if (xown) cvt_store(buf, lofs[0], v[0]);
#pragma unroll
            for (int j = 1; j < NL; ++j) cvt_store(buf, lofs[j], v[j]);
        } else {
            if (xown) cvt_store(buf, lofs[0], sidx * BK + coff[0] < d ? v[0] : z);
#pragma unroll
            for (int j = 1; j < NL; ++j) cvt_store(buf, lofs[j], sidx * BK + coff[j] < d ? v[j] : z);
        }
    };

    const int arow = 4 * (lane >> 4) + (lane & 3);
    int brow[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) brow[c] = kRouteTT + 16 * (NCH * wave + c) + (lane & 15);

    f32x4 acc[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) acc[c] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    // stages rounded up to a multiple of PF: the extra stages are all zeros (no-op
    // steps), which keeps the loop body free of conditions and every wait exact
    const int nst = (d + BK * PF - 1) / (BK * PF) * PF;
#pragma unroll
    for (int p = 0; p < PF; ++p) fetch(p, raw[p]);
    stage(0, raw[0], smem);
    fetch(PF, raw[0]);
    __syncthreads();
    // stage s: the chains consume LDS buffer s & 1; raw slot (s+1) % PF is widened into
    // the other buffer and refilled with stage s+1+PF
    for (int s0 = 0; s0 < nst; s0 += PF) {
#pragma unroll
        for (int u = 0; u < PF; ++u) {
            const int s = s0 + u;
            const float *cur = smem + (s & 1) * stage_floats;
            // operands of group g (4 steps) are read RA groups ahead of its MFMAs
            constexpr int NG = BK / 4, RA = NG < 4 ? NG : 4;
            f32x4 a[RA], b[RA][NCH];
            auto rd = [&](int g, f32x4 &ar, f32x4 (&br)[NCH]) {
                ar = *reinterpret_cast<const f32x4 *>(cur + arow * XP + 4 * g);
#pragma unroll
                for (int c = 0; c < NCH; ++c) br[c] = *reinterpret_cast<const f32x4 *>(cur + brow[c] * XP + 4 * g);
            };
#pragma unroll
            for (int g = 0; g < RA; ++g) rd(g, a[g], b[g]);
            __builtin_amdgcn_sched_barrier(0);
            // (scheduling barriers keep every read RA groups ahead of its use)
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                const f32x4 ag = a[g % RA];
                f32x4 bg[NCH];
#pragma unroll
                for (int c = 0; c < NCH; ++c) bg[c] = b[g % RA][c];
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int c = 0; c < NCH; ++c)
                        acc[c] = __builtin_amdgcn_mfma_f32_4x4x1f32(ag[q], bg[c][q], acc[c], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
                if (g + RA < NG) rd(g + RA, a[g % RA], b[g % RA]);
                __builtin_amdgcn_sched_barrier(0);
            }
            stage(s + 1, raw[(u + 1) % PF], smem + ((s + 1) & 1) * stage_floats);
            __builtin_amdgcn_sched_barrier(0);   // the loads keep their place in issue order
            fetch(s + 1 + PF, raw[(u + 1) % PF]);
            __builtin_amdgcn_sched_barrier(0);
            __syncthreads();
        }
    }

    // logits tile -> LDS (the staging area is free after the last barrier)
    const int SL = ep + 1;
    float *lg = smem;
#pragma unroll
    for (int c = 0; c < NCH; ++c)
#pragma unroll
        for (int q = 0; q < 4; ++q)
            lg[(4 * (lane >> 4) + q) * SL + 16 * (NCH * wave + c) + (lane & 15)] = acc[c][q];
    __syncthreads();

    if (logits != nullptr) {
        for (int c = tid; c < kRouteTT * E; c += blockDim.x) {
            const int r = c / E, e = c % E;
            if (t0 + r < T) logits[size_t(t0 + r) * E + e] = lg[r * SL + e];
        }
    }
    topk_rows<NV>(lg, SL, kRouteTT, t0, T, E, k, full_softmax, topk_idx, topk_w, wave, lane,
                  nwaves);
}

template <int NCH, int NV, int BK, int CPTW>
moe_status_t launch_route_mfma_cfg(const uint16_t *x, const uint16_t *w, int T, int d, int E, int k,
                                   int full, float *logits, int *idx, float *gw, hipStream_t st,
                                   int nw) {
    const int ep = 16 * NCH * nw;
    // every thread owns CPTW expert chunks, the first 16*CPR threads one token chunk
    if (ep * (BK / 8) != CPTW * 64 * nw || kRouteTT * (BK / 8) > 64 * nw) return MOE_ERR_UNSUPPORTED;
    // buffer offsets are 32-bit: the expert rows below 2^31 bytes, 16 token rows plus a
    // stage offset well below 2^32
    if (int64_t(E) * d * 2 > 0x7fffffff || d > (1 << 26)) return MOE_ERR_UNSUPPORTED;
    const size_t stage = size_t(kRouteTT + ep) * (BK + 4) * sizeof(float);
    const size_t lds = std::max(2 * stage, size_t(kRouteTT) * (ep + 1) * sizeof(float));
    if (!lds_limit_once<&k_router_mfma<NCH, NV, BK, CPTW>>(160 * 1024)) return MOE_ERR_HIP;
    hipLaunchKernelGGL((k_router_mfma<NCH, NV, BK, CPTW>), dim3(unsigned(cdiv(T, kRouteTT))),
                       dim3(64 * nw), lds, st, x, w, T, d, E, k, full, logits, idx, gw);
    return launch_status();
}

// ---------------------------------------------------------------- 16x16x1 chains
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Workgroup: TT = 16*TG tokens x EP = 64*EG padded experts, TG*EG chains of 16
// tokens x 64 experts on v_mfma_f32_16x16x1_4b_f32 (four 16x16 blocks). Lane l
// supplies row l & 15 of block l >> 4 of both operands: operand A is token l & 15 of
// the chain's token group (the same 16 tokens in every block), operand B expert l of
// its 64. Result register r of lane l is token 4*(l >> 4) + (r & 3), expert
// 16*(r >> 2) + (l & 15). Waves 0..NMW-1 compute, NC chains each (one token group,
// so operand A is read once per step for all of them); the other waves stage: raw
// bf16 rows of the next four stages in flight in their registers, widened into the
// float32 LDS stage. The two roles run separate loops with the same barriers, so
// neither holds the other's registers. Padding, zero tail and the chain order are
// those of the 4x4x1 kernel above.
template <int TG, int EG, int NC, int BK, int NLW>
__global__ __launch_bounds__(512) void k_router_mfma16(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ w, int T, int d, int E, int k,
    int full_softmax, float *__restrict__ logits, int *__restrict__ topk_idx,
    float *__restrict__ topk_w) {
    constexpr int TT = 16 * TG, EP = 64 * EG;
    constexpr int XP = BK + 4;                        // LDS row pitch (floats)
    constexpr int CPR = BK / 8;                       // 16-byte chunks per row and stage
    constexpr int PF = 4;                             // stages of raw rows in flight
    constexpr int NL = 1 + NLW;                       // loads per staging thread and stage
    constexpr int NMW = TG * EG / NC;                 // computing waves
    constexpr int STAGE = (TT + EP) * XP;
    constexpr int SL = EP + 1;                        // logits tile row pitch
    static_assert(EG % NC == 0, "the chains of a wave share one token group");
    extern __shared__ __align__(16) float smem[];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int nthreads = int(blockDim.x);
    const int t0 = blockIdx.x * TT;
    // stages rounded up to a multiple of PF (the extra ones are zeros: no-op steps)
    const int nst = (d + BK * PF - 1) / (BK * PF) * PF;
    float *lg = smem;

    if (wave >= NMW) {
        // ---- staging: chunk = 8 elements of one row; load 0 of staging thread i is
        // token chunk i % (TT*CPR) (stored by i < TT*CPR), loads 1.. expert chunks
        // i + j*nstage (the host makes EP*CPR == NLW*nstage)
        const int sti = tid - NMW * kWave;
        const int nstage = nthreads - NMW * kWave;
        const int xc = sti % (TT * CPR);
        const bool xown = sti < TT * CPR;
        const int64_t xrem = (int64_t(T) - t0) * d * 2;
        const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t *>(x + size_t(t0) * d), 0, int(xrem < 0x7fffffff ? xrem : 0x7fffffff), 0x00020000);
        const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t *>(w), 0, int(int64_t(E) * d * 2), 0x00020000);
        uint32_t voff[NL];
        int lofs[NL], coff[NL];
        {
            const int r = xc / CPR;
            coff[0] = 8 * (xc % CPR);
            voff[0] = uint32_t((min(t0 + r, T - 1) - t0) * d + coff[0]) * 2u;
            lofs[0] = r * XP + coff[0];
        }
#pragma unroll
        for (int j = 0; j < NLW; ++j) {
            const int c = sti + j * nstage;
            const int r = c / CPR;
            coff[1 + j] = 8 * (c % CPR);
            voff[1 + j] = uint32_t(min(r, E - 1) * d + coff[1 + j]) * 2u;
            lofs[1 + j] = (TT + r) * XP + coff[1 + j];
        }
        uint4 raw[PF][NL];
        auto fetch = [&](int sidx, uint4 (&dst)[NL]) {
            const int so = sidx * BK * 2;
            dst[0] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, voff[0], so, 0));
#pragma unroll
            for (int j = 1; j < NL; ++j)
                dst[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rw, voff[j], so, 0));
        };
        auto cvt_store = [&](float *buf, int lo, uint4 u) {
            float4 *dst = reinterpret_cast<float4 *>(buf + lo);
            dst[0] = make_float4(bf16_lo(u.x), bf16_hi(u.x), bf16_lo(u.y), bf16_hi(u.y));
            dst[1] = make_float4(bf16_lo(u.z), bf16_hi(u.z), bf16_lo(u.w), bf16_hi(u.w));
        };
        auto stage = [&](int sidx, const uint4 (&v)[NL], float *buf) {
            const uint4 z = make_uint4(0u, 0u, 0u, 0u);
            if ((sidx + 1) * BK <= d) {
                if (xown) cvt_store(buf, lofs[0], v[0]);
#pragma unroll
                for (int j = 1; j < NL; ++j) cvt_store(buf, lofs[j], v[j]);
            } else {
                if (xown) cvt_store(buf, lofs[0], sidx * BK + coff[0] < d ? v[0] : z);
#pragma unroll
                for (int j = 1; j < NL; ++j) cvt_store(buf, lofs[j], sidx * BK + coff[j] < d ? v[j] : z);
            }
        };
#pragma unroll
        for (int p = 0; p < PF; ++p) fetch(p, raw[p]);
        stage(0, raw[0], smem);
        fetch(PF, raw[0]);
        __syncthreads();
        for (int s0 = 0; s0 < nst; s0 += PF) {
#pragma unroll
            for (int u = 0; u < PF; ++u) {
                const int s = s0 + u;
                stage(s + 1, raw[(u + 1) % PF], smem + ((s + 1) & 1) * STAGE);
                __builtin_amdgcn_sched_barrier(0);
                fetch(s + 1 + PF, raw[(u + 1) % PF]);
                __builtin_amdgcn_sched_barrier(0);
                __syncthreads();
            }
        }
    } else {
        // ---- chains
        const int tg = wave / (EG / NC);
        const int eg0 = (wave % (EG / NC)) * NC;
        const int arow = 16 * tg + (lane & 15);
        int brow[NC];
#pragma unroll
        for (int c = 0; c < NC; ++c) brow[c] = TT + 64 * (eg0 + c) + lane;
        f32x16 acc[NC];
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[c][r] = 0.0f;
        __syncthreads();
        for (int s0 = 0; s0 < nst; s0 += PF) {
#pragma unroll
            for (int u = 0; u < PF; ++u) {
                const float *cur = smem + ((s0 + u) & 1) * STAGE;
                // operands of group g (4 steps) are read RA groups ahead of its MFMAs
                constexpr int NG = BK / 4, RA = NG < 4 ? NG : 4;
                f32x4 a[RA], b[RA][NC];
                auto rd = [&](int g, f32x4 &ar, f32x4 (&br)[NC]) {
                    ar = *reinterpret_cast<const f32x4 *>(cur + arow * XP + 4 * g);
#pragma unroll
                    for (int c = 0; c < NC; ++c) br[c] = *reinterpret_cast<const f32x4 *>(cur + brow[c] * XP + 4 * g);
                };
#pragma unroll
                for (int g = 0; g < RA; ++g) rd(g, a[g], b[g]);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int g = 0; g < NG; ++g) {
                    const f32x4 ag = a[g % RA];
                    f32x4 bg[NC];
#pragma unroll
                    for (int c = 0; c < NC; ++c) bg[c] = b[g % RA][c];
#pragma unroll
                    for (int q = 0; q < 4; ++q)
#pragma unroll
                        for (int c = 0; c < NC; ++c)
                            acc[c] = __builtin_amdgcn_mfma_f32_16x16x1f32(ag[q], bg[c][q], acc[c], 0, 0, 0);
                    __builtin_amdgcn_sched_barrier(0);
                    if (g + RA < NG) rd(g + RA, a[g % RA], b[g % RA]);
                    __builtin_amdgcn_sched_barrier(0);
                }
                __syncthreads();
            }
        }
        // logits tile -> LDS (the staging area is free after the last barrier)
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                lg[(16 * tg + 4 * (lane >> 4) + (r & 3)) * SL + 64 * (eg0 + c) + 16 * (r >> 2) + (lane & 15)] =
                    acc[c][r];
    }
    __syncthreads();

    if (logits != nullptr) {
        for (int c = tid; c < TT * E; c += nthreads) {
            const int r = c / E, e = c % E;
            if (t0 + r < T) logits[size_t(t0 + r) * E + e] = lg[r * SL + e];
        }
    }
    topk_rows<EG>(lg, SL, TT, t0, T, E, k, full_softmax, topk_idx, topk_w, wave, lane,
                  nthreads / kWave);
}

template <int TG, int EG, int NC, int BK, int NLW>
moe_status_t launch_route16_cfg(const uint16_t *x, const uint16_t *w, int T, int d, int E, int k,
                                int full, float *logits, int *idx, float *gw, hipStream_t st,
                                int nw) {
    constexpr int TT = 16 * TG, EP = 64 * EG, NMW = TG * EG / NC;
    const int nstage = kWave * (nw - NMW);
    if (E > EP || nstage <= 0 || EP * (BK / 8) != NLW * nstage || TT * (BK / 8) > nstage)
        return MOE_ERR_UNSUPPORTED;
    if (int64_t(E) * d * 2 > 0x7fffffff || d > (1 << 26)) return MOE_ERR_UNSUPPORTED;
    const size_t stage = size_t(TT + EP) * (BK + 4) * sizeof(float);
    const size_t lds = std::max(2 * stage, size_t(TT) * (EP + 1) * sizeof(float));
    if (lds > 160 * 1024) return MOE_ERR_UNSUPPORTED;
    if (!lds_limit_once<&k_router_mfma16<TG, EG, NC, BK, NLW>>(160 * 1024)) return MOE_ERR_HIP;
    hipLaunchKernelGGL((k_router_mfma16<TG, EG, NC, BK, NLW>), dim3(unsigned(cdiv(T, TT))),
                       dim3(kWave * nw), lds, st, x, w, T, d, E, k, full, logits, idx, gw);
    return launch_status();
}

moe_status_t launch_route_mfma(const void *x, const void *w, int T, int d, int E, int k, int full,
                               float *logits, int *idx, float *gw, hipStream_t st) {
    const auto xb = static_cast<const uint16_t *>(x);
    const auto wb = static_cast<const uint16_t *>(w);
    // up to 64 experts: one 16 x 16 4x4x1 chain per wave, four waves, 128-deep stages
    // (a CU holds 16 x 64 outputs at 4096 tokens: one 16x16x1 chain would leave three
    // SIMDs idle)
    if (E <= 64)
        return launch_route_mfma_cfg<1, 1, 128, 4>(xb, wb, T, d, E, k, full, logits, idx, gw, st, 4);
    // above: 32 tokens x an even number of 64-expert groups, four computing waves of
    // EG/2 chains and four staging waves, 32-deep stages
    const int eg = int(cdiv(E, 64));
    if (eg <= 2) return launch_route16_cfg<2, 2, 1, 32, 2>(xb, wb, T, d, E, k, full, logits, idx, gw, st, 8);
    if (eg <= 4) return launch_route16_cfg<2, 4, 2, 32, 4>(xb, wb, T, d, E, k, full, logits, idx, gw, st, 8);
    if (eg <= 6) return launch_route16_cfg<2, 6, 3, 32, 6>(xb, wb, T, d, E, k, full, logits, idx, gw, st, 8);
    if (eg <= 8) return launch_route16_cfg<2, 8, 4, 32, 8>(xb, wb, T, d, E, k, full, logits, idx, gw, st, 8);
    // up to 1024 experts: 16 tokens per workgroup and 8-deep stages keep two float32
    // stages of 16 + 1024 rows (100 KiB) in LDS; four waves of four chains each
    return launch_route16_cfg<1, 16, 4, 8, 4>(xb, wb, T, d, E, k, full, logits, idx, gw, st, 8);
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
    // bf16 takes up to 1024 experts; the float32 kernel keeps its logits tile and the
    // expert rows of a stage in static LDS, which holds 512
    if (k > 32 || E > (dtype == MOE_BF16 ? 1024 : 512) || T > (int64_t(1) << 31) / 64 ||
        d > (int64_t(1) << 30))
        return MOE_ERR_UNSUPPORTED;
    if (T == 0) return MOE_OK;
    if (!x || !w_router || !topk_idx || !topk_w) return MOE_ERR_INVALID_ARG;
    if ((d * elt_size(dtype)) % 16 != 0 || !aligned16(x) || !aligned16(w_router))
        return MOE_ERR_ALIGN;
    const hipStream_t st = as_stream(stream);
    if (dtype == MOE_BF16)
        return launch_route_mfma(x, w_router, int(T), int(d), E, k, flags, logits, topk_idx, topk_w,
                                 st);
    return launch_route<MOE_F32>(x, w_router, int(T), int(d), E, k, flags, logits, topk_idx,
                                 topk_w, st);
}
