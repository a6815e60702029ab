// Expert FFN: the grouped GEMM that multiplies each expert's rows by that expert's
// SwiGLU weights. [EFA] = Perplexity, "Enabling trillion-parameter models on AWS EFA"
// (2025): after dispatch, grouped GEMM kernels multiply the tokens with the expert
// weights (MoE all-to-all over EFA); the receiver moves tokens into the tensor handed
// to the grouped GEMM (Dispatch and combine). The expert form is not on the pages:
// SwiGLU without biases, h = X W1^T, u = X W3^T, a = silu(h) * u, y = a W2^T.
//
// bf16 path: v_mfma_f32_32x32x16_bf16, float32 accumulation. Workgroup tile 256 token
// rows x 256 weight rows x 64 deep, eight wavefronts (each four alternating 32-row token sub-tiles x 64 weight
// rows). For the gate/up GEMM the 256 weight rows are 128 rows of W1 and the same 128
// rows of W3, so the SwiGLU epilogue pairs h and u in registers and writes a (and h, u
// when they are saved for the backward). Tiles are double-buffered in LDS with an XOR
// swizzle of 16-byte chunks. Rows are ragged per
// expert: a tile map (m-tiles per expert, prefix-summed on the device) lets a
// persistent grid walk (expert, m-tile, n-tile) work items; the walk gives each XCD
// a contiguous run of items in every round so tiles that share A rows or weight
// panels meet in the same L2.
//
// f32 path: a plain LDS-tiled vector-ALU kernel (float32 has no dense matrix-core
// peak worth the complexity at the sizes it is used for).
#include "gemm_common.h"

#include <mutex>

namespace moe {
namespace {

enum { EPI_SWIGLU = 0, EPI_PLAIN = 1 };

typedef unsigned int v4u32 __attribute__((ext_vector_type(4)));

// Eight wavefronts, two per SIMD: wave w takes weight group w & 3 (64 weight rows)
// and token group w >> 2, the 32-row token sub-tiles (w >> 2) + 2i. Each SIMD holds
// one wave of each token group, so the MFMA work per SIMD is the same for any count of
// live token rows, and its two waves' shares differ by at most one sub-tile.
constexpr int kFwdThreads = 512;
constexpr int kLdsFwd = kLdsGemm;
// Waves 0-3 issue every stage's direct loads (each the share of two waves) and alone
// wait for the vector-memory counter; waves 4-7 carry the epilogue's global writes. So
// one item's writes drain while the next item's stages load.
constexpr int kLoaderWaves = 4;
// The split pays where an item's writes are large next to its loads (down: 256 output
// columns; gate/up when h and u are saved); gate/up writing a alone keeps every wave
// loading and writing its own share (measured: the split costs it more than it saves).

// silu(h) = h * sigmoid(h) with the hardware exp and reciprocal (the result is rounded
// to bf16, far coarser than their error)
__device__ __forceinline__ float silu_fast(float h) {
    return h * __builtin_amdgcn_rcpf(1.0f + __expf(-h));
}

// Per-item state of the bf16 grouped GEMM: buffer resources of the token tile and
// of the expert's weight panel, and per-lane byte offsets of the lane's 16-byte chunk
// in the wave's A and B groups 0 and 1 (group j + 2 lies 16 rows further on, with the
// same swizzle).
struct GemmItem {
    __amdgpu_buffer_rsrc_t ra;   // token rows from the tile's first row on
    __amdgpu_buffer_rsrc_t rw;   // the expert's weight panel
    uint32_t a_off[2], b_off[2];
    int a_groups;                // of this wave's A groups, those holding live rows
    int64_t m0, m_end;           // token rows [m0, m_end) are live in this tile
    int n0;                      // first output column
};

// Direct global->LDS loads of one stage (a group is 8 rows x 128 bytes, one 1 KiB
// wavefront instruction). Split: loading wave w moves A and B groups 8w..8w+7, the
// other waves nothing; else wave w moves groups 4w..4w+3. Buffer loads rather than
// global ones: the compiler then keeps its LDS waits exact.
template <bool SPLIT>
__device__ __forceinline__ void issue_stage(unsigned char *lds, int stage, int k0,
                                            const GemmItem &it, int wave, int K) {
    constexpr int NG = SPLIT ? 8 : 4;
    if (SPLIT && wave >= kLoaderWaves) return;
    unsigned char *As = lds + stage * (kLdsA + kLdsB);
    unsigned char *Bs = As + kLdsA;
    const uint32_t step = uint32_t(16 * K * 2);          // 16 rows
#pragma unroll
    for (int j = 0; j < NG; ++j) {
        if (j < it.a_groups)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                it.ra, (__attribute__((address_space(3))) void *)(As + (wave * NG + j) * 1024), 16,
                it.a_off[j & 1] + uint32_t(j >> 1) * step, k0 * 2, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            it.rw, (__attribute__((address_space(3))) void *)(Bs + (wave * NG + j) * 1024), 16,
            it.b_off[j & 1] + uint32_t(j >> 1) * step, k0 * 2, 0, 0);
    }
}

// LDS reads of one k16 step: the wave's two weight fragments and its NW token
// fragments (16 bytes per lane each; rows are 128 B with chunk c stored at c ^ swz(row)).
template <int NW>
__device__ __forceinline__ void read_frags(const unsigned char *As, const unsigned char *Bs,
                                           int lane, int ks, const int (&brow)[2], int trow,
                                           bf16x8 (&wf)[2], bf16x8 (&tf)[4]) {
    const int kc = ks * 2 + (lane >> 5);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        const int r = brow[s] + (lane & 31);
        wf[s] = *reinterpret_cast<const bf16x8 *>(Bs + r * 128 + ((kc ^ swz(r)) << 4));
    }
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        const int r = trow + i * 64 + (lane & 31);
        tf[i] = *reinterpret_cast<const bf16x8 *>(As + r * 128 + ((kc ^ swz(r)) << 4));
    }
}

// One work item, seen by one wave with NW (0..4) live 32-row token sub-tiles: the
// whole K loop and the epilogue, branch-free in the inner loop. A wave with no live
// rows still moves its share of every stage and joins every barrier.
template <int EPI, int NW, bool SPLIT>
__device__ __forceinline__ void run_item(unsigned char *lds, const GemmItem &it,
                                         const GemmItem &next, bool has_next, int wave,
                                         int lane, int K, int N, uint16_t *__restrict__ out,
                                         uint16_t *__restrict__ hu_save) {
    const int wn = wave & 3, wm = wave >> 2;
    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < NW; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
    // B rows of this wave's two 32-row weight sub-tiles: gate/up pairs W1 rows with
    // the same W3 rows; down takes 64 consecutive W2 rows
    int brow[2];
#pragma unroll
    for (int s = 0; s < 2; ++s)
        brow[s] = (EPI == EPI_SWIGLU) ? s * 128 + wn * 32 : wn * 64 + s * 32;
    // token sub-tiles alternate between the two groups (group wm takes 32-row
    // sub-tiles wm, wm + 2, ...), so the two wavefronts of a SIMD get equal shares of
    // a partly filled tile
    const int trow = wm * 32;

    const int KT = K / BK;
    const bool loader = !SPLIT || wave < kLoaderWaves;
    // stage 0 was issued before the previous item's epilogue (or before the first item)
    if (loader) __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < KT) issue_stage<SPLIT>(lds, cur ^ 1, (kt + 1) * BK, it, wave, K);
        if (NW > 0) {
            const unsigned char *As = lds + cur * (kLdsA + kLdsB);
            const unsigned char *Bs = As + kLdsA;
            // fragments double-buffered across the four k16 steps: the LDS reads of step
            // ks+1 are issued before the MFMAs of step ks (sched_barrier keeps that order)
            bf16x8 wf[2][2], tf[2][4];
#pragma unroll
            for (int ks = 0; ks < BK / 16; ++ks) {
                if (ks == 0) {
                    read_frags<NW>(As, Bs, lane, 0, brow, trow, wf[0], tf[0]);
                    __builtin_amdgcn_sched_barrier(0);   // step 0's reads issue first
                }
                if (ks + 1 < BK / 16)
                    read_frags<NW>(As, Bs, lane, ks + 1, brow, trow, wf[(ks + 1) & 1], tf[(ks + 1) & 1]);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int i = 0; i < NW; ++i)
#pragma unroll
                    for (int s = 0; s < 2; ++s)
                        acc[i][s] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[ks & 1][s], tf[ks & 1][i],
                                                                            acc[i][s], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        if (loader) __builtin_amdgcn_s_waitcnt(0);   // this wave's loads of the next stage landed
        __syncthreads();                 // everyone's loads landed, and cur is free
    }

    // every wave is past its last LDS read: the next item's first stage flies into buffer
    // 0 during this item's epilogue
    if (has_next) issue_stage<SPLIT>(lds, 0, 0, next, wave, K);

    if (!SPLIT) {
    // direct epilogue: D = W_tile * X_tile^T, so lane l holds token column m = l & 31 and, for
    // v = 4g + q, weight row n = 8g + 4*(l >> 5) + q: four consecutive outputs of one
    // token row, stored as one 8-byte write per (sub-tile, g)
    const int64_t mrow0 = it.m0 + trow + (lane & 31);   // sub-tile i at mrow0 + 64 i
    const int nl = 4 * (lane >> 5);
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        const int64_t m = mrow0 + i * 64;
        if (m >= it.m_end) continue;
        if (EPI == EPI_SWIGLU) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int n = it.n0 + wn * 32 + 8 * g + nl;
                if (n >= N) continue;
                float a4[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) a4[q] = silu_fast(acc[i][0][4 * g + q]) * acc[i][1][4 * g + q];
                uint2 pa;
                pa.x = pack_bf16x2(a4[0], a4[1]);
                pa.y = pack_bf16x2(a4[2], a4[3]);
                *reinterpret_cast<uint2 *>(out + m * N + n) = pa;
                if (hu_save) {
                    uint2 ph, pu;
                    ph.x = pack_bf16x2(acc[i][0][4 * g], acc[i][0][4 * g + 1]);
                    ph.y = pack_bf16x2(acc[i][0][4 * g + 2], acc[i][0][4 * g + 3]);
                    pu.x = pack_bf16x2(acc[i][1][4 * g], acc[i][1][4 * g + 1]);
                    pu.y = pack_bf16x2(acc[i][1][4 * g + 2], acc[i][1][4 * g + 3]);
                    *reinterpret_cast<uint2 *>(hu_save + m * 2 * N + n) = ph;
                    *reinterpret_cast<uint2 *>(hu_save + m * 2 * N + N + n) = pu;
                }
            }
        } else {
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int n = it.n0 + wn * 64 + s * 32 + 8 * g + nl;
                    if (n >= N) continue;
                    uint2 p;
                    p.x = pack_bf16x2(acc[i][s][4 * g], acc[i][s][4 * g + 1]);
                    p.y = pack_bf16x2(acc[i][s][4 * g + 2], acc[i][s][4 * g + 3]);
                    *reinterpret_cast<uint2 *>(out + m * N + n) = p;
                }
        }
    }
    return;
    }

    // split: epilogue through stage buffer 1 (64 KiB), CR token rows at a time. D = W_tile *
    // X_tile^T: lane l holds token row trow + 64i + (l & 31) and, for v = 4g + q, weight
    // row 8g + 4 (l >> 5) + q of sub-tile s, four consecutive outputs of one token row
    // that go to LDS as one 8-byte bf16 piece. A chunk row is RP bytes: gate/up a (128
    // columns, 256 B), with h and u behind it when they are saved; down 256 columns
    // (512 B). Its 16-byte piece p sits at p ^ (row & 15). Chunks are taken starting
    // half-way through the tile.
    const bool save = (EPI == EPI_SWIGLU) && hu_save != nullptr;
    const int RP = (EPI == EPI_SWIGLU) ? (save ? 768 : 256) : 512;
    const int CR = (EPI == EPI_SWIGLU) ? (save ? 64 : 256) : 128;
    const int nch = 256 / CR;
    unsigned char *cb = lds + (kLdsA + kLdsB);
#pragma unroll 1
    for (int cc = 0; cc < nch; ++cc) {
        const int c = (cc + nch / 2) % nch;
        const int lo = c * CR;                               // first tile row of the chunk
#pragma unroll
        for (int i = 0; i < NW; ++i) {
            const int t0 = trow + 64 * i;
            if (t0 < lo || t0 >= lo + CR) continue;
            const int rl = t0 - lo + (lane & 31);
            unsigned char *row = cb + rl * RP + (lane >> 5) * 8;
            const int sw = rl & 15;
            if (EPI == EPI_SWIGLU) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int pc = ((wn * 4 + g) ^ sw) << 4;
                    float a4[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) a4[q] = silu_fast(acc[i][0][4 * g + q]) * acc[i][1][4 * g + q];
                    *reinterpret_cast<uint2 *>(row + pc) =
                        make_uint2(pack_bf16x2(a4[0], a4[1]), pack_bf16x2(a4[2], a4[3]));
                    if (save) {
                        *reinterpret_cast<uint2 *>(row + 256 + pc) =
                            make_uint2(pack_bf16x2(acc[i][0][4 * g], acc[i][0][4 * g + 1]),
                                       pack_bf16x2(acc[i][0][4 * g + 2], acc[i][0][4 * g + 3]));
                        *reinterpret_cast<uint2 *>(row + 512 + pc) =
                            make_uint2(pack_bf16x2(acc[i][1][4 * g], acc[i][1][4 * g + 1]),
                                       pack_bf16x2(acc[i][1][4 * g + 2], acc[i][1][4 * g + 3]));
                    }
                }
            } else {
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const int pc = ((wn * 8 + s2 * 4 + g) ^ sw) << 4;
                        *reinterpret_cast<uint2 *>(row + pc) =
                            make_uint2(pack_bf16x2(acc[i][s2][4 * g], acc[i][s2][4 * g + 1]),
                                       pack_bf16x2(acc[i][s2][4 * g + 2], acc[i][s2][4 * g + 3]));
                    }
            }
        }
        __syncthreads();
        if (!loader) {
            // this wave's CR/4 rows of the chunk in whole 16-byte pieces: gate/up 16 lanes
            // per 256-byte section row (4 rows per instruction), down 32 lanes per row (2
            // rows per instruction); buffer stores from the wave's first token row (rows
            // past the item and columns past N are skipped)
            const int nr = CR / 4;
            const int r0 = (wave - kLoaderWaves) * nr;
            const int64_t m0 = it.m0 + lo + r0;
            const int live = int(max<int64_t>(0, min<int64_t>(nr, it.m_end - m0)));
            constexpr int LPR = (EPI == EPI_SWIGLU) ? 16 : 32;      // lanes per row
            constexpr int RPI = 64 / LPR;                           // rows per instruction
            const int pr = lane % LPR, rsub = lane / LPR;
            const int n = it.n0 + 8 * pr;
            const bool col = n < N;
            const int ld = 2 * N;                                   // hu_save row length
            const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
                out + m0 * N, 0, int(int64_t(live) * N * 2), 0x00020000);
#pragma unroll 4
            for (int k = 0; k < nr / RPI; ++k) {
                const int rr = k * RPI + rsub;
                const int rowb = (r0 + rr) * RP + ((pr ^ ((r0 + rr) & 15)) << 4);
                if (!(col && rr < live)) continue;
                const uint4 v = *reinterpret_cast<const uint4 *>(cb + rowb);
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u32, v), ro, (rr * N + n) * 2, 0, 0);
                if (save) {
                    const __amdgpu_buffer_rsrc_t rh = __builtin_amdgcn_make_buffer_rsrc(
                        hu_save + m0 * ld, 0, int(int64_t(live) * ld * 2), 0x00020000);
                    const uint4 h = *reinterpret_cast<const uint4 *>(cb + rowb + 256);
                    const uint4 u = *reinterpret_cast<const uint4 *>(cb + rowb + 512);
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u32, h), rh, (rr * ld + n) * 2, 0, 0);
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u32, u), rh, (rr * ld + N + n) * 2, 0, 0);
                }
            }
        }
        __syncthreads();
    }
}

// Work item -> per-wave load state. An expert's rows are split into equal m-tiles, so
// the tiles that share one weight panel run at one speed and meet in L2; rows past the
// allocation are never touched, whatever expert_off holds.
template <int EPI, bool SPLIT>
__device__ __forceinline__ GemmItem make_item(int item, const int *tile_off,
                                              const int *__restrict__ expert_off, int E,
                                              int n_tiles, const uint16_t *__restrict__ A,
                                              const uint16_t *__restrict__ W, int K, int N,
                                              int64_t rows_alloc, int wave, int lane) {
    const int Nw = (EPI == EPI_SWIGLU) ? 2 * N : N;              // weight rows per expert
    // a direct load puts lane l's 16 bytes at row l/8, physical chunk l%8 of its
    // 8-row group, so the XOR swizzle is applied on the global side
    const int lrow = lane >> 3;
    const int pchunk = lane & 7;
    const ItemCoord ic = decode_item(item, tile_off, E, n_tiles);
    const int e = ic.e;
    GemmItem it;
    const int64_t e_lo = min<int64_t>(expert_off[e], rows_alloc);
    const int64_t e_hi = min<int64_t>(expert_off[e + 1], rows_alloc);
    const int mc = tile_off[e + 1] - tile_off[e];
    const int64_t rp = (e_hi - e_lo + mc - 1) / mc;     // <= BM
    it.m0 = e_lo + int64_t(ic.mt) * rp;
    it.m_end = min<int64_t>(e_hi, it.m0 + rp);
    it.n0 = ic.nt * (EPI == EPI_SWIGLU ? BNW / 2 : BNW);
    // byte ranges of the two resources (loads past them would read zeros); the host
    // bounds the weight panel below 2^31 bytes
    it.ra = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(A + it.m0 * K), 0,
                                             int((rows_alloc - it.m0 < BM ? rows_alloc - it.m0 : BM) * K * 2),
                                             0x00020000);
    it.rw = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(W + size_t(e) * Nw * K), 0,
                                             int(size_t(Nw) * K * 2), 0x00020000);
    const int wr0 = SPLIT ? (wave & 3) * 64 : wave * 32;        // the wave's first tile row
    it.a_groups = int(min<int64_t>(SPLIT ? 8 : 4, max<int64_t>(0, (it.m_end - it.m0 - wr0 + 7) / 8)));
    // Rows past the tile's data read zeros (outside the token resource) or stay inside
    // the weight panel (gate rows past N read up rows) or past it (zeros): the outputs of
    // such rows and columns are never stored. (Offsets of non-loading waves go unused.)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int r = wr0 + j * 8 + lrow;               // tile row of group j
        const int c = pchunk ^ swz(r);
        it.a_off[j] = uint32_t((r * K + c * 8) * 2);
        const int wr = (EPI == EPI_SWIGLU) ? it.n0 + (r & 127) + (r < 128 ? 0 : N) : it.n0 + r;
        it.b_off[j] = uint32_t((size_t(wr) * K + c * 8) * 2);
    }
    return it;
}

template <int EPI, bool SPLIT>
__global__ __launch_bounds__(kFwdThreads) void k_gemm_bf16(
    const uint16_t *__restrict__ A,        // token rows [rows, K]
    const int *__restrict__ expert_off,    // [E+1]
    int E, const uint16_t *__restrict__ W, // [E, Nw, K]
    int K, int N, int64_t rows_alloc,
    uint16_t *__restrict__ out,            // [rows, N]
    uint16_t *__restrict__ hu_save,        // [rows, 2N] (gate/up only; may be null)
    int n_tiles) {
    extern __shared__ __align__(16) unsigned char lds[];   // 2 stages x (A 32 KiB + B 32 KiB)
    __shared__ int tile_off[kMaxE + 1];
    __shared__ int map_scratch[256];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wavefront
    build_tile_map(expert_off, E, BM, rows_alloc, tile_off, map_scratch);
    const int total = tile_off[E] * n_tiles;
    const int G = gridDim.x;
    // this workgroup's place in a round: XCD (blockIdx % 8) gets a contiguous run;
    // rotating the place each round spreads large and small items evenly
    const int per = G / 8;
    const int slot = (G % 8 == 0) ? (blockIdx.x % 8) * per + blockIdx.x / 8 : blockIdx.x;
    if (slot >= total) return;

    GemmItem it = make_item<EPI, SPLIT>(slot, tile_off, expert_off, E, n_tiles, A, W, K, N, rows_alloc,
                                 wave, lane);
    issue_stage<SPLIT>(lds, 0, 0, it, wave, K);
    for (int base = 0; base < total; base += G) {
        const int nbase = base + G;
        const int nitem = nbase + (slot + nbase / G) % G;
        const bool has_next = nitem < total;
        GemmItem next = it;
        if (has_next)
            next = make_item<EPI, SPLIT>(nitem, tile_off, expert_off, E, n_tiles, A, W, K, N, rows_alloc,
                                  wave, lane);
        // live 32-row token sub-tiles of this wave's token group
        const int nsub = int(min<int64_t>(8, (it.m_end - it.m0 + 31) / 32));
        const int nw = min(4, max(0, (nsub - (wave >> 2) + 1) / 2));
        switch (nw) {
        case 4: run_item<EPI, 4, SPLIT>(lds, it, next, has_next, wave, lane, K, N, out, hu_save); break;
        case 3: run_item<EPI, 3, SPLIT>(lds, it, next, has_next, wave, lane, K, N, out, hu_save); break;
        case 2: run_item<EPI, 2, SPLIT>(lds, it, next, has_next, wave, lane, K, N, out, hu_save); break;
        case 1: run_item<EPI, 1, SPLIT>(lds, it, next, has_next, wave, lane, K, N, out, hu_save); break;
        default: run_item<EPI, 0, SPLIT>(lds, it, next, has_next, wave, lane, K, N, out, hu_save); break;
        }
        if (!has_next) break;
        it = next;
    }
}

// ---------------------------------------------------------------- f32 path
// 64x64 output tile per workgroup, 16-deep LDS stages, 4x4 outputs per thread.
// Gate/up computes h and u tiles side by side (W1 rows and the matching W3 rows).
constexpr int FT = 64, FK = 16;

template <int EPI>
__global__ __launch_bounds__(256) void k_gemm_f32(const float *__restrict__ A,
                                                  const int *__restrict__ expert_off, int E,
                                                  const float *__restrict__ W, int K, int N,
                                                  int64_t rows_alloc, float *__restrict__ out,
                                                  float *__restrict__ hu_save, int n_tiles) {
    constexpr int NB = (EPI == EPI_SWIGLU) ? 2 : 1;   // weight tiles (W1, W3)
    __shared__ float As[FK][FT + 1];
    __shared__ float Bs[NB][FK][FT + 1];
    __shared__ int tile_off[kMaxE + 1];
    __shared__ int map_scratch[256];
    const int tid = threadIdx.x;
    const int tr = tid / 16, tc = tid % 16;
    const int Nw = NB * N;
    build_tile_map(expert_off, E, FT, rows_alloc, tile_off, map_scratch);
    const int total = tile_off[E] * n_tiles;
    for (int item = blockIdx.x; item < total; item += gridDim.x) {
        const ItemCoord ic = decode_item(item, tile_off, E, n_tiles);
        const int e = ic.e, nt = ic.nt;
        const int m0 = expert_off[e] + ic.mt * FT;
        const int m_end = int(min<int64_t>(expert_off[e + 1], rows_alloc));
        const int n0 = nt * FT;
        const float *We = W + size_t(e) * Nw * K;
        float acc[NB][4][4] = {};
        for (int k0 = 0; k0 < K; k0 += FK) {
            __syncthreads();
            for (int c = tid; c < FT * FK; c += 256) {
                const int r = c / FK, kk = c % FK;
                const int row = m0 + r, kg = k0 + kk;
                As[kk][r] = (row >= 0 && row < m_end && kg < K) ? A[size_t(row) * K + kg] : 0.0f;
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    const int n = n0 + r;
                    Bs[b][kk][r] = (n < N && kg < K) ? We[size_t(b * N + n) * K + kg] : 0.0f;
                }
            }
            __syncthreads();
#pragma unroll
            for (int kk = 0; kk < FK; ++kk) {
                float av[4], bv[NB][4];
#pragma unroll
                for (int i = 0; i < 4; ++i) av[i] = As[kk][tr * 4 + i];
#pragma unroll
                for (int b = 0; b < NB; ++b)
#pragma unroll
                    for (int j = 0; j < 4; ++j) bv[b][j] = Bs[b][kk][tc * 4 + j];
#pragma unroll
                for (int b = 0; b < NB; ++b)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int j = 0; j < 4; ++j) acc[b][i][j] = __builtin_fmaf(av[i], bv[b][j], acc[b][i][j]);
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = m0 + tr * 4 + i;
            if (row < 0 || row >= m_end) continue;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int col = n0 + tc * 4 + j;
                if (col >= N) continue;
                if (EPI == EPI_SWIGLU) {
                    const float h = acc[0][i][j], u = acc[NB - 1][i][j];
                    out[size_t(row) * N + col] = silu_f(h) * u;
                    if (hu_save) {
                        hu_save[size_t(row) * 2 * N + col] = h;
                        hu_save[size_t(row) * 2 * N + N + col] = u;
                    }
                } else {
                    out[size_t(row) * N + col] = acc[0][i][j];
                }
            }
        }
    }
}

bool set_lds_limits() {
    return lds_limit_once<&k_gemm_bf16<EPI_SWIGLU, false>>(kLdsFwd) &&
           lds_limit_once<&k_gemm_bf16<EPI_SWIGLU, true>>(kLdsFwd) &&
           lds_limit_once<&k_gemm_bf16<EPI_PLAIN, true>>(kLdsFwd);
}

// Workspace of the composite call: the activation a [rows, F] in dtype.
size_t ffn_ws_bytes(int64_t rows, int64_t F, moe_dtype_t dt) {
    return align256(size_t(rows) * F * elt_size(dt));
}

moe_status_t check_common(int32_t E, int64_t rows, int64_t d, int64_t F, moe_dtype_t dtype) {
    if (!valid_dtype(dtype) || E <= 0 || rows < 0 || d <= 0 || F <= 0) return MOE_ERR_INVALID_ARG;
    if (E > kMaxE || rows >= (int64_t(1) << 31) || d > (1 << 20) || F > (1 << 20))
        return MOE_ERR_UNSUPPORTED;
    if (dtype == MOE_BF16 && (d % BK != 0 || F % BK != 0)) return MOE_ERR_UNSUPPORTED;
    // one expert's weight panel (2F x d or d x F) is addressed with 32-bit byte offsets
    if (2 * F * d * int64_t(elt_size(dtype)) >= (int64_t(1) << 31)) return MOE_ERR_UNSUPPORTED;
    if ((d * elt_size(dtype)) % 16 != 0 || (F * elt_size(dtype)) % 16 != 0) return MOE_ERR_ALIGN;
    return MOE_OK;
}

moe_status_t launch_gate_up(const void *x_disp, const int32_t *expert_off, const void *w13,
                            int32_t E, int64_t rows, int64_t d, int64_t F, moe_dtype_t dtype,
                            void *act, void *hu_save, hipStream_t st) {
    if (dtype == MOE_BF16) {
        if (!set_lds_limits()) return MOE_ERR_HIP;
        const int nt = int(cdiv(F, BNW / 2));
        const int g = int(std::min<int64_t>((cdiv(rows, BM) + E) * nt, num_cus()));
        // writing h and u as well: the loader/storer split
        if (hu_save != nullptr)
            hipLaunchKernelGGL((k_gemm_bf16<EPI_SWIGLU, true>), dim3(g), dim3(kFwdThreads), kLdsFwd, st,
                               static_cast<const uint16_t *>(x_disp), expert_off, E,
                               static_cast<const uint16_t *>(w13), int(d), int(F), rows,
                               static_cast<uint16_t *>(act), static_cast<uint16_t *>(hu_save), nt);
        else
            hipLaunchKernelGGL((k_gemm_bf16<EPI_SWIGLU, false>), dim3(g), dim3(kFwdThreads), kLdsFwd, st,
                               static_cast<const uint16_t *>(x_disp), expert_off, E,
                               static_cast<const uint16_t *>(w13), int(d), int(F), rows,
                               static_cast<uint16_t *>(act), nullptr, nt);
    } else {
        const int nt = int(cdiv(F, FT));
        const int g = int(std::min<int64_t>((cdiv(rows, FT) + E) * nt, 4 * num_cus()));
        hipLaunchKernelGGL(k_gemm_f32<EPI_SWIGLU>, dim3(g), dim3(256), 0, st,
                           static_cast<const float *>(x_disp), expert_off, E,
                           static_cast<const float *>(w13), int(d), int(F), rows,
                           static_cast<float *>(act), static_cast<float *>(hu_save), nt);
    }
    return launch_status();
}

moe_status_t launch_down(const void *act, const int32_t *expert_off, const void *w2, int32_t E,
                         int64_t rows, int64_t d, int64_t F, moe_dtype_t dtype, void *y_disp,
                         hipStream_t st) {
    if (dtype == MOE_BF16) {
        if (!set_lds_limits()) return MOE_ERR_HIP;
        const int nt = int(cdiv(d, BNW));
        const int g = int(std::min<int64_t>((cdiv(rows, BM) + E) * nt, num_cus()));
        hipLaunchKernelGGL((k_gemm_bf16<EPI_PLAIN, true>), dim3(g), dim3(kFwdThreads), kLdsFwd, st,
                           static_cast<const uint16_t *>(act), expert_off, E,
                           static_cast<const uint16_t *>(w2), int(F), int(d), rows,
                           static_cast<uint16_t *>(y_disp), nullptr, nt);
    } else {
        const int nt = int(cdiv(d, FT));
        const int g = int(std::min<int64_t>((cdiv(rows, FT) + E) * nt, 4 * num_cus()));
        hipLaunchKernelGGL(k_gemm_f32<EPI_PLAIN>, dim3(g), dim3(256), 0, st,
                           static_cast<const float *>(act), expert_off, E,
                           static_cast<const float *>(w2), int(F), int(d), rows,
                           static_cast<float *>(y_disp), nullptr, nt);
    }
    return launch_status();
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" size_t moe_expert_ffn_workspace_size(int32_t E, int64_t rows, int64_t d, int64_t F,
                                                moe_dtype_t dtype) {
    (void)d;
    if (E <= 0 || rows < 0 || F <= 0 || !valid_dtype(dtype)) return 0;
    return ffn_ws_bytes(rows, F, dtype);
}

extern "C" moe_status_t moe_expert_ffn_gate_up(const void *x_disp, const int32_t *expert_off,
                                               const void *w13, int32_t E, int64_t rows,
                                               int64_t d, int64_t F, moe_dtype_t dtype, void *act,
                                               void *hu_save, void *stream) {
    const moe_status_t c = check_common(E, rows, d, F, dtype);
    if (c != MOE_OK) return c;
    if (rows == 0) return MOE_OK;
    if (!x_disp || !expert_off || !w13 || !act) return MOE_ERR_INVALID_ARG;
    if (!aligned16(x_disp) || !aligned16(w13) || !aligned16(act) || (hu_save && !aligned16(hu_save)))
        return MOE_ERR_ALIGN;
    return launch_gate_up(x_disp, expert_off, w13, E, rows, d, F, dtype, act, hu_save,
                          as_stream(stream));
}

extern "C" moe_status_t moe_expert_ffn_down(const void *act, const int32_t *expert_off,
                                            const void *w2, int32_t E, int64_t rows, int64_t d,
                                            int64_t F, moe_dtype_t dtype, void *y_disp,
                                            void *stream) {
    const moe_status_t c = check_common(E, rows, d, F, dtype);
    if (c != MOE_OK) return c;
    if (rows == 0) return MOE_OK;
    if (!act || !expert_off || !w2 || !y_disp) return MOE_ERR_INVALID_ARG;
    if (!aligned16(act) || !aligned16(w2) || !aligned16(y_disp)) return MOE_ERR_ALIGN;
    return launch_down(act, expert_off, w2, E, rows, d, F, dtype, y_disp, as_stream(stream));
}

extern "C" moe_status_t moe_expert_ffn(const void *x_disp, const int32_t *expert_off,
                                       const void *w13, const void *w2, int32_t E, int64_t rows,
                                       int64_t d, int64_t F, moe_dtype_t dtype, void *y_disp,
                                       void *hu_save, void *ws, size_t ws_bytes, void *stream) {
    const moe_status_t c = check_common(E, rows, d, F, dtype);
    if (c != MOE_OK) return c;
    if (rows == 0) return MOE_OK;
    if (!x_disp || !expert_off || !w13 || !w2 || !y_disp || !ws) return MOE_ERR_INVALID_ARG;
    if (ws_bytes < ffn_ws_bytes(rows, F, dtype)) return MOE_ERR_CAPACITY;
    if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return MOE_ERR_ALIGN;
    if (!aligned16(x_disp) || !aligned16(w13) || !aligned16(w2) || !aligned16(y_disp) ||
        (hu_save && !aligned16(hu_save)))
        return MOE_ERR_ALIGN;
    const hipStream_t st = as_stream(stream);
    const moe_status_t s1 = launch_gate_up(x_disp, expert_off, w13, E, rows, d, F, dtype, ws,
                                           hu_save, st);
    if (s1 != MOE_OK) return s1;
    return launch_down(ws, expert_off, w2, E, rows, d, F, dtype, y_disp, st);
}
