// Expert FFN: the grouped GEMM that multiplies each expert's rows by that expert's
// SwiGLU weights. [EFA] = Perplexity, "Enabling trillion-parameter models on AWS EFA"
// (2025): after dispatch, grouped GEMM kernels multiply the tokens with the expert
// weights (MoE all-to-all over EFA); the receiver moves tokens into the tensor handed
// to the grouped GEMM (Dispatch and combine). The expert form is not on the pages:
// SwiGLU without biases, h = X W1^T, u = X W3^T, a = silu(h) * u, y = a W2^T.
//
// bf16 path: v_mfma_f32_16x16x32_bf16, float32 accumulation. Workgroup tile 224 token
// rows x 384 weight rows x 64 deep, eight wavefronts, LDS-direct buffer loads into
// double-buffered stages with an XOR swizzle of 16-byte chunks. For the gate/up GEMM
// the 384 weight rows are 192 rows of W1 and the same 192 rows of W3, so the SwiGLU
// epilogue pairs h and u in registers and writes a (and h, u when they are saved for
// the backward). Rows are ragged per expert: a tile map (m-tiles per expert,
// prefix-summed on the device) lets a persistent grid walk (expert, n-tile, m-tile)
// work items; the walk gives each XCD a contiguous run of items in every round so
// tiles that share A rows or weight panels meet in the same L2.
//
// f32 path: a plain LDS-tiled vector-ALU kernel (float32 has no dense matrix-core
// peak worth the complexity at the sizes it is used for).
#include "gemm_common.h"

#include <mutex>

namespace moe {
namespace {

enum { EPI_SWIGLU = 0, EPI_PLAIN = 1 };

// Eight wavefronts, two per SIMD.
constexpr int kFwdThreads = 512;

// Workgroup barrier after this wave's LDS operations complete, without waiting for
// its global stores or direct loads (__syncthreads also waits for those). The memory
// clobber keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// silu(h) = h * sigmoid(h) with the hardware exp and reciprocal (the result is rounded
// to bf16, far coarser than their error)
__device__ __forceinline__ float silu_fast(float h) {
    return h * __builtin_amdgcn_rcpf(1.0f + __expf(-h));
}

// ---------------------------------------------------------------- wide tiles
// Tile of 224 token rows x 384 weight rows x 64 deep on v_mfma_f32_16x16x32_bf16.
// Every grouped GEMM here moves its stage loads between the L2 and the CUs at one
// aggregate rate, so its time follows the bytes it loads per flop: each stage load
// of a token row serves 384 weight rows instead of 256, and each weight row serves
// up to 224 token rows. The eight wavefronts split the tile 2 x 4: wave w takes token
// group w >> 2 (the 16-row sub-tiles (w >> 2) + 2i, up to seven) and weight group
// w & 3 (six 16-row weight blocks), 42 blocks of 16 x 16 outputs, four accumulators
// each: 168 registers per lane, which leaves room for double-buffered fragments at
// two wavefronts per SIMD. Gate/up tiles hold 192 rows of W1 (tile rows 0..191) and
// the same 192 rows of W3 (192..383), twelve 16-row blocks each; weight group g takes
// W1 blocks g, g + 4, g + 8 and the matching W3 blocks, so h and u of one output sit
// in one lane and register. Down tiles hold 384 consecutive rows of W2, 24 blocks;
// weight group g takes blocks g, g + 4, ..., g + 20. Stages load only live token and
// weight rows (an item's last n-tile may be partly past N).
constexpr int WM = 224;                           // token rows per wide tile
constexpr int WN = 384;                           // weight rows per wide tile
constexpr int kLdsWA = WM * BK * 2;               // 28 KiB
constexpr int kLdsWB = WN * BK * 2;               // 48 KiB
constexpr int kLdsWide = 2 * (kLdsWA + kLdsWB);   // 152 KiB, double buffered
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct WideItem {
    __amdgpu_buffer_rsrc_t ra;   // token rows from the tile's first row on
    __amdgpu_buffer_rsrc_t rw;   // the expert's weight panel
    uint32_t a_off;              // lane's byte offset in the wave's A group 0 (group j: +64 j rows)
    uint32_t b_off[2];           // B groups 0-2 and 3-5 (group j: + 64 (j % 3) rows)
    int a_groups;                // live A groups of this wave (0..4)
    int b_mask;                  // live B groups of this wave (bit j)
    int64_t m0, m_end;           // token rows [m0, m_end) are live in this tile
    int n0;                      // first output column
};

// Direct global->LDS loads of one stage: A groups (8 rows x 128 bytes each) wave + 8j,
// j < 4, of the 28; B groups wave + 8j, j < 6, of the 48. Weight loads carry the
// non-temporal cache-policy bit: a weight row serves only the m-tiles of its expert,
// which run side by side, while the stream of other experts' weights would otherwise
// push the token rows that each n-tile re-reads out of the caches (measured on the
// 384-expert layer: HBM fetch per gate/up launch 25.4 -> 23.9 GB, 1.005 x the
// algorithmic bytes; gate/up 4.62-4.86 -> 4.57-4.61 ms, down 2.53-2.59 -> 2.47-2.52 ms).
constexpr int kWeightNT = 2;   // the nt bit of the buffer instruction's cache policy
__device__ __forceinline__ void issue_wide(unsigned char *lds, int stage, int k0,
                                           const WideItem &it, int wave, int K) {
    unsigned char *As = lds + stage * (kLdsWA + kLdsWB);
    unsigned char *Bs = As + kLdsWA;
    const uint32_t step = uint32_t(64 * K * 2);          // 64 rows
#pragma unroll
    for (int j = 0; j < 4; ++j)
        if (j < it.a_groups)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                it.ra, (__attribute__((address_space(3))) void *)(As + (wave + 8 * j) * 1024), 16,
                it.a_off + uint32_t(j) * step, k0 * 2, 0, 0);
#pragma unroll
    for (int j = 0; j < 6; ++j)
        if ((it.b_mask >> j) & 1)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                it.rw, (__attribute__((address_space(3))) void *)(Bs + (wave + 8 * j) * 1024), 16,
                it.b_off[j / 3] + uint32_t(j % 3) * step, k0 * 2, 0, kWeightNT);
}

template <int EPI>
__device__ __forceinline__ WideItem make_wide_item(int item, const int *tile_off,
                                                   const int *__restrict__ expert_off, int E,
                                                   int n_tiles, const uint16_t *__restrict__ A,
                                                   const uint16_t *__restrict__ W, int K, int N,
                                                   int64_t rows_alloc, int wave, int lane) {
    const int Nw = (EPI == EPI_SWIGLU) ? 2 * N : N;              // weight rows per expert
    const int lrow = lane >> 3;
    const int pchunk = lane & 7;
    const ItemCoord ic = decode_item(item, tile_off, E, n_tiles);
    const int e = ic.e;
    WideItem it;
    const int64_t e_lo = min<int64_t>(expert_off[e], rows_alloc);
    const int64_t e_hi = min<int64_t>(expert_off[e + 1], rows_alloc);
    const int mc = tile_off[e + 1] - tile_off[e];
    const int64_t rp = (e_hi - e_lo + mc - 1) / mc;     // <= WM
    it.m0 = e_lo + int64_t(ic.mt) * rp;
    it.m_end = min<int64_t>(e_hi, it.m0 + rp);
    const int cols = (EPI == EPI_SWIGLU) ? WN / 2 : WN;         // output columns per tile
    it.n0 = ic.nt * cols;
    it.ra = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(A + it.m0 * K), 0,
                                             int((rows_alloc - it.m0 < WM ? rows_alloc - it.m0 : WM) * K * 2),
                                             0x00020000);
    it.rw = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(W + size_t(e) * Nw * K), 0,
                                             int(size_t(Nw) * K * 2), 0x00020000);
    // tile row of the lane's row in group wave (+ 64 j): 8 wave + lrow; its swizzle
    // depends on the row's low four bits only, the same for every j
    const int r = 8 * wave + lrow;
    const int c = pchunk ^ swz(r);
    it.a_off = uint32_t((r * K + c * 8) * 2);
    const int live = int(it.m_end - it.m0);
    it.a_groups = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        if (wave + 8 * j < WM / 8 && 8 * (wave + 8 * j) < live) it.a_groups = j + 1;
    const int ncol = N - it.n0;                          // output columns left (multiple of 64)
    it.b_mask = 0;
    if (EPI == EPI_SWIGLU) {
        // groups 0-2: W1 rows n0 + r + 64 j; groups 3-5: W3 rows N + n0 + r + 64 (j - 3)
        it.b_off[0] = uint32_t((size_t(it.n0 + r) * K + c * 8) * 2);
        it.b_off[1] = uint32_t((size_t(N + it.n0 + r) * K + c * 8) * 2);
#pragma unroll
        for (int j = 0; j < 3; ++j)
            if (8 * (wave + 8 * j) < ncol) it.b_mask |= 9 << j;
    } else {
        it.b_off[0] = uint32_t((size_t(it.n0 + r) * K + c * 8) * 2);
        it.b_off[1] = it.b_off[0] + uint32_t(3 * 64 * K * 2);
#pragma unroll
        for (int j = 0; j < 6; ++j)
            if (8 * (wave + 8 * j) < ncol) it.b_mask |= 1 << j;
    }
    return it;
}

// One work item seen by one wave with NW (0..7) live 16-row token sub-tiles. FULL:
// every weight sub-tile of the tile is live; else the wave skips the reads and MFMAs
// of its sub-tiles past N (its 16-row weight blocks are wn, wn + 4, ..., so the live
// ones of a partly filled tile spread evenly over the SIMDs).
template <int EPI, int NW, bool FULL, bool NT>
__device__ __forceinline__ void run_wide_item(unsigned char *lds, const WideItem &it,
                                              const WideItem &next, bool has_next, int wave,
                                              int lane, int K, int N,
                                              uint16_t *__restrict__ out,
                                              uint16_t *__restrict__ hu_save) {
    const int wn = wave & 3, wm = wave >> 2;
    // live weight blocks of this wave: block wn + 4j is live while it starts before N
    constexpr int J = (EPI == EPI_SWIGLU) ? 3 : 6;
    const int nb = min(J * 4, (N - it.n0) / 16);
    const int ls = FULL ? J : min(J, max(0, (nb - wn + 3) / 4));
    auto live = [&](int s) { return FULL || (s % J) < ls; };
    f32x4 acc[NW > 0 ? NW : 1][6];
#pragma unroll
    for (int i = 0; i < NW; ++i)
#pragma unroll
        for (int s = 0; s < 6; ++s) acc[i][s] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    // first tile row of each of the wave's weight sub-tiles
    int wrow[6];
#pragma unroll
    for (int s = 0; s < 6; ++s)
        wrow[s] = (EPI == EPI_SWIGLU) ? (s < 3 ? 16 * (wn + 4 * s) : WN / 2 + 16 * (wn + 4 * (s - 3)))
                                      : 16 * (wn + 4 * s);
    const int KT = K / BK;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < KT) issue_wide(lds, cur ^ 1, (kt + 1) * BK, it, wave, K);
        if (NW > 0) {
            const unsigned char *As = lds + cur * (kLdsWA + kLdsWB);
            const unsigned char *Bs = As + kLdsWA;
            // software pipeline over the stage's 2 x NW groups (k32 step ks, token
            // sub-tile i): the token fragment of group g + 1 is read while group g's
            // six MFMAs issue, and step 1's weight fragments while step 0 runs, so LDS
            // latency hides behind the matrix cores (weight and token fragments
            // double-buffered)
            bf16x8 wf[2][6], tf[2];
            auto rd_w = [&](int ks, bf16x8 (&dst)[6]) {
                const int kc = ks * 4 + (lane >> 4);
#pragma unroll
                for (int s = 0; s < 6; ++s) {
                    const int r = wrow[s] + (lane & 15);
                    if (live(s))
                        dst[s] = *reinterpret_cast<const bf16x8 *>(Bs + r * 128 + ((kc ^ swz(r)) << 4));
                }
            };
            constexpr int NWD = NW > 0 ? NW : 1;
            auto rd_t = [&](int g, bf16x8 &dst) {
                const int ks = g / NWD, i = g % NWD;
                const int kc = ks * 4 + (lane >> 4);
                const int r = 16 * (wm + 2 * i) + (lane & 15);
                dst = *reinterpret_cast<const bf16x8 *>(As + r * 128 + ((kc ^ swz(r)) << 4));
            };
            constexpr int NG = 2 * NWD;
            rd_w(0, wf[0]);
            rd_t(0, tf[0]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                if (g + 1 < NG) rd_t(g + 1, tf[(g + 1) & 1]);
                if (g == 0) rd_w(1, wf[1]);
                __builtin_amdgcn_sched_barrier(0);
                const int ks = g / NWD, i = g % NWD;
#pragma unroll
                for (int s = 0; s < 6; ++s)
                    if (live(s))
                        acc[i][s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[ks][s], tf[g & 1], acc[i][s], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        __builtin_amdgcn_s_waitcnt(0);   // this wave's loads of the next stage landed
        __syncthreads();                 // everyone's loads landed, and cur is free
    }
    // every wave is past its last LDS read: the next item's first stage flies into buffer
    // 0 during this item's epilogue
    if (has_next) issue_wide(lds, 0, 0, next, wave, K);

    // Epilogue through stage buffer 1, which is idle until the next item's first barrier.
    // D = W_tile * X_tile^T: lane l holds token column l & 15 of each token sub-tile and,
    // in register q, weight row 4 (l >> 4) + q of each weight block, so a direct store
    // would write 32-byte pieces of 16 rows. Instead each output matrix (a, and h, u
    // when saved; y for down) goes to LDS 96 tile rows at a time and from there to
    // memory as whole rows, 16 bytes per lane. The barriers here wait for LDS only: the
    // stores and the next item's first stage stay in flight.
    constexpr int COLS = (EPI == EPI_SWIGLU) ? WN / 2 : WN;   // output columns per tile
    constexpr int PPR = COLS / 8;                             // 16-byte pieces per row
    constexpr int PITCH = COLS * 2 + 16;                      // LDS row pitch (bytes)
    constexpr int CR = 96;                                    // tile rows per chunk
    static_assert(CR * PITCH <= kLdsWA + kLdsWB, "an epilogue chunk fits one stage buffer");
    unsigned char *cb = lds + (kLdsWA + kLdsWB);
    const int live_rows = int(it.m_end - it.m0);
    const int nmat = (EPI == EPI_SWIGLU && hu_save != nullptr) ? 3 : 1;
    const int tid = int(threadIdx.x);
    const int nl = 4 * (lane >> 4);
    // every wave runs the same chunks and barriers (its own sub-tiles may end sooner)
#pragma unroll
    for (int c = 0; c < (WM + CR - 1) / CR; ++c) {            // token sub-tiles 3c..3c+2
        if (c * CR >= live_rows) break;
#pragma unroll
        for (int o = 0; o < ((EPI == EPI_SWIGLU) ? 3 : 1); ++o) {
            if (o >= nmat) break;
            uint16_t *dst = o == 0 ? out : hu_save + (o == 2 ? N : 0);
            const int64_t ld = o == 0 ? N : 2 * int64_t(N);
#pragma unroll
            for (int i = 3 * c; i < NW && i < 3 * c + 3; ++i) {
                unsigned char *row = cb + (16 * (wm + 2 * (i % 3)) + (lane & 15)) * PITCH + nl * 2;
#pragma unroll
                for (int s = 0; s < ((EPI == EPI_SWIGLU) ? 3 : 6); ++s) {
                    if (!live(s)) continue;
                    float v[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        if (EPI == EPI_PLAIN) v[q] = acc[i][s][q];
                        else if (o == 0) v[q] = silu_fast(acc[i][s][q]) * acc[i][s + 3][q];
                        else v[q] = acc[i][o == 1 ? s : s + 3][q];
                    }
                    *reinterpret_cast<uint2 *>(row + 32 * (wn + 4 * s)) =
                        make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
                }
            }
            lds_barrier();
            const int rows_c = min(CR, live_rows - c * CR);
            uint16_t *base = dst + (it.m0 + int64_t(c) * CR) * ld + it.n0;
            for (int p = tid; p < rows_c * PPR; p += kFwdThreads) {
                const int r = p / PPR, cp = p - r * PPR;
                if (it.n0 + 8 * cp < N) {
                    const uint4 v = *reinterpret_cast<const uint4 *>(cb + r * PITCH + 16 * cp);
                    if (NT)
                        __builtin_nontemporal_store(__builtin_bit_cast(u32x4, v),
                                                    reinterpret_cast<u32x4 *>(base + r * ld + 8 * cp));
                    else
                        *reinterpret_cast<uint4 *>(base + r * ld + 8 * cp) = v;
                }
            }
            lds_barrier();
        }
    }
}

template <int EPI, bool FULL, bool NT>
__device__ __forceinline__ void wide_item_nw(int nw, unsigned char *lds, const WideItem &it,
                                             const WideItem &next, bool has_next, int wave,
                                             int lane, int K, int N, uint16_t *__restrict__ out,
                                             uint16_t *__restrict__ hu_save) {
    switch (nw) {
    case 7: run_wide_item<EPI, 7, FULL, NT>(lds, it, next, has_next, wave, lane, K, N, out, hu_save); break;
    case 6: run_wide_item<EPI, 6, FULL, NT>(lds, it, next, has_next, wave, lane, K, N, out, hu_save); break;
    case 5: run_wide_item<EPI, 5, FULL, NT>(lds, it, next, has_next, wave, lane, K, N, out, hu_save); break;
    case 4: run_wide_item<EPI, 4, FULL, NT>(lds, it, next, has_next, wave, lane, K, N, out, hu_save); break;
    case 3: run_wide_item<EPI, 3, FULL, NT>(lds, it, next, has_next, wave, lane, K, N, out, hu_save); break;
    case 2: run_wide_item<EPI, 2, FULL, NT>(lds, it, next, has_next, wave, lane, K, N, out, hu_save); break;
    case 1: run_wide_item<EPI, 1, FULL, NT>(lds, it, next, has_next, wave, lane, K, N, out, hu_save); break;
    default: run_wide_item<EPI, 0, FULL, NT>(lds, it, next, has_next, wave, lane, K, N, out, hu_save); break;
    }
}

// NT: non-temporal output stores
template <int EPI, bool NT>
__global__ __launch_bounds__(kFwdThreads) void k_gemm_wide(
    const uint16_t *__restrict__ A,        // token rows [rows, K]
    const int *__restrict__ expert_off,    // [E+1]
    int E, const uint16_t *__restrict__ W, // [E, Nw, K]
    int K, int N, int64_t rows_alloc,
    uint16_t *__restrict__ out,            // [rows, N]
    uint16_t *__restrict__ hu_save,        // [rows, 2N] (gate/up only; may be null)
    int n_tiles) {
    extern __shared__ __align__(16) unsigned char lds[];   // 2 stages x (A 28 KiB + B 48 KiB)
    __shared__ int tile_off[kMaxE + 1];
    __shared__ int map_scratch[256];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    build_tile_map(expert_off, E, WM, rows_alloc, tile_off, map_scratch);
    const int total = tile_off[E] * n_tiles;
    const int G = gridDim.x;
    const int per = G / 8;
    const int slot = (G % 8 == 0) ? (blockIdx.x % 8) * per + blockIdx.x / 8 : blockIdx.x;
    if (slot >= total) return;

    WideItem it = make_wide_item<EPI>(slot, tile_off, expert_off, E, n_tiles, A, W, K, N, rows_alloc,
                                      wave, lane);
    issue_wide(lds, 0, 0, it, wave, K);
    for (int base = 0; base < total; base += G) {
        const int nbase = base + G;
        const int nitem = nbase + (slot + nbase / G) % G;
        const bool has_next = nitem < total;
        WideItem next = it;
        if (has_next)
            next = make_wide_item<EPI>(nitem, tile_off, expert_off, E, n_tiles, A, W, K, N, rows_alloc,
                                       wave, lane);
        const int nsub = int(min<int64_t>(WM / 16, (it.m_end - it.m0 + 15) / 16));
        const int nw = min(7, max(0, (nsub - (wave >> 2) + 1) / 2));
        const bool full = N - it.n0 >= ((EPI == EPI_SWIGLU) ? WN / 2 : WN);
        if (full) wide_item_nw<EPI, true, NT>(nw, lds, it, next, has_next, wave, lane, K, N, out, hu_save);
        else wide_item_nw<EPI, false, NT>(nw, lds, it, next, has_next, wave, lane, K, N, out, hu_save);
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
    return lds_limit_once<&k_gemm_wide<EPI_SWIGLU, false>>(kLdsWide) &&
           lds_limit_once<&k_gemm_wide<EPI_PLAIN, false>>(kLdsWide) &&
           lds_limit_once<&k_gemm_wide<EPI_PLAIN, true>>(kLdsWide);
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
        // one persistent workgroup per CU (the stages take 152 KiB of LDS)
        const int nt = int(cdiv(F, WN / 2));
        const int g = int(std::min<int64_t>((cdiv(rows, WM) + E) * nt, num_cus()));
        hipLaunchKernelGGL((k_gemm_wide<EPI_SWIGLU, false>), dim3(g), dim3(kFwdThreads), kLdsWide, st,
                           static_cast<const uint16_t *>(x_disp), expert_off, E,
                           static_cast<const uint16_t *>(w13), int(d), int(F), rows,
                           static_cast<uint16_t *>(act), static_cast<uint16_t *>(hu_save), nt);
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
        const int nt = int(cdiv(d, WN));
        const int g = int(std::min<int64_t>((cdiv(rows, WM) + E) * nt, num_cus()));
        // y_disp larger than the 256 MB Infinity Cache cannot wait there for the combine:
        // non-temporal stores then keep it from displacing the token rows each item
        // re-reads (measured on the 384-expert layer: down 2.68 -> 2.51 ms, the combine
        // unchanged; at 100 MB the combine reads y_disp from the cache, 23 against 31 us)
        const bool nt_out = size_t(rows) * d * 2 > (size_t(256) << 20);
        if (nt_out)
            hipLaunchKernelGGL((k_gemm_wide<EPI_PLAIN, true>), dim3(g), dim3(kFwdThreads), kLdsWide, st,
                               static_cast<const uint16_t *>(act), expert_off, E,
                               static_cast<const uint16_t *>(w2), int(F), int(d), rows,
                               static_cast<uint16_t *>(y_disp), nullptr, nt);
        else
            hipLaunchKernelGGL((k_gemm_wide<EPI_PLAIN, false>), dim3(g), dim3(kFwdThreads), kLdsWide, st,
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
