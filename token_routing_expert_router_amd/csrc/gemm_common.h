// Pieces shared by the grouped-GEMM kernels (forward and backward): MFMA operand
// types, tile geometry, the LDS swizzle and the per-workgroup m-tile map.
#pragma once

#include "common.h"

#include <mutex>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 256;         // token rows per tile
constexpr int BNW = 256;        // weight rows per tile
constexpr int BK = 64;          // depth per LDS stage
constexpr int kGemmThreads = 256;
constexpr int kLdsA = BM * BK * 2;              // bytes per A stage
constexpr int kLdsB = BNW * BK * 2;             // bytes per B stage
constexpr int kLdsGemm = 2 * (kLdsA + kLdsB);   // double buffered

// 16-byte chunk c of LDS row r lives at chunk c ^ swz(r): 8 consecutive rows (and
// the even/odd rows of 16 consecutive rows) land on distinct bank groups.
__device__ __forceinline__ int swz(int r) { return ((r >> 1) & 7) ^ ((r & 1) << 2); }

__device__ __forceinline__ float silu_f(float h) { return h / (1.0f + __expf(-h)); }

// m-tiles per expert, prefix summed into LDS by every workgroup:
// toff[e] = sum_{e'<e} ceil(M_e'/tile_rows), toff[E] = total (E <= 1024). Threads
// 0..255 do the work; a larger workgroup's other threads only join the barriers.
// Doing it in the kernel keeps the grouped GEMM a single launch.
constexpr int kMaxE = 1024;
__device__ __forceinline__ void build_tile_map(const int *__restrict__ expert_off, int E,
                                               int tile_rows, int64_t rows_alloc, int *toff,
                                               int *scratch /* [256] */) {
    const int tid = threadIdx.x;     // blockDim.x >= 256
    const bool act = tid < 256;
    int cnt[4], sum = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = tid * 4 + i;
        int c = 0;
        if (act && e < E) {
            const int64_t a = min<int64_t>(expert_off[e], rows_alloc);
            const int64_t b = min<int64_t>(expert_off[e + 1], rows_alloc);
            c = b > a ? int((b - a + tile_rows - 1) / tile_rows) : 0;
        }
        cnt[i] = c;
        sum += c;
    }
    int v = sum;
    for (int off = 1; off < 256; off <<= 1) {
        if (act) scratch[tid] = v;
        __syncthreads();
        if (act && tid >= off) v += scratch[tid - off];
        __syncthreads();
    }
    if (act) {
        int run = v - sum;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = tid * 4 + i;
            if (e < E) toff[e] = run;
            run += cnt[i];
        }
        if (tid == 255) toff[E] = v;     // inclusive sum of the last thread = total
    }
    __syncthreads();
}


// Work item -> (expert, n-tile, m-tile of that expert), ordered expert-major, then
// n-tile, then m-tile: the m-tiles that share one weight panel are adjacent, so in a
// persistent round they run together on one XCD and the panel is fetched once.
struct ItemCoord {
    int e, nt, mt;
};
__device__ __forceinline__ ItemCoord decode_item(int item, const int *tile_off, int E, int n_tiles) {
    int lo = 0, hi = E;                      // largest e with tile_off[e] * n_tiles <= item
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (tile_off[mid] * n_tiles <= item) lo = mid; else hi = mid;
    }
    const int rem = item - tile_off[lo] * n_tiles;
    const int mc = tile_off[lo + 1] - tile_off[lo];   // >= 1 for the expert found
    return {lo, rem / mc, rem % mc};
}

// Compute units of the current device (queried once per device).
inline int num_cus() {
    static PerDevice<int> pd;
    return per_device(pd, [] {
        int dev = 0, v = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
            return v;
        return 256;
    });
}

}  // namespace moe
