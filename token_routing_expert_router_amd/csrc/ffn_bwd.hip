// Backward of the expert FFN: four grouped GEMMs per expert on a 256 x 256 x 64 MFMA
// tile, eight wavefronts per workgroup as in the forward. With X, dO = dy_disp rows of
// expert e, h, u from the forward (hu_save), a = silu(h) * u:
//   G1  dA = dO W2            epilogue: dh = dA u s (1 + h (1 - s)), du = dA silu(h)
//                             (s = sigmoid(h)), stored as dHU = [dh du] in bf16, and a
//                             recomputed from h, u for G3
//   G2  dX = dHU W13          -> dx_disp (bf16)
//   G3  dW2 = dO^T a          -> dw2  (fp32), contraction over the expert's rows
//   G4  dW13 = dHU^T X        -> dw13 (fp32), contraction over the expert's rows
// The MFMA's A operand indexes the output's contiguous dimension and its B operand the
// output rows. Every A operand, and the B operand of G3/G4, is stored with the
// contraction dimension strided: such a tile is copied to LDS as it lies in memory (k
// rows of 256 contiguous elements, direct loads) and transposed on the way out by
// ds_read_b64_tr_b16, whose 16-lane groups hand lane 4a+b element b of the 8-byte
// pieces read by lanes a, a+4, a+8, a+12. Reductions over rows run in one fixed order
// per output (stages in row order, MFMA k order inside), so results are bitwise
// reproducible.
// Waves 0-3 move every stage (each the share of two waves); waves 4-7 carry all of the
// epilogue's global traffic. The tile leaves through LDS as whole 1 KiB rows, and only
// the loading waves ever wait for their vector-memory counter. So the storing waves'
// writes drain while the next item's stages load, instead of delaying its first stage.
#include "gemm_common.h"

namespace moe {
namespace {

enum { G1_DA = 0, G2_DX = 1, G3_DW2 = 2, G4_DW13 = 3 };

constexpr int kBwdThreads = 512;     // 8 waves: 4 A groups (64 rows) x 2 B groups (128 rows)
constexpr int kLoaderWaves = 4;      // waves that issue the direct loads; the others store

struct BwdArgs {
    const uint16_t *x_disp, *dy_disp, *hu, *w13, *w2;
    const int *expert_off;
    uint16_t *dhu, *act, *dx_disp;
    float *dw13, *dw2;
    int E, d, F;
    int64_t rows_alloc;
};

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int v2u32 __attribute__((ext_vector_type(2)));
typedef unsigned int v4u32 __attribute__((ext_vector_type(4)));

// Transposed tiles: 64 k rows of 512 B (256 elements); 16-byte chunk c of k row r lives
// at chunk c ^ swzT(r), so the four k rows one transposing read touches fall on
// distinct bank groups.
__device__ __forceinline__ int swzT(int r) { return (r & 3) << 2; }

// One operand's load state for the current item: where its tile data starts, how many
// bytes from there belong to it (loads past them read zeros), and the lane's byte offset
// for the even and the odd ones of the wave's four 1 KiB direct-load instructions of a
// stage (instruction j + 2 reads jstep bytes further on than instruction j).
struct Opnd {
    const char *base;
    int64_t nbytes;
    uint32_t off[2];
    uint32_t jstep;
    uint32_t vstep;          // from the lane's offsets for wave w to those for wave w + 1
    uint32_t kstep;          // bytes between consecutive stages
};

// Normal operand (rows K-contiguous, `ld` elements apart; at most 256 rows, so the
// byte count fits a buffer resource): instruction j of wave w moves tile rows
// 8(4w+j) .. +7 (128 B each); stages advance along the rows.
__device__ __forceinline__ void opnd_normal(Opnd &o, const uint16_t *base, int64_t nbytes, int ld,
                                            int wave, int lane) {
    o.base = reinterpret_cast<const char *>(base);
    o.nbytes = nbytes;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int r = (wave * 4 + j) * 8 + (lane >> 3);
        const int c = (lane & 7) ^ swz(r);      // swz(r + 16) == swz(r)
        o.off[j] = uint32_t((r * ld + c * 8) * 2);
    }
    o.jstep = uint32_t(16 * ld * 2);
    o.vstep = uint32_t(32 * ld * 2);
    o.kstep = BK * 2;
}

// Transposed operand (k rows `ld` elements apart, the tile's 256 columns from col0):
// instruction j of wave w moves k rows 2(4w+j), 2(4w+j)+1 of the stage; stages advance
// by 64 k rows, and each stage gets its own resource, so the byte count may exceed
// what one resource can describe.
__device__ __forceinline__ void opnd_trans(Opnd &o, const uint16_t *base, int64_t nbytes, int ld,
                                           int col0, int wave, int lane) {
    o.base = reinterpret_cast<const char *>(base);
    o.nbytes = nbytes;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int kr = (wave * 4 + j) * 2 + (lane >> 5);
        const int c = (lane & 31) ^ swzT(kr);   // swzT(kr + 4) == swzT(kr)
        o.off[j] = uint32_t((kr * ld + col0 + c * 8) * 2);
    }
    o.jstep = uint32_t(4 * ld * 2);
    o.vstep = uint32_t(8 * ld * 2);
    o.kstep = uint32_t(BK * ld * 2);
}

// The four direct loads are written as assembly: the compiler then has no LDS write of
// its own to order the transposing reads against (it would wait for every load in
// flight, the next stage's included, before each of them). The kernel orders them
// itself: each stage ends with s_waitcnt vmcnt(0) and a barrier before anyone reads it.
__device__ __forceinline__ void dma16(unsigned char *dst, __amdgpu_buffer_rsrc_t rs, uint32_t voff,
                                      uint32_t soff) {
    // m0 and soffset are wave-uniform; readfirstlane keeps them in scalar registers
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(uint32_t(reinterpret_cast<uintptr_t>(
        (__attribute__((address_space(3))) unsigned char *)dst)));
    const uint32_t so = __builtin_amdgcn_readfirstlane(soff);
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :: "s"(m0), "v"(voff), "s"(rs), "s"(so) : "memory", "m0");
}

// A buffer resource in scalar registers: base and size pass through readfirstlane, so
// the compiler knows them to be wave-uniform (they are) and never hands the "s" operand
// of the direct load a vector register.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(const char *base, int64_t nbytes) {
    const uint64_t pb = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(pb));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(pb >> 32));
    const int n = __builtin_amdgcn_readfirstlane(int(nbytes < 0x7fffffff ? nbytes : 0x7fffffff));
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>((uint64_t(hi) << 32) | lo), 0, n,
                                             0x00020000);
}

template <bool TR>
__device__ __forceinline__ void issue_opnd(unsigned char *tile, const Opnd &o, int kt, int wave) {
    __amdgpu_buffer_rsrc_t rs;
    uint32_t soff;
    if (TR) {
        const int64_t start = int64_t(kt) * o.kstep;
        rs = uniform_rsrc(o.base + start, o.nbytes - start);   // > 0: stages start inside the data
        soff = 0;
    } else {
        rs = uniform_rsrc(o.base, o.nbytes);
        soff = uint32_t(kt) * o.kstep;
    }
    // loader wave w moves the share of waves 2w and 2w + 1 (its offsets are those of 2w)
#pragma unroll
    for (int v = 0; v < 2; ++v)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            dma16(tile + ((2 * wave + v) * 4 + j) * 1024, rs, o.off[j & 1] + uint32_t(v) * o.vstep,
                  soff + uint32_t(j >> 1) * o.jstep);
}

// MFMA fragment (32 rows from row0, k16 step ks) of a normal tile
__device__ __forceinline__ bf16x8 frag_normal(const unsigned char *tile, int row0, int ks, int lane) {
    const int r = row0 + (lane & 31);
    const int kc = ks * 2 + (lane >> 5);
    return *reinterpret_cast<const bf16x8 *>(tile + r * 128 + ((kc ^ swz(r)) << 4));
}

// The same fragment of a transposed tile: lane l needs rows row0 + (l & 31), k values
// 16 ks + 8 (l >> 5) + 0..7; source lane s of its 16-lane group points at k row
// (s >> 2) (+4 for the second read) and the four columns 4 (s & 3) .. +3 of its half.
__device__ __forceinline__ bf16x8 frag_trans(const unsigned char *tile, int row0, int ks, int lane) {
    const int s = lane & 15;
    const int kr = ks * 16 + 8 * (lane >> 5) + (s >> 2);
    const int m = row0 + 16 * ((lane >> 4) & 1) + 4 * (s & 3);
    const int off = kr * 512 + (((m >> 3) ^ swzT(kr)) << 4) + (m & 7) * 2;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4 *)(tile + off));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4 *)(tile + off + 4 * 512));
    const s16x4 v8[2] = {lo, hi};
    return __builtin_bit_cast(bf16x8, v8);
}

template <bool TR>
__device__ __forceinline__ bf16x8 frag(const unsigned char *tile, int row0, int ks, int lane) {
    if (TR) return frag_trans(tile, row0, ks, lane);
    return frag_normal(tile, row0, ks, lane);
}

struct BwdItem {
    Opnd a, b;               // A: output columns, B: output rows
    int e;
    int64_t m0, m_end;       // the expert's token rows used by this item
    int a0, b0;              // first output column / output row of the tile (matrix coords)
    int KT;                  // LDS stages
};

template <int KIND>
__device__ __forceinline__ BwdItem make_bwd_item(const BwdArgs &A, int item, const int *tile_off,
                                                 int t_tiles, int n_tiles, int wave, int lane) {
    constexpr bool DGRAD = (KIND == G1_DA || KIND == G2_DX);
    const int d = A.d, F = A.F, F2 = 2 * F;
    BwdItem it;
    if (DGRAD) {
        const ItemCoord ic = decode_item(item, tile_off, A.E, n_tiles);
        it.e = ic.e;
        const int64_t e_lo = min<int64_t>(A.expert_off[ic.e], A.rows_alloc);
        const int64_t e_hi = min<int64_t>(A.expert_off[ic.e + 1], A.rows_alloc);
        const int mc = tile_off[ic.e + 1] - tile_off[ic.e];
        const int64_t rp = (e_hi - e_lo + mc - 1) / mc;     // equal m-tiles, <= BM
        it.m0 = e_lo + int64_t(ic.mt) * rp;
        it.m_end = min<int64_t>(e_hi, it.m0 + rp);
        it.a0 = ic.nt * BNW;
        it.b0 = 0;
        const int K = (KIND == G1_DA) ? d : F2;
        it.KT = K / BK;
        // B: the tile's token rows of dO (G1) or dHU (G2); rows past m_end read zeros
        const uint16_t *tb = (KIND == G1_DA) ? A.dy_disp : A.dhu;
        opnd_normal(it.b, tb + it.m0 * K, (it.m_end - it.m0) * K * 2, K, 2 * wave, lane);
        // A: W2_e [d][F] (G1) or W13_e [2F][d] (G2), k rows along the contraction
        if (KIND == G1_DA)
            opnd_trans(it.a, A.w2 + size_t(it.e) * d * F, int64_t(d) * F * 2, F, it.a0, 2 * wave, lane);
        else
            opnd_trans(it.a, A.w13 + size_t(it.e) * F2 * d, int64_t(F2) * d * 2, d, it.a0, 2 * wave, lane);
    } else {
        it.e = item / (t_tiles * n_tiles);
        const int rem = item % (t_tiles * n_tiles);
        it.b0 = (rem / n_tiles) * BM;
        it.a0 = (rem % n_tiles) * BNW;
        it.m0 = min<int64_t>(A.expert_off[it.e], A.rows_alloc);
        it.m_end = max(it.m0, min<int64_t>(A.expert_off[it.e + 1], A.rows_alloc));
        it.KT = int((it.m_end - it.m0 + BK - 1) / BK);
        const int64_t nr = it.m_end - it.m0;               // rows past these read zeros
        if (KIND == G3_DW2) {        // dW2[i][f] = sum_r dO[r][i] a[r][f]
            opnd_trans(it.a, A.act + it.m0 * F, nr * F * 2, F, it.a0, 2 * wave, lane);
            opnd_trans(it.b, A.dy_disp + it.m0 * d, nr * d * 2, d, it.b0, 2 * wave, lane);
        } else {                     // dW13[j][i] = sum_r dHU[r][j] X[r][i]
            opnd_trans(it.a, A.x_disp + it.m0 * d, nr * d * 2, d, it.a0, 2 * wave, lane);
            opnd_trans(it.b, A.dhu + it.m0 * F2, nr * F2 * 2, F2, it.b0, 2 * wave, lane);
        }
    }
    return it;
}

template <int KIND>
__device__ __forceinline__ void issue_bwd_stage(unsigned char *buf, int kt, const BwdItem &it,
                                                int wave) {
    constexpr bool BTR = !(KIND == G1_DA || KIND == G2_DX);
    if (wave >= kLoaderWaves) return;
    issue_opnd<BTR>(buf, it.b, kt, wave);
    issue_opnd<true>(buf + kLdsA, it.a, kt, wave);
}

// MFMAs of one stage held in buf
template <int KIND, int NW>
__device__ __forceinline__ void mma_bwd_stage(const unsigned char *buf, int arow, int brow, int lane,
                                              f32x16 (&acc)[4][2]) {
    constexpr bool BTR = !(KIND == G1_DA || KIND == G2_DX);
    const unsigned char *Bs = buf;
    const unsigned char *As = buf + kLdsA;
    bf16x8 wf[2][2], tf[2][4];
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
        if (ks == 0) {
#pragma unroll
            for (int s = 0; s < 2; ++s) wf[0][s] = frag<true>(As, arow + s * 32, 0, lane);
#pragma unroll
            for (int i = 0; i < NW; ++i) tf[0][i] = frag<BTR>(Bs, brow + i * 64, 0, lane);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (ks + 1 < BK / 16) {
            const int n = (ks + 1) & 1;
#pragma unroll
            for (int s = 0; s < 2; ++s) wf[n][s] = frag<true>(As, arow + s * 32, ks + 1, lane);
#pragma unroll
            for (int i = 0; i < NW; ++i) tf[n][i] = frag<BTR>(Bs, brow + i * 64, ks + 1, lane);
        }
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

// A storing wave's 16 rows of an LDS chunk (rows lrow0..lrow0+15 of the chunk buffer,
// tile rows trow0..): one row per instruction, lane j owning tile columns 4j..4j+3.
// Chunk rows are 1 KiB of fp32 with 16-byte piece p of row r at p ^ (r & 15). Global
// accesses are buffer operations on a resource that starts at the block's first row and
// ends after its last live row, with row rr as the scalar offset (on gfx950 the range
// check covers the scalar offset too: measured, loads past the end read zeros and
// stores are dropped). Rows past the item (rr >= live, a wave-uniform test) and lanes
// past the last column are also skipped explicitly.
template <int KIND>
__device__ __forceinline__ void store_rows(const unsigned char *cb, const BwdArgs &A,
                                           const BwdItem &it, int trow0, int lrow0, int lane) {
    const int d = A.d, F = A.F, F2 = 2 * F;
    auto rd = [&](int rr) {
        return *reinterpret_cast<const float4 *>(cb + (lrow0 + rr) * 1024 + ((lane ^ rr) << 4));
    };
    const int n = it.a0 + 4 * lane;
    if (KIND == G3_DW2 || KIND == G4_DW13) {
        // the weight gradients are written once and not read again by the layer:
        // non-temporal stores (the cache-policy nt bit) keep them from displacing the
        // operands in the caches (measured: expert backward 1419 -> 1373 us)
        constexpr int kStoreNT = 2;
        const int nrows = (KIND == G3_DW2) ? d : F2;
        const int ncols = (KIND == G3_DW2) ? F : d;
        const int r0 = it.b0 + trow0;
        const int live = max(0, min(16, nrows - r0));
        const float *out = (KIND == G3_DW2) ? A.dw2 + size_t(it.e) * d * F : A.dw13 + size_t(it.e) * F2 * d;
        const __amdgpu_buffer_rsrc_t rs =
            uniform_rsrc(reinterpret_cast<const char *>(out + size_t(r0) * ncols), int64_t(live) * ncols * 4);
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            float4 v[8];
#pragma unroll
            for (int rr = 0; rr < 8; ++rr) v[rr] = rd(8 * b + rr);
            if (n < ncols) {
#pragma unroll
                for (int rr = 0; rr < 8; ++rr)
                    if (8 * b + rr < live)
                        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u32, v[rr]), rs, n * 4,
                                                               (8 * b + rr) * ncols * 4, kStoreNT);
            }
        }
    } else if (KIND == G2_DX) {
        const int64_t r0 = it.m0 + trow0;
        const int live = int(max<int64_t>(0, min<int64_t>(16, it.m_end - r0)));
        const __amdgpu_buffer_rsrc_t rs =
            uniform_rsrc(reinterpret_cast<const char *>(A.dx_disp + r0 * d), int64_t(live) * d * 2);
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            float4 v[8];
#pragma unroll
            for (int rr = 0; rr < 8; ++rr) v[rr] = rd(8 * b + rr);
            if (n < d) {
#pragma unroll
                for (int rr = 0; rr < 8; ++rr)
                    if (8 * b + rr < live)
                        __builtin_amdgcn_raw_buffer_store_b64(
                            v2u32{pack_bf16x2(v[rr].x, v[rr].y), pack_bf16x2(v[rr].z, v[rr].w)}, rs, n * 2,
                            (8 * b + rr) * d * 2, 0);
            }
        }
    } else {
        // dA -> dh = dA u s (1 + h (1 - s)) = dA u (s + silu(h) (1 - s)), du = dA silu(h),
        // a = silu(h) u, with s = sigmoid(h) and silu(h) = h s; eight rows per batch, their
        // h and u loaded together
        const int64_t r0 = it.m0 + trow0;
        const int live = int(max<int64_t>(0, min<int64_t>(16, it.m_end - r0)));
        const __amdgpu_buffer_rsrc_t rhu =
            uniform_rsrc(reinterpret_cast<const char *>(A.hu + r0 * F2), int64_t(live) * F2 * 2);
        const __amdgpu_buffer_rsrc_t rdhu =
            uniform_rsrc(reinterpret_cast<const char *>(A.dhu + r0 * F2), int64_t(live) * F2 * 2);
        const __amdgpu_buffer_rsrc_t ract =
            uniform_rsrc(reinterpret_cast<const char *>(A.act + r0 * F), int64_t(live) * F * 2);
        const bool col = n < F;
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            v2u32 hv[8], uv[8];
#pragma unroll
            for (int rr = 0; rr < 8; ++rr) {
                hv[rr] = uv[rr] = v2u32{0u, 0u};
                if (8 * b + rr < live) {
                    hv[rr] = __builtin_amdgcn_raw_buffer_load_b64(rhu, n * 2, (8 * b + rr) * F2 * 2, 0);
                    uv[rr] = __builtin_amdgcn_raw_buffer_load_b64(rhu, (F + n) * 2, (8 * b + rr) * F2 * 2, 0);
                }
            }
#pragma unroll
            for (int rr = 0; rr < 8; ++rr) {
                const float4 dv = rd(8 * b + rr);
                const float da[4] = {dv.x, dv.y, dv.z, dv.w};
                const float h[4] = {bf16_lo(hv[rr][0]), bf16_hi(hv[rr][0]), bf16_lo(hv[rr][1]), bf16_hi(hv[rr][1])};
                const float u[4] = {bf16_lo(uv[rr][0]), bf16_hi(uv[rr][0]), bf16_lo(uv[rr][1]), bf16_hi(uv[rr][1])};
                float dh[4], du[4], av[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-h[q]));
                    const float hs = h[q] * sg;
                    av[q] = hs * u[q];
                    du[q] = da[q] * hs;
                    dh[q] = (da[q] * u[q]) * __builtin_fmaf(hs, 1.0f - sg, sg);
                }
                if (col && 8 * b + rr < live) {
                    const int so2 = (8 * b + rr) * F2 * 2, so1 = (8 * b + rr) * F * 2;
                    __builtin_amdgcn_raw_buffer_store_b64(v2u32{pack_bf16x2(dh[0], dh[1]), pack_bf16x2(dh[2], dh[3])},
                                                          rdhu, n * 2, so2, 0);
                    __builtin_amdgcn_raw_buffer_store_b64(v2u32{pack_bf16x2(du[0], du[1]), pack_bf16x2(du[2], du[3])},
                                                          rdhu, (F + n) * 2, so2, 0);
                    __builtin_amdgcn_raw_buffer_store_b64(v2u32{pack_bf16x2(av[0], av[1]), pack_bf16x2(av[2], av[3])},
                                                          ract, n * 2, so1, 0);
                }
            }
        }
    }
}

// One work item seen by one wave with NW (0..4) live 32-row sub-tiles of output rows.
template <int KIND, int NW>
__device__ __forceinline__ void run_bwd_item(unsigned char *lds, const BwdArgs &A,
                                             const BwdItem &it, BwdItem &next, int nitem,
                                             const int *tile_off, int t_tiles, int n_tiles,
                                             int wave, int lane) {
    const bool loader = wave < kLoaderWaves;
    const int wn = wave & 3, wm = wave >> 2;
    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < NW; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
    // output-row sub-tiles alternate between the two groups (group wm takes 32-row
    // sub-tiles wm, wm + 2, ...), so a SIMD's two wavefronts share a partly filled tile
    // evenly
    const int arow = wn * 64, brow = wm * 32;

    // stage 0 was issued before the previous item's epilogue (or before the first item)
    if (loader) __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int kt = 0; kt < it.KT; ++kt) {
        unsigned char *cur = lds + (kt & 1) * (kLdsA + kLdsB);
        if (kt + 1 < it.KT) issue_bwd_stage<KIND>(lds + ((kt + 1) & 1) * (kLdsA + kLdsB), kt + 1, it, wave);
        if (NW > 0) mma_bwd_stage<KIND, NW>(cur, arow, brow, lane, acc);
        if (loader) __builtin_amdgcn_s_waitcnt(0);   // this wave's loads of the next stage landed
        __syncthreads();                 // everyone's loads landed, and cur is free
    }

    // every wave is past its last LDS read: the next item's first stage flies into buffer 0
    // during this item's epilogue
    if (nitem >= 0) {
        next = make_bwd_item<KIND>(A, nitem, tile_off, t_tiles, n_tiles, wave, lane);
        if (next.KT > 0) issue_bwd_stage<KIND>(lds, 0, next, wave);
    }

    // epilogue through stage buffer 1, 64 tile rows at a time. The accumulators of lane l
    // are tile row brow + 64i + (l & 31) and, for v = 4g + q, tile column arow + 32s + 8g +
    // 4 (l >> 5) + q. Chunk c = tile rows 64c..64c+63 = sub-tile i = c of both groups.
    unsigned char *cb = lds + (kLdsA + kLdsB);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        if (c < NW) {
            const int rl = 32 * wm + (lane & 31);
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int pc = wn * 16 + 8 * s + 2 * g + (lane >> 5);
                    *reinterpret_cast<float4 *>(cb + rl * 1024 + ((pc ^ (rl & 15)) << 4)) =
                        make_float4(acc[c][s][4 * g], acc[c][s][4 * g + 1], acc[c][s][4 * g + 2],
                                    acc[c][s][4 * g + 3]);
                }
        }
        __syncthreads();
        if (!loader) {
            const int r0 = (wave - kLoaderWaves) * 16;
            store_rows<KIND>(cb, A, it, 64 * c + r0, r0, lane);
        }
        __syncthreads();
    }
}

template <int KIND>
__global__ __launch_bounds__(kBwdThreads) void k_gemm_bwd(BwdArgs A, int t_tiles, int n_tiles) {
    __shared__ __align__(16) unsigned char lds[2 * (kLdsA + kLdsB)];   // two stages
    __shared__ int tile_off[kMaxE + 1];
    __shared__ int map_scratch[256];
    constexpr bool DGRAD = (KIND == G1_DA || KIND == G2_DX);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int E = A.E;
    int total;
    if (DGRAD) {
        build_tile_map(A.expert_off, E, BM, A.rows_alloc, tile_off, map_scratch);
        total = tile_off[E] * n_tiles;
    } else {
        total = E * t_tiles * n_tiles;
    }
    const int G = gridDim.x;
    const int per = G / 8;
    const int slot = (G % 8 == 0) ? (blockIdx.x % 8) * per + blockIdx.x / 8 : blockIdx.x;
    if (slot >= total) return;

    BwdItem it = make_bwd_item<KIND>(A, slot, tile_off, t_tiles, n_tiles, wave, lane);
    if (it.KT > 0) issue_bwd_stage<KIND>(lds, 0, it, wave);
    for (int base = 0; base < total; base += G) {
        // rotating the slot each round spreads large and small items evenly
        const int nbase = base + G;
        const int nitem = nbase + (slot + nbase / G) % G;
        const bool has_next = nitem < total;
        BwdItem next;
        // live 32-row sub-tiles of output rows in this wave's half
        int nsub;
        if (DGRAD) nsub = int(min<int64_t>(8, (it.m_end - it.m0 + 31) / 32));
        else nsub = min(8, (((KIND == G3_DW2) ? A.d : 2 * A.F) - it.b0 + 31) / 32);
        const int nw = min(4, max(0, (nsub - (wave >> 2) + 1) / 2));
        switch (nw) {
        case 4: run_bwd_item<KIND, 4>(lds, A, it, next, has_next ? nitem : -1, tile_off, t_tiles, n_tiles, wave, lane); break;
        case 3: run_bwd_item<KIND, 3>(lds, A, it, next, has_next ? nitem : -1, tile_off, t_tiles, n_tiles, wave, lane); break;
        case 2: run_bwd_item<KIND, 2>(lds, A, it, next, has_next ? nitem : -1, tile_off, t_tiles, n_tiles, wave, lane); break;
        case 1: run_bwd_item<KIND, 1>(lds, A, it, next, has_next ? nitem : -1, tile_off, t_tiles, n_tiles, wave, lane); break;
        default: run_bwd_item<KIND, 0>(lds, A, it, next, has_next ? nitem : -1, tile_off, t_tiles, n_tiles, wave, lane); break;
        }
        if (!has_next) break;
        it = next;
    }
}

// Workspace: dHU [rows, 2F] then a [rows, F], both bf16.
size_t bwd_dhu_bytes(int64_t rows, int64_t F) { return align256(size_t(rows) * 2 * F * 2); }
size_t bwd_ws_bytes(int64_t rows, int64_t F) {
    return bwd_dhu_bytes(rows, F) + align256(size_t(rows) * F * 2);
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" size_t moe_expert_ffn_bwd_workspace_size(int32_t E, int64_t rows, int64_t d, int64_t F,
                                                    moe_dtype_t dtype) {
    (void)d;
    if (E <= 0 || rows < 0 || F <= 0 || dtype != MOE_BF16) return 0;
    return bwd_ws_bytes(rows, F);
}

extern "C" moe_status_t moe_expert_ffn_bwd(const void *x_disp, const void *dy_disp, const void *hu_save,
                                           const int32_t *expert_off, const void *w13, const void *w2,
                                           int32_t E, int64_t rows, int64_t d, int64_t F,
                                           moe_dtype_t dtype, void *dx_disp, float *dw13, float *dw2,
                                           void *ws, size_t ws_bytes, void *stream) {
    if (!valid_dtype(dtype) || E <= 0 || rows < 0 || d <= 0 || F <= 0) return MOE_ERR_INVALID_ARG;
    if (dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
    if (E > kMaxE || rows >= (int64_t(1) << 31) || d % BK != 0 || F % BK != 0 || d > (1 << 20) ||
        F > (1 << 20) || int64_t(d) * 2 * F * 2 >= (int64_t(1) << 31))
        return MOE_ERR_UNSUPPORTED;
    if (!x_disp || !dy_disp || !hu_save || !expert_off || !w13 || !w2 || !dx_disp || !dw13 || !dw2 ||
        !ws)
        return MOE_ERR_INVALID_ARG;
    if (ws_bytes < bwd_ws_bytes(rows, F)) return MOE_ERR_CAPACITY;
    if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return MOE_ERR_ALIGN;
    if (!aligned16(x_disp) || !aligned16(dy_disp) || !aligned16(hu_save) || !aligned16(w13) ||
        !aligned16(w2) || !aligned16(dx_disp) || !aligned16(dw13) || !aligned16(dw2))
        return MOE_ERR_ALIGN;
    const hipStream_t st = as_stream(stream);
    BwdArgs A;
    A.x_disp = static_cast<const uint16_t *>(x_disp);
    A.dy_disp = static_cast<const uint16_t *>(dy_disp);
    A.hu = static_cast<const uint16_t *>(hu_save);
    A.w13 = static_cast<const uint16_t *>(w13);
    A.w2 = static_cast<const uint16_t *>(w2);
    A.expert_off = expert_off;
    A.dhu = static_cast<uint16_t *>(ws);
    A.act = reinterpret_cast<uint16_t *>(static_cast<char *>(ws) + bwd_dhu_bytes(rows, F));
    A.dx_disp = static_cast<uint16_t *>(dx_disp);
    A.dw13 = dw13;
    A.dw2 = dw2;
    A.E = E;
    A.d = int(d);
    A.F = int(F);
    A.rows_alloc = rows;
    if (rows == 0) {
        // no rows: the weight gradients are still defined (zero)
    }
    const int cus = num_cus();
    const int64_t max_mt = cdiv(rows, BM) + E;
    {   // G1: dA -> dh, du
        const int nt = int(cdiv(F, BNW));
        const int g = int(std::min<int64_t>(max_mt * nt, cus));
        if (g > 0)
            hipLaunchKernelGGL(k_gemm_bwd<G1_DA>, dim3(g), dim3(kBwdThreads), 0, st, A, 0, nt);
    }
    {   // G3: dW2 (independent of G1)
        const int tt = int(cdiv(d, BM)), nt = int(cdiv(F, BNW));
        const int g = int(std::min<int64_t>(int64_t(E) * tt * nt, cus));
        hipLaunchKernelGGL(k_gemm_bwd<G3_DW2>, dim3(g), dim3(kBwdThreads), 0, st, A, tt, nt);
    }
    {   // G4: dW13 (before G2, so dx_disp is the last thing written)
        const int tt = int(cdiv(2 * F, BM)), nt = int(cdiv(d, BNW));
        const int g = int(std::min<int64_t>(int64_t(E) * tt * nt, cus));
        hipLaunchKernelGGL(k_gemm_bwd<G4_DW13>, dim3(g), dim3(kBwdThreads), 0, st, A, tt, nt);
    }
    {   // G2: dX
        const int nt = int(cdiv(d, BNW));
        const int g = int(std::min<int64_t>(max_mt * nt, cus));
        if (g > 0)
            hipLaunchKernelGGL(k_gemm_bwd<G2_DX>, dim3(g), dim3(kBwdThreads), 0, st, A, 0, nt);
    }
    return launch_status();
}
