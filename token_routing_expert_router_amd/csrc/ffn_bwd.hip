// Backward of the expert FFN: four grouped GEMMs per expert, on the same 256 x 256 x 64
// MFMA tile as the forward. With X, dO = dy_disp rows of expert e, h, u from the
// forward (hu_save), a = silu(h) * u:
//   G1  dA = dO W2            epilogue: dh = dA u s (1 + h (1 - s)), du = dA silu(h)
//                             (s = sigmoid(h)), stored as dHU = [dh du] in bf16
//   G2  dX = dHU W13          -> dx_disp (bf16)
//   G3  dW2 = dO^T a          -> dw2  (fp32), contraction over the expert's rows
//   G4  dW13 = dHU^T X        -> dw13 (fp32), contraction over the expert's rows
// Every one of them contracts over a dimension that is strided in at least one
// operand, so next to the direct global->LDS loads of the forward there is a
// transposing loader: a thread fetches an 8 (k) x 8 (n) block of bf16 with eight
// 16-byte loads, transposes it in registers with v_perm_b32 and writes eight
// K-contiguous 16-byte rows into the same swizzled LDS layout, so the MFMA fragment
// reads are unchanged. Reductions over rows run in one fixed order per output
// (stages in row order, MFMA k order inside), so results are bitwise reproducible.
#include "gemm_common.h"

namespace moe {
namespace {

enum { G1_DA = 0, G2_DX = 1, G3_DW2 = 2, G4_DW13 = 3 };

struct BwdArgs {
    const uint16_t *x_disp, *dy_disp, *hu, *w13, *w2;
    const int *expert_off;
    uint16_t *dhu, *dx_disp;
    float *dw13, *dw2;
    int E, d, F;
    int64_t rows_alloc;
};

// 8 x 8 block of bf16: reg[r] holds row krow0 + r (8 elements along n) of the stage
// that starts at the uniform byte pointer `base` (rows ldb bytes apart). Rows at or
// past kvalid, or a block with nok false, read as zero; their loads go to row 0 of
// the stage (always inside the matrix) so the code stays branch-free.
__device__ __forceinline__ void tload(u32x4 (&reg)[8], const char *base, uint32_t ldb, int krow0,
                                      int kvalid, uint32_t noff, bool nok) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        const int kr = krow0 + r;
        const bool ok = nok && kr < kvalid;
        const uint32_t off = uint32_t(ok ? kr : 0) * ldb + (nok ? noff : 0u);
        const u32x4 v = *reinterpret_cast<const u32x4 *>(base + off);
        reg[r] = ok ? v : u32x4{0u, 0u, 0u, 0u};
    }
}

// reg[r] <- bf16(silu(h) * u) with h = reg[r], u = ureg[r] (8 values each)
__device__ __forceinline__ void swiglu_rows(u32x4 (&reg)[8], const u32x4 (&ureg)[8]) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        uint32_t o[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t hv = reg[r][j], uv = ureg[r][j];
            o[j] = pack_bf16x2(silu_f(bf16_lo(hv)) * bf16_lo(uv), silu_f(bf16_hi(hv)) * bf16_hi(uv));
        }
        reg[r] = u32x4{o[0], o[1], o[2], o[3]};
    }
}

// Transpose the 8 x 8 block and store its 8 columns as K-contiguous 16-byte chunks:
// LDS row nb*8 + c (the n index), logical chunk kb (the k block), swizzled.
__device__ __forceinline__ void tstore(const u32x4 (&reg)[8], unsigned char *tile, int nb, int kb) {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const int j = c >> 1;
        const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;   // high or low halves
        u32x4 o;
        o.x = __builtin_amdgcn_perm(reg[1][j], reg[0][j], sel);
        o.y = __builtin_amdgcn_perm(reg[3][j], reg[2][j], sel);
        o.z = __builtin_amdgcn_perm(reg[5][j], reg[4][j], sel);
        o.w = __builtin_amdgcn_perm(reg[7][j], reg[6][j], sel);
        const int row = nb * 8 + c;
        *reinterpret_cast<u32x4 *>(tile + row * 128 + ((kb ^ swz(row)) << 4)) = o;
    }
}

template <int NS>
__device__ __forceinline__ void mma_stage(const unsigned char *Ts, const unsigned char *Ws, int lane,
                                          const int (&brow)[2], f32x16 (&acc)[NS][2]) {
    bf16x8 wf[2][2], tf[2][NS];
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
        auto rd = [&](int kss, bf16x8 (&w)[2], bf16x8 (&t)[NS]) {
            const int kc = kss * 2 + (lane >> 5);
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const int r = brow[s] + (lane & 31);
                w[s] = *reinterpret_cast<const bf16x8 *>(Ws + r * 128 + ((kc ^ swz(r)) << 4));
            }
#pragma unroll
            for (int i = 0; i < NS; ++i) {
                const int r = i * 32 + (lane & 31);
                t[i] = *reinterpret_cast<const bf16x8 *>(Ts + r * 128 + ((kc ^ swz(r)) << 4));
            }
        };
        if (ks == 0) rd(0, wf[0], tf[0]);
        if (ks + 1 < BK / 16) rd(ks + 1, wf[(ks + 1) & 1], tf[(ks + 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < NS; ++i)
#pragma unroll
            for (int s = 0; s < 2; ++s)
                acc[i][s] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[ks & 1][s], tf[ks & 1][i], acc[i][s], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
    }
}

struct BwdItem {
    int e;
    int64_t m0, m_end;   // the expert's token rows used by this item
    int t0;              // first T-side row (output row) of the tile
    int n0;              // first W-side row (output column) of the tile
    int KT;              // LDS stages
};

template <int KIND, int NS>
__device__ __forceinline__ void run_bwd_item(unsigned char *lds, const BwdArgs &A, const BwdItem &it,
                                             int wave, int lane) {
    constexpr bool DGRAD = (KIND == G1_DA || KIND == G2_DX);
    const int tid = threadIdx.x;
    const int d = A.d, F = A.F;
    const int F2 = 2 * F;

    // ---------------- operand geometry
    // T side (MFMA B, 256 rows shared by all waves)
    const uint16_t *Tsrc;        // DGRAD: token rows (direct); WGRAD: [K=rows][N] matrix
    int64_t ldT;
    int nT;                      // WGRAD: size of the T side
    if (KIND == G1_DA) { Tsrc = A.dy_disp; ldT = d; nT = 0; }
    else if (KIND == G2_DX) { Tsrc = A.dhu; ldT = F2; nT = 0; }
    else if (KIND == G3_DW2) { Tsrc = A.dy_disp; ldT = d; nT = d; }
    else { Tsrc = A.dhu; ldT = F2; nT = F2; }
    // W side (MFMA A, 64 rows per wave), always loaded through the transposing path
    const uint16_t *Wsrc;
    int64_t ldW;
    int nW;
    int64_t k_endW;
    if (KIND == G1_DA) { Wsrc = A.w2 + size_t(it.e) * d * F; ldW = F; nW = F; k_endW = d; }
    else if (KIND == G2_DX) { Wsrc = A.w13 + size_t(it.e) * F2 * d; ldW = d; nW = d; k_endW = F2; }
    else if (KIND == G3_DW2) { Wsrc = A.hu; ldW = F2; nW = F; k_endW = it.m_end; }
    else { Wsrc = A.x_disp; ldW = d; nW = d; k_endW = it.m_end; }
    const int64_t kW0 = DGRAD ? 0 : it.m0;     // first k row of the W side

    const int nb = tid & 31, kb = tid >> 5;    // this thread's 8 x 8 block of a 256 x 64 tile

    // direct-load offsets of the T side (DGRAD only), as in the forward
    uint32_t a_off[8];
    int a_groups = 0;
    const char *Tb = nullptr;
    if (DGRAD) {
        const int lrow = lane >> 3, pchunk = lane & 7;
        Tb = reinterpret_cast<const char *>(Tsrc + it.m0 * ldT);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int g = wave * 8 + j;
            const int r = g * 8 + lrow;
            const int c = pchunk ^ swz(r);
            const int64_t tr = min<int64_t>(it.m0 + r, A.rows_alloc - 1);
            a_off[j] = uint32_t(((tr - it.m0) * ldT + c * 8) * 2);
            if (it.m0 + g * 8 < it.m_end) a_groups = j + 1;
        }
    }

    f32x16 acc[NS][2];
#pragma unroll
    for (int i = 0; i < NS; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
    int brow[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) brow[s] = wave * 64 + s * 32;

    u32x4 rW[8], rU[8], rT[8];
    const uint32_t ldbT = uint32_t(ldT * 2), ldbW = uint32_t(ldW * 2);
    const int krow0 = kb * 8;                 // this thread's first row inside a stage
    const uint32_t noffT = uint32_t((it.t0 + nb * 8) * 2);
    const bool nokT = it.t0 + nb * 8 < nT;
    const uint32_t noffW = uint32_t((it.n0 + nb * 8) * 2);
    const bool nokW = it.n0 + nb * 8 < nW;
    const char *Tbase = reinterpret_cast<const char *>(Tsrc) + it.m0 * ldT * 2;
    const char *Wbase = reinterpret_cast<const char *>(Wsrc) + kW0 * ldW * 2;
    auto issue = [&](int stage, int kt) {
        unsigned char *Ts = lds + stage * (kLdsA + kLdsB);
        if (DGRAD) {
            const char *Tk = Tb + size_t(kt) * BK * 2;
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (j < a_groups)
                    __builtin_amdgcn_global_load_lds(
                        Tk + a_off[j],
                        (__attribute__((address_space(3))) void *)(Ts + (wave * 8 + j) * 1024), 16, 0, 0);
        } else {
            const int kvalid = int(min<int64_t>(BK, it.m_end - it.m0 - int64_t(kt) * BK));
            tload(rT, Tbase + size_t(kt) * BK * ldbT, ldbT, krow0, kvalid, noffT, nokT);
        }
        const int kvalidW = DGRAD ? BK : int(min<int64_t>(BK, k_endW - kW0 - int64_t(kt) * BK));
        const char *Wk = Wbase + size_t(kt) * BK * ldbW;
        tload(rW, Wk, ldbW, krow0, kvalidW, noffW, nokW);
        if (KIND == G3_DW2) tload(rU, Wk + size_t(F) * 2, ldbW, krow0, kvalidW, noffW, nokW);
    };
    auto commit = [&](int stage) {
        unsigned char *Ts = lds + stage * (kLdsA + kLdsB);
        unsigned char *Ws = Ts + kLdsA;
        if (KIND == G3_DW2) swiglu_rows(rW, rU);
        tstore(rW, Ws, nb, kb);
        if (!DGRAD) tstore(rT, Ts, nb, kb);
    };

    __syncthreads();                 // the previous item's readers are done with LDS
    if (it.KT > 0) {
        issue(0, 0);
        commit(0);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }
    for (int kt = 0; kt < it.KT; ++kt) {
        const int cur = kt & 1;
        const bool more = kt + 1 < it.KT;
        if (more) issue(cur ^ 1, kt + 1);
        const unsigned char *Ts = lds + cur * (kLdsA + kLdsB);
        mma_stage<NS>(Ts, Ts + kLdsA, lane, brow, acc);
        if (more) commit(cur ^ 1);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }

    // ---------------- epilogues: lane holds T-side row (lane & 31) of each 32-row
    // sub-tile and, for v = 4g + q, W-side row 8g + 4*(lane >> 5) + q of each of its
    // two 32-row weight sub-tiles: four consecutive outputs of one output row.
    const int nl = 4 * (lane >> 5);
#pragma unroll
    for (int i = 0; i < NS; ++i) {
        if (DGRAD) {
            const int64_t m = it.m0 + i * 32 + (lane & 31);
            if (m >= it.m_end) continue;
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int n = it.n0 + wave * 64 + s * 32 + 8 * g + nl;
                    if (n >= nW) continue;
                    if (KIND == G1_DA) {
                        const uint2 hv = *reinterpret_cast<const uint2 *>(A.hu + m * F2 + n);
                        const uint2 uv = *reinterpret_cast<const uint2 *>(A.hu + m * F2 + F + n);
                        float h[4] = {bf16_lo(hv.x), bf16_hi(hv.x), bf16_lo(hv.y), bf16_hi(hv.y)};
                        float u[4] = {bf16_lo(uv.x), bf16_hi(uv.x), bf16_lo(uv.y), bf16_hi(uv.y)};
                        float dh[4], du[4];
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const float da = acc[i][s][4 * g + q];
                            const float sg = 1.0f / (1.0f + __expf(-h[q]));
                            dh[q] = da * u[q] * sg * (1.0f + h[q] * (1.0f - sg));
                            du[q] = da * h[q] * sg;
                        }
                        uint2 ph, pu;
                        ph.x = pack_bf16x2(dh[0], dh[1]);
                        ph.y = pack_bf16x2(dh[2], dh[3]);
                        pu.x = pack_bf16x2(du[0], du[1]);
                        pu.y = pack_bf16x2(du[2], du[3]);
                        *reinterpret_cast<uint2 *>(A.dhu + m * F2 + n) = ph;
                        *reinterpret_cast<uint2 *>(A.dhu + m * F2 + F + n) = pu;
                    } else {
                        uint2 p;
                        p.x = pack_bf16x2(acc[i][s][4 * g], acc[i][s][4 * g + 1]);
                        p.y = pack_bf16x2(acc[i][s][4 * g + 2], acc[i][s][4 * g + 3]);
                        *reinterpret_cast<uint2 *>(A.dx_disp + m * d + n) = p;
                    }
                }
        } else {
            const int trow = it.t0 + i * 32 + (lane & 31);
            if (trow >= nT) continue;
            float *out = (KIND == G3_DW2) ? A.dw2 + size_t(it.e) * d * F + size_t(trow) * F
                                          : A.dw13 + size_t(it.e) * F2 * d + size_t(trow) * d;
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int n = it.n0 + wave * 64 + s * 32 + 8 * g + nl;
                    if (n >= nW) continue;
                    *reinterpret_cast<float4 *>(out + n) =
                        make_float4(acc[i][s][4 * g], acc[i][s][4 * g + 1], acc[i][s][4 * g + 2],
                                    acc[i][s][4 * g + 3]);
                }
        }
    }
}

template <int KIND>
__global__ __launch_bounds__(kGemmThreads, 1) void k_gemm_bwd(BwdArgs A, int t_tiles, int n_tiles) {
    extern __shared__ __align__(16) unsigned char lds[];
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
    const int Kd = (KIND == G1_DA) ? A.d : 2 * A.F;
    const int G = gridDim.x;
    const int per = G / 8;
    const int slot = (G % 8 == 0) ? (blockIdx.x % 8) * per + blockIdx.x / 8 : blockIdx.x;
    for (int base = 0; base < total; base += G) {
        // rotating the slot each round spreads large and small items evenly
        const int item = base + (slot + base / G) % G;
        if (item >= total) break;
        BwdItem it;
        int nsub;
        if (DGRAD) {
            const ItemCoord ic = decode_item(item, tile_off, E, n_tiles);
            it.e = ic.e;
            it.m0 = int64_t(A.expert_off[ic.e]) + int64_t(ic.mt) * BM;
            it.m_end = min<int64_t>(A.expert_off[ic.e + 1], A.rows_alloc);
            it.t0 = 0;
            it.n0 = ic.nt * BNW;
            it.KT = Kd / BK;
            nsub = int(min<int64_t>(8, (it.m_end - it.m0 + 31) / 32));
        } else {
            it.e = item / (t_tiles * n_tiles);
            const int rem = item % (t_tiles * n_tiles);
            const int tt = rem / n_tiles, nt = rem % n_tiles;
            it.m0 = min<int64_t>(A.expert_off[it.e], A.rows_alloc);
            it.m_end = max(it.m0, min<int64_t>(A.expert_off[it.e + 1], A.rows_alloc));
            it.t0 = tt * BM;
            it.n0 = nt * BNW;
            it.KT = int((it.m_end - it.m0 + BK - 1) / BK);
            const int nT = (KIND == G3_DW2) ? A.d : 2 * A.F;
            nsub = min(8, (nT - it.t0 + 31) / 32);
        }
        switch (nsub) {
        case 8: run_bwd_item<KIND, 8>(lds, A, it, wave, lane); break;
        case 7: run_bwd_item<KIND, 7>(lds, A, it, wave, lane); break;
        case 6: run_bwd_item<KIND, 6>(lds, A, it, wave, lane); break;
        case 5: run_bwd_item<KIND, 5>(lds, A, it, wave, lane); break;
        case 4: run_bwd_item<KIND, 4>(lds, A, it, wave, lane); break;
        case 3: run_bwd_item<KIND, 3>(lds, A, it, wave, lane); break;
        case 2: run_bwd_item<KIND, 2>(lds, A, it, wave, lane); break;
        default: run_bwd_item<KIND, 1>(lds, A, it, wave, lane); break;
        }
    }
}

bool set_bwd_lds_limits() {
    static int ok = -1;
    if (ok < 0) {
        ok = 1;
        const void *fns[4] = {reinterpret_cast<const void *>(&k_gemm_bwd<G1_DA>),
                              reinterpret_cast<const void *>(&k_gemm_bwd<G2_DX>),
                              reinterpret_cast<const void *>(&k_gemm_bwd<G3_DW2>),
                              reinterpret_cast<const void *>(&k_gemm_bwd<G4_DW13>)};
        for (const void *f : fns)
            if (hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsGemm) != hipSuccess)
                ok = 0;
    }
    return ok == 1;
}

size_t bwd_ws_bytes(int64_t rows, int64_t F) { return align256(size_t(rows) * 2 * F * 2); }

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
        F > (1 << 20) || int64_t(d) * 2 * F >= (int64_t(1) << 31))
        return MOE_ERR_UNSUPPORTED;
    if (!x_disp || !dy_disp || !hu_save || !expert_off || !w13 || !w2 || !dx_disp || !dw13 || !dw2 ||
        !ws)
        return MOE_ERR_INVALID_ARG;
    if (ws_bytes < bwd_ws_bytes(rows, F)) return MOE_ERR_CAPACITY;
    if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return MOE_ERR_ALIGN;
    if (!aligned16(x_disp) || !aligned16(dy_disp) || !aligned16(hu_save) || !aligned16(w13) ||
        !aligned16(w2) || !aligned16(dx_disp) || !aligned16(dw13) || !aligned16(dw2))
        return MOE_ERR_ALIGN;
    if (!set_bwd_lds_limits()) return MOE_ERR_HIP;     // first HIP call: all checks done
    const hipStream_t st = as_stream(stream);
    BwdArgs A;
    A.x_disp = static_cast<const uint16_t *>(x_disp);
    A.dy_disp = static_cast<const uint16_t *>(dy_disp);
    A.hu = static_cast<const uint16_t *>(hu_save);
    A.w13 = static_cast<const uint16_t *>(w13);
    A.w2 = static_cast<const uint16_t *>(w2);
    A.expert_off = expert_off;
    A.dhu = static_cast<uint16_t *>(ws);
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
            hipLaunchKernelGGL(k_gemm_bwd<G1_DA>, dim3(g), dim3(kGemmThreads), kLdsGemm, st, A, 0, nt);
    }
    {   // G3: dW2 (independent of G1)
        const int tt = int(cdiv(d, BM)), nt = int(cdiv(F, BNW));
        const int g = int(std::min<int64_t>(int64_t(E) * tt * nt, cus));
        hipLaunchKernelGGL(k_gemm_bwd<G3_DW2>, dim3(g), dim3(kGemmThreads), kLdsGemm, st, A, tt, nt);
    }
    {   // G2: dX
        const int nt = int(cdiv(d, BNW));
        const int g = int(std::min<int64_t>(max_mt * nt, cus));
        if (g > 0)
            hipLaunchKernelGGL(k_gemm_bwd<G2_DX>, dim3(g), dim3(kGemmThreads), kLdsGemm, st, A, 0, nt);
    }
    {   // G4: dW13
        const int tt = int(cdiv(2 * F, BM)), nt = int(cdiv(d, BNW));
        const int g = int(std::min<int64_t>(int64_t(E) * tt * nt, cus));
        hipLaunchKernelGGL(k_gemm_bwd<G4_DW13>, dim3(g), dim3(kGemmThreads), kLdsGemm, st, A, tt, nt);
    }
    return launch_status();
}
