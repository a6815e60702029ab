// Dispatch: the plan (per-expert counts, offsets, a stable slot per (token, expert)
// pair) and the copy of each token into its slots, plus the copy's transpose for the
// backward. [EFA] = Perplexity, "Enabling trillion-parameter models on AWS EFA"
// (2025). Section "Dispatch and combine": per-expert token counts are accumulated
// atomically in the shared memory of one block, and their cumulative sum gives the
// offsets that pack tokens into contiguous per-destination send buffers. Section
// "Send and receive buffers": each sender's rows at a destination are one
// contiguous chunk (one write per peer); a destination receives at most
// N*T*max(R, E/N) rows.
//
// Plan kernels (deterministic, no order-dependent atomics):
//   k_plan_count  one workgroup per 256-token block of one source: every pair sets
//                 bit (t mod 256) of its expert's 256-bit mask in LDS (atomic OR,
//                 whose result does not depend on the order); popcounts are the
//                 block's per-expert counts, and a pair's rank inside its expert is the
//                 popcount of the mask bits below its token, so tokens keep their order
//                 inside every expert. The ranks (< 256) go to the workspace as bytes.
//   k_plan_scan   one workgroup: per-source counts, expert offsets, chunk offsets
//                 per destination, and the first row of every (block, expert);
//                 k_plan_scan_em is the short form for the expert-major layout.
//   k_plan_copy   one wavefront per token: its k slots (first row of its block and
//                 expert + its rank), the unused-row marks, then the row copy: the row
//                 is read once with 16-byte loads and written to each of its k rows
//                 (1 KiB per wavefront instruction).
// Prefix sums in k_plan_scan are segmented scans built from wavefront shuffles.
#include "common.h"

#include <algorithm>

namespace moe {
namespace {

constexpr int kPlanBlock = 256;                 // tokens per plan block
constexpr int kMaskWords = kPlanBlock / 64;     // 64-bit words per expert mask
constexpr int kScanThreads = 1024;
constexpr int kScanLdsInts = 32768;             // 128 KiB of LDS for the scan

struct PlanGeom {
    int T, k, E, n_src, n_dst, Ts, bps, B, epr;
    int64_t cap;
    FastDiv dE, dbps, depr, dTs, dcap;   // the same divisors, as multiply-shifts
    // rank-major layout with one plan block per source and at most 64 experts per
    // destination: the count kernel also takes each source's chunk sizes and the offset
    // of every expert inside its chunk, and the scan only joins the sources
    bool rm1;
};

PlanGeom make_geom(int64_t T, int32_t E, int32_t k, const moe_layout_t *lay) {
    PlanGeom g;
    g.T = int(T);
    g.k = k;
    g.E = E;
    g.n_src = lay ? lay->n_src : 1;
    g.n_dst = lay ? lay->n_dst : 1;
    g.cap = lay ? lay->cap_rows_per_dst : T * k;
    g.Ts = g.T / g.n_src;
    g.bps = int(cdiv(g.Ts, kPlanBlock));
    g.B = g.n_src * g.bps;
    g.epr = E / g.n_dst;
    g.dE = FastDiv(uint32_t(g.E));
    g.dbps = FastDiv(uint32_t(std::max(g.bps, 1)));
    g.depr = FastDiv(uint32_t(std::max(g.epr, 1)));
    g.dTs = FastDiv(uint32_t(std::max(g.Ts, 1)));
    g.dcap = FastDiv(uint32_t(std::max<int64_t>(std::min<int64_t>(g.cap, 0x7fffffff), 1)));
    g.rm1 = (g.n_src > 1 || g.n_dst > 1) && g.bps == 1 && g.epr <= 64 &&
            int64_t(g.n_dst) * (g.n_src + 1) <= 16384;   // its chunk table fits 64 KiB of LDS
    return g;
}

// Workspace: [0,256) status flag; blk_flags [B]; blk_counts [B][E]; blk_base [B][E];
// rank [T*k] bytes. The flag is overwritten (never accumulated across calls) and every
// other entry a call reads it has written first, so nothing needs clearing.
// With the one-block-per-source path also: within [B][E] (rows before expert e inside
// its destination chunk) and csize [B][n_dst] (rows the source sends to each
// destination).
struct WsLayout {
    size_t flags, counts, base, rank, within, csize, total;
};
WsLayout ws_layout(const PlanGeom &g) {
    WsLayout l;
    l.flags = 256;
    l.counts = l.flags + align256(size_t(g.B) * sizeof(int));
    l.base = l.counts + align256(size_t(g.B) * g.E * sizeof(int));
    l.rank = l.base + align256(size_t(g.B) * g.E * sizeof(int));
    l.within = l.rank + align256(size_t(g.T) * g.k);
    l.csize = l.within + (g.rm1 ? align256(size_t(g.B) * g.E * sizeof(int)) : 0);
    l.total = l.csize + (g.rm1 ? align256(size_t(g.B) * g.n_dst * sizeof(int)) : 0);
    return l;
}
size_t ws_bytes_for(const PlanGeom &g) { return ws_layout(g).total; }

constexpr int kMaxK = 32;

// sum_{i < n} a[i * stride] with eight LDS loads in flight
__device__ __forceinline__ int lds_strided_sum(const int *a, int n, int stride) {
    int c = 0, i = 0;
    for (; i + 8 <= n; i += 8) {
        int w[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) w[u] = a[(i + u) * stride];
#pragma unroll
        for (int u = 0; u < 8; ++u) c += w[u];
    }
    for (; i < n; ++i) c += a[i * stride];
    return c;
}


// Counts and ranks of one plan block. Thread t loads its token's k expert ids first
// (all loads in flight together), then sets its bits.
__global__ __launch_bounds__(kPlanBlock) void k_plan_count(const int *__restrict__ idx, PlanGeom g,
                                                          int *__restrict__ blk_counts,
                                                          int *__restrict__ blk_flags,
                                                          unsigned char *__restrict__ rank,
                                                          int *__restrict__ within,
                                                          int *__restrict__ csize) {
    extern __shared__ unsigned long long masks[];
    int *cnt_l = reinterpret_cast<int *>(masks + g.E * kMaskWords);   // [E], rm1 only
    __shared__ int bflag;
    const int b = blockIdx.x;
    const int s = b / g.bps, tb = (b % g.bps) * kPlanBlock;
    const int n = min(kPlanBlock, g.Ts - tb);
    const int t = threadIdx.x;
    const size_t p0 = size_t(s * g.Ts + tb + t) * g.k;      // this token's first pair
    int ev[kMaxK];
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) ev[j] = (j < g.k && t < n) ? idx[p0 + j] : -1;
    if (t == 0) bflag = 0;
    for (int i = t; i < g.E * kMaskWords; i += blockDim.x) masks[i] = 0ull;
    __syncthreads();
    const unsigned long long bit = 1ull << (t & 63);
    if (t < n) {
        int fl = 0;
#pragma unroll
        for (int j = 0; j < kMaxK; ++j) {
            if (j >= g.k) break;
            const int e = ev[j];
            if (e < 0 || e >= g.E) {
                fl = kFlagBadIndex;
                continue;
            }
            const unsigned long long old = atomicOr(&masks[e * kMaskWords + (t >> 6)], bit);
            if (old & bit) fl = kFlagBadIndex;              // expert listed twice
        }
        if (fl) atomicOr(&bflag, fl);
    }
    __syncthreads();
    if (t == 0) blk_flags[b] = bflag;
    for (int e = t; e < g.E; e += blockDim.x) {
        int c = 0;
#pragma unroll
        for (int w = 0; w < kMaskWords; ++w) c += __popcll(masks[e * kMaskWords + w]);
        blk_counts[size_t(b) * g.E + e] = c;
        if (g.rm1) cnt_l[e] = c;
    }
    if (g.rm1) {
        __syncthreads();
        // this source's rows before expert e inside its chunk for e's destination, and
        // its chunk size per destination (at most 64 experts per destination)
        for (int e = t; e < g.E; e += blockDim.x) {
            const int r0 = g.depr.div(e) * g.epr;
            within[size_t(b) * g.E + e] = lds_strided_sum(cnt_l + r0, e - r0, 1);
        }
        for (int r = t; r < g.n_dst; r += blockDim.x)
            csize[size_t(b) * g.n_dst + r] = lds_strided_sum(cnt_l + r * g.epr, g.epr, 1);
    }
    if (t < n) {
#pragma unroll
        for (int j = 0; j < kMaxK; ++j) {
            if (j >= g.k) break;
            const int e = ev[j];
            int r = 0;
            if (e >= 0 && e < g.E) {
                const unsigned long long *m = masks + e * kMaskWords;
                for (int w = 0; w < (t >> 6); ++w) r += __popcll(m[w]);
                r += __popcll(m[t >> 6] & (bit - 1ull));
            }
            rank[p0 + j] = static_cast<unsigned char>(r);
        }
    }
}

// Block-wide exclusive scan of a[0..n) in LDS, restarting at every multiple of L
// (segments of length L). Each thread scans a contiguous chunk serially; the chunk
// aggregates (segment-start flag, sum) are combined by a segmented scan with
// wavefront shuffles, then across the 16 wavefronts through LDS; the carry is added
// to the chunk's elements before its first segment start. seg_total[s] (if
// non-null) receives the sum of segment s. Two barriers, whatever n is.
__device__ void seg_exclusive_scan(int *a, int n, int L, int *seg_total, int *wf_flag,
                                   int *wf_sum /* [kScanThreads / 64] each */) {
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int per = (n + kScanThreads - 1) / kScanThreads;
    const int lo = min(n, tid * per), hi = min(n, lo + per);
    int run = 0, flag = 0;
    int seg = lo / L, pos = lo - seg * L;             // position inside the segment, tracked
    for (int i = lo; i < hi; ++i) {
        if (pos == 0) {
            run = 0;
            flag = 1;
        }
        const int v = a[i];
        a[i] = run;
        run += v;
        if (pos == L - 1) {
            if (seg_total) seg_total[seg] = v;       // keep the last value
            pos = 0;
            ++seg;
        } else {
            ++pos;
        }
    }
    // inclusive segmented scan over the lanes of this wavefront
    int f = flag, v = run;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int of = __shfl_up(f, off, 64), ov = __shfl_up(v, off, 64);
        if (lane >= off && !f) {
            v += ov;
            f = of;
        }
    }
    if (lane == 63) {
        wf_flag[wave] = f;
        wf_sum[wave] = v;
    }
    __syncthreads();
    // carry from the wavefronts before this one
    int cf = 0, cv = 0;
    for (int w = 0; w < wave; ++w) {
        if (wf_flag[w]) {
            cf = 1;
            cv = wf_sum[w];
        } else {
            cv += wf_sum[w];
        }
    }
    if (!f) v += cv;                     // this lane's inclusive value, carry included
    int prev = __shfl_up(v, 1, 64);      // exclusive carry into this chunk
    if (lane == 0) prev = cv;
    (void)cf;
    for (int i = lo, p = lo - (lo / L) * L; i < hi; ++i, ++p) {
        if (p == L) p = 0;
        if (p == 0) break;
        a[i] += prev;
    }
    __syncthreads();
    if (seg_total) {
        for (int sg = tid; sg < n / L; sg += kScanThreads) seg_total[sg] += a[sg * L + L - 1];
        __syncthreads();
    }
}


// One workgroup, everything in LDS:
//   bct [ns][E][bps]  block counts, then their prefix over the source's blocks
//   cnt [ns][E]       per-source counts, then rows before e inside its chunk
//   tot [E+1]         per-expert totals, then expert_off
//   chk [nd][ns+1]    chunk sizes (sender order), then chunk offsets
__global__ __launch_bounds__(kScanThreads) void k_plan_scan(
    const int *__restrict__ blk_counts, const int *__restrict__ blk_flags, PlanGeom g,
    int *__restrict__ counts, int *__restrict__ expert_off, int *__restrict__ chunk_off,
    int *__restrict__ blk_base, int *__restrict__ flag) {
    extern __shared__ int lds[];
    __shared__ int sflag;
    __shared__ int tf[kScanThreads / 64], ts[kScanThreads / 64];
    const int E = g.E, ns = g.n_src, nd = g.n_dst, epr = g.epr, bps = g.bps;
    int *bct = lds;
    int *cnt = bct + ns * E * bps;
    int *tot = cnt + ns * E;
    int *chk = tot + E + 1;
    int *segt = chk + nd * (ns + 1);            // [ns * nd] chunk sizes
    const int tid = threadIdx.x;
    if (tid == 0) sflag = 0;
    __syncthreads();
    for (int b = tid; b < g.B; b += kScanThreads)
        if (blk_flags[b]) atomicOr(&sflag, blk_flags[b]);
    // block counts, transposed so that one (source, expert)'s blocks are contiguous;
    // every thread loads 16 consecutive-in-memory counts per round, all in flight
    {
        const int n = g.B * E;
        for (int c0 = 0; c0 < n; c0 += 16 * kScanThreads) {
            int v[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                const int c = c0 + u * kScanThreads + tid;
                v[u] = c < n ? blk_counts[c] : 0;
            }
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                const int c = c0 + u * kScanThreads + tid;
                if (c < n) {
                    const int b = g.dE.div(c), e = c - b * E;
                    const int s = g.dbps.div(b), bb = b - s * bps;
                    bct[(s * E + e) * bps + bb] = v[u];
                }
            }
        }
    }
    __syncthreads();
    // per-source counts, prefix over each source's blocks
    for (int se = tid; se < ns * E; se += kScanThreads) {
        const int c = lds_strided_sum(bct + se * bps, bps, 1);
        cnt[se] = c;
        counts[se] = c;
    }
    __syncthreads();
    seg_exclusive_scan(bct, ns * E * bps, bps, nullptr, tf, ts);
    for (int e = tid; e < E; e += kScanThreads) tot[e] = lds_strided_sum(cnt + e, ns, E);
    __syncthreads();
    // rows before expert e inside (source s -> its destination); chunk sizes
    seg_exclusive_scan(cnt, ns * E, epr, segt, tf, ts);
    // chunk offsets of every destination in sender order: chk[r][s]
    for (int i = tid; i < nd * ns; i += kScanThreads) {
        const int r = i / ns, s = i % ns;
        chk[r * (ns + 1) + s] = segt[s * nd + r];
    }
    __syncthreads();
    for (int r = tid; r < nd; r += kScanThreads) chk[r * (ns + 1) + ns] = 0;
    __syncthreads();
    seg_exclusive_scan(chk, nd * (ns + 1), ns + 1, nullptr, tf, ts);
    for (int i = tid; i < nd * (ns + 1); i += kScanThreads) {
        chunk_off[i] = chk[i];
        if (i % (ns + 1) == ns && int64_t(chk[i]) > g.cap) atomicOr(&sflag, kFlagCapacity);
    }
    // expert offsets
    tot[E] = 0;
    __syncthreads();
    seg_exclusive_scan(tot, E + 1, E + 1, nullptr, tf, ts);
    for (int e = tid; e <= E; e += kScanThreads) expert_off[e] = tot[e];
    __syncthreads();
    if (tid == 0) *flag = sflag;      // overwrites the previous call's flag
    // first row of every (block, expert), all B*E of them in parallel
    for (int c = tid; c < g.B * E; c += kScanThreads) {
        const int b = g.dE.div(c), e = c - b * E;
        const int s = g.dbps.div(b), bb = b - s * bps;
        const int r = g.depr.div(e);
        blk_base[c] = int(int64_t(r) * g.cap) + chk[r * (ns + 1) + s] + cnt[s * E + e] +
                      bct[(s * E + e) * bps + bb];
    }
}

// The plan's scan for the rank-major layout with one block per source (rm1): the
// count kernel already left each source's chunk sizes csize[s][r] and the rows before
// every expert inside its chunk, within[s][e]; this joins the sources.
//   chunk_off[r][s] = sum_{s' < s} csize[s'][r]   (one thread per destination)
//   expert_off      = exclusive scan of sum_s counts[s][e]
//   blk_base[s][e]  = r * cap + chunk_off[r][s] + within[s][e]
__global__ __launch_bounds__(kScanThreads) void k_plan_scan_rm1(
    const int *__restrict__ blk_counts, const int *__restrict__ blk_flags,
    const int *__restrict__ within, const int *__restrict__ csize, PlanGeom g,
    int *__restrict__ counts, int *__restrict__ expert_off, int *__restrict__ chunk_off,
    int *__restrict__ blk_base, int *__restrict__ flag) {
    extern __shared__ int chk[];                // [nd][ns + 1]
    __shared__ int wsum[kScanThreads / kWave];
    __shared__ int sflag;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int E = g.E, ns = g.n_src, nd = g.n_dst;
    if (tid == 0) sflag = 0;
    __syncthreads();
    int fl = 0;
    for (int b = tid; b < ns; b += kScanThreads) fl |= blk_flags[b];
    if (fl) atomicOr(&sflag, fl);
    // chunk offsets: destination r's senders in order, eight loads in flight
    for (int r = tid; r < nd; r += kScanThreads) {
        int run = 0, s = 0;
        for (; s + 8 <= ns; s += 8) {
            int w[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) w[u] = csize[size_t(s + u) * nd + r];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                chk[r * (ns + 1) + s + u] = run;
                run += w[u];
            }
        }
        for (; s < ns; ++s) {
            const int w = csize[size_t(s) * nd + r];
            chk[r * (ns + 1) + s] = run;
            run += w;
        }
        chk[r * (ns + 1) + ns] = run;
        if (int64_t(run) > g.cap) atomicOr(&sflag, kFlagCapacity);
    }
    // per-expert totals over the sources (and the per-source counts, which are the
    // block counts here), eight loads in flight
    int tot = 0;
    if (tid < E) {
        int s = 0;
        for (; s + 8 <= ns; s += 8) {
            int w[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) w[u] = blk_counts[size_t(s + u) * E + tid];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                counts[size_t(s + u) * E + tid] = w[u];
                tot += w[u];
            }
        }
        for (; s < ns; ++s) {
            const int w = blk_counts[size_t(s) * E + tid];
            counts[size_t(s) * E + tid] = w;
            tot += w;
        }
    }
    // exclusive scan of the totals over e = tid (E <= kScanThreads)
    int v = tot;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int o = __shfl_up(v, off, kWave);
        if (lane >= off) v += o;
    }
    if (lane == kWave - 1) wsum[wave] = v;
    __syncthreads();
    int carry = 0;
    for (int w = 0; w < wave; ++w) carry += wsum[w];
    if (tid < E) expert_off[tid] = carry + v - tot;
    if (tid == E - 1) expert_off[E] = carry + v;
    for (int i = tid; i < nd * (ns + 1); i += kScanThreads) chunk_off[i] = chk[i];
    // first row of every (source, expert)
    for (int c = tid; c < ns * E; c += kScanThreads) {
        const int s = g.dE.div(c), e = c - s * E;
        const int r = g.depr.div(e);
        blk_base[c] = int(int64_t(r) * g.cap) + chk[r * (ns + 1) + s] + within[c];
    }
    __syncthreads();
    if (tid == 0) *flag = sflag;      // overwrites the previous call's flag
}

// The plan's scan for the expert-major layout (one source, one destination): thread
// e sums expert e's block counts, the experts' totals are scanned across the
// workgroup, and a second walk over the counts writes the first row of every
// (block, e) in block order. Counts are read 32 at a time (independent loads).
__global__ __launch_bounds__(kScanThreads) void k_plan_scan_em(
    const int *__restrict__ blk_counts, const int *__restrict__ blk_flags, PlanGeom g,
    int *__restrict__ counts, int *__restrict__ expert_off, int *__restrict__ chunk_off,
    int *__restrict__ blk_base, int *__restrict__ flag) {
    constexpr int kBatch = 32;
    __shared__ int wsum[kScanThreads / kWave];
    __shared__ int sflag;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int E = g.E;
    if (tid == 0) sflag = 0;
    __syncthreads();
    int fl = 0;
    for (int b = tid; b < g.B; b += kScanThreads) fl |= blk_flags[b];
    if (fl) atomicOr(&sflag, fl);
    // the first kBatch blocks' counts stay in registers for the second pass
    int tot = 0;
    int c0v[kBatch];
    if (tid < E) {
#pragma unroll
        for (int u = 0; u < kBatch; ++u) c0v[u] = (u < g.B) ? blk_counts[size_t(u) * E + tid] : 0;
#pragma unroll
        for (int u = 0; u < kBatch; ++u) tot += c0v[u];
        for (int b0 = kBatch; b0 < g.B; b0 += kBatch) {
            int c[kBatch];
#pragma unroll
            for (int u = 0; u < kBatch; ++u)
                c[u] = (b0 + u < g.B) ? blk_counts[size_t(b0 + u) * E + tid] : 0;
#pragma unroll
            for (int u = 0; u < kBatch; ++u) tot += c[u];
        }
        counts[tid] = tot;
    }
    // exclusive scan of the totals over e = tid
    int v = tot;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int o = __shfl_up(v, off, kWave);
        if (lane >= off) v += o;
    }
    if (lane == kWave - 1) wsum[wave] = v;
    __syncthreads();
    int carry = 0;
    for (int w = 0; w < wave; ++w) carry += wsum[w];
    const int off_e = carry + v - tot;
    if (tid < E) {
        expert_off[tid] = off_e;
        int run = off_e;
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            if (u < g.B) blk_base[size_t(u) * E + tid] = run;
            run += c0v[u];
        }
        for (int b0 = kBatch; b0 < g.B; b0 += kBatch) {
            int c[kBatch];
#pragma unroll
            for (int u = 0; u < kBatch; ++u)
                c[u] = (b0 + u < g.B) ? blk_counts[size_t(b0 + u) * E + tid] : 0;
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                if (b0 + u < g.B) blk_base[size_t(b0 + u) * E + tid] = run;
                run += c[u];
            }
        }
    }
    if (tid == E - 1) {
        expert_off[E] = off_e + tot;
        chunk_off[0] = 0;
        chunk_off[1] = off_e + tot;
        if (int64_t(off_e + tot) > g.cap) atomicOr(&sflag, kFlagCapacity);
    }
    __syncthreads();
    if (tid == 0) *flag = sflag;      // overwrites the previous call's flag
}

// Slots, unused-row marking and the copy, fused: one wavefront per token.
// Block-scaled fp8 payload of 16 consecutive elements (two 16-byte chunks of bf16) of
// a row, for 8-lane groups that each hold one 128-element block: m = the block's
// largest magnitude (an 8-lane max), scale = m / 448, codes = E4M3(x * (448 / m))
// rounded to nearest even (the hardware conversion, its input clamped to +-448 so it
// saturates); an all-zero block gets +0 codes.
__device__ __forceinline__ uint4 quant16_fp8(const uint4 &v0, const uint4 &v1, float &scale) {
    float f[16];
    Vec<MOE_BF16>::unpack(v0, f);
    Vec<MOE_BF16>::unpack(v1, f + 8);
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(f[i]));
#pragma unroll
    for (int off = 1; off < 8; off <<= 1) m = fmaxf(m, __shfl_xor(m, off, kWave));
    scale = m / 448.0f;
    if (m == 0.0f) return make_uint4(0u, 0u, 0u, 0u);
    const float inv = 448.0f / m;
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const float r0 = fminf(fmaxf(f[4 * q] * inv, -448.0f), 448.0f);
        const float r1 = fminf(fmaxf(f[4 * q + 1] * inv, -448.0f), 448.0f);
        const float r2 = fminf(fmaxf(f[4 * q + 2] * inv, -448.0f), 448.0f);
        const float r3 = fminf(fmaxf(f[4 * q + 3] * inv, -448.0f), 448.0f);
        int p = __builtin_amdgcn_cvt_pk_fp8_f32(r0, r1, 0, false);
        p = __builtin_amdgcn_cvt_pk_fp8_f32(r2, r3, p, true);
        w[q] = uint32_t(p);
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
}

constexpr int kCopyThreads = 256;   // four wavefronts, one token each

// Wavefront (block, wave) takes token blockIdx.x * 4 + wave: lane j < k finds the row
// of pair j (the first row of its block and expert plus its rank inside the block),
// records it in pair_slot and row_pair, and the wavefront then copies the row (or its
// fp8 payload) to the k rows. All workgroups together mark the rows that no pair uses
// with row_pair = -1.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// NT: the copied rows are stored non-temporally (see dispatch_impl)
template <bool Q8, bool NT>
__global__ __launch_bounds__(kCopyThreads) void k_plan_copy(
    const int *__restrict__ idx, PlanGeom g, const int *__restrict__ blk_base,
    const unsigned char *__restrict__ rank, const int *__restrict__ chunk_off,
    int *__restrict__ pair_slot, int *__restrict__ row_pair, int *__restrict__ flag,
    const uint4 *__restrict__ x, int rc, uint4 *__restrict__ x_disp, uint4 *__restrict__ q_disp,
    float *__restrict__ q_scale) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int t = blockIdx.x * (kCopyThreads / kWave) + wave;
    const int64_t rows_total = int64_t(g.n_dst) * g.cap;
    // rows that no pair uses
    for (int64_t row = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; row < rows_total;
         row += int64_t(gridDim.x) * blockDim.x) {
        const int r = g.dcap.div(int(row));            // row < n_dst * cap < 2^31
        if (row - int64_t(r) * g.cap >= chunk_off[r * (g.n_src + 1) + g.n_src]) row_pair[row] = -1;
    }
    if (t >= g.T) return;
    const int s = g.dTs.div(t);
    const int b = s * g.bps + (t - s * g.Ts) / kPlanBlock;
    // the token's row (plain copy) is loaded before its slots are known
    const uint4 *src = x ? x + size_t(t) * rc : nullptr;
    int my_slot = -1;
    if (lane < g.k) {
        const size_t p = size_t(t) * g.k + lane;
        const int e = idx[p];
        if (e >= 0 && e < g.E) {
            const int row = blk_base[size_t(b) * g.E + e] + int(rank[p]);
            const int r = g.depr.div(e);
            if (int64_t(row) - int64_t(r) * g.cap < g.cap) {
                my_slot = row;
                row_pair[row] = int(p);
            } else {
                atomicOr(flag, kFlagCapacity);
            }
        }
        pair_slot[p] = my_slot;
    }
    if (src == nullptr) return;
    if (Q8) {
        // a row is rc/2 pieces of 16 elements (16 code bytes); 8 lanes hold one block.
        // Batches of 8 pieces per lane (8192 elements): all their loads in flight
        // together, then the codes; the batch's 64 block scales are gathered so that
        // lane L holds block L's, and each destination row gets them in one write.
        const int rp = rc / 2, nb = rc / 16;
        for (int c0 = 0; c0 < rp; c0 += 8 * kWave) {
            uint4 v[8][2];
#pragma unroll
            for (int it = 0; it < 8; ++it) {
                const int c = c0 + it * kWave + lane;
                v[it][0] = make_uint4(0u, 0u, 0u, 0u);
                v[it][1] = make_uint4(0u, 0u, 0u, 0u);
                if (c < rp) {
                    v[it][0] = src[2 * c];
                    v[it][1] = src[2 * c + 1];
                }
            }
            uint4 code[8];
            float my_sc = 0.0f;
#pragma unroll
            for (int it = 0; it < 8; ++it) {
                float sc;
                code[it] = quant16_fp8(v[it][0], v[it][1], sc);   // every lane takes part
                // block it*8 + (lane & 7) of the batch sits in lanes 8 (lane & 7) + 0..7
                const float bs = __shfl(sc, (lane & 7) * 8, kWave);
                if ((lane >> 3) == it) my_sc = bs;
            }
            const int blk = c0 / 8 + lane;                         // block held by this lane
            for (int j = 0; j < g.k; ++j) {
                const int sj = __builtin_amdgcn_readlane(my_slot, j);
                if (sj < 0 || sj >= rows_total) continue;
#pragma unroll
                for (int it = 0; it < 8; ++it) {
                    const int c = c0 + it * kWave + lane;
                    if (c < rp) q_disp[size_t(sj) * rp + c] = code[it];
                }
                if (blk < nb) q_scale[size_t(sj) * nb + blk] = my_sc;
            }
        }
        return;
    }
    // batches of 16 KiB of the row (16 pieces per lane) with all loads in flight
    for (int c0 = 0; c0 < rc; c0 += 16 * kWave) {
        uint4 v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int c = c0 + u * kWave + lane;
            v[u] = make_uint4(0u, 0u, 0u, 0u);
            if (c < rc) v[u] = src[c];
        }
        for (int j = 0; j < g.k; ++j) {
            const int sj = __builtin_amdgcn_readlane(my_slot, j);
            if (sj < 0 || sj >= rows_total) continue;
            uint4 *dst = x_disp + size_t(sj) * rc;
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                const int c = c0 + u * kWave + lane;
                if (c < rc) {
                    if (NT)
                        __builtin_nontemporal_store(__builtin_bit_cast(u32x4_t, v[u]),
                                                    reinterpret_cast<u32x4_t *>(dst + c));
                    else
                        dst[c] = v[u];
                }
            }
        }
    }
}

// dx[t] = sum_j dx_disp[pair_slot[t,j]] + sum_j dl[t,j] * w_router[idx[t,j]]
template <int DT>
__global__ __launch_bounds__(256) void k_dispatch_bwd(const uint4 *__restrict__ dx_disp,
                                                      const int *__restrict__ pair_slot,
                                                      const int *__restrict__ topk_idx,
                                                      const float *__restrict__ dl,
                                                      const uint4 *__restrict__ w_router, int T,
                                                      int k, int E, int rc, int64_t rows_total,
                                                      uint4 *__restrict__ dx) {
    constexpr int VN = Vec<DT>::N;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave0 = __builtin_amdgcn_readfirstlane((blockIdx.x * blockDim.x + threadIdx.x) / kWave);
    const int nwaves = gridDim.x * blockDim.x / kWave;
    for (int t = wave0; t < T; t += nwaves) {
        // lane j < k holds pair j's slot, expert and router-gradient weight
        const int my_s = lane < k ? pair_slot[size_t(t) * k + lane] : -1;
        const int my_e = (lane < k && dl != nullptr) ? topk_idx[size_t(t) * k + lane] : -1;
        const float my_g = (lane < k && dl != nullptr) ? dl[size_t(t) * k + lane] : 0.0f;
        for (int c = lane; c < rc; c += kWave) {
            float acc[VN];
#pragma unroll
            for (int i = 0; i < VN; ++i) acc[i] = 0.0f;
            // the k gathered rows, eight loads in flight, summed in j order
            for (int j0 = 0; j0 < k; j0 += 8) {
                uint4 v[8];
                bool ok[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int sj = __builtin_amdgcn_readlane(my_s, min(j0 + u, kWave - 1));
                    ok[u] = j0 + u < k && sj >= 0 && sj < rows_total;   // uniform
                    v[u] = make_uint4(0u, 0u, 0u, 0u);
                    if (ok[u]) v[u] = dx_disp[size_t(sj) * rc + c];
                }
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    if (!ok[u]) continue;
                    float f[VN];
                    Vec<DT>::unpack(v[u], f);
#pragma unroll
                    for (int i = 0; i < VN; ++i) acc[i] += f[i];
                }
            }
            if (dl != nullptr) {
                for (int j0 = 0; j0 < k; j0 += 8) {
                    uint4 v[8];
                    bool ok[8];
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        const int ej = __builtin_amdgcn_readlane(my_e, min(j0 + u, kWave - 1));
                        ok[u] = j0 + u < k && ej >= 0 && ej < E;
                        v[u] = make_uint4(0u, 0u, 0u, 0u);
                        if (ok[u]) v[u] = w_router[size_t(ej) * rc + c];
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
            }
            dx[size_t(t) * rc + c] = Vec<DT>::pack(acc);
        }
    }
}

// An empty batch (T = 0): every count and offset is zero, every row of the buffer is
// unused, and the status flag is cleared, so a later consumer of the plan (combine,
// the backward) reads a valid empty plan rather than whatever the buffers held.
__global__ __launch_bounds__(256) void k_plan_empty(PlanGeom g, int *__restrict__ counts,
                                                     int *__restrict__ expert_off,
                                                     int *__restrict__ chunk_off,
                                                     int *__restrict__ row_pair,
                                                     int *__restrict__ flag) {
    const int64_t tid = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t stride = int64_t(gridDim.x) * blockDim.x;
    if (tid == 0) *flag = 0;
    for (int64_t i = tid; i < int64_t(g.n_src) * g.E; i += stride) counts[i] = 0;
    for (int64_t i = tid; i <= g.E; i += stride) expert_off[i] = 0;
    for (int64_t i = tid; i < int64_t(g.n_dst) * (g.n_src + 1); i += stride) chunk_off[i] = 0;
    for (int64_t i = tid; i < int64_t(g.n_dst) * g.cap; i += stride) row_pair[i] = -1;
}

bool set_scan_lds_limit() { return lds_limit_once<&k_plan_scan>(kScanLdsInts * int(sizeof(int))); }

// The allocation-free dispatch's workspace: one fixed array per GPU, held until the
// process ends. Its name is a host-side stand-in; kernels get the device address that
// hipGetSymbolAddress returns for the current device (looked up once per device).
constexpr size_t kNoAllocScratchBytes = size_t(4) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

void *scratch_ptr() {
    static PerDevice<void *> pd;
    return per_device(pd, []() -> void * {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
        return ptr;
    });
}

int copy_grid(int64_t T) { return int(std::min<int64_t>(cdiv(T, 4), 8192)); }

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" size_t moe_dispatch_workspace_size(int64_t T, int32_t E, int32_t k,
                                              const moe_layout_t *layout) {
    if (T < 0 || E <= 0 || k <= 0) return 0;
    if (layout && (layout->n_src <= 0 || layout->n_dst <= 0 || T % layout->n_src)) return 0;
    return ws_bytes_for(make_geom(T, E, k, layout));
}

namespace moe {
namespace {

// The plan, then either the row copy (x_disp) or the fp8 payload (q_disp, q_scale).
// noalloc: the workspace is this device's scratch array (ws and ws_bytes are ignored).
moe_status_t dispatch_impl(const void *x, const int32_t *topk_idx, int64_t T, int64_t d,
                           int32_t E, int32_t k, moe_dtype_t dtype, const moe_layout_t *layout,
                           int32_t *counts, int32_t *expert_off, int32_t *chunk_off,
                           int32_t *pair_slot, int32_t *row_pair, void *x_disp, uint8_t *q_disp,
                           float *q_scale, void *ws, size_t ws_bytes, void *stream,
                           bool noalloc = false) {
    const bool q8 = q_disp != nullptr || q_scale != nullptr;
    if (!valid_dtype(dtype) || T < 0 || d <= 0 || E <= 0 || k <= 0) return MOE_ERR_INVALID_ARG;
    if (k > E) return MOE_ERR_SHAPE;
    if (layout && (layout->n_src <= 0 || layout->n_dst <= 0 || layout->cap_rows_per_dst < 0))
        return MOE_ERR_INVALID_ARG;
    const int n_src = layout ? layout->n_src : 1, n_dst = layout ? layout->n_dst : 1;
    if (T % n_src != 0 || E % n_dst != 0) return MOE_ERR_SHAPE;
    if (E > 1024 || k > 32 || T * k >= (int64_t(1) << 31)) return MOE_ERR_UNSUPPORTED;
    const PlanGeom g = make_geom(T, E, k, layout);
    // tight form of the receive bound: a token sends at most min(k, E/N) rows to one
    // destination, so a destination receives at most n_src * Ts * min(k, E/N) rows
    const int64_t need = int64_t(n_src) * g.Ts * std::min<int64_t>(k, g.epr);
    if (g.cap < need) return MOE_ERR_CAPACITY;
    if (int64_t(n_dst) * g.cap >= (int64_t(1) << 31)) return MOE_ERR_UNSUPPORTED;
    // the expert-major layout scans with k_plan_scan_em, which walks the plan blocks in
    // batches and needs no LDS beyond its own; the rank-major scan keeps every block
    // count, per-source count and chunk size of the plan in one workgroup's LDS
    const bool expert_major = n_src == 1 && n_dst == 1;
    const size_t lds_scan = size_t(int64_t(g.B) * E + int64_t(n_src) * E + E + 1 +
                                   int64_t(n_dst) * (n_src + 1) + int64_t(n_src) * n_dst) *
                            sizeof(int);
    if (!expert_major && lds_scan > size_t(kScanLdsInts) * sizeof(int)) return MOE_ERR_UNSUPPORTED;
    if (noalloc) {
        // the plan's workspace must fit the fixed array; nothing is allocated instead
        if (ws_bytes_for(g) > kNoAllocScratchBytes) return MOE_ERR_CAPACITY;
        ws = scratch_ptr();
        if (ws == nullptr) return MOE_ERR_HIP;
        ws_bytes = kNoAllocScratchBytes;
    }
    if (T == 0) {
        // plan only: nothing to read, but the plan outputs describe an empty batch
        if (!counts || !expert_off || !chunk_off || !ws || (g.cap > 0 && !row_pair))
            return MOE_ERR_INVALID_ARG;
        if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return MOE_ERR_ALIGN;
        if (ws_bytes < ws_bytes_for(g)) return MOE_ERR_CAPACITY;
        const int64_t n = std::max<int64_t>({int64_t(n_dst) * g.cap, int64_t(E) + 1,
                                             int64_t(n_src) * E, int64_t(n_dst) * (n_src + 1)});
        hipLaunchKernelGGL(k_plan_empty, dim3(unsigned(std::min<int64_t>(cdiv(n, 256), 1024))),
                           dim3(256), 0, as_stream(stream), g, counts, expert_off, chunk_off,
                           row_pair, reinterpret_cast<int *>(ws));
        return launch_status();
    }
    if (!topk_idx || !counts || !expert_off || !chunk_off || !pair_slot || !row_pair || !ws)
        return MOE_ERR_INVALID_ARG;
    if (!q8 && (x == nullptr) != (x_disp == nullptr)) return MOE_ERR_INVALID_ARG;
    if (q8 && (!x || !q_disp || !q_scale)) return MOE_ERR_INVALID_ARG;
    if (q8 && (dtype != MOE_BF16 || d % 128 != 0)) return MOE_ERR_UNSUPPORTED;
    if (ws_bytes < ws_bytes_for(g)) return MOE_ERR_CAPACITY;
    if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return MOE_ERR_ALIGN;
    const int64_t rowb = d * elt_size(dtype);
    if (x && (rowb % 16 != 0 || !aligned16(x) || (!q8 && !aligned16(x_disp)))) return MOE_ERR_ALIGN;
    if (q8 && (!aligned16(q_disp) || !aligned16(q_scale)))
        return MOE_ERR_ALIGN;

    if (!set_scan_lds_limit()) return MOE_ERR_HIP;   // first HIP call: all checks done
    const hipStream_t st = as_stream(stream);
    char *wsb = static_cast<char *>(ws);
    const WsLayout wl = ws_layout(g);
    int *flag = reinterpret_cast<int *>(wsb);
    int *blk_flags = reinterpret_cast<int *>(wsb + wl.flags);
    int *blk_counts = reinterpret_cast<int *>(wsb + wl.counts);
    int *blk_base = reinterpret_cast<int *>(wsb + wl.base);
    unsigned char *rank = reinterpret_cast<unsigned char *>(wsb + wl.rank);
    int *within = g.rm1 ? reinterpret_cast<int *>(wsb + wl.within) : nullptr;
    int *csize = g.rm1 ? reinterpret_cast<int *>(wsb + wl.csize) : nullptr;
    const size_t lds_mask = size_t(E) * kMaskWords * sizeof(unsigned long long) +
                            (g.rm1 ? size_t(E) * sizeof(int) : 0);

    hipLaunchKernelGGL(k_plan_count, dim3(g.B), dim3(kPlanBlock), lds_mask, st, topk_idx, g,
                       blk_counts, blk_flags, rank, within, csize);
    if (g.rm1)
        hipLaunchKernelGGL(k_plan_scan_rm1, dim3(1), dim3(kScanThreads),
                           size_t(n_dst) * (n_src + 1) * sizeof(int), st, blk_counts, blk_flags,
                           within, csize, g, counts, expert_off, chunk_off, blk_base, flag);
    else if (expert_major)
        hipLaunchKernelGGL(k_plan_scan_em, dim3(1), dim3(kScanThreads), 0, st, blk_counts,
                           blk_flags, g, counts, expert_off, chunk_off, blk_base, flag);
    else
        hipLaunchKernelGGL(k_plan_scan, dim3(1), dim3(kScanThreads), lds_scan, st, blk_counts,
                           blk_flags, g, counts, expert_off, chunk_off, blk_base, flag);
    const dim3 cgrid(unsigned(cdiv(T, kCopyThreads / kWave)));
    // Copies of more than twice the 256 MB Infinity Cache go out non-temporally. The
    // copy itself gets slightly slower, but the cache is not left full of dirty rows
    // for the grouped GEMM that reads them next, which streams its weights through it
    // (measured at T=8192, E=384, 0.94 GB: dispatch 200 -> 208 us, gate/up 4.68 -> 4.50
    // ms; at 470 MB, the 32-source EP layout, the copy slowed 102 -> 115 us with no
    // gain after it, so the ordinary stores stay there).
    const bool nt = size_t(T) * g.k * rowb > (size_t(512) << 20);
    if (q8)
        hipLaunchKernelGGL((k_plan_copy<true, false>), cgrid, dim3(kCopyThreads), 0, st, topk_idx, g,
                           blk_base, rank, chunk_off, pair_slot, row_pair, flag,
                           static_cast<const uint4 *>(x), int(rowb / 16), nullptr,
                           reinterpret_cast<uint4 *>(q_disp), q_scale);
    else if (nt)
        hipLaunchKernelGGL((k_plan_copy<false, true>), cgrid, dim3(kCopyThreads), 0, st, topk_idx, g,
                           blk_base, rank, chunk_off, pair_slot, row_pair, flag,
                           static_cast<const uint4 *>(x), int(rowb / 16), static_cast<uint4 *>(x_disp),
                           nullptr, nullptr);
    else
        hipLaunchKernelGGL((k_plan_copy<false, false>), cgrid, dim3(kCopyThreads), 0, st, topk_idx, g,
                           blk_base, rank, chunk_off, pair_slot, row_pair, flag,
                           static_cast<const uint4 *>(x), int(rowb / 16), static_cast<uint4 *>(x_disp),
                           nullptr, nullptr);
    return launch_status();
}

}  // namespace
}  // namespace moe

extern "C" moe_status_t moe_dispatch(const void *x, const int32_t *topk_idx, int64_t T,
                                     int64_t d, int32_t E, int32_t k, moe_dtype_t dtype,
                                     const moe_layout_t *layout, int32_t *counts,
                                     int32_t *expert_off, int32_t *chunk_off, int32_t *pair_slot,
                                     int32_t *row_pair, void *x_disp, void *ws, size_t ws_bytes,
                                     void *stream) {
    return dispatch_impl(x, topk_idx, T, d, E, k, dtype, layout, counts, expert_off, chunk_off,
                         pair_slot, row_pair, x_disp, nullptr, nullptr, ws, ws_bytes, stream);
}

extern "C" moe_status_t moe_dispatch_noalloc(const void *x, const int32_t *topk_idx, int64_t T,
                                             int64_t d, int32_t E, int32_t k, moe_dtype_t dtype,
                                             const moe_layout_t *layout, int32_t *counts,
                                             int32_t *expert_off, int32_t *chunk_off,
                                             int32_t *pair_slot, int32_t *row_pair, void *x_disp,
                                             void *stream) {
    return dispatch_impl(x, topk_idx, T, d, E, k, dtype, layout, counts, expert_off, chunk_off,
                         pair_slot, row_pair, x_disp, nullptr, nullptr, nullptr, 0, stream,
                         /*noalloc=*/true);
}

extern "C" moe_status_t moe_dispatch_fp8(const void *x, const int32_t *topk_idx, int64_t T,
                                         int64_t d, int32_t E, int32_t k,
                                         const moe_layout_t *layout, int32_t *counts,
                                         int32_t *expert_off, int32_t *chunk_off,
                                         int32_t *pair_slot, int32_t *row_pair, uint8_t *q_disp,
                                         float *q_scale, void *ws, size_t ws_bytes, void *stream) {
    if (!q_disp || !q_scale) return MOE_ERR_INVALID_ARG;
    return dispatch_impl(x, topk_idx, T, d, E, k, MOE_BF16, layout, counts, expert_off, chunk_off,
                         pair_slot, row_pair, nullptr, q_disp, q_scale, ws, ws_bytes, stream);
}

extern "C" moe_status_t moe_dispatch_status(const void *ws, void *stream) {
    if (!ws) return MOE_ERR_INVALID_ARG;
    int flag = 0;
    if (hipStreamSynchronize(as_stream(stream)) != hipSuccess) return MOE_ERR_HIP;
    if (hipMemcpy(&flag, ws, sizeof(int), hipMemcpyDeviceToHost) != hipSuccess) return MOE_ERR_HIP;
    if (flag & kFlagBadIndex) return MOE_ERR_BAD_INDEX;
    if (flag & kFlagCapacity) return MOE_ERR_CAPACITY;
    return MOE_OK;
}

extern "C" moe_status_t moe_dispatch_bwd(const void *dx_disp, const int32_t *pair_slot,
                                         const int32_t *topk_idx, const float *dlogits_sel,
                                         const void *w_router, int64_t T, int32_t k, int64_t d,
                                         int32_t E, int64_t rows_total, moe_dtype_t dtype,
                                         void *dx, void *stream) {
    if (!valid_dtype(dtype) || T < 0 || d <= 0 || k <= 0 || rows_total < 0)
        return MOE_ERR_INVALID_ARG;
    if (k > kWave) return MOE_ERR_UNSUPPORTED;
    if (T == 0) return MOE_OK;
    if (!dx_disp || !pair_slot || !dx) return MOE_ERR_INVALID_ARG;
    if (dlogits_sel && (!topk_idx || !w_router || E <= 0)) return MOE_ERR_INVALID_ARG;
    const int64_t rowb = d * elt_size(dtype);
    if (rowb % 16 != 0 || !aligned16(dx_disp) || !aligned16(dx) ||
        (w_router && !aligned16(w_router)))
        return MOE_ERR_ALIGN;
    const hipStream_t st = as_stream(stream);
    if (dtype == MOE_BF16)
        hipLaunchKernelGGL(k_dispatch_bwd<MOE_BF16>, dim3(copy_grid(T)), dim3(256), 0, st,
                           static_cast<const uint4 *>(dx_disp), pair_slot, topk_idx, dlogits_sel,
                           static_cast<const uint4 *>(w_router), int(T), k, E, int(rowb / 16),
                           rows_total, static_cast<uint4 *>(dx));
    else
        hipLaunchKernelGGL(k_dispatch_bwd<MOE_F32>, dim3(copy_grid(T)), dim3(256), 0, st,
                           static_cast<const uint4 *>(dx_disp), pair_slot, topk_idx, dlogits_sel,
                           static_cast<const uint4 *>(w_router), int(T), k, E, int(rowb / 16),
                           rows_total, static_cast<uint4 *>(dx));
    return launch_status();
}
