// SI selection on gfx950: per query token, the forced sink and local window plus the
// top-m fill by (score descending, position ascending)
// (LongCat-Flash-Lite-Sparse summary, "Good to know" and "Technical features", first
// bullet: the selection budget is split into a fixed sink and a local window).
//
// Exact selection on a 64-bit composite key
//     comp = order_key(score) << 32 | ~position
// (larger comp = better: higher score, then lower position; composites are unique), so
// the chosen set is the set of the m largest composites among the candidates.
//   hist:     many workgroups per row count the candidates per first-level bin (top 11
//             bits of the order key) in LDS and add the counts to the row's histogram
//             with integer atomics. The indexer can build the same histogram in its
//             epilogue; then this pass is skipped.
//   filter:   many workgroups per row find the threshold bin b1 from the histogram and
//             classify their columns: candidates above b1 are set in the row's column
//             bitmap (each workgroup writes whole words of its own column range), the
//             candidates in b1 are appended to the row's tie list.
//   resolve:  one workgroup per row ranks the tie list in LDS (second-level histogram
//             of the next 12 key bits, then direct ranking of the few candidates that
//             share 23 key bits, or radix passes when many are equal), sets the chosen
//             ties in the bitmap, and compacts the bitmap into ascending positions
//             between the sink and the window. It leaves the row's histogram and
//             counters at zero for the next call. (A fused selection + attention
//             launch replaces this pass: each attention workgroup resolves the slice
//             of the row it attends over; the filter records its pick for them.)
// Kernel boundaries are the only cross-workgroup synchronisation, apart from the
// counter that tells the last of a row's sliced resolves to clear the row's counters. Membership is
// defined by the total order on composites and the output is sorted, so the result
// does not depend on the order in which atomics land.
#include "select_core.cuh"

namespace lsa {
namespace {
using namespace sel;

constexpr int kHT = 256;             // histogram and filter threads
constexpr int kRT = 1024;            // resolve threads (16 waves)
constexpr int kKeptLds = 1024;       // kept-map entries the resolve keeps in LDS
constexpr int kFC = 2048;            // filter round: 8 columns per thread
// ----------------------------------------------------------------------------- hist
__global__ __launch_bounds__(kHT) void select_hist_kernel(SelectArgs a, uint32_t *hist, int part_cols) {
    __shared__ uint32_t h[kSelBins];
    const int row = blockIdx.y;
    const int c0 = blockIdx.x * part_cols;
    const int c1 = min(a.n_cols, c0 + part_cols);
    for (int i = threadIdx.x; i < kSelBins; i += kHT) h[i] = 0;
    __syncthreads();
    const Row r = make_row(a, row);
    if (r.m > 0) {
        for (int col = c0 + 4 * threadIdx.x; col < c1; col += 4 * kHT) {
            float xs[4];
            if (a.vec && col + 3 < c1) {
                const float4 v = *reinterpret_cast<const float4 *>(r.sc + col);
                xs[0] = v.x, xs[1] = v.y, xs[2] = v.z, xs[3] = v.w;
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) xs[e] = col + e < c1 ? r.sc[col + e] : kNegInf;
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                uint64_t comp;
                if (col + e < c1 && candidate_x(a, r, col + e, xs[e], comp)) atomicAdd(&h[(uint32_t)(comp >> 32) >> kSelShift], 1u);
            }
        }
    }
    __syncthreads();
    uint32_t *g = hist + (int64_t)row * kSelBins;
    for (int i = threadIdx.x; i < kSelBins; i += kHT)
        if (h[i]) atomicAdd(&g[i], h[i]);
}

// ----------------------------------------------------------------------------- filter
// grid (parts, rows); part_cols is a multiple of 32, so each workgroup owns whole words
// of the row's column bitmap.
template <bool KEPT>
__global__ __launch_bounds__(kHT) void select_filter_kernel(SelectArgs a, Ws w, int part_cols) {
    __shared__ uint64_t tbuf[kFC];
    __shared__ uint32_t tcbuf[kFC];
    __shared__ uint32_t scr[24];
    __shared__ uint32_t tcnt, tbase;
    const int row = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63;
    const int c0 = blockIdx.x * part_cols;
    const int c1 = min(a.n_cols, c0 + part_cols);
    const Row r = make_row(a, row);
    const uint32_t m = (uint32_t)max(r.m, 0);

    // first round's scores are requested before the histogram (independent loads)
    auto load4 = [&](int col, int end) -> float4 {
        if (a.vec && col + 3 < end) return *reinterpret_cast<const float4 *>(r.sc + col);
        float4 v;
        v.x = col < end ? r.sc[col] : kNegInf;
        v.y = col + 1 < end ? r.sc[col + 1] : kNegInf;
        v.z = col + 2 < end ? r.sc[col + 2] : kNegInf;
        v.w = col + 3 < end ? r.sc[col + 3] : kNegInf;
        return v;
    };
    // both halves of a round's columns; a whole aligned round takes plain vector loads
    // (a workgroup-uniform choice: no divergent paths writing the same registers)
    float4 va, vb;
    auto load_round = [&](int base) __attribute__((always_inline)) {
        const int end = min(c1, base + kFC);
        if (a.vec && base + kFC <= c1) {
            va = *reinterpret_cast<const float4 *>(r.sc + base + 4 * tid);
            vb = *reinterpret_cast<const float4 *>(r.sc + base + kFC / 2 + 4 * tid);
        } else {
            va = load4(base + 4 * tid, end);
            vb = load4(base + kFC / 2 + 4 * tid, end);
        }
    };
    load_round(c0);
    uint32_t hv[kSelBins / kHT];  // thread t: bins from the top, 8 per thread
    {
        const uint32_t *g = w.hist + (int64_t)row * kSelBins + kSelBins - kSelBins / kHT * (tid + 1);
        const uint4 lo = *reinterpret_cast<const uint4 *>(g), hi = *reinterpret_cast<const uint4 *>(g + 4);
        hv[0] = hi.w, hv[1] = hi.z, hv[2] = hi.y, hv[3] = hi.x, hv[4] = lo.w, hv[5] = lo.z, hv[6] = lo.y, hv[7] = lo.x;
    }
    const BinPick bp = pick_bin<kHT, kSelBins / kHT>(hv, m, scr);
    uint32_t *gctr = w.ctr + (int64_t)row * kCtr;
    if (blockIdx.x == 0 && tid == 0) {  // every workgroup of the row picks the same; one records it
        gctr[1] = (uint32_t)bp.mode;
        gctr[2] = (uint32_t)bp.bin;
        gctr[3] = bp.above;
    }
    if (bp.mode == 0) return;
    const int b1 = bp.bin;
    uint64_t *gties = w.ties + (int64_t)row * w.cap;
    uint32_t *gtcols = w.tcols ? w.tcols + (int64_t)row * w.cap : nullptr;
    uint32_t *gbits = w.bits + (int64_t)row * w.words;

    for (int base = c0; base < c1; base += kFC) {
        const int end = min(c1, base + kFC);
        if (tid == 0) tcnt = 0;
        __syncthreads();
        if (base != c0) load_round(base);
        // Lane l of wave w holds columns base + 256 w + 4 l + e (va) and base + 1024 +
        // 256 w + 4 l + e (vb), e = 0..3. Per column slot i (0..7) one ballot of the columns
        // above the threshold bin and one of the ties: bitmap word k of a half-row slice
        // is interleaved from the four ballots of that half (lanes 8k .. 8k+7, bit 4 j + e
        // for lane 8k + j), and the ties take one LDS append per wave.
        const int ca = base + 4 * tid, cb = base + kFC / 2 + 4 * tid;
        uint64_t selb[8], tieb[8], comps[8];
        // flat rows: branch-free (the column is the position); a kept map needs its load
        const int lo = a.causal ? r.f_sink_end : 0;
        const int hi = a.causal ? min(r.p + 1, r.f_win_lo) : end;  // candidates: lo <= col < hi
        // kept map: the eight columns' entries requested together (clamped block index,
        // unconditional loads), so their round trips overlap
        int kbv[KEPT ? 8 : 1];
        if constexpr (KEPT) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int col = (i < 4 ? ca : cb) + (i & 3);
                kbv[i] = r.kept[min(col / a.block_size, a.n_keep - 1)];
            }
        }
        auto classify = [&](int i, int col, float x) {
            uint64_t comp = 0;
            bool cand;
            if constexpr (KEPT) {
                cand = col < end && candidate_kb(a, r, col, x, kbv[i], comp);
            } else {
                cand = x > kNegInf && col < end && col >= lo && col < hi;
                comp = ((uint64_t)order_key(x) << 32) | (uint32_t)~(uint32_t)col;
            }
            const int d1 = (int)(comp >> kB1Shift);
            selb[i] = __ballot(cand && (bp.mode == 1 || d1 > b1));
            tieb[i] = __ballot(cand && bp.mode == 2 && d1 == b1);
            comps[i] = comp;
        };
        classify(0, ca, va.x);
        classify(1, ca + 1, va.y);
        classify(2, ca + 2, va.z);
        classify(3, ca + 3, va.w);
        classify(4, cb, vb.x);
        classify(5, cb + 1, vb.y);
        classify(6, cb + 2, vb.z);
        classify(7, cb + 3, vb.w);
        // lanes 0..15: word (lane & 7) of half (lane >> 3) of this wave's slice (both
        // halves computed, one kept: no dynamic index into the ballot array)
        const int half = (lane >> 3) & 1, wk = lane & 7;
        const int wi = half * (kFC / 64) + 8 * (tid >> 6) + wk;  // word index from base
        auto spread = [&](uint64_t bsel) {  // bit j of lane 8 wk + j's byte -> bit 4 j
            uint32_t x = (uint32_t)(bsel >> (8 * wk)) & 0xFFu;
            x = (x | (x << 12)) & 0x000F000Fu;
            x = (x | (x << 6)) & 0x03030303u;
            return (x | (x << 3)) & 0x11111111u;
        };
        const uint32_t wlo = spread(selb[0]) | spread(selb[1]) << 1 | spread(selb[2]) << 2 | spread(selb[3]) << 3;
        const uint32_t whi = spread(selb[4]) | spread(selb[5]) << 1 | spread(selb[6]) << 2 | spread(selb[7]) << 3;
        const uint32_t word = half ? whi : wlo;
        uint32_t ntw = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) ntw += (uint32_t)__popcll(tieb[i]);
        if (ntw) {  // uniform per wave
            uint32_t sb = 0;
            if (lane == 0) sb = atomicAdd(&tcnt, ntw);
            sb = __builtin_amdgcn_readfirstlane(sb);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                if ((tieb[i] >> lane) & 1ull) {
                    const uint32_t slot = sb + lane_rank(tieb[i]);
                    tbuf[slot] = comps[i];
                    tcbuf[slot] = (uint32_t)((i < 4 ? ca : cb) + (i & 3));
                }
                sb += (uint32_t)__popcll(tieb[i]);
            }
        }
        __syncthreads();
        const uint32_t nt = tcnt;
        if (nt) {
            if (tid == 0) tbase = atomicAdd(&gctr[0], nt);
            __syncthreads();
            const uint32_t tb = tbase;
            for (uint32_t i = tid; i < nt; i += kHT) {
                if (tb + i < (uint32_t)w.cap) {
                    gties[tb + i] = tbuf[i];
                    if (gtcols) gtcols[tb + i] = tcbuf[i];
                }
            }
        }
        // bitmap words last (a barrier would wait for these stores)
        if (lane < 16 && base + 32 * wi < end) gbits[(base >> 5) + wi] = word;
        if (base + kFC < c1) __syncthreads();  // LDS buffers are reused by the next round
    }
}

// ----------------------------------------------------------------------------- resolve
// One workgroup per row. Ties are ranked from LDS when they fit (kTieLds), else read
// from the workspace list. LWORDS > 0: the row's bitmap (LWORDS words) is loaded into LDS
// with the first loads, the chosen ties are set there and the compaction reads it back;
// else the bitmap stays in the workspace (global atomics, then coherent reads). KEPT:
// columns map to positions through the kept map, so the chosen positions are sorted
// (bitonic, KPAD entries) before they are written.
template <bool KEPT, int KPAD>
__global__ __launch_bounds__(kRT) void select_resolve_kernel(SelectArgs a, Ws w, int lwords) {
    extern __shared__ __attribute__((aligned(16))) unsigned char dyn[];
    const int tcap = min(w.cap, kTieLds);                                        // ties held in LDS
    uint64_t *lties = reinterpret_cast<uint64_t *>(dyn);                         // [tcap]
    uint32_t *ltcols = reinterpret_cast<uint32_t *>(dyn + (size_t)tcap * 8);     // [tcap] (KEPT)
    uint32_t *lbits = reinterpret_cast<uint32_t *>(dyn + (size_t)tcap * (KEPT ? 12 : 8));  // [lwords]
    __shared__ __attribute__((aligned(16))) uint32_t h[kB2];  // second-level histogram, then the final group
    __shared__ uint32_t h256[256];
    __shared__ uint32_t scr[32];
    __shared__ uint32_t cnt[4];
    __shared__ uint32_t s_desc;  // KEPT: the kept map's valid entries do not ascend
    __shared__ int32_t fill[KEPT ? KPAD : 1];
    // KEPT: the kept map in LDS when it fits (read with the first loads; the columns of
    // the fill then map to positions without another round trip to memory)
    __shared__ int32_t skept[KEPT ? kKeptLds : 1];
    const bool kl = KEPT && a.n_keep <= kKeptLds;
    const int row = blockIdx.x;
    const int tid = threadIdx.x;
    const Row r = make_row(a, row);
    if (tid == 0) s_desc = 0;
    const uint32_t m = (uint32_t)max(r.m, 0);
    uint32_t *g1 = w.hist + (int64_t)row * kSelBins;
    uint32_t *gctr = w.ctr + (int64_t)row * kCtr;
    const uint64_t *gties = w.ties + (int64_t)row * w.cap;
    const uint32_t *gtcols = KEPT ? w.tcols + (int64_t)row * w.cap : nullptr;
    uint32_t *gbits = w.bits + (int64_t)row * w.words;

    // ---- first loads: histogram (2 bins per thread from the top), tie count, the first
    // tie entries, the bitmap; the histogram and the counters are left at zero
    uint32_t hv[2];
    hv[0] = g1[kSelBins - 1 - 2 * tid];
    hv[1] = g1[kSelBins - 2 - 2 * tid];
    const uint32_t ntie = gctr[0];
    uint64_t t0 = 0, t1 = 0;
    uint32_t tc0 = 0, tc1 = 0;
    if (tid < tcap) t0 = gties[tid];
    if (tid + kRT < tcap) t1 = gties[tid + kRT];
    if (KEPT) {
        if (tid < tcap) tc0 = gtcols[tid];
        if (tid + kRT < tcap) tc1 = gtcols[tid + kRT];
    }
    if (lwords) copy_words_to_lds<kRT, 2>(gbits, lbits, lwords);
    // KEPT: whether the kept map ascends (a kept map whose valid entries ascend, then -1,
    // as lsa_select writes it, keeps the columns in position order), read with the first loads
    bool desc = false;
    if constexpr (KEPT) {
        for (int i = tid; i < a.n_keep; i += kRT) {
            const int x = r.kept[i];
            if (kl) skept[i] = x;
            if (i + 1 < a.n_keep) {
                const int y = r.kept[i + 1];
                const bool vx = x >= 0 && x < r.nblk, vy = y >= 0 && y < r.nblk;
                desc = desc || (vy && (!vx || x >= y));
            }
        }
    }
    const BinPick bp = pick_bin<kRT, 2>(hv, m, scr);  // its barriers follow every thread's reads
    if (desc) s_desc = 1;  // (read after the compaction's barriers)
    const int b1 = bp.bin;

    auto mark = [&](int col) {
        if (lwords) atomicOr(&lbits[col >> 5], 1u << (col & 31));
        else atomicOr(&gbits[col >> 5], 1u << (col & 31));
    };
    if (bp.mode == 2) {
        const bool overflow = ntie > (uint32_t)w.cap;  // the list is incomplete
        const uint32_t nl = min(ntie, (uint32_t)w.cap);
        const bool inlds = nl <= (uint32_t)tcap;
        const uint64_t *tl = inlds ? lties : gties;            // the tie list being ranked
        const uint32_t *tcl = inlds ? ltcols : gtcols;
        const uint32_t need1 = m > bp.above ? m - bp.above : 0u;
        uint64_t thr = ~(uint64_t)0;
        if (!overflow) {
            if (inlds) {
                if ((uint32_t)tid < nl) lties[tid] = t0;
                if ((uint32_t)tid + kRT < nl) lties[tid + kRT] = t1;
                for (uint32_t i = tid + 2 * kRT; i < nl; i += kRT) lties[i] = gties[i];
                if (KEPT) {
                    if ((uint32_t)tid < nl) ltcols[tid] = tc0;
                    if ((uint32_t)tid + kRT < nl) ltcols[tid + kRT] = tc1;
                    for (uint32_t i = tid + 2 * kRT; i < nl; i += kRT) ltcols[i] = gtcols[i];
                }
            }
            for (int i = tid; i < kB2; i += kRT) h[i] = 0;
            if (tid < 4) cnt[tid] = 0;
            __syncthreads();
            for (uint32_t i = tid; i < nl; i += kRT)
                atomicAdd(&h[((uint32_t)(tl[i] >> 32) >> kL2Shift) & (kB2 - 1)], 1u);
            __syncthreads();
            uint32_t v2[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) v2[e] = h[kB2 - 1 - 4 * tid - e];
            const BinPick p2 = pick_bin<kRT, 4>(v2, need1, scr);
            if (p2.mode == 1) {
                thr = 0;  // every tie
            } else if (p2.mode == 2) {
                const int b2 = p2.bin;
                const uint32_t n2 = h[b2];
                const uint32_t need2 = need1 - p2.above;  // wanted from the (b1, b2) group
                const uint64_t pre = (uint64_t)(((uint32_t)b1 << kSelShift) | ((uint32_t)b2 << kL2Shift)) << 32;
                __syncthreads();  // h is reused below
                if (need2 == n2) {
                    thr = pre;  // the whole group
                } else if (n2 <= (uint32_t)kTiny) {
                    uint64_t *tiny = reinterpret_cast<uint64_t *>(h);
                    for (uint32_t i = tid; i < nl; i += kRT) {
                        const uint64_t c = tl[i];
                        if ((c >> kGrpShift) == (pre >> kGrpShift)) {
                            const uint32_t slot = atomicAdd(&cnt[2], 1u);
                            if (slot < (uint32_t)kTiny) tiny[slot] = c;
                        }
                    }
                    __syncthreads();
                    const uint32_t nt = min(cnt[2], (uint32_t)kTiny);
                    if ((uint32_t)tid < nt) {
                        const uint64_t c = tiny[tid];
                        uint32_t rank = 0;  // composites are unique
                        for (uint32_t j = 0; j < nt; ++j) rank += tiny[j] > c;
                        if (rank == need2 - 1) {
                            scr[20] = (uint32_t)c;
                            scr[21] = (uint32_t)(c >> 32);
                        }
                    }
                    __syncthreads();
                    thr = ((uint64_t)scr[21] << 32) | scr[20];
                } else {
                    thr = radix_kth<kRT>(ArrSrc{tl, (int)nl}, need2, pre, kGrpShift, h256, scr);
                }
            }
            for (uint32_t i = tid; i < nl; i += kRT)
                if (tl[i] >= thr) mark(KEPT ? (int)tcl[i] : comp_pos(tl[i]));
        } else {
            // the tie list overflowed: exact select inside bin b1 over the whole row
            const RowSrc rs{&a, &r};
            const uint64_t pre = (uint64_t)b1 << kB1Shift;
            thr = radix_kth<kRT>(rs, need1, pre, kB1Shift, h256, scr);
            for (int col = tid; col < a.n_cols; col += kRT) {
                uint64_t c;
                if (candidate_x(a, r, col, r.sc[col], c) && (c >> kB1Shift) == (uint64_t)b1 && c >= thr) mark(col);
            }
        }
    }
    __syncthreads();

    // ---- ascending output: sink [0, f_sink_end), the fill (strictly between sink and
    // window), the window [f_win_lo, p], then -1
    int32_t *dst = a.idx + (int64_t)row * a.K;
    const int nsink = a.causal ? r.f_sink_end : 0;
    const int nwin = a.causal ? max(0, r.p - r.f_win_lo + 1) : 0;
    uint32_t nfill = 0;
    if (bp.mode != 0) {
        auto word = [&](int i) -> uint32_t {
            return lwords ? lbits[i] : __hip_atomic_load(&gbits[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        };
        const int per = (w.words + kRT - 1) / kRT;
        const int w0 = min(w.words, tid * per), w1 = min(w.words, w0 + per);
        uint32_t c = 0;
        for (int i = w0; i < w1; ++i) c += __popc(word(i));
        uint32_t off = block_exscan<kRT>(c, scr, &nfill);
        for (int i = w0; i < w1; ++i) {
            uint32_t bits = word(i);
            while (bits) {
                const int col = i * 32 + __ffs(bits) - 1;
                bits &= bits - 1;
                if constexpr (KEPT) {
                    if (off < (uint32_t)KPAD) fill[off] = col;  // its position below
                } else {
                    if (nsink + off < (uint32_t)a.K) dst[nsink + off] = col;
                }
                ++off;
            }
        }
        if constexpr (KEPT) {
            nfill = min(nfill, (uint32_t)KPAD);
            // columns -> positions through the kept map, each thread its own entries, so the
            // loads are independent (in the bit walk each waited for the previous one)
            __syncthreads();
            for (uint32_t i = tid; i < nfill; i += kRT) {
                const int col = fill[i], blk = col / a.block_size;
                fill[i] = (kl ? skept[blk] : r.kept[blk]) * a.block_size + (col - blk * a.block_size);
            }
            // an ascending kept map leaves the fill sorted (checked with the first loads)
            __syncthreads();
            const bool ascending = s_desc == 0;
            int np = KPAD;  // the sort's size: the fill rounded up to a power of two
            while (np / 2 >= (int)nfill && np > 1) np /= 2;
            if (ascending) np = 1;
            for (int i = tid; i < np; i += kRT)
                if ((uint32_t)i >= nfill) fill[i] = 0x7FFFFFFF;
            __syncthreads();
            for (int k = 2; k <= np; k <<= 1) {
                for (int j = k >> 1; j > 0; j >>= 1) {
                    for (int i = tid; i < np; i += kRT) {
                        const int ixj = i ^ j;
                        if (ixj > i) {
                            const int x = fill[i], y = fill[ixj];
                            const bool up = (i & k) == 0;
                            if ((x > y) == up) {
                                fill[i] = y;
                                fill[ixj] = x;
                            }
                        }
                    }
                    __syncthreads();
                }
            }
            for (uint32_t i = tid; i < nfill; i += kRT)
                if (nsink + i < (uint32_t)a.K) dst[nsink + i] = fill[i];
        }
    }
    for (int s = tid; s < nsink; s += kRT) dst[s] = s;
    const int wbase = nsink + (int)nfill;
    for (int j = tid; j < nwin; j += kRT)
        if (wbase + j < a.K) dst[wbase + j] = r.f_win_lo + j;
    for (int i = wbase + nwin + tid; i < a.K; i += kRT) dst[i] = -1;
    // the histogram and the counters are left at zero (last: a barrier would wait for these stores)
    g1[kSelBins - 1 - 2 * tid] = 0;
    g1[kSelBins - 2 - 2 * tid] = 0;
    if (tid < kCtr) gctr[tid] = 0;
}

// ----------------------------------------------------------------------------- small rows
// Rows of at most kSmallCols columns (a short decode context): one workgroup per row
// runs the whole selection in one launch from the
// row's order keys held in LDS (the scores read once): first-level histogram, threshold
// bin, the bits of the columns above it and the list of its ties, the ties ranked as in
// the resolve, and the compaction. The workspace is not read; its histogram and counters for the row are left
// at zero, whatever state they came in.
// (Measured: 8 rows of 4096 columns 13 us in one launch against 18 us for the
// histogram, filter and resolve kernels; 4 rows of 16384 columns 19 us against 17: the
// single workgroup's passes over its row no longer pay for the saved launches.)
constexpr int kSmallCols = 4096;
constexpr int kSmallT = 1024;
constexpr int kSmallTies = kSmallCols;  // the list holds every column: it cannot overflow
constexpr size_t kSmallLds = (size_t)kSmallCols * 4 + (size_t)kSmallTies * 12 + (size_t)kB2 * 4 +
                             ((size_t)kSmallCols / 32 + 4) * 4;

template <bool KEPT>
__global__ __launch_bounds__(kSmallT) void select_small_kernel(SelectArgs a, Ws w) {
    extern __shared__ __attribute__((aligned(16))) unsigned char dyn[];
    constexpr int NT = kSmallT;
    uint32_t *keys = reinterpret_cast<uint32_t *>(dyn);                                  // [kSmallCols], 0: none
    uint64_t *lties = reinterpret_cast<uint64_t *>(dyn + (size_t)kSmallCols * 4);         // [kSmallTies]
    uint32_t *tcol = reinterpret_cast<uint32_t *>(lties + kSmallTies);                   // [kSmallTies]
    uint32_t *h = tcol + kSmallTies;                                                     // [kB2]
    uint32_t *lbits = h + kB2;                                                           // [words]
    __shared__ uint32_t h256[256];
    __shared__ uint32_t scr[32];
    __shared__ uint32_t s_nt, s_desc;
    const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const Row r = make_row(a, row);
    const uint32_t m = (uint32_t)max(r.m, 0);
    const int nc = a.n_cols;
    const int words = (nc + 31) / 32;
    auto pos_of = [&](int c) -> int {  // position of a candidate column
        if constexpr (KEPT) {
            const int blk = c / a.block_size;
            return r.kept[blk] * a.block_size + (c - blk * a.block_size);
        } else {
            return c;
        }
    };
    // ---- the row's keys and first-level histogram: the whole row in one round of loads
    // (16 bytes per thread for 16-byte aligned rows), requested before the histogram is
    // cleared so that their latency covers the clearing and its barrier
    constexpr int U = (kSmallCols + 4 * NT - 1) / (4 * NT);  // 16-byte groups per thread
    constexpr int US = (kSmallCols + NT - 1) / NT;          // columns per thread (unaligned rows)
    f32x4 xv[U];
    float xs[US];
    if (a.vec) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = 4 * (u * NT + tid);
            xv[u] = c < nc ? *reinterpret_cast<const f32x4 *>(r.sc + c) : f32x4{kNegInf, kNegInf, kNegInf, kNegInf};
        }
    } else {
#pragma unroll
        for (int u = 0; u < US; ++u) {
            const int c = u * NT + tid;
            xs[u] = c < nc ? r.sc[c] : kNegInf;
        }
    }
    bool desc = false;  // KEPT: the kept map's valid entries do not ascend
    if constexpr (KEPT) {
        for (int i = tid; i + 1 < a.n_keep; i += NT) {
            const int x = r.kept[i], y = r.kept[i + 1];
            const bool vx = x >= 0 && x < r.nblk, vy = y >= 0 && y < r.nblk;
            desc = desc || (vy && (!vx || x >= y));
        }
    }
    for (int i = tid; i < kSelBins; i += NT) h[i] = 0;
    if (tid == 0) {
        s_nt = 0;
        s_desc = 0;
    }
    __syncthreads();
    if (desc) s_desc = 1;  // (read after the barriers below)
    auto take = [&](int c, float x) __attribute__((always_inline)) {
        uint64_t comp = 0;
        const bool cand = c < nc && candidate_x(a, r, c, x, comp);
        const uint32_t key = cand ? (uint32_t)(comp >> 32) : 0u;
        if (c < nc) keys[c] = key;
        wave_hist_add(h, cand ? (int)(key >> kSelShift) : -1);
    };
    if (a.vec) {
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (4 * u * NT < nc)  // uniform: groups past the row are not taken
#pragma unroll
                for (int e = 0; e < 4; ++e) take(4 * (u * NT + tid) + e, xv[u][e]);
    } else {
#pragma unroll
        for (int u = 0; u < US; ++u)
            if (u * NT < nc) take(u * NT + tid, xs[u]);
    }
    __syncthreads();
    constexpr int HP = kSelBins / NT;  // first-level bins per thread
    uint32_t hv[HP];
#pragma unroll
    for (int e = 0; e < HP; ++e) hv[e] = h[kSelBins - 1 - HP * tid - e];
    const BinPick bp = pick_bin<NT, HP>(hv, m, scr);  // its barriers follow every thread's reads
    const uint32_t b1 = (uint32_t)bp.bin;
    // ---- bits of the columns above the bin (every candidate in mode 1), ties into LDS;
    // each wave takes 64 columns at a time and writes their two bitmap words
    if (bp.mode != 0) {
        constexpr int IT = kSmallCols / NT;  // 64-column groups per wave
        uint32_t kk[IT];
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int c = wave * 64 + it * NT + lane;
            kk[it] = c < nc ? keys[c] : 0u;
        }
        uint64_t tb[IT];
        uint32_t ntw = 0;
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int base = wave * 64 + it * NT;
            const uint32_t d1 = kk[it] >> kSelShift;
            const bool above = kk[it] != 0u && (bp.mode == 1 || d1 > b1);
            const uint64_t ab = __ballot(above);
            tb[it] = __ballot(kk[it] != 0u && bp.mode == 2 && d1 == b1);
            ntw += (uint32_t)__popcll(tb[it]);
            if (lane == 0 && base < words * 32) {
                lbits[base >> 5] = (uint32_t)ab;
                if ((base >> 5) + 1 < words) lbits[(base >> 5) + 1] = (uint32_t)(ab >> 32);
            }
        }
        if (ntw) {  // uniform per wave: one reservation in the tie list
            uint32_t sb = 0;
            if (lane == 0) sb = atomicAdd(&s_nt, ntw);
            sb = __builtin_amdgcn_readfirstlane(sb);
#pragma unroll
            for (int it = 0; it < IT; ++it) {
                if ((tb[it] >> lane) & 1ull) {
                    const int c = wave * 64 + it * NT + lane;
                    const uint32_t slot = sb + lane_rank(tb[it]);
                    lties[slot] = ((uint64_t)kk[it] << 32) | (uint32_t)~(uint32_t)pos_of(c);
                    tcol[slot] = (uint32_t)c;
                }
                sb += (uint32_t)__popcll(tb[it]);
            }
        }
    }
    __syncthreads();
    // ---- the chosen ties
    if (bp.mode == 2) {
        const uint32_t ntie = s_nt;
        const uint32_t need1 = m > bp.above ? m - bp.above : 0u;
        for (int i = tid; i < kB2; i += NT) h[i] = 0;
        __syncthreads();
        const uint64_t thr = tie_threshold<NT>([&](uint32_t i) { return lties[i]; }, ntie, need1, b1, h, h256, scr);
        for (uint32_t i = tid; i < ntie; i += NT)
            if (lties[i] >= thr) atomicOr(&lbits[tcol[i] >> 5], 1u << (tcol[i] & 31));
    }
    __syncthreads();
    // ---- ascending output: sink, the fill, the window, then -1
    int32_t *dst = a.idx + (int64_t)row * a.K;
    const int nsink = a.causal ? r.f_sink_end : 0;
    const int nwin = a.causal ? max(0, r.p - r.f_win_lo + 1) : 0;
    uint32_t nfill = 0;
    if (bp.mode != 0) {
        int32_t *fill = reinterpret_cast<int32_t *>(lties);  // KEPT: the fill's positions (the ties are done)
        const int per = (words + NT - 1) / NT;
        const int w0 = min(words, tid * per), w1 = min(words, w0 + per);
        uint32_t cn = 0;
        for (int i = w0; i < w1; ++i) cn += __popc(lbits[i]);
        uint32_t off = block_exscan<NT>(cn, scr, &nfill);
        nfill = min(nfill, m);
        for (int i = w0; i < w1; ++i) {
            uint32_t bits = lbits[i];
            while (bits && off < nfill) {
                const int c = i * 32 + __ffs(bits) - 1;
                bits &= bits - 1;
                if constexpr (KEPT) fill[off] = c;  // its position below
                else dst[nsink + off] = c;
                ++off;
            }
        }
        if constexpr (KEPT) {
            // columns -> positions through the kept map, each thread its own entries (the
            // loads independent of one another)
            __syncthreads();
            for (uint32_t i = tid; i < nfill; i += NT) fill[i] = pos_of(fill[i]);
            // a kept map whose valid entries ascend, then -1 (as lsa_select writes it), keeps
            // the columns in position order (checked with the loads); otherwise the fill is
            // sorted (bitonic, in LDS)
            __syncthreads();
            int np = 1;
            if (s_desc) while (np < (int)nfill) np <<= 1;
            for (int i = tid; i < np; i += NT)
                if ((uint32_t)i >= nfill) fill[i] = 0x7FFFFFFF;
            __syncthreads();
            for (int k = 2; k <= np; k <<= 1) {
                for (int j = k >> 1; j > 0; j >>= 1) {
                    for (int i = tid; i < np; i += NT) {
                        const int ixj = i ^ j;
                        if (ixj > i) {
                            const int x = fill[i], y = fill[ixj];
                            const bool up = (i & k) == 0;
                            if ((x > y) == up) {
                                fill[i] = y;
                                fill[ixj] = x;
                            }
                        }
                    }
                    __syncthreads();
                }
            }
            for (uint32_t i = tid; i < nfill; i += NT) dst[nsink + i] = fill[i];
        }
    }
    for (int s = tid; s < nsink; s += NT) dst[s] = s;
    const int wbase = nsink + (int)nfill;
    for (int j = tid; j < nwin; j += NT)
        if (wbase + j < a.K) dst[wbase + j] = r.f_win_lo + j;
    for (int i = wbase + nwin + tid; i < a.K; i += NT) dst[i] = -1;
    // the workspace's histogram and counters of this row are left at zero
    uint32_t *g1 = w.hist + (int64_t)row * kSelBins;
    for (int i = tid; i < kSelBins; i += NT) g1[i] = 0;
    if (tid < kCtr) w.ctr[(int64_t)row * kCtr + tid] = 0;
}

// ----------------------------------------------------------------------------- candidate lists
// The selection of a flat row from the candidate list its indexer wrote (every candidate
// whose bin could still reach the row's fill when it was scored; see the indexer), one
// workgroup per row with the row's state in LDS. Every candidate in a bin at or above the
// row's threshold bin is in the list, so the list's own first-level histogram agrees with
// the row's from the threshold bin up, and the threshold bin and the count above it come
// out the same. Then: candidates above the bin set their bit in an LDS bitmap of the row's
// positions, those in it go to an LDS tie list, the ties are ranked as in the resolve
// (or, when the LDS list overflows, by radix passes over the candidate list), and the
// bitmap is compacted into ascending positions.
constexpr int kCandT = 1024;
constexpr int kCandMaxWords = 16384;  // positions per row up to 2^19 (bitmap in LDS)

__global__ __launch_bounds__(kCandT) void select_cand_kernel(SelectArgs a, const uint64_t *cand,
                                                             const uint32_t *cand_cnt, int words, int tcap) {
    extern __shared__ __attribute__((aligned(16))) unsigned char dyn[];
    uint32_t *lbits = reinterpret_cast<uint32_t *>(dyn);                                  // [words]
    uint64_t *lties = reinterpret_cast<uint64_t *>(dyn + (size_t)((words + 3) & ~3) * 4);  // [tcap]
    __shared__ __attribute__((aligned(16))) uint32_t h[kB2];  // first level, then second level
    __shared__ uint32_t h256[256];
    __shared__ uint32_t scr[32];
    __shared__ uint32_t s_nt;
    constexpr int NT = kCandT;
    const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
    const Row r = make_row(a, row);
    const uint32_t m = (uint32_t)max(r.m, 0);
    const uint32_t ne = cand_cnt[row];
    const uint64_t *list = cand + (int64_t)row * a.N;

    for (int i = tid; i < words; i += NT) lbits[i] = 0;
    for (int i = tid; i < kSelBins; i += NT) h[i] = 0;
    if (tid == 0) s_nt = 0;
    __syncthreads();
    // the list in rounds of U entries per thread (U loads in flight)
    constexpr int U = 8;
    auto round = [&](uint32_t base, uint64_t (&c)[U], bool (&ok)[U]) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t i = base + u * NT + tid;
            ok[u] = i < ne;
            c[u] = list[ok[u] ? i : 0];
        }
    };
    // ---- first-level histogram of the list (lanes that share a bin add once)
    for (uint32_t base = 0; base < ne; base += U * NT) {
        uint64_t c[U];
        bool ok[U];
        round(base, c, ok);
#pragma unroll
        for (int u = 0; u < U; ++u) wave_hist_add(h, ok[u] ? (int)((uint32_t)(c[u] >> 32) >> kSelShift) : -1);
    }
    __syncthreads();
    uint32_t hv[2];
    hv[0] = h[kSelBins - 1 - 2 * tid];
    hv[1] = h[kSelBins - 2 - 2 * tid];
    const BinPick bp = pick_bin<NT, 2>(hv, m, scr);  // its barriers follow every thread's reads
    const uint32_t b1 = (uint32_t)bp.bin;

    // ---- classify: above the bin into the bitmap, in it into the tie list (one LDS
    // reservation per wave and round)
    if (bp.mode != 0) {
        for (uint32_t base = 0; base < ne; base += U * NT) {
            uint64_t c[U];
            bool ok[U];
            round(base, c, ok);
            uint64_t tb[U];
            uint32_t ntw = 0;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t d1 = (uint32_t)(c[u] >> kB1Shift);
                if (ok[u] && (bp.mode == 1 || d1 > b1)) {
                    const int pos = comp_pos(c[u]);
                    atomicOr(&lbits[pos >> 5], 1u << (pos & 31));
                }
                tb[u] = __ballot(ok[u] && bp.mode == 2 && d1 == b1);
                ntw += (uint32_t)__popcll(tb[u]);
            }
            if (ntw) {  // uniform per wave
                uint32_t sb = 0;
                if (lane == 0) sb = atomicAdd(&s_nt, ntw);
                sb = __builtin_amdgcn_readfirstlane(sb);
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    if ((tb[u] >> lane) & 1ull) {
                        const uint32_t slot = sb + lane_rank(tb[u]);
                        if (slot < (uint32_t)tcap) lties[slot] = c[u];
                    }
                    sb += (uint32_t)__popcll(tb[u]);
                }
            }
        }
    }
    __syncthreads();

    // ---- the chosen ties
    if (bp.mode == 2) {
        const uint32_t ntie = s_nt;
        const uint32_t need1 = m > bp.above ? m - bp.above : 0u;
        if (ntie <= (uint32_t)tcap) {
            for (int i = tid; i < kB2; i += NT) h[i] = 0;
            __syncthreads();
            const uint64_t thr = tie_threshold<NT>([&](uint32_t i) { return lties[i]; }, ntie, need1, b1, h, h256, scr);
            for (uint32_t i = tid; i < ntie; i += NT) {
                if (lties[i] >= thr) {
                    const int pos = comp_pos(lties[i]);
                    atomicOr(&lbits[pos >> 5], 1u << (pos & 31));
                }
            }
        } else {
            // the tie list did not fit: radix passes over the whole candidate list (entries
            // outside bin b1 do not match the prefix and are left out)
            const uint64_t pre = (uint64_t)b1 << kB1Shift;
            auto get = [&](uint32_t i) { return list[i]; };
            const uint64_t thr = radix_kth<NT>(FnSrc<decltype(get)>{get, (int)ne}, need1, pre, kB1Shift, h256, scr);
            for (uint32_t i = tid; i < ne; i += NT) {
                const uint64_t c = list[i];
                if ((c >> kB1Shift) == (uint64_t)b1 && c >= thr) {
                    const int pos = comp_pos(c);
                    atomicOr(&lbits[pos >> 5], 1u << (pos & 31));
                }
            }
        }
    }
    __syncthreads();

    // ---- ascending output: sink, the fill, the window, then -1
    int32_t *dst = a.idx + (int64_t)row * a.K;
    const int nsink = a.causal ? r.f_sink_end : 0;
    const int nwin = a.causal ? max(0, r.p - r.f_win_lo + 1) : 0;
    uint32_t nfill = 0;
    if (bp.mode != 0) {
        const int per = (words + NT - 1) / NT;
        const int w0 = min(words, tid * per), w1 = min(words, w0 + per);
        uint32_t cn = 0;
        for (int i = w0; i < w1; ++i) cn += __popc(lbits[i]);
        uint32_t off = block_exscan<NT>(cn, scr, &nfill);
        nfill = min(nfill, m);
        for (int i = w0; i < w1; ++i) {
            uint32_t bits = lbits[i];
            while (bits && off < nfill) {
                dst[nsink + off] = i * 32 + __ffs(bits) - 1;
                bits &= bits - 1;
                ++off;
            }
        }
    }
    for (int s = tid; s < nsink; s += NT) dst[s] = s;
    const int wbase = nsink + (int)nfill;
    for (int j = tid; j < nwin; j += NT)
        if (wbase + j < a.K) dst[wbase + j] = r.f_win_lo + j;
    for (int i = wbase + nwin + tid; i < a.K; i += NT) dst[i] = -1;
}

__global__ void clear_kernel(uint4 *p, size_t n16, uint8_t *tail, size_t ntail) {
    const size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t j = i; j < n16; j += stride) p[j] = make_uint4(0, 0, 0, 0);
    if (i < ntail) tail[i] = 0;
}

template <bool KEPT, int KPAD>
hipError_t launch_resolve_t(const SelectArgs &a, const Ws &w, hipStream_t s) {
    const int tcap = w.cap < kTieLds ? w.cap : kTieLds;
    const size_t tie_lds = (size_t)tcap * (KEPT ? 12 : 8);
    // the bitmap goes to LDS when it fits beside the ties and the static arrays (<= 38 KB)
    const size_t budget = (KEPT ? 122 : 126) * 1024;
    const int lwords = (w.words <= kBitsLds && tie_lds + (size_t)w.words * 4 <= budget) ? w.words : 0;
    const size_t lds = tie_lds + (size_t)lwords * 4;
    hipLaunchKernelGGL((select_resolve_kernel<KEPT, KPAD>), dim3(a.B * a.T), dim3(kRT), lds, s, a, w, lwords);
    return hipGetLastError();
}

hipError_t launch_resolve(const SelectArgs &a, const Ws &w, hipStream_t s) {
    if (!a.kept) return launch_resolve_t<false, 1>(a, w, s);
    if (a.K <= 1024) return launch_resolve_t<true, 1024>(a, w, s);
    if (a.K <= 2048) return launch_resolve_t<true, 2048>(a, w, s);
    return launch_resolve_t<true, 4096>(a, w, s);
}

// Columns per filter (and histogram) workgroup: about 1024 workgroups in all, at least
// 2048 columns each, a multiple of 32.
#ifndef LSA_FILTER_MIN_COLS
#define LSA_FILTER_MIN_COLS 2048
#endif
int part_columns(int rows, int n_cols, int &parts) {
    int p = (1024 + rows - 1) / rows;
    const int max_parts = (n_cols + LSA_FILTER_MIN_COLS - 1) / LSA_FILTER_MIN_COLS;
    if (p > max_parts) p = max_parts;
    if (p < 1) p = 1;
    int pc = (n_cols + p - 1) / p;
    pc = (pc + 31) / 32 * 32;
    parts = (n_cols + pc - 1) / pc;
    return pc;
}

}  // namespace

size_t select_workspace_bytes(int rows, int n_cols, bool kept) { return ws_total(rows, n_cols, kept); }

size_t select_zero_bytes(int rows) { return zero_bytes(rows); }

hipError_t launch_select_hist(const SelectArgs &a, void *wsp, hipStream_t s) {
    const int rows = a.B * a.T;
    if (!a.ws_clean) {
        const hipError_t e = launch_clear(wsp, zero_bytes(rows), s);
        if (e != hipSuccess) return e;
    }
    int parts;
    const int pc = part_columns(rows, a.n_cols, parts);
    const Ws w = carve(wsp, rows, a.n_cols, a.kept != nullptr);
    hipLaunchKernelGGL(select_hist_kernel, dim3(parts, rows), dim3(kHT), 0, s, a, w.hist, pc);
    return hipGetLastError();
}

hipError_t launch_select_front(const SelectArgs &a, void *wsp, hipStream_t s) {
    const int rows = a.B * a.T;
    if (!a.primed) {
        const hipError_t e = launch_select_hist(a, wsp, s);
        if (e != hipSuccess) return e;
    }
    const Ws w = carve(wsp, rows, a.n_cols, a.kept != nullptr);
    int parts;
    const int pc = part_columns(rows, a.n_cols, parts);
    if (a.kept) hipLaunchKernelGGL(select_filter_kernel<true>, dim3(parts, rows), dim3(kHT), 0, s, a, w, pc);
    else hipLaunchKernelGGL(select_filter_kernel<false>, dim3(parts, rows), dim3(kHT), 0, s, a, w, pc);
    return hipGetLastError();
}

size_t select_cand_lds(int n_cols, int &words, int &tcap) {
    words = bit_words(n_cols);
    if (words > kCandMaxWords) return 0;
    const size_t static_bytes = (size_t)kB2 * 4 + 256 * 4 + 32 * 4 + 16;
    const size_t budget = 160 * 1024 - static_bytes - 512;
    const size_t bits = (size_t)((words + 3) & ~3) * 4;
    if (bits + 1024 * 8 > budget) return 0;
    tcap = (int)min((size_t)16384, (budget - bits) / 8);
    return bits + (size_t)tcap * 8;
}

hipError_t launch_select_cand(const SelectArgs &a, const uint64_t *cand, const uint32_t *cand_cnt, hipStream_t s) {
    int words = 0, tcap = 0;
    const size_t lds = select_cand_lds(a.n_cols, words, tcap);
    if (!lds) return hipErrorInvalidValue;  // (callers check select_cand_fits first)
    hipLaunchKernelGGL(select_cand_kernel, dim3(a.B * a.T), dim3(kCandT), lds, s, a, cand, cand_cnt, words, tcap);
    return hipGetLastError();
}

bool select_cand_fits(int n_cols) {
    int words, tcap;
    return select_cand_lds(n_cols, words, tcap) != 0;
}

bool select_small(int n_cols) { return n_cols <= kSmallCols; }

hipError_t launch_select(const SelectArgs &a, void *wsp, hipStream_t s) {
    if (select_small(a.n_cols)) {
        const Ws w = carve(wsp, a.B * a.T, a.n_cols, a.kept != nullptr);
        if (a.kept) hipLaunchKernelGGL(select_small_kernel<true>, dim3(a.B * a.T), dim3(kSmallT), kSmallLds, s, a, w);
        else hipLaunchKernelGGL(select_small_kernel<false>, dim3(a.B * a.T), dim3(kSmallT), kSmallLds, s, a, w);
        return hipGetLastError();
    }
    const hipError_t e = launch_select_front(a, wsp, s);
    if (e != hipSuccess) return e;
    return launch_resolve(a, carve(wsp, a.B * a.T, a.n_cols, a.kept != nullptr), s);
}

hipError_t launch_clear(void *p, size_t bytes, hipStream_t s) {
    if (bytes == 0) return hipSuccess;
    const size_t n16 = bytes / 16;
    const size_t ntail = bytes % 16;
    uint8_t *tail = reinterpret_cast<uint8_t *>(p) + n16 * 16;
    size_t blocks = (n16 + 255) / 256;
    if (blocks < 1) blocks = 1;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(clear_kernel, dim3((unsigned)blocks), dim3(256), 0, s, reinterpret_cast<uint4 *>(p), n16, tail,
                       ntail);
    return hipGetLastError();
}

}  // namespace lsa
