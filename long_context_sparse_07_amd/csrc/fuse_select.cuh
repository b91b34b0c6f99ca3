// SI selection finished inside the indexer launch (flat token scores, one query token
// per workgroup): the workgroups that score one query's columns exchange what the
// selection needs through the workspace and two in-launch barriers per query, so the
// score row never makes a round trip through memory before the selection
// (LongCat-Flash-Lite-Sparse summary, "Good to know" and "Technical features", first
// bullet: the budget is a fixed sink, a local window and a top-k fill).
//
// Workgroup j of a query row holds its chunk's scores in LDS when the indexer loop ends.
//   A  it adds its candidate counts per first-level bin to the row's histogram (integer
//      atomics) and arrives at the row's first barrier;
//   B  every workgroup reads the whole histogram and picks the same threshold bin b1;
//      it marks its candidates above b1 in an LDS bitmap of its chunk and publishes
//      its count of them and its candidates in b1 (the ties) in its own slot of the
//      workspace, then arrives at the second barrier;
//   C  every workgroup reads every chunk's counts and the row's ties, ranks the ties
//      (the same for all), and so knows how many positions each chunk contributes:
//      its own positions go to idx at their rank in the ascending output, and it
//      writes its share of the sink, window and padding entries.
// Data crossing workgroups moves only through device-scope atomic operations and
// coherent (device-scope) loads and stores, ordered by waiting for a workgroup's memory
// operations before it arrives; no cache writeback is needed. The workgroups of a row
// are co-resident (cooperative launch); every barrier wait is bounded and records a
// flag in the workspace if it ever ran out, so no wait can hang.
#pragma once
#include "select_core.cuh"

namespace lsa {
namespace fsel {
using namespace sel;

constexpr int kSpinMax = 1 << 22;  // barrier polls before giving up (about 0.1 s)
// per-row counters (zero between calls): [0] arrivals at the first barrier, [1] at the
// second, [2] workgroups done with the row's workspace, [3] a barrier wait ran out
constexpr int kFCtr = 4;
// phase C LDS layout (bytes): chunk bitmap [0, 1024), second-level histogram [1024, 17408),
// radix histogram [17408, 18432), chosen ties per chunk [18432, 19456), then from kTieOff
// the row's tie list
constexpr int kTieOff = 19584;

__device__ __forceinline__ uint32_t ld_c(const uint32_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_c(const uint64_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_c(uint64_t *p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Arrive at a row barrier and wait for the row's nc workgroups. Every thread's memory
// operations issued before it are complete (performed) before the arrival is counted.
template <int NT>
__device__ void row_barrier(uint32_t *cnt, uint32_t nc, uint32_t *flag) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) {
        __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        int n = 0;
        while (ld_c(cnt) < nc) {
            __builtin_amdgcn_s_sleep(1);
            if (++n >= kSpinMax) {
                __hip_atomic_fetch_or(flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
        }
    }
    __syncthreads();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Phases B and C for workgroup j (of f.nc) of query row `row` (position p), chunk
// columns [c0, c1) with their scores in lsc (LDS). The row's histogram already holds
// this chunk's candidate counts (phase A adds, done by the caller). lds: scratch of
// lds_bytes (the indexer's key ring and lsc, both free from phase C on; phase B uses
// only the bytes below the key ring's end, ring_bytes).
template <int NT>
__device__ void run(const FusedSelArgs &f, int row, int j, int c0, int c1, int p, const float *lsc,
                    unsigned char *lds, int ring_bytes, int lds_bytes) {
    static_assert(kSelBins % NT == 0 && NT <= 1024 && NT >= 256, "threads per workgroup");
    __shared__ uint32_t scr[32];
    __shared__ uint32_t s_nab, s_nt;
    const int tid = threadIdx.x, lane = tid & 63;
    const int nc = f.nc;
    int sink_end, win_lo;
    forced_bounds(p, f.sink, f.window, sink_end, win_lo);
    const int nwin = max(0, p - win_lo + 1);
    const uint32_t m = (uint32_t)max(0, f.K - (sink_end + nwin));
    uint32_t *ghist = f.hist + (int64_t)row * kSelBins;
    uint32_t *gctr = f.ctr + (int64_t)row * kFCtr;
    uint64_t *gcnt = f.cnt + (int64_t)row * nc;
    uint64_t *gties = f.ties + (int64_t)row * nc * f.chunk;
    uint32_t *cb = reinterpret_cast<uint32_t *>(lds);  // chunk bitmap, [0, 1024)

    // ---- A: the row's histogram is complete once every chunk has arrived
    row_barrier<NT>(&gctr[0], (uint32_t)nc, &gctr[3]);

    // ---- B: threshold bin, then this chunk's candidates above it and in it
    constexpr int PER = kSelBins / NT;
    uint32_t hv[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) hv[e] = ld_c(&ghist[kSelBins - 1 - PER * tid - e]);
    const BinPick bp = pick_bin<NT, PER>(hv, m, scr);
    const int ncols = c1 - c0;
    for (int i = tid; i < 256; i += NT) cb[i] = 0;
    if (tid == 0) s_nab = 0, s_nt = 0;
    __syncthreads();
    uint64_t *lt = reinterpret_cast<uint64_t *>(lds + 1024);  // this chunk's ties (ring bytes only)
    const uint32_t b1 = (uint32_t)bp.bin;
    for (int base = 0; base < ncols; base += NT) {
        const int off = base + tid, col = c0 + off;
        bool cand = false;
        uint32_t key = 0;
        if (off < ncols) {
            const float x = lsc[off];
            cand = x > kNegInf && col >= sink_end && col < win_lo;  // win_lo <= p + 1
            key = order_key(x);
        }
        const uint32_t bin = key >> kSelShift;
        const uint64_t ba = __ballot(cand && (bp.mode == 1 || (bp.mode == 2 && bin > b1)));
        const uint64_t bt = __ballot(cand && bp.mode == 2 && bin == b1);
        const int w0 = base + (tid & ~63);  // this wave's first column offset (a multiple of 64)
        if (lane == 0 && w0 < ncols) {
            cb[w0 >> 5] = (uint32_t)ba;
            cb[(w0 >> 5) + 1] = (uint32_t)(ba >> 32);
            if (ba) atomicAdd(&s_nab, (uint32_t)__popcll(ba));
        }
        if (bt) {  // uniform per wave
            uint32_t sb = 0;
            if (lane == 0) sb = atomicAdd(&s_nt, (uint32_t)__popcll(bt));
            sb = __builtin_amdgcn_readfirstlane(sb);
            if ((bt >> lane) & 1ull) lt[sb + lane_rank(bt)] = ((uint64_t)key << 32) | (uint32_t)~(uint32_t)col;
        }
    }
    __syncthreads();
    const uint32_t nab = s_nab, nt = s_nt;
    for (uint32_t i = tid; i < nt; i += NT) st_c(&gties[(int64_t)j * f.chunk + i], lt[i]);
    if (tid == 0) st_c(&gcnt[j], ((uint64_t)nab << 32) | nt);

    // ---- C: every chunk's counts and the row's ties
    row_barrier<NT>(&gctr[1], (uint32_t)nc, &gctr[3]);
    uint32_t *h2 = reinterpret_cast<uint32_t *>(lds + 1024);  // [kB2]
    uint32_t *h256 = h2 + kB2;                                // [256]
    uint32_t *tcnt = h256 + 256;                              // [256] chosen ties per chunk
    __shared__ uint32_t s_tpre[257], s_nab_i[256];
    const uint64_t cv = tid < nc ? ld_c(&gcnt[tid]) : 0;
    uint32_t tot_t;
    const uint32_t ex_t = block_exscan<NT>((uint32_t)cv, scr, &tot_t);
    if (tid < nc) {
        s_tpre[tid] = ex_t;
        s_nab_i[tid] = (uint32_t)(cv >> 32);
        tcnt[tid] = 0;
    }
    if (tid == 0) s_tpre[nc] = tot_t;
    for (int i = tid; i < kB2; i += NT) h2[i] = 0;
    const uint32_t ntie = tot_t;
    const int tie_lds = (lds_bytes - kTieOff) / 8;
    uint64_t *ltr = reinterpret_cast<uint64_t *>(lds + kTieOff);
    __syncthreads();
    auto seg = [&](uint32_t e) {  // the chunk whose slot holds row tie e
        int lo = 0, hi = nc;      // s_tpre[lo] <= e < s_tpre[hi]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (s_tpre[mid] <= e) lo = mid;
            else hi = mid;
        }
        return lo;
    };
    auto gaddr = [&](uint32_t e) {
        const int s = seg(e);
        return &gties[(int64_t)s * f.chunk + (e - s_tpre[s])];
    };
    const bool in_lds = ntie <= (uint32_t)tie_lds;
    if (in_lds) {
        for (uint32_t e = tid; e < ntie; e += NT) ltr[e] = ld_c(gaddr(e));
        __syncthreads();
    }
    auto get = [&](uint32_t e) -> uint64_t { return in_lds ? ltr[e] : ld_c(gaddr(e)); };
    uint32_t above;  // candidates above the threshold bin over the whole row
    block_exscan<NT>(tid < nc ? (uint32_t)(cv >> 32) : 0u, scr, &above);
    uint32_t nfill = 0;
    if (bp.mode == 1) nfill = min(above, m);
    else if (bp.mode == 2) nfill = m;
    if (bp.mode == 2 && ntie > 0) {
        const uint32_t need1 = m > above ? m - above : 0u;
        uint64_t thr = ~(uint64_t)0;
        if (need1 > 0) thr = tie_threshold<NT>(get, ntie, need1, b1, h2, h256, scr);
        for (uint32_t e = tid; e < ntie; e += NT) {
            const uint64_t c = get(e);
            if (c >= thr) {
                const int s = seg(e);
                atomicAdd(&tcnt[s], 1u);
                if (s == j) {
                    const int off = comp_pos(c) - c0;
                    atomicOr(&cb[off >> 5], 1u << (off & 31));
                }
            }
        }
        __syncthreads();
    }
    // this chunk's first fill rank: positions contributed by the chunks before it
    const uint32_t sv = tid < nc ? s_nab_i[tid] + tcnt[tid] : 0u;
    uint32_t tot_s;
    const uint32_t ex_s = block_exscan<NT>(sv, scr, &tot_s);
    if (tid == j) scr[30] = ex_s;
    __syncthreads();
    const uint32_t off_j = scr[30];
    // ---- the chunk's positions, ascending, at their output ranks
    const int nw = (ncols + 31) >> 5;
    const uint32_t word = tid < nw ? cb[tid] : 0u;
    uint32_t tot_w;
    const uint32_t ex_w = block_exscan<NT>((uint32_t)__popc(word), scr, &tot_w);
    int32_t *out = f.idx + (int64_t)row * f.K;
    {
        // (the chunks' counts add up to nfill; the bound only keeps a miscount inside the row)
        const uint32_t fend = (uint32_t)sink_end + nfill;
        uint32_t x = word, r = sink_end + off_j + ex_w;
        while (x && r < fend) {
            const int b = __ffs(x) - 1;
            x &= x - 1;
            out[r++] = c0 + 32 * tid + b;
        }
    }
    // ---- this workgroup's share of the sink, window and padding entries
    const int k0 = (int)((int64_t)f.K * j / nc), k1 = (int)((int64_t)f.K * (j + 1) / nc);
    const int wbase = sink_end + (int)nfill;
    for (int k = k0 + tid; k < k1; k += NT) {
        if (k < sink_end) out[k] = k;
        else if (k >= wbase) out[k] = k < wbase + nwin ? win_lo + (k - wbase) : -1;
    }
    // ---- workspace hygiene: every read of the row's histogram happened before the
    // second barrier; this chunk clears its share of it. The last workgroup done with the
    // row's counters and ties clears the counters.
    const int hp = (kSelBins + nc - 1) / nc;
    for (int i = j * hp + tid; i < min(kSelBins, (j + 1) * hp); i += NT) ghist[i] = 0;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
        const uint32_t prev = __hip_atomic_fetch_add(&gctr[2], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (prev == (uint32_t)nc - 1) {
            const uint32_t fl = ld_c(&gctr[3]);
            gctr[0] = 0;
            gctr[1] = 0;
            gctr[2] = 0;
            gctr[3] = fl;  // a wait that ran out stays recorded
        }
    }
}

}  // namespace fsel
}  // namespace lsa
