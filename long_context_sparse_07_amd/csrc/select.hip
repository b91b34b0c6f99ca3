// SI selection on gfx950: per query token, the forced sink and local window plus the
// top-m fill by (score descending, position ascending)
// (LongCat-Flash-Lite-Sparse summary, "Good to know" and "Technical features", first
// bullet: the selection budget is split into a fixed sink and a local window).
//
// Exact multi-workgroup selection on a 64-bit composite key
//     comp = order_key(score) << 32 | ~position
// (larger comp = better: higher score, then lower position; composites are unique).
//   F1 hist:    every workgroup histograms the top 12 key bits of its column range in
//               LDS and adds it to the row's fine (4096-bin) and coarse (256-bin)
//               histograms with integer atomics.
//   F2 filter:  every workgroup finds the threshold bin b1 (the bin of the m-th best
//               candidate) from the coarse histogram and the 16 fine bins under it,
//               then appends the composites of its candidates in bins >= b1 to the
//               row's list (one atomic reservation per round).
//   R resolve:  one workgroup per row loads the list into LDS, finds the m-th largest
//               composite by 8-bit radix passes, marks the forced and chosen positions
//               in an LDS bitmap and writes them in ascending order (a bitonic sort
//               instead when positions exceed 2^19); it then zeroes its row's
//               histograms and counters for the next call.
// Kernel boundaries are the only cross-workgroup synchronisation (no device-scope
// fences). Membership is defined by the total order on composites and the output is
// sorted, so the result does not depend on the order in which atomics land.
#include "common.cuh"
#include "kernels.h"

namespace lsa {
namespace {

constexpr int kT = 256;
constexpr int kBins = 4096;          // 12-bit first-level digit
constexpr int kCh = 1024;            // F2 staging round (columns)
constexpr int kLcap = 4096;          // list entries resolved in LDS
constexpr int kBitmapMax = 1 << 19;  // positions handled by the LDS bitmap
constexpr int kCtr = 16;             // per-row counters

// ctr[row][*]
enum { C_NLIST = 0, C_NSURE = 1, C_MODE = 4, C_B1 = 5, C_ABOVE = 6 };

struct Ws {
    uint32_t *hist1;  // [rows][4096] fine histogram (top 12 key bits)
    uint32_t *hist0;  // [rows][256] coarse histogram (top 8 key bits)
    uint32_t *hist2;  // [rows][4096] next 12 key bits of the candidates in bin b1
    uint32_t *ctr;    // [rows][16]
    int32_t *sure;    // [rows][K] positions of candidates above bin b1
    uint64_t *list;   // [rows][cap] composites of candidates in bin b1
    int cap, K;
};

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

inline int list_cap(int n_cols) {
    int c = n_cols / 8;
    if (c < 8192) c = 8192;
    if (c > n_cols) c = n_cols;
    return (c + 63) / 64 * 64;
}

size_t zero_region_bytes(int rows) {
    return 2 * align256((size_t)rows * kBins * 4) + align256((size_t)rows * 256 * 4) + align256((size_t)rows * kCtr * 4);
}

Ws carve(void *base, int rows, int K, int n_cols) {
    Ws w;
    char *p = reinterpret_cast<char *>(base);
    w.hist1 = reinterpret_cast<uint32_t *>(p);
    p += align256((size_t)rows * kBins * 4);
    w.hist2 = reinterpret_cast<uint32_t *>(p);
    p += align256((size_t)rows * kBins * 4);
    w.hist0 = reinterpret_cast<uint32_t *>(p);
    p += align256((size_t)rows * 256 * 4);
    w.ctr = reinterpret_cast<uint32_t *>(p);
    p += align256((size_t)rows * kCtr * 4);
    w.sure = reinterpret_cast<int32_t *>(p);
    p += align256((size_t)rows * K * 4);
    w.list = reinterpret_cast<uint64_t *>(p);
    w.cap = list_cap(n_cols);
    w.K = K;
    return w;
}

size_t ws_bytes(int rows, int K, int n_cols) {
    return zero_region_bytes(rows) + align256((size_t)rows * K * 4) + align256((size_t)rows * list_cap(n_cols) * 8);
}

// Per-row context: query position, forced set, fill size.
struct Row {
    int b, t, p;
    int f_sink_end;  // sink = [0, f_sink_end)
    int f_win_lo;    // window = [f_win_lo, p] (empty when f_win_lo > p)
    int m;           // fill size
    const float *sc;
    const int32_t *kept;
    int nblk;
};

__device__ __forceinline__ Row make_row(const SelectArgs &a, int row) {
    Row r;
    r.b = row / a.T;
    r.t = row % a.T;
    int ctx = a.ctx_len ? a.ctx_len[r.b] : a.N;
    ctx = min(max(ctx, 0), a.N);
    r.p = ctx - a.T + r.t;
    if (a.causal) {
        const int pe = max(r.p + 1, 0);
        r.f_sink_end = min(a.sink, pe);
        r.f_win_lo = a.window > 0 ? max(r.f_sink_end, r.p - a.window + 1) : pe;
        r.f_win_lo = max(r.f_win_lo, 0);
        r.m = a.K - (r.f_sink_end + max(0, r.p - r.f_win_lo + 1));
    } else {
        r.f_sink_end = 0;
        r.f_win_lo = 0x7FFFFFFF;
        r.m = a.K;
    }
    r.sc = a.scores + (int64_t)row * a.n_cols;
    r.kept = a.kept ? a.kept + (int64_t)row * a.n_keep : nullptr;
    r.nblk = a.kept ? a.N / a.block_size : 0;
    return r;
}

__device__ __forceinline__ bool candidate_x(const SelectArgs &a, const Row &r, int col, float x, uint64_t &comp) {
    if (!(x > kNegInf)) return false;  // -inf and NaN are never selected
    int pos = col;
    if (r.kept) {
        const int blk = col / a.block_size;
        if (blk >= a.n_keep) return false;
        const int kb = r.kept[blk];
        if (kb < 0 || kb >= r.nblk) return false;
        pos = kb * a.block_size + (col - blk * a.block_size);
    }
    if (a.causal && (pos > r.p || pos < r.f_sink_end || pos >= r.f_win_lo)) return false;
    comp = ((uint64_t)order_key(x) << 32) | (uint32_t)(~(uint32_t)pos);
    return true;
}

__device__ __forceinline__ bool candidate(const SelectArgs &a, const Row &r, int col, uint64_t &comp) {
    return candidate_x(a, r, col, r.sc[col], comp);
}

__device__ __forceinline__ int comp_pos(uint64_t c) { return (int)(~(uint32_t)c); }

// Block-wide exclusive scan of one value per thread (256 threads, wave64).
__device__ uint32_t block_exscan(uint32_t v, uint32_t *lds4, uint32_t *total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        uint32_t y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    if (lane == 63) lds4[wave] = x;
    __syncthreads();
    uint32_t base = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        uint32_t s = lds4[w];
        if (w < wave) base += s;
        tot += s;
    }
    __syncthreads();
    *total = tot;
    return base + x - v;
}

// Threshold bin of the 4096-bin histogram h (LDS), counted from the top: the bin b with
// above(b) < need <= above(b) + h[b]. mode 0: need == 0; 1: total <= need (take all);
// 2: threshold bin found.
struct BinPick {
    int mode;
    int bin;
    uint32_t above;  // candidates in bins above `bin` (mode 2)
};

__device__ BinPick pick_bin(const uint32_t *h, uint32_t need, uint32_t *scratch) {
    const int tid = threadIdx.x;
    const int hi_bin = kBins - 1 - 16 * tid;  // thread tid owns 16 bins, walked from the top
    uint32_t s = 0;
#pragma unroll
    for (int e = 0; e < 16; ++e) s += h[hi_bin - e];
    uint32_t total;
    const uint32_t ex = block_exscan(s, scratch, &total);
    if (need == 0) return BinPick{0, kBins, 0};
    if (total <= need) return BinPick{1, -1, total};
    if (ex < need && need <= ex + s) {
        uint32_t acc = ex;
        for (int e = 0; e < 16; ++e) {
            const uint32_t c = h[hi_bin - e];
            if (acc + c >= need) {
                scratch[4] = (uint32_t)(hi_bin - e);
                break;
            }
            acc += c;
        }
    }
    __syncthreads();
    BinPick r{2, (int)scratch[4], 0};
    __syncthreads();
    return r;
}

// ----------------------------------------------------------------------------- F1
__global__ __launch_bounds__(kT) void select_hist_kernel(SelectArgs a, Ws ws, int part_cols) {
    __shared__ uint32_t h[kBins];
    const int row = blockIdx.y;
    const int c0 = blockIdx.x * part_cols;
    const int c1 = min(a.n_cols, c0 + part_cols);
    const bool vec = (a.n_cols & 3) == 0;
    for (int i = threadIdx.x; i < kBins; i += kT) h[i] = 0;
    __syncthreads();
    const Row r = make_row(a, row);
    if (r.m > 0) {
        for (int col = c0 + 4 * threadIdx.x; col < c1; col += 4 * kT) {
            float xs[4];
            if (vec && col + 3 < c1) {
                const float4 v = *reinterpret_cast<const float4 *>(r.sc + col);
                xs[0] = v.x, xs[1] = v.y, xs[2] = v.z, xs[3] = v.w;
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) xs[e] = col + e < c1 ? r.sc[col + e] : kNegInf;
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                uint64_t comp;
                if (col + e < c1 && candidate_x(a, r, col + e, xs[e], comp)) atomicAdd(&h[comp >> 52], 1u);
            }
        }
    }
    __syncthreads();
    uint32_t *g = ws.hist1 + (int64_t)row * kBins;
    uint32_t *g0 = ws.hist0 + (int64_t)row * 256;
    for (int i = threadIdx.x; i < kBins; i += kT)
        if (h[i]) atomicAdd(&g[i], h[i]);
    // coarse histogram of the top 8 bits: thread i sums fine bins [16 i, 16 i + 16)
    uint32_t s = 0;
#pragma unroll
    for (int e = 0; e < 16; ++e) s += h[16 * threadIdx.x + e];
    if (s) atomicAdd(&g0[threadIdx.x], s);
}

// Threshold bin b1 from the coarse (256) and fine (4096) row histograms: one coarse
// scan, then the 16 fine bins under the chosen coarse bin.
__device__ BinPick pick_bin2(const uint32_t *g0, const uint32_t *g1, uint32_t need, uint32_t *s16,
                             uint32_t *scratch) {
    const int tid = threadIdx.x;
    const uint32_t v = g0[255 - tid];  // thread tid owns coarse bin 255 - tid (top first)
    uint32_t total;
    const uint32_t ex = block_exscan(v, scratch, &total);
    if (need == 0) return BinPick{0, kBins, 0};
    if (total <= need) return BinPick{1, -1, total};
    if (ex < need && need <= ex + v) {
        scratch[4] = (uint32_t)(255 - tid);
        scratch[5] = ex;
    }
    __syncthreads();
    const int cb = (int)scratch[4];
    const uint32_t above = scratch[5];
    if (tid < 16) s16[tid] = g1[16 * cb + 15 - tid];  // fine bins of cb, top first
    __syncthreads();
    if (tid == 0) {
        uint32_t acc = above;
        for (int e = 0; e < 16; ++e) {
            if (acc + s16[e] >= need) {
                scratch[6] = (uint32_t)(16 * cb + 15 - e);
                scratch[7] = acc;
                break;
            }
            acc += s16[e];
        }
    }
    __syncthreads();
    BinPick r{2, (int)scratch[6], scratch[7]};
    __syncthreads();
    return r;
}

// ----------------------------------------------------------------------------- F2
__global__ __launch_bounds__(kT) void select_filter_kernel(SelectArgs a, Ws ws, int part_cols) {
    __shared__ int32_t sbuf[kCh];
    __shared__ uint64_t lbuf[kCh];
    __shared__ uint32_t h2[kBins];
    __shared__ uint32_t cnt[4];
    __shared__ uint32_t s16[16];
    __shared__ uint32_t scratch[8];
    const int row = blockIdx.y;
    const int tid = threadIdx.x;
    const int c0 = blockIdx.x * part_cols;
    const int c1 = min(a.n_cols, c0 + part_cols);
    const bool vec = (a.n_cols & 3) == 0;
    const Row r = make_row(a, row);
    uint32_t *ctr = ws.ctr + (int64_t)row * kCtr;
    int32_t *gsure = ws.sure + (int64_t)row * ws.K;
    uint64_t *glist = ws.list + (int64_t)row * ws.cap;
    if (tid < 4) cnt[tid] = 0;
    for (int i = tid; i < kBins; i += kT) h2[i] = 0;
    // the first round's scores are loaded before the threshold pick (independent loads)
    constexpr int PRE = kCh / (4 * kT);
    float4 pre[PRE];
    {
        const int end = min(c1, c0 + kCh);
#pragma unroll
        for (int u = 0; u < PRE; ++u) {
            const int col = c0 + 4 * (tid + u * kT);
            if (vec && col + 3 < end) pre[u] = *reinterpret_cast<const float4 *>(r.sc + col);
            else pre[u] = make_float4(kNegInf, kNegInf, kNegInf, kNegInf);
        }
    }
    const BinPick bp = pick_bin2(ws.hist0 + (int64_t)row * 256, ws.hist1 + (int64_t)row * kBins,
                                 (uint32_t)max(r.m, 0), s16, scratch);
    if (blockIdx.x == 0 && tid == 0) {
        ctr[C_MODE] = (uint32_t)bp.mode;
        ctr[C_B1] = (uint32_t)bp.bin;
        ctr[C_ABOVE] = bp.above;
    }
    if (bp.mode == 0) return;
    const int b1 = bp.bin;
    bool any_tie = false;
    auto classify = [&](int col, float x) {
        uint64_t comp;
        if (candidate_x(a, r, col, x, comp)) {
            const int d1 = (int)(comp >> 52);
            if (bp.mode == 1 || d1 > b1) {
                sbuf[atomicAdd(&cnt[0], 1u)] = comp_pos(comp);
            } else if (d1 == b1) {
                atomicAdd(&h2[(comp >> 40) & (kBins - 1)], 1u);
                lbuf[atomicAdd(&cnt[1], 1u)] = comp;
            }
        }
    };
    auto classify4 = [&](int col, int end, bool have, float4 v) {
        if (col >= end) return;
        if (have && col + 3 < end) {
            classify(col, v.x);
            classify(col + 1, v.y);
            classify(col + 2, v.z);
            classify(col + 3, v.w);
        } else {
            for (int e = 0; e < 4 && col + e < end; ++e) classify(col + e, r.sc[col + e]);
        }
    };
    auto flush = [&]() {
        __syncthreads();
        if (tid == 0) {
            cnt[2] = cnt[0] ? atomicAdd(&ctr[C_NSURE], cnt[0]) : 0;
            cnt[3] = cnt[1] ? atomicAdd(&ctr[C_NLIST], cnt[1]) : 0;
        }
        __syncthreads();
        const uint32_t ns = cnt[0], nl = cnt[1], os = cnt[2], ol = cnt[3];
        any_tie |= nl > 0;
        for (uint32_t i = tid; i < ns; i += kT)
            if (os + i < (uint32_t)ws.K) gsure[os + i] = sbuf[i];
        for (uint32_t i = tid; i < nl; i += kT)
            if (ol + i < (uint32_t)ws.cap) glist[ol + i] = lbuf[i];
        __syncthreads();
        if (tid < 2) cnt[tid] = 0;
        __syncthreads();
    };
    {  // first round from the prefetched registers
        const int end = min(c1, c0 + kCh);
#pragma unroll
        for (int u = 0; u < PRE; ++u) {
            const int col = c0 + 4 * (tid + u * kT);
            classify4(col, end, vec, pre[u]);
        }
        flush();
    }
    for (int base = c0 + kCh; base < c1; base += kCh) {
        const int end = min(c1, base + kCh);
        for (int col = base + 4 * tid; col < end; col += 4 * kT) {
            const bool have = vec && col + 3 < end;
            const float4 v = have ? *reinterpret_cast<const float4 *>(r.sc + col) : make_float4(0.f, 0.f, 0.f, 0.f);
            classify4(col, end, have, v);
        }
        flush();
    }
    if (any_tie) {
        uint32_t *g2 = ws.hist2 + (int64_t)row * kBins;
        for (int i = tid; i < kBins; i += kT)
            if (h2[i]) atomicAdd(&g2[i], h2[i]);
    }
}

// ----------------------------------------------------------------------------- R resolve helpers

struct ArrSrc {
    const uint64_t *p;
    int n;
    __device__ int size() const { return n; }
    __device__ bool get(int i, uint64_t &c) const {
        c = p[i];
        return true;
    }
};
struct RowSrc {
    const SelectArgs *a;
    const Row *r;
    __device__ int size() const { return a->n_cols; }
    __device__ bool get(int i, uint64_t &c) const { return candidate(*a, *r, i, c); }
};

// LDS histogram increment for digit d (-1: none) with same-digit lanes of the wave
// merged into one atomic (radix digits of nearly sorted keys are mostly equal).
__device__ __forceinline__ void wave_hist_add(uint32_t *h, int d) {
    const int d0 = __builtin_amdgcn_readfirstlane(d);
    const uint64_t same = __ballot(d == d0);
    if (d == d0) {
        if (d0 >= 0 && (int)__lane_id() == __ffsll((unsigned long long)same) - 1) atomicAdd(&h[d0], (uint32_t)__popcll(same));
    } else if (d >= 0) {
        atomicAdd(&h[d], 1u);
    }
}

__device__ __forceinline__ bool hi_match(uint64_t c, uint64_t pref, int bits) {
    return bits >= 64 ? true : (c >> bits) == (pref >> bits);
}

// need-th largest composite of the source (1 <= need <= size), by 8-bit radix passes
// from the top bit; returns the smallest composite that still belongs to the top
// `need` (every element >= it is selected, exactly `need` of them).
template <class Src>
__device__ uint64_t radix_kth(const Src &src, uint32_t need, uint32_t *h256, uint32_t *scratch) {
    uint64_t pref = 0;
    for (int sh = 56; sh >= 0; sh -= 8) {
        for (int i = threadIdx.x; i < 256; i += kT) h256[i] = 0;
        __syncthreads();
        const int n = src.size();
        const int nr = (n + kT - 1) / kT * kT;  // every lane takes part in the wave merge
        for (int i = threadIdx.x; i < nr; i += kT) {
            uint64_t c = 0;
            const bool ok = i < n && src.get(i, c) && hi_match(c, pref, sh + 8);
            wave_hist_add(h256, ok ? (int)((c >> sh) & 255) : -1);
        }
        __syncthreads();
        if (threadIdx.x < 64) {
            const int lane = threadIdx.x;
            const int hi = 255 - 4 * lane;  // lane owns 4 digits, scanned from the top
            const uint32_t s = h256[hi] + h256[hi - 1] + h256[hi - 2] + h256[hi - 3];
            uint32_t x = s;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const uint32_t y = __shfl_up(x, o, 64);
                if (lane >= o) x += y;
            }
            const uint32_t ex = x - s;
            if (ex < need && need <= x) {
                uint32_t acc = ex;
                for (int e = 0; e < 4; ++e) {
                    const uint32_t c = h256[hi - e];
                    if (acc + c >= need) {
                        scratch[0] = (uint32_t)(hi - e);
                        scratch[1] = need - acc;
                        scratch[2] = (c == need - acc);
                        break;
                    }
                    acc += c;
                }
            }
        }
        __syncthreads();
        const uint32_t d = scratch[0];
        need = scratch[1];
        const bool whole = scratch[2] != 0;
        __syncthreads();
        pref |= (uint64_t)d << sh;
        if (whole) return pref;  // lower bits zero: every element with this prefix
    }
    return pref;
}

// ----------------------------------------------------------------------------- R
// Threshold inside bin b1 from the row's second-level histogram (LDS copy h): the bin b2
// of the r1-th best tie candidate, and how many tie candidates lie above it.
__device__ void pick_bin_lds(const uint32_t *h, uint32_t need, uint32_t *scratch, int &bin, uint32_t &above) {
    const int tid = threadIdx.x;
    const int hi_bin = kBins - 1 - 16 * tid;
    uint32_t s = 0;
#pragma unroll
    for (int e = 0; e < 16; ++e) s += h[hi_bin - e];
    uint32_t total;
    const uint32_t ex = block_exscan(s, scratch, &total);
    if (ex < need && need <= ex + s) {
        uint32_t acc = ex;
        for (int e = 0; e < 16; ++e) {
            const uint32_t c = h[hi_bin - e];
            if (acc + c >= need) {
                scratch[4] = (uint32_t)(hi_bin - e);
                scratch[5] = acc;
                break;
            }
            acc += c;
        }
    }
    __syncthreads();
    bin = (int)scratch[4];
    above = scratch[5];
    __syncthreads();
}

template <int KPAD>
__global__ __launch_bounds__(kT) void select_resolve_kernel(SelectArgs a, Ws ws, int bitmap_words) {
    extern __shared__ __attribute__((aligned(16))) unsigned char dyn[];
    uint64_t *lst = reinterpret_cast<uint64_t *>(dyn);               // tie list [kLcap]
    uint32_t *area = reinterpret_cast<uint32_t *>(dyn + kLcap * 8);  // bitmap or sort buffer
    __shared__ uint32_t h[kBins];
    __shared__ uint32_t cnt[4];
    __shared__ uint32_t h256[256];
    __shared__ uint32_t scratch[8];
    __shared__ uint64_t tiny[256];
    __shared__ int32_t sure_l[KPAD];
    const int row = blockIdx.x;
    const int tid = threadIdx.x;
    const Row r = make_row(a, row);
    uint32_t *ctr = ws.ctr + (int64_t)row * kCtr;
    const uint64_t *glist = ws.list + (int64_t)row * ws.cap;
    const int32_t *gsure = ws.sure + (int64_t)row * ws.K;
    uint32_t *g2 = ws.hist2 + (int64_t)row * kBins;
    const int mode = (int)ctr[C_MODE];
    const int b1 = (int)ctr[C_B1];
    const uint32_t n_sure = mode == 0 ? 0u : min(ctr[C_NSURE], (uint32_t)ws.K);
    const uint32_t n_list = mode == 2 ? ctr[C_NLIST] : 0u;
    const uint32_t need1 = mode == 2 ? (uint32_t)max(r.m, 0) - ctr[C_ABOVE] : 0u;  // wanted from bin b1
    const bool in_lds = n_list <= (uint32_t)kLcap;
    const bool in_glb = n_list <= (uint32_t)ws.cap;
    // issue every independent load first: second-level histogram, tie list, sure list
    {
        uint32_t hv[kBins / kT];
#pragma unroll
        for (int u = 0; u < kBins / kT; ++u) hv[u] = mode == 2 ? g2[tid + u * kT] : 0u;
        constexpr int U = kLcap / kT;
        uint64_t lv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t i = tid + u * kT;
            lv[u] = (in_lds && i < n_list) ? __builtin_nontemporal_load(&glist[i]) : 0;
        }
        constexpr int US = KPAD / kT;
        int32_t sv[US];
#pragma unroll
        for (int u = 0; u < US; ++u) {
            const uint32_t i = tid + u * kT;
            sv[u] = i < n_sure ? gsure[i] : 0;
        }
#pragma unroll
        for (int u = 0; u < kBins / kT; ++u) h[tid + u * kT] = hv[u];
#pragma unroll
        for (int u = 0; u < U; ++u) lst[tid + u * kT] = lv[u];
#pragma unroll
        for (int u = 0; u < US; ++u) sure_l[tid + u * kT] = sv[u];
    }
    if (tid == 0) cnt[0] = 0;
    __syncthreads();
    // ---- threshold composite thr: the chosen tie candidates are those with comp >= thr
    uint64_t thr = 0;
    bool from_row = false;  // exact select over the whole row (large tie groups, overflowed list)
    if (mode == 2) {
        int b2;
        uint32_t above2;
        pick_bin_lds(h, need1, scratch, b2, above2);
        const uint32_t need2 = need1 - above2;                    // wanted from (b1, b2)
        const uint64_t p24 = ((uint64_t)b1 << 52) | ((uint64_t)b2 << 40);
        const uint32_t n2 = h[b2];
        if (need2 == n2) {
            thr = p24;              // the whole (b1, b2) group
            from_row = !in_glb;     // list incomplete: enumerate comp >= thr from the row
        } else if (n2 <= 256 && in_glb) {
            // the few (b1, b2) elements into LDS, then exact radix select on their composites
            auto gather = [&](uint64_t c) {
                if ((c >> 40) == (p24 >> 40)) {
                    const uint32_t slot = atomicAdd(&cnt[0], 1u);
                    if (slot < 256u) tiny[slot] = c;
                }
            };
            if (in_lds) {
                for (uint32_t i = tid; i < n_list; i += kT) gather(lst[i]);
            } else {
                for (uint32_t i = tid; i < n_list; i += kT) gather(glist[i]);
            }
            __syncthreads();
            // rank of each gathered composite (composites are unique): the need2-th largest
            // is the one with exactly need2 - 1 larger elements
            const uint32_t nt = min(cnt[0], 256u);
            if ((uint32_t)tid < nt) {
                const uint64_t c = tiny[tid];
                uint32_t rank = 0;
                for (uint32_t j = 0; j < nt; ++j) rank += tiny[j] > c;
                if (rank == need2 - 1) {
                    scratch[0] = (uint32_t)c;
                    scratch[1] = (uint32_t)(c >> 32);
                }
            }
            __syncthreads();
            thr = ((uint64_t)scratch[1] << 32) | scratch[0];
        } else {
            // many equal keys or an overflowed list: exact select over the whole row
            const RowSrc rsrc{&a, &r};
            thr = radix_kth(rsrc, (uint32_t)max(r.m, 0), h256, scratch);
            from_row = true;
        }
    }
    int32_t *dst = a.idx + (int64_t)row * a.K;
    // chosen fill positions: the sure list plus the tie candidates with comp >= thr, or,
    // when the row had to be scanned, every candidate with comp >= thr
    auto for_chosen = [&](auto &&fn) {
        if (mode == 0) return;
        if (from_row) {
            for (int i = tid; i < a.n_cols; i += kT) {
                uint64_t c;
                if (candidate(a, r, i, c) && c >= thr) fn(comp_pos(c));
            }
            return;
        }
        for (uint32_t i = tid; i < n_sure; i += kT) fn(sure_l[i]);
        if (mode != 2) return;
        if (in_lds) {
            for (uint32_t i = tid; i < n_list; i += kT)
                if (lst[i] >= thr) fn(comp_pos(lst[i]));
        } else {
            for (uint32_t i = tid; i < n_list; i += kT) {
                const uint64_t c = glist[i];
                if (c >= thr) fn(comp_pos(c));
            }
        }
    };
    // ---- ascending output: sink [0, f_sink_end), then the fill (all strictly between
    // sink and window), then the window [f_win_lo, p]
    if (bitmap_words > 0) {
        for (int i = tid; i < bitmap_words; i += kT) area[i] = 0;
        __syncthreads();
        for_chosen([&](int pos) { atomicOr(&area[pos >> 5], 1u << (pos & 31)); });
        __syncthreads();
        const int per = (bitmap_words + kT - 1) / kT;
        const int w0 = min(bitmap_words, tid * per), w1 = min(bitmap_words, w0 + per);
        uint32_t c = 0;
        for (int i = w0; i < w1; ++i) c += __popc(area[i]);
        uint32_t nfill;
        const int nsink = a.causal ? r.f_sink_end : 0;
        const int nwin = a.causal ? max(0, r.p - r.f_win_lo + 1) : 0;
        uint32_t off = nsink + block_exscan(c, scratch, &nfill);
        for (int i = w0; i < w1; ++i) {
            uint32_t bits = area[i];
            while (bits) {
                const int bpos = __ffs(bits) - 1;
                bits &= bits - 1;
                if (off < (uint32_t)a.K) dst[off] = i * 32 + bpos;
                ++off;
            }
        }
        for (int s2 = tid; s2 < nsink; s2 += kT) dst[s2] = s2;
        const int wbase = nsink + (int)nfill;
        for (int j = tid; j < nwin; j += kT)
            if (wbase + j < a.K) dst[wbase + j] = r.f_win_lo + j;
        for (int i = wbase + nwin + tid; i < a.K; i += kT) dst[i] = -1;
    } else {
        int32_t *out = reinterpret_cast<int32_t *>(area);
        for (int i = tid; i < KPAD; i += kT) out[i] = 0x7FFFFFFF;
        if (tid == 0) cnt[2] = 0;
        __syncthreads();
        auto emit = [&](int pos) {
            const uint32_t slot = atomicAdd(&cnt[2], 1u);
            if (slot < (uint32_t)KPAD) out[slot] = pos;
        };
        if (a.causal) {
            for (int s = tid; s < r.f_sink_end; s += kT) emit(s);
            for (int s = r.f_win_lo + tid; s <= r.p; s += kT) emit(s);
        }
        for_chosen(emit);
        __syncthreads();
        const uint32_t count = min(cnt[2], (uint32_t)KPAD);
        for (int k = 2; k <= KPAD; k <<= 1) {
            for (int j = k >> 1; j > 0; j >>= 1) {
                for (int i = tid; i < KPAD; i += kT) {
                    const int ixj = i ^ j;
                    if (ixj > i) {
                        const int x = out[i], y = out[ixj];
                        const bool up = (i & k) == 0;
                        if ((x > y) == up) {
                            out[i] = y;
                            out[ixj] = x;
                        }
                    }
                }
                __syncthreads();
            }
        }
        for (int i = tid; i < a.K; i += kT) dst[i] = (uint32_t)i < count ? out[i] : -1;
    }
    // ---- leave the row's histograms and counters at zero for the next call
    uint32_t *g = ws.hist1 + (int64_t)row * kBins;
    for (int i = tid; i < kBins; i += kT) {
        g[i] = 0;
        g2[i] = 0;
    }
    ws.hist0[(int64_t)row * 256 + tid] = 0;
    if (tid < kCtr) ctr[tid] = 0;
}

__global__ void clear_kernel(uint4 *p, size_t n16, uint8_t *tail, size_t ntail) {
    const size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t j = i; j < n16; j += stride) p[j] = make_uint4(0, 0, 0, 0);
    if (i < ntail) tail[i] = 0;
}

template <int KPAD>
hipError_t launch_resolve(const SelectArgs &a, const Ws &w, int rows, hipStream_t s) {
    const int64_t npos = (a.causal || a.kept) ? (int64_t)a.N : (int64_t)a.n_cols;  // positions bound
    const int words = npos <= kBitmapMax ? (int)((npos + 31) / 32) : 0;
    const size_t area = words ? (size_t)words * 4 : (size_t)KPAD * 4;
    const size_t lds = (size_t)kLcap * 8 + area;
    hipLaunchKernelGGL((select_resolve_kernel<KPAD>), dim3(rows), dim3(kT), lds, s, a, w, words);
    return hipGetLastError();
}

}  // namespace

size_t select_workspace_bytes(const SelectArgs &a) { return ws_bytes(a.B * a.T, a.K, a.n_cols); }

hipError_t launch_select(const SelectArgs &a, void *wsp, hipStream_t s) {
    const int rows = a.B * a.T;
    Ws w = carve(wsp, rows, a.K, a.n_cols);
    hipError_t e;
    if (!a.ws_clean) {
        e = launch_clear(wsp, zero_region_bytes(rows), s);
        if (e != hipSuccess) return e;
    }
    int parts = (1024 + rows - 1) / rows;
    const int max_parts = (a.n_cols + 2047) / 2048;
    if (parts > max_parts) parts = max_parts;
    if (parts < 1) parts = 1;
    int part_cols = (a.n_cols + parts - 1) / parts;
    part_cols = (part_cols + 3) / 4 * 4;
    parts = (a.n_cols + part_cols - 1) / part_cols;
    dim3 grid(parts, rows);
    hipLaunchKernelGGL(select_hist_kernel, grid, dim3(kT), 0, s, a, w, part_cols);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(select_filter_kernel, grid, dim3(kT), 0, s, a, w, part_cols);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.K <= 512) return launch_resolve<512>(a, w, rows, s);
    if (a.K <= 1024) return launch_resolve<1024>(a, w, rows, s);
    if (a.K <= 2048) return launch_resolve<2048>(a, w, rows, s);
    return launch_resolve<4096>(a, w, rows, s);
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
