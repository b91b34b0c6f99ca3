// Exact SI selection machinery shared by the selection kernels and the fused
// selection + attention kernel: the 64-bit composite order, the per-row context, block
// scans, the threshold-bin pick, radix selection inside a group, and the per-row
// workspace layout (LongCat-Flash-Lite-Sparse summary, "Good to know" and "Technical
// features": a fixed sink and local window, the rest of the budget by top-k).
#pragma once
#include "common.cuh"
#include "kernels.h"

namespace lsa {
namespace sel {

constexpr int kB2 = 4096;            // second-level bins: the next 12 key bits
constexpr int kL2Shift = kSelShift - 12;
constexpr int kGrpShift = 32 + kL2Shift;  // composite bits above it: the 23 key bits of (b1, b2)
constexpr int kB1Shift = 32 + kSelShift;  // composite bits above it: the 11 key bits of b1
constexpr int kTieLds = 8192;        // tie entries the resolve keeps in LDS
constexpr int kBitsLds = 8192;       // bitmap words the resolve keeps in LDS
constexpr int kTiny = 1024;          // a final group up to this size is ranked directly
constexpr int kCtr = 16;             // per-row counters: [0] tie count, [1..3] the filter's pick
                                     // (mode, bin, count above), [15] sliced-resolve arrivals

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Tie list capacity per row: every column when the rows together stay within 2^24
// entries, else 2^24 / rows (at least 8192); a longer threshold bin is resolved by
// rescanning the row.
inline int tie_cap(int rows, int n_cols) {
    const int64_t all = ((int64_t)n_cols + 63) / 64 * 64;
    int64_t c = ((int64_t)(1 << 24) / rows + 63) / 64 * 64;
    if (c < kTieLds) c = kTieLds;
    return (int)(all < c ? all : c);
}
inline int bit_words(int n_cols) { return (n_cols + 31) / 32; }

// Workspace: per row the first-level histogram and counters (kept at zero between
// calls), the tie list (composites, and columns when a kept map is used) and the column
// bitmap (rewritten by every call).
struct Ws {
    uint32_t *hist;   // [rows][kSelBins]
    uint32_t *ctr;    // [rows][kCtr]
    uint64_t *ties;   // [rows][cap]
    uint32_t *tcols;  // [rows][cap] (kept map only)
    uint32_t *bits;   // [rows][words]
    int cap, words;
};

inline size_t zero_bytes(int rows) { return align256((size_t)rows * kSelBins * 4) + align256((size_t)rows * kCtr * 4); }

inline Ws carve(void *base, int rows, int n_cols, bool kept) {
    Ws w;
    char *p = reinterpret_cast<char *>(base);
    w.cap = tie_cap(rows, n_cols);
    w.words = bit_words(n_cols);
    w.hist = reinterpret_cast<uint32_t *>(p);
    p += align256((size_t)rows * kSelBins * 4);
    w.ctr = reinterpret_cast<uint32_t *>(p);
    p += align256((size_t)rows * kCtr * 4);
    w.ties = reinterpret_cast<uint64_t *>(p);
    p += align256((size_t)rows * w.cap * 8);
    w.tcols = kept ? reinterpret_cast<uint32_t *>(p) : nullptr;
    if (kept) p += align256((size_t)rows * w.cap * 4);
    w.bits = reinterpret_cast<uint32_t *>(p);
    return w;
}

inline size_t ws_total(int rows, int n_cols, bool kept) {
    const int cap = tie_cap(rows, n_cols);
    return zero_bytes(rows) + align256((size_t)rows * cap * 8) + (kept ? align256((size_t)rows * cap * 4) : 0) +
           align256((size_t)rows * bit_words(n_cols) * 4);
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
        forced_bounds(r.p, a.sink, a.window, r.f_sink_end, r.f_win_lo);
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

// candidate_x with the column's kept-map entry already loaded (kb = kept[col / block_size]
// when that block index is below n_keep)
__device__ __forceinline__ bool candidate_kb(const SelectArgs &a, const Row &r, int col, float x, int kb, uint64_t &comp) {
    if (!(x > kNegInf)) return false;
    const int blk = col / a.block_size;
    if (blk >= a.n_keep || kb < 0 || kb >= r.nblk) return false;
    const int pos = kb * a.block_size + (col - blk * a.block_size);
    if (a.causal && (pos > r.p || pos < r.f_sink_end || pos >= r.f_win_lo)) return false;
    comp = ((uint64_t)order_key(x) << 32) | (uint32_t)(~(uint32_t)pos);
    return true;
}

__device__ __forceinline__ int comp_pos(uint64_t c) { return (int)(~(uint32_t)c); }

__device__ __forceinline__ uint32_t lane_rank(uint64_t mask) {  // set lanes of mask below this lane
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Block-wide exclusive scan of one value per thread (NT threads, wave64); lds >= NT/64 words.
template <int NT>
__device__ uint32_t block_exscan(uint32_t v, uint32_t *lds, uint32_t *total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    if (lane == 63) lds[wave] = x;
    __syncthreads();
    uint32_t base = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
        const uint32_t s = lds[w];
        if (w < wave) base += s;
        tot += s;
    }
    __syncthreads();
    *total = tot;
    return base + x - v;
}

// Threshold bin of an NB-bin LDS histogram counted from the top bin: the bin b with
// above(b) < need <= above(b) + h[b]. mode 0: need == 0 (nothing); 1: total <= need
// (take everything); 2: threshold bin found. scr >= 24 words.
struct BinPick {
    int mode;
    int bin;
    uint32_t above;  // elements in bins above `bin` (mode 2), or the total (mode 1)
};

// v[e] is bin NB - 1 - PER * threadIdx.x - e of an NB = NT * PER bin histogram.
template <int NT, int PER>
__device__ BinPick pick_bin(const uint32_t (&v)[PER], uint32_t need, uint32_t *scr) {
    constexpr int NB = NT * PER;
    const int top = NB - 1 - PER * (int)threadIdx.x;
    uint32_t s = 0;
#pragma unroll
    for (int e = 0; e < PER; ++e) s += v[e];
    uint32_t total;
    const uint32_t ex = block_exscan<NT>(s, scr, &total);
    if (need == 0) return BinPick{0, NB, 0};
    if (total <= need) return BinPick{1, -1, total};
    if (ex < need && need <= ex + s) {
        uint32_t acc = ex;
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            if (acc < need && need <= acc + v[e]) {
                scr[16] = (uint32_t)(top - e);
                scr[17] = acc;
            }
            acc += v[e];
        }
    }
    __syncthreads();
    const BinPick r{2, (int)scr[16], scr[17]};
    __syncthreads();
    return r;
}

// ----------------------------------------------------------------------------- radix
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
    __device__ bool get(int i, uint64_t &c) const { return candidate_x(*a, *r, i, r->sc[i], c); }
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

// need-th largest composite (1 <= need <= group size) of the group of source elements
// whose bits at and above bit `lo_bits` equal those of pref; radix passes of up to 8
// bits over the low lo_bits bits (0 < lo_bits < 64). Returns the smallest composite
// that still belongs to the group's top `need`: those are exactly the group elements
// >= it.
template <int NT, class Src>
__device__ uint64_t radix_kth(const Src &src, uint32_t need, uint64_t pref, int lo_bits, uint32_t *h256,
                              uint32_t *scr) {
    int hi = lo_bits;
    pref = pref >> hi << hi;
    while (hi > 0) {
        const int w = hi < 8 ? hi : 8;
        const int sh = hi - w;
        const uint32_t dmask = (1u << w) - 1;
        for (int i = threadIdx.x; i < 256; i += NT) h256[i] = 0;
        __syncthreads();
        const int n = src.size();
        const int nr = (n + NT - 1) / NT * NT;  // every lane takes part in the wave merge
        for (int i = threadIdx.x; i < nr; i += NT) {
            uint64_t c = 0;
            const bool ok = i < n && src.get(i, c) && (c >> hi) == (pref >> hi);
            wave_hist_add(h256, ok ? (int)((c >> sh) & dmask) : -1);
        }
        __syncthreads();
        if (threadIdx.x < 64) {
            const int lane = threadIdx.x;
            const int top = 255 - 4 * lane;  // lane owns 4 digits, scanned from the top
            const uint32_t s = h256[top] + h256[top - 1] + h256[top - 2] + h256[top - 3];
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
                    const uint32_t c = h256[top - e];
                    if (acc + c >= need) {
                        scr[0] = (uint32_t)(top - e);
                        scr[1] = need - acc;
                        scr[2] = (c == need - acc);
                        break;
                    }
                    acc += c;
                }
            }
        }
        __syncthreads();
        const uint32_t d = scr[0];
        need = scr[1];
        const bool whole = scr[2] != 0;
        __syncthreads();
        pref |= (uint64_t)d << sh;
        hi = sh;
        if (whole) return pref;  // lower bits zero: every group element with this prefix
    }
    return pref;
}

// A radix source over a tie list read through an accessor (LDS array, or the workspace
// read with coherent loads).
template <class Get>
struct FnSrc {
    Get g;
    int n;
    __device__ int size() const { return n; }
    __device__ bool get(int i, uint64_t &c) const {
        c = g(i);
        return true;
    }
};

// The smallest composite to take from the tie list of threshold bin b1 (nl entries read by
// get(i)), so that the entries >= it are the need1 largest (1 <= need1 <= nl): a
// second-level histogram of the next 12 key bits (h: kB2 words, zeroed by the caller,
// transposed as the sliced resolve stores it), then the final (b1, b2) group ranked
// directly when small or by radix passes. Returns 0 when every tie is taken.
template <int NT, class Get>
__device__ uint64_t tie_threshold(Get get, uint32_t nl, uint32_t need1, uint32_t b1, uint32_t *h, uint32_t *h256,
                                  uint32_t *scr) {
    const int tid = threadIdx.x;
    constexpr int PER = kB2 / NT;  // second-level bins per thread
    auto hslot = [](int bin) {     // transposed slot of a second-level bin
        const int rk = kB2 - 1 - bin;
        return (rk % PER) * NT + rk / PER;
    };
    uint64_t thr = ~(uint64_t)0;
    if (tid == 0) scr[24] = 0;
    for (uint32_t i = tid; i < nl; i += NT) atomicAdd(&h[hslot((int)(((uint32_t)(get(i) >> 32) >> kL2Shift) & (kB2 - 1)))], 1u);
    __syncthreads();
    uint32_t v2[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) v2[e] = h[e * NT + tid];
    const BinPick p2 = pick_bin<NT, PER>(v2, need1, scr);
    if (p2.mode == 1) {
        thr = 0;  // every tie
    } else if (p2.mode == 2) {
        const int b2 = p2.bin;
        const uint32_t n2 = h[hslot(b2)];
        const uint32_t need2 = need1 - p2.above;  // wanted from the (b1, b2) group
        const uint64_t pre = (uint64_t)((b1 << kSelShift) | ((uint32_t)b2 << kL2Shift)) << 32;
        __syncthreads();  // h is reused below
        if (need2 == n2) {
            thr = pre;  // the whole group
        } else if (n2 <= (uint32_t)kTiny) {
            uint64_t *tiny = reinterpret_cast<uint64_t *>(h);
            for (uint32_t i = tid; i < nl; i += NT) {
                const uint64_t c = get(i);
                if ((c >> kGrpShift) == (pre >> kGrpShift)) {
                    const uint32_t slot = atomicAdd(&scr[24], 1u);
                    if (slot < (uint32_t)kTiny) tiny[slot] = c;
                }
            }
            __syncthreads();
            const uint32_t nt = min(scr[24], (uint32_t)kTiny);
            for (uint32_t i = tid; i < nt; i += NT) {
                const uint64_t c = tiny[i];
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
            thr = radix_kth<NT>(FnSrc<Get>{get, (int)nl}, need2, pre, kGrpShift, h256, scr);
        }
    }
    __syncthreads();
    return thr;
}

// Copy n 32-bit words global -> LDS with several loads per thread in flight (a plain
// element loop would wait for each load before its LDS store): U 16-byte loads when
// both pointers are 16-byte aligned, else 4 U word loads. (Native vector types: arrays
// of the HIP vector classes end up in scratch memory.)
template <int NT, int U>
__device__ void copy_words_to_lds(const uint32_t *src, uint32_t *dst, int n) {
    const int tid = (int)threadIdx.x;
    if ((((uintptr_t)src | (uintptr_t)dst) & 15) == 0) {
        const int n4 = n >> 2;
        const u32x4 *s4 = reinterpret_cast<const u32x4 *>(src);
        u32x4 *d4 = reinterpret_cast<u32x4 *>(dst);
        for (int base = 0; base < n4; base += NT * U) {
            u32x4 v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int i = min(base + u * NT + tid, n4 - 1);
                v[u] = s4[i];
            }
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (base + u * NT + tid < n4) d4[base + u * NT + tid] = v[u];
        }
        for (int i = 4 * n4 + tid; i < n; i += NT) dst[i] = src[i];
    } else {
        constexpr int V = 4 * U;
        for (int base = 0; base < n; base += NT * V) {
            uint32_t v[V];
#pragma unroll
            for (int u = 0; u < V; ++u) v[u] = src[min(base + u * NT + tid, n - 1)];
#pragma unroll
            for (int u = 0; u < V; ++u)
                if (base + u * NT + tid < n) dst[base + u * NT + tid] = v[u];
        }
    }
}

// ----------------------------------------------------------------------------- sliced resolve
// Output entries [k0, k1) of a flat row (no kept map), resolved by one of several
// workgroups that each need a slice of the row. Every such workgroup ranks the row's
// tie list itself (it holds only the threshold bin's candidates), sets the chosen ties
// in its own LDS copy of the row's bitmap (or, when that does not fit, in the workspace
// bitmap: every workgroup sets the same bits) and counts set bits up to its slice, each
// thread a contiguous range of words. The threshold pick comes from the counters the
// filter recorded. lpos[k - k0] receives output entry k (a position, or -1 past the
// row's selection).
//
// LDS layouts are transposed so that the per-thread scans read consecutive words in
// consecutive lanes (no bank conflicts): thread t's j-th bitmap word (word t 2^pw_log
// + j) sits at j NT + t, and its e-th second-level bin from the top at e NT + t.
constexpr int kSliceTiesFirst = 2048;  // tie entries requested with the first loads

struct SliceLds {     // caller-provided LDS scratch (16-byte aligned pieces)
    uint64_t *ties;   // [tl]
    uint32_t *bits;   // [NT << pw_log] when bits_lds (transposed)
    uint32_t *h;      // [kB2] (transposed)
    uint32_t *h256;   // [256]
    uint32_t *scr;    // [32]
    int tl;           // tie entries held in LDS (>= kSliceTiesFirst)
    int pw_log;       // log2 of the bitmap words per thread (NT << pw_log >= words)
    bool bits_lds;
};

// Position of set bit number r (from bit 0, r < popcount(x)) of x.
__device__ __forceinline__ int select_bit(uint32_t x, uint32_t r) {
    int pos = 0;
    uint32_t c = __popc(x & 0xFFFFu);
    if (r >= c) r -= c, x >>= 16, pos += 16;
    c = __popc(x & 0xFFu);
    if (r >= c) r -= c, x >>= 8, pos += 8;
    c = __popc(x & 0xFu);
    if (r >= c) r -= c, x >>= 4, pos += 4;
    c = __popc(x & 0x3u);
    if (r >= c) r -= c, x >>= 2, pos += 2;
    return pos + (r >= (x & 1u) ? 1 : 0);
}

__host__ __device__ constexpr int ilog2(int x) { return x <= 1 ? 0 : 1 + ilog2(x >> 1); }

// Bitmap words per thread (a power of two) for an NT-thread sliced resolve.
inline int slice_pw_log(int words, int nt) {
    int l = 0;
    while ((nt << l) < words) ++l;
    return l;
}

// LDS slot of bitmap word i in the transposed layout.
template <int NT>
__device__ __forceinline__ int bit_slot(int i, int pwl) {
    return ((i & ((1 << pwl) - 1)) << ilog2(NT)) | (i >> pwl);
}

// Copy a row bitmap of `words` words global -> LDS in the transposed layout (slots of
// words past the end are left alone: the scans never read them).
template <int NT>
__device__ void copy_bits_transposed(const uint32_t *src, uint32_t *dst, int words, int pwl) {
    const int tid = (int)threadIdx.x;
    if (((uintptr_t)src & 15) == 0) {
        const int n4 = words >> 2;
        const u32x4 *s4 = reinterpret_cast<const u32x4 *>(src);
        for (int base = 0; base < n4; base += 4 * NT) {
            u32x4 v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) v[u] = s4[min(base + u * NT + tid, n4 - 1)];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int q = base + u * NT + tid;
                if (q < n4)
#pragma unroll
                    for (int e = 0; e < 4; ++e) dst[bit_slot<NT>(4 * q + e, pwl)] = v[u][e];
            }
        }
        for (int i = 4 * n4 + tid; i < words; i += NT) dst[bit_slot<NT>(i, pwl)] = src[i];
    } else {
        for (int base = 0; base < words; base += 16 * NT) {
            uint32_t v[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) v[u] = src[min(base + u * NT + tid, words - 1)];
#pragma unroll
            for (int u = 0; u < 16; ++u)
                if (base + u * NT + tid < words) dst[bit_slot<NT>(base + u * NT + tid, pwl)] = v[u];
        }
    }
}

struct NoHook {
    __device__ void operator()() const {}
};

// after_loads() is called once the first round of loads has been issued and before it is
// waited for: loads the caller issues there are not waited for by that round (the vector
// memory counter retires in issue order, so loads issued earlier would be).
template <int NT, class Hook = NoHook>
__device__ void resolve_slice(const SelectArgs &a, const Ws &w, int row, int k0, int k1, const SliceLds &S,
                              int32_t *lpos, Hook after_loads = Hook{}) {
    const int tid = threadIdx.x;
    const Row r = make_row(a, row);
    const int nsink = a.causal ? r.f_sink_end : 0;
    const int nwin = a.causal ? max(0, r.p - r.f_win_lo + 1) : 0;
    const uint32_t m = (uint32_t)max(r.m, 0);
    const uint32_t *gctr = w.ctr + (int64_t)row * kCtr;
    const uint64_t *gties = w.ties + (int64_t)row * w.cap;
    uint32_t *gbits = w.bits + (int64_t)row * w.words;
    uint32_t *scr = S.scr;

    // ---- one round of loads: the counters (one thread), the bitmap, the tie list's start.
    // When each copy takes at most four 16-byte loads per thread, every load is requested
    // before any is waited for, and after_loads() runs in between; otherwise the copies
    // run one after another and after_loads() follows them.
    const int tfirst = min(w.cap, kSliceTiesFirst);
    const int pwl = S.pw_log;
    const int n4b = S.bits_lds ? w.words >> 2 : 0, n4t = tfirst >> 1;  // 16-byte pieces
    const bool one_round = ((((uintptr_t)gbits | (uintptr_t)gties | (uintptr_t)gctr | (uintptr_t)S.ties) & 15) == 0) &&
                           (w.words & 3) == 0 && n4b <= 4 * NT && n4t <= 4 * NT && (tfirst & 1) == 0;
    if (one_round) {
        const u32x4 *sb = reinterpret_cast<const u32x4 *>(gbits);
        const u32x4 *st = reinterpret_cast<const u32x4 *>(gties);
        u32x4 vb[4], vt[4], vc = {0u, 0u, 0u, 0u};
        if (n4b > 0) {
#pragma unroll
            for (int u = 0; u < 4; ++u) vb[u] = sb[min(u * NT + tid, n4b - 1)];
        }
        if (n4t > 0) {
#pragma unroll
            for (int u = 0; u < 4; ++u) vt[u] = st[min(u * NT + tid, n4t - 1)];
        }
        if (tid == 0) vc = *reinterpret_cast<const u32x4 *>(gctr);
        after_loads();
        for (int i = tid; i < kB2; i += NT) S.h[i] = 0;  // the second-level histogram
        if (n4b > 0) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int q = u * NT + tid;
                if (q < n4b)
#pragma unroll
                    for (int e = 0; e < 4; ++e) S.bits[bit_slot<NT>(4 * q + e, pwl)] = vb[u][e];
            }
        }
        if (n4t > 0) {
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (u * NT + tid < n4t) reinterpret_cast<u32x4 *>(S.ties)[u * NT + tid] = vt[u];
        }
        if (tid == 0) {
            scr[28] = vc[0];
            scr[29] = vc[1];
            scr[30] = vc[2];
            scr[31] = vc[3];
            scr[24] = 0;
        }
    } else {
        if (tid == 0) {
            scr[28] = gctr[0];
            scr[29] = gctr[1];
            scr[30] = gctr[2];
            scr[31] = gctr[3];
        }
        if (S.bits_lds) copy_bits_transposed<NT>(gbits, S.bits, w.words, pwl);
        copy_words_to_lds<NT, 4>(reinterpret_cast<const uint32_t *>(gties), reinterpret_cast<uint32_t *>(S.ties), 2 * tfirst);
        after_loads();
        for (int i = tid; i < kB2; i += NT) S.h[i] = 0;  // the second-level histogram
        if (tid == 0) scr[24] = 0;
    }
    __syncthreads();
    const uint32_t ntie = scr[28], mode = scr[29], b1 = scr[30], above = scr[31];
    const uint32_t nfill = mode == 0 ? 0u : (mode == 1 ? min(above, m) : m);
    const int f0 = max(k0 - nsink, 0), f1 = min(k1 - nsink, (int)nfill);  // fill ranks of the slice
    const bool overflow = ntie > (uint32_t)w.cap;
    const uint32_t nl = min(ntie, (uint32_t)w.cap);
    const bool ties_lds = nl <= (uint32_t)S.tl;

    // set the chosen columns (one loop per bitmap location: the LDS copy takes LDS atomics)
    auto mark_all = [&](auto chosen, int n) __attribute__((always_inline)) {
        if (S.bits_lds) {
            for (int i = tid; i < n; i += NT) {
                const int col = chosen(i);
                if (col >= 0) atomicOr(&S.bits[bit_slot<NT>(col >> 5, pwl)], 1u << (col & 31));
            }
        } else {
            for (int i = tid; i < n; i += NT) {
                const int col = chosen(i);
                if (col >= 0) atomicOr(&gbits[col >> 5], 1u << (col & 31));
            }
        }
    };
    if (f0 < f1 && mode == 2) {
        const uint32_t need1 = m > above ? m - above : 0u;
        if (!overflow && ties_lds && nl > (uint32_t)tfirst) {  // uniform
            copy_words_to_lds<NT, 4>(reinterpret_cast<const uint32_t *>(gties + tfirst),
                                     reinterpret_cast<uint32_t *>(S.ties + tfirst), 2 * ((int)nl - tfirst));
            __syncthreads();
        }
        // rank the tie list where it lives (inlined at each call, so that the LDS copy is
        // read with LDS instructions)
        auto rank_and_mark = [&](const uint64_t *tl) __attribute__((always_inline)) {
            const uint64_t thr = tie_threshold<NT>([&](uint32_t i) { return tl[i]; }, nl, need1, b1, S.h, S.h256, scr);
            mark_all([&](int i) { return tl[i] >= thr ? comp_pos(tl[i]) : -1; }, (int)nl);
        };
        if (!overflow) {
            if (ties_lds) rank_and_mark(S.ties);
            else rank_and_mark(gties);
        } else {
            // the tie list overflowed: exact select inside bin b1 over the whole row
            const RowSrc rs{&a, &r};
            const uint64_t pre = (uint64_t)b1 << kB1Shift;
            const uint64_t thr = radix_kth<NT>(rs, need1, pre, kB1Shift, S.h256, scr);
            mark_all([&](int col) {
                uint64_t c;
                return candidate_x(a, r, col, r.sc[col], c) && (c >> kB1Shift) == (uint64_t)b1 && c >= thr ? col : -1;
            }, a.n_cols);
        }
    }
    __syncthreads();

    // ---- the slice: sink [0, nsink), the fill (ascending columns), window [f_win_lo, p], then -1
    const int wbase = nsink + (int)nfill;
    for (int k = k0 + tid; k < k1; k += NT) {
        if (k < nsink) lpos[k - k0] = k;
        else if (k >= wbase) lpos[k - k0] = k < wbase + nwin ? r.f_win_lo + (k - wbase) : -1;
    }
    if (f0 < f1) {  // uniform
        // The fill ranks [f0, f1) of this slice, found in parallel: every thread counts the
        // set bits of its contiguous word range and a block scan gives each range's first
        // rank; then one thread per wanted rank finds the range that holds it (binary
        // search over the ranges' first ranks), the word inside the range and the bit
        // inside the word. Loads go 16 at a time with clamped indices (no divergence).
        const int per = S.bits_lds ? 1 << pwl : (w.words + NT - 1) / NT;
        auto batch = [&](int i0, int wend, uint32_t(&v)[16]) __attribute__((always_inline)) {
            if (S.bits_lds) {
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const uint32_t x = S.bits[bit_slot<NT>(max(min(i0 + j, wend - 1), 0), pwl)];
                    v[j] = i0 + j < wend ? x : 0u;
                }
            } else {
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const uint32_t x = __hip_atomic_load(&gbits[max(min(i0 + j, wend - 1), 0)], __ATOMIC_RELAXED,
                                                         __HIP_MEMORY_SCOPE_AGENT);
                    v[j] = i0 + j < wend ? x : 0u;
                }
            }
        };
        const int w0 = min(w.words, tid * per), w1 = min(w.words, w0 + per);
        uint32_t c = 0;
        for (int i0 = w0; i0 < w1; i0 += 16) {
            uint32_t v[16];
            batch(i0, w1, v);
#pragma unroll
            for (int j = 0; j < 16; ++j) c += __popc(v[j]);
        }
        uint32_t tot;
        const uint32_t off = block_exscan<NT>(c, scr, &tot);
        uint32_t *offs = S.h;  // free since the ranking
        offs[tid] = off;
        __syncthreads();
        for (int q = tid; q < f1 - f0; q += NT) {
            const uint32_t k = (uint32_t)(f0 + q);
            int t = 0;  // the last range whose first rank is <= k holds rank k
#pragma unroll
            for (int step = NT / 2; step > 0; step >>= 1)
                if (offs[t + step] <= k) t += step;
            uint32_t rk = k - offs[t];
            const int tw0 = min(w.words, t * per), tw1 = min(w.words, tw0 + per);
            int col = -1;
            for (int i0 = tw0; i0 < tw1 && col < 0; i0 += 16) {
                uint32_t v[16];
                batch(i0, tw1, v);
                uint32_t wsel = 0;
                int jsel = -1;
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const uint32_t pc = __popc(v[j]);
                    const bool hit = jsel < 0 && rk < pc;
                    wsel = hit ? v[j] : wsel;
                    jsel = hit ? j : jsel;
                    rk = (jsel < 0) ? rk - pc : rk;
                }
                if (jsel >= 0) col = (i0 + jsel) * 32 + select_bit(wsel, rk);
            }
            lpos[nsink + (int)k - k0] = col;
        }
    }
    __syncthreads();  // lpos complete
}

// Workspace hygiene after a sliced resolve (global stores only: call it after the
// workgroup's last barrier, since a barrier waits for outstanding stores). Each of the
// row's workgroups clears its share of the row's histogram (the sliced resolve does not
// read it); the last one to arrive clears the row's counters.
template <int NT>
__device__ void release_slice(const Ws &w, int row, int nslices, int slice) {
    uint32_t *g1 = w.hist + (int64_t)row * kSelBins;
    uint32_t *gctr = w.ctr + (int64_t)row * kCtr;
    const int per = (kSelBins + nslices - 1) / nslices;
    const int h0 = min(kSelBins, slice * per), h1 = min(kSelBins, h0 + per);
    for (int i = h0 + (int)threadIdx.x; i < h1; i += NT) g1[i] = 0;
    if (threadIdx.x == 0) {
        const uint32_t prev = atomicAdd(&gctr[15], 1u);
        if (prev == (uint32_t)nslices - 1)
            for (int i = 0; i < kCtr; ++i) gctr[i] = 0;
    }
}
}  // namespace sel
}  // namespace lsa
