// SI selection on gfx950: per query token, the forced sink and local window plus the
// top-m fill by (score descending, position ascending)
// (LongCat-Flash-Lite-Sparse summary, "Good to know" and "Technical features", first
// bullet: the selection budget is split into a fixed sink and a local window).
//
// Exact multi-workgroup radix selection on a 64-bit composite key
//     comp = order_key(score) << 32 | ~position
// (larger comp = better: higher score, then lower position; composites are unique).
//   S1 hist:    every workgroup histograms the top 12 key bits of its column range in
//               LDS and adds it to the row histogram (integer atomics: deterministic).
//   S2 filter:  every workgroup finds the threshold bin b1 from the row histogram;
//               candidates above b1 are certainly selected ("sure" list), candidates
//               in b1 go to a composite list and into a second 12-bit histogram.
//   S3 resolve: one workgroup per row finds the second-level bin b2, then the exact
//               threshold composite inside (b1, b2) by 8-bit radix passes, gathers
//               forced + sure + chosen positions, sorts them (bitonic, LDS) and writes
//               idx; it then zeroes its row's histograms and counters.
// The result does not depend on the order atomics land in: membership is defined by
// the total order on composites, and the output is sorted.
#include "common.cuh"
#include "kernels.h"

namespace lsa {
namespace {

constexpr int kT = 256;
constexpr int kBins = 4096;  // 12-bit digits
constexpr int kCh = 1024;    // S2 staging chunk (columns per round)

struct Ws {
    uint32_t *hist1;  // [rows][4096]
    uint32_t *hist2;  // [rows][4096]
    uint32_t *ctr;    // [rows][8]: 0 n_sure, 1 n_list
    int32_t *sure;    // [rows][K]
    uint64_t *list;   // [rows][cap]
    int cap;
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

inline int list_cap(int n_cols) {
    int c = n_cols / 8;
    if (c < 4096) c = 4096;
    if (c > n_cols) c = n_cols;
    return (c + 63) / 64 * 64;
}

Ws carve(void *base, int rows, int K, int n_cols) {
    Ws w;
    char *p = reinterpret_cast<char *>(base);
    w.hist1 = reinterpret_cast<uint32_t *>(p);
    p += align256((size_t)rows * kBins * 4);
    w.hist2 = reinterpret_cast<uint32_t *>(p);
    p += align256((size_t)rows * kBins * 4);
    w.ctr = reinterpret_cast<uint32_t *>(p);
    p += align256((size_t)rows * 8 * 4);
    w.sure = reinterpret_cast<int32_t *>(p);
    p += align256((size_t)rows * K * 4);
    w.list = reinterpret_cast<uint64_t *>(p);
    w.cap = list_cap(n_cols);
    return w;
}

size_t ws_bytes(int rows, int K, int n_cols) {
    return 2 * align256((size_t)rows * kBins * 4) + align256((size_t)rows * 8 * 4) + align256((size_t)rows * K * 4) +
           align256((size_t)rows * list_cap(n_cols) * 8);
}

// Per-row context: query position, forced set, fill size.
struct Row {
    int b, t, p;
    int f_sink_end;  // sink = [0, f_sink_end)
    int f_win_lo;    // window = [f_win_lo, p] (empty when f_win_lo > p)
    int nforced;
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
        r.nforced = r.f_sink_end + max(0, r.p - r.f_win_lo + 1);
        r.m = a.K - r.nforced;
    } else {
        r.f_sink_end = 0;
        r.f_win_lo = 0;
        r.nforced = 0;
        r.m = a.K;
    }
    r.sc = a.scores + (int64_t)row * a.n_cols;
    r.kept = a.kept ? a.kept + (int64_t)row * a.n_keep : nullptr;
    r.nblk = a.kept ? a.N / a.block_size : 0;
    return r;
}

// Candidate test of column `col`; on success sets the composite key.
__device__ __forceinline__ bool candidate(const SelectArgs &a, const Row &r, int col, uint64_t &comp) {
    const float x = r.sc[col];
    if (!(x > kNegInf)) return false;  // -inf and NaN are never selected
    int pos = col;
    if (r.kept) {
        const int blk = col / a.block_size;
        if (blk >= a.n_keep) return false;
        const int kb = r.kept[blk];
        if (kb < 0 || kb >= r.nblk) return false;
        pos = kb * a.block_size + (col - blk * a.block_size);
    }
    if (a.causal) {
        if (pos > r.p || pos < r.f_sink_end || pos >= r.f_win_lo) return false;
    }
    comp = ((uint64_t)order_key(x) << 32) | (uint32_t)(~(uint32_t)pos);
    return true;
}

__device__ __forceinline__ int comp_pos(uint64_t c) { return (int)(~(uint32_t)c); }

// Block-wide exclusive scan of one value per thread (256 threads, wave64). Returns the
// exclusive prefix and writes the total to *total.
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

// Threshold bin of a 4096-bin LDS histogram, counted from the top: the bin b with
// above(b) < need <= above(b) + h[b]. Returns mode: 0 none needed (need == 0),
// 1 everything (total <= need), 2 threshold bin found.
struct BinPick {
    int mode;
    int bin;
    uint32_t above;
    uint32_t total;
};

__device__ BinPick pick_bin(const uint32_t *h, uint32_t need, uint32_t *scratch) {
    // thread i owns bins [4095 - 16 i - 15, 4095 - 16 i], walked from the top
    const int tid = threadIdx.x;
    const int hi_bin = kBins - 1 - 16 * tid;
    uint32_t s = 0;
#pragma unroll
    for (int e = 0; e < 16; ++e) s += h[hi_bin - e];
    uint32_t total;
    uint32_t ex = block_exscan(s, scratch, &total);
    BinPick r;
    r.total = total;
    if (need == 0) {
        r.mode = 0;
        r.bin = kBins;
        r.above = 0;
        return r;
    }
    if (total <= need) {
        r.mode = 1;
        r.bin = -1;
        r.above = total;
        return r;
    }
    if (ex < need && need <= ex + s) {
        uint32_t acc = ex;
        for (int e = 0; e < 16; ++e) {
            uint32_t c = h[hi_bin - e];
            if (acc + c >= need) {
                scratch[4] = (uint32_t)(hi_bin - e);
                scratch[5] = acc;
                break;
            }
            acc += c;
        }
    }
    __syncthreads();
    r.mode = 2;
    r.bin = (int)scratch[4];
    r.above = scratch[5];
    __syncthreads();
    return r;
}

// ----------------------------------------------------------------------------- S1
__global__ __launch_bounds__(kT) void select_hist_kernel(SelectArgs a, Ws ws, int part_cols) {
    __shared__ uint32_t h[kBins];
    const int row = blockIdx.y;
    const int c0 = blockIdx.x * part_cols;
    const int c1 = min(a.n_cols, c0 + part_cols);
    for (int i = threadIdx.x; i < kBins; i += kT) h[i] = 0;
    __syncthreads();
    const Row r = make_row(a, row);
    if (r.m > 0) {
        for (int col = c0 + threadIdx.x; col < c1; col += kT) {
            uint64_t comp;
            if (candidate(a, r, col, comp)) atomicAdd(&h[comp >> 52], 1u);
        }
    }
    __syncthreads();
    uint32_t *g = ws.hist1 + (int64_t)row * kBins;
    for (int i = threadIdx.x; i < kBins; i += kT)
        if (h[i]) atomicAdd(&g[i], h[i]);
}

// ----------------------------------------------------------------------------- S2
__global__ __launch_bounds__(kT) void select_filter_kernel(SelectArgs a, Ws ws, int part_cols) {
    __shared__ uint32_t h[kBins];
    __shared__ uint32_t h2[kBins];
    __shared__ int32_t sbuf[kCh];
    __shared__ uint64_t lbuf[kCh];
    __shared__ uint32_t cnt[8];
    __shared__ uint32_t scratch[8];
    const int row = blockIdx.y;
    const int c0 = blockIdx.x * part_cols;
    const int c1 = min(a.n_cols, c0 + part_cols);
    const Row r = make_row(a, row);
    const uint32_t *g1 = ws.hist1 + (int64_t)row * kBins;
    for (int i = threadIdx.x; i < kBins; i += kT) {
        h[i] = g1[i];
        h2[i] = 0;
    }
    if (threadIdx.x < 8) cnt[threadIdx.x] = 0;
    __syncthreads();
    const BinPick bp = pick_bin(h, (uint32_t)max(r.m, 0), scratch);
    if (bp.mode == 0) return;  // uniform over the workgroup
    const int b1 = bp.bin;
    for (int base = c0; base < c1; base += kCh) {
        const int end = min(c1, base + kCh);
        for (int col = base + threadIdx.x; col < end; col += kT) {
            uint64_t comp;
            if (!candidate(a, r, col, comp)) continue;
            const int d1 = (int)(comp >> 52);
            if (bp.mode == 1 || d1 > b1) {
                sbuf[atomicAdd(&cnt[0], 1u)] = comp_pos(comp);
            } else if (d1 == b1) {
                atomicAdd(&h2[(comp >> 40) & (kBins - 1)], 1u);
                lbuf[atomicAdd(&cnt[1], 1u)] = comp;
            }
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            uint32_t *ctr = ws.ctr + (int64_t)row * 8;
            cnt[2] = cnt[0] ? atomicAdd(&ctr[0], cnt[0]) : 0;
            cnt[3] = cnt[1] ? atomicAdd(&ctr[1], cnt[1]) : 0;
        }
        __syncthreads();
        const uint32_t ns = cnt[0], nl = cnt[1], bs = cnt[2], bl = cnt[3];
        int32_t *sure = ws.sure + (int64_t)row * a.K;
        uint64_t *list = ws.list + (int64_t)row * ws.cap;
        for (uint32_t i = threadIdx.x; i < ns; i += kT)
            if (bs + i < (uint32_t)a.K) sure[bs + i] = sbuf[i];
        for (uint32_t i = threadIdx.x; i < nl; i += kT)
            if (bl + i < (uint32_t)ws.cap) list[bl + i] = lbuf[i];
        __syncthreads();
        if (threadIdx.x < 2) cnt[threadIdx.x] = 0;
        __syncthreads();
    }
    if (bp.mode == 2) {
        uint32_t *g2 = ws.hist2 + (int64_t)row * kBins;
        for (int i = threadIdx.x; i < kBins; i += kT)
            if (h2[i]) atomicAdd(&g2[i], h2[i]);
    }
}

// ----------------------------------------------------------------------------- S3

// Elements for the exact stage: the composite list, or (when it overflowed) the row.
struct ListSrc {
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

// need-th largest composite among elements whose bits above `lo_bit` equal those of
// `prefix` (need >= 1 and at most the number of such elements).
template <class Src>
__device__ uint64_t radix_kth(const Src &src, uint64_t prefix, int lo_bit, uint32_t need, uint32_t *h256,
                              uint32_t *scratch) {
    uint64_t pref = prefix;
    for (int sh = lo_bit - 8; sh >= 0; sh -= 8) {
        for (int i = threadIdx.x; i < 256; i += kT) h256[i] = 0;
        __syncthreads();
        const int n = src.size();
        for (int i = threadIdx.x; i < n; i += kT) {
            uint64_t c;
            if (src.get(i, c) && (c >> (sh + 8)) == (pref >> (sh + 8))) atomicAdd(&h256[(c >> sh) & 255], 1u);
        }
        __syncthreads();
        if (threadIdx.x < 64) {
            // lane l owns digits [255 - 4l - 3, 255 - 4l], scanned from the top
            const int lane = threadIdx.x;
            const int hi = 255 - 4 * lane;
            uint32_t s = h256[hi] + h256[hi - 1] + h256[hi - 2] + h256[hi - 3];
            uint32_t x = s;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                uint32_t y = __shfl_up(x, o, 64);
                if (lane >= o) x += y;
            }
            const uint32_t ex = x - s;
            if (ex < need && need <= x) {
                uint32_t acc = ex;
                for (int e = 0; e < 4; ++e) {
                    uint32_t c = h256[hi - e];
                    if (acc + c >= need) {
                        scratch[0] = (uint32_t)(hi - e);
                        scratch[1] = need - acc;            // still needed inside this digit
                        scratch[2] = (c == need - acc);     // the whole digit is taken
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
        pref = (pref & ~((uint64_t)255 << sh)) | ((uint64_t)d << sh);
        if (whole) return pref & ~(((uint64_t)1 << sh) - 1);  // every element with this prefix
    }
    return pref;
}

template <int KPAD>
__global__ __launch_bounds__(kT) void select_resolve_kernel(SelectArgs a, Ws ws) {
    __shared__ uint32_t h[kBins];
    __shared__ int32_t out[KPAD];
    __shared__ uint32_t ocount;
    __shared__ uint32_t scratch[8];
    const int row = blockIdx.x;
    const Row r = make_row(a, row);
    const int tid = threadIdx.x;
    uint32_t *g1 = ws.hist1 + (int64_t)row * kBins;
    uint32_t *g2 = ws.hist2 + (int64_t)row * kBins;
    uint32_t *ctr = ws.ctr + (int64_t)row * 8;
    for (int i = tid; i < KPAD; i += kT) out[i] = 0x7FFFFFFF;
    for (int i = tid; i < kBins; i += kT) h[i] = g1[i];
    if (tid == 0) ocount = 0;
    __syncthreads();

    auto emit = [&](int pos) {
        uint32_t slot = atomicAdd(&ocount, 1u);
        if (slot < (uint32_t)KPAD) out[slot] = pos;
    };

    // forced set: sink [0, f_sink_end) and window [f_win_lo, p] (disjoint by construction)
    if (a.causal) {
        for (int s = tid; s < r.f_sink_end; s += kT) emit(s);
        for (int s = r.f_win_lo + tid; s <= r.p; s += kT) emit(s);
    }
    const BinPick bp = pick_bin(h, (uint32_t)max(r.m, 0), scratch);
    const uint32_t n_sure = min(ctr[0], (uint32_t)a.K);
    const uint32_t n_list = ctr[1];
    const int32_t *sure = ws.sure + (int64_t)row * a.K;
    const uint64_t *list = ws.list + (int64_t)row * ws.cap;
    if (bp.mode != 0) {
        for (uint32_t i = tid; i < n_sure; i += kT) emit(sure[i]);
    }
    if (bp.mode == 2) {
        const int b1 = bp.bin;
        const uint32_t r1 = (uint32_t)r.m - bp.above;  // still needed from bin b1 (>= 1)
        const uint32_t n1 = h[b1];
        const bool overflow = n1 > (uint32_t)ws.cap || n_list != n1;
        ListSrc ls{list, (int)min(n_list, (uint32_t)ws.cap)};
        RowSrc rs{&a, &r};
        if (r1 == n1) {
            // the whole bin is selected
            if (!overflow) {
                for (int i = tid; i < ls.n; i += kT) emit(comp_pos(list[i]));
            } else {
                for (int i = tid; i < a.n_cols; i += kT) {
                    uint64_t c;
                    if (rs.get(i, c) && (int)(c >> 52) == b1) emit(comp_pos(c));
                }
            }
        } else {
            __syncthreads();
            for (int i = tid; i < kBins; i += kT) h[i] = g2[i];
            __syncthreads();
            const BinPick bq = pick_bin(h, r1, scratch);
            const int b2 = bq.bin;
            const uint32_t r2 = r1 - bq.above;
            const uint32_t n2 = h[b2];
            const uint64_t p24 = ((uint64_t)b1 << 52) | ((uint64_t)b2 << 40);
            __syncthreads();  // every thread has read h[b2] before radix_kth reuses h
            uint64_t thr = p24;
            if (r2 < n2) {
                thr = overflow ? radix_kth(rs, p24, 40, r2, h, scratch) : radix_kth(ls, p24, 40, r2, h, scratch);
            }
            // take every element of bin b1 with digit2 > b2, and those of (b1, b2) with comp >= thr
            auto take = [&](uint64_t c) {
                if ((int)(c >> 52) != b1) return false;
                const uint64_t d2 = (c >> 40) & (kBins - 1);
                if (d2 > (uint64_t)b2) return true;
                return d2 == (uint64_t)b2 && c >= thr;
            };
            if (!overflow) {
                for (int i = tid; i < ls.n; i += kT)
                    if (take(list[i])) emit(comp_pos(list[i]));
            } else {
                for (int i = tid; i < a.n_cols; i += kT) {
                    uint64_t c;
                    if (rs.get(i, c) && take(c)) emit(comp_pos(c));
                }
            }
        }
    }
    __syncthreads();
    const uint32_t count = min(ocount, (uint32_t)KPAD);
    // bitonic sort of out[0, KPAD) ascending (padding 0x7FFFFFFF sorts last)
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
    int32_t *dst = a.idx + (int64_t)row * a.K;
    for (int i = tid; i < a.K; i += kT) dst[i] = (uint32_t)i < count ? out[i] : -1;
    // return this row's workspace to zero for the next call
    for (int i = tid; i < kBins; i += kT) {
        g1[i] = 0;
        g2[i] = 0;
    }
    if (tid < 8) ctr[tid] = 0;
}

__global__ void clear_kernel(uint4 *p, size_t n16, uint8_t *tail, size_t ntail) {
    size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t j = i; j < n16; j += stride) p[j] = make_uint4(0, 0, 0, 0);
    if (i < ntail) tail[i] = 0;
}

template <int KPAD>
hipError_t launch_resolve(const SelectArgs &a, const Ws &w, int rows, hipStream_t s) {
    hipLaunchKernelGGL((select_resolve_kernel<KPAD>), dim3(rows), dim3(kT), 0, s, a, w);
    return hipGetLastError();
}

}  // namespace

size_t select_workspace_bytes(const SelectArgs &a) { return ws_bytes(a.B * a.T, a.K, a.n_cols); }

hipError_t launch_select(const SelectArgs &a, void *wsp, hipStream_t s) {
    const int rows = a.B * a.T;
    Ws w = carve(wsp, rows, a.K, a.n_cols);
    int parts = (1024 + rows - 1) / rows;
    const int max_parts = (a.n_cols + 2047) / 2048;
    if (parts > max_parts) parts = max_parts;
    if (parts < 1) parts = 1;
    int part_cols = (a.n_cols + parts - 1) / parts;
    parts = (a.n_cols + part_cols - 1) / part_cols;
    dim3 grid(parts, rows);
    hipLaunchKernelGGL(select_hist_kernel, grid, dim3(kT), 0, s, a, w, part_cols);
    hipError_t e = hipGetLastError();
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
