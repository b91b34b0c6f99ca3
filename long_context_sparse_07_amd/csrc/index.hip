// Indexer kernels of the LSA hot path on gfx950.
//
// index_tokens_kernel: I[t,s] = scale[s] * sum_h w[t,h] * ReLU(q[t,h] . k[s]) (reading R1
// of the DSA-style indexer that LSA extends, molayo1419.me LongCat-2.0 article, section
// "The sparse attention problem at 1M tokens"). The key cache is streamed once, HBM
// coalesced, by direct-to-LDS DMA (global_load_lds_dwordx4) into a 4-stage ring of
// 128-key tiles (three tiles in flight per workgroup); the (query-head rows) x (keys)
// contraction runs on
// v_mfma_f32_32x32x16_bf16 with fp8 keys widened exactly to bf16 in registers; the
// ReLU, head weights, head sum, per-token scale and causal mask are fused into the
// MFMA epilogue. With fp8 queries (an option for fp8 keys: each query row quantised
// like a key row, its scale folded into the head weight, since ReLU(s x) = s ReLU(x)
// for s > 0) the contraction runs on v_mfma_f32_32x32x64_f8f6f4 straight from the fp8
// key bytes in LDS.
//
// index_blocks_kernel: coarse HI block scores max_h w * ReLU(q . kbar) in fp32 (VALU),
// so that the block means are not rounded to bf16 (LongCat-Flash-Lite-Sparse summary,
// "Technical features", third bullet: coarse candidate blocks first).
//
// block_means_kernel: kbar[j] = mean of the dequantised keys of block j, fp32.
#include <hip/hip_ext.h>

#include "common.cuh"
#include "kernels.h"

namespace lsa {
namespace {

constexpr int kThreads = 256;
constexpr int kKT = 128;  // keys per LDS tile (4 waves x 32)

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

// s_waitcnt vmcnt(n) (gfx9 encoding: expcnt and lgkmcnt left at their maxima)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// LDS add without return, issued as inline asm. Written as a plain atomic, the compiler
// orders it after every outstanding direct-to-LDS DMA (s_waitcnt vmcnt(0)), which would
// drain the key ring on every tile. The histogram and the ring never overlap.
__device__ __forceinline__ void lds_add_u32(uint32_t *p, uint32_t v) {
    const uint32_t la = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) uint32_t *)p);
    asm volatile("ds_add_u32 %0, %1" ::"v"(la), "v"(v) : "memory");
}
__device__ __forceinline__ void lds_wait_all() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// set lanes of mask below this lane
__device__ __forceinline__ uint32_t lane_rank64(uint64_t mask) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Workgroup barrier for the key ring: this wave's LDS operations complete first, its
// outstanding vector memory operations do not (a workgroup fence would also wait for the
// direct-to-LDS DMA still in flight, i.e. drain the ring). The memory clobber keeps the
// compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Query-row layouts of one MFMA row group.
enum { ONEQ = 0, Q4 = 4, Q8 = 8, Q16 = 16 };

template <int D, bool FP8, int NST_>
struct Tile {
    static constexpr int RB = FP8 ? D : 2 * D;        // bytes per key row
    static constexpr int CPR = RB / 16;               // 16-byte chunks per row
    static constexpr int BYTES = kKT * RB;
    static constexpr int KINSTR = BYTES / 1024;       // 64-lane x 16-byte DMA instructions per tile
    static constexpr int PER_WAVE = KINSTR / 4 + (FP8 ? 1 : 0);  // + one scale DMA per wave
    static constexpr int SBYTES = FP8 ? kKT * 4 : 0;  // per-token scales of a tile
    static constexpr int STAGE = BYTES + SBYTES;
    static constexpr int NST = NST_;                  // ring: one tile computed, NST-1 in flight
    static_assert(KINSTR % 4 == 0, "tile must split evenly over 4 waves");
    static_assert(PER_WAVE * (NST - 2) < 64, "vmcnt budget");
    static constexpr int RPB = CPR >= 16 ? 1 : 16 / CPR;  // rows per 256-byte bank row
    // XOR swizzle of the 16-byte chunks: 16 lanes reading the same logical chunk of
    // 16 consecutive rows land on 16 distinct groups of 4 banks.
    __device__ static __forceinline__ int swz(int row, int c) { return c ^ ((row / RPB) & (CPR - 1)); }
};

// Wait until at most n tiles' DMA instructions (PW per tile, n <= MAXN) are pending.
template <int PW, int MAXN>
__device__ __forceinline__ void wait_tiles(int n) {
    if constexpr (MAXN > 0) {
        if (n >= MAXN) {
            wait_vmcnt<MAXN * PW>();
            return;
        }
        wait_tiles<PW, MAXN - 1>(n);
    } else {
        wait_vmcnt<0>();
    }
}

// Chunk c (16 bytes) of bf16 query row n in the LDS copy of the query: XOR-permuted so that
// 16 lanes reading one logical chunk of 16 consecutive rows hit 16 distinct bank groups.
template <int D>
__device__ __forceinline__ int qswz(int n, int c) {
    constexpr int CPR = D / 8, RPB = CPR >= 16 ? 1 : 16 / CPR;
    return c ^ ((n / RPB) & (CPR - 1));
}

// Row i of the (query, head) row space of group `grp` -> (t, h); ok = a real row.
template <int MODE>
__device__ __forceinline__ void row_to_th(int grp, int i, int H, int T, int &t, int &h, bool &ok) {
    if constexpr (MODE == ONEQ) {
        t = grp;
        h = i;
        ok = (i < H) && (t < T);
    } else {
        constexpr int QPG = 32 / MODE;
        t = grp * QPG + i / MODE;
        h = i % MODE;
        ok = t < T;
    }
}

// HIST (one query per workgroup): the epilogue also counts the selection candidates of
// its columns per first-level bin of the selection histogram (finite scores at visible
// positions outside the sink and the window) and adds the counts to sel_hist.
// EMIT (four query groups a workgroup, one query and its whole row per wave): each wave
// keeps an LDS histogram of its row's candidates in 1024 bins (the positive scores by their
// top 11 order-key bits, as the selection bins them; every negative score in the lowest
// bin) and, from it, the running threshold: the bin where the candidates counted so far
// from the top reach the fill size. The threshold only rises as candidates arrive, so a
// candidate in a bin below it can no longer be among the row's K - |forced| largest; the
// others are appended to the row's candidate list. At the end every candidate in a bin
// at or above the final threshold, and so every one the selection can take, is listed.
template <int D, bool FP8, bool QF8, int MODE, int HB, bool HI, bool PRE, bool HIST, int NST, bool EMIT = false>
__global__ __launch_bounds__(PRE ? kThreads : 2 * kThreads) void index_tokens_kernel(IndexTokensArgs a, int groups,
                                                                                      int chunk) {
    using G = Tile<D, FP8, NST>;
    static_assert(!QF8 || FP8, "fp8 queries need fp8 keys");
    // SPLIT (one query group per workgroup): waves 0-3 compute, waves 4-7 only stream the
    // key tiles into the LDS ring, so a DMA issue that stalls on a full memory queue
    // never holds up the MFMA and VALU work. Otherwise (four query groups share each
    // tile, 4 waves) every wave does both.
    constexpr bool SPLIT = !PRE;
    constexpr int NT = SPLIT ? 2 * kThreads : kThreads;
    constexpr int KSTEPS = D / 16;
    constexpr int QPG = MODE == ONEQ ? 1 : 32 / MODE;
    extern __shared__ __attribute__((aligned(16))) unsigned char ring[];  // NST x (keys, scales)
    __shared__ int tpos[HI ? G::NST : 1][kKT];                            // HI: position of each row
    __shared__ uint32_t shist[HIST ? kSelBins : 1];                      // HIST: candidate counts
    static_assert(!HIST || (MODE == ONEQ && !PRE), "the histogram needs one query per workgroup");
    static_assert(!EMIT || (MODE == ONEQ && PRE && !HI), "emission: one whole flat row per wave");
    constexpr int kEB = 1024;  // EMIT: running-threshold bins
    __shared__ uint32_t whist[EMIT ? 4 : 1][EMIT ? kEB : 1];
    // SPLIT: the query's rows (64 rows: bf16, or fp8 codes with their row scales) and head
    // weights pass through LDS, loaded (and quantised) once per workgroup, each compute wave
    // a quarter of the rows, instead of by every compute wave for its whole A operand
    constexpr bool QSHARE = SPLIT;
    __shared__ __attribute__((aligned(16))) uint32_t sqb[QSHARE ? 64 * D / (QF8 ? 4 : 2) : 1];
    __shared__ float sqs[QSHARE && QF8 ? 64 : 1];
    __shared__ float sw[QSHARE ? 64 : 1];

    const int tid = threadIdx.x;
    const int lane = tid & 63, half = lane >> 5, l32 = lane & 31;
    const int wave = (tid >> 6) & 3;               // compute wave, or the producer of its rows
    const bool producer = SPLIT && (tid >> 6) >= 4;
    const int b = blockIdx.z;
    const int c0 = blockIdx.x * chunk;
    if (c0 >= a.n_out) return;
    const int c1 = min(a.n_out, c0 + chunk);
    const int T = a.T, H = a.H, N = a.N;
    int ctx = a.ctx_len ? a.ctx_len[b] : N;
    ctx = min(max(ctx, 0), N);

    constexpr bool OWN = !PRE;
    const int grp = PRE ? blockIdx.y * 4 + wave : blockIdx.y;
    const bool active = grp < groups;
    int f_se = 0, f_wl = 0;  // HIST / EMIT: forced set of the workgroup's (wave's) query
    if constexpr (HIST) {
        for (int i = tid; i < kSelBins; i += NT) shist[i] = 0;
        forced_bounds(ctx - T + grp, a.sink, a.window, f_se, f_wl);
    }
    if constexpr (HIST) __syncthreads();
    // EMIT: this wave's fill size, running threshold bin and list length (wave-uniform)
    uint32_t e_m = 0, e_thr = 0, e_cnt = 0;
    uint64_t *e_row = nullptr;
    if constexpr (EMIT) {
        forced_bounds(ctx - T + grp, a.sink, a.window, f_se, f_wl);
        const int pq = ctx - T + grp;
        e_m = (uint32_t)max(0, a.K - (f_se + max(0, pq - f_wl + 1)));
        if (e_m == 0) e_thr = kEB;  // an empty fill lists nothing
        for (int i = lane; i < kEB; i += 64) whist[wave][i] = 0;  // each wave only touches its own
        e_row = a.cand + (int64_t)(b * T + min(grp, T - 1)) * a.N;
    }

    // ---- query fragments (A operand, rows = query heads) and head weights (compute waves)
    // lane (l32, half) holds dims (D / 2) half .. +D/2 of row 32 hb + l32
    constexpr int KF8 = D / 64;  // fp8 MFMA steps: dims (D / 2) half + 32 kk .. +32
    bf16x8 aq[HB][QF8 ? 1 : KSTEPS];
    i32x8 aq8[HB][QF8 ? KF8 : 1];
    float wreg[HB][16];
#pragma unroll
    for (int hb = 0; hb < HB && !QSHARE; ++hb) {
        int t, h;
        bool ok;
        row_to_th<MODE>(grp, 32 * hb + l32, H, T, t, h, ok);
        ok = ok && active && !producer;
        const uint16_t *qrow = a.q + ((int64_t)(b * T + t) * H + h) * D + (D / 2) * half;
        u32x4 qv[KSTEPS];
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            u32x4 v = {0, 0, 0, 0};
            if (ok) v = *reinterpret_cast<const u32x4 *>(qrow + 8 * ks);
            qv[ks] = v;
            if constexpr (!QF8) aq[hb][ks] = __builtin_bit_cast(bf16x8, v);
        }
        float qs = 1.0f;  // QF8: the row's scale, max(amax, 1e-12) / 448
        if constexpr (QF8 && !QSHARE) {
            float amax = 0.0f;
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    amax = fmaxf(amax, fmaxf(fabsf(bf16lo(qv[ks][e])), fabsf(bf16hi(qv[ks][e]))));
            amax = fmaxf(amax, __shfl_xor(amax, 32, 64));  // the row's other half
            qs = fmaxf(amax, 1e-12f) / 448.0f;
            auto code = [&](float x) { return fminf(fmaxf(x / qs, -448.0f), 448.0f); };
#pragma unroll
            for (int kk = 0; kk < KF8; ++kk)
#pragma unroll
                for (int wi = 0; wi < 8; ++wi) {  // bytes 4 wi .. +3: dims 32 kk + 4 wi .. +3
                    const int dd = 32 * kk + 4 * wi;
                    const uint32_t lo = qv[dd / 8][(dd % 8) / 2], hi = qv[dd / 8][(dd % 8) / 2 + 1];
                    uint32_t wv = __builtin_amdgcn_cvt_pk_fp8_f32(code(bf16lo(lo)), code(bf16hi(lo)), 0, false);
                    wv = __builtin_amdgcn_cvt_pk_fp8_f32(code(bf16lo(hi)), code(bf16hi(hi)), wv, true);
                    aq8[hb][kk][wi] = (int)wv;
                }
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int rb = 8 * (r / 4) + 4 * half + (r % 4);  // C row within the block
            const int i = 32 * hb + rb;
            row_to_th<MODE>(grp, i, H, T, t, h, ok);
            float wv = (ok && active && !producer) ? a.w[(int64_t)(b * T + t) * H + h] : 0.0f;
            if constexpr (QF8 && !QSHARE) wv *= __shfl(qs, rb, 64);  // lane rb holds row rb's scale
            wreg[hb][r] = wv;
        }
    }
    if constexpr (QSHARE) {
        // compute wave w, lane l: row 16 w + l / 4, dims (D / 4) (l % 4) .. +D/4 of the query,
        // and (l % 4 == 0) the row's head weight. bf16 rows keep their 16-byte chunks
        // XOR-permuted (qswz), so the 16 lanes of an operand read hit 16 bank groups.
        if (!producer) {
            constexpr int DPL = D / 4;
            const int i = 16 * wave + (lane >> 2), d0 = DPL * (lane & 3);
            int t, h;
            bool ok;
            row_to_th<MODE>(grp, i, H, T, t, h, ok);
            ok = ok && active && i < 32 * HB;
            u32x4 qv[DPL / 8];
            const uint16_t *qrow = a.q + ((int64_t)(b * T + t) * H + h) * D + d0;
#pragma unroll
            for (int j = 0; j < DPL / 8; ++j) {
                u32x4 v = {0, 0, 0, 0};
                if (ok) v = *reinterpret_cast<const u32x4 *>(qrow + 8 * j);
                qv[j] = v;
            }
            const float wv = ok ? a.w[(int64_t)(b * T + t) * H + h] : 0.0f;
            if constexpr (QF8) {
                static_assert(DPL == 32, "fp8 queries: D = 128");
                float amax = 0.0f;
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        amax = fmaxf(amax, fmaxf(fabsf(bf16lo(qv[j][e])), fabsf(bf16hi(qv[j][e]))));
                amax = fmaxf(amax, __shfl_xor(amax, 1, 64));  // the row's four lanes
                amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
                const float qs = fmaxf(amax, 1e-12f) / 448.0f;
                auto code = [&](float x) { return fminf(fmaxf(x / qs, -448.0f), 448.0f); };
                uint32_t cw[8];
#pragma unroll
                for (int wi = 0; wi < 8; ++wi) {  // bytes 4 wi .. +3: dims d0 + 4 wi .. +3
                    const uint32_t lo = qv[wi / 2][2 * (wi % 2)], hi = qv[wi / 2][2 * (wi % 2) + 1];
                    uint32_t c = __builtin_amdgcn_cvt_pk_fp8_f32(code(bf16lo(lo)), code(bf16hi(lo)), 0, false);
                    cw[wi] = __builtin_amdgcn_cvt_pk_fp8_f32(code(bf16lo(hi)), code(bf16hi(hi)), c, true);
                }
                u32x4 *dst = reinterpret_cast<u32x4 *>(sqb + i * (D / 4) + d0 / 4);
                dst[0] = u32x4{cw[0], cw[1], cw[2], cw[3]};
                dst[1] = u32x4{cw[4], cw[5], cw[6], cw[7]};
                if ((lane & 3) == 0) sqs[i] = qs;
            } else {
                u32x4 *drow = reinterpret_cast<u32x4 *>(sqb + i * (D / 2));
#pragma unroll
                for (int j = 0; j < DPL / 8; ++j) drow[qswz<D>(i, (DPL / 8) * (lane & 3) + j)] = qv[j];
            }
            if ((lane & 3) == 0) sw[i] = wv;
        }
    }
    // SPLIT: the compute waves wait for their query and weight loads here, before any
    // score store is pending (the compiler then knows them complete inside the loop);
    // the producers have nothing outstanding yet
    if constexpr (SPLIT) wait_vmcnt<0>();

    // Last visible position over every query of this workgroup (flat mode skips tiles past it).
    int last_t;
    if constexpr (PRE) last_t = min(T - 1, (int)blockIdx.y * 4 + 3);
    else last_t = min(T - 1, grp * QPG + QPG - 1);
    const int maxp = ctx - T + last_t;

    // HI: the query whose kept list maps columns to positions (one query per group).
    const int32_t *kept_row = HI ? a.kept + (int64_t)(b * T + grp) * a.n_keep : nullptr;
    const int nblk_cache = HI ? N / a.block_size : 0;

    auto col_pos = [&](int col) -> int {  // position of a column, -1 if none
        if (col >= c1) return -1;
        if constexpr (HI) {
            int blk = col / a.block_size;
            int kb = kept_row[blk];
            if (kb < 0 || kb >= nblk_cache) return -1;
            return kb * a.block_size + (col - blk * a.block_size);
        } else {
            return col < N ? col : -1;
        }
    };

    const unsigned char *kbase = reinterpret_cast<const unsigned char *>(a.k) + (int64_t)b * N * G::RB;
    const float *sbase = FP8 ? a.k_scale + (int64_t)b * N : nullptr;

    // DMA of one tile into ring stage `st`: key instruction n (of KINSTR) fills LDS chunks
    // [64 n, 64 n + 64) of the stage; lane l fills physical chunk L = 64 n + l, i.e. row
    // L / CPR, physical chunk pc = L % CPR, which holds logical chunk pc ^ swz(row) (the
    // XOR swizzle is applied on the global side, so each row is still read as one
    // contiguous line). Rows without a position read the cache start (masked later).
    // SPLIT: producer w loads exactly the 32 rows compute wave w uses. Otherwise (four
    // query groups share each tile) the waves split every tile.
    auto instr = [&](int j) { return OWN ? wave * (G::KINSTR / 4) + j : j * 4 + wave; };
    // Flat mode: a lane's byte offset from the tile's first row is the same for every
    // tile, so a tile whose rows all exist only adds the tile offset.
    int roff[G::KINSTR / 4];
#pragma unroll
    for (int j = 0; j < G::KINSTR / 4; ++j) {
        const int L = 64 * instr(j) + lane;
        const int row = L / G::CPR, pc = L % G::CPR;
        roff[j] = row * G::RB + G::swz(row, pc) * 16;
    }
    const int full_end = min(c1, N);  // flat: tiles ending at or before it need no masking
    auto issue_tile = [&](int tc0, int st) {
        unsigned char *stage = ring + st * G::STAGE;
        const bool full = !HI && tc0 + kKT <= full_end;
        const unsigned char *src[G::KINSTR / 4];
        if (full) {
            const unsigned char *tb = kbase + (int64_t)tc0 * G::RB;
#pragma unroll
            for (int j = 0; j < G::KINSTR / 4; ++j) src[j] = tb + roff[j];
        } else {
#pragma unroll
            for (int j = 0; j < G::KINSTR / 4; ++j) {
                const int L = 64 * instr(j) + lane;
                const int row = L / G::CPR, pc = L % G::CPR;
                const int pos = col_pos(tc0 + row);
                src[j] = kbase + (pos >= 0 ? (int64_t)pos * G::RB + G::swz(row, pc) * 16 : 0);
            }
        }
#pragma unroll
        for (int j = 0; j < G::KINSTR / 4; ++j)
            __builtin_amdgcn_global_load_lds((const glb_void_t *)src[j], (lds_void_t *)(stage + 1024 * instr(j)), 16,
                                             0, 0);
        if constexpr (FP8) {
            // wave w loads the scales of rows [32 w, 32 w + 32): 32 active lanes x 4 bytes
            if (lane < 32) {
                const int row = 32 * wave + lane;
                const int pos = full ? tc0 + row : col_pos(tc0 + row);
                __builtin_amdgcn_global_load_lds((const glb_void_t *)(sbase + (pos >= 0 ? pos : 0)),
                                                 (lds_void_t *)(stage + G::BYTES + 128 * wave), 4, 0, 0);
            }
        }
        if constexpr (HI) {  // positions of these rows (read back by the wave that computes them)
            if (lane < 32) tpos[st][32 * wave + lane] = col_pos(tc0 + 32 * wave + lane);
        }
    };

    auto write_score = [&](int t, int col, float v) {
        a.scores[(int64_t)(b * T + t) * a.n_out + col] = v;
    };

    const int ntiles = (c1 - c0 + kKT - 1) / kKT;
    // Flat mode: a tile is skipped when its first column lies past every query's
    // position; visibility only shrinks with the column, so skipped tiles form a suffix.
    int nvis = ntiles;
    if constexpr (!HI) nvis = maxp < c0 ? 0 : min(ntiles, (maxp - c0) / kKT + 1);
    if (!SPLIT || producer) {
#pragma unroll
        for (int p = 0; p < G::NST - 1; ++p)
            if (p < nvis) issue_tile(c0 + p * kKT, p);
    }
    if constexpr (QSHARE) {
        lds_barrier();  // the query rows and weights in LDS (the DMA above keeps streaming)
        if (!producer) {
#pragma unroll
            for (int hb = 0; hb < HB; ++hb) {
                const int qr = 32 * hb + l32;
                if constexpr (QF8) {
                    // A operand: row qr, bytes (D / 2) half + 32 kk .. +32
                    const u32x4 *src = reinterpret_cast<const u32x4 *>(sqb + qr * (D / 4) + (D / 8) * half);
#pragma unroll
                    for (int kk = 0; kk < KF8; ++kk) {
                        const u32x4 x0 = src[2 * kk], x1 = src[2 * kk + 1];
                        aq8[hb][kk] = i32x8{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3],
                                            (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
                    }
                } else {
                    // A operand: row qr, dims (D / 2) half + 8 ks .. +8 (chunk (D / 16) half + ks)
                    const u32x4 *srow = reinterpret_cast<const u32x4 *>(sqb + qr * (D / 2));
#pragma unroll
                    for (int ks = 0; ks < KSTEPS; ++ks)
                        aq[hb][ks] = __builtin_bit_cast(bf16x8, srow[qswz<D>(qr, (D / 16) * half + ks)]);
                }
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int i = 32 * hb + 8 * (r / 4) + 4 * half + (r % 4);
                    wreg[hb][r] = QF8 ? sw[i] * sqs[i] : sw[i];
                }
            }
        }
    }
    // the query and weight loads were issued before the ring DMA and so have landed once
    // at most the DMA instructions are pending; waiting here (no store is pending yet, so
    // the count is exact) lets the loop use them without a full drain of the ring
    if (!SPLIT) wait_tiles<G::PER_WAVE, G::NST - 1>(min(nvis, G::NST - 1));

    // ---- one sub-tile of 32 rows: LDS operands (load_k), then MFMA accumulators (mma)
    constexpr int NKV = FP8 ? KSTEPS / 2 : KSTEPS;  // 16-byte key fragments per lane
    struct KFrag {
        u32x4 v[NKV];
    };
    auto load_k = [&](const unsigned char *tile, int row, KFrag &kf) {
        const unsigned char *trow = tile + row * G::RB;
#pragma unroll
        for (int j = 0; j < NKV; ++j)  // bytes (D / 2 or D) * half + 16 j of the row
            kf.v[j] = *reinterpret_cast<const u32x4 *>(trow + G::swz(row, NKV * half + j) * 16);
    };
    auto mma = [&](const KFrag &kf, f32x16(&acc)[HB]) {
#pragma unroll
        for (int hb = 0; hb < HB; ++hb)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[hb][r] = 0.0f;
        if constexpr (QF8) {
            // the key bytes (D / 2) half + 32 kk .. +32 of the row, as they sit in LDS
#pragma unroll
            for (int kk = 0; kk < KF8; ++kk) {
                const u32x4 k0 = kf.v[2 * kk], k1 = kf.v[2 * kk + 1];
                const i32x8 kb = {(int)k0[0], (int)k0[1], (int)k0[2], (int)k0[3],
                                  (int)k1[0], (int)k1[1], (int)k1[2], (int)k1[3]};
#pragma unroll
                for (int hb = 0; hb < HB; ++hb) acc[hb] = mfma32_fp8(aq8[hb][kk], kb, acc[hb]);
            }
        } else if constexpr (FP8) {
#pragma unroll
            for (int kk = 0; kk < NKV; ++kk) {
                bf16x8 f0, f1;
                fp8x16_to_frags(kf.v[kk], f0, f1);
#pragma unroll
                for (int hb = 0; hb < HB; ++hb) {
                    acc[hb] = mfma32(aq[hb][2 * kk], f0, acc[hb]);
                    acc[hb] = mfma32(aq[hb][2 * kk + 1], f1, acc[hb]);
                }
            }
        } else {
#pragma unroll
            for (int ks = 0; ks < NKV; ++ks) {
                const bf16x8 f = __builtin_bit_cast(bf16x8, kf.v[ks]);
#pragma unroll
                for (int hb = 0; hb < HB; ++hb) acc[hb] = mfma32(aq[hb][ks], f, acc[hb]);
            }
        }
    };
    auto mfma_tile = [&](const unsigned char *tile, int row, f32x16(&acc)[HB]) {
        KFrag kf;
        load_k(tile, row, kf);  // every LDS operand of the sub-tile is requested before the first MFMA
        mma(kf, acc);
    };

    // ---- epilogue of one sub-tile: ReLU, head weights, head sum, scale, causal mask
    // (col: the lane's column; pos: its cache position or -1; sc: its per-token scale)
    auto epilogue = [&](const f32x16(&acc)[HB], int col, int pos, float sc) {
        if constexpr (MODE == ONEQ) {
            // head sum in four independent chains, then the other half-wave's heads
            float s4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int hb = 0; hb < HB; ++hb)
#pragma unroll
                for (int r = 0; r < 16; ++r) s4[r & 3] += wreg[hb][r] * relu_bits(acc[hb][r]);
            const float s = half_pair_sum((s4[0] + s4[1]) + (s4[2] + s4[3]));
            const int t = grp;
            const int p = ctx - T + t;
            bool emit = false;
            uint64_t comp = 0;
            if (half == 0 && col < c1) {
                const bool vis = pos >= 0 && pos <= p;
                const float v = vis ? s * sc : kNegInf;
                if (!EMIT || a.scores) write_score(t, col, v);
                if constexpr (HIST)
                    if (vis && pos >= f_se && pos < f_wl && v > kNegInf) lds_add_u32(&shist[order_key(v) >> kSelShift], 1u);
                if constexpr (EMIT) {
                    if (vis && pos >= f_se && pos < f_wl && v > kNegInf) {
                        const uint32_t key = order_key(v);
                        // the positive scores' quarter-octave bins (the selection's own
                        // resolution); every negative score in bin 0, below them all
                        const uint32_t bin = key >= 0x80000000u ? (key >> kSelShift) - 1024u : 0u;
                        lds_add_u32(&whist[wave][bin], 1u);
                        emit = bin >= e_thr;
                        comp = ((uint64_t)key << 32) | (uint32_t)~(uint32_t)pos;
                    }
                }
            }
            if constexpr (EMIT) {  // the whole wave takes part (uniform call)
                const uint64_t eb = __ballot(emit);
                if (emit) e_row[e_cnt + lane_rank64(eb)] = comp;
                e_cnt += (uint32_t)__popcll(eb);
            }
        } else if constexpr (MODE == Q4) {
            float part[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int r = 0; r < 16; ++r) part[r / 4] += wreg[0][r] * relu_bits(acc[0][r]);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int t = grp * QPG + 2 * j + half;
                const int p = ctx - T + t;
                if (t < T && col < c1) write_score(t, col, (pos >= 0 && pos <= p) ? part[j] * sc : kNegInf);
            }
        } else {
            float part[QPG];
#pragma unroll
            for (int j = 0; j < QPG; ++j) part[j] = 0.0f;
#pragma unroll
            for (int r = 0; r < 16; ++r) part[(8 * (r / 4)) / MODE] += wreg[0][r] * relu_bits(acc[0][r]);
#pragma unroll
            for (int j = 0; j < QPG; ++j) {
                part[j] += __shfl_xor(part[j], 32, 64);
                const int t = grp * QPG + j;
                const int p = ctx - T + t;
                if (half == 0 && t < T && col < c1) write_score(t, col, (pos >= 0 && pos <= p) ? part[j] * sc : kNegInf);
            }
        }
    };

    // ---- ring wait + refill at the top of iteration `it`
    auto advance = [&](int it) {
        // this wave's DMA of tile `it` is complete once at most `ahead` later tiles'
        // instructions are pending (vector memory operations retire in issue order)
        wait_tiles<G::PER_WAVE, G::NST - 2>(min(G::NST - 2, nvis - 1 - it));
        // OWN: this wave's rows of tile `it` landed and it has finished reading its rows of
        // tile it-1 (the stage refilled next). Shared tiles: every wave's part landed and
        // every wave is done with tile it-1.
        if constexpr (!OWN) __syncthreads();
        if (it + G::NST - 1 < nvis)
            issue_tile(c0 + (it + G::NST - 1) * kKT, (it + G::NST - 1) % G::NST);
    };

    // SPLIT: tile `it` is in the ring once every producer's DMA of it landed (each waits
    // for its own), and its stage may be refilled once every compute wave is done with
    // tile it-1: one workgroup barrier (LDS ordering only) per tile covers both.
    auto sync_tile = [&](int it) {
        if (producer) wait_tiles<G::PER_WAVE, G::NST - 2>(min(G::NST - 2, nvis - 1 - it));
        lds_barrier();
        if (producer && it + G::NST - 1 < nvis)
            issue_tile(c0 + (it + G::NST - 1) * kKT, (it + G::NST - 1) % G::NST);
    };

    if constexpr (PRE) {
        // four query groups share each tile: every wave computes all four sub-tiles
        for (int it = 0; it < nvis; ++it) {
            advance(it);
            const int st = it % G::NST;
            const unsigned char *tile = ring + st * G::STAGE;
            const float *tscale = reinterpret_cast<const float *>(tile + G::BYTES);
            if (active) {
                // the MFMAs of sub-tile sb + 1 are issued before the epilogue of sub-tile sb
                // (accumulators alternate), so the matrix core and the VALU overlap
                f32x16 acc[2][HB];
                mfma_tile(tile, l32, acc[0]);
#pragma unroll
                for (int sb = 0; sb < 4; ++sb) {
                    const int row = sb * 32 + l32;
                    if (sb + 1 < 4) mfma_tile(tile, row + 32, acc[(sb + 1) & 1]);
                    const int col = c0 + it * kKT + row;
                    epilogue(acc[sb & 1], col, col < c1 && col < N ? col : -1, FP8 ? tscale[row] : 1.0f);
                }
                if constexpr (EMIT) {
                    // the running threshold, every fourth tile: lane l sums bins 1023 - 16 l - e
                    // (from the top), a wave scan finds the lane where the count reaches the
                    // fill size, that lane the bin (this wave's own adds are ordered before)
                    if ((it & 3) == 3) {
                        lds_wait_all();
                        uint32_t hv[16], sum = 0;
#pragma unroll
                        for (int e = 0; e < 16; ++e) {
                            hv[e] = whist[wave][kEB - 1 - 16 * lane - e];
                            sum += hv[e];
                        }
                        uint32_t cum = sum;
#pragma unroll
                        for (int o = 1; o < 64; o <<= 1) {
                            const uint32_t y = __shfl_up(cum, o, 64);
                            if (lane >= o) cum += y;
                        }
                        const uint64_t reach = __ballot(e_m > 0 && cum >= e_m);
                        if (reach) {
                            const int L = __ffsll((unsigned long long)reach) - 1;
                            int bin = 0;
                            uint32_t acc2 = cum - sum;
#pragma unroll
                            for (int e = 0; e < 16; ++e) {
                                acc2 += hv[e];
                                if (bin == 0 && acc2 >= e_m) bin = kEB - 1 - 16 * lane - e;
                            }
                            e_thr = (uint32_t)__builtin_amdgcn_readlane(bin, L);
                        }
                    }
                }
            }
        }
    } else {
        // (one query group per workgroup: every compute wave is active)
        // Software pipeline over this wave's 32 rows of each tile: the MFMAs of tile `it`
        // are issued before the epilogue of tile it-1 (accumulators alternate), so the
        // matrix core and the VALU work on different tiles at the same time. The scale
        // and position of a tile are read while its stage is current (the producers
        // refill that stage after the next barrier).
        const int row = wave * 32 + l32;
        f32x16 acc0[HB], acc1[HB];
        int pcol = 0, ppos = -1;
        float psc = 0.0f;
        auto step = [&](int it, f32x16(&cur)[HB], const f32x16(&prev)[HB]) {
            const int st = it % G::NST;
            const unsigned char *tile = ring + st * G::STAGE;
            const float sc = FP8 ? reinterpret_cast<const float *>(tile + G::BYTES)[row] : 1.0f;
            const int col = c0 + it * kKT + row;
            int pos;
            if constexpr (HI) pos = tpos[st][row];
            else pos = col < c1 && col < N ? col : -1;
            mfma_tile(tile, row, cur);
            if (it > 0) epilogue(prev, pcol, ppos, psc);
            pcol = col;
            ppos = pos;
            psc = sc;
        };
        for (int it = 0; it < nvis; it += 2) {
            sync_tile(it);
            if (!producer) step(it, acc0, acc1);
            if (it + 1 < nvis) {
                sync_tile(it + 1);
                if (!producer) step(it + 1, acc1, acc0);
            }
        }
        if (!producer && nvis > 0) {
            if (nvis & 1) epilogue(acc0, pcol, ppos, psc);
            else epilogue(acc1, pcol, ppos, psc);
        }
    }
    if constexpr (EMIT)
        if (active && lane == 0) a.cand_cnt[b * T + grp] = e_cnt;
    {  // tiles past every query's position: -inf
        constexpr int NQ = PRE ? 4 : QPG;
        for (int e = nvis * kKT + tid; e < ntiles * kKT * NQ; e += NT) {
            // e runs over (query q, column offset) of the skipped tiles
            int q = e / (ntiles * kKT);
            int off = e % (ntiles * kKT);
            if (off < nvis * kKT) continue;
            int col = c0 + off;
            int t = PRE ? ((int)blockIdx.y * 4 + q) : grp * QPG + q;
            if (col < c1 && t < T && (!EMIT || a.scores)) write_score(t, col, kNegInf);
        }
    }
    if constexpr (HIST) {
        // the histogram adds above are inline asm (not tracked by the compiler); the LDS-only
        // barrier does not wait for the score stores still in flight
        lds_barrier();
        if (active) {
            uint32_t *g = a.sel_hist + (int64_t)(b * T + grp) * kSelBins;
            for (int i = tid; i < kSelBins; i += NT) {
                const uint32_t v = shist[i];
                if (v) atomicAdd(&g[i], v);
            }
        }
    }
}

// ---------------------------------------------------------------------------- blocks

// One thread per block j; the query token's (H x D) rows staged in LDS as fp32, the
// block's mean key held in registers (all its loads in flight at once), the head dots
// summed in dimension order.
template <int D>
__global__ __launch_bounds__(256) void index_blocks_kernel(IndexBlocksArgs a) {
    extern __shared__ float qs[];  // [H][D]
    // sel_hist (priming a selection without causal mask or forced set): this workgroup's
    // count of finite scores per first-level bin, added to the row's histogram at the end
    __shared__ uint32_t shist[kSelBins];
    const bool prime = a.sel_hist != nullptr;
    const int b = blockIdx.z, t = blockIdx.y;
    const int H = a.H, T = a.T;
    if (prime)
        for (int i = threadIdx.x; i < kSelBins; i += blockDim.x) shist[i] = 0;
    const int64_t qoff = ((int64_t)b * T + t) * H * D;
    for (int e = threadIdx.x; e < H * D; e += blockDim.x) {
        uint16_t bits = a.q[qoff + e];
        qs[e] = u2f((uint32_t)bits << 16);
    }
    const int j = blockIdx.x * blockDim.x + threadIdx.x;
    const bool in = j < a.n_blocks;
    float kv[D];
    {
        const float4 *kb4 = reinterpret_cast<const float4 *>(a.kbar + ((int64_t)b * a.n_blocks + (in ? j : 0)) * D);
#pragma unroll
        for (int d4 = 0; d4 < D / 4; ++d4) {
            const float4 v = kb4[d4];
            kv[4 * d4] = v.x, kv[4 * d4 + 1] = v.y, kv[4 * d4 + 2] = v.z, kv[4 * d4 + 3] = v.w;
        }
    }
    __syncthreads();
    if (!in && !prime) return;
    int ctx = a.ctx_len ? a.ctx_len[b] : a.N;
    ctx = min(max(ctx, 0), a.N);
    const int p = ctx - T + t;
    const int Bs = a.block_size;
    // eligibility: complete, visible, and at least one non-forced position (reading R9)
    const int64_t lo = (int64_t)j * Bs, hi = lo + Bs - 1;  // inclusive
    bool ok = in && hi <= p;
    if (ok) {
        int64_t nf = 0;
        const int64_t s_hi = min((int64_t)a.sink, (int64_t)p + 1) - 1;  // sink [0, s_hi]
        const int64_t w_lo = a.window > 0 ? max((int64_t)0, (int64_t)p - a.window + 1) : (int64_t)p + 1;
        auto overlap = [](int64_t a0, int64_t a1, int64_t b0, int64_t b1) -> int64_t {
            int64_t l = max(a0, b0), r = min(a1, b1);
            return r >= l ? r - l + 1 : 0;
        };
        nf += overlap(lo, hi, 0, s_hi);
        nf += overlap(lo, hi, w_lo, p);
        nf -= overlap(lo, hi, max((int64_t)0, w_lo), min(s_hi, (int64_t)p));  // sink and window overlap
        ok = nf < Bs;
    }
    float best = kNegInf;
    if (ok) {
        const float *wt = a.w + ((int64_t)b * T + t) * H;
        for (int h = 0; h < H; ++h) {
            float dot = 0.0f;
            const float *qh = qs + h * D;
#pragma unroll
            for (int d = 0; d < D; ++d) dot = fmaf(qh[d], kv[d], dot);
            const float v = wt[h] * fmaxf(dot, 0.0f);
            best = h == 0 ? v : fmaxf(best, v);
        }
    }
    if (in) a.scores[((int64_t)b * T + t) * a.n_blocks + j] = best;
    if (prime) {
        if (in && best > kNegInf) atomicAdd(&shist[order_key(best) >> kSelShift], 1u);
        __syncthreads();
        uint32_t *g = a.sel_hist + ((int64_t)b * T + t) * kSelBins;
        for (int i = threadIdx.x; i < kSelBins; i += blockDim.x) {
            const uint32_t v = shist[i];
            if (v) atomicAdd(&g[i], v);
        }
    }
}

// ---------------------------------------------------------------------------- block means

// One workgroup of D threads per (block j, sequence b); thread d sums dimension d.
__global__ __launch_bounds__(128) void block_means_kernel(BlockMeansArgs a) {
    const int j = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
    if (d >= a.D) return;
    const int Bs = a.block_size, D = a.D;
    const int64_t row0 = (int64_t)b * a.N + (int64_t)j * Bs;
    a.kbar[((int64_t)b * a.n_blocks + j) * D + d] = block_mean_d(a.k, a.fp8, a.k_scale, row0, Bs, D, d);
}

int compute_units() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
        n = 256;
    return n;
}

// Decode (SPLIT) workgroups per compute unit over the launch (one resident at a time: the
// ring takes more than half of the LDS); a build may set another count to compare.
#ifndef LSA_DECODE_WG_PER_CU
#define LSA_DECODE_WG_PER_CU 1
#endif
constexpr int kDecodeWgPerCu = LSA_DECODE_WG_PER_CU;

// Measurement hook (lsa_index_launch_events): the next token-indexer launch on this host
// thread records its own start and end into these events, from the dispatch itself.
thread_local hipEvent_t t_ev_start = nullptr, t_ev_stop = nullptr;

#define LSA_LAUNCH_TOKENS(K, GRID, BLOCK, LDS, S, ...)                                                      \
    do {                                                                                                     \
        if (t_ev_start || t_ev_stop) {                                                                       \
            hipEvent_t e0_ = t_ev_start, e1_ = t_ev_stop;                                                    \
            t_ev_start = t_ev_stop = nullptr;                                                                \
            hipExtLaunchKernelGGL(K, GRID, BLOCK, (uint32_t)(LDS), S, e0_, e1_, 0, __VA_ARGS__);             \
        } else {                                                                                             \
            hipLaunchKernelGGL(K, GRID, BLOCK, LDS, S, __VA_ARGS__);                                         \
        }                                                                                                    \
    } while (0)

template <int D, bool FP8, bool QF8, int MODE, int HB, bool HI, bool PRE, bool HIST = false>
hipError_t launch_tokens_t(const IndexTokensArgs &a, hipStream_t s) {
    constexpr int NST = 4;  // one tile computed, three in flight (deeper rings measured no faster)
    using G = Tile<D, FP8, NST>;
    const int QPG = MODE == ONEQ ? 1 : 32 / MODE;
    const int groups = (a.T + QPG - 1) / QPG;
    const int gy = PRE ? (groups + 3) / 4 : groups;
    const int max_chunks = (a.n_out + kKT - 1) / kKT;
    // SPLIT kernels (8 waves, 2 per SIMD): one workgroup per CU, every wave of a CU the
    // same age, so no workgroup is starved by the oldest-first issue arbitration of an
    // older one on the same CU; shared tiles (4 waves): two per CU
    const int target = PRE ? 512 : kDecodeWgPerCu * compute_units();
    int want = (target + a.B * gy - 1) / (a.B * gy);
    int chunks = want < 1 ? 1 : (want > max_chunks ? max_chunks : want);
    int chunk = (a.n_out + chunks - 1) / chunks;
    chunk = (chunk + kKT - 1) / kKT * kKT;
    chunks = (a.n_out + chunk - 1) / chunk;
    dim3 grid(chunks, gy, a.B);
    const size_t lds = (size_t)G::NST * G::STAGE;
    LSA_LAUNCH_TOKENS((index_tokens_kernel<D, FP8, QF8, MODE, HB, HI, PRE, HIST, NST>), grid,
                      dim3(PRE ? kThreads : 2 * kThreads), lds, s, a, groups, chunk);
    return hipGetLastError();
}

// Candidate emission (a.cand): the shared-tile kernel with one whole row per wave, a
// 3-stage key ring (the four waves' running-threshold histograms take the fourth stage's
// LDS, so two workgroups still fit on a compute unit).
template <int D, bool FP8, bool QF8, int HB>
hipError_t launch_tokens_emit(const IndexTokensArgs &a, hipStream_t s) {
    constexpr int NST = 3;
    using G = Tile<D, FP8, NST>;
    const int groups = a.T;
    const dim3 grid(1, (groups + 3) / 4, a.B);
    const size_t lds = (size_t)G::NST * G::STAGE;
    LSA_LAUNCH_TOKENS((index_tokens_kernel<D, FP8, QF8, ONEQ, HB, false, true, false, NST, true>), grid,
                      dim3(kThreads), lds, s, a, groups, a.n_out);
    return hipGetLastError();
}

template <int D, bool FP8, bool QF8 = false>
hipError_t launch_tokens_d(const IndexTokensArgs &a, hipStream_t s) {
    if (a.cand) return a.H == 32 ? launch_tokens_emit<D, FP8, QF8, 1>(a, s) : launch_tokens_emit<D, FP8, QF8, 2>(a, s);
    const bool hi = a.kept != nullptr;
    if (a.sel_hist) {  // one query per workgroup: the epilogue builds the selection histogram
        if (hi) {
            if (a.H <= 32) return launch_tokens_t<D, FP8, QF8, ONEQ, 1, true, false, true>(a, s);
            return launch_tokens_t<D, FP8, QF8, ONEQ, 2, true, false, true>(a, s);
        }
        if (a.H == 32) return launch_tokens_t<D, FP8, QF8, ONEQ, 1, false, false, true>(a, s);
        return launch_tokens_t<D, FP8, QF8, ONEQ, 2, false, false, true>(a, s);
    }
    if (hi) {
        if (a.H <= 32) return launch_tokens_t<D, FP8, QF8, ONEQ, 1, true, false>(a, s);
        return launch_tokens_t<D, FP8, QF8, ONEQ, 2, true, false>(a, s);
    }
    switch (a.H) {
        case 4: return launch_tokens_t<D, FP8, QF8, Q4, 1, false, false>(a, s);
        case 8: return launch_tokens_t<D, FP8, QF8, Q8, 1, false, false>(a, s);
        case 16: return launch_tokens_t<D, FP8, QF8, Q16, 1, false, false>(a, s);
        case 32:
            if (a.T >= 64) return launch_tokens_t<D, FP8, QF8, ONEQ, 1, false, true>(a, s);
            return launch_tokens_t<D, FP8, QF8, ONEQ, 1, false, false>(a, s);
        default:
            if (a.T >= 64) return launch_tokens_t<D, FP8, QF8, ONEQ, 2, false, true>(a, s);
            return launch_tokens_t<D, FP8, QF8, ONEQ, 2, false, false>(a, s);
    }
}

}  // namespace

bool index_tokens_fused_hist(int H, int T, bool hi) {
    if (hi) return true;
    return (H == 32 || H == 64) && T < 64;
}

bool index_tokens_emits(int B, int T, int N, int H, int D, bool hi) {
    // the shared-tile kernel (T >= 64) with whole rows per workgroup: at least as many
    // groups of four query tokens as the 512 workgroups it aims for
    (void)N;
    if (hi || !(H == 32 || H == 64) || (D != 64 && D != 128) || T < 64) return false;
    return (int64_t)B * ((T + 3) / 4) >= 512;
}

bool index_tokens_supported(int H, int D, bool hi) {
    if (D != 64 && D != 128) return false;
    if (hi) return H >= 1 && H <= 64;
    return H == 4 || H == 8 || H == 16 || H == 32 || H == 64;
}

void set_index_launch_events(hipEvent_t start, hipEvent_t stop) {
    t_ev_start = start;
    t_ev_stop = stop;
}

hipError_t launch_index_tokens(const IndexTokensArgs &a, hipStream_t s) {
    if (a.qf8) return launch_tokens_d<128, true, true>(a, s);  // fp8 keys, D = 128 (checked by the caller)
    if (a.D == 64) return a.fp8 ? launch_tokens_d<64, true>(a, s) : launch_tokens_d<64, false>(a, s);
    return a.fp8 ? launch_tokens_d<128, true>(a, s) : launch_tokens_d<128, false>(a, s);
}

hipError_t launch_index_blocks(const IndexBlocksArgs &a, hipStream_t s) {
    dim3 grid((a.n_blocks + 255) / 256, a.T, a.B);
    size_t lds = (size_t)a.H * a.D * sizeof(float);
    if (a.D == 64) hipLaunchKernelGGL(index_blocks_kernel<64>, grid, dim3(256), lds, s, a);
    else hipLaunchKernelGGL(index_blocks_kernel<128>, grid, dim3(256), lds, s, a);
    return hipGetLastError();
}

hipError_t launch_block_means(const BlockMeansArgs &a, hipStream_t s) {
    dim3 grid(a.n_blocks, a.B);
    hipLaunchKernelGGL(block_means_kernel, grid, dim3(128), 0, s, a);
    return hipGetLastError();
}

}  // namespace lsa
