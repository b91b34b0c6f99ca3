// Sparse attention over the selected rows only (LongCat-2.0 summary, aitrends.kr,
// "Technical features": no attention matrix over all token pairs), for MQA/GQA and
// MLA latent KV, several CLI layers per launch.
//
// One workgroup = (layer, sequence, query token, KV head, split of the K selected
// rows); wave w owns 16 query heads of the KV head's group. Per tile of 32 selected
// rows:
//   - the rows are gathered HBM -> LDS by direct-to-LDS DMA (global_load_lds_dwordx4)
//     into a 3-stage ring (two tiles in flight while one is computed). A row is cut
//     into blocks of four 16-byte chunks; block k of all 32 rows forms 2 KB of LDS,
//     row r at 64 r, its chunks XOR-permuted by (r >> 2) & 3. One DMA instruction
//     fills one block for 16 rows, every lane's source and destination is fixed for
//     the whole launch, and both LDS read patterns below are free of bank conflicts;
//   - S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (lane = one head, 8 rows), so the
//     online-softmax statistics of a head stay inside one lane group;
//   - P^T is packed to bf16 straight from the S^T accumulators (no LDS round trip)
//     and O^T += V^T P^T accumulates on MFMA in fp32; the V^T operand comes from LDS
//     transpose reads (ds_read_b64_tr_b16).
// Splits write partials (o / l as bf16 rows, m and l in fp32) that a second kernel
// merges in split order.
//
// Fused selection: a workgroup can also resolve its own split of the selection (the
// selection's last pass, for flat rows) before it gathers: the LDS tile ring is free
// then and holds the pass's working set, and the positions land straight in the LDS
// position list, with no kernel boundary and no round trip of the index list through
// memory in between.
#include <mutex>

#include <hip/hip_ext.h>

#include "select_core.cuh"

namespace lsa {
namespace {

// Split partials of lsa_attend_noalloc, for callers that cannot allocate: one copy per
// GPU, held until the process ends, shared by every such call on that GPU (calls that
// overlap on one GPU race for it). Host code takes its device address from
// hipGetSymbolAddress, never from this name.
static __device__ __align__(256) unsigned char scratch[kAttendStaticScratchBytes];

constexpr int kRows = 32;     // selected rows per tile
constexpr int kMaxR = 2048;   // selected rows per split (positions staged in LDS)
constexpr int kBlk = 2048;    // LDS bytes of one block (4 chunks) of the 32 rows
// up to 16 query heads per KV head (one wave of heads): workgroups aimed for, three per
// compute unit in one generation
constexpr int kOneHeadTarget = 768;
constexpr size_t kLdsPerCu = 160 * 1024;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((__vector_size__(8 * sizeof(short)))) short s16x8;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) unsigned char lds_u8;

// s_waitcnt vmcnt(n) (gfx9 encoding: expcnt and lgkmcnt left at their maxima)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

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

// Physical chunk slot (0..3) of logical chunk j of row r inside a block.
__device__ __forceinline__ int slot(int j, int r) { return j ^ ((r >> 2) & 3); }

// Fused selection resolve: the selection's arguments and workspace, and the share of the
// tile ring its working set takes (tie entries held in LDS, the row bitmap in LDS or not).
struct FuseArgs {
    SelectArgs sa;
    sel::Ws w;
    int tl;
    int pw_log;
    int bits_lds;
};

template <int DQK, int DV, int HW, bool MLA, bool OUTF32, int NSTC = 4>
struct AttTile {
    static constexpr int NT = 64 * HW;
    static constexpr int KB = DQK * 2 / 64;           // K blocks per row (MLA 18, else 4)
    static constexpr int VB = MLA ? 0 : DV * 2 / 64;  // V blocks (separate V cache)
    static constexpr int STAGE = (KB + VB) * kBlk;
    static constexpr int INSTR = 2 * (KB + VB);       // DMA instructions per tile (16 rows each)
    static_assert(INSTR % HW == 0, "tile must split evenly over the waves");
    static constexpr int PER_WAVE = INSTR / HW;
    // tiles in LDS: one computed, NST-1 in flight; as many as the LDS (with the position
    // list) and the 6-bit vmcnt allow, at most NSTC
    static constexpr int LDS_MAX = 160 * 1024 - kMaxR * 4 - kMaxR / 32 * 4;
    static constexpr int NST_LDS = LDS_MAX / STAGE;
    static constexpr int NST_V = 63 / PER_WAVE + 1;
    static constexpr int NST_A = NST_LDS < NST_V ? NST_LDS : NST_V;
    static constexpr int NST = NST_A < NSTC ? NST_A : NSTC;
    static_assert(NST >= 2, "two stages at least");
    static_assert(PER_WAVE * (NST - 1) < 64, "vmcnt budget");
    static_assert(!MLA || DV == 512, "MLA values are the first 512 columns (16 blocks)");
};

template <int DQK, int DV, int HW, bool MLA, bool OUTF32, bool FUSED, int NSTC = 4>
__global__ __launch_bounds__(64 * HW) void attend_kernel(AttendArgs a, uint16_t *po, float *pml, int R, FuseArgs f) {
    using G = AttTile<DQK, DV, HW, MLA, OUTF32, NSTC>;
    constexpr int NT = G::NT;
    constexpr int KSQ = DQK / 32;
    constexpr int NCB = DV / 16;
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    int *posbuf = reinterpret_cast<int *>(lds + G::NST * G::STAGE);  // [R] (R <= kMaxR, a multiple of 32)
    uint32_t *vmask = reinterpret_cast<uint32_t *>(posbuf + R);       // [R / 32] valid rows per tile

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int hl = lane & 15, q4 = lane >> 4;
    const int B = a.B, T = a.T, Hq = a.Hq, Hkv = a.Hkv, K = a.K;
    const int split = blockIdx.x;
    const int t = blockIdx.y / Hkv, kvh = blockIdx.y % Hkv;
    const int layer = blockIdx.z / B, b = blockIdx.z % B;
    const int g = Hq / Hkv;
    const int hg = 16 * wave + hl;  // head inside the group
    const bool hvalid = hg < g;
    const int hq = kvh * g + (hvalid ? hg : 0);
    const int r0 = split * R;
    const int nrows = max(0, min(K, r0 + R) - r0);
    const int nsplit = gridDim.x;
    const int ntile = (nrows + kRows - 1) / kRows;

    // Q as the B operand of S^T = K Q^T: lane holds head hl, dims 32 ks + 8 q4 .. +8
    bf16x8 bq[KSQ];
    auto load_q = [&]() __attribute__((always_inline)) {
        const uint16_t *qp = a.q + layer * a.lsq + (((int64_t)b * T + t) * Hq + hq) * DQK + 8 * q4;
#pragma unroll
        for (int ks = 0; ks < KSQ; ++ks) {
            u32x4 v = {0, 0, 0, 0};
            if (hvalid) v = *reinterpret_cast<const u32x4 *>(qp + 32 * ks);
            bq[ks] = __builtin_bit_cast(bf16x8, v);
        }
    };
    const int64_t selrow = (int64_t)b * T + t;
    // paged caches: one row pool per layer (no per-sequence offset), position s of
    // sequence b at row bt[b][s / page_size] * page_size + s % page_size
    const int64_t bofs_k = a.bt ? 0 : b * a.ksb, bofs_v = a.bt ? 0 : b * a.vsb;
    auto phys = [&](int s) -> int {  // cache row of position s in [0, N), -1 if its page is unmapped
        if (!a.bt) return s;
        const int pg = s / a.page_size;
        if (pg >= a.max_pages) return -1;
        const int pp = a.bt[(int64_t)b * a.max_pages + pg];
        return (pp >= 0 && pp < a.num_pages) ? pp * a.page_size + (s - pg * a.page_size) : -1;
    };
    // the workgroups sharing a selection row: splits x KV heads x layers
    const int nslices = nsplit * Hkv * a.L, slice = split + nsplit * (kvh + Hkv * layer);
    if constexpr (FUSED) {
        // resolve rows r0 .. r0 + nrows - 1 of the selection into the position list;
        // its working set lives in the tile ring (ties, histograms, scratch, bitmap)
        sel::SliceLds S;
        unsigned char *p = lds;
        S.ties = reinterpret_cast<uint64_t *>(p);
        p += (size_t)f.tl * 8;
        S.h = reinterpret_cast<uint32_t *>(p);
        p += sel::kB2 * 4;
        S.h256 = reinterpret_cast<uint32_t *>(p);
        p += 256 * 4;
        S.scr = reinterpret_cast<uint32_t *>(p);
        p += 32 * 4;
        S.bits = reinterpret_cast<uint32_t *>(p);
        S.tl = f.tl;
        S.pw_log = f.pw_log;
        S.bits_lds = f.bits_lds != 0;
        // Q is requested once the selection's first loads are (their wait does not cover it)
        sel::resolve_slice<NT>(f.sa, f.w, (int)selrow, r0, r0 + nrows, S, posbuf,
                               [&]() __attribute__((always_inline)) { load_q(); });  // ends with a barrier
        if (kvh == 0 && layer == 0) {
            int32_t *dst = f.sa.idx + selrow * K + r0;
            for (int i = tid; i < nrows; i += NT) dst[i] = posbuf[i];
        }
        if (a.bt) {  // positions -> cache rows (or -1), each thread its own entries
            for (int i = tid; i < nrows; i += NT) {
                const int ps = posbuf[i];
                posbuf[i] = (ps >= 0 && ps < a.N) ? phys(ps) : -1;
            }
            __syncthreads();
        }
    }
    // shared selection (draft tokens): one index row per sequence; token t attends only
    // over its entries at positions <= its own p
    const int32_t *idxrow = FUSED ? nullptr : a.idx + (a.idx_shared ? (int64_t)b : selrow) * K + r0;
    const int pmax = a.idx_shared ? (a.ctx_len ? a.ctx_len[b] : a.N) - T + t : 0x7FFFFFFF;
    const uint16_t *kbase = a.k + layer * a.lsk + bofs_k + kvh * a.ksh;
    const uint16_t *vbase = MLA ? kbase : a.v + layer * a.lsv + bofs_v + kvh * a.vsh;

    // ---- DMA: instruction n of a tile fills block n / 2 (K blocks, then V blocks) for
    // rows 16 (n & 1) .. +15; lane l writes 16 bytes at 16 l: row 16 (n & 1) + l / 4,
    // slot l & 3, which holds logical chunk slot(l & 3, row) of the block.
    const int drow = lane >> 2;                            // + 16 (n & 1)
    const int dchk0 = slot(lane & 3, drow), dchk1 = slot(lane & 3, drow + 16);  // (row + 16) >> 2 & 3 == row >> 2 & 3
    auto issue_tile = [&](int it, int p0, int p1) {  // p0, p1: positions of rows drow, drow + 16
        lds_u8 *stage = (lds_u8 *)lds + (it % G::NST) * G::STAGE;
#pragma unroll
        for (int jj = 0; jj < G::PER_WAVE; ++jj) {
            const int n = jj * HW + wave;
            const int blk = n >> 1, hi = n & 1;
            const bool isv = blk >= G::KB;
            const int cb = isv ? blk - G::KB : blk;  // block within the K or V row
            const int pos = hi ? p1 : p0;
            const int chk = 4 * cb + (hi ? dchk1 : dchk0);
            const uint16_t *src = (isv ? vbase + (int64_t)pos * a.vsn : kbase + (int64_t)pos * a.ksn) + 8 * chk;
            __builtin_amdgcn_global_load_lds((const glb_void_t *)src, (lds_void_t *)(stage + blk * kBlk + 1024 * hi), 16,
                                             0, 0);
        }
    };

    // ---- prologue. Vector memory operations retire in issue order, so each wait below
    // only covers what it needs: the selected positions come first (tile 0's DMA and the
    // LDS position list need them), then tile 0's DMA, then Q (the first MFMA waits for
    // Q, and so for tile 0, but not for the later tiles), then the DMA of tiles
    // 1 .. NST-2. The position list is written to LDS last, ready by the loop's first
    // barrier. Without the fused resolve the positions come from the index list: every
    // entry this thread needs is requested at once (the DMA rows of the first tiles and
    // its entries of the LDS list), then checked, then, for a paged cache, mapped to cache
    // rows by a second batch of block-table loads, so the round trips overlap instead of
    // following one another.
    constexpr int PIT = kMaxR / NT;   // LDS list entries per thread, at most
    const int nlist = ntile * kRows;  // LDS list length (whole tiles)
    int dpos[G::NST - 1][2];
    int lpos[PIT];                    // entries tid + NT j of the LDS list (without the fused resolve)
    if constexpr (FUSED) {
#pragma unroll
        for (int p = 0; p < G::NST - 1; ++p)
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const int i = p * kRows + drow + 16 * r;
                const int ps = i < nrows ? posbuf[i] : -1;  // cache rows when paged
                dpos[p][r] = (ps >= 0 && (a.bt || ps < a.N)) ? ps : -1;
            }
    } else {
        auto raw = [&](int i) -> int {  // entry i of the split's index list (nrows > 0), -1 past it
            const int v = idxrow[min(i, nrows - 1)];
            return i < nrows ? v : -1;
        };
        auto check = [&](int ps) { return (ps >= 0 && ps < a.N && ps <= pmax) ? ps : -1; };
#pragma unroll
        for (int p = 0; p < G::NST - 1; ++p) dpos[p][0] = dpos[p][1] = -1;
#pragma unroll
        for (int j = 0; j < PIT; ++j) lpos[j] = -1;
        if (nrows > 0) {  // unconditional loads (clamped indices), so they issue back to back
#pragma unroll
            for (int p = 0; p < G::NST - 1; ++p) {
                dpos[p][0] = raw(p * kRows + drow);
                dpos[p][1] = raw(p * kRows + drow + 16);
            }
#pragma unroll
            for (int j = 0; j < PIT; ++j) lpos[j] = raw(tid + NT * j);
        }
#pragma unroll
        for (int p = 0; p < G::NST - 1; ++p) {
            dpos[p][0] = check(dpos[p][0]);
            dpos[p][1] = check(dpos[p][1]);
        }
#pragma unroll
        for (int j = 0; j < PIT; ++j) lpos[j] = check(lpos[j]);
        if (a.bt) {
            // page of each position (page 0 for none), its block-table entry, then the row
            auto page = [&](int ps) { return ps >= 0 ? min(ps / a.page_size, a.max_pages - 1) : 0; };
            auto row = [&](int ps, int pp) -> int {
                if (ps < 0 || ps / a.page_size >= a.max_pages || pp < 0 || pp >= a.num_pages) return -1;
                return pp * a.page_size + ps % a.page_size;
            };
            const int32_t *btrow = a.bt + (int64_t)b * a.max_pages;
            int dpp[G::NST - 1][2], lpp[PIT];
#pragma unroll
            for (int p = 0; p < G::NST - 1; ++p) {
                dpp[p][0] = btrow[page(dpos[p][0])];
                dpp[p][1] = btrow[page(dpos[p][1])];
            }
#pragma unroll
            for (int j = 0; j < PIT; ++j) lpp[j] = btrow[page(lpos[j])];
#pragma unroll
            for (int p = 0; p < G::NST - 1; ++p) {
                dpos[p][0] = row(dpos[p][0], dpp[p][0]);
                dpos[p][1] = row(dpos[p][1], dpp[p][1]);
            }
#pragma unroll
            for (int j = 0; j < PIT; ++j) lpos[j] = row(lpos[j], lpp[j]);
        }
    }
    // invalid rows read row 0 (finite values; zero probability)
    if (ntile > 0) issue_tile(0, max(dpos[0][0], 0), max(dpos[0][1], 0));
    if constexpr (!FUSED) load_q();
#pragma unroll
    for (int p = 1; p < G::NST - 1; ++p)
        if (p < ntile) issue_tile(p, max(dpos[p][0], 0), max(dpos[p][1], 0));
    // (FUSED: entries are rewritten in place, each by the thread that reads it; the DMA
    // positions read above take max(., 0) and so agree with either value)
#pragma unroll
    for (int j = 0; j < PIT; ++j) {
        if (NT * j >= nlist) break;
        const int i = tid + NT * j;
        const bool in = i < nlist;
        int ps = -1;
        if constexpr (FUSED) {
            const int v = in && i < nrows ? posbuf[i] : -1;
            ps = (v >= 0 && (a.bt || v < a.N)) ? v : -1;
        } else {
            ps = lpos[j];
        }
        if (in) posbuf[i] = max(ps, 0);
        const uint64_t bal = __ballot(in && ps >= 0);
        if (lane == 0 && in) {
            vmask[i >> 5] = (uint32_t)bal;
            if (i + 32 < nlist) vmask[(i >> 5) + 1] = (uint32_t)(bal >> 32);
        }
    }

    f32x4 o[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) o[cb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    float m_run = kNegInf, l_run = 0.0f;
    const float sl2 = a.scale * kLog2e;
    // ---- per-lane LDS read bases (constant offsets added per block)
    // K fragment (A operand of S^T): row 16 rb + hl, logical chunk q4 of block ks
    const int kr0 = hl, kr1 = 16 + hl;
    const int koff0 = kr0 * 64 + slot(q4, kr0) * 16, koff1 = kr1 * 64 + slot(q4, kr1) * 16;
    // V^T transpose reads: row 4 q4 + hl / 4 (+16), dims 16 cb + 4 (hl & 3) .. +4, i.e.
    // logical chunk 2 (cb & 1) + (hl & 3) / 2 of block cb / 2, bytes 8 (hl & 1)
    const int vr = 4 * q4 + (hl >> 2);
    const int vj = (hl & 3) >> 1;
    const int voffe = vr * 64 + slot(vj, vr) * 16 + 8 * (hl & 1);
    const int voffo = vr * 64 + slot(vj + 2, vr) * 16 + 8 * (hl & 1);

    for (int it = 0; it < ntile; ++it) {
        // this wave's loads of tile `it` have landed once at most (ahead * PER_WAVE) are pending
        wait_tiles<G::PER_WAVE, G::NST - 2>(min(G::NST - 2, ntile - 1 - it));
        __syncthreads();  // every wave's loads of tile `it` landed; tile it-1 no longer read
        if (it + G::NST - 1 < ntile) {
            const int nt = it + G::NST - 1;
            issue_tile(nt, posbuf[nt * kRows + drow], posbuf[nt * kRows + drow + 16]);
        }
        const lds_u8 *kt = (const lds_u8 *)lds + (it % G::NST) * G::STAGE;
        const lds_u8 *vt = MLA ? kt : kt + G::KB * kBlk;
        const uint32_t vm = vmask[it];
        if (16 * wave >= g) continue;  // a wave without query heads only loads tiles

        // ---- S^T tile (32 rows x 16 heads): st[rb][r] = row 16 rb + 4 q4 + r, head hl
        f32x4 st[2] = {f32x4{0.0f, 0.0f, 0.0f, 0.0f}, f32x4{0.0f, 0.0f, 0.0f, 0.0f}};
        {
            const lds_u32x4 *k0 = (const lds_u32x4 *)(kt + koff0);
            const lds_u32x4 *k1 = (const lds_u32x4 *)(kt + koff1);
            u32x4 f0[2], f1[2];
            f0[0] = k0[0];
            f1[0] = k1[0];
#pragma unroll
            for (int ks = 0; ks < KSQ; ++ks) {
                if (ks + 1 < KSQ) {
                    f0[(ks + 1) & 1] = k0[(ks + 1) * (kBlk / 16)];
                    f1[(ks + 1) & 1] = k1[(ks + 1) * (kBlk / 16)];
                }
                st[0] = mfma16(__builtin_bit_cast(bf16x8, f0[ks & 1]), bq[ks], st[0]);
                st[1] = mfma16(__builtin_bit_cast(bf16x8, f1[ks & 1]), bq[ks], st[1]);
            }
        }
        // ---- online softmax (log2 domain), rows of this lane: 16 rb + 4 q4 + r.
        // The reference maximum m_run only moves when the tile maximum exceeds it by more
        // than 8 (probabilities stay <= 2^8), so O is rescaled rarely; o / l and the
        // log-sum-exp do not depend on which reference is used.
        float z[8];
        float mt = kNegInf;
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const bool ok = (vm >> (16 * rb + 4 * q4 + r)) & 1u;
                const float v = ok ? st[rb][r] * sl2 : kNegInf;
                z[4 * rb + r] = v;
                mt = fmaxf(mt, v);
            }
        mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
        mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
        const bool bump = mt > m_run + 8.0f;  // also when m_run is -inf and the tile is not empty
        if (__ballot(bump)) {
            const float m_new = bump ? mt : m_run;
            const float alpha = m_run == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(m_run - m_new);
            // o is still zero for a head that has seen no row yet: only rescale when some
            // head of the wave had a reference before
            if (__ballot(bump && m_run != kNegInf)) {
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb) o[cb] *= alpha;
            }
            l_run *= alpha;
            m_run = m_new;
        }
        const float m_use = m_run == kNegInf ? 0.0f : m_run;
        float p[8];
        float psum = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            p[i] = z[i] == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(z[i] - m_use);
            psum += p[i];
        }
        l_run += psum;
        // P^T as the B operand of O^T = V^T P^T: k index 8 q4 + e <-> row (e < 4 ? 4 q4 + e : 16 + 4 q4 + e - 4)
        typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16v8;
        const bf16v8 pb = {(__bf16)p[0], (__bf16)p[1], (__bf16)p[2], (__bf16)p[3],
                           (__bf16)p[4], (__bf16)p[5], (__bf16)p[6], (__bf16)p[7]};
        const bf16x8 bp = __builtin_bit_cast(bf16x8, pb);
        // ---- O^T += V^T P^T. A operand (dv 16 cb + hl, the same 8 rows) by two LDS
        // transpose reads: lane i of a 16-lane group points at V[row 4 q4 + i/4][dv 4 (i%4)]
        // and receives V[4 q4 .. 4 q4 + 3][dv i] (then rows 16 + 4 q4 ..); 2-deep ring.
        {
            // one base address per parity of cb, opaque to the compiler so that it keeps
            // the per-block constants as instruction offsets (instead of hoisting 32
            // precomputed addresses and adding the stage base to each)
            uint32_t ea = (uint32_t)(uintptr_t)(vt + voffe), oa = (uint32_t)(uintptr_t)(vt + voffo);
            asm volatile("" : "+v"(ea), "+v"(oa));
            const lds_s16x4 *ve = (const lds_s16x4 *)(uintptr_t)ea;
            const lds_s16x4 *vo = (const lds_s16x4 *)(uintptr_t)oa;
            auto vread = [&](int cb, int half) -> s16x4 {  // rows +16 * half: 1024 bytes on
                const lds_s16x4 *bse = (cb & 1) ? vo : ve;
                return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    const_cast<lds_s16x4 *>(bse + ((cb >> 1) * kBlk + 1024 * half) / 8));
            };
            s16x4 x0[2], x1[2];
            x0[0] = vread(0, 0);
            x1[0] = vread(0, 1);
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                if (cb + 1 < NCB) {
                    x0[(cb + 1) & 1] = vread(cb + 1, 0);
                    x1[(cb + 1) & 1] = vread(cb + 1, 1);
                }
                const s16x8 av = __builtin_shufflevector(x0[cb & 1], x1[cb & 1], 0, 1, 2, 3, 4, 5, 6, 7);
                o[cb] = mfma16(__builtin_bit_cast(bf16x8, av), bp, o[cb]);
            }
        }
    }

    // ---- finish: the 4 lane groups hold disjoint rows of the same head
    float l_tot = l_run + __shfl_xor(l_run, 16, 64);
    l_tot += __shfl_xor(l_tot, 32, 64);
    const int64_t ohead = (((int64_t)b * T + t) * Hq + hq);
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    if (OUTF32 && nsplit == 1) {
        if (hvalid) {
            float *out = reinterpret_cast<float *>(a.out) + layer * a.lso + ohead * DV + 4 * q4;
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) *reinterpret_cast<f32x4 *>(out + 16 * cb) = o[cb] * inv;
            if (a.lse && lane < 16)
                a.lse[layer * a.lsl + ohead] = l_tot > 0.0f ? (m_run + __builtin_log2f(l_tot)) * kLn2 : kNegInf;
        }
        if constexpr (FUSED) sel::release_slice<NT>(f.w, (int)selrow, nslices, slice);
        return;
    }
    // bf16 rows o / l (the output, or a split's normalised partial) staged per wave in
    // LDS (the tile ring is free once every wave is done), then written one whole row
    // (DV values) per store instruction.
    constexpr int RB = DV * 2;             // bytes per bf16 row
    constexpr int RS = RB + 16;            // LDS row stride (padding: conflict-free staging)
    constexpr int LPR = RB / 16;           // lanes per row when storing 16 bytes each
    constexpr int HPI = 64 / LPR;          // rows (heads) per store instruction
    static_assert(HW * 16 * RS <= G::NST * G::STAGE, "staging fits the ring");
    __syncthreads();
    lds_u8 *wst = (lds_u8 *)lds + wave * 16 * RS;
    if (hvalid) {
        typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16v4;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
            const bf16v4 w4 = {(__bf16)(o[cb][0] * inv), (__bf16)(o[cb][1] * inv), (__bf16)(o[cb][2] * inv),
                               (__bf16)(o[cb][3] * inv)};
            *(__attribute__((address_space(3))) bf16v4 *)(wst + hl * RS + 2 * (16 * cb + 4 * q4)) = w4;
        }
    }
    const int64_t pbase = (int64_t)layer * B * T * Hq;  // heads before this layer
    // the wave's LDS writes precede its reads (in-order LDS per wave)
#pragma unroll
    for (int h0 = 0; h0 < 16; h0 += HPI) {
        const int h = h0 + lane / LPR;
        if (16 * wave + h >= g) continue;
        const int64_t oh = ((int64_t)b * T + t) * Hq + kvh * g + 16 * wave + h;
        const u32x4 v = *(const lds_u32x4 *)(wst + h * RS + 16 * (lane % LPR));
        uint16_t *row = nsplit == 1 ? reinterpret_cast<uint16_t *>(a.out) + layer * a.lso + oh * DV
                                    : reinterpret_cast<uint16_t *>(po) + ((pbase + oh) * nsplit + split) * DV;
        *reinterpret_cast<u32x4 *>(row + 8 * (lane % LPR)) = v;
    }
    if (hvalid && lane < 16) {
        if (nsplit == 1) {
            if (a.lse) a.lse[layer * a.lsl + ohead] = l_tot > 0.0f ? (m_run + __builtin_log2f(l_tot)) * kLn2 : kNegInf;
        } else {
            const int64_t pidx = (pbase + ohead) * nsplit + split;
            pml[2 * pidx] = m_run;
            pml[2 * pidx + 1] = l_tot;
        }
    }
    if constexpr (FUSED) sel::release_slice<NT>(f.w, (int)selrow, nslices, slice);
}

// ----------------------------------------------------------------------------- MLA, 32 heads
// MLA latent rows (576 wide, V = the first 512 columns) with a multiple of 32 query heads
// per KV head. One workgroup = (layer, sequence, query token, KV head, 32-head block, split
// of the selected rows), 4 waves, rounds of 128 selected rows:
//   - wave w gathers tile w of the round (32 rows, 36 KB) into its own LDS slot (the same
//     block layout and DMA as above; each wave waits for its own loads only) and computes
//     S^T = K Q^T for its 32 rows and the block's 32 heads on v_mfma_f32_32x32x16_bf16,
//     with the 32 heads' Q held in registers;
//   - the waves agree on each head's reference maximum through LDS and write their
//     probabilities (bf16, in the B-operand layout of the value product) to LDS;
//   - wave w accumulates O^T for value columns 128 w .. 128 w + 127 over the round's four
//     tiles, V^T by LDS transpose reads.
// Every K and V byte in LDS is read once per 32 heads (twice as few reads as the 16-head
// layout above), and a split covers 128 rows, so the split partials of the 128K decode are
// half as many.
constexpr int kMRound = 128;   // selected rows per round (4 waves x 32)
constexpr int kMMaxPos = 1024; // rows per split held in the LDS position list (fused resolve)
constexpr int kMKB = 18;       // 64-byte blocks per 576-wide row
constexpr int kMStage = kMKB * kBlk;
constexpr int kMLdsFixed = 4 * kMStage + 8192 + 1024;  // slots, probabilities, maxima and sums
static_assert(32 * 576 * 2 == kMKB * kBlk && 4 * (kMKB / 2) * 1024 == kMKB * kBlk, "Q of 32 heads fills one slot");

template <bool OUTF32, bool FUSED>
__global__ __launch_bounds__(256) void attend_mla_kernel(AttendArgs a, uint16_t *po, float *pml, int R, int HB,
                                                         FuseArgs f) {
    constexpr int NT = 256, KS = 36, DV = 512;
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    u32x4 *pbuf = reinterpret_cast<u32x4 *>(lds + 4 * kMStage);     // [4 tiles][2 K-blocks][64 lanes]
    float *mx = reinterpret_cast<float *>(lds + 4 * kMStage + 8192);  // [4][32] tile maxima
    float *lsm = mx + 128;                                            // [4][32] row sums
    int *posbuf = reinterpret_cast<int *>(lds + kMLdsFixed);         // [R] (FUSED)

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n32 = lane & 31, g = lane >> 5;
    const int T = a.T, Hq = a.Hq, Hkv = a.Hkv, K = a.K;
    const int nsplit = gridDim.x / HB;
    const int split = blockIdx.x % nsplit, hb = blockIdx.x / nsplit;
    const int t = blockIdx.y / Hkv, kvh = blockIdx.y % Hkv;
    const int layer = blockIdx.z / a.B, b = blockIdx.z % a.B;
    const int gq = Hq / Hkv;
    const int hq = kvh * gq + 32 * hb + n32;  // this lane's query head
    const int r0 = split * R;
    const int nrows = max(0, min(K, r0 + R) - r0);
    const int ntile = (nrows + 31) / 32;
    const int nround = (ntile + 3) / 4;
    const int64_t selrow = (int64_t)b * T + t;
    const int64_t bofs = a.bt ? 0 : b * a.ksb;
    auto phys = [&](int s) -> int {  // cache row of position s, -1 if its page is unmapped
        if (!a.bt) return s;
        const int pg = s / a.page_size;
        if (pg >= a.max_pages) return -1;
        const int pp = a.bt[(int64_t)b * a.max_pages + pg];
        return (pp >= 0 && pp < a.num_pages) ? pp * a.page_size + (s - pg * a.page_size) : -1;
    };
    bf16x8 bq[KS];  // B operand of S^T: head n32, dims 16 ks + 8 g .. +8
    // The block's Q (32 rows of 1152 bytes, contiguous: 36 KB, one slot) is copied into
    // slot 3 once per workgroup by DMA (while the fused selection runs in slots 0-2), and
    // every wave takes its fragments from there: each wave loading all of Q from memory had
    // made the workgroup take in 144 KB of Q beside its 147 KB of rows
    // In the slot, row n's 16-byte chunk c sits at chunk c ^ ((n >> 1) & 7) of the row (the
    // XOR stays inside aligned groups of 8 of its 72 chunks), so that the 16 lanes of a
    // fragment read (rows n32 .. n32 + 15, one chunk each) hit 16 distinct bank groups:
    // unswizzled, the 1152-byte row stride put them on two. The permutation is applied
    // on the global side of the DMA (each lane's LDS destination is fixed).
    lds_u8 *qslot = (lds_u8 *)lds + 3 * kMStage;
    auto dma_q = [&]() __attribute__((always_inline)) {
        const unsigned char *qsrc =
            reinterpret_cast<const unsigned char *>(a.q + layer * a.lsq + (selrow * Hq + kvh * gq + 32 * hb) * 576);
#pragma unroll
        for (int j = 0; j < kMKB / 2; ++j) {  // 1 KB pieces wave * 9 + j of 36
            const int n = wave * (kMKB / 2) + j;
            const int L = 64 * n + lane, row = L / 72, pc = L % 72;  // LDS chunk L: row, physical chunk
            __builtin_amdgcn_global_load_lds((const glb_void_t *)(qsrc + 1152 * row + 16 * (pc ^ ((row >> 1) & 7))),
                                             (lds_void_t *)(qslot + 1024 * n), 16, 0, 0);
        }
    };
    auto lds_q = [&]() __attribute__((always_inline)) {
        // fragment ks: logical chunk 2 ks + g = 8 (ks / 4) + 2 (ks % 4) + g of row n32
        const int sw = (n32 >> 1) & 7;
        const lds_u8 *qp = qslot + n32 * 1152;
        int qo[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) qo[k] = 16 * ((2 * k + g) ^ sw);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            bq[ks] = __builtin_bit_cast(bf16x8, *(const lds_u32x4 *)(qp + 128 * (ks / 4) + qo[ks % 4]));
    };
    const int nslices = nsplit * HB * Hkv * a.L;
    const int slice = split + nsplit * (hb + HB * (kvh + Hkv * layer));
    if constexpr (FUSED) {
        sel::SliceLds S;
        unsigned char *p = lds;
        S.ties = reinterpret_cast<uint64_t *>(p);
        p += (size_t)f.tl * 8;
        S.h = reinterpret_cast<uint32_t *>(p);
        p += sel::kB2 * 4;
        S.h256 = reinterpret_cast<uint32_t *>(p);
        p += 256 * 4;
        S.scr = reinterpret_cast<uint32_t *>(p);
        p += 32 * 4;
        S.bits = reinterpret_cast<uint32_t *>(p);
        S.tl = f.tl;
        S.pw_log = f.pw_log;
        S.bits_lds = f.bits_lds != 0;
        // Q's DMA is issued once the selection's first loads are (its latency then hides
        // under the selection's later phases, and the selection's first wait does not cover
        // it); the selection's working set stays in slots 0-2
        sel::resolve_slice<NT>(f.sa, f.w, (int)selrow, r0, r0 + nrows, S, posbuf,
                               [&]() __attribute__((always_inline)) { dma_q(); });  // ends with a barrier
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's share of Q landed
        if (kvh == 0 && layer == 0 && hb == 0) {
            int32_t *dst = f.sa.idx + selrow * K + r0;
            for (int i = tid; i < nrows; i += NT) dst[i] = posbuf[i];
        }
        if (a.bt) {  // positions -> cache rows (or -1), each thread its own entries
            for (int i = tid; i < nrows; i += NT) {
                const int ps = posbuf[i];
                posbuf[i] = (ps >= 0 && ps < a.N) ? phys(ps) : -1;
            }
        }
        __syncthreads();  // the working set (slots 0-2) is free, the list complete, Q in slot 3
        lds_q();
        __syncthreads();  // slot 3 read by every wave (wave 3's tile goes there)
    }
    const int32_t *idxrow = FUSED ? nullptr : a.idx + (a.idx_shared ? (int64_t)b : selrow) * K + r0;
    const int pmax = a.idx_shared ? (a.ctx_len ? a.ctx_len[b] : a.N) - T + t : 0x7FFFFFFF;
    const uint16_t *kbase = a.k + layer * a.lsk + bofs + kvh * a.ksh;
    auto rowpos = [&](int i) {  // (fused resolve) cache row of selected row i of the split, -1 if none
        const int s = i < nrows ? posbuf[i] : -1;
        return (s >= 0 && (a.bt || s < a.N)) ? s : -1;
    };
    // ---- DMA of tile j into this wave's slot: instruction n fills block n / 2 for rows
    // 16 (n & 1) .. +15; lane l writes row 16 (n & 1) + l / 4, physical chunk l & 3
    const int drow = lane >> 2;
    const int dchk0 = slot(lane & 3, drow), dchk1 = slot(lane & 3, drow + 16);
    lds_u8 *myslot = (lds_u8 *)lds + wave * kMStage;
    auto issue = [&](int p0, int p1) {  // positions (>= 0) of rows drow, drow + 16
        const uint16_t *s0 = kbase + (int64_t)p0 * a.ksn, *s1 = kbase + (int64_t)p1 * a.ksn;
#pragma unroll
        for (int n = 0; n < 2 * kMKB; ++n) {
            const int blk = n >> 1, hi = n & 1;
            const uint16_t *src = (hi ? s1 : s0) + 8 * (4 * blk + (hi ? dchk1 : dchk0));
            __builtin_amdgcn_global_load_lds((const glb_void_t *)src, (lds_void_t *)(myslot + blk * kBlk + 1024 * hi),
                                             16, 0, 0);
        }
    };
    // rows of this wave's tile in round rd: positions of rows drow, drow + 16, and the mask
    // of valid rows (bit r: row r)
    auto tile_rows = [&](int rd, int &p0, int &p1) {
        const int j = 4 * rd + wave;
        if constexpr (FUSED) {
            p0 = j < ntile ? rowpos(32 * j + drow) : -1;
            p1 = j < ntile ? rowpos(32 * j + drow + 16) : -1;
        } else {
            // both entries requested together (clamped indices, unconditional loads), then
            // checked and, paged, mapped to cache rows by a second pair of loads
            p0 = p1 = -1;
            if (nrows > 0) {
                const int i0 = 32 * j + drow, i1 = i0 + 16;
                const int v0 = idxrow[min(i0, nrows - 1)], v1 = idxrow[min(i1, nrows - 1)];
                p0 = i0 < nrows ? v0 : -1;
                p1 = i1 < nrows ? v1 : -1;
            }
            auto check = [&](int ps) { return (ps >= 0 && ps < a.N && ps <= pmax) ? ps : -1; };
            p0 = check(p0);
            p1 = check(p1);
            if (a.bt) {
                auto page = [&](int ps) { return ps >= 0 ? min(ps / a.page_size, a.max_pages - 1) : 0; };
                auto row = [&](int ps, int pp) -> int {
                    if (ps < 0 || ps / a.page_size >= a.max_pages || pp < 0 || pp >= a.num_pages) return -1;
                    return pp * a.page_size + ps % a.page_size;
                };
                const int32_t *btrow = a.bt + (int64_t)b * a.max_pages;
                const int pp0 = btrow[page(p0)], pp1 = btrow[page(p1)];
                p0 = row(p0, pp0);
                p1 = row(p1, pp1);
            }
        }
    };
    auto tile_mask = [&](int p0, int p1) -> uint32_t {
        const int a0 = __shfl(p0, 4 * (lane & 15), 64), a1 = __shfl(p1, 4 * (lane & 15), 64);
        const bool ok = lane < 32 && (lane < 16 ? a0 : a1) >= 0;
        return (uint32_t)__ballot(ok);
    };
    // the positions first; without the fused resolve, Q then goes into slot 3 by DMA (once
    // per workgroup) while waves 0-2 already request their tiles; once every wave has taken
    // its Q fragments from slot 3, wave 3 requests its tile there
    int cp0, cp1;
    tile_rows(0, cp0, cp1);
    if constexpr (FUSED) {
        if (wave < ntile) issue(max(cp0, 0), max(cp1, 0));
    } else {
        dma_q();
        const bool early = wave < 3 && wave < ntile;
        if (early) {
            issue(max(cp0, 0), max(cp1, 0));
            wait_vmcnt<2 * kMKB>();  // this wave's share of Q landed (its tile may not have)
        } else {
            wait_vmcnt<0>();
        }
        __syncthreads();  // Q in slot 3
        lds_q();
        __syncthreads();  // slot 3 read by every wave
        if (wave == 3 && wave < ntile) issue(max(cp0, 0), max(cp1, 0));
    }
    uint32_t vm = tile_mask(cp0, cp1);

    f32x16 o[4];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[db][e] = 0.0f;
    float m_run = kNegInf, l_run = 0.0f;
    const float sl2 = a.scale * kLog2e;
    // K fragment (A operand of S^T): row n32, dims 16 ks + 8 g .. +8 = block ks / 2,
    // logical chunk 2 (ks & 1) + g
    const int koff0 = n32 * 64 + slot(g, n32) * 16, koff1 = n32 * 64 + slot(2 + g, n32) * 16;
    // V^T transpose reads (A operand of O^T): 16-lane group c = lane / 16 reads rows
    // 16 kb + 8 h + 4 g .. +3 and value columns 32 db + 16 (c & 1) .. +15: lane i of the
    // group points at row +i/4, columns +4 (i & 3) (chunk 2 (c & 1) + (i & 3) / 2, bytes
    // 8 (i & 1)) and receives the column 32 db + (lane & 31) of the four rows
    const int vi = lane & 15, vc = (lane >> 4) & 1;
    const int vchunk = 2 * vc + ((vi & 3) >> 1);
    int voff[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int row = 16 * kb + 8 * h + 4 * g + (vi >> 2);
            voff[kb][h] = row * 64 + slot(vchunk, row) * 16 + 8 * (vi & 1);
        }

    for (int rd = 0; rd < nround; ++rd) {
        const int j = 4 * rd + wave;
        const bool have = j < ntile;
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's tile (and Q) landed
        int np0 = -1, np1 = -1;
        if (rd + 1 < nround) tile_rows(rd + 1, np0, np1);
        // ---- S^T for this wave's tile: st[e] = row 8 (e / 4) + 4 g + (e & 3), head n32
        float z[16];
        float mt = kNegInf;
        if (have) {
            f32x16 st;
#pragma unroll
            for (int e = 0; e < 16; ++e) st[e] = 0.0f;
            const lds_u32x4 *k0 = (const lds_u32x4 *)(myslot + koff0);
            const lds_u32x4 *k1 = (const lds_u32x4 *)(myslot + koff1);
            auto kload = [&](int ks) { return (ks & 1) ? k1[(ks >> 1) * (kBlk / 16)] : k0[(ks >> 1) * (kBlk / 16)]; };
            // K fragments four steps ahead, two accumulator chains (even and odd steps), so
            // neither the LDS latency nor the accumulation dependency stalls each step
            constexpr int PF = 4;
            u32x4 kf[PF];
#pragma unroll
            for (int i = 0; i < PF; ++i) kf[i] = kload(i);
            f32x16 st1;
#pragma unroll
            for (int e = 0; e < 16; ++e) st1[e] = 0.0f;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf16x8 ka = __builtin_bit_cast(bf16x8, kf[ks % PF]);
                if (ks + PF < KS) kf[ks % PF] = kload(ks + PF);
                if (ks & 1) st1 = mfma32(ka, bq[ks], st1);
                else st = mfma32(ka, bq[ks], st);
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int e = 0; e < 16; ++e) st[e] += st1[e];
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int row = 8 * (e >> 2) + 4 * g + (e & 3);
                const float v = ((vm >> row) & 1u) ? st[e] * sl2 : kNegInf;
                z[e] = v;
                mt = fmaxf(mt, v);
            }
            mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
        }
        if (lane < 32) mx[wave * 32 + n32] = mt;
        __syncthreads();
        // ---- the round's reference: every wave takes the same decisions from the same maxima
        const float mr = fmaxf(fmaxf(mx[n32], mx[32 + n32]), fmaxf(mx[64 + n32], mx[96 + n32]));
        const bool bump = mr > m_run + 8.0f;  // also when m_run is -inf and the round is not empty
        if (__ballot(bump)) {
            const float m_new = bump ? mr : m_run;
            const float alpha = m_run == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(m_run - m_new);
            if (__ballot(bump && m_run != kNegInf)) {
#pragma unroll
                for (int db = 0; db < 4; ++db) o[db] *= alpha;
            }
            l_run *= alpha;
            m_run = m_new;
        }
        if (have) {
            const float m_use = m_run == kNegInf ? 0.0f : m_run;
            float p[16];
            float psum = 0.0f;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                p[e] = z[e] == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(z[e] - m_use);
                psum += p[e];
            }
            l_run += psum;
            // P^T (B operand of O^T, K-block kb): k slot e of lane group g <-> row
            // 16 kb + 8 (e / 4) + 4 g + (e & 3), i.e. this lane's own p[8 kb + e]
            typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16v8;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const bf16v8 pb = {(__bf16)p[8 * kb], (__bf16)p[8 * kb + 1], (__bf16)p[8 * kb + 2], (__bf16)p[8 * kb + 3],
                                   (__bf16)p[8 * kb + 4], (__bf16)p[8 * kb + 5], (__bf16)p[8 * kb + 6], (__bf16)p[8 * kb + 7]};
                pbuf[(wave * 2 + kb) * 64 + lane] = __builtin_bit_cast(u32x4, pb);
            }
        }
        __syncthreads();
        // ---- O^T += V^T P^T over the round's tiles, value columns 128 wave .. +127
        // batches (tile jj, K-block kb) in order; the next batch's LDS reads are issued
        // before the current batch's products (two register sets)
        const int nb = 2 * min(4, ntile - 4 * rd);
        struct VB {
            s16x4 x[4][2];
            bf16x8 bp;
        };
        auto vload = [&](int i, VB &v) __attribute__((always_inline)) {
            const int jj = i >> 1, kb = i & 1;
            const lds_u8 *vt = (const lds_u8 *)lds + jj * kMStage + 4 * wave * kBlk;
            v.bp = __builtin_bit_cast(bf16x8, pbuf[i * 64 + lane]);
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    v.x[db][h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        const_cast<lds_s16x4 *>((const lds_s16x4 *)(vt + db * kBlk + (kb ? voff[1][h] : voff[0][h]))));
        };
        auto vmma = [&](const VB &v) __attribute__((always_inline)) {
#pragma unroll
            for (int db = 0; db < 4; ++db) {
                const s16x8 av = __builtin_shufflevector(v.x[db][0], v.x[db][1], 0, 1, 2, 3, 4, 5, 6, 7);
                o[db] = mfma32(__builtin_bit_cast(bf16x8, av), v.bp, o[db]);
            }
        };
        VB va, vb;
        vload(0, va);
        if (nb == 8) {  // a full round, straight-line (exact LDS wait counts)
#pragma unroll
            for (int i = 0; i < 8; i += 2) {
                vload(i + 1, vb);
                __builtin_amdgcn_sched_barrier(0);
                vmma(va);
                __builtin_amdgcn_sched_barrier(0);
                if (i + 2 < 8) vload(i + 2, va);
                __builtin_amdgcn_sched_barrier(0);
                vmma(vb);
                __builtin_amdgcn_sched_barrier(0);
            }
        } else
        for (int i = 0; i < nb; i += 2) {
            if (i + 1 < nb) vload(i + 1, vb);
            __builtin_amdgcn_sched_barrier(0);  // the next batch's reads stay ahead of these products
            vmma(va);
            __builtin_amdgcn_sched_barrier(0);
            if (i + 1 < nb) {
                if (i + 2 < nb) vload(i + 2, va);
                __builtin_amdgcn_sched_barrier(0);
                vmma(vb);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        if (rd + 1 < nround) {
            __syncthreads();  // every wave is done with the slots, maxima and probabilities
            if (4 * (rd + 1) + wave < ntile) issue(max(np0, 0), max(np1, 0));
            vm = tile_mask(np0, np1);
        }
    }

    // ---- finish: row sums over the lane pair and the four waves (fixed order)
    const float lw = l_run + __shfl_xor(l_run, 32, 64);
    if (lane < 32) lsm[wave * 32 + n32] = lw;
    __syncthreads();  // also: every wave is done with the slots (staging below)
    const float l_tot = ((lsm[n32] + lsm[32 + n32]) + lsm[64 + n32]) + lsm[96 + n32];
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    const int64_t pbase = (int64_t)layer * a.B * T * Hq;  // heads before this layer
    const int64_t ohead = selrow * Hq + hq;
    // O^T value (column 32 db' + 8 (e / 4) + 4 g + (e & 3) of this wave's 128, head n32),
    // staged per wave in LDS as rows of the 32 heads, then written in 16-byte pieces
    if (OUTF32 && nsplit == 1) {
        constexpr int RS = 512 + 16;  // bytes per staged row (128 fp32 + padding)
        lds_u8 *wst = (lds_u8 *)lds + wave * 32 * RS;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                *(__attribute__((address_space(3))) f32x4 *)(wst + n32 * RS + 4 * (32 * db + 8 * q + 4 * g)) =
                    f32x4{o[db][4 * q] * inv, o[db][4 * q + 1] * inv, o[db][4 * q + 2] * inv, o[db][4 * q + 3] * inv};
        asm volatile("" ::: "memory");  // the wave's staging writes before its reads
#pragma unroll
        for (int it = 0; it < 16; ++it) {
            const int h = 2 * it + (lane >> 5);
            const u32x4 v = *(const lds_u32x4 *)(wst + h * RS + 16 * (lane & 31));
            const int64_t oh = selrow * Hq + kvh * gq + 32 * hb + h;
            float *row = reinterpret_cast<float *>(a.out) + layer * a.lso + oh * DV + 128 * wave;
            *reinterpret_cast<u32x4 *>(row + 4 * (lane & 31)) = v;
        }
    } else {
        constexpr int RS = 256 + 16;  // bytes per staged row (128 bf16 + padding)
        lds_u8 *wst = (lds_u8 *)lds + wave * 32 * RS;
        typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16v4;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const bf16v4 w4 = {(__bf16)(o[db][4 * q] * inv), (__bf16)(o[db][4 * q + 1] * inv),
                                   (__bf16)(o[db][4 * q + 2] * inv), (__bf16)(o[db][4 * q + 3] * inv)};
                *(__attribute__((address_space(3))) bf16v4 *)(wst + n32 * RS + 2 * (32 * db + 8 * q + 4 * g)) = w4;
            }
        asm volatile("" ::: "memory");  // the wave's staging writes before its reads
#pragma unroll
        for (int it = 0; it < 8; ++it) {
            const int h = 4 * it + (lane >> 4);
            const u32x4 v = *(const lds_u32x4 *)(wst + h * RS + 16 * (lane & 15));
            const int64_t oh = selrow * Hq + kvh * gq + 32 * hb + h;
            uint16_t *row = nsplit == 1 ? reinterpret_cast<uint16_t *>(a.out) + layer * a.lso + oh * DV
                                        : po + ((pbase + oh) * nsplit + split) * DV;
            *reinterpret_cast<u32x4 *>(row + 128 * wave + 8 * (lane & 15)) = v;
        }
    }
    if (wave == 0 && lane < 32) {
        if (nsplit == 1) {
            if (a.lse) a.lse[layer * a.lsl + ohead] = l_tot > 0.0f ? (m_run + __builtin_log2f(l_tot)) * kLn2 : kNegInf;
        } else {
            const int64_t pidx = (pbase + ohead) * nsplit + split;
            pml[2 * pidx] = m_run;
            pml[2 * pidx + 1] = l_tot;
        }
    }
    if constexpr (FUSED) sel::release_slice<NT>(f.w, (int)selrow, nslices, slice);
}

// Merge the split partials of HPW heads of one (layer, b, t). Wave h < HPW turns head h's
// (m, l) pairs into weights l 2^(m - M) (M = the largest m) for the normalised rows. A
// head's DV values are split into 8-value chunks, one lane each, and its splits into SG
// groups (split s to group s % SG): every thread has its group's loads in flight at once
// and sums them in split order, then the group-0 thread of each chunk adds the SG partial
// sums in group order (a fixed order: the same bits every run).
constexpr int kCombT = 256;
constexpr int kMaxSplits = kAttendMaxSplits;

template <int DV, int HPW, bool OUTF32>
__global__ __launch_bounds__(kCombT) void attend_combine_kernel(AttendArgs a, const uint16_t *po, const float *pml, int S) {
    constexpr int LPR = DV / 8;                 // lanes per row (8 values each)
    constexpr int SG = kCombT / (HPW * LPR);    // split groups per head
    static_assert(SG >= 1 && HPW * SG * LPR == kCombT && HPW <= 4, "thread layout");
    static_assert(kMaxSplits <= 128, "two (m, l) pairs per lane");
    constexpr int PER = (kMaxSplits + SG - 1) / SG;  // splits per group at most
    __shared__ float wgt[HPW][kMaxSplits];
    __shared__ float linv[HPW];
    __shared__ __attribute__((aligned(16))) float part[HPW][SG][DV];
    const int bt = blockIdx.y, layer = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t hbase = (int64_t)layer * a.B * a.T * a.Hq + (int64_t)bt * a.Hq;  // partial heads of (layer, b, t)
    // The weights' inputs come first: wave w < HPW loads the (m, l) pairs of head w of the
    // workgroup (two per lane at most). Then every thread requests its first round of
    // partial rows, and only then are the weights formed, so that their wait does not
    // cover the rows (the counter retires in order) and the rows' latency overlaps it.
    const int hw = blockIdx.x * HPW + wave;
    const bool wwave = wave < HPW && hw < a.Hq;  // uniform per wave
    float2 ml0 = {kNegInf, 0.0f}, ml1 = {kNegInf, 0.0f};
    if (wwave) {
        const float2 *ml = reinterpret_cast<const float2 *>(pml + (hbase + hw) * S * 2);
        if (lane < S) ml0 = ml[lane];
        if (lane + 64 < S) ml1 = ml[lane + 64];
    }
    auto form_weights = [&]() __attribute__((always_inline)) {
        if (!wwave) return;
        float M = fmaxf(ml0.x, ml1.x);
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
        auto weight = [&](float2 v) { return (M == kNegInf || v.x == kNegInf) ? 0.0f : __builtin_amdgcn_exp2f(v.x - M) * v.y; };
        const float w0 = weight(ml0), w1 = weight(ml1);
        if (lane < S) wgt[wave][lane] = w0;
        if (lane + 64 < S) wgt[wave][lane + 64] = w1;
        float L = w0 + w1;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) L += __shfl_xor(L, o, 64);  // the same tree every run
        if (lane == 0) {
            linv[wave] = L > 0.0f ? 1.0f / L : 0.0f;
            if (a.lse) a.lse[layer * a.lsl + (int64_t)bt * a.Hq + hw] = L > 0.0f ? (M + __builtin_log2f(L)) * kLn2 : kNegInf;
        }
    };
    // ---- this thread's splits (group sg) of chunk c of head hl, all loads in flight
    const int hl = tid / (SG * LPR), sg = (tid / LPR) % SG, c = tid % LPR;
    const int hq = blockIdx.x * HPW + hl;
    const bool live = hq < a.Hq;
    const u32x4 *src = reinterpret_cast<const u32x4 *>(po + (hbase + (live ? hq : 0)) * S * DV) + c;
    constexpr int RU = DV / 8;  // u32x4 per row
    // rounds of up to 8 of the group's splits in flight (one round for the default splits)
    constexpr int U = PER < 8 ? PER : 8;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
    for (int base = 0; base < PER; base += U) {
        u32x4 v[U];
        // unconditional loads (a split past S reads the last one and is not accumulated), so
        // every path issues the same loads and the waits below can count them
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int sp = sg + (base + u) * SG;
            v[u] = src[(int64_t)min(sp, S - 1) * RU];
        }
        if (base == 0) {  // (uniform: every thread runs round 0)
            form_weights();
            __syncthreads();  // the weights
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int sp = sg + (base + u) * SG;
            if (live && sp < S) {
                const float w = wgt[hl][sp];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    acc[2 * q] += w * bf16lo(v[u][q]);
                    acc[2 * q + 1] += w * bf16hi(v[u][q]);
                }
            }
        }
        if (sg + (base + U) * SG >= S) break;  // uniform per group; no barrier follows in the loop
    }
    *reinterpret_cast<f32x4 *>(&part[hl][sg][8 * c]) = f32x4{acc[0], acc[1], acc[2], acc[3]};
    *reinterpret_cast<f32x4 *>(&part[hl][sg][8 * c + 4]) = f32x4{acc[4], acc[5], acc[6], acc[7]};
    __syncthreads();
    if (sg != 0 || !live) return;
    float r[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = 0.0f;
    for (int g = 0; g < SG; ++g) {
        const f32x4 x0 = *reinterpret_cast<const f32x4 *>(&part[hl][g][8 * c]);
        const f32x4 x1 = *reinterpret_cast<const f32x4 *>(&part[hl][g][8 * c + 4]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            r[e] += x0[e];
            r[4 + e] += x1[e];
        }
    }
    const float inv = linv[hl];
    const int64_t ob = layer * a.lso + ((int64_t)bt * a.Hq + hq) * DV + 8 * c;
    if constexpr (OUTF32) {
        float *out = reinterpret_cast<float *>(a.out) + ob;
        *reinterpret_cast<f32x4 *>(out) = f32x4{r[0] * inv, r[1] * inv, r[2] * inv, r[3] * inv};
        *reinterpret_cast<f32x4 *>(out + 4) = f32x4{r[4] * inv, r[5] * inv, r[6] * inv, r[7] * inv};
    } else {
        typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16v8;
        const bf16v8 w8 = {(__bf16)(r[0] * inv), (__bf16)(r[1] * inv), (__bf16)(r[2] * inv), (__bf16)(r[3] * inv),
                           (__bf16)(r[4] * inv), (__bf16)(r[5] * inv), (__bf16)(r[6] * inv), (__bf16)(r[7] * inv)};
        *reinterpret_cast<bf16v8 *>(reinterpret_cast<uint16_t *>(a.out) + ob) = w8;
    }
}

// Measurement hook (lsa_attend_launch_events): the next attention call on this host thread
// records its start from the dispatch of its first kernel and its end from that of its
// last one (the merge, or the attention itself with one split).
thread_local hipEvent_t t_att_start = nullptr, t_att_stop = nullptr;

#define LSA_LAUNCH_ATT(LAST, K, GRID, BLOCK, LDS, S, ...)                                                   \
    do {                                                                                                     \
        if (t_att_start || t_att_stop) {                                                                     \
            hipEvent_t e0_ = t_att_start, e1_ = (LAST) ? t_att_stop : nullptr;                               \
            t_att_start = nullptr;                                                                           \
            if (LAST) t_att_stop = nullptr;                                                                  \
            hipExtLaunchKernelGGL(K, GRID, BLOCK, (uint32_t)(LDS), S, e0_, e1_, 0, __VA_ARGS__);             \
        } else {                                                                                             \
            hipLaunchKernelGGL(K, GRID, BLOCK, LDS, S, __VA_ARGS__);                                         \
        }                                                                                                    \
    } while (0)

// The merge launch: one head a workgroup for 128-wide rows (16 split groups), two for
// 512-wide rows (2 split groups each).
#ifndef LSA_COMBINE_HEADS_512
#define LSA_COMBINE_HEADS_512 2
#endif
template <int DV, bool OUTF32>
hipError_t launch_combine(const AttendArgs &a, const uint16_t *po, const float *pml, int S, hipStream_t s) {
    constexpr int HPW = DV >= 512 ? LSA_COMBINE_HEADS_512 : 1;
    dim3 cgrid((a.Hq + HPW - 1) / HPW, a.B * a.T, a.L);
    LSA_LAUNCH_ATT(true, (attend_combine_kernel<DV, HPW, OUTF32>), cgrid, dim3(kCombT), 0, s, a, po, pml, S);
    return hipGetLastError();
}

int rows_per_split(const AttendArgs &a) {
    int R = (a.K + a.n_splits - 1) / a.n_splits;
    return (R + kRows - 1) / kRows * kRows;
}

// Split partials in the workspace: bf16 rows [L][B][T][Hq][S][DV], then fp32 (m, l)
// [L][B][T][Hq][S][2].
size_t partial_rows_bytes(const AttendArgs &a, int S) {
    return ((size_t)a.L * a.B * a.T * a.Hq * S * a.d_v * 2 + 255) & ~(size_t)255;
}

template <int DQK, int DV, int HW, bool MLA, bool OUTF32, int NSTC = 4>
hipError_t launch_t(const AttendArgs &a, void *ws, hipStream_t s, const FuseArgs *fuse) {
    const int R = rows_per_split(a);
    const int S = (a.K + R - 1) / R;
    uint16_t *po = reinterpret_cast<uint16_t *>(ws);
    float *pml = S > 1 ? reinterpret_cast<float *>(reinterpret_cast<char *>(ws) + partial_rows_bytes(a, S)) : nullptr;
    dim3 grid(S, a.T * a.Hkv, a.B * a.L);
    using G = AttTile<DQK, DV, HW, MLA, OUTF32, NSTC>;
    // the ring, then the split's position list and row masks (sized by the split, so that
    // short splits leave room for more workgroups per compute unit)
    const size_t lds = (size_t)G::NST * G::STAGE + (size_t)R * sizeof(int) + (size_t)(R / 32) * sizeof(uint32_t);
    if (fuse) {
        // (the chain runs only with four waves of heads and the 4-stage ring:
        // launch_select_attend decides)
        if constexpr (HW != 4 || NSTC != 4) {
            return hipErrorInvalidValue;
        } else {
            // the resolve's working set in the tile ring: histograms and scratch, the row
            // bitmap when it fits beside the first tie entries, the rest for ties
            FuseArgs f = *fuse;
            constexpr size_t ring = (size_t)G::NST * G::STAGE;
            constexpr size_t fixed = sel::kB2 * 4 + 256 * 4 + 32 * 4;
            f.pw_log = sel::slice_pw_log(f.w.words, G::NT);
            const size_t bb = ((size_t)G::NT << f.pw_log) * 4;  // transposed bitmap
            static_assert(ring >= fixed + sel::kSliceTiesFirst * 8, "tile ring too small for the resolve");
            f.bits_lds = ring >= fixed + bb + (size_t)sel::kSliceTiesFirst * 8;
            f.tl = (int)(((ring - fixed - (f.bits_lds ? bb : 0)) / 8) & ~(size_t)1);
            LSA_LAUNCH_ATT(S == 1, (attend_kernel<DQK, DV, HW, MLA, OUTF32, true, NSTC>), grid, dim3(64 * HW), lds, s,
                           a, po, pml, R, f);
        }
    } else {
        LSA_LAUNCH_ATT(S == 1, (attend_kernel<DQK, DV, HW, MLA, OUTF32, false, NSTC>), grid, dim3(64 * HW), lds, s, a,
                       po, pml, R, FuseArgs{});
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || S == 1) return e;
    return launch_combine<DV, OUTF32>(a, po, pml, S, s);
}

// The 32-head MLA kernel: MLA rows and a multiple of 32 query heads per KV head.
bool mla32(const AttendArgs &a) { return a.d_qk == 576 && (a.Hq / a.Hkv) % 32 == 0; }

template <bool OUTF32>
hipError_t launch_mla(const AttendArgs &a, void *ws, hipStream_t s, const FuseArgs *fuse) {
    const int R = rows_per_split(a);
    const int S = (a.K + R - 1) / R;
    const int HB = (a.Hq / a.Hkv) / 32;
    uint16_t *po = reinterpret_cast<uint16_t *>(ws);
    float *pml = S > 1 ? reinterpret_cast<float *>(reinterpret_cast<char *>(ws) + partial_rows_bytes(a, S)) : nullptr;
    // the two 32-head blocks of a split S workgroups apart: on one XCD (one L2) when S % 8 == 0
    dim3 grid(S * HB, a.T * a.Hkv, a.B * a.L);
    if (fuse) {
        if (R > kMMaxPos) return hipErrorInvalidValue;  // (launch_select_attend checks first)
        FuseArgs f = *fuse;
        constexpr size_t ring = (size_t)3 * kMStage;  // slot 3 takes Q meanwhile
        constexpr size_t fixed = sel::kB2 * 4 + 256 * 4 + 32 * 4;
        f.pw_log = sel::slice_pw_log(f.w.words, 256);
        const size_t bb = ((size_t)256 << f.pw_log) * 4;  // transposed bitmap
        static_assert(ring >= fixed + sel::kSliceTiesFirst * 8, "slots too small for the resolve");
        f.bits_lds = ring >= fixed + bb + (size_t)sel::kSliceTiesFirst * 8;
        f.tl = (int)(((ring - fixed - (f.bits_lds ? bb : 0)) / 8) & ~(size_t)1);
        const size_t lds = kMLdsFixed + (size_t)R * sizeof(int);
        LSA_LAUNCH_ATT(S == 1, (attend_mla_kernel<OUTF32, true>), grid, dim3(256), lds, s, a, po, pml, R, HB, f);
    } else {
        LSA_LAUNCH_ATT(S == 1, (attend_mla_kernel<OUTF32, false>), grid, dim3(256), (size_t)kMLdsFixed, s, a, po, pml,
                       R, HB, FuseArgs{});
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || S == 1) return e;
    return launch_combine<512, OUTF32>(a, po, pml, S, s);
}

template <int DQK, int DV, bool MLA>
hipError_t launch_d(const AttendArgs &a, void *ws, hipStream_t s, const FuseArgs *fuse) {
    if constexpr (MLA) {
        if (mla32(a)) return a.out_f32 ? launch_mla<true>(a, ws, s, fuse) : launch_mla<false>(a, ws, s, fuse);
    }
    const int g = a.Hq / a.Hkv;
    const int HW = (g + 15) / 16;
    if (HW == 1) {
        // one wave of query heads: four waves share the tile loads (three of them compute
        // nothing), so a workgroup keeps more DMA in flight than one wave's 6-bit vmcnt
        // allows. A 3-stage ring when three workgroups then fit on a compute unit, else a
        // 2-stage ring when that fits more of them (long splits: their position lists take
        // the LDS).
        using G3 = AttTile<DQK, DV, 4, MLA, false, 3>;
        using G2 = AttTile<DQK, DV, 4, MLA, false, 2>;
        const int R = rows_per_split(a);
        const size_t list = (size_t)R * sizeof(int) + (size_t)(R / 32) * sizeof(uint32_t);
        const int n3 = (int)(kLdsPerCu / ((size_t)G3::NST * G3::STAGE + list));
        const int n2 = (int)(kLdsPerCu / ((size_t)G2::NST * G2::STAGE + list));
        const bool two = n3 < 3 && n2 > n3;
        if (a.out_f32)
            return two ? launch_t<DQK, DV, 4, MLA, true, 2>(a, ws, s, fuse) : launch_t<DQK, DV, 4, MLA, true, 3>(a, ws, s, fuse);
        return two ? launch_t<DQK, DV, 4, MLA, false, 2>(a, ws, s, fuse) : launch_t<DQK, DV, 4, MLA, false, 3>(a, ws, s, fuse);
    }
    if (a.out_f32) {
        if (HW == 2) return launch_t<DQK, DV, 2, MLA, true>(a, ws, s, fuse);
        return launch_t<DQK, DV, 4, MLA, true>(a, ws, s, fuse);
    }
    if (HW == 2) return launch_t<DQK, DV, 2, MLA, false>(a, ws, s, fuse);
    return launch_t<DQK, DV, 4, MLA, false>(a, ws, s, fuse);
}

}  // namespace

bool attend_supported(int d_qk, int d_v, int g) {
    // one wave per 16 query heads of a KV head: 1, 2 or 4 waves per workgroup
    if (g < 1 || g > 64 || (g + 15) / 16 == 3) return false;
    return (d_qk == 128 && d_v == 128) || (d_qk == 576 && d_v == 512);
}

void set_attend_launch_events(hipEvent_t start, hipEvent_t stop) {
    t_att_start = start;
    t_att_stop = stop;
}

int attend_default_splits(const AttendArgs &a) {
    const int g = a.Hq / a.Hkv;
    const int HW = (g + 15) / 16;
    const long units = (long)a.L * a.B * a.T * a.Hkv;
    if (mla32(a)) {
        // 32-head blocks: about 256 workgroups, at least one round (128 rows) per split
        const long wg = units * (g / 32);
        long s = (256 + wg - 1) / wg;
        const long smax = (a.K + kMRound - 1) / kMRound;
        if (s > smax) s = smax;
        if (s > kAttendMaxSplits) s = kAttendMaxSplits;
        return (int)(s < 1 ? 1 : s);
    }
    // four waves of heads: one workgroup per compute unit; one wave of heads: three per
    // compute unit in one generation; else four workgroups per compute unit over the launch
    const long target = HW == 4 ? 256 : HW == 1 ? kOneHeadTarget : 1024;
    long s = (target + units - 1) / units;
    const long smax = (a.K + kRows - 1) / kRows;
    const long smin = (a.K + kMaxR - 1) / kMaxR;
    if (s > smax) s = smax;
    if (s < smin) s = smin;
    if (s < 1) s = 1;
    return (int)s;
}

size_t attend_workspace_bytes(const AttendArgs &a) {
    const int R = rows_per_split(a);
    const int S = (a.K + R - 1) / R;
    if (S <= 1) return 0;
    return partial_rows_bytes(a, S) + (size_t)a.L * a.B * a.T * a.Hq * S * 2 * sizeof(float);
}

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxScratchDevices] = {};
}  // namespace

hipError_t attend_static_scratch(int dev, void **ptr) {
    if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        // each GPU holds its own copy of the array at its own address: look it up with
        // that device current, once
        int cur = 0;
        hipError_t e = hipGetDevice(&cur);
        if (e != hipSuccess) return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        const hipError_t e2 = cur != dev ? hipSetDevice(cur) : hipSuccess;
        if (e != hipSuccess) return e;
        if (e2 != hipSuccess) return e2;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

hipError_t launch_attend(const AttendArgs &a, void *ws, hipStream_t s) {
    const bool mla = a.d_qk == 576;
    if (mla) return launch_d<576, 512, true>(a, ws, s, nullptr);
    return launch_d<128, 128, false>(a, ws, s, nullptr);
}

hipError_t launch_select_attend(const SelectArgs &sa, void *sel_ws, const AttendArgs &a, void *ws, hipStream_t s) {
    // Every attention workgroup sharing a selection row repeats the row-level part of the
    // selection. That is paid back only when four waves resolve together (more than 48
    // query heads per KV head) and one KV head of one layer reads each row; otherwise the
    // selection's own resolve kernel and then the plain attention run (same results).
    if (!(a.Hq / a.Hkv > 48 && a.Hkv * a.L == 1) || (mla32(a) && rows_per_split(a) > kMMaxPos) ||
        select_small(sa.n_cols)) {
        const hipError_t e = launch_select(sa, sel_ws, s);
        if (e != hipSuccess) return e;
        AttendArgs a2 = a;
        a2.idx = sa.idx;
        return launch_attend(a2, ws, s);
    }
    const hipError_t e = launch_select_front(sa, sel_ws, s);
    if (e != hipSuccess) return e;
    FuseArgs f{};
    f.sa = sa;
    f.w = sel::carve(sel_ws, sa.B * sa.T, sa.n_cols, false);
    if (a.d_qk == 576) return launch_d<576, 512, true>(a, ws, s, &f);
    return launch_d<128, 128, false>(a, ws, s, &f);
}

}  // namespace lsa
