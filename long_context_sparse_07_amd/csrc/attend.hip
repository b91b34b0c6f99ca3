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
#include "select_core.cuh"

namespace lsa {
namespace {

constexpr int kRows = 32;     // selected rows per tile
constexpr int kMaxR = 2048;   // selected rows per split (positions staged in LDS)
constexpr int kBlk = 2048;    // LDS bytes of one block (4 chunks) of the 32 rows
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

template <int DQK, int DV, int HW, bool MLA, bool OUTF32>
struct AttTile {
    static constexpr int NT = 64 * HW;
    static constexpr int KB = DQK * 2 / 64;           // K blocks per row (MLA 18, else 4)
    static constexpr int VB = MLA ? 0 : DV * 2 / 64;  // V blocks (separate V cache)
    static constexpr int STAGE = (KB + VB) * kBlk;
    static constexpr int INSTR = 2 * (KB + VB);       // DMA instructions per tile (16 rows each)
    static_assert(INSTR % HW == 0, "tile must split evenly over the waves");
    static constexpr int PER_WAVE = INSTR / HW;
    // tiles in LDS: one computed, NST-1 in flight; as many as the LDS (with the position
    // list) and the 6-bit vmcnt allow, at most 4
    static constexpr int LDS_MAX = 160 * 1024 - kMaxR * 4 - kMaxR / 32 * 4;
    static constexpr int NST_LDS = LDS_MAX / STAGE;
    static constexpr int NST_V = 63 / PER_WAVE + 1;
    static constexpr int NST = NST_LDS < NST_V ? (NST_LDS < 4 ? NST_LDS : 4) : (NST_V < 4 ? NST_V : 4);
    static_assert(NST >= 2, "two stages at least");
    static_assert(PER_WAVE * (NST - 1) < 64, "vmcnt budget");
    static_assert(!MLA || DV == 512, "MLA values are the first 512 columns (16 blocks)");
};

template <int DQK, int DV, int HW, bool MLA, bool OUTF32, bool FUSED>
__global__ __launch_bounds__(64 * HW) void attend_kernel(AttendArgs a, uint16_t *po, float *pml, int R, FuseArgs f) {
    using G = AttTile<DQK, DV, HW, MLA, OUTF32>;
    constexpr int NT = G::NT;
    constexpr int KSQ = DQK / 32;
    constexpr int NCB = DV / 16;
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    int *posbuf = reinterpret_cast<int *>(lds + G::NST * G::STAGE);  // [kMaxR]
    uint32_t *vmask = reinterpret_cast<uint32_t *>(posbuf + kMaxR);   // [kMaxR / 32] valid rows per tile

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
    // FUSED: Q is requested first, its latency hidden under the selection's
    if constexpr (FUSED) load_q();
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
        sel::resolve_slice<NT>(f.sa, f.w, (int)selrow, r0, r0 + nrows, S, posbuf);  // ends with a barrier
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
    // barrier.
    auto rowpos = [&](int i) {  // cache row of selected row i of the split, -1 if none
        if constexpr (FUSED) {  // the position list holds cache rows when paged
            const int s = i < nrows ? posbuf[i] : -1;
            return (s >= 0 && (a.bt || s < a.N)) ? s : -1;
        } else {
            const int s = i < nrows ? idxrow[i] : -1;
            return (s >= 0 && s < a.N && s <= pmax) ? phys(s) : -1;
        }
    };
    const int lpos0 = rowpos(tid);  // this thread's first entry of the LDS position list
    int dpos[G::NST - 1][2];
#pragma unroll
    for (int p = 0; p < G::NST - 1; ++p) {
        dpos[p][0] = rowpos(p * kRows + drow);
        dpos[p][1] = rowpos(p * kRows + drow + 16);
    }
    // invalid rows read row 0 (finite values; zero probability)
    if (ntile > 0) issue_tile(0, max(dpos[0][0], 0), max(dpos[0][1], 0));
    if constexpr (!FUSED) load_q();
#pragma unroll
    for (int p = 1; p < G::NST - 1; ++p)
        if (p < ntile) issue_tile(p, max(dpos[p][0], 0), max(dpos[p][1], 0));
    // (FUSED: entries are rewritten in place, each by the thread that reads it; the DMA
    // positions read above take max(., 0) and so agree with either value)
    for (int i = tid; i < ntile * kRows; i += NT) {
        const int ps = i == tid ? lpos0 : rowpos(i);
        posbuf[i] = max(ps, 0);
        const uint64_t bal = __ballot(ps >= 0);
        if (lane == 0) {
            vmask[i >> 5] = (uint32_t)bal;
            if (i + 32 < ntile * kRows) vmask[(i >> 5) + 1] = (uint32_t)(bal >> 32);
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
        const int ahead = min(G::NST - 2, ntile - 1 - it);
        if constexpr (G::NST >= 4) {
            if (ahead >= 2) wait_vmcnt<(G::NST >= 4 ? 2 * G::PER_WAVE : 0)>();
            else if (ahead == 1) wait_vmcnt<G::PER_WAVE>();
            else wait_vmcnt<0>();
        } else {
            if (ahead >= 1) wait_vmcnt<G::PER_WAVE>();
            else wait_vmcnt<0>();
        }
        __syncthreads();  // every wave's loads of tile `it` landed; tile it-1 no longer read
        if (it + G::NST - 1 < ntile) {
            const int nt = it + G::NST - 1;
            issue_tile(nt, posbuf[nt * kRows + drow], posbuf[nt * kRows + drow + 16]);
        }
        const lds_u8 *kt = (const lds_u8 *)lds + (it % G::NST) * G::STAGE;
        const lds_u8 *vt = MLA ? kt : kt + G::KB * kBlk;
        const uint32_t vm = vmask[it];

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

// Merge the split partials of HPW heads of one (layer, b, t) in split order. Lane l of
// the head's lane group owns the 8 values 8 l .. 8 l + 7 of its row; one wave turns a
// head's (m, l) pairs into weights l 2^(m - M) (M = the largest m) for the normalised
// rows, then every lane accumulates its 8 values over the splits, 16-byte loads issued
// eight splits at a time.
constexpr int kCombT = 256;
constexpr int kMaxSplits = kAttendMaxSplits;

template <int DV, bool OUTF32>
__global__ __launch_bounds__(kCombT) void attend_combine_kernel(AttendArgs a, const uint16_t *po, const float *pml, int S) {
    constexpr int LPR = DV / 8;          // lanes per head row
    constexpr int HPW = kCombT / LPR;    // heads per workgroup
    constexpr int HPV = HPW / 4;         // heads per wave
    __shared__ float wgt[HPW][kMaxSplits];
    __shared__ float linv[HPW];
    const int bt = blockIdx.y, layer = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t hbase = (int64_t)layer * a.B * a.T * a.Hq + (int64_t)bt * a.Hq;  // partial heads of (layer, b, t)
    // ---- weights: wave w handles heads HPV w .. HPV w + HPV - 1 of the group
    for (int k = 0; k < HPV; ++k) {
        const int hl = wave * HPV + k;
        const int hq = blockIdx.x * HPW + hl;
        if (hq >= a.Hq) break;
        const float *ml = pml + (hbase + hq) * S * 2;
        float M = kNegInf;
        for (int s = lane; s < S; s += 64) M = fmaxf(M, ml[2 * s]);
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
        float L = 0.0f;
        for (int s = lane; s < S; s += 64) {
            const float m = ml[2 * s];
            const float wl = (M == kNegInf || m == kNegInf) ? 0.0f : __builtin_amdgcn_exp2f(m - M) * ml[2 * s + 1];
            wgt[hl][s] = wl;
            L += wl;
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) L += __shfl_xor(L, o, 64);  // the same tree every run
        if (lane == 0) {
            linv[hl] = L > 0.0f ? 1.0f / L : 0.0f;
            if (a.lse) a.lse[layer * a.lsl + (int64_t)bt * a.Hq + hq] = L > 0.0f ? (M + __builtin_log2f(L)) * kLn2 : kNegInf;
        }
    }
    __syncthreads();
    // ---- weighted sum of the rows
    const int hl = tid / LPR, c = tid % LPR;
    const int hq = blockIdx.x * HPW + hl;
    if (hq >= a.Hq) return;
    const u32x4 *src = reinterpret_cast<const u32x4 *>(po + (hbase + hq) * S * DV) + c;
    constexpr int RU = DV / 8;  // u32x4 per row
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
    auto add = [&](const u32x4 v, float w) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            acc[2 * q] += w * bf16lo(v[q]);
            acc[2 * q + 1] += w * bf16hi(v[q]);
        }
    };
    int s = 0;
    for (; s + 8 <= S; s += 8) {
        u32x4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = src[(int64_t)(s + u) * RU];
#pragma unroll
        for (int u = 0; u < 8; ++u) add(v[u], wgt[hl][s + u]);
    }
    for (; s < S; ++s) add(src[(int64_t)s * RU], wgt[hl][s]);
    const float inv = linv[hl];
    const int64_t ob = layer * a.lso + ((int64_t)bt * a.Hq + hq) * DV + 8 * c;
    if constexpr (OUTF32) {
        float *out = reinterpret_cast<float *>(a.out) + ob;
        *reinterpret_cast<f32x4 *>(out) = f32x4{acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
        *reinterpret_cast<f32x4 *>(out + 4) = f32x4{acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv};
    } else {
        typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16v8;
        const bf16v8 w8 = {(__bf16)(acc[0] * inv), (__bf16)(acc[1] * inv), (__bf16)(acc[2] * inv),
                           (__bf16)(acc[3] * inv), (__bf16)(acc[4] * inv), (__bf16)(acc[5] * inv),
                           (__bf16)(acc[6] * inv), (__bf16)(acc[7] * inv)};
        *reinterpret_cast<bf16v8 *>(reinterpret_cast<uint16_t *>(a.out) + ob) = w8;
    }
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

template <int DQK, int DV, int HW, bool MLA, bool OUTF32>
hipError_t launch_t(const AttendArgs &a, void *ws, hipStream_t s, const FuseArgs *fuse) {
    const int R = rows_per_split(a);
    const int S = (a.K + R - 1) / R;
    uint16_t *po = reinterpret_cast<uint16_t *>(ws);
    float *pml = S > 1 ? reinterpret_cast<float *>(reinterpret_cast<char *>(ws) + partial_rows_bytes(a, S)) : nullptr;
    dim3 grid(S, a.T * a.Hkv, a.B * a.L);
    using G = AttTile<DQK, DV, HW, MLA, OUTF32>;
    const size_t lds = (size_t)G::NST * G::STAGE + (size_t)kMaxR * sizeof(int) + (size_t)(kMaxR / 32) * sizeof(uint32_t);
    if (fuse) {
        // (the chain runs only with four waves a workgroup: launch_select_attend decides)
        if constexpr (HW != 4) return hipErrorInvalidValue;
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
        if constexpr (HW == 4)
            hipLaunchKernelGGL((attend_kernel<DQK, DV, HW, MLA, OUTF32, true>), grid, dim3(64 * HW), lds, s, a, po, pml,
                               R, f);
    } else {
        hipLaunchKernelGGL((attend_kernel<DQK, DV, HW, MLA, OUTF32, false>), grid, dim3(64 * HW), lds, s, a, po, pml, R,
                           FuseArgs{});
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || S == 1) return e;
    constexpr int HPW = kCombT / (DV / 8);
    dim3 cgrid((a.Hq + HPW - 1) / HPW, a.B * a.T, a.L);
    hipLaunchKernelGGL((attend_combine_kernel<DV, OUTF32>), cgrid, dim3(kCombT), 0, s, a, po, pml, S);
    return hipGetLastError();
}

template <int DQK, int DV, bool MLA>
hipError_t launch_d(const AttendArgs &a, void *ws, hipStream_t s, const FuseArgs *fuse) {
    const int g = a.Hq / a.Hkv;
    const int HW = (g + 15) / 16;
    if (a.out_f32) {
        if (HW == 1) return launch_t<DQK, DV, 1, MLA, true>(a, ws, s, fuse);
        if (HW == 2) return launch_t<DQK, DV, 2, MLA, true>(a, ws, s, fuse);
        return launch_t<DQK, DV, 4, MLA, true>(a, ws, s, fuse);
    }
    if (HW == 1) return launch_t<DQK, DV, 1, MLA, false>(a, ws, s, fuse);
    if (HW == 2) return launch_t<DQK, DV, 2, MLA, false>(a, ws, s, fuse);
    return launch_t<DQK, DV, 4, MLA, false>(a, ws, s, fuse);
}

}  // namespace

bool attend_supported(int d_qk, int d_v, int g) {
    // one wave per 16 query heads of a KV head: 1, 2 or 4 waves per workgroup
    if (g < 1 || g > 64 || (g + 15) / 16 == 3) return false;
    return (d_qk == 128 && d_v == 128) || (d_qk == 576 && d_v == 512);
}

int attend_default_splits(const AttendArgs &a) {
    const int g = a.Hq / a.Hkv;
    const int HW = (g + 15) / 16;
    const long units = (long)a.L * a.B * a.T * a.Hkv;
    const long target = HW == 4 ? 256 : 1024;
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
    if (!(a.Hq / a.Hkv > 48 && a.Hkv * a.L == 1)) {
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
