// Sparse attention over the selected rows only (LongCat-2.0 summary, aitrends.kr,
// "Technical features": no attention matrix over all token pairs), for MQA/GQA and
// MLA latent KV, several CLI layers per launch.
//
// One workgroup = (layer, sequence, query token, KV head, split of the K selected
// rows); wave w owns 16 query heads of the KV head's group. Per tile of 32 selected
// rows:
//   - the rows are gathered HBM -> LDS by direct-to-LDS DMA (global_load_lds_dwordx4,
//     16-byte chunks, each row contiguous) into a 3-stage ring: two tiles in flight
//     while one is computed; positions of the whole split are staged in LDS first;
//   - S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (lane = one head, 8 rows), so the
//     online-softmax statistics of a head stay inside one lane group;
//   - P^T is packed to bf16 straight from the S^T accumulators (no LDS round trip)
//     and O^T += V^T P^T accumulates on MFMA in fp32; the V^T operand comes from LDS
//     transpose reads (ds_read_b64_tr_b16).
// Splits write (o, m, l) partials that a second kernel merges in split order.
#include "common.cuh"
#include "kernels.h"

namespace lsa {
namespace {

constexpr int kRows = 32;     // selected rows per tile
constexpr int kMaxR = 2048;   // selected rows per split (positions staged in LDS)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// s_waitcnt vmcnt(n) (gfx9 encoding: expcnt and lgkmcnt left at their maxima)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <int DQK, int DV, int HW, bool MLA, bool OUTF32>
struct AttTile {
    static constexpr int NT = 64 * HW;
    static constexpr int KCH = DQK * 2 / 16;          // 16-byte chunks of a K row
    static constexpr int VCH = MLA ? 0 : DV * 2 / 16;  // of a V row (separate V cache)
    static constexpr int KCP = KCH + 1;               // + 1 padding chunk: conflict-free LDS reads
    static constexpr int VCP = MLA ? 0 : VCH + 1;
    static constexpr int KST = KCP * 16, VST = MLA ? KST : VCP * 16;
    static constexpr int CHUNKS = kRows * (KCP + VCP);
    static constexpr int INSTR = ((CHUNKS + 63) / 64 + HW - 1) / HW * HW;  // 64-lane DMA instructions per tile
    static constexpr int PER_WAVE = INSTR / HW;
    static constexpr int STAGE = INSTR * 64 * 16;     // bytes per stage
    // tiles in LDS: computing one, NST-1 in flight (bounded by the 6-bit vmcnt)
    static constexpr int NST = PER_WAVE * 2 < 64 ? 3 : 2;
    static_assert(PER_WAVE * (NST - 1) < 64, "vmcnt budget");
};

template <int DQK, int DV, int HW, bool MLA, bool OUTF32>
__global__ __launch_bounds__(64 * HW) void attend_kernel(AttendArgs a, float *po, float *pml, int R) {
    using G = AttTile<DQK, DV, HW, MLA, OUTF32>;
    constexpr int NT = G::NT;
    constexpr int KSQ = DQK / 32;
    constexpr int NCB = DV / 16;
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    int *posbuf = reinterpret_cast<int *>(lds + G::NST * G::STAGE);

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

    const int32_t *idxrow = a.idx + ((int64_t)b * T + t) * K + r0;
    for (int i = tid; i < nrows; i += NT) {
        const int s = idxrow[i];
        posbuf[i] = (s >= 0 && s < a.N) ? s : -1;
    }
    // Q as the B operand of S^T = K Q^T: lane holds head hl, dims 32 ks + 8 q4 .. +8
    bf16x8 bq[KSQ];
    {
        const uint16_t *qp = a.q + layer * a.lsq + (((int64_t)b * T + t) * Hq + hq) * DQK + 8 * q4;
#pragma unroll
        for (int ks = 0; ks < KSQ; ++ks) {
            u32x4 v = {0, 0, 0, 0};
            if (hvalid) v = *reinterpret_cast<const u32x4 *>(qp + 32 * ks);
            bq[ks] = __builtin_bit_cast(bf16x8, v);
        }
    }
    f32x4 o[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) o[cb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    float m_run = kNegInf, l_run = 0.0f;
    const float sl2 = a.scale * kLog2e;
    const uint16_t *kbase = a.k + layer * a.lsk + b * a.ksb + kvh * a.ksh;
    const uint16_t *vbase = MLA ? kbase : a.v + layer * a.lsv + b * a.vsb + kvh * a.vsh;

    // DMA one tile: instruction n of the tile fills LDS chunks [64 n, 64 n + 64) of the
    // stage; lane l loads chunk 64 n + l. Padding chunks and invalid rows read row 0
    // (finite values; their probabilities are zero).
    auto issue_tile = [&](int it) {
        unsigned char *stage = lds + (it % G::NST) * G::STAGE;
        const uint16_t *src[G::PER_WAVE];
#pragma unroll
        for (int j = 0; j < G::PER_WAVE; ++j) {  // all addresses first (positions from LDS)
            const int n = j * HW + wave;
            const int ci = 64 * n + lane;
            src[j] = kbase;
            if (ci < G::CHUNKS) {
                const bool isk = ci < kRows * G::KCP;
                const int cc = isk ? ci : ci - kRows * G::KCP;
                const int row = isk ? cc / G::KCP : cc / G::VCP;
                const int c = isk ? cc % G::KCP : cc % G::VCP;
                const int ri = it * kRows + row;
                const int pos = ri < nrows ? posbuf[ri] : -1;
                const int lim = isk ? G::KCH : G::VCH;
                if (pos >= 0 && c < lim) src[j] = (isk ? kbase + pos * a.ksn : vbase + pos * a.vsn) + c * 8;
            }
        }
#pragma unroll
        for (int j = 0; j < G::PER_WAVE; ++j)  // then the DMA instructions back to back
            __builtin_amdgcn_global_load_lds((const glb_void_t *)src[j], (lds_void_t *)(stage + 1024 * (j * HW + wave)),
                                             16, 0, 0);
    };

    const int ntile = (nrows + kRows - 1) / kRows;
    __syncthreads();  // posbuf
    // prologue: tiles 0 .. NST-2 in flight
#pragma unroll
    for (int p = 0; p < G::NST - 1; ++p)
        if (p < ntile) issue_tile(p);

    for (int it = 0; it < ntile; ++it) {
        // this wave's loads of tile `it` have landed once at most (ahead * PER_WAVE) are pending
        const int ahead = min(G::NST - 2, ntile - 1 - it);
        if (ahead >= 1) wait_vmcnt<G::PER_WAVE>();
        else wait_vmcnt<0>();
        __syncthreads();  // every wave's loads of tile `it` landed; tile it-1 no longer read
        if (it + G::NST - 1 < ntile) issue_tile(it + G::NST - 1);
        const unsigned char *kt = lds + (it % G::NST) * G::STAGE;
        const unsigned char *vt = MLA ? kt : kt + kRows * G::KST;

        // ---- S^T tile (32 rows x 16 heads): st[rb][r] = row 16 rb + 4 q4 + r, head hl.
        // K fragments come from LDS through a 2-deep register ring (loads one step ahead).
        f32x4 st[2] = {f32x4{0.0f, 0.0f, 0.0f, 0.0f}, f32x4{0.0f, 0.0f, 0.0f, 0.0f}};
        {
            const unsigned char *k0 = kt + hl * G::KST + 16 * q4;
            const unsigned char *k1 = k0 + 16 * G::KST;
            u32x4 f0[2], f1[2];
            f0[0] = *reinterpret_cast<const u32x4 *>(k0);
            f1[0] = *reinterpret_cast<const u32x4 *>(k1);
#pragma unroll
            for (int ks = 0; ks < KSQ; ++ks) {
                if (ks + 1 < KSQ) {
                    f0[(ks + 1) & 1] = *reinterpret_cast<const u32x4 *>(k0 + 64 * (ks + 1));
                    f1[(ks + 1) & 1] = *reinterpret_cast<const u32x4 *>(k1 + 64 * (ks + 1));
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
                const int ri = it * kRows + 16 * rb + 4 * q4 + r;
                const bool ok = ri < nrows && posbuf[ri] >= 0;
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
            l_run *= alpha;
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) o[cb] *= alpha;
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
        const u32x4 pp = {pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3]), pack_bf16(p[4], p[5]), pack_bf16(p[6], p[7])};
        const bf16x8 bp = __builtin_bit_cast(bf16x8, pp);
        // ---- O^T += V^T P^T. A operand (dv 16 cb + hl, the same 8 rows) by two LDS
        // transpose reads: lane i of a 16-lane group points at V[row 4 q4 + i/4][dv 4 (i%4)]
        // and receives V[4 q4 .. 4 q4 + 3][dv i] (then rows 16 + 4 q4 ..); 2-deep ring.
        {
            typedef __attribute__((__vector_size__(8 * sizeof(short)))) short s16x8;
            const unsigned char *va = vt + (4 * q4 + (hl >> 2)) * G::VST + 8 * (hl & 3);
            const unsigned char *vb = va + 16 * G::VST;
            s16x4 x0[2], x1[2];
            x0[0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)va);
            x1[0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)vb);
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                if (cb + 1 < NCB) {
                    x0[(cb + 1) & 1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(va + 32 * (cb + 1)));
                    x1[(cb + 1) & 1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(vb + 32 * (cb + 1)));
                }
                const s16x8 av = __builtin_shufflevector(x0[cb & 1], x1[cb & 1], 0, 1, 2, 3, 4, 5, 6, 7);
                o[cb] = mfma16(__builtin_bit_cast(bf16x8, av), bp, o[cb]);
            }
        }
    }

    // ---- finish: the 4 lane groups hold disjoint rows of the same head
    float l_tot = l_run + __shfl_xor(l_run, 16, 64);
    l_tot += __shfl_xor(l_tot, 32, 64);
    if (!hvalid) return;
    const int64_t ohead = (((int64_t)b * T + t) * Hq + hq);
    if (nsplit == 1) {
        const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
        if constexpr (OUTF32) {
            float *out = reinterpret_cast<float *>(a.out) + layer * a.lso + ohead * DV + 4 * q4;
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) *reinterpret_cast<f32x4 *>(out + 16 * cb) = o[cb] * inv;
        } else {
            uint16_t *out = reinterpret_cast<uint16_t *>(a.out) + layer * a.lso + ohead * DV + 4 * q4;
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                uint2 w2;
                w2.x = pack_bf16(o[cb][0] * inv, o[cb][1] * inv);
                w2.y = pack_bf16(o[cb][2] * inv, o[cb][3] * inv);
                *reinterpret_cast<uint2 *>(out + 16 * cb) = w2;
            }
        }
        if (a.lse && lane < 16)
            a.lse[layer * a.lsl + ohead] = l_tot > 0.0f ? (m_run + __builtin_log2f(l_tot)) * kLn2 : kNegInf;
    } else {
        const int64_t pidx = ((int64_t)layer * B * T * Hq + ohead) * nsplit + split;
        float *dst = po + pidx * DV + 4 * q4;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) *reinterpret_cast<f32x4 *>(dst + 16 * cb) = o[cb];
        if (lane < 16) {
            pml[2 * pidx] = m_run;
            pml[2 * pidx + 1] = l_tot;
        }
    }
}

// Merge the split partials of one (layer, b, t, hq) in split order.
template <int DV, bool OUTF32>
__global__ __launch_bounds__(64) void attend_combine_kernel(AttendArgs a, const float *po, const float *pml, int S) {
    const int hq = blockIdx.x, bt = blockIdx.y, layer = blockIdx.z;
    const int64_t ohead = (int64_t)bt * a.Hq + hq;
    const int64_t pbase = ((int64_t)layer * a.B * a.T * a.Hq + ohead) * S;
    float M = kNegInf;
    for (int s = 0; s < S; ++s) M = fmaxf(M, pml[2 * (pbase + s)]);
    float L = 0.0f;
    constexpr int PER = DV / 64;
    float acc[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] = 0.0f;
    if (M != kNegInf) {
        for (int s = 0; s < S; ++s) {
            const float m = pml[2 * (pbase + s)];
            const float wgt = m == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(m - M);
            L += wgt * pml[2 * (pbase + s) + 1];
            const float *src = po + (pbase + s) * DV;
#pragma unroll
            for (int e = 0; e < PER; ++e) acc[e] += wgt * src[threadIdx.x + 64 * e];
        }
    }
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    if constexpr (OUTF32) {
        float *out = reinterpret_cast<float *>(a.out) + layer * a.lso + ohead * DV;
#pragma unroll
        for (int e = 0; e < PER; ++e) out[threadIdx.x + 64 * e] = acc[e] * inv;
    } else {
        uint16_t *out = reinterpret_cast<uint16_t *>(a.out) + layer * a.lso + ohead * DV;
#pragma unroll
        for (int e = 0; e < PER; ++e) out[threadIdx.x + 64 * e] = (uint16_t)f2bf(acc[e] * inv);
    }
    if (a.lse && threadIdx.x == 0)
        a.lse[layer * a.lsl + ohead] = L > 0.0f ? (M + __builtin_log2f(L)) * kLn2 : kNegInf;
}

int rows_per_split(const AttendArgs &a) {
    int R = (a.K + a.n_splits - 1) / a.n_splits;
    return (R + kRows - 1) / kRows * kRows;
}

template <int DQK, int DV, int HW, bool MLA, bool OUTF32>
hipError_t launch_t(const AttendArgs &a, void *ws, hipStream_t s) {
    const int R = rows_per_split(a);
    const int S = (a.K + R - 1) / R;
    float *po = reinterpret_cast<float *>(ws);
    float *pml = po + (size_t)a.L * a.B * a.T * a.Hq * S * DV;
    dim3 grid(S, a.T * a.Hkv, a.B * a.L);
    using G = AttTile<DQK, DV, HW, MLA, OUTF32>;
    const size_t lds = (size_t)G::NST * G::STAGE + (size_t)kMaxR * sizeof(int);
    hipLaunchKernelGGL((attend_kernel<DQK, DV, HW, MLA, OUTF32>), grid, dim3(64 * HW), lds, s, a, po, pml, R);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || S == 1) return e;
    dim3 cgrid(a.Hq, a.B * a.T, a.L);
    hipLaunchKernelGGL((attend_combine_kernel<DV, OUTF32>), cgrid, dim3(64), 0, s, a, po, pml, S);
    return hipGetLastError();
}

template <int DQK, int DV, bool MLA>
hipError_t launch_d(const AttendArgs &a, void *ws, hipStream_t s) {
    const int g = a.Hq / a.Hkv;
    const int HW = (g + 15) / 16;
    if (a.out_f32) {
        if (HW == 1) return launch_t<DQK, DV, 1, MLA, true>(a, ws, s);
        if (HW == 2) return launch_t<DQK, DV, 2, MLA, true>(a, ws, s);
        return launch_t<DQK, DV, 4, MLA, true>(a, ws, s);
    }
    if (HW == 1) return launch_t<DQK, DV, 1, MLA, false>(a, ws, s);
    if (HW == 2) return launch_t<DQK, DV, 2, MLA, false>(a, ws, s);
    return launch_t<DQK, DV, 4, MLA, false>(a, ws, s);
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
    const long target = HW == 4 ? 128 : 1024;
    long s = (target + units - 1) / units;
    const long smax = (a.K + kRows - 1) / kRows;
    const long smin = (a.K + kMaxR - 1) / kMaxR;
    if (s > smax) s = smax;
    if (s < smin) s = smin;
    if (s < 1) s = 1;
    return (int)s;
}

size_t attend_workspace_bytes(const AttendArgs &a) {
    AttendArgs c = a;
    const int R = rows_per_split(c);
    const int S = (a.K + R - 1) / R;
    if (S <= 1) return 0;
    const size_t heads = (size_t)a.L * a.B * a.T * a.Hq * S;
    return heads * a.d_v * sizeof(float) + heads * 2 * sizeof(float);
}

hipError_t launch_attend(const AttendArgs &a, void *ws, hipStream_t s) {
    const bool mla = a.d_qk == 576;
    if (mla) return launch_d<576, 512, true>(a, ws, s);
    return launch_d<128, 128, false>(a, ws, s);
}

}  // namespace lsa
