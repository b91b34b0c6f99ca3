// Backward of the sparse attention (training): gradients of q and of the selected K/V rows,
// the selection held fixed. LSA is trained with its sparse operators and those operators
// are deterministic (molayo1419.me LongCat-2.0 article, sections "The sparse attention
// problem at 1M tokens" and "Training on 50,000 Chinese ASICs"), so every sum below runs in
// a fixed order and no floating-point atomics are used.
//
// With z = scale q . K_s, P = exp(z - lse), dP = dO . V_s, D = dO . O, dS = P (dP - D):
//   dq_h = scale sum_s dS K_s,  dK_s = scale sum_(t,h) dS q_h,  dV_s = sum_(t,h) P dO_h.
//
// bwd_rows_kernel (one workgroup per query token, KV head and tile of 32 selected rows):
//   the tile's K (and V) rows are gathered into LDS; q . K and dO . V for every head of
//   the group and row of the tile on the matrix cores, then P and scale * dS; then the
//   rows' gradient contributions of this query (G: scale sum_h dS q_h, and sum_h P dO_h)
//   and this tile's part of dq.
// bwd_dq_kernel: dq = the tiles' parts, added in tile order.
// bwd_kv_kernel (one workgroup per tile of 16 cache positions and KV head): the
//   contributions G of every query that selected one of the positions, added in ascending
//   query order; only the positions some query selected are written. With one query token
//   per sequence each position has a single contribution, and bwd_rows_kernel writes the
//   row gradients straight to dk / dv instead (no G, no position sweep).
// target_tile_kernel, kl_kernel: the indexer distillation target (head-averaged attention
//   over the selected rows), its KL against the indexer's softmax, and the KL's gradient
//   with respect to the indexer scores.
#include "common.cuh"
#include "kernels.h"

namespace lsa {
namespace {

constexpr int kBT = 256;  // threads per workgroup
constexpr int kRT = 32;   // selected rows per bwd_rows workgroup
constexpr int kPT = 16;   // cache positions per bwd_kv workgroup (LDS: 16 x 576 fp32)
constexpr int kMaxG = 64; // query heads per KV head

__device__ __forceinline__ float dot8(u32x4 x, u32x4 y) {
    float s = 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) s += bf16lo(x[e]) * bf16lo(y[e]) + bf16hi(x[e]) * bf16hi(y[e]);
    return s;
}

__device__ __forceinline__ float bf16_at(const uint16_t *p) { return u2f((uint32_t)*p << 16); }

// G row width: MLA one latent row (dK + dV on its first DV columns); else K then V
template <int DQK, int DV, bool MLA>
constexpr int g_width() { return MLA ? DQK : DQK + DV; }

// DIRECT (one query token per sequence): the contributions are the row gradients
// themselves; row r goes to dk (and dv) at its position, not to G.
template <int DQK, int DV, bool MLA, bool DIRECT>
__global__ __launch_bounds__(kBT) void bwd_rows_kernel(AttendBwdArgs a, float *G, float *dqp) {
    constexpr int GW = g_width<DQK, DV, MLA>();
    __shared__ __attribute__((aligned(16))) uint16_t kt[kRT][DQK];
    __shared__ __attribute__((aligned(16))) uint16_t vt[MLA ? 1 : kRT][DV];
    __shared__ __attribute__((aligned(16))) float Ps[kMaxG][kRT];
    __shared__ __attribute__((aligned(16))) float dSs[kMaxG][kRT];  // scale * dS
    __shared__ float Zs[kMaxG][kRT], DPs[kMaxG][kRT];  // q . K_r and dO . V_r (unscaled)
    __shared__ float Dh[kMaxG], lseh[kMaxG];
    __shared__ int rowpos[kRT];

    const int tid = threadIdx.x;
    const int tile = blockIdx.x, bt = blockIdx.y, kvh = blockIdx.z;
    const int b = bt / a.T;
    const int g = a.Hq / a.Hkv;
    const int r0 = tile * kRT;
    const int nrows = min(kRT, a.K - r0);
    const int ntiles = gridDim.x;
    const int64_t qh0 = (int64_t)bt * a.Hq + kvh * g;  // first query head row of the group

    if (tid < kRT) {
        const int s = tid < nrows ? a.idx[(int64_t)bt * a.K + r0 + tid] : -1;
        rowpos[tid] = (s >= 0 && s < a.N) ? s : -1;
    }
    __syncthreads();
    // gather the tile's rows (invalid rows: zeros)
    const uint16_t *kb = a.k + b * a.ksb + kvh * a.ksh;
    for (int i = tid; i < kRT * DQK / 8; i += kBT) {
        const int r = i / (DQK / 8), c = i % (DQK / 8);
        const int s = rowpos[r];
        u32x4 v = {0, 0, 0, 0};
        if (s >= 0) v = *reinterpret_cast<const u32x4 *>(kb + (int64_t)s * a.ksn + 8 * c);
        *reinterpret_cast<u32x4 *>(&kt[r][8 * c]) = v;
    }
    if constexpr (!MLA) {
        const uint16_t *vb = a.v + b * a.vsb + kvh * a.vsh;
        for (int i = tid; i < kRT * DV / 8; i += kBT) {
            const int r = i / (DV / 8), c = i % (DV / 8);
            const int s = rowpos[r];
            u32x4 v = {0, 0, 0, 0};
            if (s >= 0) v = *reinterpret_cast<const u32x4 *>(vb + (int64_t)s * a.vsn + 8 * c);
            *reinterpret_cast<u32x4 *>(&vt[r][8 * c]) = v;
        }
    }
    // D = dO . O and lse per head: four threads per head
    const int h = tid >> 2, part = tid & 3;
    {
        float d = 0.0f;
        if (h < g) {
            const uint16_t *o = a.out + (qh0 + h) * DV, *dob = a.dout + (qh0 + h) * DV;
            for (int c = part; c < DV / 8; c += 4)
                d += dot8(*reinterpret_cast<const u32x4 *>(o + 8 * c), *reinterpret_cast<const u32x4 *>(dob + 8 * c));
        }
        d += __shfl_xor(d, 1, 64);
        d += __shfl_xor(d, 2, 64);
        if (h < g && part == 0) {
            Dh[h] = d;
            lseh[h] = a.lse[qh0 + h];
        }
    }
    __syncthreads();

    // z^T = K_tile q^T and dP^T = V_tile dO^T on v_mfma_f32_32x32x16_bf16 (bf16 products,
    // fp32 sums): one 32 rows x 32 heads block per wave, z blocks first, then dP blocks
    {
        const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, half = lane >> 5;
        const int nhb = (g + 31) / 32;
        if (wave < 2 * nhb) {
            const bool isdp = wave >= nhb;
            const int head = 32 * (isdp ? wave - nhb : wave) + l32;
            const bool hok = head < g;
            f32x16 acc;
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
            // A: key row l32, dims 16 st + 8 half .. +8 (LDS); B: head `head`, the same dims
            if (!isdp) {
                const uint16_t *qp = a.q + (qh0 + (hok ? head : 0)) * DQK + 8 * half;
#pragma unroll 4
                for (int st = 0; st < DQK / 16; ++st) {
                    u32x4 bv = {0, 0, 0, 0};
                    if (hok) bv = *reinterpret_cast<const u32x4 *>(qp + 16 * st);
                    const u32x4 av = *reinterpret_cast<const u32x4 *>(&kt[l32][16 * st + 8 * half]);
                    acc = mfma32(__builtin_bit_cast(bf16x8, av), __builtin_bit_cast(bf16x8, bv), acc);
                }
            } else {
                const uint16_t *op = a.dout + (qh0 + (hok ? head : 0)) * DV + 8 * half;
#pragma unroll 4
                for (int st = 0; st < DV / 16; ++st) {
                    u32x4 bv = {0, 0, 0, 0};
                    if (hok) bv = *reinterpret_cast<const u32x4 *>(op + 16 * st);
                    const uint16_t *vr = MLA ? &kt[l32][16 * st + 8 * half] : &vt[MLA ? 0 : l32][16 * st + 8 * half];
                    const u32x4 av = *reinterpret_cast<const u32x4 *>(vr);
                    acc = mfma32(__builtin_bit_cast(bf16x8, av), __builtin_bit_cast(bf16x8, bv), acc);
                }
            }
            // C: lane holds head column l32, rows 8 (r / 4) + 4 half + r % 4
            float(*dst)[kRT] = isdp ? DPs : Zs;
            if (hok) {
#pragma unroll
                for (int r = 0; r < 16; ++r) dst[head][8 * (r / 4) + 4 * half + (r % 4)] = acc[r];
            }
        }
    }
    __syncthreads();
    // P and scale * dS: thread (h, part) takes rows part + 4 j
    if (h < g) {
        const float lse = lseh[h], D = Dh[h];
#pragma unroll
        for (int j = 0; j < kRT / 4; ++j) {
            const int r = part + 4 * j;
            // a query with no valid row has lse = -inf and no row here with rowpos >= 0
            const float p = (rowpos[r] >= 0 && lse > kNegInf) ? expf(a.scale * Zs[h][r] - lse) : 0.0f;
            Ps[h][r] = p;
            dSs[h][r] = a.scale * (p * (DPs[h][r] - D));
        }
    }
    __syncthreads();

    // The two remaining products run on v_mfma_f32_32x32x16_bf16 too. Their fp32 factors
    // (scale dS, P) enter as a sum of two bf16 values, hi = bf16(x) and lo = bf16(x - hi),
    // so each product carries about 16 significant bits of the factor (two instructions);
    // q, dO and the K rows are bf16 already. Heads past g count as zero.
    const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, half = lane >> 5;
    auto split8 = [](const float (&x)[8], bf16x8 &hi, bf16x8 &lo) {
        u32x4 h, l;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t h0 = f2bf(x[2 * e]), h1 = f2bf(x[2 * e + 1]);
            h[e] = h0 | (h1 << 16);
            l[e] = f2bf(x[2 * e] - u2f(h0 << 16)) | (f2bf(x[2 * e + 1] - u2f(h1 << 16)) << 16);
        }
        hi = __builtin_bit_cast(bf16x8, h);
        lo = __builtin_bit_cast(bf16x8, l);
    };
    const int nks = (g + 15) / 16;  // 16-head steps

    // G rows of this query, 32 columns a block: row r, column c = sum_h A[r][h] B[h][c] with
    // A = scale dS^T and B = q (K part), A = P^T and B = dO (V part; MLA: the first DV
    // columns of the same row)
    float *gout = G + (((int64_t)bt * a.Hkv + kvh) * a.K + r0) * GW;
    for (int cb = wave; cb < GW / 32; cb += kBT / 64) {
        const int c = 32 * cb + l32;
        const bool kpart = 32 * cb < DQK;
        const bool vpart = MLA ? 32 * cb < DV : !kpart;
        const int vc = MLA ? c : c - DQK;
        f32x16 acc;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
        for (int ks = 0; ks < nks; ++ks) {
            const int hb0 = 16 * ks + 8 * half;  // this lane's 8 heads
#pragma unroll
            for (int part = 0; part < 2; ++part) {
                if (part == 0 ? !kpart : !vpart) continue;
                float x[8];
                u32x4 bw;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int hh = hb0 + e;
                    x[e] = hh < g ? (part == 0 ? dSs[hh][l32] : Ps[hh][l32]) : 0.0f;
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    uint32_t w2 = 0;
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
                        const int hh = hb0 + 2 * e + u;
                        const uint32_t v = hh < g ? (uint32_t)(part == 0 ? a.q[(qh0 + hh) * DQK + c]
                                                                           : a.dout[(qh0 + hh) * DV + vc])
                                                  : 0u;
                        w2 |= v << (16 * u);
                    }
                    bw[e] = w2;
                }
                bf16x8 ahi, alo;
                split8(x, ahi, alo);
                const bf16x8 bv = __builtin_bit_cast(bf16x8, bw);
                acc = mfma32(ahi, bv, acc);
                acc = mfma32(alo, bv, acc);
            }
        }
        // C: lane holds column c, rows 8 (r / 4) + 4 half + r % 4
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = 8 * (r / 4) + 4 * half + (r % 4);
            if constexpr (DIRECT) {
                const int pos = rowpos[row];  // -1 for padding and rows past nrows
                if (pos >= 0) {
                    const int64_t rk = ((int64_t)b * a.N + pos) * a.Hkv + kvh;
                    if (c < DQK) a.dk[rk * DQK + c] = acc[r];
                    else a.dv[rk * DV + (c - DQK)] = acc[r];
                }
            } else {
                if (row < nrows) gout[(int64_t)row * GW + c] = acc[r];
            }
        }
    }

    // this tile's part of dq: head h, dim d = sum_r (scale dS)[h][r] K_r[d]
    float *dq = dqp + (((int64_t)bt * a.Hkv + kvh) * ntiles + tile) * g * DQK;
    const int nhb = (g + 31) / 32;
    for (int blk = wave; blk < nhb * (DQK / 32); blk += kBT / 64) {
        const int hb = blk / (DQK / 32), cb = blk % (DQK / 32);
        const int head = 32 * hb + l32, d = 32 * cb + l32;
        f32x16 acc;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
#pragma unroll
        for (int ks = 0; ks < kRT / 16; ++ks) {
            const int rr0 = 16 * ks + 8 * half;  // this lane's 8 rows
            float x[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = head < g ? dSs[head][rr0 + e] : 0.0f;
            u32x4 bw;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                bw[e] = (uint32_t)kt[rr0 + 2 * e][d] | ((uint32_t)kt[rr0 + 2 * e + 1][d] << 16);
            bf16x8 ahi, alo;
            split8(x, ahi, alo);
            const bf16x8 bv = __builtin_bit_cast(bf16x8, bw);
            acc = mfma32(ahi, bv, acc);
            acc = mfma32(alo, bv, acc);
        }
        // C: lane holds dim d, heads 32 hb + 8 (r / 4) + 4 half + r % 4
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int hh = 32 * hb + 8 * (r / 4) + 4 * half + (r % 4);
            if (hh < g) dq[hh * DQK + d] = acc[r];
        }
    }
}

template <int DQK>
__global__ __launch_bounds__(64) void bwd_dq_kernel(AttendBwdArgs a, const float *dqp, int ntiles) {
    const int qh = blockIdx.x;  // (b, t, head) row
    const int g = a.Hq / a.Hkv;
    const int hq = qh % a.Hq, bt = qh / a.Hq;
    const int kvh = hq / g, hh = hq % g;
    const float *src = dqp + (((int64_t)bt * a.Hkv + kvh) * ntiles) * g * DQK + hh * DQK;
    for (int d = threadIdx.x; d < DQK; d += 64) {
        float s = 0.0f;
        for (int t0 = 0; t0 < ntiles; t0 += 8) {  // eight loads in flight, added in tile order
            float v[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = t0 + j < ntiles ? src[(int64_t)(t0 + j) * g * DQK + d] : 0.0f;
#pragma unroll
            for (int j = 0; j < 8; ++j) s += v[j];
        }
        a.dq[(int64_t)qh * DQK + d] = s;
    }
}

// One wave finds the run of slots of an index row (valid entries ascending, padding last)
// whose positions lie in [p0, p0 + kPT): each round samples 64 slots at once and keeps the
// interval where the first slot >= p0 lies, so a row of 2048 entries costs three rounds of
// loads (a binary search by one thread: eleven, then up to kPT more for the run).
__device__ __forceinline__ void wave_find_run(const int32_t *row, int K, int p0, int &lo, int &cnt) {
    const int ln = threadIdx.x & 63;
    auto key = [&](int slot) { const int s = row[slot]; return s < 0 ? 0x7FFFFFFF : s; };
    int lb = 0, hb = K;  // the first slot with key >= p0 lies in [lb, hb] (hb: none below K)
    while (hb - lb > 64) {
        const int S = (hb - lb + 63) / 64;
        const int sl = lb + ln * S;
        const int n = __popcll(__ballot(sl < hb && key(sl) < p0));  // samples below p0 (a prefix)
        if (n == 0) {
            hb = lb;
            break;
        }
        const int nlb = lb + (n - 1) * S + 1;
        hb = min(lb + n * S, hb);
        lb = nlb;
    }
    if (hb > lb) lb += __popcll(__ballot(lb + ln < hb && key(lb + ln) < p0));
    lo = lb;
    cnt = __popcll(__ballot(ln < kPT && lo + ln < K && key(lo + ln) < p0 + kPT));
}

template <int DQK, int DV, bool MLA>
__global__ __launch_bounds__(kBT) void bwd_kv_kernel(AttendBwdArgs a, const float *G) {
    constexpr int GW = g_width<DQK, DV, MLA>();
    constexpr int NC = (GW + kBT - 1) / kBT;  // columns per thread
    __shared__ __attribute__((aligned(16))) float acc[kPT][GW];
    __shared__ int lo_s[kBT], cnt_s[kBT];
    __shared__ int hit[kPT];  // a query selected position p0 + r
    const int tid = threadIdx.x;
    const int p0 = blockIdx.x * kPT, b = blockIdx.y, kvh = blockIdx.z;
    bool touched = false;  // some query selected a position of the tile (uniform)
    for (int t0 = 0; t0 < a.T; t0 += kBT) {
        // thread j finds the slots of query t0 + j whose positions fall in [p0, p0 + kPT):
        // valid entries ascend and padding (-1) comes last, so they are one run of slots
        const int t = t0 + tid;
        int lo = 0, cnt = 0, entry = tid;  // entry: the lo_s / cnt_s slot this thread fills, or -1
        if (a.T <= kBT / 64) {
            // few queries (decode): wave w searches query w, 64 slots per round of loads
            const int w = tid >> 6;
            entry = (tid & 63) == 0 ? w : -1;
            if (w < a.T) wave_find_run(a.idx + ((int64_t)b * a.T + w) * a.K, a.K, p0, lo, cnt);
        } else if (t < a.T) {
            const int32_t *row = a.idx + ((int64_t)b * a.T + t) * a.K;
            auto key = [&](int slot) { const int s = row[slot]; return s < 0 ? 0x7FFFFFFF : s; };
            int hi = a.K;
            while (lo < hi) {  // first slot with key >= p0
                const int mid = (lo + hi) >> 1;
                if (key(mid) < p0) lo = mid + 1;
                else hi = mid;
            }
            while (lo + cnt < a.K && cnt < kPT && key(lo + cnt) < p0 + kPT) ++cnt;
        }
        __syncthreads();  // the previous chunk is done with lo_s / cnt_s
        if (entry >= 0) {
            lo_s[entry] = lo;
            cnt_s[entry] = cnt;
        }
        const bool any = __syncthreads_or(entry >= 0 && cnt > 0);
        if (!any) continue;
        if (!touched) {  // first contributions: clear the accumulators
            for (int i = tid; i < kPT * GW; i += kBT) (&acc[0][0])[i] = 0.0f;
            if (tid < kPT) hit[tid] = 0;
            __syncthreads();
            touched = true;
        }
        const int nt = min(kBT, a.T - t0);
        for (int j = 0; j < nt; ++j) {  // ascending query order
            const int tt = t0 + j;
            const int32_t *row = a.idx + ((int64_t)b * a.T + tt) * a.K;
            const float *gq = G + (((int64_t)b * a.T + tt) * a.Hkv + kvh) * a.K * GW;
            for (int e = 0; e < cnt_s[j]; ++e) {
                const int slot = lo_s[j] + e;
                const int pos = row[slot];
                if (pos < p0 || pos >= p0 + kPT || pos >= a.N) continue;  // (rows not ascending: skipped)
                const float *gr = gq + (int64_t)slot * GW;
                if (tid == 0) hit[pos - p0] = 1;
#pragma unroll
                for (int i = 0; i < NC; ++i) {
                    const int c = tid + kBT * i;
                    if (c < GW) acc[pos - p0][c] += gr[c];
                }
            }
        }
    }
    if (!touched) return;  // nothing selected a position of the tile: nothing is written
    __syncthreads();
    // the selected positions of the tile: 16-byte stores
    for (int e = tid; e < kPT * GW / 4; e += kBT) {
        const int r = e / (GW / 4), c = 4 * (e % (GW / 4));
        const int pos = p0 + r;
        if (pos >= a.N) break;
        if (!hit[r]) continue;
        const int64_t rowk = ((int64_t)b * a.N + pos) * a.Hkv + kvh;
        float *dst = c < DQK ? a.dk + rowk * DQK + c : a.dv + rowk * DV + (c - DQK);
        *reinterpret_cast<f32x4 *>(dst) = *reinterpret_cast<const f32x4 *>(&acc[r][c]);
    }
}

// ---- indexer distillation target
// target_tile_kernel (one workgroup per query token and 32 selected rows): for each KV head
// in turn, the rows are gathered into LDS and q . K of every head of the group comes from
// the matrix cores; each row's thread adds exp(scale z - lse) over the heads (KV heads in
// order), then divides by Hq.
template <int DQK>
__global__ __launch_bounds__(kBT) void target_tile_kernel(IndexTargetArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t kt[kRT][DQK];
    __shared__ float Zs[kMaxG][kRT];
    __shared__ int rowpos[kRT];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l32 = lane & 31, half = lane >> 5;
    const int tile = blockIdx.x, bt = blockIdx.y;
    const int b = bt / a.T;
    const int g = a.Hq / a.Hkv;
    const int r0 = tile * kRT;
    const int nrows = min(kRT, a.K - r0);
    if (tid < kRT) {
        const int s = tid < nrows ? a.idx[(int64_t)bt * a.K + r0 + tid] : -1;
        rowpos[tid] = (s >= 0 && s < a.N) ? s : -1;
    }
    float tgt = 0.0f;  // thread r < kRT: row r's sum over heads
    for (int kvh = 0; kvh < a.Hkv; ++kvh) {
        __syncthreads();  // rowpos written; the previous head's kt and Zs no longer read
        const uint16_t *kb = a.k + b * a.ksb + kvh * a.ksh;
        for (int i = tid; i < kRT * DQK / 8; i += kBT) {
            const int r = i / (DQK / 8), c = i % (DQK / 8);
            const int s = rowpos[r];
            u32x4 v = {0, 0, 0, 0};
            if (s >= 0) v = *reinterpret_cast<const u32x4 *>(kb + (int64_t)s * a.ksn + 8 * c);
            *reinterpret_cast<u32x4 *>(&kt[r][8 * c]) = v;
        }
        __syncthreads();
        const int64_t qh0 = (int64_t)bt * a.Hq + kvh * g;
        if (wave < (g + 31) / 32) {  // z^T block: 32 rows x 32 heads
            const int head = 32 * wave + l32;
            const bool hok = head < g;
            const uint16_t *qp = a.q + (qh0 + (hok ? head : 0)) * DQK + 8 * half;
            f32x16 acc;
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
#pragma unroll 4
            for (int st = 0; st < DQK / 16; ++st) {
                u32x4 bv = {0, 0, 0, 0};
                if (hok) bv = *reinterpret_cast<const u32x4 *>(qp + 16 * st);
                const u32x4 av = *reinterpret_cast<const u32x4 *>(&kt[l32][16 * st + 8 * half]);
                acc = mfma32(__builtin_bit_cast(bf16x8, av), __builtin_bit_cast(bf16x8, bv), acc);
            }
            if (hok) {
#pragma unroll
                for (int r = 0; r < 16; ++r) Zs[head][8 * (r / 4) + 4 * half + (r % 4)] = acc[r];
            }
        }
        __syncthreads();
        if (tid < kRT && rowpos[tid] >= 0) {
            for (int hh = 0; hh < g; ++hh) {
                const float lse = a.lse[qh0 + hh];
                if (lse > kNegInf) tgt += expf(a.scale * Zs[hh][tid] - lse);
            }
        }
    }
    if (tid < nrows) a.target[(int64_t)bt * a.K + r0 + tid] = rowpos[tid] >= 0 ? tgt / (float)a.Hq : 0.0f;
}

// fixed-order sum or maximum over the workgroup (kBT threads)
template <bool MAX>
__device__ float block_reduce(float v, float *scr) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float w = __shfl_xor(v, o, 64);
        v = MAX ? fmaxf(v, w) : v + w;
    }
    __syncthreads();  // scr free
    if ((tid & 63) == 0) scr[tid >> 6] = v;
    __syncthreads();
    float r = scr[0];
    for (int i = 1; i < kBT / 64; ++i) r = MAX ? fmaxf(r, scr[i]) : r + scr[i];
    return r;
}

// kl_kernel (one workgroup per query token): u = softmax of the indexer scores over the
// valid entries, loss = sum target (log target - log u), grad = u - target
__global__ __launch_bounds__(kBT) void kl_kernel(IndexTargetArgs a) {
    __shared__ float scr[kBT / 64];
    const int tid = threadIdx.x, bt = blockIdx.x;
    const int32_t *row = a.idx + (int64_t)bt * a.K;
    const float *sc = a.scores + (int64_t)bt * a.n_cols;
    const float *tg = a.target + (int64_t)bt * a.K;
    float m = kNegInf;
    for (int j = tid; j < a.K; j += kBT) {
        const int s = row[j];
        if (s >= 0 && s < a.N) m = fmaxf(m, sc[s]);
    }
    m = block_reduce<true>(m, scr);
    float se = 0.0f;
    for (int j = tid; j < a.K; j += kBT) {
        const int s = row[j];
        if (s >= 0 && s < a.N) se += expf(sc[s] - m);
    }
    se = block_reduce<false>(se, scr);
    const float lz = m + logf(se);  // log of the softmax denominator
    float loss = 0.0f;
    for (int j = tid; j < a.K; j += kBT) {
        const int s = row[j];
        const bool ok = s >= 0 && s < a.N && m > kNegInf;
        const float lu = ok ? sc[s] - lz : 0.0f, t = tg[j];
        if (ok && t > 0.0f) loss += t * (logf(t) - lu);
        a.grad[(int64_t)bt * a.K + j] = ok ? expf(lu) - t : 0.0f;
    }
    loss = block_reduce<false>(loss, scr);
    if (tid == 0) a.loss[bt] = loss;
}

struct BwdLayout {
    size_t g_off, g_bytes, dq_off, dq_bytes, total;
    int ntiles;
};

BwdLayout bwd_layout(const AttendBwdArgs &a) {
    const int DQK = a.mla ? 576 : 128, DV = a.mla ? 512 : 128;
    const int GW = a.mla ? DQK : DQK + DV;
    BwdLayout l;
    l.ntiles = (a.K + kRT - 1) / kRT;
    l.g_off = 0;
    l.g_bytes = a.T == 1 ? 0 : (size_t)a.B * a.T * a.Hkv * a.K * GW * sizeof(float);  // T == 1: no G
    l.dq_off = (l.g_bytes + 255) / 256 * 256;
    l.dq_bytes = (size_t)a.B * a.T * a.Hq * l.ntiles * DQK * sizeof(float);
    l.total = l.dq_off + l.dq_bytes;
    return l;
}

template <int DQK, int DV, bool MLA>
hipError_t launch_bwd_t(const AttendBwdArgs &a, void *ws, hipStream_t s) {
    const BwdLayout l = bwd_layout(a);
    float *G = reinterpret_cast<float *>(static_cast<unsigned char *>(ws) + l.g_off);
    float *dqp = reinterpret_cast<float *>(static_cast<unsigned char *>(ws) + l.dq_off);
    const dim3 rgrid(l.ntiles, a.B * a.T, a.Hkv);
    if (a.T == 1) hipLaunchKernelGGL((bwd_rows_kernel<DQK, DV, MLA, true>), rgrid, dim3(kBT), 0, s, a, G, dqp);
    else hipLaunchKernelGGL((bwd_rows_kernel<DQK, DV, MLA, false>), rgrid, dim3(kBT), 0, s, a, G, dqp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_dq_kernel<DQK>), dim3(a.B * a.T * a.Hq), dim3(64), 0, s, a, dqp, l.ntiles);
    if ((e = hipGetLastError()) != hipSuccess || a.T == 1) return e;
    hipLaunchKernelGGL((bwd_kv_kernel<DQK, DV, MLA>), dim3((a.N + kPT - 1) / kPT, a.B, a.Hkv), dim3(kBT), 0, s, a, G);
    return hipGetLastError();
}

}  // namespace

size_t attend_bwd_workspace_bytes(const AttendBwdArgs &a) { return bwd_layout(a).total; }

hipError_t launch_index_target(const IndexTargetArgs &a, hipStream_t s) {
    const dim3 grid((a.K + kRT - 1) / kRT, a.B * a.T);
    if (a.dqk == 576) hipLaunchKernelGGL(target_tile_kernel<576>, grid, dim3(kBT), 0, s, a);
    else hipLaunchKernelGGL(target_tile_kernel<128>, grid, dim3(kBT), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kl_kernel, dim3(a.B * a.T), dim3(kBT), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_attend_bwd(const AttendBwdArgs &a, void *ws, hipStream_t s) {
    return a.mla ? launch_bwd_t<576, 512, true>(a, ws, s) : launch_bwd_t<128, 128, false>(a, ws, s);
}

}  // namespace lsa
