// Device helpers shared by the LSA kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lsa {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// ---- MFMA (gfx950). Lane layouts verified on the device:
// 16x16x32: A lane l holds A[l%16][8*(l/16)+e], B lane l holds B[8*(l/16)+e][l%16],
//           D lane l holds D[4*(l/16)+r][l%16], r = 0..3.
// 32x32x16: A lane l holds A[l%32][8*(l/32)+e], B lane l holds B[8*(l/32)+e][l%32],
//           D lane l holds D[8*(r/4)+4*(l/32)+r%4][l%32], r = 0..15.
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// 32x32 fp32 += (32 x 64 e4m3) x (64 x 32 e4m3), unscaled (v_mfma_f32_32x32x64_f8f6f4):
// lane l supplies 32 bytes of row (A) / column (B) l % 32; lanes l and l + 32 hold
// complementary halves of the 64-long contraction, the same for A and B, so any fixed
// assignment of contraction indices to (lane half, byte) shared by both operands sums
// every index once
typedef __attribute__((ext_vector_type(8))) int i32x8;
__device__ __forceinline__ f32x16 mfma32_fp8(i32x8 a, i32x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// ---- bit casts
__device__ __forceinline__ uint32_t f2u(float x) { return __builtin_bit_cast(uint32_t, x); }
__device__ __forceinline__ float u2f(uint32_t x) { return __builtin_bit_cast(float, x); }

// bf16 bits -> fp32 (exact)
__device__ __forceinline__ float bf16lo(uint32_t two) { return u2f(two << 16); }
__device__ __forceinline__ float bf16hi(uint32_t two) { return u2f(two & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even (finite values)
__device__ __forceinline__ uint32_t f2bf(float x) {
    uint32_t u = f2u(x);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) { return f2bf(lo) | (f2bf(hi) << 16); }

// Upper halves of two fp32 words -> one packed bf16 pair (exact for values that are
// already bf16-representable, e.g. widened fp8).
__device__ __forceinline__ uint32_t hi_halves(uint32_t lo_word, uint32_t hi_word) {
    return __builtin_amdgcn_perm(hi_word, lo_word, 0x07060302u);
}

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;

// Four OCP e4m3fn bytes (one dword) -> four bf16 (two dwords), exact (every e4m3 value
// is a bf16 value): gfx950 v_cvt_scalef32_pk_bf16_fp8 with scale 1.
__device__ __forceinline__ void fp8x4_to_bf16x4(uint32_t v, uint32_t &o0, uint32_t &o1) {
    o0 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v, 1.0f, false));
    o1 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v, 1.0f, true));
}

// max(x, 0) on the bit pattern: a float with the sign bit set is a negative int32.
__device__ __forceinline__ float relu_bits(float x) {
    return __builtin_bit_cast(float, max(__builtin_bit_cast(int32_t, x), 0));
}

// 16 fp8 bytes -> two bf16x8 fragments (first 8 bytes, last 8 bytes).
__device__ __forceinline__ void fp8x16_to_frags(u32x4 v, bf16x8 &f0, bf16x8 &f1) {
    uint32_t a0, a1, a2, a3, b0, b1, b2, b3;
    fp8x4_to_bf16x4(v[0], a0, a1);
    fp8x4_to_bf16x4(v[1], a2, a3);
    fp8x4_to_bf16x4(v[2], b0, b1);
    fp8x4_to_bf16x4(v[3], b2, b3);
    u32x4 a = {a0, a1, a2, a3};
    u32x4 b = {b0, b1, b2, b3};
    f0 = __builtin_bit_cast(bf16x8, a);
    f1 = __builtin_bit_cast(bf16x8, b);
}

// ---- order-preserving fp32 -> uint32 map (larger float -> larger key).
// -0.0 is folded onto +0.0 first so that the two compare equal.
__device__ __forceinline__ uint32_t order_key(float x) {
    uint32_t u = f2u(x + 0.0f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---- HI block summary: element d of the mean dequantised key of the Bs rows starting at
// row0 (fp8 bytes times the per-token scale, or bf16), summed in row order in fp32. The
// summary kernel and the cache append both use this, so their results agree bit for bit.
// Loads go 64 rows at a time (clamped to the block; one memory round trip for a block of
// 64, the key type chosen outside the unrolled loads); the sum stays in row order, one
// fused multiply-add per fp8 row.
__device__ __forceinline__ float block_mean_d(const void *k, bool fp8, const float *k_scale, int64_t row0, int Bs,
                                              int D, int d) {
    constexpr int R = 64;
    float acc = 0.0f;
    if (fp8) {
        const uint8_t *k8 = reinterpret_cast<const uint8_t *>(k);
        for (int s0 = 0; s0 < Bs; s0 += R) {
            uint32_t byte[R];
            float sc[R];
#pragma unroll
            for (int u = 0; u < R; ++u) {
                const int64_t r = row0 + min(s0 + u, Bs - 1);
                byte[u] = k8[r * D + d];
                sc[u] = k_scale[r];
            }
#pragma unroll
            for (int u = 0; u < R; ++u)
                if (s0 + u < Bs) acc = __builtin_fmaf(sc[u], __builtin_amdgcn_cvt_pk_f32_fp8(byte[u], false)[0], acc);
        }
    } else {
        const uint16_t *k16 = reinterpret_cast<const uint16_t *>(k);
        for (int s0 = 0; s0 < Bs; s0 += R) {
            uint32_t h[R];
#pragma unroll
            for (int u = 0; u < R; ++u) h[u] = k16[(row0 + min(s0 + u, Bs - 1)) * D + d];
#pragma unroll
            for (int u = 0; u < R; ++u)
                if (s0 + u < Bs) acc += u2f(h[u] << 16);
        }
    }
    return acc / (float)Bs;
}

// ---- SI forced set at query position p: sink [0, sink_end) and window [win_lo, p]
// (empty when win_lo > p); where the two overlap the window starts after the sink.
__device__ __forceinline__ void forced_bounds(int p, int sink, int window, int &sink_end, int &win_lo) {
    const int pe = max(p + 1, 0);
    sink_end = min(sink, pe);
    win_lo = window > 0 ? max(sink_end, p - window + 1) : pe;
    win_lo = max(win_lo, 0);
}

// First-level selection histogram: candidates counted per bin order_key(score) >> 21
// (sign, exponent and two mantissa bits). Written by the selection's histogram pass or
// by the indexer epilogue, read by the selection's row pass.
constexpr int kSelBins = 2048;
constexpr int kSelShift = 21;

// ---- wave reductions (wave64)

// v[l] + v[l ^ 32] in every lane. v_permlane32_swap exchanges the upper half-wave of
// its first operand with the lower half-wave of its second; with both operands holding
// v, the two results hold v[l] and v[l ^ 32] between them. Written as inline asm with
// both operands read-write: this compiler's builtin for the instruction returns the
// first result for both. The s_nop pads cover the VALU-write -> permlane-read hazard.
__device__ __forceinline__ float half_pair_sum(float v) {
    uint32_t x = __builtin_bit_cast(uint32_t, v), y = x;
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(x), "+v"(y));
    return __builtin_bit_cast(float, x) + __builtin_bit_cast(float, y);
}
__device__ __forceinline__ float wave_xor_f(float v, int mask) { return __shfl_xor(v, mask, 64); }

template <typename T>
__device__ __forceinline__ T ld_nt(const T *p) { return __builtin_nontemporal_load(p); }

}  // namespace lsa
