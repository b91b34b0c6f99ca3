// Cache append: the write side of a decode step. SI's local window ends at the current
// token, so a step's new rows must be in the caches before the step reads them; HI's
// coarse pass reads one summary per key block, which is brought up to date when an append
// writes a block's last row ("LongCat-Flash-Lite-Sparse" summary, aitrends.kr,
// "Technical features", first and third bullets).
//
// append_kernel: one wave per new token. The indexer key (bf16) is quantised per token:
//   scale = max(max_d |k|, 1e-12) / 448, byte = e4m3fn(clamp(k / scale, +-448)),
// in fp32 with correctly rounded divisions and the hardware's round-to-nearest-even
// conversion (or copied to a bf16 key cache); the token's KV rows are copied with 16-byte
// loads and stores.
// append_kbar_kernel (second launch, after every key is written): for each block whose
// last row the append wrote, the block's mean dequantised key, computed exactly as the
// summary kernel does.
#include "common.cuh"
#include "kernels.h"

namespace lsa {
namespace {

template <int D>
__global__ __launch_bounds__(64) void append_kernel(CacheAppendArgs a) {
    const int t = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
    const int p0 = a.pos0 ? a.pos0[b] : a.N - a.T;
    const int s = p0 + t;
    if (s < 0 || s >= a.N) return;
    constexpr int PER = D / 64;  // key elements per lane
    const uint16_t *kn = a.k_new + ((int64_t)b * a.T + t) * D;
    float v[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) v[e] = u2f((uint32_t)kn[lane + 64 * e] << 16);
    const int64_t row = (int64_t)b * a.N + s;
    if (a.fp8) {
        float m = 0.0f;
#pragma unroll
        for (int e = 0; e < PER; ++e) m = fmaxf(m, fabsf(v[e]));
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
        const float scale = fmaxf(m, 1e-12f) / 448.0f;
        uint8_t *kc = reinterpret_cast<uint8_t *>(a.k_cache) + row * D;
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            const float y = fminf(fmaxf(v[e] / scale, -448.0f), 448.0f);
            kc[lane + 64 * e] = (uint8_t)(__builtin_amdgcn_cvt_pk_fp8_f32(y, y, 0, false) & 0xFF);
        }
        if (lane == 0) a.k_scale[row] = scale;
    } else {
        uint16_t *kc = reinterpret_cast<uint16_t *>(a.k_cache) + row * D;
#pragma unroll
        for (int e = 0; e < PER; ++e) kc[lane + 64 * e] = kn[lane + 64 * e];
    }
    for (int r = 0; r < a.n_rows; ++r) {
        const u32x4 *src = reinterpret_cast<const u32x4 *>(a.rows_new[r] + ((int64_t)b * a.T + t) * a.row_elems[r]);
        u32x4 *dst = reinterpret_cast<u32x4 *>(a.rows_cache[r] + b * a.stride_b[r] + (int64_t)s * a.stride_n[r]);
        const int n16 = (int)(a.row_elems[r] / 8);
        for (int i = lane; i < n16; i += 64) dst[i] = src[i];
    }
}

// blockIdx.x = k: the k-th row in [p0, p0 + T) that ends a block.
__global__ __launch_bounds__(128) void append_kbar_kernel(CacheAppendArgs a) {
    const int k = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
    if (d >= a.D) return;
    const int Bs = a.block_size;
    const int p0 = a.pos0 ? a.pos0[b] : a.N - a.T;
    const int lo = max(p0, 0), hi = min(p0 + a.T, a.N);  // rows written: [lo, hi)
    const int64_t first = ((int64_t)lo + Bs) / Bs * Bs - 1;  // smallest row >= lo ending a block
    const int64_t last_row = first + (int64_t)k * Bs;
    if (last_row >= hi) return;
    const int64_t j = last_row / Bs;
    if (j >= a.n_blocks) return;
    const int64_t row0 = (int64_t)b * a.N + j * Bs;
    a.kbar[((int64_t)b * a.n_blocks + j) * a.D + d] = block_mean_d(a.k_cache, a.fp8, a.k_scale, row0, Bs, a.D, d);
}

}  // namespace

hipError_t launch_cache_append(const CacheAppendArgs &a, hipStream_t s) {
    if (a.D == 64) hipLaunchKernelGGL(append_kernel<64>, dim3(a.T, a.B), dim3(64), 0, s, a);
    else hipLaunchKernelGGL(append_kernel<128>, dim3(a.T, a.B), dim3(64), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !a.kbar) return e;
    const int nb = a.T / a.block_size + 1;  // rows ending a block among T consecutive rows
    hipLaunchKernelGGL(append_kbar_kernel, dim3(nb, a.B), dim3(128), 0, s, a);
    return hipGetLastError();
}

}  // namespace lsa
