// nvfp4_norm.hip -- residual add + RMSNorm for gfx950, the step that produces a
// projection's activations (the Qwen3.8-27B-NVFP4 blueprint page's kernel
// table: norm::residual_add_rms_norm; kern's gemma_rms_norm is the variant
// with the Gemma offset).
//
// Per row: v = bf16(r + h) is the new residual stream (stored as r_out, which
// may be r itself), x = bf16(v * w' / sqrt(mean(v^2) + eps)) with w' = w or
// 1 + w; fp32 arithmetic.  One workgroup per row; each thread keeps its
// chunks of v in registers between the sum of squares and the scaling, so an
// in-place residual never has to be read back.  The sum of squares runs in a
// fixed order (per thread, then a fixed butterfly, then waves in order):
// results are bitwise deterministic.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nvfp4_internal.h"

namespace nvfp4 {
namespace {

constexpr int kNormThreads = 256;
constexpr int kRsrcWord3 = 0x00020000;
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

struct NormArgs {
    const uint16_t *r, *h, *w;
    uint16_t *r_out, *x;
    int k, rows, gemma_offset;
    float eps;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, kRsrcWord3);
}

__device__ __forceinline__ float lo_f(uint32_t u) { return __builtin_bit_cast(float, u << 16); }
__device__ __forceinline__ float hi_f(uint32_t u) { return __builtin_bit_cast(float, u & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even (NaN stays a quiet NaN)
__device__ __forceinline__ uint32_t rne(float f) {
    const uint32_t u = __builtin_bit_cast(uint32_t, f);
    const uint32_t r = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
    return (u & 0x7FFFFFFFu) > 0x7F800000u ? ((u >> 16) | 0x40u) : r;
}

// CPT: 16-byte chunks (8 values) per thread, kNormThreads * CPT * 8 >= k.
template <int CPT>
__global__ __launch_bounds__(kNormThreads) void norm_kernel(NormArgs a) {
    __shared__ float wsum[kNormThreads / 64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const size_t row0 = (size_t)blockIdx.x * a.k;
    const uint32_t rb = (uint32_t)a.k * 2;
    const __amdgpu_buffer_rsrc_t rr = make_rsrc(a.r + row0, rb), hr = make_rsrc(a.h + row0, rb);
    const __amdgpu_buffer_rsrc_t ror = make_rsrc(a.r_out + row0, rb), xr = make_rsrc(a.x + row0, rb);
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(a.w, rb);
    // pass 1: v = bf16(r + h), stored; sum of squares
    u32x4_t v[CPT];
    float ss = 0.0f;
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
        const int off = (tid + kNormThreads * j) * 16;   // past the row: loads read 0, stores are dropped
        const u32x4_t rv = __builtin_amdgcn_raw_buffer_load_b128(rr, off, 0, 0);
        const u32x4_t hv = __builtin_amdgcn_raw_buffer_load_b128(hr, off, 0, 0);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t lo = rne(lo_f(rv[e]) + lo_f(hv[e])), hi = rne(hi_f(rv[e]) + hi_f(hv[e]));
            v[j][e] = lo | (hi << 16);
            const float fl = lo_f(v[j][e]), fh = hi_f(v[j][e]);
            ss = __builtin_fmaf(fl, fl, ss);
            ss = __builtin_fmaf(fh, fh, ss);
        }
        __builtin_amdgcn_raw_buffer_store_b128(v[j], ror, off, 0, 0);
    }
    // fixed-order reduction: butterfly within the wave, then the waves in order
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m);
    if (lane == 0) wsum[wave] = ss;
    __syncthreads();
    float tot = wsum[0];
#pragma unroll
    for (int i = 1; i < kNormThreads / 64; ++i) tot += wsum[i];
    const float inv = 1.0f / __builtin_sqrtf(tot / (float)a.k + a.eps);
    // pass 2: x = bf16(v * inv * w')
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
        const int off = (tid + kNormThreads * j) * 16;
        const u32x4_t wv = __builtin_amdgcn_raw_buffer_load_b128(wr, off, 0, 0);
        u32x4_t xv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float wl = lo_f(wv[e]), wh = hi_f(wv[e]);
            if (a.gemma_offset) {
                wl += 1.0f;
                wh += 1.0f;
            }
            xv[e] = rne(lo_f(v[j][e]) * inv * wl) | (rne(hi_f(v[j][e]) * inv * wh) << 16);
        }
        __builtin_amdgcn_raw_buffer_store_b128(xv, xr, off, 0, 0);
    }
}

template <int CPT>
hipError_t launch_cpt(const NormArgs &a, hipStream_t s) {
    hipLaunchKernelGGL(norm_kernel<CPT>, dim3((unsigned)a.rows), dim3(kNormThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace

int64_t norm_max_k() { return (int64_t)kNormThreads * 32 * 8; }

hipError_t launch_residual_rmsnorm(const void *r, const void *h, const void *w, int64_t k, int rows, float eps,
                                   int gemma_offset, void *r_out, void *x, hipStream_t stream) {
    NormArgs a{};
    a.r = static_cast<const uint16_t *>(r);
    a.h = static_cast<const uint16_t *>(h);
    a.w = static_cast<const uint16_t *>(w);
    a.r_out = static_cast<uint16_t *>(r_out);
    a.x = static_cast<uint16_t *>(x);
    a.k = (int)k;
    a.rows = rows;
    a.gemma_offset = gemma_offset;
    a.eps = eps;
    const int64_t chunks = (k / 8 + kNormThreads - 1) / kNormThreads;
    if (chunks <= 1) return launch_cpt<1>(a, stream);
    if (chunks <= 2) return launch_cpt<2>(a, stream);
    if (chunks <= 4) return launch_cpt<4>(a, stream);
    if (chunks <= 8) return launch_cpt<8>(a, stream);
    if (chunks <= 16) return launch_cpt<16>(a, stream);
    if (chunks <= 32) return launch_cpt<32>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace nvfp4
