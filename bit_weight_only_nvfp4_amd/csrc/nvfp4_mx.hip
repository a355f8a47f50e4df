// nvfp4_mx.hip -- MXFP4 projection for gfx950: E2M1 codes with one E8M0
// power-of-two scale per 32 consecutive k of a row (the microscaling format
// the pages name through the kern build's gpu_mxfp4 kernels), read in the
// format's own row-major layout: codes [n][k/2] (low nibble first), scales
// [n][k/32].
//
// y[r][j] = sum_k e2m1(code[j][k]) * 2^(scale[j][k/32] - 127) * x[r][k], fp32
// accumulation, rows <= 16 per launch.
//
// gfx950 converts E2M1 pairs to bf16 with a power-of-two scale applied by the
// conversion itself (v_cvt_scalef32_pk_bf16_fp4 takes the scale's exponent):
// with the E8M0 byte placed in an fp32 exponent, one instruction dequantizes
// two weights exactly (a code has 2 significant bits; bf16 holds every
// code * 2^e for e in -126..125).  The activations then feed the bf16 matrix
// cores as stored: no activation staging, no scale multiply.
//   * one workgroup per 64 features (four 16-feature products), 4 waves each
//     over a quarter of k in steps of 128; two steps in flight;
//   * per step a lane (q, n) takes k = 32 q .. 32 q + 31 of the step -- one MX
//     block, so one scale byte per feature block -- as 16 bytes of codes per
//     feature block and 64 bytes of its activation row; product m of the step
//     uses k = 32 q + 8 m .. + 7 in both operands;
//   * the waves' sums are added in LDS in wave order (deterministic).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nvfp4_internal.h"

namespace nvfp4 {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kMxFB = 4;            // 16-feature blocks per workgroup
constexpr int kMxFeatures = 16 * kMxFB;
constexpr int kMxWaves = 4;
constexpr int kMxStepK = 128;
// Steps in flight per wave.  Measured on a [151936 x 5120] matrix: 2 (116
// registers, four waves per SIMD) 130 us at 1 row against 138 with 4 (176
// registers); 128 features per workgroup with 3 steps 134 us.  The kernel is
// far from its bytes (about 3 TB/s): each step also makes as many scale-byte
// requests (16 rows per feature block) as code requests.
constexpr int kMxBufs = 2;
constexpr int kRsrcWord3 = 0x00020000;
constexpr int kDeviceCoherent = 16;
constexpr int kDropped = 0x7fffffff;
// An offset past every buffer of a workgroup (codes: at most 64 x 2^23 bytes,
// scales 64 x 2^19, activations 16 x 2^25): the load reads zeros.
constexpr int kOutside = 1 << 30;

struct MxArgs {
    const uint8_t *codes, *scales;
    const uint16_t *x;
    void *y;
    int n, k, rows, out_f32;
    int kw;   // k per wave, a multiple of kMxStepK
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, kRsrcWord3);
}

struct MxStep {
    u32x4_t c[kMxFB];     // codes: k = 32 q .. + 31 of each feature block's row n
    uint32_t s[kMxFB];    // its E8M0 scale byte
    u32x4_t a[4];         // activations of row n, k = 32 q .. + 31
};

__device__ __forceinline__ void load_step(__amdgpu_buffer_rsrc_t cr, __amdgpu_buffer_rsrc_t sr,
                                          __amdgpu_buffer_rsrc_t xr, int k0, int kend, int k, int q, int n16,
                                          MxStep &st) {
    const int kk = k0 + 32 * q;
    const bool in = kk < kend;   // k is a multiple of 32: a lane's block is all in or all out
    const int kh = k / 2, kb = k / 32;
    const int co = in ? n16 * kh + kk / 2 : kOutside;
    const int so = in ? n16 * kb + kk / 32 : kOutside;
    const int xo = in ? (n16 * k + kk) * 2 : kOutside;
#pragma unroll
    for (int fb = 0; fb < kMxFB; ++fb) {
        st.c[fb] = __builtin_amdgcn_raw_buffer_load_b128(cr, co + fb * 16 * kh, 0, 0);
        st.s[fb] = __builtin_amdgcn_raw_buffer_load_b8(sr, so + fb * 16 * kb, 0, 0);
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) st.a[m] = __builtin_amdgcn_raw_buffer_load_b128(xr, xo + 16 * m, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
}

// Eight codes (one word, low nibble first) times 2^(e - 127) as bf16.
__device__ __forceinline__ bf16x8_t dequant8(uint32_t w, float scale) {
    const bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0);
    const bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1);
    const bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2);
    const bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3);
    return bf16x8_t{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

__device__ __forceinline__ void mac_step(const MxStep &st, f32x4_t (&d)[kMxFB]) {
    float sc[kMxFB];
#pragma unroll
    for (int fb = 0; fb < kMxFB; ++fb) sc[fb] = __builtin_bit_cast(float, (st.s[fb] & 0xffu) << 23);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const bf16x8_t a = __builtin_bit_cast(bf16x8_t, st.a[m]);
#pragma unroll
        for (int fb = 0; fb < kMxFB; ++fb)
            d[fb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, dequant8(st.c[fb][m], sc[fb]), d[fb], 0, 0, 0);
    }
}

__device__ __forceinline__ uint16_t bf16_rne(float f) {
    const uint32_t u = __builtin_bit_cast(uint32_t, f);
    const uint32_t rne = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
    const uint32_t nan = (u >> 16) | 0x40u;
    return (uint16_t)((u & 0x7FFFFFFFu) > 0x7F800000u ? nan : rne);
}

__global__ __launch_bounds__(kMxWaves * 64) void mx_kernel(MxArgs a) {
    __shared__ float red[kMxWaves][kMxFB][16][16];   // [wave][feature block][row][feature]
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int q = lane >> 4, n16 = lane & 15;
    const int f0 = blockIdx.x * kMxFeatures;
    const int nf = min(kMxFeatures, a.n - f0);
    const __amdgpu_buffer_rsrc_t cr = make_rsrc(a.codes + (size_t)f0 * (a.k / 2), (uint32_t)((size_t)nf * a.k / 2));
    const __amdgpu_buffer_rsrc_t sr = make_rsrc(a.scales + (size_t)f0 * (a.k / 32), (uint32_t)((size_t)nf * a.k / 32));
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.x, (uint32_t)((size_t)a.rows * a.k * 2));
    const int kb = wave * a.kw, ke = min(a.k, kb + a.kw);
    const int steps = ke > kb ? (ke - kb + kMxStepK - 1) / kMxStepK : 0;
    f32x4_t d[kMxFB];
#pragma unroll
    for (int fb = 0; fb < kMxFB; ++fb) d[fb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    MxStep st[kMxBufs];
#pragma unroll
    for (int i = 0; i < kMxBufs; ++i) load_step(cr, sr, xr, kb + i * kMxStepK, ke, a.k, q, n16, st[i]);
    // steps past the wave's last are loaded (reading nothing) but not used,
    // so the loads in flight never depend on control flow
    for (int j = 0; j < steps; j += kMxBufs) {
#pragma unroll
        for (int i = 0; i < kMxBufs; ++i) {
            if (j + i < steps) mac_step(st[i], d);
            load_step(cr, sr, xr, kb + (j + i + kMxBufs) * kMxStepK, ke, a.k, q, n16, st[i]);
        }
    }
#pragma unroll
    for (int fb = 0; fb < kMxFB; ++fb)
#pragma unroll
        for (int v = 0; v < 4; ++v) red[wave][fb][4 * q + v][n16] = d[fb][v];
    __syncthreads();
    const __amdgpu_buffer_rsrc_t yr = make_rsrc(a.y, (uint32_t)((size_t)a.rows * a.n * (a.out_f32 ? 4 : 2)));
#pragma unroll
    for (int o = tid; o < 16 * kMxFeatures; o += kMxWaves * 64) {
        const int r = o / kMxFeatures, f = o % kMxFeatures;
        float t = red[0][f >> 4][r][f & 15];
#pragma unroll
        for (int w = 1; w < kMxWaves; ++w) t += red[w][f >> 4][r][f & 15];
        const int at = r * a.n + f0 + f;
        const bool keep = r < a.rows && f < nf;
        if (a.out_f32)
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, t), yr, keep ? at * 4 : kDropped, 0,
                                                  kDeviceCoherent);
        else
            __builtin_amdgcn_raw_buffer_store_b16(bf16_rne(t), yr, keep ? at * 2 : kDropped, 0, kDeviceCoherent);
    }
}

}  // namespace

hipError_t launch_mx(const void *codes, const void *scales, int64_t n, int64_t k, const void *x, int rows, void *y,
                     int out_f32, hipStream_t stream) {
    MxArgs a{};
    a.codes = static_cast<const uint8_t *>(codes);
    a.scales = static_cast<const uint8_t *>(scales);
    a.x = static_cast<const uint16_t *>(x);
    a.y = y;
    a.n = (int)n;
    a.k = (int)k;
    a.rows = rows;
    a.out_f32 = out_f32;
    const int64_t per = (k + kMxWaves - 1) / kMxWaves;
    a.kw = (int)((per + kMxStepK - 1) / kMxStepK * kMxStepK);
    const unsigned grid = (unsigned)((n + kMxFeatures - 1) / kMxFeatures);
    hipLaunchKernelGGL(mx_kernel, dim3(grid), dim3(kMxWaves * 64), 0, stream, a);
    return hipGetLastError();
}

}  // namespace nvfp4
