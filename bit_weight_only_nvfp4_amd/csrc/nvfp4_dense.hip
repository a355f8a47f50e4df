// nvfp4_dense.hip -- dense bf16 projection for gfx950: the lm head, whose
// weights stay bf16 (the Qwen3.8-27B-NVFP4 blueprint page, "Precision" table:
// bf16 x bf16 nodes next to the nvfp4/g16 ones; its kernel table names the
// step gemv::dense_gemv_bf16).
//
// y[r][j] = sum_k W[j][k] x[r][k], W bf16 [n][k] row-major as stored, x bf16
// [rows][k] (rows <= 16 per launch), fp32 accumulation, bf16 (RNE) or fp32 out.
//
// The weight stream is the whole cost (2 bytes per weight against 4.5 bits for
// NVFP4), so the kernel is shaped for it:
//   * one workgroup per 32 features (two 16-feature matrix-core products), 4
//     waves each taking a quarter of k; many more workgroups than CUs (several
//     resident per CU), so the hardware's dispatcher balances them.  Measured
//     on a [151936 x 5120] head against 8 waves per workgroup: 4.8% faster at
//     1 row; 2 waves, 64 features per workgroup, or 5-6 steps in flight were
//     slower, 3 steps equal;
//   * a wave's k-range in steps of 64: per step a lane loads 32 contiguous
//     bytes of each of its two weight rows (16 rows x 128 bytes per product:
//     whole lines) and 32 bytes of its activation row, four steps in flight;
//   * v_mfma_f32_16x16x32_bf16, A = activations (16 product rows: the call's
//     rows, zeros past them), B = weights.  A lane holds k = 16 q + 8 m .. + 7
//     of product m of the step in both operands: any assignment of k to the
//     operand's k slots gives the same sum as long as A and B share it;
//   * the waves' sums are added in LDS in wave order (deterministic), one
//     output per lane, and stored through buffer resources whose bounds drop
//     the rows past the call's and the features past n.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nvfp4_internal.h"

namespace nvfp4 {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kDenseFB = 2;          // 16-feature blocks per workgroup
constexpr int kDenseFeatures = 16 * kDenseFB;
constexpr int kDenseWaves = 4;
constexpr int kDenseStepK = 64;
constexpr int kDenseBufs = 4;        // steps in flight per wave
constexpr int kDropped = 0x7fffffff; // past any buffer: loads read 0, stores are dropped
constexpr int kRsrcWord3 = 0x00020000;
constexpr int kDeviceCoherent = 16;

struct DenseArgs {
    const uint16_t *w;
    const uint16_t *x;
    void *y;
    int n, k, rows, out_f32;
    int kw;   // k per wave, a multiple of kDenseStepK
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, kRsrcWord3);
}

// One step's operands of this lane: two weight rows (feature blocks) and the
// activation row, 32 bytes each (k = k0 + 16 q .. + 15).
struct DenseStep {
    u32x4_t b[kDenseFB][2];
    u32x4_t a[2];
};

// Offsets past every buffer of a workgroup (its weight rows take at most
// 32 x 2^24 x 2 = 2^30 bytes): the load reads zeros.  Each lane selects one
// base offset and the loads add constants to it (folded into the
// instructions), so no lane branches and the waits stay exact.
constexpr int kOutside = 1 << 30;

__device__ __forceinline__ void load_step(__amdgpu_buffer_rsrc_t wr, __amdgpu_buffer_rsrc_t xr, int k0, int kend,
                                          int k, int q, int n16, int row, DenseStep &s) {
    const int kk = k0 + 16 * q;
    const bool in = kk < kend;   // k is a multiple of 16: a lane's 16 values are all in or all out
    const int wo = in ? (n16 * k + kk) * 2 : kOutside;
    const int fbo = 16 * k * 2;   // the next feature block's rows
#pragma unroll
    for (int fb = 0; fb < kDenseFB; ++fb) {
        s.b[fb][0] = __builtin_amdgcn_raw_buffer_load_b128(wr, wo + fb * fbo, 0, 0);
        s.b[fb][1] = __builtin_amdgcn_raw_buffer_load_b128(wr, wo + fb * fbo + 16, 0, 0);
    }
    const int xo = in ? (row * k + kk) * 2 : kOutside;
    s.a[0] = __builtin_amdgcn_raw_buffer_load_b128(xr, xo, 0, 0);
    s.a[1] = __builtin_amdgcn_raw_buffer_load_b128(xr, xo + 16, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ void mac_step(const DenseStep &s, f32x4_t (&d)[kDenseFB]) {
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        const bf16x8_t a = __builtin_bit_cast(bf16x8_t, s.a[m]);
#pragma unroll
        for (int fb = 0; fb < kDenseFB; ++fb)
            d[fb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8_t, s.b[fb][m]), d[fb], 0,
                                                            0, 0);
    }
}

__device__ __forceinline__ uint16_t bf16_rne(float f) {
    const uint32_t u = __builtin_bit_cast(uint32_t, f);
    const uint32_t rne = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
    const uint32_t nan = (u >> 16) | 0x40u;
    return (uint16_t)((u & 0x7FFFFFFFu) > 0x7F800000u ? nan : rne);
}

__global__ __launch_bounds__(kDenseWaves * 64) void dense_kernel(DenseArgs a) {
    __shared__ float red[kDenseWaves][kDenseFB][16][16];   // [wave][feature block][row][feature]
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int q = lane >> 4, n16 = lane & 15;
    const int f0 = blockIdx.x * kDenseFeatures;
    // this workgroup's weight rows (up to 32, fewer at the end of W)
    const int nf = min(kDenseFeatures, a.n - f0);
    const __amdgpu_buffer_rsrc_t wr =
        make_rsrc(a.w + (size_t)f0 * a.k, (uint32_t)((size_t)nf * a.k * 2));
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.x, (uint32_t)((size_t)a.rows * a.k * 2));
    const int kb = wave * a.kw, ke = min(a.k, kb + a.kw);
    const int steps = ke > kb ? (ke - kb + kDenseStepK - 1) / kDenseStepK : 0;
    f32x4_t d[kDenseFB];
#pragma unroll
    for (int fb = 0; fb < kDenseFB; ++fb) d[fb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    DenseStep s[kDenseBufs];
#pragma unroll
    for (int i = 0; i < kDenseBufs; ++i) load_step(wr, xr, kb + i * kDenseStepK, ke, a.k, q, n16, n16, s[i]);
    // steps past the wave's last are loaded (reading nothing) but not used,
    // so the loads in flight never depend on control flow
    for (int j = 0; j < steps; j += kDenseBufs) {
#pragma unroll
        for (int i = 0; i < kDenseBufs; ++i) {
            if (j + i < steps) mac_step(s[i], d);
            load_step(wr, xr, kb + (j + i + kDenseBufs) * kDenseStepK, ke, a.k, q, n16, n16, s[i]);
        }
    }
    // lane (q, n16) holds rows 4 q .. 4 q + 3 of features 16 fb + n16
#pragma unroll
    for (int fb = 0; fb < kDenseFB; ++fb)
#pragma unroll
        for (int v = 0; v < 4; ++v) red[wave][fb][4 * q + v][n16] = d[fb][v];
    __syncthreads();
    // 16 rows x kDenseFeatures outputs, summed in wave order
    const __amdgpu_buffer_rsrc_t yr = make_rsrc(a.y, (uint32_t)((size_t)a.rows * a.n * (a.out_f32 ? 4 : 2)));
#pragma unroll
    for (int o = tid; o < 16 * kDenseFeatures; o += kDenseWaves * 64) {
        const int r = o / kDenseFeatures, f = o % kDenseFeatures;
        float t = red[0][f >> 4][r][f & 15];
#pragma unroll
        for (int w = 1; w < kDenseWaves; ++w) t += red[w][f >> 4][r][f & 15];
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

hipError_t launch_dense(const void *w, int64_t n, int64_t k, const void *x, int rows, void *y, int out_f32,
                        hipStream_t stream) {
    DenseArgs a{};
    a.w = static_cast<const uint16_t *>(w);
    a.x = static_cast<const uint16_t *>(x);
    a.y = y;
    a.n = (int)n;
    a.k = (int)k;
    a.rows = rows;
    a.out_f32 = out_f32;
    const int64_t per = (k + kDenseWaves - 1) / kDenseWaves;
    a.kw = (int)((per + kDenseStepK - 1) / kDenseStepK * kDenseStepK);
    const unsigned grid = (unsigned)((n + kDenseFeatures - 1) / kDenseFeatures);
    hipLaunchKernelGGL(dense_kernel, dim3(grid), dim3(kDenseWaves * 64), 0, stream, a);
    return hipGetLastError();
}

}  // namespace nvfp4
