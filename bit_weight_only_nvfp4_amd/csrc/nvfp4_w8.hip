// nvfp4_w8.hip -- W8G32_F16S projection for gfx950: signed 8-bit weights
// with one fp16 scale per 32 consecutive k of a row, symmetric (the encoding
// the pages name for the DFlash2 drafter's matrices), read in row-major form:
// codes int8 [n][k], scales fp16 [n][k/32].
//
// y[r][j] = sum_k code[j][k] * scale[j][k/32] * x[r][k], fp32 accumulation,
// rows <= 16 per launch.
//
// A code times an fp16 scale has up to 19 significant bits, which no 16-bit
// operand holds, so the scale is not folded into the weights: each 16x16x32
// bf16 product covers exactly one 32-k group (the codes are exact in bf16),
// starts from zero, and its fp32 result is multiplied by the group's scale
// into the accumulator (one scale per lane: a lane's four results share a
// feature).
//   * one workgroup per 32 features (two 16-feature products), 4 waves each
//     over a quarter of k in steps of 128 (four groups); two steps in flight.
//     Measured on [17408 x 5120] and [5120 x 17408]: 64 features per
//     workgroup 25-70% slower (too few workgroups on the second), 16
//     features, 8 waves or three steps in flight 4-30% slower;
//   * a lane (q, n) loads group q of the step whole (32 bytes of row n, so
//     each row is read as 128 contiguous bytes: with 8-byte pieces per lane
//     the same kernel took 49% longer); a cross-lane transpose then gives
//     product m of the step group m, lane (q, n) holding k = 32 m + 8 q .. + 7
//     of row n in both operands (16 bytes of activations, loaded in place);
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

constexpr int kMxStepK = 128;       // four 32-k groups
constexpr int kRsrcWord3 = 0x00020000;
constexpr int kDeviceCoherent = 16;
constexpr int kDropped = 0x7fffffff;
// An offset past every buffer of a workgroup (codes: at most 64 x 2^24 bytes
// = 2^30, scales 64 x 2^20, activations 16 x 2^25): the load reads zeros.
constexpr int kOutside = 1 << 30;

struct MxArgs {
    const int8_t *codes;
    const uint16_t *scales;
    const uint16_t *x;
    void *y;
    int n, k, rows, out_f32;
    int kw;   // k per wave, a multiple of kMxStepK
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, kRsrcWord3);
}

template <int FB>
struct MxStep {
    u32x4_t c[FB][2];       // codes of group q: k = 32 q .. + 31 of each feature block's row n
    uint32_t s[FB][2];      // the four groups' fp16 scales of each row (same for every q)
    u32x4_t a[4];              // activations of row n for each group m
};

template <int FB>
__device__ __forceinline__ void load_step(__amdgpu_buffer_rsrc_t cr, __amdgpu_buffer_rsrc_t sr,
                                          __amdgpu_buffer_rsrc_t xr, int k0, int kend, int k, int q, int n16,
                                          MxStep<FB> &st) {
    const bool in = k0 < kend;   // steps and k are multiples of 128: a step is all in or all out
    const int kb = k / 32;
    const int co = in ? n16 * k + k0 + 32 * q : kOutside;
    const int so = in ? (n16 * kb + k0 / 32) * 2 : kOutside;
    const int xo = in ? (n16 * k + k0 + 8 * q) * 2 : kOutside;
#pragma unroll
    for (int fb = 0; fb < FB; ++fb) {
        // k is a multiple of 128 (checked by the host): every offset here is
        // 16-byte aligned and every group of a step lies inside the row
        st.c[fb][0] = __builtin_amdgcn_raw_buffer_load_b128(cr, co + fb * 16 * k, 0, 0);
        st.c[fb][1] = __builtin_amdgcn_raw_buffer_load_b128(cr, co + fb * 16 * k + 16, 0, 0);
        const auto sv = __builtin_amdgcn_raw_buffer_load_b64(sr, so + fb * 16 * kb * 2, 0, 0);
        st.s[fb][0] = sv[0];
        st.s[fb][1] = sv[1];
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) st.a[m] = __builtin_amdgcn_raw_buffer_load_b128(xr, xo + 64 * m, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
}

// Eight signed bytes (two words) as bf16, exactly.
__device__ __forceinline__ bf16x8_t int8x8_to_bf16(uint32_t lo, uint32_t hi) {
    bf16x8_t r;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        r[j] = (__bf16)(float)(int)(int8_t)(lo >> (8 * j));
        r[4 + j] = (__bf16)(float)(int)(int8_t)(hi >> (8 * j));
    }
    return r;
}

// A lane (q, n) loads group q of the step whole (32 bytes, so the four lanes
// of a row read 128 contiguous bytes); product m needs k = 32 m + 8 q .. + 7
// in lane q.  Seen as a 4 x 4 matrix E[q][j] of 8-byte pieces (lane quarter
// q, words 2 j and 2 j + 1), that is the transpose: one v_permlane32_swap
// stage swaps the off-diagonal 2 x 2 blocks between the half-waves, one
// v_permlane16_swap stage transposes each 2 x 2 block between 16-lane rows.
__device__ __forceinline__ void transpose_groups(const u32x4_t (&c)[2], uint32_t (&w)[8]) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        w[t] = c[0][t];
        w[4 + t] = c[1][t];
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const auto r = __builtin_amdgcn_permlane32_swap(w[t], w[t + 4], false, false);
        w[t] = r[0];
        w[t + 4] = r[1];
    }
#pragma unroll
    for (int t = 0; t < 8; t += (t & 1) ? 3 : 1) {   // t = 0, 1, 4, 5
        const auto r = __builtin_amdgcn_permlane16_swap(w[t], w[t + 2], false, false);
        w[t] = r[0];
        w[t + 2] = r[1];
    }
}

template <int FB>
__device__ __forceinline__ void mac_step(const MxStep<FB> &st, int groups, f32x4_t (&d)[FB]) {
    uint32_t w[FB][8];
#pragma unroll
    for (int fb = 0; fb < FB; ++fb) transpose_groups(st.c[fb], w[fb]);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        if (m >= groups) break;   // uniform: past the end of k
        const bf16x8_t a = __builtin_bit_cast(bf16x8_t, st.a[m]);
#pragma unroll
        for (int fb = 0; fb < FB; ++fb) {
            const f32x4_t p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                a, int8x8_to_bf16(w[fb][2 * m], w[fb][2 * m + 1]), f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
            const uint32_t sw = st.s[fb][m >> 1];
            const float sc = (float)__builtin_bit_cast(_Float16, (uint16_t)((m & 1) ? sw >> 16 : sw & 0xffffu));
#pragma unroll
            for (int v = 0; v < 4; ++v) d[fb][v] = __builtin_fmaf(p[v], sc, d[fb][v]);
        }
    }
}

__device__ __forceinline__ uint16_t bf16_rne(float f) {
    const uint32_t u = __builtin_bit_cast(uint32_t, f);
    const uint32_t rne = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
    const uint32_t nan = (u >> 16) | 0x40u;
    return (uint16_t)((u & 0x7FFFFFFFu) > 0x7F800000u ? nan : rne);
}

// FB 16-feature blocks per workgroup, WAVES waves over parts of k, BUFS steps
// in flight per wave.
template <int FB, int WAVES, int BUFS>
__global__ __launch_bounds__(WAVES * 64) void w8_kernel(MxArgs a) {
    constexpr int kFeatures = 16 * FB;
    __shared__ float red[WAVES][FB][16][16];   // [wave][feature block][row][feature]
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int q = lane >> 4, n16 = lane & 15;
    const int f0 = blockIdx.x * kFeatures;
    const int nf = min(kFeatures, a.n - f0);
    const __amdgpu_buffer_rsrc_t cr = make_rsrc(a.codes + (size_t)f0 * a.k, (uint32_t)((size_t)nf * a.k));
    const __amdgpu_buffer_rsrc_t sr = make_rsrc(a.scales + (size_t)f0 * (a.k / 32), (uint32_t)((size_t)nf * (a.k / 32) * 2));
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.x, (uint32_t)((size_t)a.rows * a.k * 2));
    const int kb = wave * a.kw, ke = min(a.k, kb + a.kw);
    const int steps = ke > kb ? (ke - kb + kMxStepK - 1) / kMxStepK : 0;
    f32x4_t d[FB];
#pragma unroll
    for (int fb = 0; fb < FB; ++fb) d[fb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    MxStep<FB> st[BUFS];
#pragma unroll
    for (int i = 0; i < BUFS; ++i) load_step(cr, sr, xr, kb + i * kMxStepK, ke, a.k, q, n16, st[i]);
    // steps past the wave's last are loaded (reading nothing) but not used,
    // so the loads in flight never depend on control flow
    for (int j = 0; j < steps; j += BUFS) {
#pragma unroll
        for (int i = 0; i < BUFS; ++i) {
            if (j + i < steps) mac_step(st[i], min(4, (ke - (kb + (j + i) * kMxStepK)) / 32), d);
            load_step(cr, sr, xr, kb + (j + i + BUFS) * kMxStepK, ke, a.k, q, n16, st[i]);
        }
    }
#pragma unroll
    for (int fb = 0; fb < FB; ++fb)
#pragma unroll
        for (int v = 0; v < 4; ++v) red[wave][fb][4 * q + v][n16] = d[fb][v];
    __syncthreads();
    const __amdgpu_buffer_rsrc_t yr = make_rsrc(a.y, (uint32_t)((size_t)a.rows * a.n * (a.out_f32 ? 4 : 2)));
#pragma unroll
    for (int o = tid; o < 16 * kFeatures; o += WAVES * 64) {
        const int r = o / kFeatures, f = o % kFeatures;
        float t = red[0][f >> 4][r][f & 15];
#pragma unroll
        for (int w = 1; w < WAVES; ++w) t += red[w][f >> 4][r][f & 15];
        const int at = r * a.n + f0 + f;
        const bool keep = r < a.rows && f < nf;
        if (a.out_f32)
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, t), yr, keep ? at * 4 : kDropped, 0,
                                                  kDeviceCoherent);
        else
            __builtin_amdgcn_raw_buffer_store_b16(bf16_rne(t), yr, keep ? at * 2 : kDropped, 0, kDeviceCoherent);
    }
}

template <int FB, int WAVES, int BUFS>
hipError_t launch_cfg(MxArgs &a, int64_t n, int64_t k, hipStream_t stream) {
    const int64_t per = (k + WAVES - 1) / WAVES;
    a.kw = (int)((per + kMxStepK - 1) / kMxStepK * kMxStepK);
    const unsigned grid = (unsigned)((n + 16 * FB - 1) / (16 * FB));
    hipLaunchKernelGGL((w8_kernel<FB, WAVES, BUFS>), dim3(grid), dim3(WAVES * 64), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_w8(const void *codes, const void *scales, int64_t n, int64_t k, const void *x, int rows, void *y,
                     int out_f32, hipStream_t stream) {
    MxArgs a{};
    a.codes = static_cast<const int8_t *>(codes);
    a.scales = static_cast<const uint16_t *>(scales);
    a.x = static_cast<const uint16_t *>(x);
    a.y = y;
    a.n = (int)n;
    a.k = (int)k;
    a.rows = rows;
    a.out_f32 = out_f32;
    // 16 features per workgroup where that still leaves two workgroups per CU
    // (28.2 us against 31.0 on [17408 x 5120] at 1 row, 35.6 against 35.7 at
    // 8), else 32 ([5120 x 17408]: 30.7 us against 34.2 with 16).  Either way
    // each feature's sum runs over the same 4 quarters of k in the same order.
    if (n >= 16 * 512) return launch_cfg<1, 4, 2>(a, n, k, stream);
    return launch_cfg<2, 4, 2>(a, n, k, stream);
}

}  // namespace nvfp4
