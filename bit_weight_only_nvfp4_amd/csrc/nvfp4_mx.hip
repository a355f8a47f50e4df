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
//   * one workgroup per 64 features (four 16-feature products), 2 waves
//     each over half of k in steps of 256; below 32768 features one per 32
//     features with one wave over all of k, so that small matrices still
//     give two workgroups per CU; two steps in flight per wave;
//   * per step a lane (q, n) takes k = 64 q .. 64 q + 63 of the step -- two
//     MX blocks, so two scale bytes per feature block -- as 32 contiguous
//     bytes of codes per feature block (a row's four lanes read 128
//     contiguous bytes) and 128 bytes of its activation row; product m of
//     the step uses word m & 3 of block m >> 2 in both operands.  Measured on
//     a [151936 x 5120] matrix: 126 us at 1 row against 130 with one block
//     per lane in steps of 128 (116 registers, four waves per SIMD); 32
//     features per workgroup or three steps in flight slower;
//   * scale bytes: byte loads cost more than their bytes (the same kernel
//     with no scale loads took 85 us instead of 126), so where k is a
//     multiple of 256 the row's 8 scale bytes of a step are one 8-byte load
//     shared by its four lanes: 104 us;
//   * the waves' sums are added in LDS in wave order (deterministic; a
//     feature's sum depends on the matrix's width class, not on the rows).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nvfp4_internal.h"

namespace nvfp4 {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kMxStepK = 256;
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

template <int FB>
struct MxStep {
    u32x4_t c[FB][2];     // codes: blocks 2 q and 2 q + 1 (k = 64 q .. + 63) of each feature block's row n
    uint32_t s[FB][2];    // their E8M0 scale bytes, or (WIDE) the row's 8 scale bytes of the step
    u32x4_t a[8];         // activations of row n, k = 64 q .. + 63
};

// WIDE (k a multiple of 256, scales 8-byte aligned): the four lanes of a row
// load the row's 8 scale bytes of the step as one 8-byte word (one address,
// merged), each picking its two bytes when it computes; otherwise each lane
// loads its two bytes.
template <int FB, bool WIDE>
__device__ __forceinline__ void load_step(__amdgpu_buffer_rsrc_t cr, __amdgpu_buffer_rsrc_t sr,
                                          __amdgpu_buffer_rsrc_t xr, int k0, int kend, int k, int q, int n16,
                                          MxStep<FB> &st) {
    // k is a multiple of 32: each of a lane's two blocks is all in or all out
    const int kk = k0 + 64 * q;
    const bool in0 = kk < kend, in1 = kk + 32 < kend;
    const int kh = k / 2, kb = k / 32;
    const int co0 = in0 ? n16 * kh + kk / 2 : kOutside, co1 = in1 ? n16 * kh + kk / 2 + 16 : kOutside;
    const int so0 = in0 ? n16 * kb + kk / 32 : kOutside, so1 = in1 ? n16 * kb + kk / 32 + 1 : kOutside;
    const int xo0 = in0 ? (n16 * k + kk) * 2 : kOutside, xo1 = in1 ? (n16 * k + kk) * 2 + 64 : kOutside;
#pragma unroll
    for (int fb = 0; fb < FB; ++fb) {
        st.c[fb][0] = __builtin_amdgcn_raw_buffer_load_b128(cr, co0 + fb * 16 * kh, 0, 0);
        st.c[fb][1] = __builtin_amdgcn_raw_buffer_load_b128(cr, co1 + fb * 16 * kh, 0, 0);
        if constexpr (WIDE) {
            // steps are whole (k and the waves' k ranges are multiples of 256):
            // so0 is the row's first scale of the step, 8-byte aligned
            const auto v = __builtin_amdgcn_raw_buffer_load_b64(sr, so0 - (in0 ? q * 2 : 0) + fb * 16 * kb, 0, 0);
            st.s[fb][0] = v[0];
            st.s[fb][1] = v[1];
        } else {
            st.s[fb][0] = __builtin_amdgcn_raw_buffer_load_b8(sr, so0 + fb * 16 * kb, 0, 0);
            st.s[fb][1] = __builtin_amdgcn_raw_buffer_load_b8(sr, so1 + fb * 16 * kb, 0, 0);
        }
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        st.a[m] = __builtin_amdgcn_raw_buffer_load_b128(xr, xo0 + 16 * m, 0, 0);
        st.a[4 + m] = __builtin_amdgcn_raw_buffer_load_b128(xr, xo1 + 16 * m, 0, 0);
    }
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

// Product m of the step takes word m & 3 of block m >> 2 in both operands: a
// lane's codes are dequantized with its own block's scale, so a product may
// mix the blocks of different lanes.
template <int FB, bool WIDE>
__device__ __forceinline__ void mac_step(const MxStep<FB> &st, int q, f32x4_t (&d)[FB]) {
    float sc[FB][2];
#pragma unroll
    for (int fb = 0; fb < FB; ++fb) {
        uint32_t b0 = st.s[fb][0], b1 = st.s[fb][1];
        if constexpr (WIDE) {   // bytes 2 q and 2 q + 1 of the row's 8
            const uint32_t w = (q & 2) ? st.s[fb][1] : st.s[fb][0];
            b0 = w >> (16 * (q & 1));
            b1 = b0 >> 8;
        }
        sc[fb][0] = __builtin_bit_cast(float, (b0 & 0xffu) << 23);
        sc[fb][1] = __builtin_bit_cast(float, (b1 & 0xffu) << 23);
    }
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const bf16x8_t a = __builtin_bit_cast(bf16x8_t, st.a[m]);
#pragma unroll
        for (int fb = 0; fb < FB; ++fb)
            d[fb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, dequant8(st.c[fb][m >> 2][m & 3], sc[fb][m >> 2]),
                                                            d[fb], 0, 0, 0);
    }
}

__device__ __forceinline__ uint16_t bf16_rne(float f) {
    const uint32_t u = __builtin_bit_cast(uint32_t, f);
    const uint32_t rne = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
    const uint32_t nan = (u >> 16) | 0x40u;
    return (uint16_t)((u & 0x7FFFFFFFu) > 0x7F800000u ? nan : rne);
}

// FB 16-feature blocks per workgroup, WAVES waves over parts of k, BUFS
// steps in flight per wave.
template <int FB, int WAVES, int BUFS, bool WIDE>
__global__ __launch_bounds__(WAVES * 64) void mx_kernel(MxArgs a) {
    constexpr int kMxFeatures = 16 * FB;
    __shared__ float red[WAVES][FB][16][16];   // [wave][feature block][row][feature]
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
    f32x4_t d[FB];
#pragma unroll
    for (int fb = 0; fb < FB; ++fb) d[fb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    MxStep<FB> st[BUFS];
#pragma unroll
    for (int i = 0; i < BUFS; ++i) load_step<FB, WIDE>(cr, sr, xr, kb + i * kMxStepK, ke, a.k, q, n16, st[i]);
    // steps past the wave's last are loaded (reading nothing) but not used,
    // so the loads in flight never depend on control flow
    for (int j = 0; j < steps; j += BUFS) {
#pragma unroll
        for (int i = 0; i < BUFS; ++i) {
            if (j + i < steps) mac_step<FB, WIDE>(st[i], q, d);
            load_step<FB, WIDE>(cr, sr, xr, kb + (j + i + BUFS) * kMxStepK, ke, a.k, q, n16, st[i]);
        }
    }
#pragma unroll
    for (int fb = 0; fb < FB; ++fb)
#pragma unroll
        for (int v = 0; v < 4; ++v) red[wave][fb][4 * q + v][n16] = d[fb][v];
    __syncthreads();
    const __amdgpu_buffer_rsrc_t yr = make_rsrc(a.y, (uint32_t)((size_t)a.rows * a.n * (a.out_f32 ? 4 : 2)));
#pragma unroll
    for (int o = tid; o < 16 * kMxFeatures; o += WAVES * 64) {
        const int r = o / kMxFeatures, f = o % kMxFeatures;
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
    constexpr int BUFS = 2;
    const bool wide = k % 256 == 0 && reinterpret_cast<uintptr_t>(scales) % 8 == 0;
    // Below 512 groups of 64 features (two workgroups per CU), groups of 32
    // features, one wave over all of k: twice the workgroups and 20 steps per
    // wave at k = 5120 (17.5 us against 20.0 with four waves over quarters of
    // k on [17408 x 5120] at 1 row, 21.6 against 24.1 at 8).  From there on,
    // groups of 64 features, two waves over halves of k (105 us against 106
    // with four waves, 120 with one, on [151936 x 5120]).
    auto wave_k = [&](int waves) {
        const int64_t per = (k + waves - 1) / waves;
        return (int)((per + kMxStepK - 1) / kMxStepK * kMxStepK);
    };
    if (n < 32768) {
        constexpr int FB = 2, W = 1;
        a.kw = wave_k(W);
        const unsigned grid = (unsigned)((n + 16 * FB - 1) / (16 * FB));
        if (wide) hipLaunchKernelGGL((mx_kernel<FB, W, BUFS, true>), dim3(grid), dim3(W * 64), 0, stream, a);
        else hipLaunchKernelGGL((mx_kernel<FB, W, BUFS, false>), dim3(grid), dim3(W * 64), 0, stream, a);
    } else {
        constexpr int FB = 4, W = 2;
        a.kw = wave_k(W);
        const unsigned grid = (unsigned)((n + 16 * FB - 1) / (16 * FB));
        if (wide) hipLaunchKernelGGL((mx_kernel<FB, W, BUFS, true>), dim3(grid), dim3(W * 64), 0, stream, a);
        else hipLaunchKernelGGL((mx_kernel<FB, W, BUFS, false>), dim3(grid), dim3(W * 64), 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace nvfp4
