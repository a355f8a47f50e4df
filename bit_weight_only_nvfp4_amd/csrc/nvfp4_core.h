// nvfp4_core.h -- per-super-tile compute cores of the gfx950 NVFP4 projection.
//
// A wave holds one super-tile of one strip in registers: lane l owns output
// feature 64*s + l and, per 32-k tile t, 16 bytes of E2M1 codes (two 16-element
// groups, low nibble first) plus the 16 E4M3 scales of its feature in a 16-byte
// scale chunk.  The activation rows of the super-tile's 256 k sit in LDS, row r
// at xw + r * xstride.  Each core adds sum_k (code * scale) * x[r][k] into
// acc[m][r] (fp32); s_g is applied by the caller's epilogue.
#pragma once

#include "nvfp4_internal.h"

namespace nvfp4 {
namespace core {

__device__ __forceinline__ uint32_t word_of(const uint4 &v, int i) {
    switch (i & 3) {
        case 0: return v.x;
        case 1: return v.y;
        case 2: return v.z;
        default: return v.w;
    }
}

__device__ __forceinline__ float dot2(bf16x2_t w, uint32_t xbits, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(w, __builtin_bit_cast(bf16x2_t, xbits), acc, false);
}

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bf16x4_t as_bf16x4(uint32_t lo, uint32_t hi) {
    const u32x2_t v = {lo, hi};
    return __builtin_bit_cast(bf16x4_t, v);
}

// Keep each 16-element group's work in place.  Left alone, the compiler hoists
// every group's activation reads ahead and sinks the arithmetic behind them
// (it does so for the gate/up pair), which multiplies register pressure.  An
// empty asm statement that takes the accumulators as in/out operands and
// clobbers memory is a compiler-only barrier: the group's arithmetic must be
// done before it and later LDS reads cannot move above it.  It emits no
// instruction and no wait.
template <int NMAT, int ROWS>
__device__ __forceinline__ void pin_group(float (&acc)[NMAT][ROWS]) {
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int r = 0; r < ROWS; ++r) __asm__ volatile("" : "+v"(acc[m][r])::"memory");
}

// Dot-product core: per 16-element group, 8 v_dot2 (two bf16 weights x two
// bf16 activations into fp32) per activation row, then one fma with the
// group's E4M3 scale.  Activations are wave-uniform LDS broadcasts.
template <int ROWS, int NMAT>
__device__ __forceinline__ void core_dot2(const uint4 (&wc)[NMAT][kTilesPerSuper], const uint4 (&wsc)[NMAT],
                                          const uint16_t *xw, int xstride, float (&acc)[NMAT][ROWS]) {
#pragma unroll
    for (int t = 0; t < kTilesPerSuper; ++t) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            uint4 xa[ROWS], xb[ROWS];
#pragma unroll
            for (int r = 0; r < ROWS; ++r) {
                const uint4 *xp = reinterpret_cast<const uint4 *>(xw + r * xstride + 32 * t + 16 * h);
                xa[r] = xp[0];
                xb[r] = xp[1];
            }
#pragma unroll
            for (int m = 0; m < NMAT; ++m) {
                const uint32_t d0 = word_of(wc[m][t], 2 * h);
                const uint32_t d1 = word_of(wc[m][t], 2 * h + 1);
                const bf16x2_t w0 = e2m1x2_to_bf16x2<0>(d0), w1 = e2m1x2_to_bf16x2<1>(d0);
                const bf16x2_t w2 = e2m1x2_to_bf16x2<2>(d0), w3 = e2m1x2_to_bf16x2<3>(d0);
                const bf16x2_t w4 = e2m1x2_to_bf16x2<0>(d1), w5 = e2m1x2_to_bf16x2<1>(d1);
                const bf16x2_t w6 = e2m1x2_to_bf16x2<2>(d1), w7 = e2m1x2_to_bf16x2<3>(d1);
                const int g = 2 * t + h;
                const float sc = e4m3_to_f32_dyn(word_of(wsc[m], g >> 2), g & 3);
#pragma unroll
                for (int r = 0; r < ROWS; ++r) {
                    float part = 0.0f;
                    part = dot2(w0, xa[r].x, part);
                    part = dot2(w1, xa[r].y, part);
                    part = dot2(w2, xa[r].z, part);
                    part = dot2(w3, xa[r].w, part);
                    part = dot2(w4, xb[r].x, part);
                    part = dot2(w5, xb[r].y, part);
                    part = dot2(w6, xb[r].z, part);
                    part = dot2(w7, xb[r].w, part);
                    acc[m][r] = __builtin_fmaf(part, sc, acc[m][r]);
                }
            }
            pin_group(acc);
        }
    }
}

// Matrix-core: v_mfma_f32_4x4x4_16b_bf16 runs 16 independent 4x4x4 products.
// Block b (lanes 4b..4b+3) takes as B the 4 weights (4 consecutive k) of the 4
// features 4b..4b+3 -- lane l keeps feature l, as in the packed layout -- and,
// broadcast from block 0 (cbsz 4, abid 0), A = 4 activation rows x the same 4
// k; lane l receives D[row 0..3][feature l].  Four such products cover one
// 16-element group; the group sum is scaled into the fp32 accumulators, so
// each weight costs half a convert and ROWS/16 fma instead of ROWS/2 dot2.
template <int ROWS, int NMAT>
__device__ __forceinline__ void core_mfma(const uint4 (&wc)[NMAT][kTilesPerSuper], const uint4 (&wsc)[NMAT],
                                          const uint16_t *xw, int xstride, int lane, float (&acc)[NMAT][ROWS]) {
    constexpr int RB = (ROWS + 3) / 4;   // blocks of 4 activation rows
    const f32x4_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int t = 0; t < kTilesPerSuper; ++t) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            // A operands: lane i (mod 4) holds activation row 4*rb+i, 16 k of the group
            uint4 xa[RB], xb[RB];
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const int row = min(4 * rb + (lane & 3), ROWS - 1);
                const uint4 *xp = reinterpret_cast<const uint4 *>(xw + row * xstride + 32 * t + 16 * h);
                xa[rb] = xp[0];
                xb[rb] = xp[1];
            }
#pragma unroll
            for (int m = 0; m < NMAT; ++m) {
                const uint32_t d0 = word_of(wc[m][t], 2 * h);
                const uint32_t d1 = word_of(wc[m][t], 2 * h + 1);
                const bf16x4_t b0 = __builtin_shufflevector(e2m1x2_to_bf16x2<0>(d0), e2m1x2_to_bf16x2<1>(d0), 0, 1, 2, 3);
                const bf16x4_t b1 = __builtin_shufflevector(e2m1x2_to_bf16x2<2>(d0), e2m1x2_to_bf16x2<3>(d0), 0, 1, 2, 3);
                const bf16x4_t b2 = __builtin_shufflevector(e2m1x2_to_bf16x2<0>(d1), e2m1x2_to_bf16x2<1>(d1), 0, 1, 2, 3);
                const bf16x4_t b3 = __builtin_shufflevector(e2m1x2_to_bf16x2<2>(d1), e2m1x2_to_bf16x2<3>(d1), 0, 1, 2, 3);
                const int g = 2 * t + h;
                const float sc = e4m3_to_f32_dyn(word_of(wsc[m], g >> 2), g & 3);
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    f32x4_t d = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(as_bf16x4(xa[rb].x, xa[rb].y), b0, zero, 4, 0, 0);
                    d = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(as_bf16x4(xa[rb].z, xa[rb].w), b1, d, 4, 0, 0);
                    d = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(as_bf16x4(xb[rb].x, xb[rb].y), b2, d, 4, 0, 0);
                    d = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(as_bf16x4(xb[rb].z, xb[rb].w), b3, d, 4, 0, 0);
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (4 * rb + i < ROWS) acc[m][4 * rb + i] = __builtin_fmaf(d[i], sc, acc[m][4 * rb + i]);
                }
            }
            pin_group(acc);
        }
    }
}

}  // namespace core
}  // namespace nvfp4
