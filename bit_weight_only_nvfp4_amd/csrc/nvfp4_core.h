// nvfp4_core.h -- per-super-tile arithmetic of the gfx950 NVFP4 projection on
// the matrix cores: bf16 products of the activations exactly as stored and the
// E2M1 codes, one 16-element group per product row, with the E4M3 group scale
// folded into an fp32 accumulator (v_mfma_f32_16x16x32_bf16).
//
// Why this arithmetic.  A bf16 activation times an E2M1 code is exact in fp32
// (8 x 2 significant bits), and so is every code in bf16; the E4M3 group scale
// has 4 significant bits and only a power-of-two part can ride in the code
// conversion (v_cvt_scalef32_pk_bf16_fp4 applies the exponent of its scale
// operand alone), so the scale multiplies the group's sum instead.  The
// activations need no conversion or rescaling at all, whatever their range,
// and every row of a call is computed by the same instructions in the same
// positions whatever the number of rows, so a row's result does not depend on
// how many rows share the call.
//
// One product covers 16 features x 32 k (two 16-element groups).  Its 16 A
// rows ("slots") are (group half h, activation row r) pairs: slot s holds row
// 2 (s & 3) + (s >> 3) of the row set restricted to the group h = (s >> 2) & 1
// of the product's 32 k (the other group's k are zero), so D row s of feature
// j is one 16-element group sum.  With the D layout below, lane group q of the
// result holds group half q & 1 and rows 2 v + (q >> 1), v = 0..3: one fused
// multiply-add by the lane's E4M3 scale per v covers all four lane groups.  A
// row set is 8 rows; more rows take more row sets, sharing the converted codes.
//
// Operand lane layouts of the 16x16x32 bf16 product (measured on gfx950):
//   A: lane 16 q + i holds row i, k = 8 q .. 8 q + 7;
//   B: lane 16 q + n holds column n, k = 8 q .. 8 q + 7;
//   D: lane 16 q + n holds rows 4 q .. 4 q + 3 of column n.
// So B lanes q = 0, 1 carry the product's first group and q = 2, 3 its second,
// and A lane (q, s) is non-zero only where q >> 1 equals slot s's group half.
//
// Inside one product the hardware adds the 8 products of each lane group
// without rounding and combines the lane groups' sums in fp32 (measured:
// 2^24 + 1 - 2^24 within one lane group gives 1, across lane groups 0); bf16
// and fp32 subnormals are kept.
#pragma once

#include "nvfp4_internal.h"

namespace nvfp4 {
namespace core {

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

// LDS image of one super-tile's activations, per wave: rows of 256 bf16 as
// stored, 528 bytes apart (rows start 4 banks apart), then 16 zero bytes read
// by the masked product rows.
template <int ROWS>
struct XStageG {
    static constexpr int XR = (ROWS * 32 + 63) / 64;   // 16-byte activation chunks per lane
    static constexpr int RA = 2 * XR;                  // rows staged: ROWS rounded up to even
    static constexpr int ROW_BYTES = 528;
    static constexpr int ZERO_OFF = RA * ROW_BYTES;
    static constexpr int BYTES = ZERO_OFF + 16;
    static constexpr int RS = (ROWS + 7) / 8;                       // row sets
    static constexpr int NV = ((ROWS < 8 ? ROWS : 8) + 1) / 2;      // D rows per lane in use
};

__device__ __forceinline__ uint32_t word_of(const uint4 &v, int i) {
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// Store this lane's activation chunks: chunk c = lane + 64 i is row c / 32,
// k = 8 (c % 32) .. + 7 of the super-tile (rows past the call's are zeros).
template <int ROWS>
__device__ __forceinline__ void stage_g(const uint4 (&xv)[XStageG<ROWS>::XR], uint8_t *xs, int lane) {
    using S = XStageG<ROWS>;
#pragma unroll
    for (int i = 0; i < S::XR; ++i) {
        const int c = lane + 64 * i;
        *reinterpret_cast<uint4 *>(xs + (c >> 5) * S::ROW_BYTES + (c & 31) * 16) = xv[i];
    }
}

// acc[fb][rs][v] += this super-tile's group sums times their E4M3 scales for
// feature 16 fb + n, row 8 rs + 2 v + (q >> 1), group half q & 1 (lane 16 q + n).
//
// Packed layout version 3 (one super-tile = 64 features x 256 k): wc[c] is the
// lane's 16 bytes of code chunk c; its dword j holds the 8 codes of feature
// 16 (c >> 1) + n for k = 32 (4 (c & 1) + j) + 8 q .. + 7, i.e. product
// (fb, ks) -- k step ks of 32 k -- takes dword ks & 3 of chunk 2 fb + (ks >> 2).
// ws is the lane's scale entry: byte 8 b + ks is the scale of feature
// 16 (2 (q >> 1) + b) + n, group 2 ks + (q & 1) of the super-tile; lanes q and
// q ^ 2 need the same 32 scale bytes and hold half of them each.
// The 16 codes of product (fb, ks) as a bf16 B operand.
__device__ __forceinline__ bf16x8_t codes_bf16(uint32_t w) {
    const bf16x2_t b0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 0);
    const bf16x2_t b1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 1);
    const bf16x2_t b2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 2);
    const bf16x2_t b3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 3);
    return bf16x8_t{b0.x, b0.y, b1.x, b1.y, b2.x, b2.y, b3.x, b3.y};
}

// Software pipeline over the 8 k steps of a super-tile: while the products
// of step ks run on the matrix core, the vector unit converts the codes of
// step ks + 1 and scales the results of step ks - 1 into the accumulators
// (a product's result is read 2 steps of conversions after it was issued,
// so neither unit waits for the other).
template <int ROWS>
__device__ __forceinline__ void core_g(const uint4 (&wc)[kCodeChunks], const uint4 &ws, const uint8_t *xs, int lane,
                                       float (&acc)[4][XStageG<ROWS>::RS][XStageG<ROWS>::NV]) {
    using S = XStageG<ROWS>;
    constexpr int RS = S::RS, NV = S::NV;
    const int q = lane >> 4, i = lane & 15;
    // the scale bytes of feature blocks 0, 1 (sl[0]) and 2, 3 (sl[1])
    uint32_t sl[2][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const auto r = __builtin_amdgcn_permlane32_swap(word_of(ws, j), word_of(ws, j), false, false);
        sl[0][j] = r[0];
        sl[1][j] = r[1];
    }
    // this lane's A slot: group half and row of the row set
    const int sh = (i >> 2) & 1, sr = 2 * (i & 3) + (i >> 3);
    int abase[RS], astep[RS];
#pragma unroll
    for (int rs = 0; rs < RS; ++rs) {
        const bool live = sh == (q >> 1) && 8 * rs + sr < ROWS;
        abase[rs] = live ? (8 * rs + sr) * S::ROW_BYTES + 16 * q : S::ZERO_OFF;
        astep[rs] = live ? 64 : 0;
    }
    // E4M3 scale of feature block fb at k step ks
    // E4M3 scales of feature block fb at k steps ks and ks + 1 (ks even): one
    // packed conversion of the two bytes
    auto scale_pair = [&](int fb, int ks) {
        const uint32_t w = sl[fb >> 1][2 * (fb & 1) + (ks >> 2)];
        return (ks & 2) ? __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true) : __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
    };
    float sn[4];   // the scale of the odd k step, converted with the even one
    if constexpr (RS >= 2) {
        // Two or more row sets: the products of a k step are already 8 or more
        // in flight, enough to cover the matrix core's latency without the
        // pipeline, whose second set of results would not fit in registers.
        // Same products, same multiply-adds in the same order per accumulator.
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            bf16x8_t A[RS], B[4];
#pragma unroll
            for (int rs = 0; rs < RS; ++rs)
                A[rs] = *reinterpret_cast<const bf16x8_t *>(xs + abase[rs] + astep[rs] * ks);
#pragma unroll
            for (int fb = 0; fb < 4; ++fb) B[fb] = codes_bf16(word_of(wc[2 * fb + (ks >> 2)], ks & 3));
            f32x4_t D[4][RS];
#pragma unroll
            for (int fb = 0; fb < 4; ++fb)
#pragma unroll
                for (int rs = 0; rs < RS; ++rs) {
                    const f32x4_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
                    D[fb][rs] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[rs], B[fb], zero, 0, 0, 0);
                }
#pragma unroll
            for (int fb = 0; fb < 4; ++fb) {
                float sc;
                if ((ks & 1) == 0) {
                    const auto p = scale_pair(fb, ks);
                    sc = p[0];
                    sn[fb] = p[1];
                } else {
                    sc = sn[fb];
                }
#pragma unroll
                for (int rs = 0; rs < RS; ++rs)
#pragma unroll
                    for (int v = 0; v < NV; ++v) acc[fb][rs][v] = __builtin_fmaf(D[fb][rs][v], sc, acc[fb][rs][v]);
            }
        }
        return;
    }
    bf16x8_t B[4], Bn[4];
    f32x4_t D[4][RS], Dp[4][RS];
    float sp[4];
#pragma unroll
    for (int fb = 0; fb < 4; ++fb) Bn[fb] = codes_bf16(word_of(wc[2 * fb], 0));
#pragma unroll
    for (int ks = 0; ks <= 8; ++ks) {
        if (ks < 8) {
            bf16x8_t A[RS];
#pragma unroll
            for (int rs = 0; rs < RS; ++rs)
                A[rs] = *reinterpret_cast<const bf16x8_t *>(xs + abase[rs] + astep[rs] * ks);
#pragma unroll
            for (int fb = 0; fb < 4; ++fb) B[fb] = Bn[fb];
#pragma unroll
            for (int fb = 0; fb < 4; ++fb)
#pragma unroll
                for (int rs = 0; rs < RS; ++rs) {
                    const f32x4_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
                    D[fb][rs] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[rs], B[fb], zero, 0, 0, 0);
                }
            if (ks + 1 < 8) {
#pragma unroll
                for (int fb = 0; fb < 4; ++fb) Bn[fb] = codes_bf16(word_of(wc[2 * fb + ((ks + 1) >> 2)], (ks + 1) & 3));
            }
        }
        if (ks > 0) {
#pragma unroll
            for (int fb = 0; fb < 4; ++fb)
#pragma unroll
                for (int rs = 0; rs < RS; ++rs)
#pragma unroll
                    for (int v = 0; v < NV; ++v) acc[fb][rs][v] = __builtin_fmaf(Dp[fb][rs][v], sp[fb], acc[fb][rs][v]);
        }
        if (ks < 8) {
#pragma unroll
            for (int fb = 0; fb < 4; ++fb) {
                if ((ks & 1) == 0) {
                    const auto p = scale_pair(fb, ks);
                    sp[fb] = p[0];
                    sn[fb] = p[1];
                } else {
                    sp[fb] = sn[fb];
                }
#pragma unroll
                for (int rs = 0; rs < RS; ++rs) Dp[fb][rs] = D[fb][rs];
            }
        }
    }
}

}  // namespace core
}  // namespace nvfp4
