// nvfp4_core.h -- per-super-tile compute of the gfx950 NVFP4 projection on the
// matrix cores, on one of two paths: block-scaled fp8 x fp4 products
// (v_mfma_scale_f32_16x16x128_f8f6f4: stage_x, core_mx; up to 4 activation
// rows) or fp16 products of dequantized weights (v_mfma_f32_16x16x32_f16:
// stage_x16, core_f16; 5-16 rows), described before each.
//
// fp8 x fp4 path: the E2M1 codes are the fp4 B operand exactly as stored (no
// per-weight conversion).  One product covers 16 features x 64 k and 16 "slots" (rows of
// A): slot 4 G + R is activation row 4 rq + R restricted to group G (16 k) of
// the 64-k block.  Each activation value is split exactly into an fp8 E4M3
// high part and an fp8 low part (x = hi + lo for all values within 13 binades
// of their group's largest), both scaled by powers of two that ride in the
// instruction's per-block E8M0 A scales.  The 128-k operand holds the block's
// 64 codes twice: the high parts meet the first copy, the low parts the
// second, so each slot's result is already hi + lo.  The result for slot
// (G, R) of feature j is then a 16-element group sum, multiplied by the E4M3
// group scale of (j, G) and accumulated in fp32.
//
// Operand lane layouts of the 16x16x128 product (measured on gfx950):
//   A (fp8, 32 B per lane): lane 16 q + i holds row i, bytes 0..15 = k 16 q ..,
//     bytes 16..31 = k 64 + 16 q ..;
//   B (fp4, 16 B per lane): lane 16 q + n holds column n, k = 32 q .. 32 q + 31;
//   A scale of (row i, 32-k block b): lane 16 b + i; B scale likewise;
//   D: lane 16 q + n holds rows 4 q .. 4 q + 3 of column n.
#pragma once

#include "nvfp4_internal.h"

namespace nvfp4 {
namespace core {

typedef int32_t i32x8_t __attribute__((ext_vector_type(8)));
typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef short i16x2_t __attribute__((ext_vector_type(2)));
typedef uint16_t u16x2_t __attribute__((ext_vector_type(2)));

// LDS image of one super-tile's activations, per wave.
template <int ROWS>
struct XStage {
    static constexpr int NRQ = (ROWS + 3) / 4;             // quads of activation rows
    static constexpr int XR = (ROWS * 32 + 63) / 64;       // 16-byte activation chunks per lane
    // slot (kb, rq, G, R): 16 bytes hi then 16 bytes lo, 16 consecutive k
    static constexpr int SLOT_BYTES = 4 * NRQ * 16 * 32;
    // per slot: E8M0 exponent of the hi part | (of the lo part << 8)
    static constexpr int EXP_OFF = SLOT_BYTES;
    static constexpr int ZERO_OFF = EXP_OFF + 4 * NRQ * 16 * 4;   // 32 zero bytes
    static constexpr int BYTES = ZERO_OFF + 32;
};

__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t,
                              __builtin_elementwise_max(__builtin_bit_cast(u16x2_t, a), __builtin_bit_cast(u16x2_t, b)));
}

__device__ __forceinline__ uint32_t word_of(const uint4 &v, int i) {
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// Split the super-tile's activation chunks into hi/lo fp8 parts and stage them.
// Chunk c = lane + 64 i holds row c / 32, k = 8 (c % 32) .. + 7 of the
// super-tile; lanes l and l ^ 1 hold the two halves of one 16-element group.
// Group exponent: the largest |x| of the group is below 2^(E+1); the hi parts
// are x / 2^(E-7) (below 256, inside E4M3's range) and the lo parts
// (x - hi) / 2^(E-12) (below 256 again: |x - hi| <= 2^(E-4)).
template <int ROWS>
__device__ __forceinline__ void stage_x(const uint4 (&xv)[XStage<ROWS>::XR], uint8_t *xs, int lane) {
    using S = XStage<ROWS>;
#pragma unroll
    for (int i = 0; i < S::XR; ++i) {
        const int c = lane + 64 * i;
        const int r = c >> 5, kk = (c & 31) * 8;
        const int gt = kk >> 4, h = (kk >> 3) & 1;
        const int slot = (((gt >> 2) * S::NRQ + (r >> 2)) * 4 + (gt & 3)) * 4 + (r & 3);
        const uint32_t d[4] = {xv[i].x, xv[i].y, xv[i].z, xv[i].w};
        uint32_t m = pk_max_u16(pk_max_u16(d[0] & 0x7fff7fffu, d[1] & 0x7fff7fffu),
                                pk_max_u16(d[2] & 0x7fff7fffu, d[3] & 0x7fff7fffu));
        m = max(m & 0xffffu, m >> 16);
        m = max(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0xB1, 0xF, 0xF, false));   // lane ^ 1
        const int ef = (int)(m >> 7);   // biased bf16 exponent of the group's largest |x|
        const int ehi = max(ef, 8) - 7, elo = max(ef, 13) - 12;
        const float shi = __builtin_bit_cast(float, ehi << 23), slo = __builtin_bit_cast(float, elo << 23);
        i16x2_t hw0 = {0, 0}, hw1 = {0, 0};
        hw0 = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(hw0, __builtin_bit_cast(bf16x2_t, d[0]), shi, false);
        hw0 = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(hw0, __builtin_bit_cast(bf16x2_t, d[1]), shi, true);
        hw1 = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(hw1, __builtin_bit_cast(bf16x2_t, d[2]), shi, false);
        hw1 = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(hw1, __builtin_bit_cast(bf16x2_t, d[3]), shi, true);
        const uint32_t h0 = __builtin_bit_cast(uint32_t, hw0), h1 = __builtin_bit_cast(uint32_t, hw1);
        const f32x2_t back[4] = {__builtin_amdgcn_cvt_scalef32_pk_f32_fp8(h0, shi, false),
                                 __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(h0, shi, true),
                                 __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(h1, shi, false),
                                 __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(h1, shi, true)};
        float lo[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {   // exact: x and hi share the exponent range
            lo[2 * q] = __builtin_bit_cast(float, d[q] << 16) - back[q].x;
            lo[2 * q + 1] = __builtin_bit_cast(float, d[q] & 0xffff0000u) - back[q].y;
        }
        i16x2_t lw0 = {0, 0}, lw1 = {0, 0};
        lw0 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lw0, lo[0], lo[1], slo, false);
        lw0 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lw0, lo[2], lo[3], slo, true);
        lw1 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lw1, lo[4], lo[5], slo, false);
        lw1 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lw1, lo[6], lo[7], slo, true);
        uint8_t *p = xs + slot * 32 + h * 8;
        *reinterpret_cast<uint2 *>(p) = make_uint2(h0, h1);
        *reinterpret_cast<uint2 *>(p + 16) =
            make_uint2(__builtin_bit_cast(uint32_t, lw0), __builtin_bit_cast(uint32_t, lw1));
        *reinterpret_cast<uint32_t *>(xs + S::EXP_OFF + slot * 4) = (uint32_t)ehi | ((uint32_t)elo << 8);
    }
}

// Duplicate a 1 KB load of code chunks (c | c + 1) -- lanes 0..31 hold chunk
// c, lanes 32..63 chunk c + 1 -- into the two matrix-core operands
// (c | c) and (c + 1 | c + 1): the 128-k operand holds a 64-k block twice.
__device__ __forceinline__ void dup_halves(const uint4 &v, i32x4_t &lo, i32x4_t &hi) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const auto r = __builtin_amdgcn_permlane32_swap(w[q], w[q], false, false);
        lo[q] = (int32_t)r[0];
        hi[q] = (int32_t)r[1];
    }
}

// acc[fb][r] += this lane's share of one matrix's super-tile.  Lane 16 g + n
// accumulates feature 16 fb + n over the groups 4 kb + g; the four lane groups
// together hold the super-tile's sums.  wc[l] is the super-tile's l-th KB of
// codes (chunks 2 l, 2 l + 1) as loaded by lane 16 g + n at 16 * lane; ws is
// scale entry 16 g + n.
template <int ROWS>
__device__ __forceinline__ void core_mx(const uint4 (&wc)[kCodeChunks / 2], const uint4 &ws, const uint8_t *xs,
                                        int lane, float (&acc)[4][ROWS]) {
    using S = XStage<ROWS>;
    const int g = lane >> 4, i = lane & 15, G = i >> 2, R = i & 3;
    const bool data_lane = g == G;                         // holds slot i's parts
    const bool hi_scale = g == (G >> 1), lo_scale = g == 2 + (G >> 1);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
        const uint32_t sw = word_of(ws, kb);   // bytes fb = 0..3: scales of group 4 kb + g
        const f32x2_t s01 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(sw, 1.0f, false);
        const f32x2_t s23 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(sw, 1.0f, true);
        const float sc[4] = {s01.x, s01.y, s23.x, s23.y};
        i32x4_t b4[4];
        dup_halves(wc[2 * kb], b4[0], b4[1]);
        dup_halves(wc[2 * kb + 1], b4[2], b4[3]);
#pragma unroll
        for (int rq = 0; rq < S::NRQ; ++rq) {
            const int slot = ((kb * S::NRQ + rq) * 4 + G) * 4 + R;
            const i32x8_t A = *reinterpret_cast<const i32x8_t *>(xs + (data_lane ? slot * 32 : S::ZERO_OFF));
            const uint32_t e = *reinterpret_cast<const uint32_t *>(xs + S::EXP_OFF + slot * 4);
            const int sa = hi_scale ? (int)(e & 0xff) : lo_scale ? (int)((e >> 8) & 0xff) : 127;
#pragma unroll
            for (int fb = 0; fb < 4; ++fb) {
                const i32x8_t B = __builtin_shufflevector(b4[fb], b4[fb], 0, 1, 2, 3, -1, -1, -1, -1);
                const f32x4_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
                // A: fp8 E4M3 (format 0), B: fp4 E2M1 (format 4), B scale 2^0
                const f32x4_t D = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, zero, 0, 4, 0, sa, 0, 127);
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    if (4 * rq + v < ROWS) acc[fb][4 * rq + v] = __builtin_fmaf(D[v], sc[fb], acc[fb][4 * rq + v]);
            }
        }
        // one k block at a time: bounds the products in flight (registers)
        if (ROWS > 4) __builtin_amdgcn_sched_barrier(0);
    }
}

// One activation row (the fp8 x fp4 path mapped for it): a product covers 16
// features x 128 k -- the codes of two 64-k blocks of one feature block after
// one v_permlane32_swap, already the B layout above -- and its 16 slots are
// the 8 groups of those 128 k, hi and lo part each: slot m = 2 G + part holds
// group G (k 16 G .. 16 G + 15) of part m % 2, zero elsewhere, so a super-tile
// takes 8 products where the general mapping takes 16 (it fills only one of
// its 4 row slots with one row).  D rows 4 q + v of lane group q are groups
// 2 q + v / 2: their sums are D[0] + D[1] and D[2] + D[3].
struct XStage1 {
    static constexpr int XR = 1;
    // pair p (64-k blocks 2 p, 2 p + 1), slot m: 32 bytes in the A lane layout
    // (group G < 4 in bytes 0..15, G >= 4 in bytes 16..31, the other half zero)
    static constexpr int EXP_OFF = 2 * 16 * 32;        // pair p, slot m: E8M0 byte
    static constexpr int ZERO_OFF = EXP_OFF + 32;      // 32 zero bytes
    static constexpr int WS_OFF = ZERO_OFF + 32;       // the lanes' 16-byte group-scale entries
    static constexpr int BYTES = WS_OFF + 1024;
};

// Zero the slot image once: the half of each slot entry that holds no group
// is never written afterwards.
__device__ __forceinline__ void init_x1(uint8_t *xs, int lane) {
    *reinterpret_cast<uint4 *>(xs + lane * 16) = make_uint4(0u, 0u, 0u, 0u);
    if (lane < 8) reinterpret_cast<uint32_t *>(xs + XStage1::ZERO_OFF)[lane] = 0u;
}

// As stage_x (same hi / lo split and exponents), into the one-row slot image.
// Lane l < 32 holds k = 8 l .. 8 l + 7: group l / 2 of the super-tile.
__device__ __forceinline__ void stage_x1(const uint4 (&xv)[1], uint8_t *xs, int lane) {
    using S = XStage1;
    const uint32_t d[4] = {xv[0].x, xv[0].y, xv[0].z, xv[0].w};
    uint32_t m = pk_max_u16(pk_max_u16(d[0] & 0x7fff7fffu, d[1] & 0x7fff7fffu),
                            pk_max_u16(d[2] & 0x7fff7fffu, d[3] & 0x7fff7fffu));
    m = max(m & 0xffffu, m >> 16);
    m = max(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0xB1, 0xF, 0xF, false));   // lane ^ 1
    const int ef = (int)(m >> 7);
    const int ehi = max(ef, 8) - 7, elo = max(ef, 13) - 12;
    const float shi = __builtin_bit_cast(float, ehi << 23), slo = __builtin_bit_cast(float, elo << 23);
    i16x2_t hw0 = {0, 0}, hw1 = {0, 0};
    hw0 = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(hw0, __builtin_bit_cast(bf16x2_t, d[0]), shi, false);
    hw0 = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(hw0, __builtin_bit_cast(bf16x2_t, d[1]), shi, true);
    hw1 = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(hw1, __builtin_bit_cast(bf16x2_t, d[2]), shi, false);
    hw1 = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(hw1, __builtin_bit_cast(bf16x2_t, d[3]), shi, true);
    const uint32_t h0 = __builtin_bit_cast(uint32_t, hw0), h1 = __builtin_bit_cast(uint32_t, hw1);
    const f32x2_t back[4] = {__builtin_amdgcn_cvt_scalef32_pk_f32_fp8(h0, shi, false),
                             __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(h0, shi, true),
                             __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(h1, shi, false),
                             __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(h1, shi, true)};
    float lo[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {   // exact: x and hi share the exponent range
        lo[2 * q] = __builtin_bit_cast(float, d[q] << 16) - back[q].x;
        lo[2 * q + 1] = __builtin_bit_cast(float, d[q] & 0xffff0000u) - back[q].y;
    }
    i16x2_t lw0 = {0, 0}, lw1 = {0, 0};
    lw0 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lw0, lo[0], lo[1], slo, false);
    lw0 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lw0, lo[2], lo[3], slo, true);
    lw1 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lw1, lo[4], lo[5], slo, false);
    lw1 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lw1, lo[6], lo[7], slo, true);
    if (lane < 32) {
        const int gt = lane >> 1, h = lane & 1, p = gt >> 3, G = gt & 7;
        uint8_t *e = xs + p * 512 + 2 * G * 32 + (G >> 2) * 16 + h * 8;   // slot 2 G (hi); 2 G + 1 (lo) is 32 on
        *reinterpret_cast<uint2 *>(e) = make_uint2(h0, h1);
        *reinterpret_cast<uint2 *>(e + 32) =
            make_uint2(__builtin_bit_cast(uint32_t, lw0), __builtin_bit_cast(uint32_t, lw1));
        if (h == 0)
            *reinterpret_cast<uint16_t *>(xs + S::EXP_OFF + p * 16 + 2 * G) = (uint16_t)(ehi | (elo << 8));
    }
}

// acc[fb] += this lane's share of one matrix's super-tile (lane group q: groups
// 8 p + 2 q, 8 p + 2 q + 1 of each k pair p); wc, ws as for core_mx.
__device__ __forceinline__ void core_mx1(const uint4 (&wc)[kCodeChunks / 2], const uint4 &ws, uint8_t *xs, int lane,
                                         float (&acc)[4][1]) {
    using S = XStage1;
    const int q = lane >> 4, i = lane & 15;
    *reinterpret_cast<uint4 *>(xs + S::WS_OFF + lane * 16) = ws;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        // E4M3 scales of this lane's groups 8 p + 2 q + t, from lanes 16 (2 (q % 2) + t) + n
        float sc[2][4];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int src = 16 * (2 * (q & 1) + t) + i;
            const uint32_t w = *reinterpret_cast<const uint32_t *>(xs + S::WS_OFF + src * 16 + 4 * (2 * p + (q >> 1)));
            const f32x2_t s01 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, false);
            const f32x2_t s23 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, true);
            sc[t][0] = s01.x;
            sc[t][1] = s01.y;
            sc[t][2] = s23.x;
            sc[t][3] = s23.y;
        }
        // A: slot i; data in lane group (i / 2) % 4, the E8M0 scale in lane group i / 4
        const int G = i >> 1;
        const i32x8_t A = *reinterpret_cast<const i32x8_t *>(xs + (q == (G & 3) ? p * 512 + i * 32 : S::ZERO_OFF));
        const uint32_t e2 = *reinterpret_cast<const uint16_t *>(xs + S::EXP_OFF + p * 16 + (i & ~1));
        const int sa = q == (i >> 2) ? (int)((i & 1) ? (e2 >> 8) : (e2 & 0xff)) : 127;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint32_t x[4] = {wc[4 * p + h].x, wc[4 * p + h].y, wc[4 * p + h].z, wc[4 * p + h].w};
            const uint32_t y[4] = {wc[4 * p + 2 + h].x, wc[4 * p + 2 + h].y, wc[4 * p + 2 + h].z, wc[4 * p + 2 + h].w};
            i32x4_t b[2];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const auto r = __builtin_amdgcn_permlane32_swap(x[j], y[j], false, false);
                b[0][j] = (int32_t)r[0];
                b[1][j] = (int32_t)r[1];
            }
#pragma unroll
            for (int o = 0; o < 2; ++o) {
                const int fb = 2 * h + o;
                const i32x8_t B = __builtin_shufflevector(b[o], b[o], 0, 1, 2, 3, -1, -1, -1, -1);
                const f32x4_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
                const f32x4_t D = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, zero, 0, 4, 0, sa, 0, 127);
                acc[fb][0] = __builtin_fmaf(D[0] + D[1], sc[0][fb], acc[fb][0]);
                acc[fb][0] = __builtin_fmaf(D[2] + D[3], sc[1][fb], acc[fb][0]);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// fp16 path (v_mfma_f32_16x16x32_f16).  Each code times its E4M3 group scale
// is exact in fp16 (at most 6 significant bits, magnitudes 2^-10 .. 2688), and
// so is each activation times one power of two per (row, super-tile) for the
// values within 31 binades of that row's largest in the super-tile (the rest,
// below 2^-31 of it, round to the nearest 2^-24 step of the scaled values).
// The products are then ordinary fp16 x fp16 -> fp32 matrix products with no
// masked rows: A rows are the activation rows, B the dequantized weights.
//
// Operand lane layouts of the 16x16x32 product (measured on gfx950): A: lane
// 16 q + i holds row i, k = 8 q .. 8 q + 7; B: lane 16 q + n holds column n,
// k = 8 q .. 8 q + 7; D: lane 16 q + n holds rows 4 q .. 4 q + 3 of column n.
// Any assignment of actual k to the products' k slots is a valid product as
// long as A and B use the same one; here lane group q of the products of k
// pair p (64-k blocks 2 p, 2 p + 1) and step s covers k = K(q) + 8 s + e with
// K(q) = 64 (2 p + q / 2) + 32 (q % 2): exactly the 32 codes the lane holds
// after one v_permlane32_swap of two of its code registers.

// LDS image of one super-tile's activations for the fp16 path, per wave.
template <int ROWS>
struct XStage16 {
    static constexpr int XR = (ROWS * 32 + 63) / 64;   // 16-byte activation chunks per lane
    static constexpr int RA = 2 * XR;                  // rows staged: ROWS rounded up to even
    static constexpr int ROW_BYTES = 528;              // 256 fp16 + 16 (rows start 4 banks apart)
    static constexpr int ZERO_OFF = RA * ROW_BYTES;    // 16 zero bytes: the A rows past ROWS
    // per product row (16): the float undoing its row's scale (zero past RA,
    // zeroed with the 16 bytes before it, once per launch)
    static constexpr int SCALE_OFF = ZERO_OFF + 16;
    static constexpr int WS_OFF = SCALE_OFF + 64;      // the lanes' 16-byte group-scale entries
    static constexpr int BYTES = WS_OFF + 1024;
    static constexpr int ZERO_WORDS = 20;              // zero bytes and row scales, as words
};

// Largest of the two 16-bit halves of m over the 32 lanes of each half-wave:
// within rows of 16 lanes by DPP (quads, half-rows, rows), then across the
// two rows of a half-wave with one v_permlane16_swap, whose two results hold
// rows 2 h and 2 h + 1 in some order (the maximum does not depend on it).
__device__ __forceinline__ uint32_t halfwave_max_u16x2(uint32_t m) {
    m = pk_max_u16(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0xB1, 0xF, 0xF, false));    // quad_perm 1,0,3,2
    m = pk_max_u16(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0x4E, 0xF, 0xF, false));    // quad_perm 2,3,0,1
    m = pk_max_u16(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0x141, 0xF, 0xF, false));   // row_half_mirror
    m = pk_max_u16(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0x140, 0xF, 0xF, false));   // row_mirror
    const auto r = __builtin_amdgcn_permlane16_swap(m, m, false, false);
    return pk_max_u16(r[0], r[1]);
}

// Two fp32 values times sc, each rounded once to fp16 (nearest even, fp16
// denormals kept), packed low first: one v_fma_mixlo_f16 and one
// v_fma_mixhi_f16 into the same register (the compiler splits such pairs
// into multiplies, conversions and packs).
__device__ __forceinline__ uint32_t mul_pk_f16(float lo, float hi, float sc) {
    uint32_t out;
    asm("v_fma_mixlo_f16 %0, %1, %2, 0 op_sel_hi:[0,0,0]\n\t"
        "v_fma_mixhi_f16 %0, %3, %2, 0 op_sel_hi:[0,0,0]"
        : "=&v"(out)
        : "v"(lo), "v"(sc), "v"(hi));
    return out;
}

// Stage the super-tile's activations as fp16, each row scaled by 2^(14 - E)
// where its largest |x| in the super-tile is below 2^(E+1).  Chunk c = lane +
// 64 i holds row c / 32, k = 8 (c % 32) .. + 7: the 32 lanes of a half-wave
// hold one row.  Rows past ROWS are zeros (their loads read nothing) and are
// staged like the others; no lane branches.
template <int ROWS>
__device__ __forceinline__ void stage_x16(const uint4 (&xv)[XStage16<ROWS>::XR], uint8_t *xs, int lane) {
    using S = XStage16<ROWS>;
    constexpr int XR = S::XR, NP = (XR + 1) / 2;
    // |x| maxima of each chunk, two chunks per word (chunk 2 j low, 2 j + 1 high)
    uint32_t mp[NP];
#pragma unroll
    for (int j = 0; j < NP; ++j) mp[j] = 0u;
#pragma unroll
    for (int i = 0; i < XR; ++i) {
        uint32_t m = pk_max_u16(pk_max_u16(xv[i].x & 0x7fff7fffu, xv[i].y & 0x7fff7fffu),
                                pk_max_u16(xv[i].z & 0x7fff7fffu, xv[i].w & 0x7fff7fffu));
        m = max(m & 0xffffu, m >> 16);
        mp[i >> 1] |= (i & 1) ? m << 16 : m;
    }
#pragma unroll
    for (int j = 0; j < NP; ++j) mp[j] = halfwave_max_u16x2(mp[j]);
#pragma unroll
    for (int i = 0; i < XR; ++i) {
        const int c = lane + 64 * i;
        const int r = c >> 5, kk = (c & 31) * 8;
        const uint32_t m = (i & 1) ? mp[i >> 1] >> 16 : mp[i >> 1] & 0xffffu;
        // biased exponent of the row's largest |x|, kept where both scales are
        // normal floats (rows of all zeros or of tiny values take the bottom)
        const int ef = min(max((int)(m >> 7), 15), 254);
        const float sc = __builtin_bit_cast(float, (268 - ef) << 23);    // 2^(141 - ef) = 2^(14 - E)
        const float un = __builtin_bit_cast(float, (ef - 14) << 23);     // 2^(E - 14)
        const uint32_t d[4] = {xv[i].x, xv[i].y, xv[i].z, xv[i].w};
        uint32_t h[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
            h[q] = mul_pk_f16(__builtin_bit_cast(float, d[q] << 16), __builtin_bit_cast(float, d[q] & 0xffff0000u), sc);
        *reinterpret_cast<uint4 *>(xs + r * S::ROW_BYTES + kk * 2) = make_uint4(h[0], h[1], h[2], h[3]);
        *reinterpret_cast<float *>(xs + S::SCALE_OFF + r * 4) = un;   // the row's 32 lanes store the same value
    }
}

// acc[fb][v] += this super-tile's sum for feature 16 fb + n, row 4 q + v: a
// lane keeps only the rows its products hold (lane group q; rows past ROWS
// stay zero).  wc, ws as for core_mx.
template <int ROWS>
__device__ __forceinline__ void core_f16(const uint4 (&wc)[kCodeChunks / 2], const uint4 &ws, uint8_t *xs, int lane,
                                         float (&acc)[4][4]) {
    using S = XStage16<ROWS>;
    typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
    typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
    const int q = lane >> 4, n = lane & 15;
    // group-scale entries: lane (q, n) needs those of lanes 16 (2 (q % 2) + t) + n
    *reinterpret_cast<uint4 *>(xs + S::WS_OFF + lane * 16) = ws;
    f32x4_t D[4];
#pragma unroll
    for (int fb = 0; fb < 4; ++fb) D[fb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        // scales of this lane's two groups (t), for each feature block
        half2_t sh[2][4];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int src = 16 * (2 * (q & 1) + t) + n;
            const uint32_t w = *reinterpret_cast<const uint32_t *>(xs + S::WS_OFF + src * 16 + 4 * (2 * p + (q >> 1)));
            const f32x2_t s01 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, false);
            const f32x2_t s23 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, true);
            const float sv[4] = {s01.x, s01.y, s23.x, s23.y};
#pragma unroll
            for (int fb = 0; fb < 4; ++fb) sh[t][fb] = half2_t{(_Float16)sv[fb], (_Float16)sv[fb]};
        }
        // codes of k pair p: feature blocks 2 h, 2 h + 1 from one swap per register
        uint32_t cb[4][4];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint32_t x[4] = {wc[4 * p + h].x, wc[4 * p + h].y, wc[4 * p + h].z, wc[4 * p + h].w};
            const uint32_t y[4] = {wc[4 * p + 2 + h].x, wc[4 * p + 2 + h].y, wc[4 * p + 2 + h].z, wc[4 * p + 2 + h].w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const auto r = __builtin_amdgcn_permlane32_swap(x[j], y[j], false, false);
                cb[2 * h][j] = r[0];
                cb[2 * h + 1][j] = r[1];
            }
        }
        const int K = 64 * (2 * p + (q >> 1)) + 32 * (q & 1);
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const half8_t A = *reinterpret_cast<const half8_t *>(
                xs + (n < ROWS ? n * S::ROW_BYTES + (K + 8 * st) * 2 : S::ZERO_OFF));
#pragma unroll
            for (int fb = 0; fb < 4; ++fb) {
                const uint32_t w = cb[fb][st];
                const half2_t g = sh[st >> 1][fb];
                const half2_t b0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * g;
                const half2_t b1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * g;
                const half2_t b2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * g;
                const half2_t b3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * g;
                const half8_t B = {b0.x, b0.y, b1.x, b1.y, b2.x, b2.y, b3.x, b3.y};
                D[fb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, B, D[fb], 0, 0, 0);
            }
        }
    }
    const f32x4_t un = *reinterpret_cast<const f32x4_t *>(xs + S::SCALE_OFF + 16 * q);
#pragma unroll
    for (int fb = 0; fb < 4; ++fb)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[fb][v] = __builtin_fmaf(D[fb][v], un[v], acc[fb][v]);
}

// Sum over the four lane groups; lane 16 g + n returns the total of feature
// 16 g + n (the strip's features in lane order).
__device__ __forceinline__ float strip_total(const float (&a)[4], int lane) {
    float t[4];
#pragma unroll
    for (int fb = 0; fb < 4; ++fb) {
        float v = a[fb];
        v += __shfl_xor(v, 16);
        v += __shfl_xor(v, 32);
        t[fb] = v;
    }
    const int g = lane >> 4;
    return g == 0 ? t[0] : g == 1 ? t[1] : g == 2 ? t[2] : t[3];
}

}  // namespace core
}  // namespace nvfp4
