// nvfp4_gemv.hip -- weight-only NVFP4 projection kernels for gfx950.
//
// y[r][j] = s_g * sum_k (code * scale)[j][k] * x[r][k], 1..8 activation rows,
// and the fused gate/up pair o = silu(g) * u.  The blueprint page for the
// NVFP4 27B model lists these as the w4a16_gemv family ("Kernels" table) with
// weights nvfp4/g16 and bf16 activations ("Precision" table); its planner's
// row_tiers=by_rows picks a variant per row count, here a template per count.
//
// Work decomposition (one kernel launch):
//   * a wave owns one strip of 64 output features (lane l = feature 64*s + l)
//     and one super-tile of 256 k: 8 code loads + 1 scale load of 16 bytes per
//     lane, each a whole aligned 1 KB run for the wave;
//   * a workgroup = `waves` waves on the same strip and consecutive
//     super-tiles; the activation rows of its k-range are staged in LDS once
//     and read back as wave-uniform broadcasts;
//   * the k extent of a strip is split over `parts` workgroups (split-K for the
//     skinny shapes); partial sums go to a caller workspace and the last
//     workgroup to arrive at a strip (arrival counter) adds them in part order
//     0..P-1, so results are bitwise deterministic with no float atomics.
// Decode: two E2M1 codes -> two bf16 (exact), v_dot2 with two bf16 activations
// into an fp32 partial per 16-element group, then one fma with the group's E4M3
// scale; s_g multiplies the reduced sum in the epilogue.
#include "nvfp4_internal.h"

namespace nvfp4 {
namespace {

struct GemvArgs {
    const uint8_t *w0;   // packed weight (gate for the pair)
    const uint8_t *w1;   // packed up weight (pair only)
    const uint16_t *x;   // [ROWS][k] bf16
    void *y;             // [ROWS][n]
    float *partial;      // [P][NMAT][ROWS][n_pad]
    unsigned *counters;  // [S]
    int n, k, T, P, spp, n_pad, out_f32;
};

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

template <int ROWS, int NMAT, bool MFMA>
__global__ __launch_bounds__(256) void gemv_kernel(GemvArgs a) {
    extern __shared__ __align__(16) unsigned char smem[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nthreads = blockDim.x, nwaves = nthreads >> 6;
    const int s = blockIdx.x / a.P, p = blockIdx.x - s * a.P;
    const int u0 = p * a.spp;
    const int u1 = min(a.T, u0 + a.spp);
    const int kbase = u0 * kSuperK;
    const int xstride = a.spp * kSuperK;       // bf16 elements per LDS row
    uint16_t *xs = reinterpret_cast<uint16_t *>(smem);
    float *red = reinterpret_cast<float *>(smem + (size_t)ROWS * xstride * 2);

    // 1. activation chunks (8 bf16 each) of this workgroup's k-range; zero past k.
    //    Issued before the weight loads and without branches, so the wait for
    //    them does not also wait for the weights (the vector memory counter
    //    drains in issue order and the compiler can count exactly).
    constexpr int XMAX = (ROWS + 1) / 2;       // spp == nwaves: ROWS*32*spp / (64*nwaves)
    const int xchunks_per_row = xstride / 8;
    uint4 xr[XMAX];
#pragma unroll
    for (int i = 0; i < XMAX; ++i) {
        const int c = tid + i * nthreads;
        const int r = c / xchunks_per_row;
        const int kk = (c - r * xchunks_per_row) * 8;
        const bool in = r < ROWS && kbase + kk < a.k;
        const size_t off = in ? (size_t)r * a.k + kbase + kk : 0;   // row 0, k 0 is always valid
        xr[i] = *reinterpret_cast<const uint4 *>(a.x + off);
        if (!in) xr[i] = make_uint4(0u, 0u, 0u, 0u);
    }

    // 2. this wave's super-tile of every matrix.  A wave past the end of the
    //    part (only when the part is short) re-reads the part's last super-tile,
    //    which another wave of this workgroup is reading (an L2 hit), and
    //    discards it; keeping the loads unconditional keeps the waits exact.
    const bool active = u0 + wave < u1;
    const int u = active ? u0 + wave : u1 - 1;
    uint4 wc[NMAT][kTilesPerSuper];
    uint4 wsc[NMAT];
#pragma unroll
    for (int m = 0; m < NMAT; ++m) {
        const uint8_t *base = (m == 0 ? a.w0 : a.w1) + kHeaderBytes + ((size_t)s * a.T + u) * kSuperBytes + lane * 16;
#pragma unroll
        for (int t = 0; t < kTilesPerSuper; ++t)
            wc[m][t] = *reinterpret_cast<const uint4 *>(base + t * kChunkBytes);
        wsc[m] = *reinterpret_cast<const uint4 *>(base + kScaleOffset);
    }

    // 3. activations to LDS
#pragma unroll
    for (int i = 0; i < XMAX; ++i) {
        const int c = tid + i * nthreads;
        const int r = c / xchunks_per_row;
        const int kk = (c - r * xchunks_per_row) * 8;
        if (r < ROWS) *reinterpret_cast<uint4 *>(xs + r * xstride + kk) = xr[i];
    }
    __syncthreads();

    // 4. per-lane dot products over the super-tile
    float acc[NMAT][ROWS];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int r = 0; r < ROWS; ++r) acc[m][r] = 0.0f;
    const uint16_t *xw = xs + (u - u0) * kSuperK;
    if (MFMA) core_mfma<ROWS, NMAT>(wc, wsc, xw, xstride, lane, acc);
    else core_dot2<ROWS, NMAT>(wc, wsc, xw, xstride, acc);

    // 5. reduce over the waves of the workgroup, in wave order, into the slots
    //    of wave 0.  Row r is finalized by wave r % nwaves (a runtime loop over
    //    values kept in LDS, so no register arrays indexed by row), so the
    //    split-K and epilogue work of several rows runs on several waves.
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int r = 0; r < ROWS; ++r)
            red[((wave * NMAT + m) * ROWS + r) * kStripN + lane] = active ? acc[m][r] : 0.0f;
    __syncthreads();
    for (int r = wave; r < ROWS; r += nwaves) {
#pragma unroll
        for (int m = 0; m < NMAT; ++m) {
            float t = red[(m * ROWS + r) * kStripN + lane];
            for (int w = 1; w < nwaves; ++w) t += red[((w * NMAT + m) * ROWS + r) * kStripN + lane];
            red[(m * ROWS + r) * kStripN + lane] = t;
        }
    }

    const int f = s * kStripN + lane;

    // 6. split-K: publish this part, the last arrival sums parts 0..P-1 in order.
    //    Partials and counters are touched only by device-scope atomic accesses
    //    (sc1: performed at the device coherence point, past the per-XCD L2), so
    //    no cache-wide writeback or invalidate is needed; the explicit wait makes
    //    every wave's stores complete before the barrier and the arrival count,
    //    and the reader's loads are issued only after the count returns.
    if (a.P > 1) {
        __shared__ unsigned s_last;
        for (int r = wave; r < ROWS; r += nwaves) {
#pragma unroll
            for (int m = 0; m < NMAT; ++m)
                __hip_atomic_store(&a.partial[(((size_t)p * NMAT + m) * ROWS + r) * a.n_pad + f],
                                   red[(m * ROWS + r) * kStripN + lane], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_waitcnt(0);
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __syncthreads();
        if (tid == 0)
            s_last = __hip_atomic_fetch_add(&a.counters[s], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                     (unsigned)(a.P - 1);
        __syncthreads();
        if (!s_last) return;
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        constexpr int QB = 8;   // partial loads in flight per matrix before the in-order adds
        for (int r = wave; r < ROWS; r += nwaves) {
            float t[NMAT];
#pragma unroll
            for (int m = 0; m < NMAT; ++m) t[m] = 0.0f;
            for (int q0 = 0; q0 < a.P; q0 += QB) {
                float pv[NMAT][QB];
#pragma unroll
                for (int j = 0; j < QB; ++j) {
                    const int q = min(q0 + j, a.P - 1);
#pragma unroll
                    for (int m = 0; m < NMAT; ++m)
                        pv[m][j] = __hip_atomic_load(&a.partial[(((size_t)q * NMAT + m) * ROWS + r) * a.n_pad + f],
                                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
#pragma unroll
                for (int j = 0; j < QB; ++j)
                    if (q0 + j < a.P)
#pragma unroll
                        for (int m = 0; m < NMAT; ++m) t[m] += pv[m][j];
            }
#pragma unroll
            for (int m = 0; m < NMAT; ++m) red[(m * ROWS + r) * kStripN + lane] = t[m];
        }
        if (tid == 0) __hip_atomic_store(&a.counters[s], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    // 7. epilogue: global scale, SiLU(g) * u for the pair, bf16 RNE or fp32
    if (f >= a.n) return;
    const float sg0 = *reinterpret_cast<const float *>(a.w0);
    const float sg1 = NMAT == 2 ? *reinterpret_cast<const float *>(a.w1) : 0.0f;
    for (int r = wave; r < ROWS; r += nwaves) {
        float out;
        if (NMAT == 1) {
            out = red[r * kStripN + lane] * sg0;
        } else {
            const float g = red[r * kStripN + lane] * sg0;
            const float uu = red[(ROWS + r) * kStripN + lane] * sg1;
            out = g / (1.0f + expf(-g)) * uu;
        }
        const size_t at = (size_t)r * a.n + f;
        if (a.out_f32) reinterpret_cast<float *>(a.y)[at] = out;
        else reinterpret_cast<uint16_t *>(a.y)[at] = f32_to_bf16_rne(out);
    }
}

template <int ROWS, int NMAT>
hipError_t launch_one(const GemvPlan &pl, const GemvArgs &args, hipStream_t stream) {
    GemvArgs a = args;
    void *kargs[] = {&a};
    const void *fn = pl.mfma ? reinterpret_cast<const void *>(&gemv_kernel<ROWS, NMAT, true>)
                             : reinterpret_cast<const void *>(&gemv_kernel<ROWS, NMAT, false>);
    return hipLaunchKernel(fn,
                           dim3((unsigned)(pl.strips * pl.parts)), dim3((unsigned)(64 * pl.waves)), kargs,
                           pl.lds_bytes, stream);
}

template <int NMAT>
hipError_t launch_rows(const GemvPlan &pl, const GemvArgs &a, hipStream_t stream) {
    switch (pl.rows) {
        case 1: return launch_one<1, NMAT>(pl, a, stream);
        case 2: return launch_one<2, NMAT>(pl, a, stream);
        case 3: return launch_one<3, NMAT>(pl, a, stream);
        case 4: return launch_one<4, NMAT>(pl, a, stream);
        case 5: return launch_one<5, NMAT>(pl, a, stream);
        case 6: return launch_one<6, NMAT>(pl, a, stream);
        case 7: return launch_one<7, NMAT>(pl, a, stream);
        case 8: return launch_one<8, NMAT>(pl, a, stream);
        default: return hipErrorInvalidValue;
    }
}

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

}  // namespace

GemvPlan make_gemv_plan(int64_t n, int64_t k, int rows, int dual) {
    GemvPlan pl{};
    pl.n = n;
    pl.k = k;
    pl.rows = rows;
    pl.nmat = dual ? 2 : 1;
    pl.strips = (int)num_strips(n);
    pl.supers = (int)num_supers(k);
    pl.waves = pl.supers < 4 ? pl.supers : 4;
    pl.supers_per_part = pl.waves;
    pl.parts = (int)ceil_div(pl.supers, pl.supers_per_part);
    pl.mfma = rows >= NVFP4_MFMA_MIN_ROWS;
    if (pl.parts > 1) {
        pl.counter_bytes = kCounterRegionBytes;
        pl.partial_bytes = (size_t)pl.parts * pl.nmat * rows * (size_t)pl.strips * kStripN * sizeof(float);
    }
    pl.lds_bytes = (size_t)rows * pl.supers_per_part * kSuperK * 2 +
                   (size_t)pl.waves * pl.nmat * rows * kStripN * sizeof(float);
    return pl;
}

hipError_t launch_gemv(const GemvPlan &pl, const void *w0, const void *w1, const void *x, void *y,
                       int out_f32, void *workspace, hipStream_t stream) {
    GemvArgs a{};
    a.w0 = static_cast<const uint8_t *>(w0);
    a.w1 = static_cast<const uint8_t *>(w1);
    a.x = static_cast<const uint16_t *>(x);
    a.y = y;
    a.counters = static_cast<unsigned *>(workspace);
    a.partial = pl.parts > 1 ? reinterpret_cast<float *>(static_cast<uint8_t *>(workspace) + pl.counter_bytes)
                             : nullptr;
    a.n = (int)pl.n;
    a.k = (int)pl.k;
    a.T = pl.supers;
    a.P = pl.parts;
    a.spp = pl.supers_per_part;
    a.n_pad = pl.strips * kStripN;
    a.out_f32 = out_f32;
    return pl.nmat == 2 ? launch_rows<2>(pl, a, stream) : launch_rows<1>(pl, a, stream);
}

}  // namespace nvfp4
