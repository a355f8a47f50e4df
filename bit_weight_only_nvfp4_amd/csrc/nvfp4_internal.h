// nvfp4_internal.h -- layout constants, device codecs and launcher declarations
// shared by the translation units of the gfx950 NVFP4 library.
//
// Device codecs (verified exhaustively against the CPU oracle through
// nvfp4_dequant and the quantizer tests):
//   * E2M1 pair -> bf16 pair: v_cvt_scalef32_pk_bf16_fp4 with scale 1.0.  The
//     instruction applies only the exponent of its fp32 scale operand, so the
//     E4M3 group scale (which has mantissa bits) is applied separately; the low
//     nibble becomes the low bf16.
//   * OCP E4M3 byte -> fp32: v_cvt_f32_fp8 (OCP encoding on gfx950, NaN kept).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nvfp4.h"

namespace nvfp4 {

// ---- packed layout (version 2) -------------------------------------------
// A super-tile (strip s of 64 features, k from 256 u) is an array of 16-byte
// entries: 16 code chunks of 32 entries (chunk c = 4 kb + fb, entry 16 h + j:
// codes of feature 16 fb + j, k = 64 kb + 32 h .. + 31 of the super-tile),
// then 64 scale entries (entry 16 g + j, byte 4 kb + fb: scale of feature
// 16 fb + j, group 4 kb + g of the super-tile).
constexpr int kHeaderBytes = 256;
constexpr int kStripN = 64;        // output features per strip
constexpr int kSuperK = 256;       // k per super-tile
constexpr int kFeatureBlock = 16;  // features per matrix-core product
constexpr int kKBlock = 64;        // k per matrix-core product
constexpr int kCodeChunks = (kStripN / kFeatureBlock) * (kSuperK / kKBlock);   // 16
constexpr int kCodeChunkBytes = kFeatureBlock * kKBlock / 2;                    // 512
constexpr int kScaleOffset = kCodeChunks * kCodeChunkBytes;                     // 8192
constexpr int kSuperBytes = kScaleOffset + 16 * kStripN;                        // 9216
constexpr int kEntriesPerSuper = kSuperBytes / 16;                              // 576

// Byte offset, within a super-tile, of the code entry holding feature f (0..63
// in the strip) and k = kr .. kr + 31 (kr a multiple of 32 below 256).
__host__ __device__ inline int code_entry_offset(int f, int kr) {
    return ((kr >> 6) * 4 + (f >> 4)) * kCodeChunkBytes + ((((kr >> 5) & 1) << 4) + (f & 15)) * 16;
}
// Byte offset, within a super-tile, of the scale of feature f, group gt (0..15).
__host__ __device__ inline int scale_byte_offset(int f, int gt) {
    return kScaleOffset + (((gt & 3) << 4) + (f & 15)) * 16 + (gt >> 2) * 4 + (f >> 4);
}

// Projection workspace layout.  Fixed regions that do not depend on the
// call's shape, so partial sums of one call can never land where another
// call's counters are: a zero-filled workspace stays valid for calls of any
// shape, since every launch returns its counters to zero.
//   [0, 32 KiB): split-K arrival counters, one per 128-byte line for each of
//                up to 256 shared strips (a call has fewer shared strips
//                than workgroups);
//   [32 KiB, 64 KiB): one 128-byte line per workgroup of a multi-call launch:
//                word 0 = the last call it may go past;
//   [64 KiB, 65 KiB): word 0 = set when a wait between calls timed out,
//                word 32 = arrivals between calls, word 64 = workgroups
//                done with the launch (one 128-byte line each);
//   [65 KiB, ...): fp32 partial sums of the call running.
constexpr int64_t kMaxN = (int64_t)1 << 20;
constexpr size_t kSyncOffset = 32 * 1024;
constexpr size_t kFlagOffset = 64 * 1024;
constexpr size_t kPartialOffset = 65 * 1024;

// Bytes 32..255 of the header are always zero (pack and quantize write them);
// kernels use them as a 16-byte source of zeros.
constexpr int kHeaderZeroOffset = 64;

struct Header {
    float global_scale;
    uint32_t magic;
    uint32_t layout;
    uint32_t reserved;
    int64_t n;
    int64_t k;
};

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t num_strips(int64_t n) { return ceil_div(n, kStripN); }
inline int64_t num_supers(int64_t k) { return ceil_div(k, kSuperK); }

// ---- device codecs ----------------------------------------------------------
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// byte `sel` of `word` (two E2M1 codes) -> two bf16, low nibble first
template <int SEL>
__device__ __forceinline__ bf16x2_t e2m1x2_to_bf16x2(uint32_t word) {
    return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, 1.0f, SEL);
}

// byte `sel` of `word` (OCP E4M3) -> fp32
template <int SEL>
__device__ __forceinline__ float e4m3_to_f32(uint32_t word) {
    return __builtin_amdgcn_cvt_f32_fp8(word, SEL);
}

__device__ __forceinline__ float e4m3_to_f32_dyn(uint32_t word, int sel) {
    switch (sel & 3) {
        case 0: return e4m3_to_f32<0>(word);
        case 1: return e4m3_to_f32<1>(word);
        case 2: return e4m3_to_f32<2>(word);
        default: return e4m3_to_f32<3>(word);
    }
}

__device__ __forceinline__ float bf16_lo_to_f32(bf16x2_t v) {
    return __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, v) << 16);
}
__device__ __forceinline__ float bf16_hi_to_f32(bf16x2_t v) {
    return __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, v) & 0xFFFF0000u);
}

// fp32 -> bf16 bits, round to nearest even (NaN stays a quiet NaN)
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    const uint32_t u = __builtin_bit_cast(uint32_t, f);
    const uint32_t rne = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
    const uint32_t nan = (u >> 16) | 0x40u;   // quiet NaN, sign and payload top kept
    return (uint16_t)((u & 0x7FFFFFFFu) > 0x7F800000u ? nan : rne);   // a select, no branch
}

// Launch shape of the persistent streaming projection kernel.
constexpr int kMaxWorkgroups = 256;      // one per CU on MI355X
constexpr int kOwnerMinStrips = 160;     // from here on, whole strips per workgroup
constexpr size_t kOneWorkgroupPerCuLds = 82 * 1024;   // > half of the 160 KB LDS of a CU
constexpr int kMaxWavesPerWg = 8;
// Rows one kernel call computes (the instantiated row counts are 1..16);
// calls of more rows are cut into row chunks by the host.
constexpr int kKernelMaxRows = 16;
static_assert(NVFP4_MAX_ROWS >= kKernelMaxRows, "the ABI's row limit covers the kernel's");
// Waves per workgroup and super-tiles each wave keeps in flight (NB, even,
// so that a pair's gate and up super-tiles of one position are always in
// flight together).  The super-tiles in flight live in registers.  Two waves
// per SIMD with two super-tiles each fit in 256 registers at every row count
// (about 145 at 1 row, 245 at 8).  Measured against it on the decode-step
// sweep: one wave per SIMD with six in flight and three waves per SIMD with
// two were 6-15% slower at 1-2 rows, and four in flight at two waves per SIMD
// (1-2 rows, 225-252 registers) within 1% either way.  The calls of a decode
// step are short (a few super-tiles per wave), and what a call costs beyond
// its bytes is latency at its start and end, which more bytes in flight do
// not shorten.  A wave can have at most 63 vector-memory loads outstanding (a
// super-tile takes 9 plus one per 64 lanes of activations), which bounds NB
// at 6 (1-2 rows) or 4 (up to 8 rows).
__host__ __device__ constexpr int max_waves_for_rows(int rows) { return 8; }
__host__ __device__ constexpr int pipe_depth_for_rows(int rows) { return 2; }
// Super-tile arithmetic: the fp16 matrix-core path (dequantized weights, fp16
// activations) from 5 rows on, the block-scaled fp8 x fp4 path below; and the
// per-wave LDS bytes of its staged activations (core::XStage16, core::XStage1
// at one row, core::XStage).
// The fp8 path masks 3 of every 4 product rows and splits each activation in
// two; the fp16 path pays instead for converting every code (about 512 vector
// instructions per super-tile, whatever the row count).  Measured on the
// decode-step sweep, fp16 is 8-12% slower at 1-4 rows (one row quad: 16
// products per super-tile on the fp8 path) and 1.4-4.7% faster at 5-8 (two
// row quads, 32 products).
constexpr int kF16FromRows = 5;
__host__ __device__ constexpr bool use_f16_core(int rows) { return rows >= kF16FromRows; }
__host__ __device__ constexpr int x_stage_bytes(int rows) {
    return use_f16_core(rows) ? (rows + 1) / 2 * 2 * 528 + 16 + 64 + 1024 : rows == 1 ? 2112 : 2304 * ((rows + 3) / 4) + 32;
}

// Rows per wave-reduction slot (a wave's sums of one matrix for one strip):
// on the fp16 path each lane stores the rows of its own products, all 16.
__host__ __device__ constexpr int red_rows(int rows) { return use_f16_core(rows) ? 16 : rows; }

struct StreamPlan {
    int64_t n, k;
    int rows, nmat;
    int strips, supers;       // S, T
    int G, F, R;              // workgroups, owned strips per workgroup, shared strips
    int waves;                // waves per workgroup taking part in the call
    int max_pieces;           // most pieces any shared strip is cut into
    size_t partial_bytes;     // fp32 partial sums [R][max_pieces][nmat][rows][64] (0 if no strip is cut)
    size_t lds_bytes;
};

// One projection call of a launch: its plan and operands (w1 = nullptr for a
// single projection).
struct StreamCall {
    StreamPlan plan;
    const void *w0, *w1, *x;
    void *y;
    int out_f32;
};

StreamPlan make_stream_plan(int64_t n, int64_t k, int rows, int dual);
size_t stream_lds_bytes(int rows, int waves);
// Workspace bytes for these calls run by launch_sequence (one call: what
// nvfp4_gemv needs; several: the completion counts too).
size_t sequence_workspace_bytes(const StreamCall *calls, int ncalls);
// Whether several calls can share one launch on this device (cooperative launch).
bool cooperative_ok();
// Run the calls in order on `stream`: runs of calls with the same row count
// share one launch when cooperative launches are available.
hipError_t launch_sequence(const StreamCall *calls, int ncalls, void *workspace, hipStream_t stream);
// Launches launch_sequence makes for these calls.
int sequence_launches(const StreamCall *calls, int ncalls);

// Dense bf16 projection (rows <= kKernelMaxRows): y[r][j] = sum_k W[j][k] x[r][k].
hipError_t launch_dense(const void *w, int64_t n, int64_t k, const void *x, int rows, void *y, int out_f32,
                        hipStream_t stream);

// MXFP4 projection (rows <= kKernelMaxRows): codes [n][k/2], E8M0 scales [n][k/32].
hipError_t launch_mx(const void *codes, const void *scales, int64_t n, int64_t k, const void *x, int rows, void *y,
                     int out_f32, hipStream_t stream);

// W8G32_F16S projection (rows <= kKernelMaxRows, k % 128 == 0): int8 codes [n][k],
// fp16 scales [n][k/32].
hipError_t launch_w8(const void *codes, const void *scales, int64_t n, int64_t k, const void *x, int rows, void *y,
                     int out_f32, hipStream_t stream);

// Residual add + RMSNorm, one workgroup per row (k <= norm_max_k()).
int64_t norm_max_k();
hipError_t launch_residual_rmsnorm(const void *r, const void *h, const void *w, int64_t k, int rows, float eps,
                                   int gemma_offset, void *r_out, void *x, hipStream_t stream);

hipError_t launch_pack(const uint8_t *codes, const uint8_t *scales, float global_scale,
                       int64_t n, int64_t k, void *packed, hipStream_t stream);
hipError_t launch_unpack(const void *packed, int64_t n, int64_t k, uint8_t *codes,
                         uint8_t *scales, float *global_scale, hipStream_t stream);
hipError_t launch_dequant(const void *packed, int64_t n, int64_t k, float *out,
                          hipStream_t stream);
size_t quantize_workspace_bytes(int64_t n, int64_t k);
hipError_t launch_quantize(const float *W, int64_t n, int64_t k, void *packed,
                           void *workspace, hipStream_t stream);

}  // namespace nvfp4
