// nvfp4_internal.h -- layout constants, device codecs and launcher declarations
// shared by the translation units of the gfx950 NVFP4 library.
//
// Device codecs (verified exhaustively against the CPU oracle through
// nvfp4_dequant and the quantizer tests):
//   * E2M1 pair -> bf16 pair: v_cvt_scalef32_pk_bf16_fp4 with scale 1.0.  The
//     instruction applies only the exponent of its fp32 scale operand (measured:
//     scale 1.5 leaves a code as is, 3.0 doubles it), so the E4M3 group scale
//     (which has mantissa bits) is applied separately; the low nibble becomes
//     the low bf16.
//   * OCP E4M3 byte -> fp32: v_cvt_f32_fp8 (OCP encoding on gfx950, NaN kept).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nvfp4.h"

namespace nvfp4 {

// ---- packed layout (version 3) -------------------------------------------
// A super-tile (strip s of 64 features, k from 256 u) is 8 code chunks of
// 1 KB, then a 1 KB scale chunk.  Lane l = 16 q + n of a wave reads bytes
// 16 l .. 16 l + 15 of each chunk:
//   code chunk c, dword j: the 8 codes (4 bytes, low nibble first) of feature
//     16 (c >> 1) + n, k = 32 (4 (c & 1) + j) + 8 q .. + 7 of the super-tile;
//   scale chunk, byte 8 b + t: the E4M3 scale of feature 16 (2 (q >> 1) + b) + n,
//     group 2 t + (q & 1) of the super-tile.
// This is the B operand of the 16x16x32 matrix-core product exactly as one
// lane needs it (nvfp4_core.h), and every wave load is a run of whole,
// aligned 128-byte lines.
constexpr int kHeaderBytes = 256;
constexpr int kStripN = 64;        // output features per strip
constexpr int kSuperK = 256;       // k per super-tile
constexpr int kCodeChunks = 8;
constexpr int kCodeChunkBytes = 1024;
constexpr int kScaleOffset = kCodeChunks * kCodeChunkBytes;                     // 8192
constexpr int kSuperBytes = kScaleOffset + 16 * kStripN;                        // 9216
constexpr int kEntriesPerSuper = kSuperBytes / 16;                              // 576

// Byte offset, within a super-tile, of the 4 code bytes of feature f (0..63 in
// the strip) for k = kp .. kp + 7 (kp a multiple of 8 below 256).
__host__ __device__ inline int code_piece_offset(int f, int kp) {
    const int ks = kp >> 5, q = (kp >> 3) & 3;
    return (2 * (f >> 4) + (ks >> 2)) * kCodeChunkBytes + (16 * q + (f & 15)) * 16 + 4 * (ks & 3);
}
// Byte offset, within a super-tile, of the scale of feature f, group gt (0..15).
__host__ __device__ inline int scale_byte_offset(int f, int gt) {
    const int fb = f >> 4, q = 2 * (fb >> 1) + (gt & 1);
    return kScaleOffset + (16 * q + (f & 15)) * 16 + 8 * (fb & 1) + (gt >> 1);
}

// Projection workspace layout.  Fixed regions that do not depend on the
// call's shape, so partial sums of one call can never land where another
// call's counters are: a zero-filled workspace stays valid for calls of any
// shape, since every launch returns its counters to zero.
//   [0, 32 KiB): split-K arrival counters of region 0, one per 128-byte line
//                for each of up to 256 shared strips (a call has fewer shared
//                strips than workgroups);
//   [32 KiB, 64 KiB): one 128-byte line per workgroup of a multi-call launch:
//                word 0 = the last wait it may go past;
//   [64 KiB, 65 KiB): word 0 = set when a wait between calls timed out,
//                word 32 = arrivals at waits, word 64 = workgroups done with
//                the launch (one 128-byte line each);
//   [65 KiB, 161 KiB): the split-K counters of regions 1, 2, 3;
//   [161 KiB, ...): fp32 partial sums, region 0 first, then (in a launch of
//                several calls) regions 1, 2, 3, each P bytes rounded up to 256.
// A launch of several calls runs consecutive calls that do not depend on each
// other without a wait between them, so up to kRegions calls are in flight
// at once, each with counters and partial sums of its own (its region).
constexpr int64_t kMaxN = (int64_t)1 << 20;
constexpr size_t kSyncOffset = 32 * 1024;
constexpr size_t kFlagOffset = 64 * 1024;
constexpr size_t kCounterBytes = 32 * 1024;
constexpr size_t kCounterTailOffset = 65 * 1024;
constexpr int kRegions = 4;
constexpr size_t kPartialOffset = kCounterTailOffset + (kRegions - 1) * kCounterBytes;
static_assert(kFlagOffset == NVFP4_WS_WAIT_FLAG_OFFSET, "the wait flag sits where the ABI says");
static_assert(kPartialOffset == NVFP4_WS_STATE_BYTES, "the state every launch leaves at zero, as the ABI says");
constexpr size_t round_partial(size_t p) { return (p + 255) & ~(size_t)255; }
// Workspace bytes of a launch of several calls whose largest partial sums
// take `partial` bytes.
constexpr size_t sequence_workspace(size_t partial) { return kPartialOffset + kRegions * round_partial(partial); }

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
constexpr int kLeftoverPieces = 4;       // pieces per strip left over past whole strips per workgroup, at most
constexpr size_t kOneWorkgroupPerCuLds = 82 * 1024;   // > half of the 160 KB LDS of a CU
constexpr int kMaxWavesPerWg = 8;
// Rows one kernel call computes; calls of more rows are cut into row chunks
// by the host.  A call runs on the kernel instantiated for the smallest of
// 1, 2, 4, 6, 8, 12, 16 rows that holds it: the rows past the call's read
// zero activations and their outputs are dropped.  Every row is computed by
// the same instructions in the same product positions at every row count, so
// padding changes no result.
constexpr int kKernelMaxRows = 16;
static_assert(NVFP4_MAX_ROWS >= kKernelMaxRows, "the ABI's row limit covers the kernel's");
__host__ __device__ constexpr int kernel_rows(int rows) {
    return rows <= 1 ? 1 : rows <= 2 ? 2 : rows <= 4 ? 4 : rows <= 6 ? 6 : rows <= 8 ? 8 : rows <= 12 ? 12 : 16;
}
// Waves per workgroup and super-tiles each wave keeps in flight (NB, even,
// so that a pair's gate and up super-tiles of one position are always in
// flight together).  The super-tiles in flight live in registers.  Neither
// depends on the row count: the plan, and with it every summation order, is
// the same for every row count.
__host__ __device__ constexpr int max_waves_for_rows(int) { return 8; }
__host__ __device__ constexpr int pipe_depth_for_rows(int) { return 2; }
// Per-wave LDS bytes of the staged activations (core::XStageG) and rows per
// wave-reduction slot (the D rows the lanes hold: 2 per v, 8 per row set).
__host__ __device__ constexpr int x_stage_bytes(int krows) { return 2 * ((krows + 1) / 2) * 528 + 16; }
__host__ __device__ constexpr int red_rows(int krows) {
    return 8 * ((krows + 7) / 8 - 1) + 2 * (((krows < 8 ? krows : 8) + 1) / 2);
}
// Segment ends without a workgroup barrier (up to 4 rows: each wave stores
// its slot and goes on, wave 0 sums them once all are stored), or with
// barriers and the rows' sums spread over the waves (from 6 rows on, where
// wave 0 summing every row alone costs more than the barriers).  Measured on
// the decode step: 3%, 5% and 1% faster at 1, 2 and 4 rows, 2.5-5% slower at
// 6-8 rows.
__host__ __device__ constexpr bool barrier_free_segments(int krows) { return krows <= 4; }
// Buffers of wave-reduction slots, consecutive segments alternating: without
// barriers a wave waits for wave 0's reads of a segment only two segments
// later; with barriers (6-8 rows) a wave writing a segment's slots has passed
// the previous segment's barriers, which wave 0 reaches only after reading
// the sums of the one before, so no barrier opens a segment end (0.4-0.5%
// faster decode step at 6 and 8 rows).  One buffer from 12 rows on, where
// the LDS holds no second one: a barrier opens each segment end there.
__host__ __device__ constexpr int red_buffers(int krows) { return krows <= 8 ? 2 : 1; }

struct StreamPlan {
    int64_t n, k;
    int rows, krows, nmat;    // rows of the call, rows of the kernel that runs it
    int strips, supers;       // S, T
    int G, F, R;              // workgroups, owned strips per workgroup, shared strips
    int Gs;                   // the last Gs workgroups take the shared strips' units
    int waves;                // waves per workgroup taking part in the call
    int max_pieces;           // most pieces any shared strip is cut into
    size_t partial_bytes;     // fp32 partial sums [R][max_pieces][nmat][krows][64] (0 if no strip is cut)
    size_t lds_bytes;
};

// One projection call of a launch: its plan and operands (w1 = nullptr for a
// single projection).
struct StreamCall {
    StreamPlan plan;
    const void *w0, *w1, *x;
    void *y;
    int out_f32;
    // a residual add + RMSNorm call when norm != 0 (1, or 2 with the Gemma
    // offset): x = residual, w0 = delta, w1 = weight, y = normalized output,
    // aux = residual_out; plan.rows rows of plan.k values, no tiles
    int norm;
    const void *aux;
    float eps;
};

// The plan of a residual add + RMSNorm call of a sequence: rows workgroups,
// one row each, no tiles and no workspace.
StreamPlan make_norm_plan(int64_t k, int rows);

StreamPlan make_stream_plan(int64_t n, int64_t k, int rows, int dual);
size_t stream_lds_bytes(int krows, int waves);
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
// Waits between calls those launches make where every run of calls of one
// row count shares a launch (a device with cooperative launches).
int sequence_waits(const StreamCall *calls, int ncalls);
// The same in two steps: build_launches writes the launches of these calls
// (sequence_launches of them, launch_rec_bytes() each, 8-byte aligned) into
// recs and returns their count; launch_recs enqueues them with a workspace.
size_t launch_rec_bytes();
int build_launches(const StreamCall *calls, int ncalls, void *recs);
hipError_t launch_recs(const void *recs, int nrec, void *workspace, hipStream_t stream);

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

// Streaming-read ceiling: read `bytes` (a multiple of 16) once; 256 words to `sink`.
hipError_t launch_read_ceiling(const void *buf, size_t bytes, void *sink, hipStream_t stream);

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
