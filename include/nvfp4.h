/*
 * nvfp4.h -- C ABI of the MI355X (gfx950) weight-only NVFP4 projection library.
 *
 * Weight-only 4-bit projection ("w4a16" GEMV): weights are NVFP4 -- E2M1 codes,
 * one OCP E4M3 scale per 16 consecutive weights of an output row, one FP32
 * per-tensor scale -- and activations are bf16, 1..128 rows per call.  The
 * format and kernel family are the ones named on the Qwen3.8-27B-NVFP4
 * blueprint page: "Precision" table (weights nvfp4/g16, activations bf16) and
 * "Kernels" table (w4a16_gemv_qg / _sw / _dual / _dual_sw, with the planner
 * setting row_tiers=by_rows choosing a variant per row count).
 *
 * Conventions for every entry point:
 *   - Device pointers are device memory of the current HIP device; host
 *     pointers are marked "host".  The caller owns every buffer; the library
 *     never allocates, frees, or keeps a pointer after returning.
 *   - All work is enqueued on `stream` (a hipStream_t, NULL = default stream)
 *     with no synchronization, so calls are capturable in a HIP graph.
 *   - Status: 0 (NVFP4_OK) or a negative NVFP4_E_* code, returned
 *     synchronously.  Every argument check happens before any HIP call, so
 *     argument errors never touch the device.  nvfp4_last_error() gives a
 *     thread-local message for the last failure.  Faults inside a kernel
 *     surface asynchronously, at the caller's next synchronization.
 *   - The library refuses devices other than gfx950 (NVFP4_E_DEVICE), with a
 *     message naming the architecture found and the one required -- as the
 *     TensorFold issue #603 thread asks of an engine: refuse a format the device
 *     cannot run and name the missing capability.
 *
 * Canonical (unpacked) NVFP4 tensors, row-major:
 *   codes  [n][k/2]  byte j of a row: element 2j in bits 0..3, 2j+1 in bits 4..7;
 *                    code bit 3 = sign, bits 2..1 = exponent (bias 1), bit 0 =
 *                    mantissa: magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6;
 *   scales [n][k/16] OCP E4M3 byte per group of 16 consecutive k (bytes 0x7F
 *                    and 0xFF are NaN; the quantizer never produces them);
 *   global_scale     FP32 multiplier s_g: weight = code * scale * s_g.
 *   k must be a positive multiple of 16 and at most 2^24; 1 <= n <= 2^20.
 *
 * Packed (device-tiled) weight, produced by nvfp4_pack / nvfp4_quantize:
 *   [256-byte header][strip 0: super-tiles 0..T-1][strip 1 ...] ...
 *   strip = 64 output features, super-tile = 64 features x 256 k = 9216 bytes
 *   (layout version 3): 8 code chunks of 1 KB, then a 1 KB scale chunk, each
 *   64 entries of 16 bytes (entry l = 16 q + j is what lane l of a wave reads):
 *     code chunk c, entry l, dword d: the 8 codes (4 canonical bytes) of
 *       feature 64 s + 16 (c >> 1) + j for k = 256 u + 32 (4 (c & 1) + d) + 8 q
 *       .. + 7;
 *     scale chunk, entry l, byte 8 b + t: the E4M3 scale of feature
 *       64 s + 16 (2 (q >> 1) + b) + j, group 16 u + 2 t + (q & 1).
 *   Features >= n and k >= k are zero padding.  Each lane's 16 code bytes hold
 *   the weight operands of four 16x16x32 matrix-core products, and one wave
 *   instruction reads one whole, aligned 1 KB run of 128-byte lines.
 *   The header holds s_g (float at byte 0), the layout magic and version, n, k.
 *
 * Arithmetic of the projections (nvfp4_gemv, the pair, nvfp4_gemv_sequence):
 * every product of a bf16 activation, exactly as stored, and an E2M1 code is
 * exact; each 16-element group's sum comes from the matrix core in fp32 and is
 * multiplied by its E4M3 group scale into an fp32 accumulator; s_g multiplies
 * the fp32 total.  This holds for every finite bf16 activation, subnormals
 * included (fp32 subnormal products are kept).  A row's result is
 * bit-identical whatever the number of rows in the call (1..NVFP4_MAX_ROWS)
 * and run to run.
 */
#ifndef NVFP4_H
#define NVFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NVFP4_ABI_VERSION 2
#define NVFP4_LAYOUT_MAGIC 0x34465056u /* "VPF4" */
#define NVFP4_LAYOUT_VERSION 3u
#define NVFP4_MAX_ROWS 128

enum {
    NVFP4_OK = 0,
    NVFP4_E_NULL = -1,      /* a required pointer is NULL                      */
    NVFP4_E_SHAPE = -2,     /* n or k out of range, k % 16 != 0, mismatched pair */
    NVFP4_E_ROWS = -3,      /* rows outside 1..NVFP4_MAX_ROWS                  */
    NVFP4_E_ALIGN = -4,     /* a pointer is not aligned as documented          */
    NVFP4_E_DTYPE = -5,     /* unknown out_dtype                               */
    NVFP4_E_WORKSPACE = -6, /* workspace missing or smaller than required      */
    NVFP4_E_LAYOUT = -7,    /* nvfp4_weight magic/version/size mismatch        */
    NVFP4_E_DEVICE = -8,    /* no HIP device, or not gfx950                    */
    NVFP4_E_HIP = -9,       /* a HIP runtime call or launch failed             */
    NVFP4_E_OVERLAP = -10   /* an output overlaps an input or the workspace    */
};

enum { NVFP4_OUT_BF16 = 0, NVFP4_OUT_F32 = 1 };

/* Descriptor of a packed weight.  A plain value: copy it freely.  `data` is
 * caller-owned device memory of nvfp4_packed_bytes(n, k) bytes, 16-byte
 * aligned. */
typedef struct nvfp4_weight {
    uint32_t magic;   /* NVFP4_LAYOUT_MAGIC                         */
    uint32_t layout;  /* NVFP4_LAYOUT_VERSION                       */
    int64_t n;        /* output features                            */
    int64_t k;        /* input features, multiple of 16             */
    void *data;       /* device: header + super-tiles               */
} nvfp4_weight;

int nvfp4_abi_version(void);
const char *nvfp4_strerror(int status);
/* thread-local detail of the last failure on this thread ("" if none) */
const char *nvfp4_last_error(void);

/* Bytes of the packed buffer for an [n x k] weight; 0 if the shape is invalid. */
size_t nvfp4_packed_bytes(int64_t n, int64_t k);

/* Re-tile canonical codes/scales (device) into the packed layout and write the
 * header (s_g = global_scale).  The weight-preparation step that the pages'
 * runtimes run on the device before decode (kern README: "weight_prep" kernel
 * and the device "load" program that assembles fused qkv / gate_up buffers).
 * Byte permutation only -- no arithmetic.  codes/scales need no alignment;
 * packed must be 16-byte aligned with packed_bytes >= nvfp4_packed_bytes(n,k).
 * *out (host) is filled on success. */
int nvfp4_pack(const uint8_t *codes, const uint8_t *scales, float global_scale,
               int64_t n, int64_t k, void *packed, size_t packed_bytes,
               nvfp4_weight *out, void *stream);

/* Inverse of nvfp4_pack (test and inspection use): writes canonical codes
 * [n][k/2], scales [n][k/16] and, if global_scale is not NULL, s_g (device
 * float). */
int nvfp4_unpack(const nvfp4_weight *w, uint8_t *codes, uint8_t *scales,
                 float *global_scale, void *stream);

/* Dequantize to fp32 out[n][k] = fp32(fp32(e2m1 * e4m3) * s_g) (test and
 * inspection use).  The codes go through the conversion instruction the
 * projection kernels use (v_cvt_scalef32_pk_bf16_fp4, exact); the scale and
 * s_g are applied in fp32 here, while the projections apply the scale to each
 * group's sum and s_g to the total.  out 16-byte aligned. */
int nvfp4_dequant(const nvfp4_weight *w, float *out, void *stream);

/* Quantize fp32 weights W[n][k] (device, 16-byte aligned) straight into the
 * packed layout: s_g = amax/(448*6); per 16-group E4M3 scale
 * RNE_sat((amax_g/6)/s_g); codes E2M1 RNE_sat(w / (e4m3(scale)*s_g)); a group
 * whose scale decodes to 0 gets all-zero codes.  Bit-identical to the CPU
 * quantizer it is tested against.  The step before the projection: the
 * veloGB10 setup page's "--quantize all" from the bf16 checkpoint, which it
 * says gives output identical to the published NVFP4 artifact.
 * workspace: device, >= nvfp4_quantize_workspace_bytes(n, k) bytes, 16-byte
 * aligned; no initialization needed.  The status word (int32 at workspace
 * byte 0) is set by the device to nonzero if a weight is not finite (the
 * packed contents are then unspecified) and to zero otherwise. */
size_t nvfp4_quantize_workspace_bytes(int64_t n, int64_t k);
int nvfp4_quantize(const float *W, int64_t n, int64_t k, void *packed, size_t packed_bytes,
                   void *workspace, size_t workspace_bytes, nvfp4_weight *out, void *stream);

/* Workspace needed by nvfp4_gemv (dual = 0) or nvfp4_gemv_dual_silu (dual = 1)
 * for this shape and row count: split-K partial sums plus arrival counters.
 * 0 means none.  Deterministic in (n, k, rows, dual). */
size_t nvfp4_workspace_bytes(int64_t n, int64_t k, int rows, int dual);

/* y[r][j] = s_g * sum_k (code * scale)[j][k] * x[r][k]  for r < rows, j < n.
 * x: device bf16 [rows][k], 16-byte aligned.  y: device [rows][n], bf16
 * (NVFP4_OUT_BF16, round to nearest even) or fp32 (NVFP4_OUT_F32), aligned
 * to its element size; y must not overlap x, the weight or the workspace
 * (NVFP4_E_OVERLAP).  fp32 accumulation; results are bitwise deterministic
 * run to run.  A kernel computes up to 16 rows; a call of more rows runs as
 * ceil(rows / 16) chunks of balanced row counts, each reading the weights
 * once (the pages' wider row tiers: up to 32 draft and 128 multi-sequence
 * rows).  A row's result does not depend on the call's row count.
 * workspace: >= nvfp4_workspace_bytes(n, k, rows, 0) bytes, 16-byte aligned,
 * ZERO-FILLED before its first use.  Its first 65 KiB hold counters at fixed
 * positions and every call returns them to zero, so one workspace serves any
 * sequence of calls of any shape on one stream; calls that may run
 * concurrently need distinct workspaces. */
int nvfp4_gemv(const nvfp4_weight *w, const void *x, int rows, void *y, int out_dtype,
               void *workspace, size_t workspace_bytes, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): nvfp4_gemv
 * with the workspace taken from a static array inside the library (one per
 * device, NVFP4_NOALLOC_SCRATCH_BYTES, held until the process ends) instead of
 * the caller's.  Same arguments, results (bit for bit) and errors as
 * nvfp4_gemv; it allocates and frees nothing.  The array holds the largest
 * workspace any valid call needs (at most 255 shared strips of at most 16 rows
 * in fewer than 768 pieces: under 3.2 MB of partial sums per region, four
 * regions for a call of more than 16 rows, plus 161 KiB of counters); a call
 * whose workspace would exceed it is refused with
 * NVFP4_E_WORKSPACE before anything is launched.  Every call on one device shares that device's
 * array, which keeps the last call's contents: calls that may overlap in time
 * on one device (different streams without ordering) race and must not be
 * made.  The array starts at zero and every call leaves its counters at zero. */
#define NVFP4_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int nvfp4_gemv_noalloc(const nvfp4_weight *w, const void *x, int rows, void *y, int out_dtype, void *stream);

/* Fused gate/up pair of the SwiGLU FFN: o = silu(g) * u with
 * g = x W_gate^T, u = x W_up^T (both as in nvfp4_gemv, fp32), silu(g) =
 * g / (1 + exp(-g)), evaluated after the full reduction -- the blueprint
 * page's w4a16_gemv_dual kernels with the silu_mul step (its planner splits
 * that step out as decode_split_silu; here it is the epilogue).  gate and up
 * must have the same n and k.  workspace as for nvfp4_gemv with dual = 1. */
int nvfp4_gemv_dual_silu(const nvfp4_weight *gate, const nvfp4_weight *up, const void *x,
                         int rows, void *y, int out_dtype, void *workspace,
                         size_t workspace_bytes, void *stream);

/* Residual add + RMSNorm inside a sequence (the blueprint page's
 * norm::residual_add_rms_norm between a decoder's projections): the same
 * operation as nvfp4_residual_rmsnorm, run by the sequence's own launch between
 * two of its calls instead of as a launch of its own. */
typedef struct nvfp4_norm {
    const void *residual;    /* device bf16 [rows][k], 16-byte aligned                   */
    const void *delta;       /* device bf16 [rows][k], 16-byte aligned                   */
    const void *weight;      /* device bf16 [k], 16-byte aligned                         */
    void *residual_out;      /* device bf16 [rows][k], 16-byte aligned; may be residual  */
    int64_t k;               /* positive multiple of 16, at most 65536                   */
    float eps;               /* finite, >= 0                                             */
    int gemma_offset;        /* nonzero: w' = 1 + weight                                 */
} nvfp4_norm;

/* One call of a sequence: a projection (norm == NULL, up == NULL), a gate/up
 * pair (norm == NULL, up != NULL), or a residual add + RMSNorm (norm != NULL;
 * then w, up and x must be NULL, y receives the normalized rows -- bf16
 * [rows][norm->k], 16-byte aligned, out_dtype NVFP4_OUT_BF16 -- and a later
 * call may take y as its x and norm->residual_out as a later norm's
 * residual). */
typedef struct nvfp4_call {
    const nvfp4_weight *w;   /* the projection's weight; the gate weight of a pair */
    const nvfp4_weight *up;  /* NULL, or the pair's up weight (same n, k as w)     */
    const void *x;           /* device bf16 [rows][k], 16-byte aligned             */
    void *y;                 /* device [rows][n], bf16 or fp32 per out_dtype       */
    int rows;                /* 1..NVFP4_MAX_ROWS                                  */
    int out_dtype;           /* NVFP4_OUT_BF16 or NVFP4_OUT_F32                    */
    const nvfp4_norm *norm;  /* NULL, or the residual add + RMSNorm this call is   */
} nvfp4_call;

/* Byte offset, in a projection workspace, of the uint32 wait flag: a launch
 * sets it to nonzero if one of its bounded waits gave up -- a wait between the
 * calls of a launch of several calls (nvfp4_gemv_sequence), or, in a launch
 * with a workspace, a wave of a workgroup waiting for the others at the end of
 * a strip segment -- after 2^18 polls (well under a second); it then goes on
 * so that no launch can hang, and that launch's results are not reliable.
 * Nothing clears it but the caller: read it after a synchronization to check
 * a run of launches. */
#define NVFP4_WS_WAIT_FLAG_OFFSET 65536

/* The first NVFP4_WS_STATE_BYTES of a projection workspace hold counters and
 * wait words that every launch leaves at zero (the wait flag aside); the
 * partial sums follow. */
#define NVFP4_WS_STATE_BYTES ((size_t)161 << 10)

/* Workspace for nvfp4_gemv_sequence: for one call what nvfp4_gemv needs;
 * for several, NVFP4_WS_STATE_BYTES + 4 x the largest partial sums any of its
 * calls needs (rounded up to 256 bytes): up to four consecutive calls that do
 * not depend on each other run at once, each with counters and partial sums
 * of its own. */
size_t nvfp4_sequence_workspace_bytes(const nvfp4_call *calls, int ncalls);

/* Enqueue a whole decode step's projections with one host call: every call is
 * validated first (nothing is launched if any is invalid; the message names
 * the failing call's index), then the calls run in order on `stream`, each
 * computing exactly what nvfp4_gemv / nvfp4_gemv_dual_silu would (bit for
 * bit), sharing the one workspace.  The pages drive a decode step of several
 * hundred launches as one captured graph (kern README, "decode" programs; the
 * NVFP4 blueprint's 755 launches per step); here runs of up to 256 consecutive
 * calls with the same row count share one cooperative launch.  A call that
 * reads what an earlier call of the launch writes, or writes what one reads or
 * writes (by address ranges), starts only after every workgroup has finished
 * every earlier call (a wait); calls that depend on none of the calls since
 * the last wait run without one, up to four at a time (a call's next weight
 * tiles are fetched across either).  So a call may read the y of an earlier
 * call as its x, and the results are those of the calls made one by one.
 * No call's y may overlap any call's weight, its own x or the workspace
 * (NVFP4_E_OVERLAP).
 * Residual add + RMSNorm calls (norm != NULL) run inside the same launch, one
 * workgroup per row, with the arithmetic and summation order of
 * nvfp4_residual_rmsnorm: both outputs are bit-identical to it.  A norm's
 * delta may be an earlier call's y; its outputs may not overlap any weight or
 * the workspace, and its residual_out no other call's y.
 * events: NULL, or 2*ncalls hipEvent_t handles (entries may be NULL); with
 * events every call gets a launch of its own, events[2i] is recorded on
 * `stream` right before call i and events[2i+1] right after it, for
 * per-launch device timing. */
int nvfp4_gemv_sequence(const nvfp4_call *calls, int ncalls, void *workspace, size_t workspace_bytes,
                        void *const *events, void *stream);

/* Waits between calls the launches of nvfp4_gemv_sequence make for these
 * calls on a device with cooperative launches (calls of one row count share
 * a launch): the calls that depend on an earlier call of their launch, plus
 * one for every fifth call of a run of independent ones.  The calls are
 * validated as nvfp4_gemv_sequence validates them (but for the workspace);
 * a negative NVFP4_E_* status if one is invalid. */
int nvfp4_sequence_waits(const nvfp4_call *calls, int ncalls);

/* A call list validated once and kept, for a decode step launched many times
 * (the pages capture a step once and replay it: kern README, "Layout").
 * nvfp4_sequence_plan_bytes: host bytes of the plan of these calls, 0 if a
 * call is invalid (nvfp4_last_error says which).  nvfp4_sequence_plan:
 * validates the calls exactly as nvfp4_gemv_sequence does (but for the
 * workspace) and writes the plan -- the kernel launches with every argument
 * but the workspace -- into `plan`: caller-owned host memory, 16-byte aligned,
 * at least nvfp4_sequence_plan_bytes long (NVFP4_E_WORKSPACE otherwise).  The
 * plan holds the calls' device pointers: their buffers must stay allocated
 * and the plan unchanged while it is used, on the device current when it was
 * made.  nvfp4_sequence_plan_launch: enqueues the plan's launches on `stream`
 * -- the same work as nvfp4_gemv_sequence with no events, bit for bit --
 * after checking only the plan's header, the workspace (size, alignment, no
 * overlap with any output) and the device: O(ncalls) host work. */
size_t nvfp4_sequence_plan_bytes(const nvfp4_call *calls, int ncalls);
int nvfp4_sequence_plan(const nvfp4_call *calls, int ncalls, void *plan, size_t plan_bytes);
int nvfp4_sequence_plan_launch(const void *plan, void *workspace, size_t workspace_bytes, void *stream);

/* Dense bf16 projection, for the projection whose weights stay bf16: the lm
 * head (the Qwen3.8-27B-NVFP4 blueprint page, "Precision" table, bf16 x bf16
 * nodes; its kernel table names the step gemv::dense_gemv_bf16).
 * y[r][j] = sum_k W[j][k] x[r][k] for r < rows, j < n, fp32 accumulation.
 * W: device bf16 [n][k] row-major (as stored), 16-byte aligned; n, k as for
 * the NVFP4 calls (1 <= n <= 2^20, k a positive multiple of 16, k <= 2^24).
 * x: device bf16 [rows][k], 16-byte aligned, rows 1..NVFP4_MAX_ROWS (a kernel
 * pass takes up to 16 rows; more run as balanced row chunks, each reading W
 * once).  y: device [rows][n], bf16 (NVFP4_OUT_BF16, RNE) or fp32, aligned to
 * its element size, not overlapping W or x (NVFP4_E_OVERLAP).  No workspace;
 * bitwise deterministic; enqueued on `stream`. */
int nvfp4_dense_gemv_bf16(const void *W, int64_t n, int64_t k, const void *x, int rows, void *y,
                          int out_dtype, void *stream);

/* MXFP4 projection, the microscaling format variant (E2M1 codes with one E8M0
 * power-of-two scale per 32 consecutive k of a row, no tensor scale; the
 * pages name it through the kern build's gpu_mxfp4 kernels), in the format's
 * own row-major layout, no repacking:
 *   y[r][j] = sum_k e2m1(code[j][k]) * 2^(scale[j][k/32] - 127) * x[r][k].
 * codes: device [n][k/2] bytes (element 2i in the low nibble of byte i),
 * 16-byte aligned; scales: device [n][k/32] E8M0 bytes (255, NaN, gives NaN
 * results); 1 <= n <= 2^20, k a positive multiple of 32, k <= 2^24; x, rows,
 * y, out_dtype as for nvfp4_gemv (more than 16 rows run as row chunks, each
 * reading the weight once).  No workspace; bitwise deterministic. */
int nvfp4_mxfp4_gemv(const void *codes, const void *scales, int64_t n, int64_t k, const void *x, int rows,
                     void *y, int out_dtype, void *stream);

/* W8G32_F16S projection, the 8-bit format variant (signed 8-bit weights with
 * one fp16 scale per 32 consecutive k of a row, symmetric; the pages name this
 * encoding for the DFlash2 drafter's matrices), row-major:
 *   y[r][j] = sum_k code[j][k] * scale[j][k/32] * x[r][k].
 * codes: device int8 [n][k], 16-byte aligned; scales: device fp16 [n][k/32],
 * 8-byte aligned; 1 <= n <= 2^20, k a positive multiple of 128, k <= 2^24;
 * x, rows, y, out_dtype as for nvfp4_gemv (more than 16 rows run as row
 * chunks).  No workspace; bitwise deterministic. */
int nvfp4_w8g32_gemv(const void *codes, const void *scales, int64_t n, int64_t k, const void *x, int rows,
                     void *y, int out_dtype, void *stream);

/* Residual add + RMSNorm, the step that produces a projection's activations
 * (the blueprint page's kernel table: norm::residual_add_rms_norm; kern's
 * gemma_rms_norm is the variant with the Gemma offset).  Per row r < rows:
 *   residual_out[r] = bf16(residual[r] + delta[r])            (RNE)
 *   x[r][j] = bf16(residual_out[r][j] * w'[j] / sqrt(mean_j(residual_out[r]^2) + eps))
 * with w' = weight, or 1 + weight when gemma_offset != 0; fp32 arithmetic.
 * residual, delta, residual_out, x: device bf16 [rows][k]; weight: device bf16
 * [k]; every buffer 16-byte aligned; k a positive multiple of 16, at most
 * 65536; rows 1..2^20; eps finite and >= 0.  residual_out may be residual
 * itself (in-place update); no other overlap (NVFP4_E_OVERLAP).  Bitwise
 * deterministic; enqueued on `stream`. */
int nvfp4_residual_rmsnorm(const void *residual, const void *delta, const void *weight, int64_t k, int rows,
                           float eps, int gemma_offset, void *residual_out, void *x, void *stream);

/* Number of kernel launches nvfp4_gemv_sequence makes for these calls without
 * events on the current device (one per call where shared launches are not
 * available); 0 if ncalls <= 0 or calls is NULL. */
int nvfp4_sequence_launches(const nvfp4_call *calls, int ncalls);

/* Measurement aid, not part of the method: read `bytes` of device memory at
 * `buf` once with the projection kernel's launch shape (16-byte nontemporal
 * loads, one 512-thread workgroup per CU) and nothing else -- the streaming
 * read ceiling the projections are compared with beside the nominal HBM peak.
 * buf 16-byte aligned, bytes a positive multiple of 16; sink: device, 256
 * uint32 (4-byte aligned), receives a fold of the bytes read. */
int nvfp4_read_ceiling(const void *buf, size_t bytes, void *sink, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* NVFP4_H */
