// nvfp4_stream.hip -- persistent streaming NVFP4 projection kernel for gfx950.
//
// y[r][j] = s_g * sum_k (code * scale)[j][k] * x[r][k] for 1..16 activation rows,
// and the gate/up pair o = silu(g) * u (the w4a16_gemv / w4a16_gemv_dual kernel
// family of the Qwen3.8-27B-NVFP4 blueprint page, "Kernels" table).
//
// One launch runs an ordered list of projection calls (one call for
// nvfp4_gemv, a decode step's projections for nvfp4_gemv_sequence).  Decode
// GEMVs are bound by the HBM weight stream, so the launch is shaped for the
// stream rather than for the arithmetic:
//   * at most one workgroup per CU (G <= 256), all resident at once (a
//     cooperative launch when there are several calls);
//   * two waves per SIMD, each running a pipeline of NB = 2 super-tiles (64
//     features x 256 k) in registers: the codes, scales and activation window
//     of super-tile i+1 are in flight while super-tile i is computed.  The
//     activation window travels with its weights, so it is never stuck
//     behind other waves' weight loads;
//   * the pipeline runs across calls: while a call's last tiles are computed
//     and its results written, the first NB super-tiles of the next call are
//     already in flight;
//   * a workgroup owns whole strips of 64 features where it can (no split-K,
//     no cross-workgroup traffic); skinny shapes are cut into balanced pieces
//     of strips over all workgroups ("stream-K"), and the strips left over
//     past whole strips per workgroup into at most 4 pieces each, on the last
//     workgroups (those a narrower call before them left idle);
//   * pieces of a strip are summed in piece order by the last to arrive (an
//     arrival counter), so results are bitwise deterministic with no float
//     atomics, and identical whether a call runs alone or in a sequence;
//   * a call that depends on an earlier call of the launch (reads what it
//     writes, or writes what it reads or writes) starts only after every
//     workgroup has finished every earlier call (a completion count per
//     launch); independent calls follow each other without a wait, up to
//     four at once, each with its own workspace region;
//   * the waves of a workgroup meet only where they must: up to 4 rows a
//     segment end takes no barrier (LDS counters), from 6 rows on it takes
//     barriers and spreads the sums over the waves;
//   * the workgroup's geometry of every call is computed once per launch
//     (LDS table), and up to 4 rows a tile's weights are read through a
//     buffer resource over the super-tile (no per-load address arithmetic).
// Everything one workgroup writes to global memory -- outputs, partial sums,
// counters -- is written by its wave 0 with device-coherent (sc1) accesses, and
// wave 0 is the only wave with no loads in flight across a call boundary, so it
// can wait for its own writes to complete before it counts the call done
// without waiting for the other waves' next weight loads.  Activations are read
// with device-coherent loads as well.  No cache-wide flushes.
//
// Work units of a call: strip s in [0, S) x super-tile u in [0, T).  G
// workgroups; the first G*F strips are owned, F per workgroup; the R = S - G*F
// remaining strips form R*T shared units split into Gs contiguous ranges
// [s*RT/Gs, (s+1)*RT/Gs) of the last Gs workgroups (s = g - (G - Gs); Gs = G
// for skinny shapes), cut at strip boundaries into pieces.
#include <algorithm>
#include <atomic>
#include <type_traits>
#include <vector>

#include "nvfp4_core.h"

namespace nvfp4 {
namespace {
using namespace core;

// One call of a launch.
// A residual add + RMSNorm call (kNorm) reuses the fields: x = residual,
// w0 = delta, w1 = the norm weight (bf16 [k]), y = the normalized output,
// aux = residual_out, n = k = the row length, eps; it has no tiles (waves 0).
struct CallDesc {
    const uint8_t *w0;    // packed weight (gate of the pair)
    const uint8_t *w1;    // packed up weight of a pair; w0 otherwise
    const uint16_t *x;    // [rows][k] bf16
    void *y;              // [rows][n]
    void *aux;            // norm: residual_out
    int n, k, T;
    int G, F, R;          // workgroups taking part, owned strips each, shared strips
    union {
        int max_pieces;   // pieces a shared strip is cut into, at most
        float eps;        // norm: added to the mean square
    };
    int waves;            // waves taking part
    int flags;            // kPair | kOutF32 | kReloadX
    int rows;             // the call's rows (the kernel's ROWS may be more: those rows read and write nothing)
};
constexpr int kPair = 1, kOutF32 = 2, kNorm = 8, kGemma = 16;
// The call waits for every earlier call of the launch to complete before it
// starts (it reads or overwrites what one of them writes or reads); without
// it the call starts as soon as this workgroup is done with the call before.
constexpr int kWaitBefore = 32;
// Bits 8..9: the call's workspace region (counters and partial sums).
constexpr int kRegionShift = 8;
// Bits 16..23: the workgroups the shared strips are spread over, minus one
// (the last of the call's G; the others own whole strips only).
constexpr int kShareShift = 16;
// x is written by the call before this one in the same launch: the activations
// of a super-tile fetched before the call started are fetched again.
constexpr int kReloadX = 4;
// Calls per launch: a decode step's 256 projection calls in one launch.  The
// call table travels in the kernel arguments (80 bytes a call, 20 KB here) and
// is copied into LDS once per workgroup.
constexpr int kSeqMax = 256;

// 16 zero bytes for the dummy loads of a norm call (a packed weight's header
// holds its own: a norm's buffers may be shorter than a header)
__device__ __align__(16) uint8_t g_zero16[16];

__device__ __forceinline__ const uint8_t *zero_of(const CallDesc &d) {
    return (d.flags & kNorm) ? g_zero16 : d.w0 + kHeaderZeroOffset;
}

// What every call of a launch shares: the workspace regions and the grid.
// In the kernel, partial and counters are those of the call running (its
// region); in the arguments, region 0's.
struct LaunchShared {
    float *partial;       // [R][max_pieces][nmat][rows][64] of the call running
    unsigned *counters;   // arrival count of shared strip sh at word 32 sh (one 128-byte line each)
    unsigned *sync;       // word 32 g: the last wait workgroup g may go past (one 128-byte line each)
    unsigned *flags;      // word 0: a wait between calls timed out; 32: arrivals; 64: workgroups exited
    unsigned *counters_tail;   // the counters of regions 1..
    int pstride;          // floats from one region's partial sums to the next
    int ncalls;
    int G;                // workgroups of the launch
};
// Kernel arguments: the shared part and a table of N calls (N = 1 for a
// launch of one call, so that it copies no more than it needs).
template <int N>
struct KernelArgs {
    LaunchShared s;
    CallDesc call[N];
};
using SeqArgs = KernelArgs<kSeqMax>;
static_assert(sizeof(SeqArgs) <= 24 * 1024, "kernel arguments of a launch (measured to work up to 32 KB)");
static_assert(sizeof(CallDesc) % 4 == 0, "call descriptors are copied as words");

constexpr int kSC1 = 16;                          // cache policy: device-coherent access
constexpr int kNT = 2;                            // cache policy: nontemporal (streamed once)
constexpr int kBufferLoadRowsCut = 4;             // tile weight loads through a buffer resource up to here
constexpr int kDroppedOffset = 0x7fffffff;        // past any buffer: loads read 0, stores are dropped
constexpr int kRsrcWord3 = 0x00020000;            // raw buffer, 32-bit data format
// Polls a wait between calls makes before it gives up (each poll is a round
// trip to memory, about a microsecond): counted rather than timed, so a
// dispatch that the scheduler pauses cannot run out of time while paused.
constexpr unsigned kMaxPolls = 1u << 18;

// Workgroup whose shared range [floor(g*U/G), floor((g+1)*U/G)) holds shared
// unit v: the largest g with g*U < (v+1)*G, i.e. ((v+1)*G - 1) / U.
__host__ __device__ __forceinline__ int owner_wg(long long v, long long U, int G) {
    return (int)(((v + 1) * G - 1) / U);
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

typedef const __attribute__((address_space(1))) u32x4_t *global_u32x4_ptr;

// Streamed-once weight bytes: nontemporal loads keep them from displacing the
// activations and partials in the caches.  The pointer is declared global:
// where the compiler cannot prove it (a pointer carried across calls), it
// would otherwise emit a flat load, which also counts against the LDS wait
// counter and makes every later LDS wait wait for the weights.
__device__ __forceinline__ uint4 load_nt(const uint8_t *p) {
    const u32x4_t t = __builtin_nontemporal_load((global_u32x4_ptr)(p));
    return make_uint4(t.x, t.y, t.z, t.w);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, kRsrcWord3);
}

// One super-tile of one matrix in registers: its 8 KB of codes as 8 wave-wide
// 1 KB loads (lane l: bytes 16 l of each KB), the scale entry of the lane and
// this lane's chunks of the activation window.
template <int ROWS>
struct Tile {
    static constexpr int XR = core::XStageG<ROWS>::XR;
    uint4 wc[kCodeChunks];
    uint4 ws;
    uint4 xv[XR];
};

// Where a super-tile's loads read from.  A dummy (real == false) reads the
// packed header's zero bytes and no activations, so the number of loads in
// flight never depends on control flow and the compiler can count them
// exactly; its contents are never used, or used with zero scales.
struct TileSrc {
    const uint8_t *base;            // the super-tile, or the zero bytes
    __amdgpu_buffer_rsrc_t xr;      // the call's activations
    int kbase, k;
    bool real;                      // weights: the super-tile's, else the zero bytes
    bool xreal;                     // activations: the window's, else zeros
};

// This lane's chunks of the activation window: chunk c = lane + 64 i is row
// c / 32, k = kbase + 8 (c % 32) .. + 7.  Chunks past the activations read
// zeros (out-of-range buffer loads): always issued, never masked afterwards.
template <int ROWS>
__device__ __forceinline__ void load_x(const TileSrc &t, int lane, uint4 (&xv)[Tile<ROWS>::XR]) {
#pragma unroll
    for (int i = 0; i < Tile<ROWS>::XR; ++i) {
        const int c = lane + 64 * i;
        const int r = c >> 5, kk = (c & 31) * 8;
        const bool in = t.xreal && r < ROWS && t.kbase + kk < t.k;
        const int off = in ? (r * t.k + t.kbase + kk) * 2 : kDroppedOffset;
        const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(t.xr, off, 0, kSC1);
        xv[i] = make_uint4(v.x, v.y, v.z, v.w);
    }
}

// Weight loads of a tile through a buffer resource (up to CUT rows), else
// as global loads with per-lane addresses.  Same bytes either way; measured
// on the decode step: the buffer form 3.5% faster at 1 row and 2.3% at 4,
// 1.9% slower at 8 (its tile loop schedules worse there).
constexpr bool kBufferTileLoads(int rows) { return rows <= kBufferLoadRowsCut; }

template <int ROWS, bool WITH_X>
__device__ __forceinline__ void load_tile(const TileSrc &t, const uint8_t *zero, int lane, Tile<ROWS> &b) {
    // the activation window first: it is consumed first (staged into LDS)
    // and, issued first, it can be waited for while the codes are in flight
    if (WITH_X) {
        load_x<ROWS>(t, lane, b.xv);
        __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (!kBufferTileLoads(ROWS)) {
#pragma unroll
        for (int l = 0; l < kCodeChunks; ++l)
            b.wc[l] = load_nt(t.real ? t.base + l * kCodeChunkBytes + lane * 16 : zero);
        b.ws = load_nt(t.real ? t.base + kScaleOffset + lane * 16 : zero);
        __builtin_amdgcn_sched_barrier(0);
        return;
    }
    // The weights through a buffer resource over the super-tile (its base is
    // wave-uniform: scalar registers): the lane's offset is one register for
    // every chunk, the chunk's a constant, so no address arithmetic per load.
    // A dummy gets an empty resource: its loads read zeros without touching
    // memory.
    const uint8_t *base = t.real ? t.base : zero;
    const uint64_t bu = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(uintptr_t)base)) |
                        ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)((uintptr_t)base >> 32)) << 32);
    const __amdgpu_buffer_rsrc_t wr = rsrc(reinterpret_cast<const void *>(bu), t.real ? (uint32_t)kSuperBytes : 0u);
    const int vo = lane * 16;
#pragma unroll
    for (int l = 0; l < kCodeChunks; ++l) {
        const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(wr, vo + (l & 3) * kCodeChunkBytes,
                                                                (l >> 2) * 4 * kCodeChunkBytes, kNT);
        b.wc[l] = make_uint4(v.x, v.y, v.z, v.w);
    }
    {
        const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(wr, vo, kScaleOffset, kNT);
        b.ws = make_uint4(v.x, v.y, v.z, v.w);
    }
    // keep the whole tile's loads ahead of what follows (the scheduler would
    // otherwise sink them into the previous tile's arithmetic, after its wait)
    __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ TileSrc pick(bool first, const TileSrc &a, const TileSrc &b) {
    TileSrc t;
    t.base = first ? a.base : b.base;
    t.xr = first ? a.xr : b.xr;
    t.kbase = first ? a.kbase : b.kbase;
    t.k = first ? a.k : b.k;
    t.real = first ? a.real : b.real;
    t.xreal = first ? a.xreal : b.xreal;
    return t;
}

// Buffer resource over a call's outputs: stores at an offset past its size
// are dropped by the hardware, which masks the lanes past the last feature
// and the kernel rows past the call's without a branch.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t output_rsrc(const CallDesc &d) {
    return rsrc(d.y, (uint32_t)(d.rows * d.n * ((d.flags & kOutF32) ? 4 : 2)));
}

// Buffer resource over a call's activations: loads past them (the kernel
// rows past the call's, k past the last) read zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t x_rsrc(const CallDesc &d) {
    return rsrc(d.x, (uint32_t)(d.rows * d.k * 2));
}

// Apply the tensor scales and the SiLU product (pair) to the strip sums g, u
// of row r and store the row's outputs of strip s.
template <int ROWS>
__device__ __forceinline__ void epilogue(const CallDesc &d, __amdgpu_buffer_rsrc_t yr, float g, float u,
                                         const float (&sg)[2], int s, int r, int lane) {
    const int f = s * kStripN + lane;
    const float gs = g * sg[0];
    const float out = (d.flags & kPair) ? gs / (1.0f + expf(-gs)) * (u * sg[1]) : gs;
    const int at = r * d.n + f;
    if (d.flags & kOutF32)
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, out), yr,
                                              f < d.n ? at * 4 : kDroppedOffset, 0, kSC1);
    else
        __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16_rne(out), yr, f < d.n ? at * 2 : kDroppedOffset, 0,
                                              kSC1);
}

// The work of workgroup g in one call as one sequence of super-tiles, in
// segments: first its F owned strips, then its shared range [su0, su1) of the
// R*T shared units, cut at strip boundaries (nsh segments).  Every quantity
// here derives from kernel arguments and the workgroup index only, so the
// compiler keeps it, and every branch on it, on the scalar unit.
struct Geometry {
    int su0, su1, fs, nsh, nseg, total;
    // A shared range never exceeds one strip's T super-tiles, so it touches at
    // most two shared strips: fs, whose pieces may start in an earlier
    // workgroup (this one is piece `piece0` of `np0`), and fs + 1, which
    // starts here (piece 0 of `np1`).
    int piece0, np0, np1;
};

// Owner of shared unit v, in 32-bit arithmetic: v < U = R*T < 2^24 (R < 256,
// T <= 2^16) and G <= 256, so (v + 1) * G < 2^32.
__device__ __forceinline__ int owner_wg32(uint32_t v, uint32_t U, uint32_t G) {
    return (int)(((v + 1u) * G - 1u) / U);
}

__device__ __forceinline__ Geometry make_geometry(const CallDesc &d, int g) {
    Geometry q;
    q.su0 = q.su1 = q.fs = q.nsh = q.nseg = q.total = 0;
    q.piece0 = q.np0 = q.np1 = 1;
    if (g >= d.G) return q;   // not taking part in this call
    // g * U and (g + 1) * U stay below 256 * 2^24 = 2^32.  The shared units
    // are spread over the call's last G workgroups here (G <= the call's),
    // s = 0 .. G - 1 in order: a call of fewer strips than workgroups runs on
    // the first ones, so the last are the least loaded in a run of calls.
    const uint32_t U = (uint32_t)d.R * (uint32_t)d.T, T = (uint32_t)d.T;
    const uint32_t G = (uint32_t)((d.flags >> kShareShift) & 0xff) + 1u;
    const int s = g - (d.G - (int)G);
    if (s >= 0) {
        q.su0 = (int)((uint32_t)s * U / G);
        q.su1 = (int)((uint32_t)(s + 1) * U / G);
    }
    q.fs = q.su1 > q.su0 ? (int)((uint32_t)q.su0 / T) : 0;
    q.nsh = q.su1 > q.su0 ? (int)((uint32_t)(q.su1 - 1) / T) - q.fs + 1 : 0;
    q.nseg = d.F + q.nsh;
    q.total = d.F * d.T + (q.su1 - q.su0);
    if (q.nsh > 0) {
        const int first = owner_wg32((uint32_t)q.fs * T, U, G);
        q.piece0 = s - first;
        q.np0 = owner_wg32((uint32_t)(q.fs + 1) * T - 1u, U, G) - first + 1;
        // strip fs + 1 (used only when this range reaches it, i.e. fs + 1 < R)
        q.np1 = owner_wg32(min((uint32_t)(q.fs + 2) * T - 1u, U - 1u), U, G) - s + 1;
    }
    return q;
}

// Segment k of the sequence: positions [start, end), strip, first super-tile.
struct Cursor {
    int k, start, end, strip, u0;
};

// Shared-strip index of segment k, or -1 for an owned strip.
__device__ __forceinline__ int segment_shared(const CallDesc &d, const Geometry &q, int k) {
    return k >= d.F ? q.fs + (k - d.F) : -1;
}

__device__ __forceinline__ Cursor cursor_at(const CallDesc &d, const Geometry &q, int g, int k) {
    const int sh = segment_shared(d, q, k);
    const int v0 = max(q.su0, sh * d.T), v1 = min(q.su1, (sh + 1) * d.T);
    const int shared_base = d.F * d.T;
    Cursor c;
    c.k = k;
    const bool live = k < q.nseg, shared = sh >= 0;
    c.start = !live ? 0x7fffffff : shared ? shared_base + v0 - q.su0 : k * d.T;
    c.end = !live ? 0x7fffffff : shared ? shared_base + v1 - q.su0 : (k + 1) * d.T;
    c.strip = shared ? d.G * d.F + sh : g * d.F + k;
    c.u0 = shared ? v0 - sh * d.T : 0;
    return c;
}

// Segment ends without a workgroup barrier (barrier_free_segments(ROWS)).
// Buffer b (of red_buffers(ROWS))
// of the wave-reduction slots serves segments b, b + red_buffers(ROWS), ...
// of the workgroup's sequence, counted across calls; arr[b] counts the waves
// other than wave 0 that have stored their slots for its segment, done[b] is
// the last segment whose slots wave 0 has read from it.  The LDS executes
// each wave's instructions in order, so a count that wave 0 reads comes after
// the slots it counts, and a done that a wave reads after the reads it
// reports; the signal fences keep the compiler from moving LDS accesses
// across these words.
struct SegSync {
    unsigned arr[2];
    int done[2];
};

// Wave-uniform spin until *w >= v, bounded: past kMaxPolls polls the wait
// flag is set and the wave goes on (it never hangs).
__device__ __forceinline__ void lds_wait_ge(const int *w, int v, const LaunchShared &a, int lane) {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    unsigned polls = 0;
    while (__builtin_amdgcn_readfirstlane(__hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) < v &&
           polls < kMaxPolls) {
        __builtin_amdgcn_s_sleep(1);
        ++polls;
    }
    if (polls >= kMaxPolls && a.flags && lane == 0)
        __hip_atomic_store(a.flags, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Close segment k (the workgroup's segment number seg, counted across calls):
// every wave stores its accumulators' sums in its slot; the slots are summed
// in wave order; then wave 0 either writes the strip's outputs, or stores
// this piece of a shared strip in the partials and marks it in pub[] (strip
// fs or fs + 1).  Arrivals are counted, and the last piece's workgroup sums
// the pieces, once the call's tiles are done.  Every wave calls this for
// every segment, in order, and leaves with its accumulators cleared and seg
// advanced.  Without barriers (barrier_free_segments) a wave stores its slot
// and goes on, and waits only where it would overwrite slots that wave 0 has
// not read yet (a segment that used the same buffer); wave 0 waits for the
// other waves' slots and sums them alone.  With barriers, the waves store
// their slots, sum some rows each, and wave 0 reads the sums.
//
// This runs inside the tile loop, so its loops over values are fully
// unrolled with wave-uniform guards: a divergent branch there makes the
// compiler assume that tile loads may still be in flight at the top of the
// tile loop, and wait for them.
template <int ROWS>
using Acc = float[2][4][core::XStageG<ROWS>::RS][core::XStageG<ROWS>::NV];

template <int ROWS>
__device__ __forceinline__ void finish_segment(const LaunchShared &a, const CallDesc &d, const Geometry &q, int g,
                                               int k, float *red0, const float (&sg)[2],
                                               __amdgpu_buffer_rsrc_t yr, int wave, int sw, int nwc, int lane,
                                               Acc<ROWS> &acc, int (&pub)[2], int &seg, SegSync &ss) {
    using XS = core::XStageG<ROWS>;
    const bool pair = d.flags & kPair;
    constexpr int RR = red_rows(ROWS);   // rows per slot of `red`
    constexpr int NBUF = red_buffers(ROWS);
    constexpr bool kBarrierFree = barrier_free_segments(ROWS);
    const int nwb = blockDim.x >> 6;
    const int b = seg % NBUF;
    float *red = red0 + (size_t)b * nwb * 2 * RR * kStripN;
    if constexpr (kBarrierFree) {
        // the slots of buffer b are free once wave 0 has read them for segment seg - NBUF
        if (wave != 0) lds_wait_ge(&ss.done[b], seg - NBUF, a, lane);
    } else if constexpr (NBUF == 1) {
        __syncthreads();   // the previous segment's reads of `red` are done
    }
    // Slots in position order (sw): the sums below run in that order.  A
    // pair's accumulators are its gate and up sums; a single projection's
    // are two halves of its sum (even and odd tiles of the wave).  Lane
    // 16 q + n holds group half q & 1 of rows 8 rs + 2 v + (q >> 1) of feature
    // 16 fb + n: the two halves are added across lanes 16 apart, and both
    // lanes store the same sum (every D row of the slot is written, the rows
    // past ROWS being sums of zeros).
    const int n = lane & 15, rp = lane >> 5;
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int fb = 0; fb < 4; ++fb)
#pragma unroll
            for (int rs = 0; rs < XS::RS; ++rs)
#pragma unroll
                for (int v = 0; v < XS::NV; ++v) {
                    float t = m == 0 ? (pair ? acc[0][fb][rs][v] : acc[0][fb][rs][v] + acc[1][fb][rs][v])
                                     : acc[1][fb][rs][v];
                    t += __shfl_xor(t, 16);
                    if (m == 0 || pair)
                        red[((sw * 2 + m) * RR + 8 * rs + 2 * v + rp) * kStripN + 16 * fb + n] = t;
                }
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int fb = 0; fb < 4; ++fb)
#pragma unroll
            for (int rs = 0; rs < XS::RS; ++rs)
#pragma unroll
                for (int v = 0; v < XS::NV; ++v) acc[m][fb][rs][v] = 0.0f;
    const int this_seg = seg++;
    if constexpr (kBarrierFree) {
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        if (wave != 0) {
            if (lane == 0) __hip_atomic_fetch_add(&ss.arr[b], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            return;
        }
        lds_wait_ge(reinterpret_cast<const int *>(&ss.arr[b]), nwb - 1, a, lane);
        if (lane == 0) __hip_atomic_store(&ss.arr[b], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    } else {
        __syncthreads();
        // From 6 rows on the rows are spread over the waves (row r by wave r
        // mod the waves), each sum stored over slot 0's entry, and wave 0
        // reads the sums after one more barrier: summing every row's slots
        // alone made the other waves wait for it at the next segment (16% of
        // a long 8-row call).  Same order, same sums.
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int r = 0; r < ROWS; ++r)
                if ((m == 0 || pair) && r % nwb == wave) {
                    float t = red[(m * RR + r) * kStripN + lane];
#pragma unroll
                    for (int w = 1; w < kMaxWavesPerWg; ++w)
                        if (w < nwc) t += red[((w * 2 + m) * RR + r) * kStripN + lane];
                    red[(m * RR + r) * kStripN + lane] = t;
                }
        __syncthreads();
        if (wave != 0) return;
    }
    // The slots of a row are summed in position order.
    float v[2][ROWS];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int r = 0; r < ROWS; ++r) {
            float t = 0.0f;
            if (m == 0 || pair) {
                t = red[(m * RR + r) * kStripN + lane];
                if constexpr (kBarrierFree) {
#pragma unroll
                    for (int w = 1; w < kMaxWavesPerWg; ++w)
                        if (w < nwc) t += red[((w * 2 + m) * RR + r) * kStripN + lane];
                }
            }
            v[m][r] = t;
        }
    if constexpr (kBarrierFree) {
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        if (lane == 0) __hip_atomic_store(&ss.done[b], this_seg, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    const int sh = segment_shared(d, q, k);
    const bool head = sh == q.fs;
    const int np = head ? q.np0 : q.np1;
    if (sh >= 0 && np > 1) {
        const int nmat = pair ? 2 : 1;
        const size_t slot = ((size_t)sh * d.max_pieces + (head ? q.piece0 : 0)) * nmat;
#pragma unroll
        for (int m = 0; m < 2; ++m)
            if (m == 0 || pair)
#pragma unroll
                for (int r = 0; r < ROWS; ++r)
                    __hip_atomic_store(&a.partial[((slot + m) * ROWS + r) * kStripN + lane], v[m][r],
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        pub[head ? 0 : 1] = 1;   // its arrival is counted after the call's tiles
        return;
    }
    const int strip = sh >= 0 ? d.G * d.F + sh : g * d.F + k;
#pragma unroll
    for (int r = 0; r < ROWS; ++r) epilogue<ROWS>(d, yr, v[0][r], v[1][r], sg, strip, r, lane);
}

// Pieces of a shared strip are summed in piece order, gate and up (NM = 2) or
// the projection alone (NM = 1), 32 values per lane in flight per round trip
// to memory (16 at one row: measured 1% faster on the decode step there, 1%
// slower at two rows; loads past the last piece read the last one again,
// which measured faster than skipping them behind branches).  Pieces per
// round trip for one wave holding every row:
template <int ROWS, int NM>
__host__ __device__ constexpr int final_sum_qb() {
    return ROWS == 1 ? 16 / NM : (32 / NM) / ROWS > 0 ? (32 / NM) / ROWS : 1;
}

// Wave 0: sum the pieces of shared strip sh for every row at once, QB pieces
// per round, and write its outputs.
template <int ROWS, int NM>
__device__ __forceinline__ void final_sum(const LaunchShared &a, const CallDesc &d, int sh, int np,
                                          const float (&sg)[2], __amdgpu_buffer_rsrc_t yr, int lane) {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    constexpr int QB = final_sum_qb<ROWS, NM>();
    float tq[ROWS][NM];
#pragma unroll
    for (int r = 0; r < ROWS; ++r)
#pragma unroll
        for (int m = 0; m < NM; ++m) tq[r][m] = 0.0f;
    for (int q0 = 0; q0 < np; q0 += QB) {
        float pv[ROWS][NM][QB];
#pragma unroll
        for (int j = 0; j < QB; ++j) {
            const size_t qs = ((size_t)sh * d.max_pieces + min(q0 + j, np - 1)) * NM;
#pragma unroll
            for (int m = 0; m < NM; ++m)
#pragma unroll
                for (int r = 0; r < ROWS; ++r)
                    pv[r][m][j] = __hip_atomic_load(&a.partial[((qs + m) * ROWS + r) * kStripN + lane],
                                                    __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
#pragma unroll
        for (int j = 0; j < QB; ++j)
            if (q0 + j < np)
#pragma unroll
                for (int r = 0; r < ROWS; ++r)
#pragma unroll
                    for (int m = 0; m < NM; ++m) tq[r][m] += pv[r][m][j];
    }
#pragma unroll
    for (int r = 0; r < ROWS; ++r)
        epilogue<ROWS>(d, yr, tq[r][0], tq[r][NM - 1], sg, d.G * d.F + sh, r, lane);
}

// The same sums spread over the workgroup's waves: wave w takes rows w,
// w + nwb, ..., each in rounds of 32 / NM pieces, into fs[m][r][lane] (LDS)
// for wave 0 to write.  The order of every sum is the one above.
template <int ROWS, int NM>
__device__ __forceinline__ void sum_pieces(const LaunchShared &a, const CallDesc &d, int sh, int np, int wave, int nwb,
                                           int lane, float *fs) {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    constexpr int QB = 32 / NM;
    for (int r = wave; r < ROWS; r += nwb) {
        float t[NM];
#pragma unroll
        for (int m = 0; m < NM; ++m) t[m] = 0.0f;
        for (int q0 = 0; q0 < np; q0 += QB) {
            float pv[NM][QB];
#pragma unroll
            for (int j = 0; j < QB; ++j) {
                const size_t qs = ((size_t)sh * d.max_pieces + min(q0 + j, np - 1)) * NM;
#pragma unroll
                for (int m = 0; m < NM; ++m)
                    pv[m][j] = __hip_atomic_load(&a.partial[((qs + m) * ROWS + r) * kStripN + lane],
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
#pragma unroll
            for (int j = 0; j < QB; ++j)
                if (q0 + j < np)
#pragma unroll
                    for (int m = 0; m < NM; ++m) t[m] += pv[m][j];
        }
#pragma unroll
        for (int m = 0; m < NM; ++m) fs[(m * ROWS + r) * kStripN + lane] = t[m];
    }
}

// Wait until every load and store of this wave issued so far has completed.
__device__ __forceinline__ void wait_all_loads() {
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0); expcnt and lgkmcnt not waited for
}

// Wave 0: wait until every earlier write of this wave has completed.  All of
// them are device-coherent, so completion makes them visible to every CU.
__device__ __forceinline__ void wait_own_writes() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Counter accesses of wave 0, made by its lane 0 alone (device-scope
// atomics), with the result broadcast to the wave.  They sit outside the tile
// loop, where the divergent branch costs nothing.
__device__ __forceinline__ unsigned lane0_add(unsigned *p, int lane) {
    unsigned old = 0;
    if (lane == 0) old = __hip_atomic_fetch_add(p, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return (unsigned)__builtin_amdgcn_readfirstlane((int)old);
}

__device__ __forceinline__ unsigned lane0_load(unsigned *p, int lane) {
    unsigned v = 0;
    if (lane == 0) v = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return (unsigned)__builtin_amdgcn_readfirstlane((int)v);
}

__device__ __forceinline__ void lane0_store(unsigned *p, unsigned v, int lane) {
    if (lane == 0) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wave 0: count this workgroup's pieces of shared strips fs and fs + 1
// (pub[h] set: a piece of strip fs + h was stored), lanes 0 and 1 at once, so
// that two pieces cost one round trip to memory.  Bit h of the result is set
// where this workgroup's count completes strip fs + h: it clears the counter
// and sums the strip.
__device__ __forceinline__ unsigned arrive_pieces(const LaunchShared &a, const Geometry &q, const int (&pub)[2],
                                                  int lane) {
    const bool mine = (lane == 0 && pub[0]) || (lane == 1 && pub[1]);
    unsigned *cnt = a.counters + (q.fs + (lane & 1)) * 32;
    const unsigned np = (unsigned)(lane == 1 ? q.np1 : q.np0);
    unsigned old = 0;
    if (mine) old = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = mine && old == np - 1u;
    if (last) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return (unsigned)__ballot(last) & 3u;
}

// Wave 0: the wait between calls (epoch e = calls finished so far).  Each
// workgroup counts itself in one arrival counter once its writes of the call
// are complete; the workgroup whose count completes epoch e stores e in every
// workgroup's release word, each in a 128-byte line of its own that only its
// workgroup polls, and goes on without waiting (returns true).  A wait of
// more than kMaxPolls polls sets the wait flag and goes on: it never hangs.
__device__ __forceinline__ bool arrive_call(const LaunchShared &a, int g, unsigned e, int lane) {
    wait_own_writes();
    const bool last = lane0_add(a.flags + 32, lane) + 1u == e * (unsigned)a.G;
    if (last) {
#pragma unroll
        for (int i = 0; i < kMaxWorkgroups / 64; ++i) {
            const int w = lane + 64 * i;
            if (w < a.G) __hip_atomic_store(a.sync + w * 32, e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    return last;
}

// One poll at a time.  Measured against it on the decode-step sweep: four
// polls in flight (a new one every ~0.2 us) was 2-5% slower (256 workgroups
// polling that often slow the weight stream), and polling before wave 0's
// fetch of the next call's first items (a poll's result waits for every load
// issued before it) 0.4-2.6% slower.
__device__ __forceinline__ void wait_release(const LaunchShared &a, int g, unsigned e, int lane) {
    unsigned polls = 0;
    while (lane0_load(a.sync + g * 32, lane) < e && polls < kMaxPolls) {
        __builtin_amdgcn_s_sleep(1);
        ++polls;
    }
    if (polls >= kMaxPolls) lane0_store(a.flags, 1u, lane);
}

// Residual add + RMSNorm of one row, by every wave of workgroup `row`: v =
// bf16(residual + delta) is stored as residual_out, then x = bf16(v * inv *
// w') with inv = 1 / sqrt(mean(v^2) + eps) and w' = w or 1 + w, fp32
// arithmetic.  The sum of squares takes the order of the stand-alone norm
// kernel (its thread t of 256 sums chunks of 8 values t, t + 256, ... in
// order; a butterfly per wave of 64; the 4 waves' sums in order): waves 0-3
// here are its waves (with fewer waves, each takes several in turn), so the
// two give the same bits.  Chunks go 4 per thread at a time, all loads in
// flight together; up to 8192 values the whole row is one such block and
// (in kernels of up to 8 rows) v stays in registers, otherwise the second
// pass reads v back from residual_out (the thread's own writes, after
// waiting for them), which is also correct when residual_out is the residual
// itself.  Every wave waits for its writes
// before the workgroup goes on: wave 0 then counts the call done.
__device__ __forceinline__ float bf_lo(uint32_t u) { return __builtin_bit_cast(float, u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __builtin_bit_cast(float, u & 0xffff0000u); }

// KEEP: the row may stay in registers (kernels of up to 8 rows; beside the
// 12- and 16-row kernels' registers it would spill).
template <bool KEEP>
__device__ __forceinline__ void norm_row(const CallDesc &d, int row, int wave, int nwb, int lane, float *s_ss) {
    const int k = d.n;
    const uint32_t rb = (uint32_t)k * 2;
    const size_t row0 = (size_t)row * k;
    const __amdgpu_buffer_rsrc_t rr = rsrc(d.x + row0, rb);
    const __amdgpu_buffer_rsrc_t hr = rsrc(reinterpret_cast<const uint16_t *>(d.w0) + row0, rb);
    const __amdgpu_buffer_rsrc_t wr = rsrc(d.w1, rb);
    const __amdgpu_buffer_rsrc_t orr = rsrc(static_cast<uint16_t *>(d.aux) + row0, rb);
    const __amdgpu_buffer_rsrc_t xr = rsrc(static_cast<uint16_t *>(d.y) + row0, rb);
    constexpr int kBlock = 4 * 256 * 8;   // values per block: 4 chunks of 8 per thread
    const bool keep = KEEP && k <= kBlock && nwb >= 4;   // v of the one block stays in registers
    const bool gemma = d.flags & kGemma;
    u32x4_t vk[4], wk[4];
    for (int vw = wave; vw < 4; vw += nwb) {
        const int t = 64 * vw + lane;
        float ss = 0.0f;
        for (int c0 = 0; c0 < k; c0 += kBlock) {   // past the row: loads read 0, stores are dropped
            u32x4_t rv[4], hv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int off = c0 * 2 + (t + 256 * i) * 16;
                rv[i] = __builtin_amdgcn_raw_buffer_load_b128(rr, off, 0, kSC1);
                hv[i] = __builtin_amdgcn_raw_buffer_load_b128(hr, off, 0, kSC1);
                if (keep) wk[i] = __builtin_amdgcn_raw_buffer_load_b128(wr, off, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int off = c0 * 2 + (t + 256 * i) * 16;
                u32x4_t v;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t lo = f32_to_bf16_rne(bf_lo(rv[i][e]) + bf_lo(hv[i][e]));
                    const uint32_t hi = f32_to_bf16_rne(bf_hi(rv[i][e]) + bf_hi(hv[i][e]));
                    v[e] = lo | (hi << 16);
                    const float fl = bf_lo(v[e]), fh = bf_hi(v[e]);
                    ss = __builtin_fmaf(fl, fl, ss);
                    ss = __builtin_fmaf(fh, fh, ss);
                }
                __builtin_amdgcn_raw_buffer_store_b128(v, orr, off, 0, kSC1);
                vk[i] = v;
            }
        }
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m);
        if (lane == 0) s_ss[vw] = ss;
    }
    __syncthreads();
    const float tot = ((s_ss[0] + s_ss[1]) + s_ss[2]) + s_ss[3];
    const float inv = 1.0f / __builtin_sqrtf(tot / (float)k + d.eps);
    if (!keep) wait_own_writes();
    for (int vw = wave; vw < 4; vw += nwb) {
        const int t = 64 * vw + lane;
        for (int c0 = 0; c0 < k; c0 += kBlock) {
            u32x4_t v[4], wv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int off = c0 * 2 + (t + 256 * i) * 16;
                v[i] = keep ? vk[i] : __builtin_amdgcn_raw_buffer_load_b128(orr, off, 0, kSC1);
                wv[i] = keep ? wk[i] : __builtin_amdgcn_raw_buffer_load_b128(wr, off, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int off = c0 * 2 + (t + 256 * i) * 16;
                u32x4_t xv;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float wl = bf_lo(wv[i][e]), wh = bf_hi(wv[i][e]);
                    if (gemma) {
                        wl += 1.0f;
                        wh += 1.0f;
                    }
                    xv[e] = (uint32_t)f32_to_bf16_rne(bf_lo(v[i][e]) * inv * wl) |
                            ((uint32_t)f32_to_bf16_rne(bf_hi(v[i][e]) * inv * wh) << 16);
                }
                __builtin_amdgcn_raw_buffer_store_b128(xv, xr, off, 0, kSC1);
            }
        }
    }
    wait_own_writes();
    __syncthreads();
}

// SEQ: several calls per launch (the cross-call pipeline and the completion
// counts); without it the launch runs call 0 alone.
template <int ROWS, bool SEQ>
__global__ __launch_bounds__(max_waves_for_rows(ROWS) * 64) void seq_kernel(KernelArgs<SEQ ? kSeqMax : 1> args) {
    LaunchShared a = args.s;   // partial and counters: the running call's region
    extern __shared__ __align__(16) unsigned char smem[];
    const int tid = threadIdx.x, lane = tid & 63;
    // the wave index is uniform across the wave; saying so keeps every loop and
    // branch below on the scalar unit (no exec-masked control flow around loads)
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nwb = blockDim.x >> 6;
    const int g = blockIdx.x;
    // Position order of the waves: wave 0 comes last, so it gets the fewest
    // super-tiles -- it also reduces and writes every result.
    const int sw = wave == 0 ? nwb - 1 : wave - 1;
    using XS = core::XStageG<ROWS>;
    static_assert(XS::BYTES == x_stage_bytes(ROWS), "host LDS sizing assumes this staging size");
    static_assert(XS::XR == Tile<ROWS>::XR, "one activation chunk layout");
    uint8_t *xs = smem + (size_t)wave * XS::BYTES;   // this wave's staged activations
    float *red = reinterpret_cast<float *>(smem + (size_t)nwb * XS::BYTES);
    if (lane < 4) reinterpret_cast<uint32_t *>(xs + XS::ZERO_OFF)[lane] = 0u;   // the staging's zero bytes
    // one staging and one product per super-tile
    auto stage = [&](const Tile<ROWS> &t) { core::stage_g<ROWS>(t.xv, xs, lane); };
    auto product = [&](const Tile<ROWS> &t, float (&ac)[4][XS::RS][XS::NV]) {
        core::core_g<ROWS>(t.wc, t.ws, xs, lane, ac);
    };

    Acc<ROWS> acc;
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int fb = 0; fb < 4; ++fb)
#pragma unroll
            for (int rs = 0; rs < XS::RS; ++rs)
#pragma unroll
                for (int v = 0; v < XS::NV; ++v) acc[m][fb][rs][v] = 0.0f;
    // The call table, copied into LDS once: reading a call's descriptor from
    // the kernel arguments at the start of every call costs a cache miss each
    // time; from LDS it is a few cycles.  The words are wave-uniform.
    __shared__ CallDesc s_calls[SEQ ? kSeqMax : 1];
    __shared__ unsigned s_fin;   // shared strips this workgroup completes (bits 0, 1)
    __shared__ float s_ss[4];    // a norm call's sums of squares, by wave of the stand-alone kernel
    __shared__ SegSync s_seg;    // segment ends (finish_segment)
    int seg = 0;                 // segments this workgroup has closed
    if (tid < 2) {
        s_seg.arr[tid] = 0u;
        s_seg.done[tid] = tid - red_buffers(ROWS);
    }
    // This workgroup's geometry of every call of the launch, computed once
    // here (one call per thread) rather than by every wave a call ahead: its
    // divisions are no small part of a short call (measured: computing it
    // twice per call made the 1-row decode step 5% longer).
    __shared__ Geometry s_geo[SEQ ? kSeqMax : 1];
    constexpr int kDescWords = sizeof(CallDesc) / 4;
    constexpr int kGeoWords = sizeof(Geometry) / 4;
    static_assert(sizeof(Geometry) % 4 == 0, "geometries are read as words");
    if (SEQ) {
        const uint32_t *src = reinterpret_cast<const uint32_t *>(args.call);
        uint32_t *dst = reinterpret_cast<uint32_t *>(s_calls);
        for (int i = tid; i < a.ncalls * kDescWords; i += blockDim.x) dst[i] = src[i];
        __syncthreads();
        for (int c = tid; c < a.ncalls; c += blockDim.x) {
            const CallDesc &dc = s_calls[c];
            s_geo[c] = make_geometry(dc, !(dc.flags & kNorm) ? g : kMaxWorkgroups);
        }
    }
    __syncthreads();
    auto desc = [&](int c) {
        if (!SEQ) return args.call[0];
        CallDesc v;
        const uint32_t *p = reinterpret_cast<const uint32_t *>(&s_calls[c]);
        uint32_t *o = reinterpret_cast<uint32_t *>(&v);
#pragma unroll
        for (int i = 0; i < kDescWords; ++i) o[i] = (uint32_t)__builtin_amdgcn_readfirstlane((int)p[i]);
        return v;
    };

    // Everything a wave needs to start call k: its descriptor and geometry,
    // the wave's number of positions, and the sources of its first NB items
    // (the wave's stream of super-tiles in a call, item t: of a single
    // projection, position sw + t * waves, with its activation window; of a
    // pair, position sw + (t / 2) * waves, gate (t even, with the window) or
    // up (t odd); items past the wave's last are dummies).  Prepared one call
    // ahead, before the wait between calls, so none of it is on the path from
    // one call's end to the next one's first tile.
    constexpr int NB = pipe_depth_for_rows(ROWS);
    static_assert(NB % 2 == 0, "a pair's gate and up super-tiles share a buffer pair");
    struct Prep {
        CallDesc d;
        Geometry q;
        int nw;          // this wave's positions
        bool fetch;      // its first NB items are fetched during the call before
        float sg[2];     // tensor scales (wave 0 only)
    };
    const int ncalls = SEQ ? a.ncalls : 1;
    auto prepare = [&](int k) {
        Prep p;
        const bool live = k < ncalls;
        p.d = desc(live ? k : ncalls - 1);
        const CallDesc &d = p.d;
        if (SEQ && live) {
            const uint32_t *gp = reinterpret_cast<const uint32_t *>(&s_geo[k]);
            uint32_t *go = reinterpret_cast<uint32_t *>(&p.q);
#pragma unroll
            for (int i = 0; i < kGeoWords; ++i) go[i] = (uint32_t)__builtin_amdgcn_readfirstlane((int)gp[i]);
        } else {
            p.q = make_geometry(d, live && !(d.flags & kNorm) ? g : kMaxWorkgroups);
        }
        const Geometry &q = p.q;
        p.nw = sw < d.waves && sw < q.total ? (q.total - sw + d.waves - 1) / d.waves : 0;
        p.fetch = p.nw > 0;
        // Tensor scales from the packed headers, for wave 0, which writes every
        // result.  Scalar loads, issued a call ahead: a value loaded into a
        // vector register and used in a loop that stores makes the compiler
        // wait for every load in flight before entering that loop (which the
        // segment-closing loops are), and the scalar counter is only waited on
        // by the next LDS access, long after these have landed.
        p.sg[0] = p.sg[1] = 0.0f;
        if (wave == 0) {
            typedef const __attribute__((address_space(4))) float *const_float_ptr;
            p.sg[0] = *(const_float_ptr)(uintptr_t)d.w0;
            p.sg[1] = *(const_float_ptr)(uintptr_t)d.w1;
        }
        return p;
    };
    // Item t of prepared call p, for a first fetch (t < NB); `cu` is a cursor
    // over p's segments that only moves forward, so t must not decrease
    // between uses of one cursor.  `mine` false makes it a dummy.
    auto first_item = [&](const Prep &p, Cursor &cu, int t, bool mine) {
        const CallDesc &d = p.d;
        const bool pair = d.flags & kPair;
        const bool real = mine && p.fetch && t < (pair ? 2 * p.nw : p.nw), up = pair && (t & 1);
        const int i = sw + (pair ? t >> 1 : t) * d.waves;
        if (real)
            while (i >= cu.end) cu = cursor_at(d, p.q, g, cu.k + 1);
        TileSrc s;
        const int u = cu.u0 + (i - cu.start);
        s.base = (up ? d.w1 : d.w0) + kHeaderBytes + ((size_t)cu.strip * d.T + u) * kSuperBytes;
        s.xr = x_rsrc(d);
        s.kbase = u * kSuperK;
        s.k = d.k;
        s.real = real;
        s.xreal = real && !up;
        return s;
    };

    // b[] holds the first NB items of the call about to start: call 0's are
    // fetched here, every later call's during the call before it (items of a
    // wave with no positions are dummies, never used)
    Tile<ROWS> b[NB];
    Prep cur = prepare(0);
    Prep nxt = prepare(1);
    {
        Cursor c0 = cursor_at(cur.d, cur.q, g, 0);
#pragma unroll
        for (int i = 0; i < NB; ++i)
            load_tile<ROWS, true>(first_item(cur, c0, i, true), zero_of(cur.d), lane, b[i]);
    }
    unsigned waits = 0;   // waits between calls passed so far
    for (int c = 0; c < ncalls; ++c) {
        const CallDesc d = cur.d;
        const Geometry q = cur.q;
        const int nw = cur.nw;
        const bool has_next = SEQ && c + 1 < ncalls;
        // the next call waits for this one (and every other before it)
        const bool wait_next = has_next && (nxt.d.flags & kWaitBefore);
        if (SEQ) {
            const int reg = (d.flags >> kRegionShift) & (kRegions - 1);
            a.partial = args.s.partial + (size_t)reg * args.s.pstride;
            a.counters = reg ? args.s.counters_tail + (reg - 1) * (int)(kCounterBytes / 4) : args.s.counters;
        }
        const bool pair = d.flags & kPair;
        const int nwc = d.waves;
        const uint8_t *zero = zero_of(d);
        const __amdgpu_buffer_rsrc_t xr = x_rsrc(d);
        const __amdgpu_buffer_rsrc_t yr = output_rsrc(d);
        const float sg[2] = {cur.sg[0], cur.sg[1]};
        // The next call's first NB items, fetched while this call ends.  Wave
        // 0 fetches its own only once it has counted this call done: it writes
        // every result, and waits for its writes to complete first.  Up to 4
        // rows every wave waits until then (kLateFetch): the end of a call is a
        // chain of dependent round trips to memory (partial sums, counts, the
        // final sums, outputs, the wait), each slowed by any burst of loads in
        // flight.  Measured on the decode step with barrier-free segment ends:
        // 3.6% faster at 1 row, 1% at 4; at 6-8 rows (more arithmetic per
        // byte, segment barriers) 4-6% slower.
        constexpr bool kLateFetch = ROWS <= 4;
        // A workgroup normalizing a row (a norm call) fetches the next call's
        // first items only after it: its loads would return behind them.
        const bool norm_here = (d.flags & kNorm) && g < d.rows;
        const bool nreal = !kLateFetch && nxt.fetch && wave != 0 && !norm_here;
        const Cursor nc0 = cursor_at(nxt.d, nxt.q, g, 0);

        int pub[2] = {0, 0};   // pieces of shared strips fs, fs + 1 stored here
        bool released = false;   // this workgroup completed the call's epoch (wave 0)
        Cursor lc = cursor_at(d, q, g, 0), cc = lc;   // load cursor (runs ahead), segment being accumulated
        auto item = [&](int t) {
            const bool up = pair && (t & 1);
            const int pos = sw + (pair ? t >> 1 : t) * nwc;
            const bool real = (pair ? t >> 1 : t) < nw;
            if (real)
                while (pos >= lc.end) lc = cursor_at(d, q, g, lc.k + 1);
            TileSrc s;
            const int u = lc.u0 + (pos - lc.start);
            s.base = real ? (up ? d.w1 : d.w0) + kHeaderBytes + ((size_t)lc.strip * d.T + u) * kSuperBytes : zero;
            s.xr = xr;
            s.kbase = u * kSuperK;
            s.k = d.k;
            s.real = real;
            s.xreal = real && !up;
            return s;
        };
        // close every segment that ends before position i
        auto close_before = [&](int i) {
            while (i >= cc.end) {
                finish_segment<ROWS>(a, d, q, g, cc.k, red, sg, yr, wave, sw, nwc, lane, acc, pub, seg, s_seg);
                cc = cursor_at(d, q, g, cc.k + 1);
            }
        };
        if (nw > 0 && (d.flags & kReloadX)) {
#pragma unroll
            for (int i = 0; i < NB; ++i)
                if (!pair || !(i & 1)) load_x<ROWS>(item(i), lane, b[i].xv);
        }
        // Items NB j + i (buffer i) per iteration, all NB in flight at the top;
        // each buffer is refilled with the item NB ahead as soon as it has been
        // consumed, and past the call's last items with the next call's first
        // NB.  A wave with no positions that fetches for the next call runs one
        // iteration that only fetches, so that the buffers are written in one
        // place only -- a second place costs registers at the merge.  The loop
        // has one exit, and no wait at its head other than for the data it
        // consumes.
        const int nitems = pair ? 2 * nw : nw;
        const int iters = nw > 0 ? (nitems + NB - 1) / NB : nreal ? 1 : 0;
        // Every load issued before the loop has completed here (the first
        // items arrived during the wait between calls; reloaded activation
        // windows are cache hits).  Saying so costs little and lets the
        // compiler count the loop's own loads exactly: otherwise its wait at
        // the loop head merges the state of the way in, where the first items'
        // loads are the most recent, and it waits for nearly every load in
        // flight at the top of every iteration.
        if (iters > 0) wait_all_loads();
        for (int j = 0; j < iters; ++j) {
            const int t = NB * j;
            const bool more = j + 1 < iters;   // another iteration follows
            Cursor nc = nc0;   // over the next call's first items
#pragma unroll
            for (int i = 0; i < NB; ++i) {
                const int ti = t + i;
                // Items past the wave's last are fetched (the loads in flight
                // must not depend on control flow) but not computed; a pair's
                // up super-tile uses the window its gate staged.
                const bool live = ti < nitems;
                if (live && (!pair || !(i & 1))) stage(b[i]);
                // past the last item this closes every segment left
                close_before(sw + (pair ? ti >> 1 : ti) * nwc);
                if (live) product(b[i], acc[i & 1]);
                const TileSrc next_call = first_item(nxt, nc, i, !kLateFetch && wave != 0);
                load_tile<ROWS, true>(pick(more, item(ti + NB), next_call), zero, lane, b[i]);
            }
        }
        while (cc.k < q.nseg) {
            finish_segment<ROWS>(a, d, q, g, cc.k, red, sg, yr, wave, sw, nwc, lane, acc, pub, seg, s_seg);
            cc = cursor_at(d, q, g, cc.k + 1);
        }
        if (norm_here) norm_row<(ROWS <= 8)>(d, g, wave, nwb, lane, s_ss);
        // Pieces of shared strips: wave 0 counts them; where this workgroup's
        // count completes a strip, it is summed either by wave 0 alone or by
        // every wave, some rows each, into LDS (`red`, free once wave 0 has
        // read its last segment's sums), and wave 0 writes the outputs.
        // Whether a piece was published follows from the geometry, so every
        // wave takes the same branch.
        const bool pieces = (q.nsh > 0 && q.np0 > 1) || (q.nsh > 1 && q.np1 > 1);
        // Wave 0 alone needs a round trip per QB pieces; the other waves have
        // the next call's first super-tiles in flight (from 3 rows on), and
        // their loads wait behind those: they help only where wave 0 alone
        // would need more than 4 rounds (measured: 2 rounds alone beat help).
        const int qb0 = pair ? final_sum_qb<ROWS, 2>() : final_sum_qb<ROWS, 1>();
        const int np_max = max(q.nsh > 0 ? q.np0 : 1, q.nsh > 1 ? q.np1 : 1);
        const bool spread = !kLateFetch && nwb > 1 && np_max > 4 * qb0;
        if (pieces && !spread) {
            if (wave == 0) {
                wait_own_writes();   // the partials are visible before they are counted
                const unsigned fin = arrive_pieces(a, q, pub, lane);
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int np = h ? q.np1 : q.np0;
                    if (fin & (1u << h)) {
                        if (pair) final_sum<ROWS, 2>(a, d, q.fs + h, np, sg, yr, lane);
                        else final_sum<ROWS, 1>(a, d, q.fs + h, np, sg, yr, lane);
                    }
                }
            }
        } else if (pieces) {
            if (wave == 0) {
                wait_own_writes();   // the partials are visible before they are counted
                const unsigned fin = arrive_pieces(a, q, pub, lane);
                if (lane == 0) s_fin = fin;
            }
            __syncthreads();
            const unsigned fin = (unsigned)__builtin_amdgcn_readfirstlane((int)s_fin);
            if (fin) {
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    if (fin & (1u << h)) {
                        float *fs = red + 2 * h * ROWS * kStripN;
                        if (pair) sum_pieces<ROWS, 2>(a, d, q.fs + h, h ? q.np1 : q.np0, wave, nwb, lane, fs);
                        else sum_pieces<ROWS, 1>(a, d, q.fs + h, h ? q.np1 : q.np0, wave, nwb, lane, fs);
                    }
                __syncthreads();
                if (wave == 0) {
#pragma unroll
                    for (int h = 0; h < 2; ++h)
                        if (fin & (1u << h))
#pragma unroll
                            for (int r = 0; r < ROWS; ++r)
                                epilogue<ROWS>(d, yr, red[((2 * h) * ROWS + r) * kStripN + lane],
                                               red[((2 * h + 1) * ROWS + r) * kStripN + lane], sg,
                                               d.G * d.F + q.fs + h, r, lane);
                }
                // the next segment's slots overwrite these sums
                __syncthreads();
            }
        }
        if (wait_next) ++waits;
        if (wave == 0 && wait_next) released = arrive_call(a, g, waits, lane);
        // Without a wait before the next call no barrier ends this one either:
        // the other waves start the next call while wave 0 still completes
        // this one's shared strips, and wave 0 catches up at the next
        // segment's end (with barriers there, they meet it).
        if (has_next) {
            if (kLateFetch && wait_next) __syncthreads();   // wave 0 has counted the call done
            if ((kLateFetch || wave == 0 || norm_here) && nxt.fetch) {
                // wave 0's writes are complete: its loads in flight delay only its polls
                Cursor nc = nc0;
#pragma unroll
                for (int i = 0; i < NB; ++i) load_tile<ROWS, true>(first_item(nxt, nc, i, true), zero, lane, b[i]);
            }
            // the call after next, prepared while the workgroups finish this one
            cur = nxt;
            nxt = prepare(c + 2);
            if (wave == 0 && wait_next && !released) wait_release(a, g, waits, lane);
            if (wait_next) __syncthreads();   // the next call starts in every wave
        }
    }
    if (SEQ && wave == 0) {
        // Back to zero for the next launch: this workgroup's release word (no
        // release is stored after the last wait), and, by the last workgroup
        // out, the arrival and exit counts.
        wait_own_writes();
        lane0_store(a.sync + g * 32, 0u, lane);
        if (lane0_add(a.flags + 64, lane) == (unsigned)(a.G - 1)) {
            lane0_store(a.flags + 32, 0u, lane);
            lane0_store(a.flags + 64, 0u, lane);
        }
    }
}

template <int ROWS, bool SEQ>
hipError_t launch_kernel(const LaunchShared &sh, const CallDesc *calls, int waves, size_t lds, hipStream_t stream) {
    const void *fn = reinterpret_cast<const void *>(&seq_kernel<ROWS, SEQ>);
    // dynamic LDS beyond the default limit needs the attribute, set once per
    // instantiation: what the CU's 160 KB leave beside the kernel's static LDS
    // (the call table of a sequence kernel)
    static std::atomic<int> lds_set{0};
    if (lds_set.load(std::memory_order_acquire) == 0) {
        hipFuncAttributes attr{};
        hipError_t e = hipFuncGetAttributes(&attr, fn);
        if (e != hipSuccess) return e;
        e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                (int)(160 * 1024 - attr.sharedSizeBytes));
        if (e != hipSuccess) return e;
        lds_set.store(1, std::memory_order_release);
    }
    KernelArgs<SEQ ? kSeqMax : 1> a;   // the table past ncalls is never read
    a.s = sh;
    for (int i = 0; i < (SEQ ? sh.ncalls : 1); ++i) a.call[i] = calls[i];
    void *kargs[] = {&a};
    const dim3 grid((unsigned)a.s.G), block((unsigned)(64 * waves));
    // workgroups that wait for each other must all be resident: a cooperative launch
    if (SEQ) return hipLaunchCooperativeKernel(fn, grid, block, kargs, (unsigned)lds, stream);
    return hipLaunchKernel(fn, grid, block, kargs, lds, stream);
}

template <int ROWS>
hipError_t launch_rows(const LaunchShared &a, const CallDesc *c, int waves, size_t lds, hipStream_t s) {
    return a.ncalls > 1 ? launch_kernel<ROWS, true>(a, c, waves, lds, s) : launch_kernel<ROWS, false>(a, c, waves, lds, s);
}

hipError_t launch_args(int krows, const LaunchShared &a, const CallDesc *c, int waves, size_t lds, hipStream_t s) {
    switch (krows) {
        case 1: return launch_rows<1>(a, c, waves, lds, s);
        case 2: return launch_rows<2>(a, c, waves, lds, s);
        case 4: return launch_rows<4>(a, c, waves, lds, s);
        case 6: return launch_rows<6>(a, c, waves, lds, s);
        case 8: return launch_rows<8>(a, c, waves, lds, s);
        case 12: return launch_rows<12>(a, c, waves, lds, s);
        case 16: return launch_rows<16>(a, c, waves, lds, s);
        default: return hipErrorInvalidValue;
    }
}

bool ranges_overlap(const void *a, size_t na, const void *b, size_t nb) {
    const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
    return pa < pb + nb && pb < pa + na;
}

}  // namespace

// Whether this device runs launches whose workgroups wait for each other.
bool cooperative_ok() {
    static std::atomic<int> state{-1};
    int s = state.load(std::memory_order_acquire);
    if (s < 0) {
        int dev = 0, coop = 0, cus = 0;
        s = hipGetDevice(&dev) == hipSuccess &&
                    hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev) == hipSuccess &&
                    hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
                    coop != 0 && cus >= kMaxWorkgroups
                ? 1
                : 0;
        state.store(s, std::memory_order_release);
    }
    return s == 1;
}

StreamPlan make_norm_plan(int64_t k, int rows) {
    StreamPlan pl{};
    pl.n = k;
    pl.k = k;
    pl.rows = rows;
    // the kernel of the row chunks a projection of as many rows runs as, so
    // that the norm shares their launch
    const int chunks = (rows + kKernelMaxRows - 1) / kKernelMaxRows;
    pl.krows = kernel_rows((rows + chunks - 1) / chunks);
    pl.nmat = 1;
    pl.strips = 0;
    pl.supers = 1;
    pl.G = rows;      // workgroup r normalizes row r
    pl.Gs = rows;
    pl.F = 0;
    pl.R = 0;
    pl.waves = 0;     // no tiles
    pl.max_pieces = 1;
    pl.partial_bytes = 0;
    pl.lds_bytes = stream_lds_bytes(pl.krows, 1);
    return pl;
}

StreamPlan make_stream_plan(int64_t n, int64_t k, int rows, int dual) {
    StreamPlan pl{};
    pl.n = n;
    pl.k = k;
    pl.rows = rows;
    pl.krows = kernel_rows(rows);
    pl.nmat = dual ? 2 : 1;
    const int S = (int)num_strips(n), T = (int)num_supers(k);
    pl.strips = S;
    pl.supers = T;
    const long long units = (long long)S * T;
    if ((S >= kOwnerMinStrips || T <= 4) && S <= kMaxWorkgroups) {
        pl.G = S;                      // one owned strip per workgroup (also for short k)
        pl.F = 1;
    } else if (S > kMaxWorkgroups) {
        pl.G = kMaxWorkgroups;         // whole strips plus balanced pieces of the rest
        pl.F = S / kMaxWorkgroups;
    } else {
        // skinny: balanced pieces only, as many workgroups as keeps them equal
        const long long per = (units + kMaxWorkgroups - 1) / kMaxWorkgroups;
        pl.G = (int)((units + per - 1) / per);
        pl.F = 0;
    }
    pl.R = S - pl.G * pl.F;
    // Waves per workgroup: each keeps pipe_depth_for_rows(rows) super-tiles
    // (9 KB each) in flight, so this sets the bytes in flight per CU -- enough
    // to cover the memory latency at full bandwidth.
    int waves = max_waves_for_rows(rows);
    // Strips left over past whole strips per workgroup are spread over the
    // last Gs workgroups, so that each is cut into at most kLeftoverPieces
    // pieces (every piece adds a partial sum, and the strip's completion waits
    // for the last of them), and every one of those workgroups gets at least
    // one unit (one without units would be counted as a piece that never
    // arrives).
    pl.Gs = pl.G;
    if (pl.F > 0 && pl.R > 0) {
        const long long gs = std::min<long long>((long long)pl.R * kLeftoverPieces, (long long)pl.R * T);
        if (gs < pl.G) pl.Gs = (int)gs;
    }
    const long long per_wg = pl.F * (long long)T + (pl.R ? ((long long)pl.R * T + pl.Gs - 1) / pl.Gs : 0);
    // When the others can take everything in their first fetch, wave 0 takes
    // no position: in a sequence each wave's first items arrive ahead of the
    // call, except wave 0's (it writes the results and cannot have loads in
    // flight while it waits for them), so a position of its own would be the
    // last to arrive.
    const int ahead = pipe_depth_for_rows(rows) / pl.nmat;   // positions of a wave's first fetch
    if (per_wg <= (long long)ahead * (waves - 1)) waves -= 1;
    if (waves > per_wg) waves = (int)per_wg;
    if (waves < 1) waves = 1;
    pl.waves = waves;
    pl.max_pieces = 1;
    if (pl.R > 0) {
        const long long U = (long long)pl.R * T;
        for (int sh = 0; sh < pl.R; ++sh) {
            const int np = owner_wg((long long)sh * T + T - 1, U, pl.Gs) - owner_wg((long long)sh * T, U, pl.Gs) + 1;
            if (np > pl.max_pieces) pl.max_pieces = np;
        }
    }
    if (pl.max_pieces > 1)
        pl.partial_bytes = (size_t)pl.R * pl.max_pieces * pl.nmat * pl.krows * kStripN * sizeof(float);
    pl.lds_bytes = stream_lds_bytes(pl.krows, pl.waves);
    return pl;
}

size_t stream_lds_bytes(int krows, int waves) {
    const size_t lds_x = (size_t)waves * x_stage_bytes(krows);
    // the wave-reduction slots; they also hold the final sums of up to two
    // shared strips (4 x rows x 64 floats), hence at least two waves' worth
    const size_t lds_red = (size_t)red_buffers(krows) * (waves < 2 ? 2 : waves) * 2 * red_rows(krows) * kStripN *
                           sizeof(float);
    // at least ~81 KB so that no CU ever holds two of these workgroups
    return lds_x + lds_red < kOneWorkgroupPerCuLds ? kOneWorkgroupPerCuLds : lds_x + lds_red;
}

size_t sequence_workspace_bytes(const StreamCall *calls, int ncalls) {
    size_t partial = 0;
    for (int i = 0; i < ncalls; ++i)
        if (calls[i].plan.partial_bytes > partial) partial = calls[i].plan.partial_bytes;
    // several calls in one launch keep their waits in the sync region and
    // may run in up to kRegions regions at once
    if (ncalls > 1) return sequence_workspace(partial);
    if (partial > 0) return kPartialOffset + partial;
    return 0;
}

namespace {
// End of the launch that starts at call i0: a run of calls with the same row
// count, cut into launches of at most kSeqMax calls, as equal as possible.
int launch_end(const StreamCall *calls, int ncalls, int i0, bool shared) {
    if (!shared) return i0 + 1;
    int run = i0 + 1;
    while (run < ncalls && calls[run].plan.krows == calls[i0].plan.krows) ++run;
    const int left = run - i0, parts = (left + kSeqMax - 1) / kSeqMax;
    return i0 + (left + parts - 1) / parts;
}
}  // namespace

int sequence_launches(const StreamCall *calls, int ncalls) {
    const bool shared = ncalls > 1 && cooperative_ok();
    int n = 0;
    for (int i0 = 0; i0 < ncalls; i0 = launch_end(calls, ncalls, i0, shared)) ++n;
    return n;
}

// One launch of a sequence, complete but for the workspace pointers.
struct LaunchRec {
    int krows, waves;
    size_t lds;
    size_t partial_bytes;     // a region's partial sums (the list's largest)
    LaunchShared s;           // workspace pointers set at launch
    CallDesc call[kSeqMax];   // the first s.ncalls are the launch's calls
};

size_t launch_rec_bytes() { return sizeof(LaunchRec); }

namespace {
// The bytes a call reads (weights, activations; a norm call: delta, norm
// weight, residual) and writes (outputs; a norm call: x and residual_out).
struct Span {
    const void *p;
    size_t n;
};
int reads_of(const StreamCall &c, Span (&s)[3]) {
    const size_t xb = (size_t)c.plan.rows * c.plan.k * 2;
    if (c.norm) {
        s[0] = {c.w0, xb};
        s[1] = {c.w1, (size_t)c.plan.k * 2};
    } else {
        s[0] = {c.w0, nvfp4_packed_bytes(c.plan.n, c.plan.k)};
        s[1] = {c.w1, c.w1 ? nvfp4_packed_bytes(c.plan.n, c.plan.k) : 0};
    }
    s[2] = {c.x, xb};
    return 3;
}
int writes_of(const StreamCall &c, Span (&s)[2]) {
    s[0] = {c.y, (size_t)c.plan.rows * c.plan.n * (c.out_f32 ? 4 : 2)};
    s[1] = {c.aux, c.norm ? (size_t)c.plan.rows * c.plan.k * 2 : 0};
    return 2;
}
bool spans_overlap(const Span *a, int na, const Span *b, int nb) {
    for (int i = 0; i < na; ++i)
        for (int j = 0; j < nb; ++j)
            if (a[i].n && b[j].n && ranges_overlap(a[i].p, a[i].n, b[j].p, b[j].n)) return true;
    return false;
}
// Call i must wait for call j (earlier in the launch): it reads what j
// writes, or writes what j reads or writes.
bool depends(const StreamCall &j, const StreamCall &i) {
    Span rj[3], wj[2], ri[3], wi[2];
    reads_of(j, rj);
    writes_of(j, wj);
    reads_of(i, ri);
    writes_of(i, wi);
    return spans_overlap(wj, 2, ri, 3) || spans_overlap(rj, 3, wi, 2) || spans_overlap(wj, 2, wi, 2);
}

// The wait, region and reload flags of the calls [i0, i1) of one launch.
void mark_runs(const StreamCall *calls, int i0, int i1, int *flags) {
    int run = i0, prev_run = i0;   // first call of the current run and of the run before
    for (int i = i0; i < i1; ++i) {
        const StreamCall &sc = calls[i];
        int f = 0;
        if (i > i0) {
            bool wait = i - run >= kRegions;
            for (int j = run; j < i && !wait; ++j) wait = depends(calls[j], sc);
            if (wait) {
                prev_run = run;
                run = i;
                f |= kWaitBefore;
                const Span xs[1] = {{sc.x, (size_t)sc.plan.rows * sc.plan.k * 2}};
                for (int j = prev_run; j < i; ++j) {
                    Span wj[2];
                    writes_of(calls[j], wj);
                    if (spans_overlap(wj, 2, xs, 1)) f |= kReloadX;
                }
            }
        }
        flags[i - i0] = f | ((i - run) << kRegionShift);
    }
}
}  // namespace

int sequence_waits(const StreamCall *calls, int ncalls) {
    std::vector<int> flags((size_t)ncalls);
    int waits = 0;
    for (int i0 = 0; i0 < ncalls;) {
        const int i1 = launch_end(calls, ncalls, i0, ncalls > 1);
        mark_runs(calls, i0, i1, flags.data());
        for (int i = 0; i < i1 - i0; ++i) waits += (flags[i] & kWaitBefore) ? 1 : 0;
        i0 = i1;
    }
    return waits;
}

// Calls of a launch run as runs of mutually independent calls: a call waits
// (kWaitBefore) for every earlier call when it depends on a call of the
// current run, or when the run already holds kRegions calls; the calls of a
// run take workspace regions 0, 1, ... in order.  A call that waits has its
// first tiles fetched during the run before, so it fetches their activations
// again when a call of that run writes them (kReloadX).
int build_launches(const StreamCall *calls, int ncalls, void *recs) {
    LaunchRec *out = static_cast<LaunchRec *>(recs);
    const bool shared = ncalls > 1 && cooperative_ok();
    size_t partial = 0;   // the largest partial sums of the list: a region's size
    for (int i = 0; i < ncalls; ++i)
        if (calls[i].plan.partial_bytes > partial) partial = calls[i].plan.partial_bytes;
    int nrec = 0;
    for (int i0 = 0; i0 < ncalls; ++nrec) {
        const int i1 = launch_end(calls, ncalls, i0, shared);
        LaunchRec &r = out[nrec];
        r.s = LaunchShared{};
        r.s.pstride = (int)(round_partial(partial) / sizeof(float));
        r.partial_bytes = partial;
        const int krows = calls[i0].plan.krows;
        r.s.ncalls = i1 - i0;
        int G = 1, waves = 1;
        int marks[kSeqMax];
        mark_runs(calls, i0, i1, marks);
        for (int i = i0; i < i1; ++i) {
            const StreamCall &sc = calls[i];
            const StreamPlan &pl = sc.plan;
            CallDesc &d = r.call[i - i0];
            d = CallDesc{};
            d.w0 = static_cast<const uint8_t *>(sc.w0);
            d.w1 = static_cast<const uint8_t *>(sc.w1 ? sc.w1 : sc.w0);
            d.x = static_cast<const uint16_t *>(sc.x);
            d.y = sc.y;
            d.n = (int)pl.n;
            d.k = (int)pl.k;
            d.T = pl.supers;
            d.G = pl.G;
            d.F = pl.F;
            d.R = pl.R;
            d.max_pieces = pl.max_pieces;
            d.waves = pl.waves;
            d.flags = (pl.nmat == 2 ? kPair : 0) | (sc.out_f32 ? kOutF32 : 0) | ((pl.Gs - 1) << kShareShift);
            d.rows = pl.rows;
            d.aux = nullptr;
            if (sc.norm) {
                d.flags = kNorm | (sc.norm == 2 ? kGemma : 0);
                d.aux = const_cast<void *>(sc.aux);
                d.eps = sc.eps;
            }
            d.flags |= marks[i - i0];
            if (pl.G > G) G = pl.G;
            if (pl.waves > waves) waves = pl.waves;
        }
        r.s.G = G;
        r.krows = krows;
        r.waves = waves;
        r.lds = stream_lds_bytes(krows, waves);
        i0 = i1;
    }
    return nrec;
}

hipError_t launch_recs(const void *recs, int nrec, void *workspace, hipStream_t stream) {
    const LaunchRec *in = static_cast<const LaunchRec *>(recs);
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    for (int i = 0; i < nrec; ++i) {
        LaunchShared a = in[i].s;
        a.counters = reinterpret_cast<unsigned *>(ws);
        a.sync = ws ? reinterpret_cast<unsigned *>(ws + kSyncOffset) : nullptr;
        a.flags = ws ? reinterpret_cast<unsigned *>(ws + kFlagOffset) : nullptr;
        a.partial = ws ? reinterpret_cast<float *>(ws + kPartialOffset) : nullptr;
        a.counters_tail = ws ? reinterpret_cast<unsigned *>(ws + kCounterTailOffset) : nullptr;
        hipError_t e = launch_args(in[i].krows, a, in[i].call, in[i].waves, in[i].lds, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_sequence(const StreamCall *calls, int ncalls, void *workspace, hipStream_t stream) {
    std::vector<LaunchRec> recs((size_t)sequence_launches(calls, ncalls));
    const int nrec = build_launches(calls, ncalls, recs.data());
    return launch_recs(recs.data(), nrec, workspace, stream);
}

}  // namespace nvfp4
