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
//     no cross-workgroup traffic); the remaining units of work are cut into
//     balanced pieces of strips ("stream-K");
//   * pieces of a strip are summed in piece order by the last to arrive (an
//     arrival counter), so results are bitwise deterministic with no float
//     atomics, and identical whether a call runs alone or in a sequence;
//   * calls run in order: a call starts computing only after every workgroup
//     has finished the previous one (a completion count per launch), so a call
//     may read an earlier call's output as its activations.
// Everything one workgroup writes to global memory -- outputs, partial sums,
// counters -- is written by its wave 0 with device-coherent (sc1) accesses, and
// wave 0 is the only wave with no loads in flight across a call boundary, so it
// can wait for its own writes to complete before it counts the call done
// without waiting for the other waves' next weight loads.  Activations are read
// with device-coherent loads as well.  No cache-wide flushes.
//
// Work units of a call: strip s in [0, S) x super-tile u in [0, T).  G
// workgroups; the first G*F strips are owned, F per workgroup; the R = S - G*F
// remaining strips form R*T shared units split into G contiguous ranges
// [g*RT/G, (g+1)*RT/G), cut at strip boundaries into pieces.
#include <atomic>
#include <type_traits>

#include "nvfp4_core.h"

namespace nvfp4 {
namespace {
using namespace core;

// One call of a launch.
struct CallDesc {
    const uint8_t *w0;    // packed weight (gate of the pair)
    const uint8_t *w1;    // packed up weight of a pair; w0 otherwise
    const uint16_t *x;    // [rows][k] bf16
    void *y;              // [rows][n]
    int n, k, T;
    int G, F, R;          // workgroups taking part, owned strips each, shared strips
    int max_pieces;
    int waves;            // waves taking part
    int flags;            // kPair | kOutF32 | kReloadX
    int pad;
};
constexpr int kPair = 1, kOutF32 = 2;
// x is written by the call before this one in the same launch: the activations
// of a super-tile fetched before the call started are fetched again.
constexpr int kReloadX = 4;
constexpr int kSeqMax = 40;   // calls per launch (the kernel arguments stay below 4 KB)

struct SeqArgs {
    CallDesc call[kSeqMax];
    float *partial;       // [R][max_pieces][nmat][rows][64] of the call running
    unsigned *counters;   // arrival count of shared strip sh at word 32 sh (one 128-byte line each)
    unsigned *sync;       // word 32 g: the last call workgroup g may go past (one 128-byte line each)
    unsigned *flags;      // word 0: a wait between calls timed out; 32: arrivals; 64: workgroups exited
    int ncalls;
    int G;                // workgroups of the launch
};
static_assert(sizeof(SeqArgs) <= 3072, "kernel arguments must stay small");
static_assert(sizeof(CallDesc) % 4 == 0, "call descriptors are copied as words");

constexpr int kSC1 = 16;                          // cache policy: device-coherent access
constexpr int kDroppedOffset = 0x7fffffff;        // past any buffer: loads read 0, stores are dropped
constexpr int kRsrcWord3 = 0x00020000;            // raw buffer, 32-bit data format
constexpr uint64_t kWaitTicks = 20000000;         // 0.2 s of the 100 MHz real-time clock

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
    static constexpr int XR = core::XStage<ROWS>::XR;
    uint4 wc[kCodeChunks / 2];
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

template <int ROWS, bool WITH_X>
__device__ __forceinline__ void load_tile(const TileSrc &t, const uint8_t *zero, int lane, Tile<ROWS> &b) {
    // the activation window first: it is consumed first (staged into LDS)
    // and, issued first, it can be waited for while the codes are in flight
    if (WITH_X) {
        load_x<ROWS>(t, lane, b.xv);
        __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int l = 0; l < kCodeChunks / 2; ++l)
        b.wc[l] = load_nt(t.real ? t.base + l * 2 * kCodeChunkBytes + lane * 16 : zero);
    b.ws = load_nt(t.real ? t.base + kScaleOffset + lane * 16 : zero);
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
// without a branch.
template <int ROWS>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t output_rsrc(const CallDesc &d) {
    return rsrc(d.y, (uint32_t)(ROWS * d.n * ((d.flags & kOutF32) ? 4 : 2)));
}

template <int ROWS>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t x_rsrc(const CallDesc &d) {
    return rsrc(d.x, (uint32_t)(ROWS * d.k * 2));
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
    // g * U and (g + 1) * U stay below 256 * 2^24 = 2^32
    const uint32_t U = (uint32_t)d.R * (uint32_t)d.T, G = (uint32_t)d.G, T = (uint32_t)d.T;
    q.su0 = (int)((uint32_t)g * U / G);
    q.su1 = (int)((uint32_t)(g + 1) * U / G);
    q.fs = q.su1 > q.su0 ? (int)((uint32_t)q.su0 / T) : 0;
    q.nsh = q.su1 > q.su0 ? (int)((uint32_t)(q.su1 - 1) / T) - q.fs + 1 : 0;
    q.nseg = d.F + q.nsh;
    q.total = d.F * d.T + (q.su1 - q.su0);
    if (q.nsh > 0) {
        const int first = owner_wg32((uint32_t)q.fs * T, U, G);
        q.piece0 = g - first;
        q.np0 = owner_wg32((uint32_t)(q.fs + 1) * T - 1u, U, G) - first + 1;
        // strip fs + 1 (used only when this range reaches it, i.e. fs + 1 < R)
        q.np1 = owner_wg32(min((uint32_t)(q.fs + 2) * T - 1u, U - 1u), U, G) - g + 1;
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

// Close segment k: reduce the waves' accumulators in wave order; then wave 0
// either writes the strip's outputs, or stores this piece of a shared strip
// in the partials and marks it in pub[] (strip fs or fs + 1).  Arrivals are
// counted, and the last piece's workgroup sums the pieces, once the call's
// tiles are done.  Every wave calls this for every segment, in order, and
// leaves with its accumulators cleared.
//
// This runs inside the tile loop, so its loops are fully unrolled with
// wave-uniform guards: a rolled loop or a divergent branch there makes the
// compiler assume that tile loads may still be in flight at the top of the
// tile loop, and wait for them.
template <int ROWS, int AR>
__device__ __forceinline__ void finish_segment(const SeqArgs &a, const CallDesc &d, const Geometry &q, int g,
                                               int k, float *red, const float (&sg)[2],
                                               __amdgpu_buffer_rsrc_t yr, int wave, int sw, int nwc, int lane,
                                               float (&acc)[2][4][AR], int (&pub)[2]) {
    const bool pair = d.flags & kPair;
    constexpr int RR = red_rows(ROWS);   // rows per slot of `red`
    __syncthreads();   // the previous segment's reads of `red` are done
    // slots in position order (sw): the sums below run in that order
    // a pair's accumulators are its gate and up sums; a single projection's
    // are two halves of its sum (even and odd tiles of the wave)
    if constexpr (use_f16_core(ROWS)) {
        // lane 16 q + n holds rows 4 q + v of features 16 fb + n, already
        // summed over k: each lane writes its own, rows past ROWS (exact
        // zeros) included, since the slots have 16 rows on this path
        float *base = red + (sw * 2 * RR + 4 * (lane >> 4)) * kStripN + (lane & 15);
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
            for (int fb = 0; fb < 4; ++fb) {
                base[v * kStripN + 16 * fb] = pair ? acc[0][fb][v] : acc[0][fb][v] + acc[1][fb][v];
                if (pair) base[(RR + v) * kStripN + 16 * fb] = acc[1][fb][v];
                acc[0][fb][v] = 0.0f;
                acc[1][fb][v] = 0.0f;
            }
    } else {
#pragma unroll
        for (int r = 0; r < ROWS; ++r) {
            float g4[4], u4[4];
#pragma unroll
            for (int fb = 0; fb < 4; ++fb) {
                g4[fb] = pair ? acc[0][fb][r] : acc[0][fb][r] + acc[1][fb][r];
                u4[fb] = acc[1][fb][r];
                acc[0][fb][r] = 0.0f;
                acc[1][fb][r] = 0.0f;
            }
            red[((sw * 2 + 0) * RR + r) * kStripN + lane] = core::strip_total(g4, lane);
            if (pair) red[((sw * 2 + 1) * RR + r) * kStripN + lane] = core::strip_total(u4, lane);
        }
    }
    __syncthreads();
    if (wave != 0) return;
    float v[2][ROWS];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int r = 0; r < ROWS; ++r) {
            float t = 0.0f;
            if (m == 0 || pair) {
                t = red[(m * RR + r) * kStripN + lane];
#pragma unroll
                for (int w = 1; w < kMaxWavesPerWg; ++w)
                    if (w < nwc) t += red[((w * 2 + m) * RR + r) * kStripN + lane];
            }
            v[m][r] = t;
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
__device__ __forceinline__ void final_sum(const SeqArgs &a, const CallDesc &d, int sh, int np,
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
__device__ __forceinline__ void sum_pieces(const SeqArgs &a, const CallDesc &d, int sh, int np, int wave, int nwb,
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

// Wave 0: count this workgroup's piece of shared strip sh; true for the
// workgroup whose count completes it, which clears the counter and sums the
// strip.
__device__ __forceinline__ bool arrive_piece(const SeqArgs &a, int sh, int np, int lane) {
    unsigned *cnt = a.counters + sh * 32;
    if (lane0_add(cnt, lane) != (unsigned)(np - 1)) return false;
    lane0_store(cnt, 0u, lane);
    return true;
}

// Wave 0: the wait between calls (epoch e = calls finished so far).  Each
// workgroup counts itself in one arrival counter once its writes of the call
// are complete; the workgroup whose count completes epoch e stores e in every
// workgroup's release word, each in a 128-byte line of its own that only its
// workgroup polls, and goes on without waiting (returns true).  A wait that
// exceeds kWaitTicks sets a flag and goes on: it never hangs.
__device__ __forceinline__ bool arrive_call(const SeqArgs &a, int g, unsigned e, int lane) {
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
__device__ __forceinline__ void wait_release(const SeqArgs &a, int g, unsigned e, int lane) {
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    bool late = false;
    while (lane0_load(a.sync + g * 32, lane) < e && !late) {
        __builtin_amdgcn_s_sleep(1);
        late = __builtin_amdgcn_s_memrealtime() - t0 > kWaitTicks;
    }
    if (late) lane0_store(a.flags, 1u, lane);
}

// SEQ: several calls per launch (the cross-call pipeline and the completion
// counts); without it the launch runs call 0 alone.
template <int ROWS, bool SEQ>
__global__ __launch_bounds__(max_waves_for_rows(ROWS) * 64) void seq_kernel(SeqArgs a) {
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
    constexpr bool kF16 = use_f16_core(ROWS), kOne = !kF16 && ROWS == 1;
    using XS = std::conditional_t<kF16, core::XStage16<ROWS>,
                                  std::conditional_t<kOne, core::XStage1, core::XStage<ROWS>>>;
    static_assert(XS::BYTES == x_stage_bytes(ROWS), "host LDS sizing assumes this staging size");
    static_assert(XS::XR == Tile<ROWS>::XR, "one activation chunk layout");
    uint8_t *xs = smem + (size_t)wave * XS::BYTES;   // this wave's staged activations
    float *red = reinterpret_cast<float *>(smem + (size_t)nwb * XS::BYTES);
    constexpr int kZeroWords = kF16 ? core::XStage16<ROWS>::ZERO_WORDS : 8;   // the staging's zero bytes
    if constexpr (kOne) core::init_x1(xs, lane);
    else if (lane < kZeroWords) reinterpret_cast<uint32_t *>(xs + XS::ZERO_OFF)[lane] = 0u;
    // one staging and one product per super-tile, on the path chosen for ROWS
    auto stage = [&](const Tile<ROWS> &t) {
        if constexpr (kF16) core::stage_x16<ROWS>(t.xv, xs, lane);
        else if constexpr (kOne) core::stage_x1(t.xv, xs, lane);
        else core::stage_x<ROWS>(t.xv, xs, lane);
    };
    // Accumulators: the fp16 path's lanes hold 4 rows each (their products'
    // rows), the other paths every row in every lane.
    constexpr int AR = kF16 ? 4 : ROWS;
    auto product = [&](const Tile<ROWS> &t, float (&ac)[4][AR]) {
        if constexpr (kF16) core::core_f16<ROWS>(t.wc, t.ws, xs, lane, ac);
        else if constexpr (kOne) core::core_mx1(t.wc, t.ws, xs, lane, ac);
        else core::core_mx<ROWS>(t.wc, t.ws, xs, lane, ac);
    };

    float acc[2][4][AR];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int fb = 0; fb < 4; ++fb)
#pragma unroll
            for (int r = 0; r < AR; ++r) acc[m][fb][r] = 0.0f;
    // The call table, copied into LDS once: reading a call's descriptor from
    // the kernel arguments at the start of every call costs a cache miss each
    // time; from LDS it is a few cycles.  The words are wave-uniform.
    __shared__ CallDesc s_calls[SEQ ? kSeqMax : 1];
    __shared__ unsigned s_fin;   // shared strips this workgroup completes (bits 0, 1)
    constexpr int kDescWords = sizeof(CallDesc) / 4;
    if (SEQ) {
        const uint32_t *src = reinterpret_cast<const uint32_t *>(a.call);
        uint32_t *dst = reinterpret_cast<uint32_t *>(s_calls);
        for (int i = tid; i < a.ncalls * kDescWords; i += blockDim.x) dst[i] = src[i];
        __syncthreads();
    }
    auto desc = [&](int c) {
        if (!SEQ) return a.call[0];
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
        p.q = make_geometry(d, live ? g : kMaxWorkgroups);
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
        s.xr = x_rsrc<ROWS>(d);
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
            load_tile<ROWS, true>(first_item(cur, c0, i, true), cur.d.w0 + kHeaderZeroOffset, lane, b[i]);
    }
    for (int c = 0; c < ncalls; ++c) {
        const CallDesc d = cur.d;
        const Geometry q = cur.q;
        const int nw = cur.nw;
        const bool has_next = SEQ && c + 1 < ncalls;
        const bool pair = d.flags & kPair;
        const int nwc = d.waves;
        const uint8_t *zero = d.w0 + kHeaderZeroOffset;
        const __amdgpu_buffer_rsrc_t xr = x_rsrc<ROWS>(d);
        const __amdgpu_buffer_rsrc_t yr = output_rsrc<ROWS>(d);
        const float sg[2] = {cur.sg[0], cur.sg[1]};
        // The next call's first NB items, fetched while this call ends.  Wave
        // 0 fetches its own only once it has counted this call done: it writes
        // every result, and waits for its writes to complete first.  At 1-2
        // rows every wave waits until then (kLateFetch): the end of a call is a
        // chain of dependent round trips to memory (partial sums, counts, the
        // final sums, outputs, the wait), each slowed by any burst of loads in
        // flight, and the calls are short enough that the chain, not the
        // stream, sets their length (measured 1-2% faster on a decode step; at
        // 4-8 rows, with more arithmetic per byte, 4-6% slower).
        constexpr bool kLateFetch = ROWS <= 2;
        const bool nreal = !kLateFetch && nxt.fetch && wave != 0;
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
                finish_segment<ROWS, AR>(a, d, q, g, cc.k, red, sg, yr, wave, sw, nwc, lane, acc, pub);
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
            finish_segment<ROWS, AR>(a, d, q, g, cc.k, red, sg, yr, wave, sw, nwc, lane, acc, pub);
            cc = cursor_at(d, q, g, cc.k + 1);
        }
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
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int np = h ? q.np1 : q.np0;
                    if (pub[h] && arrive_piece(a, q.fs + h, np, lane)) {
                        if (pair) final_sum<ROWS, 2>(a, d, q.fs + h, np, sg, yr, lane);
                        else final_sum<ROWS, 1>(a, d, q.fs + h, np, sg, yr, lane);
                    }
                }
            }
        } else if (pieces) {
            if (wave == 0) {
                wait_own_writes();   // the partials are visible before they are counted
                unsigned fin = 0;
                if (pub[0] && arrive_piece(a, q.fs, q.np0, lane)) fin |= 1u;
                if (pub[1] && arrive_piece(a, q.fs + 1, q.np1, lane)) fin |= 2u;
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
            }
        }
        if (wave == 0 && has_next) released = arrive_call(a, g, (unsigned)(c + 1), lane);
        if (has_next) {
            if (kLateFetch) __syncthreads();   // wave 0 has counted the call done
            if ((kLateFetch || wave == 0) && nxt.fetch) {
                // wave 0's writes are complete: its loads in flight delay only its polls
                Cursor nc = nc0;
#pragma unroll
                for (int i = 0; i < NB; ++i) load_tile<ROWS, true>(first_item(nxt, nc, i, true), zero, lane, b[i]);
            }
            // the call after next, prepared while the workgroups finish this one
            cur = nxt;
            nxt = prepare(c + 2);
            if (wave == 0 && !released) wait_release(a, g, (unsigned)(c + 1), lane);
            __syncthreads();   // the next call starts in every wave
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
hipError_t launch_kernel(const SeqArgs &args, int waves, size_t lds, hipStream_t stream) {
    const void *fn = reinterpret_cast<const void *>(&seq_kernel<ROWS, SEQ>);
    // dynamic LDS beyond the default limit needs the attribute, set once per instantiation
    static std::atomic<int> lds_set{0};
    if (lds_set.load(std::memory_order_acquire) == 0) {
        hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, 152 * 1024);
        if (e != hipSuccess) return e;
        lds_set.store(1, std::memory_order_release);
    }
    SeqArgs a = args;
    void *kargs[] = {&a};
    const dim3 grid((unsigned)a.G), block((unsigned)(64 * waves));
    // workgroups that wait for each other must all be resident: a cooperative launch
    if (SEQ) return hipLaunchCooperativeKernel(fn, grid, block, kargs, (unsigned)lds, stream);
    return hipLaunchKernel(fn, grid, block, kargs, lds, stream);
}

template <int ROWS>
hipError_t launch_rows(const SeqArgs &a, int waves, size_t lds, hipStream_t s) {
    return a.ncalls > 1 ? launch_kernel<ROWS, true>(a, waves, lds, s) : launch_kernel<ROWS, false>(a, waves, lds, s);
}

hipError_t launch_args(int rows, const SeqArgs &a, int waves, size_t lds, hipStream_t s) {
    switch (rows) {
        case 1: return launch_rows<1>(a, waves, lds, s);
        case 2: return launch_rows<2>(a, waves, lds, s);
        case 3: return launch_rows<3>(a, waves, lds, s);
        case 4: return launch_rows<4>(a, waves, lds, s);
        case 5: return launch_rows<5>(a, waves, lds, s);
        case 6: return launch_rows<6>(a, waves, lds, s);
        case 7: return launch_rows<7>(a, waves, lds, s);
        case 8: return launch_rows<8>(a, waves, lds, s);
        case 9: return launch_rows<9>(a, waves, lds, s);
        case 10: return launch_rows<10>(a, waves, lds, s);
        case 11: return launch_rows<11>(a, waves, lds, s);
        case 12: return launch_rows<12>(a, waves, lds, s);
        case 13: return launch_rows<13>(a, waves, lds, s);
        case 14: return launch_rows<14>(a, waves, lds, s);
        case 15: return launch_rows<15>(a, waves, lds, s);
        case 16: return launch_rows<16>(a, waves, lds, s);
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

StreamPlan make_stream_plan(int64_t n, int64_t k, int rows, int dual) {
    StreamPlan pl{};
    pl.n = n;
    pl.k = k;
    pl.rows = rows;
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
    const long long per_wg = pl.F * (long long)T + (pl.R ? ((long long)pl.R * T + pl.G - 1) / pl.G : 0);
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
            const int np = owner_wg((long long)sh * T + T - 1, U, pl.G) - owner_wg((long long)sh * T, U, pl.G) + 1;
            if (np > pl.max_pieces) pl.max_pieces = np;
        }
    }
    if (pl.max_pieces > 1) pl.partial_bytes = (size_t)pl.R * pl.max_pieces * pl.nmat * rows * kStripN * sizeof(float);
    pl.lds_bytes = stream_lds_bytes(rows, pl.waves);
    return pl;
}

size_t stream_lds_bytes(int rows, int waves) {
    const size_t lds_x = (size_t)waves * x_stage_bytes(rows);
    // the wave-reduction slots; they also hold the final sums of up to two
    // shared strips (4 x rows x 64 floats), hence at least two waves' worth
    const size_t lds_red = (size_t)(waves < 2 ? 2 : waves) * 2 * red_rows(rows) * kStripN * sizeof(float);
    // at least ~81 KB so that no CU ever holds two of these workgroups
    return lds_x + lds_red < kOneWorkgroupPerCuLds ? kOneWorkgroupPerCuLds : lds_x + lds_red;
}

size_t sequence_workspace_bytes(const StreamCall *calls, int ncalls) {
    size_t partial = 0;
    for (int i = 0; i < ncalls; ++i)
        if (calls[i].plan.partial_bytes > partial) partial = calls[i].plan.partial_bytes;
    // several calls in one launch keep their waits in the sync region
    if (ncalls > 1 || partial > 0) return kPartialOffset + partial;
    return 0;
}

namespace {
// End of the launch that starts at call i0: a run of calls with the same row
// count, cut into launches of at most kSeqMax calls, as equal as possible.
int launch_end(const StreamCall *calls, int ncalls, int i0, bool shared) {
    if (!shared) return i0 + 1;
    int run = i0 + 1;
    while (run < ncalls && calls[run].plan.rows == calls[i0].plan.rows) ++run;
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

hipError_t launch_sequence(const StreamCall *calls, int ncalls, void *workspace, hipStream_t stream) {
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    const bool shared = ncalls > 1 && cooperative_ok();
    for (int i0 = 0; i0 < ncalls;) {
        const int i1 = launch_end(calls, ncalls, i0, shared);
        const int rows = calls[i0].plan.rows;
        SeqArgs a{};
        a.ncalls = i1 - i0;
        a.counters = reinterpret_cast<unsigned *>(ws);
        a.sync = ws ? reinterpret_cast<unsigned *>(ws + kSyncOffset) : nullptr;
        a.flags = ws ? reinterpret_cast<unsigned *>(ws + kFlagOffset) : nullptr;
        a.partial = ws ? reinterpret_cast<float *>(ws + kPartialOffset) : nullptr;
        int G = 1, waves = 1;
        for (int i = i0; i < i1; ++i) {
            const StreamCall &sc = calls[i];
            const StreamPlan &pl = sc.plan;
            CallDesc &d = a.call[i - i0];
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
            d.flags = (pl.nmat == 2 ? kPair : 0) | (sc.out_f32 ? kOutF32 : 0);
            if (i > i0) {
                const StreamCall &p = calls[i - 1];
                const size_t ybytes = (size_t)p.plan.rows * p.plan.n * (p.out_f32 ? 4 : 2);
                if (ranges_overlap(sc.x, (size_t)rows * pl.k * 2, p.y, ybytes)) d.flags |= kReloadX;
            }
            if (pl.G > G) G = pl.G;
            if (pl.waves > waves) waves = pl.waves;
        }
        a.G = G;
        hipError_t e = launch_args(rows, a, waves, stream_lds_bytes(rows, waves), stream);
        if (e != hipSuccess) return e;
        i0 = i1;
    }
    return hipSuccess;
}

}  // namespace nvfp4
