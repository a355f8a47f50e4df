// nvfp4_stream.hip -- persistent streaming NVFP4 projection kernel for gfx950.
//
// y[r][j] = s_g * sum_k (code * scale)[j][k] * x[r][k] for 1..8 activation rows,
// and the gate/up pair o = silu(g) * u (the w4a16_gemv / w4a16_gemv_dual kernel
// family of the Qwen3.8-27B-NVFP4 blueprint page, "Kernels" table).
//
// Decode GEMVs are bound by the HBM weight stream, so the launch is shaped for
// the stream rather than for the arithmetic:
//   * at most one workgroup per CU (G <= 256), all resident at once: no second
//     dispatch round and no per-workgroup start-up in the middle of the stream;
//   * every wave runs a two-deep pipeline over its super-tiles (64 features x
//     256 k): the codes, scales and activation window of super-tile i+1 are in
//     flight while super-tile i is computed.  The activation window travels
//     with its weights, so it is never stuck behind other waves' weight loads;
//   * a workgroup owns whole strips of 64 features where it can (no split-K,
//     no cross-workgroup traffic); the remaining units of work are cut into
//     balanced pieces of strips ("stream-K").  A workgroup processes its pieces
//     first, so their publish / last-arrival handshake overlaps the rest of the
//     stream, and finishes with the strips it owns outright;
//   * pieces of a strip are summed in piece order by the last to arrive (an
//     arrival counter), so results are bitwise deterministic with no float
//     atomics.  Partials and counters are accessed only with device-scope
//     atomics (sc1), ordered by explicit waits -- no cache-wide flushes.
//
// Work units: strip s in [0, S) x super-tile u in [0, T).  G workgroups; the
// first G*F strips are owned, F per workgroup; the R = S - G*F remaining
// strips form R*T shared units split into G contiguous ranges
// [g*RT/G, (g+1)*RT/G), cut at strip boundaries into pieces.
#include <atomic>
#include <type_traits>

#include "nvfp4_core.h"

namespace nvfp4 {
namespace {
using namespace core;

struct StreamArgs {
    const uint8_t *w0;    // packed weight (gate of the pair)
    const uint8_t *w1;    // packed up weight (pair only)
    const uint16_t *x;    // [ROWS][k] bf16
    void *y;              // [ROWS][n]
    float *partial;       // [R][max_pieces][NMAT][ROWS][64]
    unsigned *counters;   // [R]
    int n, k, T;
    int G, F, R;
    int max_pieces;
    int out_f32;
};

// Workgroup whose shared range [floor(g*U/G), floor((g+1)*U/G)) holds shared
// unit v: the largest g with g*U < (v+1)*G, i.e. ((v+1)*G - 1) / U.
__host__ __device__ __forceinline__ int owner_wg(long long v, long long U, int G) {
    return (int)(((v + 1) * G - 1) / U);
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Streamed-once weight bytes: nontemporal loads keep them from displacing the
// activations and partials in the caches.
__device__ __forceinline__ uint4 load_nt(const uint8_t *p) {
    const u32x4_t t = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
    return make_uint4(t.x, t.y, t.z, t.w);
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

// Issue the loads of super-tile u of strip s of matrix w (with its activation
// window when WITH_X).  With real == false the same loads read an always-valid
// location (the weight's first super-tile, the header's zero bytes), so the
// number of loads in flight never depends on control flow and the compiler can
// count them exactly; those results are never used.
template <int ROWS, bool WITH_X>
__device__ __forceinline__ void load_tile(const StreamArgs &a, const uint8_t *w, int s, int u, bool real,
                                          int lane, Tile<ROWS> &b) {
    const size_t off = real ? ((size_t)s * a.T + u) * kSuperBytes : 0;
    const uint8_t *base = w + kHeaderBytes + off;
    // the activation window first: it is consumed first (staged into LDS)
    // and, issued first, it can be waited for while the codes are in flight
    if (WITH_X) {
        const int kbase = u * kSuperK;
#pragma unroll
        for (int i = 0; i < Tile<ROWS>::XR; ++i) {
            const int c = lane + 64 * i;
            const int r = c >> 5, kk = (c & 31) * 8;
            const bool in = real && r < ROWS && kbase + kk < a.k;
            // chunks past the activations read 16 zero bytes from the packed
            // header's padding instead: always issued, never masked afterwards
            // (both addresses are formed, then one is selected: no branch)
            const uint8_t *xp = reinterpret_cast<const uint8_t *>(a.x + (size_t)min(r, ROWS - 1) * a.k + kbase + kk);
            const uint8_t *src = in ? xp : a.w0 + kHeaderZeroOffset;
            b.xv[i] = *reinterpret_cast<const uint4 *>(src);
        }
    }
#pragma unroll
    for (int l = 0; l < kCodeChunks / 2; ++l) b.wc[l] = load_nt(base + l * 2 * kCodeChunkBytes + lane * 16);
    b.ws = load_nt(base + kScaleOffset + lane * 16);
    // keep the whole tile's loads ahead of what follows (the scheduler would
    // otherwise sink them into the previous tile's arithmetic, after its wait)
    __builtin_amdgcn_sched_barrier(0);
}

// Buffer resource over the outputs: stores at an offset past its size are
// dropped by the hardware, which masks the lanes past the last feature without
// a branch.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t output_rsrc(const StreamArgs &a, int rows) {
    const int bytes = rows * a.n * (a.out_f32 ? 4 : 2);
    return __builtin_amdgcn_make_buffer_rsrc(a.y, (short)0, bytes, 0x00020000);
}

constexpr int kDroppedOffset = 0x7fffffff;

// Apply the tensor scales (sg[m] of matrix m) and the SiLU product, and store
// row r of a strip's outputs.
template <int ROWS, int NMAT>
__device__ __forceinline__ void epilogue(const StreamArgs &a, __amdgpu_buffer_rsrc_t yr, const float *red,
                                         const float (&sg)[NMAT], int s, int r, int lane) {
    const int f = s * kStripN + lane;
    float out;
    if (NMAT == 1) {
        out = red[r * kStripN + lane] * sg[0];
    } else {
        const float g = red[r * kStripN + lane] * sg[0];
        const float u = red[(ROWS + r) * kStripN + lane] * sg[NMAT - 1];
        out = g / (1.0f + expf(-g)) * u;
    }
    const int at = r * a.n + f;
    if (a.out_f32)
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, out), yr,
                                              f < a.n ? at * 4 : kDroppedOffset, 0, 0);
    else
        __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16_rne(out), yr, f < a.n ? at * 2 : kDroppedOffset, 0, 0);
}

// The work of workgroup g as one sequence of super-tiles, in segments: first
// its shared range [su0, su1) of the R*T shared units, cut at strip
// boundaries (nsh segments), then its F owned strips.  Every quantity here
// derives from kernel arguments and the workgroup index only, so the compiler
// keeps it, and every branch on it, on the scalar unit.
struct Geometry {
    int g, su0, su1, fs, nsh, nseg, total;
    // A shared range never exceeds one strip's T super-tiles, so it touches at
    // most two shared strips: fs, whose pieces may start in an earlier
    // workgroup (this one is piece `piece0` of `np0`), and fs + 1, which
    // starts here (piece 0 of `np1`).
    int piece0, np0, np1;
};

__device__ __forceinline__ Geometry make_geometry(const StreamArgs &a) {
    Geometry q;
    q.g = blockIdx.x;
    const long long U = (long long)a.R * a.T;
    q.su0 = (int)((long long)q.g * U / a.G);
    q.su1 = (int)((long long)(q.g + 1) * U / a.G);
    q.fs = q.su1 > q.su0 ? q.su0 / a.T : 0;
    q.nsh = q.su1 > q.su0 ? (q.su1 - 1) / a.T - q.fs + 1 : 0;
    q.nseg = q.nsh + a.F;
    q.total = (q.su1 - q.su0) + a.F * a.T;
    q.piece0 = q.np0 = q.np1 = 1;
    if (q.nsh > 0) {
        const int first = owner_wg((long long)q.fs * a.T, U, a.G);
        q.piece0 = q.g - first;
        q.np0 = owner_wg((long long)(q.fs + 1) * a.T - 1, U, a.G) - first + 1;
        q.np1 = owner_wg((long long)(q.fs + 2) * a.T - 1, U, a.G) - q.g + 1;
    }
    return q;
}

// Segment k of the sequence: positions [start, end), strip, first super-tile.
struct Cursor {
    int k, start, end, strip, u0;
};

// Segment order within a workgroup's sequence: its shared pieces before or
// after its owned strips.
#ifndef NVFP4_SHARED_FIRST
#define NVFP4_SHARED_FIRST 0
#endif
constexpr bool kSharedFirst = NVFP4_SHARED_FIRST != 0;

// Shared-strip index of segment k, or -1 for an owned strip.
__device__ __forceinline__ int segment_shared(const StreamArgs &a, const Geometry &q, int k) {
    if (kSharedFirst) return k < q.nsh ? q.fs + k : -1;
    return k >= a.F ? q.fs + (k - a.F) : -1;
}

// Index among the workgroup's owned strips of an owned segment k.
__device__ __forceinline__ int segment_owned(const Geometry &q, int k) {
    return kSharedFirst ? k - q.nsh : k;
}

__device__ __forceinline__ Cursor cursor_at(const StreamArgs &a, const Geometry &q, int k) {
    const int sh = segment_shared(a, q, k);
    const int f = segment_owned(q, k);
    const int shared_base = kSharedFirst ? 0 : a.F * a.T;
    const int owned_base = kSharedFirst ? q.su1 - q.su0 : 0;
    const int v0 = max(q.su0, sh * a.T), v1 = min(q.su1, (sh + 1) * a.T);
    Cursor c;
    c.k = k;
    const bool live = k < q.nseg, shared = sh >= 0;
    c.start = !live ? 0x7fffffff : shared ? shared_base + v0 - q.su0 : owned_base + f * a.T;
    c.end = !live ? 0x7fffffff : shared ? shared_base + v1 - q.su0 : owned_base + (f + 1) * a.T;
    c.strip = shared ? a.G * a.F + sh : q.g * a.F + f;
    c.u0 = shared ? v0 - sh * a.T : 0;
    return c;
}

// Close segment k: reduce the waves' accumulators in wave order, then either
// write the strip's outputs, or store this piece of a shared strip in the
// partials and mark it in pub[] (strip fs or fs + 1).  Arrivals are counted,
// and the last piece's workgroup sums the pieces, once the tile loop is over.
// Every wave calls this for every segment, in order, and leaves with its
// accumulators cleared.  Rows r = wave, wave + nwaves, ... are this wave's.
//
// This runs inside the tile loop, so its loops are fully unrolled with
// wave-uniform guards: a rolled loop or a divergent branch there makes the
// compiler assume that tile loads may still be in flight at the top of the
// tile loop, and wait for them.
template <int ROWS, int NMAT>
__device__ __forceinline__ void finish_segment(const StreamArgs &a, const Geometry &q, int k, float *red,
                                               const float (&sg)[NMAT], __amdgpu_buffer_rsrc_t yr,
                                               int wave, int nwaves, int lane, float (&acc)[NMAT][4][ROWS],
                                               int (&pub)[2]) {
    __syncthreads();   // the previous segment's reads of `red` are done
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int r = 0; r < ROWS; ++r) {
            const float a4[4] = {acc[m][0][r], acc[m][1][r], acc[m][2][r], acc[m][3][r]};
            red[((wave * NMAT + m) * ROWS + r) * kStripN + lane] = core::strip_total(a4, lane);
#pragma unroll
            for (int fb = 0; fb < 4; ++fb) acc[m][fb][r] = 0.0f;
        }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < ROWS; ++t) {
        const int r = wave + t * nwaves;
        if (r < ROWS) {
#pragma unroll
            for (int m = 0; m < NMAT; ++m) {
                float v = red[(m * ROWS + r) * kStripN + lane];
#pragma unroll
                for (int w = 1; w < kMaxWavesPerWg; ++w)
                    if (w < nwaves) v += red[((w * NMAT + m) * ROWS + r) * kStripN + lane];
                red[(m * ROWS + r) * kStripN + lane] = v;
            }
        }
    }
    const int sh = segment_shared(a, q, k);
    const bool head = sh == q.fs;
    const int np = head ? q.np0 : q.np1;
    if (sh >= 0 && np > 1) {
        const size_t slot = ((size_t)sh * a.max_pieces + (head ? q.piece0 : 0)) * NMAT;
#pragma unroll
        for (int t = 0; t < ROWS; ++t) {
            const int r = wave + t * nwaves;
            if (r < ROWS) {
#pragma unroll
                for (int m = 0; m < NMAT; ++m)
                    __hip_atomic_store(&a.partial[((slot + m) * ROWS + r) * kStripN + lane],
                                       red[(m * ROWS + r) * kStripN + lane], __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        pub[head ? 0 : 1] = 1;   // its arrival is counted after the tile loop
        return;
    }
    const int strip = sh >= 0 ? a.G * a.F + sh : q.g * a.F + segment_owned(q, k);
#pragma unroll
    for (int t = 0; t < ROWS; ++t) {
        const int r = wave + t * nwaves;
        if (r < ROWS) epilogue<ROWS, NMAT>(a, yr, red, sg, strip, r, lane);
    }
}

// Sum the pieces of shared strip sh in piece order and write its outputs
// (done by the workgroup whose piece arrived last), then clear its counter.
template <int ROWS, int NMAT>
__device__ __forceinline__ void final_sum(const StreamArgs &a, int sh, int np, float *red, const float (&sg)[NMAT],
                                          __amdgpu_buffer_rsrc_t yr, int wave, int nwaves, int lane) {
    __syncthreads();   // earlier reads of `red` are done
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    constexpr int QB = 8;   // partial loads in flight per matrix before the in-order adds
    for (int r = wave; r < ROWS; r += nwaves) {
        float tq[NMAT];
#pragma unroll
        for (int m = 0; m < NMAT; ++m) tq[m] = 0.0f;
        for (int q0 = 0; q0 < np; q0 += QB) {
            float pv[NMAT][QB];
#pragma unroll
            for (int j = 0; j < QB; ++j) {
                const int pq = min(q0 + j, np - 1);
                const size_t qs = ((size_t)sh * a.max_pieces + pq) * NMAT;
#pragma unroll
                for (int m = 0; m < NMAT; ++m)
                    pv[m][j] = __hip_atomic_load(&a.partial[((qs + m) * ROWS + r) * kStripN + lane],
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
#pragma unroll
            for (int j = 0; j < QB; ++j)
                if (q0 + j < np)
#pragma unroll
                    for (int m = 0; m < NMAT; ++m) tq[m] += pv[m][j];
        }
#pragma unroll
        for (int m = 0; m < NMAT; ++m) red[(m * ROWS + r) * kStripN + lane] = tq[m];
        epilogue<ROWS, NMAT>(a, yr, red, sg, a.G * a.F + sh, r, lane);
    }
    if (wave == 0) __hip_atomic_store(&a.counters[sh], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int ROWS, int NMAT>
__global__ __launch_bounds__(max_waves_for_rows(ROWS) * 64) void stream_kernel(StreamArgs a) {
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ unsigned s_last[2];
    const int tid = threadIdx.x, lane = tid & 63;
    // the wave index is uniform across the wave; saying so keeps every loop and
    // branch below on the scalar unit (no exec-masked control flow around loads)
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nwaves = blockDim.x >> 6;
    using XS = core::XStage<ROWS>;
    static_assert(XS::BYTES == 2304 * ((ROWS + 3) / 4) + 32, "host LDS sizing assumes this staging size");
    uint8_t *xs = smem + (size_t)wave * XS::BYTES;   // this wave's staged activations
    float *red = reinterpret_cast<float *>(smem + (size_t)nwaves * XS::BYTES);
    if (lane < 8) reinterpret_cast<uint32_t *>(xs + XS::ZERO_OFF)[lane] = 0u;
    const Geometry q = make_geometry(a);
    // tensor scales, loaded before any tile so that no later wait is for them
    float sg[NMAT];
    sg[0] = *reinterpret_cast<const float *>(a.w0);
    if (NMAT == 2) sg[NMAT - 1] = *reinterpret_cast<const float *>(a.w1);
    const __amdgpu_buffer_rsrc_t yr = output_rsrc(a, ROWS);

    // Wave w takes positions w, w + nwaves, ... of the workgroup's sequence,
    // through all its segments, two deep: the loads of the next super-tile are
    // in flight while one is computed and while a segment is closed.
    const int nw = wave < q.total ? (q.total - wave + nwaves - 1) / nwaves : 0;
    float acc[NMAT][4][ROWS];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int fb = 0; fb < 4; ++fb)
#pragma unroll
            for (int r = 0; r < ROWS; ++r) acc[m][fb][r] = 0.0f;
    int pub[2] = {0, 0};   // pieces of shared strips fs, fs + 1 stored here
    Cursor lc, cc;   // load cursor (runs ahead) and the segment being accumulated
    lc = cursor_at(a, q, 0);
    cc = lc;
    Tile<ROWS> b0, b1;
    // issue the loads of matrix w at position i (dummy loads past the wave's last tile)
    auto load_pos = [&](const uint8_t *w, int i, bool real, Tile<ROWS> &b, auto with_x) {
        if (real)
            while (i >= lc.end) lc = cursor_at(a, q, lc.k + 1);
        load_tile<ROWS, decltype(with_x)::value>(a, w, lc.strip, lc.u0 + (i - lc.start), real, lane, b);
    };
    // close every segment that ends before position i
    auto close_before = [&](int i) {
        while (i >= cc.end) {
            finish_segment<ROWS, NMAT>(a, q, cc.k, red, sg, yr, wave, nwaves, lane, acc, pub);
            cc = cursor_at(a, q, cc.k + 1);
        }
    };
    using WithX = std::true_type;
    using NoX = std::false_type;
    if (NMAT == 1) {
        // Two positions per iteration.  A tile's activations are staged into
        // LDS (their registers freed) before the next tile's loads are issued;
        // its codes are consumed after.  The wave's tile count is padded to
        // even with one dummy tile whose scales are zeroed, so both tiles of
        // every iteration are consumed and the loop has one exit: on the way
        // back to its head the only loads in flight are those of the next
        // tile, and no wait is needed before reusing registers.
        if (nw > 0) {
            load_pos(a.w0, wave, true, b0, WithX{});
            for (int j = 0; j < nw; j += 2) {
                const int i0 = wave + j * nwaves, i1 = i0 + nwaves;
                const bool r1 = j + 1 < nw, r2 = j + 2 < nw;
                core::stage_x<ROWS>(b0.xv, xs, lane);
                load_pos(a.w0, i1, r1, b1, WithX{});
                close_before(i0);
                core::core_mx<ROWS>(b0.wc, b0.ws, xs, lane, acc[0]);
                core::stage_x<ROWS>(b1.xv, xs, lane);
                load_pos(a.w0, i1 + nwaves, r2, b0, WithX{});
                if (!r1) b1.ws = make_uint4(0, 0, 0, 0);
                close_before(i1);   // past the last tile this closes every segment left
                core::core_mx<ROWS>(b1.wc, b1.ws, xs, lane, acc[0]);
            }
        }
    } else {
        // One position per iteration: the gate super-tile (with the activation
        // window, staged once) then the up super-tile of the same position,
        // each in flight while the other is computed.
        if (nw > 0) {
            load_pos(a.w0, wave, true, b0, WithX{});
            for (int j = 0; j < nw; ++j) {
                const int i0 = wave + j * nwaves;
                core::stage_x<ROWS>(b0.xv, xs, lane);
                load_pos(a.w1, i0, true, b1, NoX{});
                close_before(i0);
                core::core_mx<ROWS>(b0.wc, b0.ws, xs, lane, acc[0]);
                load_pos(a.w0, i0 + nwaves, j + 1 < nw, b0, WithX{});
                core::core_mx<ROWS>(b1.wc, b1.ws, xs, lane, acc[NMAT - 1]);
            }
        }
    }
    while (cc.k < q.nseg) {
        finish_segment<ROWS, NMAT>(a, q, cc.k, red, sg, yr, wave, nwaves, lane, acc, pub);
        cc = cursor_at(a, q, cc.k + 1);
    }
    if (pub[0] | pub[1]) {
        // Every wave's partial stores have completed (they are in the
        // device-coherent level) before the arrivals are counted.
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_waitcnt(0);
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __syncthreads();
        if (tid == 0) {
            s_last[0] = pub[0] && __hip_atomic_fetch_add(&a.counters[q.fs], 1u, __ATOMIC_RELAXED,
                                                          __HIP_MEMORY_SCOPE_AGENT) == (unsigned)(q.np0 - 1);
            s_last[1] = pub[1] && __hip_atomic_fetch_add(&a.counters[q.fs + 1], 1u, __ATOMIC_RELAXED,
                                                          __HIP_MEMORY_SCOPE_AGENT) == (unsigned)(q.np1 - 1);
        }
        __syncthreads();
        if (s_last[0]) final_sum<ROWS, NMAT>(a, q.fs, q.np0, red, sg, yr, wave, nwaves, lane);
        if (s_last[1]) final_sum<ROWS, NMAT>(a, q.fs + 1, q.np1, red, sg, yr, wave, nwaves, lane);
    }
}

template <int ROWS, int NMAT>
hipError_t launch_stream_rows(const StreamPlan &pl, const StreamArgs &args, hipStream_t stream) {
    const void *fn = reinterpret_cast<const void *>(&stream_kernel<ROWS, NMAT>);
    // dynamic LDS beyond the default limit needs the attribute, set once per instantiation
    static std::atomic<int> lds_set{0};
    if (lds_set.load(std::memory_order_acquire) == 0) {
        hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024 - 1024);
        if (e != hipSuccess) return e;
        lds_set.store(1, std::memory_order_release);
    }
    StreamArgs a = args;
    void *kargs[] = {&a};
    return hipLaunchKernel(fn, dim3((unsigned)pl.G), dim3((unsigned)(64 * pl.waves)), kargs, pl.lds_bytes, stream);
}

template <int NMAT>
hipError_t launch_stream_nmat(const StreamPlan &pl, const StreamArgs &a, hipStream_t stream) {
    switch (pl.rows) {
        case 1: return launch_stream_rows<1, NMAT>(pl, a, stream);
        case 2: return launch_stream_rows<2, NMAT>(pl, a, stream);
        case 3: return launch_stream_rows<3, NMAT>(pl, a, stream);
        case 4: return launch_stream_rows<4, NMAT>(pl, a, stream);
        case 5: return launch_stream_rows<5, NMAT>(pl, a, stream);
        case 6: return launch_stream_rows<6, NMAT>(pl, a, stream);
        case 7: return launch_stream_rows<7, NMAT>(pl, a, stream);
        case 8: return launch_stream_rows<8, NMAT>(pl, a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

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
    // Waves per workgroup: each keeps about two super-tiles in flight, so this
    // sets the bytes in flight per CU (about 18 KB per wave for one matrix, 36 KB
    // for the pair) -- enough to cover the memory latency at full bandwidth,
    // and few enough that the first tiles arrive early.
    int waves = pl.nmat == 1 ? kStreamWavesSingle : kStreamWavesPair;
    if (waves > max_waves_for_rows(rows)) waves = max_waves_for_rows(rows);
    const long long per_wg = pl.F * (long long)T + (pl.R ? ((long long)pl.R * T + pl.G - 1) / pl.G : 0);
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
    if (pl.max_pieces > 1) {
        pl.counter_bytes = kCounterRegionBytes;
        pl.partial_bytes = (size_t)pl.R * pl.max_pieces * pl.nmat * rows * kStripN * sizeof(float);
    }
    const size_t lds_x = (size_t)pl.waves * (2304 * ((rows + 3) / 4) + 32);   // core::XStage<rows>::BYTES
    const size_t lds_red = (size_t)pl.waves * pl.nmat * rows * kStripN * sizeof(float);
    // at least ~81 KB so that no CU ever holds two of these workgroups
    pl.lds_bytes = lds_x + lds_red < kOneWorkgroupPerCuLds ? kOneWorkgroupPerCuLds : lds_x + lds_red;
    return pl;
}

hipError_t launch_stream(const StreamPlan &pl, const void *w0, const void *w1, const void *x, void *y, int out_f32,
                         void *workspace, hipStream_t stream) {
    StreamArgs a{};
    a.w0 = static_cast<const uint8_t *>(w0);
    a.w1 = static_cast<const uint8_t *>(w1);
    a.x = static_cast<const uint16_t *>(x);
    a.y = y;
    a.counters = static_cast<unsigned *>(workspace);
    a.partial = pl.max_pieces > 1
                    ? reinterpret_cast<float *>(static_cast<uint8_t *>(workspace) + pl.counter_bytes)
                    : nullptr;
    a.n = (int)pl.n;
    a.k = (int)pl.k;
    a.T = pl.supers;
    a.G = pl.G;
    a.F = pl.F;
    a.R = pl.R;
    a.max_pieces = pl.max_pieces;
    a.out_f32 = out_f32;
    return pl.nmat == 2 ? launch_stream_nmat<2>(pl, a, stream) : launch_stream_nmat<1>(pl, a, stream);
}

}  // namespace nvfp4
