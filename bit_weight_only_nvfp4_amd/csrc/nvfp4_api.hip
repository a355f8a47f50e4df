// nvfp4_api.hip -- the C ABI declared in include/nvfp4.h: argument validation
// (all of it before any HIP call), the gfx950 capability check, and dispatch to
// the kernels' launchers on the caller's stream.  No allocation, no
// synchronization, no state other than the thread-local error message and a
// per-device cache of the architecture check.
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <vector>

#include "nvfp4_internal.h"

using namespace nvfp4;

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return status;
}

int ok() {
    g_err[0] = '\0';
    return NVFP4_OK;
}

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool valid_shape(int64_t n, int64_t k) {
    return n >= 1 && k >= 16 && k % 16 == 0 && n <= kMaxN && k <= (int64_t)1 << 24;
}

// 0 = unknown, 1 = gfx950, 2 = other
std::atomic<int> g_dev_state[64];

int check_device(const char *fn) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0)
        return fail(NVFP4_E_DEVICE, "%s: no HIP device available (%s); NVFP4 on this library needs gfx950", fn,
                    hipGetErrorString(e));
    if (dev < 64) {
        int st = g_dev_state[dev].load(std::memory_order_relaxed);
        if (st == 1) return NVFP4_OK;
    }
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return fail(NVFP4_E_HIP, "%s: hipGetDeviceProperties: %s", fn, hipGetErrorString(e));
    const bool is950 = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    if (dev < 64) g_dev_state[dev].store(is950 ? 1 : 2, std::memory_order_relaxed);
    if (!is950)
        return fail(NVFP4_E_DEVICE,
                    "%s: device %d is %s; NVFP4 weights on this library need gfx950 (E2M1/E4M3 conversion and "
                    "bf16 dot instructions)",
                    fn, dev, prop.gcnArchName);
    return NVFP4_OK;
}

int hip_status(const char *fn, hipError_t e) {
    if (e != hipSuccess) return fail(NVFP4_E_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return ok();
}

int check_weight(const char *fn, const char *name, const nvfp4_weight *w) {
    if (!w) return fail(NVFP4_E_NULL, "%s: %s is NULL", fn, name);
    if (w->magic != NVFP4_LAYOUT_MAGIC || w->layout != NVFP4_LAYOUT_VERSION)
        return fail(NVFP4_E_LAYOUT, "%s: %s has magic 0x%08x layout %u, expected 0x%08x layout %u", fn, name,
                    w->magic, w->layout, NVFP4_LAYOUT_MAGIC, NVFP4_LAYOUT_VERSION);
    if (!valid_shape(w->n, w->k))
        return fail(NVFP4_E_SHAPE, "%s: %s has n=%lld k=%lld (need 1 <= n <= 2^20, k a positive multiple of 16, k <= 2^24)", fn,
                    name, (long long)w->n, (long long)w->k);
    if (!w->data) return fail(NVFP4_E_NULL, "%s: %s->data is NULL", fn, name);
    if (!aligned(w->data, 16)) return fail(NVFP4_E_ALIGN, "%s: %s->data is not 16-byte aligned", fn, name);
    return NVFP4_OK;
}

int check_gemv_args(const char *fn, const void *x, int rows, const void *y, int out_dtype) {
    if (!x) return fail(NVFP4_E_NULL, "%s: x is NULL", fn);
    if (!y) return fail(NVFP4_E_NULL, "%s: y is NULL", fn);
    if (rows < 1 || rows > NVFP4_MAX_ROWS)
        return fail(NVFP4_E_ROWS, "%s: rows=%d outside 1..%d", fn, rows, NVFP4_MAX_ROWS);
    if (out_dtype != NVFP4_OUT_BF16 && out_dtype != NVFP4_OUT_F32)
        return fail(NVFP4_E_DTYPE, "%s: out_dtype=%d (0 = bf16, 1 = fp32)", fn, out_dtype);
    if (!aligned(x, 16)) return fail(NVFP4_E_ALIGN, "%s: x is not 16-byte aligned", fn);
    if (!aligned(y, out_dtype == NVFP4_OUT_F32 ? 4 : 2))
        return fail(NVFP4_E_ALIGN, "%s: y is not aligned to its element size", fn);
    return NVFP4_OK;
}

int check_workspace(const char *fn, const void *workspace, size_t workspace_bytes, size_t need) {
    if (need == 0) return NVFP4_OK;
    if (!workspace) return fail(NVFP4_E_WORKSPACE, "%s: workspace is NULL but %zu bytes are needed", fn, need);
    if (workspace_bytes < need)
        return fail(NVFP4_E_WORKSPACE, "%s: workspace has %zu bytes, %zu needed", fn, workspace_bytes, need);
    if (!aligned(workspace, 16)) return fail(NVFP4_E_ALIGN, "%s: workspace is not 16-byte aligned", fn);
    return NVFP4_OK;
}

bool overlap(const void *a, size_t na, const void *b, size_t nb) {
    const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
    return na && nb && pa < pb + nb && pb < pa + na;
}

size_t x_bytes(const StreamCall &c) { return (size_t)c.plan.rows * c.plan.k * 2; }
size_t y_bytes(const StreamCall &c) { return (size_t)c.plan.rows * c.plan.n * (c.out_f32 ? 4 : 2); }
// the bytes a call reads from w0 and w1 (a norm call: delta and weight)
size_t w_bytes(const StreamCall &c) {
    return c.norm ? (size_t)c.plan.rows * c.plan.k * 2 : nvfp4_packed_bytes(c.plan.n, c.plan.k);
}
size_t w1_bytes(const StreamCall &c) {
    return c.norm ? (size_t)c.plan.k * 2 : (c.w1 ? nvfp4_packed_bytes(c.plan.n, c.plan.k) : 0);
}

// A call's outputs may not overlap its own activations, the workspace or any
// weight of the launch (weights are read ahead across calls).  A norm call's
// delta is read as an activation, after the calls before it have finished, so
// an earlier call may write it; its residual_out may be its own residual, and
// a later call may read it (a norm's residual, a projection's x).
int check_overlaps(const char *fn, const StreamCall *calls, int ncalls, const void *workspace, size_t ws_bytes) {
    for (int i = 0; i < ncalls; ++i) {
        const StreamCall &c = calls[i];
        const size_t yb = y_bytes(c), rb = c.norm ? x_bytes(c) : 0;
        if (overlap(c.y, yb, c.x, x_bytes(c)))
            return fail(NVFP4_E_OVERLAP, "%s: call %d: y overlaps its x", fn, i);
        if (overlap(c.y, yb, workspace, ws_bytes) || overlap(c.aux, rb, workspace, ws_bytes))
            return fail(NVFP4_E_OVERLAP, "%s: call %d: an output overlaps the workspace", fn, i);
        for (int j = 0; j < ncalls; ++j) {
            const StreamCall &o = calls[j];
            const bool w0 = !o.norm;   // a norm's w0 is its delta
            if ((w0 && overlap(c.y, yb, o.w0, w_bytes(o))) || (o.w1 && overlap(c.y, yb, o.w1, w1_bytes(o))))
                return fail(NVFP4_E_OVERLAP, "%s: call %d: y overlaps the weight of call %d", fn, i, j);
            if ((w0 && overlap(c.aux, rb, o.w0, w_bytes(o))) || (o.w1 && overlap(c.aux, rb, o.w1, w1_bytes(o))))
                return fail(NVFP4_E_OVERLAP, "%s: call %d: residual_out overlaps the weight of call %d", fn, i, j);
            if (j != i && overlap(c.aux, rb, o.y, y_bytes(o)))
                return fail(NVFP4_E_OVERLAP, "%s: call %d: residual_out overlaps the y of call %d", fn, i, j);
        }
    }
    return NVFP4_OK;
}

// A call of more than kKernelMaxRows rows runs as ceil(rows / 16) calls of
// balanced row counts; each chunk reads the weights once.  A row's result does
// not depend on the chunk it falls in (every row count runs the same
// arithmetic per row).
int num_chunks(int rows) { return (rows + kKernelMaxRows - 1) / kKernelMaxRows; }

void chunk_of(int rows, int j, int &r0, int &nr) {
    const int nch = num_chunks(rows), base = rows / nch, extra = rows % nch;
    r0 = j * base + (j < extra ? j : extra);
    nr = base + (j < extra ? 1 : 0);
}

// Append the calls one projection or pair call runs as (one per row chunk).
void add_calls(std::vector<StreamCall> &out, const nvfp4_weight *w, const nvfp4_weight *up, const void *x,
               int rows, void *y, int out_dtype) {
    const size_t ybytes = out_dtype == NVFP4_OUT_F32 ? 4 : 2;
    for (int j = 0; j < num_chunks(rows); ++j) {
        int r0, nr;
        chunk_of(rows, j, r0, nr);
        StreamCall c{};
        c.plan = make_stream_plan(w->n, w->k, nr, up != nullptr);
        c.w0 = w->data;
        c.w1 = up ? up->data : nullptr;
        c.x = static_cast<const uint8_t *>(x) + (size_t)r0 * w->k * 2;
        c.y = static_cast<uint8_t *>(y) + (size_t)r0 * w->n * ybytes;
        c.out_f32 = out_dtype == NVFP4_OUT_F32;
        out.push_back(c);
    }
}

// Plans only (for the size queries): the chunk row counts of a call.
void add_plans(std::vector<StreamCall> &out, int64_t n, int64_t k, int rows, bool dual) {
    for (int j = 0; j < num_chunks(rows); ++j) {
        int r0, nr;
        chunk_of(rows, j, r0, nr);
        StreamCall c{};
        c.plan = make_stream_plan(n, k, nr, dual);
        out.push_back(c);
    }
}

// A call's outputs may not overlap its own activations (checked on the whole
// call, before it is cut into row chunks).
int check_self_overlap(const char *fn, const nvfp4_weight *w, const void *x, int rows, const void *y,
                       int out_dtype) {
    const size_t xb = (size_t)rows * w->k * 2, yb = (size_t)rows * w->n * (out_dtype == NVFP4_OUT_F32 ? 4 : 2);
    if (overlap(y, yb, x, xb)) return fail(NVFP4_E_OVERLAP, "%s: y overlaps its x", fn);
    return NVFP4_OK;
}

// Validate one projection or pair call (everything but the workspace).
int check_call(const char *fn, const nvfp4_weight *w, const nvfp4_weight *up, const void *x, int rows,
               const void *y, int out_dtype) {
    int st = check_weight(fn, up ? "gate" : "w", w);
    if (st) return st;
    if (up) {
        st = check_weight(fn, "up", up);
        if (st) return st;
        if (w->n != up->n || w->k != up->k)
            return fail(NVFP4_E_SHAPE, "%s: gate is %lldx%lld but up is %lldx%lld", fn, (long long)w->n,
                        (long long)w->k, (long long)up->n, (long long)up->k);
    }
    return check_gemv_args(fn, x, rows, y, out_dtype);
}

// The projection workspace of nvfp4_gemv_noalloc: a file-scope device array,
// one per device the library runs on, held until the process ends.  It is
// zero when the code object is loaded, and every launch leaves its counters
// at zero again (the partial sums are written before they are read), so it
// never needs clearing.  Host code never passes the array's name to a kernel
// or a copy (that is a host-side stand-in, not a device address): it uses the
// device address hipGetSymbolAddress returned for the current device.
constexpr size_t kScratchBytes = NVFP4_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];   // device address of `scratch` on device d, set once

// The device address of the current device's scratch array, looked up on the
// first call on that device (with it current) and kept.
int scratch_address(const char *fn, void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0) return fail(NVFP4_E_DEVICE, "%s: no HIP device (%s)", fn, hipGetErrorString(e));
    if (dev >= kMaxDevices) return fail(NVFP4_E_DEVICE, "%s: device %d beyond the %d this library tracks", fn, dev,
                                        kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(NVFP4_E_HIP, "%s: hipGetSymbolAddress(scratch) on device %d: %s", fn, dev,
                        hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return NVFP4_OK;
}

// Validate a residual add + RMSNorm call of a sequence and append it.
int add_norm_call(const char *fn, const nvfp4_call &c, std::vector<StreamCall> &out) {
    const nvfp4_norm *nm = c.norm;
    if (c.w || c.up || c.x) return fail(NVFP4_E_NULL, "%s: a norm call must have w, up and x NULL", fn);
    if (!nm->residual || !nm->delta || !nm->weight || !nm->residual_out || !c.y)
        return fail(NVFP4_E_NULL, "%s: a norm buffer or y is NULL", fn);
    if (nm->k < 16 || nm->k % 16 != 0 || nm->k > norm_max_k())
        return fail(NVFP4_E_SHAPE, "%s: k=%lld (need a positive multiple of 16, at most %lld)", fn,
                    (long long)nm->k, (long long)norm_max_k());
    if (c.rows < 1 || c.rows > NVFP4_MAX_ROWS)
        return fail(NVFP4_E_ROWS, "%s: rows=%d outside 1..%d", fn, c.rows, NVFP4_MAX_ROWS);
    if (c.out_dtype != NVFP4_OUT_BF16) return fail(NVFP4_E_DTYPE, "%s: a norm call writes bf16", fn);
    if (!(nm->eps >= 0.0f) || nm->eps > 3.0e38f) return fail(NVFP4_E_SHAPE, "%s: eps must be finite and >= 0", fn);
    for (const void *p : {nm->residual, nm->delta, nm->weight, (const void *)nm->residual_out, (const void *)c.y})
        if (!aligned(p, 16)) return fail(NVFP4_E_ALIGN, "%s: every norm buffer must be 16-byte aligned", fn);
    const size_t rb = (size_t)c.rows * nm->k * 2, wb = (size_t)nm->k * 2;
    if (nm->residual_out != nm->residual && overlap(nm->residual_out, rb, nm->residual, rb))
        return fail(NVFP4_E_OVERLAP, "%s: residual_out overlaps residual without being it", fn);
    if (overlap(nm->residual_out, rb, nm->delta, rb) || overlap(nm->residual_out, rb, nm->weight, wb))
        return fail(NVFP4_E_OVERLAP, "%s: residual_out overlaps delta or weight", fn);
    if (overlap(c.y, rb, nm->residual, rb) || overlap(c.y, rb, nm->delta, rb) || overlap(c.y, rb, nm->weight, wb) ||
        overlap(c.y, rb, nm->residual_out, rb))
        return fail(NVFP4_E_OVERLAP, "%s: y overlaps another norm buffer", fn);
    StreamCall s{};
    s.plan = make_norm_plan(nm->k, c.rows);
    s.w0 = nm->delta;
    s.w1 = nm->weight;
    s.x = nm->residual;
    s.y = c.y;
    s.out_f32 = 0;
    s.norm = nm->gemma_offset ? 2 : 1;
    s.aux = nm->residual_out;
    s.eps = nm->eps;
    out.push_back(s);
    return NVFP4_OK;
}

// Validate every call of a sequence and turn it into the calls one launch
// runs (a projection of more than kKernelMaxRows rows: one per row chunk);
// call i runs as out[first[i] .. first[i + 1]).
int build_sequence(const char *fn, const nvfp4_call *calls, int ncalls, std::vector<StreamCall> &out,
                   std::vector<int> &first) {
    if (!calls) return fail(NVFP4_E_NULL, "%s: calls is NULL", fn);
    char name[64];
    out.clear();
    first.assign((size_t)ncalls + 1, 0);
    for (int i = 0; i < ncalls; ++i) {
        const nvfp4_call &c = calls[i];
        snprintf(name, sizeof name, "%s call %d", fn, i);
        first[i] = (int)out.size();
        if (c.norm) {
            int st = add_norm_call(name, c, out);
            if (st) return st;
            continue;
        }
        int st = check_call(name, c.w, c.up, c.x, c.rows, c.y, c.out_dtype);
        if (st) return st;
        st = check_self_overlap(name, c.w, c.x, c.rows, c.y, c.out_dtype);
        if (st) return st;
        add_calls(out, c.w, c.up, c.x, c.rows, c.y, c.out_dtype);
    }
    first[ncalls] = (int)out.size();
    return NVFP4_OK;
}

// A sequence plan (nvfp4_sequence_plan): header, launch records, then the
// byte ranges of every output (checked against the workspace at launch).
constexpr uint32_t kPlanMagic = 0x50535650;   // "PVSP"
struct PlanHeader {
    uint32_t magic, abi;
    size_t bytes, workspace_bytes;
    int device, nrec, nout, pad;
};
struct OutRange {
    uintptr_t p;
    size_t n;
};
struct PlanLayout {
    size_t rec_off, out_off, total;
};
size_t round16(size_t v) { return (v + 15) & ~(size_t)15; }
PlanLayout plan_layout_of(int nrec, int nout) {
    PlanLayout L;
    L.rec_off = round16(sizeof(PlanHeader));
    L.out_off = round16(L.rec_off + (size_t)nrec * launch_rec_bytes());
    L.total = L.out_off + (size_t)nout * sizeof(OutRange);
    return L;
}
PlanLayout plan_layout(const std::vector<StreamCall> &sc) {
    int nout = 0;
    for (const StreamCall &c : sc) nout += c.norm ? 2 : 1;
    return plan_layout_of(sequence_launches(sc.data(), (int)sc.size()), nout);
}

int run_one(const char *fn, const nvfp4_weight *w, const nvfp4_weight *up, const void *x, int rows, void *y,
            int out_dtype, void *workspace, size_t workspace_bytes, void *stream) {
    int st = check_call(fn, w, up, x, rows, y, out_dtype);
    if (st) return st;
    st = check_self_overlap(fn, w, x, rows, y, out_dtype);
    if (st) return st;
    std::vector<StreamCall> sc;
    add_calls(sc, w, up, x, rows, y, out_dtype);
    const int nc = (int)sc.size();
    st = check_workspace(fn, workspace, workspace_bytes, sequence_workspace_bytes(sc.data(), nc));
    if (st) return st;
    st = check_overlaps(fn, sc.data(), nc, workspace, workspace_bytes);
    if (st) return st;
    st = check_device(fn);
    if (st) return st;
    return hip_status(fn, launch_sequence(sc.data(), nc, workspace, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

int nvfp4_abi_version(void) { return NVFP4_ABI_VERSION; }

const char *nvfp4_strerror(int status) {
    switch (status) {
        case NVFP4_OK: return "ok";
        case NVFP4_E_NULL: return "null pointer";
        case NVFP4_E_SHAPE: return "invalid shape";
        case NVFP4_E_ROWS: return "rows out of range";
        case NVFP4_E_ALIGN: return "misaligned pointer";
        case NVFP4_E_DTYPE: return "invalid dtype";
        case NVFP4_E_WORKSPACE: return "workspace missing or too small";
        case NVFP4_E_LAYOUT: return "packed weight layout mismatch";
        case NVFP4_E_DEVICE: return "unsupported device";
        case NVFP4_E_HIP: return "HIP runtime error";
        case NVFP4_E_OVERLAP: return "an output overlaps an input or the workspace";
        default: return "unknown status";
    }
}

const char *nvfp4_last_error(void) { return g_err; }

size_t nvfp4_packed_bytes(int64_t n, int64_t k) {
    if (!valid_shape(n, k)) return 0;
    return (size_t)kHeaderBytes + (size_t)num_strips(n) * (size_t)num_supers(k) * kSuperBytes;
}

int nvfp4_pack(const uint8_t *codes, const uint8_t *scales, float global_scale, int64_t n, int64_t k,
               void *packed, size_t packed_bytes, nvfp4_weight *out, void *stream) {
    static const char *fn = "nvfp4_pack";
    if (!codes || !scales || !packed || !out) return fail(NVFP4_E_NULL, "%s: a pointer argument is NULL", fn);
    if (!valid_shape(n, k))
        return fail(NVFP4_E_SHAPE, "%s: n=%lld k=%lld (need 1 <= n <= 2^20, k a positive multiple of 16, k <= 2^24)", fn,
                    (long long)n, (long long)k);
    if (!aligned(packed, 16)) return fail(NVFP4_E_ALIGN, "%s: packed is not 16-byte aligned", fn);
    const size_t need = nvfp4_packed_bytes(n, k);
    if (packed_bytes < need)
        return fail(NVFP4_E_LAYOUT, "%s: packed buffer has %zu bytes, %zu needed", fn, packed_bytes, need);
    int st = check_device(fn);
    if (st) return st;
    st = hip_status(fn, launch_pack(codes, scales, global_scale, n, k, packed, static_cast<hipStream_t>(stream)));
    if (st) return st;
    out->magic = NVFP4_LAYOUT_MAGIC;
    out->layout = NVFP4_LAYOUT_VERSION;
    out->n = n;
    out->k = k;
    out->data = packed;
    return NVFP4_OK;
}

int nvfp4_unpack(const nvfp4_weight *w, uint8_t *codes, uint8_t *scales, float *global_scale, void *stream) {
    static const char *fn = "nvfp4_unpack";
    int st = check_weight(fn, "w", w);
    if (st) return st;
    if (!codes || !scales) return fail(NVFP4_E_NULL, "%s: codes or scales is NULL", fn);
    if (global_scale && !aligned(global_scale, 4))
        return fail(NVFP4_E_ALIGN, "%s: global_scale is not 4-byte aligned", fn);
    st = check_device(fn);
    if (st) return st;
    return hip_status(fn, launch_unpack(w->data, w->n, w->k, codes, scales, global_scale,
                                        static_cast<hipStream_t>(stream)));
}

int nvfp4_dequant(const nvfp4_weight *w, float *out, void *stream) {
    static const char *fn = "nvfp4_dequant";
    int st = check_weight(fn, "w", w);
    if (st) return st;
    if (!out) return fail(NVFP4_E_NULL, "%s: out is NULL", fn);
    if (!aligned(out, 16)) return fail(NVFP4_E_ALIGN, "%s: out is not 16-byte aligned", fn);
    st = check_device(fn);
    if (st) return st;
    return hip_status(fn, launch_dequant(w->data, w->n, w->k, out, static_cast<hipStream_t>(stream)));
}

size_t nvfp4_quantize_workspace_bytes(int64_t n, int64_t k) {
    if (!valid_shape(n, k)) return 0;
    return quantize_workspace_bytes(n, k);
}

int nvfp4_quantize(const float *W, int64_t n, int64_t k, void *packed, size_t packed_bytes, void *workspace,
                   size_t workspace_bytes, nvfp4_weight *out, void *stream) {
    static const char *fn = "nvfp4_quantize";
    if (!W || !packed || !workspace || !out) return fail(NVFP4_E_NULL, "%s: a pointer argument is NULL", fn);
    if (!valid_shape(n, k))
        return fail(NVFP4_E_SHAPE, "%s: n=%lld k=%lld (need 1 <= n <= 2^20, k a positive multiple of 16, k <= 2^24)", fn,
                    (long long)n, (long long)k);
    if (!aligned(W, 16) || !aligned(packed, 16) || !aligned(workspace, 16))
        return fail(NVFP4_E_ALIGN, "%s: W, packed and workspace must be 16-byte aligned", fn);
    const size_t need = nvfp4_packed_bytes(n, k);
    if (packed_bytes < need)
        return fail(NVFP4_E_LAYOUT, "%s: packed buffer has %zu bytes, %zu needed", fn, packed_bytes, need);
    const size_t wneed = quantize_workspace_bytes(n, k);
    if (workspace_bytes < wneed)
        return fail(NVFP4_E_WORKSPACE, "%s: workspace has %zu bytes, %zu needed", fn, workspace_bytes, wneed);
    int st = check_device(fn);
    if (st) return st;
    st = hip_status(fn, launch_quantize(W, n, k, packed, workspace, static_cast<hipStream_t>(stream)));
    if (st) return st;
    out->magic = NVFP4_LAYOUT_MAGIC;
    out->layout = NVFP4_LAYOUT_VERSION;
    out->n = n;
    out->k = k;
    out->data = packed;
    return NVFP4_OK;
}

size_t nvfp4_workspace_bytes(int64_t n, int64_t k, int rows, int dual) {
    if (!valid_shape(n, k) || rows < 1 || rows > NVFP4_MAX_ROWS) return 0;
    std::vector<StreamCall> sc;
    add_plans(sc, n, k, rows, dual != 0);
    return sequence_workspace_bytes(sc.data(), (int)sc.size());
}

int nvfp4_gemv(const nvfp4_weight *w, const void *x, int rows, void *y, int out_dtype, void *workspace,
               size_t workspace_bytes, void *stream) {
    return run_one("nvfp4_gemv", w, nullptr, x, rows, y, out_dtype, workspace, workspace_bytes, stream);
}

int nvfp4_gemv_noalloc(const nvfp4_weight *w, const void *x, int rows, void *y, int out_dtype, void *stream) {
    static const char *fn = "nvfp4_gemv_noalloc";
    int st = check_call(fn, w, nullptr, x, rows, y, out_dtype);
    if (st) return st;
    st = check_self_overlap(fn, w, x, rows, y, out_dtype);
    if (st) return st;
    std::vector<StreamCall> sc;
    add_calls(sc, w, nullptr, x, rows, y, out_dtype);
    const int nc = (int)sc.size();
    const size_t need = sequence_workspace_bytes(sc.data(), nc);
    if (need > kScratchBytes)
        return fail(NVFP4_E_WORKSPACE,
                    "%s: this call needs %zu bytes of workspace; the static scratch holds %zu (use nvfp4_gemv "
                    "with a workspace of nvfp4_workspace_bytes(n, k, rows, 0) bytes)",
                    fn, need, kScratchBytes);
    st = check_device(fn);
    if (st) return st;
    void *ws = nullptr;
    st = scratch_address(fn, &ws);
    if (st) return st;
    st = check_overlaps(fn, sc.data(), nc, ws, need);
    if (st) return st;
    return hip_status(fn, launch_sequence(sc.data(), nc, need ? ws : nullptr, static_cast<hipStream_t>(stream)));
}

int nvfp4_gemv_dual_silu(const nvfp4_weight *gate, const nvfp4_weight *up, const void *x, int rows, void *y,
                         int out_dtype, void *workspace, size_t workspace_bytes, void *stream) {
    if (!up) return fail(NVFP4_E_NULL, "nvfp4_gemv_dual_silu: up is NULL");
    return run_one("nvfp4_gemv_dual_silu", gate, up, x, rows, y, out_dtype, workspace, workspace_bytes, stream);
}

size_t nvfp4_sequence_workspace_bytes(const nvfp4_call *calls, int ncalls) {
    if (!calls || ncalls <= 0) return 0;
    std::vector<StreamCall> sc;
    sc.reserve(ncalls);
    for (int i = 0; i < ncalls; ++i) {
        const nvfp4_call &c = calls[i];
        if (c.norm) {
            sc.push_back(StreamCall{});   // no partial sums; counts as a call of the launch
            continue;
        }
        if (!c.w || !valid_shape(c.w->n, c.w->k) || c.rows < 1 || c.rows > NVFP4_MAX_ROWS) continue;
        add_plans(sc, c.w->n, c.w->k, c.rows, c.up != nullptr);
    }
    return sequence_workspace_bytes(sc.data(), (int)sc.size());
}

int nvfp4_sequence_launches(const nvfp4_call *calls, int ncalls) {
    if (!calls || ncalls <= 0) return 0;
    std::vector<StreamCall> sc;
    sc.reserve(ncalls);
    for (int i = 0; i < ncalls; ++i) {
        const nvfp4_call &c = calls[i];
        if (c.rows < 1 || c.rows > NVFP4_MAX_ROWS) continue;
        if (c.norm) {
            StreamCall s{};
            s.plan = make_norm_plan(16, c.rows);
            sc.push_back(s);
            continue;
        }
        for (int j = 0; j < num_chunks(c.rows); ++j) {
            int r0, nr;
            chunk_of(c.rows, j, r0, nr);
            StreamCall s{};
            s.plan.rows = nr;
            s.plan.krows = kernel_rows(nr);
            sc.push_back(s);
        }
    }
    return sequence_launches(sc.data(), (int)sc.size());
}

int nvfp4_dense_gemv_bf16(const void *W, int64_t n, int64_t k, const void *x, int rows, void *y, int out_dtype,
                          void *stream) {
    static const char *fn = "nvfp4_dense_gemv_bf16";
    if (!W) return fail(NVFP4_E_NULL, "%s: W is NULL", fn);
    if (!valid_shape(n, k))
        return fail(NVFP4_E_SHAPE, "%s: n=%lld k=%lld (need 1 <= n <= 2^20, k a positive multiple of 16, k <= 2^24)",
                    fn, (long long)n, (long long)k);
    if (!aligned(W, 16)) return fail(NVFP4_E_ALIGN, "%s: W is not 16-byte aligned", fn);
    int st = check_gemv_args(fn, x, rows, y, out_dtype);
    if (st) return st;
    const size_t xb = (size_t)rows * k * 2, yb = (size_t)rows * n * (out_dtype == NVFP4_OUT_F32 ? 4 : 2);
    if (overlap(y, yb, x, xb)) return fail(NVFP4_E_OVERLAP, "%s: y overlaps x", fn);
    if (overlap(y, yb, W, (size_t)n * k * 2)) return fail(NVFP4_E_OVERLAP, "%s: y overlaps W", fn);
    st = check_device(fn);
    if (st) return st;
    const size_t ye = out_dtype == NVFP4_OUT_F32 ? 4 : 2;
    for (int j = 0; j < num_chunks(rows); ++j) {
        int r0, nr;
        chunk_of(rows, j, r0, nr);
        hipError_t e = launch_dense(W, n, k, static_cast<const uint8_t *>(x) + (size_t)r0 * k * 2, nr,
                                    static_cast<uint8_t *>(y) + (size_t)r0 * n * ye, out_dtype == NVFP4_OUT_F32,
                                    static_cast<hipStream_t>(stream));
        if (e != hipSuccess) return hip_status(fn, e);
    }
    return ok();
}

int nvfp4_mxfp4_gemv(const void *codes, const void *scales, int64_t n, int64_t k, const void *x, int rows, void *y,
                     int out_dtype, void *stream) {
    static const char *fn = "nvfp4_mxfp4_gemv";
    if (!codes) return fail(NVFP4_E_NULL, "%s: codes is NULL", fn);
    if (!scales) return fail(NVFP4_E_NULL, "%s: scales is NULL", fn);
    if (n < 1 || n > kMaxN || k < 32 || k % 32 != 0 || k > ((int64_t)1 << 24))
        return fail(NVFP4_E_SHAPE, "%s: n=%lld k=%lld (need 1 <= n <= 2^20, k a positive multiple of 32, k <= 2^24)",
                    fn, (long long)n, (long long)k);
    if (!aligned(codes, 16)) return fail(NVFP4_E_ALIGN, "%s: codes are not 16-byte aligned", fn);
    int st = check_gemv_args(fn, x, rows, y, out_dtype);
    if (st) return st;
    const size_t ye = out_dtype == NVFP4_OUT_F32 ? 4 : 2;
    const size_t xb = (size_t)rows * k * 2, yb = (size_t)rows * n * ye;
    if (overlap(y, yb, x, xb)) return fail(NVFP4_E_OVERLAP, "%s: y overlaps x", fn);
    if (overlap(y, yb, codes, (size_t)n * k / 2) || overlap(y, yb, scales, (size_t)n * k / 32))
        return fail(NVFP4_E_OVERLAP, "%s: y overlaps the weight", fn);
    st = check_device(fn);
    if (st) return st;
    for (int j = 0; j < num_chunks(rows); ++j) {
        int r0, nr;
        chunk_of(rows, j, r0, nr);
        hipError_t e = launch_mx(codes, scales, n, k, static_cast<const uint8_t *>(x) + (size_t)r0 * k * 2, nr,
                                 static_cast<uint8_t *>(y) + (size_t)r0 * n * ye, out_dtype == NVFP4_OUT_F32,
                                 static_cast<hipStream_t>(stream));
        if (e != hipSuccess) return hip_status(fn, e);
    }
    return ok();
}

int nvfp4_w8g32_gemv(const void *codes, const void *scales, int64_t n, int64_t k, const void *x, int rows, void *y,
                     int out_dtype, void *stream) {
    static const char *fn = "nvfp4_w8g32_gemv";
    if (!codes) return fail(NVFP4_E_NULL, "%s: codes is NULL", fn);
    if (!scales) return fail(NVFP4_E_NULL, "%s: scales is NULL", fn);
    if (n < 1 || n > kMaxN || k < 128 || k % 128 != 0 || k > ((int64_t)1 << 24))
        return fail(NVFP4_E_SHAPE, "%s: n=%lld k=%lld (need 1 <= n <= 2^20, k a positive multiple of 128, k <= 2^24)",
                    fn, (long long)n, (long long)k);
    if (!aligned(codes, 16) || !aligned(scales, 8))
        return fail(NVFP4_E_ALIGN, "%s: codes must be 16-byte and scales 8-byte aligned", fn);
    int st = check_gemv_args(fn, x, rows, y, out_dtype);
    if (st) return st;
    const size_t ye = out_dtype == NVFP4_OUT_F32 ? 4 : 2;
    const size_t xb = (size_t)rows * k * 2, yb = (size_t)rows * n * ye;
    if (overlap(y, yb, x, xb)) return fail(NVFP4_E_OVERLAP, "%s: y overlaps x", fn);
    if (overlap(y, yb, codes, (size_t)n * k) || overlap(y, yb, scales, (size_t)n * k / 16))
        return fail(NVFP4_E_OVERLAP, "%s: y overlaps the weight", fn);
    st = check_device(fn);
    if (st) return st;
    for (int j = 0; j < num_chunks(rows); ++j) {
        int r0, nr;
        chunk_of(rows, j, r0, nr);
        hipError_t e = launch_w8(codes, scales, n, k, static_cast<const uint8_t *>(x) + (size_t)r0 * k * 2, nr,
                                 static_cast<uint8_t *>(y) + (size_t)r0 * n * ye, out_dtype == NVFP4_OUT_F32,
                                 static_cast<hipStream_t>(stream));
        if (e != hipSuccess) return hip_status(fn, e);
    }
    return ok();
}

int nvfp4_residual_rmsnorm(const void *residual, const void *delta, const void *weight, int64_t k, int rows,
                           float eps, int gemma_offset, void *residual_out, void *x, void *stream) {
    static const char *fn = "nvfp4_residual_rmsnorm";
    if (!residual) return fail(NVFP4_E_NULL, "%s: residual is NULL", fn);
    if (!delta) return fail(NVFP4_E_NULL, "%s: delta is NULL", fn);
    if (!weight) return fail(NVFP4_E_NULL, "%s: weight is NULL", fn);
    if (!residual_out) return fail(NVFP4_E_NULL, "%s: residual_out is NULL", fn);
    if (!x) return fail(NVFP4_E_NULL, "%s: x is NULL", fn);
    if (k < 16 || k % 16 != 0 || k > norm_max_k())
        return fail(NVFP4_E_SHAPE, "%s: k=%lld (need a positive multiple of 16, at most %lld)", fn, (long long)k,
                    (long long)norm_max_k());
    if (rows < 1 || rows > (1 << 20)) return fail(NVFP4_E_ROWS, "%s: rows=%d outside 1..2^20", fn, rows);
    if (!(eps >= 0.0f) || eps > 3.0e38f) return fail(NVFP4_E_SHAPE, "%s: eps must be finite and >= 0", fn);
    for (const void *p : {residual, delta, weight, (const void *)residual_out, (const void *)x})
        if (!aligned(p, 16)) return fail(NVFP4_E_ALIGN, "%s: every buffer must be 16-byte aligned", fn);
    const size_t rb = (size_t)rows * k * 2, wb = (size_t)k * 2;
    // the residual may be updated in place (residual_out == residual), nothing else may overlap
    if (residual_out != residual && overlap(residual_out, rb, residual, rb))
        return fail(NVFP4_E_OVERLAP, "%s: residual_out overlaps residual without being it", fn);
    if (overlap(residual_out, rb, delta, rb) || overlap(residual_out, rb, weight, wb))
        return fail(NVFP4_E_OVERLAP, "%s: residual_out overlaps delta or weight", fn);
    if (overlap(x, rb, residual, rb) || overlap(x, rb, delta, rb) || overlap(x, rb, weight, wb) ||
        overlap(x, rb, residual_out, rb))
        return fail(NVFP4_E_OVERLAP, "%s: x overlaps another buffer", fn);
    int st = check_device(fn);
    if (st) return st;
    return hip_status(fn, launch_residual_rmsnorm(residual, delta, weight, k, rows, eps, gemma_offset != 0,
                                                  residual_out, x, static_cast<hipStream_t>(stream)));
}

int nvfp4_read_ceiling(const void *buf, size_t bytes, void *sink, void *stream) {
    static const char *fn = "nvfp4_read_ceiling";
    if (!buf || !sink) return fail(NVFP4_E_NULL, "%s: buf or sink is NULL", fn);
    if (bytes == 0 || bytes % 16 != 0) return fail(NVFP4_E_SHAPE, "%s: bytes=%zu (need a positive multiple of 16)", fn, bytes);
    if (!aligned(buf, 16) || !aligned(sink, 4)) return fail(NVFP4_E_ALIGN, "%s: buf must be 16-byte and sink 4-byte aligned", fn);
    int st = check_device(fn);
    if (st) return st;
    return hip_status(fn, launch_read_ceiling(buf, bytes, sink, static_cast<hipStream_t>(stream)));
}

int nvfp4_gemv_sequence(const nvfp4_call *calls, int ncalls, void *workspace, size_t workspace_bytes,
                        void *const *events, void *stream) {
    static const char *fn = "nvfp4_gemv_sequence";
    if (ncalls < 0) return fail(NVFP4_E_SHAPE, "%s: ncalls=%d", fn, ncalls);
    if (ncalls == 0) return ok();
    std::vector<StreamCall> sc;
    std::vector<int> first;   // call i runs as sc[first[i] .. first[i + 1])
    int st = build_sequence(fn, calls, ncalls, sc, first);
    if (st) return st;
    const int nsc = (int)sc.size();
    st = check_workspace(fn, workspace, workspace_bytes, sequence_workspace_bytes(sc.data(), nsc));
    if (st) return st;
    st = check_overlaps(fn, sc.data(), nsc, workspace, workspace_bytes);
    if (st) return st;
    st = check_device(fn);
    if (st) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (!events) return hip_status(fn, launch_sequence(sc.data(), nsc, workspace, s));
    // per-call timing: each call (all its row chunks) launched between its two events
    for (int i = 0; i < ncalls; ++i) {
        if (events[2 * i]) {
            hipError_t e = hipEventRecord(static_cast<hipEvent_t>(events[2 * i]), s);
            if (e != hipSuccess) return fail(NVFP4_E_HIP, "%s: hipEventRecord before call %d: %s", fn, i,
                                             hipGetErrorString(e));
        }
        hipError_t e = hipSuccess;
        for (int j = first[i]; j < first[i + 1] && e == hipSuccess; ++j) e = launch_sequence(&sc[j], 1, workspace, s);
        if (e != hipSuccess) return fail(NVFP4_E_HIP, "%s: launch of call %d failed: %s", fn, i, hipGetErrorString(e));
        if (events[2 * i + 1]) {
            e = hipEventRecord(static_cast<hipEvent_t>(events[2 * i + 1]), s);
            if (e != hipSuccess) return fail(NVFP4_E_HIP, "%s: hipEventRecord after call %d: %s", fn, i,
                                             hipGetErrorString(e));
        }
    }
    return ok();
}

int nvfp4_sequence_waits(const nvfp4_call *calls, int ncalls) {
    static const char *fn = "nvfp4_sequence_waits";
    if (ncalls < 0) return fail(NVFP4_E_SHAPE, "%s: ncalls=%d", fn, ncalls);
    if (ncalls == 0) return 0;
    std::vector<StreamCall> sc;
    std::vector<int> first;
    int st = build_sequence(fn, calls, ncalls, sc, first);
    if (st) return st;
    st = check_overlaps(fn, sc.data(), (int)sc.size(), nullptr, 0);
    if (st) return st;
    return sequence_waits(sc.data(), (int)sc.size());
}

size_t nvfp4_sequence_plan_bytes(const nvfp4_call *calls, int ncalls) {
    static const char *fn = "nvfp4_sequence_plan_bytes";
    if (ncalls <= 0 || !calls) return 0;
    std::vector<StreamCall> sc;
    std::vector<int> first;
    if (build_sequence(fn, calls, ncalls, sc, first)) return 0;
    return plan_layout(sc).total;
}

int nvfp4_sequence_plan(const nvfp4_call *calls, int ncalls, void *plan, size_t plan_bytes) {
    static const char *fn = "nvfp4_sequence_plan";
    if (ncalls <= 0) return fail(NVFP4_E_SHAPE, "%s: ncalls=%d (need at least one call)", fn, ncalls);
    if (!plan) return fail(NVFP4_E_NULL, "%s: plan is NULL", fn);
    if (!aligned(plan, 16)) return fail(NVFP4_E_ALIGN, "%s: plan is not 16-byte aligned", fn);
    std::vector<StreamCall> sc;
    std::vector<int> first;
    int st = build_sequence(fn, calls, ncalls, sc, first);
    if (st) return st;
    const int nsc = (int)sc.size();
    // the plan's outputs against any workspace are checked at launch; here
    // every other overlap rule (no workspace yet)
    st = check_overlaps(fn, sc.data(), nsc, nullptr, 0);
    if (st) return st;
    const PlanLayout L = plan_layout(sc);
    if (plan_bytes < L.total)
        return fail(NVFP4_E_WORKSPACE, "%s: plan has %zu bytes, %zu needed", fn, plan_bytes, L.total);
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) dev = -1;
    uint8_t *base = static_cast<uint8_t *>(plan);
    PlanHeader h{};
    h.magic = kPlanMagic;
    h.abi = NVFP4_ABI_VERSION;
    h.bytes = L.total;
    h.workspace_bytes = sequence_workspace_bytes(sc.data(), nsc);
    h.device = dev;
    h.nrec = build_launches(sc.data(), nsc, base + L.rec_off);
    h.nout = 0;
    OutRange *outs = reinterpret_cast<OutRange *>(base + L.out_off);
    for (const StreamCall &c : sc) {
        outs[h.nout++] = OutRange{reinterpret_cast<uintptr_t>(c.y), y_bytes(c)};
        if (c.norm) outs[h.nout++] = OutRange{reinterpret_cast<uintptr_t>(c.aux), x_bytes(c)};
    }
    *reinterpret_cast<PlanHeader *>(base) = h;
    return ok();
}

int nvfp4_sequence_plan_launch(const void *plan, void *workspace, size_t workspace_bytes, void *stream) {
    static const char *fn = "nvfp4_sequence_plan_launch";
    if (!plan) return fail(NVFP4_E_NULL, "%s: plan is NULL", fn);
    if (!aligned(plan, 16)) return fail(NVFP4_E_ALIGN, "%s: plan is not 16-byte aligned", fn);
    const uint8_t *base = static_cast<const uint8_t *>(plan);
    const PlanHeader &h = *reinterpret_cast<const PlanHeader *>(base);
    if (h.magic != kPlanMagic || h.abi != NVFP4_ABI_VERSION)
        return fail(NVFP4_E_LAYOUT, "%s: not a plan written by nvfp4_sequence_plan of this library", fn);
    int st = check_workspace(fn, workspace, workspace_bytes, h.workspace_bytes);
    if (st) return st;
    const PlanLayout L = plan_layout_of(h.nrec, h.nout);
    const OutRange *outs = reinterpret_cast<const OutRange *>(base + L.out_off);
    for (int i = 0; i < h.nout; ++i)
        if (overlap(reinterpret_cast<const void *>(outs[i].p), outs[i].n, workspace, workspace_bytes))
            return fail(NVFP4_E_OVERLAP, "%s: an output of the plan overlaps the workspace", fn);
    st = check_device(fn);
    if (st) return st;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev != h.device)
        return fail(NVFP4_E_DEVICE, "%s: the plan was made on device %d, the current device is %d", fn, h.device,
                    dev);
    return hip_status(fn, launch_recs(base + L.rec_off, h.nrec, workspace, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
