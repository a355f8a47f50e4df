// Drives the host side of the HIP library -- argument validation, the
// sequence builder and the plan writer -- for a build whose host code has
// AddressSanitizer and UndefinedBehaviorSanitizer.  Every buffer address is
// fake (never dereferenced): each call returns an error before touching the
// device, or NVFP4_E_DEVICE where every check passed and no gfx950 device is
// present (on a machine with one, those calls are not made).  Plans are
// written into exactly sized heap buffers.  Exits 0 when every status is the
// documented one.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "nvfp4.h"

static int failures = 0;
#define EXPECT_EQ(a, b)                                                                                  \
    do {                                                                                                 \
        const long long va = (long long)(a), vb = (long long)(b);                                        \
        if (va != vb) {                                                                                  \
            std::fprintf(stderr, "%s:%d: %s = %lld, expected %lld (%s)\n", __FILE__, __LINE__, #a, va, vb, \
                         nvfp4_last_error());                                                            \
            ++failures;                                                                                  \
        }                                                                                                \
    } while (0)

// small weights at FAKE, activations at XF, outputs at YF, workspaces at WF,
// large weights from 4 GiB up: no two ranges overlap unless a check plants it
static const uintptr_t FAKE = 0x10000, XF = 0x1000000, YF = 0x2000000, WF = 0x3000000, BIG = 0x100000000ull;
static void *P(uintptr_t a) { return reinterpret_cast<void *>(a); }
static const uint8_t *B(uintptr_t a) { return reinterpret_cast<const uint8_t *>(a); }

static nvfp4_weight weight(int64_t n, int64_t k, uintptr_t data) {
    nvfp4_weight w{};
    w.magic = NVFP4_LAYOUT_MAGIC;
    w.layout = NVFP4_LAYOUT_VERSION;
    w.n = n;
    w.k = k;
    w.data = P(data);
    return w;
}

int main() {
    const bool no_device = std::getenv("NVFP4_SAN_HAS_DEVICE") == nullptr;
    EXPECT_EQ(nvfp4_abi_version(), NVFP4_ABI_VERSION);
    for (int s = 1; s >= -12; --s) (void)nvfp4_strerror(s);

    // single calls
    nvfp4_weight w = weight(256, 512, FAKE), big = weight(5120, 17408, BIG);
    EXPECT_EQ(nvfp4_gemv(nullptr, P(XF), 1, P(YF), 0, nullptr, 0, nullptr), NVFP4_E_NULL);
    EXPECT_EQ(nvfp4_gemv(&w, P(XF), 0, P(YF), 0, nullptr, 0, nullptr), NVFP4_E_ROWS);
    EXPECT_EQ(nvfp4_gemv(&w, P(XF), 129, P(YF), 0, nullptr, 0, nullptr), NVFP4_E_ROWS);
    EXPECT_EQ(nvfp4_gemv(&w, P(XF + 2), 1, P(YF), 0, nullptr, 0, nullptr), NVFP4_E_ALIGN);
    EXPECT_EQ(nvfp4_gemv(&w, P(XF), 1, P(YF), 7, nullptr, 0, nullptr), NVFP4_E_DTYPE);
    EXPECT_EQ(nvfp4_gemv(&w, P(XF), 1, P(XF), 0, nullptr, 0, nullptr), NVFP4_E_OVERLAP);
    const size_t need = nvfp4_workspace_bytes(5120, 17408, 8, 0);
    EXPECT_EQ(nvfp4_gemv(&big, P(XF), 8, P(YF), 0, P(WF), need - 1, nullptr), NVFP4_E_WORKSPACE);
    if (no_device) EXPECT_EQ(nvfp4_gemv(&big, P(XF), 8, P(YF), 0, P(WF), need, nullptr), NVFP4_E_DEVICE);
    nvfp4_weight bad = w;
    bad.layout = 2;
    EXPECT_EQ(nvfp4_gemv(&bad, P(XF), 1, P(YF), 0, nullptr, 0, nullptr), NVFP4_E_LAYOUT);
    EXPECT_EQ(nvfp4_gemv_noalloc(&big, P(XF), 200, P(YF), 0, nullptr), NVFP4_E_ROWS);
    nvfp4_weight out{};
    const size_t pb = nvfp4_packed_bytes(256, 512);
    EXPECT_EQ(nvfp4_pack(B(FAKE), B(FAKE), 1.0f, 256, 520, P(FAKE), pb, &out, nullptr), NVFP4_E_SHAPE);
    EXPECT_EQ(nvfp4_pack(B(FAKE), B(FAKE), 1.0f, 256, 512, P(FAKE), pb - 1, &out, nullptr), NVFP4_E_LAYOUT);
    EXPECT_EQ(nvfp4_residual_rmsnorm(P(XF), P(WF), P(FAKE), 24, 2, 1e-6f, 0, P(YF), P(YF + 0x100000), nullptr),
              NVFP4_E_SHAPE);
    EXPECT_EQ(nvfp4_residual_rmsnorm(P(XF), P(WF), P(FAKE), 512, 2, NAN, 0, P(YF), P(YF + 0x100000), nullptr),
              NVFP4_E_SHAPE);
    EXPECT_EQ(nvfp4_dense_gemv_bf16(P(FAKE), 256, 520, P(XF), 1, P(YF), 0, nullptr), NVFP4_E_SHAPE);
    EXPECT_EQ(nvfp4_mxfp4_gemv(P(FAKE), P(FAKE + 4096 * 4), 256, 512, P(XF), 0, P(YF), 0, nullptr), NVFP4_E_ROWS);
    EXPECT_EQ(nvfp4_w8g32_gemv(P(FAKE), P(FAKE), 256, 500, P(XF), 1, P(YF), 0, nullptr), NVFP4_E_SHAPE);
    EXPECT_EQ(nvfp4_read_ceiling(P(XF), 24, P(YF), nullptr), NVFP4_E_SHAPE);

    // a 64-layer decode step with norms: 384 calls, 129 distinct weights
    const int layers = 64, per = 6, ncalls = layers * per;
    std::vector<nvfp4_weight> ws;
    ws.reserve(layers * 5);
    std::vector<nvfp4_norm> norms(2 * layers);
    std::vector<nvfp4_call> calls(ncalls);
    // decode-step buffers 16 MiB apart (the largest, at 100 rows, is 3.4 MB)
    const uintptr_t R = 0x10000000, XN = R + 0x1000000, A = R + 0x2000000, QKV = R + 0x3000000, O = R + 0x4000000,
                    H = R + 0x5000000, D = R + 0x6000000;
    for (int l = 0; l < layers; ++l) {
        const uintptr_t base = BIG + (uintptr_t)l * 0x40000000ull;
        ws.push_back(weight(12288, 5120, base));
        ws.push_back(weight(5120, 6144, base + 0x4000000));
        ws.push_back(weight(17408, 5120, base + 0x8000000));
        ws.push_back(weight(17408, 5120, base + 0xC000000));
        ws.push_back(weight(5120, 17408, base + 0x10000000));
        nvfp4_weight *lw = &ws[ws.size() - 5];
        for (int j = 0; j < 2; ++j) {
            nvfp4_norm &nm = norms[2 * l + j];
            nm.residual = P(R);
            nm.residual_out = P(R);
            nm.delta = P(j ? O : D);
            nm.weight = P(base + 0x20000000 + j * 0x10000);
            nm.k = 5120;
            nm.eps = 1e-6f;
            nm.gemma_offset = 1;
        }
        nvfp4_call *c = &calls[l * per];
        c[0] = nvfp4_call{nullptr, nullptr, nullptr, P(XN), 8, 0, &norms[2 * l]};
        c[1] = nvfp4_call{&lw[0], nullptr, P(XN), P(QKV), 8, 0, nullptr};
        c[2] = nvfp4_call{&lw[1], nullptr, P(A), P(O), 8, 0, nullptr};
        c[3] = nvfp4_call{nullptr, nullptr, nullptr, P(XN), 8, 0, &norms[2 * l + 1]};
        c[4] = nvfp4_call{&lw[2], &lw[3], P(XN), P(H), 8, 0, nullptr};
        c[5] = nvfp4_call{&lw[4], nullptr, P(H), P(D), 8, 0, nullptr};
    }
    const size_t sneed = nvfp4_sequence_workspace_bytes(calls.data(), ncalls);
    EXPECT_EQ(sneed > 65 * 1024, 1);
    EXPECT_EQ(nvfp4_sequence_launches(calls.data(), ncalls) >= 1, 1);
    if (no_device) EXPECT_EQ(nvfp4_gemv_sequence(calls.data(), ncalls, P(WF), sneed, nullptr, nullptr), NVFP4_E_DEVICE);
    const size_t nb = nvfp4_sequence_plan_bytes(calls.data(), ncalls);
    EXPECT_EQ(nb > 0, 1);
    void *raw = std::aligned_alloc(16, (nb + 15) / 16 * 16);
    EXPECT_EQ(nvfp4_sequence_plan(calls.data(), ncalls, raw, nb - 1), NVFP4_E_WORKSPACE);
    EXPECT_EQ(nvfp4_sequence_plan(calls.data(), ncalls, raw, nb), NVFP4_OK);
    EXPECT_EQ(nvfp4_sequence_plan_launch(raw, P(WF), sneed - 16, nullptr), NVFP4_E_WORKSPACE);
    EXPECT_EQ(nvfp4_sequence_plan_launch(raw, P(D), sneed, nullptr), NVFP4_E_OVERLAP);
    if (no_device) EXPECT_EQ(nvfp4_sequence_plan_launch(raw, P(WF), sneed, nullptr), NVFP4_E_DEVICE);
    std::free(raw);
    // rows past one kernel call: row chunks
    for (nvfp4_call &c : calls) c.rows = 100;
    const size_t nb2 = nvfp4_sequence_plan_bytes(calls.data(), ncalls);
    EXPECT_EQ(nb2 > nb, 1);
    raw = std::aligned_alloc(16, (nb2 + 15) / 16 * 16);
    EXPECT_EQ(nvfp4_sequence_plan(calls.data(), ncalls, raw, nb2), NVFP4_OK);
    std::free(raw);
    // errors found while building
    calls[7].rows = 0;
    EXPECT_EQ(nvfp4_sequence_plan_bytes(calls.data(), ncalls), 0);
    EXPECT_EQ(nvfp4_gemv_sequence(calls.data(), ncalls, P(WF), sneed, nullptr, nullptr), NVFP4_E_ROWS);
    calls[7].rows = 100;
    norms[5].k = 5121;
    EXPECT_EQ(nvfp4_gemv_sequence(calls.data(), ncalls, P(WF), sneed, nullptr, nullptr), NVFP4_E_SHAPE);
    norms[5].k = 5120;
    const size_t sneed2 = nvfp4_sequence_workspace_bytes(calls.data(), ncalls);
    calls[11].y = P(BIG + 0x4000000 + 4096);   // into layer 0's o weight
    EXPECT_EQ(nvfp4_gemv_sequence(calls.data(), ncalls, P(WF), sneed2, nullptr, nullptr), NVFP4_E_OVERLAP);

    if (failures) {
        std::fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    std::printf("host driver: ok\n");
    return 0;
}
