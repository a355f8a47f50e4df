// nvfp4_bw.hip -- the streaming-read ceiling: a kernel that only reads a
// buffer once (16 bytes per lane per load, nontemporal, every byte once), the
// practical HBM read rate on this device that the projection kernels are
// compared with beside the nominal peak.  The same launch shape as the
// projection kernel (one 512-thread workgroup per CU, 8 loads in flight per
// lane); every loaded word is folded into one xor per workgroup written to
// `sink`, so the loads cannot be removed.
#include "nvfp4_internal.h"

namespace nvfp4 {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef const __attribute__((address_space(1))) u32x4_t *global_u32x4_ptr;

constexpr int kBwThreads = 512;
constexpr int kBwUnroll = 8;

__global__ __launch_bounds__(kBwThreads) void read_kernel(const uint8_t *__restrict__ buf, int64_t n16,
                                                          uint32_t *__restrict__ sink) {
    const int64_t stride = (int64_t)gridDim.x * kBwThreads;
    int64_t i = (int64_t)blockIdx.x * kBwThreads + threadIdx.x;
    uint32_t acc = 0;
    // full rounds of kBwUnroll loads in flight per lane
    for (; i + (kBwUnroll - 1) * stride < n16; i += kBwUnroll * stride) {
        u32x4_t v[kBwUnroll];
#pragma unroll
        for (int u = 0; u < kBwUnroll; ++u)
            v[u] = __builtin_nontemporal_load((global_u32x4_ptr)(buf + (i + u * stride) * 16));
#pragma unroll
        for (int u = 0; u < kBwUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n16; i += stride) {
        const u32x4_t v = __builtin_nontemporal_load((global_u32x4_ptr)(buf + i * 16));
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    __shared__ uint32_t s[kBwThreads / 64];
    for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o);
    if ((threadIdx.x & 63) == 0) s[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t t = 0;
        for (int w = 0; w < kBwThreads / 64; ++w) t ^= s[w];
        sink[blockIdx.x] = t;
    }
}

}  // namespace

hipError_t launch_read_ceiling(const void *buf, size_t bytes, void *sink, hipStream_t stream) {
    hipLaunchKernelGGL(read_kernel, dim3(kMaxWorkgroups), dim3(kBwThreads), 0, stream,
                       static_cast<const uint8_t *>(buf), (int64_t)(bytes / 16), static_cast<uint32_t *>(sink));
    return hipGetLastError();
}

}  // namespace nvfp4
