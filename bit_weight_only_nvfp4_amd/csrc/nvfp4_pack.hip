// nvfp4_pack.hip -- weight preparation on the device for gfx950:
//   pack     canonical codes/scales -> super-tiled layout (byte permutation);
//   unpack   the inverse;
//   dequant  packed -> fp32 (codes converted by the same instruction the
//            projection kernels use; scales and s_g applied in fp32);
//   quantize fp32 weights -> packed NVFP4 (the step before the projection).
// The kern README describes this stage as device-side weight preparation
// ("weight_prep" kernel, a "load" program that fills fused qkv / gate_up
// buffers); the veloGB10 setup page quantizes a bf16 checkpoint itself with
// "--quantize all".
#include "nvfp4_internal.h"

namespace nvfp4 {
namespace {


// the whole 256-byte header: fields in the first 32 bytes, zeros after
__device__ void write_header(void *packed, float global_scale, int64_t n, int64_t k) {
    uint4 *h = static_cast<uint4 *>(packed);
    h[0] = make_uint4(__builtin_bit_cast(uint32_t, global_scale), NVFP4_LAYOUT_MAGIC, NVFP4_LAYOUT_VERSION, 0u);
    h[1] = make_uint4((uint32_t)(uint64_t)n, (uint32_t)((uint64_t)n >> 32), (uint32_t)(uint64_t)k,
                      (uint32_t)((uint64_t)k >> 32));
    for (int i = 2; i < kHeaderBytes / 16; ++i) h[i] = make_uint4(0u, 0u, 0u, 0u);
}

// Entry e of a super-tile (16 bytes, read by lane l = e % 64 of a wave):
// code entries e < 512 (chunk c = e / 64), then the 64 scale entries.
//   code entry: dword j = the 8 codes of feature 16 (c >> 1) + n for
//     k = 32 (4 (c & 1) + j) + 8 q .. + 7 (q = l >> 4, n = l & 15);
//   scale entry: byte b = the scale of feature 16 (2 (q >> 1) + (b >> 3)) + n,
//     group 2 (b & 7) + (q & 1).
struct Entry {
    bool code;
    int c, q, n;
};
__device__ __forceinline__ Entry entry_of(int e) {
    Entry d;
    d.code = e < kCodeChunks * 64;
    const int l = d.code ? (e & 63) : e - kCodeChunks * 64;
    d.c = d.code ? e >> 6 : 0;
    d.q = l >> 4;
    d.n = l & 15;
    return d;
}
// code entry: feature (in the strip) and first k (in the super-tile) of dword j
__device__ __forceinline__ int code_f(const Entry &d) { return 16 * (d.c >> 1) + d.n; }
__device__ __forceinline__ int code_k(const Entry &d, int j) { return 32 * (4 * (d.c & 1) + j) + 8 * d.q; }
// scale entry: feature (in the strip) and group (in the super-tile) of byte b
__device__ __forceinline__ int scale_f(const Entry &d, int b) { return 16 * (2 * (d.q >> 1) + (b >> 3)) + d.n; }
__device__ __forceinline__ int scale_g(const Entry &d, int b) { return 2 * (b & 7) + (d.q & 1); }

__device__ __forceinline__ uint4 pack16(const uint8_t (&b)[16]) {
    uint4 o;
    o.x = b[0] | (b[1] << 8) | (b[2] << 16) | ((uint32_t)b[3] << 24);
    o.y = b[4] | (b[5] << 8) | (b[6] << 16) | ((uint32_t)b[7] << 24);
    o.z = b[8] | (b[9] << 8) | (b[10] << 16) | ((uint32_t)b[11] << 24);
    o.w = b[12] | (b[13] << 8) | (b[14] << 16) | ((uint32_t)b[15] << 24);
    return o;
}

// one thread per 16-byte entry of the packed body
__global__ __launch_bounds__(256) void pack_kernel(const uint8_t *__restrict__ codes,
                                                   const uint8_t *__restrict__ scales, float global_scale,
                                                   int64_t n, int64_t k, int64_t T, int64_t total,
                                                   uint8_t *__restrict__ packed) {
    const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (id == 0) write_header(packed, global_scale, n, k);
    if (id >= total) return;
    const int64_t st = id / kEntriesPerSuper;
    const int e = (int)(id - st * kEntriesPerSuper);
    const int64_t s = st / T, u = st % T;
    const Entry d = entry_of(e);
    uint8_t b[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) b[i] = 0;
    if (d.code) {
        const int64_t f = s * kStripN + code_f(d);
        if (f < n) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t k0 = u * kSuperK + code_k(d, j);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (k0 + 2 * i < k) b[4 * j + i] = codes[f * (k / 2) + k0 / 2 + i];
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int64_t f = s * kStripN + scale_f(d, i), gi = u * (kSuperK / 16) + scale_g(d, i);
            if (f < n && gi < k / 16) b[i] = scales[f * (k / 16) + gi];
        }
    }
    *reinterpret_cast<uint4 *>(packed + kHeaderBytes + st * kSuperBytes + e * 16) = pack16(b);
}

__global__ __launch_bounds__(256) void unpack_kernel(const uint8_t *__restrict__ packed, int64_t n, int64_t k,
                                                     int64_t T, int64_t total, uint8_t *__restrict__ codes,
                                                     uint8_t *__restrict__ scales, float *global_scale) {
    const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (id == 0 && global_scale) *global_scale = reinterpret_cast<const Header *>(packed)->global_scale;
    if (id >= total) return;
    const int64_t st = id / kEntriesPerSuper;
    const int e = (int)(id - st * kEntriesPerSuper);
    const int64_t s = st / T, u = st % T;
    const Entry d = entry_of(e);
    const uint4 o = *reinterpret_cast<const uint4 *>(packed + kHeaderBytes + st * kSuperBytes + e * 16);
    const uint32_t w[4] = {o.x, o.y, o.z, o.w};
    if (d.code) {
        const int64_t f = s * kStripN + code_f(d);
        if (f >= n) return;
        for (int j = 0; j < 4; ++j) {
            const int64_t k0 = u * kSuperK + code_k(d, j);
            for (int i = 0; i < 4; ++i)
                if (k0 + 2 * i < k) codes[f * (k / 2) + k0 / 2 + i] = (uint8_t)(w[j] >> (8 * i));
        }
    } else {
        for (int i = 0; i < 16; ++i) {
            const int64_t f = s * kStripN + scale_f(d, i), gi = u * (kSuperK / 16) + scale_g(d, i);
            if (f < n && gi < k / 16) scales[f * (k / 16) + gi] = (uint8_t)(w[i >> 2] >> (8 * (i & 3)));
        }
    }
}

// one thread per code entry: 4 runs of 8 weights of one feature, each run
// converted by the instruction the projection kernels use for the codes
// (v_cvt_scalef32_pk_bf16_fp4, exact) and multiplied by its group's E4M3 scale
// (exact: at most 6 significant bits), then by s_g (one rounding)
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t *__restrict__ packed, int64_t n, int64_t k,
                                                      int64_t T, int64_t total, float *__restrict__ out) {
    const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (id >= total) return;
    const int64_t st = id / (kCodeChunks * 64);
    const int e = (int)(id - st * (kCodeChunks * 64));
    const int64_t s = st / T, u = st % T;
    const Entry d = entry_of(e);
    const int fs = code_f(d);
    const int64_t f = s * kStripN + fs;
    if (f >= n) return;
    const uint8_t *sup = packed + kHeaderBytes + st * kSuperBytes;
    const uint4 cw = *reinterpret_cast<const uint4 *>(sup + e * 16);
    const float sg = reinterpret_cast<const Header *>(packed)->global_scale;
    const uint32_t cwv[4] = {cw.x, cw.y, cw.z, cw.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int kp = code_k(d, j);
        const int64_t k0 = u * kSuperK + kp;
        if (k0 >= k) continue;
        const float sc = e4m3_to_f32<0>(sup[scale_byte_offset(fs, kp >> 4)]);
        const uint32_t word = cwv[j];
        const bf16x2_t p[4] = {e2m1x2_to_bf16x2<0>(word), e2m1x2_to_bf16x2<1>(word),
                               e2m1x2_to_bf16x2<2>(word), e2m1x2_to_bf16x2<3>(word)};
        float *dst = out + f * k + k0;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            dst[2 * b] = (bf16_lo_to_f32(p[b]) * sc) * sg;
            dst[2 * b + 1] = (bf16_hi_to_f32(p[b]) * sc) * sg;
        }
    }
}

// ---- quantizer --------------------------------------------------------------

constexpr int kAmaxBlocks = 512;

// OCP E4M3 encode of t >= 0 (possibly +inf): round to nearest even, saturate
// to 448, keep subnormals, never NaN.
__device__ __forceinline__ uint32_t e4m3_encode_rne_sat(float t) {
    if (!(t < 448.0f)) return 0x7Eu;
    if (t < 0x1p-6f) return (uint32_t)__builtin_rintf(t * 512.0f);   // quantum 2^-9, 0..8
    const uint32_t u = __builtin_bit_cast(uint32_t, t);
    // keep 3 mantissa bits with round-half-even; the fp32 exponent field maps
    // to the E4M3 one by subtracting 120 (127 - 7), i.e. 960 after the shift
    return ((u + 0x7FFFFu + ((u >> 20) & 1u)) >> 20) - 960u;
}

// E2M1 encode of q: nearest of 0 .5 1 1.5 2 3 4 6 (ties to the even mantissa
// bit), saturating at 6, sign kept (a negative that rounds to 0 gives 0x8).
__device__ __forceinline__ uint32_t e2m1_encode_rne_sat(float q) {
    const float a = __builtin_fabsf(q);
    const uint32_t mag = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                         (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
                         (uint32_t)(a > 5.0f);
    return mag | ((__builtin_bit_cast(uint32_t, q) >> 31) << 3);
}

// pass 1: per-block max |w| and a non-finite flag
__global__ __launch_bounds__(256) void amax_kernel(const float *__restrict__ W, int64_t count4,
                                                   float *__restrict__ bmax, int *__restrict__ bbad) {
    __shared__ float smax[256];
    __shared__ int sbad[256];
    float m = 0.0f;
    int bad = 0;
    const float4 *W4 = reinterpret_cast<const float4 *>(W);
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count4;
         i += (int64_t)gridDim.x * blockDim.x) {
        const float4 v = W4[i];
        const float a[4] = {__builtin_fabsf(v.x), __builtin_fabsf(v.y), __builtin_fabsf(v.z), __builtin_fabsf(v.w)};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            bad |= !(a[j] <= 3.4028234663852886e38f);   // Inf or NaN
            m = a[j] > m ? a[j] : m;
        }
    }
    smax[threadIdx.x] = m;
    sbad[threadIdx.x] = bad;
    __syncthreads();
    for (int off = 128; off > 0; off >>= 1) {
        if ((int)threadIdx.x < off) {
            const float o = smax[threadIdx.x + off];
            smax[threadIdx.x] = o > smax[threadIdx.x] ? o : smax[threadIdx.x];
            sbad[threadIdx.x] |= sbad[threadIdx.x + off];
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        bmax[blockIdx.x] = smax[0];
        bbad[blockIdx.x] = sbad[0];
    }
}

// pass 2: one thread per 16-weight group of the padded [n_pad][k_pad/16] grid
__global__ __launch_bounds__(256) void quantize_kernel(const float *__restrict__ W, int64_t n, int64_t k,
                                                       int64_t T, int64_t groups_total, int nblocks_amax,
                                                       const float *__restrict__ bmax, const int *__restrict__ bbad,
                                                       int *__restrict__ status, uint8_t *__restrict__ packed) {
    __shared__ float s_sg;
    if (threadIdx.x == 0) {
        float m = 0.0f;
        int bad = 0;
        for (int i = 0; i < nblocks_amax; ++i) {
            m = bmax[i] > m ? bmax[i] : m;
            bad |= bbad[i];
        }
        const float sg = m / 2688.0f;   // amax / (448 * 6), correctly rounded
        s_sg = sg;
        if (blockIdx.x == 0) {
            write_header(packed, sg, n, k);
            *status = bad;
        }
    }
    __syncthreads();
    const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (id >= groups_total) return;
    const float sg = s_sg;
    const int64_t gp = T * (kSuperK / 16);                 // groups per padded row
    const int64_t f = id / gp, g = id - f * gp;
    uint32_t lo = 0, hi = 0, e = 0;
    if (f < n && g < k / 16) {
        const float4 *src = reinterpret_cast<const float4 *>(W + f * k + 16 * g);
        float w[16];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float4 v = src[j];
            w[4 * j] = v.x;
            w[4 * j + 1] = v.y;
            w[4 * j + 2] = v.z;
            w[4 * j + 3] = v.w;
        }
        float a = 0.0f;
#pragma unroll
        for (int j = 0; j < 16; ++j) a = __builtin_fabsf(w[j]) > a ? __builtin_fabsf(w[j]) : a;
        if (sg != 0.0f) e = e4m3_encode_rne_sat((a / 6.0f) / sg);
        const float S = e4m3_to_f32<0>(e) * sg;
        if (S != 0.0f) {
#pragma unroll
            for (int j = 0; j < 8; ++j) lo |= e2m1_encode_rne_sat(w[j] / S) << (4 * j);
#pragma unroll
            for (int j = 0; j < 8; ++j) hi |= e2m1_encode_rne_sat(w[8 + j] / S) << (4 * j);
        }
    }
    const int64_t s = f / kStripN, fs = f % kStripN;
    const int64_t u = g / (kSuperK / 16), q = g % (kSuperK / 16);
    uint8_t *sup = packed + kHeaderBytes + (s * T + u) * kSuperBytes;
    *reinterpret_cast<uint32_t *>(sup + code_piece_offset((int)fs, (int)q * 16)) = lo;
    *reinterpret_cast<uint32_t *>(sup + code_piece_offset((int)fs, (int)q * 16 + 8)) = hi;
    sup[scale_byte_offset((int)fs, (int)q)] = (uint8_t)e;
}

inline unsigned grid_for(int64_t total, int block) { return (unsigned)ceil_div(total, block); }

}  // namespace

hipError_t launch_pack(const uint8_t *codes, const uint8_t *scales, float global_scale, int64_t n, int64_t k,
                       void *packed, hipStream_t stream) {
    const int64_t T = num_supers(k);
    const int64_t total = num_strips(n) * T * kEntriesPerSuper;
    hipLaunchKernelGGL(pack_kernel, dim3(grid_for(total, 256)), dim3(256), 0, stream, codes, scales,
                       global_scale, n, k, T, total, static_cast<uint8_t *>(packed));
    return hipGetLastError();
}

hipError_t launch_unpack(const void *packed, int64_t n, int64_t k, uint8_t *codes, uint8_t *scales,
                         float *global_scale, hipStream_t stream) {
    const int64_t T = num_supers(k);
    const int64_t total = num_strips(n) * T * kEntriesPerSuper;
    hipLaunchKernelGGL(unpack_kernel, dim3(grid_for(total, 256)), dim3(256), 0, stream,
                       static_cast<const uint8_t *>(packed), n, k, T, total, codes, scales, global_scale);
    return hipGetLastError();
}

hipError_t launch_dequant(const void *packed, int64_t n, int64_t k, float *out, hipStream_t stream) {
    const int64_t T = num_supers(k);
    const int64_t total = num_strips(n) * T * kCodeChunks * 64;
    hipLaunchKernelGGL(dequant_kernel, dim3(grid_for(total, 256)), dim3(256), 0, stream,
                       static_cast<const uint8_t *>(packed), n, k, T, total, out);
    return hipGetLastError();
}

size_t quantize_workspace_bytes(int64_t, int64_t) {
    return 256 + (size_t)kAmaxBlocks * (sizeof(float) + sizeof(int));
}

hipError_t launch_quantize(const float *W, int64_t n, int64_t k, void *packed, void *workspace,
                           hipStream_t stream) {
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    int *status = reinterpret_cast<int *>(ws);
    float *bmax = reinterpret_cast<float *>(ws + 256);
    int *bbad = reinterpret_cast<int *>(ws + 256 + kAmaxBlocks * sizeof(float));
    const int64_t count4 = n * k / 4;   // k % 16 == 0
    int64_t nb = ceil_div(count4, 256 * 16);
    if (nb > kAmaxBlocks) nb = kAmaxBlocks;
    if (nb < 1) nb = 1;
    hipLaunchKernelGGL(amax_kernel, dim3((unsigned)nb), dim3(256), 0, stream, W, count4, bmax, bbad);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t T = num_supers(k);
    const int64_t groups_total = num_strips(n) * kStripN * T * (kSuperK / 16);
    hipLaunchKernelGGL(quantize_kernel, dim3(grid_for(groups_total, 256)), dim3(256), 0, stream, W, n, k, T,
                       groups_total, (int)nb, bmax, bbad, status, static_cast<uint8_t *>(packed));
    return hipGetLastError();
}

}  // namespace nvfp4
