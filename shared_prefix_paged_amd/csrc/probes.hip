// HIP measurement probes for gfx950 (MI355X) and their C ABI entry points:
// what this device achieves on a streaming read and on bf16 MFMA, beside its
// published peaks.  No attention kernel lives here.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <string>

#include "internal.h"

using spkv::fail;

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// The read takes block-contiguous 32 KB chunks (each lane 8 nontemporal
// 16-byte loads in flight, 16 blocks per CU, grid-stride over chunks): of the
// read shapes tried on MI355X (lane- or block-strided, 1 to 16 loads in
// flight, with and without the streaming hint, register loads and
// global->LDS rings) this one and a contiguous LDS ring reach the highest
// rate, about 7.1 TB/s.
constexpr int kProbeLoads = 8;
constexpr int kProbeBlocksPerCu = 16;

__global__ __launch_bounds__(256) void probe_read_kernel(const u32x4_t *src, int64_t n16, uint32_t *sink) {
    constexpr int64_t kChunk = 256 * kProbeLoads;
    uint32_t acc = 0;
    for (int64_t c = blockIdx.x; c * kChunk < n16; c += gridDim.x) {
        const int64_t b = c * kChunk + threadIdx.x;
        if (c * kChunk + kChunk <= n16) {
            u32x4_t v[kProbeLoads];
#pragma unroll
            for (int u = 0; u < kProbeLoads; ++u) v[u] = __builtin_nontemporal_load(src + b + u * 256);
            __builtin_amdgcn_sched_barrier(0);      // all loads issued before the first use
#pragma unroll
            for (int u = 0; u < kProbeLoads; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
        } else {
            for (int u = 0; u < kProbeLoads; ++u)
                if (b + u * 256 < n16) {
                    const u32x4_t v = __builtin_nontemporal_load(src + b + u * 256);
                    acc ^= v.x ^ v.y ^ v.z ^ v.w;
                }
        }
    }
    acc ^= __shfl_xor(acc, 32, 64);
    acc ^= __shfl_xor(acc, 16, 64);
    acc ^= __shfl_xor(acc, 8, 64);
    acc ^= __shfl_xor(acc, 4, 64);
    acc ^= __shfl_xor(acc, 2, 64);
    acc ^= __shfl_xor(acc, 1, 64);
    // one plain store per wave: atomics from every wave of a streaming read
    // cost about a sixth of its rate on MI355X, plain stores nothing
    if ((threadIdx.x & 63) == 0) sink[(blockIdx.x * blockDim.x + threadIdx.x) >> 6] = acc;
}

__global__ __launch_bounds__(256) void probe_mfma_kernel(int iters, float *sink) {
    const int lane = threadIdx.x & 63;
    const int wave = (int)((blockIdx.x * blockDim.x + threadIdx.x) >> 6);
    bf16x8_t a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = (__bf16)(0.001f * (float)((lane + e) & 7));
        b[e] = (__bf16)(0.001f * (float)((lane * 3 + e) & 7));
    }
    f32x16_t acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[c][j] = 0.f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
    }
    float t = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int j = 0; j < 16; ++j) t += acc[c][j];
    for (int off = 32; off > 0; off >>= 1) t += __shfl_xor(t, off, 64);
    if (lane == 0) sink[wave] = t;
}

spkv_status launched(const char *what) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(SPKV_E_HIP, std::string(what) + ": " + hipGetErrorString(e));
    return SPKV_OK;
}

}  // namespace

extern "C" {

spkv_status spkv_probe_read(const void *src, size_t bytes, uint32_t *sink, int32_t sink_words, void *stream) {
    if (!src || !sink || bytes == 0 || bytes % 16 || ((uintptr_t)src & 15) || sink_words < 4)
        return fail(SPKV_E_INVAL, "probe_read: src must be 16-byte aligned, bytes a positive multiple of 16, "
                                  "sink_words >= 4");
    int cus = 0;
    if (spkv_device_cus(&cus) != SPKV_OK) return SPKV_E_HIP;
    const int64_t n16 = (int64_t)(bytes / 16);
    const int64_t chunks = (n16 + 256 * kProbeLoads - 1) / (256 * kProbeLoads);
    const int64_t blocks = std::min<int64_t>(std::min<int64_t>((int64_t)cus * kProbeBlocksPerCu, chunks),
                                             sink_words / 4);
    hipLaunchKernelGGL(probe_read_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                       (const u32x4_t *)src, n16, sink);
    return launched("probe_read_kernel");
}

spkv_status spkv_probe_mfma(int32_t waves, int32_t iters, float *sink, void *stream) {
    if (!sink || waves <= 0 || waves % 4 || iters <= 0) return fail(SPKV_E_INVAL, "probe_mfma: bad size");
    hipLaunchKernelGGL(probe_mfma_kernel, dim3((unsigned)(waves / 4)), dim3(256), 0, (hipStream_t)stream, iters, sink);
    return launched("probe_mfma_kernel");
}

}  // extern "C"
