// probe.hip -- diagnostic kernels that measure this GPU's own ceilings,
// so that measured throughput can be stated against both the data-sheet
// peaks and what a trivial kernel reaches on the same part: a streaming read
// of a device buffer (HBM) and a loop of independent bf16 matrix-core
// products (v_mfma_f32_32x32x16_bf16), and an empty kernel for the launch
// floor.  None is part of the matmul path.
#include "common.h"

namespace coli {

typedef __bf16 pr_bf16x8 __attribute__((ext_vector_type(8)));
typedef float pr_f32x16 __attribute__((ext_vector_type(16)));

// every lane reads 16-byte chunks, 8 in flight, grid-stride over the buffer;
// the xor of all words is stored only if it equals a value no input makes
// likely, which keeps the loads alive without a global reduction
__global__ __launch_bounds__(256) void k_probe_read(const u32x4 *__restrict__ buf, int64_t n16,
                                                    uint32_t never, float *sink) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    uint32_t acc = 0;
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    for (; i + 7 * stride < n16; i += 8 * stride) {
        u32x4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(buf + i + u * stride);
#pragma unroll
        for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n16; i += stride) {
        const u32x4 v = __builtin_nontemporal_load(buf + i);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (acc == never)
        sink[0] = (float)acc;
}

// each wavefront keeps 8 independent 32x32 accumulators busy for `iters`
// rounds: 8 * iters products of 32 x 32 x 16 per wavefront
__global__ __launch_bounds__(256) void k_probe_mfma(int iters, float never, float *sink) {
    pr_f32x16 acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
    pr_bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = (__bf16)(float)((threadIdx.x + e) & 7);
        b[e] = (__bf16)(float)((threadIdx.x * 3 + e) & 7);
    }
    for (int it = 0; it < iters; ++it)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[j][r];
    if (s == never)
        sink[0] = s;
}

// a kernel that does nothing: the launch floor of this GPU and runtime
// (back-to-back launches on one stream, or replayed from a graph)
__global__ __launch_bounds__(256) void k_probe_empty(float never, float *sink) {
    if (threadIdx.x == 1024)  // never: blocks have 256 threads
        sink[0] = never;
}

}  // namespace coli

using namespace coli;

extern "C" int coli_probe_read(const void *buf, size_t bytes, float *sink, void *stream) {
    if (!buf || !sink || bytes < 16 || bytes % 16 != 0 || (uintptr_t)buf % 16 != 0)
        return decline("probe_read: need a 16-byte aligned buffer of a multiple of 16 bytes "
                       "and a sink");
    hipLaunchKernelGGL(k_probe_read, dim3(4096), dim3(256), 0, (hipStream_t)stream,
                       (const u32x4 *)buf, (int64_t)(bytes / 16), 0x9E3779B9u, sink);
    return after_launch("probe_read");
}

extern "C" int coli_probe_mfma(int workgroups, int iters, float *sink, void *stream) {
    if (!sink || workgroups < 1 || iters < 1)
        return decline("probe_mfma: need workgroups >= 1, iters >= 1 and a sink");
    hipLaunchKernelGGL(k_probe_mfma, dim3((unsigned)workgroups), dim3(256), 0, (hipStream_t)stream,
                       iters, -1.2345e30f, sink);
    return after_launch("probe_mfma");
}

extern "C" int coli_probe_launch(int workgroups, float *sink, void *stream) {
    if (!sink || workgroups < 1)
        return decline("probe_launch: need workgroups >= 1 and a sink");
    hipLaunchKernelGGL(k_probe_empty, dim3((unsigned)workgroups), dim3(256), 0, (hipStream_t)stream,
                       -1.2345e30f, sink);
    return after_launch("probe_launch");
}
