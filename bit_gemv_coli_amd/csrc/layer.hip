// layer.hip -- the steps of a decode layer around the expert block
// (colibri-strix commit log, full decode layer commit: the post-attention RMSNorm in front of the shared expert, router
// and experts, and the residual add after them).
//   k_rmsnorm       one workgroup per row: f64 sum of squares (each thread a
//                   strided share, wavefront sums, then the four wavefronts in
//                   order), inv = 1 / sqrt(ms + eps) in f64, every output the
//                   f32 rounding of x * inv * w computed in f64;
//   k_residual_add  out = h + y elementwise (out may be h) -- where the
//                   producer of y is not a matrix-core decode kernel, which
//                   adds the residual in its own epilogue.
#include "common.h"
#include "layer.h"
#include "rms.h"

namespace coli {

template <bool VEC>
__global__ __launch_bounds__(256) void k_rmsnorm(const float *__restrict__ x, int D,
                                                 const float *__restrict__ w, double eps,
                                                 float *__restrict__ y) {
    __shared__ double part[4];
    const int t = threadIdx.x;
    const float *xr = x + (int64_t)blockIdx.x * D;
    float *yr = y + (int64_t)blockIdx.x * D;
    const double inv = row_rms_inv<VEC>(xr, D, eps, part);
    if constexpr (VEC) {
        for (int d = 4 * t; d < D; d += 1024) {
            const f32x4 v = gload<f32x4>(xr + d);
            const f32x4 g = w ? gload<f32x4>(w + d) : f32x4{1.f, 1.f, 1.f, 1.f};
            f32x4 o;
            o.x = rms_apply(v.x, inv, g.x);
            o.y = rms_apply(v.y, inv, g.y);
            o.z = rms_apply(v.z, inv, g.z);
            o.w = rms_apply(v.w, inv, g.w);
            *(f32x4 *)(yr + d) = o;
        }
    } else {
        for (int d = t; d < D; d += 256)
            yr[d] = rms_apply(xr[d], inv, w ? w[d] : 1.0f);
    }
}

__global__ __launch_bounds__(256) void k_residual_add(const float *h, const float *__restrict__ y,
                                                      float *out, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n)
        out[i] = h[i] + y[i];
}

// The two routings of a two-phase block: slot i keeps its expert in ida when
// it is resident (late[i] == 0) and in idb when it is late; the other list
// holds -1 there, which the block skips.
__global__ __launch_bounds__(256) void k_split_ids(const int32_t *__restrict__ ids,
                                                   const int32_t *__restrict__ late, int n,
                                                   int32_t *__restrict__ ida,
                                                   int32_t *__restrict__ idb) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n) {
        const int32_t e = ids[i];
        const bool l = late[i] != 0;
        ida[i] = l ? -1 : e;
        idb[i] = l ? e : -1;
    }
}

int launch_split_ids(const int32_t *ids, const int32_t *late, int n, int32_t *ida, int32_t *idb,
                     hipStream_t st) {
    ProfScope ps("split_ids", st);
    hipLaunchKernelGGL(k_split_ids, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, ids, late,
                       n, ida, idb);
    return after_launch("split_ids");
}

int launch_rmsnorm(const float *x, int S, int D, const float *w, double eps, float *y,
                   hipStream_t st) {
    ProfScope ps("rmsnorm", st);
    const bool vec = D % 4 == 0 && (uintptr_t)x % 16 == 0 && (uintptr_t)y % 16 == 0 &&
                     (uintptr_t)w % 16 == 0;
    if (vec)
        hipLaunchKernelGGL(k_rmsnorm<true>, dim3((unsigned)S), dim3(256), 0, st, x, D, w, eps, y);
    else
        hipLaunchKernelGGL(k_rmsnorm<false>, dim3((unsigned)S), dim3(256), 0, st, x, D, w, eps, y);
    return after_launch("rmsnorm");
}

int launch_residual_add(const float *h, const float *y, float *out, int64_t n, hipStream_t st) {
    ProfScope ps("residual_add", st);
    hipLaunchKernelGGL(k_residual_add, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, h, y,
                       out, n);
    return after_launch("residual_add");
}

}  // namespace coli
