// rms.h -- the RMSNorm reduction shared by the norm kernel and the router
// that folds the norm in: both must reach the same 1 / rms bit for bit.
#pragma once
#include "common.h"

namespace coli {

__device__ __forceinline__ double rms_shfl_xor(double v, int m) {
    const int2 p = __builtin_bit_cast(int2, v);
    int2 q;
    q.x = __shfl_xor(p.x, m);
    q.y = __shfl_xor(p.y, m);
    return __builtin_bit_cast(double, q);
}

// inv = 1 / sqrt(sum x^2 / D + eps) of one row, in f64, by a workgroup of
// 256 threads in one fixed order: each thread a strided share (VEC: four
// consecutive inputs in every 1024), wavefront butterfly sums, then the four
// wavefronts' sums in order.  part: 4 doubles of LDS for this row; every
// thread returns inv.  Contains a workgroup barrier.
template <bool VEC>
__device__ __forceinline__ double row_rms_inv(const float *__restrict__ xr, int D, double eps,
                                              double *part) {
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    double ss = 0.0;
    if constexpr (VEC) {
        for (int d = 4 * t; d < D; d += 1024) {
            const f32x4 v = gload<f32x4>(xr + d);
            ss = fma((double)v.x, (double)v.x, ss);
            ss = fma((double)v.y, (double)v.y, ss);
            ss = fma((double)v.z, (double)v.z, ss);
            ss = fma((double)v.w, (double)v.w, ss);
        }
    } else {
        for (int d = t; d < D; d += 256) ss = fma((double)xr[d], (double)xr[d], ss);
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) ss += rms_shfl_xor(ss, m);
    if (lane == 0)
        part[wv] = ss;
    __syncthreads();
    const double tot = ((part[0] + part[1]) + part[2]) + part[3];
    return 1.0 / sqrt(tot / (double)D + eps);
}

// one normalised input: the f32 rounding of x * inv * w, computed in f64
__device__ __forceinline__ float rms_apply(float x, double inv, float w) {
    return (float)((double)x * inv * (double)w);
}

}  // namespace coli
