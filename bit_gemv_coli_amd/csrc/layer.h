// layer.h -- launchers of the decode-layer steps around the expert block
// (layer.hip): the per-row RMSNorm, the residual add and the routing split of
// the two-phase block.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace coli {

int launch_rmsnorm(const float *x, int S, int D, const float *w, double eps, float *y,
                   hipStream_t st);
int launch_residual_add(const float *h, const float *y, float *out, int64_t n, hipStream_t st);
int launch_split_ids(const int32_t *ids, const int32_t *late, int n, int32_t *ida, int32_t *idb,
                     hipStream_t st);

}  // namespace coli
