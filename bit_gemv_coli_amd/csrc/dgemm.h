// dgemm.h -- the split-K prefill GEMM for packed int4 tensors (dgemm.hip)
#pragma once
#include "common.h"

namespace coli {

// workspace bytes for (W, S): the input rows as bf16 fragments, rows padded
// to whole 144-row tiles and inputs to whole groups of four 128-input
// blocks; 0 when the kernel does not take W
size_t dgemm_ws_bytes(const coli_qtensor *W, int S);
// y = W x for S input rows with the inputs prepared in ws; 1 done, 0 not
// taken (layout, alignment, workspace), <0 error
int launch_dgemm(const coli_qtensor *W, const float *x, float *y, int S, void *ws, size_t ws_bytes,
                 hipStream_t st);

}  // namespace coli
