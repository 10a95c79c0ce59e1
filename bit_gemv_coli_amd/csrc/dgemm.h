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
// y1 = W1 x and y2 = W2 x (single matrices of the same input count, both
// grouped int4 or both per-row int4) in one launch after one input
// preparation; workspace dgemm_ws_bytes(W1, S).  1 done, 0 not taken, <0 error
int launch_dgemm_pair(const coli_qtensor *W1, const coli_qtensor *W2, const float *x, float *y1,
                      float *y2, int S, void *ws, size_t ws_bytes, hipStream_t st);

// nb products on row ranges of one packed matrix W (a single matrix): batch
// b computes y_b[m][n] = sum_k W[row0 + b row_step + n][k] x_b[m][k] for S
// rows m and N outputs n, x_b = x + b x_bstride (rows ldx apart), y_b = y +
// b y_bstride (rows ldy apart); row0 and row_step multiples of 16.
// Workspace: dgemm_heads_ws_bytes(W, S, nb).  1 done, 0 not taken, <0 error
size_t dgemm_heads_ws_bytes(const coli_qtensor *W, int S, int nb);
// whether launch_dgemm_heads takes these shapes (pointers and workspace aside)
bool dgemm_heads_takes(const coli_qtensor *W, int row0, int row_step, int N, int nb, int S);
int launch_dgemm_heads(const coli_qtensor *W, int row0, int row_step, int N, int nb, const float *x,
                       int64_t ldx, int64_t x_bstride, float *y, int64_t ldy, int64_t y_bstride, int S,
                       void *ws, size_t ws_bytes, hipStream_t st);

}  // namespace coli
