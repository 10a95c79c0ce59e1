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

// The input preparation's layout: the 8 inputs x[m][k .. k + 7] (k a
// multiple of 8) as bf16 (round to nearest even, v_cvt_pk_bf16_f32) at this
// byte offset of a batch's preparation; nkb4 = the 128-input blocks rounded
// up to a multiple of 4; rows up to whole 144-row tiles, inputs up to nkb4
// blocks (inputs past K must be zero, rows past S may hold anything: their
// outputs are not written).
__host__ __device__ inline int64_t dgemm_frag_offset(int m, int k, int nkb4) {
    const int kb = k / 128, c8 = (k % 128) / 8;
    return ((int64_t)(m / 16) * nkb4 + kb) * 4096 + (c8 & 3) * 1024 + (16 * (c8 >> 2) + m % 16) * 16;
}
inline int dgemm_nkb4(const coli_qtensor *W) { return ((W->I + 127) / 128 + 3) / 4 * 4; }
__device__ __forceinline__ uint32_t dgemm_bf16x2(float lo, float hi) {
    uint32_t r;
    asm("v_cvt_pk_bf16_f32 %0, %1, %2" : "=v"(r) : "v"(lo), "v"(hi));
    return r;
}

// nb products on row ranges of one packed matrix W (a single matrix): batch
// b computes y_b[m][n] = sum_k W[row0 + b row_step + n][k] x_b[m][k] for S
// rows m and N outputs n, x_b = x + b x_bstride (rows ldx apart), y_b = y +
// b y_bstride (rows ldy apart); row0 and row_step multiples of 16.
// Workspace: dgemm_heads_ws_bytes(W, S, nb), batch b's input preparation at
// b dgemm_ws_bytes(W, S); with prepared, the caller has written it there
// already (x unused).  1 done, 0 not taken, <0 error
size_t dgemm_heads_ws_bytes(const coli_qtensor *W, int S, int nb);
// whether launch_dgemm_heads takes these shapes (pointers and workspace aside)
bool dgemm_heads_takes(const coli_qtensor *W, int row0, int row_step, int N, int nb, int S);
int launch_dgemm_heads(const coli_qtensor *W, int row0, int row_step, int N, int nb, const float *x,
                       int64_t ldx, int64_t x_bstride, float *y, int64_t ldy, int64_t y_bstride, int S,
                       void *ws, size_t ws_bytes, hipStream_t st, bool prepared = false);

}  // namespace coli
