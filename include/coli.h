/*
 * coli.h -- C ABI of the MI355X (gfx950) quantized-weight matmul library
 * (libcoli.so): the colibri engine's quantized matmul and batched MoE expert
 * block, as hand-written HIP kernels.
 *
 * Sources (pages describing the colibri engine; cited as in every file):
 *   colibri PR #298, commit adding fmt=4 to the CUDA backend  -- grouped int4:
 *       fmt=2 nibble layout plus one f32 scale per gs inputs along I, folded in
 *       per group during accumulation; tensor upload takes gs and sizes the
 *       scale buffer O*ceil(I/gs).
 *   colibri PR #298, commit adding the matmul_i4_grouped test -- offset
 *       nibbles (0x0 -> -8, 0xF -> +7), partial last group, tolerances judged
 *       against the sum of |terms|.
 *   colibri PR #298, commit adding fmt=4 to the Metal mm_gemv -- fmt 1-3 scale
 *       once per row after the dot product; fmt 4 per group.
 *   colibri PR #298, commit making the CUDA ABI return 0 for fmt=4 -- an entry
 *       that cannot honour its input returns 0: a declined call is a fallback, not a wrong result.
 *   colibri-strix commit log, batched expert-block commit -- gate/up -> SiLU -> down for a whole expert block in one
 *       submission, ragged per-row routing, weighted scatter-add.
 *   colibri-strix commit log, shared-expert fusion commit -- the shared
 *       expert joins the block as an extra expert with weight 1.0 on every row.
 *   colibri-strix commit log, prefill GEMM routing commit
 *       -- large row batches (prefill) take a GEMM path, small ones a GEMV.
 *
 * Conventions shared by every entry point
 *   Return value: COLI_OK (1) work validated and enqueued on `stream`;
 *   COLI_DECLINED (0) the call cannot be honoured (unknown or unsupported
 *   format, group size, shape, NULL or misaligned pointer, workspace too small,
 *   fault injection tripped): NOTHING was written or enqueued, and
 *   coli_last_reason() says why; COLI_HIP_ERROR (-1) the HIP runtime reported
 *   an error (coli_last_error()).
 *   Memory: every data pointer is a DEVICE pointer owned by the caller (for
 *   example a torch tensor's data_ptr()); the library allocates and frees no
 *   device memory in these calls and keeps no pointer past the call, except
 *   that enqueued kernels read/write the buffers until they complete.
 *   Streams: `stream` is a hipStream_t (NULL = the null stream).  All work is
 *   asynchronous; the caller synchronises.
 *   Layouts are row-major and dense.  Activations and outputs are f32.
 *   Reentrancy: calls on different streams may overlap; a workspace must not be
 *   shared by two calls that may run at the same time.
 */
#ifndef COLI_H
#define COLI_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define COLI_OK 1
#define COLI_DECLINED 0
#define COLI_HIP_ERROR (-1)

/* Weight formats (colibri's QT fmt codes). */
#define COLI_FMT_I8_ROW 1  /* int8 two's complement, one f32 scale per row      */
#define COLI_FMT_I4_ROW 2  /* int4 offset (nibble-8), one f32 scale per row     */
#define COLI_FMT_I2_ROW 3  /* int2 offset (code-2), one f32 scale per row       */
#define COLI_FMT_I4_GRP 4  /* int4 offset, one f32 scale per gs inputs (groups) */

/*
 * A quantized matrix, or a stack of n equally shaped matrices (experts).
 * Filled and validated by coli_tensor_upload; treat the fields as read-only.
 *
 * Codes q: bytes [n][O][row_bytes], each row starting on a byte boundary:
 *   fmt 1: row_bytes = I,         byte i = int8 value v
 *   fmt 2/4: row_bytes = ceil(I/2), element i in byte i/2, LOW nibble for even
 *            i, high nibble for odd i; v = nibble - 8 (0x0 -> -8, 0xF -> +7)
 *   fmt 3: row_bytes = ceil(I/4), element i in byte i/4 at bits 2*(i%4)..+1;
 *          v = code - 2
 * Scales s: f32 [n][O] for fmt 1-3; f32 [n][O][ng] for fmt 4 with
 *   ng = ceil(I/gs), group g covering inputs [g*gs, min((g+1)*gs, I)).
 * Weight value: w(o,i) = s[o] * v (fmt 1-3), s[o][i/gs] * v (fmt 4).
 */
typedef struct coli_qtensor {
    int32_t fmt;
    int32_t n;         /* matrices in the stack, >= 1                       */
    int32_t O, I;      /* rows (outputs) and inputs of each matrix          */
    int32_t gs;        /* fmt 4: inputs per scale group; fmt 1-3: 0         */
    int32_t ng;        /* fmt 4: ceil(I/gs); fmt 1-3: 1                     */
    int64_t row_bytes; /* bytes per row of codes                            */
    int64_t q_stride;  /* bytes between matrices   = O * row_bytes          */
    int64_t s_stride;  /* floats between matrices  = O * ng                 */
    const void *q;     /* device codes                                      */
    const float *s;    /* device scales                                     */
    uint32_t magic;    /* set by coli_tensor_upload                         */
    uint32_t flags;    /* internal: which kernel paths the layout allows    */
    /* Optional repacked copy (coli_tensor_pack); NULL until packed.  The
     * matrix-core decode kernels read it instead of q/s. */
    const void *pk;    /* device: packed codes and scales                   */
    int64_t pk_stride; /* bytes between matrices in the packed copy         */
    int64_t pk_scale_off; /* byte offset of the packed scales within pk     */
} coli_qtensor;

/*
 * coli_tensor_upload -- describe caller-owned device codes and scales as a
 * quantized tensor (colibri PR #298, CUDA fmt=4 commit: the grouped upload
 * takes gs and allocates O*ceil(I/gs) scales; the per-row upload is gs=0).
 *   t      host record to fill (written only on success)
 *   fmt    1..4;  n >= 1;  O, I >= 1
 *   gs     fmt 4: group size >= 1 (any value; multiples of 16 take the fast
 *          kernels, others a slower exact path); fmt 1-3: must be 0
 *   ng     fmt 4: must equal ceil(I/gs); fmt 1-3: must be 1
 *   q_dev, s_dev  device pointers (non-NULL); nothing is copied -- the record
 *          refers to the caller's buffers, which must outlive its use.
 * Returns COLI_OK or COLI_DECLINED (bad fmt, gs, ng, shape or NULL pointer).
 * Launches nothing.
 */
int coli_tensor_upload(coli_qtensor *t, int fmt, int n, int O, int I, int gs, int ng,
                       const void *q_dev, const float *s_dev);

/*
 * coli_packed_bytes -- device bytes the repacked copy of a tensor of this
 * shape needs (0 when the format / layout has no packed form: packing needs
 * I % 32 == 0, and for fmt 4 gs of 32, 64 or a multiple of 128).
 */
size_t coli_packed_bytes(int fmt, int n, int O, int I, int gs);

/*
 * coli_tensor_pack -- write a repacked copy of the tensor's codes (and fmt-4
 * scales) into caller-owned device memory and attach it to the record; an
 * upload-time layout conversion in the spirit of the pages' upload-time
 * offset_to_signed_s4 (colibri PR #298, CUDA fmt=4 commit).  Layout: every
 * 16-row x 128-input tile becomes one contiguous block in the order the
 * matrix-core decode kernels load it (so each wavefront load is one request):
 * fmt 2 / 4 1 KiB of two's-complement nibbles q - 8; fmt 1 2 KiB of the int8
 * codes, each lane's 32 inputs as the 16 even ones then the 16 odd ones;
 * fmt 3 512 bytes of two's-complement 2-bit values q - 2 in the same
 * even / odd split.  The fmt-4 group scales follow, one run per (tile, 4
 * blocks, row) so a lane fetches a whole batch's scales at once (per-row
 * scales stay in the original s); rows and inputs past O and I are padded
 * with zero weights.  The represented weights are unchanged.  Only fmt 2 / 4
 * packed copies serve the MoE block and the prefill kernels; fmt 1 / 3
 * packed copies serve coli_qmatmul and coli_qmatmul_group at S <= 4.
 *   t         record from coli_tensor_upload (updated on success)
 *   packed    device buffer of at least coli_packed_bytes(...) bytes, 256-byte
 *             aligned, owned by the caller, kept alive while t is used
 * The original q/s must stay valid too (other kernels read them).  Packing is
 * enqueued on `stream`; calls on other streams must be ordered after it.
 * Returns COLI_OK, COLI_DECLINED (no packed form, small or misaligned buffer)
 * or COLI_HIP_ERROR.
 */
int coli_tensor_pack(coli_qtensor *t, void *packed, size_t bytes, void *stream);

/*
 * coli_qmatmul -- y = W x for every matrix of the stack
 * (colibri PR #298 commits: fmt 4 folds the group scale in per group, fmt 1-3
 * scale once per row; colibri-strix prefill GEMM routing commit: large row batches take the GEMM path).
 *   W   tensor from coli_tensor_upload (n matrices [O][I])
 *   x   device f32 [S][I]          y   device f32 [n][S][O]
 *   S   >= 1 input rows.  S <= coli_gemv_max_rows() (default 4) runs the
 *       fp32 GEMV kernels; larger S runs the bf16 matrix-core GEMM (weights
 *       and x rounded to bf16, fp32 accumulation; error <= 4e-3 * A per
 *       output, A = sum_i |w_i||x_i|).
 *       Decode error (S <= 4), per output:
 *         vector-ALU kernels (no packed copy, or coli_set_decode_kernel(1)):
 *           <= 1e-5 * A -- they multiply the f32 inputs themselves;
 *         matrix-core kernels (tensors with a packed copy):
 *           <= 1e-5 * A + 2^-29 * Ahat,
 *           Ahat = sum over the 128-input blocks b of the row of
 *                  max(max_{i in b} |x_i|, 2^-97) * sum_{i in b} |w_i|.
 *         The matrix-core kernels hold each (input row, 128-input block) as
 *         integers under one power of two, so an input's resolution is
 *         2^-29 of its block's largest |x|.  For activations like the
 *         workloads' N(0,1) inputs Ahat is a few times A and the term is
 *         ~1e-8 A; an input ~1e6 times larger than the rest of its block at
 *         a column whose weights are zero makes it exceed 1e-5 A.  Callers
 *         whose inputs have such outliers take the vector-ALU kernels.
 * x and y must not overlap.  Returns COLI_OK / COLI_DECLINED / COLI_HIP_ERROR.
 */
int coli_qmatmul(const coli_qtensor *W, const float *x, float *y, int S, void *stream);

/*
 * coli_qmatmul_ws -- coli_qmatmul with a caller workspace, for prefill rows
 * (same pages as coli_qmatmul: large row batches take a GEMM path).
 *   workspace  device buffer of at least coli_qmatmul_workspace_bytes(W, S)
 *              bytes, 256-byte aligned, not shared with a call that may run
 *              at the same time; contents on entry do not matter
 * For S > coli_gemv_max_rows() on a packed int4 tensor (fmt 2, or fmt 4
 * with groups of 32, 64 or multiples of 128) the input rows are first
 * rounded to bf16 into the workspace in the order the matrix cores read
 * them; then every 144 x 96 output tile runs on one workgroup whose four
 * wavefronts each sum a quarter of every 128 inputs, the quarters added in a
 * fixed order.  Same bound as the GEMM of coli_qmatmul (weights bf16(s (q -
 * 8)), x bf16, fp32 accumulation: error <= 4e-3 * A); results are repeatable
 * but not bit-identical to coli_qmatmul's (another summation order).  Any
 * other case -- decode rows, no packed copy, workspace NULL or too small --
 * runs exactly as coli_qmatmul.  Returns COLI_OK / COLI_DECLINED /
 * COLI_HIP_ERROR.
 */
int coli_qmatmul_ws(const coli_qtensor *W, const float *x, float *y, int S, void *workspace,
                    size_t ws_bytes, void *stream);
/* Workspace bytes coli_qmatmul_ws uses for (W, S); 0 when it uses none. */
size_t coli_qmatmul_workspace_bytes(const coli_qtensor *W, int S);

/*
 * coli_qmatmul_group -- y[g] = W[g] x[g] for n independent matrices in one
 * submission (colibri-strix commit log, full decode layer commit: the projections of a layer go to the GPU together, not one
 * dispatch each).  Each member is computed exactly as coli_qmatmul computes it
 * (same kernels, same bounds, bit-identical results); members need not share
 * shapes.
 *   n      1 .. COLI_GROUP_MAX members
 *   W[g]   tensor from coli_tensor_upload (for one launch: a single matrix
 *          with a packed copy, all members the same fmt, fmt-4 members with
 *          the same scale slots per 128 inputs; otherwise the members run one
 *          launch each, still in this call)
 *   x[g]   device f32 [S][I_g]      y[g]   device f32 [n_g][S][O_g]
 *   S      >= 1 input rows, the same for all members
 * The host arrays W, x, y are read during the call only.  Members' outputs
 * must not overlap each other or any input.  Every member is validated
 * before anything is enqueued.  Returns COLI_OK / COLI_DECLINED /
 * COLI_HIP_ERROR.
 */
#define COLI_GROUP_MAX 8
int coli_qmatmul_group(int n, const coli_qtensor *const *W, const float *const *x,
                       float *const *y, int S, void *stream);

/* Largest S served by the fp32 GEMV path (env COLI_GEMV_MAX_ROWS, 1..4). */
int coli_gemv_max_rows(void);
/* Set it (1..4); returns the previous value, or 0 if the value is refused. */
int coli_set_gemv_max_rows(int s);

/* Kernel family of the fp32 decode path: 0 (default) uses the matrix-core
 * decode kernels for tensors that carry a packed copy (coli_tensor_pack) and
 * the vector-ALU kernels elsewhere; 1 uses the vector-ALU kernels everywhere
 * (error <= 1e-5 * A whatever the inputs' spread; the matrix-core kernels add
 * up to 2^-29 * Ahat, see coli_qmatmul).
 * Environment: COLI_DECODE_KERNEL=valu.  Returns the previous mode, -1 if
 * `mode` is refused. */
int coli_set_decode_kernel(int mode);

/*
 * coli_dequantize -- w_out[e][o][i] = (float)(s * v), the exact product
 * rounded once to f32 (test hook; bit-exact with the oracle).
 *   w_out  device f32 [n][O][I].  Returns COLI_OK / COLI_DECLINED / -1.
 */
int coli_dequantize(const coli_qtensor *W, float *w_out, void *stream);

/*
 * coli_moe_route -- the block's routing table (colibri-strix "batched
 * moe_block": per-row ragged expert routing).
 *   ids     device int32 [S][K] expert ids; ids outside [0,E) are left out
 *   counts  device int32 [E]     pairs routed to each expert
 *   offsets device int32 [E+1]   exclusive prefix sum; offsets[E] = valid pairs
 *   perm    device int32 [S*K]   valid pair indices p = s*K+k grouped by
 *           ascending expert, ascending p within an expert; entries past
 *           offsets[E] are set to -1
 *   n_bad   device int32 [1]     number of ids outside [0,E)
 * Limits: 1 <= E <= 4096, K >= 1, S >= 0.  Bit-exact with the oracle.
 */
int coli_moe_route(const int32_t *ids, int S, int K, int E, int32_t *counts,
                   int32_t *offsets, int32_t *perm, int32_t *n_bad, void *stream);

/*
 * coli_moe_block -- the batched MoE expert block in one submission
 * (colibri-strix "batched moe_block": gate/up -> SiLU -> down per expert, then
 * the weighted combine; shared-expert fusion commit: the shared expert adds with
 * weight 1.0 on every row):
 *   out[s] = sum_k w[s][k] * D_e (silu(G_e x_s) * (U_e x_s)),  e = ids[s][k]
 *            + D_sh (silu(G_sh x_s) * (U_sh x_s))            (if given)
 *   gate, up   stacks of E matrices [F][Dm]   (same fmt and gs)
 *   down       stack of E matrices [Dm][F]
 *   x          device f32 [S][Dm];  ids device int32 [S][K];  w device f32 [S][K]
 *   sh_gate, sh_up, sh_down  all NULL, or one matrix each with the routed
 *              stacks' shapes, fmt and gs (a group-size mix is declined)
 *   out        device f32 [S][Dm] (overwritten)
 *   workspace  device buffer of at least coli_moe_workspace_bytes(...) bytes,
 *              256-byte aligned
 * Routing weights are used as given (no renormalisation).  Pairs whose id lies
 * outside [0,E) contribute nothing (their count is reported by
 * coli_moe_route); duplicate ids in a row are independent terms.  The combine
 * adds k in ascending order with no atomics, so reruns are bit-identical.
 * S <= coli_gemv_max_rows() runs fp32 GEMV kernels (packed stacks: the
 * matrix-core kernels, each GEMV within the coli_qmatmul bound, with x as the
 * input of gate/up and h as the input of down); larger S runs bf16
 * matrix-core grouped GEMMs over the routing table.
 * Limits: 1 <= E <= 4096, 1 <= K <= 64, S >= 1.
 */
int coli_moe_block(const coli_qtensor *gate, const coli_qtensor *up, const coli_qtensor *down,
                   const float *x, int S, const int32_t *ids, const float *w, int K,
                   const coli_qtensor *sh_gate, const coli_qtensor *sh_up,
                   const coli_qtensor *sh_down, float *out, void *workspace,
                   size_t ws_bytes, void *stream);

/*
 * coli_moe_hidden -- the first half of coli_moe_block on its own (test hook):
 * h[p] = silu(G_e x_s) * (U_e x_s) for routed pair p = s*K+k (zero when the id
 * is out of range), then h[S*K+s] for the shared expert when given.
 *   h_out  device f32 [S*K (+S)][F].  Same kernels, precision and workspace
 *          rules as coli_moe_block with the same S.
 */
int coli_moe_hidden(const coli_qtensor *gate, const coli_qtensor *up, const float *x, int S,
                    const int32_t *ids, int K, const coli_qtensor *sh_gate,
                    const coli_qtensor *sh_up, float *h_out, void *workspace,
                    size_t ws_bytes, void *stream);

/* Workspace bytes coli_moe_block / coli_moe_hidden need (0 on bad input). */
size_t coli_moe_workspace_bytes(int E, int S, int K, int F, int Dm, int has_shared);

/*
 * coli_moe_block_begin / coli_moe_block_end -- the expert block in two
 * submissions (colibri-strix commit log, disk/GPU overlap commit: the resident experts and the shared expert go
 * to the GPU first, the experts still being loaded follow in a second submit
 * once they are in place).  Here a slot (s, k) is late when late[s][k] != 0:
 * begin computes out = the block over the resident slots (+ the shared
 * expert); end, enqueued once the late experts' weights are in the stacks,
 * adds the block over the late slots:
 *     out[s] = (sum_{k resident} w y + shared) + (sum_{k late} w y)
 * each sum in ascending k (deterministic; the same value as coli_moe_block up
 * to the order of that one extra addition, within the same bounds).
 *   begin: arguments as coli_moe_block plus late, device int32 [S][K];
 *   end:   the same tensors, x, S, w, K, whether begin had a shared expert,
 *          and out as written by begin.
 *   workspace: device memory of coli_moe_block_two_phase_workspace_bytes(E,
 *   S, K, F, D, has_shared) bytes, 256-byte aligned, the same buffer for both
 *   calls (begin leaves the late slots' routing in it) and not used by
 *   anything else in between.  Both calls on one stream, or ordered.
 * Returns COLI_OK, COLI_DECLINED (as coli_moe_block, NULL late) or
 * COLI_HIP_ERROR.
 */
size_t coli_moe_block_two_phase_workspace_bytes(int E, int S, int K, int F, int Dm, int has_shared);
int coli_moe_block_begin(const coli_qtensor *gate, const coli_qtensor *up, const coli_qtensor *down,
                         const float *x, int S, const int32_t *ids, const float *w, int K,
                         const int32_t *late, const coli_qtensor *sh_gate,
                         const coli_qtensor *sh_up, const coli_qtensor *sh_down, float *out,
                         void *workspace, size_t ws_bytes, void *stream);
int coli_moe_block_end(const coli_qtensor *gate, const coli_qtensor *up, const coli_qtensor *down,
                       const float *x, int S, const float *w, int K, int has_shared, float *out,
                       void *workspace, size_t ws_bytes, void *stream);

/*
 * coli_moe_block_noalloc -- coli_moe_block for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation): the same block, same kernels and results, with the
 * library's own static device scratch in place of the caller's workspace.
 * Arguments as coli_moe_block without workspace / ws_bytes; the caller still
 * passes x, ids, w and out.
 *   Limit: blocks whose coli_moe_workspace_bytes(...) exceeds
 *   COLI_NOALLOC_SCRATCH_BYTES are declined (COLI_DECLINED, nothing written;
 *   the decode shapes of the pages' model -- S <= 4, K = 8, F = 2048,
 *   D = 6144, shared expert -- need about 1.2 MB).
 *   The scratch is one static array per GPU, held by every GPU the library
 *   runs on until the process ends; it keeps the last call's contents (the
 *   block clears what must start at zero itself).  Calls that may overlap on
 *   one GPU (other streams, other threads) race on it: serialise them.
 *   Allocates nothing (no hipMalloc / hipFree; the scratch address is looked
 *   up once per device on the first call there).
 * Returns COLI_OK, COLI_DECLINED or COLI_HIP_ERROR.
 */
#define COLI_NOALLOC_SCRATCH_BYTES (8u << 20)
int coli_moe_block_noalloc(const coli_qtensor *gate, const coli_qtensor *up,
                           const coli_qtensor *down, const float *x, int S, const int32_t *ids,
                           const float *w, int K, const coli_qtensor *sh_gate,
                           const coli_qtensor *sh_up, const coli_qtensor *sh_down, float *out,
                           void *stream);

/* ---------------------------------------------------------------------- */
/* Diagnostics (colibri PR #298, HIP single-source merge: a fault-injection */
/* control proves GPU calls really executed; issue #585: fallbacks must be  */
/* loud).                                                                   */
/* ---------------------------------------------------------------------- */

/*
 * coli_moe_router -- the router in front of the expert block and its exact
 * top-K selection (colibri-strix commit log, full decode layer commit: router matvec + sigmoid, greedy argmax over sigmoid + bias
 * with the CPU's tie order, top-p truncation, norm_topk, routed_scale).
 *   x    f32 [S][D] input rows;  R  f32 [E][D] router weights (row-major);
 *   bias f32 [E] added to the sigmoid score for the choice only (NULL: none);
 *   for each row: z = R x (exact f64 products, f64 sums), p = 1/(1+exp(-z)),
 *   K greedy picks of the largest p + bias, the smaller expert index among
 *   equal keys; 0 < topp < 1 keeps the picks up to and including the first at
 *   which the running sum of p reaches topp times the sum over the K picks
 *   (topp 0 or 1 keeps all); weights = p of the kept picks, divided by their
 *   sum when norm_topk != 0, times routed_scale;
 *   ids i32 [S][K] in pick order (dropped slots -1), w f32 [S][K] (dropped 0);
 *   workspace: device memory of coli_moe_router_workspace_bytes(S, E) bytes,
 *   8-byte aligned, caller-owned, contents undefined between calls.
 * ids and w feed coli_moe_block directly.  Limits: 1 <= E <= 512,
 * 1 <= K <= min(16, E).  Returns COLI_OK, COLI_DECLINED (bad sizes, NULL
 * pointers, small workspace, topp outside [0,1]) or COLI_HIP_ERROR.
 */
size_t coli_moe_router_workspace_bytes(int S, int E);
int coli_moe_router(const float *x, int S, int D, const float *R, const float *bias, int E, int K,
                    float topp, int norm_topk, float routed_scale, int32_t *ids, float *w,
                    void *workspace, size_t ws_bytes, void *stream);

/*
 * coli_rmsnorm -- per-row RMSNorm (colibri-strix commit log, full decode layer commit: the post-attention norm in front of
 * the shared expert and the router; the pages name the step only, the usual
 * root-mean-square norm with a per-feature weight is taken):
 *   y[s][d] = x[s][d] / sqrt(mean_d x[s][d]^2 + eps) * w[d]
 * with the mean of squares and the product in f64 and one rounding to f32.
 *   x, y  f32 [S][D] device rows (y may equal x); w f32 [D] or NULL (ones);
 *   eps   finite, >= 0.
 * Returns COLI_OK, COLI_DECLINED (NULL x/y, bad sizes, bad eps) or
 * COLI_HIP_ERROR.
 */
int coli_rmsnorm(const float *x, int S, int D, const float *w, float eps, float *y, void *stream);

/*
 * coli_moe_layer -- the expert half of a decode layer in one submission
 * (colibri-strix commit log, full decode layer commit: post-attention norm, shared expert, router with the exact top-K,
 * routed experts, then the residual add), for S >= 1 rows:
 *   xn      = coli_rmsnorm(h, ln_w, eps)                   (kept in workspace)
 *   ids, w  = coli_moe_router(xn, R, bias, K, topp, norm_topk, routed_scale)
 *   out     = h + coli_moe_block(xn, ids, w; shared expert if given)
 * Arguments as in those calls: gate/up/down are the expert stacks (E = gate's
 * matrix count, F its rows, D its columns), R f32 [E][D], h and out f32
 * [S][D] (out may equal h: the add is elementwise and last).  ln_w, bias and
 * the shared expert (all three or none) may be NULL.  Limits: the block's
 * (one fmt and gs, whole 16-byte packets) and the router's (E <= 512,
 * K <= min(16, E)).
 *   workspace: device memory of coli_moe_layer_workspace_bytes(E, S, K, F, D,
 *   has_shared) bytes, 256-byte aligned, caller-owned, contents undefined
 *   between calls.  Everything is validated before the first launch; nothing
 *   is allocated and the host never waits, so the call can be captured in a
 *   graph.
 * Returns COLI_OK, COLI_DECLINED or COLI_HIP_ERROR.
 */
size_t coli_moe_layer_workspace_bytes(int E, int S, int K, int F, int D, int has_shared);
int coli_moe_layer(const coli_qtensor *gate, const coli_qtensor *up, const coli_qtensor *down,
                   const float *h, int S, const float *ln_w, float eps, const float *R,
                   const float *bias, int K, float topp, int norm_topk, float routed_scale,
                   const coli_qtensor *sh_gate, const coli_qtensor *sh_up,
                   const coli_qtensor *sh_down, float *out, void *workspace, size_t ws_bytes,
                   void *stream);

/*
 * Decode attention of one MLA layer (colibri-strix commit log: the fused
 * decode attention commit (Phase 2) runs q_a -> RMSNorm -> q_b -> RoPE, kv_a ->
 * RMSNorm of the latent and RoPE of the rotary key written to the latent and
 * rotary caches, the absorption core (qabs, score, softmax, clat, ctx) and
 * o_proj in one submission; the S <= 4 commit after it gives every step a
 * query-row dimension, row s attending keys [0, pos_base + s]; issue #585
 * thread: kv_b is grouped int4 on that path).
 *
 * Dimensions (the pages compile them in without printing them; the reading
 * here takes them from the layer's projection shapes): D hidden, qr = q_a
 * rows, L latent width, H heads of d_nope + d_rope query components and d_v
 * value components:
 *   q_a [qr][D]   q_b [H (d_nope + d_rope)][qr], head h's rows h (d_nope +
 *                 d_rope) + j, the d_nope position-free ones first
 *   kv_a [L + d_rope][D]: the latent, then the rotary key shared by all heads
 *   kv_b [H (d_nope + d_v)][L]: head h's d_nope key rows, then its d_v value
 *                 rows                       o_proj [D][H d_v]
 *   q_norm [qr], kv_norm [L]: f32 RMSNorm weights (NULL: ones)
 * RoPE turns consecutive pairs (2i, 2i+1) by pos * rope_theta^(-2i/d_rope);
 * RMSNorm is x / sqrt(mean x^2 + eps) * w; the softmax scale is
 * 1/sqrt(d_nope + d_rope).  All five matrices are single coli_qtensors (any
 * format for the projections; kv_b fmt 4 with gs % 8 == 0, or fmt 2, latent
 * width L a multiple of 32 up to 4096, codes 16-byte aligned).
 */
typedef struct coli_mla_layer {
    const coli_qtensor *q_a, *q_b, *kv_a, *kv_b, *o_proj;
    const float *q_norm, *kv_norm;
    int32_t H, d_nope, d_rope, d_v;
    float eps, rope_theta;
} coli_mla_layer;

#define COLI_MLA_STAGES 10
/* Most query rows one coli_mla_decode / coli_layer_decode call takes. */
#define COLI_MLA_MAX_ROWS 4096
/* Workspace bytes of coli_mla_decode for S rows and caches of T_cap rows
 * (0 on bad input). */
size_t coli_mla_workspace_bytes(const coli_mla_layer *layer, int S, int T_cap);
/* Where each step leaves its result in that workspace (for inspection after
 * the call): byte offsets of f32 arrays, in order cq_raw [S][qr], ckv_raw
 * [S][L + d_rope], cq [S][qr], q [S][H (d_nope + d_rope)], qabs [S][H][L],
 * qpe [S][H][d_rope] (rotated), scores [S][H][T_cap] (scaled, keys 0 ..
 * pos_base + s), p [S][H][T_cap], clat [S][H][L], ctx [S][H d_v].  Returns
 * the total bytes (0 on bad input). */
size_t coli_mla_workspace_layout(const coli_mla_layer *layer, int S, int T_cap,
                                 size_t offsets[COLI_MLA_STAGES]);
/*
 * coli_mla_decode -- the attention for S = 1..COLI_MLA_MAX_ROWS rows x [S][D]
 * at positions pos_base .. pos_base + S - 1 (S <= 4: decode; more rows:
 * prefill, the same steps for every row, row s attending keys 0 ..
 * pos_base + s):
 *   writes cache rows Lc[pos_base + s] (f32 [T_cap][L]) and Rc[pos_base + s]
 *   (f32 [T_cap][d_rope]); reads rows 0 .. pos_base + s for row s (rows below
 *   pos_base are the earlier tokens', supplied by the caller);
 *   out f32 [S][D] = o_proj ctx.
 * Requires pos_base >= 0 and pos_base + S <= T_cap.  The projections run
 * coli_qmatmul's kernels with its bounds (S <= 4: the fp32 decode GEMVs;
 * more rows: the bf16 prefill GEMMs).  The core is fp32; for more than 4
 * rows it runs on the fp32 matrix cores after every row's cache rows are
 * written, in groups of at most 192 rows, and with a packed kv_b whose head
 * blocks are whole 16-row tiles the value absorption runs on the bf16
 * prefill GEMM (its bound).  Nothing is allocated and the host never waits
 * (graph-capturable).  x, out, Lc, Rc and the workspace must not overlap.
 *   workspace: coli_mla_workspace_bytes(layer, S, T_cap) bytes, 256-byte
 *   aligned, caller-owned; its stage arrays hold this call's intermediates.
 * Returns COLI_OK, COLI_DECLINED or COLI_HIP_ERROR.
 */
int coli_mla_decode(const coli_mla_layer *layer, const float *x, int S, int pos_base, float *Lc,
                    float *Rc, int T_cap, float *out, void *workspace, size_t ws_bytes,
                    void *stream);

/*
 * coli_layer_decode -- a whole decode layer in one submission (colibri-strix
 * commit log, full decode layer commit: in_ln RMSNorm -> fused attention ->
 * residual add -> post_ln RMSNorm -> shared expert, router with the exact
 * top-K, routed experts -> residual add):
 *   xn  = coli_rmsnorm(x, in_ln, eps)
 *   a   = coli_mla_decode(attn, xn, pos_base; caches Lc, Rc)
 *   h   = x + a                                               (f32)
 *   out = coli_moe_layer(h, post_ln, eps, R, bias, K, topp, norm_topk,
 *                        routed_scale; experts gate/up/down, shared expert)
 * Arguments as in those calls (S = 1..COLI_MLA_MAX_ROWS: S <= 4 decode, more
 * rows prefill with coli_mla_decode's and coli_moe_layer's prefill kernels;
 * in_ln, post_ln, bias and the shared expert may be NULL); out may equal x.  Everything is validated before the
 * first launch; nothing is allocated and the host never waits.  Where the
 * matrix-core decode kernels run (S <= 4), the two norms and both residual
 * adds are folded into neighbouring launches (11 launches per layer instead of 16):
 * the residual adds and the post_ln norm give the bits the separate steps
 * give; the in_ln norm sums its squares in another order, so xn may differ
 * from coli_rmsnorm's in the last place (both within one f32 rounding of the
 * exact norm).
 *   workspace: coli_layer_decode_workspace_bytes(attn, gate, S, K, T_cap,
 *   has_shared) bytes, 256-byte aligned.  coli_layer_decode_workspace_layout
 *   gives the byte offsets of xn [S][D], a [S][D], h [S][D], the attention's
 *   workspace (coli_mla_workspace_layout applies from there) and the expert
 *   half's workspace.
 * Returns COLI_OK, COLI_DECLINED or COLI_HIP_ERROR.
 */
#define COLI_LAYER_STAGES 5
size_t coli_layer_decode_workspace_bytes(const coli_mla_layer *attn, const coli_qtensor *gate,
                                         int S, int K, int T_cap, int has_shared);
size_t coli_layer_decode_workspace_layout(const coli_mla_layer *attn, const coli_qtensor *gate,
                                          int S, int K, int T_cap, int has_shared,
                                          size_t offsets[COLI_LAYER_STAGES]);
int coli_layer_decode(const coli_mla_layer *attn, const float *in_ln, const coli_qtensor *gate,
                      const coli_qtensor *up, const coli_qtensor *down, const float *post_ln,
                      const float *R, const float *bias, int K, float topp, int norm_topk,
                      float routed_scale, const coli_qtensor *sh_gate, const coli_qtensor *sh_up,
                      const coli_qtensor *sh_down, float eps, const float *x, int S, int pos_base,
                      float *Lc, float *Rc, int T_cap, float *out, void *workspace,
                      size_t ws_bytes, void *stream);

/* Why the last call on this thread returned COLI_DECLINED ("" if none). */
const char *coli_last_reason(void);
/* Last HIP error text on this thread ("" if none). */
const char *coli_last_error(void);
/* Counters since load: compute calls, declined calls, kernel launches. */
void coli_stats(uint64_t *calls, uint64_t *declined, uint64_t *launches);
/* Fault injection: after n more successful compute calls every compute call
 * returns COLI_DECLINED and writes nothing; n < 0 disables.  The environment
 * variable COLI_FAIL_AFTER sets the initial value. */
void coli_set_fail_after(int64_t n);

/* Kernel timing with HIP events recorded around every launch while enabled
 * (on the launch stream).  coli_prof_read sums completed launches whose kernel
 * tag equals `tag` (e.g. "moe_gateup_decode"); returns the count or -1. */
void coli_prof_enable(int on);
void coli_prof_reset(void);
int64_t coli_prof_read(const char *tag, double *total_ms);
/* Tag of the i-th distinct kernel seen by the profiler (NULL past the end). */
const char *coli_prof_tag(int i);

/* Ceilings of this GPU measured by trivial kernels (diagnostics; not part
 * of the matmul path), timed by the caller around the call on `stream`:
 *   coli_probe_read   streams `bytes` (a multiple of 16) of the device buffer
 *                     `buf` (16-byte aligned) once through the vector loads;
 *   coli_probe_mfma   runs `workgroups` x 4 wavefronts, each issuing
 *                     8 * iters independent v_mfma_f32_32x32x16_bf16
 *                     (32768 flops each) -- the bf16 matrix-core rate.
 * `sink` is one device float that is written only in a case the inputs make
 * impossible.  Returns COLI_OK, COLI_DECLINED on bad arguments, or
 * COLI_HIP_ERROR. */
int coli_probe_read(const void *buf, size_t bytes, float *sink, void *stream);
int coli_probe_mfma(int workgroups, int iters, float *sink, void *stream);
/* coli_probe_launch: one launch of an empty kernel of `workgroups` x 256
 * threads -- the launch floor (back to back on a stream, or from a graph).
 * `sink` as above.  Returns COLI_OK, COLI_DECLINED or COLI_HIP_ERROR. */
int coli_probe_launch(int workgroups, float *sink, void *stream);

/* Library version string. */
const char *coli_version(void);

#ifdef __cplusplus
}
#endif

#endif /* COLI_H */
