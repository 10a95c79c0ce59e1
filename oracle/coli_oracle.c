/*
 * coli_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, double-precision CPU statement of what the colibri quantized
 * weight matmul and batched MoE expert block compute.  It exists so that the
 * GPU library can be checked against something that is obviously correct.
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load it; the GPU library never calls it, and the two share no code.
 *
 * Sources (pages describing the colibri engine):
 *   [P4-cuda]   colibri PR #298, commit adding fmt=4 to the CUDA backend:
 *               grouped int4 keeps the fmt=2 nibble layout and carries one f32
 *               scale per gs inputs along I, applied per group during the
 *               accumulation; the scale buffer holds O*ceil(I/gs) floats.
 *   [P4-test]   colibri PR #298, commit adding the matmul_i4_grouped test:
 *               the double-precision reference dequantises nibble -> (v-8)
 *               times scale[i/gs] and accumulates in double; nibbles are
 *               offset-encoded (0x0 -> -8, 0xF -> +7); the last group may be
 *               partial; the error is judged against the sum of |terms|.
 *   [P4-metal]  colibri PR #298, commit adding fmt=4 to the Metal mm_gemv:
 *               fmt 1-3 apply one per-row scale after the full dot product,
 *               fmt 4 folds its group scale in per group.
 *   [P4-addrow] colibri PR #298, commit making qt_addrow/qt_matvec_rows refuse
 *               unknown formats: fmt=1 raw bytes, fmt=3 row stride (I+3)/4,
 *               one scale per row for fmt 1/2/3.
 *   [P3-moe]    colibri-strix commit log, batched expert-block commit: gate/up -> SiLU -> down per expert,
 *               per-row ragged routing, weighted scatter-add of the results.
 *   [P3-shared] colibri-strix commit log, shared-expert fusion commit: the shared expert is an
 *               extra expert with routing weight 1.0 over every row.
 *   [P3-layer]  colibri-strix commit log, full decode layer commit: the router is a matvec followed by a
 *               sigmoid, then an exact top-K phase: greedy argmax over the
 *               sigmoid score plus a per-expert bias with the CPU's tie order,
 *               top-p truncation, norm_topk and routed_scale.
 *
 * Readings where the pages are silent (each also listed with the design notes):
 *   - element 2j of a byte pair is the LOW nibble, 2j+1 the high nibble;
 *   - each row starts on a byte boundary (strides I, ceil(I/2), ceil(I/4));
 *   - fmt 3 packs four 2-bit codes per byte, lowest bits first, value code-2;
 *   - fmt 1 bytes are two's-complement int8;
 *   - fmt 4 scales are row-major [O][ng], ng = ceil(I/gs), the last group
 *     holds I-(ng-1)*gs inputs;
 *   - SiLU(z) = z / (1 + exp(-z)); the gate feeds SiLU, the up projection is
 *     linear; routing weights are used exactly as given;
 *   - an expert id outside [0,E) contributes nothing and is counted.
 *
 * Arithmetic: every weight is s*v with s an f32 and |v| <= 128, so the f64
 * product is exact; every product with an f32 (or f64-held f32) input is exact
 * in f64 as well.  Sums run sequentially over the input index in f64.
 *
 * Parallelism: the optional OpenMP pragmas only split independent output rows
 * (or independent routed pairs) across threads; they change no arithmetic.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------ */
/* Formats                                                             */
/* ------------------------------------------------------------------ */

/* Bytes per weight row: fmt 1 one byte per input, fmt 2/4 two nibbles per
 * byte, fmt 3 four 2-bit codes per byte ([P4-addrow] gives (I+3)/4). */
int64_t oracle_row_bytes(int fmt, int64_t I)
{
    switch (fmt) {
    case 1: return I;
    case 2: case 4: return (I + 1) / 2;
    case 3: return (I + 3) / 4;
    default: return -1;
    }
}

/* 1 when (fmt, O, I, gs, ng) is a shape the oracle understands. */
int oracle_shape_ok(int fmt, int64_t O, int64_t I, int64_t gs, int64_t ng)
{
    if (fmt < 1 || fmt > 4 || O < 0 || I < 0)
        return 0;
    if (fmt == 4) {
        if (gs < 1) return 0;
        if (ng != (I + gs - 1) / gs) return 0;
    }
    return 1;
}

/* Integer code of weight (o, i): the stored value with its offset removed. */
static int weight_code(int fmt, const uint8_t *q, int64_t rb, int64_t o, int64_t i)
{
    const uint8_t *row = q + o * rb;
    if (fmt == 1)
        return (int)(int8_t)row[i];
    if (fmt == 2 || fmt == 4) {
        uint8_t b = row[i / 2];
        int nib = (i % 2 == 0) ? (b & 0x0F) : (b >> 4);
        return nib - 8;
    }
    /* fmt 3 */
    {
        uint8_t b = row[i / 4];
        int code = (b >> (2 * (i % 4))) & 0x3;
        return code - 2;
    }
}

/* Scale that multiplies weight (o, i): per row for fmt 1-3, per group of gs
 * inputs for fmt 4 ([P4-cuda], [P4-test]). */
static double weight_scale(int fmt, const float *s, int64_t ng, int64_t gs,
                           int64_t o, int64_t i)
{
    if (fmt == 4)
        return (double)s[o * ng + i / gs];
    return (double)s[o];
}

/* Exact weight value s * v. */
static double weight_value(int fmt, const uint8_t *q, const float *s, int64_t rb,
                           int64_t ng, int64_t gs, int64_t o, int64_t i)
{
    return weight_scale(fmt, s, ng, gs, o, i) * (double)weight_code(fmt, q, rb, o, i);
}

/* Integer codes of a whole [O][I] matrix. */
void oracle_decode_codes(int fmt, int64_t O, int64_t I, const uint8_t *q, int32_t *v)
{
    int64_t rb = oracle_row_bytes(fmt, I);
    for (int64_t o = 0; o < O; o++)
        for (int64_t i = 0; i < I; i++)
            v[o * I + i] = weight_code(fmt, q, rb, o, i);
}

/* Dequantised weights rounded once to f32: (float)((double)s * v). */
void oracle_dequant_f32(int fmt, int64_t O, int64_t I, int64_t gs, int64_t ng,
                        const uint8_t *q, const float *s, float *w)
{
    int64_t rb = oracle_row_bytes(fmt, I);
    for (int64_t o = 0; o < O; o++)
        for (int64_t i = 0; i < I; i++)
            w[o * I + i] = (float)weight_value(fmt, q, s, rb, ng, gs, o, i);
}

/* Dequantised weights kept exact in f64. */
void oracle_dequant_f64(int fmt, int64_t O, int64_t I, int64_t gs, int64_t ng,
                        const uint8_t *q, const float *s, double *w)
{
    int64_t rb = oracle_row_bytes(fmt, I);
    for (int64_t o = 0; o < O; o++)
        for (int64_t i = 0; i < I; i++)
            w[o * I + i] = weight_value(fmt, q, s, rb, ng, gs, o, i);
}

/* ------------------------------------------------------------------ */
/* Quantized matmul: y[s][o] = sum_i w(o,i) * x[s][i]                  */
/* ------------------------------------------------------------------ */

/* One output: the plain sequential sum over i in f64, plus the magnitude
 * A = sum_i |w(o,i)| * |x[i]| that tolerances are measured against
 * ([P4-test]: cancellation makes |result|-relative checks misfire). */
static void dot_row(int fmt, const uint8_t *q, const float *s, int64_t rb,
                    int64_t ng, int64_t gs, int64_t I, int64_t o,
                    const double *x, double *y, double *A)
{
    double acc = 0.0, mag = 0.0;
    for (int64_t i = 0; i < I; i++) {
        double w = weight_value(fmt, q, s, rb, ng, gs, o, i);
        acc += w * x[i];
        mag += fabs(w) * fabs(x[i]);
    }
    *y = acc;
    *A = mag;
}

/* y, A: [S][O] in f64 (A may be NULL).  x: [S][I] f64 inputs. */
void oracle_qmatmul_f64in(int fmt, int64_t O, int64_t I, int64_t gs, int64_t ng,
                          const uint8_t *q, const float *s, int64_t S,
                          const double *x, double *y, double *A, int nthreads)
{
    int64_t rb = oracle_row_bytes(fmt, I);
    (void)nthreads;
    for (int64_t t = 0; t < S; t++) {
#ifdef _OPENMP
#pragma omp parallel for schedule(static) num_threads(nthreads > 0 ? nthreads : 1)
#endif
        for (int64_t o = 0; o < O; o++) {
            double yy, aa;
            dot_row(fmt, q, s, rb, ng, gs, I, o, x + t * I, &yy, &aa);
            y[t * O + o] = yy;
            if (A)
                A[t * O + o] = aa;
        }
    }
}

/* Same with f32 inputs x: [S][I]; every f32 is exact in f64. */
void oracle_qmatmul(int fmt, int64_t O, int64_t I, int64_t gs, int64_t ng,
                    const uint8_t *q, const float *s, int64_t S, const float *x,
                    double *y, double *A, int nthreads)
{
    double *xd = (double *)malloc(sizeof(double) * (size_t)(S * I > 0 ? S * I : 1));
    for (int64_t k = 0; k < S * I; k++)
        xd[k] = (double)x[k];
    oracle_qmatmul_f64in(fmt, O, I, gs, ng, q, s, S, xd, y, A, nthreads);
    free(xd);
}

/* ------------------------------------------------------------------ */
/* MoE expert block                                                    */
/* ------------------------------------------------------------------ */

/* SiLU(z) = z * sigmoid(z) = z / (1 + exp(-z)) in f64. */
double oracle_silu(double z)
{
    return z / (1.0 + exp(-z));
}

/* Routing table ([P3-moe] "per-row ragged expert routing"):
 *   counts[e]  = number of (s,k) with ids[s][k] == e,
 *   offsets[e] = exclusive prefix sum of counts (offsets[E] = valid pairs),
 *   perm       = every valid pair index p = s*K + k, grouped by expert in
 *                ascending e, ascending p inside each expert.
 * Returns the number of pairs whose id lies outside [0,E) (left out). */
int64_t oracle_moe_route(const int32_t *ids, int64_t S, int64_t K, int64_t E,
                         int32_t *counts, int32_t *offsets, int32_t *perm)
{
    int64_t bad = 0;
    for (int64_t e = 0; e < E; e++)
        counts[e] = 0;
    for (int64_t p = 0; p < S * K; p++) {
        int32_t e = ids[p];
        if (e < 0 || e >= E)
            bad++;
        else
            counts[e]++;
    }
    offsets[0] = 0;
    for (int64_t e = 0; e < E; e++)
        offsets[e + 1] = offsets[e] + counts[e];
    /* stable placement: walk pairs in ascending p, append to their expert */
    {
        int32_t *fill = (int32_t *)malloc(sizeof(int32_t) * (size_t)(E > 0 ? E : 1));
        for (int64_t e = 0; e < E; e++)
            fill[e] = offsets[e];
        for (int64_t p = 0; p < S * K; p++) {
            int32_t e = ids[p];
            if (e >= 0 && e < E)
                perm[fill[e]++] = (int32_t)p;
        }
        free(fill);
    }
    return bad;
}

/* One quantized matrix inside a stack of experts. */
typedef struct oracle_qt {
    int32_t fmt;
    int32_t O, I;
    int32_t gs, ng;
    int32_t pad_;
    int64_t q_stride; /* bytes between consecutive experts' codes   */
    int64_t s_stride; /* floats between consecutive experts' scales */
    const uint8_t *q;
    const float *s;
} oracle_qt;

static const uint8_t *qt_q(const oracle_qt *t, int64_t e) { return t->q + e * t->q_stride; }
static const float *qt_s(const oracle_qt *t, int64_t e) { return t->s + e * t->s_stride; }

/* One expert MLP on one input row ([P3-moe]):
 *   g = G x, u = U x, h_j = silu(g_j) * u_j, y = D h.
 * x is f64 [D_in]; g, u, h, Ag, Au are [F]; y is evaluated only at the
 * requested output rows (all rows when rows == NULL). */
static void expert_mlp(const oracle_qt *G, const oracle_qt *U, const oracle_qt *Dn,
                       int64_t e, const double *x, double *g, double *u, double *h,
                       double *Ag, double *Au, int64_t nrows, const int32_t *rows,
                       double *y)
{
    int64_t F = G->O, Din = G->I, Dout = Dn->O;
    int64_t rbg = oracle_row_bytes(G->fmt, Din);
    int64_t rbu = oracle_row_bytes(U->fmt, Din);
    int64_t rbd = oracle_row_bytes(Dn->fmt, F);
    for (int64_t j = 0; j < F; j++) {
        dot_row(G->fmt, qt_q(G, e), qt_s(G, e), rbg, G->ng, G->gs, Din, j, x, &g[j], &Ag[j]);
        dot_row(U->fmt, qt_q(U, e), qt_s(U, e), rbu, U->ng, U->gs, Din, j, x, &u[j], &Au[j]);
        h[j] = oracle_silu(g[j]) * u[j];
    }
    int64_t n = rows ? nrows : Dout;
    for (int64_t r = 0; r < n; r++) {
        int64_t o = rows ? rows[r] : r;
        double a;
        dot_row(Dn->fmt, qt_q(Dn, e), qt_s(Dn, e), rbd, Dn->ng, Dn->gs, F, o, h, &y[r], &a);
    }
}

/* The batched expert block:
 *   out[s] = sum_k w[s][k] * MLP_{ids[s][k]}(x[s])  (+ 1.0 * MLP_shared(x[s]))
 * gate/up: stacks of E matrices [F][D]; down: E matrices [D][F]; the shared
 * triple (all three NULL or none) holds one matrix each.
 * x: f32 [S][D].  ids, w: [S][K].  out: f64 [S][nout] where nout = nrows when
 * rows != NULL (only those output rows are evaluated) else D.
 * Optional per-pair intermediates, each [P][F] with P = S*K (+S when a shared
 * expert is given; routed pair p = s*K+k first, then shared row s at S*K+s):
 * g, u, h, Ag, Au.  An id outside [0,E) contributes nothing; the count of such
 * pairs is returned. */
int64_t oracle_moe_block(const oracle_qt *gate, const oracle_qt *up, const oracle_qt *down,
                         int64_t E, const float *x, int64_t S, const int32_t *ids,
                         const float *w, int64_t K, const oracle_qt *sh_gate,
                         const oracle_qt *sh_up, const oracle_qt *sh_down,
                         int64_t nrows, const int32_t *rows, double *out,
                         double *g_out, double *u_out, double *h_out, double *Ag_out,
                         double *Au_out, int nthreads)
{
    int64_t F = gate->O, D = gate->I;
    int64_t nout = rows ? nrows : down->O;
    int64_t has_shared = (sh_gate && sh_up && sh_down) ? 1 : 0;
    int64_t P = S * K + (has_shared ? S : 0);
    int64_t bad = 0;
    (void)nthreads;

    double *ybuf = (double *)malloc(sizeof(double) * (size_t)((P > 0 ? P : 1) * (nout > 0 ? nout : 1)));
    int8_t *valid = (int8_t *)calloc((size_t)(P > 0 ? P : 1), 1);

    for (int64_t p = 0; p < S * K; p++) {
        int32_t e = ids[p];
        if (e < 0 || e >= E)
            bad++;
        else
            valid[p] = 1;
    }
    for (int64_t p = S * K; p < P; p++)
        valid[p] = 1;

#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads > 0 ? nthreads : 1)
#endif
    for (int64_t p = 0; p < P; p++) {
        if (!valid[p])
            continue;
        int64_t s = (p < S * K) ? p / K : p - S * K;
        const oracle_qt *G = gate, *U = up, *Dn = down;
        int64_t e;
        if (p < S * K) {
            e = ids[p];
        } else {
            G = sh_gate; U = sh_up; Dn = sh_down;
            e = 0;
        }
        double *xd = (double *)malloc(sizeof(double) * (size_t)(D > 0 ? D : 1));
        double *g = (double *)malloc(sizeof(double) * (size_t)(F > 0 ? F : 1) * 5);
        double *u = g + F, *h = u + F, *Ag = h + F, *Au = Ag + F;
        for (int64_t i = 0; i < D; i++)
            xd[i] = (double)x[s * D + i];
        expert_mlp(G, U, Dn, e, xd, g, u, h, Ag, Au, nrows, rows, ybuf + p * nout);
        if (g_out) memcpy(g_out + p * F, g, sizeof(double) * (size_t)F);
        if (u_out) memcpy(u_out + p * F, u, sizeof(double) * (size_t)F);
        if (h_out) memcpy(h_out + p * F, h, sizeof(double) * (size_t)F);
        if (Ag_out) memcpy(Ag_out + p * F, Ag, sizeof(double) * (size_t)F);
        if (Au_out) memcpy(Au_out + p * F, Au, sizeof(double) * (size_t)F);
        free(g);
        free(xd);
    }

    /* weighted combine in ascending k, then the shared expert with weight 1 */
    for (int64_t s = 0; s < S; s++) {
        for (int64_t r = 0; r < nout; r++) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; k++) {
                int64_t p = s * K + k;
                if (valid[p])
                    acc += (double)w[p] * ybuf[p * nout + r];
            }
            if (has_shared)
                acc += ybuf[(S * K + s) * nout + r];
            out[s * nout + r] = acc;
        }
    }
    free(valid);
    free(ybuf);
    return bad;
}

/* ------------------------------------------------------------------ */
/* Router and exact top-K ([P3-layer])                                 */
/* ------------------------------------------------------------------ */

/* For every input row s (readings where the one-line description is silent):
 *   z[e] = sum_d R[e][d] * x[s][d] in f64 (exact products, sequential sum);
 *   p[e] = 1 / (1 + exp(-z[e]));  selection key c[e] = p[e] + bias[e];
 *   K greedy rounds, each taking the not yet chosen expert with the largest
 *   key, the smallest index among equal keys (a scan keeping its first
 *   maximum);
 *   top-p (0 < topp < 1): the picks, in pick order, are kept up to and
 *   including the first at which the running sum of p reaches
 *   topp * (sum of p over all K picks); later slots become id -1, weight 0;
 *   topp <= 0 or >= 1 keeps all K;
 *   weight of a kept pick = its p (the bias steers the choice only); with
 *   norm_topk the kept weights are divided by their sum; finally every weight
 *   is multiplied by routed_scale.
 * ids[s][K], w[s][K] (f64); z_out[s][E] the logits when not NULL.
 * bias may be NULL (all zero). */
void oracle_moe_router(const float *x, int64_t S, int64_t D, const float *R,
                       const float *bias, int64_t E, int64_t K, double topp,
                       int norm_topk, double routed_scale, int32_t *ids, double *w,
                       double *z_out)
{
    double *z = (double *)malloc(sizeof(double) * (size_t)(E > 0 ? E : 1));
    double *c = (double *)malloc(sizeof(double) * (size_t)(E > 0 ? E : 1));
    double *pr = (double *)malloc(sizeof(double) * (size_t)(E > 0 ? E : 1));
    char *taken = (char *)malloc((size_t)(E > 0 ? E : 1));
    for (int64_t s = 0; s < S; s++) {
        for (int64_t e = 0; e < E; e++) {
            double acc = 0.0;
            for (int64_t d = 0; d < D; d++)
                acc += (double)R[e * D + d] * (double)x[s * D + d];
            z[e] = acc;
            pr[e] = 1.0 / (1.0 + exp(-acc));
            c[e] = pr[e] + (bias ? (double)bias[e] : 0.0);
            taken[e] = 0;
            if (z_out)
                z_out[s * E + e] = acc;
        }
        /* greedy picks */
        double total = 0.0;
        for (int64_t k = 0; k < K; k++) {
            int64_t best = -1;
            for (int64_t e = 0; e < E; e++)
                if (!taken[e] && (best < 0 || c[e] > c[best]))
                    best = e;
            taken[best] = 1;
            ids[s * K + k] = (int32_t)best;
            w[s * K + k] = pr[best];
            total += pr[best];
        }
        /* top-p truncation */
        int64_t keep = K;
        if (topp > 0.0 && topp < 1.0) {
            double run = 0.0;
            for (int64_t k = 0; k < K; k++) {
                run += w[s * K + k];
                if (run >= topp * total) {
                    keep = k + 1;
                    break;
                }
            }
        }
        for (int64_t k = keep; k < K; k++) {
            ids[s * K + k] = -1;
            w[s * K + k] = 0.0;
        }
        if (norm_topk) {
            double sum = 0.0;
            for (int64_t k = 0; k < keep; k++)
                sum += w[s * K + k];
            for (int64_t k = 0; k < keep; k++)
                w[s * K + k] /= sum;
        }
        for (int64_t k = 0; k < keep; k++)
            w[s * K + k] *= routed_scale;
    }
    free(taken);
    free(pr);
    free(c);
    free(z);
}

/* ------------------------------------------------------------------ */

/* RMSNorm of each row (colibri-strix commit log, full decode layer commit: the post-attention norm in front of the expert
 * half of the layer).  The pages name the step only; the reading taken is
 * the usual root-mean-square norm with a per-feature weight:
 *   ms      = (sum_d x[s][d]^2) / D          (f64, sequential sum)
 *   y[s][d] = x[s][d] / sqrt(ms + eps) * w[d] (f64)
 * w may be NULL (all ones). */
void oracle_rmsnorm(const float *x, int64_t S, int64_t D, const float *w, double eps, double *y)
{
    for (int64_t s = 0; s < S; s++) {
        const float *xr = x + s * D;
        double ss = 0.0;
        for (int64_t d = 0; d < D; d++)
            ss += (double)xr[d] * (double)xr[d];
        const double inv = 1.0 / sqrt(ss / (double)D + eps);
        for (int64_t d = 0; d < D; d++)
            y[s * D + d] = (double)xr[d] * inv * (w ? (double)w[d] : 1.0);
    }
}

/* ------------------------------------------------------------------ */
/* MLA decode attention                                                */
/* ------------------------------------------------------------------ */
/*
 * Sources (colibri-strix commit log):
 *   [P3-attn]   fused decode attention commit (Phase 2): one decode attention
 *               layer is q_a -> RMSNorm -> q_b -> RoPE on the query path;
 *               kv_a -> RMSNorm of the latent and RoPE of the rotary key at
 *               the token's position, both written to the latent / rotary
 *               caches (Lc, Rc); the MLA absorption core (qabs, score,
 *               softmax, clat, ctx); then o_proj.
 *   [P3-attnS4] fused attention for S <= 4 (MTP verify): every core step
 *               gains a query-row dimension; query row s attends the keys
 *               [0, pos_base + s].
 *   [P3-attnT]  standalone fused-attention regression tests: the CPU chain
 *               per head is qabs, score, softmax, clat, ctx; checked at
 *               S = 1/3/4 and pos_base 0/12/37 including the cache rows.
 *   [P1]        issue #585 thread: kv_b, the MLA absorption weight, is
 *               grouped int4 (fmt 4) on the fused path.
 *
 * Readings where the pages are silent (each also in the design notes):
 *   - dimensions: H heads, each query head has d_nope "no position" and
 *     d_rope rotary components (q_b rows h*(d_nope+d_rope) + j, the no-
 *     position ones first); kv_a gives the latent (kv_rank) then the shared
 *     rotary key (d_rope); kv_b rows h*(d_nope+d_v) + j hold head h's key
 *     absorption rows (j < d_nope) then its value rows; ctx is [h*d_v + v];
 *   - RoPE rotates consecutive pairs (2i, 2i+1) of a rotary vector by
 *     pos * theta^(-2i/d_rope);
 *   - RMSNorm as oracle_rmsnorm (eps inside the square root, per-feature
 *     weight), on the query latent and on the kv latent;
 *   - the softmax scale is 1/sqrt(d_nope + d_rope);
 *   - the caches store f32 (the rows this call writes are rounded to f32
 *     before any score reads them).
 * Absorption: score = q . k with k = [W_UK Lc, Rc] equals
 * (W_UK^T q_nope) . Lc + q_rope . Rc, and sum_t p_t W_UV Lc_t equals
 * W_UV (sum_t p_t Lc_t); the pins check this against the expanded form.
 */

/* RoPE of one rotary vector of 2*npair components at position pos. */
void oracle_rope(const double *in, int64_t npair, int64_t pos, double theta, double *out)
{
    for (int64_t i = 0; i < npair; i++) {
        double ang = (double)pos * pow(theta, -(double)(2 * i) / (double)(2 * npair));
        double c = cos(ang), s = sin(ang);
        double a = in[2 * i], b = in[2 * i + 1];
        out[2 * i] = a * c - b * s;
        out[2 * i + 1] = a * s + b * c;
    }
}

/* RMSNorm of one f64 vector (the oracle_rmsnorm formula). */
static void rms_f64(const double *x, int64_t n, const float *w, double eps, double *y)
{
    double ss = 0.0;
    for (int64_t d = 0; d < n; d++)
        ss += x[d] * x[d];
    const double inv = 1.0 / sqrt(ss / (double)n + eps);
    for (int64_t d = 0; d < n; d++)
        y[d] = x[d] * inv * (w ? (double)w[d] : 1.0);
}

/* One weight of matrix 0 of a stack. */
static double qt_w(const oracle_qt *t, int64_t o, int64_t i)
{
    return weight_value(t->fmt, t->q, t->s, oracle_row_bytes(t->fmt, t->I), t->ng, t->gs, o, i);
}

/* qabs[s][h][c] = sum_{j < dn} q[s][h*(dn+dr)+j] * kv_b[h*(dn+dv)+j][c]
 * (the key absorption); A the matching sum of |terms|.  q: [S][H*(dn+dr)]. */
void oracle_mla_qabs(const oracle_qt *kv_b, int64_t H, int64_t dn, int64_t dr, int64_t dv,
                     const double *q, int64_t S, double *qabs, double *A)
{
    const int64_t L = kv_b->I;
    for (int64_t s = 0; s < S; s++)
#ifdef _OPENMP
#pragma omp parallel for schedule(static)
#endif
        for (int64_t h = 0; h < H; h++)
            for (int64_t c = 0; c < L; c++) {
                double acc = 0.0, mag = 0.0;
                for (int64_t j = 0; j < dn; j++) {
                    double w = qt_w(kv_b, h * (dn + dv) + j, c);
                    double v = q[s * H * (dn + dr) + h * (dn + dr) + j];
                    acc += v * w;
                    mag += fabs(v) * fabs(w);
                }
                qabs[(s * H + h) * L + c] = acc;
                if (A)
                    A[(s * H + h) * L + c] = mag;
            }
}

/* scores[s][h][t] = scale * (qabs[s][h] . Lc[t] + qpe[s][h] . Rc[t]) for
 * t <= pos_base + s; entries past it are set to 0 (never read).  Ts = the
 * row stride of scores (>= pos_base + S).  A: the sum of |terms| times scale. */
void oracle_mla_scores(const double *qabs, const double *qpe, const float *Lc, const float *Rc,
                       int64_t S, int64_t H, int64_t L, int64_t dr, int64_t pos_base, int64_t Ts,
                       double scale, double *scores, double *A)
{
    for (int64_t s = 0; s < S; s++)
        for (int64_t h = 0; h < H; h++) {
            const double *qa = qabs + (s * H + h) * L, *qp = qpe + (s * H + h) * dr;
            for (int64_t t = 0; t < Ts; t++) {
                double acc = 0.0, mag = 0.0;
                if (t <= pos_base + s) {
                    for (int64_t c = 0; c < L; c++) {
                        acc += qa[c] * (double)Lc[t * L + c];
                        mag += fabs(qa[c]) * fabs((double)Lc[t * L + c]);
                    }
                    for (int64_t r = 0; r < dr; r++) {
                        acc += qp[r] * (double)Rc[t * dr + r];
                        mag += fabs(qp[r]) * fabs((double)Rc[t * dr + r]);
                    }
                }
                scores[(s * H + h) * Ts + t] = acc * scale;
                if (A)
                    A[(s * H + h) * Ts + t] = mag * scale;
            }
        }
}

/* p[s][h][t] = exp(z_t - max) / sum over t <= pos_base + s; 0 past it. */
void oracle_mla_softmax(const double *scores, int64_t S, int64_t H, int64_t pos_base, int64_t Ts,
                        double *p)
{
    for (int64_t s = 0; s < S; s++)
        for (int64_t h = 0; h < H; h++) {
            const double *z = scores + (s * H + h) * Ts;
            double *pr = p + (s * H + h) * Ts;
            const int64_t n = pos_base + s + 1;
            double mx = z[0];
            for (int64_t t = 1; t < n; t++)
                mx = z[t] > mx ? z[t] : mx;
            double sum = 0.0;
            for (int64_t t = 0; t < n; t++)
                sum += exp(z[t] - mx);
            for (int64_t t = 0; t < Ts; t++)
                pr[t] = t < n ? exp(z[t] - mx) / sum : 0.0;
        }
}

/* clat[s][h][c] = sum_{t <= pos_base+s} p[s][h][t] * Lc[t][c]; A its sum of
 * |terms|. */
void oracle_mla_clat(const double *p, const float *Lc, int64_t S, int64_t H, int64_t L,
                     int64_t pos_base, int64_t Ts, double *clat, double *A)
{
    for (int64_t s = 0; s < S; s++)
        for (int64_t h = 0; h < H; h++)
            for (int64_t c = 0; c < L; c++) {
                double acc = 0.0, mag = 0.0;
                for (int64_t t = 0; t <= pos_base + s; t++) {
                    double v = p[(s * H + h) * Ts + t] * (double)Lc[t * L + c];
                    acc += v;
                    mag += fabs(v);
                }
                clat[(s * H + h) * L + c] = acc;
                if (A)
                    A[(s * H + h) * L + c] = mag;
            }
}

/* ctx[s][h*dv+v] = sum_c kv_b[h*(dn+dv)+dn+v][c] * clat[s][h][c] (the value
 * absorption); A its sum of |terms|. */
void oracle_mla_ctx(const oracle_qt *kv_b, int64_t H, int64_t dn, int64_t dv, const double *clat,
                    int64_t S, double *ctx, double *A)
{
    const int64_t L = kv_b->I;
    for (int64_t s = 0; s < S; s++)
#ifdef _OPENMP
#pragma omp parallel for schedule(static)
#endif
        for (int64_t h = 0; h < H; h++)
            for (int64_t v = 0; v < dv; v++) {
                double acc = 0.0, mag = 0.0;
                for (int64_t c = 0; c < L; c++) {
                    double w = qt_w(kv_b, h * (dn + dv) + dn + v, c);
                    double z = clat[(s * H + h) * L + c];
                    acc += w * z;
                    mag += fabs(w) * fabs(z);
                }
                ctx[s * H * dv + h * dv + v] = acc;
                if (A)
                    A[s * H * dv + h * dv + v] = mag;
            }
}

/* One matrix of a stack times f64 rows: y[s][o] = sum_i w(o,i) x[s][i]. */
static void qt_gemv(const oracle_qt *t, const double *x, int64_t S, double *y, int nthreads)
{
    (void)nthreads;
    for (int64_t s = 0; s < S; s++)
#ifdef _OPENMP
#pragma omp parallel for schedule(static) num_threads(nthreads > 0 ? nthreads : 1)
#endif
        for (int64_t o = 0; o < t->O; o++) {
            double acc = 0.0;
            for (int64_t i = 0; i < t->I; i++)
                acc += qt_w(t, o, i) * x[s * t->I + i];
            y[s * t->O + o] = acc;
        }
}

/* The whole decode attention for S rows at positions pos_base .. pos_base+S-1
 * ([P3-attn], [P3-attnS4]), every step above in order:
 *   cq_raw = q_a x;  cq = RMSNorm(cq_raw) * q_norm;  q = q_b cq
 *   ckv_raw = kv_a x;  Lc[pos] = f32(RMSNorm(latent) * kv_norm);
 *   Rc[pos] = f32(RoPE(rotary key, pos))                  (pos = pos_base+s)
 *   qpe = RoPE(q rotary part, pos);  qabs;  scores;  p;  clat;  ctx;
 *   out = o_proj ctx
 * x f32 [S][D]; Lc f32 [>= pos_base+S][kv_rank], Rc f32 [..][d_rope]: rows
 * below pos_base are inputs, rows pos_base.. are written.  out f64 [S][D].
 * st (optional, NULL entries skipped) receives the stages in f64:
 * 0 cq_raw [S][qr], 1 ckv_raw [S][L+dr], 2 cq [S][qr], 3 q [S][H(dn+dr)],
 * 4 qabs [S][H][L], 5 qpe [S][H][dr], 6 scores [S][H][pos_base+S],
 * 7 p [same], 8 clat [S][H][L], 9 ctx [S][H dv].  nthreads: OpenMP threads
 * over the output rows of the four projections (no change to the arithmetic). */
void oracle_mla_decode(const oracle_qt *q_a, const float *q_norm, const oracle_qt *q_b,
                       const oracle_qt *kv_a, const float *kv_norm, const oracle_qt *kv_b,
                       const oracle_qt *o_proj, int64_t H, int64_t dn, int64_t dr, int64_t dv,
                       double eps, double theta, const float *x, int64_t S, int64_t pos_base,
                       float *Lc, float *Rc, double *out, double **st, int nthreads)
{
    const int64_t D = q_a->I, qr = q_a->O, L = kv_b->I, Ts = pos_base + S;
    const int64_t nq = H * (dn + dr);
    double *xd = (double *)calloc((size_t)(S * D), sizeof(double));
    double *cq_raw = (double *)calloc((size_t)(S * qr), sizeof(double));
    double *ckv = (double *)calloc((size_t)(S * (L + dr)), sizeof(double));
    double *cq = (double *)calloc((size_t)(S * qr), sizeof(double));
    double *q = (double *)calloc((size_t)(S * nq), sizeof(double));
    double *qabs = (double *)calloc((size_t)(S * H * L), sizeof(double));
    double *qpe = (double *)calloc((size_t)(S * H * dr), sizeof(double));
    double *sc = (double *)calloc((size_t)(S * H * Ts), sizeof(double));
    double *p = (double *)calloc((size_t)(S * H * Ts), sizeof(double));
    double *clat = (double *)calloc((size_t)(S * H * L), sizeof(double));
    double *ctx = (double *)calloc((size_t)(S * H * dv), sizeof(double));
    double *tmp = (double *)calloc((size_t)(L > dr ? L : dr), sizeof(double));

    for (int64_t i = 0; i < S * D; i++)
        xd[i] = (double)x[i];
    /* query path */
    qt_gemv(q_a, xd, S, cq_raw, nthreads);
    for (int64_t s = 0; s < S; s++)
        rms_f64(cq_raw + s * qr, qr, q_norm, eps, cq + s * qr);
    qt_gemv(q_b, cq, S, q, nthreads);
    /* kv path: cache rows of this call's positions */
    qt_gemv(kv_a, xd, S, ckv, nthreads);
    for (int64_t s = 0; s < S; s++) {
        const int64_t pos = pos_base + s;
        rms_f64(ckv + s * (L + dr), L, kv_norm, eps, tmp);
        for (int64_t c = 0; c < L; c++)
            Lc[pos * L + c] = (float)tmp[c];
        oracle_rope(ckv + s * (L + dr) + L, dr / 2, pos, theta, tmp);
        for (int64_t r = 0; r < dr; r++)
            Rc[pos * dr + r] = (float)tmp[r];
    }
    /* absorption core */
    for (int64_t s = 0; s < S; s++)
        for (int64_t h = 0; h < H; h++)
            oracle_rope(q + s * nq + h * (dn + dr) + dn, dr / 2, pos_base + s, theta,
                        qpe + (s * H + h) * dr);
    oracle_mla_qabs(kv_b, H, dn, dr, dv, q, S, qabs, NULL);
    oracle_mla_scores(qabs, qpe, Lc, Rc, S, H, L, dr, pos_base, Ts, 1.0 / sqrt((double)(dn + dr)),
                      sc, NULL);
    oracle_mla_softmax(sc, S, H, pos_base, Ts, p);
    oracle_mla_clat(p, Lc, S, H, L, pos_base, Ts, clat, NULL);
    oracle_mla_ctx(kv_b, H, dn, dv, clat, S, ctx, NULL);
    qt_gemv(o_proj, ctx, S, out, nthreads);

    if (st) {
        const double *src[10] = {cq_raw, ckv, cq, q, qabs, qpe, sc, p, clat, ctx};
        const int64_t n[10] = {S * qr, S * (L + dr), S * qr, S * nq, S * H * L, S * H * dr,
                               S * H * Ts, S * H * Ts, S * H * L, S * H * dv};
        for (int k = 0; k < 10; k++)
            if (st[k])
                memcpy(st[k], src[k], sizeof(double) * (size_t)n[k]);
    }
    free(xd); free(cq_raw); free(ckv); free(cq); free(q); free(qabs); free(qpe);
    free(sc); free(p); free(clat); free(ctx); free(tmp);
}
