// gemv.hip -- fp32 decode kernels for gfx950: quantized GEMV (S <= 4 input
// rows), the decode MoE block (dual gate/up + SiLU, down + weighted combine),
// and the exact dequantizer.
//
// What is computed (colibri PR #298, CUDA fmt=4 and Metal mm_gemv fmt=4
// commits): y[s][o] = sum_i w(o,i) x[s][i] with w = scale * v; fmt 4 applies
// its per-group scale to each group's partial sum during the accumulation,
// fmt 1-3 apply the row scale once after the dot product.
//
// How (MI355X design, not the pages' Metal/CUDA kernels):
//   * one 64-lane wavefront owns R weight rows; every lane streams 16-byte
//     packets (32 int4 / 32 int2 / 16 int8 codes) with non-temporal loads, so a
//     row chunk of 64 packets is one fully coalesced 1 KiB request;
//   * codes are turned into floats with one SDWA v_cvt_f32_i32 per code after
//     a couple of bit operations per 32-bit word (the code's offset is removed
//     exactly, see common.h), then fp32 FMAs against the inputs;
//   * fmt-4 group scales are loaded once per packet and folded into each
//     lane's per-packet partial (gs a multiple of 32: one scale per packet;
//     gs a multiple of 16: two);
//   * the lane partials are summed across the wavefront with cross-lane
//     shuffles; no LDS, no atomics, so every result is deterministic.
#include <stdarg.h>

#include "common.h"

namespace coli {

// ---------------------------------------------------------------------------
// Exact dequantizer (test hook): w = (float)(s * v), one rounding.
// ---------------------------------------------------------------------------

__device__ __forceinline__ int code_at(int fmt, const uint8_t *row, int64_t i) {
    if (fmt == 1)
        return (int)(int8_t)row[i];
    if (fmt == 3)
        return (int)((row[i >> 2] >> (2 * (i & 3))) & 3) - 2;
    const uint8_t b = row[i >> 1];
    return (int)((i & 1) ? (b >> 4) : (b & 15)) - 8;
}

__global__ void k_dequant(int fmt, const uint8_t *__restrict__ q, const float *__restrict__ s,
                          int64_t rows, int64_t I, int64_t rb, int ng, int gs,
                          float *__restrict__ w) {
    const int64_t total = rows * I;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
         t += (int64_t)gridDim.x * blockDim.x) {
        const int64_t g = t / I, i = t - g * I;
        const int v = code_at(fmt, q + g * rb, i);
        const float sc = (fmt == 4) ? s[g * ng + i / gs] : s[g];
        w[t] = __fmul_rn(sc, (float)v);
    }
}

int launch_dequant(const coli_qtensor *W, float *w, hipStream_t st) {
    const int64_t rows = (int64_t)W->n * W->O;
    const int64_t total = rows * W->I;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    ProfScope ps("dequant", st);
    hipLaunchKernelGGL(k_dequant, dim3((unsigned)blocks), dim3(256), 0, st, W->fmt,
                       (const uint8_t *)W->q, W->s, rows, (int64_t)W->I, W->row_bytes, W->ng,
                       W->gs > 0 ? W->gs : 1, w);
    return after_launch("dequant");
}

// ---------------------------------------------------------------------------
// Exact-shape fallback GEMV: any fmt, gs, I, alignment.  One wavefront per
// (row, input row); lanes stride over the inputs.  Used when the layout does
// not allow packet loads.
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void k_gemv_any(int fmt, const uint8_t *__restrict__ q,
                                                  const float *__restrict__ s,
                                                  const float *__restrict__ x,
                                                  float *__restrict__ y, int rows, int O, int I,
                                                  int64_t rb, int ng, int gs, int S) {
    const int lane = threadIdx.x & 63;
    const int g = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int t = blockIdx.y;
    if (g >= rows)
        return;
    const uint8_t *row = q + (int64_t)g * rb;
    const float *xs = x + (int64_t)t * I;
    float acc = 0.f;
    for (int64_t i = lane; i < I; i += 64) {
        const float sc = (fmt == 4) ? s[(int64_t)g * ng + i / gs] : s[g];
        const float wv = __fmul_rn(sc, (float)code_at(fmt, row, i));
        acc = fmaf(wv, xs[i], acc);
    }
    acc = wave_sum(acc);
    if (lane == 0) {
        const int e = g / O, o = g - e * O;
        y[((int64_t)e * S + t) * O + o] = acc;
    }
}

// ---------------------------------------------------------------------------
// Packet GEMV core
// ---------------------------------------------------------------------------

// GM: 0 = per-row scale (fmt 1-3), 1 = one group scale per packet,
//     2 = two group scales per packet (16 inputs each).
template <int FMT, int GM>
struct PacketDot {
    static constexpr int CP = packet_cols(FMT);
    static constexpr int PB = packet_bytes(FMT);

    // Accumulate the packet's contribution for NS input rows:
    //   acc[t] += scale * sum_j f_j * xv[t][j]     (GM 1/2)
    //   acc[t] += sum_j f_j * xv[t][j]             (GM 0)
    template <int NS>
    __device__ __forceinline__ static void run(const Packet<FMT> &pk, const float (&xv)[NS][CP],
                                               float s0, float s1, float (&acc)[NS]) {
        float f[CP];
        decode_packet<FMT>(pk, f);
#pragma unroll
        for (int t = 0; t < NS; ++t) {
            if constexpr (GM == 2) {
                float pa = 0.f, pb = 0.f;
#pragma unroll
                for (int j = 0; j < CP / 2; ++j) pa = fmaf(f[j], xv[t][j], pa);
#pragma unroll
                for (int j = CP / 2; j < CP; ++j) pb = fmaf(f[j], xv[t][j], pb);
                acc[t] = fmaf(s0, pa, acc[t]);
                acc[t] = fmaf(s1, pb, acc[t]);
            } else {
                float pa = 0.f, pb = 0.f;
#pragma unroll
                for (int j = 0; j < CP; j += 2) {
                    pa = fmaf(f[j], xv[t][j], pa);
                    pb = fmaf(f[j + 1], xv[t][j + 1], pb);
                }
                const float p = pa + pb;
                if constexpr (GM == 1)
                    acc[t] = fmaf(s0, p, acc[t]);
                else
                    acc[t] += p;
            }
        }
    }
};

template <int CP>
__device__ __forceinline__ void load_x(const float *__restrict__ xp, float (&xv)[CP]) {
    const f32x4 *p4 = reinterpret_cast<const f32x4 *>(xp);
#pragma unroll
    for (int j = 0; j < CP / 4; ++j) {
        const f32x4 v = p4[j];
        xv[4 * j + 0] = v.x;
        xv[4 * j + 1] = v.y;
        xv[4 * j + 2] = v.z;
        xv[4 * j + 3] = v.w;
    }
}

// Group scale(s) of the packet starting at input col0 for row `row`.
template <int GM>
__device__ __forceinline__ void packet_scales(const float *__restrict__ s, int64_t row, int ng,
                                              int gs, int col0, float &s0, float &s1) {
    if constexpr (GM == 1) {
        s0 = s[row * ng + col0 / gs];
        s1 = 0.f;
    } else if constexpr (GM == 2) {
        s0 = s[row * ng + col0 / gs];
        s1 = s[row * ng + (col0 + 16) / gs];
    } else {
        s0 = s1 = 0.f;
    }
}

// y[e][t][o] for R consecutive rows per wavefront, S input rows (S <= 4).
template <int FMT, int S, int R, int GM>
__global__ __launch_bounds__(256) void k_gemv(const uint8_t *__restrict__ q,
                                              const float *__restrict__ sc,
                                              const float *__restrict__ x, float *__restrict__ y,
                                              int rows, int O, int I, int64_t rb, int ng, int gs,
                                              int ldx, int Sy) {
    constexpr int CP = packet_cols(FMT), PB = packet_bytes(FMT);
    using Dot = PacketDot<FMT, GM>;
    const int lane = threadIdx.x & 63;
    const int r0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * R;
    if (r0 >= rows)
        return;
    const int nchunks = (I + 64 * CP - 1) / (64 * CP);

    int64_t rowi[R];
#pragma unroll
    for (int r = 0; r < R; ++r) rowi[r] = (r0 + r < rows) ? (r0 + r) : (rows - 1);

    float acc[R][S];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int t = 0; t < S; ++t) acc[r][t] = 0.f;

    Packet<FMT> nxt[R];
    {
        const int col0 = lane * CP;
        if (col0 < I) {
#pragma unroll
            for (int r = 0; r < R; ++r)
                nxt[r] = load_packet<FMT>(q + rowi[r] * rb + (int64_t)lane * PB);
        }
    }
    for (int c = 0; c < nchunks; ++c) {
        const int col0 = c * 64 * CP + lane * CP;
        const bool live = col0 < I;
        Packet<FMT> cur[R];
#pragma unroll
        for (int r = 0; r < R; ++r) cur[r] = nxt[r];
        const int coln = col0 + 64 * CP;
        if (c + 1 < nchunks && coln < I) {
#pragma unroll
            for (int r = 0; r < R; ++r)
                nxt[r] = load_packet<FMT>(q + rowi[r] * rb + (int64_t)coln / CP * PB);
        }
        if (live) {
            float xv[S][CP];
#pragma unroll
            for (int t = 0; t < S; ++t) load_x<CP>(x + (int64_t)t * ldx + col0, xv[t]);
#pragma unroll
            for (int r = 0; r < R; ++r) {
                float s0, s1;
                packet_scales<GM>(sc, rowi[r], ng, gs, col0, s0, s1);
                Dot::template run<S>(cur[r], xv, s0, s1, acc[r]);
            }
        }
    }
    constexpr float inv = 1.0f / Mult<FMT>::value;
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
        for (int t = 0; t < S; ++t) {
            const float v = wave_sum(acc[r][t]);
            if (lane == 0 && r0 + r < rows) {
                const int g = r0 + r;
                const int e = g / O, o = g - e * O;
                const float out = (GM == 0) ? (v * inv) * sc[g] : v * inv;
                y[((int64_t)e * Sy + t) * O + o] = out;
            }
        }
    }
}

template <int FMT, int GM>
static void launch_gemv_t(const coli_qtensor *W, const float *x, float *y, int S, int Sy,
                          hipStream_t st) {
    const int rows = W->n * W->O;
    const int R = 4;
    const unsigned blocks = (unsigned)((rows + 4 * R - 1) / (4 * R));
    const uint8_t *q = (const uint8_t *)W->q;
    const int gs = W->gs > 0 ? W->gs : 1;
#define COLI_GEMV_CASE(SS)                                                                     \
    hipLaunchKernelGGL((k_gemv<FMT, SS, R, GM>), dim3(blocks), dim3(256), 0, st, q, W->s, x, y, \
                       rows, W->O, W->I, W->row_bytes, W->ng, gs, W->I, Sy)
    switch (S) {
    case 1: COLI_GEMV_CASE(1); break;
    case 2: COLI_GEMV_CASE(2); break;
    case 3: COLI_GEMV_CASE(3); break;
    default: COLI_GEMV_CASE(4); break;
    }
#undef COLI_GEMV_CASE
}

// y = W x for S input rows.  Packet kernels take up to 4 input rows per
// launch (larger S is split into blocks of 4); the fallback takes any S.
int launch_gemv(const coli_qtensor *W, const float *x, float *y, int S, hipStream_t st) {
    const int rows = W->n * W->O;
    const bool fast = (W->flags & QF_FAST) &&
                      (W->fmt != 4 || (W->flags & (QF_GROUP32 | QF_GROUP16))) &&
                      ((uintptr_t)x % 16 == 0);
    if (!fast) {
        ProfScope ps("gemv_any", st);
        hipLaunchKernelGGL(k_gemv_any, dim3((unsigned)((rows + 3) / 4), (unsigned)S), dim3(256), 0,
                           st, W->fmt, (const uint8_t *)W->q, W->s, x, y, rows, W->O, W->I,
                           W->row_bytes, W->ng, W->gs > 0 ? W->gs : 1, S);
        return after_launch("gemv_any");
    }
    for (int t0 = 0; t0 < S; t0 += 4) {
        const int ns = (S - t0) < 4 ? (S - t0) : 4;
        const float *xb = x + (int64_t)t0 * W->I;
        float *yb = y + (int64_t)t0 * W->O;
        ProfScope ps("gemv", st);
        switch (W->fmt) {
        case 1: launch_gemv_t<1, 0>(W, xb, yb, ns, S, st); break;
        case 2: launch_gemv_t<2, 0>(W, xb, yb, ns, S, st); break;
        case 3: launch_gemv_t<3, 0>(W, xb, yb, ns, S, st); break;
        default:
            if (W->flags & QF_GROUP32)
                launch_gemv_t<4, 1>(W, xb, yb, ns, S, st);
            else
                launch_gemv_t<4, 2>(W, xb, yb, ns, S, st);
            break;
        }
        int rc = after_launch("gemv");
        if (rc != COLI_OK)
            return rc;
    }
    return COLI_OK;
}

// ---------------------------------------------------------------------------
// Decode MoE block (S <= 4)
//
// colibri-strix "batched moe_block": per expert gate/up -> SiLU -> down, then
// the weighted scatter-add; "fuse shared expert": the shared expert is one
// more expert with weight 1 on every row.  Here: one launch computes every
// routed pair's hidden vector h = silu(G x) * (U x) (gate row j and up row j
// in the same wavefront -- one pass over x for both), a second launch computes
// every output row's sum over the pairs of its token of w * (D_e h), ascending
// k, plus the shared expert.
// ---------------------------------------------------------------------------

struct QView {  // one stack (or the shared matrix) as the kernels see it
    const uint8_t *q;
    const float *s;
    int64_t rb, q_stride, s_stride;
    int ng, gs;
};

static QView view_of(const coli_qtensor *t) {
    QView v;
    v.q = (const uint8_t *)t->q;
    v.s = t->s;
    v.rb = t->row_bytes;
    v.q_stride = t->q_stride;
    v.s_stride = t->s_stride;
    v.ng = t->ng;
    v.gs = t->gs > 0 ? t->gs : 1;
    return v;
}

__device__ __forceinline__ float silu_f32(float z) { return z / (1.0f + expf(-z)); }

// grid: x = ceil(F / (4 * R)), y = pair index (routed pairs, then shared rows)
template <int FMT, int R, int GM>
__global__ __launch_bounds__(256) void k_moe_gateup_decode(QView G, QView U, QView SG, QView SU,
                                                           const float *__restrict__ x,
                                                           const int32_t *__restrict__ ids, int S,
                                                           int K, int E, int F, int D,
                                                           float *__restrict__ h) {
    constexpr int CP = packet_cols(FMT), PB = packet_bytes(FMT);
    using Dot = PacketDot<FMT, GM>;
    const int lane = threadIdx.x & 63;
    const int p = blockIdx.y;
    const int j0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * R;
    if (j0 >= F)
        return;
    int s, e;
    QView g = G, u = U;
    if (p < S * K) {
        s = p / K;
        e = ids[p];
        if (e < 0 || e >= E) {  // left out: h = 0
            if (lane < R && j0 + lane < F)
                h[(int64_t)p * F + j0 + lane] = 0.f;
            return;
        }
    } else {
        s = p - S * K;
        e = 0;
        g = SG;
        u = SU;
    }
    const uint8_t *gq = g.q + (int64_t)e * g.q_stride;
    const uint8_t *uq = u.q + (int64_t)e * u.q_stride;
    const float *gsc = g.s + (int64_t)e * g.s_stride;
    const float *usc = u.s + (int64_t)e * u.s_stride;
    const float *xs = x + (int64_t)s * D;

    int64_t rowi[R];
#pragma unroll
    for (int r = 0; r < R; ++r) rowi[r] = (j0 + r < F) ? (j0 + r) : (F - 1);

    float ag[R][1], au[R][1];
#pragma unroll
    for (int r = 0; r < R; ++r) ag[r][0] = au[r][0] = 0.f;

    const int nchunks = (D + 64 * CP - 1) / (64 * CP);
    Packet<FMT> ng_[R], nu_[R];
    if (lane * CP < D) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            ng_[r] = load_packet<FMT>(gq + rowi[r] * g.rb + (int64_t)lane * PB);
            nu_[r] = load_packet<FMT>(uq + rowi[r] * u.rb + (int64_t)lane * PB);
        }
    }
    for (int c = 0; c < nchunks; ++c) {
        const int col0 = c * 64 * CP + lane * CP;
        Packet<FMT> cg[R], cu[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            cg[r] = ng_[r];
            cu[r] = nu_[r];
        }
        const int coln = col0 + 64 * CP;
        if (c + 1 < nchunks && coln < D) {
            const int64_t off = (int64_t)coln / CP * PB;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                ng_[r] = load_packet<FMT>(gq + rowi[r] * g.rb + off);
                nu_[r] = load_packet<FMT>(uq + rowi[r] * u.rb + off);
            }
        }
        if (col0 < D) {
            float xv[1][CP];
            load_x<CP>(xs + col0, xv[0]);
#pragma unroll
            for (int r = 0; r < R; ++r) {
                float s0, s1;
                packet_scales<GM>(gsc, rowi[r], g.ng, g.gs, col0, s0, s1);
                Dot::template run<1>(cg[r], xv, s0, s1, ag[r]);
                packet_scales<GM>(usc, rowi[r], u.ng, u.gs, col0, s0, s1);
                Dot::template run<1>(cu[r], xv, s0, s1, au[r]);
            }
        }
    }
    constexpr float inv = 1.0f / Mult<FMT>::value;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        float gv = wave_sum(ag[r][0]) * inv;
        float uv = wave_sum(au[r][0]) * inv;
        if (GM == 0) {
            gv *= gsc[rowi[r]];
            uv *= usc[rowi[r]];
        }
        if (lane == 0 && j0 + r < F)
            h[(int64_t)p * F + j0 + r] = silu_f32(gv) * uv;
    }
}

// grid: x = ceil(D / (4 * R)), y = token s
template <int FMT, int R, int GM>
__global__ __launch_bounds__(256) void k_moe_down_decode(QView Dn, QView SD, int has_shared,
                                                         const float *__restrict__ h,
                                                         const int32_t *__restrict__ ids,
                                                         const float *__restrict__ w, int S, int K,
                                                         int E, int F, int D,
                                                         float *__restrict__ out) {
    constexpr int CP = packet_cols(FMT), PB = packet_bytes(FMT);
    using Dot = PacketDot<FMT, GM>;
    const int lane = threadIdx.x & 63;
    const int s = blockIdx.y;
    const int o0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * R;
    if (o0 >= D)
        return;
    int64_t rowi[R];
#pragma unroll
    for (int r = 0; r < R; ++r) rowi[r] = (o0 + r < D) ? (o0 + r) : (D - 1);

    float tot[R];
#pragma unroll
    for (int r = 0; r < R; ++r) tot[r] = 0.f;

    const int nchunks = (F + 64 * CP - 1) / (64 * CP);
    const int npairs = K + (has_shared ? 1 : 0);
    for (int k = 0; k < npairs; ++k) {
        QView d = Dn;
        int e;
        float wk;
        int64_t p;
        if (k < K) {
            p = (int64_t)s * K + k;
            e = ids[p];
            if (e < 0 || e >= E)
                continue;
            wk = w[p];
        } else {
            p = (int64_t)S * K + s;
            e = 0;
            wk = 1.0f;
            d = SD;
        }
        const uint8_t *dq = d.q + (int64_t)e * d.q_stride;
        const float *dsc = d.s + (int64_t)e * d.s_stride;
        const float *hp = h + p * F;
        float part[R][1];
#pragma unroll
        for (int r = 0; r < R; ++r) part[r][0] = 0.f;
        for (int c = 0; c < nchunks; ++c) {
            const int col0 = c * 64 * CP + lane * CP;
            if (col0 < F) {
                Packet<FMT> pk[R];
#pragma unroll
                for (int r = 0; r < R; ++r)
                    pk[r] = load_packet<FMT>(dq + rowi[r] * d.rb + (int64_t)col0 / CP * PB);
                float xv[1][CP];
                load_x<CP>(hp + col0, xv[0]);
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    float s0, s1;
                    packet_scales<GM>(dsc, rowi[r], d.ng, d.gs, col0, s0, s1);
                    Dot::template run<1>(pk[r], xv, s0, s1, part[r]);
                }
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float f = (GM == 0) ? wk * dsc[rowi[r]] : wk;
            tot[r] = fmaf(f, part[r][0], tot[r]);
        }
    }
    constexpr float inv = 1.0f / Mult<FMT>::value;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const float v = wave_sum(tot[r]);
        if (lane == 0 && o0 + r < D)
            out[(int64_t)s * D + o0 + r] = v * inv;
    }
}

size_t moe_decode_ws_bytes(int S, int K, int F, int has_shared) {
    const size_t P = (size_t)S * K + (has_shared ? S : 0);
    return ((P * F * sizeof(float) + 255) / 256) * 256;
}

template <int FMT, int GM>
static int moe_decode_t(const MoeArgs &a, float *h) {
    const QView G = view_of(a.gate), U = view_of(a.up);
    const QView Dn = a.down ? view_of(a.down) : G;
    const bool has_sh = a.sg != nullptr;
    const QView SG = has_sh ? view_of(a.sg) : G, SU = has_sh ? view_of(a.su) : U;
    const QView SD = (has_sh && a.sd) ? view_of(a.sd) : Dn;
    const int P = a.S * a.K + (has_sh ? a.S : 0);
    {
        constexpr int R = 2;
        ProfScope ps("moe_gateup_decode", a.st);
        hipLaunchKernelGGL((k_moe_gateup_decode<FMT, R, GM>),
                           dim3((unsigned)((a.F + 4 * R - 1) / (4 * R)), (unsigned)P), dim3(256), 0,
                           a.st, G, U, SG, SU, a.x, a.ids, a.S, a.K, a.E, a.F, a.D, h);
        int rc = after_launch("moe_gateup_decode");
        if (rc != COLI_OK)
            return rc;
    }
    if (a.out == nullptr || a.down == nullptr)
        return COLI_OK;
    {
        constexpr int R = 2;
        ProfScope ps("moe_down_decode", a.st);
        hipLaunchKernelGGL((k_moe_down_decode<FMT, R, GM>),
                           dim3((unsigned)((a.D + 4 * R - 1) / (4 * R)), (unsigned)a.S), dim3(256),
                           0, a.st, Dn, SD, has_sh ? 1 : 0, h, a.ids, a.w, a.S, a.K, a.E, a.F, a.D,
                           a.out);
        return after_launch("moe_down_decode");
    }
}

int launch_moe_decode(const MoeArgs &a) {
    float *h = a.h_out ? a.h_out : (float *)a.ws;
    switch (a.gate->fmt) {
    case 1: return moe_decode_t<1, 0>(a, h);
    case 2: return moe_decode_t<2, 0>(a, h);
    case 3: return moe_decode_t<3, 0>(a, h);
    default: {
        // one scale per packet when every tensor's gs is a multiple of 32
        const coli_qtensor *all[6] = {a.gate, a.up, a.down, a.sg, a.su, a.sd};
        bool g32 = true;
        for (const coli_qtensor *t : all)
            if (t && !(t->flags & QF_GROUP32)) g32 = false;
        return g32 ? moe_decode_t<4, 1>(a, h) : moe_decode_t<4, 2>(a, h);
    }
    }
}

}  // namespace coli
