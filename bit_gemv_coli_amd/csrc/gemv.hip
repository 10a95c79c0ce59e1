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
#include <string.h>

#include "common.h"
#include "layer.h"

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
// Packet row-dot core
//
// A workgroup of 4 wavefronts owns a range of weight rows of one matrix (or of
// a gate/up pair of matrices) and the input vector(s) they multiply.  The
// inputs are staged once per workgroup into LDS in "packet-major" order --
// float4 j of lane l's packet in chunk c sits at ((c*NJ + j)*64 + l) -- so the
// 64 lanes of a wavefront read 64 consecutive float4 (no bank conflicts).
// Each wavefront takes R rows at a time and walks the row in chunks of 64
// packets; the packets and group scales of chunk c+1 are requested before
// chunk c is computed, and the inputs come from LDS, so the vector-memory
// queue always holds the next chunk.
// ---------------------------------------------------------------------------

// GM: 0 = per-row scale (fmt 1-3), 1 = one group scale per packet,
//     2 = two group scales per packet (16 inputs each).
template <int FMT, int GM>
struct PacketDot {
    static constexpr int CP = packet_cols(FMT);

    // acc[t] += scale * sum_j f_j * x[t][j]   (GM 1/2; GM 0 without scale)
    template <int NS>
    __device__ __forceinline__ static void run(const Packet<FMT> &pk, const f32x4 (&xv)[NS][CP / 4],
                                               float s0, float s1, float (&acc)[NS]) {
        float f[CP];
        decode_packet<FMT>(pk, f);
#pragma unroll
        for (int t = 0; t < NS; ++t) {
            float pa = 0.f, pb = 0.f;
            if constexpr (GM == 2) {
#pragma unroll
                for (int j = 0; j < CP / 8; ++j) {
                    pa = fmaf(f[4 * j + 0], xv[t][j].x, pa);
                    pa = fmaf(f[4 * j + 1], xv[t][j].y, pa);
                    pa = fmaf(f[4 * j + 2], xv[t][j].z, pa);
                    pa = fmaf(f[4 * j + 3], xv[t][j].w, pa);
                }
#pragma unroll
                for (int j = CP / 8; j < CP / 4; ++j) {
                    pb = fmaf(f[4 * j + 0], xv[t][j].x, pb);
                    pb = fmaf(f[4 * j + 1], xv[t][j].y, pb);
                    pb = fmaf(f[4 * j + 2], xv[t][j].z, pb);
                    pb = fmaf(f[4 * j + 3], xv[t][j].w, pb);
                }
                acc[t] = fmaf(s0, pa, acc[t]);
                acc[t] = fmaf(s1, pb, acc[t]);
            } else {
#pragma unroll
                for (int j = 0; j < CP / 4; ++j) {
                    pa = fmaf(f[4 * j + 0], xv[t][j].x, pa);
                    pb = fmaf(f[4 * j + 1], xv[t][j].y, pb);
                    pa = fmaf(f[4 * j + 2], xv[t][j].z, pa);
                    pb = fmaf(f[4 * j + 3], xv[t][j].w, pb);
                }
                if constexpr (GM == 1)
                    acc[t] = fmaf(s0, pa + pb, acc[t]);
                else
                    acc[t] += pa + pb;
            }
        }
    }
};

// Stage columns [c0*64*CP, c0*64*CP + nch*64*CP) (clipped to I) of NS input
// rows into LDS, packet-major.  lds holds NS * nch * 64 * CP floats.
template <int CP>
__device__ __forceinline__ void stage_x(const float *__restrict__ x, int64_t ldx, int NS, int I,
                                        int c0, int nch, f32x4 *lds) {
    constexpr int NJ = CP / 4, UN = 8;
    const int colb = c0 * 64 * CP;
    const int ncols = min(I - colb, nch * 64 * CP);
    const int n4 = ncols / 4;
    const int total = NS * n4;
    // UN loads in flight per thread before the LDS writes
    for (int base = 0; base < total; base += UN * (int)blockDim.x) {
        f32x4 v[UN];
#pragma unroll
        for (int u = 0; u < UN; ++u) {
            const int idx = min(base + u * (int)blockDim.x + (int)threadIdx.x, total - 1);
            const int t = idx / n4, r = idx - t * n4;
            v[u] = gload<f32x4>(x + t * ldx + colb + 4 * r);
        }
#pragma unroll
        for (int u = 0; u < UN; ++u) {
            const int idx = base + u * (int)blockDim.x + (int)threadIdx.x;
            if (idx < total) {
                const int t = idx / n4, r = idx - t * n4;
                const int col = 4 * r;
                const int c = col / (64 * CP), rem = col - c * 64 * CP;
                const int l = rem / CP, j = (rem % CP) / 4;
                lds[((t * nch + c) * NJ + j) * 64 + l] = v[u];
            }
        }
    }
}

// gshift = log2(gs) when gs is a power of two (a shift instead of a divide)
__device__ __forceinline__ int group_of(int col, int gs, int gshift) {
    return gshift >= 0 ? (col >> gshift) : (col / gs);
}

template <int GM>
__device__ __forceinline__ void packet_scales(const float *__restrict__ s, int64_t row, int ng,
                                              int gs, int gshift, int col0, float &s0, float &s1) {
    if constexpr (GM == 1) {
        s0 = gload<float>(s + row * ng + group_of(col0, gs, gshift));
        s1 = 0.f;
    } else if constexpr (GM == 2) {
        s0 = gload<float>(s + row * ng + group_of(col0, gs, gshift));
        s1 = gload<float>(s + row * ng + group_of(col0 + 16, gs, gshift));
    } else {
        s0 = s1 = 0.f;
    }
}

// Epilogues
enum { EPI_Y = 0, EPI_SILU = 1, EPI_PART = 2 };

struct RowDotArgs {
    // weight stacks (NMAT of them, same shape and format): matrix e of stack m
    // starts at q[m] + e*q_stride, its scales at s[m] + e*s_stride
    const uint8_t *q[2];
    const float *s[2];
    const uint8_t *sq[2];  // shared-expert matrices (MoE modes)
    const float *ss[2];
    int64_t rb, q_stride, s_stride;
    int ng, gs, gshift;    // gshift = log2(gs) if gs is a power of two, else -1
    int O, I;              // rows per matrix, inputs
    const float *x;        // inputs
    int64_t ldx;
    // MoE pair mapping (mode 1): pair p = blockIdx.y; p < S*K routed, else shared
    int moe;
    const int32_t *ids;
    int S, K, E;
    int x_by_pair;         // inputs row = pair (down) instead of token (gate/up)
    float *out;
    int Sy;                // EPI_Y: input rows per matrix in the output
    int rows_per_wg;       // multiple of 4*R
    int segc;              // chunks per LDS segment
    int nseg;              // number of segments
};

template <int FMT, int GM, int NS, int R, int NMAT, int EPI>
__global__ __launch_bounds__(256) void k_rowdot(RowDotArgs a) {
    constexpr int CP = packet_cols(FMT), PB = packet_bytes(FMT), NJ = CP / 4;
    // chunks requested together: up to 3 (a 6144-input int4 row) when the
    // wavefront holds few rows, fewer when it holds many
    constexpr int NB = (NMAT * R * NS <= 4) ? 3 : ((NMAT * R * NS <= 8) ? 2 : 1);
    using Dot = PacketDot<FMT, GM>;
    extern __shared__ f32x4 xl[];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int I = a.I, O = a.O;

    // --- which matrix and which input rows --------------------------------
    const uint8_t *q[NMAT];
    const float *sc[NMAT];
    const float *xin;
    int64_t p = blockIdx.y;
    int valid = 1;
    if (a.moe) {
        int e, s;
        bool shared = p >= (int64_t)a.S * a.K;
        if (!shared) {
            s = (int)(p / a.K);
            e = gload<int32_t>(a.ids + p);
            valid = (e >= 0 && e < a.E);
        } else {
            s = (int)(p - (int64_t)a.S * a.K);
            e = 0;
        }
#pragma unroll
        for (int m = 0; m < NMAT; ++m) {
            q[m] = (shared ? a.sq[m] : a.q[m]) + (int64_t)(valid ? e : 0) * a.q_stride;
            sc[m] = (shared ? a.ss[m] : a.s[m]) + (int64_t)(valid ? e : 0) * a.s_stride;
        }
        xin = a.x + (a.x_by_pair ? p : (int64_t)s) * a.ldx;
    } else {
#pragma unroll
        for (int m = 0; m < NMAT; ++m) {
            q[m] = a.q[m] + p * a.q_stride;
            sc[m] = a.s[m] + p * a.s_stride;
        }
        xin = a.x;
    }
    const int row_beg = blockIdx.x * a.rows_per_wg;
    const int row_end = min(O, row_beg + a.rows_per_wg);
    if (!valid) {
        // pair left out (expert id outside [0,E)): its hidden vector is zero
        if (EPI == EPI_SILU)
            for (int j = row_beg + threadIdx.x; j < row_end; j += blockDim.x)
                a.out[p * O + j] = 0.f;
        return;
    }
    const int nch_all = (I + 64 * CP - 1) / (64 * CP);

    if (a.nseg == 1) {  // the whole input fits: stage once
        stage_x<CP>(xin, a.ldx, NS, I, 0, nch_all, xl);
        __syncthreads();
    }

    for (int rg = row_beg + wave * R; rg < row_beg + a.rows_per_wg; rg += 4 * R) {
        const bool live = rg < row_end;
        int64_t rowi[R];
#pragma unroll
        for (int r = 0; r < R; ++r) rowi[r] = min(rg + r, O - 1);
        float acc[NMAT][R][NS];
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int t = 0; t < NS; ++t) acc[m][r][t] = 0.f;

        for (int sg = 0; sg < a.nseg; ++sg) {
            const int c0 = sg * a.segc;
            const int nch = min(a.segc, nch_all - c0);
            if (a.nseg > 1) {
                __syncthreads();
                stage_x<CP>(xin, a.ldx, NS, I, c0, nch, xl);
                __syncthreads();
            }
            if (!live)
                continue;
            // chunks in batches of NB: every packet and scale of a batch is
            // requested before any is used, with no branches between the
            // requests (out-of-range chunks/lanes re-read the row's last
            // packet and are not used); latency is hidden by the other
            // wavefronts of the CU.
            const int last_pk = I / CP - 1;
            for (int cb = 0; cb < nch; cb += NB) {
                Packet<FMT> cq[NB][NMAT][R];
                float cs0[NB][NMAT][R], cs1[NB][NMAT][R];
#pragma unroll
                for (int i = 0; i < NB; ++i) {
                    const int pk = min((c0 + cb + i) * 64 + lane, last_pk);
#pragma unroll
                    for (int m = 0; m < NMAT; ++m)
#pragma unroll
                        for (int r = 0; r < R; ++r) {
                            packet_scales<GM>(sc[m], rowi[r], a.ng, a.gs, a.gshift, pk * CP,
                                              cs0[i][m][r], cs1[i][m][r]);
                            cq[i][m][r] = load_packet<FMT>(q[m] + rowi[r] * a.rb + (int64_t)pk * PB);
                        }
                }
#pragma unroll
                for (int i = 0; i < NB; ++i) {
                    const int col0 = (c0 + cb + i) * 64 * CP + lane * CP;
                    if (cb + i < nch && col0 < I) {
                        f32x4 xv[NS][NJ];
#pragma unroll
                        for (int t = 0; t < NS; ++t)
#pragma unroll
                            for (int j = 0; j < NJ; ++j)
                                xv[t][j] = xl[((t * nch + cb + i) * NJ + j) * 64 + lane];
#pragma unroll
                        for (int m = 0; m < NMAT; ++m)
#pragma unroll
                            for (int r = 0; r < R; ++r)
                                Dot::template run<NS>(cq[i][m][r], xv, cs0[i][m][r], cs1[i][m][r],
                                                      acc[m][r]);
                    }
                }
            }
        }
        if (!live)
            continue;
        // --- reduce across the wavefront and write -----------------------
        constexpr float inv = 1.0f / Mult<FMT>::value;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int row = rg + r;
            if constexpr (EPI == EPI_SILU) {
                float g = wave_sum(acc[0][r][0]) * inv;
                float u = wave_sum(acc[NMAT - 1][r][0]) * inv;
                if (GM == 0) {
                    g *= gload<float>(sc[0] + rowi[r]);
                    u *= gload<float>(sc[NMAT - 1] + rowi[r]);
                }
                if (lane == 0 && row < row_end)
                    a.out[p * O + row] = (g / (1.0f + expf(-g))) * u;
            } else {
#pragma unroll
                for (int t = 0; t < NS; ++t) {
                    float v = wave_sum(acc[0][r][t]) * inv;
                    if (GM == 0)
                        v *= gload<float>(sc[0] + rowi[r]);
                    if (lane == 0 && row < row_end) {
                        if (EPI == EPI_Y)
                            a.out[(p * a.Sy + t) * O + row] = v;
                        else
                            a.out[p * O + row] = v;
                    }
                }
            }
        }
    }
}

#ifndef COLI_VALU_WANT_WGS
#define COLI_VALU_WANT_WGS 1024
#endif
// LDS budget for the staged inputs of one workgroup.
constexpr int LDS_X_BYTES = 32 * 1024;

template <int FMT>
static void plan_segments(int I, int NS, int &segc, int &nseg, size_t &lds) {
    constexpr int CP = packet_cols(FMT);
    const int nch = (I + 64 * CP - 1) / (64 * CP);
    const int per_chunk = NS * 64 * CP * 4;
    segc = LDS_X_BYTES / per_chunk;
    if (segc < 1) segc = 1;
    if (segc >= nch) segc = nch;
    nseg = (nch + segc - 1) / segc;
    lds = (size_t)segc * per_chunk;
}

// Rows per workgroup: enough workgroups to fill the chip, and enough rows
// per workgroup to amortize the input staging.
static int rows_per_wg(int O, int groups, int R, int want_wgs) {
    const int unit = 4 * R;
    int per = (int)(((int64_t)O * groups + want_wgs - 1) / want_wgs);
    per = ((per + unit - 1) / unit) * unit;
    if (per < unit) per = unit;
    const int cap = ((O + unit - 1) / unit) * unit;
    return per > cap ? cap : per;
}

template <int FMT, int GM, int NS, int R, int NMAT, int EPI>
static void launch_rowdot(const RowDotArgs &a0, int groups, hipStream_t st) {
    RowDotArgs a = a0;
    size_t lds;
    plan_segments<FMT>(a.I, NS, a.segc, a.nseg, lds);
    const dim3 grid((unsigned)((a.O + a.rows_per_wg - 1) / a.rows_per_wg), (unsigned)groups);
    hipLaunchKernelGGL((k_rowdot<FMT, GM, NS, R, NMAT, EPI>), grid, dim3(256), lds, st, a);
}

static RowDotArgs args_for(const coli_qtensor *W) {
    RowDotArgs a;
    memset(&a, 0, sizeof a);
    a.q[0] = a.q[1] = (const uint8_t *)W->q;
    a.s[0] = a.s[1] = W->s;
    a.rb = W->row_bytes;
    a.q_stride = W->q_stride;
    a.s_stride = W->s_stride;
    a.ng = W->ng;
    a.gs = W->gs > 0 ? W->gs : 1;
    a.gshift = -1;
    for (int b = 0; b < 31; ++b)
        if ((1 << b) == a.gs) a.gshift = b;
    a.O = W->O;
    a.I = W->I;
    return a;
}

template <int FMT, int GM>
static void launch_gemv_t(const coli_qtensor *W, const float *x, float *y, int S, int Sy,
                          hipStream_t st) {
    RowDotArgs a = args_for(W);
    a.x = x;
    a.ldx = W->I;
    a.out = y;
    a.Sy = Sy;
    constexpr int R = 2;
    a.rows_per_wg = rows_per_wg(W->O, W->n, R, 2048);
    switch (S) {
    case 1: launch_rowdot<FMT, GM, 1, R, 1, EPI_Y>(a, W->n, st); break;
    case 2: launch_rowdot<FMT, GM, 2, R, 1, EPI_Y>(a, W->n, st); break;
    case 3: launch_rowdot<FMT, GM, 3, R, 1, EPI_Y>(a, W->n, st); break;
    default: launch_rowdot<FMT, GM, 4, R, 1, EPI_Y>(a, W->n, st); break;
    }
}

static int group_mode(const coli_qtensor *const *ts, int n) {
    // 1: every tensor's gs is a multiple of 32; 2: multiples of 16
    for (int i = 0; i < n; ++i)
        if (ts[i] && !(ts[i]->flags & QF_GROUP32)) return 2;
    return 1;
}

// y = W x for S input rows.  Packet kernels take up to 4 input rows per
// launch (larger S is split into blocks of 4); the fallback takes any S.
static int launch_gemv_y(const coli_qtensor *W, const float *x, float *y, int S, hipStream_t st);

int launch_gemv(const coli_qtensor *W, const float *x, float *y, int S, hipStream_t st,
                const float *radd, float *ysum) {
    if (ysum == nullptr)
        return launch_gemv_y(W, x, y, S, st);
    if (W->n != 1 || radd == nullptr)
        return decline("gemv: a residual add takes one matrix and its addend");
    const bool fast = (W->flags & QF_FAST) &&
                      (W->fmt != 4 || (W->flags & (QF_GROUP32 | QF_GROUP16))) &&
                      ((uintptr_t)x % 16 == 0);
    if (fast && S <= 4 && decode_kernel_mode() == 0) {
        const int r = launch_mgemv(W, x, y, S, st, radd, ysum);
        if (r == 1)
            return COLI_OK;
        if (r < 0)
            return COLI_HIP_ERROR;
    }
    const int rc = launch_gemv_y(W, x, y, S, st);
    if (rc != COLI_OK)
        return rc;
    return launch_residual_add(radd, y, ysum, (int64_t)S * W->n * W->O, st);
}

static int launch_gemv_y(const coli_qtensor *W, const float *x, float *y, int S, hipStream_t st) {
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
    if (S <= 4 && decode_kernel_mode() == 0) {
        const int r = launch_mgemv(W, x, y, S, st);
        if (r == 1)
            return COLI_OK;
        if (r < 0)
            return COLI_HIP_ERROR;
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
            if (group_mode(&W, 1) == 1)
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
// the weighted scatter-add; shared-expert fusion commit: the shared expert is one
// more expert with weight 1 on every row.  Here, per routed pair p = s*K+k
// (then one pair per token for the shared expert):
//   launch 1  h[p]  = silu(G_e x_s) * (U_e x_s)   gate row j and up row j in
//                                                 the same wavefront: one pass
//   launch 2  yp[p] = D_e h[p]
//   launch 3  out[s] = sum_k w[s][k] yp[s*K+k] (+ yp[shared s]), ascending k,
//             one thread per output, no atomics: reruns are bit-identical.
//             (The matrix-core path folds launch 3 into launch 2.)
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void k_moe_combine(const float *__restrict__ yp,
                                                     const int32_t *__restrict__ ids,
                                                     const float *__restrict__ w, int S, int K,
                                                     int E, int D, int has_shared,
                                                     float *__restrict__ out) {
    const int s = blockIdx.y;
    const int o = blockIdx.x * blockDim.x + threadIdx.x;
    if (o >= D)
        return;
    // all K loads of a chunk are issued before the sums (ascending k)
    float acc = 0.f;
    for (int k0 = 0; k0 < K; k0 += 8) {
        float v[8], wk[8];
        bool ok[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int k = min(k0 + u, K - 1);
            const int64_t p = (int64_t)s * K + k;
            const int e = ids[p];
            ok[u] = (k0 + u < K) && e >= 0 && e < E;
            wk[u] = w[p];
            v[u] = yp[p * D + o];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
            acc = ok[u] ? fmaf(wk[u], v[u], acc) : acc;
    }
    if (has_shared)
        acc += yp[((int64_t)S * K + s) * D + o];
    out[(int64_t)s * D + o] = acc;
}

size_t moe_decode_ws_bytes(int S, int K, int F, int D, int has_shared) {
    const size_t P = (size_t)S * K + (has_shared ? S : 0);
    const size_t hb = ((P * F * sizeof(float) + 255) / 256) * 256;
    const size_t yb = ((P * D * sizeof(float) + 255) / 256) * 256;
    const size_t cb = (((size_t)(D + 15) / 16 * sizeof(int) + 255) / 256) * 256;  // counters
    return hb + yb + cb;
}

static void fill_pair_args(RowDotArgs &a, const coli_qtensor *m0, const coli_qtensor *m1,
                           const coli_qtensor *s0, const coli_qtensor *s1) {
    a = args_for(m0);
    a.q[1] = (const uint8_t *)m1->q;
    a.s[1] = m1->s;
    a.sq[0] = s0 ? (const uint8_t *)s0->q : a.q[0];
    a.ss[0] = s0 ? s0->s : a.s[0];
    a.sq[1] = s1 ? (const uint8_t *)s1->q : a.q[1];
    a.ss[1] = s1 ? s1->s : a.s[1];
    a.moe = 1;
}

template <int FMT, int GM>
static int moe_decode_t(const MoeArgs &a, float *h, float *yp) {
    const bool has_sh = a.sg != nullptr;
    const int P = a.S * a.K + (has_sh ? a.S : 0);
    constexpr int R = 2;
    {
        RowDotArgs r;
        fill_pair_args(r, a.gate, a.up, a.sg, a.su);
        r.x = a.x;
        r.ldx = a.D;
        r.ids = a.ids;
        r.S = a.S; r.K = a.K; r.E = a.E;
        r.x_by_pair = 0;
        r.out = h;
        r.rows_per_wg = rows_per_wg(a.F, P, R, COLI_VALU_WANT_WGS);
        ProfScope ps("moe_gateup_decode", a.st);
        launch_rowdot<FMT, GM, 1, R, 2, EPI_SILU>(r, P, a.st);
        int rc = after_launch("moe_gateup_decode");
        if (rc != COLI_OK)
            return rc;
    }
    if (a.out == nullptr || a.down == nullptr)
        return COLI_OK;
    {
        RowDotArgs r;
        fill_pair_args(r, a.down, a.down, a.sd, a.sd);
        r.x = h;
        r.ldx = a.F;
        r.ids = a.ids;
        r.S = a.S; r.K = a.K; r.E = a.E;
        r.x_by_pair = 1;
        r.out = yp;
        r.rows_per_wg = rows_per_wg(a.D, P, R, 1024);
        ProfScope ps("moe_down_decode", a.st);
        launch_rowdot<FMT, GM, 1, R, 1, EPI_PART>(r, P, a.st);
        int rc = after_launch("moe_down_decode");
        if (rc != COLI_OK)
            return rc;
    }
    return COLI_OK;
}

static int moe_combine(const MoeArgs &a, const float *yp) {
    ProfScope ps("moe_combine", a.st);
    hipLaunchKernelGGL(k_moe_combine, dim3((unsigned)((a.D + 255) / 256), (unsigned)a.S),
                       dim3(256), 0, a.st, yp, a.ids, a.w, a.S, a.K, a.E, a.D,
                       a.sg != nullptr ? 1 : 0, a.out);
    return after_launch("moe_combine");
}

int launch_moe_decode(const MoeArgs &a) {
    const bool has_sh = a.sg != nullptr;
    const size_t P = (size_t)a.S * a.K + (has_sh ? a.S : 0);
    float *h = a.h_out ? a.h_out : (float *)a.ws;
    float *yp = (float *)((char *)a.ws + ((P * a.F * sizeof(float) + 255) / 256) * 256);
    int *cnt = (int *)((char *)yp + ((P * a.D * sizeof(float) + 255) / 256) * 256);
    const coli_qtensor *all[6] = {a.gate, a.up, a.down, a.sg, a.su, a.sd};
    int rc = 0;
    if (decode_kernel_mode() == 0)
        rc = launch_mgemv_moe(a, h, yp, cnt);  // matrix-core kernels, combine folded in
    if (rc < 0)
        return COLI_HIP_ERROR;
    if (rc == 1)
        return COLI_OK;  // (the residual add, if asked for, is in the combine)
    {
        switch (a.gate->fmt) {
        case 1: rc = moe_decode_t<1, 0>(a, h, yp); break;
        case 2: rc = moe_decode_t<2, 0>(a, h, yp); break;
        case 3: rc = moe_decode_t<3, 0>(a, h, yp); break;
        default:
            rc = group_mode(all, 6) == 1 ? moe_decode_t<4, 1>(a, h, yp)
                                         : moe_decode_t<4, 2>(a, h, yp);
        }
        if (rc != COLI_OK)
            return rc;
    }
    if (a.out == nullptr || a.down == nullptr)
        return COLI_OK;
    rc = moe_combine(a, yp);
    if (rc != COLI_OK || a.resid == nullptr)
        return rc;
    return launch_residual_add(a.resid, a.out, a.out_res, (int64_t)a.S * a.D, a.st);
}

}  // namespace coli
