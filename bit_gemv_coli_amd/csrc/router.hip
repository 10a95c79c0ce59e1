// router.hip -- the MoE router and its exact top-K selection on the GPU
// (colibri-strix commit log, full decode layer commit: router matvec + sigmoid, then greedy argmax over sigmoid + bias
// with the CPU's tie order, top-p truncation, norm_topk, routed_scale).
//
// Decisions are taken on f64 numbers: every logit is a sum of exact f64
// products of f32 operands, the sigmoid and the key p + bias are f64, so the
// picks do not depend on the order the GPU sums in (beyond 2^-53 relative),
// and equal logits give equal keys and the smaller expert index.
//   k_router_logits     z[s][e] for up to 4 input rows (decode): a workgroup
//                       per expert, its wavefronts on quarters of the inputs,
//                       lanes on 16-byte loads, one f64 FMA per product,
//                       wavefront sums then quarters added in order; in a
//                       decode layer it also applies the RMSNorm in front of
//                       the router (every workgroup reduces the rows the
//                       way k_rmsnorm does, the first writes them out);
//   k_router_logits_mx  z for many rows: f64 16x16x4 matrix-core products
//                       (f32 operands widened exactly), a 32 x 32 block of
//                       (rows, experts) per workgroup, the inputs split over
//                       its four wavefronts and over P workgroups; partial sums
//                       added in a fixed order;
//   k_router_topk       one workgroup per input row: sigmoid and key per
//                       expert into LDS, every expert's rank under (key
//                       descending, index ascending) counted by four threads
//                       over quarters of the experts, the K smallest ranks
//                       are the greedy picks in order; top-p, norm_topk and
//                       routed_scale per pick.
#include <algorithm>

#include "common.h"
#include "layer.h"
#include "rms.h"

namespace coli {

constexpr int RT_MAXE = 512;   // experts (8 per lane)
constexpr int RT_MAXK = 16;    // picks per row
constexpr int RT_MAXP = 8;     // partial sums of the many-row logits

__device__ __forceinline__ double rt_shfl_xor(double v, int m) {
    const int2 p = __builtin_bit_cast(int2, v);
    int2 q;
    q.x = __shfl_xor(p.x, m);
    q.y = __shfl_xor(p.y, m);
    return __builtin_bit_cast(double, q);
}

// z for TE experts x TT input rows per wavefront (WS == 1), or per
// workgroup with its four wavefronts on four contiguous quarters of the
// inputs (WS == 4, quarters added in wavefront order).  Every lane takes 4
// consecutive inputs (one 16-byte load per expert row and input row) of each
// 256-input stretch, U stretches requested before they are used.
// NORM (WS == 4, VEC): x holds the rows before the RMSNorm in front of the
// router; every workgroup reduces them to 1 / rms exactly as k_rmsnorm does
// and normalises each input as it loads it (the same f32 values k_rmsnorm
// writes), and the first workgroup also writes the normalised rows to xn.
template <int TT, int TE, int U, bool VEC, int WS, bool NORM = false>
__global__ __launch_bounds__(256) void k_router_logits(const float *__restrict__ x, int S, int D,
                                                       const float *__restrict__ R, int E,
                                                       double *__restrict__ z,
                                                       const float *__restrict__ lnw = nullptr,
                                                       double eps = 0.0,
                                                       float *__restrict__ xn = nullptr) {
    static_assert(WS == 1 || WS == 4, "one or four wavefronts per block of experts");
    static_assert(!NORM || (WS == 4 && VEC), "the folded norm takes whole workgroups, 16-byte rows");
    __shared__ double sp[WS == 4 ? 3 : 1][TE * TT];
    __shared__ double npart[NORM ? TT : 1][4];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int e0 = (WS == 4 ? (int)blockIdx.x : (int)blockIdx.x * 4 + wv) * TE;
    const int s0 = blockIdx.y * TT;
    if (e0 >= E)
        return;  // whole wavefront (whole workgroup when WS == 4)
    const int q = WS == 4 ? wv : 0;
    const int dlo = (int)((int64_t)(D / 4) * q / WS) * 4;
    const int dhi = q == WS - 1 ? D : (int)((int64_t)(D / 4) * (q + 1) / WS) * 4;
    // rows past the end read the last row again and are not written
    const float *rr[TE];
    const float *xr[TT];
#pragma unroll
    for (int i = 0; i < TE; ++i) rr[i] = R + (int64_t)min(e0 + i, E - 1) * D;
#pragma unroll
    for (int t = 0; t < TT; ++t) xr[t] = x + (int64_t)min(s0 + t, S - 1) * D;
    // one batch of U stretches: expert rows, input rows and (NORM) the norm
    // weights; the first batch is requested before the norm's own loads, so
    // all of it arrives in the same memory round trip
    f32x4 rv[U][TE], xv[U][TT], gv[U];
    const int nfull = VEC ? dlo + (dhi - dlo) / (256 * U) * (256 * U) : dlo;
    auto load_batch = [&](int d0) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int d = d0 + 256 * u + 4 * lane;
#pragma unroll
            for (int i = 0; i < TE; ++i) rv[u][i] = gload<f32x4>(rr[i] + d);
#pragma unroll
            for (int t = 0; t < TT; ++t) xv[u][t] = gload<f32x4>(xr[t] + d);
            if constexpr (NORM)
                gv[u] = lnw ? gload<f32x4>(lnw + d) : f32x4{1.f, 1.f, 1.f, 1.f};
        }
    };
    if constexpr (VEC) {
        if (dlo < nfull)
            load_batch(dlo);
    }
    double inv[TT];
    if constexpr (NORM) {
#pragma unroll
        for (int t = 0; t < TT; ++t) inv[t] = row_rms_inv<true>(xr[t], D, eps, npart[t]);
        if (blockIdx.x == 0)
            for (int t = 0; t < TT && s0 + t < S; ++t)
                for (int d = 4 * (int)threadIdx.x; d < D; d += 1024) {
                    const f32x4 v = gload<f32x4>(xr[t] + d);
                    const f32x4 g = lnw ? gload<f32x4>(lnw + d) : f32x4{1.f, 1.f, 1.f, 1.f};
                    *(f32x4 *)(xn + (int64_t)(s0 + t) * D + d) =
                        f32x4{rms_apply(v.x, inv[t], g.x), rms_apply(v.y, inv[t], g.y),
                              rms_apply(v.z, inv[t], g.z), rms_apply(v.w, inv[t], g.w)};
                }
    }
    // the normalised inputs (NORM) of row t at d
    auto norm4 = [&](f32x4 v, int t, int d) -> f32x4 {
        if constexpr (NORM) {
            const f32x4 g = lnw ? gload<f32x4>(lnw + d) : f32x4{1.f, 1.f, 1.f, 1.f};
            return f32x4{rms_apply(v.x, inv[t], g.x), rms_apply(v.y, inv[t], g.y),
                         rms_apply(v.z, inv[t], g.z), rms_apply(v.w, inv[t], g.w)};
        } else {
            return v;
        }
    };
    double acc[TE][TT];
#pragma unroll
    for (int i = 0; i < TE; ++i)
#pragma unroll
        for (int t = 0; t < TT; ++t) acc[i][t] = 0.0;
    if constexpr (VEC) {
        for (int d0 = dlo; d0 < nfull; d0 += 256 * U) {
            if (d0 != dlo)
                load_batch(d0);
            if constexpr (NORM) {
#pragma unroll
                for (int u = 0; u < U; ++u)
#pragma unroll
                    for (int t = 0; t < TT; ++t) {
                        const f32x4 v = xv[u][t], g = gv[u];
                        xv[u][t] = f32x4{rms_apply(v.x, inv[t], g.x), rms_apply(v.y, inv[t], g.y),
                                         rms_apply(v.z, inv[t], g.z), rms_apply(v.w, inv[t], g.w)};
                    }
            }
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int i = 0; i < TE; ++i)
#pragma unroll
                    for (int t = 0; t < TT; ++t) {
                        acc[i][t] = fma((double)rv[u][i].x, (double)xv[u][t].x, acc[i][t]);
                        acc[i][t] = fma((double)rv[u][i].y, (double)xv[u][t].y, acc[i][t]);
                        acc[i][t] = fma((double)rv[u][i].z, (double)xv[u][t].z, acc[i][t]);
                        acc[i][t] = fma((double)rv[u][i].w, (double)xv[u][t].w, acc[i][t]);
                    }
        }
        for (int d = nfull + 4 * lane; d < dhi; d += 256) {
#pragma unroll
            for (int i = 0; i < TE; ++i) {
                const f32x4 r = gload<f32x4>(rr[i] + d);
#pragma unroll
                for (int t = 0; t < TT; ++t) {
                    const f32x4 v = norm4(gload<f32x4>(xr[t] + d), t, d);
                    acc[i][t] = fma((double)r.x, (double)v.x, acc[i][t]);
                    acc[i][t] = fma((double)r.y, (double)v.y, acc[i][t]);
                    acc[i][t] = fma((double)r.z, (double)v.z, acc[i][t]);
                    acc[i][t] = fma((double)r.w, (double)v.w, acc[i][t]);
                }
            }
        }
    } else {
        for (int d = dlo + lane; d < dhi; d += 64)
#pragma unroll
            for (int i = 0; i < TE; ++i) {
                const double r = (double)rr[i][d];
#pragma unroll
                for (int t = 0; t < TT; ++t) acc[i][t] = fma(r, (double)xr[t][d], acc[i][t]);
            }
    }
    // wavefront sums; lane i * TT + t keeps (expert e0 + i, row s0 + t)
    double mine = 0.0;
#pragma unroll
    for (int i = 0; i < TE; ++i)
#pragma unroll
        for (int t = 0; t < TT; ++t) {
            double v = acc[i][t];
#pragma unroll
            for (int m = 32; m >= 1; m >>= 1) v += rt_shfl_xor(v, m);
            mine = (lane == i * TT + t) ? v : mine;
        }
    if constexpr (WS == 4) {
        if (wv > 0 && lane < TE * TT)
            sp[wv - 1][lane] = mine;
        __syncthreads();
        if (wv > 0)
            return;
        if (lane < TE * TT)
            mine = ((mine + sp[0][lane]) + sp[1][lane]) + sp[2][lane];
    }
    if (lane < TE * TT) {
        const int e = e0 + lane / TT, s = s0 + lane % TT;
        if (e < E && s < S)
            z[(int64_t)s * E + e] = mine;
    }
}

typedef double f64x4 __attribute__((ext_vector_type(4)));

// Partial logits zp[p][s][e] over the p-th of P shares of the inputs, for the
// 32 rows x 32 experts at (blockIdx.y, blockIdx.x).  Matrix-core layout of
// the f64 16x16x4 product: lane l holds A[l%16][l/16] and B[l/16][l%16] and
// keeps D[l/16 + 4v][l%16] in its v-th f64 of the result.  A lane loads 4 consecutive inputs d+4g..d+4g+3
// (g = l/16) of its row and of its expert, and product c of the four uses
// input d+4g+c as contraction index g, so every 16 inputs are 4 products.
// Needs D % 4 == 0 and 16-byte aligned rows.
template <int U>
__global__ __launch_bounds__(256) void k_router_logits_mx(const float *__restrict__ x, int S, int D,
                                                          const float *__restrict__ R, int E,
                                                          double *__restrict__ zp) {
    __shared__ double sred[3][16][64];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int i16 = lane & 15, g = lane >> 4;
    const int s0 = blockIdx.y * 32, e0 = blockIdx.x * 32;
    const int nst = (D + 15) / 16;
    const int part = blockIdx.z * 4 + wv, nparts = gridDim.z * 4;
    const int st0 = (int)((int64_t)nst * part / nparts);
    const int st1 = (int)((int64_t)nst * (part + 1) / nparts);
    // rows and experts past the end read the last one again and are not written
    const float *xa[2], *rb[2];
#pragma unroll
    for (int a = 0; a < 2; ++a) {
        xa[a] = x + (int64_t)min(s0 + 16 * a + i16, S - 1) * D + 4 * g;
        rb[a] = R + (int64_t)min(e0 + 16 * a + i16, E - 1) * D + 4 * g;
    }
    f64x4 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = f64x4{0.0, 0.0, 0.0, 0.0};
    auto mma = [&](const f32x4 (&xv)[2], const f32x4 (&rv)[2]) {
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int b = 0; b < 2; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_f64_16x16x4f64((double)xv[a][c], (double)rv[b][c],
                                                                    acc[a][b], 0, 0, 0);
    };
    // whole steps through a ring of U register slots: slot u is used for
    // step st + u and refilled at once with step st + u + U (the last whole
    // step again near the end, so every load stays in bounds)
    const int stf = max(st0, min(st1, D / 16));
    int st = st0;
    if (stf - st0 >= U) {
        f32x4 rx[U][2], rr[U][2];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int a = 0; a < 2; ++a) {
                rx[u][a] = gload<f32x4>(xa[a] + (st0 + u) * 16);
                rr[u][a] = gload<f32x4>(rb[a] + (st0 + u) * 16);
            }
        // keeps the first fill and the refills distinct loads, so the
        // compiler cannot merge them into one load at the top of the loop
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int a = 0; a < 2; ++a) asm volatile("" : "+v"(rx[u][a]), "+v"(rr[u][a]));
        for (; st + U <= stf; st += U) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                mma(rx[u], rr[u]);
                const int sn = min(st + U + u, stf - 1) * 16;
#pragma unroll
                for (int a = 0; a < 2; ++a) {
                    rx[u][a] = gload<f32x4>(xa[a] + sn);
                    rr[u][a] = gload<f32x4>(rb[a] + sn);
                }
            }
        }
    }
    // the rest one step at a time; inputs past D count as zeros
    for (; st < st1; ++st) {
        const int d = st * 16;
        const bool ok = d + 4 * g < D;
        f32x4 xv[2], rv[2];
#pragma unroll
        for (int a = 0; a < 2; ++a) {
            xv[a] = ok ? gload<f32x4>(xa[a] + d) : f32x4{0.f, 0.f, 0.f, 0.f};
            rv[a] = ok ? gload<f32x4>(rb[a] + d) : f32x4{0.f, 0.f, 0.f, 0.f};
        }
        mma(xv, rv);
    }
    // the four wavefronts' sums, added in wavefront order
    if (wv > 0) {
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int v = 0; v < 4; ++v) sred[wv - 1][(a * 2 + b) * 4 + v][lane] = acc[a][b][v];
    }
    __syncthreads();
    if (wv > 0)
        return;
#pragma unroll
    for (int q = 0; q < 3; ++q)
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int v = 0; v < 4; ++v) acc[a][b][v] += sred[q][(a * 2 + b) * 4 + v][lane];
    double *zo = zp + (int64_t)blockIdx.z * S * E;
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const int e = e0 + 16 * b + i16;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int s = s0 + 16 * a + g + 4 * v;
                if (s < S && e < E)
                    zo[(int64_t)s * E + e] = acc[a][b][v];
            }
        }
}

// One workgroup (1024 threads) per input row; z is the sum of P partial
// logits zp[p][s][e], added for p = 0, 1, ... in that order.  Thread t
// serves experts t % 256 and t % 256 + 256 over the quarter t / 256 of the
// experts compared against.
__global__ __launch_bounds__(1024) void k_router_topk(const double *__restrict__ zp, int P, int S,
                                                      int E, const float *__restrict__ bias, int K,
                                                      double topp, int norm_topk, double scale,
                                                      int32_t *__restrict__ ids, float *__restrict__ w) {
    __shared__ __align__(16) double skey[RT_MAXE];
    __shared__ double spr[RT_MAXE];
    __shared__ int srank[4][RT_MAXE];
    __shared__ int spick[RT_MAXK];
    __shared__ double spp[RT_MAXK];
    const int t = threadIdx.x, s = blockIdx.x;
    const int et = t & 255, q = t >> 8;
    if (t < RT_MAXE) {
        const int e = t;
        if (e < E) {
            double zz = zp[(int64_t)s * E + e];
            for (int p = 1; p < P; ++p) zz += zp[((int64_t)p * S + s) * E + e];
            const double pr = 1.0 / (1.0 + exp(-zz));
            spr[e] = pr;
            skey[e] = pr + (bias ? (double)bias[e] : 0.0);
        }
    }
    if (t < RT_MAXK) {
        spick[t] = -1;
        spp[t] = 0.0;
    }
    __syncthreads();
    // rank of expert e: experts with a larger key, or an equal key and a
    // smaller index, counted over j in this thread's quarter
    const int jq = (E + 31) / 32 * 8;  // quarters of whole 8-key groups
    const int j0 = min(E, q * jq), j1 = min(E, (q + 1) * jq);
#pragma unroll
    for (int h = 0; h < RT_MAXE / 256; ++h) {
        const int e = et + 256 * h;
        if (e < E) {
            const double ke = skey[e];
            int r = 0;
            int j = j0;
            for (; j + 8 <= j1; j += 8) {
                double kj[8];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const double2 v = *(const double2 *)&skey[j + 2 * u];
                    kj[2 * u] = v.x;
                    kj[2 * u + 1] = v.y;
                }
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    r += (int)(kj[u] > ke) + ((int)(kj[u] == ke) & (int)(j + u < e));  // no branches
            }
            for (; j < j1; ++j) {
                const double kj = skey[j];
                r += (int)(kj > ke) + ((int)(kj == ke) & (int)(j < e));
            }
            srank[q][e] = r;
        }
    }
    __syncthreads();
    if (t < RT_MAXE && t < E) {
        const int r = srank[0][t] + srank[1][t] + srank[2][t] + srank[3][t];
        if (r < K) {
            spick[r] = t;
            spp[r] = spr[t];
        }
    }
    __syncthreads();
    // every pick's lane runs the same serial top-p and sums over the picks
    if (t < K) {
        double total = 0.0;
        for (int k = 0; k < K; ++k) total += spp[k];
        int keep = K;
        if (topp > 0.0 && topp < 1.0) {
            double run = 0.0;
            for (int k = 0; k < K; ++k) {
                run += spp[k];
                if (run >= topp * total) {
                    keep = k + 1;
                    break;
                }
            }
        }
        double sum = 0.0;
        for (int k = 0; k < keep; ++k) sum += spp[k];
        const bool kept = t < keep;
        double v = kept ? spp[t] : 0.0;
        if (kept && norm_topk)
            v /= sum;
        ids[(int64_t)s * K + t] = kept ? spick[t] : -1;
        w[(int64_t)s * K + t] = (float)(v * (kept ? scale : 0.0));
    }
}

size_t router_ws_bytes(int S, int E) { return (size_t)RT_MAXP * S * E * sizeof(double); }

static int launch_topk(const double *z, int P, int S, int E, const float *bias, int K, float topp,
                       int norm_topk, float routed_scale, int32_t *ids, float *w, hipStream_t st) {
    ProfScope ps("router_topk", st);
    hipLaunchKernelGGL(k_router_topk, dim3((unsigned)S), dim3(1024), 0, st, z, P, S, E, bias, K,
                       (double)topp, norm_topk, (double)routed_scale, ids, w);
    return after_launch("router_topk");
}

// The RMSNorm in front of the router folded into the decode logits kernel
// (S <= 4 rows, 16-byte aligned rows): one launch fewer; xn gets the same
// values a separate norm launch writes.  Otherwise the two launches.
int launch_norm_router(const float *h, int S, int D, const float *lnw, double eps, float *xn,
                       const float *R, const float *bias, int E, int K, float topp, int norm_topk,
                       float routed_scale, int32_t *ids, float *w, void *ws, hipStream_t st) {
    const bool fold = S >= 1 && S <= 4 && D % 4 == 0 && (uintptr_t)h % 16 == 0 &&
                      (uintptr_t)xn % 16 == 0 && (uintptr_t)lnw % 16 == 0 && (uintptr_t)R % 16 == 0;
    if (!fold) {
        const int rc = launch_rmsnorm(h, S, D, lnw, eps, xn, st);
        if (rc != COLI_OK) return rc;
        return launch_router(xn, S, D, R, bias, E, K, topp, norm_topk, routed_scale, ids, w, ws, st);
    }
    double *z = (double *)ws;
    {
        ProfScope ps("router_logits", st);
        const dim3 grid((unsigned)E, 1u);
        if (S == 1)
            hipLaunchKernelGGL((k_router_logits<1, 1, 6, true, 4, true>), grid, dim3(256), 0, st, h, S, D,
                               R, E, z, lnw, eps, xn);
        else
            hipLaunchKernelGGL((k_router_logits<4, 1, 6, true, 4, true>), grid, dim3(256), 0, st, h, S, D,
                               R, E, z, lnw, eps, xn);
        const int rc = after_launch("router_logits");
        if (rc != COLI_OK) return rc;
    }
    return launch_topk(z, 1, S, E, bias, K, topp, norm_topk, routed_scale, ids, w, st);
}

int launch_router(const float *x, int S, int D, const float *R, const float *bias, int E, int K,
                  float topp, int norm_topk, float routed_scale, int32_t *ids, float *w, void *ws,
                  hipStream_t st) {
    double *z = (double *)ws;
    const bool vec = D % 4 == 0 && (uintptr_t)x % 16 == 0 && (uintptr_t)R % 16 == 0;
    int P = 1;
    {
        ProfScope ps("router_logits", st);
        if (S <= 4) {
            // decode rows: a workgroup per expert, each router row read once
            const dim3 grid((unsigned)E, 1u);
            if (S == 1 && vec)
                hipLaunchKernelGGL((k_router_logits<1, 1, 6, true, 4>), grid, dim3(256), 0, st, x, S, D, R, E, z);
            else if (S == 1)
                hipLaunchKernelGGL((k_router_logits<1, 1, 6, false, 4>), grid, dim3(256), 0, st, x, S, D, R, E, z);
            else if (vec)
                hipLaunchKernelGGL((k_router_logits<4, 1, 6, true, 4>), grid, dim3(256), 0, st, x, S, D, R, E, z);
            else
                hipLaunchKernelGGL((k_router_logits<4, 1, 6, false, 4>), grid, dim3(256), 0, st, x, S, D, R, E, z);
        } else if (vec) {
            // at least ~512 workgroups: split the inputs P ways (each of a
            // workgroup's 4 wavefronts keeps 4 or more 16-input steps)
            const int nt = ((E + 31) / 32) * ((S + 31) / 32);
            const int nst = (D + 15) / 16;
            P = std::max(1, std::min({RT_MAXP, (512 + nt - 1) / nt, nst / 16}));
            const dim3 grid((unsigned)((E + 31) / 32), (unsigned)((S + 31) / 32), (unsigned)P);
            hipLaunchKernelGGL((k_router_logits_mx<4>), grid, dim3(256), 0, st, x, S, D, R, E, z);
        } else {
            const dim3 grid((unsigned)((E + 31) / 32), (unsigned)((S + 7) / 8));
            hipLaunchKernelGGL((k_router_logits<8, 8, 1, false, 1>), grid, dim3(256), 0, st, x, S, D, R, E, z);
        }
        int rc = after_launch("router_logits");
        if (rc != COLI_OK) return rc;
    }
    return launch_topk(z, P, S, E, bias, K, topp, norm_topk, routed_scale, ids, w, st);
}

}  // namespace coli
