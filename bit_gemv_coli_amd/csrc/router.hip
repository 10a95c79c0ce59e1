// router.hip -- the MoE router and its exact top-K selection on the GPU
// (colibri-strix commit log, "metal: full decode layer in ONE command
// buffer": router matvec + sigmoid, then greedy argmax over sigmoid + bias
// with the CPU's tie order, top-p truncation, norm_topk, routed_scale).
//
// Decisions are taken on f64 numbers: every logit is a sum of exact f64
// products of f32 operands, the sigmoid and the key p + bias are f64, so the
// picks do not depend on the order the GPU sums in (beyond 2^-53 relative),
// and equal logits give equal keys and the smaller expert index.
//   k_router_logits  z[s][e] for 8 input rows x 1 expert per wavefront: lanes
//                    split the inputs (16-byte loads), one f64 FMA per product,
//                    a wavefront sum at the end;
//   k_router_topk    one wavefront per input row: lane l holds experts
//                    l, l + 64, ...; K rounds of a wavefront argmax on
//                    (key, index); top-p, norm_topk and routed_scale on lane 0.
#include "common.h"

namespace coli {

constexpr int RT_TOK = 8;      // input rows per logits wavefront
constexpr int RT_MAXE = 512;   // experts (8 per lane)
constexpr int RT_MAXK = 16;    // picks per row

__device__ __forceinline__ double rt_shfl_xor(double v, int m) {
    const int2 p = __builtin_bit_cast(int2, v);
    int2 q;
    q.x = __shfl_xor(p.x, m);
    q.y = __shfl_xor(p.y, m);
    return __builtin_bit_cast(double, q);
}

template <bool VEC>
__global__ __launch_bounds__(256) void k_router_logits(const float *__restrict__ x, int S, int D,
                                                       const float *__restrict__ R, int E,
                                                       double *__restrict__ z) {
    const int lane = threadIdx.x & 63;
    const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int s0 = blockIdx.y * RT_TOK;
    if (e >= E)
        return;  // whole wavefront
    const int ns = min(RT_TOK, S - s0);
    const float *rr = R + (int64_t)e * D;
    double acc[RT_TOK];
#pragma unroll
    for (int t = 0; t < RT_TOK; ++t) acc[t] = 0.0;
    if constexpr (VEC) {
        for (int d = 4 * lane; d < D; d += 256) {
            const f32x4 r = gload<f32x4>(rr + d);
#pragma unroll
            for (int t = 0; t < RT_TOK; ++t) {
                if (t < ns) {
                    const f32x4 v = gload<f32x4>(x + (int64_t)(s0 + t) * D + d);
                    acc[t] = fma((double)r.x, (double)v.x, acc[t]);
                    acc[t] = fma((double)r.y, (double)v.y, acc[t]);
                    acc[t] = fma((double)r.z, (double)v.z, acc[t]);
                    acc[t] = fma((double)r.w, (double)v.w, acc[t]);
                }
            }
        }
    } else {
        for (int d = lane; d < D; d += 64) {
            const double r = (double)rr[d];
#pragma unroll
            for (int t = 0; t < RT_TOK; ++t)
                if (t < ns)
                    acc[t] = fma(r, (double)x[(int64_t)(s0 + t) * D + d], acc[t]);
        }
    }
#pragma unroll
    for (int t = 0; t < RT_TOK; ++t)
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) acc[t] += rt_shfl_xor(acc[t], m);
    if (lane < ns) {
        double v = acc[0];
#pragma unroll
        for (int t = 1; t < RT_TOK; ++t) v = (lane == t) ? acc[t] : v;
        z[(int64_t)(s0 + lane) * E + e] = v;
    }
}

__global__ __launch_bounds__(256) void k_router_topk(const double *__restrict__ z, int S, int E,
                                                     const float *__restrict__ bias, int K,
                                                     double topp, int norm_topk, double scale,
                                                     int32_t *__restrict__ ids, float *__restrict__ w) {
    const int lane = threadIdx.x & 63;
    const int s = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (s >= S)
        return;  // whole wavefront
    constexpr int EPL = RT_MAXE / 64;
    double key[EPL], pr[EPL];
    const double neg = -__builtin_huge_val();
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = lane + 64 * i;
        if (e < E) {
            const double zz = z[(int64_t)s * E + e];
            pr[i] = 1.0 / (1.0 + exp(-zz));
            key[i] = pr[i] + (bias ? (double)bias[e] : 0.0);
        } else {
            pr[i] = 0.0;
            key[i] = neg;
        }
    }
    unsigned taken = 0;
    int pick[RT_MAXK];
    double pp[RT_MAXK];
    for (int k = 0; k < K; ++k) {
        // this lane's best untaken expert: largest key, smaller index on ties
        double bk = neg, bp = 0.0;
        int be = 0x7fffffff;
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            const int e = lane + 64 * i;
            const bool ok = e < E && !((taken >> i) & 1u);
            if (ok && (key[i] > bk || be == 0x7fffffff)) {
                bk = key[i];
                bp = pr[i];
                be = e;
            }
        }
        // wavefront argmax on (key, index)
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) {
            const double ok2 = rt_shfl_xor(bk, m), op2 = rt_shfl_xor(bp, m);
            const int oe = __shfl_xor(be, m);
            const bool better = (oe != 0x7fffffff) &&
                                (be == 0x7fffffff || ok2 > bk || (ok2 == bk && oe < be));
            if (better) {
                bk = ok2;
                bp = op2;
                be = oe;
            }
        }
        if ((be & 63) == lane && be != 0x7fffffff)
            taken |= 1u << (be >> 6);
        pick[k] = be;
        pp[k] = bp;
    }
    if (lane == 0) {
        double total = 0.0;
        for (int k = 0; k < K; ++k) total += pp[k];
        int keep = K;
        if (topp > 0.0 && topp < 1.0) {
            double run = 0.0;
            for (int k = 0; k < K; ++k) {
                run += pp[k];
                if (run >= topp * total) {
                    keep = k + 1;
                    break;
                }
            }
        }
        double sum = 0.0;
        for (int k = 0; k < keep; ++k) sum += pp[k];
        for (int k = 0; k < K; ++k) {
            const bool kept = k < keep;
            double v = kept ? pp[k] : 0.0;
            if (kept && norm_topk)
                v /= sum;
            ids[(int64_t)s * K + k] = kept ? pick[k] : -1;
            w[(int64_t)s * K + k] = (float)(v * (kept ? scale : 0.0));
        }
    }
}

size_t router_ws_bytes(int S, int E) { return (size_t)S * E * sizeof(double); }

int launch_router(const float *x, int S, int D, const float *R, const float *bias, int E, int K,
                  float topp, int norm_topk, float routed_scale, int32_t *ids, float *w, void *ws,
                  hipStream_t st) {
    double *z = (double *)ws;
    const bool vec = D % 4 == 0 && (uintptr_t)x % 16 == 0 && (uintptr_t)R % 16 == 0;
    {
        ProfScope ps("router_logits", st);
        const dim3 grid((unsigned)((E + 3) / 4), (unsigned)((S + RT_TOK - 1) / RT_TOK));
        if (vec)
            hipLaunchKernelGGL(k_router_logits<true>, grid, dim3(256), 0, st, x, S, D, R, E, z);
        else
            hipLaunchKernelGGL(k_router_logits<false>, grid, dim3(256), 0, st, x, S, D, R, E, z);
        int rc = after_launch("router_logits");
        if (rc != COLI_OK) return rc;
    }
    ProfScope ps("router_topk", st);
    hipLaunchKernelGGL(k_router_topk, dim3((unsigned)((S + 3) / 4)), dim3(256), 0, st, z, S, E, bias, K,
                       (double)topp, norm_topk, (double)routed_scale, ids, w);
    return after_launch("router_topk");
}

}  // namespace coli
