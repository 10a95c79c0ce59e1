// gemm.hip -- prefill path (S > 4 input rows): the quantized matmul as a bf16
// matrix-core GEMM for gfx950, dense and over the ragged MoE routing table.
//
// What is computed (colibri PR #298, CUDA fmt=4 commit: the group scale is
// applied to each group's partial sum during accumulation; colibri-strix
// commit log, prefill GEMM routing commit: large row
// batches take a GEMM path; batched expert-block commit: per-row ragged
// routing, gate/up -> SiLU -> down, weighted scatter-add):
//     Y[m][n] = sum_g scale(n, g) * sum_{k in g} v(n, k) * X[m][k]
//
// How (MI355X design):
//   * a workgroup of 4 wavefronts owns a BM x BN output tile (inputs x weight
//     rows), 2 x 2 wavefronts; K advances 64 inputs per step;
//   * each step the weight codes of the tile are loaded as 16-byte packets,
//     turned into the exact small integers MULT*v (one SDWA conversion per
//     code) and stored to LDS as bf16 -- exact, since |MULT*v| <= 128 -- next
//     to the inputs rounded to bf16;
//   * v_mfma_f32_16x16x32_bf16 accumulates in fp32; for grouped int4 every
//     group's partial sum is formed in a fresh accumulator and added to the
//     output with its f32 scale, so only the inputs are rounded to bf16
//     (bf16 keeps 8 significant bits: error <= 2^-8 * sum |w||x| plus fp32
//     accumulation);
//   * MoE: a routing kernel builds the table and a tile list (expert, first
//     row); the inputs are gathered to bf16 in routing order once; gate and up
//     share a workgroup (one pass over the inputs) and write
//     h = silu(g) * u in bf16; down writes per-pair rows; a combine kernel
//     adds them per token in ascending k (no atomics).
#include <string.h>

#include <algorithm>

#include "common.h"

namespace coli {

typedef __bf16 bf16_t;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4v __attribute__((ext_vector_type(4)));

constexpr int G_BK = 64;          // inputs per K step
constexpr int G_LDK = G_BK + 8;   // LDS row stride in bf16 (pad against bank conflicts)

enum { GE_DENSE = 0, GE_GATEUP = 1, GE_DOWN = 2 };

struct GemmArgs {
    // inputs: X rows (f32 when xf32, else bf16), row stride ldx elements
    const void *x;
    int64_t ldx;
    int M, K;                 // dense: M input rows; MoE: unused (tiles say)
    // weights: NMAT stacks (gate, up) or one; matrix e at q[m] + e*q_stride
    const uint8_t *q[2];
    const float *s[2];
    const uint8_t *sq[2];     // shared expert (MoE, tile expert == E)
    const float *ss[2];
    int64_t rb, q_stride, s_stride;
    int ng, gs, N;            // N = rows per matrix
    // MoE tile list
    const int32_t *tiles;     // [2*t] expert, [2*t+1] first row
    const int32_t *n_tiles;
    const int32_t *counts, *offsets;
    int E, SK, S;
    // outputs
    void *y;
    int64_t ldy;
};

__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + expf(-z)); }

// Store CP exact values f[] as bf16 into LDS.
template <int CP>
__device__ __forceinline__ void store_bf16(bf16_t *dst, const float *f) {
#pragma unroll
    for (int j = 0; j < CP; j += 8) {
        bf16x8 v;
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = (bf16_t)f[j + i];
        *reinterpret_cast<bf16x8 *>(dst + j) = v;
    }
}

template <int FMT, int BM, int BN, int NMAT, int EPI, bool XF32>
__global__ __launch_bounds__(256) void k_gemm(GemmArgs a) {
    constexpr int CP = packet_cols(FMT), PB = packet_bytes(FMT);
    constexpr int WTM = BM / 2, WTN = BN / 2;       // wavefront tile
    constexpr int MB = WTM / 16, NB = WTN / 16;     // 16x16 blocks per wavefront
    constexpr int PPR = G_BK / CP;                  // packets per row per K step
    constexpr int WPK = (BN * PPR + 255) / 256;     // packets per thread per matrix
    constexpr bool GROUPED = (FMT == 4);
    constexpr float INV = 1.0f / Mult<FMT>::value;

    __shared__ __attribute__((aligned(16))) bf16_t Ws[NMAT][BN * G_LDK];
    __shared__ __attribute__((aligned(16))) bf16_t Xs[BM * G_LDK];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int n0 = blockIdx.y * BN;
    const int K = a.K;

    // --- which rows of X, which weight matrices --------------------------
    int m_count, xrow0, e = 0;
    bool shared = false;
    if (EPI == GE_DENSE) {
        xrow0 = blockIdx.x * BM;
        m_count = min(BM, a.M - xrow0);
    } else {
        const int t = blockIdx.x;
        if (t >= gload<int32_t>(a.n_tiles))
            return;
        e = gload<int32_t>(a.tiles + 2 * t);
        const int m0 = gload<int32_t>(a.tiles + 2 * t + 1);
        if (e >= a.E) {
            shared = true;
            m_count = min(BM, a.S - m0);
            xrow0 = a.SK + m0;
        } else {
            m_count = min(BM, gload<int32_t>(a.counts + e) - m0);
            xrow0 = gload<int32_t>(a.offsets + e) + m0;
        }
    }
    const uint8_t *wq[NMAT];
    const float *wsc[NMAT];
#pragma unroll
    for (int m = 0; m < NMAT; ++m) {
        wq[m] = shared ? a.sq[m] : a.q[m] + (int64_t)e * a.q_stride;
        wsc[m] = shared ? a.ss[m] : a.s[m] + (int64_t)e * a.s_stride;
    }

    f32x4v acc[NMAT][MB][NB], cg[NMAT][MB][NB];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                acc[m][i][j] = f32x4v{0.f, 0.f, 0.f, 0.f};
                cg[m][i][j] = f32x4v{0.f, 0.f, 0.f, 0.f};
            }

    for (int k0 = 0; k0 < K; k0 += G_BK) {
        const int kslices = min(G_BK, K - k0) / 32;  // K % 32 == 0
        // ---- weights: packets -> exact bf16 integers in LDS --------------
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int w = 0; w < WPK; ++w) {
                const int pidx = tid + w * 256;
                if (pidx < BN * PPR) {
                    const int r = pidx / PPR, pk = pidx % PPR;
                    const int row = min(n0 + r, a.N - 1);
                    const int col = k0 + pk * CP;
                    float f[CP];
                    if (col < K) {
                        const Packet<FMT> p = load_packet<FMT>(wq[m] + row * a.rb + (int64_t)(col / CP) * PB);
                        decode_packet<FMT>(p, f);
                    } else {
#pragma unroll
                        for (int i = 0; i < CP; ++i) f[i] = 0.f;
                    }
                    store_bf16<CP>(&Ws[m][r * G_LDK + pk * CP], f);
                }
            }
        // ---- inputs: BM rows x 64 -> bf16 in LDS ---------------------------
        if constexpr (XF32) {
            // 16 floats per thread-iteration
            for (int idx = tid; idx < BM * (G_BK / 16); idx += 256) {
                const int r = idx / (G_BK / 16), c = (idx % (G_BK / 16)) * 16;
                const int xr = xrow0 + min(r, max(m_count - 1, 0));
                const float *src = (const float *)a.x + (int64_t)xr * a.ldx + k0 + c;
                bf16x8 v0, v1;
                if (k0 + c < K) {
                    const f32x4 p0 = gload<f32x4>(src), p1 = gload<f32x4>(src + 4);
                    const f32x4 p2 = gload<f32x4>(src + 8), p3 = gload<f32x4>(src + 12);
                    v0 = bf16x8{(bf16_t)p0.x, (bf16_t)p0.y, (bf16_t)p0.z, (bf16_t)p0.w,
                                (bf16_t)p1.x, (bf16_t)p1.y, (bf16_t)p1.z, (bf16_t)p1.w};
                    v1 = bf16x8{(bf16_t)p2.x, (bf16_t)p2.y, (bf16_t)p2.z, (bf16_t)p2.w,
                                (bf16_t)p3.x, (bf16_t)p3.y, (bf16_t)p3.z, (bf16_t)p3.w};
                } else {
                    v0 = v1 = bf16x8{};
                }
                *reinterpret_cast<bf16x8 *>(&Xs[r * G_LDK + c]) = v0;
                *reinterpret_cast<bf16x8 *>(&Xs[r * G_LDK + c + 8]) = v1;
            }
        } else {
            for (int idx = tid; idx < BM * (G_BK / 8); idx += 256) {
                const int r = idx / (G_BK / 8), c = (idx % (G_BK / 8)) * 8;
                const int xr = xrow0 + min(r, max(m_count - 1, 0));
                const bf16_t *src = (const bf16_t *)a.x + (int64_t)xr * a.ldx + k0 + c;
                bf16x8 v = (k0 + c < K) ? gload<bf16x8>(src) : bf16x8{};
                *reinterpret_cast<bf16x8 *>(&Xs[r * G_LDK + c]) = v;
            }
        }
        __syncthreads();

        // ---- matrix cores ----------------------------------------------------
        for (int ks = 0; ks < kslices; ++ks) {
            const int kk = ks * 32;
            const int kglob = k0 + kk;
            bf16x8 af[MB], bfr[NMAT][NB];
#pragma unroll
            for (int i = 0; i < MB; ++i)
                af[i] = *reinterpret_cast<const bf16x8 *>(
                    &Xs[(wm * WTM + i * 16 + (lane & 15)) * G_LDK + kk + 8 * (lane >> 4)]);
#pragma unroll
            for (int m = 0; m < NMAT; ++m)
#pragma unroll
                for (int j = 0; j < NB; ++j)
                    bfr[m][j] = *reinterpret_cast<const bf16x8 *>(
                        &Ws[m][(wn * WTN + j * 16 + (lane & 15)) * G_LDK + kk + 8 * (lane >> 4)]);
            if constexpr (GROUPED) {
                const bool first = (kglob % a.gs) == 0;
                const bool last = ((kglob + 32) % a.gs) == 0 || (kglob + 32 >= K);
#pragma unroll
                for (int m = 0; m < NMAT; ++m)
#pragma unroll
                    for (int i = 0; i < MB; ++i)
#pragma unroll
                        for (int j = 0; j < NB; ++j)
                            cg[m][i][j] = first
                                ? __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[m][j], f32x4v{0.f, 0.f, 0.f, 0.f}, 0, 0, 0)
                                : __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[m][j], cg[m][i][j], 0, 0, 0);
                if (last) {
                    const int g = kglob / a.gs;
#pragma unroll
                    for (int m = 0; m < NMAT; ++m)
#pragma unroll
                        for (int j = 0; j < NB; ++j) {
                            const int row = min(n0 + wn * WTN + j * 16 + (lane & 15), a.N - 1);
                            const float sc = gload<float>(wsc[m] + (int64_t)row * a.ng + g) * INV;
#pragma unroll
                            for (int i = 0; i < MB; ++i) {
                                acc[m][i][j].x = fmaf(sc, cg[m][i][j].x, acc[m][i][j].x);
                                acc[m][i][j].y = fmaf(sc, cg[m][i][j].y, acc[m][i][j].y);
                                acc[m][i][j].z = fmaf(sc, cg[m][i][j].z, acc[m][i][j].z);
                                acc[m][i][j].w = fmaf(sc, cg[m][i][j].w, acc[m][i][j].w);
                            }
                        }
                }
            } else {
#pragma unroll
                for (int m = 0; m < NMAT; ++m)
#pragma unroll
                    for (int i = 0; i < MB; ++i)
#pragma unroll
                        for (int j = 0; j < NB; ++j)
                            acc[m][i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[m][j], acc[m][i][j], 0, 0, 0);
            }
        }
        __syncthreads();
    }

    // ---- epilogue ------------------------------------------------------------
#pragma unroll
    for (int j = 0; j < NB; ++j) {
        const int n = n0 + wn * WTN + j * 16 + (lane & 15);
        if (n >= a.N)
            continue;
        float rs[NMAT];
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
            rs[m] = GROUPED ? 1.0f : gload<float>(wsc[m] + n) * INV;
#pragma unroll
        for (int i = 0; i < MB; ++i) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int mr = wm * WTM + i * 16 + 4 * (lane >> 4) + c;
                if (mr >= m_count)
                    continue;
                const float v0 = acc[0][i][j][c] * rs[0];
                if constexpr (EPI == GE_GATEUP) {
                    const float v1 = acc[NMAT - 1][i][j][c] * rs[NMAT - 1];
                    ((bf16_t *)a.y)[(int64_t)(xrow0 + mr) * a.ldy + n] = (bf16_t)(silu_f(v0) * v1);
                } else {
                    ((float *)a.y)[(int64_t)(xrow0 + mr) * a.ldy + n] = v0;
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Dense entry (coli_qmatmul with S > the GEMV limit)
// ---------------------------------------------------------------------------

size_t gemm_workspace_bytes(int S, int I) { (void)S; (void)I; return 0; }

static GemmArgs gemm_args_for(const coli_qtensor *W) {
    GemmArgs a;
    memset(&a, 0, sizeof a);
    a.q[0] = a.q[1] = (const uint8_t *)W->q;
    a.s[0] = a.s[1] = W->s;
    a.rb = W->row_bytes;
    a.q_stride = W->q_stride;
    a.s_stride = W->s_stride;
    a.ng = W->ng;
    a.gs = W->gs > 0 ? W->gs : 1;
    a.N = W->O;
    a.K = W->I;
    return a;
}

static bool mfma_ok(const coli_qtensor *W) {
    if (!(W->flags & QF_FAST) || W->I % 32 != 0)
        return false;
    return W->fmt != 4 || W->gs % 32 == 0;
}

template <int FMT>
static void launch_dense_t(const coli_qtensor *W, const float *x, float *y, int S, hipStream_t st) {
    constexpr int BM = 64, BN = 128;
    for (int e = 0; e < W->n; ++e) {
        GemmArgs a = gemm_args_for(W);
        a.q[0] = (const uint8_t *)W->q + (int64_t)e * W->q_stride;
        a.s[0] = W->s + (int64_t)e * W->s_stride;
        a.x = x;
        a.ldx = W->I;
        a.M = S;
        a.y = y + (int64_t)e * S * W->O;
        a.ldy = W->O;
        const dim3 grid((unsigned)((S + BM - 1) / BM), (unsigned)((W->O + BN - 1) / BN));
        hipLaunchKernelGGL((k_gemm<FMT, BM, BN, 1, GE_DENSE, true>), grid, dim3(256), 0, st, a);
    }
}

int launch_gemm(const coli_qtensor *W, const float *x, float *y, int S, void *ws, size_t ws_bytes,
                hipStream_t st) {
    (void)ws; (void)ws_bytes;
    const int pr = launch_pgemm_dense(W, x, y, S, st);  // int4 formats
    if (pr != 0)
        return pr > 0 ? COLI_OK : COLI_HIP_ERROR;
    if (!mfma_ok(W) || (uintptr_t)x % 16 != 0)
        return launch_gemv(W, x, y, S, st);  // exact fp32 path for other layouts
    ProfScope ps("gemm_dense", st);
    switch (W->fmt) {
    case 1: launch_dense_t<1>(W, x, y, S, st); break;
    case 2: launch_dense_t<2>(W, x, y, S, st); break;
    case 3: launch_dense_t<3>(W, x, y, S, st); break;
    default: launch_dense_t<4>(W, x, y, S, st); break;
    }
    return after_launch("gemm_dense");
}

// ---------------------------------------------------------------------------
// Prefill MoE block
// ---------------------------------------------------------------------------

constexpr int MOE_BM = 32, MOE_BN = 128;

struct PrefillWs {
    int32_t *counts, *offsets, *perm, *n_bad, *inv, *tiles, *n_tiles, *tiles_s, *n_tiles_s;
    bf16_t *xg, *hg;
    float *y;
    size_t bytes;
    int max_tiles, max_short;
};

static size_t al(size_t b) { return (b + 255) / 256 * 256; }

static PrefillWs prefill_layout(void *base, int E, int S, int K, int F, int D, int has_shared) {
    PrefillWs w;
    const size_t SK = (size_t)S * K, R = SK + (has_shared ? S : 0);
    w.max_tiles = (int)(std::min<size_t>((size_t)E, SK) + (SK + MOE_BM - 1) / MOE_BM +
                        (has_shared ? (S + MOE_BM - 1) / MOE_BM : 0));
    char *p = (char *)base;
    size_t off = 0;
    auto take = [&](size_t b) { char *q = p ? p + off : nullptr; off += al(b); return q; };
    w.counts = (int32_t *)take(sizeof(int32_t) * E);
    w.offsets = (int32_t *)take(sizeof(int32_t) * (E + 1));
    w.perm = (int32_t *)take(sizeof(int32_t) * std::max<size_t>(SK, 1));
    w.n_bad = (int32_t *)take(sizeof(int32_t));
    w.inv = (int32_t *)take(sizeof(int32_t) * std::max<size_t>(SK, 1));
    w.tiles = (int32_t *)take(sizeof(int32_t) * 2 * w.max_tiles);
    w.n_tiles = (int32_t *)take(sizeof(int32_t));
    w.max_short = (int)std::min<size_t>((size_t)E, SK);
    w.tiles_s = (int32_t *)take(sizeof(int32_t) * 2 * std::max(w.max_short, 1));
    w.n_tiles_s = (int32_t *)take(sizeof(int32_t));
    w.xg = (bf16_t *)take(sizeof(bf16_t) * R * D);
    w.hg = (bf16_t *)take(sizeof(bf16_t) * R * F);
    w.y = (float *)take(sizeof(float) * R * D);
    w.bytes = off;
    return w;
}

size_t moe_prefill_ws_bytes(int E, int S, int K, int F, int D, int has_shared) {
    return prefill_layout(nullptr, E, S, K, F, D, has_shared).bytes;
}

// xg[pos] = bf16(x[token of perm[pos]]) for valid routed rows; shared rows
// SK+s take x[s].
__global__ __launch_bounds__(256) void k_gather_x(const float *__restrict__ x, int D, int K, int SK,
                                                  int S, int has_shared,
                                                  const int32_t *__restrict__ perm,
                                                  const int32_t *__restrict__ offsets, int E,
                                                  bf16_t *__restrict__ xg) {
    const int pos = blockIdx.x;
    int tok;
    if (pos < SK) {
        if (pos >= gload<int32_t>(offsets + E))
            return;
        tok = gload<int32_t>(perm + pos) / K;
    } else {
        tok = pos - SK;
    }
    const float *src = x + (int64_t)tok * D;
    bf16_t *dst = xg + (int64_t)pos * D;
    for (int c = threadIdx.x * 8; c < D; c += 256 * 8) {
        const f32x4 p0 = gload<f32x4>(src + c), p1 = gload<f32x4>(src + c + 4);
        *reinterpret_cast<bf16x8 *>(dst + c) =
            bf16x8{(bf16_t)p0.x, (bf16_t)p0.y, (bf16_t)p0.z, (bf16_t)p0.w,
                   (bf16_t)p1.x, (bf16_t)p1.y, (bf16_t)p1.z, (bf16_t)p1.w};
    }
}

// out[s][o] = sum_k w[s][k] * y[inv[s*K+k]][o] (ascending k) + y[SK+s][o]
__global__ __launch_bounds__(256) void k_prefill_combine(const float *__restrict__ y,
                                                         const int32_t *__restrict__ inv,
                                                         const float *__restrict__ w, int S, int K,
                                                         int D, int has_shared,
                                                         float *__restrict__ out) {
    const int s = blockIdx.y;
    const int o = (blockIdx.x * 256 + threadIdx.x) * 4;
    if (o >= D)
        return;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < K; ++k) {
        const int64_t p = (int64_t)s * K + k;
        const int pos = gload<int32_t>(inv + p);
        if (pos < 0)
            continue;
        const float wk = gload<float>(w + p);
        const f32x4 v = gload<f32x4>(y + (int64_t)pos * D + o);
        acc.x = fmaf(wk, v.x, acc.x);
        acc.y = fmaf(wk, v.y, acc.y);
        acc.z = fmaf(wk, v.z, acc.z);
        acc.w = fmaf(wk, v.w, acc.w);
    }
    if (has_shared) {
        const f32x4 v = gload<f32x4>(y + ((int64_t)S * K + s) * D + o);
        acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
    float *dst = out + (int64_t)s * D + o;  // caller's buffer: 4-byte alignment only
    dst[0] = acc.x;
    dst[1] = acc.y;
    dst[2] = acc.z;
    dst[3] = acc.w;
}

// h_out[p] = f32(hg[inv[p]]) (0 when left out); h_out[SK+s] = f32(hg[SK+s])
__global__ __launch_bounds__(256) void k_hidden_out(const bf16_t *__restrict__ hg,
                                                    const int32_t *__restrict__ inv, int SK,
                                                    int F, float *__restrict__ h) {
    const int p = blockIdx.x;
    const int pos = p < SK ? gload<int32_t>(inv + p) : p;
    for (int j = threadIdx.x; j < F; j += 256)
        h[(int64_t)p * F + j] = pos < 0 ? 0.f : (float)hg[(int64_t)pos * F + j];
}

static int moe_gather(const MoeArgs &a, const PrefillWs &w) {
    const bool has_sh = a.sg != nullptr;
    const int SK = a.S * a.K;
    const int R = SK + (has_sh ? a.S : 0);
    ProfScope ps("moe_gather", a.st);
    hipLaunchKernelGGL(k_gather_x, dim3((unsigned)R), dim3(256), 0, a.st, a.x, a.D, a.K, SK, a.S,
                       has_sh ? 1 : 0, w.perm, w.offsets, a.E, w.xg);
    return after_launch("moe_gather");
}

static int moe_hidden_out(const MoeArgs &a, const PrefillWs &w) {
    const int SK = a.S * a.K;
    const int R = SK + (a.sg != nullptr ? a.S : 0);
    ProfScope ps("moe_hidden_out", a.st);
    hipLaunchKernelGGL(k_hidden_out, dim3((unsigned)R), dim3(256), 0, a.st, w.hg, w.inv, SK, a.F,
                       a.h_out);
    return after_launch("moe_hidden_out");
}

static int moe_combine(const MoeArgs &a, const PrefillWs &w) {
    ProfScope ps("moe_prefill_combine", a.st);
    hipLaunchKernelGGL(k_prefill_combine, dim3((unsigned)((a.D / 4 + 255) / 256), (unsigned)a.S),
                       dim3(256), 0, a.st, w.y, w.inv, a.w, a.S, a.K, a.D,
                       a.sg != nullptr ? 1 : 0, a.out);
    return after_launch("moe_prefill_combine");
}

template <int FMT>
static int moe_prefill_t(const MoeArgs &a, const PrefillWs &w) {
    const bool has_sh = a.sg != nullptr;
    const int SK = a.S * a.K;
    int rc = moe_gather(a, w);
    if (rc != COLI_OK)
        return rc;
    {
        GemmArgs g = gemm_args_for(a.gate);
        g.q[1] = (const uint8_t *)a.up->q;
        g.s[1] = a.up->s;
        g.sq[0] = has_sh ? (const uint8_t *)a.sg->q : g.q[0];
        g.ss[0] = has_sh ? a.sg->s : g.s[0];
        g.sq[1] = has_sh ? (const uint8_t *)a.su->q : g.q[1];
        g.ss[1] = has_sh ? a.su->s : g.s[1];
        g.x = w.xg;
        g.ldx = a.D;
        g.tiles = w.tiles; g.n_tiles = w.n_tiles; g.counts = w.counts; g.offsets = w.offsets;
        g.E = a.E; g.SK = SK; g.S = a.S;
        g.y = w.hg;
        g.ldy = a.F;
        const dim3 grid((unsigned)w.max_tiles, (unsigned)((a.F + MOE_BN - 1) / MOE_BN));
        ProfScope ps("moe_gateup_gemm", a.st);
        hipLaunchKernelGGL((k_gemm<FMT, MOE_BM, MOE_BN, 2, GE_GATEUP, false>), grid, dim3(256), 0,
                           a.st, g);
        int rc = after_launch("moe_gateup_gemm");
        if (rc != COLI_OK) return rc;
    }
    if (a.h_out)
        return moe_hidden_out(a, w);
    {
        GemmArgs g = gemm_args_for(a.down);
        g.sq[0] = g.sq[1] = has_sh ? (const uint8_t *)a.sd->q : g.q[0];
        g.ss[0] = g.ss[1] = has_sh ? a.sd->s : g.s[0];
        g.x = w.hg;
        g.ldx = a.F;
        g.tiles = w.tiles; g.n_tiles = w.n_tiles; g.counts = w.counts; g.offsets = w.offsets;
        g.E = a.E; g.SK = SK; g.S = a.S;
        g.y = w.y;
        g.ldy = a.D;
        const dim3 grid((unsigned)w.max_tiles, (unsigned)((a.D + MOE_BN - 1) / MOE_BN));
        ProfScope ps("moe_down_gemm", a.st);
        hipLaunchKernelGGL((k_gemm<FMT, MOE_BM, MOE_BN, 1, GE_DOWN, false>), grid, dim3(256), 0,
                           a.st, g);
        int rc = after_launch("moe_down_gemm");
        if (rc != COLI_OK) return rc;
    }
    return moe_combine(a, w);
}

// the int4 formats on the newer matrix-core kernels (routed tiles of `rows`)
static int moe_prefill_pg(const MoeArgs &a, const PrefillWs &w, int rows) {
    const bool has_sh = a.sg != nullptr;
    const size_t SK = (size_t)a.S * a.K;
    const int max_tiles = (int)(std::min<size_t>((size_t)a.E, SK) + (SK + rows - 1) / rows +
                                (has_sh ? ((size_t)a.S + rows - 1) / rows : 0));
    int rc = moe_gather(a, w);
    if (rc != COLI_OK)
        return rc;
    const bool short_tiles = rows == PG_MOE_ROWS_PACKED && PG_MOE_ROWS_SHORT > 0;
    rc = launch_pgemm_moe(a, rows, w.xg, w.hg, a.h_out ? nullptr : w.y, w.tiles, w.n_tiles,
                          w.counts, w.offsets, max_tiles, short_tiles ? w.tiles_s : nullptr,
                          short_tiles ? w.n_tiles_s : nullptr, short_tiles ? w.max_short : 0);
    if (rc != COLI_OK)
        return rc;
    return a.h_out ? moe_hidden_out(a, w) : moe_combine(a, w);
}

int launch_moe_prefill(const MoeArgs &a) {
    const bool has_sh = a.sg != nullptr;
    // the matrix-core kernels need whole 32-input slices and gs % 32 == 0
    const coli_qtensor *all[6] = {a.gate, a.up, a.down, a.sg, a.su, a.sd};
    for (const coli_qtensor *t : all)
        if (t && !mfma_ok(t))
            return decline("moe_block (S > %d): tensor layout needs I %% 32 == 0 and gs %% 32 == 0 "
                           "for the matrix-core path", coli_gemv_max_rows());
    if (a.D % 8 != 0)
        return decline("moe_block (S > %d): hidden size must be a multiple of 8",
                       coli_gemv_max_rows());
    const PrefillWs w = prefill_layout(a.ws, a.E, a.S, a.K, a.F, a.D, has_sh);
    if (w.bytes > a.ws_bytes)
        return decline("moe_block: workspace %zu bytes < %zu needed", a.ws_bytes, w.bytes);
    const int pg_rows = (uintptr_t)a.ws % 16 == 0 ? pgemm_moe_rows(a) : 0;
    const int bm_s = pg_rows == PG_MOE_ROWS_PACKED ? PG_MOE_ROWS_SHORT : 0;
    int rc = launch_route(a.ids, a.S, a.K, a.E, w.counts, w.offsets, w.perm, w.n_bad, w.inv,
                          w.tiles, w.n_tiles, pg_rows ? pg_rows : MOE_BM, has_sh ? a.S : 0, a.st,
                          bm_s ? w.tiles_s : nullptr, bm_s ? w.n_tiles_s : nullptr, bm_s);
    if (rc != COLI_OK)
        return rc;
    if (pg_rows)
        return moe_prefill_pg(a, w, pg_rows);
    switch (a.gate->fmt) {
    case 1: return moe_prefill_t<1>(a, w);
    case 2: return moe_prefill_t<2>(a, w);
    case 3: return moe_prefill_t<3>(a, w);
    default: return moe_prefill_t<4>(a, w);
    }
}

}  // namespace coli
