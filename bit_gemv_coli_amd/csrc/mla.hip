// mla.hip -- attention of one MLA layer: decode (S <= 4 query rows) and prefill
// (colibri-strix commit log, fused decode attention commit (Phase 2) and the
// S <= 4 commit after it; issue #585 thread: kv_b, the absorption weight, is
// grouped int4):
//   query path  cq_raw = q_a x;  cq = RMSNorm(cq_raw) q_norm;  q = q_b cq
//   kv path     ckv = kv_a x;  Lc[pos] = RMSNorm(latent) kv_norm;
//               Rc[pos] = RoPE(rotary key, pos)                 (pos = pos_base + s)
//   core        qpe = RoPE(rotary part of q);  qabs = W_UK^T q_nope (per head);
//               score_t = (qabs . Lc[t] + qpe . Rc[t]) / sqrt(d_nope + d_rope)
//               for t <= pos (row s sees keys 0 .. pos_base + s);  p = softmax;
//               clat = sum_t p_t Lc[t];  ctx = W_UV clat (per head)
//   output      out = o_proj ctx
// The four projections are the library's decode GEMVs (q_a and kv_a share x
// and go out as one grouped launch); the kernels here are the steps between
// them.  Every step is a separate launch on one stream, so each reads what the
// one before wrote; nothing waits on the host.  The query latent's RMSNorm
// is folded into q_b's input staging when the matrix-core GEMV runs q_b (the
// layer's input norm likewise into the q_a / kv_a launch), and the key side
// (latent norm, rotary key, cache rows) runs in the key-absorption launch.
//
// Kernels (all HBM- or latency-bound at decode sizes; the weights they read,
// kv_b's key and value rows, are 64 x 448 x 512 int4 = 8.3 MB for the
// pages' model):
//   k_mla_qnorm       (when q_b does not fold it) one workgroup per row: f64
//                     sum of squares, f32 rounding of x * inv * w in f64
//   k_mla_qabs        4 workgroups per head, each summing a quarter of its
//                     key rows (lanes own 8 columns, 8 rows in flight per
//                     wavefront) into a partial; workgroup 0 of each head
//                     rotates the query's rotary part; one more column of
//                     workgroups normalises each new row's latent, rotates
//                     its rotary key (cos / sin in f64) and writes both
//                     cache rows
//   k_mla_scores      partial scores over a third of the L + d_rope components:
//                     4 heads x 64 keys per workgroup, the split's component
//                     chunks requested together (16-byte loads) and passed
//                     through two LDS buffers; adds the qabs partials while
//                     staging
//   k_mla_softmax_clat per 64-key chunk: the softmax statistics of each
//                     wavefront's head over all keys (the first 9 keys per
//                     lane requested together and kept in registers), then
//                     the chunk's share of clat (4 heads x 64 columns per
//                     workgroup)
//   k_mla_ctx         16 value rows per wavefront, 4 lanes per row with
//                     16-byte code loads, requested before clat (the chunks'
//                     shares added in order) is formed in LDS
// Prefill groups (more than 4 rows, up to MLA_GROUP per launch set) run the
// core on the fp32 matrix cores (v_mfma_f32_16x16x4f32, 64-row tiles):
//   k_mla_qabs_mx     once for the rows of all prefill groups, ahead of them:
//                     a 64-row tile x 64 latent columns of one head per
//                     workgroup, kv_b's key rows decoded into LDS; more
//                     workgroups of the same launch do the key side (every
//                     row's cache rows) and the query rotation
//   k_mla_scores_mx   the group's queries resident in LDS, 64-key tiles
//                     streamed; four workgroups per (head, component split)
//   k_mla_softmax_rows each row's statistics from its scores kept in
//                     registers; writes every key's score and probability
//   k_mla_clat_mx     per 64-key chunk and head: probabilities times the
//                     chunk's latent rows, column tiles through LDS
//   k_mla_clat_sum_frag adds the chunks' partials when the value absorption
//                     of all rows follows on the bf16 GEMM, writing clat also
//                     as that GEMM's prepared inputs
// At decode sizes each of these is a few dependent memory round trips of
// ~2 us each (measured per workgroup), so every kernel requests what it can
// before its first wait.
// Every partial sum is added in a fixed order by the next kernel, so reruns
// are bit-identical.
#include <algorithm>

#include "common.h"
#include "dgemm.h"
#include "layer.h"
#include "mla.h"

namespace coli {

__device__ __forceinline__ double mla_shfl_xor(double v, int m) {
    const int2 p = __builtin_bit_cast(int2, v);
    int2 q;
    q.x = __shfl_xor(p.x, m);
    q.y = __shfl_xor(p.y, m);
    return __builtin_bit_cast(double, q);
}

// rotation of pair i of a d_rope-wide rotary vector at position pos
__device__ __forceinline__ void rope_pair(float a, float b, int i, int dr, int pos, double theta,
                                          float *oa, float *ob) {
    const double ang = (double)pos * pow(theta, -(double)(2 * i) / (double)dr);
    double sn, cs;
    sincos(ang, &sn, &cs);
    *oa = (float)((double)a * cs - (double)b * sn);
    *ob = (float)((double)a * sn + (double)b * cs);
}

// ---- norms, rotary key, cache rows ----------------------------------------
// RMSNorm of one row of n inputs by a workgroup of NTH threads: f64 sum of
// squares (strided per thread, wavefront sums, wavefronts in order), every
// output the f32 rounding of x * inv * w computed in f64; part: NTH / 64
// doubles of LDS.  Contains a workgroup barrier.
template <int NTH>
__device__ __forceinline__ void mla_row_norm(const float *__restrict__ xr, int n,
                                             const float *__restrict__ w, double eps,
                                             float *__restrict__ yr, double *part) {
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    double ss = 0.0;
    for (int d = t; d < n; d += NTH) ss = fma((double)xr[d], (double)xr[d], ss);
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) ss += mla_shfl_xor(ss, m);
    if (lane == 0)
        part[wv] = ss;
    __syncthreads();
    double tot = part[0];
#pragma unroll
    for (int i = 1; i < NTH / 64; ++i) tot += part[i];
    const double inv = 1.0 / sqrt(tot / (double)n + eps);
    for (int d = t; d < n; d += NTH)
        yr[d] = (float)((double)xr[d] * inv * (w ? (double)w[d] : 1.0));
}

// the query latent's norm, one workgroup per row (when the q_b launch does
// not fold it into its input staging)
__global__ __launch_bounds__(256) void k_mla_qnorm(const float *__restrict__ cq_raw, int qr,
                                                   const float *__restrict__ qn, double eps,
                                                   float *__restrict__ cq) {
    __shared__ double part[4];
    const int s = blockIdx.x;
    mla_row_norm<256>(cq_raw + (int64_t)s * qr, qr, qn, eps, cq + (int64_t)s * qr, part);
}

// ---- key absorption and the query's rotary part ----------------------------
// grid (head, QA_SPLIT row splits): each workgroup sums its share of the
// head's d_nope key rows into its own partial (qabs_part[split]); the scores
// kernel adds the QA_SPLIT partials in split order.  A lane owns 8 columns
// (one word of codes per row); the 8 wavefronts take every 8th row of the
// split, all of a wavefront's rows requested before any is used.
constexpr int QA_NW = 8;      // wavefronts per workgroup
constexpr int QA_COLS = 512;  // latent columns per pass (8 per lane)
constexpr int QA_RB = 8;      // rows per wavefront in flight

// The extra column of workgroups (blockIdx.x == H) takes the new tokens' key
// side: workgroup (H, s) normalises row s's latent into cache row
// pos_base + s of Lc and rotates its rotary key into the same row of Rc.
template <int S, bool GRP>
__global__ __launch_bounds__(QA_NW * 64) void k_mla_qabs(MlaKvb kb, int H, int dn, int dr, int dv,
                                                         int L, const float *__restrict__ q,
                                                         int pos_base, double theta,
                                                         float *__restrict__ part,
                                                         float *__restrict__ qpe,
                                                         const float *__restrict__ ckv,
                                                         const float *__restrict__ kn, double eps,
                                                         float *__restrict__ Lc,
                                                         float *__restrict__ Rc, int nrows,
                                                         int rbase) {
    __shared__ float red[QA_NW][S][QA_COLS];
    const int h = blockIdx.x, split = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // this workgroup's S rows: rz .. rz + S - 1 of a group of nrows (the
    // partials' row count), MLA_CHUNK rows per blockIdx.z
    const int rz = rbase + MLA_CHUNK * (int)blockIdx.z;
    q += (int64_t)rz * H * (dn + dr);
    qpe += (int64_t)rz * H * dr;
    ckv += (int64_t)rz * (L + dr);
    pos_base += rz;
    if (h == H) {
        __shared__ double npart[QA_NW];
        const int s = split;
        if (s >= S)
            return;
        const int pos = pos_base + s;
        const float *xr = ckv + (int64_t)s * (L + dr);
        mla_row_norm<QA_NW * 64>(xr, L, kn, eps, Lc + (int64_t)pos * L, npart);
        for (int i = tid; i < dr / 2; i += QA_NW * 64)
            rope_pair(xr[L + 2 * i], xr[L + 2 * i + 1], i, dr, pos, theta,
                      Rc + (int64_t)pos * dr + 2 * i, Rc + (int64_t)pos * dr + 2 * i + 1);
        return;
    }
    const int nq = H * (dn + dr);
    const int rows = (dn + MLA_QA_SPLIT - 1) / MLA_QA_SPLIT;
    const int j0 = split * rows, j1 = min(dn, j0 + rows);
    const float *qh = q + (int64_t)h * (dn + dr);
    for (int col0 = 0; col0 < L; col0 += QA_COLS) {
        const int c0 = col0 + 8 * lane;  // this lane's 8 columns
        const bool live = c0 < L;
        float acc[S][8];
#pragma unroll
        for (int s = 0; s < S; ++s)
#pragma unroll
            for (int k = 0; k < 8; ++k) acc[s][k] = 0.f;
        for (int jb = j0 + wave; jb < j1; jb += QA_NW * QA_RB) {
            uint32_t wd[QA_RB];
            float sc[QA_RB], qs[QA_RB][S];
#pragma unroll
            for (int r = 0; r < QA_RB; ++r) {
                const int j = min(jb + r * QA_NW, j1 - 1);
                const int64_t row = (int64_t)h * (dn + dv) + j;
                wd[r] = live ? gload<uint32_t>(kb.q + row * kb.rb + c0 / 2) : 0x88888888u;
                sc[r] = GRP ? (live ? gload<float>(kb.s + row * kb.ng + c0 / kb.gs) : 0.f)
                            : gload<float>(kb.s + row);
#pragma unroll
                for (int s = 0; s < S; ++s) qs[r][s] = gload<float>(qh + (int64_t)s * nq + j);
            }
#pragma unroll
            for (int r = 0; r < QA_RB; ++r) {
                if (jb + r * QA_NW >= j1)
                    break;
                float f[8];
                decode_nib_word(wd[r], f);  // 16 (nibble - 8)
#pragma unroll
                for (int s = 0; s < S; ++s) {
                    const float w = qs[r][s] * sc[r] * 0.0625f;
#pragma unroll
                    for (int k = 0; k < 8; ++k) acc[s][k] = fmaf(w, f[k], acc[s][k]);
                }
            }
        }
#pragma unroll
        for (int s = 0; s < S; ++s)
#pragma unroll
            for (int k = 0; k < 8; ++k) red[wave][s][8 * lane + k] = acc[s][k];
        __syncthreads();
        for (int idx = tid; idx < S * QA_COLS; idx += QA_NW * 64) {
            const int s = idx / QA_COLS, c = idx % QA_COLS;
            if (col0 + c < L) {
                float v = red[0][s][c];
#pragma unroll
                for (int w = 1; w < QA_NW; ++w) v += red[w][s][c];
                part[(((int64_t)split * nrows + rz + s) * H + h) * L + col0 + c] = v;
            }
        }
        __syncthreads();
    }
    if (split == 0)
        for (int idx = tid; idx < S * (dr / 2); idx += QA_NW * 64) {
            const int s = idx / (dr / 2), i = idx % (dr / 2);
            const float *qr = q + (int64_t)s * nq + (int64_t)h * (dn + dr) + dn;
            float *o = qpe + ((int64_t)s * H + h) * dr;
            rope_pair(qr[2 * i], qr[2 * i + 1], i, dr, pos_base + s, theta, o + 2 * i, o + 2 * i + 1);
        }
}

// Prefill rows (all rows of the prefill groups, before the first group's
// scores): the key absorption on the fp32 matrix cores, with the key side and
// the query rotation as other workgroups of the same launch.  Workgroups
// [0, nrt * H * ncol): qabs[s][h][c] = sum_j q[s][h][j] W_UK[h][j][c] for one
// 64-row tile x 64 latent columns of head h, over the
// d_nope key rows in chunks of 64 (query values and kv_b's key rows, the
// latter decoded to s * (q - 8) exactly as the vector kernel forms them and
// stored column-major, through LDS; the next chunk requested while the
// current one is multiplied); wavefront w takes rows 16 w .. 16 w + 15 as
// four 16 x 16 tiles of v_mfma_f32_16x16x4f32, product j giving lane group
// g = l / 16 key row 4 g + j of each 16-row block (16-byte LDS operand
// reads).  The next S workgroups: the key side of row s (latent RMSNorm into
// cache row pos_base + s of Lc, rotary key into the same row of Rc); the last
// S: the rotation of row s's query rotary parts into qpe.
constexpr int QX_T = 64;             // rows, key rows and columns per tile
constexpr int QX_LD = QX_T + 4;      // LDS row stride
template <bool GRP>
__global__ __launch_bounds__(256) void k_mla_qabs_mx(MlaKvb kb, int S, int H, int dn, int dr,
                                                     int dv, int L, const float *__restrict__ q,
                                                     int pos_base, double theta,
                                                     float *__restrict__ qabs,
                                                     float *__restrict__ qpe,
                                                     const float *__restrict__ ckv,
                                                     const float *__restrict__ kn, double eps,
                                                     float *__restrict__ Lc,
                                                     float *__restrict__ Rc) {
    __shared__ __attribute__((aligned(16))) float qa[QX_T][QX_LD];  // [row][key row]
    __shared__ __attribute__((aligned(16))) float wt[QX_T][QX_LD];  // [column][key row]
    __shared__ double npart[4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int ncol = (L + QX_T - 1) / QX_T;
    const int nrt = (S + QX_T - 1) / QX_T;
    const int nq = H * (dn + dr);
    int bx = blockIdx.x;
    if (bx >= nrt * H * ncol) {
        bx -= nrt * H * ncol;
        if (bx < S) {  // key side of row bx
            const int pos = pos_base + bx;
            const float *xr = ckv + (int64_t)bx * (L + dr);
            mla_row_norm<256>(xr, L, kn, eps, Lc + (int64_t)pos * L, npart);
            for (int i = tid; i < dr / 2; i += 256)
                rope_pair(xr[L + 2 * i], xr[L + 2 * i + 1], i, dr, pos, theta,
                          Rc + (int64_t)pos * dr + 2 * i, Rc + (int64_t)pos * dr + 2 * i + 1);
        } else if (bx < 2 * S) {  // query rotation of row bx - S
            const int srow = bx - S;
            for (int idx = tid; idx < H * (dr / 2); idx += 256) {
                const int h = idx / (dr / 2), i = idx % (dr / 2);
                const float *qr = q + (int64_t)srow * nq + (int64_t)h * (dn + dr) + dn;
                float *o = qpe + ((int64_t)srow * H + h) * dr;
                rope_pair(qr[2 * i], qr[2 * i + 1], i, dr, pos_base + srow, theta, o + 2 * i, o + 2 * i + 1);
            }
        }
        return;
    }
    // this workgroup's row tile: rows r0 .. r0 + Sl - 1 of the call
    const int r0 = (bx / (H * ncol)) * QX_T;
    bx %= H * ncol;
    const int Sl = min(QX_T, S - r0);
    q += (int64_t)r0 * nq;
    qabs += (int64_t)r0 * H * L;
    const int h = bx / ncol, c0 = (bx % ncol) * QX_T;
    const int rr = tid >> 4, j4 = 4 * (tid & 15);  // query staging: rows rr + 16 i, key rows j4 .. + 3
    // the query rows' 4-value runs are 16-byte aligned (16-byte aligned q,
    // head strides a multiple of 4 values)
    const bool qvec = (uintptr_t)q % 16 == 0 && (dn + dr) % 4 == 0;
    const int wr = tid >> 2, w8 = 16 * (tid & 3);  // weight staging: key row wr, columns w8 .. + 15
    f32x4 qv[4];
    float wv[16];
    auto request = [&](int j0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = rr + 16 * i, j = j0 + j4;
            f32x4 v = {0.f, 0.f, 0.f, 0.f};
            if (r < Sl) {
                const float *qr = q + (int64_t)r * nq + (int64_t)h * (dn + dr);
                if (qvec && j + 4 <= dn) {
                    v = gload<f32x4>(qr + j);  // one 16-byte load
                } else {
                    float e[4];
#pragma unroll
                    for (int k = 0; k < 4; ++k) e[k] = j + k < dn ? qr[j + k] : 0.f;
                    v = f32x4{e[0], e[1], e[2], e[3]};
                }
            }
            qv[i] = v;
        }
        const int j = j0 + wr;
        const int64_t row = (int64_t)h * (dn + dv) + min(j, dn - 1);
        const int c = c0 + w8;  // 16 columns (a multiple of 16, so c < L covers all 16)
        uint32_t w2[2] = {0x88888888u, 0x88888888u};
        float sc2[2] = {0.f, 0.f};
        if (j < dn && c < L) {
            // both code words in one 8-byte load; one scale when the 16
            // columns share a group
            const u32x2 v = gload<u32x2>(kb.q + row * kb.rb + c / 2);
            w2[0] = v.x;
            w2[1] = v.y;
            if (!GRP) {
                sc2[0] = sc2[1] = gload<float>(kb.s + row);
            } else if (kb.gs % 16 == 0) {
                sc2[0] = sc2[1] = gload<float>(kb.s + row * kb.ng + c / kb.gs);
            } else {
                sc2[0] = gload<float>(kb.s + row * kb.ng + c / kb.gs);
                sc2[1] = gload<float>(kb.s + row * kb.ng + (c + 8) / kb.gs);
            }
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            float f[8];
            decode_nib_word(w2[u], f);  // 16 (nibble - 8)
            const float k16 = sc2[u] * 0.0625f;
#pragma unroll
            for (int k = 0; k < 8; ++k) wv[8 * u + k] = f[k] * k16;
        }
    };
    const int am = 16 * wave + (lane & 15), bn = lane & 15, g4 = 4 * (lane >> 4);
    f32x4 acc[4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    request(0);
    for (int j0 = 0; j0 < dn; j0 += QX_T) {
        __syncthreads();  // the previous chunk's products are done with qa and wt
#pragma unroll
        for (int i = 0; i < 4; ++i) *reinterpret_cast<f32x4 *>(&qa[rr + 16 * i][j4]) = qv[i];
#pragma unroll
        for (int k = 0; k < 16; ++k) wt[w8 + k][wr] = wv[k];
        __syncthreads();
        if (j0 + QX_T < dn)
            request(j0 + QX_T);
#pragma unroll
        for (int kb4 = 0; kb4 < QX_T; kb4 += 16) {
            const f32x4 a4 = *reinterpret_cast<const f32x4 *>(&qa[am][kb4 + g4]);
            f32x4 b4[4];
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) b4[nb] = *reinterpret_cast<const f32x4 *>(&wt[16 * nb + bn][kb4 + g4]);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
#pragma unroll
                for (int nb = 0; nb < 4; ++nb)
                    acc[nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a4[jj], b4[nb][jj], acc[nb], 0, 0, 0);
        }
    }
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 16 * wave + 4 * (lane >> 4) + i, c = c0 + 16 * nb + (lane & 15);
            if (r < Sl && c < L)
                qabs[((int64_t)r * H + h) * L + c] = acc[nb][i];
        }
}

// ---- scores ----------------------------------------------------------------
// Partial scores over one third of the L + d_rope components (Q = [qabs,
// qpe], K = [Lc, Rc]): grid (64-key tiles, 4-head groups, row x MLA_SC_SPLIT).
// A workgroup takes 4 heads (one per wavefront) x 64 keys (one per lane);
// its components go through LDS in chunks of 64 (keys padded to 65 floats),
// the next chunk's loads issued before the current one is used; each chunk is
// summed on its own and then added.  The softmax kernel adds the splits in
// order and scales.  qabs is the sum of the key-absorption partials, formed
// while staging; the first key tile stores it.
constexpr int SC_KEYS = 64;
constexpr int SC_HEADS = 4;
constexpr int SC_CH = 64;
constexpr int SC_MAXCH = 3;  // component chunks requested together (decode kernel)

__global__ __launch_bounds__(256) void k_mla_scores(const float *__restrict__ part,
                                                    const float *__restrict__ qpe,
                                                    const float *__restrict__ Lc,
                                                    const float *__restrict__ Rc, int S, int H,
                                                    int L, int dr, int pos_base, int Tcap,
                                                    int lvec, float *__restrict__ qabs,
                                                    float *__restrict__ sc_part) {
    __shared__ float kt[2][SC_KEYS][SC_CH + 1];
    __shared__ float qt[2][SC_HEADS][SC_CH];
    const int t0 = blockIdx.x * SC_KEYS, h0 = blockIdx.y * SC_HEADS;
    const int s = blockIdx.z / MLA_SC_SPLIT, split = blockIdx.z % MLA_SC_SPLIT;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int last = pos_base + s;  // keys 0 .. last
    if (t0 > last)
        return;
    const int C = L + dr;
    const int nch_all = (C + SC_CH - 1) / SC_CH;
    const int per = (nch_all + MLA_SC_SPLIT - 1) / MLA_SC_SPLIT;
    const int ch0 = split * per, ch1 = min(nch_all, ch0 + per);
    const int64_t pstride = (int64_t)S * H * L;
    // key components: thread t takes 4 consecutive components (c4 = 4 (t % 16))
    // of keys t / 16 + 16 i; the latent part with 16-byte loads (L % 4 == 0,
    // lvec: Lc 16-byte aligned), the rotary part component by component
    const int kk = tid >> 4, c4 = 4 * (tid & 15);
    auto fetch = [&](f32x4 (&kr)[4], float &qv, int c0) {
        const int c = c0 + c4;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = t0 + kk + 16 * i;
            f32x4 v = {0.f, 0.f, 0.f, 0.f};
            if (t <= last) {
                if (c + 4 <= L && lvec) {
                    v = gload<f32x4>(Lc + (int64_t)t * L + c);
                } else {
                    float e[4];
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const int ck = c + k;
                        e[k] = ck < L ? Lc[(int64_t)t * L + ck] : (ck < C ? Rc[(int64_t)t * dr + (ck - L)] : 0.f);
                    }
                    v = f32x4{e[0], e[1], e[2], e[3]};
                }
            }
            kr[i] = v;
        }
        const int hh = tid / SC_CH, cq = tid % SC_CH;  // 4 heads x 64 components
        const int h = h0 + hh, cc = c0 + cq;
        float v = 0.f;
        if (h < H && cc < C) {
            if (cc < L) {
                const float *pp = part + ((int64_t)s * H + h) * L + cc;
                v = pp[0];
#pragma unroll
                for (int k = 1; k < MLA_QA_SPLIT; ++k) v += pp[k * pstride];
            } else {
                v = qpe[((int64_t)s * H + h) * dr + (cc - L)];
            }
        }
        qv = v;
    };
    auto store = [&](int buf, const f32x4 (&kr)[4], float qv, int c0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float *row = &kt[buf][kk + 16 * i][c4];
            row[0] = kr[i].x; row[1] = kr[i].y; row[2] = kr[i].z; row[3] = kr[i].w;
        }
        const int hh = tid / SC_CH, cq = tid % SC_CH;
        qt[buf][hh][cq] = qv;
        if (blockIdx.x == 0 && h0 + hh < H && c0 + cq < L)
            qabs[((int64_t)s * H + h0 + hh) * L + c0 + cq] = qv;
    };
    // up to SC_MAXCH chunks are requested together (one memory round trip for
    // all of them), then go through the two LDS buffers in turn; the chunk
    // sums are added in chunk order
    float tot = 0.f;
    for (int g0 = ch0; g0 < ch1; g0 += SC_MAXCH) {
        f32x4 kr[SC_MAXCH][4];
        float qv[SC_MAXCH];
#pragma unroll
        for (int j = 0; j < SC_MAXCH; ++j)
            fetch(kr[j], qv[j], min(g0 + j, ch1 - 1) * SC_CH);
#pragma unroll
        for (int j = 0; j < SC_MAXCH; ++j) {
            if (g0 + j >= ch1)
                break;
            store(j & 1, kr[j], qv[j], (g0 + j) * SC_CH);
            __syncthreads();
            float a = 0.f;
#pragma unroll 16
            for (int cc = 0; cc < SC_CH; ++cc) a = fmaf(qt[j & 1][wave][cc], kt[j & 1][lane][cc], a);
            tot += a;
        }
        __syncthreads();
    }
    const int t = t0 + lane, h = h0 + wave;
    if (t <= last && h < H)
        sc_part[(((int64_t)split * S + s) * H + h) * Tcap + t] = tot;
}

// Prefill rows on the fp32 matrix cores: partial scores over one third of
// the L + d_rope components for one head and a 64-row tile of the group;
// grid (SX_KW key-tile lanes, heads, row tiles x MLA_SC_SPLIT): workgroup x takes the
// 64-key tiles x, x + SX_KW, ...  The query tile of the split (qabs, then
// qpe) is staged once into LDS and stays there while the key tiles stream
// through, component chunk by chunk (64
// components; the next chunk requested into registers while the current one
// is multiplied).  Wavefront w takes rows 16 w .. 16 w + 15 against the 64
// keys of a tile as four 16 x 16 tiles of v_mfma_f32_16x16x4f32 (A lane l =
// Q[l % 16][k], B lane l = K[k][l % 16] for the product's k index l / 16,
// result lane l register i = row 4 (l / 16) + i, key l % 16); within each
// 16-component block, product j gives lane group g = l / 16 component
// 4 g + j, so a lane reads its four components with one 16-byte LDS read
// (the sum over the block is the same up to rounding order).  Rows past S, keys past the group's last
// position and scores past a row's own position are neither loaded nor
// stored.  A split of more than SX_QCH chunks stages its query chunks again
// for every key tile.
constexpr int SX_T = 64;    // rows = keys per tile
// workgroups per (head, split), along the key tiles
#ifndef COLI_MLA_SX_KW
#define COLI_MLA_SX_KW 4
#endif
constexpr int SX_KW = COLI_MLA_SX_KW;
constexpr int SX_QCH = 3;   // query chunks kept in LDS
constexpr int SX_LD = SC_CH + 4;  // LDS row stride (16-byte rows for the 4-component reads)
__global__ __launch_bounds__(256) void k_mla_scores_mx(const float *__restrict__ qabs,
                                                       const float *__restrict__ qpe,
                                                       const float *__restrict__ Lc,
                                                       const float *__restrict__ Rc, int S, int H,
                                                       int L, int dr, int pos_base, int Tcap,
                                                       int lvec, float *__restrict__ sc_part) {
    __shared__ __attribute__((aligned(16))) float qs[SX_QCH][SX_T][SX_LD];
    __shared__ __attribute__((aligned(16))) float ks[SX_T][SX_LD];
    // grid z: (row tile, split); this workgroup's rows r0 .. r0 + Sl - 1
    const int h = blockIdx.y, split = (int)blockIdx.z % MLA_SC_SPLIT;
    const int r0 = ((int)blockIdx.z / MLA_SC_SPLIT) * SX_T, Sl = min(SX_T, S - r0);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int last_max = pos_base + r0 + Sl - 1;  // keys 0 .. last of the tile's last row
    const int nkt = last_max / SX_T + 1;
    const int C = L + dr;
    const int nch_all = (C + SC_CH - 1) / SC_CH;
    const int per = (nch_all + MLA_SC_SPLIT - 1) / MLA_SC_SPLIT;
    // rotary runs of 4 on 16-byte boundaries (L is a multiple of 32)
    const bool rvec = lvec && dr % 4 == 0 && (uintptr_t)qpe % 16 == 0 && (uintptr_t)Rc % 16 == 0;
    // (a split with no chunks, when L + d_rope is short, stores zero partials)
    const int ch0 = split * per, ch1 = min(nch_all, ch0 + per);
    // staging: thread t takes 4 consecutive components (4 (t % 16)) of rows /
    // keys t / 16 + 16 i, i < 4
    const int rr = tid >> 4, c4 = 4 * (tid & 15);
    auto qload = [&](f32x4 (&qv)[4], int c0) {
        const int c = c0 + c4;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = rr + 16 * i;
            f32x4 q = {0.f, 0.f, 0.f, 0.f};
            if (r < Sl) {
                if (c + 4 <= L) {
                    q = gload<f32x4>(qabs + ((int64_t)(r0 + r) * H + h) * L + c);
                } else if (rvec && c >= L && c + 4 <= C) {  // rotary part, 16-byte aligned
                    q = gload<f32x4>(qpe + ((int64_t)(r0 + r) * H + h) * dr + (c - L));
                } else {
                    float e[4];
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const int ck = c + k;
                        e[k] = ck < L ? qabs[((int64_t)(r0 + r) * H + h) * L + ck]
                                      : (ck < C ? qpe[((int64_t)(r0 + r) * H + h) * dr + (ck - L)] : 0.f);
                    }
                    q = f32x4{e[0], e[1], e[2], e[3]};
                }
            }
            qv[i] = q;
        }
    };
    auto kload = [&](f32x4 (&kv)[4], int t0, int c0) {
        const int c = c0 + c4;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = t0 + rr + 16 * i;
            f32x4 k4 = {0.f, 0.f, 0.f, 0.f};
            if (t <= last_max) {
                if (c + 4 <= L && lvec) {
                    k4 = gload<f32x4>(Lc + (int64_t)t * L + c);
                } else if (rvec && c >= L && c + 4 <= C) {  // rotary key, 16-byte aligned
                    k4 = gload<f32x4>(Rc + (int64_t)t * dr + (c - L));
                } else {
                    float e[4];
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const int ck = c + k;
                        e[k] = ck < L ? Lc[(int64_t)t * L + ck] : (ck < C ? Rc[(int64_t)t * dr + (ck - L)] : 0.f);
                    }
                    k4 = f32x4{e[0], e[1], e[2], e[3]};
                }
            }
            kv[i] = k4;
        }
    };
    auto put = [&](float (*dst)[SX_LD], const f32x4 (&v)[4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) *reinterpret_cast<f32x4 *>(&dst[rr + 16 * i][c4]) = v[i];
    };
    const bool qres = ch1 - ch0 <= SX_QCH;  // the split's query chunks stay in LDS
    const int am = 16 * wave + (lane & 15), bn = lane & 15, g4 = 4 * (lane >> 4);
    bool qdone = false;
    for (int kt = blockIdx.x; kt < nkt; kt += gridDim.x) {
        const int t0 = kt * SX_T;
        f32x4 acc[4];
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
        f32x4 qv[4], kv[4];
        // chunk c's query values (when not resident) and keys are requested
        // during chunk c - 1
        auto request = [&](int ch) {
            if (!qres || !qdone)
                qload(qv, ch * SC_CH);
            kload(kv, t0, ch * SC_CH);
        };
        if (ch0 < ch1)
            request(ch0);
        for (int ch = ch0; ch < ch1; ++ch) {
            const int qi = qres ? ch - ch0 : 0;
            __syncthreads();  // the previous chunk's products are done with ks (and qs[qi])
            if (!qres || !qdone)
                put(qs[qi], qv);
            put(ks, kv);
            __syncthreads();
            if (ch + 1 < ch1)
                request(ch + 1);
#pragma unroll
            for (int kb = 0; kb < SC_CH; kb += 16) {
                const f32x4 a4 = *reinterpret_cast<const f32x4 *>(&qs[qi][am][kb + g4]);
                f32x4 b4[4];
#pragma unroll
                for (int nb = 0; nb < 4; ++nb)
                    b4[nb] = *reinterpret_cast<const f32x4 *>(&ks[16 * nb + bn][kb + g4]);
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int nb = 0; nb < 4; ++nb)
                        acc[nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a4[j], b4[nb][j], acc[nb], 0, 0, 0);
            }
        }
        qdone = true;
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * wave + 4 * (lane >> 4) + i, t = t0 + 16 * nb + (lane & 15);
                if (r < Sl && t <= pos_base + r0 + r)
                    sc_part[(((int64_t)split * S + r0 + r) * H + h) * Tcap + t] = acc[nb][i];
            }
    }
}

// ---- softmax and the latent context ----------------------------------------
// grid (64-key chunks, 64-column tiles, 4-head groups x rows).  Each wavefront
// first forms its head's scores z_t = scale * (sum of the score splits in
// order) over keys 0 .. pos_base + s and their softmax statistics (strided
// max and sum of exp(z - max), then wavefront shuffles in a fixed order);
// then its workgroup's chunk: p = exp(z - max) / sum for 64 keys in LDS, the
// chunk's Lc rows in LDS, and the chunk's share of clat[h][c] = sum_t p Lc[t][c]
// into its own partial.  The value-absorption kernel adds the partials in
// chunk order.  Column tile 0 stores the chunk's scores and probabilities.
constexpr int CL_COLS = 64;
constexpr int CL_HEADS = 4;
constexpr int CL_KEYS = 64;
// keys per lane whose scores are requested together
#ifndef COLI_MLA_SM_KJ
#define COLI_MLA_SM_KJ 9
#endif
constexpr int SM_KJ = COLI_MLA_SM_KJ;

__device__ __forceinline__ float mla_score(const float *__restrict__ sc_part, int64_t sstride,
                                           int64_t at, float scale) {
    float z = sc_part[at];
#pragma unroll
    for (int k = 1; k < MLA_SC_SPLIT; ++k) z += sc_part[at + k * sstride];
    return z * scale;
}

__global__ __launch_bounds__(256) void k_mla_softmax_clat(const float *__restrict__ sc_part,
                                                          const float *__restrict__ Lc, int S, int H,
                                                          int L, int pos_base, int Tcap, float scale,
                                                          float *__restrict__ scores,
                                                          float *__restrict__ p,
                                                          float *__restrict__ cl_part) {
    __shared__ float lt[CL_KEYS][CL_COLS + 1];
    __shared__ float pt[CL_HEADS][CL_KEYS];
    const int chunk = blockIdx.x, t0 = chunk * CL_KEYS, c0 = blockIdx.y * CL_COLS;
    const int ng = (H + CL_HEADS - 1) / CL_HEADS;
    const int s = blockIdx.z / ng, h0 = (blockIdx.z % ng) * CL_HEADS;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = pos_base + s + 1;
    if (t0 >= n)
        return;
    const int64_t sstride = (int64_t)S * H * Tcap;
    // this chunk's Lc rows: requested first, they do not depend on the scores
    float lr[CL_KEYS * CL_COLS / 256];
#pragma unroll
    for (int i = 0; i < CL_KEYS * CL_COLS / 256; ++i) {
        const int idx = tid + 256 * i, tt = idx / CL_COLS, c = idx % CL_COLS;
        const int t = t0 + tt;
        lr[i] = (t < n && c0 + c < L) ? Lc[(int64_t)t * L + c0 + c] : 0.f;
    }
    // softmax statistics of this wavefront's head: lane l takes keys l, l + 64,
    // ...; the first SM_KJ of them are requested together and kept (a key
    // past n reads as -inf: it moves neither the maximum nor the sum), later
    // ones are read again for the sum
    const int h = h0 + wave;
    const int64_t zrow = ((int64_t)s * H + min(h, H - 1)) * Tcap;
    float zk[SM_KJ];
#pragma unroll
    for (int j = 0; j < SM_KJ; ++j) {
        const int t = lane + 64 * j;
        const float z = mla_score(sc_part, sstride, zrow + min(t, n - 1), scale);
        zk[j] = t < n ? z : -__builtin_inff();
    }
    float m = -__builtin_inff();
#pragma unroll
    for (int j = 0; j < SM_KJ; ++j) m = fmaxf(m, zk[j]);
    for (int t = lane + 64 * SM_KJ; t < n; t += 64) m = fmaxf(m, mla_score(sc_part, sstride, zrow + t, scale));
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    float e = 0.f;
#pragma unroll
    for (int j = 0; j < SM_KJ; ++j) e += expf(zk[j] - m);
    for (int t = lane + 64 * SM_KJ; t < n; t += 64) e += expf(mla_score(sc_part, sstride, zrow + t, scale) - m);
    e = wave_sum(e);
    {
        const int t = t0 + lane;
        float pv = 0.f;
        if (h < H && t < n) {
            float z = zk[0];
#pragma unroll
            for (int j = 1; j < SM_KJ; ++j) z = chunk == j ? zk[j] : z;
            if (chunk >= SM_KJ)
                z = mla_score(sc_part, sstride, zrow + t, scale);
            pv = expf(z - m) / e;
            if (blockIdx.y == 0) {
                scores[zrow + t] = z;
                p[zrow + t] = pv;
            }
        }
        pt[wave][lane] = pv;
    }
#pragma unroll
    for (int i = 0; i < CL_KEYS * CL_COLS / 256; ++i) {
        const int idx = tid + 256 * i;
        lt[idx / CL_COLS][idx % CL_COLS] = lr[i];
    }
    __syncthreads();
    float a = 0.f;
#pragma unroll 16
    for (int tt = 0; tt < CL_KEYS; ++tt) a = fmaf(pt[wave][tt], lt[tt][lane], a);
    const int c = c0 + lane;
    if (h < H && c < L)
        cl_part[(((int64_t)chunk * S + s) * H + h) * L + c] = a;
}

// Prefill rows: the softmax of each (row, head) -- the same strided max and
// sum of exp(z - max) as above, in the same order (the first SM_KJ keys per
// lane requested together and kept) -- then the row's scores and
// probabilities p = exp(z - max) / sum for every key; grid (rows, 4-head
// groups), a wavefront per head.
__global__ __launch_bounds__(256) void k_mla_softmax_rows(const float *__restrict__ sc_part,
                                                          int S, int H, int pos_base, int Tcap,
                                                          float scale, float *__restrict__ scores,
                                                          float *__restrict__ p) {
    const int s = blockIdx.x, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int h = blockIdx.y * CL_HEADS + wave;
    if (h >= H)
        return;  // whole wavefront
    const int n = pos_base + s + 1;
    const int64_t sstride = (int64_t)S * H * Tcap;
    const int64_t zrow = ((int64_t)s * H + h) * Tcap;
    float zk[SM_KJ];
#pragma unroll
    for (int j = 0; j < SM_KJ; ++j) {
        const int t = lane + 64 * j;
        const float z = mla_score(sc_part, sstride, zrow + min(t, n - 1), scale);
        zk[j] = t < n ? z : -__builtin_inff();
    }
    float m = -__builtin_inff();
#pragma unroll
    for (int j = 0; j < SM_KJ; ++j) m = fmaxf(m, zk[j]);
    for (int t = lane + 64 * SM_KJ; t < n; t += 64) m = fmaxf(m, mla_score(sc_part, sstride, zrow + t, scale));
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    float e = 0.f;
#pragma unroll
    for (int j = 0; j < SM_KJ; ++j) e += expf(zk[j] - m);
    for (int t = lane + 64 * SM_KJ; t < n; t += 64) e += expf(mla_score(sc_part, sstride, zrow + t, scale) - m);
    e = wave_sum(e);
#pragma unroll
    for (int j = 0; j < SM_KJ; ++j) {
        const int t = lane + 64 * j;
        if (t < n) {
            scores[zrow + t] = zk[j];
            p[zrow + t] = expf(zk[j] - m) / e;
        }
    }
    for (int t = lane + 64 * SM_KJ; t < n; t += 64) {
        const float z = mla_score(sc_part, sstride, zrow + t, scale);
        scores[zrow + t] = z;
        p[zrow + t] = expf(z - m) / e;
    }
}

// Prefill rows on the fp32 matrix cores: one 64-key chunk's share of clat
// for one head and a 64-row tile of the group; grid (64-key chunks, CX_CW
// column groups, row tiles x heads), each workgroup taking every CX_CW-th 64-column
// tile; the partials k_mla_softmax_clat writes for decode rows
// (cl_part[chunk][s][h][c] for the chunks that hold keys of row s).  The
// chunk's probabilities (written by k_mla_softmax_rows) are staged once into
// LDS; the column tiles of the chunk's Lc rows follow one another through LDS
// (transposed, key-contiguous; the next tile requested while the current one
// is multiplied).  Wavefront w takes rows 16 w .. 16 w + 15 x the 64 columns
// as four 16 x 16 tiles of v_mfma_f32_16x16x4f32 over the 64 keys, product j
// giving lane group g = l / 16 key 4 g + j of each 16-key block (16-byte LDS
// operand reads).
constexpr int CX_T = 64;               // rows, keys and columns per tile
constexpr int CX_LD = CX_T + 4;        // LDS row stride
#ifndef COLI_MLA_CX_CW
#define COLI_MLA_CX_CW 4
#endif
constexpr int CX_CW = COLI_MLA_CX_CW;  // workgroups per (chunk, head), along the column tiles
static_assert(CX_T == CL_KEYS, "the partials are per key chunk of CL_KEYS");
__global__ __launch_bounds__(256) void k_mla_clat_mx(const float *__restrict__ p,
                                                     const float *__restrict__ Lc, int S, int H,
                                                     int L, int pos_base, int Tcap, int lvec,
                                                     float *__restrict__ cl_part) {
    __shared__ __attribute__((aligned(16))) float ps[CX_T][CX_LD];  // [row][key]
    __shared__ __attribute__((aligned(16))) float lt[CX_T][CX_LD];  // [column][key]
    // grid z: (row tile, head); this workgroup's rows r0 .. r0 + Sl - 1
    const int chunk = blockIdx.x, t0 = chunk * CX_T, h = (int)blockIdx.z % H;
    const int r0 = ((int)blockIdx.z / H) * CX_T, Sl = min(CX_T, S - r0);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n_max = pos_base + r0 + Sl;  // keys of the tile's last row
    if (t0 >= n_max)
        return;
    const int rr = tid >> 4, c4 = 4 * (tid & 15);
    const int nct = (L + CX_T - 1) / CX_T;
    // the Lc rows of a column tile (keys rr + 16 i, columns c0 + c4 .. + 3)
    f32x4 lv[4];
    auto lload = [&](int c0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = t0 + rr + 16 * i, c = c0 + c4;
            f32x4 v = {0.f, 0.f, 0.f, 0.f};
            if (t < n_max) {
                if (c + 4 <= L && lvec) {
                    v = gload<f32x4>(Lc + (int64_t)t * L + c);
                } else {
                    float e[4];
#pragma unroll
                    for (int k = 0; k < 4; ++k) e[k] = c + k < L ? Lc[(int64_t)t * L + c + k] : 0.f;
                    v = f32x4{e[0], e[1], e[2], e[3]};
                }
            }
            lv[i] = v;
        }
    };
    if (blockIdx.y < nct)
        lload(blockIdx.y * CX_T);  // requested first: it does not depend on the scores
    // probabilities of rows rr + 16 i at keys t0 + c4 .. + 3 (requested at
    // once at clamped addresses, zero past each row's own position)
    float pz[4][4];
    const bool pvec = (uintptr_t)p % 16 == 0 && Tcap % 4 == 0 && t0 + c4 + 4 <= Tcap;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t prow = ((int64_t)(r0 + min(rr + 16 * i, Sl - 1)) * H + h) * Tcap;
        if (pvec) {  // one 16-byte load
            const f32x4 v = gload<f32x4>(p + prow + t0 + c4);
            pz[i][0] = v.x; pz[i][1] = v.y; pz[i][2] = v.z; pz[i][3] = v.w;
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) pz[i][k] = p[prow + min(t0 + c4 + k, Tcap - 1)];
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = rr + 16 * i;
        float pv[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) pv[k] = (r < Sl && t0 + c4 + k < pos_base + r0 + r + 1) ? pz[i][k] : 0.f;
        *reinterpret_cast<f32x4 *>(&ps[r][c4]) = f32x4{pv[0], pv[1], pv[2], pv[3]};
    }
    const int am = 16 * wave + (lane & 15), bn = lane & 15, g4 = 4 * (lane >> 4);
    for (int ct = blockIdx.y; ct < nct; ct += gridDim.y) {
        const int c0 = ct * CX_T;
        __syncthreads();  // the previous tile's products are done with lt
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int kk = rr + 16 * i;
            lt[c4][kk] = lv[i].x;
            lt[c4 + 1][kk] = lv[i].y;
            lt[c4 + 2][kk] = lv[i].z;
            lt[c4 + 3][kk] = lv[i].w;
        }
        __syncthreads();
        if (ct + (int)gridDim.y < nct)
            lload(c0 + (int)gridDim.y * CX_T);
        f32x4 acc[4];
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < CX_T; kb += 16) {
            const f32x4 a4 = *reinterpret_cast<const f32x4 *>(&ps[am][kb + g4]);
            f32x4 b4[4];
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) b4[nb] = *reinterpret_cast<const f32x4 *>(&lt[16 * nb + bn][kb + g4]);
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int nb = 0; nb < 4; ++nb)
                    acc[nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a4[j], b4[nb][j], acc[nb], 0, 0, 0);
        }
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * wave + 4 * (lane >> 4) + i, c = c0 + 16 * nb + (lane & 15);
                if (r < Sl && c < L && t0 < pos_base + r0 + r + 1)
                    cl_part[(((int64_t)chunk * S + r0 + r) * H + h) * L + c] = acc[nb][i];
            }
    }
}

// Prefill rows whose value absorption runs on the matrix cores afterwards:
// clat[s][h][c] = the key chunks' partials of row s (one per kpp keys) added
// in chunk order, written as f32 and as the split-K GEMM's prepared bf16
// inputs (batch h of the value absorption at xf + h per: row r0 + s, input
// c; the inputs from L up to nkb4 blocks zero); one thread per 8 values.
__global__ __launch_bounds__(256) void k_mla_clat_sum_frag(const float *__restrict__ cl_part, int S,
                                                           int H, int L, int pos_base, int kpp,
                                                           float *__restrict__ clat, int r0,
                                                           uint8_t *__restrict__ xf, int64_t per,
                                                           int nkb4) {
    const int L8 = nkb4 * 128 / 8;  // 8-input groups per row, padding included
    const int64_t n8 = (int64_t)S * H * L8;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n8)
        return;
    const int s = (int)(i / ((int64_t)H * L8));
    const int h = (int)((i / L8) % H), c = 8 * (int)(i % L8);
    f32x4 v0 = {0.f, 0.f, 0.f, 0.f}, v1 = v0;
    if (c < L) {
        const int64_t n = (int64_t)S * H * L, o = ((int64_t)s * H + h) * L + c;
        const int nchunk = (pos_base + s + 1 + kpp - 1) / kpp;
        v0 = gload<f32x4>(cl_part + o);
        v1 = gload<f32x4>(cl_part + o + 4);
        for (int k = 1; k < nchunk; ++k) {
            v0 += gload<f32x4>(cl_part + o + (int64_t)k * n);
            v1 += gload<f32x4>(cl_part + o + (int64_t)k * n + 4);
        }
        *reinterpret_cast<f32x4 *>(clat + o) = v0;
        *reinterpret_cast<f32x4 *>(clat + o + 4) = v1;
    }
    const u32x4 b = {dgemm_bf16x2(v0.x, v0.y), dgemm_bf16x2(v0.z, v0.w), dgemm_bf16x2(v1.x, v1.y),
                     dgemm_bf16x2(v1.z, v1.w)};
    *reinterpret_cast<u32x4 *>(xf + (int64_t)h * per + dgemm_frag_offset(r0 + s, c, nkb4)) = b;
}

// ---- value absorption --------------------------------------------------------
// ctx[h][v] = sum_c kv_b[h (dn+dv) + dn + v][c] clat[h][c]: a wavefront takes
// 16 value rows, 4 lanes per row, each lane 16-byte loads (32 columns) of its
// row at chunks q, q+4, ... (the 4 lanes of a row read 64 contiguous bytes);
// clat of the head sits in LDS; the 4 lanes' sums are combined by two xor
// shuffles.  Needs L % 32 == 0.
constexpr int CX_ROWS = 64;  // value rows per workgroup (16 per wavefront)
constexpr int CX_CH = 4;     // 32-column chunks per lane whose codes are requested up front
constexpr int CX_KC = 16;    // key chunks of latent-context partials requested together

template <int S, bool GRP>
__global__ __launch_bounds__(256) void k_mla_ctx(MlaKvb kb, int H, int dn, int dv, int L,
                                                 int pos_base, const float *__restrict__ cl_part,
                                                 float *__restrict__ clat,
                                                 float *__restrict__ ctx, int nrows, int rbase) {
    extern __shared__ __attribute__((aligned(16))) float cl[];  // [S][L]
    const int h = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // rows rz .. rz + S - 1 of a group of nrows (the partials' row count)
    const int rz = rbase + MLA_CHUNK * (int)blockIdx.z;
    cl_part += (int64_t)rz * H * L;
    clat += (int64_t)rz * H * L;
    ctx += (int64_t)rz * H * dv;
    pos_base += rz;
    const int v = blockIdx.y * CX_ROWS + wave * 16 + (lane >> 2);
    const int q = lane & 3;
    const bool live = v < dv;
    const int64_t row = (int64_t)h * (dn + dv) + dn + min(v, dv - 1);
    const int nch = L / 32;
    // the value rows' codes and scales of this lane's first CX_CH chunks,
    // requested before the latent context is summed (one memory round trip
    // for both)
    u32x4 wq[CX_CH];
    float wsc[CX_CH][4];
#pragma unroll
    for (int u = 0; u < CX_CH; ++u) {
        const int ch = min(q + 4 * u, nch - 1);
        wq[u] = live ? gload<u32x4>(kb.q + row * kb.rb + 16 * ch)
                     : u32x4{0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u};
#pragma unroll
        for (int k = 0; k < 4; ++k)
            wsc[u][k] = GRP ? gload<float>(kb.s + row * kb.ng + (32 * ch + 8 * k) / kb.gs) : 1.f;
    }
    // clat = the key chunks' partials of row s, added in chunk order (the
    // first CX_KC requested together); the first row tile stores it
    for (int i = tid; i < S * L; i += 256) {
        const int s = i / L, c = i % L;
        const int nchunk = (pos_base + s + 1 + CL_KEYS - 1) / CL_KEYS;
        const float *pp = cl_part + ((int64_t)s * H + h) * L + c;
        float pk[CX_KC];
#pragma unroll
        for (int k = 0; k < CX_KC; ++k) pk[k] = pp[(int64_t)min(k, nchunk - 1) * nrows * H * L];
        float v = pk[0];
#pragma unroll
        for (int k = 1; k < CX_KC; ++k) v = k < nchunk ? v + pk[k] : v;
        for (int k = CX_KC; k < nchunk; ++k) v += pp[(int64_t)k * nrows * H * L];
        cl[i] = v;
        if (blockIdx.y == 0)
            clat[((int64_t)s * H + h) * L + c] = v;
    }
    __syncthreads();
    float part[S];
#pragma unroll
    for (int s = 0; s < S; ++s) part[s] = 0.f;
    for (int ch = q, u = 0; ch < nch; ch += 4, ++u) {
        u32x4 w4 = wq[0];
        float scu[4] = {wsc[0][0], wsc[0][1], wsc[0][2], wsc[0][3]};
#pragma unroll
        for (int j = 1; j < CX_CH; ++j)
            if (u == j) {
                w4 = wq[j];
#pragma unroll
                for (int k = 0; k < 4; ++k) scu[k] = wsc[j][k];
            }
        if (u >= CX_CH) {
            w4 = live ? gload<u32x4>(kb.q + row * kb.rb + 16 * ch)
                      : u32x4{0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u};
#pragma unroll
            for (int k = 0; k < 4; ++k)
                scu[k] = GRP ? gload<float>(kb.s + row * kb.ng + (32 * ch + 8 * k) / kb.gs) : 1.f;
        }
        const uint32_t wds[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int c = 32 * ch + 8 * k;
            const float sc = scu[k];
            float f[8];
            decode_nib_word(wds[k], f);
#pragma unroll
            for (int s = 0; s < S; ++s) {
                const f32x4 a = *reinterpret_cast<const f32x4 *>(cl + s * L + c);
                const f32x4 b = *reinterpret_cast<const f32x4 *>(cl + s * L + c + 4);
                float d = f[0] * a.x;
                d = fmaf(f[1], a.y, d); d = fmaf(f[2], a.z, d); d = fmaf(f[3], a.w, d);
                d = fmaf(f[4], b.x, d); d = fmaf(f[5], b.y, d); d = fmaf(f[6], b.z, d);
                d = fmaf(f[7], b.w, d);
                part[s] = fmaf(sc, d, part[s]);
            }
        }
    }
    const float rs = GRP ? 0.0625f : gload<float>(kb.s + row) * 0.0625f;
#pragma unroll
    for (int s = 0; s < S; ++s) {
        float t = part[s] + __shfl_xor(part[s], 1, 4);
        t += __shfl_xor(t, 2, 4);
        if (q == 0 && live)
            ctx[(int64_t)s * H * dv + (int64_t)h * dv + v] = t * rs;
    }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------

// prefill rows (S > MLA_CHUNK): whether the value absorption of all rows
// runs as per-head products on the matrix cores (kv_b with a packed int4 copy)
static bool mla_ctx_on_gemm(const coli_mla_layer &m, int S) {
    return S > MLA_CHUNK &&
           dgemm_heads_takes(m.kv_b, m.d_nope, m.d_nope + m.d_v, m.d_v, m.H, S);
}

// prefill rows: the largest input preparation of the four projections and
// (when it runs there) the value absorption on the split-K GEMM, else 0
size_t mla_proj_ws(const coli_mla_layer &m, int S) {
    if (S <= MLA_CHUNK)
        return 0;
    size_t b = 0;
    for (const coli_qtensor *W : {m.q_a, m.kv_a, m.q_b, m.o_proj})
        b = std::max(b, dgemm_ws_bytes(W, S));
    if (mla_ctx_on_gemm(m, S))
        b = std::max(b, dgemm_heads_ws_bytes(m.kv_b, S, m.H));
    return b;
}

MlaLayout mla_layout(int S, int H, int dn, int dr, int dv, int qr, int L, int Tcap, size_t proj_ws) {
    MlaLayout l;
    size_t o = 0;
    auto take = [&](size_t floats) {
        const size_t at = o;
        o += (floats * sizeof(float) + 255) / 256 * 256;
        return at;
    };
    l.off[MLA_CQ_RAW] = take((size_t)S * qr);
    l.off[MLA_CKV_RAW] = take((size_t)S * (L + dr));
    l.off[MLA_CQ] = take((size_t)S * qr);
    l.off[MLA_Q] = take((size_t)S * H * (dn + dr));
    l.off[MLA_QABS] = take((size_t)S * H * L);
    l.off[MLA_QPE] = take((size_t)S * H * dr);
    l.off[MLA_SCORES] = take((size_t)S * H * Tcap);
    l.off[MLA_P] = take((size_t)S * H * Tcap);
    l.off[MLA_CLAT] = take((size_t)S * H * L);
    l.off[MLA_CTX] = take((size_t)S * H * dv);
    // the core runs on groups of at most MLA_GROUP rows: partial sums for one
    const int Sc = S < MLA_GROUP ? S : MLA_GROUP;
    l.qabs_part = take((size_t)MLA_QA_SPLIT * Sc * H * L);
    l.sc_part = take((size_t)MLA_SC_SPLIT * Sc * H * Tcap);
    l.cl_part = take((size_t)((Tcap + CL_KEYS - 1) / CL_KEYS) * Sc * H * L);
    l.xprep = take((proj_ws + sizeof(float) - 1) / sizeof(float));
    l.xprep_bytes = proj_ws;
    l.total = o;
    return l;
}

static int gemv_pair(const coli_qtensor *A, const coli_qtensor *B, const float *x, float *ya,
                     float *yb, int S, hipStream_t st) {
    if (decode_kernel_mode() == 0) {
        const coli_qtensor *W[2] = {A, B};
        const float *xs[2] = {x, x};
        float *ys[2] = {ya, yb};
        const int r = launch_mgemv_group(2, W, xs, ys, S, st);
        if (r == 1)
            return COLI_OK;
        if (r < 0)
            return COLI_HIP_ERROR;
    }
    int rc = launch_gemv(A, x, ya, S, st);
    if (rc != COLI_OK)
        return rc;
    return launch_gemv(B, x, yb, S, st);
}

// chunked launch of the key absorption or the value absorption: rows
// rbase + 4 z .. of a group of nrows, MLA_CHUNK rows per workgroup along z
template <int SC>
static void qabs_launch(bool grp, unsigned nz, int rbase, int nrows, const MlaKvb &kb, int H,
                        int dn, int dr, int dv, int L, const float *q, int pos_base, double theta,
                        float *part, float *qpe, const float *ckv, const float *kn, double eps,
                        float *Lc, float *Rc, hipStream_t st) {
    // (one more column of workgroups for the key side of the new rows)
    static_assert(MLA_QA_SPLIT >= MLA_CHUNK, "a workgroup per new row of a chunk");
    const dim3 grid((unsigned)H + 1, (unsigned)MLA_QA_SPLIT, nz);
    if (grp)
        hipLaunchKernelGGL((k_mla_qabs<SC, true>), grid, dim3(QA_NW * 64), 0, st, kb, H, dn, dr, dv,
                           L, q, pos_base, theta, part, qpe, ckv, kn, eps, Lc, Rc, nrows, rbase);
    else
        hipLaunchKernelGGL((k_mla_qabs<SC, false>), grid, dim3(QA_NW * 64), 0, st, kb, H, dn, dr,
                           dv, L, q, pos_base, theta, part, qpe, ckv, kn, eps, Lc, Rc, nrows, rbase);
}

template <int SC>
static void ctx_launch(bool grp, unsigned nz, int rbase, int nrows, const MlaKvb &kb, int H,
                       int dn, int dv, int L, int pos_base, const float *cl_part, float *clat,
                       float *ctx, hipStream_t st) {
    const dim3 grid((unsigned)H, (unsigned)((dv + CX_ROWS - 1) / CX_ROWS), nz);
    const size_t lds = (size_t)SC * L * sizeof(float);
    if (grp)
        hipLaunchKernelGGL((k_mla_ctx<SC, true>), grid, dim3(256), lds, st, kb, H, dn, dv, L,
                           pos_base, cl_part, clat, ctx, nrows, rbase);
    else
        hipLaunchKernelGGL((k_mla_ctx<SC, false>), grid, dim3(256), lds, st, kb, H, dn, dv, L,
                           pos_base, cl_part, clat, ctx, nrows, rbase);
}

// kv_b as the absorption kernels read it
static MlaKvb mla_kvb(const coli_mla_layer &m) {
    const bool grp = m.kv_b->fmt == COLI_FMT_I4_GRP;
    MlaKvb kb;
    kb.q = (const uint8_t *)m.kv_b->q;
    kb.s = m.kv_b->s;
    kb.rb = m.kv_b->row_bytes;
    kb.ng = m.kv_b->ng;
    kb.gs = grp ? m.kv_b->gs : 1;
    return kb;
}

// The core for a group of G rows r0 .. r0 + G - 1 (G <= MLA_GROUP) at
// positions pos_base + r0 ..: stage pointers start at row r0, the partial
// sums are the group's own.  The key and value absorptions run MLA_CHUNK rows
// per workgroup (whole chunks in one launch, a last partial chunk in a second);
// scores and softmax take the G rows directly.
static int launch_core(const MlaArgs &a, const MlaLayout &l, char *ws, hipStream_t st, int r0,
                       int G, bool ctx_later) {
    const coli_mla_layer &m = *a.layer;
    const int H = m.H, dn = m.d_nope, dr = m.d_rope, dv = m.d_v;
    const int L = m.kv_b->I;
    const bool grp = m.kv_b->fmt == COLI_FMT_I4_GRP;
    const MlaKvb kb = mla_kvb(m);
    const int64_t R = r0;
    const int pos_base = a.pos_base + r0;
    const float *q = (const float *)(ws + l.off[MLA_Q]) + R * H * (dn + dr);
    float *qabs = (float *)(ws + l.off[MLA_QABS]) + R * H * L;
    float *qpe = (float *)(ws + l.off[MLA_QPE]) + R * H * dr;
    float *sc = (float *)(ws + l.off[MLA_SCORES]) + R * H * a.T_cap;
    float *p = (float *)(ws + l.off[MLA_P]) + R * H * a.T_cap;
    float *clat = (float *)(ws + l.off[MLA_CLAT]) + R * H * L;
    float *ctx = (float *)(ws + l.off[MLA_CTX]) + R * H * dv;
    const float *ckv = (const float *)(ws + l.off[MLA_CKV_RAW]) + R * (L + dr);
    float *part = (float *)(ws + l.qabs_part);
    float *sc_part = (float *)(ws + l.sc_part);
    float *cl_part = (float *)(ws + l.cl_part);
    const double theta = (double)m.rope_theta;
    const double eps = (double)m.eps;
    const unsigned nfull = (unsigned)(G / MLA_CHUNK);
    const int rem = G % MLA_CHUNK, rrem = (int)nfull * MLA_CHUNK;
    if (G <= MLA_CHUNK) {  // (a prefill group's qabs, key side and qpe are formed before the groups)
        ProfScope ps("mla_qabs", st);
        {
            if (nfull > 0)
                qabs_launch<MLA_CHUNK>(grp, nfull, 0, G, kb, H, dn, dr, dv, L, q, pos_base, theta, part,
                                       qpe, ckv, m.kv_norm, eps, a.Lc, a.Rc, st);
            switch (rem) {
                case 1: qabs_launch<1>(grp, 1, rrem, G, kb, H, dn, dr, dv, L, q, pos_base, theta, part,
                                       qpe, ckv, m.kv_norm, eps, a.Lc, a.Rc, st); break;
                case 2: qabs_launch<2>(grp, 1, rrem, G, kb, H, dn, dr, dv, L, q, pos_base, theta, part,
                                       qpe, ckv, m.kv_norm, eps, a.Lc, a.Rc, st); break;
                case 3: qabs_launch<3>(grp, 1, rrem, G, kb, H, dn, dr, dv, L, q, pos_base, theta, part,
                                       qpe, ckv, m.kv_norm, eps, a.Lc, a.Rc, st); break;
                default: break;
            }
            const int rc = after_launch("mla_qabs");
            if (rc != COLI_OK) return rc;
        }
    }
    {
        ProfScope ps("mla_scores", st);
        const int nkeys = pos_base + G;
        const dim3 grid((unsigned)((nkeys + SC_KEYS - 1) / SC_KEYS),
                        (unsigned)((H + SC_HEADS - 1) / SC_HEADS), (unsigned)(G * MLA_SC_SPLIT));
        if (G > MLA_CHUNK) {
            const int lvec = (uintptr_t)a.Lc % 16 == 0;
            const int nkt = (nkeys + SX_T - 1) / SX_T;
            const dim3 gridx((unsigned)(nkt < SX_KW ? nkt : SX_KW), (unsigned)H,
                             (unsigned)(MLA_SC_SPLIT * ((G + SX_T - 1) / SX_T)));
            hipLaunchKernelGGL(k_mla_scores_mx, gridx, dim3(256), 0, st, (const float *)qabs,
                               (const float *)qpe, (const float *)a.Lc, (const float *)a.Rc, G, H,
                               L, dr, pos_base, a.T_cap, lvec, sc_part);
        } else {
            const int lvec = (uintptr_t)a.Lc % 16 == 0;
            hipLaunchKernelGGL(k_mla_scores, grid, dim3(256), 0, st, (const float *)part,
                               (const float *)qpe, (const float *)a.Lc, (const float *)a.Rc, G, H,
                               L, dr, pos_base, a.T_cap, lvec, qabs, sc_part);
        }
        const int rc = after_launch("mla_scores");
        if (rc != COLI_OK) return rc;
    }
    {
        ProfScope ps("mla_softmax_clat", st);
        const int nkeys = pos_base + G;
        const float scale = (float)(1.0 / sqrt((double)(dn + dr)));
        const dim3 grid((unsigned)((nkeys + CL_KEYS - 1) / CL_KEYS),
                        (unsigned)((L + CL_COLS - 1) / CL_COLS),
                        (unsigned)(G * ((H + CL_HEADS - 1) / CL_HEADS)));
        if (G > MLA_CHUNK) {
            hipLaunchKernelGGL(k_mla_softmax_rows, dim3((unsigned)G, (unsigned)((H + CL_HEADS - 1) / CL_HEADS)),
                               dim3(256), 0, st, (const float *)sc_part, G, H, pos_base, a.T_cap,
                               scale, sc, p);
            const int lvec = (uintptr_t)a.Lc % 16 == 0;
            const int nct = (L + CX_T - 1) / CX_T;
            const dim3 gridx((unsigned)((nkeys + CX_T - 1) / CX_T), (unsigned)(nct < CX_CW ? nct : CX_CW),
                             (unsigned)(H * ((G + CX_T - 1) / CX_T)));
            hipLaunchKernelGGL(k_mla_clat_mx, gridx, dim3(256), 0, st, (const float *)p,
                               (const float *)a.Lc, G, H, L, pos_base, a.T_cap, lvec, cl_part);
        } else {
            hipLaunchKernelGGL(k_mla_softmax_clat, grid, dim3(256), 0, st, (const float *)sc_part,
                               (const float *)a.Lc, G, H, L, pos_base, a.T_cap, scale, sc, p,
                               cl_part);
        }
        const int rc = after_launch("mla_softmax_clat");
        if (rc != COLI_OK) return rc;
    }
    {
        ProfScope ps("mla_ctx", st);
        if (ctx_later) {  // the group's clat only, written also as the value absorption's
                          // prepared inputs; that GEMM follows for all rows
            const int nkb4 = dgemm_nkb4(m.kv_b);
            const int64_t n8 = (int64_t)G * H * (nkb4 * 128 / 8);
            hipLaunchKernelGGL(k_mla_clat_sum_frag, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, st,
                               (const float *)cl_part, G, H, L, pos_base, CL_KEYS, clat, r0,
                               (uint8_t *)(ws + l.xprep), (int64_t)dgemm_ws_bytes(m.kv_b, a.S), nkb4);
            return after_launch("mla_ctx");
        }
        if (nfull > 0)
            ctx_launch<MLA_CHUNK>(grp, nfull, 0, G, kb, H, dn, dv, L, pos_base, cl_part, clat, ctx,
                                  st);
        switch (rem) {
            case 1: ctx_launch<1>(grp, 1, rrem, G, kb, H, dn, dv, L, pos_base, cl_part, clat, ctx,
                                  st); break;
            case 2: ctx_launch<2>(grp, 1, rrem, G, kb, H, dn, dv, L, pos_base, cl_part, clat, ctx,
                                  st); break;
            case 3: ctx_launch<3>(grp, 1, rrem, G, kb, H, dn, dv, L, pos_base, cl_part, clat, ctx,
                                  st); break;
            default: break;
        }
        const int rc = after_launch("mla_ctx");
        if (rc != COLI_OK) return rc;
    }
    return COLI_OK;
}

// the core over all S rows, at most MLA_GROUP rows per launch set (each group's key
// rows are in the caches before the next group's scores read them)
static int launch_core_rows(const MlaArgs &a, const MlaLayout &l, char *ws, hipStream_t st) {
    const coli_mla_layer &m = *a.layer;
    const bool ctx_later = mla_ctx_on_gemm(m, a.S) && l.xprep_bytes > 0;
    // groups of near-equal size, at most MLA_GROUP rows each, whole chunks
    // of MLA_CHUNK rows but the last
    const int ngroups = (a.S + MLA_GROUP - 1) / MLA_GROUP;
    const int gnom = ((a.S + ngroups - 1) / ngroups + MLA_CHUNK - 1) / MLA_CHUNK * MLA_CHUNK;
    // the rows of the groups of more than MLA_CHUNK rows (all but a last
    // group of at most MLA_CHUNK, which takes the decode kernels): their
    // qabs, key side (cache rows) and qpe in one launch ahead of the groups,
    // since none of it depends on another row's scores
    const int last = a.S - (a.S - 1) / gnom * gnom;  // rows of the last group
    const int big = a.S <= MLA_CHUNK ? 0 : (last <= MLA_CHUNK ? a.S - last : a.S);
    if (big > 0) {
        ProfScope ps("mla_qabs", st);
        const int H = m.H, dn = m.d_nope, dr = m.d_rope, dv = m.d_v, L = m.kv_b->I;
        const MlaKvb kb = mla_kvb(m);
        const float *q = (const float *)(ws + l.off[MLA_Q]);
        float *qabs = (float *)(ws + l.off[MLA_QABS]);
        float *qpe = (float *)(ws + l.off[MLA_QPE]);
        const float *ckv = (const float *)(ws + l.off[MLA_CKV_RAW]);
        const double theta = (double)m.rope_theta, eps = (double)m.eps;
        const unsigned nblk = (unsigned)(((big + QX_T - 1) / QX_T) * H * ((L + QX_T - 1) / QX_T) + 2 * big);
        if (m.kv_b->fmt == COLI_FMT_I4_GRP)
            hipLaunchKernelGGL(k_mla_qabs_mx<true>, dim3(nblk), dim3(256), 0, st, kb, big, H, dn, dr, dv,
                               L, q, a.pos_base, theta, qabs, qpe, ckv, m.kv_norm, eps, a.Lc, a.Rc);
        else
            hipLaunchKernelGGL(k_mla_qabs_mx<false>, dim3(nblk), dim3(256), 0, st, kb, big, H, dn, dr, dv,
                               L, q, a.pos_base, theta, qabs, qpe, ckv, m.kv_norm, eps, a.Lc, a.Rc);
        const int rc = after_launch("mla_qabs");
        if (rc != COLI_OK) return rc;
    }
    for (int r0 = 0; r0 < a.S; r0 += gnom) {
        const int G = a.S - r0 < gnom ? a.S - r0 : gnom;
        const int rc = launch_core(a, l, ws, st, r0, G, ctx_later);
        if (rc != COLI_OK) return rc;
    }
    if (!ctx_later)
        return COLI_OK;
    // value absorption of all rows: head h's value rows of kv_b times its
    // latent context, on the bf16 matrix cores (the prefill precision)
    const int H = m.H, dn = m.d_nope, dv = m.d_v, L = m.kv_b->I;
    const int r = launch_dgemm_heads(m.kv_b, dn, dn + dv, dv, H, (const float *)(ws + l.off[MLA_CLAT]),
                                     (int64_t)H * L, L, (float *)(ws + l.off[MLA_CTX]),
                                     (int64_t)H * dv, dv, a.S, ws + l.xprep, l.xprep_bytes, st,
                                     true);  // inputs prepared by the groups' clat sums
    return r > 0 ? COLI_OK : COLI_HIP_ERROR;  // (shapes checked by mla_ctx_on_gemm)
}

// one projection of S > MLA_CHUNK rows: the prefill GEMM (bf16 matrix cores),
// the split-K kernel with the inputs prepared in the workspace when it takes W
static int proj_rows(const coli_qtensor *W, const float *x, float *y, int S, hipStream_t st,
                     char *ws, const MlaLayout &l) {
    if (l.xprep_bytes > 0) {
        const int r = launch_dgemm(W, x, y, S, ws + l.xprep, l.xprep_bytes, st);
        if (r != 0)
            return r > 0 ? COLI_OK : COLI_HIP_ERROR;
    }
    return launch_gemm(W, x, y, S, nullptr, 0, st);
}

// q_a and kv_a of S > MLA_CHUNK rows (same inputs): one launch of the
// split-K kernel for both when it takes them, else one projection each
static int proj_rows_pair(const coli_qtensor *W1, const coli_qtensor *W2, const float *x, float *y1,
                          float *y2, int S, hipStream_t st, char *ws, const MlaLayout &l) {
    if (l.xprep_bytes > 0) {
        const int r = launch_dgemm_pair(W1, W2, x, y1, y2, S, ws + l.xprep, l.xprep_bytes, st);
        if (r != 0)
            return r > 0 ? COLI_OK : COLI_HIP_ERROR;
    }
    const int rc = proj_rows(W1, x, y1, S, st, ws, l);
    return rc != COLI_OK ? rc : proj_rows(W2, x, y2, S, st, ws, l);
}

int launch_mla_decode(const MlaArgs &a) {
    const coli_mla_layer &m = *a.layer;
    const int S = a.S;
    const int H = m.H, dn = m.d_nope, dr = m.d_rope, dv = m.d_v;
    const int qr = m.q_a->O, L = m.kv_b->I;
    const MlaLayout l = mla_layout(S, H, dn, dr, dv, qr, L, a.T_cap, mla_proj_ws(m, S));
    char *ws = (char *)a.ws;
    const hipStream_t st = a.st;
    float *cq_raw = (float *)(ws + l.off[MLA_CQ_RAW]);
    float *ckv = (float *)(ws + l.off[MLA_CKV_RAW]);
    float *cq = (float *)(ws + l.off[MLA_CQ]);
    float *q = (float *)(ws + l.off[MLA_Q]);
    float *ctx = (float *)(ws + l.off[MLA_CTX]);
    int rc;
    if (S > MLA_CHUNK) {
        // prefill rows: the projections on the prefill GEMM, the norms and
        // the layer's residual add launches of their own, the core in
        // chunks of rows
        const float *xin = a.x;
        if (a.in_norm) {
            rc = launch_rmsnorm(a.x, S, m.q_a->I, a.in_norm_w, a.in_eps, a.xn, st);
            if (rc != COLI_OK) return rc;
            xin = a.xn;
        }
        rc = proj_rows_pair(m.q_a, m.kv_a, xin, cq_raw, ckv, S, st, ws, l);
        if (rc != COLI_OK) return rc;
        {
            ProfScope ps("mla_qnorm", st);
            hipLaunchKernelGGL(k_mla_qnorm, dim3((unsigned)S), dim3(256), 0, st,
                               (const float *)cq_raw, qr, m.q_norm, (double)m.eps, cq);
            rc = after_launch("mla_qnorm");
            if (rc != COLI_OK) return rc;
        }
        rc = proj_rows(m.q_b, cq, q, S, st, ws, l);
        if (rc != COLI_OK) return rc;
        rc = launch_core_rows(a, l, ws, st);
        if (rc != COLI_OK) return rc;
        rc = proj_rows(m.o_proj, ctx, a.out, S, st, ws, l);
        if (rc != COLI_OK || a.hsum == nullptr) return rc;
        return launch_residual_add(a.resid, a.out, a.hsum, (int64_t)S * m.o_proj->O, st);
    }
    // q_a and kv_a (the layer's input norm folded in when the matrix-core
    // kernel takes it, else a norm launch first)
    bool done = false;
    const float *xin = a.x;
    if (a.in_norm) {
        if (decode_kernel_mode() == 0) {
            const coli_qtensor *W[2] = {m.q_a, m.kv_a};
            const float *xs[2] = {a.x, a.x};
            float *ys[2] = {cq_raw, ckv};
            const InNorm nr{a.in_norm_w, a.in_eps, a.xn};
            const int r = launch_mgemv_group(2, W, xs, ys, S, st, &nr);
            if (r < 0) return COLI_HIP_ERROR;
            done = r == 1;
        }
        if (!done) {
            rc = launch_rmsnorm(a.x, S, m.q_a->I, a.in_norm_w, a.in_eps, a.xn, st);
            if (rc != COLI_OK) return rc;
            xin = a.xn;
        }
    }
    if (!done) {
        rc = gemv_pair(m.q_a, m.kv_a, xin, cq_raw, ckv, S, st);
        if (rc != COLI_OK) return rc;
    }
    // q_b on the query latent's norm (folded in the same way); the key
    // side's norm and rotation run beside the key absorption
    done = false;
    if (decode_kernel_mode() == 0) {
        const InNorm nr{m.q_norm, (double)m.eps, cq};
        const int r = launch_mgemv(m.q_b, cq_raw, q, S, st, nullptr, nullptr, &nr);
        if (r < 0) return COLI_HIP_ERROR;
        done = r == 1;
    }
    if (!done) {
        {
            ProfScope ps("mla_qnorm", st);
            hipLaunchKernelGGL(k_mla_qnorm, dim3((unsigned)S), dim3(256), 0, st,
                               (const float *)cq_raw, qr, m.q_norm, (double)m.eps, cq);
            rc = after_launch("mla_qnorm");
            if (rc != COLI_OK) return rc;
        }
        rc = launch_gemv(m.q_b, cq, q, S, st);
        if (rc != COLI_OK) return rc;
    }
    rc = launch_core_rows(a, l, ws, st);
    if (rc != COLI_OK) return rc;
    return launch_gemv(m.o_proj, ctx, a.out, S, st, a.resid, a.hsum);
}

}  // namespace coli
