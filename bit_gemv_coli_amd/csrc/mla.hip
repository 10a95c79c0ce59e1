// mla.hip -- decode attention of one MLA layer for S <= 4 query rows
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
// one before wrote; nothing waits on the host.
//
// Kernels (all HBM- or latency-bound at decode sizes; the weights they read,
// kv_b's key and value rows, are 64 x 448 x 512 int4 = 8.3 MB for the
// pages' model):
//   k_mla_norm_rope   one workgroup per (row, latent): f64 sum of squares,
//                     f32 rounding of x * inv * w in f64; the kv workgroup
//                     also rotates the rotary key (cos / sin in f64) and
//                     writes both cache rows
//   k_mla_qabs        one workgroup per (head, 512-column slab): each lane
//                     owns 8 columns (one word of codes per kv_b row), the
//                     8 wavefronts take every 8th key row, then sum in LDS in
//                     wavefront order; workgroup 0 of each head rotates the
//                     query's rotary part
//   k_mla_scores      one workgroup per (64 keys, head, row): qabs and qpe in
//                     LDS, a wavefront per 16 keys, lanes across the latent
//                     (coalesced cache rows), wavefront sums
//   k_mla_softmax_clat one workgroup per (row, head, 256 latent columns): max
//                     and sum by fixed-order LDS trees, p by exp and one
//                     division, then clat with the probabilities staged in LDS
//   k_mla_ctx         one workgroup per (head, 16 value rows): lanes own 8
//                     latent columns, wavefront sums
#include "common.h"
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
__global__ __launch_bounds__(256) void k_mla_norm_rope(const float *__restrict__ cq_raw, int qr,
                                                       const float *__restrict__ qn,
                                                       const float *__restrict__ ckv, int L, int dr,
                                                       const float *__restrict__ kn, double eps,
                                                       double theta, int pos_base,
                                                       float *__restrict__ cq, float *__restrict__ Lc,
                                                       float *__restrict__ Rc) {
    __shared__ double part[4];
    const int s = blockIdx.x, t = threadIdx.x, lane = t & 63, wv = t >> 6;
    const bool kv = blockIdx.y == 1;
    const int pos = pos_base + s;
    const float *xr = kv ? ckv + (int64_t)s * (L + dr) : cq_raw + (int64_t)s * qr;
    const int n = kv ? L : qr;
    const float *w = kv ? kn : qn;
    float *yr = kv ? Lc + (int64_t)pos * L : cq + (int64_t)s * qr;
    double ss = 0.0;
    for (int d = t; d < n; d += 256) ss = fma((double)xr[d], (double)xr[d], ss);
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) ss += mla_shfl_xor(ss, m);
    if (lane == 0)
        part[wv] = ss;
    __syncthreads();
    const double tot = ((part[0] + part[1]) + part[2]) + part[3];
    const double inv = 1.0 / sqrt(tot / (double)n + eps);
    for (int d = t; d < n; d += 256)
        yr[d] = (float)((double)xr[d] * inv * (w ? (double)w[d] : 1.0));
    if (kv)
        for (int i = t; i < dr / 2; i += 256)
            rope_pair(xr[L + 2 * i], xr[L + 2 * i + 1], i, dr, pos, theta,
                      Rc + (int64_t)pos * dr + 2 * i, Rc + (int64_t)pos * dr + 2 * i + 1);
}

// ---- key absorption and the query's rotary part ----------------------------
constexpr int QA_NW = 8;      // wavefronts per workgroup
constexpr int QA_COLS = 512;  // latent columns per workgroup (8 per lane)

template <int S, bool GRP>
__global__ __launch_bounds__(QA_NW * 64) void k_mla_qabs(MlaKvb kb, int H, int dn, int dr, int dv,
                                                         int L, const float *__restrict__ q,
                                                         int pos_base, double theta,
                                                         float *__restrict__ qabs,
                                                         float *__restrict__ qpe) {
    __shared__ float red[QA_NW][S][QA_COLS];
    const int h = blockIdx.x, col0 = blockIdx.y * QA_COLS;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nq = H * (dn + dr);
    const int c0 = col0 + 8 * lane;  // this lane's 8 columns
    const bool live = c0 < L;
    float acc[S][8];
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[s][k] = 0.f;
    for (int j = wave; j < dn; j += QA_NW) {
        const int64_t row = (int64_t)h * (dn + dv) + j;
        const float sc = GRP ? (live ? gload<float>(kb.s + row * kb.ng + c0 / kb.gs) : 0.f)
                             : gload<float>(kb.s + row);
        const uint32_t wd = live ? gload<uint32_t>(kb.q + row * kb.rb + c0 / 2) : 0x88888888u;
        float f[8];
        decode_nib_word(wd, f);  // 16 (nibble - 8)
#pragma unroll
        for (int s = 0; s < S; ++s) {
            const float qs = gload<float>(q + (int64_t)s * nq + (int64_t)h * (dn + dr) + j) * sc *
                             0.0625f;
#pragma unroll
            for (int k = 0; k < 8; ++k) acc[s][k] = fmaf(qs, f[k], acc[s][k]);
        }
    }
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
        for (int k = 0; k < 8; ++k) red[wave][s][8 * lane + k] = acc[s][k];
    __syncthreads();
    for (int idx = tid; idx < S * QA_COLS; idx += QA_NW * 64) {
        const int s = idx / QA_COLS, c = idx % QA_COLS;
        if (col0 + c >= L)
            continue;
        float v = red[0][s][c];
#pragma unroll
        for (int w = 1; w < QA_NW; ++w) v += red[w][s][c];
        qabs[((int64_t)s * H + h) * L + col0 + c] = v;
    }
    if (blockIdx.y == 0)
        for (int idx = tid; idx < S * (dr / 2); idx += QA_NW * 64) {
            const int s = idx / (dr / 2), i = idx % (dr / 2);
            const float *qr = q + (int64_t)s * nq + (int64_t)h * (dn + dr) + dn;
            float *o = qpe + ((int64_t)s * H + h) * dr;
            rope_pair(qr[2 * i], qr[2 * i + 1], i, dr, pos_base + s, theta, o + 2 * i, o + 2 * i + 1);
        }
}

// ---- scores ----------------------------------------------------------------
constexpr int SC_KEYS = 64;  // keys per workgroup (16 per wavefront)

__global__ __launch_bounds__(256) void k_mla_scores(const float *__restrict__ qabs,
                                                    const float *__restrict__ qpe,
                                                    const float *__restrict__ Lc,
                                                    const float *__restrict__ Rc, int H, int L,
                                                    int dr, int pos_base, int Tcap, float scale,
                                                    float *__restrict__ scores) {
    extern __shared__ float sq[];  // [L] qabs then [dr] qpe of this (row, head)
    const int t0 = blockIdx.x * SC_KEYS, h = blockIdx.y, s = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int last = pos_base + s;  // keys 0 .. last
    if (t0 > last)
        return;
    const float *qa = qabs + ((int64_t)s * H + h) * L;
    const float *qp = qpe + ((int64_t)s * H + h) * dr;
    for (int c = tid; c < L; c += 256) sq[c] = qa[c];
    for (int r = tid; r < dr; r += 256) sq[L + r] = qp[r];
    __syncthreads();
    float *zrow = scores + ((int64_t)s * H + h) * Tcap;
    const int tb = t0 + wave * (SC_KEYS / 4);
    for (int k = 0; k < SC_KEYS / 4; ++k) {
        const int t = tb + k;
        if (t > last)
            break;
        const float *lr = Lc + (int64_t)t * L;
        const float *rr = Rc + (int64_t)t * dr;
        float a = 0.f;
        for (int c = lane; c < L; c += 64) a = fmaf(sq[c], lr[c], a);
        for (int r = lane; r < dr; r += 64) a = fmaf(sq[L + r], rr[r], a);
        a = wave_sum(a);
        if (lane == 0)
            zrow[t] = a * scale;
    }
}

// ---- softmax and the latent context ----------------------------------------
__device__ __forceinline__ float block_reduce_256(float v, float *buf, bool is_max) {
    // fixed-order tree over the 256 threads (deterministic)
    const int tid = threadIdx.x;
    buf[tid] = v;
    __syncthreads();
    for (int off = 128; off >= 1; off >>= 1) {
        if (tid < off)
            buf[tid] = is_max ? fmaxf(buf[tid], buf[tid + off]) : buf[tid] + buf[tid + off];
        __syncthreads();
    }
    const float r = buf[0];
    __syncthreads();
    return r;
}

__global__ __launch_bounds__(256) void k_mla_softmax_clat(const float *__restrict__ scores,
                                                          const float *__restrict__ Lc, int H, int L,
                                                          int pos_base, int Tcap,
                                                          float *__restrict__ p,
                                                          float *__restrict__ clat) {
    __shared__ float buf[256];
    __shared__ float pl[256];
    const int sh = blockIdx.x, s = sh / H;
    const int tid = threadIdx.x;
    const int n = pos_base + s + 1;
    const float *z = scores + (int64_t)sh * Tcap;
    float m = -__builtin_inff();
    for (int t = tid; t < n; t += 256) m = fmaxf(m, z[t]);
    m = block_reduce_256(m, buf, true);
    float e = 0.f;
    for (int t = tid; t < n; t += 256) e += expf(z[t] - m);
    const float sum = block_reduce_256(e, buf, false);
    const int c = blockIdx.y * 256 + tid;
    float acc = 0.f;
    for (int tb = 0; tb < n; tb += 256) {
        const int t = tb + tid;
        const float pv = t < n ? expf(z[t] - m) / sum : 0.f;
        pl[tid] = pv;
        if (blockIdx.y == 0 && t < n)
            p[(int64_t)sh * Tcap + t] = pv;
        __syncthreads();
        if (c < L) {
            const int nk = min(256, n - tb);
            for (int k = 0; k < nk; ++k) acc = fmaf(pl[k], Lc[(int64_t)(tb + k) * L + c], acc);
        }
        __syncthreads();
    }
    if (c < L)
        clat[(int64_t)sh * L + c] = acc;
}

// ---- value absorption --------------------------------------------------------
constexpr int CX_ROWS = 16;  // value rows per workgroup (4 per wavefront)

template <int S, bool GRP>
__global__ __launch_bounds__(256) void k_mla_ctx(MlaKvb kb, int H, int dn, int dv, int L,
                                                 const float *__restrict__ clat,
                                                 float *__restrict__ ctx) {
    const int h = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nwd = L / 8;  // words of codes per row
    for (int r = 0; r < CX_ROWS / 4; ++r) {
        const int v = blockIdx.y * CX_ROWS + wave * (CX_ROWS / 4) + r;
        if (v >= dv)
            break;
        const int64_t row = (int64_t)h * (dn + dv) + dn + v;
        float part[S];
#pragma unroll
        for (int s = 0; s < S; ++s) part[s] = 0.f;
        for (int wd = lane; wd < nwd; wd += 64) {
            const int c0 = 8 * wd;
            const float sc = GRP ? gload<float>(kb.s + row * kb.ng + c0 / kb.gs) : 1.f;
            float f[8];
            decode_nib_word(gload<uint32_t>(kb.q + row * kb.rb + c0 / 2), f);
#pragma unroll
            for (int s = 0; s < S; ++s) {
                const float *cl = clat + ((int64_t)s * H + h) * L + c0;
                const f32x4 a = gload<f32x4>(cl), b = gload<f32x4>(cl + 4);
                float d = f[0] * a.x;
                d = fmaf(f[1], a.y, d); d = fmaf(f[2], a.z, d); d = fmaf(f[3], a.w, d);
                d = fmaf(f[4], b.x, d); d = fmaf(f[5], b.y, d); d = fmaf(f[6], b.z, d);
                d = fmaf(f[7], b.w, d);
                part[s] = fmaf(sc, d, part[s]);
            }
        }
        const float rs = GRP ? 0.0625f : gload<float>(kb.s + row) * 0.0625f;
#pragma unroll
        for (int s = 0; s < S; ++s) {
            const float tot = wave_sum(part[s]);
            if (lane == 0)
                ctx[(int64_t)s * H * dv + (int64_t)h * dv + v] = tot * rs;
        }
    }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------

MlaLayout mla_layout(int S, int H, int dn, int dr, int dv, int qr, int L, int Tcap) {
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

template <int S>
static int launch_core(const MlaArgs &a, const MlaLayout &l, char *ws, hipStream_t st) {
    const coli_mla_layer &m = *a.layer;
    const int H = m.H, dn = m.d_nope, dr = m.d_rope, dv = m.d_v;
    const int L = m.kv_b->I;
    const bool grp = m.kv_b->fmt == COLI_FMT_I4_GRP;
    MlaKvb kb;
    kb.q = (const uint8_t *)m.kv_b->q;
    kb.s = m.kv_b->s;
    kb.rb = m.kv_b->row_bytes;
    kb.ng = m.kv_b->ng;
    kb.gs = grp ? m.kv_b->gs : 1;
    const float *q = (const float *)(ws + l.off[MLA_Q]);
    float *qabs = (float *)(ws + l.off[MLA_QABS]);
    float *qpe = (float *)(ws + l.off[MLA_QPE]);
    float *sc = (float *)(ws + l.off[MLA_SCORES]);
    float *p = (float *)(ws + l.off[MLA_P]);
    float *clat = (float *)(ws + l.off[MLA_CLAT]);
    float *ctx = (float *)(ws + l.off[MLA_CTX]);
    const double theta = (double)m.rope_theta;
    {
        ProfScope ps("mla_qabs", st);
        const dim3 grid((unsigned)H, (unsigned)((L + QA_COLS - 1) / QA_COLS));
        if (grp)
            hipLaunchKernelGGL((k_mla_qabs<S, true>), grid, dim3(QA_NW * 64), 0, st, kb, H, dn, dr,
                               dv, L, q, a.pos_base, theta, qabs, qpe);
        else
            hipLaunchKernelGGL((k_mla_qabs<S, false>), grid, dim3(QA_NW * 64), 0, st, kb, H, dn,
                               dr, dv, L, q, a.pos_base, theta, qabs, qpe);
        const int rc = after_launch("mla_qabs");
        if (rc != COLI_OK) return rc;
    }
    {
        ProfScope ps("mla_scores", st);
        const int nkeys = a.pos_base + S;
        const dim3 grid((unsigned)((nkeys + SC_KEYS - 1) / SC_KEYS), (unsigned)H, (unsigned)S);
        const float scale = (float)(1.0 / sqrt((double)(dn + dr)));
        hipLaunchKernelGGL(k_mla_scores, grid, dim3(256), (size_t)(L + dr) * sizeof(float), st,
                           (const float *)qabs, (const float *)qpe, (const float *)a.Lc,
                           (const float *)a.Rc, H, L, dr, a.pos_base, a.T_cap, scale, sc);
        const int rc = after_launch("mla_scores");
        if (rc != COLI_OK) return rc;
    }
    {
        ProfScope ps("mla_softmax_clat", st);
        const dim3 grid((unsigned)(S * H), (unsigned)((L + 255) / 256));
        hipLaunchKernelGGL(k_mla_softmax_clat, grid, dim3(256), 0, st, (const float *)sc,
                           (const float *)a.Lc, H, L, a.pos_base, a.T_cap, p, clat);
        const int rc = after_launch("mla_softmax_clat");
        if (rc != COLI_OK) return rc;
    }
    {
        ProfScope ps("mla_ctx", st);
        const dim3 grid((unsigned)H, (unsigned)((dv + CX_ROWS - 1) / CX_ROWS));
        if (grp)
            hipLaunchKernelGGL((k_mla_ctx<S, true>), grid, dim3(256), 0, st, kb, H, dn, dv, L,
                               (const float *)clat, ctx);
        else
            hipLaunchKernelGGL((k_mla_ctx<S, false>), grid, dim3(256), 0, st, kb, H, dn, dv, L,
                               (const float *)clat, ctx);
        const int rc = after_launch("mla_ctx");
        if (rc != COLI_OK) return rc;
    }
    return COLI_OK;
}

int launch_mla_decode(const MlaArgs &a) {
    const coli_mla_layer &m = *a.layer;
    const int S = a.S;
    const int H = m.H, dn = m.d_nope, dr = m.d_rope, dv = m.d_v;
    const int qr = m.q_a->O, L = m.kv_b->I;
    const MlaLayout l = mla_layout(S, H, dn, dr, dv, qr, L, a.T_cap);
    char *ws = (char *)a.ws;
    const hipStream_t st = a.st;
    float *cq_raw = (float *)(ws + l.off[MLA_CQ_RAW]);
    float *ckv = (float *)(ws + l.off[MLA_CKV_RAW]);
    float *cq = (float *)(ws + l.off[MLA_CQ]);
    float *q = (float *)(ws + l.off[MLA_Q]);
    float *ctx = (float *)(ws + l.off[MLA_CTX]);
    int rc = gemv_pair(m.q_a, m.kv_a, a.x, cq_raw, ckv, S, st);
    if (rc != COLI_OK) return rc;
    {
        ProfScope ps("mla_norm_rope", st);
        hipLaunchKernelGGL(k_mla_norm_rope, dim3((unsigned)S, 2), dim3(256), 0, st,
                           (const float *)cq_raw, qr, m.q_norm, (const float *)ckv, L, dr,
                           m.kv_norm, (double)m.eps, (double)m.rope_theta, a.pos_base, cq, a.Lc,
                           a.Rc);
        rc = after_launch("mla_norm_rope");
        if (rc != COLI_OK) return rc;
    }
    rc = launch_gemv(m.q_b, cq, q, S, st);
    if (rc != COLI_OK) return rc;
    switch (S) {
        case 1: rc = launch_core<1>(a, l, ws, st); break;
        case 2: rc = launch_core<2>(a, l, ws, st); break;
        case 3: rc = launch_core<3>(a, l, ws, st); break;
        default: rc = launch_core<4>(a, l, ws, st); break;
    }
    if (rc != COLI_OK) return rc;
    return launch_gemv(m.o_proj, ctx, a.out, S, st);
}

}  // namespace coli
