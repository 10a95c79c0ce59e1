// pgemm.hip -- prefill GEMM (S > 4 input rows) for the int4 formats on the
// gfx950 matrix cores: Y[m][n] = sum_k w(n, k) * X[m][k].
//
// What is computed (colibri PR #298, CUDA fmt=4 commit: w = scale(n, k/gs) *
// (q - 8), the group scale applied inline; colibri-strix "route large
// row-batch matmul_qt GEMMs to the GPU": large row batches take a GEMM path).
//
// Precision (the bf16 envelope): every weight is dequantized once per
// workgroup to bf16(s * (q - 8)) -- one rounding of the exact product -- and
// every input to bf16(x); products accumulate in fp32 on
// v_mfma_f32_32x32x16_bf16.  |error| <= (2 * 2^-9 + 2^-18) * sum |w||x| plus
// the fp32 accumulation, inside 4e-3 * sum |w||x|.
//
// Shape of one workgroup (8 wavefronts, 512 threads, output tile BM x 128:
// BM input rows x 128 weight rows -- for gate/up 64 gate rows then the same
// 64 up rows), K advancing 64 inputs per step through a double-buffered LDS
// tile (rows padded to 72 elements), one barrier per step:
//   * 4 producer wavefronts request each step's codes (32 per thread), group
//     scales and inputs four steps ahead, turn codes into bf16(s * v) and
//     inputs into bf16, and store the next tile;
//   * 4 consumer wavefronts (2 x 2, each BM/2 rows x 64 weight rows) run
//     v_mfma_f32_32x32x16_bf16 on the current tile.
// Each SIMD thus holds one producer and one consumer wavefront, so the
// conversion work on the vector ALUs runs beside the matrix cores instead of
// between their instructions.
#include <string.h>

#include <algorithm>

#include "common.h"

namespace coli {

typedef __bf16 pg_bf16;
typedef __bf16 pg_bf16x8 __attribute__((ext_vector_type(8)));
typedef float pg_f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t pg_u32x2 __attribute__((ext_vector_type(2)));

constexpr int PG_BK = 64;         // inputs per K step
constexpr int PG_LD = PG_BK + 8;  // LDS row stride (bf16 elements)
constexpr int PG_BN = 128;        // weight rows per tile (all matrices)
constexpr int PG_PD = 4;          // steps requested ahead by the producers (even)

enum { PG_Y = 0, PG_SILU = 1, PG_PART = 2 };

struct PgArgs {
    const void *x;  // f32 [M][K] (AF32) or bf16 rows
    int64_t ldx;
    int M, K;
    const uint8_t *q[2];
    const float *s[2];
    int64_t rb;     // code bytes per weight row
    int ng, gshift, N;  // groups per row (fmt 4), log2 of the group size, weight rows
    int fmt;
    void *y;
    int64_t ldy;
};

// bf16 of two floats packed low | high (round to nearest even)
__device__ __forceinline__ uint32_t pk_bf16(float lo, float hi) {
    uint32_t r;
    asm("v_cvt_pk_bf16_f32 %0, %1, %2" : "=v"(r) : "v"(lo), "v"(hi));
    return r;
}

template <int BM, int NMAT, int EPI, bool AF32>
__global__ __launch_bounds__(512) void k_pg(PgArgs a) {
    static_assert(BM == 64 || BM == 128, "tile rows");
    constexpr int MBK = BM / 64;       // 32-row blocks per consumer wavefront
    constexpr int NPM = PG_BN / NMAT;  // weight rows per matrix
    __shared__ __attribute__((aligned(16))) pg_bf16 As[2][BM * PG_LD];
    __shared__ __attribute__((aligned(16))) pg_bf16 Bs[2][PG_BN * PG_LD];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    // XCD-aware tile order: workgroup w runs on XCD w % 8 (round-robin
    // dispatch); give each XCD a contiguous run of tiles in M-major order so
    // its L2 holds the input rows of at most two M tiles
    int mt, nt;
    {
        const int ntm = gridDim.x, ntn = gridDim.y, tiles = ntm * ntn;
        const int w = blockIdx.y * ntm + blockIdx.x;
        const int per = (tiles + 7) / 8;
        const int xcd = w % 8, idx = w / 8;
        int t = xcd * per + idx;
        if (tiles % 8 != 0 || t >= tiles)
            t = w;  // uneven split: keep the plain order
        mt = t / ntn;
        nt = t % ntn;
    }
    const int m0 = mt * BM;
    const int n0 = nt * NPM;
    const int K = a.K;
    const int nsteps = (K + PG_BK - 1) / PG_BK;
    // both roles run the same padded number of steps (and barriers); steps
    // past the last one move data nobody reads
    const int npad = (nsteps + PG_PD - 1) / PG_PD * PG_PD;
    // LDS hand-over between the wavefronts (no wait on outstanding loads)
    auto lds_barrier = []() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); };

    if (wave >= 4) {
        // ================= producers: requests, conversion, LDS ==============
        const int pt = tid - 256;
        // weight row rB, 32 codes (16 bytes) at 32 * pB
        const int rB = pt >> 1, pB = pt & 1;
        const int mat = rB / NPM;
        const int nrow = min(n0 + rB % NPM, a.N - 1);
        const uint8_t *qrow = a.q[mat] + (int64_t)nrow * a.rb;
        const float *srow = a.s[mat] + (a.fmt == 4 ? (int64_t)nrow * a.ng : (int64_t)nrow);
        // inputs: request i of a lane covers 16 bytes of input row
        // aro + ARI * i + lane / LPR at input column acol, so that LPR
        // consecutive lanes read one row's step slice (coalesced)
        constexpr int ESZ = AF32 ? 4 : 2;          // bytes per input element
        constexpr int EPL = 16 / ESZ;              // elements per 16-byte request
        constexpr int LPR = PG_BK / EPL;           // lanes per row slice (16 or 8)
        constexpr int ARI = 64 / LPR;              // rows per request (4 or 8)
        constexpr int NA = BM * PG_BK / (256 * EPL);  // requests per thread
        const int pw = pt >> 6, pl = pt & 63;
        const int aro = pw * (BM / 4) + pl / LPR;  // first row of this lane
        const int acol = EPL * (pl % LPR);
        const int64_t xoff0 = (int64_t)min(m0 + aro, a.M - 1) * a.ldx;
        int64_t xstep[NA];  // row offset of request i (rows clamped to M-1)
#pragma unroll
        for (int i = 0; i < NA; ++i) xstep[i] = (int64_t)min(m0 + aro + ARI * i, a.M - 1) * a.ldx;
        (void)xoff0;

        struct Stage {
            u32x4 c;              // 32 codes
            float s;              // their scale (gs >= 32: one group)
            bool cin;             // the codes lie below K
            u32x4 xr[NA];         // inputs (16 bytes per request)
        };
        // requests are unconditional: addresses clamped in range, codes past K
        // replaced by zero weights afterwards (inputs past K then add nothing)
        auto request = [&](Stage &sg, int step) {
            const int k = step * PG_BK;
            const int kc = k + 32 * pB;
            const bool cin = kc < K;
            const int kcc = min(kc, K - 32);
            // (the values are only looked at in deposit: using them here would
            // wait for these very requests)
            sg.c = gload<u32x4>(qrow + kcc / 2);
            sg.s = (a.fmt == 4) ? gload<float>(srow + (kcc >> a.gshift)) : gload<float>(srow);
            sg.cin = cin;
            const int ka = min(k + acol, K - EPL);
#pragma unroll
            for (int i = 0; i < NA; ++i)
                sg.xr[i] = gload<u32x4>((const char *)a.x + (xstep[i] + ka) * ESZ);
        };
        // codes -> bf16(s * (q - 8)) in natural input order, inputs -> bf16
        auto deposit = [&](Stage &sg, int buf) {
            // the stage's values enter the conversion here and not earlier:
            // an early conversion would wait for requests just issued
            asm volatile("" : "+v"(sg.c), "+v"(sg.s));
#pragma unroll
            for (int i = 0; i < NA; ++i) asm volatile("" : "+v"(sg.xr[i]));
            const float s16 = sg.cin ? sg.s * 0.0625f : 0.f;  // the signed bytes below hold 16 * v
            u32x4 *bd = reinterpret_cast<u32x4 *>(&Bs[buf][rB * PG_LD + 32 * pB]);
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                const uint32_t w = sg.c[h] ^ 0x88888888u;   // nibbles v = q - 8
                const uint32_t ev = (w << 4) & 0xF0F0F0F0u;  // inputs 0, 2, 4, 6
                const uint32_t od = w & 0xF0F0F0F0u;         // inputs 1, 3, 5, 7
                bd[h] = u32x4{pk_bf16(sbyte<0>(ev) * s16, sbyte<0>(od) * s16),
                              pk_bf16(sbyte<1>(ev) * s16, sbyte<1>(od) * s16),
                              pk_bf16(sbyte<2>(ev) * s16, sbyte<2>(od) * s16),
                              pk_bf16(sbyte<3>(ev) * s16, sbyte<3>(od) * s16)};
            }
#pragma unroll
            for (int i = 0; i < NA; ++i) {
                pg_bf16 *ad = &As[buf][(aro + ARI * i) * PG_LD + acol];
                if constexpr (AF32) {
                    const f32x4 f = __builtin_bit_cast(f32x4, sg.xr[i]);
                    typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
                    *reinterpret_cast<u32x2v *>(ad) = u32x2v{pk_bf16(f.x, f.y), pk_bf16(f.z, f.w)};
                } else {
                    *reinterpret_cast<u32x4 *>(ad) = sg.xr[i];
                }
            }
        };

        // a ring of PG_PD stages: stage u holds the requests of steps u, u+PG_PD,
        // ...; past the last step a request repeats it (its tile goes to a
        // buffer nobody reads).  The loop is unrolled by PG_PD so every stage
        // index is a constant.
        Stage st[PG_PD];
#pragma unroll
        for (int u = 0; u < PG_PD; ++u) request(st[u], min(u, nsteps - 1));
        deposit(st[0], 0);
        request(st[0], min(PG_PD, nsteps - 1));
        lds_barrier();  // tile 0 ready
        for (int base = 0; base < npad; base += PG_PD) {
#pragma unroll
            for (int u = 0; u < PG_PD; ++u) {
                const int step = base + u;  // the tile the consumers use now
                deposit(st[(u + 1) % PG_PD], (u + 1) & 1);  // tile step+1
                __builtin_amdgcn_sched_barrier(0);
                request(st[(u + 1) % PG_PD], min(step + 1 + PG_PD, nsteps - 1));
                __builtin_amdgcn_sched_barrier(0);
                lds_barrier();
            }
        }
        return;
    }

    // ================= consumers: matrix cores on the LDS tiles ===============
    const int wm = wave >> 1, wn = wave & 1;  // rows [wm*BM/2, +BM/2), weight rows [64*wn, +64)
    pg_f32x16 acc[MBK][2];
#pragma unroll
    for (int i = 0; i < MBK; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    // 32x32x16 operands: lane l holds row l % 32, inputs 8 * (l / 32) .. +8
    const int fr = lane & 31, fk = 8 * (lane >> 5);
    auto compute = [&](int buf) {
#pragma unroll
        for (int ks = 0; ks < PG_BK / 16; ++ks) {
            pg_bf16x8 bfr[2], afr[MBK];
#pragma unroll
            for (int j = 0; j < 2; ++j)
                bfr[j] = *reinterpret_cast<const pg_bf16x8 *>(
                    &Bs[buf][(64 * wn + 32 * j + fr) * PG_LD + 16 * ks + fk]);
#pragma unroll
            for (int i = 0; i < MBK; ++i)
                afr[i] = *reinterpret_cast<const pg_bf16x8 *>(
                    &As[buf][(wm * (BM / 2) + 32 * i + fr) * PG_LD + 16 * ks + fk]);
#pragma unroll
            for (int i = 0; i < MBK; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(afr[i], bfr[j], acc[i][j], 0, 0, 0);
        }
    };
    lds_barrier();  // tile 0 ready
    for (int step = 0; step < npad; step += 2) {
        if (step < nsteps)
            compute(0);
        lds_barrier();
        if (step + 1 < nsteps)
            compute(1);
        lds_barrier();
    }

    // ---- epilogue: C row (8 * (r / 4) + 4 * (l / 32) + r % 4), column l % 32
    const int ccol = lane & 31, crow = 4 * (lane >> 5);
    if constexpr (EPI == PG_Y) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int n = n0 + 64 * wn + 32 * j + ccol;
            if (n >= a.N)
                continue;
#pragma unroll
            for (int i = 0; i < MBK; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int m = m0 + wm * (BM / 2) + 32 * i + 8 * (r / 4) + crow + (r % 4);
                    if (m < a.M)
                        ((float *)a.y)[(int64_t)m * a.ldy + n] = acc[i][j][r];
                }
        }
    }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------

// The int4 formats with whole 32-input packets, 8-byte aligned rows and (fmt
// 4) a power-of-two group size of at least 32.
bool pgemm_ok(const coli_qtensor *W) {
    if (W->fmt != 2 && W->fmt != 4)
        return false;
    if (!(W->flags & QF_FAST) || W->I % 32 != 0 || W->row_bytes % 8 != 0)
        return false;
    return W->fmt != 4 || (W->gs >= 32 && (W->gs & (W->gs - 1)) == 0);
}

int launch_pgemm_dense(const coli_qtensor *W, const float *x, float *y, int S, hipStream_t st) {
    if (!pgemm_ok(W) || S < 1 || (uintptr_t)x % 16 != 0 || W->I % 16 != 0)
        return 0;
    ProfScope ps("gemm_dense", st);
    for (int e = 0; e < W->n; ++e) {
        PgArgs a;
        memset(&a, 0, sizeof a);
        a.x = x;
        a.ldx = W->I;
        a.M = S;
        a.K = W->I;
        a.q[0] = a.q[1] = (const uint8_t *)W->q + (int64_t)e * W->q_stride;
        a.s[0] = a.s[1] = W->s + (int64_t)e * W->s_stride;
        a.rb = W->row_bytes;
        a.ng = W->ng;
        a.gshift = W->fmt == 4 ? __builtin_ctz((unsigned)W->gs) : 0;
        a.N = W->O;
        a.fmt = W->fmt;
        a.y = y + (int64_t)e * S * W->O;
        a.ldy = W->O;
        if (S > 64) {
            const dim3 grid((unsigned)((S + 127) / 128), (unsigned)((W->O + PG_BN - 1) / PG_BN));
            hipLaunchKernelGGL((k_pg<128, 1, PG_Y, true>), grid, dim3(512), 0, st, a);
        } else {
            const dim3 grid((unsigned)((S + 63) / 64), (unsigned)((W->O + PG_BN - 1) / PG_BN));
            hipLaunchKernelGGL((k_pg<64, 1, PG_Y, true>), grid, dim3(512), 0, st, a);
        }
    }
    return after_launch("gemm_dense") == COLI_OK ? 1 : -1;
}

}  // namespace coli
