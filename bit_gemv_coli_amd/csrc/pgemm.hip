// pgemm.hip -- prefill GEMM (S > 4 input rows) for the int4 formats on the
// gfx950 matrix cores: Y[m][n] = sum_k w(n, k) * X[m][k].  Two kernels:
//   k_pg  producer/consumer wavefronts with a double-buffered LDS tile for
//         both operands (dense rows; plain int4 experts in the MoE block);
//   k_sg  weight streaming for packed experts in the MoE block (further down).
//
// What is computed (colibri PR #298, CUDA fmt=4 commit: w = scale(n, k/gs) *
// (q - 8), the group scale applied inline; colibri-strix prefill GEMM routing commit: large row batches take a GEMM path).
//
// Precision (the bf16 envelope): every weight is dequantized once per
// workgroup to bf16(s * (q - 8)) -- one rounding of the exact product -- and
// every input to bf16(x); products accumulate in fp32 on
// v_mfma_f32_32x32x16_bf16.  bf16 keeps 8 significant bits (each rounding
// within 2^-8 relative), so |error| <= (2^-7 + 2^-16) * sum |w||x| plus the
// fp32 accumulation; with no single product carrying most of sum |w||x| the
// roundings average out far inside 4e-3 * sum |w||x|.
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
    // routed (MoE) tiles: tile t = (expert tiles[2t], first row tiles[2t+1]);
    // expert E is the shared expert (rows SK ..); weights of expert e at
    // q[m] + e * q_stride
    const uint8_t *sq[2];
    const float *ss[2];
    int64_t q_stride, s_stride;
    const int32_t *tiles, *n_tiles, *counts, *offsets;
    int E, SK, S;
    int nkb, nkq, cbs, rtn;  // packed copy: blocks per row, quads, scale slots, 16-row tiles
    int mchunk;              // weight-streaming kernel: row tiles run together on one XCD
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

template <int BM, int NMAT, int EPI, bool AF32, bool MOE>
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
    if (MOE) {
        // routed tiles (gridDim.x a multiple of 8): tile mt runs on XCD mt % 8
        // -- unused tiles at the end of the list spread over all XCDs -- and
        // each XCD takes its tiles one after the other with all their
        // weight-row tiles together, so a tile's input rows stay in that L2
        const int w = blockIdx.y * gridDim.x + blockIdx.x, ntn = gridDim.y;
        const int xcd = w % 8, idx = w / 8;
        mt = 8 * (idx / ntn) + xcd;
        nt = idx % ntn;
    } else {
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
    // rows of this tile: X rows xr0 .. xr0 + mcount - 1 (routing order for
    // MoE), weights of expert e
    int xr0, mcount;
    const uint8_t *wq[NMAT];
    const float *wsc[NMAT];
    if (MOE) {
        if (mt >= gload<int32_t>(a.n_tiles))
            return;  // whole workgroup: the tile list is shorter than the grid
        const int e = gload<int32_t>(a.tiles + 2 * mt);
        const int r0 = gload<int32_t>(a.tiles + 2 * mt + 1);
        const bool shared = e >= a.E;
        xr0 = (shared ? a.SK : gload<int32_t>(a.offsets + e)) + r0;
        mcount = min(BM, (shared ? a.S : gload<int32_t>(a.counts + e)) - r0);
#pragma unroll
        for (int m = 0; m < NMAT; ++m) {
            wq[m] = shared ? a.sq[m] : a.q[m] + (int64_t)e * a.q_stride;
            wsc[m] = shared ? a.ss[m] : a.s[m] + (int64_t)e * a.s_stride;
        }
    } else {
        xr0 = mt * BM;
        mcount = min(BM, a.M - xr0);
#pragma unroll
        for (int m = 0; m < NMAT; ++m) {
            wq[m] = a.q[m];
            wsc[m] = a.s[m];
        }
    }
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
        const uint8_t *qrow = wq[mat] + (int64_t)nrow * a.rb;
        const float *srow = wsc[mat] + (a.fmt == 4 ? (int64_t)nrow * a.ng : (int64_t)nrow);
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
        int64_t xstep[NA];  // row offset of request i (rows past the tile clamped)
#pragma unroll
        for (int i = 0; i < NA; ++i)
            xstep[i] = (int64_t)(xr0 + min(aro + ARI * i, mcount - 1)) * a.ldx;

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
    if constexpr (EPI == PG_SILU) {
        // gate values sit in the wn = 0 wavefronts, up values of the same
        // outputs in wn = 1: up goes through LDS (the producers have ended)
        float *ex = reinterpret_cast<float *>(&Bs[0][0]);  // [BM][64] f32
        if (wn == 1) {
#pragma unroll
            for (int i = 0; i < MBK; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int m = wm * (BM / 2) + 32 * i + 8 * (r / 4) + crow + (r % 4);
                        ex[m * 64 + 32 * j + ccol] = acc[i][j][r];
                    }
        }
        lds_barrier();
        if (wn == 0) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int n = n0 + 32 * j + ccol;
                if (n >= a.N)
                    continue;
#pragma unroll
                for (int i = 0; i < MBK; ++i)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int m = wm * (BM / 2) + 32 * i + 8 * (r / 4) + crow + (r % 4);
                        if (m < mcount) {
                            const float g = acc[i][j][r], u = ex[m * 64 + 32 * j + ccol];
                            ((pg_bf16 *)a.y)[(int64_t)(xr0 + m) * a.ldy + n] =
                                (pg_bf16)((g / (1.0f + expf(-g))) * u);
                        }
                    }
            }
        }
    } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int n = n0 + 64 * wn + 32 * j + ccol;
            if (n >= a.N)
                continue;
#pragma unroll
            for (int i = 0; i < MBK; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int m = wm * (BM / 2) + 32 * i + 8 * (r / 4) + crow + (r % 4);
                    if (m < mcount)
                        ((float *)a.y)[(int64_t)(xr0 + m) * a.ldy + n] = acc[i][j][r];
                }
        }
    }
}

// ---------------------------------------------------------------------------
// Weight-streaming GEMM for short row tiles (the routed MoE experts), on the
// packed copy of the weights: 16-row tiles of 128-input blocks, 1 KiB each,
// lane l = 16 j + r holding row r, inputs 32 j .. 32 j + 31 as
// two's-complement nibbles, plus per (tile, 4 blocks, row, group slot) runs
// of 4 scales.  Every wavefront streams its own tiles straight into registers
// (one contiguous KiB per tile and block, four blocks in flight, scale runs
// once per four blocks), turns the nibbles into bf16 there and runs
// v_mfma_f32_16x16x32_bf16 against the input rows, which the workgroup
// stages through LDS one block ahead (one barrier per block).  No weight
// passes through LDS.
//
// Inputs inside a block: lane (n = l % 16, g = l / 16) holds inputs
// 32 g .. 32 g + 31 of weight row n; MFMA slice s (0..3) takes inputs
// 32 g + 8 s .. + 8 from each lane, and the input rows are read from LDS at the
// same columns, so every slice sums 32 distinct inputs and the four slices
// cover the block.
//
// Scales and conversion (SM): with groups of >= 128 inputs (and the
// per-row format) a block lies inside one group.  There the code q becomes
// the bf16 number 2 + q / 8 by placing its bits in the mantissa (two shifts,
// two masks and four byte permutes per 8 codes), so that
// sum (q - 8) x = 8 (sum (2 + q / 8) x - 3 sum x); a fifth MFMA per row block
// adds -3 sum x (a constant -3 weight row), and the group's scale times 8 is
// applied once to the group sum in fp32 (SM_GRP1: groups of one block, the
// group sum starts from zero in the MFMA; SM_GRPN: longer groups; SM_ROW: the
// per-row format, one group per row).  The byte permutes pair inputs 0-2, 4-6, 1-3, 5-7, so the
// input rows are stored in LDS in that order within every 8 inputs.  Groups
// of 32 or 64 (SM_FOLD) fold the scale into the bf16 weights instead, each
// lane's 32 inputs lying in one group.
constexpr int SG_KC = 128;         // inputs per block
constexpr int SG_LDA = SG_KC + 8;  // LDS row stride of the input tile (bf16 elements)
constexpr int SG_NB = 4;           // blocks in flight (= blocks per scale run)

typedef float sg_f32x4 __attribute__((ext_vector_type(4)));
enum { SM_FOLD = 0, SM_GRP1 = 1, SM_GRPN = 2, SM_ROW = 3 };

template <int MB, int NCT, int NMAT, int EPI, bool MOE, int SM>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_sg(PgArgs a) {
    constexpr int TM = 16 * MB;       // input rows per tile
    constexpr int TPM = NCT / NMAT;   // 16-row weight tiles per matrix per wavefront
    constexpr int WCOL = 16 * TPM;    // output columns per wavefront
    static_assert(NCT % NMAT == 0, "tiles per matrix");
    __shared__ __attribute__((aligned(16))) pg_bf16 As[2][TM * SG_LDA];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int mt, nt;
    {
        // XCD-aware order (workgroup w runs on XCD w % 8; gridDim.x a multiple
        // of 8 L): runs of L = mchunk consecutive row tiles go to one XCD,
        // which takes their column tiles one by one with the L row tiles of
        // each side by side, so the L tiles (usually one expert's) read every
        // weight slice together and share it through that XCD's L2, while
        // their input rows stay there too.  L = 1: row tile mt on XCD mt % 8
        // with all its column tiles together.
        const int w = blockIdx.y * gridDim.x + blockIdx.x, ntn = gridDim.y;
        const int L = a.mchunk > 0 ? a.mchunk : 1;
        if (gridDim.x % (8 * L) == 0) {
            const int xcd = w % 8, j = w / 8, per = L * ntn;
            const int r = j / per, q = j % per;
            nt = q / L;
            mt = (r * 8 + xcd) * L + q % L;
        } else {
            mt = blockIdx.x;
            nt = blockIdx.y;
        }
    }
    int xr0, mcount;
    const uint8_t *wq[NMAT];  // packed codes of the matrix
    const float *wsc[NMAT];   // its packed scale runs (fmt 4) or row scales (fmt 2)
    if (MOE) {
        if (mt >= gload<int32_t>(a.n_tiles))
            return;  // whole workgroup: the tile list is shorter than the grid
        const int e = gload<int32_t>(a.tiles + 2 * mt);
        const int r0 = gload<int32_t>(a.tiles + 2 * mt + 1);
        const bool shared = e >= a.E;
        xr0 = (shared ? a.SK : gload<int32_t>(a.offsets + e)) + r0;
        mcount = min(TM, (shared ? a.S : gload<int32_t>(a.counts + e)) - r0);
#pragma unroll
        for (int m = 0; m < NMAT; ++m) {
            wq[m] = shared ? a.sq[m] : a.q[m] + (int64_t)e * a.q_stride;
            wsc[m] = shared ? a.ss[m] : a.s[m] + (int64_t)e * a.s_stride;
        }
    } else {
        xr0 = mt * TM;
        mcount = min(TM, a.M - xr0);
#pragma unroll
        for (int m = 0; m < NMAT; ++m) {
            wq[m] = a.q[m];
            wsc[m] = a.s[m];
        }
    }
    const int K = a.K;
    const int nch = a.nkb;  // blocks (the last one zero-padded past K)
    const int npad = (nch + SG_NB - 1) / SG_NB * SG_NB;
    const int ln = lane & 15, lg = lane >> 4;
    const int c0 = nt * (4 * WCOL) + wave * WCOL;  // first output column of this wavefront

    // ---- weight tiles of this wavefront (tiles past the matrix clamped; their
    // outputs are dropped): code and scale-run offsets within the matrix
    int qoff[NCT], soff[NCT];
    float rsc[NCT];  // per-row scale (SM_ROW)
    constexpr bool SF = SM == SM_FOLD;
    const int cb = SF ? (lg >> (a.gshift - 5)) : 0;  // this lane's group slot in a block
#pragma unroll
    for (int t = 0; t < NCT; ++t) {
        const int tile = min((c0 + 16 * (t % TPM)) >> 4, a.rtn - 1);
        qoff[t] = tile * a.nkb * 1024 + 16 * lane;
        soff[t] = ((tile * a.nkq * 16 + ln) * a.cbs + cb) * 4;
        if (SM == SM_ROW)
            rsc[t] = gload<float>(wsc[t / TPM] + min(c0 + 16 * (t % TPM) + ln, a.N - 1));
    }
    struct BSlot {
        u32x4 c[NCT];
    };
    // unconditional requests at clamped addresses: blocks past the last one
    // meet zero inputs (the LDS tile is zero there)
    auto bload = [&](BSlot &b, int c) {
        const int cc = min(c, nch - 1);
#pragma unroll
        for (int t = 0; t < NCT; ++t) b.c[t] = gload<u32x4>(wq[t / TPM] + (qoff[t] + cc * 1024));
    };
    auto rload = [&](sg_f32x4 *run, int kq) {
        const int kqc = min(kq, a.nkq - 1);
        if constexpr (SM != SM_ROW)
#pragma unroll
            for (int t = 0; t < NCT; ++t) run[t] = gload<sg_f32x4>(wsc[t / TPM] + (soff[t] + kqc * 64 * a.cbs));
    };

    // ---- input rows: 8 bf16 per 16-byte request, 16 lanes per row
    constexpr int ALPR = SG_KC / 8;
    constexpr int AROWS = 256 / ALPR;
    constexpr int NAQ = TM / AROWS;
    static_assert(NAQ >= 1, "tile rows");
    const int arow0 = tid / ALPR, acol = 8 * (tid % ALPR);
    int64_t aoff[NAQ];
#pragma unroll
    for (int i = 0; i < NAQ; ++i)
        aoff[i] = (int64_t)(xr0 + min(arow0 + AROWS * i, mcount - 1)) * a.ldx;
    struct ASlot {
        u32x4 v[NAQ];
    };
    auto aload = [&](ASlot &sl, int c) {
        const int kk = min(min(c, nch - 1) * SG_KC + acol, K - 8);
#pragma unroll
        for (int i = 0; i < NAQ; ++i)
            sl.v[i] = gload<u32x4>((const pg_bf16 *)a.x + (aoff[i] + kk));
    };
    // inputs of block c to LDS, every 8 in the order 0 2 4 6 1 3 5 7; columns
    // past K (and blocks past the last) as zeros
    auto astore = [&](ASlot &sl, int stage, int c) {
#pragma unroll
        for (int i = 0; i < NAQ; ++i) asm volatile("" : "+v"(sl.v[i]));
        const bool zero = c * SG_KC + acol >= K;
#pragma unroll
        for (int i = 0; i < NAQ; ++i) {
            const u32x4 v = sl.v[i];
            const u32x4 o = {__builtin_amdgcn_perm(v.y, v.x, 0x05040100u), __builtin_amdgcn_perm(v.w, v.z, 0x05040100u),
                             __builtin_amdgcn_perm(v.y, v.x, 0x07060302u), __builtin_amdgcn_perm(v.w, v.z, 0x07060302u)};
            *reinterpret_cast<u32x4 *>(&As[stage][(arow0 + AROWS * i) * SG_LDA + acol]) =
                zero ? u32x4{0u, 0u, 0u, 0u} : o;
        }
    };
    auto lds_barrier = []() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); };

    // ---- accumulators: C tile (i, t), lane holds rows 4 (l / 16) + r, column l % 16
    const sg_f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
    sg_f32x4 acc[MB][NCT], accg[MB][NCT], corr[MB];
#pragma unroll
    for (int i = 0; i < MB; ++i) {
        corr[i] = zero4;
#pragma unroll
        for (int t = 0; t < NCT; ++t) {
            acc[i][t] = zero4;
            accg[i][t] = zero4;
        }
    }
    // bf16 -3 in every element: the weight row that adds -3 sum x
    const pg_bf16x8 neg3 = __builtin_bit_cast(pg_bf16x8, u32x4{0xC040C040u, 0xC040C040u, 0xC040C040u, 0xC040C040u});
    // a group ends after block c when c + 1 is a multiple of the blocks per
    // group (never inside a row for the per-row format) or at the last block
    const int gblk = a.ng;

    // block c = 4 kq + u with the scale runs of quad kq
    auto compute = [&](BSlot &b, const sg_f32x4 *run, int u, int stage, int c) {
#pragma unroll
        for (int t = 0; t < NCT; ++t) asm volatile("" : "+v"(b.c[t]));
        float f[NCT];
#pragma unroll
        for (int t = 0; t < NCT; ++t)  // SM_FOLD weights hold 16 (q - 8), the others (q - 8) / 8
            f[t] = (SM == SM_ROW ? rsc[t] : run[t][u]) * (SF ? 0.0625f : 8.0f);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            pg_bf16x8 afr[MB];
#pragma unroll
            for (int i = 0; i < MB; ++i)
                afr[i] = *reinterpret_cast<const pg_bf16x8 *>(
                    &As[stage][(16 * i + ln) * SG_LDA + 32 * lg + 8 * s]);
            const bool fresh = SM == SM_GRP1 && s == 0;  // the group sum starts here
            if constexpr (!SF) {
#pragma unroll
                for (int i = 0; i < MB; ++i)
                    corr[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr[i], neg3, fresh ? zero4 : corr[i], 0, 0, 0);
            }
#pragma unroll
            for (int t = 0; t < NCT; ++t) {
                const uint32_t w = b.c[t][s];  // two's-complement nibbles q - 8
                u32x4 bw;
                if constexpr (SF) {
                    const uint32_t ev = (w << 4) & 0xF0F0F0F0u;  // 16 (q - 8) of inputs 0, 2, 4, 6
                    const uint32_t od = w & 0xF0F0F0F0u;         // of inputs 1, 3, 5, 7
                    const float sc = f[t];
                    bw = u32x4{pk_bf16(sbyte<0>(ev) * sc, sbyte<1>(ev) * sc),
                               pk_bf16(sbyte<2>(ev) * sc, sbyte<3>(ev) * sc),
                               pk_bf16(sbyte<0>(od) * sc, sbyte<1>(od) * sc),
                               pk_bf16(sbyte<2>(od) * sc, sbyte<3>(od) * sc)};
                } else {
                    // q << 3 in the low mantissa byte of bf16 0x40nn: 2 + q / 8
                    const uint32_t lo = ((w << 3) & 0x78787878u) ^ 0x40404040u;  // inputs 0, 2, 4, 6
                    const uint32_t hi = ((w >> 1) & 0x78787878u) ^ 0x40404040u;  // inputs 1, 3, 5, 7
                    bw = u32x4{__builtin_amdgcn_perm(0x40404040u, lo, 0x05010400u),
                               __builtin_amdgcn_perm(0x40404040u, lo, 0x05030402u),
                               __builtin_amdgcn_perm(0x40404040u, hi, 0x05010400u),
                               __builtin_amdgcn_perm(0x40404040u, hi, 0x05030402u)};
                }
                const pg_bf16x8 bfr = __builtin_bit_cast(pg_bf16x8, bw);
#pragma unroll
                for (int i = 0; i < MB; ++i)
                    accg[i][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr[i], bfr, fresh ? zero4 : accg[i][t], 0, 0, 0);
            }
        }
        const bool gend = SM == SM_GRP1 || (SM == SM_GRPN && (c + 1) % gblk == 0) || c + 1 == nch;
        if (!SF && c < nch && gend) {
#pragma unroll
            for (int i = 0; i < MB; ++i)
#pragma unroll
                for (int t = 0; t < NCT; ++t)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        acc[i][t][r] = fmaf(f[t], accg[i][t][r] + corr[i][r], acc[i][t][r]);
                        if (SM != SM_GRP1)
                            accg[i][t][r] = 0.f;
                    }
            if (SM != SM_GRP1)
#pragma unroll
                for (int i = 0; i < MB; ++i) corr[i] = zero4;
        }
    };

    // ---- pipeline: the codes and inputs of block c are requested SG_NB blocks
    // earlier (inputs first), the scale runs of a quad one quad earlier, the
    // inputs go to LDS at the end of block c - 1.  Requests complete in order,
    // so waiting for the inputs of block c + 1 only forces code requests of
    // blocks up to c + 1.
    BSlot bs[SG_NB];
    ASlot as[SG_NB];
    sg_f32x4 run[NCT], runn[NCT];
#pragma unroll
    for (int u = 0; u < SG_NB; ++u) {
        aload(as[u], u);
        bload(bs[u], u);
    }
    rload(runn, 0);
    astore(as[0], 0, 0);
    lds_barrier();  // block 0 in LDS
    for (int base = 0; base < npad; base += SG_NB) {
#pragma unroll
        for (int t = 0; t < NCT; ++t) {
            asm volatile("" : "+v"(runn[t]));
            run[t] = runn[t];
        }
        rload(runn, base / SG_NB + 1);
#pragma unroll
        for (int u = 0; u < SG_NB; ++u) {
            const int c = base + u;
            aload(as[u], c + SG_NB);
            __builtin_amdgcn_sched_barrier(0);
            compute(bs[u], run, u, u % 2, c);
            __builtin_amdgcn_sched_barrier(0);
            bload(bs[u], c + SG_NB);
            __builtin_amdgcn_sched_barrier(0);
            astore(as[(u + 1) % SG_NB], (u + 1) % 2, c + 1);
            lds_barrier();
        }
    }
    if (SF) {
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int t = 0; t < NCT; ++t) acc[i][t] = accg[i][t];
    }

    // ---- epilogue
    if constexpr (EPI == PG_SILU) {
#pragma unroll
        for (int t = 0; t < TPM; ++t) {
            const int n = c0 + 16 * t + ln;
            if (n >= a.N)
                continue;
#pragma unroll
            for (int i = 0; i < MB; ++i)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int m = 16 * i + 4 * lg + r;
                    if (m < mcount) {
                        const float g = acc[i][t][r], u = acc[i][t + TPM][r];
                        ((pg_bf16 *)a.y)[(int64_t)(xr0 + m) * a.ldy + n] =
                            (pg_bf16)((g / (1.0f + expf(-g))) * u);
                    }
                }
        }
    } else {
#pragma unroll
        for (int t = 0; t < NCT; ++t) {
            const int n = c0 + 16 * t + ln;
            if (n >= a.N)
                continue;
#pragma unroll
            for (int i = 0; i < MB; ++i)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int m = 16 * i + 4 * lg + r;
                    if (m < mcount)
                        ((float *)a.y)[(int64_t)(xr0 + m) * a.ldy + n] = acc[i][t][r];
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
            hipLaunchKernelGGL((k_pg<128, 1, PG_Y, true, false>), grid, dim3(512), 0, st, a);
        } else {
            const dim3 grid((unsigned)((S + 63) / 64), (unsigned)((W->O + PG_BN - 1) / PG_BN));
            hipLaunchKernelGGL((k_pg<64, 1, PG_Y, true, false>), grid, dim3(512), 0, st, a);
        }
    }
    return after_launch("gemm_dense") == COLI_OK ? 1 : -1;
}

// ---- prefill MoE stages over the routed tile list (gridDim.x = max_tiles
// rounded up to 8): gate/up + SiLU into bf16 h (routing order), down into f32
// rows.  Tensors with a packed copy run the weight-streaming kernel on 32-row
// tiles, the others the producer/consumer kernel on 64-row tiles.

static bool moe_all(const MoeArgs &m, bool (*ok)(const coli_qtensor *)) {
    const coli_qtensor *all[6] = {m.gate, m.up, m.down, m.sg, m.su, m.sd};
    for (const coli_qtensor *t : all)
        if (t && !ok(t))
            return false;
    return true;
}

int pgemm_moe_rows(const MoeArgs &m) {
    if (m.D % 32 != 0 || m.F % 32 != 0)
        return 0;
    if (moe_all(m, mgemv_int4_ok))
        return PG_MOE_ROWS_PACKED;
    if (moe_all(m, pgemm_ok))
        return PG_MOE_ROWS;
    return 0;
}

// operands of one projection (matrix index mi of the pair) for either kernel
static void pg_operand(PgArgs &a, int mi, const coli_qtensor *T, const coli_qtensor *Sh, bool packed) {
    if (packed) {
        a.q[mi] = (const uint8_t *)T->pk;
        a.s[mi] = T->fmt == 4 ? (const float *)((const uint8_t *)T->pk + T->pk_scale_off) : T->s;
        a.q_stride = T->pk_stride;
        a.s_stride = T->fmt == 4 ? T->pk_stride / 4 : T->s_stride;
        const coli_qtensor *H = Sh ? Sh : T;
        a.sq[mi] = Sh ? (const uint8_t *)H->pk : a.q[mi];
        a.ss[mi] = Sh ? (H->fmt == 4 ? (const float *)((const uint8_t *)H->pk + H->pk_scale_off) : H->s)
                      : a.s[mi];
        a.nkb = (T->I + 127) / 128;
        a.nkq = (a.nkb + 3) / 4;
        a.cbs = (T->fmt != 4 || T->gs % 128 == 0) ? 1 : 128 / T->gs;
        a.rtn = (T->O + 15) / 16;
        // blocks per scale group (the per-row format: never inside a row)
        a.ng = T->fmt == 4 ? std::max(1, T->gs / 128) : a.nkb + 1;
        a.gshift = (T->fmt == 4 && T->gs < 128) ? __builtin_ctz((unsigned)T->gs) : 0;
    } else {
        a.q[mi] = (const uint8_t *)T->q;
        a.s[mi] = T->s;
        a.q_stride = T->q_stride;
        a.s_stride = T->s_stride;
        a.sq[mi] = Sh ? (const uint8_t *)Sh->q : a.q[mi];
        a.ss[mi] = Sh ? Sh->s : a.s[mi];
        a.ng = T->ng;
        a.gshift = T->fmt == 4 ? __builtin_ctz((unsigned)T->gs) : 0;
    }
    a.rb = T->row_bytes;
    a.N = T->O;
    a.fmt = T->fmt;
}

// 16-row weight tiles per wavefront in the weight-streaming kernel (measured:
// 2 instead of 4 is 8% slower on the Zipf(1.1) S=544 block; 64-row input
// tiles, which need 2 to fit the registers, 1.5x slower)
#ifndef COLI_SG_NCT
#define COLI_SG_NCT 4
#endif

template <int SM, int MB>
static void sg_launch(const PgArgs &a, unsigned gx, bool down, hipStream_t st) {
    constexpr int NCT = COLI_SG_NCT;
    // output columns per workgroup: 4 wavefronts x 16 NCT / NMAT
    if (!down)
        hipLaunchKernelGGL((k_sg<MB, NCT, 2, PG_SILU, true, SM>),
                           dim3(gx, (unsigned)((a.N + 32 * NCT - 1) / (32 * NCT))), dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL((k_sg<MB, NCT, 1, PG_PART, true, SM>),
                           dim3(gx, (unsigned)((a.N + 64 * NCT - 1) / (64 * NCT))), dim3(256), 0, st, a);
}

template <int MB>
static void sg_stage(const PgArgs &a, unsigned gx, bool down, const coli_qtensor *T, hipStream_t st) {
    if (T->fmt == 4 && T->gs < 128) sg_launch<SM_FOLD, MB>(a, gx, down, st);
    else if (T->fmt == 4 && T->gs == 128) sg_launch<SM_GRP1, MB>(a, gx, down, st);
    else if (T->fmt == 4) sg_launch<SM_GRPN, MB>(a, gx, down, st);
    else sg_launch<SM_ROW, MB>(a, gx, down, st);
}

// one projection stage over the routed tiles; packed experts: the row tiles
// of PG_MOE_ROWS_PACKED rows, then (gx_s > 0) the short tiles of experts with
// at most PG_MOE_ROWS_SHORT rows, which halve the matrix-core and input work
// of the many lightly routed experts
// row tiles of one XCD run (see k_sg) in the pass over the longer tiles
// (measured on the S=544 Zipf(1.1) / Zipf(2.5) blocks: 1, 2, 4 within noise
// of each other, 8 slower on Zipf(2.5); the repeated weight reads of the
// multi-tile experts are served by the last-level cache either way)
#ifndef COLI_SG_MCHUNK
#define COLI_SG_MCHUNK 2
#endif

static void pg_moe_stage(const PgArgs &a, unsigned gx, bool down, bool packed, const coli_qtensor *T,
                         hipStream_t st, const int32_t *tiles_s, const int32_t *n_tiles_s,
                         unsigned gx_s) {
    if (packed) {
        PgArgs b = a;
        b.mchunk = COLI_SG_MCHUNK;
        const unsigned g8 = 8u * COLI_SG_MCHUNK;
        sg_stage<PG_MOE_ROWS_PACKED / 16>(b, (gx + g8 - 1) / g8 * g8, down, T, st);
        if constexpr (PG_MOE_ROWS_SHORT > 0) {
            if (gx_s > 0) {
                b.mchunk = 1;
                b.tiles = tiles_s;
                b.n_tiles = n_tiles_s;
                sg_stage<PG_MOE_ROWS_SHORT / 16>(b, gx_s, down, T, st);
            }
        }
    } else if (!down) {
        hipLaunchKernelGGL((k_pg<PG_MOE_ROWS, 2, PG_SILU, false, true>),
                           dim3(gx, (unsigned)((a.N + 63) / 64)), dim3(512), 0, st, a);
    } else {
        hipLaunchKernelGGL((k_pg<PG_MOE_ROWS, 1, PG_PART, false, true>),
                           dim3(gx, (unsigned)((a.N + 127) / 128)), dim3(512), 0, st, a);
    }
}

int launch_pgemm_moe(const MoeArgs &m, int rows, const void *xg, void *hg, float *y,
                     const int32_t *tiles, const int32_t *n_tiles, const int32_t *counts,
                     const int32_t *offsets, int max_tiles, const int32_t *tiles_s,
                     const int32_t *n_tiles_s, int max_short) {
    const bool packed = rows > 0 && moe_all(m, mgemv_int4_ok);
    const unsigned gx = (unsigned)((max_tiles + 7) / 8 * 8);
    const unsigned gx_s = (packed && tiles_s && n_tiles_s && max_short > 0)
                              ? (unsigned)((max_short + 7) / 8 * 8) : 0u;
    PgArgs a;
    memset(&a, 0, sizeof a);
    a.tiles = tiles; a.n_tiles = n_tiles; a.counts = counts; a.offsets = offsets;
    a.E = m.E; a.SK = m.S * m.K; a.S = m.S;
    {
        pg_operand(a, 0, m.gate, m.sg, packed);
        pg_operand(a, 1, m.up, m.su, packed);
        a.x = xg;
        a.ldx = m.D;
        a.K = m.D;
        a.y = hg;
        a.ldy = m.F;
        ProfScope ps("moe_gateup_gemm", m.st);
        pg_moe_stage(a, gx, false, packed, m.gate, m.st, tiles_s, n_tiles_s, gx_s);
        int rc = after_launch("moe_gateup_gemm");
        if (rc != COLI_OK) return rc;
    }
    if (y == nullptr)
        return COLI_OK;
    {
        pg_operand(a, 0, m.down, m.sd, packed);
        pg_operand(a, 1, m.down, m.sd, packed);
        a.x = hg;
        a.ldx = m.F;
        a.K = m.F;
        a.y = y;
        a.ldy = m.D;
        ProfScope ps("moe_down_gemm", m.st);
        pg_moe_stage(a, gx, true, packed, m.down, m.st, tiles_s, n_tiles_s, gx_s);
        return after_launch("moe_down_gemm");
    }
}

}  // namespace coli
