// mgemv.hip -- decode GEMV on the matrix cores (gfx950), for the int4 formats
// (fmt 4 grouped, fmt 2 per row) at S <= 4 input rows.
//
// What is computed (colibri PR #298, CUDA fmt=4 commit: every group's scale
// multiplies that group's partial sum; Metal mm_gemv fmt=4 commit: fmt 2
// scales once per row after the dot product):
//     y[t][o] = sum_g s[o][g] * sum_{i in g} (q(o,i) - 8) * x[t][i]
//
// Why matrix cores for a bandwidth-bound GEMV: at 8 TB/s an int4 GEMV has to
// retire ~14e12 weights/s, and converting codes to floats one by one on the
// vector ALUs takes most of the VALU issue budget.  Here the products are
// exact integer products on v_mfma_i32_16x16x64_i8:
//   weights  the packed copy holds each code as the two's-complement nibble
//            v = q - 8 (the pages' upload-time offset_to_signed_s4).  For a
//            word of 8 nibbles, w & 0xF0F0F0F0 is 16*v of the odd inputs as
//            four int8 and (w << 4) & 0xF0F0F0F0 is 16*v of the even inputs:
//            two 16-byte B operands from 12 VALU instructions per 32 codes.
//   inputs   per (input row, 128-input block) a power of two 2^e brings
//            max|x| into [2^29, 2^30); X = trunc(x * 2^e) is an int32 within
//            2^-29 max|x| 2^e of x 2^e, and X = d0 + 2^8 d1 + 2^16 d2 + 2^24 d3
//            with signed byte digits: the bytes of (X + 0x808080) XOR
//            0x808080.  The digits, moved into one row per digit, are the
//            int8 A operand.
//   sums     exact in int32 per 128-input block (|sum| < 2^22); the group
//            scale, 2^-e, the digit weight and 1/16 are applied in fp32.
// Accuracy: the represented input is within 2^-e <= 2^-29 max|x| of its
// block (2^-126 for blocks below 2^-96), so an output moves by at most
// 2^-29 * sum_b max_b|x| * sum_{i in b} |w_i| on top of the fp32 rounding
// (1e-5 * sum |w||x|).  For activations of similar magnitude that term is
// ~1e-8 of sum |w||x|; one input far above the rest of its block where the
// weights are zero makes it dominate (the vector-ALU kernels have no such
// term).
//
// Layout of one matrix-core step (16 weight rows x 128 inputs):
//   lane l: weight row n = l % 16, input quarter j = l / 16; it loads the 16
//   code bytes of row n at inputs [32j, 32j+32) of the block (one 1 KiB
//   request per wavefront in the packed copy).  Its even and odd inputs form
//   the B operands of two MFMAs.  A row r of a set = (combination c of group-
//   in-block and input row, digit r % 4) with c = 4 * set + r / 4; an A lane
//   whose inputs belong to another group than its row's reads zeros, so each
//   group's sum lands in its own output rows.  C rows 4j .. 4j+3 of a lane are
//   the four digits of combination 4 * set + j.
#include <string.h>

#include <algorithm>

#include <hip/hip_ext.h>

#include "common.h"
#include "rms.h"

namespace coli {

typedef int i32x4 __attribute__((ext_vector_type(4)));

// 16*v of the odd / even inputs of a word of 8 two's-complement nibbles
__device__ __forceinline__ uint32_t odd_x16(uint32_t w) { return w & 0xF0F0F0F0u; }
__device__ __forceinline__ uint32_t even_x16(uint32_t w) { return (w << 4) & 0xF0F0F0F0u; }

// int32 -> four signed byte digits, X = d0 + 2^8 d1 + 2^16 d2 + 2^24 d3
// (|X| < 2^30): byte i of (X + 0x808080) is d_i + 128 for i < 3
__device__ __forceinline__ uint32_t digits_of(float xs) {
    return ((uint32_t)(int)xs + 0x808080u) ^ 0x808080u;
}

// 4x4 byte transpose: out[d] byte b = byte d of in[b]
__device__ __forceinline__ void transpose4(uint32_t a, uint32_t b, uint32_t c, uint32_t d,
                                           uint32_t out[4]) {
    // v_perm_b32 selects bytes of {S0 (bytes 4-7), S1 (bytes 0-3)}
    const uint32_t ab0 = __builtin_amdgcn_perm(b, a, 0x05010400u);  // a0 b0 a1 b1
    const uint32_t ab1 = __builtin_amdgcn_perm(b, a, 0x07030602u);  // a2 b2 a3 b3
    const uint32_t cd0 = __builtin_amdgcn_perm(d, c, 0x05010400u);
    const uint32_t cd1 = __builtin_amdgcn_perm(d, c, 0x07030602u);
    out[0] = __builtin_amdgcn_perm(cd0, ab0, 0x05040100u);  // a0 b0 c0 d0
    out[1] = __builtin_amdgcn_perm(cd0, ab0, 0x07060302u);
    out[2] = __builtin_amdgcn_perm(cd1, ab1, 0x05040100u);
    out[3] = __builtin_amdgcn_perm(cd1, ab1, 0x07060302u);
}

// epilogues: y; SiLU(gate) * up; partial rows for the combine; y with the
// input rows RMS-normalised as they are staged (MG_YN)
enum { MG_Y = 0, MG_SILU = 1, MG_PART = 2, MG_YN = 3 };

// one member of a grouped GEMV: a single packed matrix, its input rows and
// its output rows
constexpr int MG_MAXGRP = 8;
struct MgGroup {
    const uint8_t *pk;
    const float *s;  // original per-row scales (fmt 2)
    const float *x;
    float *out;
    int64_t pk_stride, pk_scale_off;
    int nkb, O, I, kseg, nseg, wg0;
};

struct MgArgs {
    // packed copies (see coli_tensor_pack): matrix e of stack m at pk[m] + e*pk_stride
    const uint8_t *pk[2];
    const uint8_t *spk[2];  // shared expert's packed copies (MoE)
    int64_t pk_stride, pk_scale_off;
    int nkb, cbs;           // 128-input blocks per row; scale slots per block
    const float *s[2];      // original scales (fmt 2: per row)
    const float *ss[2];
    int64_t s_stride;
    int ng, gs;
    int O, I;
    const float *x;
    int64_t ldx;
    int moe;
    const int32_t *ids;
    int S, K, E;
    int x_by_pair;
    float *out;
    int Sy;
    int kseg;   // inputs per LDS segment (multiple of 128)
    int nseg;
    // MoE down with the top-k combine folded in (cnt != nullptr): arrival
    // counters per workgroup column, routing weights, final output [S][O]
    int *cnt;
    int ncnt;   // counters the gate/up launch clears
    const float *wts;
    float *yfin;
    int has_sh;
    // residual add (single-matrix MG_Y, and the combine): yres = radd + y,
    // same [S][O] layout as the output
    const float *radd;
    float *yres;
    // MG_YN: norm weights (NULL: 1), eps, and where workgroup (0, 0) writes
    // the normalised input rows [Sy][I]
    const float *nw;
    double neps;
    float *nxo;
    // grouped GEMV (ngrp > 0, MG_Y only): independent matrices with their own
    // inputs and outputs in one launch; workgroups from grp[g].wg0 on belong
    // to member g
    int ngrp;
    MgGroup grp[MG_MAXGRP];
};

// Partial rows that another workgroup sums are stored and loaded with
// device-scope relaxed atomics: those go to the point of coherence shared by
// all XCDs (their L2s are not coherent with each other for plain accesses), so
// no cache-wide write-back or invalidate is needed.
//
// What orders them (the combine tail below): the HIP memory model gives a
// relaxed atomic no ordering against another, so the order rests on the gfx9
// (CDNA4) ISA, not on the source-level model:
//   * agent-scope relaxed atomic loads and stores are emitted as global
//     loads / stores with the sc1 bit, which the L2 of each XCD serves
//     write-through / miss-always, i.e. at the memory-side coherence point;
//   * on gfx9 the vector memory counter (vmcnt) counts stores as well as
//     loads, and a store leaves it only once the memory side has acknowledged
//     it, so `s_waitcnt vmcnt(0)` (inside s_waitcnt(0)) returns after this
//     wave's partial rows are at the coherence point;
//   * the counter add is issued after that wait and the workgroup barrier,
//     and the last workgroup issues its sc1 loads only after the add has
//     returned -- so they observe every partial row counted before it.
// A release/acquire pair would say the same thing in the source model, but
// agent-scope release on gfx950 writes back the whole L2 of the XCD
// (measured: about five times this kernel's time); the tests check the
// combined rows against the oracle and their bit-repeatability.
__device__ __forceinline__ void store_coherent(float *p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// After a workgroup has stored its partial rows of one 16*TPW-row column, it
// counts itself in; the last of the column's gridDim.y workgroups writes
// out[s][row] = sum_k w[s][k] * yp[s*K+k][row] (+ yp[shared s][row]) for the
// column: k ascending, ids outside [0,E) skipped, one thread per output.
// Arrival order only decides which workgroup sums, never the order of the
// sum, so reruns are bit-identical.
template <int TPW>
__device__ __forceinline__ void mg_combine_tail(const MgArgs &a) {
    const int nth = blockDim.x;
    __shared__ int last;
    __builtin_amdgcn_s_waitcnt(0);  // this thread's partial stores have completed
    __syncthreads();
    if (threadIdx.x == 0)
        last = __hip_atomic_fetch_add(a.cnt + blockIdx.x, 1, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT) == (int)gridDim.y - 1;
    __syncthreads();
    if (!last)
        return;
    constexpr int ROWS = 16 * TPW;
    const int O = a.O, K = a.K;
    for (int idx = threadIdx.x; idx < ROWS * a.S; idx += nth) {
        const int s = idx / ROWS, row = blockIdx.x * ROWS + idx % ROWS;
        if (row >= O)
            continue;
        float acc = 0.f;
        for (int k0 = 0; k0 < K; k0 += 8) {
            float v[8], wk[8];
            bool ok[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int k = min(k0 + u, K - 1);
                const int64_t p = (int64_t)s * K + k;
                const int e = gload<int32_t>(a.ids + p);
                ok[u] = (k0 + u < K) && e >= 0 && e < a.E;
                wk[u] = gload<float>(a.wts + p);
                v[u] = load_coherent(a.out + p * O + row);
            }
#pragma unroll
            for (int u = 0; u < 8; ++u)
                acc = ok[u] ? fmaf(wk[u], v[u], acc) : acc;
        }
        if (a.has_sh)
            acc += load_coherent(a.out + ((int64_t)a.S * K + s) * O + row);
        a.yfin[(int64_t)s * O + row] = acc;
        if (a.yres != nullptr)
            a.yres[(int64_t)s * O + row] = a.radd[(int64_t)s * O + row] + acc;
    }
}

// launch shapes: KS wavefronts along the inputs of one 16-row tile, NW
// wavefronts per workgroup (NW / KS tiles); measured best for the decode MoE
// block: gate/up 2 x 4, down 1 x 4; for one 6144 x 6144 matrix 3 x 6 (two
// tiles share a workgroup's input staging: 7.7 us at S = 1 against 8.5 us
// for 4 x 4, 18.7 against 22.8 us at S = 4)
#ifndef COLI_MG_KS_GATEUP
#define COLI_MG_KS_GATEUP 2
#endif
#ifndef COLI_MG_NW_GATEUP
#define COLI_MG_NW_GATEUP 4
#endif
#ifndef COLI_MG_KS_DOWN
#define COLI_MG_KS_DOWN 1
#endif
#ifndef COLI_MG_NW_DOWN
#define COLI_MG_NW_DOWN 4
#endif
#ifndef COLI_MG_KS_DENSE
#define COLI_MG_KS_DENSE 3
#endif
#ifndef COLI_MG_NW_DENSE
#define COLI_MG_NW_DENSE 6
#endif
// longest input segment staged at once (a multiple of 512).  Rows longer
// than this restage their inputs once per segment; in exchange the LDS
// footprint stays small enough for several workgroups per compute unit
// (measured on the 75-layer stream with grouped projections: 64.5 us/layer
// at 8192 against 71.1 with o_proj's 16384 inputs in one segment; 4096
// slows the 6144-input matrices by a third)
#ifndef COLI_MG_KSEG_MAX
#define COLI_MG_KSEG_MAX 8192
#endif
// weight requests after the first input staging instead of before it
#ifndef COLI_MG_STAGE_FIRST
#define COLI_MG_STAGE_FIRST 0
#endif
// stacks of matrices with enough rows for at least COLI_MG_WIDE_MIN_WG
// workgroups of 16 * NW_WIDE / KS_WIDE rows take the wider shape (measured on
// a ring of 6144 x 6144 fmt-4 stacks of 8: 3 x 12 against 3 x 6 is 8.84 ->
// 5.65 us per matrix at S = 4 and 4.11 -> 3.96 at S = 1; one matrix per
// launch is slower with it: 96 workgroups for 256 compute units).  Not for
// 4 scale slots per block (gs 32), whose S >= 3 kernels would spill.
#ifndef COLI_MG_KS_WIDE
#define COLI_MG_KS_WIDE 3
#endif
#ifndef COLI_MG_NW_WIDE
#define COLI_MG_NW_WIDE 12
#endif
// ... and at S = 1 two wavefronts along the inputs x 4 tiles (8 wavefronts):
// stacked 6144 x 6144 fmt 4 g64 3.97 -> 3.58 us per matrix, 1024 x 2048
// stacks of 64 0.42 -> 0.27 us (2048 inputs are 4 quads: no uneven 3-way
// split); slower than 3 x 12 at S = 4 (5.61 -> 5.89 us)
#ifndef COLI_MG_KS_WIDE1
#define COLI_MG_KS_WIDE1 2
#endif
#ifndef COLI_MG_NW_WIDE1
#define COLI_MG_NW_WIDE1 8
#endif
static_assert(COLI_MG_NW_WIDE / COLI_MG_KS_WIDE == COLI_MG_NW_WIDE1 / COLI_MG_KS_WIDE1,
              "both wide shapes cover the same rows per workgroup");
#ifndef COLI_MG_WIDE_MIN_WG
#define COLI_MG_WIDE_MIN_WG 512
#endif
// quads of blocks in flight per wavefront in the dense GEMV and the MoE block
#ifndef COLI_MG_NBQ_DENSE
#define COLI_MG_NBQ_DENSE 2
#endif
#ifndef COLI_MG_NBQ_GATEUP
#define COLI_MG_NBQ_GATEUP 2
#endif
// gate/up with more workgroups than fit at once with two quads in flight
// (138 VGPRs + 64 AGPRs: 2 per compute unit, 512 on the chip): one quad in
// flight compiled for 4 wavefronts per SIMD (116 VGPRs), so e.g. the 9 pairs
// of 8 routed + 1 shared expert (576 workgroups) start together (measured on
// the 75-layer stream: 42.0 against 43.1 us per block; the 8-pair block keeps
// two quads: 35.0 against 35.4 us)
#ifndef COLI_MG_GATEUP_SLOTS
#define COLI_MG_GATEUP_SLOTS 512
#endif
// (down: one quad; measured 13.6 against 14.1 us per down launch with two,
// 16.5 with four, in the 8-of-256-expert block)
#ifndef COLI_MG_NBQ_DOWN
#define COLI_MG_NBQ_DOWN 1
#endif
// 128-input blocks requested together per wavefront: one quad, whose group
// scales sit together in the packed copy
constexpr int MG_NBK = 4;
// groups of 8 inputs per thread in one input staging step (with the input
// norm folded in: fewer, so the norm weights fit beside them)
constexpr int MG_UN = 4;
constexpr int MG_UN_YN = 2;
// buffer resource word 3 for raw (untyped) buffer loads; reads past
// num_records return zeros
constexpr int MG_RSRC_W3 = 0x00020000;
// load aux bits: nontemporal (streamed once)
constexpr int MG_AUX_NT = 2;

// LDS bytes of one k_mgemv launch (digits, zero block, reduction, factors)
__host__ __device__ constexpr int mg_nset(int CB, int NT) { return (CB * NT + 3) / 4; }

// NT input rows per tile (1..4); CB groups per 128-input block (1, 2, 4);
// KS wavefronts share one 16-row tile along the inputs; NMAT matrices (gate
// and up share their rows); NBQ quads of blocks in flight per wavefront.
// QB: bits per code in the packed copy -- 4 (fmt 2 / 4: nibbles, B bytes
// 16 v), 8 (fmt 1: int8 codes, B bytes v), 2 (fmt 3: 2-bit codes moved to the
// top of each byte, B bytes 64 v).
// Occupancy: 4 wavefronts per SIMD for gate/up with one quad in flight, and
// for one input row with the input norm folded in (122-128 VGPRs): at 3 per
// SIMD only one 6-wavefront workgroup fits a compute unit (its wavefronts go
// round-robin over the 4 SIMDs), so q_b's 512 workgroups ran in two rounds
// (measured: starts spread over 5.7 us).  The other shapes keep the
// compiler's choice.
template <int NT, int CB, bool GROUPED, int NMAT, int EPI, int KS, int NW, int NBQ = 2, int QB = 4>
__global__ __launch_bounds__(NW * 64, ((NMAT == 2 && NBQ == 1) || (EPI == MG_YN && NT == 1 && CB <= 2)) ? 4 : 1) void k_mgemv(MgArgs a) {
    static_assert(NW % KS == 0, "whole tiles per workgroup");
    static_assert(QB == 4 || ((QB == 8 || QB == 2) && !GROUPED && EPI == MG_Y), "code width");
    constexpr bool YOUT = EPI == MG_Y || EPI == MG_YN;
    constexpr int LB = 4 * QB;   // code bytes per lane and 128-input block
    constexpr int BLK = 64 * LB; // bytes per 16-row x 128-input tile block
    constexpr int TPW = NW / KS;
    constexpr int NTH = NW * 64;
    constexpr int NCOMBO = CB * NT;          // (group-in-block, input row) combinations
    constexpr int NSET = mg_nset(CB, NT);    // A-row sets of 4 combinations x 4 digits
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int tile_w = wave / KS, ks = wave % KS;
    int bx = blockIdx.x;
    if constexpr (YOUT) {
        if (a.ngrp > 0) {
            // this workgroup's member (constant indices only, so the
            // arguments stay in scalar registers)
            int g = 0;
#pragma unroll
            for (int i = 1; i < MG_MAXGRP; ++i) g = (i < a.ngrp && bx >= a.grp[i].wg0) ? i : g;
#pragma unroll
            for (int i = 0; i < MG_MAXGRP; ++i)
                if (i == g) {
                    const MgGroup &m = a.grp[i];
                    a.pk[0] = m.pk;
                    a.s[0] = m.s;
                    a.x = m.x;
                    a.ldx = m.I;
                    a.out = m.out;
                    a.pk_stride = m.pk_stride;
                    a.pk_scale_off = m.pk_scale_off;
                    a.nkb = m.nkb;
                    a.O = m.O;
                    a.I = m.I;
                    a.kseg = m.kseg;
                    a.nseg = m.nseg;
                    bx -= m.wg0;
                }
        }
    }
    const int I = a.I, O = a.O;
    const int KSEG = a.kseg;

    // LDS: digits [NT][4][KSEG] int8 | zero row [KSEG] | reduction [4][NMAT][NSET][16][16] f32 |
    //      exponent factors [NT][KSEG/128]
    char *xs = smem;
    char *zero = smem + (size_t)NT * 4 * KSEG;
    float *red = (float *)(zero + KSEG);
    float *xfac = red + NW * NMAT * NSET * 256;
    const int fstride = (KSEG / 128 + 3) & ~3;  // whole quads: one 16-byte read per batch

    // --- which matrix, which inputs ---------------------------------------
    const int64_t p = blockIdx.y;
    const uint8_t *pkm[NMAT];  // packed copy of the matrix
    const float *sc[NMAT];     // original per-row scales (fmt 2)
    int xrow[NT];
    int valid = 1;
    if (a.moe) {
        const bool shared = p >= (int64_t)a.S * a.K;
        int e = 0, s;
        if (!shared) {
            s = (int)(p / a.K);
            // scalar load: the scalar cache path does not queue behind this
            // CU's vector weight requests
            e = *(const __attribute__((address_space(4))) int32_t *)(a.ids + p);
            valid = (e >= 0 && e < a.E);
            if (!valid) e = 0;
        } else {
            s = (int)(p - (int64_t)a.S * a.K);
        }
#pragma unroll
        for (int m = 0; m < NMAT; ++m) {
            pkm[m] = (shared ? a.spk[m] : a.pk[m]) + (int64_t)e * a.pk_stride;
            sc[m] = (shared ? a.ss[m] : a.s[m]) + (int64_t)e * a.s_stride;
        }
        xrow[0] = a.x_by_pair ? (int)p : s;
    } else {
#pragma unroll
        for (int m = 0; m < NMAT; ++m) {
            pkm[m] = a.pk[m] + p * a.pk_stride;
            sc[m] = a.s[m] + p * a.s_stride;
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) xrow[t] = t;
    }
    // inputs of one staging step: UN groups of 8 per thread.  The first step's
    // loads are issued here, ahead of every weight request (loads complete in
    // order), so the staging overlaps the first weight batches.
    constexpr int UN = EPI == MG_YN ? MG_UN_YN : MG_UN;
    const int kpad = (I + 127) / 128 * 128;
    float xv[UN][8];
    auto stage_load = [&](int k0, int nb8, int base) {
#pragma unroll
        for (int u = 0; u < UN; ++u) {
            const int idx = min(base + u * NTH + tid, NT * nb8 - 1);
            const int t = idx / nb8, b8 = idx % nb8;
            const int k = k0 + b8 * 8;
            const float *xr = a.x + (int64_t)xrow[t] * a.ldx + min(k, I - 8);
            const f32x4 p0 = gload<f32x4>(xr), p1 = gload<f32x4>(xr + 4);
            const bool in = k < I;
            xv[u][0] = in ? p0.x : 0.f; xv[u][1] = in ? p0.y : 0.f;
            xv[u][2] = in ? p0.z : 0.f; xv[u][3] = in ? p0.w : 0.f;
            xv[u][4] = in ? p1.x : 0.f; xv[u][5] = in ? p1.y : 0.f;
            xv[u][6] = in ? p1.z : 0.f; xv[u][7] = in ? p1.w : 0.f;
        }
    };
    stage_load(0, min(KSEG, kpad) / 8, 0);
    // MG_YN: the norm weights of the same inputs, requested before the
    // weights so that the staging does not wait behind them (loads complete
    // in order)
    float gv[EPI == MG_YN ? UN : 1][8];
    if constexpr (EPI == MG_YN) {
        const int nb8 = min(KSEG, kpad) / 8;
#pragma unroll
        for (int u = 0; u < UN; ++u) {
            const int idx = min(u * NTH + tid, NT * nb8 - 1);
            const int k = min((idx % nb8) * 8, I - 8);
            f32x4 g0{1.f, 1.f, 1.f, 1.f}, g1{1.f, 1.f, 1.f, 1.f};
            if (a.nw != nullptr) {
                g0 = gload<f32x4>(a.nw + k);
                g1 = gload<f32x4>(a.nw + k + 4);
            }
            gv[u][0] = g0.x; gv[u][1] = g0.y; gv[u][2] = g0.z; gv[u][3] = g0.w;
            gv[u][4] = g1.x; gv[u][5] = g1.y; gv[u][6] = g1.z; gv[u][7] = g1.w;
        }
    }

    const int tile = bx * TPW + tile_w;
    const int row0 = tile * 16;
    if constexpr (EPI == MG_SILU) {
        if (a.cnt != nullptr && blockIdx.x == 0 && blockIdx.y == 0)
            for (int i = tid; i < a.ncnt; i += NTH)
                __hip_atomic_store(a.cnt + i, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (!valid) {
        if (EPI == MG_SILU && ks == 0 && lane < 16 && row0 + lane < O)
            a.out[p * O + row0 + lane] = 0.f;
        if constexpr (EPI == MG_PART) {
            if (a.cnt != nullptr)
                mg_combine_tail<TPW>(a);
        }
        return;
    }

    // --- lane roles ----------------------------------------------------------
    const int n = lane & 15, j = lane >> 4;                   // B: weight row, input quarter
    const int lg = (CB == 1) ? 0 : (CB == 2 ? (j >> 1) : j);  // group slot of the lane's inputs
    // A row n of set st: combination c = 4*st + n/4 = (slot c / NT, input row
    // c % NT), digit n % 4; inactive lanes read the zero row
    int aoff[NSET];
    // C rows 4j .. 4j+3: the digits of combination 4*st + j
    int ccb[NSET], ct[NSET];
#pragma unroll
    for (int st = 0; st < NSET; ++st) {
        const int c = st * 4 + (n >> 2);
        const bool act = c < NCOMBO && c / NT == lg;
        aoff[st] = act ? (((c % NT) * 4 + (n & 3)) * KSEG + 32 * j) : (int)(zero - xs);
        const int cr = min(st * 4 + j, NCOMBO - 1);
        ccb[st] = cr / NT;
        ct[st] = cr % NT;
    }
    // this lane's 16 bytes of every packed 1 KiB tile block, and its scale runs
    // (a wavefront past the last tile of a ragged column reads the last tile
    // again and writes nothing)
    const int tile_ld = min(tile, (O + 15) / 16 - 1);
    const int nkq = (a.nkb + 3) / 4;
    // codes and scales of the matrix as buffer resources; per lane a fixed
    // byte offset, per request a wave-uniform one
    __amdgpu_buffer_rsrc_t qrs[NMAT], srs[NMAT];
#pragma unroll
    for (int m = 0; m < NMAT; ++m) {
        qrs[m] = __builtin_amdgcn_make_buffer_rsrc((void *)pkm[m], (short)0, (int)a.pk_scale_off,
                                                   MG_RSRC_W3);
        srs[m] = __builtin_amdgcn_make_buffer_rsrc((void *)(pkm[m] + a.pk_scale_off), (short)0,
                                                   (int)(a.pk_stride - a.pk_scale_off), MG_RSRC_W3);
    }
    const int qoff = tile_ld * a.nkb * BLK + LB * lane;  // this lane's bytes of block 0
    int soff[NSET];  // row n's 4 scales (one per block) of its C rows' group slot, quad 0
#pragma unroll
    for (int st = 0; st < NSET; ++st) soff[st] = ((tile_ld * nkq * 16 + n) * CB + ccb[st]) * 16;

    float acc[NSET][NMAT][4];
#pragma unroll
    for (int st = 0; st < NSET; ++st)
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[st][m][q] = 0.f;

    // requests for one quad of 128-input blocks (codes and group scales);
    // NBQ batches rotate: each is re-requested as soon as it is computed
    struct Batch {
        u32x4 cw[MG_NBK][NMAT][QB == 8 ? 2 : 1];  // (QB 2: 8 bytes in .x, .y)
        f32x4 sq[NMAT][GROUPED ? NSET : 1];  // the quad's 4 scales of each set's group slot
    };
    Batch bq[NBQ];
    // kbg: first block of a quad (a multiple of 4); blocks past kb_last
    // re-read kb_last (requests are unconditional, so the compiler's load
    // counting sees straight-line code and waits for one batch at a time)
    auto load_batch = [&](Batch &bt, int kbg, int kb_last) {
#pragma unroll
        for (int i = 0; i < MG_NBK; ++i) {
            const int kglob = __builtin_amdgcn_readfirstlane(max(min(kbg + i, kb_last), 0));
#pragma unroll
            for (int m = 0; m < NMAT; ++m) {
                if constexpr (QB == 2) {
                    const u32x2 v = __builtin_bit_cast(
                        u32x2, __builtin_amdgcn_raw_buffer_load_b64(qrs[m], qoff, kglob * BLK, MG_AUX_NT));
                    bt.cw[i][m][0] = u32x4{v.x, v.y, 0u, 0u};
                } else {
#pragma unroll
                    for (int h = 0; h < (QB == 8 ? 2 : 1); ++h)
                        bt.cw[i][m][h] = __builtin_bit_cast(
                            u32x4, __builtin_amdgcn_raw_buffer_load_b128(qrs[m], qoff + 16 * h, kglob * BLK,
                                                                         MG_AUX_NT));
                }
            }
        }
        if constexpr (GROUPED) {
            const int sq0 = __builtin_amdgcn_readfirstlane((max(min(kbg, kb_last), 0) / 4) * 16 * CB * 16);
#pragma unroll
            for (int m = 0; m < NMAT; ++m)
#pragma unroll
                for (int st = 0; st < NSET; ++st)
                    bt.sq[m][st] = __builtin_bit_cast(
                        f32x4, __builtin_amdgcn_raw_buffer_load_b128(srs[m], soff[st], sq0, 0));
        }
    };
    // blocks [kb_beg, kb_end) of a segment of nkbs blocks for wavefront ks:
    // whole quads split evenly over the KS wavefronts
    auto share = [&](int nkbs, int &kb_beg, int &kb_end) {
        const int nq = (nkbs + 3) / 4;
        kb_beg = 4 * ((ks * nq) / KS);
        kb_end = min(4 * (((ks + 1) * nq) / KS), nkbs);
    };

    // ---- staging of one step of inputs as four int8 digits under one power
    //      of two per (input row, 128-input block): 16 consecutive threads
    //      own one block, each 8 inputs (one word of a 32-input quarter);
    //      digit row d holds, per quarter, the even inputs' bytes then the odd
    //      inputs' bytes
    auto stage_store = [&](int nb8, int base) {
        auto &v = xv;
#pragma unroll
        for (int u = 0; u < UN; ++u) {
            const int idx = base + u * NTH + tid;
            float mx = 0.f;
            bool bad = false;  // NaN or beyond 3e38 (fmaxf would drop a NaN)
#pragma unroll
            for (int w = 0; w < 8; ++w) {
                mx = fmaxf(mx, fabsf(v[u][w]));
                bad |= !(fabsf(v[u][w]) <= 3.0e38f);
            }
            if (bad)
                mx = __builtin_inff();
#pragma unroll
            for (int off = 8; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 16));
            // 2^e2 * max|x| in [2^29, 2^30) (tiny blocks: e2 <= 126 keeps
            // 2^-e2 normal); non-finite blocks give a NaN factor
            int e2 = 0;
            if (mx > 0.f && mx <= 3.0e38f) {
                (void)frexpf(mx, &e2);  // mx < 2^e2
                e2 = min(30 - e2, 126);
            }
            if (idx < NT * nb8) {
                const int t = idx / nb8, b8 = idx % nb8;
                uint32_t wd[8];
#pragma unroll
                for (int w = 0; w < 8; ++w)
                    wd[w] = (mx <= 3.0e38f) ? digits_of(ldexpf(v[u][w], e2)) : 0u;
                // byte b of the even word: input 2b of the 8; odd word: 2b+1
                uint32_t ev[4], od[4];
                transpose4(wd[0], wd[2], wd[4], wd[6], ev);
                transpose4(wd[1], wd[3], wd[5], wd[7], od);
                char *dst = xs + t * 4 * KSEG + (b8 >> 2) * 32 + (b8 & 3) * 4;
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    *reinterpret_cast<uint32_t *>(dst + d * KSEG) = ev[d];
                    *reinterpret_cast<uint32_t *>(dst + d * KSEG + 16) = od[d];
                }
                if ((b8 & 15) == 0)
                    xfac[t * fstride + b8 / 16] =
                        (mx <= 3.0e38f) ? ldexpf(1.0f, -e2) : __builtin_nanf("");
            }
        }
    };
    // one quad (segment blocks kb .. kb+3); blocks at or past kb_end add
    // nothing (zero factor), so every quad runs the same straight-line code
    auto compute_batch = [&](Batch &bt, int kb, int kb_end) {
        f32x4 fq[NSET];  // 2^-e of the quad's blocks for each set's input row
#pragma unroll
        for (int st = 0; st < NSET; ++st)
            fq[st] = *reinterpret_cast<const f32x4 *>(&xfac[ct[st] * fstride + kb]);
#pragma unroll
        for (int i = 0; i < MG_NBK; ++i) {
            const bool live = kb + i < kb_end;
            i32x4 a0[NSET], a1[NSET];
#pragma unroll
            for (int st = 0; st < NSET; ++st) {
                const char *ap = xs + aoff[st] + (kb + i) * 128;
                a0[st] = *reinterpret_cast<const i32x4 *>(ap);
                a1[st] = *reinterpret_cast<const i32x4 *>(ap + 16);
            }
#pragma unroll
            for (int m = 0; m < NMAT; ++m) {
                const u32x4 w = bt.cw[i][m][0];
                i32x4 be, bo;  // B operands: the lane's even inputs, its odd inputs
                if constexpr (QB == 4) {
                    be = i32x4{(int)even_x16(w.x), (int)even_x16(w.y), (int)even_x16(w.z),
                               (int)even_x16(w.w)};
                    bo = i32x4{(int)odd_x16(w.x), (int)odd_x16(w.y), (int)odd_x16(w.z),
                               (int)odd_x16(w.w)};
                } else if constexpr (QB == 8) {
                    be = __builtin_bit_cast(i32x4, w);
                    bo = __builtin_bit_cast(i32x4, bt.cw[i][m][QB == 8 ? 1 : 0]);
                } else {
                    be = i32x4{(int)((w.x << 6) & 0xC0C0C0C0u), (int)((w.x << 4) & 0xC0C0C0C0u),
                               (int)((w.x << 2) & 0xC0C0C0C0u), (int)(w.x & 0xC0C0C0C0u)};
                    bo = i32x4{(int)((w.y << 6) & 0xC0C0C0C0u), (int)((w.y << 4) & 0xC0C0C0C0u),
                               (int)((w.y << 2) & 0xC0C0C0C0u), (int)(w.y & 0xC0C0C0C0u)};
                }
#pragma unroll
                for (int st = 0; st < NSET; ++st) {
                    i32x4 c = {0, 0, 0, 0};
                    c = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0[st], be, c, 0, 0, 0);
                    c = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1[st], bo, c, 0, 0, 0);
                    const float g = live ? (GROUPED ? bt.sq[m][st][i] : 1.0f) * fq[st][i] : 0.0f;
#pragma unroll
                    for (int q = 0; q < 4; ++q) acc[st][m][q] = fmaf(g, (float)c[q], acc[st][m][q]);
                }
            }
        }
    };
    // MG_YN: the first staging step holds every input of the NT rows (the
    // host checks NT * nb8 <= UN * NTH and one segment); gv holds the norm
    // weights of the same inputs.  Each row's f64 sum
    // of squares (per thread, wavefront sums, wavefronts in order -- the same
    // in every workgroup of the launch), then x * inv * w in place;
    // workgroup (0, 0) also writes the normalised rows out.
    auto prenorm = [&](int nb8) {
        double ssq[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) ssq[t] = 0.0;
#pragma unroll
        for (int u = 0; u < UN; ++u) {
            const int idx = u * NTH + tid;
            if (idx < NT * nb8) {
                double s2 = 0.0;
#pragma unroll
                for (int w = 0; w < 8; ++w) s2 = fma((double)xv[u][w], (double)xv[u][w], s2);
                const int t = idx / nb8;
#pragma unroll
                for (int tt = 0; tt < NT; ++tt) ssq[tt] += (tt == t) ? s2 : 0.0;
            }
        }
        double *nred = reinterpret_cast<double *>(red);
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
            double v = ssq[tt];
#pragma unroll
            for (int m = 32; m >= 1; m >>= 1) v += rms_shfl_xor(v, m);
            if (lane == 0)
                nred[wave * NT + tt] = v;
        }
        __syncthreads();
        double inv[NT];
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
            double tot = 0.0;
            for (int w2 = 0; w2 < NW; ++w2) tot += nred[w2 * NT + tt];
            inv[tt] = 1.0 / sqrt(tot / (double)I + a.neps);
        }
        const bool wr = a.nxo != nullptr && blockIdx.x == 0 && blockIdx.y == 0;
#pragma unroll
        for (int u = 0; u < UN; ++u) {
            const int idx = u * NTH + tid;
            const int t = idx / nb8, k = (idx % nb8) * 8;
            if (idx < NT * nb8 && k < I) {  // I % 8 == 0: all 8 inputs are real
                double iv = inv[0];
#pragma unroll
                for (int tt = 1; tt < NT; ++tt) iv = (tt == t) ? inv[tt] : iv;
#pragma unroll
                for (int w = 0; w < 8; ++w) xv[u][w] = rms_apply(xv[u][w], iv, gv[u][w]);
                if (wr) {
                    float *o = a.nxo + (int64_t)t * I + k;
                    *reinterpret_cast<f32x4 *>(o) = f32x4{xv[u][0], xv[u][1], xv[u][2], xv[u][3]};
                    *reinterpret_cast<f32x4 *>(o + 4) = f32x4{xv[u][4], xv[u][5], xv[u][6], xv[u][7]};
                }
            }
        }
    };
    // LDS hand-over between the wavefronts (no wait on outstanding loads)
    auto lds_barrier = [&]() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); };

    // ---- segment 0: its first staging step's inputs are already requested;
    //      the first two weight batches go out before the staging uses them
    int kb_beg, kb_end;
    {
        const int klen = min(KSEG, kpad);
        const int nb8 = klen / 8;
        share(klen / 128, kb_beg, kb_end);
#if !COLI_MG_STAGE_FIRST
#pragma unroll
        for (int u = 0; u < NBQ; ++u) {
            load_batch(bq[u], kb_beg + u * MG_NBK, kb_end - 1);
            __builtin_amdgcn_sched_barrier(0);
        }
#endif
        if constexpr (EPI == MG_YN)
            prenorm(nb8);
        stage_store(nb8, 0);
        for (int base = UN * NTH; base < NT * nb8; base += UN * NTH) {
            stage_load(0, nb8, base);
            stage_store(nb8, base);
        }
        for (int idx = tid; idx < KSEG / 16; idx += NTH)
            reinterpret_cast<u32x4 *>(zero)[idx] = u32x4{0u, 0u, 0u, 0u};
        lds_barrier();
#if COLI_MG_STAGE_FIRST
#pragma unroll
        for (int u = 0; u < NBQ; ++u) {
            load_batch(bq[u], kb_beg + u * MG_NBK, kb_end - 1);
            __builtin_amdgcn_sched_barrier(0);
        }
#endif
    }
    for (int sgi = 0;;) {
        const int kg0 = sgi * (KSEG / 128);
        // all NBQ batches are in flight; each is re-requested as soon as it
        // is consumed
        const int nq = (kb_end - kb_beg + 3) / 4;
        int kb = kb_beg;
        // (scheduling fences keep each batch's use after the other's request,
        // so the wait before a batch never covers the batch behind it)
        for (int q = 0; q + NBQ < nq; q += NBQ, kb += NBQ * MG_NBK) {
#pragma unroll
            for (int u = 0; u < NBQ; ++u) {
                compute_batch(bq[u], kb + u * MG_NBK, kb_end);
                __builtin_amdgcn_sched_barrier(0);
                load_batch(bq[u], kg0 + kb + (u + NBQ) * MG_NBK, kg0 + kb_end - 1);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
#pragma unroll
        for (int u = 0; u < NBQ; ++u) {
            compute_batch(bq[u], kb + u * MG_NBK, kb_end);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (++sgi >= a.nseg)
            break;
        // ---- next segment: restage the inputs, then its first two batches
        const int k0 = sgi * KSEG;
        const int klen = min(KSEG, kpad - k0);
        const int nb8 = klen / 8;
        lds_barrier();  // every wavefront is done with the previous digits
        for (int base = 0; base < NT * nb8; base += UN * NTH) {
            stage_load(k0, nb8, base);
            stage_store(nb8, base);
        }
        lds_barrier();
        share(klen / 128, kb_beg, kb_end);
#pragma unroll
        for (int u = 0; u < NBQ; ++u) {
            load_batch(bq[u], k0 / 128 + kb_beg + u * MG_NBK, k0 / 128 + kb_end - 1);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // --- reduce: KS wavefronts x group slots x digits -> one value per (row, input row)
#pragma unroll
    for (int st = 0; st < NSET; ++st)
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                red[(((wave * NMAT + m) * NSET + st) * 16 + 4 * j + q) * 16 + n] = acc[st][m][q];
    __syncthreads();
    const int t = lane >> 4, nn = lane & 15;
    const int row = row0 + nn;
    if (ks == 0 && lane < 16 * NT && row < O) {
        float v[NMAT];
#pragma unroll
        for (int m = 0; m < NMAT; ++m) {
            float sum = 0.f;
            for (int w2 = 0; w2 < KS; ++w2)
#pragma unroll
                for (int cb = 0; cb < CB; ++cb) {
                    const int c = cb * NT + t;
                    const float *rr =
                        &red[(((tile_w * KS + w2) * NMAT + m) * NSET + c / 4) * 256 + (c % 4) * 64 + nn];
                    sum += ((rr[0] + rr[16] * 0x1p8f) + rr[32] * 0x1p16f) + rr[48] * 0x1p24f;
                }
            // the weights entered as 16 v (int4), v (int8) or 64 v (int2)
            sum *= (QB == 4) ? 0.0625f : (QB == 2 ? 0.015625f : 1.0f);
            if (!GROUPED)
                sum *= gload<float>(sc[m] + row);
            v[m] = sum;
        }
        if constexpr (EPI == MG_SILU) {
            const float g = v[0], u = v[NMAT - 1];
            a.out[p * O + row] = (g / (1.0f + expf(-g))) * u;
        } else if constexpr (EPI == MG_PART) {
            if (a.cnt != nullptr)
                store_coherent(a.out + p * O + row, v[0]);
            else
                a.out[p * O + row] = v[0];
        } else {
            const int64_t oi = (p * a.Sy + t) * O + row;
            a.out[oi] = v[0];
            if (a.yres != nullptr)
                a.yres[oi] = a.radd[oi] + v[0];
        }
    }
    if constexpr (EPI == MG_PART) {
        if (a.cnt != nullptr)
            mg_combine_tail<TPW>(a);
    }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------

// Which layouts have a packed form: int4 codes in whole 32-input packets, and
// for fmt 4 a group size of 32, 64 or a multiple of 128.
static bool packable(int fmt, int I, int gs) {
    if (fmt < 1 || fmt > 4)
        return false;
    if (I % 32 != 0 || I < 32)
        return false;
    if (fmt == 4 && !(gs == 32 || gs == 64 || (gs > 0 && gs % 128 == 0)))
        return false;
    return true;
}

static int cbs_of(int fmt, int gs) {  // scale slots per 128-input block
    if (fmt != 4 || gs % 128 == 0) return 1;
    return gs == 64 ? 2 : 4;
}

struct PackGeom {
    int rt, nkb, cbs;
    int64_t code_bytes, scale_off, stride;
};

// code bytes of one lane in one 128-input block of a packed tile (32 inputs)
static int lane_bytes(int fmt) { return fmt == 1 ? 32 : (fmt == 3 ? 8 : 16); }

static PackGeom pack_geom(int fmt, int O, int I, int gs) {
    PackGeom g;
    g.rt = (O + 15) / 16;
    g.nkb = (I + 127) / 128;
    g.cbs = cbs_of(fmt, gs);
    g.code_bytes = (int64_t)g.rt * g.nkb * 64 * lane_bytes(fmt);
    g.scale_off = g.code_bytes;
    const int64_t nkq = (g.nkb + 3) / 4;
    const int64_t sb = (fmt == 4) ? (int64_t)g.rt * nkq * 16 * 4 * g.cbs * 4 : 0;
    g.stride = (g.code_bytes + sb + 255) / 256 * 256;
    return g;
}

size_t packed_bytes(int fmt, int n, int O, int I, int gs) {
    if (n < 1 || O < 1 || !packable(fmt, I, gs))
        return 0;
    return (size_t)pack_geom(fmt, O, I, gs).stride * n;
}

// packed codes: tile block (e, rt, kb) = 1 KiB, lane l = 16*j + r holds row
// 16*rt + r, inputs kb*128 + 32*j .. +32 (16 bytes) as two's-complement
// nibbles q - 8 (code XOR 8); padding 0
__global__ __launch_bounds__(256) void k_pack_codes(const uint8_t *__restrict__ q, int64_t rb,
                                                    int64_t q_stride, int n, int O, int I, int rt,
                                                    int nkb, int64_t stride,
                                                    uint8_t *__restrict__ pk) {
    const int64_t total = (int64_t)n * rt * nkb * 64;
    for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < total;
         c += (int64_t)gridDim.x * 256) {
        const int l = (int)(c % 64);
        const int64_t blk = c / 64;
        const int kb = (int)(blk % nkb);
        const int64_t t2 = blk / nkb;
        const int tr = (int)(t2 % rt);
        const int e = (int)(t2 / rt);
        const int r = l & 15, j = l >> 4;
        const int row = tr * 16 + r;
        const int k = kb * 128 + 32 * j;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (row < O && k < I) {
            const u32x4 c = gload<u32x4>(q + (int64_t)e * q_stride + (int64_t)row * rb + k / 2);
            v = u32x4{c.x ^ 0x88888888u, c.y ^ 0x88888888u, c.z ^ 0x88888888u, c.w ^ 0x88888888u};
        }
        *reinterpret_cast<u32x4 *>(pk + (int64_t)e * stride + ((int64_t)tr * nkb + kb) * 1024 + 16 * l) = v;
    }
}

// packed fmt-1 / fmt-3 codes: tile block (e, rt, kb) of 64 lanes x LB bytes,
// lane l = 16*j + r holding row 16*rt + r, inputs kb*128 + 32*j .. +32, ordered
// for the two B operands (even inputs, odd inputs): fmt 1 (LB 32) the 16
// even inputs' int8 codes, then the 16 odd ones'; fmt 3 (LB 8) two words, word
// 0 for the even inputs, word 1 for the odd ones, whose byte b bits 2k, 2k+1
// hold v = code - 2 (two's complement) of the input at position 4k + b of
// that list.  Padding 0.
__global__ __launch_bounds__(256) void k_pack_codes_row(int fmt, const uint8_t *__restrict__ q,
                                                        int64_t rb, int64_t q_stride, int n, int O,
                                                        int I, int rt, int nkb, int64_t stride,
                                                        uint8_t *__restrict__ pk) {
    const int LB = fmt == 1 ? 32 : 8;
    const int64_t total = (int64_t)n * rt * nkb * 64;
    for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < total;
         c += (int64_t)gridDim.x * 256) {
        const int l = (int)(c % 64);
        const int64_t blk = c / 64;
        const int kb = (int)(blk % nkb);
        const int64_t t2 = blk / nkb;
        const int tr = (int)(t2 % rt);
        const int e = (int)(t2 / rt);
        const int r = l & 15, j = l >> 4;
        const int row = tr * 16 + r;
        const int k0 = kb * 128 + 32 * j;
        uint8_t out[32];
        for (int i = 0; i < 32; ++i) out[i] = 0;
        if (row < O) {
            const uint8_t *src = q + (int64_t)e * q_stride + (int64_t)row * rb;
            for (int i = 0; i < 32; ++i) {
                const int k = k0 + i;
                if (k >= I)
                    break;
                const int half = i & 1, m = i >> 1;  // odd / even list, position in it
                if (fmt == 1) {
                    out[half * 16 + m] = src[k];
                } else {
                    const int v = ((src[k >> 2] >> (2 * (k & 3))) & 3) - 2;
                    out[half * 4 + (m & 3)] |= (uint8_t)((v & 3) << (2 * (m >> 2)));
                }
            }
        }
        uint8_t *dst = pk + (int64_t)e * stride + ((int64_t)tr * nkb + kb) * 64 * LB + (int64_t)LB * l;
        for (int i = 0; i < LB; ++i) dst[i] = out[i];
    }
}

// packed fmt-4 scales: for (e, rt, quad kq of 4 blocks, row r, group slot cb)
// a run of 4 floats, block i: s[16*rt + r][group of slot cb of block 4*kq + i];
// one lane reads the run of its row and slot for a whole quad.  Padding 0.
__global__ __launch_bounds__(256) void k_pack_scales(const float *__restrict__ s, int64_t s_stride,
                                                     int ng, int gs, int n, int O, int rt, int nkb,
                                                     int cbs, int64_t stride, int64_t scale_off,
                                                     uint8_t *__restrict__ pk) {
    const int nkq = (nkb + 3) / 4;
    const int64_t total = (int64_t)n * rt * nkq * 16 * 4 * cbs;
    for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < total;
         c += (int64_t)gridDim.x * 256) {
        int64_t t = c;
        const int i = (int)(t % 4);
        t /= 4;
        const int cb = (int)(t % cbs);
        t /= cbs;
        const int r = (int)(t % 16);
        t /= 16;
        const int kq = (int)(t % nkq);
        t /= nkq;
        const int tr = (int)(t % rt);
        const int e = (int)(t / rt);
        const int row = tr * 16 + r;
        const int kb = 4 * kq + i;
        const int g = (cbs == 1) ? (kb * 128) / gs : kb * cbs + cb;
        float v = 0.f;
        if (row < O && kb < nkb && g < ng)
            v = gload<float>(s + (int64_t)e * s_stride + (int64_t)row * ng + g);
        float *dst = (float *)(pk + (int64_t)e * stride + scale_off);
        dst[c - (int64_t)e * ((int64_t)rt * nkq * 16 * 4 * cbs)] = v;
    }
}

int launch_pack(coli_qtensor *t, void *packed, hipStream_t st) {
    const PackGeom g = pack_geom(t->fmt, t->O, t->I, t->gs);
    {
        const int64_t total = (int64_t)t->n * g.rt * g.nkb * 64;
        const unsigned blocks = (unsigned)std::min<int64_t>((total + 255) / 256, 65536);
        ProfScope ps("pack", st);
        if (t->fmt == 1 || t->fmt == 3)
            hipLaunchKernelGGL(k_pack_codes_row, dim3(blocks), dim3(256), 0, st, t->fmt,
                               (const uint8_t *)t->q, t->row_bytes, t->q_stride, t->n, t->O, t->I,
                               g.rt, g.nkb, g.stride, (uint8_t *)packed);
        else
            hipLaunchKernelGGL(k_pack_codes, dim3(blocks), dim3(256), 0, st, (const uint8_t *)t->q,
                               t->row_bytes, t->q_stride, t->n, t->O, t->I, g.rt, g.nkb, g.stride,
                               (uint8_t *)packed);
        int rc = after_launch("pack");
        if (rc != COLI_OK) return rc;
    }
    if (t->fmt == 4) {
        const int64_t total = (int64_t)t->n * g.rt * ((g.nkb + 3) / 4) * 16 * 4 * g.cbs;
        const unsigned blocks = (unsigned)std::min<int64_t>((total + 255) / 256, 65536);
        ProfScope ps("pack", st);
        hipLaunchKernelGGL(k_pack_scales, dim3(blocks), dim3(256), 0, st, t->s, t->s_stride, t->ng,
                           t->gs, t->n, t->O, g.rt, g.nkb, g.cbs, g.stride, g.scale_off,
                           (uint8_t *)packed);
        int rc = after_launch("pack");
        if (rc != COLI_OK) return rc;
    }
    t->pk = packed;
    t->pk_stride = g.stride;
    t->pk_scale_off = g.scale_off;
    t->flags |= QF_PACKED;
    return COLI_OK;
}

// The matrix-core GEMV runs on tensors that carry a packed copy.
// (Buffer resources address one packed matrix with 32-bit byte offsets.)
bool mgemv_ok(const coli_qtensor *W) {
    return (W->flags & QF_PACKED) && W->pk != nullptr && packable(W->fmt, W->I, W->gs) &&
           W->pk_stride < ((int64_t)1 << 31);
}

// the int4 formats, which the MoE block and prefill kernels take
bool mgemv_int4_ok(const coli_qtensor *W) {
    return mgemv_ok(W) && (W->fmt == 2 || W->fmt == 4);
}

static int cb_of(const coli_qtensor *W) { return cbs_of(W->fmt, W->gs); }

static void plan_lds(int NT, int CB, int NMAT, int NW, int I, int &kseg, int &nseg, size_t &bytes) {
    const int kpad = (I + 127) / 128 * 128;
    // inputs per segment: 4 digit bytes each + zero row, within 112 KiB of
    // LDS (one segment covers 6144 inputs up to S = 4: restaging between
    // segments stalls the weight stream; 12.9 against 19.2 us at S = 4)
    const int cap = (112 * 1024) / (NT * 4 + 1);
    kseg = std::min(cap / 512 * 512, COLI_MG_KSEG_MAX);
    if (kseg > kpad) kseg = kpad;
    nseg = (kpad + kseg - 1) / kseg;  // segments hold whole quads (kseg % 512 == 0)
    bytes = (size_t)NT * 4 * kseg + kseg + (size_t)NW * NMAT * mg_nset(CB, NT) * 256 * 4 +
            (size_t)NT * ((kseg / 128 + 3) & ~3) * 4 + 64;
}

static MgArgs mg_args_for(const coli_qtensor *W) {
    MgArgs a;
    memset(&a, 0, sizeof a);
    a.pk[0] = a.pk[1] = (const uint8_t *)W->pk;
    a.spk[0] = a.spk[1] = (const uint8_t *)W->pk;
    a.pk_stride = W->pk_stride;
    a.pk_scale_off = W->pk_scale_off;
    a.nkb = (W->I + 127) / 128;
    a.cbs = cbs_of(W->fmt, W->gs);
    a.s[0] = a.s[1] = W->s;
    a.ss[0] = a.ss[1] = W->s;
    a.s_stride = W->s_stride;
    a.ng = W->ng;
    a.gs = W->gs > 0 ? W->gs : 1;
    a.O = W->O;
    a.I = W->I;
    return a;
}

template <int NT, int CB, bool GROUPED, int NMAT, int EPI, int KS, int NW, int NBQ, int QB = 4>
static void mg_launch(MgArgs a, int groups, hipStream_t st, const ProfScope &ps) {
    size_t lds;
    plan_lds(NT, CB, NMAT, NW, a.I, a.kseg, a.nseg, lds);
    constexpr int TPW = NW / KS;
    const int tiles = (a.O + 15) / 16;
    const dim3 grid((unsigned)((tiles + TPW - 1) / TPW), (unsigned)groups);
    hipExtLaunchKernelGGL((k_mgemv<NT, CB, GROUPED, NMAT, EPI, KS, NW, NBQ, QB>), grid, dim3(NW * 64),
                          (uint32_t)lds, st, ps.start(), ps.stop(), 0, a);
}

template <int NT, bool GROUPED, int NMAT, int EPI, int KS, int NW, int NBQ = 2>
static int mg_dispatch_cb(int cb, const MgArgs &a, int groups, hipStream_t st, const ProfScope &ps) {
    switch (cb) {
    case 1: mg_launch<NT, 1, GROUPED, NMAT, EPI, KS, NW, NBQ>(a, groups, st, ps); return 1;
    case 2: mg_launch<NT, 2, GROUPED, NMAT, EPI, KS, NW, NBQ>(a, groups, st, ps); return 1;
    default: mg_launch<NT, 4, GROUPED, NMAT, EPI, KS, NW, NBQ>(a, groups, st, ps); return 1;
    }
}

// Whether an input RMSNorm folds into a launch of NW-wavefront workgroups on
// the int4 formats: the S rows fit one staging step of one segment.
static bool prenorm_fits(const InNorm *nrm, const coli_qtensor *W, int S, int NW) {
    if (!nrm || !nrm->xn || (uintptr_t)nrm->xn % 16 != 0 || (uintptr_t)nrm->w % 16 != 0 ||
        W->I % 8 != 0 || !(W->fmt == 2 || W->fmt == 4) || !(nrm->eps >= 0.0))
        return false;
    int kseg, nseg;
    size_t lds;
    plan_lds(S, cb_of(W), 1, NW, W->I, kseg, nseg, lds);
    const int kpad = (W->I + 127) / 128 * 128;
    return nseg == 1 && (int64_t)S * (std::min(kseg, kpad) / 8) <= (int64_t)MG_UN_YN * NW * 64;
}

// Dense GEMV y[e][t][o] for S <= 4 input rows.  Returns 0 when the layout or
// (S, gs) combination is not taken (caller falls back to the VALU kernels).
// radd / ysum: also ysum = radd + y (one matrix); nrm: the input rows
// RMS-normalised first (int4 formats, rows that fit one staging step).
int launch_mgemv(const coli_qtensor *W, const float *x, float *y, int S, hipStream_t st,
                 const float *radd, float *ysum, const InNorm *nrm) {
    if (!mgemv_ok(W) || S < 1 || S > 4)
        return 0;
    if ((radd != nullptr) != (ysum != nullptr) || (ysum != nullptr && W->n != 1))
        return 0;
    const int cb = cb_of(W);
    MgArgs a = mg_args_for(W);
    a.x = x;
    a.ldx = W->I;
    a.out = y;
    a.Sy = S;
    a.radd = radd;
    a.yres = ysum;
    const bool g = W->fmt == 4;
    if (nrm != nullptr) {
        if (!prenorm_fits(nrm, W, S, COLI_MG_NW_DENSE))
            return 0;
        a.nw = nrm->w;
        a.neps = nrm->eps;
        a.nxo = nrm->xn;
        ProfScope ps("mgemv", st, true);
        switch (S) {
#define MG_NCASE(NTV)                                                                               \
    case NTV:                                                                                       \
        if (g) mg_dispatch_cb<NTV, true, 1, MG_YN, COLI_MG_KS_DENSE, COLI_MG_NW_DENSE, COLI_MG_NBQ_DENSE>(cb, a, W->n, st, ps); \
        else mg_dispatch_cb<NTV, false, 1, MG_YN, COLI_MG_KS_DENSE, COLI_MG_NW_DENSE, COLI_MG_NBQ_DENSE>(cb, a, W->n, st, ps); \
        break;
        MG_NCASE(1) MG_NCASE(2) MG_NCASE(3) default: MG_NCASE(4)
#undef MG_NCASE
        }
        return after_launch("mgemv") == COLI_OK ? 1 : -1;
    }
    constexpr int ROWS_WIDE = 16 * (COLI_MG_NW_WIDE / COLI_MG_KS_WIDE);
    const bool wide = cb <= 2 && (int64_t)W->n * ((W->O + ROWS_WIDE - 1) / ROWS_WIDE) >= COLI_MG_WIDE_MIN_WG;
    ProfScope ps("mgemv", st, true);
    int ok;
#define MG_KSW(NTV) ((NTV) == 1 ? COLI_MG_KS_WIDE1 : COLI_MG_KS_WIDE)
#define MG_NWW(NTV) ((NTV) == 1 ? COLI_MG_NW_WIDE1 : COLI_MG_NW_WIDE)
#define MG_ROWFMT(NTV, QBV)                                                                   \
    (wide ? (mg_launch<NTV, 1, false, 1, MG_Y, MG_KSW(NTV), MG_NWW(NTV), COLI_MG_NBQ_DENSE, QBV>(a, W->n, st, ps), 1) \
          : (mg_launch<NTV, 1, false, 1, MG_Y, COLI_MG_KS_DENSE, COLI_MG_NW_DENSE, COLI_MG_NBQ_DENSE, QBV>(a, W->n, st, ps), 1))
#define MG_CASE(NTV)                                                                          \
    if (W->fmt == 1)                                                                          \
        ok = MG_ROWFMT(NTV, 8);                                                               \
    else if (W->fmt == 3)                                                                     \
        ok = MG_ROWFMT(NTV, 2);                                                               \
    else if (wide)                                                                            \
        ok = g ? mg_dispatch_cb<NTV, true, 1, MG_Y, MG_KSW(NTV), MG_NWW(NTV), COLI_MG_NBQ_DENSE>(cb, a, W->n, st, ps) \
               : mg_dispatch_cb<NTV, false, 1, MG_Y, MG_KSW(NTV), MG_NWW(NTV), COLI_MG_NBQ_DENSE>(cb, a, W->n, st, ps); \
    else                                                                                      \
        ok = g ? mg_dispatch_cb<NTV, true, 1, MG_Y, COLI_MG_KS_DENSE, COLI_MG_NW_DENSE, COLI_MG_NBQ_DENSE>(cb, a, W->n, st, ps) \
               : mg_dispatch_cb<NTV, false, 1, MG_Y, COLI_MG_KS_DENSE, COLI_MG_NW_DENSE, COLI_MG_NBQ_DENSE>(cb, a, W->n, st, ps)
    switch (S) {
    case 1: MG_CASE(1); break;
    case 2: MG_CASE(2); break;
    case 3: MG_CASE(3); break;
    default: MG_CASE(4); break;
    }
#undef MG_CASE
#undef MG_ROWFMT
#undef MG_KSW
#undef MG_NWW
    if (!ok)
        return 0;
    return after_launch("mgemv") == COLI_OK ? 1 : -1;
}

// launch shape of the grouped GEMV (75-layer stream with the four projections
// grouped: 3 x 6 64.0-64.7 us per layer, 2 x 4 64.9-65.2, 2 x 8 66.8-68.2)
#ifndef COLI_MG_KS_GROUP
#define COLI_MG_KS_GROUP COLI_MG_KS_DENSE
#endif
#ifndef COLI_MG_NW_GROUP
#define COLI_MG_NW_GROUP COLI_MG_NW_DENSE
#endif

// Grouped GEMV: n independent single matrices (same format class, each with a
// packed copy) with their own inputs x[g] [S][I_g] and outputs y[g] [S][O_g],
// one launch.  Returns 0 when the group is not taken (the caller then runs
// the members one by one).
int launch_mgemv_group(int n, const coli_qtensor *const *W, const float *const *x,
                       float *const *y, int S, hipStream_t st, const InNorm *nrm) {
    if (n < 1 || n > MG_MAXGRP || S < 1 || S > 4)
        return 0;
    for (int g = 0; g < n; ++g)
        if (!mgemv_ok(W[g]) || W[g]->n != 1 || W[g]->fmt != W[0]->fmt || cb_of(W[g]) != cb_of(W[0]))
            return 0;
    // an input norm: every member takes the same rows (normalised in each
    // workgroup; the first workgroup writes them out)
    if (nrm != nullptr)
        for (int g = 0; g < n; ++g)
            if (x[g] != x[0] || W[g]->I != W[0]->I || !prenorm_fits(nrm, W[g], S, COLI_MG_NW_GROUP))
                return 0;
    constexpr int TPW = COLI_MG_NW_GROUP / COLI_MG_KS_GROUP;
    MgArgs a = mg_args_for(W[0]);
    a.Sy = S;
    a.ngrp = n;
    if (nrm != nullptr) {
        a.nw = nrm->w;
        a.neps = nrm->eps;
        a.nxo = nrm->xn;
    }
    size_t lds_max = 0;
    int wg = 0;
    // members with the longest rows first: their workgroups run longest, so
    // they start at once and the short ones fill the remaining compute units
    int order[MG_MAXGRP];
    for (int g = 0; g < n; ++g) order[g] = g;
    std::stable_sort(order, order + n, [&](int u, int v) { return W[u]->I > W[v]->I; });
    for (int k = 0; k < n; ++k) {
        const int g = order[k];
        MgGroup &m = a.grp[k];
        m.pk = (const uint8_t *)W[g]->pk;
        m.s = W[g]->s;
        m.x = x[g];
        m.out = y[g];
        m.pk_stride = W[g]->pk_stride;
        m.pk_scale_off = W[g]->pk_scale_off;
        m.nkb = (W[g]->I + 127) / 128;
        m.O = W[g]->O;
        m.I = W[g]->I;
        size_t lds;
        plan_lds(S, cb_of(W[g]), 1, COLI_MG_NW_GROUP, m.I, m.kseg, m.nseg, lds);
        lds_max = std::max(lds_max, lds);
        m.wg0 = wg;
        wg += ((m.O + 15) / 16 + TPW - 1) / TPW;
    }
    const int cb = cb_of(W[0]);
    const bool grouped = W[0]->fmt == 4;
    ProfScope ps("mgemv_group", st, true);
    int ok = 1;
#define MG_G(NTV, CBV)                                                                             \
    if (nrm) hipExtLaunchKernelGGL((k_mgemv<NTV, CBV, true, 1, MG_YN, COLI_MG_KS_GROUP, COLI_MG_NW_GROUP, \
                                   COLI_MG_NBQ_DENSE>),                                            \
                          dim3((unsigned)wg, 1u), dim3(COLI_MG_NW_GROUP * 64), (uint32_t)lds_max, st, \
                          ps.start(), ps.stop(), 0, a);                                            \
    else hipExtLaunchKernelGGL((k_mgemv<NTV, CBV, true, 1, MG_Y, COLI_MG_KS_GROUP, COLI_MG_NW_GROUP, \
                                   COLI_MG_NBQ_DENSE>),                                            \
                          dim3((unsigned)wg, 1u), dim3(COLI_MG_NW_GROUP * 64), (uint32_t)lds_max, st, \
                          ps.start(), ps.stop(), 0, a)
#define MG_R(NTV)                                                                                  \
    if (nrm) hipExtLaunchKernelGGL((k_mgemv<NTV, 1, false, 1, MG_YN, COLI_MG_KS_GROUP, COLI_MG_NW_GROUP, \
                                   COLI_MG_NBQ_DENSE>),                                            \
                          dim3((unsigned)wg, 1u), dim3(COLI_MG_NW_GROUP * 64), (uint32_t)lds_max, st, \
                          ps.start(), ps.stop(), 0, a);                                            \
    else hipExtLaunchKernelGGL((k_mgemv<NTV, 1, false, 1, MG_Y, COLI_MG_KS_GROUP, COLI_MG_NW_GROUP, \
                                   COLI_MG_NBQ_DENSE>),                                            \
                          dim3((unsigned)wg, 1u), dim3(COLI_MG_NW_GROUP * 64), (uint32_t)lds_max, st, \
                          ps.start(), ps.stop(), 0, a)
#define MG_Q(NTV, QBV)                                                                             \
    hipExtLaunchKernelGGL((k_mgemv<NTV, 1, false, 1, MG_Y, COLI_MG_KS_GROUP, COLI_MG_NW_GROUP,     \
                                   COLI_MG_NBQ_DENSE, QBV>),                                       \
                          dim3((unsigned)wg, 1u), dim3(COLI_MG_NW_GROUP * 64), (uint32_t)lds_max, st, \
                          ps.start(), ps.stop(), 0, a)
#define MG_NT(NTV)                                   \
    if (W[0]->fmt == 1) { MG_Q(NTV, 8); }            \
    else if (W[0]->fmt == 3) { MG_Q(NTV, 2); }       \
    else if (!grouped) { MG_R(NTV); }                \
    else if (cb == 1) { MG_G(NTV, 1); }              \
    else if (cb == 2) { MG_G(NTV, 2); }              \
    else { MG_G(NTV, 4); }
    switch (S) {
    case 1: MG_NT(1); break;
    case 2: MG_NT(2); break;
    case 3: MG_NT(3); break;
    default: MG_NT(4); break;
    }
#undef MG_NT
#undef MG_Q
#undef MG_R
#undef MG_G
    if (!ok)
        return 0;
    return after_launch("mgemv_group") == COLI_OK ? 1 : -1;
}

// Decode MoE block on the matrix cores: gate/up + SiLU (dual), then down per
// pair with the weighted top-k combine done by the last workgroup of each row
// column (cnt: one arrival counter per column, cleared by the gate/up launch).
// Returns 1 when the whole block was launched, 0 when not taken.
int launch_mgemv_moe(const MoeArgs &m, float *h, float *yp, int *cnt) {
    const coli_qtensor *all[6] = {m.gate, m.up, m.down, m.sg, m.su, m.sd};
    for (const coli_qtensor *t : all)
        if (t && !mgemv_int4_ok(t))
            return 0;
    const int cb = cb_of(m.gate);
    const bool g = m.gate->fmt == 4;
    const bool has_sh = m.sg != nullptr;
    const int P = m.S * m.K + (has_sh ? m.S : 0);
    {
        MgArgs a = mg_args_for(m.gate);
        a.pk[1] = (const uint8_t *)m.up->pk;
        a.s[1] = m.up->s;
        a.spk[0] = has_sh ? (const uint8_t *)m.sg->pk : a.pk[0];
        a.ss[0] = has_sh ? m.sg->s : a.s[0];
        a.spk[1] = has_sh ? (const uint8_t *)m.su->pk : a.pk[1];
        a.ss[1] = has_sh ? m.su->s : a.s[1];
        a.x = m.x;
        a.ldx = m.D;
        a.moe = 1;
        a.ids = m.ids;
        a.S = m.S; a.K = m.K; a.E = m.E;
        a.out = h;
        if (m.out != nullptr && m.down != nullptr) {
            a.cnt = cnt;
            a.ncnt = (m.D + 15) / 16;
        }
        ProfScope ps("moe_gateup_decode", m.st, true);
        constexpr int TPWG = COLI_MG_NW_GATEUP / COLI_MG_KS_GATEUP;
        const int64_t wgs = (int64_t)P * (((m.F + 15) / 16 + TPWG - 1) / TPWG);
        const bool many = wgs > COLI_MG_GATEUP_SLOTS;
        if (!(many ? (g ? mg_dispatch_cb<1, true, 2, MG_SILU, COLI_MG_KS_GATEUP, COLI_MG_NW_GATEUP, 1>(cb, a, P, m.st, ps)
                        : mg_dispatch_cb<1, false, 2, MG_SILU, COLI_MG_KS_GATEUP, COLI_MG_NW_GATEUP, 1>(cb, a, P, m.st, ps))
                   : (g ? mg_dispatch_cb<1, true, 2, MG_SILU, COLI_MG_KS_GATEUP, COLI_MG_NW_GATEUP, COLI_MG_NBQ_GATEUP>(cb, a, P, m.st, ps)
                        : mg_dispatch_cb<1, false, 2, MG_SILU, COLI_MG_KS_GATEUP, COLI_MG_NW_GATEUP, COLI_MG_NBQ_GATEUP>(cb, a, P, m.st, ps))))
            return 0;
        int rc = after_launch("moe_gateup_decode");
        if (rc != COLI_OK) return rc;
    }
    if (m.out == nullptr || m.down == nullptr)
        return 1;
    {
        MgArgs a = mg_args_for(m.down);
        a.spk[0] = a.spk[1] = has_sh ? (const uint8_t *)m.sd->pk : a.pk[0];
        a.ss[0] = a.ss[1] = has_sh ? m.sd->s : a.s[0];
        a.x = h;
        a.ldx = m.F;
        a.moe = 1;
        a.x_by_pair = 1;
        a.ids = m.ids;
        a.S = m.S; a.K = m.K; a.E = m.E;
        a.out = yp;
        a.cnt = cnt;
        a.wts = m.w;
        a.yfin = m.out;
        a.has_sh = has_sh ? 1 : 0;
        a.radd = m.resid;
        a.yres = m.resid ? m.out_res : nullptr;
        ProfScope ps("moe_down_decode", m.st, true);
        if (!(g ? mg_dispatch_cb<1, true, 1, MG_PART, COLI_MG_KS_DOWN, COLI_MG_NW_DOWN, COLI_MG_NBQ_DOWN>(cb, a, P, m.st, ps)
                : mg_dispatch_cb<1, false, 1, MG_PART, COLI_MG_KS_DOWN, COLI_MG_NW_DOWN, COLI_MG_NBQ_DOWN>(cb, a, P, m.st, ps)))
            return 0;
        int rc = after_launch("moe_down_decode");
        if (rc != COLI_OK) return rc;
    }
    return 1;
}

}  // namespace coli
