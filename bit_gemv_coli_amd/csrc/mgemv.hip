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
// vector ALUs costs ~2.5-3.5 instructions per weight -- close to all of the
// VALU issue budget.  Here each 32-bit word of 8 codes becomes four packed
// fp16 pairs of the exact integers (q-8) or 16*(q-8) in 9 VALU instructions
// (one shift, four v_and_or_b32 with the 1024 magic exponent, four
// v_pk_add_f16), and v_mfma_f32_16x16x32_f16 does the multiply-add.
//
// Precision: the inputs are split as x * 2^e = hi + lo with hi, lo in fp16
// (e a per-input-row power of two putting max|x| just below 2^15), so the
// represented input is within 2^-22 of x relative; products with the exact
// integer weights are exact, accumulation is fp32, the group scale is applied
// in fp32 once per 128 inputs.  The error stays far inside 1e-5 * sum |w||x|.
//
// Layout of one matrix-core step (16 weight rows x 128 inputs):
//   lane l: weight row n = l % 16, input quarter j = l / 16; it loads the 16
//   code bytes of row n at inputs [32j, 32j+32) of the block (one fully used
//   64-byte segment per row and 4 lanes).  Its 4 words feed 4 MFMAs (word m
//   covers inputs 32j+8m .. +8).  The MFMA's B operand is those weights; the
//   A operand rows are (group-in-block, input row, hi/lo) combinations of the
//   inputs read from LDS, zero where the lane's inputs belong to another
//   group, so one MFMA sums each group separately into its own output row.
#include <string.h>

#include <algorithm>

#include "common.h"

namespace coli {

typedef _Float16 f16_t;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4m __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t o) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(m), "v"(o));
    return r;
}

// 8 codes (one word; inputs 0..7, low nibble first) -> B operand slots
// [i0, i4, i1, i5, i2, i6, i3, i7] holding q-8 (even slots of pairs 0 and 2)
// and 16*(q-8) (pairs 1 and 3).
__device__ __forceinline__ f16x8 codes_to_f16(uint32_t w, uint32_t magic) {
    const uint32_t w8 = w >> 8;
    const uint32_t p0 = and_or(w, 0x000F000Fu, magic);
    const uint32_t p1 = and_or(w, 0x00F000F0u, magic);
    const uint32_t p2 = and_or(w8, 0x000F000Fu, magic);
    const uint32_t p3 = and_or(w8, 0x00F000F0u, magic);
    const f16x2 o1 = {(f16_t)-1032.0f, (f16_t)-1032.0f};   // 1024 + 8
    const f16x2 o16 = {(f16_t)-1152.0f, (f16_t)-1152.0f};  // 1024 + 16*8
    const f16x2 h0 = __builtin_bit_cast(f16x2, p0) + o1;
    const f16x2 h1 = __builtin_bit_cast(f16x2, p1) + o16;
    const f16x2 h2 = __builtin_bit_cast(f16x2, p2) + o1;
    const f16x2 h3 = __builtin_bit_cast(f16x2, p3) + o16;
    return f16x8{h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
}

// Input slot of element w (0..7) of an 8-block, and whether its weight comes
// out multiplied by 16 (then the input is stored divided by 16).
__device__ __forceinline__ int slot_of(int w) { return w < 4 ? 2 * w : 2 * (w - 4) + 1; }
__device__ __forceinline__ bool times16(int w) { return (w & 1) != 0; }

enum { MG_Y = 0, MG_SILU = 1, MG_PART = 2 };

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
};

// Partial rows that another workgroup sums are stored and loaded with
// device-scope relaxed atomics: those go to the point of coherence shared by
// all XCDs (their L2s are not coherent with each other for plain accesses), so
// no cache-wide write-back or invalidate is needed.
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
    for (int idx = threadIdx.x; idx < ROWS * a.S; idx += 256) {
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
    }
}

#ifndef COLI_MG_NBK
#define COLI_MG_NBK 4
#endif
#ifndef COLI_MG_KS_GATEUP
#define COLI_MG_KS_GATEUP 2
#endif
#ifndef COLI_MG_KS_DOWN
#define COLI_MG_KS_DOWN 1
#endif
#ifndef COLI_MG_KS_DENSE
#define COLI_MG_KS_DENSE 4
#endif
constexpr int MG_NBK = COLI_MG_NBK;  // 128-input blocks requested together per wavefront
constexpr int MG_ZERO_BYTES = MG_NBK * 256 + 64;

// NT input rows per tile (1..4); CB groups per 128-input block (1, 2, 4);
// KS wavefronts share one 16-row tile along the inputs; NMAT matrices (gate
// and up share their rows).
template <int NT, int CB, bool GROUPED, int NMAT, int EPI, int KS>
__global__ __launch_bounds__(256) void k_mgemv(MgArgs a) {
    constexpr int TPW = 4 / KS;
    constexpr int AROWS = CB * 2 * NT;  // live A rows (<= 16)
    static_assert(AROWS <= 16, "too many A rows");
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int tile_w = wave / KS, ks = wave % KS;
    const int I = a.I, O = a.O;
    const int KSEG = a.kseg;

    // LDS: [NT][2][KSEG] fp16 inputs | zero block | reduction [4][NMAT][16][16] f32 | misc
    f16_t *xs = (f16_t *)smem;
    char *zero = smem + (size_t)NT * 2 * KSEG * 2;
    float *red = (float *)(zero + MG_ZERO_BYTES);
    float *misc = red + 4 * NMAT * 256;

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
            e = gload<int32_t>(a.ids + p);
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
    const int tile = blockIdx.x * TPW + tile_w;
    const int row0 = tile * 16;
    if constexpr (EPI == MG_SILU) {
        if (a.cnt != nullptr && blockIdx.x == 0 && blockIdx.y == 0)
            for (int i = tid; i < a.ncnt; i += 256)
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
    const int n = lane & 15, j = lane >> 4;         // B: weight row, input quarter
    const int ar = lane & 15;                        // A row
    const int acb = ar / (2 * NT), at = (ar % (2 * NT)) / 2, ahl = ar & 1;
    const int lg = (CB == 1) ? 0 : (CB == 2 ? (j >> 1) : j);
    const bool aact = (ar < AROWS) && (acb == lg);
    // this lane's 16 bytes of every packed 1 KiB tile block, and its scale runs
    // (a wavefront past the last tile of a ragged column reads the last tile
    // again and writes nothing)
    const int tile_ld = min(tile, (O + 15) / 16 - 1);
    const uint8_t *qtile[NMAT];
    const float *stile[NMAT];
#pragma unroll
    for (int m = 0; m < NMAT; ++m) {
        qtile[m] = pkm[m] + (int64_t)tile_ld * a.nkb * 1024 + 16 * lane;
        stile[m] = (const float *)(pkm[m] + a.pk_scale_off) + (int64_t)tile_ld * a.nkb * a.cbs * 16 + n;
    }
    // C rows of this lane: 4*j .. 4*j+3 (j doubles as the C row quarter)
    const int cr0 = 4 * j;
    const int ccb0 = min(cr0, AROWS - 1) / (2 * NT);
    const int ccb1 = min(cr0 + 2, AROWS - 1) / (2 * NT);
    const int kpad = (I + 127) / 128 * 128;
    const uint32_t magic = 0x64006400u;

    float acc[NMAT][4];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[m][i] = 0.f;

    // exponent factors 2^-e per (input row, 128-input block) of the segment
    float *xfac = misc;  // [NT][kseg/128]
    const int fstride = KSEG / 128;

    // requests for one batch of 128-input blocks (codes and group scales);
    // two batches alternate so one is in flight while the other is computed
    struct Batch {
        u32x4 cw[MG_NBK][NMAT];
        float s0[MG_NBK][NMAT], s1[MG_NBK][NMAT];
    };
    Batch bA, bB;
    auto load_batch = [&](Batch &bt, int kbg, int kb_last) {
        auto &cw = bt.cw;
        auto &s0 = bt.s0;
        auto &s1 = bt.s1;
#pragma unroll
        for (int i = 0; i < MG_NBK; ++i) {
            const int kglob = min(kbg + i, kb_last);
#pragma unroll
            for (int m = 0; m < NMAT; ++m) {
                cw[i][m] = __builtin_nontemporal_load(
                    (const COLI_GLOBAL u32x4 *)(qtile[m] + (int64_t)kglob * 1024));
                if constexpr (GROUPED) {
                    const float *sb = stile[m] + (int64_t)kglob * a.cbs * 16;
                    s0[i][m] = gload<float>(sb + ccb0 * 16);
                    s1[i][m] = (((2 * NT) % 4) == 0) ? s0[i][m] : gload<float>(sb + ccb1 * 16);
                } else {
                    s0[i][m] = s1[i][m] = 1.0f;
                }
            }
        }
    };

    // the first batch is requested before the inputs are staged
    int seg0_beg, seg0_end;
    {
        const int klen = min(KSEG, kpad);
        const int nkb = klen / 128;
        seg0_beg = (ks * nkb) / KS;
        seg0_end = ((ks + 1) * nkb) / KS;
        if (seg0_beg < seg0_end)
            load_batch(bA, seg0_beg, seg0_end - 1);
    }

    for (int sgi = 0; sgi < a.nseg; ++sgi) {
        const int k0 = sgi * KSEG;
        const int klen = min(KSEG, kpad - k0);
        const int nkb = klen / 128;
        // ---- stage this segment's inputs: hi / lo fp16 in slot order, one
        //      power-of-two exponent per (input row, 128-input block): 16
        //      consecutive threads own one block, each 8 inputs -------------
        __syncthreads();
        {
            constexpr int UN = 4;
            const int nb8 = klen / 8;
            for (int base = 0; base < NT * nb8; base += UN * 256) {
                float v[UN][8];
#pragma unroll
                for (int u = 0; u < UN; ++u) {
                    const int idx = min(base + u * 256 + tid, NT * nb8 - 1);
                    const int t = idx / nb8, b8 = idx % nb8;
                    const int k = k0 + b8 * 8;
                    const float *xr = a.x + (int64_t)xrow[t] * a.ldx + min(k, I - 8);
                    const f32x4 p0 = gload<f32x4>(xr), p1 = gload<f32x4>(xr + 4);
                    const bool in = k < I;
                    v[u][0] = in ? p0.x : 0.f; v[u][1] = in ? p0.y : 0.f;
                    v[u][2] = in ? p0.z : 0.f; v[u][3] = in ? p0.w : 0.f;
                    v[u][4] = in ? p1.x : 0.f; v[u][5] = in ? p1.y : 0.f;
                    v[u][6] = in ? p1.z : 0.f; v[u][7] = in ? p1.w : 0.f;
                }
#pragma unroll
                for (int u = 0; u < UN; ++u) {
                    const int idx = base + u * 256 + tid;
                    float mx = 0.f;
#pragma unroll
                    for (int w = 0; w < 8; ++w) mx = fmaxf(mx, fabsf(v[u][w]));
#pragma unroll
                    for (int off = 8; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 16));
                    int e2 = 0;
                    if (mx > 0.f && mx <= 3.0e38f) {
                        (void)frexpf(mx, &e2);  // mx < 2^e2
                        e2 = 15 - e2;
                    }
                    if (idx < NT * nb8) {
                        const int t = idx / nb8, b8 = idx % nb8;
                        f16x8 hv, lv;
#pragma unroll
                        for (int w = 0; w < 8; ++w) {
                            const float vs = ldexpf(v[u][w], e2 - (times16(w) ? 4 : 0));
                            const f16_t h = (f16_t)vs;
                            hv[slot_of(w)] = h;
                            lv[slot_of(w)] = (f16_t)(vs - (float)h);
                        }
                        *reinterpret_cast<f16x8 *>(&xs[(t * 2 + 0) * KSEG + b8 * 8]) = hv;
                        *reinterpret_cast<f16x8 *>(&xs[(t * 2 + 1) * KSEG + b8 * 8]) = lv;
                        if ((b8 & 15) == 0)
                            xfac[t * fstride + b8 / 16] = ldexpf(1.0f, -e2);
                    }
                }
            }
            for (int idx = tid; idx < MG_ZERO_BYTES / 16; idx += 256)
                reinterpret_cast<u32x4 *>(zero)[idx] = u32x4{0u, 0u, 0u, 0u};
        }
        __syncthreads();

        // ---- this wavefront's share of the segment's 128-input blocks ------
        const int kb_beg = (ks * nkb) / KS, kb_end = ((ks + 1) * nkb) / KS;
        const char *abase = (const char *)&xs[(at * 2 + ahl) * KSEG + 32 * j];
        // token of each of this lane's C rows (rows cr0, cr0+1 / cr0+2, cr0+3)
        const int ct0 = (min(cr0, AROWS - 1) % (2 * NT)) / 2;
        const int ct1 = (min(cr0 + 2, AROWS - 1) % (2 * NT)) / 2;

        auto compute_batch = [&](Batch &bt, int kb) {
            // inactive lanes read the zero block (it covers a whole batch)
            const char *ap = aact ? abase + kb * 256 : zero;
#pragma unroll
            for (int i = 0; i < MG_NBK; ++i) {
                if (kb + i >= kb_end)
                    break;
                f16x8 av[4];
#pragma unroll
                for (int mm = 0; mm < 4; ++mm)
                    av[mm] = *reinterpret_cast<const f16x8 *>(ap + i * 256 + 16 * mm);
                const float f0 = xfac[ct0 * fstride + kb + i];
                const float f1 = xfac[ct1 * fstride + kb + i];
#pragma unroll
                for (int m = 0; m < NMAT; ++m) {
                    const u32x4 w = bt.cw[i][m];
                    f32x4m c = {0.f, 0.f, 0.f, 0.f};
                    c = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[0], codes_to_f16(w.x, magic), c, 0, 0, 0);
                    c = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[1], codes_to_f16(w.y, magic), c, 0, 0, 0);
                    c = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[2], codes_to_f16(w.z, magic), c, 0, 0, 0);
                    c = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[3], codes_to_f16(w.w, magic), c, 0, 0, 0);
                    const float g0 = bt.s0[i][m] * f0, g1 = bt.s1[i][m] * f1;
                    acc[m][0] = fmaf(g0, c[0], acc[m][0]);
                    acc[m][1] = fmaf(g0, c[1], acc[m][1]);
                    acc[m][2] = fmaf(g1, c[2], acc[m][2]);
                    acc[m][3] = fmaf(g1, c[3], acc[m][3]);
                }
            }
        };
        const int kg0 = k0 / 128;
        if (sgi > 0 && kb_beg < kb_end)
            load_batch(bA, kg0 + kb_beg, kg0 + kb_end - 1);
        for (int kb = kb_beg; kb < kb_end; kb += 2 * MG_NBK) {
            const bool hasB = kb + MG_NBK < kb_end;
            if (hasB)
                load_batch(bB, kg0 + kb + MG_NBK, kg0 + kb_end - 1);
            compute_batch(bA, kb);
            if (kb + 2 * MG_NBK < kb_end)
                load_batch(bA, kg0 + kb + 2 * MG_NBK, kg0 + kb_end - 1);
            if (hasB)
                compute_batch(bB, kb + MG_NBK);
        }
    }

    // --- reduce: KS wavefronts x (group, hi/lo) rows -> one value per (row, input row)
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[((wave * NMAT + m) * 16 + cr0 + i) * 16 + n] = acc[m][i];
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
                for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                    for (int hl = 0; hl < 2; ++hl)
                        sum += red[(((tile_w * KS + w2) * NMAT + m) * 16 + cb * 2 * NT + 2 * t + hl) * 16 + nn];
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
            a.out[(p * a.Sy + t) * O + row] = v[0];
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
    if (fmt != 2 && fmt != 4)
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

static PackGeom pack_geom(int fmt, int O, int I, int gs) {
    PackGeom g;
    g.rt = (O + 15) / 16;
    g.nkb = (I + 127) / 128;
    g.cbs = cbs_of(fmt, gs);
    g.code_bytes = (int64_t)g.rt * g.nkb * 1024;
    g.scale_off = g.code_bytes;
    const int64_t sb = (fmt == 4) ? (int64_t)g.rt * g.nkb * g.cbs * 16 * 4 : 0;
    g.stride = (g.code_bytes + sb + 255) / 256 * 256;
    return g;
}

size_t packed_bytes(int fmt, int n, int O, int I, int gs) {
    if (n < 1 || O < 1 || !packable(fmt, I, gs))
        return 0;
    return (size_t)pack_geom(fmt, O, I, gs).stride * n;
}

// packed codes: tile block (e, rt, kb) = 1 KiB, lane l = 16*j + r holds row
// 16*rt + r, inputs kb*128 + 32*j .. +32 (16 bytes); padding codes 0x88 (= 0)
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
        u32x4 v = {0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u};
        if (row < O && k < I)
            v = gload<u32x4>(q + (int64_t)e * q_stride + (int64_t)row * rb + k / 2);
        *reinterpret_cast<u32x4 *>(pk + (int64_t)e * stride + ((int64_t)tr * nkb + kb) * 1024 + 16 * l) = v;
    }
}

// packed fmt-4 scales: for (e, rt, kb) a run of cbs x 16 floats: slot cb, row r
// holds s[16*rt + r][group of the 128-input block's slot cb]; padding 0
__global__ __launch_bounds__(256) void k_pack_scales(const float *__restrict__ s, int64_t s_stride,
                                                     int ng, int gs, int n, int O, int rt, int nkb,
                                                     int cbs, int64_t stride, int64_t scale_off,
                                                     uint8_t *__restrict__ pk) {
    const int64_t total = (int64_t)n * rt * nkb * cbs * 16;
    for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < total;
         c += (int64_t)gridDim.x * 256) {
        const int r = (int)(c % 16);
        int64_t t = c / 16;
        const int cb = (int)(t % cbs);
        t /= cbs;
        const int kb = (int)(t % nkb);
        t /= nkb;
        const int tr = (int)(t % rt);
        const int e = (int)(t / rt);
        const int row = tr * 16 + r;
        const int g = (cbs == 1) ? (kb * 128) / gs : kb * cbs + cb;
        float v = 0.f;
        if (row < O && g < ng)
            v = gload<float>(s + (int64_t)e * s_stride + (int64_t)row * ng + g);
        float *dst = (float *)(pk + (int64_t)e * stride + scale_off);
        dst[(((int64_t)tr * nkb + kb) * cbs + cb) * 16 + r] = v;
    }
}

int launch_pack(coli_qtensor *t, void *packed, hipStream_t st) {
    const PackGeom g = pack_geom(t->fmt, t->O, t->I, t->gs);
    {
        const int64_t total = (int64_t)t->n * g.rt * g.nkb * 64;
        const unsigned blocks = (unsigned)std::min<int64_t>((total + 255) / 256, 65536);
        ProfScope ps("pack", st);
        hipLaunchKernelGGL(k_pack_codes, dim3(blocks), dim3(256), 0, st, (const uint8_t *)t->q,
                           t->row_bytes, t->q_stride, t->n, t->O, t->I, g.rt, g.nkb, g.stride,
                           (uint8_t *)packed);
        int rc = after_launch("pack");
        if (rc != COLI_OK) return rc;
    }
    if (t->fmt == 4) {
        const int64_t total = (int64_t)t->n * g.rt * g.nkb * g.cbs * 16;
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
bool mgemv_ok(const coli_qtensor *W) {
    return (W->flags & QF_PACKED) && W->pk != nullptr && packable(W->fmt, W->I, W->gs);
}

static int cb_of(const coli_qtensor *W) { return cbs_of(W->fmt, W->gs); }

static void plan_lds(int NT, int NMAT, int I, int &kseg, int &nseg, size_t &bytes) {
    const int kpad = (I + 127) / 128 * 128;
    const int cap = (48 * 1024) / (NT * 2 * 2);          // inputs per segment
    kseg = cap / 128 * 128;
    if (kseg > kpad) kseg = kpad;
    nseg = (kpad + kseg - 1) / kseg;
    bytes = (size_t)NT * 2 * kseg * 2 + MG_ZERO_BYTES + 4 * NMAT * 256 * 4 +
            (size_t)NT * (kseg / 128) * 4 + 64;
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

template <int NT, int CB, bool GROUPED, int NMAT, int EPI, int KS>
static void mg_launch(MgArgs a, int groups, hipStream_t st) {
    size_t lds;
    plan_lds(NT, NMAT, a.I, a.kseg, a.nseg, lds);
    constexpr int TPW = 4 / KS;
    const int tiles = (a.O + 15) / 16;
    const dim3 grid((unsigned)((tiles + TPW - 1) / TPW), (unsigned)groups);
    hipLaunchKernelGGL((k_mgemv<NT, CB, GROUPED, NMAT, EPI, KS>), grid, dim3(256), lds, st, a);
}

template <int NT, bool GROUPED, int NMAT, int EPI, int KS>
static int mg_dispatch_cb(int cb, const MgArgs &a, int groups, hipStream_t st) {
    switch (cb) {
    case 1: mg_launch<NT, 1, GROUPED, NMAT, EPI, KS>(a, groups, st); return 1;
    case 2:
        if constexpr (NT <= 4) { mg_launch<NT, 2, GROUPED, NMAT, EPI, KS>(a, groups, st); return 1; }
        return 0;
    default:
        if constexpr (NT <= 2) { mg_launch<NT, 4, GROUPED, NMAT, EPI, KS>(a, groups, st); return 1; }
        return 0;
    }
}

// Dense GEMV y[e][t][o] for S <= 4 input rows.  Returns 0 when the layout or
// (S, gs) combination is not taken (caller falls back to the VALU kernels).
int launch_mgemv(const coli_qtensor *W, const float *x, float *y, int S, hipStream_t st) {
    if (!mgemv_ok(W) || S < 1 || S > 4)
        return 0;
    const int cb = cb_of(W);
    if (cb * 2 * S > 16)
        return 0;
    MgArgs a = mg_args_for(W);
    a.x = x;
    a.ldx = W->I;
    a.out = y;
    a.Sy = S;
    const bool g = W->fmt == 4;
    ProfScope ps("mgemv", st);
    int ok;
#define MG_CASE(NTV)                                                                          \
    ok = g ? mg_dispatch_cb<NTV, true, 1, MG_Y, COLI_MG_KS_DENSE>(cb, a, W->n, st)            \
           : mg_dispatch_cb<NTV, false, 1, MG_Y, COLI_MG_KS_DENSE>(cb, a, W->n, st)
    switch (S) {
    case 1: MG_CASE(1); break;
    case 2: MG_CASE(2); break;
    case 3: MG_CASE(3); break;
    default: MG_CASE(4); break;
    }
#undef MG_CASE
    if (!ok)
        return 0;
    return after_launch("mgemv") == COLI_OK ? 1 : -1;
}

// Decode MoE block on the matrix cores: gate/up + SiLU (dual), then down per
// pair with the weighted top-k combine done by the last workgroup of each row
// column (cnt: one arrival counter per column, cleared by the gate/up launch).
// Returns 1 when the whole block was launched, 0 when not taken.
int launch_mgemv_moe(const MoeArgs &m, float *h, float *yp, int *cnt) {
    const coli_qtensor *all[6] = {m.gate, m.up, m.down, m.sg, m.su, m.sd};
    for (const coli_qtensor *t : all)
        if (t && !mgemv_ok(t))
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
        ProfScope ps("moe_gateup_decode", m.st);
        if (!(g ? mg_dispatch_cb<1, true, 2, MG_SILU, COLI_MG_KS_GATEUP>(cb, a, P, m.st)
                : mg_dispatch_cb<1, false, 2, MG_SILU, COLI_MG_KS_GATEUP>(cb, a, P, m.st)))
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
        ProfScope ps("moe_down_decode", m.st);
        if (!(g ? mg_dispatch_cb<1, true, 1, MG_PART, COLI_MG_KS_DOWN>(cb, a, P, m.st)
                : mg_dispatch_cb<1, false, 1, MG_PART, COLI_MG_KS_DOWN>(cb, a, P, m.st)))
            return 0;
        int rc = after_launch("moe_down_decode");
        if (rc != COLI_OK) return rc;
    }
    return 1;
}

}  // namespace coli
