// dgemm.hip -- prefill GEMM (S > 4 input rows) for packed int4 tensors, with
// the K dimension split over the four wavefronts of a workgroup:
// Y[m][n] = sum_k w(n, k) * X[m][k], w(n, k) = scale(n, k) * (q - 8) (colibri
// PR #298, CUDA fmt=4 commit: the group scale applied inline; colibri-strix
// prefill GEMM routing commit: large row batches take a GEMM path).
//
// Two launches:
//   k_dg_xprep  the input rows once to bf16, in the order the matrix cores
//               read them (fragments of 16 rows x 8 inputs, 1 KiB per
//               wavefront request), rows padded to whole tiles with zeros;
//   k_dg        one workgroup per 144 x 96 output tile (of one matrix, or
//               of two with the same inputs, the grid's z choosing the
//               matrix): each wavefront takes one quarter (a 32-input
//               slice) of every 128-input block and accumulates the whole
//               tile for it, so every weight is turned
//               into bf16 once per 144 input rows and no operand passes
//               between wavefronts; the four partial tiles are added in a
//               fixed order at the end.
//
// Precision (the bf16 envelope): weight bf16(f32(s * (q - 8))), input
// bf16(x), products summed in fp32 on v_mfma_f32_16x16x32_bf16.  bf16 keeps
// 8 significant bits (each rounding within 2^-8 relative), so |error| <=
// (2^-7 + 2^-16) * sum |w||x| plus the fp32 accumulation; with no single
// product carrying most of sum |w||x| the roundings average out far inside
// 4e-3 * sum |w||x|.
//
// Per wavefront and block: its 9 input fragments go straight to LDS
// (global_load_lds_dwordx4, no registers), its 6 code words and scales to
// registers, all DG_PD blocks ahead in a ring of DG_PD + 1 slots; then the 9
// fragments come back from LDS, each code word becomes 8 bf16 weights and the
// 54 products of the slice run.  A wavefront only touches its own LDS slots,
// so the main loop has no barrier.
//
// 256 tiles for the 544 x 6144 x 6144 shape: 4 row tiles (the last with 112
// rows) x 64 column tiles, one per compute unit; the tiles of one XCD share
// their row tile (its inputs stay in that XCD's L2).
#include <string.h>

#include "dgemm.h"

namespace coli {

typedef __bf16 dg_bf16x8 __attribute__((ext_vector_type(8)));

constexpr int DG_MB = 9;                 // 16-row input blocks per tile
constexpr int DG_NT = 6;                 // 16-row weight tiles per tile
constexpr int DG_TM = 16 * DG_MB;        // 144 input rows
constexpr int DG_TN = 16 * DG_NT;        // 96 outputs
constexpr int DG_SLOT = DG_MB * 1024;    // one wavefront's inputs of one block (bytes)
constexpr int DG_RSRC_W3 = 0x00020000;   // raw buffer loads; past the size: zeros
static_assert(DG_MB * (DG_NT / 2) * 1024 <= 4 * DG_SLOT, "a partial half tile fits in one slot array");

enum { DG_GRP = 0, DG_ROW = 1 };

struct DgArgs {
    const uint8_t *xf;  // bf16 input fragments (k_dg_xprep)
    const uint8_t *pq;  // packed codes
    const float *ps;    // packed scale runs (fmt 4) or row scales (fmt 2)
    int xbytes, qbytes, sbytes;  // their sizes
    int nkb, nkq, cbs, gshift, rtn;
    int M, N, nmt, nnt;
    float *y;
    int64_t ldy;
    // batches along the grid's y: batch b takes the fragments at byte
    // b * xf_bstride, weight tiles rt0 + b * rt_bstride + (0 .. rtn - 1) and
    // outputs at y + b * y_bstride (one batch: all zero)
    int xf_bstride, rt0, rt_bstride, Otot;
    int64_t y_bstride;
};
// one or two matrices per launch: grid z picks the matrix (two matrices of
// the same inputs, each with its own tiles; a workgroup past its matrix's
// tiles ends at once)
struct DgPair {
    DgArgs m[2];
};


// acc += A B on the matrix cores, accumulating in place in acc's registers
// (the builtin lets the register allocator move the 216 accumulators between
// registers every block).  The two wait states ahead cover an operand just
// written by a vector instruction; results are read back only after the
// loop, behind dg_mfma_drain.
__device__ __forceinline__ void dg_mfma(f32x4 &acc, const u32x4 &a, const u32x4 &b) {
    asm volatile("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// wait states between the last matrix-core result and any other read of it
__device__ __forceinline__ void dg_mfma_drain() { asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 15" ::: "memory"); }

// One weight tile of one block: the 9 products acc[i][t] += a[i] b (b the
// tile's bf16 weights), with the next tile's 8 codes (word w, two's-complement
// nibbles) turned into bf16 weights w * s16 * 16 between them, so the vector
// instructions issue while the matrix cores run.  The two wait states before
// the first product cover b having just been written by a vector instruction.
// Returns the next tile's bf16 weights (inputs 0..7 in order).
template <int NT>
__device__ __forceinline__ u32x4 dg_tile(f32x4 (&acc)[DG_MB][NT], int t, const u32x4 (&a)[DG_MB],
                                         const u32x4 &b, uint32_t w, float s16) {
    uint32_t ev, od, b0, b1, b2, b3;
    float f0, f1;
    asm volatile(
        "s_nop 1\n\t"
        "v_mfma_f32_16x16x32_bf16 %0, %17, %26, %0\n\t"
        "v_lshlrev_b32 %9, 4, %27\n\t"
        "v_and_b32 %9, 0xf0f0f0f0, %9\n\t"
        "v_and_b32 %10, 0xf0f0f0f0, %27\n\t"
        "v_mfma_f32_16x16x32_bf16 %1, %18, %26, %1\n\t"
        "v_cvt_f32_i32_sdwa %11, sext(%9) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_0\n\t"
        "v_cvt_f32_i32_sdwa %12, sext(%10) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_0\n\t"
        "v_mul_f32 %11, %11, %28\n\t"
        "v_mfma_f32_16x16x32_bf16 %2, %19, %26, %2\n\t"
        "v_mul_f32 %12, %12, %28\n\t"
        "v_cvt_pk_bf16_f32 %13, %11, %12\n\t"
        "v_cvt_f32_i32_sdwa %11, sext(%9) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_1\n\t"
        "v_mfma_f32_16x16x32_bf16 %3, %20, %26, %3\n\t"
        "v_cvt_f32_i32_sdwa %12, sext(%10) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_1\n\t"
        "v_mul_f32 %11, %11, %28\n\t"
        "v_mul_f32 %12, %12, %28\n\t"
        "v_mfma_f32_16x16x32_bf16 %4, %21, %26, %4\n\t"
        "v_cvt_pk_bf16_f32 %14, %11, %12\n\t"
        "v_cvt_f32_i32_sdwa %11, sext(%9) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_2\n\t"
        "v_cvt_f32_i32_sdwa %12, sext(%10) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_2\n\t"
        "v_mfma_f32_16x16x32_bf16 %5, %22, %26, %5\n\t"
        "v_mul_f32 %11, %11, %28\n\t"
        "v_mul_f32 %12, %12, %28\n\t"
        "v_cvt_pk_bf16_f32 %15, %11, %12\n\t"
        "v_mfma_f32_16x16x32_bf16 %6, %23, %26, %6\n\t"
        "v_cvt_f32_i32_sdwa %11, sext(%9) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_3\n\t"
        "v_cvt_f32_i32_sdwa %12, sext(%10) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_3\n\t"
        "v_mul_f32 %11, %11, %28\n\t"
        "v_mfma_f32_16x16x32_bf16 %7, %24, %26, %7\n\t"
        "v_mul_f32 %12, %12, %28\n\t"
        "v_cvt_pk_bf16_f32 %16, %11, %12\n\t"
        "v_mfma_f32_16x16x32_bf16 %8, %25, %26, %8"
        : "+a"(acc[0][t]), "+a"(acc[1][t]), "+a"(acc[2][t]), "+a"(acc[3][t]), "+a"(acc[4][t]),
          "+a"(acc[5][t]), "+a"(acc[6][t]), "+a"(acc[7][t]), "+a"(acc[8][t]), "=&v"(ev), "=&v"(od),
          "=&v"(f0), "=&v"(f1), "=&v"(b0), "=&v"(b1), "=&v"(b2), "=&v"(b3)
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]),
          "v"(a[8]), "v"(b), "v"(w), "v"(s16));
    return u32x4{b0, b1, b2, b3};
}

// s_waitcnt with only the vector-memory count constrained (gfx9 encoding)
template <int N>
__device__ __forceinline__ void dg_wait_vm() {
    static_assert(N >= 0 && N <= 63, "vmcnt");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// workgroup barrier for LDS hand-overs: waits for this wavefront's LDS
// accesses only (global stores may still be in flight)
__device__ __forceinline__ void dg_lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Fragment block (mb, kb) = 4 KiB at xf + (mb * nkb4 + kb) * 4096 (nkb4: the
// 128-input blocks rounded up to a multiple of 4): slice s (1 KiB), lane
// l = 16 j + r holds bf16 of x[16 mb + r][128 kb + 32 j + 8 s .. + 8]; zero
// past M rows or K inputs.  One workgroup per (mb, block): thread t takes
// row t / 16, inputs 8 (t % 16) .. + 8 (rows read contiguously); a workgroup
// per block rather than per 4 blocks keeps more loads in flight (measured on
// the 544 x 6144 x 6144 GEMM: ~2 us less per call).
__global__ __launch_bounds__(256) void k_dg_xprep(const float *__restrict__ x, int64_t ldx, int M,
                                                  int K, int nkb4, uint8_t *__restrict__ xf,
                                                  int64_t x_bstride, int64_t xf_bstride) {
    // batch blockIdx.z: inputs at x + z * x_bstride, fragments at xf + z * xf_bstride
    x += (int64_t)blockIdx.z * x_bstride;
    xf += (int64_t)blockIdx.z * xf_bstride;
    const int mb = blockIdx.x, kb = blockIdx.y;
    const int t = threadIdx.x, r = t >> 4, c8 = t & 15;
    const int row = 16 * mb + r;
    const int k = 128 * kb + 8 * c8;
    f32x4 a = {0.f, 0.f, 0.f, 0.f}, b = a;
    if (row < M && k < K) {
        const float *p = x + (int64_t)row * ldx + k;
        a = gload<f32x4>(p);
        b = gload<f32x4>(p + 4);
    }
    const u32x4 o = {dgemm_bf16x2(a.x, a.y), dgemm_bf16x2(a.z, a.w), dgemm_bf16x2(b.x, b.y),
                     dgemm_bf16x2(b.z, b.w)};
    *reinterpret_cast<u32x4 *>(xf + dgemm_frag_offset(row, k, nkb4)) = o;
}

template <int SM>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_dg(DgPair pr) {
    const DgArgs &a = pr.m[blockIdx.z];
    if ((int)blockIdx.x >= a.nmt * a.nnt)
        return;
    // ring slot u (one array each, so the compiler sees the slots apart): the
    // four wavefronts' inputs of one block, DG_SLOT bytes each
    __shared__ __attribute__((aligned(16))) uint8_t rs0[4 * DG_SLOT], rs1[4 * DG_SLOT],
        rs2[4 * DG_SLOT], rs3[4 * DG_SLOT];
    auto ring = [&](int u) -> uint8_t * { return u == 0 ? rs0 : u == 1 ? rs1 : u == 2 ? rs2 : rs3; };
    const int tid = threadIdx.x, lane = tid & 63, ln = lane & 15, lg = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // = the slice it takes
    int mt, nt;
    {
        // XCD-aware order (workgroup w runs on XCD w % 8): each XCD takes a
        // contiguous run of tiles in row-tile-major order
        const int w = blockIdx.x, tot = a.nmt * a.nnt;
        int tile = w;
        if (tot % 8 == 0)
            tile = (w % 8) * (tot / 8) + w / 8;
        mt = tile / a.nnt;
        nt = tile % a.nnt;
    }
    const int nkb = a.nkb, nkb4 = (nkb + 3) / 4 * 4;

    // weight word `wave` of this lane in every block of the 6 tiles (tiles
    // past the matrix clamped; their outputs are dropped) and its scales, as
    // buffer loads: per lane a fixed byte offset, per request a uniform one
    const __amdgpu_buffer_rsrc_t qrs =
        __builtin_amdgcn_make_buffer_rsrc((void *)a.pq, (short)0, a.qbytes, DG_RSRC_W3);
    const __amdgpu_buffer_rsrc_t srs =
        __builtin_amdgcn_make_buffer_rsrc((void *)a.ps, (short)0, a.sbytes, DG_RSRC_W3);
    const __amdgpu_buffer_rsrc_t xrs =
        __builtin_amdgcn_make_buffer_rsrc((void *)a.xf, (short)0, a.xbytes, DG_RSRC_W3);
    int rt[DG_NT];
    float rsc[DG_NT];
#pragma unroll
    for (int t = 0; t < DG_NT; ++t) {
        rt[t] = a.rt0 + (int)blockIdx.y * a.rt_bstride + min(nt * DG_NT + t, a.rtn - 1);
        rsc[t] = SM == DG_ROW ? gload<float>(a.ps + min(16 * rt[t] + ln, a.Otot - 1)) : 0.f;
    }
    const int qv = 16 * lane + 4 * wave;
    const int cb = a.cbs == 1 ? 0 : (lg >> (a.gshift - 5));  // group slot of the lane's 32 inputs
    const int sv = (ln * a.cbs + cb) * 16;                     // its scale run in a quad (bytes)
    // this wavefront's input fragments: row block i of block kb at byte
    // ((mt * 9 + i) * nkb4 + kb) * 4096 + 1024 wave + 16 lane; the blocks past
    // nkb hold zero inputs, so the clamped codes there add nothing
    const int xv = wave * 1024 + 16 * lane;
    const int xrow = mt * DG_MB * nkb4 + (int)blockIdx.y * (a.xf_bstride / 4096);
    const int wofs = wave * DG_SLOT;
    // inputs of block kb (clamped to the padded blocks) into ring slot u
    auto issue = [&](int u, int kb) {
        const int kx = min(kb, nkb4 - 1);
#pragma unroll
        for (int i = 0; i < DG_MB; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                xrs, (__attribute__((address_space(3))) void *)(ring(u) + wofs + i * 1024), 16, xv,
                ((xrow + i * nkb4) + kx) * 4096, 0, 0);
    };
    // code words and scales of the 4 blocks (one scale quad) of trip T
    // (blocks clamped to the last)
    struct BT {
        uint32_t c[4][DG_NT];
        f32x4 s[DG_NT];
    };
    auto bload = [&](BT &bt, int T) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int kc = min(4 * T + v, nkb - 1);
#pragma unroll
            for (int t = 0; t < DG_NT; ++t)
                bt.c[v][t] = __builtin_amdgcn_raw_buffer_load_b32(qrs, qv, (rt[t] * nkb + kc) * 1024, 0);
        }
        if (SM == DG_GRP) {
            const int kq = min(T, a.nkq - 1);
#pragma unroll
            for (int t = 0; t < DG_NT; ++t)
                bt.s[t] = __builtin_bit_cast(
                    f32x4, __builtin_amdgcn_raw_buffer_load_b128(srs, sv, (rt[t] * a.nkq + kq) * 16 * a.cbs * 16, 0));
        }
    };

    f32x4 acc[DG_MB][DG_NT];
#pragma unroll
    for (int i = 0; i < DG_MB; ++i)
#pragma unroll
        for (int t = 0; t < DG_NT; ++t) acc[i][t] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Blocks go 4 to a trip; block c's inputs sit in ring slot c % 4 and are
    // requested during block c - 4 (tile 4), its code words and scales with
    // the rest of its trip at the start of the trip before.  At most 63
    // vector-memory requests are in flight (the counter's range).  Tile 3 of
    // block c waits for block c + 1's inputs and reads them from LDS.
    constexpr int NB = 4 * DG_NT + (SM == DG_GRP ? DG_NT : 0);  // code and scale requests per trip
    static_assert(3 * DG_MB + NB <= 63, "vmcnt range");
    BT bc, bn;
    u32x4 af[2][DG_MB];  // inputs of even / odd blocks
    bload(bc, 0);
#pragma unroll
    for (int p = 0; p < 3; ++p) issue(p, p);
    dg_wait_vm<2 * DG_MB>();  // block 0's inputs (and the codes before them)
#pragma unroll
    for (int i = 0; i < DG_MB; ++i)
        af[0][i] = *reinterpret_cast<const u32x4 *>(ring(0) + wofs + i * 1024 + 16 * lane);
    asm volatile("" ::: "memory");
    issue(3, 3);
    auto s16of = [&](const BT &bt, int v, int t) -> float {
        return (SM == DG_GRP ? bt.s[t][v] : rsc[t]) * 0.0625f;
    };
    u32x4 bw;  // bf16 weights of the tile about to be multiplied
    {
        const float s16 = s16of(bc, 0, 0);
        const uint32_t w = bc.c[0][0];
        const uint32_t ev = (w << 4) & 0xF0F0F0F0u, od = w & 0xF0F0F0F0u;
        bw = u32x4{dgemm_bf16x2(sbyte<0>(ev) * s16, sbyte<0>(od) * s16), dgemm_bf16x2(sbyte<1>(ev) * s16, sbyte<1>(od) * s16),
                   dgemm_bf16x2(sbyte<2>(ev) * s16, sbyte<2>(od) * s16), dgemm_bf16x2(sbyte<3>(ev) * s16, sbyte<3>(od) * s16)};
    }
    for (int T = 0; 4 * T < nkb4; ++T) {
        bload(bn, T + 1);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int c = 4 * T + u, p = u % 2, q = (u + 1) % 2;
#pragma unroll
            for (int t = 0; t < DG_NT; ++t) {
                if (t == 3) {
                    // requests after block c + 1's inputs: blocks c + 2 and c + 3's
                    // (and, for u < 3, the next trip's codes)
                    if (u < 3)
                        dg_wait_vm<2 * DG_MB + NB>();
                    else
                        dg_wait_vm<2 * DG_MB>();
#pragma unroll
                    for (int i = 0; i < DG_MB; ++i)
                        af[q][i] = *reinterpret_cast<const u32x4 *>(ring((u + 1) % 4) + wofs + i * 1024 + 16 * lane);
                }
                if (t == 4) {
                    asm volatile("" ::: "memory");  // (slot u was read during block c - 1)
                    issue(u, c + 4);
                }
                // the next tile's code word and scale (tile 0 of block c + 1 after the last)
                const uint32_t wn = t + 1 < DG_NT ? bc.c[u][t + 1] : (u < 3 ? bc.c[u + 1][0] : bn.c[0][0]);
                const float sn = t + 1 < DG_NT ? s16of(bc, u, t + 1) : (u < 3 ? s16of(bc, u + 1, 0) : s16of(bn, 0, 0));
                bw = dg_tile(acc, t, af[p], bw, wn, sn);
            }
        }
        bc = bn;
    }
    dg_mfma_drain();
    __builtin_amdgcn_s_waitcnt(0);  // no request into the ring left in flight
    __syncthreads();

    // ---- the four partial tiles, added in wavefront order, half the weight
    // tiles at a time: wavefront w stores its 27 fragments (i, t) of the half
    // in slot array w (lane l's 4 values together), then each wavefront sums
    // a share of the fragments over the four arrays and writes them; lane
    // (ln, lg) of fragment (i, t) holds rows 16 i + 4 lg + r, column 16 t + ln.
    // The barriers wait for LDS only, so the first half's output stores stay
    // in flight during the second half (measured: 2-3 us less per call).
    const int m0 = mt * DG_TM, n0 = nt * DG_TN;
    float *const yb = a.y + (int64_t)blockIdx.y * a.y_bstride;
    f32x4 *mine = reinterpret_cast<f32x4 *>(ring(wave));
    const f32x4 *p0 = reinterpret_cast<const f32x4 *>(rs0), *p1 = reinterpret_cast<const f32x4 *>(rs1);
    const f32x4 *p2 = reinterpret_cast<const f32x4 *>(rs2), *p3 = reinterpret_cast<const f32x4 *>(rs3);
    constexpr int HT = DG_NT / 2, NF = DG_MB * HT;  // 27 fragments per half
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int i = 0; i < DG_MB; ++i)
#pragma unroll
            for (int tt = 0; tt < HT; ++tt) mine[(i * HT + tt) * 64 + lane] = acc[i][h * HT + tt];
        dg_lds_barrier();
        for (int f = wave; f < NF; f += 4) {
            const int o = f * 64 + lane;
            const f32x4 v = ((p0[o] + p1[o]) + p2[o]) + p3[o];
            const int i = f / HT, tt = f % HT;
            const int gn = n0 + 16 * (h * HT + tt) + ln;
            if (gn < a.N) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int gm = m0 + 16 * i + 4 * lg + r;
                    if (gm < a.M)
                        yb[(int64_t)gm * a.ldy + gn] = v[r];
                }
            }
        }
        dg_lds_barrier();
    }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------

// packed int4 tensors (fmt 2, or fmt 4 with groups of 32, 64 or whole
// 128-input blocks)
static bool dg_ok(const coli_qtensor *W) {
    return mgemv_int4_ok(W) && W->I % 32 == 0;
}

size_t dgemm_ws_bytes(const coli_qtensor *W, int S) {
    if (!dg_ok(W) || S < 1)
        return 0;
    const int64_t nmt = (S + DG_TM - 1) / DG_TM, nkb4 = ((W->I + 127) / 128 + 3) / 4 * 4;
    return (size_t)(nmt * DG_MB * nkb4 * 4096);
}

// the arguments for matrix e of W's stack: y = W_e x over S rows, inputs
// prepared in ws
static DgArgs dg_args(const coli_qtensor *W, int e, int S, const void *ws, float *y) {
    const int nkb = (W->I + 127) / 128;
    DgArgs a;
    memset(&a, 0, sizeof a);
    a.xf = (const uint8_t *)ws;
    a.pq = (const uint8_t *)W->pk + (int64_t)e * W->pk_stride;
    a.ps = W->fmt == 4 ? (const float *)((const uint8_t *)W->pk + (int64_t)e * W->pk_stride + W->pk_scale_off)
                       : W->s + (int64_t)e * W->s_stride;
    a.xbytes = (int)dgemm_ws_bytes(W, S);
    a.qbytes = (int)W->pk_scale_off;
    a.sbytes = W->fmt == 4 ? (int)(W->pk_stride - W->pk_scale_off) : (int)(W->O * sizeof(float));
    a.nkb = nkb;
    a.nkq = (nkb + 3) / 4;
    a.cbs = (W->fmt != 4 || W->gs % 128 == 0) ? 1 : 128 / W->gs;
    a.gshift = (W->fmt == 4 && W->gs < 128) ? __builtin_ctz((unsigned)W->gs) : 5;
    a.rtn = (W->O + 15) / 16;
    a.Otot = W->O;
    a.M = S;
    a.N = W->O;
    a.nmt = (S + DG_TM - 1) / DG_TM;
    a.nnt = (W->O + DG_TN - 1) / DG_TN;
    a.y = y;
    a.ldy = W->O;
    return a;
}

static bool dg_launch_ok(const coli_qtensor *W, const float *x, int S, const void *ws, size_t ws_bytes) {
    return dg_ok(W) && S >= 1 && (uintptr_t)x % 16 == 0 && ws != nullptr && (uintptr_t)ws % 256 == 0 &&
           ws_bytes >= dgemm_ws_bytes(W, S) && dgemm_ws_bytes(W, S) < ((size_t)1 << 31);
}

static void dg_xprep(const coli_qtensor *W, const float *x, int S, void *ws, hipStream_t st) {
    const int nkb4 = ((W->I + 127) / 128 + 3) / 4 * 4;
    const int nmt = (S + DG_TM - 1) / DG_TM;
    hipLaunchKernelGGL(k_dg_xprep, dim3((unsigned)(nmt * DG_MB), (unsigned)nkb4), dim3(256), 0, st,
                       x, (int64_t)W->I, S, W->I, nkb4, (uint8_t *)ws, (int64_t)0, (int64_t)0);
}

int launch_dgemm(const coli_qtensor *W, const float *x, float *y, int S, void *ws, size_t ws_bytes,
                 hipStream_t st) {
    if (!dg_launch_ok(W, x, S, ws, ws_bytes))
        return 0;
    ProfScope ps("gemm_dense", st);
    // every matrix of a stack takes the same input rows
    dg_xprep(W, x, S, ws, st);
    for (int e = 0; e < W->n; ++e) {
        DgPair pr;
        pr.m[0] = dg_args(W, e, S, ws, y + (int64_t)e * S * W->O);
        pr.m[1] = pr.m[0];
        const dim3 grid((unsigned)(pr.m[0].nmt * pr.m[0].nnt));
        if (W->fmt == 4)
            hipLaunchKernelGGL(k_dg<DG_GRP>, grid, dim3(256), 0, st, pr);
        else
            hipLaunchKernelGGL(k_dg<DG_ROW>, grid, dim3(256), 0, st, pr);
    }
    return after_launch("gemm_dense") == COLI_OK ? 1 : -1;
}

int launch_dgemm_pair(const coli_qtensor *W1, const coli_qtensor *W2, const float *x, float *y1,
                      float *y2, int S, void *ws, size_t ws_bytes, hipStream_t st) {
    if (!dg_launch_ok(W1, x, S, ws, ws_bytes) || !dg_launch_ok(W2, x, S, ws, ws_bytes) ||
        W1->n != 1 || W2->n != 1 || W1->I != W2->I || (W1->fmt == 4) != (W2->fmt == 4))
        return 0;
    ProfScope ps("gemm_dense", st);
    dg_xprep(W1, x, S, ws, st);
    DgPair pr;
    pr.m[0] = dg_args(W1, 0, S, ws, y1);
    pr.m[1] = dg_args(W2, 0, S, ws, y2);
    // the larger tile count rounded to whole XCD rounds, so that workgroup
    // w of either matrix runs on XCD w % 8
    const int t1 = pr.m[0].nmt * pr.m[0].nnt, t2 = pr.m[1].nmt * pr.m[1].nnt;
    const int gx = ((t1 > t2 ? t1 : t2) + 7) / 8 * 8;
    const dim3 grid((unsigned)gx, 1u, 2u);
    if (W1->fmt == 4)
        hipLaunchKernelGGL(k_dg<DG_GRP>, grid, dim3(256), 0, st, pr);
    else
        hipLaunchKernelGGL(k_dg<DG_ROW>, grid, dim3(256), 0, st, pr);
    return after_launch("gemm_dense") == COLI_OK ? 1 : -1;
}

// Per-head products on row ranges of one packed matrix (the MLA value
// absorption: head h's value rows of kv_b times its latent context).
size_t dgemm_heads_ws_bytes(const coli_qtensor *W, int S, int nb) {
    if (nb < 1)
        return 0;
    return dgemm_ws_bytes(W, S) * (size_t)nb;
}

bool dgemm_heads_takes(const coli_qtensor *W, int row0, int row_step, int N, int nb, int S) {
    const size_t per = dgemm_ws_bytes(W, S);
    return dg_ok(W) && W->n == 1 && S >= 1 && nb >= 1 && N >= 1 && row0 % 16 == 0 &&
           row_step % 16 == 0 && row0 + (int64_t)(nb - 1) * row_step + N <= W->O && per > 0 &&
           per * nb < ((size_t)1 << 31);
}

int launch_dgemm_heads(const coli_qtensor *W, int row0, int row_step, int N, int nb, const float *x,
                       int64_t ldx, int64_t x_bstride, float *y, int64_t ldy, int64_t y_bstride, int S,
                       void *ws, size_t ws_bytes, hipStream_t st, bool prepared) {
    const size_t per = dgemm_ws_bytes(W, S);
    if (!dgemm_heads_takes(W, row0, row_step, N, nb, S) || ws == nullptr ||
        (uintptr_t)ws % 256 != 0 || ws_bytes < per * nb ||
        (!prepared && ((uintptr_t)x % 16 != 0 || ldx % 4 != 0 || x_bstride % 4 != 0)))
        return 0;
    ProfScope ps("gemm_heads", st);
    const int nkb = (W->I + 127) / 128, nkb4 = (nkb + 3) / 4 * 4;
    const int nmt = (S + DG_TM - 1) / DG_TM, nnt = (N + DG_TN - 1) / DG_TN;
    if (!prepared)
        hipLaunchKernelGGL(k_dg_xprep, dim3((unsigned)(nmt * DG_MB), (unsigned)nkb4, (unsigned)nb),
                           dim3(256), 0, st, x, ldx, S, W->I, nkb4, (uint8_t *)ws, x_bstride, (int64_t)per);
    DgArgs a;
    memset(&a, 0, sizeof a);
    a.xf = (const uint8_t *)ws;
    a.pq = (const uint8_t *)W->pk;
    a.ps = W->fmt == 4 ? (const float *)((const uint8_t *)W->pk + W->pk_scale_off) : W->s;
    a.xbytes = (int)(per * nb);
    a.qbytes = (int)W->pk_scale_off;
    a.sbytes = W->fmt == 4 ? (int)(W->pk_stride - W->pk_scale_off) : (int)(W->O * sizeof(float));
    a.nkb = nkb;
    a.nkq = (nkb + 3) / 4;
    a.cbs = (W->fmt != 4 || W->gs % 128 == 0) ? 1 : 128 / W->gs;
    a.gshift = (W->fmt == 4 && W->gs < 128) ? __builtin_ctz((unsigned)W->gs) : 5;
    a.rtn = (N + 15) / 16;
    a.Otot = W->O;
    a.M = S;
    a.N = N;
    a.nmt = nmt;
    a.nnt = nnt;
    a.y = y;
    a.ldy = ldy;
    a.xf_bstride = (int)per;
    a.rt0 = row0 / 16;
    a.rt_bstride = row_step / 16;
    a.y_bstride = y_bstride;
    const dim3 grid((unsigned)(nmt * nnt), (unsigned)nb);
    DgPair pr;
    pr.m[0] = a;
    pr.m[1] = a;
    if (W->fmt == 4)
        hipLaunchKernelGGL(k_dg<DG_GRP>, grid, dim3(256), 0, st, pr);
    else
        hipLaunchKernelGGL(k_dg<DG_ROW>, grid, dim3(256), 0, st, pr);
    return after_launch("gemm_heads") == COLI_OK ? 1 : -1;
}

}  // namespace coli
