// common.h -- internal declarations of libcoli (gfx950 HIP).  Not part of the
// public ABI (include/coli.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/coli.h"

namespace coli {

// ---------------------------------------------------------------------------
// Host-side plumbing shared by the launchers
// ---------------------------------------------------------------------------

// Record a declined call: sets the thread's reason and returns COLI_DECLINED.
int decline(const char *fmt, ...);
// Record a HIP error: sets the thread's error text and returns COLI_HIP_ERROR.
int hip_fail(hipError_t e, const char *where);
// Check hipGetLastError after a launch; counts the launch.
int after_launch(const char *tag);

// Profiling scope: records HIP events around one kernel launch when enabled.
struct ProfScope {
    int slot;
    hipStream_t stream;
    bool ext;
    // ext: the launch records the events itself (hipExtLaunchKernelGGL start
    // and stop events, stamped by the dispatch), which times the kernel alone
    ProfScope(const char *tag, hipStream_t s, bool ext = false);
    ~ProfScope();
    hipEvent_t start() const;  // nullptr unless profiling (ext mode)
    hipEvent_t stop() const;
};

// Flags stored in coli_qtensor::flags by coli_tensor_upload.
enum : uint32_t {
    QF_FAST = 1u,     // packet loads allowed: aligned rows, row_bytes % packet == 0
    QF_GROUP32 = 2u,  // fmt 4: gs % 32 == 0 (one scale per 32-input packet)
    QF_GROUP16 = 4u,  // fmt 4: gs % 16 == 0 but not 32 (two scales per packet)
    QF_PACKED = 8u,   // carries a packed copy (coli_tensor_pack)
};

constexpr uint32_t QT_MAGIC = 0xC0117E45u;

// Bytes of one packet (the unit a lane loads) and inputs it covers.
__host__ __device__ constexpr int packet_bytes(int fmt) { return fmt == 3 ? 8 : 16; }
__host__ __device__ constexpr int packet_cols(int fmt) { return fmt == 1 ? 16 : 32; }

// Launchers (defined in gemv.hip / gemm.hip / route.hip).
int launch_dequant(const coli_qtensor *W, float *w, hipStream_t st);
// y = W x; with radd and ysum also ysum = radd + y (a residual add, in the
// matrix-core kernel's epilogue when that kernel runs)
int launch_gemv(const coli_qtensor *W, const float *x, float *y, int S, hipStream_t st,
                const float *radd = nullptr, float *ysum = nullptr);
// an RMSNorm applied to a GEMV's input rows as they are staged: x * inv * w
// (w may be NULL: 1), inv = 1 / sqrt(mean x^2 + eps) per row in f64; the
// normalised rows [S][I] are written to xn
struct InNorm {
    const float *w;
    double eps;
    float *xn;
};
int launch_gemm(const coli_qtensor *W, const float *x, float *y, int S, void *ws, size_t ws_bytes,
                hipStream_t st);
size_t gemm_workspace_bytes(int S, int I);
int launch_route(const int32_t *ids, int S, int K, int E, int32_t *counts, int32_t *offsets,
                 int32_t *perm, int32_t *n_bad, int32_t *inv, int32_t *tiles, int32_t *n_tiles,
                 int bm, int shared_rows, hipStream_t st, int32_t *tiles_s = nullptr,
                 int32_t *n_tiles_s = nullptr, int bm_s = 0);

struct MoeArgs {
    const coli_qtensor *gate, *up, *down;
    const coli_qtensor *sg, *su, *sd;  // shared triple or NULLs
    const float *x;
    int S, K, E, F, D;
    const int32_t *ids;
    const float *w;
    float *out;    // NULL for hidden-only
    float *h_out;  // hidden-only destination (f32) or NULL
    void *ws;
    size_t ws_bytes;
    hipStream_t st;
    // decode layer: also out_res = resid + out (the residual add), folded
    // into the combine when the matrix-core kernels run, else a launch of its
    // own (S <= 4 only)
    const float *resid = nullptr;
    float *out_res = nullptr;
};
int launch_moe_decode(const MoeArgs &a);
int launch_moe_prefill(const MoeArgs &a);
// router logits (f64, into ws) and exact top-K (router.hip)
size_t router_ws_bytes(int S, int E);
int launch_router(const float *x, int S, int D, const float *R, const float *bias, int E, int K,
                  float topp, int norm_topk, float routed_scale, int32_t *ids, float *w, void *ws,
                  hipStream_t st);
// RMSNorm (weights lnw, may be NULL) of h into xn, then the router on xn
int launch_norm_router(const float *h, int S, int D, const float *lnw, double eps, float *xn,
                       const float *R, const float *bias, int E, int K, float topp, int norm_topk,
                       float routed_scale, int32_t *ids, float *w, void *ws, hipStream_t st);
size_t moe_decode_ws_bytes(int S, int K, int F, int D, int has_shared);
// matrix-core decode kernels (mgemv.hip); return 1 done, 0 not taken, <0 error
bool mgemv_ok(const coli_qtensor *W);
bool mgemv_int4_ok(const coli_qtensor *W);
size_t packed_bytes(int fmt, int n, int O, int I, int gs);
int launch_pack(coli_qtensor *t, void *packed, hipStream_t st);
int launch_mgemv(const coli_qtensor *W, const float *x, float *y, int S, hipStream_t st,
                 const float *radd = nullptr, float *ysum = nullptr, const InNorm *nrm = nullptr);
int launch_mgemv_group(int n, const coli_qtensor *const *W, const float *const *x,
                       float *const *y, int S, hipStream_t st, const InNorm *nrm = nullptr);
int launch_mgemv_moe(const MoeArgs &m, float *h, float *yp, int *cnt);
// prefill GEMM on the matrix cores for the int4 formats (pgemm.hip); 1 done,
// 0 not taken, <0 error
bool pgemm_ok(const coli_qtensor *W);
int launch_pgemm_dense(const coli_qtensor *W, const float *x, float *y, int S, hipStream_t st);
// prefill MoE on the matrix cores: routed tiles of pgemm_moe_rows(m) rows
// (0: neither kernel takes these tensors; tile list, counts and offsets from
// launch_route), bf16 gathered inputs xg, bf16 SiLU products hg, f32 down
// rows y (skipped when y is null)
constexpr int PG_MOE_ROWS = 64;         // producer/consumer kernel
#ifndef COLI_SG_ROWS
#define COLI_SG_ROWS 32
#endif
constexpr int PG_MOE_ROWS_PACKED = COLI_SG_ROWS;  // weight-streaming kernel (packed copies)
// experts with 1 .. PG_MOE_ROWS_SHORT rows take one tile of that many rows in
// the weight-streaming kernel instead of a PG_MOE_ROWS_PACKED-row tile (0: off)
#ifndef COLI_SG_SHORT_ROWS
#define COLI_SG_SHORT_ROWS 16
#endif
constexpr int PG_MOE_ROWS_SHORT = COLI_SG_SHORT_ROWS;
int pgemm_moe_rows(const MoeArgs &m);
int launch_pgemm_moe(const MoeArgs &m, int rows, const void *xg, void *hg, float *y,
                     const int32_t *tiles, const int32_t *n_tiles, const int32_t *counts,
                     const int32_t *offsets, int max_tiles, const int32_t *tiles_s = nullptr,
                     const int32_t *n_tiles_s = nullptr, int max_short = 0);
// 0: matrix-core decode kernels where the layout allows, 1: vector-ALU kernels only
int decode_kernel_mode();
size_t moe_prefill_ws_bytes(int E, int S, int K, int F, int D, int has_shared);

// ---------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------

// Signed byte k of v converted to f32 in one SDWA instruction.
template <int K>
__device__ __forceinline__ float sbyte(uint32_t v);
template <>
__device__ __forceinline__ float sbyte<0>(uint32_t v) {
    float r;
    asm("v_cvt_f32_i32_sdwa %0, sext(%1) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_0"
        : "=v"(r) : "v"(v));
    return r;
}
template <>
__device__ __forceinline__ float sbyte<1>(uint32_t v) {
    float r;
    asm("v_cvt_f32_i32_sdwa %0, sext(%1) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_1"
        : "=v"(r) : "v"(v));
    return r;
}
template <>
__device__ __forceinline__ float sbyte<2>(uint32_t v) {
    float r;
    asm("v_cvt_f32_i32_sdwa %0, sext(%1) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_2"
        : "=v"(r) : "v"(v));
    return r;
}
template <>
__device__ __forceinline__ float sbyte<3>(uint32_t v) {
    float r;
    asm("v_cvt_f32_i32_sdwa %0, sext(%1) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_3"
        : "=v"(r) : "v"(v));
    return r;
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Pointers into global memory (address space 1), so loads through them are
// global_load (vector-memory counter only) rather than flat loads, which
// would also hold up the LDS counter.
#define COLI_GLOBAL __attribute__((address_space(1)))

template <typename T>
__device__ __forceinline__ T gload(const void *p) {
    return *(const COLI_GLOBAL T *)(p);
}

// Packet of codes as loaded by one lane (streamed once: non-temporal loads).
template <int FMT>
struct Packet { u32x4 v; };
template <>
struct Packet<3> { u32x2 v; };

template <int FMT>
__device__ __forceinline__ Packet<FMT> load_packet(const uint8_t *p) {
    Packet<FMT> k;
    k.v = __builtin_nontemporal_load((const COLI_GLOBAL u32x4 *)p);
    return k;
}
template <>
__device__ __forceinline__ Packet<3> load_packet<3>(const uint8_t *p) {
    Packet<3> k;
    k.v = __builtin_nontemporal_load((const COLI_GLOBAL u32x2 *)p);
    return k;
}

// The decoded value of every input of a packet is MULT * v exactly, with
//   fmt 2/4: v = nibble - 8, MULT 16  (nibble ^ 8 is v in 4-bit two's
//            complement; moved to the top of a byte it reads as 16*v)
//   fmt 3:   v = code - 2,   MULT 64  (code ^ 2, moved to the top two bits)
//   fmt 1:   v = int8 byte,  MULT 1
template <int FMT>
struct Mult { static constexpr float value = 1.0f; };
template <>
struct Mult<2> { static constexpr float value = 16.0f; };
template <>
struct Mult<4> { static constexpr float value = 16.0f; };
template <>
struct Mult<3> { static constexpr float value = 64.0f; };

// Decode a packet into f[packet_cols] (input order), values MULT * v.
template <int FMT>
__device__ __forceinline__ void decode_packet(const Packet<FMT> &k, float *f);

__device__ __forceinline__ void decode_nib_word(uint32_t w, float *f) {
    // byte b holds inputs 2b (low nibble) and 2b+1 (high nibble)
    const uint32_t a = w ^ 0x88888888u;
    const uint32_t hi = a & 0xF0F0F0F0u;
    const uint32_t lo = (a << 4) & 0xF0F0F0F0u;
    f[0] = sbyte<0>(lo); f[1] = sbyte<0>(hi);
    f[2] = sbyte<1>(lo); f[3] = sbyte<1>(hi);
    f[4] = sbyte<2>(lo); f[5] = sbyte<2>(hi);
    f[6] = sbyte<3>(lo); f[7] = sbyte<3>(hi);
}

template <>
__device__ __forceinline__ void decode_packet<4>(const Packet<4> &k, float *f) {
    decode_nib_word(k.v.x, f + 0);
    decode_nib_word(k.v.y, f + 8);
    decode_nib_word(k.v.z, f + 16);
    decode_nib_word(k.v.w, f + 24);
}
template <>
__device__ __forceinline__ void decode_packet<2>(const Packet<2> &k, float *f) {
    decode_nib_word(k.v.x, f + 0);
    decode_nib_word(k.v.y, f + 8);
    decode_nib_word(k.v.z, f + 16);
    decode_nib_word(k.v.w, f + 24);
}

__device__ __forceinline__ void decode_i8_word(uint32_t w, float *f) {
    f[0] = sbyte<0>(w); f[1] = sbyte<1>(w); f[2] = sbyte<2>(w); f[3] = sbyte<3>(w);
}
template <>
__device__ __forceinline__ void decode_packet<1>(const Packet<1> &k, float *f) {
    decode_i8_word(k.v.x, f + 0);
    decode_i8_word(k.v.y, f + 4);
    decode_i8_word(k.v.z, f + 8);
    decode_i8_word(k.v.w, f + 12);
}

__device__ __forceinline__ void decode_i2_word(uint32_t w, float *f) {
    // byte b holds inputs 4b..4b+3, lowest bits first
    const uint32_t a = w ^ 0xAAAAAAAAu;
    const uint32_t c0 = (a << 6) & 0xC0C0C0C0u;
    const uint32_t c1 = (a << 4) & 0xC0C0C0C0u;
    const uint32_t c2 = (a << 2) & 0xC0C0C0C0u;
    const uint32_t c3 = a & 0xC0C0C0C0u;
    f[0] = sbyte<0>(c0); f[1] = sbyte<0>(c1); f[2] = sbyte<0>(c2); f[3] = sbyte<0>(c3);
    f[4] = sbyte<1>(c0); f[5] = sbyte<1>(c1); f[6] = sbyte<1>(c2); f[7] = sbyte<1>(c3);
    f[8] = sbyte<2>(c0); f[9] = sbyte<2>(c1); f[10] = sbyte<2>(c2); f[11] = sbyte<2>(c3);
    f[12] = sbyte<3>(c0); f[13] = sbyte<3>(c1); f[14] = sbyte<3>(c2); f[15] = sbyte<3>(c3);
}
template <>
__device__ __forceinline__ void decode_packet<3>(const Packet<3> &k, float *f) {
    decode_i2_word(k.v.x, f + 0);
    decode_i2_word(k.v.y, f + 16);
}

// Sum over the 64 lanes of a wavefront (every lane receives the total).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        v += __shfl_xor(v, off, 64);
    return v;
}

}  // namespace coli
