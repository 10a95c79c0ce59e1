// mla.h -- the decode attention launcher (mla.hip) and its workspace layout.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/coli.h"

namespace coli {

// stage buffers inside the workspace, in this order (offsets are public via
// coli_mla_workspace_layout)
enum { MLA_CQ_RAW = 0, MLA_CKV_RAW, MLA_CQ, MLA_Q, MLA_QABS, MLA_QPE, MLA_SCORES, MLA_P, MLA_CLAT,
       MLA_CTX, MLA_NSTAGE };
static_assert(MLA_NSTAGE == COLI_MLA_STAGES, "stage count");

// key-absorption row splits per head (their partial sums sit in the workspace
// after the public stages)
constexpr int MLA_QA_SPLIT = 4;
// score splits over the L + d_rope components
constexpr int MLA_SC_SPLIT = 3;
// query rows per workgroup of the absorption kernels, and rows per launch set
// of the core (more rows: several sets in order; a multiple of MLA_CHUNK)
constexpr int MLA_CHUNK = 4;
#ifndef COLI_MLA_GROUP
#define COLI_MLA_GROUP 192
#endif
constexpr int MLA_GROUP = COLI_MLA_GROUP;
static_assert(MLA_GROUP % MLA_CHUNK == 0, "whole chunks per group");

struct MlaLayout {
    size_t off[MLA_NSTAGE];
    size_t qabs_part, sc_part, cl_part;  // partial sums (internal)
    size_t xprep, xprep_bytes;           // prefill rows: the projections' prepared inputs
    size_t total;
};
// proj_ws: bytes the prefill projections' prepared inputs take (mla_proj_ws)
MlaLayout mla_layout(int S, int H, int dn, int dr, int dv, int qr, int L, int Tcap, size_t proj_ws);
size_t mla_proj_ws(const coli_mla_layer &m, int S);

// kv_b's codes and scales as the absorption kernels read them
struct MlaKvb {
    const uint8_t *q;
    const float *s;
    int64_t rb;  // bytes per row
    int ng, gs;  // fmt 4 groups per row and group size (fmt 2: 1, 1)
};

struct MlaArgs {
    const coli_mla_layer *layer;
    const float *x;
    int S, pos_base, T_cap;
    float *Lc, *Rc, *out;
    void *ws;
    hipStream_t st;
    // decode layer: also hsum = resid + out (the residual add after the
    // attention), in o_proj's epilogue when the matrix-core kernel runs it
    const float *resid = nullptr;
    float *hsum = nullptr;
    // decode layer: x is the layer input; the attention's input is its
    // RMSNorm with in_norm_w (may be NULL) and in_eps, written to xn --
    // folded into the q_a / kv_a launch when the matrix-core kernel runs it
    bool in_norm = false;
    const float *in_norm_w = nullptr;
    double in_eps = 0.0;
    float *xn = nullptr;
};
int launch_mla_decode(const MlaArgs &a);

}  // namespace coli
