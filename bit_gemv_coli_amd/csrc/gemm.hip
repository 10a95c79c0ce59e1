// gemm.hip -- prefill path (S > 4): bf16 matrix-core GEMM.  Placeholder that
// serves the dense case with the fp32 packet GEMV in blocks of four rows.
#include "common.h"

namespace coli {

size_t gemm_workspace_bytes(int S, int I) { (void)S; (void)I; return 0; }

int launch_gemm(const coli_qtensor *W, const float *x, float *y, int S, void *ws, size_t ws_bytes,
                hipStream_t st) {
    (void)ws; (void)ws_bytes;
    return launch_gemv(W, x, y, S, st);
}

size_t moe_prefill_ws_bytes(int E, int S, int K, int F, int D, int has_shared) {
    (void)E;
    return moe_decode_ws_bytes(S, K, F, D, has_shared);
}

int launch_moe_prefill(const MoeArgs &a) {
    (void)a;
    return decline("moe_block: the S > 4 prefill path is not available in this build");
}

}  // namespace coli
