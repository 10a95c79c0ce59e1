// abi.hip -- the extern "C" entry points of libcoli: validation, dispatch,
// diagnostics.  Conventions (colibri PR #298, commit making the CUDA ABI return
// 0 for fmt=4: a declined call is a fallback, not a wrong result; issue #585 thread: silent
// fallbacks mislead, so every refusal names its reason; colibri PR #298, HIP
// single-source merge: a fault-injection control proves GPU calls executed):
//   * every entry validates everything it can see on the host before enqueuing
//     any work; a refusal returns COLI_DECLINED, writes nothing, and records
//     the reason (coli_last_reason, and on stderr when COLI_NOTICE=1);
//   * COLI_FAIL_AFTER=n makes every compute call after the first n decline.
#include <atomic>
#include <mutex>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include <string>
#include <vector>

#include "common.h"
#include "layer.h"
#include "dgemm.h"
#include "mla.h"

namespace coli {

static thread_local char g_reason[512];
static thread_local char g_error[512];
static std::atomic<uint64_t> g_calls{0}, g_declined{0}, g_launches{0};
static std::atomic<int64_t> g_fail_after{-2};  // -2: not read from env yet
static std::atomic<int> g_gemv_max{0};
static std::atomic<int> g_decode_mode{-1};

int decode_kernel_mode() {
    int v = g_decode_mode.load();
    if (v < 0) {
        const char *e = getenv("COLI_DECODE_KERNEL");
        v = (e && strcmp(e, "valu") == 0) ? 1 : 0;
        int z = -1;
        g_decode_mode.compare_exchange_strong(z, v);
        v = g_decode_mode.load();
    }
    return v;
}
static int g_notice = -1;

static void notice(const char *what, const char *msg) {
    if (g_notice < 0) {
        const char *e = getenv("COLI_NOTICE");
        g_notice = (e && atoi(e) > 0) ? 1 : 0;
    }
    if (g_notice)
        fprintf(stderr, "[coli] %s: %s\n", what, msg);
}

int decline(const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_reason, sizeof g_reason, fmt, ap);
    va_end(ap);
    g_declined.fetch_add(1);
    notice("declined", g_reason);
    return COLI_DECLINED;
}

int hip_fail(hipError_t e, const char *where) {
    snprintf(g_error, sizeof g_error, "%s: %s", where, hipGetErrorString(e));
    notice("hip error", g_error);
    return COLI_HIP_ERROR;
}

int after_launch(const char *tag) {
    g_launches.fetch_add(1);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return hip_fail(e, tag);
    return COLI_OK;
}

// --- profiling -------------------------------------------------------------

struct ProfRec {
    std::string tag;
    hipEvent_t a, b;
};
static std::mutex g_prof_mu;
static bool g_prof_on = false;
static std::vector<ProfRec> g_prof;       // recorded launches
static std::vector<hipEvent_t> g_evpool;  // free events
static std::vector<std::string> g_tags;   // distinct tags seen

static hipEvent_t take_event() {
    if (!g_evpool.empty()) {
        hipEvent_t e = g_evpool.back();
        g_evpool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess)
        return nullptr;
    return e;
}

ProfScope::ProfScope(const char *tag, hipStream_t s, bool ext_) : slot(-1), stream(s), ext(ext_) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    if (!g_prof_on)
        return;
    ProfRec r;
    r.tag = tag;
    r.a = take_event();
    r.b = take_event();
    if (!r.a || !r.b)
        return;
    bool known = false;
    for (auto &t : g_tags) known |= (t == r.tag);
    if (!known) g_tags.push_back(r.tag);
    if (!ext)
        (void)hipEventRecord(r.a, s);
    slot = (int)g_prof.size();
    g_prof.push_back(r);
}

ProfScope::~ProfScope() {
    if (slot < 0 || ext)
        return;
    std::lock_guard<std::mutex> lk(g_prof_mu);
    if (slot < (int)g_prof.size())
        (void)hipEventRecord(g_prof[slot].b, stream);
}

hipEvent_t ProfScope::start() const {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    return (ext && slot >= 0 && slot < (int)g_prof.size()) ? g_prof[slot].a : nullptr;
}

hipEvent_t ProfScope::stop() const {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    return (ext && slot >= 0 && slot < (int)g_prof.size()) ? g_prof[slot].b : nullptr;
}

static bool gate_call() {
    g_calls.fetch_add(1);
    int64_t f = g_fail_after.load();
    if (f == -2) {
        const char *e = getenv("COLI_FAIL_AFTER");
        int64_t v = e ? atoll(e) : -1;
        int64_t expect = -2;
        g_fail_after.compare_exchange_strong(expect, v);
        f = g_fail_after.load();
    }
    if (f < 0)
        return true;
    if (f == 0) {
        decline("fault injection (COLI_FAIL_AFTER) tripped");
        return false;
    }
    g_fail_after.fetch_sub(1);
    return true;
}

// --- validation ------------------------------------------------------------

static int check_qt(const coli_qtensor *t, const char *name) {
    if (!t)
        return decline("%s: NULL tensor", name);
    if (t->magic != QT_MAGIC)
        return decline("%s: not filled by coli_tensor_upload", name);
    return COLI_OK;
}

static bool dev_aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Device scratch of coli_moe_block_noalloc: one array per GPU (every device
// the library runs on holds its own copy until the process ends).  The host
// name `scratch` is a host-side stand-in, not a device address; the device
// address comes from hipGetSymbolAddress, taken once per device with that
// device current, and only that address is ever passed to kernels.
static __device__ __align__(256) unsigned char scratch[COLI_NOALLOC_SCRATCH_BYTES];

constexpr int SCRATCH_MAX_DEVICES = 64;
static std::mutex g_scratch_mu;
static void *g_scratch_ptr[SCRATCH_MAX_DEVICES];

// COLI_OK with *out = this device's scratch address, or the decline / error
static int scratch_on_current_device(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= SCRATCH_MAX_DEVICES)
        return decline("moe_block_noalloc: device %d beyond the %d the scratch table covers", dev,
                       SCRATCH_MAX_DEVICES);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (p == nullptr)
            return hip_fail(hipErrorInvalidSymbol, "hipGetSymbolAddress(scratch) gave NULL");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return COLI_OK;
}

}  // namespace coli

using namespace coli;

extern "C" {

const char *coli_version(void) { return "libcoli 0.1 (gfx950)"; }

const char *coli_last_reason(void) { return g_reason; }
const char *coli_last_error(void) { return g_error; }

void coli_stats(uint64_t *calls, uint64_t *declined, uint64_t *launches) {
    if (calls) *calls = g_calls.load();
    if (declined) *declined = g_declined.load();
    if (launches) *launches = g_launches.load();
}

void coli_set_fail_after(int64_t n) { g_fail_after.store(n < 0 ? -1 : n); }

int coli_gemv_max_rows(void) {
    int v = g_gemv_max.load();
    if (v == 0) {
        const char *e = getenv("COLI_GEMV_MAX_ROWS");
        v = e ? atoi(e) : 4;
        if (v < 1 || v > 4) v = 4;
        int z = 0;
        g_gemv_max.compare_exchange_strong(z, v);
        v = g_gemv_max.load();
    }
    return v;
}

int coli_set_decode_kernel(int mode) {
    if (mode != 0 && mode != 1)
        return -1;
    const int old = decode_kernel_mode();
    g_decode_mode.store(mode);
    return old;
}

int coli_set_gemv_max_rows(int s) {
    if (s < 1 || s > 4)
        return 0;
    const int old = coli_gemv_max_rows();
    g_gemv_max.store(s);
    return old;
}

void coli_prof_enable(int on) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_prof_on = on != 0;
}

void coli_prof_reset(void) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    for (auto &r : g_prof) {
        g_evpool.push_back(r.a);
        g_evpool.push_back(r.b);
    }
    g_prof.clear();
}

int64_t coli_prof_read(const char *tag, double *total_ms) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    if (!tag)
        return -1;
    double sum = 0.0;
    int64_t n = 0;
    for (auto &r : g_prof) {
        if (r.tag != tag)
            continue;
        if (hipEventQuery(r.b) != hipSuccess)
            continue;
        float ms = 0.f;
        if (hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess)
            continue;
        sum += ms;
        ++n;
    }
    if (total_ms) *total_ms = sum;
    return n;
}

const char *coli_prof_tag(int i) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    if (i < 0 || i >= (int)g_tags.size())
        return nullptr;
    return g_tags[i].c_str();
}

int coli_tensor_upload(coli_qtensor *t, int fmt, int n, int O, int I, int gs, int ng,
                       const void *q_dev, const float *s_dev) {
    if (!t)
        return decline("tensor_upload: NULL record");
    if (fmt < 1 || fmt > 4)
        return decline("tensor_upload: unknown fmt %d (supported: 1 int8/row, 2 int4/row, "
                       "3 int2/row, 4 grouped int4)", fmt);
    if (n < 1 || O < 1 || I < 1)
        return decline("tensor_upload: bad shape n=%d O=%d I=%d", n, O, I);
    if ((int64_t)n * O > (int64_t)INT32_MAX / 2)
        return decline("tensor_upload: n*O=%lld too large", (long long)n * O);
    if (!q_dev || !s_dev)
        return decline("tensor_upload: NULL codes or scales");
    if (!dev_aligned(s_dev, 4))
        return decline("tensor_upload: scales not 4-byte aligned");
    if (fmt == 4) {
        if (gs < 1)
            return decline("tensor_upload: fmt 4 needs gs >= 1 (got %d)", gs);
        const int want = (int)(((int64_t)I + gs - 1) / gs);
        if (ng != want)
            return decline("tensor_upload: ng=%d but ceil(I/gs)=%d (I=%d gs=%d)", ng, want, I, gs);
    } else {
        if (gs != 0)
            return decline("tensor_upload: fmt %d has per-row scales; gs must be 0 (got %d)",
                           fmt, gs);
        if (ng != 1)
            return decline("tensor_upload: fmt %d has per-row scales; ng must be 1 (got %d)",
                           fmt, ng);
    }
    coli_qtensor r;
    memset(&r, 0, sizeof r);
    r.fmt = fmt;
    r.n = n;
    r.O = O;
    r.I = I;
    r.gs = gs;
    r.ng = ng;
    r.row_bytes = fmt == 1 ? I : (fmt == 3 ? ((int64_t)I + 3) / 4 : ((int64_t)I + 1) / 2);
    r.q_stride = (int64_t)O * r.row_bytes;
    r.s_stride = (int64_t)O * ng;
    r.q = q_dev;
    r.s = s_dev;
    r.magic = QT_MAGIC;
    const int pb = packet_bytes(fmt), pc = packet_cols(fmt);
    if (I % pc == 0 && r.row_bytes % pb == 0 && dev_aligned(q_dev, pb))
        r.flags |= QF_FAST;
    if (fmt == 4) {
        if (gs % 32 == 0)
            r.flags |= QF_GROUP32;
        else if (gs % 16 == 0)
            r.flags |= QF_GROUP16;
    }
    *t = r;
    return COLI_OK;
}

size_t coli_packed_bytes(int fmt, int n, int O, int I, int gs) {
    return packed_bytes(fmt, n, O, I, gs);
}

int coli_tensor_pack(coli_qtensor *t, void *packed, size_t bytes, void *stream) {
    if (check_qt(t, "tensor_pack") != COLI_OK)
        return COLI_DECLINED;
    const size_t need = packed_bytes(t->fmt, t->n, t->O, t->I, t->gs);
    if (need == 0)
        return decline("tensor_pack: no packed form for fmt %d, I=%d, gs=%d (needs fmt 2/4, "
                       "I %% 32 == 0, gs 32, 64 or a multiple of 128)", t->fmt, t->I, t->gs);
    if (!(t->flags & QF_FAST))
        return decline("tensor_pack: codes not 16-byte aligned");
    if (!packed || !dev_aligned(packed, 256))
        return decline("tensor_pack: packed buffer NULL or not 256-byte aligned");
    if (bytes < need)
        return decline("tensor_pack: packed buffer %zu bytes < %zu needed", bytes, need);
    if (!gate_call())
        return COLI_DECLINED;
    return launch_pack(t, packed, (hipStream_t)stream);
}

int coli_dequantize(const coli_qtensor *W, float *w_out, void *stream) {
    if (check_qt(W, "dequantize") != COLI_OK)
        return COLI_DECLINED;
    if (!w_out)
        return decline("dequantize: NULL output");
    if (!gate_call())
        return COLI_DECLINED;
    return launch_dequant(W, w_out, (hipStream_t)stream);
}

int coli_qmatmul(const coli_qtensor *W, const float *x, float *y, int S, void *stream) {
    if (check_qt(W, "qmatmul") != COLI_OK)
        return COLI_DECLINED;
    if (!x || !y)
        return decline("qmatmul: NULL x or y");
    if (S < 1)
        return decline("qmatmul: S=%d < 1", S);
    if (!dev_aligned(x, 4) || !dev_aligned(y, 4))
        return decline("qmatmul: x or y not 4-byte aligned");
    if (!gate_call())
        return COLI_DECLINED;
    if (S <= coli_gemv_max_rows())
        return launch_gemv(W, x, y, S, (hipStream_t)stream);
    return launch_gemm(W, x, y, S, nullptr, 0, (hipStream_t)stream);
}

size_t coli_qmatmul_workspace_bytes(const coli_qtensor *W, int S) {
    if (!W || S <= coli_gemv_max_rows())
        return 0;
    return dgemm_ws_bytes(W, S);
}

int coli_qmatmul_ws(const coli_qtensor *W, const float *x, float *y, int S, void *workspace,
                    size_t ws_bytes, void *stream) {
    if (check_qt(W, "qmatmul_ws") != COLI_OK)
        return COLI_DECLINED;
    if (!x || !y)
        return decline("qmatmul_ws: NULL x or y");
    if (S < 1)
        return decline("qmatmul_ws: S=%d < 1", S);
    if (!dev_aligned(x, 4) || !dev_aligned(y, 4))
        return decline("qmatmul_ws: x or y not 4-byte aligned");
    if (!gate_call())
        return COLI_DECLINED;
    if (S <= coli_gemv_max_rows())
        return launch_gemv(W, x, y, S, (hipStream_t)stream);
    const int r = launch_dgemm(W, x, y, S, workspace, ws_bytes, (hipStream_t)stream);
    if (r != 0)
        return r > 0 ? COLI_OK : COLI_HIP_ERROR;
    return launch_gemm(W, x, y, S, nullptr, 0, (hipStream_t)stream);
}

int coli_qmatmul_group(int n, const coli_qtensor *const *W, const float *const *x,
                       float *const *y, int S, void *stream) {
    if (n < 1 || n > COLI_GROUP_MAX || !W || !x || !y)
        return decline("qmatmul_group: n=%d outside 1..%d or NULL array", n, COLI_GROUP_MAX);
    if (S < 1)
        return decline("qmatmul_group: S=%d < 1", S);
    for (int g = 0; g < n; ++g) {
        if (check_qt(W[g], "qmatmul_group") != COLI_OK)
            return COLI_DECLINED;
        if (!x[g] || !y[g])
            return decline("qmatmul_group: NULL x or y of member %d", g);
        if (!dev_aligned(x[g], 4) || !dev_aligned(y[g], 4))
            return decline("qmatmul_group: x or y of member %d not 4-byte aligned", g);
    }
    if (!gate_call())
        return COLI_DECLINED;
    const hipStream_t st = (hipStream_t)stream;
    if (S <= coli_gemv_max_rows() && decode_kernel_mode() == 0) {
        const int r = launch_mgemv_group(n, W, x, y, S, st);
        if (r == 1)
            return COLI_OK;
        if (r < 0)
            return COLI_HIP_ERROR;
    }
    // not one launch (format mix, no packed copy, stacks, S > 4): member by member
    for (int g = 0; g < n; ++g) {
        const int rc = S <= coli_gemv_max_rows() ? launch_gemv(W[g], x[g], y[g], S, st)
                                                 : launch_gemm(W[g], x[g], y[g], S, nullptr, 0, st);
        if (rc != COLI_OK)
            return rc;
    }
    return COLI_OK;
}

int coli_moe_route(const int32_t *ids, int S, int K, int E, int32_t *counts, int32_t *offsets,
                   int32_t *perm, int32_t *n_bad, void *stream) {
    if (!ids || !counts || !offsets || !perm || !n_bad)
        return decline("moe_route: NULL pointer");
    if (S < 0 || K < 1 || E < 1 || E > 4096)
        return decline("moe_route: bad S=%d K=%d E=%d (E must be 1..4096)", S, K, E);
    if ((int64_t)S * K > INT32_MAX / 4)
        return decline("moe_route: S*K too large");
    if (!gate_call())
        return COLI_DECLINED;
    return launch_route(ids, S, K, E, counts, offsets, perm, n_bad, nullptr, nullptr, nullptr, 0,
                        0, (hipStream_t)stream);
}

size_t coli_moe_router_workspace_bytes(int S, int E) {
    if (S < 1 || E < 1)
        return 0;
    return router_ws_bytes(S, E);
}

int coli_moe_router(const float *x, int S, int D, const float *R, const float *bias, int E, int K,
                    float topp, int norm_topk, float routed_scale, int32_t *ids, float *w,
                    void *workspace, size_t ws_bytes, void *stream) {
    if (!x || !R || !ids || !w || !workspace)
        return decline("moe_router: NULL pointer (only bias may be NULL)");
    if (S < 1 || D < 1 || E < 1 || E > 512 || K < 1 || K > 16 || K > E)
        return decline("moe_router: bad S=%d D=%d E=%d K=%d (E 1..512, K 1..min(16,E))", S, D, E, K);
    if (!(topp >= 0.0f && topp <= 1.0f) || !(routed_scale == routed_scale))
        return decline("moe_router: topp must lie in [0,1] and routed_scale must be a number");
    if ((uintptr_t)workspace % 8 != 0 || ws_bytes < router_ws_bytes(S, E))
        return decline("moe_router: workspace %zu bytes (8-byte aligned) < %zu needed", ws_bytes,
                       router_ws_bytes(S, E));
    if ((int64_t)S * D > INT32_MAX || (int64_t)E * D > INT32_MAX)
        return decline("moe_router: S*D or E*D too large");
    if (!gate_call())
        return COLI_DECLINED;
    return launch_router(x, S, D, R, bias, E, K, topp, norm_topk, routed_scale, ids, w, workspace,
                         (hipStream_t)stream);
}

size_t coli_moe_workspace_bytes(int E, int S, int K, int F, int Dm, int has_shared) {
    if (E < 1 || S < 1 || K < 1 || F < 1 || Dm < 1)
        return 0;
    if (S <= coli_gemv_max_rows())
        return moe_decode_ws_bytes(S, K, F, Dm, has_shared);
    return moe_prefill_ws_bytes(E, S, K, F, Dm, has_shared);
}

static int check_moe(const coli_qtensor *gate, const coli_qtensor *up, const coli_qtensor *down,
                     const float *x, int S, const int32_t *ids, int K,
                     const coli_qtensor *sg, const coli_qtensor *su, const coli_qtensor *sd,
                     const char *who) {
    // down / sd may be NULL for the hidden-only entry point
    if (gate == nullptr || gate->magic != QT_MAGIC) return decline("%s: bad gate tensor", who);
    if (up == nullptr || up->magic != QT_MAGIC) return decline("%s: bad up tensor", who);
    if (down != nullptr && down->magic != QT_MAGIC) return decline("%s: bad down tensor", who);
    if (!x || !ids)
        return decline("%s: NULL x or ids", who);
    if (S < 1 || K < 1 || K > 64)
        return decline("%s: bad S=%d K=%d (K must be 1..64)", who, S, K);
    const int E = gate->n, F = gate->O, D = gate->I;
    if (E > 4096)
        return decline("%s: E=%d > 4096", who, E);
    if (up->n != E || up->O != F || up->I != D)
        return decline("%s: up [%d][%d][%d] != gate [%d][%d][%d]", who, up->n, up->O, up->I, E, F, D);
    if (down && (down->n != E || down->O != D || down->I != F))
        return decline("%s: down [%d][%d][%d] must be [%d][%d][%d]", who, down->n, down->O,
                       down->I, E, D, F);
    const coli_qtensor *all[6] = {gate, up, down, sg, su, sd};
    // without a down stack (hidden-only) the shared down matrix is not needed
    const int nsh = (sg != nullptr) + (su != nullptr) + (down ? (sd != nullptr) : (sg != nullptr));
    if (nsh != 0 && nsh != 3)
        return decline("%s: shared expert needs all of its matrices", who);
    for (int i = 0; i < 6; ++i) {
        const coli_qtensor *t = all[i];
        if (!t) continue;
        if (t->magic != QT_MAGIC)
            return decline("%s: tensor %d not filled by coli_tensor_upload", who, i);
        if (t->fmt != gate->fmt)
            return decline("%s: tensor %d has fmt %d, gate has fmt %d (one format per block)",
                           who, i, t->fmt, gate->fmt);
        if (t->gs != gate->gs)
            return decline("%s: tensor %d has gs %d, gate has gs %d (mixed group sizes in one "
                           "block)", who, i, t->gs, gate->gs);
        if (!(t->flags & QF_FAST))
            return decline("%s: tensor %d layout unsupported by the block kernels (needs rows "
                           "of whole 16-byte packets: I %% %d == 0, aligned codes)", who, i,
                           packet_cols(t->fmt));
        if (t->fmt == 4 && !(t->flags & (QF_GROUP32 | QF_GROUP16)))
            return decline("%s: tensor %d gs=%d; the block kernels need gs %% 16 == 0", who, i,
                           t->gs);
    }
    if (nsh == 3) {
        if (sg->n != 1 || su->n != 1 || (sd && sd->n != 1))
            return decline("%s: shared tensors must hold one matrix each", who);
        if (sg->O != F || sg->I != D || su->O != F || su->I != D ||
            (sd && (sd->O != D || sd->I != F)))
            return decline("%s: shared expert shapes differ from the routed experts", who);
    }
    if (!dev_aligned(x, 16))
        return decline("%s: x must be 16-byte aligned", who);
    return COLI_OK;
}

int coli_moe_block(const coli_qtensor *gate, const coli_qtensor *up, const coli_qtensor *down,
                   const float *x, int S, const int32_t *ids, const float *w, int K,
                   const coli_qtensor *sh_gate, const coli_qtensor *sh_up,
                   const coli_qtensor *sh_down, float *out, void *workspace, size_t ws_bytes,
                   void *stream) {
    if (check_moe(gate, up, down, x, S, ids, K, sh_gate, sh_up, sh_down, "moe_block") != COLI_OK)
        return COLI_DECLINED;
    if (!w || !out)
        return decline("moe_block: NULL w or out");
    if (!workspace || !dev_aligned(workspace, 256))
        return decline("moe_block: workspace NULL or not 256-byte aligned");
    const int has_sh = sh_gate != nullptr;
    const size_t need = coli_moe_workspace_bytes(gate->n, S, K, gate->O, gate->I, has_sh);
    if (ws_bytes < need)
        return decline("moe_block: workspace %zu bytes < %zu needed", ws_bytes, need);
    if (!gate_call())
        return COLI_DECLINED;
    MoeArgs a;
    a.gate = gate; a.up = up; a.down = down;
    a.sg = sh_gate; a.su = sh_up; a.sd = sh_down;
    a.x = x; a.S = S; a.K = K; a.E = gate->n; a.F = gate->O; a.D = gate->I;
    a.ids = ids; a.w = w; a.out = out; a.h_out = nullptr;
    a.ws = workspace; a.ws_bytes = ws_bytes; a.st = (hipStream_t)stream;
    if (S <= coli_gemv_max_rows())
        return launch_moe_decode(a);
    return launch_moe_prefill(a);
}

// two-phase block workspace: [block][resident ids][late ids][late experts' output]
struct TwoPhaseWs {
    size_t blk, ida, idb, y, total;
};
static TwoPhaseWs two_phase_ws(int E, int S, int K, int F, int D, int has_sh) {
    TwoPhaseWs t;
    auto al = [](size_t b) { return (b + 255) / 256 * 256; };
    t.blk = 0;
    const size_t b = coli_moe_workspace_bytes(E, S, K, F, D, has_sh);
    t.ida = al(b);
    t.idb = t.ida + al(sizeof(int32_t) * (size_t)S * K);
    t.y = t.idb + al(sizeof(int32_t) * (size_t)S * K);
    t.total = b == 0 ? 0 : t.y + al(sizeof(float) * (size_t)S * D);
    return t;
}

size_t coli_moe_block_two_phase_workspace_bytes(int E, int S, int K, int F, int Dm, int has_shared) {
    if (E < 1 || S < 1 || K < 1 || F < 1 || Dm < 1)
        return 0;
    return two_phase_ws(E, S, K, F, Dm, has_shared ? 1 : 0).total;
}

static int moe_run(const coli_qtensor *gate, const coli_qtensor *up, const coli_qtensor *down,
                   const float *x, int S, const int32_t *ids, const float *w, int K,
                   const coli_qtensor *sg, const coli_qtensor *su, const coli_qtensor *sd, float *out,
                   void *ws, size_t ws_bytes, hipStream_t st) {
    MoeArgs a;
    a.gate = gate; a.up = up; a.down = down;
    a.sg = sg; a.su = su; a.sd = sd;
    a.x = x; a.S = S; a.K = K; a.E = gate->n; a.F = gate->O; a.D = gate->I;
    a.ids = ids; a.w = w; a.out = out; a.h_out = nullptr;
    a.ws = ws; a.ws_bytes = ws_bytes; a.st = st;
    return S <= coli_gemv_max_rows() ? launch_moe_decode(a) : launch_moe_prefill(a);
}

int coli_moe_block_begin(const coli_qtensor *gate, const coli_qtensor *up, const coli_qtensor *down,
                         const float *x, int S, const int32_t *ids, const float *w, int K,
                         const int32_t *late, const coli_qtensor *sh_gate,
                         const coli_qtensor *sh_up, const coli_qtensor *sh_down, float *out,
                         void *workspace, size_t ws_bytes, void *stream) {
    if (check_moe(gate, up, down, x, S, ids, K, sh_gate, sh_up, sh_down, "moe_block_begin") != COLI_OK)
        return COLI_DECLINED;
    if (!down || !w || !out || !late)
        return decline("moe_block_begin: NULL down, w, out or late");
    if (!workspace || !dev_aligned(workspace, 256))
        return decline("moe_block_begin: workspace NULL or not 256-byte aligned");
    if ((int64_t)S * K > INT32_MAX / 2)
        return decline("moe_block_begin: S*K too large");
    const TwoPhaseWs t = two_phase_ws(gate->n, S, K, gate->O, gate->I, sh_gate != nullptr);
    if (t.total == 0 || ws_bytes < t.total)
        return decline("moe_block_begin: workspace %zu bytes < %zu needed", ws_bytes, t.total);
    if (!gate_call())
        return COLI_DECLINED;
    const hipStream_t st = (hipStream_t)stream;
    char *ws = (char *)workspace;
    int32_t *ida = (int32_t *)(ws + t.ida), *idb = (int32_t *)(ws + t.idb);
    int rc = launch_split_ids(ids, late, S * K, ida, idb, st);
    if (rc != COLI_OK) return rc;
    return moe_run(gate, up, down, x, S, ida, w, K, sh_gate, sh_up, sh_down, out, ws, t.ida, st);
}

int coli_moe_block_end(const coli_qtensor *gate, const coli_qtensor *up, const coli_qtensor *down,
                       const float *x, int S, const float *w, int K, int has_shared, float *out,
                       void *workspace, size_t ws_bytes, void *stream) {
    if (!workspace || !dev_aligned(workspace, 256))
        return decline("moe_block_end: workspace NULL or not 256-byte aligned");
    // the late routing sits in the workspace; any non-NULL ids pointer passes here
    if (check_moe(gate, up, down, x, S, (const int32_t *)workspace, K, nullptr, nullptr, nullptr,
                  "moe_block_end") != COLI_OK)
        return COLI_DECLINED;
    if (!down || !w || !out)
        return decline("moe_block_end: NULL down, w or out");
    const TwoPhaseWs t = two_phase_ws(gate->n, S, K, gate->O, gate->I, has_shared ? 1 : 0);
    const int32_t *idb = (const int32_t *)((char *)workspace + t.idb);
    if (t.total == 0 || ws_bytes < t.total)
        return decline("moe_block_end: workspace %zu bytes < %zu needed", ws_bytes, t.total);
    if (!gate_call())
        return COLI_DECLINED;
    const hipStream_t st = (hipStream_t)stream;
    char *ws = (char *)workspace;
    float *y = (float *)(ws + t.y);
    int rc = moe_run(gate, up, down, x, S, idb, w, K, nullptr, nullptr, nullptr, y, ws, t.ida, st);
    if (rc != COLI_OK) return rc;
    return launch_residual_add(out, y, out, (int64_t)S * gate->I, st);
}

int coli_moe_hidden(const coli_qtensor *gate, const coli_qtensor *up, const float *x, int S,
                    const int32_t *ids, int K, const coli_qtensor *sh_gate,
                    const coli_qtensor *sh_up, float *h_out, void *workspace, size_t ws_bytes,
                    void *stream) {
    if ((sh_gate == nullptr) != (sh_up == nullptr))
        return decline("moe_hidden: shared expert needs both gate and up");
    if (check_moe(gate, up, nullptr, x, S, ids, K, sh_gate, sh_up, nullptr,
                  "moe_hidden") != COLI_OK)
        return COLI_DECLINED;
    if (!h_out || !dev_aligned(h_out, 16))
        return decline("moe_hidden: h_out NULL or not 16-byte aligned");
    if (!workspace || !dev_aligned(workspace, 256))
        return decline("moe_hidden: workspace NULL or not 256-byte aligned");
    const int has_sh = sh_gate != nullptr;
    const size_t need = coli_moe_workspace_bytes(gate->n, S, K, gate->O, gate->I, has_sh);
    if (ws_bytes < need)
        return decline("moe_hidden: workspace %zu bytes < %zu needed", ws_bytes, need);
    if (!gate_call())
        return COLI_DECLINED;
    MoeArgs a;
    a.gate = gate; a.up = up; a.down = nullptr;
    a.sg = sh_gate; a.su = sh_up; a.sd = nullptr;
    a.x = x; a.S = S; a.K = K; a.E = gate->n; a.F = gate->O; a.D = gate->I;
    a.ids = ids; a.w = nullptr; a.out = nullptr; a.h_out = h_out;
    a.ws = workspace; a.ws_bytes = ws_bytes; a.st = (hipStream_t)stream;
    if (S <= coli_gemv_max_rows())
        return launch_moe_decode(a);
    return launch_moe_prefill(a);
}

int coli_rmsnorm(const float *x, int S, int D, const float *w, float eps, float *y, void *stream) {
    if (!x || !y)
        return decline("rmsnorm: NULL x or y");
    if (S < 1 || D < 1 || (int64_t)S * D > INT32_MAX)
        return decline("rmsnorm: bad S=%d D=%d", S, D);
    if (!(eps >= 0.0f) || eps == __builtin_huge_valf())
        return decline("rmsnorm: eps must be finite and >= 0");
    if (!gate_call())
        return COLI_DECLINED;
    return launch_rmsnorm(x, S, D, w, (double)eps, y, (hipStream_t)stream);
}

static size_t al256(size_t b) { return (b + 255) / 256 * 256; }

// workspace of coli_moe_layer: xn | ids | w | router | block output | block
struct LayerWs {
    size_t xn, ids, w, rt, y, blk, total;
};
static LayerWs layer_ws(int E, int S, int K, int F, int D, int has_shared) {
    LayerWs l{};
    const size_t blk = coli_moe_workspace_bytes(E, S, K, F, D, has_shared);
    if (blk == 0)
        return l;
    l.xn = 0;
    l.ids = l.xn + al256((size_t)S * D * sizeof(float));
    l.w = l.ids + al256((size_t)S * K * sizeof(int32_t));
    l.rt = l.w + al256((size_t)S * K * sizeof(float));
    l.y = l.rt + al256(router_ws_bytes(S, E));
    l.blk = l.y + al256((size_t)S * D * sizeof(float));
    l.total = l.blk + blk;
    return l;
}

size_t coli_moe_layer_workspace_bytes(int E, int S, int K, int F, int D, int has_shared) {
    if (E < 1 || S < 1 || K < 1 || F < 1 || D < 1)
        return 0;
    return layer_ws(E, S, K, F, D, has_shared).total;
}

// validation of the expert half of a layer (everything but the workspace)
static int check_moe_layer(const coli_qtensor *gate, const coli_qtensor *up,
                           const coli_qtensor *down, const float *h, int S, float eps,
                           const float *R, int K, float topp, float routed_scale,
                           const coli_qtensor *sh_gate, const coli_qtensor *sh_up,
                           const coli_qtensor *sh_down, const void *ids_probe, const char *who) {
    if (!h || !R)
        return decline("%s: NULL input rows or router weights", who);
    // the routing lands in the workspace; any non-NULL ids pointer passes here
    if (check_moe(gate, up, down, h, S, (const int32_t *)ids_probe, K, sh_gate, sh_up, sh_down,
                  who) != COLI_OK)
        return COLI_DECLINED;
    if (!down)
        return decline("%s: NULL down tensor", who);
    const int E = gate->n, D = gate->I;
    if (E > 512 || K > 16 || K > E)
        return decline("%s: E=%d K=%d (router: E 1..512, K 1..min(16,E))", who, E, K);
    if (!(topp >= 0.0f && topp <= 1.0f) || !(routed_scale == routed_scale))
        return decline("%s: topp must lie in [0,1] and routed_scale must be a number", who);
    if (!(eps >= 0.0f) || eps == __builtin_huge_valf())
        return decline("%s: eps must be finite and >= 0", who);
    if ((int64_t)S * D > INT32_MAX || (int64_t)E * D > INT32_MAX)
        return decline("%s: S*D or E*D too large", who);
    return COLI_OK;
}

// the expert half's launches: norm, router, block (shared expert included),
// residual add
static int launch_moe_layer(const coli_qtensor *gate, const coli_qtensor *up,
                            const coli_qtensor *down, const float *h, int S, const float *ln_w,
                            float eps, const float *R, const float *bias, int K, float topp,
                            int norm_topk, float routed_scale, const coli_qtensor *sh_gate,
                            const coli_qtensor *sh_up, const coli_qtensor *sh_down, float *out,
                            char *ws, size_t ws_bytes, const LayerWs &l, hipStream_t st) {
    const int E = gate->n, F = gate->O, D = gate->I;
    float *xn = (float *)(ws + l.xn);
    int32_t *ids = (int32_t *)(ws + l.ids);
    float *w = (float *)(ws + l.w);
    float *y = (float *)(ws + l.y);
    int rc = launch_norm_router(h, S, D, ln_w, (double)eps, xn, R, bias, E, K, topp, norm_topk,
                                routed_scale, ids, w, ws + l.rt, st);
    if (rc != COLI_OK) return rc;
    MoeArgs a;
    a.gate = gate; a.up = up; a.down = down;
    a.sg = sh_gate; a.su = sh_up; a.sd = sh_down;
    a.x = xn; a.S = S; a.K = K; a.E = E; a.F = F; a.D = D;
    a.ids = ids; a.w = w; a.out = y; a.h_out = nullptr;
    a.ws = ws + l.blk; a.ws_bytes = ws_bytes - l.blk; a.st = st;
    if (S <= coli_gemv_max_rows()) {
        a.resid = h;  // out = h + y in the block's combine
        a.out_res = out;
        return launch_moe_decode(a);
    }
    rc = launch_moe_prefill(a);
    if (rc != COLI_OK) return rc;
    return launch_residual_add(h, y, out, (int64_t)S * D, st);
}

int coli_moe_layer(const coli_qtensor *gate, const coli_qtensor *up, const coli_qtensor *down,
                   const float *h, int S, const float *ln_w, float eps, const float *R,
                   const float *bias, int K, float topp, int norm_topk, float routed_scale,
                   const coli_qtensor *sh_gate, const coli_qtensor *sh_up,
                   const coli_qtensor *sh_down, float *out, void *workspace, size_t ws_bytes,
                   void *stream) {
    if (!h || !R || !out || !workspace)
        return decline("moe_layer: NULL h, R, out or workspace (ln_w, bias and the shared "
                       "expert may be NULL)");
    if (!dev_aligned(workspace, 256))
        return decline("moe_layer: workspace not 256-byte aligned");
    if (check_moe_layer(gate, up, down, h, S, eps, R, K, topp, routed_scale, sh_gate, sh_up,
                        sh_down, workspace, "moe_layer") != COLI_OK)
        return COLI_DECLINED;
    const LayerWs l = layer_ws(gate->n, S, K, gate->O, gate->I, sh_gate != nullptr);
    if (l.total == 0 || ws_bytes < l.total)
        return decline("moe_layer: workspace %zu bytes < %zu needed", ws_bytes, l.total);
    if (!gate_call())
        return COLI_DECLINED;
    return launch_moe_layer(gate, up, down, h, S, ln_w, eps, R, bias, K, topp, norm_topk,
                            routed_scale, sh_gate, sh_up, sh_down, out, (char *)workspace,
                            ws_bytes, l, (hipStream_t)stream);
}

// ---------------------------------------------------------------------------
// Decode attention (MLA)
// ---------------------------------------------------------------------------

// shapes and limits of a coli_mla_layer; fills the layout for S rows and
// T_cap cache rows
static int check_mla(const coli_mla_layer *m, int S, int T_cap, MlaLayout *lay, const char *who) {
    if (!m)
        return decline("%s: NULL layer", who);
    const coli_qtensor *ts[5] = {m->q_a, m->q_b, m->kv_a, m->kv_b, m->o_proj};
    const char *nm[5] = {"q_a", "q_b", "kv_a", "kv_b", "o_proj"};
    for (int i = 0; i < 5; ++i) {
        if (check_qt(ts[i], nm[i]) != COLI_OK)
            return decline("%s: %s not filled by coli_tensor_upload", who, nm[i]);
        if (ts[i]->n != 1)
            return decline("%s: %s must be a single matrix", who, nm[i]);
    }
    const int H = m->H, dn = m->d_nope, dr = m->d_rope, dv = m->d_v;
    if (H < 1 || H > 256 || dn < 1 || dn > 1024 || dr < 2 || dr > 256 || dr % 2 || dv < 1 ||
        dv > 1024)
        return decline("%s: bad heads/dims H=%d d_nope=%d d_rope=%d d_v=%d (H 1..256, d_nope "
                       "1..1024, d_rope even 2..256, d_v 1..1024)", who, H, dn, dr, dv);
    const int D = m->q_a->I, qr = m->q_a->O, L = m->kv_b->I;
    if (m->q_b->I != qr || m->q_b->O != H * (dn + dr))
        return decline("%s: q_b is [%d][%d], expected [%d][%d]", who, m->q_b->O, m->q_b->I,
                       H * (dn + dr), qr);
    if (m->kv_a->I != D || m->kv_a->O != L + dr)
        return decline("%s: kv_a is [%d][%d], expected [%d][%d]", who, m->kv_a->O, m->kv_a->I,
                       L + dr, D);
    if (m->kv_b->O != H * (dn + dv))
        return decline("%s: kv_b has %d rows, expected %d", who, m->kv_b->O, H * (dn + dv));
    if (m->o_proj->O != D || m->o_proj->I != H * dv)
        return decline("%s: o_proj is [%d][%d], expected [%d][%d]", who, m->o_proj->O,
                       m->o_proj->I, D, H * dv);
    const coli_qtensor *kb = m->kv_b;
    if (!(kb->fmt == COLI_FMT_I4_ROW || (kb->fmt == COLI_FMT_I4_GRP && kb->gs % 8 == 0)))
        return decline("%s: kv_b must be fmt 2, or fmt 4 with gs %% 8 == 0 (fmt %d gs %d)", who,
                       kb->fmt, kb->gs);
    if (L % 32 != 0 || L > 4096 || !dev_aligned(kb->q, 16))
        return decline("%s: latent width %d must be a multiple of 32 up to 4096 with 16-byte "
                       "aligned kv_b codes", who, L);
    if (S < 1 || S > COLI_MLA_MAX_ROWS)
        return decline("%s: S=%d outside 1..%d", who, S, COLI_MLA_MAX_ROWS);
    if (T_cap < S || (int64_t)T_cap * (L + dr) > INT32_MAX)
        return decline("%s: bad T_cap=%d", who, T_cap);
    if (!(m->eps >= 0.0f) || m->eps == __builtin_huge_valf() ||
        !(m->rope_theta > 0.0f) || m->rope_theta == __builtin_huge_valf())
        return decline("%s: eps must be finite >= 0 and rope_theta finite > 0", who);
    *lay = mla_layout(S, H, dn, dr, dv, qr, L, T_cap, mla_proj_ws(*m, S));
    return COLI_OK;
}

size_t coli_mla_workspace_layout(const coli_mla_layer *layer, int S, int T_cap,
                                 size_t offsets[COLI_MLA_STAGES]) {
    MlaLayout l;
    if (check_mla(layer, S, T_cap, &l, "mla_workspace_layout") != COLI_OK)
        return 0;
    if (offsets)
        for (int i = 0; i < MLA_NSTAGE; ++i) offsets[i] = l.off[i];
    return l.total;
}

size_t coli_mla_workspace_bytes(const coli_mla_layer *layer, int S, int T_cap) {
    return coli_mla_workspace_layout(layer, S, T_cap, nullptr);
}

int coli_mla_decode(const coli_mla_layer *layer, const float *x, int S, int pos_base, float *Lc,
                    float *Rc, int T_cap, float *out, void *workspace, size_t ws_bytes,
                    void *stream) {
    MlaLayout l;
    if (check_mla(layer, S, T_cap, &l, "mla_decode") != COLI_OK)
        return COLI_DECLINED;
    if (!x || !Lc || !Rc || !out)
        return decline("mla_decode: NULL x, Lc, Rc or out");
    if (!dev_aligned(x, 16) || !dev_aligned(out, 4) || !dev_aligned(Lc, 4) || !dev_aligned(Rc, 4))
        return decline("mla_decode: x must be 16-byte aligned (out, Lc, Rc 4-byte)");
    if (pos_base < 0 || pos_base > T_cap - S)
        return decline("mla_decode: pos_base=%d with S=%d outside a cache of %d rows", pos_base, S,
                       T_cap);
    if (!workspace || !dev_aligned(workspace, 256) || ws_bytes < l.total)
        return decline("mla_decode: workspace NULL, not 256-byte aligned or %zu < %zu bytes",
                       ws_bytes, l.total);
    if (!gate_call())
        return COLI_DECLINED;
    MlaArgs a;
    a.layer = layer;
    a.x = x;
    a.S = S;
    a.pos_base = pos_base;
    a.T_cap = T_cap;
    a.Lc = Lc;
    a.Rc = Rc;
    a.out = out;
    a.ws = workspace;
    a.st = (hipStream_t)stream;
    return launch_mla_decode(a);
}

// ---------------------------------------------------------------------------
// Full decode layer: in_ln -> attention -> residual -> expert half
// ---------------------------------------------------------------------------

struct FullLayerWs {
    size_t off[COLI_LAYER_STAGES];  // xn, attn, h, attention workspace, expert-half workspace
    size_t mla_bytes, moe_bytes, total;
};

static int full_layer_ws(const coli_mla_layer *attn, const coli_qtensor *gate, int S, int K,
                         int T_cap, int has_shared, FullLayerWs *f, const char *who) {
    MlaLayout ml;
    if (check_mla(attn, S, T_cap, &ml, who) != COLI_OK)
        return COLI_DECLINED;
    if (check_qt(gate, "gate") != COLI_OK)
        return COLI_DECLINED;
    const int D = attn->q_a->I;
    if (gate->I != D)
        return decline("%s: experts take %d inputs, the attention's hidden size is %d", who,
                       gate->I, D);
    const LayerWs l = layer_ws(gate->n, S, K, gate->O, D, has_shared);
    if (l.total == 0)
        return decline("%s: bad expert-half sizes", who);
    const size_t rows = al256((size_t)S * D * sizeof(float));
    f->off[0] = 0;
    f->off[1] = rows;
    f->off[2] = 2 * rows;
    f->off[3] = 3 * rows;
    f->off[4] = 3 * rows + ml.total;
    f->mla_bytes = ml.total;
    f->moe_bytes = l.total;
    f->total = f->off[4] + l.total;
    return COLI_OK;
}

size_t coli_layer_decode_workspace_layout(const coli_mla_layer *attn, const coli_qtensor *gate,
                                          int S, int K, int T_cap, int has_shared,
                                          size_t offsets[COLI_LAYER_STAGES]) {
    FullLayerWs f;
    if (full_layer_ws(attn, gate, S, K, T_cap, has_shared ? 1 : 0, &f, "layer_decode_workspace") !=
        COLI_OK)
        return 0;
    if (offsets)
        for (int i = 0; i < COLI_LAYER_STAGES; ++i) offsets[i] = f.off[i];
    return f.total;
}

size_t coli_layer_decode_workspace_bytes(const coli_mla_layer *attn, const coli_qtensor *gate,
                                         int S, int K, int T_cap, int has_shared) {
    return coli_layer_decode_workspace_layout(attn, gate, S, K, T_cap, has_shared, nullptr);
}

int coli_layer_decode(const coli_mla_layer *attn, const float *in_ln, const coli_qtensor *gate,
                      const coli_qtensor *up, const coli_qtensor *down, const float *post_ln,
                      const float *R, const float *bias, int K, float topp, int norm_topk,
                      float routed_scale, const coli_qtensor *sh_gate, const coli_qtensor *sh_up,
                      const coli_qtensor *sh_down, float eps, const float *x, int S, int pos_base,
                      float *Lc, float *Rc, int T_cap, float *out, void *workspace,
                      size_t ws_bytes, void *stream) {
    const char *who = "layer_decode";
    FullLayerWs f;
    if (full_layer_ws(attn, gate, S, K, T_cap, sh_gate != nullptr, &f, who) != COLI_OK)
        return COLI_DECLINED;
    if (!x || !Lc || !Rc || !out || !workspace)
        return decline("%s: NULL x, Lc, Rc, out or workspace", who);
    if (!dev_aligned(x, 16) || !dev_aligned(out, 4) || !dev_aligned(Lc, 4) || !dev_aligned(Rc, 4))
        return decline("%s: x must be 16-byte aligned (out, Lc, Rc 4-byte)", who);
    if (pos_base < 0 || pos_base > T_cap - S)
        return decline("%s: pos_base=%d with S=%d outside a cache of %d rows", who, pos_base, S,
                       T_cap);
    if (!dev_aligned(workspace, 256) || ws_bytes < f.total)
        return decline("%s: workspace not 256-byte aligned or %zu < %zu bytes", who, ws_bytes,
                       f.total);
    char *ws = (char *)workspace;
    const float *h = (const float *)(ws + f.off[2]);
    if (check_moe_layer(gate, up, down, h, S, eps, R, K, topp, routed_scale, sh_gate, sh_up,
                        sh_down, ws, who) != COLI_OK)
        return COLI_DECLINED;
    if (!gate_call())
        return COLI_DECLINED;
    const hipStream_t st = (hipStream_t)stream;
    const int D = attn->q_a->I;
    float *xn = (float *)(ws + f.off[0]);
    float *a = (float *)(ws + f.off[1]);
    float *hh = (float *)(ws + f.off[2]);
    MlaArgs m;
    m.layer = attn;
    m.x = x;
    m.in_norm = true;  // xn = in_ln RMSNorm of x, folded into q_a / kv_a when it can be
    m.in_norm_w = in_ln;
    m.in_eps = (double)eps;
    m.xn = xn;
    m.S = S;
    m.pos_base = pos_base;
    m.T_cap = T_cap;
    m.Lc = Lc;
    m.Rc = Rc;
    m.out = a;
    m.ws = ws + f.off[3];
    m.st = st;
    m.resid = x;  // h = x + a in o_proj's epilogue
    m.hsum = hh;
    const int rc = launch_mla_decode(m);
    if (rc != COLI_OK) return rc;
    const LayerWs l = layer_ws(gate->n, S, K, gate->O, D, sh_gate != nullptr);
    return launch_moe_layer(gate, up, down, hh, S, post_ln, eps, R, bias, K, topp, norm_topk,
                            routed_scale, sh_gate, sh_up, sh_down, out, ws + f.off[4], f.moe_bytes,
                            l, st);
}

// ---------------------------------------------------------------------------
// coli_moe_block_noalloc: the expert block with the library's own device
// scratch instead of a caller workspace (for callers that cannot allocate).
// ---------------------------------------------------------------------------

int coli_moe_block_noalloc(const coli_qtensor *gate, const coli_qtensor *up,
                           const coli_qtensor *down, const float *x, int S, const int32_t *ids,
                           const float *w, int K, const coli_qtensor *sh_gate,
                           const coli_qtensor *sh_up, const coli_qtensor *sh_down, float *out,
                           void *stream) {
    if (check_moe(gate, up, down, x, S, ids, K, sh_gate, sh_up, sh_down, "moe_block_noalloc") !=
        COLI_OK)
        return COLI_DECLINED;
    const size_t need =
        coli_moe_workspace_bytes(gate->n, S, K, gate->O, gate->I, sh_gate != nullptr);
    if (need == 0 || need > (size_t)COLI_NOALLOC_SCRATCH_BYTES)
        return decline("moe_block_noalloc: this block needs %zu bytes of scratch; the library's "
                       "static scratch holds %zu (use coli_moe_block with a workspace)",
                       need, (size_t)COLI_NOALLOC_SCRATCH_BYTES);
    void *ws = nullptr;
    const int rc = scratch_on_current_device(&ws);
    if (rc != COLI_OK)
        return rc;
    return coli_moe_block(gate, up, down, x, S, ids, w, K, sh_gate, sh_up, sh_down, out, ws,
                          (size_t)COLI_NOALLOC_SCRATCH_BYTES, stream);
}

}  // extern "C"
