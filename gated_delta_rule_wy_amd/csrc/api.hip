// C ABI of libgdn2 (declared in include/gdn2.h): argument validation, the
// per-thread stream, and dispatch to the kernels. Nothing is enqueued unless
// every check passes.
#include "../../include/gdn2.h"
#include "gdn2_launch.hpp"

#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <vector>

namespace {

thread_local hipStream_t g_stream = nullptr;

// Per-thread kernel timing state (gdn2_profile_*).
struct Prof {
    bool on = false;          // recording requested
    bool active = false;      // the current call is being recorded
    int max_calls = 0, calls = 0;
    std::vector<hipEvent_t> ev;
    size_t used = 0;
    struct Rec { const char *name; size_t e0; };
    std::vector<Rec> recs;
    void release() {
        for (hipEvent_t e : ev) (void)hipEventDestroy(e);
        ev.clear();
        recs.clear();
        used = 0;
        calls = 0;
        on = active = false;
    }
    // no destructor: events are left to the process teardown, whose order
    // relative to the HIP runtime's is not defined
};
thread_local Prof g_prof;

// Events created up front per recorded call; the pool grows past this on
// demand (a segmented prefill launches two kernels per segment), up to a cap.
constexpr size_t kEventsPerCall = 64;
constexpr size_t kMaxProfEvents = 1u << 17;

bool prof_grow(size_t n)
{
    while (g_prof.ev.size() < n) {
        hipEvent_t e = nullptr;
        if (g_prof.ev.size() >= kMaxProfEvents || hipEventCreate(&e) != hipSuccess) return false;
        g_prof.ev.push_back(e);
    }
    return true;
}

// Marks the start of a library call: decides whether its kernels are timed.
void prof_call()
{
    g_prof.active = g_prof.on && g_prof.calls < g_prof.max_calls;
    if (g_prof.active) ++g_prof.calls;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

bool head_dim_ok(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }

} // namespace

namespace gdn2 {

void prof_before(const char *kernel, hipStream_t st)
{
    if (!g_prof.active || !prof_grow(g_prof.used + 2)) return;
    (void)hipEventRecord(g_prof.ev[g_prof.used], st);
    g_prof.recs.push_back({kernel, g_prof.used});
    g_prof.used += 1;
}

void prof_after(hipStream_t st)
{
    if (!g_prof.active || g_prof.recs.empty() || g_prof.recs.back().e0 + 1 != g_prof.used) return;
    (void)hipEventRecord(g_prof.ev[g_prof.used], st);
    g_prof.used += 1;
}

} // namespace gdn2

extern "C" {

int gdn2_profile_begin(int max_calls)
{
    if (max_calls < 1 || max_calls > 4096) return GDN2_ERR_INVALID;
    g_prof.release();
    if (!prof_grow(std::min((size_t)max_calls * kEventsPerCall, kMaxProfEvents))) {
        g_prof.release();
        return GDN2_ERR_HIP;
    }
    g_prof.max_calls = max_calls;
    g_prof.on = true;
    return GDN2_OK;
}

int gdn2_profile_end(void)
{
    g_prof.on = g_prof.active = false;
    return g_prof.calls;
}

int gdn2_profile_kernel(int idx, const char **name, int *launches, double *total_ms)
{
    // distinct names in order of first launch
    std::vector<const char *> names;
    for (const auto &r : g_prof.recs) {
        bool seen = false;
        for (const char *n : names) seen = seen || strcmp(n, r.name) == 0;
        if (!seen) names.push_back(r.name);
    }
    if (idx < 0 || idx >= (int)names.size()) return GDN2_ERR_INVALID;
    int cnt = 0;
    double tot = 0.0;
    for (const auto &r : g_prof.recs) {
        if (strcmp(r.name, names[idx]) != 0 || r.e0 + 1 >= g_prof.used) continue;
        float ms = 0.f;
        if (hipEventSynchronize(g_prof.ev[r.e0 + 1]) != hipSuccess) return GDN2_ERR_HIP;
        if (hipEventElapsedTime(&ms, g_prof.ev[r.e0], g_prof.ev[r.e0 + 1]) != hipSuccess) return GDN2_ERR_HIP;
        ++cnt;
        tot += ms;
    }
    if (name) *name = names[idx];
    if (launches) *launches = cnt;
    if (total_ms) *total_ms = tot;
    return GDN2_OK;
}

int gdn2_set_stream(void *hip_stream)
{
    g_stream = (hipStream_t)hip_stream;
    return GDN2_OK;
}

void *gdn2_get_stream(void) { return (void *)g_stream; }

const char *gdn2_status_string(int status)
{
    switch (status) {
    case GDN2_OK: return "GDN2_OK";
    case GDN2_ERR_INVALID: return "GDN2_ERR_INVALID: invalid argument";
    case GDN2_ERR_UNSUPPORTED: return "GDN2_ERR_UNSUPPORTED: sizes or dtypes not supported";
    case GDN2_ERR_WORKSPACE: return "GDN2_ERR_WORKSPACE: workspace missing or too small";
    case GDN2_ERR_HIP: return "GDN2_ERR_HIP: HIP runtime error";
    }
    return "GDN2: unknown status";
}

static int chunk_fwd_impl(const void *q, const void *k, const void *v, const float *log_alpha,
                          const void *b, const void *w, int gates, const gdn2_short_conv *conv, const float *S0,
                          void *o, float *ST, const int32_t *cu_seqlens, int B, int T, int N, int H, int dk,
                          int dv, int in_dtype, int out_dtype, void *workspace,
                          size_t workspace_bytes, int chunk = 64);

static int chunk_check(int B, int T, int N, int H, int dk, int dv, int in_dtype, int varlen,
                       gdn2::ChunkPlan *plan, int chunk = 64)
{
    if (chunk != 32 && chunk != 64 && chunk != 128) return GDN2_ERR_INVALID;
    if (B <= 0 || T < 0 || N <= 0 || H <= 0 || dk <= 0 || dv <= 0) return GDN2_ERR_INVALID;
    if (in_dtype != GDN2_F32 && in_dtype != GDN2_BF16) return GDN2_ERR_INVALID;
    if (varlen ? B != 1 : N != B) return GDN2_ERR_INVALID;
    if (!head_dim_ok(dk) || !head_dim_ok(dv)) return GDN2_ERR_UNSUPPORTED;
    if (H > 65535) return GDN2_ERR_UNSUPPORTED;   // grid y dimension
    if ((long long)B * T > 0x7fffffffLL) return GDN2_ERR_UNSUPPORTED;
    // (each factor is bounded above, so the product cannot overflow)
    if ((long long)B * T * H * (dk > dv ? dk : dv) > 0x7fffffffLL * 16LL) return GDN2_ERR_UNSUPPORTED;
    if (!gdn2::chunk_plan(B, T, N, H, dk, dv, in_dtype == GDN2_BF16, varlen != 0, plan, chunk))
        return GDN2_ERR_UNSUPPORTED;
    return GDN2_OK;
}

size_t gdn2_chunk_fwd_sized_workspace_bytes(int B, int T, int N, int H, int dk, int dv, int in_dtype,
                                            int varlen, int chunk)
{
    gdn2::ChunkPlan plan;
    if (chunk_check(B, T, N, H, dk, dv, in_dtype, varlen, &plan, chunk) != GDN2_OK) return 0;
    return plan.total_bytes > 0 ? plan.total_bytes : 256;
}

size_t gdn2_chunk_fwd_workspace_bytes(int B, int T, int N, int H, int dk, int dv,
                                      int in_dtype, int varlen)
{
    gdn2::ChunkPlan plan;
    if (chunk_check(B, T, N, H, dk, dv, in_dtype, varlen, &plan) != GDN2_OK) return 0;
    return plan.total_bytes > 0 ? plan.total_bytes : 256;
}

int gdn2_chunk_fwd(const void *q, const void *k, const void *v, const float *log_alpha,
                   const void *b, const void *w, const float *S0, void *o, float *ST,
                   const int32_t *cu_seqlens, int B, int T, int N, int H, int dk, int dv,
                   int in_dtype, int out_dtype, void *workspace,
                   size_t workspace_bytes)
{
    return gdn2_chunk_fwd_gates(q, k, v, log_alpha, b, w, GDN2_GATES_PER_CHANNEL, S0, o, ST, cu_seqlens, B, T,
                                N, H, dk, dv, in_dtype, out_dtype, workspace, workspace_bytes);
}

} // extern "C"

// Workspace of gdn2_chunk_fwd_noalloc, for callers that cannot allocate:
// one copy per device, held until the process ends, shared by every call on
// that device (calls that overlap on one device race on it).
static constexpr size_t kScratchBytes = (size_t)GDN2_NOALLOC_WORKSPACE_MAX;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

// Device address of `scratch` on the current device, looked up with that
// device current on its first use and kept per device. (In host code the
// array's name stands for a host-side shadow, not for device memory.)
static int scratch_address(void **out)
{
    constexpr int kMaxDev = 64;
    static std::atomic<void *> addr[kMaxDev];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return GDN2_ERR_HIP;
    void *p = addr[dev].load(std::memory_order_acquire);
    if (!p) {
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return GDN2_ERR_HIP;
        addr[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return GDN2_OK;
}

extern "C" {

int gdn2_chunk_fwd_noalloc(const void *q, const void *k, const void *v, const float *log_alpha,
                           const void *b, const void *w, const float *S0, void *o, float *ST,
                           const int32_t *cu_seqlens, int B, int T, int N, int H, int dk, int dv,
                           int in_dtype, int out_dtype)
{
    const size_t need = gdn2_chunk_fwd_workspace_bytes(B, T, N, H, dk, dv, in_dtype, cu_seqlens != nullptr);
    if (need == 0 || need > kScratchBytes) {
        // invalid sizes report their own status; valid ones over the limit
        // report the workspace (nothing is launched either way)
        const int st = chunk_fwd_impl(q, k, v, log_alpha, b, w, GDN2_GATES_PER_CHANNEL, nullptr, S0, o, ST,
                                      cu_seqlens, B, T, N, H, dk, dv, in_dtype, out_dtype, nullptr, 0);
        return st == GDN2_OK ? GDN2_ERR_WORKSPACE : st;
    }
    void *ws = nullptr;
    const int st = scratch_address(&ws);
    if (st != GDN2_OK) return st;
    return chunk_fwd_impl(q, k, v, log_alpha, b, w, GDN2_GATES_PER_CHANNEL, nullptr, S0, o, ST, cu_seqlens, B, T,
                          N, H, dk, dv, in_dtype, out_dtype, ws, kScratchBytes);
}

// The convolution parameters of a *_prologue call: weights required, biases
// optional, history in / out each all-or-none.
static int conv_args(const gdn2_short_conv *c, gdn2::Prologue *p)
{
    if (!c) return GDN2_ERR_INVALID;
    const void *req[] = {c->weight_q, c->weight_k, c->weight_v};
    for (const void *x : req)
        if (!x || !aligned16(x)) return GDN2_ERR_INVALID;
    const void *opt[] = {c->bias_q, c->bias_k, c->bias_v, c->state_in_q, c->state_in_k, c->state_in_v,
                         c->state_out_q, c->state_out_k, c->state_out_v};
    for (const void *x : opt)
        if (x && !aligned16(x)) return GDN2_ERR_INVALID;
    const int nin = !!c->state_in_q + !!c->state_in_k + !!c->state_in_v;
    const int nout = !!c->state_out_q + !!c->state_out_k + !!c->state_out_v;
    if ((nin != 0 && nin != 3) || (nout != 0 && nout != 3)) return GDN2_ERR_INVALID;
    p->on = true;
    p->q = {c->weight_q, c->bias_q, c->state_in_q, c->state_out_q};
    p->k = {c->weight_k, c->bias_k, c->state_in_k, c->state_out_k};
    p->v = {c->weight_v, c->bias_v, c->state_in_v, c->state_out_v};
    return GDN2_OK;
}

static int chunk_fwd_impl(const void *q, const void *k, const void *v, const float *log_alpha,
                          const void *b, const void *w, int gates, const gdn2_short_conv *conv, const float *S0,
                          void *o, float *ST, const int32_t *cu_seqlens, int B, int T, int N, int H, int dk,
                          int dv, int in_dtype, int out_dtype, void *workspace,
                          size_t workspace_bytes, int chunk)
{
    if (gates & ~(GDN2_GATE_B_PER_HEAD | GDN2_GATE_W_PER_HEAD | GDN2_GATE_ALPHA_PER_HEAD)) return GDN2_ERR_INVALID;
    gdn2::ChunkPlan plan;
    const int varlen = cu_seqlens != nullptr;
    int st = chunk_check(B, T, N, H, dk, dv, in_dtype, varlen, &plan, chunk);
    if (st != GDN2_OK) return st;
    if (out_dtype != GDN2_F32) return out_dtype == GDN2_BF16 ? GDN2_ERR_UNSUPPORTED : GDN2_ERR_INVALID;
    const bool have_tokens = (long long)B * T > 0;
    if (have_tokens && (!q || !k || !v || !log_alpha || !b || !w || !o)) return GDN2_ERR_INVALID;
    const void *ptrs[] = {q, k, v, log_alpha, b, w, S0, o, ST, cu_seqlens, workspace};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return GDN2_ERR_INVALID;
    gdn2::ChunkArgs a;
    if (conv && (st = conv_args(conv, &a.pro)) != GDN2_OK) return st;
    if (!workspace || workspace_bytes < plan.total_bytes) return GDN2_ERR_WORKSPACE;

    a.q = q; a.k = k; a.v = v; a.b = b; a.w = w;
    a.log_alpha = log_alpha;
    a.S0 = S0;
    a.o = o;
    a.ST = ST;
    a.cu_seqlens = cu_seqlens;
    a.B = B; a.T = T; a.N = N; a.H = H; a.dk = dk; a.dv = dv;
    a.gates = gates;
    a.bf16 = in_dtype == GDN2_BF16;
    a.workspace = workspace;
    a.workspace_bytes = workspace_bytes;
    prof_call();
    if (gdn2::launch_chunk_fwd(a, plan, g_stream) != hipSuccess) return GDN2_ERR_HIP;
    return GDN2_OK;
}

int gdn2_chunk_fwd_gates(const void *q, const void *k, const void *v, const float *log_alpha,
                         const void *b, const void *w, int gates, const float *S0, void *o, float *ST,
                         const int32_t *cu_seqlens, int B, int T, int N, int H, int dk, int dv,
                         int in_dtype, int out_dtype, void *workspace,
                         size_t workspace_bytes)
{
    return chunk_fwd_impl(q, k, v, log_alpha, b, w, gates, nullptr, S0, o, ST, cu_seqlens, B, T, N, H, dk, dv,
                          in_dtype, out_dtype, workspace, workspace_bytes);
}

int gdn2_chunk_fwd_sized(const void *q, const void *k, const void *v, const float *log_alpha, const void *b,
                         const void *w, const float *S0, void *o, float *ST, const int32_t *cu_seqlens, int B,
                         int T, int N, int H, int dk, int dv, int in_dtype, int out_dtype,
                         int chunk, void *workspace, size_t workspace_bytes)
{
    return chunk_fwd_impl(q, k, v, log_alpha, b, w, GDN2_GATES_PER_CHANNEL, nullptr, S0, o, ST, cu_seqlens, B, T,
                          N, H, dk, dv, in_dtype, out_dtype, workspace, workspace_bytes, chunk);
}

int gdn2_chunk_fwd_prologue(const void *q_raw, const void *k_raw, const void *v_raw, const float *log_alpha,
                            const void *b_logit, const void *w_logit, const gdn2_short_conv *conv,
                            const float *S0, void *o, float *ST, const int32_t *cu_seqlens, int B, int T,
                            int N, int H, int dk, int dv, int in_dtype, int out_dtype,
                            void *workspace, size_t workspace_bytes)
{
    if (!conv) return GDN2_ERR_INVALID;
    return chunk_fwd_impl(q_raw, k_raw, v_raw, log_alpha, b_logit, w_logit, GDN2_GATES_PER_CHANNEL, conv, S0, o,
                          ST, cu_seqlens, B, T, N, H, dk, dv, in_dtype, out_dtype, workspace, workspace_bytes);
}

int gdn2_decode_step(const void *q, const void *k, const void *v, const float *log_alpha,
                     const void *b, const void *w, float *S, void *o, int N, int H, int dk,
                     int dv, int in_dtype, int out_dtype)
{
    return gdn2_decode_step_gates(q, k, v, log_alpha, b, w, GDN2_GATES_PER_CHANNEL, S, o, N, H, dk, dv, in_dtype,
                                  out_dtype);
}

size_t gdn2_chunk_bwd_workspace_bytes(int B, int T, int N, int H, int dk, int dv,
                                      int in_dtype, int varlen)
{
    gdn2::ChunkPlan plan;
    if (chunk_check(B, T, N, H, dk, dv, in_dtype, varlen, &plan) != GDN2_OK) return 0;
    gdn2::BwdPlan bp;
    if (!gdn2::chunk_bwd_plan(B, T, N, H, dk, dv, in_dtype == GDN2_BF16, varlen != 0, &bp)) return 0;
    return bp.total_bytes > 0 ? bp.total_bytes : 256;
}

// gdn2_chunk_bwd and its two halves (part: gdn2::kBwdAll, kBwdForward,
// kBwdFromKept); every check runs before anything is launched
static int chunk_bwd_impl(const void *q, const void *k, const void *v, const float *log_alpha, const void *b,
                          const void *w, const float *S0, const float *dO, const float *dST,
                          const int32_t *cu_seqlens, int B, int T, int N, int H, int dk, int dv, int in_dtype,
                          float *dq, float *dk_, float *dv_, float *dlog_alpha, float *db, float *dw, float *dS0,
                          void *o, float *ST, int part, void *workspace, size_t workspace_bytes)
{
    gdn2::ChunkPlan plan;
    const int varlen = cu_seqlens != nullptr;
    int st = chunk_check(B, T, N, H, dk, dv, in_dtype, varlen, &plan);
    if (st != GDN2_OK) return st;
    gdn2::BwdPlan bp;
    if (!gdn2::chunk_bwd_plan(B, T, N, H, dk, dv, in_dtype == GDN2_BF16, varlen != 0, &bp))
        return GDN2_ERR_UNSUPPORTED;
    const bool have_tokens = (long long)B * T > 0;
    if (have_tokens && (!q || !k || !v || !log_alpha || !b || !w)) return GDN2_ERR_INVALID;
    if (part == gdn2::kBwdForward && have_tokens && !o) return GDN2_ERR_INVALID;
    if (part != gdn2::kBwdForward && have_tokens && (!dO || !dq || !dk_ || !dv_ || !dlog_alpha || !db || !dw))
        return GDN2_ERR_INVALID;
    const void *ptrs[] = {q, k, v, log_alpha, b, w, S0, dO, dST, cu_seqlens, dq, dk_, dv_, dlog_alpha, db, dw, dS0,
                          o, ST, workspace};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return GDN2_ERR_INVALID;
    if (!workspace || workspace_bytes < bp.total_bytes) return GDN2_ERR_WORKSPACE;
    gdn2::ChunkBwdArgs a;
    a.q = q; a.k = k; a.v = v; a.b = b; a.w = w;
    a.log_alpha = log_alpha;
    a.S0 = S0;
    a.dO = dO;
    a.dST = dST;
    a.cu_seqlens = cu_seqlens;
    a.B = B; a.T = T; a.N = N; a.H = H; a.dk = dk; a.dv = dv;
    a.bf16 = in_dtype == GDN2_BF16;
    a.dq = dq; a.dk_ = dk_; a.dv_ = dv_; a.dlog_alpha = dlog_alpha; a.db = db; a.dw = dw;
    a.dS0 = dS0;
    a.workspace = workspace;
    a.workspace_bytes = workspace_bytes;
    a.part = part;
    a.o = o;
    a.ST = ST;
    prof_call();
    if (gdn2::launch_chunk_bwd(a, bp, g_stream) != hipSuccess) return GDN2_ERR_HIP;
    return GDN2_OK;
}

int gdn2_chunk_bwd(const void *q, const void *k, const void *v, const float *log_alpha,
                   const void *b, const void *w, const float *S0, const float *dO, const float *dST,
                   const int32_t *cu_seqlens, int B, int T, int N, int H, int dk, int dv,
                   int in_dtype, float *dq, float *dk_, float *dv_, float *dlog_alpha,
                   float *db, float *dw, float *dS0, void *workspace, size_t workspace_bytes)
{
    return chunk_bwd_impl(q, k, v, log_alpha, b, w, S0, dO, dST, cu_seqlens, B, T, N, H, dk, dv, in_dtype, dq, dk_,
                          dv_, dlog_alpha, db, dw, dS0, nullptr, nullptr, gdn2::kBwdAll, workspace, workspace_bytes);
}

int gdn2_chunk_fwd_keep(const void *q, const void *k, const void *v, const float *log_alpha,
                        const void *b, const void *w, const float *S0, void *o, float *ST,
                        const int32_t *cu_seqlens, int B, int T, int N, int H, int dk, int dv,
                        int in_dtype, int out_dtype, void *workspace, size_t workspace_bytes)
{
    if (out_dtype != GDN2_F32) return out_dtype == GDN2_BF16 ? GDN2_ERR_UNSUPPORTED : GDN2_ERR_INVALID;
    return chunk_bwd_impl(q, k, v, log_alpha, b, w, S0, nullptr, nullptr, cu_seqlens, B, T, N, H, dk, dv, in_dtype,
                          nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, o, ST, gdn2::kBwdForward,
                          workspace, workspace_bytes);
}

int gdn2_chunk_bwd_kept(const void *q, const void *k, const void *v, const float *log_alpha,
                        const void *b, const void *w, const float *S0, const float *dO, const float *dST,
                        const int32_t *cu_seqlens, int B, int T, int N, int H, int dk, int dv,
                        int in_dtype, float *dq, float *dk_, float *dv_, float *dlog_alpha,
                        float *db, float *dw, float *dS0, void *workspace, size_t workspace_bytes)
{
    return chunk_bwd_impl(q, k, v, log_alpha, b, w, S0, dO, dST, cu_seqlens, B, T, N, H, dk, dv, in_dtype, dq, dk_,
                          dv_, dlog_alpha, db, dw, dS0, nullptr, nullptr, gdn2::kBwdFromKept, workspace,
                          workspace_bytes);
}

static int decode_impl(const void *q, const void *k, const void *v, const float *log_alpha,
                       const void *b, const void *w, int gates, const gdn2_short_conv *conv, float *S, void *o,
                       int N, int H, int dk, int dv, int in_dtype, int out_dtype)
{
    if (gates & ~(GDN2_GATE_B_PER_HEAD | GDN2_GATE_W_PER_HEAD | GDN2_GATE_ALPHA_PER_HEAD)) return GDN2_ERR_INVALID;
    if (N <= 0 || H <= 0 || dk <= 0 || dv <= 0) return GDN2_ERR_INVALID;
    if (in_dtype != GDN2_F32 && in_dtype != GDN2_BF16) return GDN2_ERR_INVALID;
    if (out_dtype != GDN2_F32) return out_dtype == GDN2_BF16 ? GDN2_ERR_UNSUPPORTED : GDN2_ERR_INVALID;
    if (!head_dim_ok(dk) || !head_dim_ok(dv)) return GDN2_ERR_UNSUPPORTED;
    if ((long long)N * H > 0x7fffffffLL) return GDN2_ERR_UNSUPPORTED;
    const void *ptrs[] = {q, k, v, log_alpha, b, w, S, o};
    for (const void *p : ptrs)
        if (!p || !aligned16(p)) return GDN2_ERR_INVALID;
    gdn2::DecodeArgs a;
    int st;
    if (conv && (st = conv_args(conv, &a.pro)) != GDN2_OK) return st;
    a.q = q; a.k = k; a.v = v; a.b = b; a.w = w;
    a.log_alpha = log_alpha;
    a.S = S;
    a.o = o;
    a.N = N; a.H = H; a.dk = dk; a.dv = dv;
    a.gates = gates;
    a.bf16 = in_dtype == GDN2_BF16;
    prof_call();
    if (gdn2::launch_decode(a, g_stream) != hipSuccess) return GDN2_ERR_HIP;
    return GDN2_OK;
}

int gdn2_decode_step_gates(const void *q, const void *k, const void *v, const float *log_alpha,
                           const void *b, const void *w, int gates, float *S, void *o, int N, int H, int dk,
                           int dv, int in_dtype, int out_dtype)
{
    return decode_impl(q, k, v, log_alpha, b, w, gates, nullptr, S, o, N, H, dk, dv, in_dtype, out_dtype);
}

int gdn2_decode_step_prologue(const void *q_raw, const void *k_raw, const void *v_raw, const float *log_alpha,
                              const void *b_logit, const void *w_logit, const gdn2_short_conv *conv, float *S,
                              void *o, int N, int H, int dk, int dv, int in_dtype, int out_dtype)
{
    if (!conv) return GDN2_ERR_INVALID;
    return decode_impl(q_raw, k_raw, v_raw, log_alpha, b_logit, w_logit, GDN2_GATES_PER_CHANNEL, conv, S, o, N, H,
                       dk, dv, in_dtype, out_dtype);
}

} // extern "C"
