// C ABI of the GQE library: argument checks, then kernel launches on the
// caller's stream.  Nothing here allocates, frees or synchronises.
#include "gqe.h"

#include <hip/hip_runtime.h>

#include "gqe_launch.h"

namespace {

constexpr int kMaxHq = 64;   // experts a router workgroup keeps in LDS
constexpr int kMaxK = 8;     // kept experts per group held in registers

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

struct Shape {
    int B, T, dm, Hq, G, E, k, D, ns, causal, mode, S;
    bool bf16;
    long long BT;
};

// Shared checks of the descriptor.  Returns GQE_OK or a negative status.
int check_desc(const gqe_desc* d, Shape& s)
{
    if (!d) return GQE_ERR_INVALID;
    if (d->B < 0 || d->T < 0 || d->d_model < 1 || d->H_q < 1 || d->H_kv < 1) return GQE_ERR_INVALID;
    if (d->H_q % d->H_kv != 0) return GQE_ERR_INVALID;
    const int E = d->H_q / d->H_kv;
    if (d->k < 1 || d->k > E) return GQE_ERR_INVALID;
    if (d->n_shared != 0 && d->n_shared != 1) return GQE_ERR_INVALID;
    if (d->causal != 0 && d->causal != 1) return GQE_ERR_INVALID;
    if (d->route_mode < 0 || d->route_mode > 3) return GQE_ERR_INVALID;
    if (d->dtype != GQE_F32 && d->dtype != GQE_BF16) return GQE_ERR_INVALID;
    if (d->d_head != 32 && d->d_head != 64 && d->d_head != 128) return GQE_ERR_UNSUPPORTED;
    if (d->H_q > kMaxHq || d->k > kMaxK) return GQE_ERR_UNSUPPORTED;
    if (d->dtype == GQE_BF16 && d->d_model % 64 != 0) return GQE_ERR_UNSUPPORTED;
    const long long BT = (long long)d->B * d->T;
    // every index that reaches an int in a kernel stays below 2^31
    if (BT * d->H_kv * d->k >= (1ll << 31) || (long long)d->T * d->k >= (1ll << 31) - 256) return GQE_ERR_UNSUPPORTED;
    s.B = d->B; s.T = d->T; s.dm = d->d_model; s.Hq = d->H_q; s.G = d->H_kv; s.E = E; s.k = d->k;
    s.D = d->d_head; s.ns = d->n_shared; s.causal = d->causal; s.mode = d->route_mode;
    s.S = d->k * d->H_kv + (d->route_mode == 0 ? 1 : d->route_mode == 1 ? d->H_kv : 0) + d->n_shared;   // modes 2, 3: none
    s.bf16 = d->dtype == GQE_BF16;
    s.BT = BT;
    return GQE_OK;
}

// A required pointer: non-NULL and 16-byte aligned.
int need(const void* p)
{
    if (!p) return GQE_ERR_INVALID;
    return aligned16(p) ? GQE_OK : GQE_ERR_ALIGN;
}
// An optional pointer: NULL or 16-byte aligned.
int maybe(const void* p) { return (!p || aligned16(p)) ? GQE_OK : GQE_ERR_ALIGN; }

#define GQE_TRY(expr)                \
    do {                             \
        const int _rc = (expr);      \
        if (_rc != GQE_OK) return _rc; \
    } while (0)

int launch_status(int rc)
{
    if (rc == -2) return GQE_ERR_UNSUPPORTED;
    return rc == 0 ? GQE_OK : GQE_ERR_LAUNCH;
}

size_t prefill_ws_bytes(const Shape& s)
{
    return gqe::prefill_workspace_bytes(s.B, s.T, s.G, s.k, s.D, s.ns, s.causal, s.bf16);
}

int prefill_common(const gqe_desc* desc, const void* q_routed, const void* q_shared, const void* k, const void* v,
                   const float* p_tilde, float* out, void* workspace, size_t workspace_bytes, void* stream,
                   bool assemble, float* lse = nullptr)
{
    Shape s;
    GQE_TRY(check_desc(desc, s));
    if (s.BT == 0) return GQE_OK;
    // a NULL q_routed / q_shared leaves that part out of this call; the
    // weighted slots need the routed hard slots
    if (assemble) GQE_TRY(need(q_routed));
    GQE_TRY(maybe(q_routed));
    GQE_TRY(maybe(q_shared));
    const bool shared = s.ns && q_shared;
    if (!q_routed && !shared) return GQE_OK;
    GQE_TRY(need(k));
    GQE_TRY(need(v));
    if (assemble) GQE_TRY(need(p_tilde));
    GQE_TRY(need(out));
    GQE_TRY(maybe(workspace));
    if (workspace && workspace_bytes < prefill_ws_bytes(s)) return GQE_ERR_WORKSPACE;
    gqe::PrefillArgs a{q_routed, shared ? q_shared : nullptr, k, v, p_tilde, out, workspace,
                       s.B, s.T, s.G, s.k, s.D, s.ns, s.causal, s.mode, s.S, s.bf16};
    a.lse = lse;
    return launch_status(assemble ? gqe::launch_prefill(a, (hipStream_t)stream)
                                  : gqe::launch_prefill_heads(a, (hipStream_t)stream));
}

int attn_backward_common(const gqe_desc* desc, const void* q_routed, const void* q_shared, const void* k,
                         const void* v, const float* out, const float* d_hard, const float* dout, const float* lse,
                         float* dq_routed, float* dq_shared, float* dk, float* dv, void* workspace,
                         size_t workspace_bytes, void* stream)
{
    Shape s;
    GQE_TRY(check_desc(desc, s));
    if (!s.bf16) return GQE_ERR_UNSUPPORTED;
    if (s.BT == 0) return GQE_OK;
    GQE_TRY(need(q_routed));
    GQE_TRY(need(k));
    GQE_TRY(need(v));
    GQE_TRY(need(out));
    GQE_TRY(need(d_hard));
    GQE_TRY(need(dq_routed));
    GQE_TRY(need(dk));
    GQE_TRY(need(dv));
    if (s.ns) {
        GQE_TRY(need(q_shared));
        GQE_TRY(need(dout));
        GQE_TRY(need(dq_shared));
    }
    if (!workspace) return GQE_ERR_WORKSPACE;
    GQE_TRY(need(workspace));
    if (workspace_bytes < gqe::attn_bwd_workspace_bytes(s.B, s.T, s.G, s.k, s.ns)) return GQE_ERR_WORKSPACE;
    const long long rows = (long long)s.B * s.G * s.T * s.k + (s.ns ? s.BT : 0);
    gqe::AttnBwdArgs a{q_routed, s.ns ? q_shared : nullptr, k, v, out, d_hard, s.ns ? dout : nullptr, dq_routed,
                       s.ns ? dq_shared : nullptr, dk, dv, (float*)workspace, (float*)workspace + rows,
                       s.B, s.T, s.G, s.k, s.S, s.D, s.causal, s.ns,
                       1.4426950408889634f / sqrtf((float)s.D), 1.f / sqrtf((float)s.D)};
    if (lse) {
        // the forward's statistics take the workspace's first half's place; the kernels do not write them
        a.lse = const_cast<float*>(lse);
        a.lse_given = true;
    }
    return launch_status(gqe::launch_attn_bwd(a, (hipStream_t)stream));
}

}  // namespace

extern "C" {

int gqe_num_slots(const gqe_desc* desc)
{
    Shape s;
    if (check_desc(desc, s) != GQE_OK) return -1;
    return s.S;
}

const char* gqe_status_string(int status)
{
    switch (status) {
    case GQE_OK: return "ok";
    case GQE_ERR_INVALID: return "invalid argument";
    case GQE_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case GQE_ERR_ALIGN: return "pointer not 16-byte aligned";
    case GQE_ERR_LAUNCH: return "kernel launch failed";
    case GQE_ERR_WORKSPACE: return "workspace missing or too small";
    case GQE_ERR_SCRATCH: return "call needs more than the static scratch holds";
    default: return "unknown status";
    }
}

size_t gqe_route_workspace_bytes(const gqe_desc* desc)
{
    Shape s;
    if (check_desc(desc, s) != GQE_OK) return 0;
    return gqe::route_workspace_bytes((int)s.BT, s.Hq);
}

int gqe_route(const gqe_desc* desc, const void* x, const void* w_router, const float* b_router, int32_t* sel,
              float* p_tilde, int32_t* counts, int32_t* offsets, int32_t* rows, double* logits, void* workspace,
              size_t workspace_bytes, void* stream)
{
    Shape s;
    GQE_TRY(check_desc(desc, s));
    GQE_TRY(need(counts));
    GQE_TRY(need(offsets));
    if (s.BT > 0) {
        GQE_TRY(need(x));
        GQE_TRY(need(w_router));
        GQE_TRY(maybe(b_router));
        GQE_TRY(need(sel));
        GQE_TRY(need(p_tilde));
        GQE_TRY(need(rows));
        GQE_TRY(maybe(logits));
        if (!workspace) return GQE_ERR_WORKSPACE;
        GQE_TRY(need(workspace));
        if (workspace_bytes < gqe::route_workspace_bytes((int)s.BT, s.Hq)) return GQE_ERR_WORKSPACE;
    }
    gqe::RouteArgs a{x, w_router, b_router, sel, p_tilde, counts, offsets, rows, logits, workspace,
                     (int)s.BT, s.dm, s.G, s.E, s.k, s.bf16};
    a.renorm = s.mode != 3;
    return launch_status(gqe::launch_route(a, (hipStream_t)stream));
}

int gqe_qproj(const gqe_desc* desc, const void* x, const void* w_q, const int32_t* sel, const int32_t* counts,
              const int32_t* offsets, const int32_t* rows, void* q_routed, void* q_shared, void* stream)
{
    Shape s;
    GQE_TRY(check_desc(desc, s));
    if (s.BT == 0) return GQE_OK;
    // a NULL q_routed / q_shared leaves that part out of this call
    GQE_TRY(maybe(q_routed));
    GQE_TRY(maybe(q_shared));
    const bool shared = s.ns && q_shared;
    if (!q_routed && !shared) return GQE_OK;
    GQE_TRY(need(x));
    GQE_TRY(need(w_q));
    if (q_routed) {
        GQE_TRY(need(sel));
        GQE_TRY(need(counts));
        GQE_TRY(need(offsets));
        GQE_TRY(need(rows));
    }
    gqe::QprojArgs a{x, w_q, sel, counts, offsets, rows, q_routed, shared ? q_shared : nullptr,
                     s.B, s.T, s.dm, s.G, s.E, s.k, s.D, s.ns, s.bf16};
    return launch_status(gqe::launch_qproj(a, (hipStream_t)stream));
}

size_t gqe_attn_prefill_workspace_bytes(const gqe_desc* desc)
{
    Shape s;
    if (check_desc(desc, s) != GQE_OK) return 0;
    return prefill_ws_bytes(s);
}

int64_t gqe_attn_prefill_plan(const gqe_desc* desc, int split, int32_t* items, int64_t max_items)
{
    Shape s;
    GQE_TRY(check_desc(desc, s));
    if (!s.bf16) return GQE_ERR_UNSUPPORTED;
    if (max_items < 0) return GQE_ERR_INVALID;
    return gqe::prefill_plan(s.B, s.T, s.G, s.k, s.D, s.ns, s.causal, split != 0 && prefill_ws_bytes(s) > 0, items,
                             max_items);
}

int gqe_attn_prefill(const gqe_desc* desc, const void* q_routed, const void* q_shared, const void* k, const void* v,
                     const float* p_tilde, float* out, void* workspace, size_t workspace_bytes, void* stream)
{
    return prefill_common(desc, q_routed, q_shared, k, v, p_tilde, out, workspace, workspace_bytes, stream, true);
}

int gqe_attn_prefill_heads(const gqe_desc* desc, const void* q_routed, const void* q_shared, const void* k,
                           const void* v, float* out, void* workspace, size_t workspace_bytes, void* stream)
{
    return prefill_common(desc, q_routed, q_shared, k, v, nullptr, out, workspace, workspace_bytes, stream, false);
}

int gqe_attn_prefill_heads_lse(const gqe_desc* desc, const void* q_routed, const void* q_shared, const void* k,
                               const void* v, float* out, float* lse, void* workspace, size_t workspace_bytes,
                               void* stream)
{
    Shape s;
    GQE_TRY(check_desc(desc, s));
    if (!s.bf16) return GQE_ERR_UNSUPPORTED;
    if (s.BT == 0) return GQE_OK;
    GQE_TRY(need(lse));
    return prefill_common(desc, q_routed, q_shared, k, v, nullptr, out, workspace, workspace_bytes, stream, false,
                          lse);
}

int gqe_assemble(const gqe_desc* desc, const float* p_tilde, float* out, void* stream)
{
    Shape s;
    GQE_TRY(check_desc(desc, s));
    if (s.BT == 0) return GQE_OK;
    GQE_TRY(need(p_tilde));
    GQE_TRY(need(out));
    return launch_status(gqe::launch_assemble(p_tilde, out, s.BT, s.G, s.k, s.D, s.S, s.mode, (hipStream_t)stream));
}

size_t gqe_route_backward_workspace_bytes(const gqe_desc* desc)
{
    Shape s;
    if (check_desc(desc, s) != GQE_OK) return 0;
    return gqe::route_bwd_workspace_bytes(s.BT, s.Hq, s.dm);
}

int gqe_route_backward(const gqe_desc* desc, const float* dout, const float* out, const int32_t* sel,
                       const float* p_tilde, const void* x, const void* w_router, float* d_hard, float* d_logits,
                       float* dw_router, float* db_router, float* dx, void* workspace, size_t workspace_bytes,
                       void* stream)
{
    Shape s;
    GQE_TRY(check_desc(desc, s));
    if (s.BT * s.dm >= (1ll << 40)) return GQE_ERR_UNSUPPORTED;
    // route mode 3 scales the hard slots by the group softmax, whose gradient
    // reaches experts that were not kept; not built
    if (s.mode == 3) return GQE_ERR_UNSUPPORTED;
    if (s.BT == 0) return GQE_OK;
    GQE_TRY(need(dout));
    GQE_TRY(need(out));
    GQE_TRY(need(sel));
    GQE_TRY(need(p_tilde));
    GQE_TRY(need(d_hard));
    GQE_TRY(need(d_logits));
    GQE_TRY(maybe(dw_router));
    GQE_TRY(maybe(db_router));
    GQE_TRY(maybe(dx));
    if (db_router && !dw_router) return GQE_ERR_INVALID;
    if (dw_router) GQE_TRY(need(x));
    if (dx) GQE_TRY(need(w_router));
    if (dw_router) {
        if (!workspace) return GQE_ERR_WORKSPACE;
        GQE_TRY(need(workspace));
        if (workspace_bytes < gqe::route_bwd_workspace_bytes(s.BT, s.Hq, s.dm)) return GQE_ERR_WORKSPACE;
    }
    gqe::RouteBwdArgs a{dout, out, sel, p_tilde, x, w_router, d_hard, d_logits, dw_router, db_router, dx,
                        workspace, s.BT, s.G, s.E, s.k, s.D, s.dm, s.S, s.mode, s.bf16};
    return launch_status(gqe::launch_route_bwd(a, (hipStream_t)stream));
}

int gqe_route_stats(const gqe_desc* desc, const double* logits, float* importance, void* stream)
{
    Shape s;
    GQE_TRY(check_desc(desc, s));
    GQE_TRY(need(importance));
    if (s.BT > 0) GQE_TRY(need(logits));   // (with no tokens every importance is 0)
    return launch_status(gqe::launch_route_stats(logits, s.BT, s.G, s.E, importance, (hipStream_t)stream));
}

size_t gqe_attn_backward_workspace_bytes(const gqe_desc* desc)
{
    Shape s;
    if (check_desc(desc, s) != GQE_OK) return 0;
    return gqe::attn_bwd_workspace_bytes(s.B, s.T, s.G, s.k, s.ns);
}


int gqe_attn_backward(const gqe_desc* desc, const void* q_routed, const void* q_shared, const void* k,
                      const void* v, const float* out, const float* d_hard, const float* dout, float* dq_routed,
                      float* dq_shared, float* dk, float* dv, void* workspace, size_t workspace_bytes, void* stream)
{
    return attn_backward_common(desc, q_routed, q_shared, k, v, out, d_hard, dout, nullptr, dq_routed, dq_shared, dk,
                                dv, workspace, workspace_bytes, stream);
}

int gqe_attn_backward_lse(const gqe_desc* desc, const void* q_routed, const void* q_shared, const void* k,
                          const void* v, const float* out, const float* d_hard, const float* dout, const float* lse,
                          float* dq_routed, float* dq_shared, float* dk, float* dv, void* workspace,
                          size_t workspace_bytes, void* stream)
{
    Shape s;
    GQE_TRY(check_desc(desc, s));
    if (!s.bf16) return GQE_ERR_UNSUPPORTED;
    if (s.BT == 0) return GQE_OK;
    GQE_TRY(need(lse));
    return attn_backward_common(desc, q_routed, q_shared, k, v, out, d_hard, dout, lse, dq_routed, dq_shared, dk, dv,
                                workspace, workspace_bytes, stream);
}


int gqe_kv_proj(const gqe_desc* desc, const void* x, const void* w_k, const void* w_v, void* k, void* v,
                void* stream)
{
    Shape s;
    GQE_TRY(check_desc(desc, s));
    if (s.BT * s.G >= (1ll << 31)) return GQE_ERR_UNSUPPORTED;
    if (s.BT == 0) return GQE_OK;
    GQE_TRY(need(x));
    GQE_TRY(need(w_k));
    GQE_TRY(need(w_v));
    GQE_TRY(need(k));
    GQE_TRY(need(v));
    gqe::KvProjArgs a{x, w_k, w_v, k, v, s.B, s.T, s.dm, s.G, s.D, s.bf16};
    return launch_status(gqe::launch_kv_proj(a, (hipStream_t)stream));
}

int gqe_qkv_proj(const gqe_desc* desc, const void* x, const void* w_q, const void* w_k, const void* w_v,
                 const int32_t* sel, const int32_t* counts, const int32_t* offsets, const int32_t* rows,
                 const int32_t* positions, float rope_base, void* q_routed, void* q_shared, void* k, void* v,
                 void* stream)
{
    Shape s;
    GQE_TRY(check_desc(desc, s));
    if (!(rope_base == 0.f || rope_base > 1.f) || !(rope_base < 3.0e38f)) return GQE_ERR_INVALID;
    if (s.BT * s.G >= (1ll << 31)) return GQE_ERR_UNSUPPORTED;
    if (s.BT == 0) return GQE_OK;
    GQE_TRY(need(x));
    GQE_TRY(need(w_q));
    GQE_TRY(need(w_k));
    GQE_TRY(need(w_v));
    GQE_TRY(need(sel));
    GQE_TRY(need(counts));
    GQE_TRY(need(offsets));
    GQE_TRY(need(rows));
    GQE_TRY(maybe(positions));
    GQE_TRY(need(q_routed));
    if (s.ns) GQE_TRY(need(q_shared));
    GQE_TRY(need(k));
    GQE_TRY(need(v));
    gqe::QkvProjArgs a{};
    a.x = x; a.w_q = w_q; a.w_k = w_k; a.w_v = w_v; a.sel = sel; a.counts = counts; a.offsets = offsets;
    a.rows = rows; a.positions = positions; a.q_routed = q_routed; a.q_shared = q_shared; a.k = k; a.v = v;
    a.rope_base = rope_base;
    a.B = s.B; a.T = s.T; a.d_model = s.dm; a.G = s.G; a.E = s.E; a.k_ = s.k; a.d_head = s.D; a.n_shared = s.ns;
    a.H_kv = s.G; a.bf16 = s.bf16;
    return launch_status(gqe::launch_qkv_proj(a, (hipStream_t)stream));
}

size_t gqe_qkv_proj_backward_workspace_bytes(const gqe_desc* desc, int32_t with_kv)
{
    Shape s;
    if (check_desc(desc, s) != GQE_OK || !s.bf16 || s.BT == 0) return 0;
    gqe::ProjBwdArgs a{};
    a.B = s.B; a.T = s.T; a.d_model = s.dm; a.G = s.G; a.E = s.E; a.k = s.k; a.D = s.D; a.ns = s.ns;
    a.nkv = with_kv ? s.G : 0;
    return gqe::proj_bwd_workspace_bytes(a);
}

int gqe_qkv_proj_backward(const gqe_desc* desc, const void* x, const void* w_q, const void* w_k, const void* w_v,
                          const int32_t* sel, const int32_t* counts, const int32_t* offsets, const int32_t* rows,
                          const int32_t* positions, float rope_base, const float* dq_routed, const float* dq_shared,
                          const float* dk, const float* dv, float* dw_q, float* dw_k, float* dw_v, float* dx,
                          void* workspace, size_t workspace_bytes, void* stream)
{
    Shape s;
    GQE_TRY(check_desc(desc, s));
    if (!s.bf16) return GQE_ERR_UNSUPPORTED;
    if (!(rope_base == 0.f || rope_base > 1.f) || !(rope_base < 3.0e38f)) return GQE_ERR_INVALID;
    if ((dk == nullptr) != (dv == nullptr)) return GQE_ERR_INVALID;
    if (!dk && (dw_k || dw_v)) return GQE_ERR_INVALID;
    if (s.BT * s.G >= (1ll << 31) || s.BT * s.dm >= (1ll << 40)) return GQE_ERR_UNSUPPORTED;
    if (s.BT == 0) return GQE_OK;
    if (!dw_q && !dw_k && !dw_v && !dx) return GQE_OK;
    GQE_TRY(need(sel));
    GQE_TRY(need(counts));
    GQE_TRY(need(offsets));
    GQE_TRY(need(rows));
    GQE_TRY(maybe(positions));
    GQE_TRY(need(dq_routed));
    if (s.ns) GQE_TRY(need(dq_shared));
    GQE_TRY(maybe(dk));
    GQE_TRY(maybe(dv));
    GQE_TRY(maybe(dw_q));
    GQE_TRY(maybe(dw_k));
    GQE_TRY(maybe(dw_v));
    GQE_TRY(maybe(dx));
    GQE_TRY(maybe(workspace));
    if (dw_q || dw_k || dw_v) GQE_TRY(need(x));
    if (dx) {
        GQE_TRY(need(w_q));
        if (dk) {
            GQE_TRY(need(w_k));
            GQE_TRY(need(w_v));
        }
    }
    gqe::ProjBwdArgs a{};
    a.x = (const uint16_t*)x; a.w_q = (const uint16_t*)w_q; a.w_k = (const uint16_t*)w_k;
    a.w_v = (const uint16_t*)w_v; a.sel = sel; a.counts = counts; a.offsets = offsets; a.rows = rows;
    a.positions = positions; a.dq_routed = dq_routed; a.dq_shared = dq_shared; a.dk = dk; a.dv = dv;
    a.dw_q = dw_q; a.dw_k = dw_k; a.dw_v = dw_v; a.dx = dx;
    a.B = s.B; a.T = s.T; a.d_model = s.dm; a.G = s.G; a.E = s.E; a.k = s.k; a.D = s.D; a.ns = s.ns;
    a.nkv = dk ? s.G : 0;
    a.rope_log2_base = rope_base > 0.f ? log2((double)rope_base) : 0.0;
    if (workspace && workspace_bytes < gqe::proj_bwd_workspace_bytes(a)) return GQE_ERR_WORKSPACE;
    return launch_status(gqe::launch_proj_bwd(a, workspace, workspace_bytes, (hipStream_t)stream));
}

int gqe_out_proj(const gqe_desc* desc, float* out, const float* p_tilde, const void* w_o, float* y,
                 int32_t write_weighted, void* stream)
{
    Shape s;
    GQE_TRY(check_desc(desc, s));
    if (write_weighted != 0 && write_weighted != 1) return GQE_ERR_INVALID;
    if ((long long)s.dm * s.S * s.D >= (1ll << 31)) return GQE_ERR_UNSUPPORTED;
    if (s.BT == 0) return GQE_OK;
    GQE_TRY(need(out));
    GQE_TRY(need(p_tilde));
    GQE_TRY(need(w_o));
    GQE_TRY(need(y));
    gqe::OutProjArgs a;
    a.out = out; a.p_tilde = p_tilde; a.w_o = w_o; a.y = y; a.BT = s.BT;
    a.d_model = s.dm; a.G = s.G; a.k = s.k; a.d_head = s.D; a.n_shared = s.ns; a.route_mode = s.mode; a.S = s.S;
    a.write_weighted = write_weighted; a.bf16 = s.bf16;
    return launch_status(gqe::launch_out_proj(a, (hipStream_t)stream));
}

size_t gqe_out_proj_packed_bytes(const gqe_desc* desc)
{
    Shape s;
    if (check_desc(desc, s) != GQE_OK || !s.bf16) return 0;
    if ((long long)s.dm * s.S * s.D >= (1ll << 31) || !gqe::out_proj_tile_fits(s.S * s.D, s.dm)) return 0;
    return (size_t)s.dm * s.S * s.D * 2;
}

int gqe_out_proj_pack(const gqe_desc* desc, const void* w_o, void* w_packed, void* stream)
{
    if (gqe_out_proj_packed_bytes(desc) == 0) {
        Shape s;
        GQE_TRY(check_desc(desc, s));
        return GQE_ERR_UNSUPPORTED;
    }
    Shape s;
    GQE_TRY(check_desc(desc, s));
    GQE_TRY(need(w_o));
    GQE_TRY(need(w_packed));
    return launch_status(gqe::launch_out_proj_pack(w_o, w_packed, s.dm, s.S * s.D, (hipStream_t)stream));
}

int gqe_out_proj_packed(const gqe_desc* desc, float* out, const float* p_tilde, const void* w_packed, float* y,
                        int32_t write_weighted, void* stream)
{
    Shape s;
    GQE_TRY(check_desc(desc, s));
    if (write_weighted != 0 && write_weighted != 1) return GQE_ERR_INVALID;
    if (gqe_out_proj_packed_bytes(desc) == 0) return GQE_ERR_UNSUPPORTED;
    if (s.BT == 0) return GQE_OK;
    GQE_TRY(need(out));
    GQE_TRY(need(p_tilde));
    GQE_TRY(need(w_packed));
    GQE_TRY(need(y));
    gqe::OutProjArgs a;
    a.out = out; a.p_tilde = p_tilde; a.w_o = nullptr; a.w_packed = w_packed; a.y = y; a.BT = s.BT;
    a.d_model = s.dm; a.G = s.G; a.k = s.k; a.d_head = s.D; a.n_shared = s.ns; a.route_mode = s.mode; a.S = s.S;
    a.write_weighted = write_weighted; a.bf16 = true;
    return launch_status(gqe::launch_out_proj(a, (hipStream_t)stream));
}

size_t gqe_decode_workspace_bytes(const gqe_desc* desc, int32_t L_max)
{
    Shape s;
    if (check_desc(desc, s) != GQE_OK || L_max < 1) return 0;
    return gqe::decode_workspace_bytes(s.B, s.G, s.k, s.ns, s.D, L_max, s.bf16);
}

int gqe_attn_decode(const gqe_desc* desc, const void* q_routed, const void* q_shared, const void* k_cache,
                    const void* v_cache, int32_t L_max, const int32_t* lens, const float* p_tilde, float* out,
                    void* workspace, size_t workspace_bytes, void* stream)
{
    Shape s;
    GQE_TRY(check_desc(desc, s));
    if (s.T != 1 || L_max < 1) return GQE_ERR_INVALID;
    if ((long long)s.B * s.G * L_max * s.D >= (1ll << 40)) return GQE_ERR_UNSUPPORTED;
    if (s.B == 0) return GQE_OK;
    GQE_TRY(need(q_routed));
    if (s.ns) GQE_TRY(need(q_shared));
    GQE_TRY(need(k_cache));
    GQE_TRY(need(v_cache));
    GQE_TRY(need(lens));
    GQE_TRY(need(p_tilde));
    GQE_TRY(need(out));
    if (!workspace) return GQE_ERR_WORKSPACE;
    GQE_TRY(need(workspace));
    if (workspace_bytes < gqe::decode_workspace_bytes(s.B, s.G, s.k, s.ns, s.D, L_max, s.bf16))
        return GQE_ERR_WORKSPACE;
    gqe::DecodeArgs a{q_routed, q_shared, k_cache, v_cache, lens, p_tilde, out, workspace,
                      s.B, s.G, s.k, s.D, s.ns, s.mode, s.S, L_max, s.bf16};
    return launch_status(gqe::launch_decode(a, (hipStream_t)stream));
}

int gqe_decode_route_qproj(const gqe_desc* desc, const void* x, const void* w_router, const float* b_router,
                           const void* w_q, const int32_t* positions, float rope_base, int32_t* sel, float* p_tilde,
                           void* q_routed, void* q_shared, double* logits, void* stream)
{
    Shape s;
    GQE_TRY(check_desc(desc, s));
    if (s.T != 1) return GQE_ERR_INVALID;
    if (!(rope_base == 0.f || rope_base > 1.f) || !(rope_base < 3.0e38f)) return GQE_ERR_INVALID;
    if (rope_base > 0.f && !positions) return GQE_ERR_INVALID;
    if (s.B == 0) return GQE_OK;
    GQE_TRY(need(x));
    GQE_TRY(need(w_router));
    GQE_TRY(maybe(b_router));
    GQE_TRY(need(w_q));
    GQE_TRY(maybe(positions));
    GQE_TRY(need(sel));
    GQE_TRY(need(p_tilde));
    GQE_TRY(need(q_routed));
    if (s.ns) GQE_TRY(need(q_shared));
    GQE_TRY(maybe(logits));
    gqe::DecodePreArgs a{};
    a.x = x; a.w_router = w_router; a.b_router = b_router; a.w_q = w_q; a.positions = positions; a.sel = sel;
    a.p_tilde = p_tilde; a.q_routed = q_routed; a.q_shared = s.ns ? q_shared : nullptr; a.logits = logits;
    a.B = s.B; a.d_model = s.dm; a.G = s.G; a.E = s.E; a.k = s.k; a.d_head = s.D; a.bf16 = s.bf16;
    a.renorm = s.mode != 3;
    a.rope_log2_base = rope_base > 0.f ? log2((double)rope_base) : 0.0;
    return launch_status(gqe::launch_decode_preamble(a, (hipStream_t)stream));
}

int gqe_attn_decode_noalloc(const gqe_desc* desc, const void* q_routed, const void* q_shared, const void* k_cache,
                            const void* v_cache, int32_t L_max, const int32_t* lens, const float* p_tilde, float* out,
                            void* stream)
{
    static_assert(GQE_DECODE_SCRATCH_BYTES == gqe::kDecodeScratchBytes, "scratch size in gqe.h");
    Shape s;
    GQE_TRY(check_desc(desc, s));
    if (s.T != 1 || L_max < 1) return GQE_ERR_INVALID;
    if ((long long)s.B * s.G * L_max * s.D >= (1ll << 40)) return GQE_ERR_UNSUPPORTED;
    if (s.B == 0) return GQE_OK;
    GQE_TRY(need(q_routed));
    if (s.ns) GQE_TRY(need(q_shared));
    GQE_TRY(need(k_cache));
    GQE_TRY(need(v_cache));
    GQE_TRY(need(lens));
    GQE_TRY(need(p_tilde));
    GQE_TRY(need(out));
    if (gqe::decode_workspace_bytes(s.B, s.G, s.k, s.ns, s.D, L_max, s.bf16) > gqe::kDecodeScratchBytes)
        return GQE_ERR_SCRATCH;
    void* scratch = nullptr;
    if (gqe::decode_scratch(&scratch) != 0) return GQE_ERR_LAUNCH;
    gqe::DecodeArgs a{q_routed, q_shared, k_cache, v_cache, lens, p_tilde, out, scratch,
                      s.B, s.G, s.k, s.D, s.ns, s.mode, s.S, L_max, s.bf16};
    return launch_status(gqe::launch_decode(a, (hipStream_t)stream));
}

int gqe_check_decode_inputs(const gqe_desc* desc, const int32_t* lens, int32_t L_max, const int32_t* block_table,
                            int32_t num_pages, int32_t page_size, int32_t max_pages, int32_t* bad, void* stream)
{
    Shape s;
    GQE_TRY(check_desc(desc, s));
    if (L_max < 1) return GQE_ERR_INVALID;
    GQE_TRY(need(lens));
    GQE_TRY(need(bad));
    GQE_TRY(maybe(block_table));
    if (block_table) {
        if (num_pages < 1 || max_pages < 1 || page_size < 1) return GQE_ERR_INVALID;
        if ((long long)max_pages * page_size < L_max) return GQE_ERR_INVALID;
    }
    return launch_status(gqe::launch_decode_check(lens, s.B, L_max, block_table, page_size, max_pages, num_pages,
                                                  bad, (hipStream_t)stream));
}

int gqe_attn_decode_paged(const gqe_desc* desc, const void* q_routed, const void* q_shared, const void* k_pages,
                          const void* v_pages, int32_t num_pages, int32_t page_size, int32_t max_pages,
                          const int32_t* block_table, const int32_t* lens, const float* p_tilde, float* out,
                          void* workspace, size_t workspace_bytes, void* stream)
{
    Shape s;
    GQE_TRY(check_desc(desc, s));
    if (s.T != 1 || num_pages < 1 || max_pages < 1) return GQE_ERR_INVALID;
    if (page_size < 8 || page_size > 4096 || (page_size & (page_size - 1)) != 0) return GQE_ERR_INVALID;
    const long long L_max = (long long)max_pages * page_size;
    if (L_max >= (1ll << 30) || (long long)num_pages * s.G * page_size * s.D >= (1ll << 40)) return GQE_ERR_UNSUPPORTED;
    if (s.B == 0) return GQE_OK;
    GQE_TRY(need(q_routed));
    if (s.ns) GQE_TRY(need(q_shared));
    GQE_TRY(need(k_pages));
    GQE_TRY(need(v_pages));
    GQE_TRY(need(block_table));
    GQE_TRY(need(lens));
    GQE_TRY(need(p_tilde));
    GQE_TRY(need(out));
    if (!workspace) return GQE_ERR_WORKSPACE;
    GQE_TRY(need(workspace));
    if (workspace_bytes < gqe::decode_workspace_bytes(s.B, s.G, s.k, s.ns, s.D, (int)L_max, s.bf16))
        return GQE_ERR_WORKSPACE;
    gqe::DecodeArgs a{q_routed, q_shared, k_pages, v_pages, lens, p_tilde, out, workspace,
                      s.B, s.G, s.k, s.D, s.ns, s.mode, s.S, (int)L_max, s.bf16};
    a.block_table = block_table;
    a.page_shift = __builtin_ctz((unsigned)page_size);
    a.max_pages = max_pages;
    a.num_pages = num_pages;
    return launch_status(gqe::launch_decode(a, (hipStream_t)stream));
}

}  // extern "C"
