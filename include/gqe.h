/*
 * gqe.h -- C ABI of the GQE (Grouped Query Experts) attention forward library
 * for AMD Instinct MI355X (gfx950).
 *
 * The method (GQE study note, dimensionstp.github.io, §3-2 (1)-(5)): the H_q
 * query heads of grouped-query attention form G = H_kv groups of E = H_q / G
 * query-head "experts".  For every token and group a router scores the E
 * experts, keeps the top k and renormalises their softmax probabilities over
 * the kept ones; only the kept experts are projected and attend, causally,
 * the group's single dense KV head.  The output of a token is the
 * concatenation of the k*G hard-selected head outputs, a router-weighted sum
 * of them, and one always-on shared head.
 *
 * Conventions used throughout
 *   G = H_kv, E = H_q / H_kv, N = G * E (routed experts), global expert index
 *   n = g * E + e (the GQA query-head index of the GQA tutorial, freeguideonline,
 *   "GQA 核心原理与计算流程" step 3).  BT = B * T.
 *   S = k*G + R + n_shared output slots per token, R = 1, G, 0 or 0 weighted
 *   slots for route_mode 0, 1, 2 or 3.
 *   Slot order: hard slots g-major then ascending expert index, weighted
 *   slot(s), shared slot.  The shared head's projection is W_q row block N
 *   and it attends KV head 0.  Attention scale is 1/sqrt(d_head).
 *
 * Pointers: every tensor pointer is a DEVICE pointer owned by the caller,
 * contiguous, row-major in the layout given, and 16-byte aligned.  The
 * library never allocates, frees or synchronises; every call enqueues its
 * kernels on `stream` (a hipStream_t, NULL = the default stream) and returns.
 * Outputs are fully overwritten.  Calls keep no state between them and may
 * be made from several host threads.
 *
 * Errors: arguments are checked on the host before anything is enqueued;
 * a negative gqe_status is returned and nothing runs.  A failed launch
 * returns GQE_ERR_LAUNCH.  Device-side preconditions that the host cannot
 * see (decode lengths in 1..L_max, sel values in 0..E-1 handed to gqe_qproj)
 * are the caller's responsibility.
 */
#ifndef GQE_H
#define GQE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GQE_OK = 0,
    GQE_ERR_INVALID = -1,      /* bad shape, NULL required pointer, k outside 1..E, ... */
    GQE_ERR_UNSUPPORTED = -2,  /* valid but not built: d_head, dtype, too many experts */
    GQE_ERR_ALIGN = -3,        /* a pointer is not 16-byte aligned */
    GQE_ERR_LAUNCH = -4,       /* the HIP runtime rejected a launch */
    GQE_ERR_WORKSPACE = -5,    /* workspace missing or smaller than required */
    GQE_ERR_SCRATCH = -6       /* gqe_attn_decode_noalloc: more than GQE_DECODE_SCRATCH_BYTES needed */
} gqe_status;

typedef enum { GQE_F32 = 0, GQE_BF16 = 1 } gqe_dtype;

/* Shapes and flags of one call.  Problem statement of the GQE study note §1-1
 * (H_q, H_kv, G, E) and §3-2 (2) (top-k per group); d_head is the per-head
 * width d of the attention equation in §1-1. */
typedef struct {
    int32_t B;          /* sequences */
    int32_t T;          /* prefill: tokens per sequence; decode: must be 1 */
    int32_t d_model;    /* width of x; multiple of 64 for bf16, of 4 for f32 */
    int32_t H_q;        /* query heads = routed experts N; at most 64 */
    int32_t H_kv;       /* KV heads = groups G; H_q % H_kv == 0 */
    int32_t k;          /* experts kept per group and token, 1 <= k <= E, k <= 8 */
    int32_t d_head;     /* 32, 64 or 128 */
    int32_t n_shared;   /* 0 or 1: the always-on shared head (reads KV head 0) */
    int32_t causal;     /* 1: key s is visible to query t iff s <= t; 0: all keys */
    int32_t route_mode; /* 0: one weighted slot summed over groups (study note
                           §3-2 (4)); 1: one weighted slot per group; 2: no
                           weighted slot (the "hard concat only" row of the
                           study note's §5-1 ablation table); 3: no weighted
                           slot, each hard slot scaled by its kept expert's
                           group softmax probability, not renormalised (the
                           table's "weighted concat, no renormalized slot"
                           row) */
    int32_t dtype;      /* gqe_dtype of x, W_router, W_q, q, K, V; outputs are fp32 */
} gqe_desc;

/* Number of output slots S per token for this descriptor (or -1 if invalid). */
int gqe_num_slots(const gqe_desc* desc);

/* Human-readable name of a status code (static string). */
const char* gqe_status_string(int status);

/* Bytes of device workspace gqe_route needs (per-block expert counts). */
size_t gqe_route_workspace_bytes(const gqe_desc* desc);

/*
 * gqe_route -- router, in-group softmax, top-k, renormalisation and the
 * expert compaction, for all B*T tokens.
 *
 * Defines (GQE study note §3-2 (2) and (4)):
 *   s[t,n]  = x[t,:] . W_router[n,:] + b_router[n]          (router score)
 *   p[t,g,e] = softmax over the E experts of group g
 *   S[t,g]  = the k largest scores of the group (ties: lower e first),
 *             written in ascending expert index
 *   p~[t,g,j] = p[t,g,S_j] / sum_j' p[t,g,S_j']   (route mode 3: p[t,g,S_j])
 *   counts[n] = tokens that kept expert n;  offsets = exclusive prefix sum,
 *   offsets[N] = BT*G*k;  rows[offsets[n] + r] = the r-th smallest token id
 *   (b*T + t) that kept n.
 *
 * In:  x [BT, d_model] (dtype), w_router [N, d_model] (dtype),
 *      b_router [N] fp32 or NULL (no bias).
 * Out: sel [BT, G, k] int32, p_tilde [BT, G, k] fp32, counts [N] int32,
 *      offsets [N+1] int32, rows [BT*G*k] int32,
 *      logits [BT, N] double or NULL (the router scores, for auditing ties).
 * Workspace: gqe_route_workspace_bytes(desc) bytes of device memory, no
 *      initialisation needed, contents undefined afterwards.
 * Scores accumulate exactly-rounded partial sums of at most 32 products in
 * fp32 into double totals; the comparison that picks the experts is made on
 * those totals.
 */
int gqe_route(const gqe_desc* desc, const void* x, const void* w_router, const float* b_router,
              int32_t* sel, float* p_tilde, int32_t* counts, int32_t* offsets, int32_t* rows,
              double* logits, void* workspace, size_t workspace_bytes, void* stream);

/*
 * gqe_qproj -- routed query projection (grouped GEMM over the compacted rows)
 * plus the shared head.  Each kept expert is its own query projection and
 * unselected experts are never computed (ai-feeds summary of arXiv 2606.20945,
 * 方法/核心模块; GQE study note §3-2 (2), last sentence; §3-2 (5)).
 *
 *   q_routed[b, g, t, j, :] = W_q[g*E + S[t,g]_j] x[b,t,:]     (no bias)
 *   q_shared[b, t, :]       = W_q[N] x[b,t,:]                  (if n_shared)
 *
 * In:  x [BT, d_model]; w_q [N + n_shared, d_head, d_model] (dtype);
 *      sel, counts, offsets, rows as produced by gqe_route (only read, and only
 *      required, when q_routed is given).
 * Out: q_routed [B, G, T, k, d_head] (dtype; bf16 rounds to nearest even from
 *      an fp32 accumulator), q_shared [B, T, d_head].
 * Either output may be NULL: that part is then not computed by this call (with
 * n_shared = 0 q_shared is ignored).  The shared head needs no routing, so a
 * caller can project it on a second stream while gqe_route runs.
 * Within one (b, g) the routed queries form a dense [T*k, d_head] matrix whose
 * row r belongs to position r / k.
 */
int gqe_qproj(const gqe_desc* desc, const void* x, const void* w_q, const int32_t* sel,
              const int32_t* counts, const int32_t* offsets, const int32_t* rows,
              void* q_routed, void* q_shared, void* stream);

/*
 * Bytes of device workspace that lets gqe_attn_prefill / gqe_attn_prefill_heads
 * split the longest causal query tiles (bf16 only; 0 when no tile would be
 * split: f32, non-causal or short sequences).
 *
 * With a workspace, each causal query tile that needs more than 32 key tiles
 * of 64 keys is computed by two workgroups over the two halves of its key
 * range; the one that finishes second merges the two partial softmax states
 * (running reference, row sum, unnormalised output), adding part 0's term
 * first, so the result does not depend on which half finished first.  It
 * differs from the unsplit result only by that regrouping of fp32 sums.  The
 * split keeps the launch's longest workgroups near the average load of a
 * workgroup slot (the causal tile with the most keys otherwise sets the
 * kernel's end).
 *
 * Layout: one int32 counter per split tile (padded to 256 bytes), then the
 * partial states.  The counters must hold even values (zero) before the first
 * call with a buffer -- allocate it zeroed once -- and every completed call
 * leaves them at zero.  Calls that share a workspace must not overlap, except
 * a routed-only and a shared-only call of the same shape (see
 * gqe_attn_prefill_heads).
 */
size_t gqe_attn_prefill_workspace_bytes(const gqe_desc* desc);

/*
 * gqe_attn_prefill_plan -- the work items of one bf16 prefill attention launch,
 * in launch order (for inspection and host tests; computes nothing on the GPU).
 * split != 0 gives the plan used with a workspace.  Writes at most max_items
 * items of 5 int32 each to `items` (host memory, may be NULL):
 *   b, head (H_kv = the shared head), query tile (128 rows; 256 at d_head
 *   128, where a workgroup has eight waves instead of four), part (-1 whole
 *   tile, 0 / 1 first / second half of its key tiles), split-pair index (-1
 *   for a whole tile).
 * Items are ordered by decreasing number of key tiles.  Returns the number of
 * items (the launch's workgroup count) or a negative status.
 */
int64_t gqe_attn_prefill_plan(const gqe_desc* desc, int split, int32_t* items, int64_t max_items);

/*
 * gqe_attn_prefill -- attention of every routed and shared query row against
 * its group's dense, unchanged KV head, then slot assembly.
 *
 *   o = softmax_s(q . K[b,g,s] / sqrt(d_head)) V[b,g,s],  s <= t if causal
 *   (attention equation of GQE study note §1-1; scale as IBM "什么是分组查询注意力")
 *   out[b,t, g*k+j]  = o of routed row (g, j)                 (hard slots, §3-2 (3))
 *   mode 0: out[b,t,kG] = sum_g sum_j p~[t,g,j] o(g,j)         (§3-2 (4))
 *   mode 1: out[b,t,kG+g] = sum_j p~[t,g,j] o(g,j)
 *   mode 3: out[b,t,g*k+j] = p~[t,g,j] o(g,j), p~ then being the group softmax
 *           of the kept expert (study note §5-1 ablation table), no weighted slot
 *   out[b,t,S-1] = o of the shared row against KV head 0       (§3-2 (5))
 *
 * In:  q_routed [B, G, T, k, d_head], q_shared [B, T, d_head] or NULL (the
 *      shared slot is then not written), k, v [B, H_kv, T, d_head] (dtype),
 *      p_tilde [BT, G, k] fp32.
 * Out: out [B, T, S, d_head] fp32.
 * Workspace: NULL (no split tiles) or gqe_attn_prefill_workspace_bytes(desc)
 *      bytes of device memory prepared as described there; a smaller size
 *      returns GQE_ERR_WORKSPACE.
 * bf16: QK^T and PV run on bf16 MFMA with fp32 accumulation; the softmax is
 * fp32 and the probabilities are rounded to bf16 for the PV product.
 */
int gqe_attn_prefill(const gqe_desc* desc, const void* q_routed, const void* q_shared,
                     const void* k, const void* v, const float* p_tilde, float* out,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * gqe_attn_prefill_heads -- the attention part of gqe_attn_prefill alone
 * (same definition, GQE study note §1-1 and §3-2 (3), (5)): writes the hard
 * slots out[b,t,g*k+j] and the shared slot out[b,t,S-1]; the weighted slot(s)
 * of `out` are left as they were.  Together with gqe_assemble it computes
 * exactly what gqe_attn_prefill computes with the same workspace choice
 * (bitwise).
 * In/Out/Workspace: as gqe_attn_prefill, without p_tilde; here q_routed may be
 * NULL too.  A call with only q_routed and one with only q_shared compute
 * exactly what one call with both computes, and may run at the same time on
 * two streams with one workspace (their split tiles use disjoint parts of it).
 */
int gqe_attn_prefill_heads(const gqe_desc* desc, const void* q_routed, const void* q_shared,
                           const void* k, const void* v, float* out, void* workspace,
                           size_t workspace_bytes, void* stream);

/*
 * gqe_attn_prefill_heads_lse -- gqe_attn_prefill_heads (same slots, bit for
 * bit) that also keeps each query row's softmax statistic for the backward:
 *   lse[r] = log2 sum_s 2^(q_r . K_s log2(e) / sqrt(d_head))   (keys s as masked)
 * i.e. the base-2 log of the softmax denominator of the attention equation
 * (GQE study note §1-1), formed from the running reference and row sum the
 * kernel already holds.  bf16 only (GQE_ERR_UNSUPPORTED for fp32).
 * Out: lse [B*G*T*k + B*T] fp32: routed row t*k + j of (b, g) at
 *      (b*G + g)*T*k + t*k + j, then shared row (b, t) at B*G*T*k + b*T + t;
 *      only the rows this call computes are written.
 * Everything else: as gqe_attn_prefill_heads.
 */
int gqe_attn_prefill_heads_lse(const gqe_desc* desc, const void* q_routed, const void* q_shared,
                               const void* k, const void* v, float* out, float* lse, void* workspace,
                               size_t workspace_bytes, void* stream);

/*
 * gqe_assemble -- the weighted slot(s) of B*T output rows from their hard
 * slots (GQE study note §3-2 (4)):
 *   mode 0: out[t, kG]   = sum_g sum_j p~[t,g,j] out[t, g*k+j]
 *   mode 1: out[t, kG+g] = sum_j p~[t,g,j] out[t, g*k+j]
 * summed in fp32 in that fixed order (g, then j).  Reads only the hard slots.
 * mode 3: out[t, g*k+j] *= p~[t,g,j] in place (so a second call scales again).
 * mode 2: nothing to do.
 * In:  p_tilde [B*T, G, k] fp32.  In/Out: out [B*T, S, d_head] fp32.
 * Works for decode outputs too (T = 1).
 */
int gqe_assemble(const gqe_desc* desc, const float* p_tilde, float* out, void* stream);

/*
 * gqe_route_stats -- per-expert router importance, the load statistic a
 * balance loss is formed from together with the per-expert counts gqe_route
 * returns (GQE study note §4 names the loss without its exact form):
 *   importance[g*E + e] = sum over tokens t of softmax_e(logits[t, g, :])
 * (study note §3-2 (2)), accumulated in fp64 in a fixed order, stored fp32.
 * In:  logits [B*T, N] fp64 as gqe_route writes them (may be NULL when
 *      B*T = 0).  Out: importance [N] fp32 (all 0 when B*T = 0).
 */
int gqe_route_stats(const gqe_desc* desc, const double* logits, float* importance, void* stream);

/* Bytes of device workspace gqe_attn_backward needs (two floats per query row). */
size_t gqe_attn_backward_workspace_bytes(const gqe_desc* desc);

/*
 * gqe_attn_backward -- gradients of the routed and shared attention (GQE
 * study note §3-2 (3); GQA tutorial, step 4 of the GQA computation) given the
 * gradient of the hard and shared slots.  Per head, S = q K^T / sqrt(d_head)
 * with the forward's masking, P = softmax(S), O = P V, and
 *   dV = P^T dO,  dS = P o (dO V^T - rowsum(dO o O)),
 *   dq = dS K / sqrt(d_head),  dK = dS^T q / sqrt(d_head),
 * dK and dV of KV head 0 also summing the shared rows' terms.  Routed row
 * t*k + j of group g has dO = d_hard[t, g*k + j] and O = out[t, g*k + j]; a
 * shared row has dout[t, S-1] and out[t, S-1].
 * bf16 only (GQE_ERR_UNSUPPORTED for fp32): q, K, V as the forward reads them;
 * dO, P and dS are rounded to bf16 for the matrix products, which accumulate
 * in fp32.  Deterministic (no atomics; every sum in a fixed order).
 * In:  q_routed [B, G, T*k, d_head], q_shared [B, T, d_head] (n_shared = 1),
 *      k, v [B, H_kv, T, d_head]; out [B*T, S, d_head] fp32 (the forward's
 *      slots), d_hard [B*T, G*k, d_head] fp32 (as gqe_route_backward gives
 *      it: the weighted slot's share already added), dout [B*T, S, d_head] fp32
 *      (only the shared slot is read; n_shared = 1).
 * Out: dq_routed [B, G, T*k, d_head], dq_shared [B, T, d_head] (n_shared = 1),
 *      dk, dv [B, H_kv, T, d_head], all fp32, every element written.
 * Workspace: gqe_attn_backward_workspace_bytes(desc) bytes; no initialisation.
 * q_shared, dout and dq_shared are ignored when n_shared = 0.
 */
int gqe_attn_backward(const gqe_desc* desc, const void* q_routed, const void* q_shared, const void* k,
                      const void* v, const float* out, const float* d_hard, const float* dout,
                      float* dq_routed, float* dq_shared, float* dk, float* dv, void* workspace,
                      size_t workspace_bytes, void* stream);

/*
 * gqe_attn_backward_lse -- gqe_attn_backward given the forward's row
 * statistics (lse as gqe_attn_prefill_heads_lse wrote them, every row), so
 * the pass that recomputes them from q K^T is skipped.  Same definitions and
 * outputs; the results differ from gqe_attn_backward's only by the rounding
 * of lse (forward's reference + log2 of its row sum, against the backward's
 * recomputation).  lse is read, not written.  Workspace: as gqe_attn_backward.
 */
int gqe_attn_backward_lse(const gqe_desc* desc, const void* q_routed, const void* q_shared, const void* k,
                          const void* v, const float* out, const float* d_hard, const float* dout,
                          const float* lse, float* dq_routed, float* dq_shared, float* dk, float* dv,
                          void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace gqe_route_backward needs when it computes dw_router. */
size_t gqe_route_backward_workspace_bytes(const gqe_desc* desc);

/*
 * gqe_route_backward -- gradients through slot assembly and routing: what
 * the weighted slot carries back to the router, its differentiable learning
 * path (GQE study note §3-2 (4)), and the hard slots' share of dout.  With the
 * kept sets held fixed, p~ is the softmax of the kept scores alone, so
 *   d_hard[t, h]  = dout[t, h] + p~[t, h] dout[t, w(h)]   (w(h): the weighted
 *                   slot that sums hard slot h; none in route mode 2)
 *   dp~[t, h]     = <dout[t, w(h)], out[t, h]>
 *   d_logits[t, g*E + S_j] = p~_j (dp~_j - sum_i p~_i dp~_i), 0 for experts not kept
 *   dw_router     = sum_t d_logits[t]^T x[t],   db_router = sum_t d_logits[t]
 *   dx            = d_logits W_router  (the router's part of dx only)
 * In:  dout [B*T, S, d_head] fp32 (gradient of every slot; the shared slot's
 *      is not used here), out [B*T, S, d_head] fp32 (its hard slots are read),
 *      sel, p_tilde [B*T, G, k] as gqe_route gives them, x [B*T, d_model] and
 *      w_router [N, d_model] (dtype).
 * Out: d_hard [B*T, G*k, d_head] fp32, d_logits [B*T, N] fp32; optional (NULL
 *      skips): dw_router [N, d_model] fp32, db_router [N] fp32 (only with
 *      dw_router), dx [B*T, d_model] fp32.
 * Sums run in fixed order (dw_router: partial sums over blocks of 256 tokens,
 * then the blocks in order), so results do not depend on timing.
 * Workspace: gqe_route_backward_workspace_bytes(desc) bytes when dw_router is
 * given (else may be NULL); no initialisation needed.
 * Route mode 3 returns GQE_ERR_UNSUPPORTED (its weights are the group softmax,
 * whose gradient reaches experts that were not kept; not built).
 */
int gqe_route_backward(const gqe_desc* desc, const float* dout, const float* out, const int32_t* sel,
                       const float* p_tilde, const void* x, const void* w_router, float* d_hard,
                       float* d_logits, float* dw_router, float* db_router, float* dx, void* workspace,
                       size_t workspace_bytes, void* stream);

/*
 * gqe_kv_proj -- the K and V projections ahead of the path (GQA tutorial,
 * freeguideonline, "GQA 核心原理与计算流程" step 2: the input is projected
 * linearly to K and V, split into H_kv heads as wide as a query head):
 *   k[b, h, t, :] = W_k[h] x[b*T + t],   v[b, h, t, :] = W_v[h] x[b*T + t]
 * In:  x [B*T, d_model], w_k, w_v [H_kv, d_head, d_model] (dtype).
 * Out: k, v [B, H_kv, T, d_head] (dtype; bf16 results are fp32 sums rounded
 *      to nearest even), the layout gqe_attn_prefill reads.
 * Only B, T, d_model, H_kv, d_head and dtype of desc are used (plus its
 * validity checks).
 */
int gqe_kv_proj(const gqe_desc* desc, const void* x, const void* w_k, const void* w_v, void* k, void* v,
                void* stream);

/*
 * gqe_qkv_proj -- the whole Q/K/V preamble of the layer from one read of x
 * (GQA tutorial, freeguideonline, "GQA 核心原理与计算流程" step 2: x is
 * projected to Q, K and V; GQE study note §3-2 (2) and (5): only the kept
 * experts and the shared head are projected for Q), in one launch: the kept
 * experts over their compacted rows exactly as gqe_qproj, the shared head, and
 * the H_kv K and V heads exactly as gqe_kv_proj, with the k*G + 1 + 2*H_kv
 * projections of each x row served from one XCD's L2.
 * Optional rotary position embedding (the pages give none; the RoFormer
 * form, rotate-half pairing): with rope_base > 1, every routed and shared query
 * row and every K row at position p has each pair (c, c + d_head/2),
 * c < d_head/2, rotated by the angle p * rope_base^(-2c/d_head):
 *   (u, w) -> (u cos - w sin, w cos + u sin),
 * in fp32 on the fp32 sums before the one rounding to bf16 (V is not
 * rotated).  Positions: positions[b*T + t] (int32, device, >= 0) or, with
 * positions NULL, t.  A decode step passes T = 1 and positions = lens - 1.
 * rope_base = 0 applies no rotation (then the outputs equal gqe_qproj's and
 * gqe_kv_proj's bit for bit).
 * In:  x [BT, d_model]; w_q [N + n_shared, d_head, d_model]; w_k, w_v [H_kv,
 *      d_head, d_model] (dtype); sel, counts, offsets, rows from gqe_route.
 * Out: q_routed [B, G, T, k, d_head], q_shared [B, T, d_head] (n_shared = 1),
 *      k, v [B, H_kv, T, d_head] (dtype).
 * Errors: rope_base not 0 and not above 1 (or not finite) is GQE_ERR_INVALID.
 */
int gqe_qkv_proj(const gqe_desc* desc, const void* x, const void* w_q, const void* w_k, const void* w_v,
                 const int32_t* sel, const int32_t* counts, const int32_t* offsets, const int32_t* rows,
                 const int32_t* positions, float rope_base, void* q_routed, void* q_shared, void* k, void* v,
                 void* stream);

/*
 * gqe_qkv_proj_backward -- gradients of the Q/K/V preamble's weights and of x,
 * given the gradients of its outputs (from gqe_attn_backward): the backward
 * of gqe_qkv_proj with the same routing, positions and rope_base.  With the
 * kept sets fixed (each kept expert its own projection of x_t, GQE study note
 * §3-2 (2); unselected experts get no gradient) and R_t the rotary embedding
 * of the forward (identity when rope_base = 0):
 *   dw_q[n] = sum over tokens t that kept n of (R_t^T dq_{t,n})^T x_t,
 *   dw_q[N] = sum over t of (R_t^T dq_sh_t)^T x_t,
 *   dw_k[h] = sum_t (R_t^T dk_{t,h})^T x_t,   dw_v[h] = sum_t dv_{t,h}^T x_t,
 *   dx_t = sum_{kept n} W_q[n]^T R_t^T dq_{t,n} + W_q[N]^T R_t^T dq_sh_t
 *          + sum_h (W_k[h]^T R_t^T dk_{t,h} + W_v[h]^T dv_{t,h}).
 * (The router's share of dx comes from gqe_route_backward; add the two.)
 * bf16 only (GQE_ERR_UNSUPPORTED for fp32): the fp32 gradients are rotated
 * back in fp32 and rounded to bf16 for the MFMA products, which accumulate in
 * fp32; deterministic (fixed order, no atomics).
 * In:  x [BT, d_model], w_q [N + n_shared, d_head, d_model], w_k, w_v [H_kv,
 *      d_head, d_model] (bf16); sel, counts, offsets, rows from gqe_route;
 *      positions and rope_base as given to gqe_qkv_proj;
 *      dq_routed [B, G, T*k, d_head] and dq_shared [B, T, d_head] fp32 (as
 *      gqe_attn_backward gives them; dq_shared only with n_shared = 1);
 *      dk, dv [B, H_kv, T, d_head] fp32, both or neither (NULL: the K/V
 *      projections are left out, of dx too).
 * Out (each may be NULL to skip it): dw_q [N + n_shared, d_head, d_model],
 *      dw_k, dw_v [H_kv, d_head, d_model] (need dk, dv), dx [BT, d_model],
 *      all fp32, every element written.
 * Workspace: NULL, or gqe_qkv_proj_backward_workspace_bytes(desc, dk != NULL)
 *      bytes (a smaller size returns GQE_ERR_WORKSPACE): with it the weight
 *      gradient splits each head's rows into chunks, summed in chunk order
 *      (the same definition; only the grouping of the fp32 sums differs), so
 *      that the launch fills the chip.  No initialisation needed.
 */
size_t gqe_qkv_proj_backward_workspace_bytes(const gqe_desc* desc, int32_t with_kv);
int gqe_qkv_proj_backward(const gqe_desc* desc, const void* x, const void* w_q, const void* w_k, const void* w_v,
                          const int32_t* sel, const int32_t* counts, const int32_t* offsets, const int32_t* rows,
                          const int32_t* positions, float rope_base, const float* dq_routed, const float* dq_shared,
                          const float* dk, const float* dv, float* dw_q, float* dw_k, float* dw_v, float* dx,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * gqe_out_proj -- the attention output projection, fused with slot assembly.
 * The S slots of a token are concatenated in slot order into h_t (width
 * S*d_head) and passed through one linear map, y_t = W_o h_t, no bias (GQA
 * tutorial, freeguideonline, "GQA 核心原理与计算流程" step 5: concatenate the
 * head outputs, then one final linear projection; GQE study note §3-2 (5) and
 * (7): in GQE the concatenation is of the kG+2 slots).  The weighted slot(s)
 * are not read: they are formed from the hard slots inside the call exactly
 * as gqe_assemble forms them.  Route modes 2 and 3 have no weighted slot: the
 * slots are projected as given (mode 3: pass the scaled hard slots that
 * gqe_attn_prefill or gqe_attn_decode write).
 * In:  out [B*T, S, d_head] fp32 with the hard and shared slots written (as
 *      gqe_attn_prefill_heads or gqe_attn_decode leave them);
 *      p_tilde [B*T, G, k] fp32; w_o [d_model, S*d_head] (dtype), row-major.
 * Out: y [B*T, d_model] fp32.  With write_weighted = 1 the weighted slot(s)
 *      of `out` are written too, bit for bit what gqe_assemble writes; with 0
 *      `out` is only read.
 * bf16: each slot value is rounded to bf16 (nearest even) before the product,
 * which accumulates in fp32; fp32: fp32 throughout.  Works for decode outputs
 * too (T = 1).  d_model * S * d_head must stay below 2^31.
 */
int gqe_out_proj(const gqe_desc* desc, float* out, const float* p_tilde, const void* w_o, float* y,
                 int32_t write_weighted, void* stream);

/*
 * Packed output-projection weights (bf16 only).  The same projection as
 * gqe_out_proj (GQA tutorial step 5; GQE study note §3-2 (5), (7)) with W_o
 * first rearranged once into the order the kernel's matrix-core fragments are
 * read in, so that every weight load is a run of consecutive bytes:
 *   packed[((ct*(K/16) + ks)*2 + cb)*512 + (32*h + c)*8 + e]
 *     = W_o[64*ct + 32*cb + c][16*ks + 8*h + e],   K = S*d_head,
 *   c < 32, h < 2, e < 8.
 * gqe_out_proj_packed_bytes: bytes of the packed weights (d_model*K*2), or 0
 *   when this shape has no packed form (fp32, or K too large for the
 *   kernel's 64-token tile of bf16 slots to fit in LDS: 64*(K+8)*2 bytes
 *   above 160 KiB) -- use gqe_out_proj there.
 * gqe_out_proj_pack: w_o [d_model, K] bf16 -> w_packed (caller-owned, that
 *   many bytes); GQE_ERR_UNSUPPORTED where the size is 0.
 * gqe_out_proj_packed: y and the optional weighted-slot write-back exactly as
 *   gqe_out_proj defines them (the same bf16 rounding of every slot value;
 *   fp32 sums in a different order), from the packed weights.
 */
size_t gqe_out_proj_packed_bytes(const gqe_desc* desc);
int gqe_out_proj_pack(const gqe_desc* desc, const void* w_o, void* w_packed, void* stream);
int gqe_out_proj_packed(const gqe_desc* desc, float* out, const float* p_tilde, const void* w_packed, float* y,
                        int32_t write_weighted, void* stream);

/*
 * gqe_attn_decode_paged -- gqe_attn_decode over a paged KV cache, the layout
 * of paged attention (GQA tutorial, freeguideonline, "推理优化：连续批处理与
 * 分页注意力": GQA pairs with continuous batching and paged attention, the
 * cache being stored per KV group).  Same definition and outputs as
 * gqe_attn_decode; only where the keys and values live differs.
 * In:  k_pages, v_pages [num_pages, H_kv, page_size, d_head] (dtype): each page
 *      holds page_size consecutive positions of every KV head;
 *      block_table [B, max_pages] int32: position p of sequence b is row
 *      p % page_size of page block_table[b, p / page_size];
 *      lens [B] int32 with 1 <= lens[b] <= max_pages * page_size (out-of-range
 *      lengths behave as for gqe_attn_decode);
 *      q_routed, q_shared, p_tilde as for gqe_attn_decode.
 * page_size is a power of two from 8 to 4096.  Page ids outside
 * 0 .. num_pages-1 are clamped into that range (a bad table gives wrong
 * results, never an access outside the pages).
 * Out: out [B, S, d_head] fp32.
 * Workspace: gqe_decode_workspace_bytes(desc, max_pages * page_size) bytes.
 */
int gqe_attn_decode_paged(const gqe_desc* desc, const void* q_routed, const void* q_shared,
                          const void* k_pages, const void* v_pages, int32_t num_pages, int32_t page_size,
                          int32_t max_pages, const int32_t* block_table, const int32_t* lens,
                          const float* p_tilde, float* out, void* workspace, size_t workspace_bytes,
                          void* stream);

/*
 * gqe_check_decode_inputs -- audit of the decode preconditions the host cannot
 * see, for callers that want them checked (the decode calls clamp such values
 * instead of faulting, so a violation gives wrong results, not an error).
 * Counts, on the device, the sequences with lens[b] outside 1 .. L_max into
 * bad[0] and, when block_table is given, the block-table entries a sequence
 * uses (its first ceil(lens[b] / page_size) columns) whose page id is outside
 * 0 .. num_pages-1 into bad[1].  bad [2] int32 (device) is written, not added
 * to; synchronise the stream before reading it.  For a paged cache pass
 * L_max = max_pages * page_size; block_table NULL audits lens only.
 */
int gqe_check_decode_inputs(const gqe_desc* desc, const int32_t* lens, int32_t L_max,
                            const int32_t* block_table, int32_t num_pages, int32_t page_size,
                            int32_t max_pages, int32_t* bad, void* stream);

/*
 * gqe_decode_route_qproj -- the decode step's routing and query projection in
 * one launch, for one new token per sequence (desc->T == 1): what gqe_route
 * and gqe_qproj compute for it (GQE study note §3-2 (2), (4), (5): scores,
 * in-group softmax, the top k with lower-index ties, the weights renormalised
 * over the kept ones -- route mode 3: not renormalised --, then only the kept
 * experts' and the shared head's query rows), without the compaction, which
 * decode does not need.  bf16 scores are exact products added in double in a
 * fixed tree order (gqe_route instead adds fp32 partial sums of up to 32
 * products, so the two can differ by that rounding and split a near-tie
 * differently; each agrees with the exact score to well under 1e-6);
 * fp32 scores take gqe_route's fp64 FMA chain, bit for bit.  Each query
 * row is an fp32 sum rounded once (bf16).
 * Optional rotary embedding of the query rows (as gqe_qkv_proj) at
 * positions[b] (required when rope_base > 1; a decode step passes lens - 1).
 * In:  x [B, d_model], w_router [N, d_model], b_router [N] or NULL,
 *      w_q [N + n_shared, d_head, d_model] (dtype).
 * Out: sel [B, G, k] int32, p_tilde [B, G, k] fp32, q_routed [B, G, 1, k,
 *      d_head], q_shared [B, 1, d_head] (n_shared = 1), logits [B, N] fp64
 *      or NULL.
 */
int gqe_decode_route_qproj(const gqe_desc* desc, const void* x, const void* w_router, const float* b_router,
                           const void* w_q, const int32_t* positions, float rope_base, int32_t* sel, float* p_tilde,
                           void* q_routed, void* q_shared, double* logits, void* stream);

/* Bytes of device workspace gqe_attn_decode needs for a cache of L_max positions. */
size_t gqe_decode_workspace_bytes(const gqe_desc* desc, int32_t L_max);

/*
 * gqe_attn_decode -- one new token per sequence (desc->T == 1) against a KV
 * cache that already holds that token's K and V (decode reads the whole
 * cache: GQA tutorial, freeguideonline, "自回归推理中的内存带宽优势").
 *
 * In:  q_routed [B, G, 1, k, d_head], q_shared [B, 1, d_head] or NULL,
 *      k_cache, v_cache [B, H_kv, L_max, d_head] (dtype), lens [B] int32 with
 *      1 <= lens[b] <= L_max (positions >= lens[b] are never read; a length
 *      above L_max is read as L_max and one below 1 makes that sequence's
 *      slots NaN, with no access outside the cache or the workspace),
 *      p_tilde [B, G, k] fp32.
 * Out: out [B, S, d_head] fp32, slots as in gqe_attn_prefill.
 * Workspace: gqe_decode_workspace_bytes(desc, L_max) bytes of device memory
 *      for split-KV partial results; no initialisation needed.
 * The partial results of fixed-size key chunks are merged in chunk order, so
 * the result does not depend on scheduling.
 */
int gqe_attn_decode(const gqe_desc* desc, const void* q_routed, const void* q_shared,
                    const void* k_cache, const void* v_cache, int32_t L_max, const int32_t* lens,
                    const float* p_tilde, float* out, void* workspace, size_t workspace_bytes,
                    void* stream);

/* Bytes of the static device scratch gqe_attn_decode_noalloc uses (16 MiB). */
#define GQE_DECODE_SCRATCH_BYTES ((size_t)16 << 20)

/*
 * gqe_attn_decode_noalloc -- gqe_attn_decode for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same kernels and results, bit for bit,
 * with the split-KV partials kept in a static device array of the library
 * (GQE_DECODE_SCRATCH_BYTES, one copy per GPU, held until the process ends)
 * instead of a caller's workspace.  Nothing is allocated or freed; the
 * array's device address is looked up on the first call on each device.
 * In/Out: as gqe_attn_decode, without the workspace arguments.
 * Returns GQE_ERR_SCRATCH, with nothing enqueued, when
 * gqe_decode_workspace_bytes(desc, L_max) exceeds GQE_DECODE_SCRATCH_BYTES
 * (e.g. B = 64, L_max = 8192, H_kv = 8, k = 1, d_head = 64 needs 5.9 MB).
 * Every call on one GPU uses that GPU's one array: calls that overlap on a
 * GPU (two streams, two host threads) race and must be ordered by the caller.
 * The partials need no initialisation (every chunk a call reads it writes).
 */
int gqe_attn_decode_noalloc(const gqe_desc* desc, const void* q_routed, const void* q_shared,
                            const void* k_cache, const void* v_cache, int32_t L_max, const int32_t* lens,
                            const float* p_tilde, float* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GQE_H */
