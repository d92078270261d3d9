// Host-side launch interface between the C ABI layer (gqe_api.cpp) and the
// kernel files.  Arguments have been validated before any of these run.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gqe {

struct RouteArgs {
    const void* x;
    const void* w_router;
    const float* b_router;
    int32_t* sel;
    float* p_tilde;
    int32_t* counts;
    int32_t* offsets;
    int32_t* rows;
    double* logits;
    void* workspace;
    int BT, d_model, G, E, k;
    bool bf16;
    bool renorm = true;   // false (route mode 3): p_tilde holds the group softmax of the kept experts
};
size_t route_workspace_bytes(int BT, int N);
int launch_route(const RouteArgs& a, hipStream_t st);

struct QprojArgs {
    const void* x;
    const void* w_q;
    const int32_t* sel;
    const int32_t* counts;
    const int32_t* offsets;
    const int32_t* rows;
    void* q_routed;   // NULL: the routed experts are not projected by this call
    void* q_shared;   // NULL: the shared head is not projected by this call
    int B, T, d_model, G, E, k, d_head, n_shared;
    bool bf16;
};
int launch_qproj(const QprojArgs& a, hipStream_t st);

struct RouteBwdArgs {
    const float* dout;      // [BT, S, d_head]
    const float* out;       // [BT, S, d_head]: the hard slots are read
    const int32_t* sel;     // [BT, G, k]
    const float* p_tilde;   // [BT, G, k]
    const void* x;          // [BT, d_model]
    const void* w_router;   // [N, d_model]
    float* d_hard;          // [BT, G*k, d_head]
    float* d_logits;        // [BT, N]
    float* dw_router;       // [N, d_model] or NULL (then db_router is NULL too)
    float* db_router;       // [N] or NULL
    float* dx;              // [BT, d_model] or NULL
    void* workspace;        // route_bwd_workspace_bytes(), needed when dw_router is set
    long long BT;
    int G, E, k, d_head, d_model, S, route_mode;
    bool bf16;
};
size_t route_bwd_workspace_bytes(long long BT, int N, int C);
int launch_route_bwd(const RouteBwdArgs& a, hipStream_t st);
int launch_route_stats(const double* logits, long long BT, int G, int E, float* importance, hipStream_t st);

struct AttnBwdArgs {
    const void* q_routed;   // [B, G, T*k, d_head] bf16, row t*k + j
    const void* q_shared;   // [B, T, d_head] bf16 (n_shared = 1)
    const void* k_;         // [B, G, T, d_head] bf16
    const void* v_;         // [B, G, T, d_head] bf16
    const float* out;       // [B*T, S, d_head]: the hard and shared slots are read
    const float* d_hard;    // [B*T, G*k, d_head]
    const float* dout;      // [B*T, S, d_head]: the shared slot is read (n_shared = 1)
    float* dq_routed;       // [B, G, T*k, d_head]
    float* dq_shared;       // [B, T, d_head] (n_shared = 1)
    float* dk;              // [B, G, T, d_head]
    float* dv;              // [B, G, T, d_head]
    float* lse;             // one base-2 log-sum-exp per row (routed rows, then shared): the workspace,
                            // or the forward's own when lse_given
    float* delta;           // workspace: one <dO, O> per row
    int B, T, G, k, S, d_head, causal, n_shared;
    float qscale2, inv_sqrt_d;
    bool lse_given = false; // lse holds the forward's values: the dq kernel reads them instead of recomputing
};
size_t attn_bwd_workspace_bytes(int B, int T, int G, int k, int n_shared);
int launch_attn_bwd(const AttnBwdArgs& a, hipStream_t st);

struct KvProjArgs {
    const void* x;     // [B*T, d_model]
    const void* w_k;   // [H_kv, d_head, d_model]
    const void* w_v;
    void* k;           // [B, H_kv, T, d_head]
    void* v;
    int B, T, d_model, H_kv, d_head;
    bool bf16;
};
int launch_kv_proj(const KvProjArgs& a, hipStream_t st);

// K and V of every token as one dense GEMM (bf16): kvproj.hip.
struct KvDenseArgs {
    const uint16_t* x;          // [B*T, d_model]
    const uint16_t* w_k;        // [H, d_head, d_model]
    const uint16_t* w_v;
    void* k_out;                // [B, H, T, d_head]
    void* v_out;
    const int32_t* positions;   // [B*T] or NULL (position t)
    int B, T, d_model, H, d_head;
    double rope_log2_base;      // 0: no rotary embedding of K
};
int launch_kv_dense(const KvDenseArgs& a, hipStream_t st);

struct QkvProjArgs {
    const void* x;            // [B*T, d_model]
    const void* w_q;          // [N + n_shared, d_head, d_model]
    const void* w_k;          // [H_kv, d_head, d_model]
    const void* w_v;
    const int32_t* sel;
    const int32_t* counts;
    const int32_t* offsets;
    const int32_t* rows;
    const int32_t* positions; // [B*T] or NULL (position t)
    void* q_routed;           // [B, G, T, k, d_head]
    void* q_shared;           // [B, T, d_head] (n_shared = 1)
    void* k;                  // [B, H_kv, T, d_head]
    void* v;
    float rope_base;          // 0: no rotary embedding
    int B, T, d_model, G, E, k_, d_head, n_shared, H_kv;
    bool bf16;
};
int launch_qkv_proj(const QkvProjArgs& a, hipStream_t st);

// Backward of the Q/K/V projections.  Heads: [0, N) routed experts, ns shared,
// nkv K heads, nkv V heads (nkv = 0 when dk / dv are not given).
struct ProjBwdArgs {
    const uint16_t* x;          // [B*T, d_model] bf16
    const uint16_t* w_q;        // [N + ns, D, d_model]
    const uint16_t* w_k;        // [H_kv, D, d_model]
    const uint16_t* w_v;
    const int32_t* sel;
    const int32_t* counts;
    const int32_t* offsets;
    const int32_t* rows;
    const int32_t* positions;   // [B*T] or NULL (t)
    const float* dq_routed;     // [B, G, T*k, D]
    const float* dq_shared;     // [B, T, D]
    const float* dk;            // [B, H_kv, T, D]
    const float* dv;
    float* dw_q;                // [N + ns, D, d_model] or NULL
    float* dw_k;                // [H_kv, D, d_model] or NULL
    float* dw_v;
    float* dx;                  // [B*T, d_model] or NULL
    int B, T, d_model, G, E, k, D, ns, nkv;
    double rope_log2_base;      // > 0: the forward rotated q and K
};
// Bytes of workspace that let the weight gradient split each head's rows into
// chunks (0: one chunk is enough).
size_t proj_bwd_workspace_bytes(const ProjBwdArgs& a);
int launch_proj_bwd(const ProjBwdArgs& a, void* workspace, size_t workspace_bytes, hipStream_t st);

struct PrefillArgs {
    const void* q_routed;   // NULL: the routed heads are not computed by this call
    const void* q_shared;   // NULL: the shared head is not computed by this call
    const void* kmat;
    const void* vmat;
    const float* p_tilde;
    float* out;
    void* workspace;   // NULL: no split tiles; else prefill_workspace_bytes() bytes, counters even
    int B, T, G, k, d_head, n_shared, causal, route_mode, S;
    bool bf16;
    float* lse = nullptr;   // bf16 only: each row's base-2 log-sum-exp (routed rows, then shared rows)
};
size_t prefill_workspace_bytes(int B, int T, int G, int k, int d_head, int n_shared, int causal, bool bf16);
// The launch's work items in launch order, 5 ints each (b, h, tile, part, pair);
// returns their number and writes at most max_items of them.
long long prefill_plan(int B, int T, int G, int k, int d_head, int n_shared, int causal, bool split, int32_t* items,
                       long long max_items);
// Attention only: hard and shared slots of `out`; the weighted slots are not written.
int launch_prefill_heads(const PrefillArgs& a, hipStream_t st);
// Attention, then the weighted slots.
int launch_prefill(const PrefillArgs& a, hipStream_t st);
// Weighted slot(s) of n_tok output rows [n_tok, S, D] from their hard slots.
int launch_assemble(const float* p_tilde, float* out, long long n_tok, int G, int k, int D, int S, int route_mode,
                    hipStream_t st);

struct OutProjArgs {
    float* out;            // [BT, S, d_head] fp32: hard and shared slots read, weighted slot(s) optionally written
    const float* p_tilde;  // [BT, G, k] fp32
    const void* w_o;       // [d_model, S * d_head] (dtype)
    float* y;              // [BT, d_model] fp32
    long long BT;
    int d_model, G, k, d_head, n_shared, route_mode, S, write_weighted;
    bool bf16;
    const void* w_packed = nullptr;   // bf16: W_o in fragment order (launch_out_proj_pack); used instead of w_o
};
int launch_out_proj(const OutProjArgs& a, hipStream_t st);
// Whether the token-tile kernel takes this shape (K = S * d_head): the packed form exists only then.
bool out_proj_tile_fits(int K, int d_model);
int launch_out_proj_pack(const void* w_o, void* w_packed, int d_model, int K, hipStream_t st);

struct DecodeArgs {
    const void* q_routed;
    const void* q_shared;
    const void* k_cache;
    const void* v_cache;
    const int32_t* lens;
    const float* p_tilde;
    float* out;
    void* workspace;
    int B, G, k, d_head, n_shared, route_mode, S, L_max;
    bool bf16;
    // paged cache (block_table != NULL): k_cache / v_cache are [num_pages, G, page_size, d_head],
    // position p of sequence b is row p % page_size of page block_table[b * max_pages + p / page_size];
    // L_max = max_pages * page_size.  page_size is a power of two.
    const int32_t* block_table = nullptr;
    int page_shift = 0, max_pages = 0, num_pages = 0;
};
struct DecodePreArgs {
    const void* x;            // [B, d_model]
    const void* w_router;     // [N, d_model]
    const float* b_router;    // [N] or NULL
    const void* w_q;          // [N + n_shared, d_head, d_model]
    const int32_t* positions; // [B] rotary positions (needed when rope_log2_base > 0)
    int32_t* sel;             // [B, G, k]
    float* p_tilde;           // [B, G, k]
    void* q_routed;           // [B, G, 1, k, d_head]
    void* q_shared;           // [B, 1, d_head] or NULL (no shared head)
    double* logits;           // [B, N] or NULL
    int B, d_model, G, E, k, d_head;
    bool bf16, renorm;
    double rope_log2_base;
};
int launch_decode_preamble(const DecodePreArgs& a, hipStream_t st);

size_t decode_workspace_bytes(int B, int G, int k, int n_shared, int d_head, int L_max, bool bf16);
// Size of the static device array gqe_attn_decode_noalloc keeps its partials in.
constexpr size_t kDecodeScratchBytes = (size_t)16 << 20;
// Device address of the current device's static decode scratch (0), or -1.
int decode_scratch(void** ptr);
int launch_decode_check(const int32_t* lens, int B, int L_max, const int32_t* block_table, int page_size,
                        int max_pages, int num_pages, int32_t* bad, hipStream_t st);
int launch_decode(const DecodeArgs& a, hipStream_t st);

}  // namespace gqe
