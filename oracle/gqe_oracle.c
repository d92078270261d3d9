/*
 * GQE attention forward -- CPU ORACLE.  TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously correct definition of the Grouped Query Experts
 * (GQE) attention forward pass, written out step by step in double precision.
 * It exists to check the HIP library against.  Only the test suite, the smoke
 * check and the CPU-baseline leg of the benchmark may load it; the library
 * never calls it and the two share no code, headers or tables.
 *
 * Pages followed (cited by title and section):
 *   [note]  "Grouped Query Experts" study note, dimensionstp.github.io
 *   [sum]   "Grouped Query Experts: GQA自注意力上的混合专家", ai-feeds.com
 *   [tut]   "分组查询注意力 GQA：效率与质量的平衡方案", freeguideonline.com
 *   [ibm]   "什么是分组查询注意力 (GQA)？", ibm.com
 *
 * Notation ([note] §1-1, §3-2 (1)): G = H_kv groups, E = H_q / G query experts
 * per group, N = G*E routed experts with global index n = g*E + e (the GQA
 * query-head index, [tut] "GQA 核心原理与计算流程" step 3).  The shared head's
 * projection is row N of W_q.
 *
 * Every input is taken as exact double values (bf16 and fp32 both convert to
 * double without rounding).  All sums accumulate in double.  Rows are
 * independent, so OpenMP splits them across threads without changing any
 * result.
 *
 * Readings where the pages leave a step open (each is also listed with the
 * design notes):
 *   - the router is one linear map of x_t per group, plus an optional bias;
 *   - top-k ranks by logit (softmax is monotone, so this is the order of p),
 *     ties go to the lower expert index, and the kept set is stored in
 *     ascending expert index;
 *   - the shared head attends KV head 0 and takes no part in the weighted slot;
 *   - attention scale 1/sqrt(d_head); causal means key position s <= t;
 *   - slot order: hard slots group-major then ascending expert index, then the
 *     weighted slot(s), then the shared slot.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORA_TIE_MARGIN 1e-6
#define ORA_MAX_E 256

typedef struct {
    int32_t B, T, d_model, H_q, H_kv, k, d_head, n_shared, causal, route_mode;
} ora_desc;

/* Weighted slots: route_mode 0 one summed over groups ([note] §3-2 (4)), 1 one
 * per group, 2 none (the "hard concat only" row of the [note] §5-1 ablation
 * table), 3 none (the "weighted concat, no renormalized slot" row, read as:
 * each hard slot scaled by its kept expert's group softmax probability, not
 * renormalised over the kept ones, and no weighted-sum slot). */
static int ora_nroute(const ora_desc* D)
{
    return D->route_mode == 0 ? 1 : D->route_mode == 1 ? D->H_kv : 0;
}

static int ora_nslots(const ora_desc* D)
{
    int G = D->H_kv;
    return D->k * G + ora_nroute(D) + D->n_shared;
}

int ora_num_slots(const ora_desc* D) { return ora_nslots(D); }

/* Threads an OpenMP parallel region of the oracle uses. */
int ora_num_threads(void) { return omp_get_max_threads(); }

static double dot(const double* a, const double* b, int64_t n)
{
    double s = 0.0;
    for (int64_t i = 0; i < n; ++i) s += a[i] * b[i];
    return s;
}

/*
 * Steps 1-4 for n_tok token rows of x [n_tok, d_model].
 *   logits[t, n]   s_{t,g,e} = r_g(x_t)_e, the router score       ([note] §3-2 (2))
 *   probs[t, n]    p_{t,g,e}: softmax over the E experts of group g ([note] §3-2 (2))
 *   sel[t, g, j]   S_{t,g} = TopK(p_{t,g,1:E}, k), ascending index  ([note] §3-2 (2))
 *   ptilde[t,g,j]  p renormalised over the kept experts              ([note] §3-2 (4));
 *                  in route mode 3 p itself (the group softmax of the kept expert)
 *   tie[t, g]      1 when the k-th and (k+1)-th largest logits are closer than
 *                  1e-6, so either choice is a correct selection.
 * Any output pointer except sel may be NULL.
 */
int ora_route(const ora_desc* D, int64_t n_tok, const double* x, const double* w_router,
              const double* b_router, double* logits, double* probs, int32_t* sel,
              double* ptilde, uint8_t* tie)
{
    const int G = D->H_kv, E = D->H_q / D->H_kv, k = D->k, dm = D->d_model, N = D->H_q;
    if (E > ORA_MAX_E || k < 1 || k > E) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < n_tok; ++t) {
        const double* xt = x + t * dm;
        for (int g = 0; g < G; ++g) {
            double s[ORA_MAX_E], p[ORA_MAX_E];
            int chosen[ORA_MAX_E];
            for (int e = 0; e < E; ++e) {
                int n = g * E + e;
                s[e] = dot(xt, w_router + (int64_t)n * dm, dm) + (b_router ? b_router[n] : 0.0);
                chosen[e] = 0;
            }
            /* softmax within the group, exact two-pass form */
            double m = s[0];
            for (int e = 1; e < E; ++e) if (s[e] > m) m = s[e];
            double z = 0.0;
            for (int e = 0; e < E; ++e) { p[e] = exp(s[e] - m); z += p[e]; }
            for (int e = 0; e < E; ++e) p[e] /= z;
            /* top-k: k rounds of "largest not yet chosen"; a strict > keeps
             * the lowest index among equal logits */
            int last = -1;
            for (int r = 0; r < k; ++r) {
                int best = -1;
                for (int e = 0; e < E; ++e)
                    if (!chosen[e] && (best < 0 || s[e] > s[best])) best = e;
                chosen[best] = 1;
                last = best;
            }
            if (tie) {
                uint8_t flag = 0;
                if (k < E) {
                    double next = -INFINITY;
                    for (int e = 0; e < E; ++e) if (!chosen[e] && s[e] > next) next = s[e];
                    flag = (s[last] - next) < ORA_TIE_MARGIN;
                }
                tie[t * G + g] = flag;
            }
            int j = 0;
            double den = 0.0;
            for (int e = 0; e < E; ++e)
                if (chosen[e]) { sel[(t * G + g) * k + j] = e; den += p[e]; ++j; }
            if (ptilde)
                for (j = 0; j < k; ++j)
                    ptilde[(t * G + g) * k + j] = p[sel[(t * G + g) * k + j]] / (D->route_mode == 3 ? 1.0 : den);
            if (logits) for (int e = 0; e < E; ++e) logits[t * N + g * E + e] = s[e];
            if (probs) for (int e = 0; e < E; ++e) probs[t * N + g * E + e] = p[e];
        }
    }
    return 0;
}

/*
 * Step 5: bucket the (token, group, kept expert) triples by global expert n.
 *   counts[n]     number of tokens that kept expert n
 *   offsets[n]    exclusive prefix sum of counts, offsets[N] = n_tok*G*k
 *   rows[offsets[n] + r]  the r-th smallest token id that kept n
 * Unselected experts never appear, which is what lets the projection and
 * attention skip them ([sum] 方法/核心模块; [note] §3-2 (2)).
 */
void ora_compact(const ora_desc* D, int64_t n_tok, const int32_t* sel, int32_t* counts,
                 int32_t* offsets, int32_t* rows)
{
    const int G = D->H_kv, E = D->H_q / D->H_kv, k = D->k, N = D->H_q;
    for (int n = 0; n < N; ++n) counts[n] = 0;
    for (int64_t t = 0; t < n_tok; ++t)
        for (int g = 0; g < G; ++g)
            for (int j = 0; j < k; ++j) counts[g * E + sel[(t * G + g) * k + j]]++;
    offsets[0] = 0;
    for (int n = 0; n < N; ++n) offsets[n + 1] = offsets[n] + counts[n];
    int32_t* cursor = (int32_t*)malloc(sizeof(int32_t) * (size_t)N);
    for (int n = 0; n < N; ++n) cursor[n] = offsets[n];
    for (int64_t t = 0; t < n_tok; ++t)
        for (int g = 0; g < G; ++g)
            for (int j = 0; j < k; ++j) rows[cursor[g * E + sel[(t * G + g) * k + j]]++] = (int32_t)t;
    free(cursor);
}

/* q = W_q[n] x_t, one d_head vector: each kept expert is its own query
 * projection ([sum] 方法/核心模块; [note] §3-2 (2), last sentence). */
static void project(const ora_desc* D, const double* xt, const double* w_q, int n, double* q)
{
    const int dm = D->d_model, dh = D->d_head;
    for (int d = 0; d < dh; ++d) q[d] = dot(xt, w_q + ((int64_t)n * dh + d) * dm, dm);
}

/*
 * Step 6 for a list of tokens.  q_routed[i, g, j, :] is the projection of
 * token tok[i] by its j-th kept expert of group g; q_shared[i, :] (if the
 * shared head exists and the pointer is not NULL) uses W_q[N].
 */
void ora_qproj_rows(const ora_desc* D, int64_t n_list, const int64_t* tok, const double* x,
                    const double* w_q, const int32_t* sel, double* q_routed, double* q_shared)
{
    const int G = D->H_kv, E = D->H_q / D->H_kv, k = D->k, dh = D->d_head, N = D->H_q;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n_list; ++i) {
        const int64_t t = tok[i];
        const double* xt = x + t * D->d_model;
        for (int g = 0; g < G; ++g)
            for (int j = 0; j < k; ++j)
                project(D, xt, w_q, g * E + sel[(t * G + g) * k + j], q_routed + ((i * G + g) * k + j) * dh);
        if (D->n_shared && q_shared) project(D, xt, w_q, N, q_shared + i * dh);
    }
}

/*
 * The K and V projections ahead of the path ([tut] "GQA 核心原理与计算流程",
 * step 2: the input is projected linearly to K and V, split into g = H_kv
 * heads each as wide as a query head).  x [B*T, d_model]; w [H_kv, d_head,
 * d_model]; out[b, h, t, :] = w[h] x[b*T + t], out [B, H_kv, T, d_head].
 * Called once with W_k and once with W_v.
 */
void ora_kv_proj(const ora_desc* D, const double* x, const double* w, double* out)
{
    const int G = D->H_kv, dh = D->d_head, T = D->T;
    const int64_t BT = (int64_t)D->B * T;
#pragma omp parallel for schedule(static)
    for (int64_t tk = 0; tk < BT; ++tk) {
        const int64_t b = tk / T, t = tk % T;
        for (int h = 0; h < G; ++h) project(D, x + tk * D->d_model, w, h, out + ((b * G + h) * T + t) * dh);
    }
}

/*
 * Step 7, one query row: scaled dot-product attention over n_keys keys
 * ([note] §1-1, Attention(Q,K,V) = softmax(QK^T / sqrt(d)) V; scale
 * 1/sqrt(d_k) as in [ibm]).  Kh, Vh point at key 0 of one KV head, rows
 * d_head apart.  Exact two-pass softmax; w is caller scratch of n_keys.
 */
static void attend(const double* q, const double* Kh, const double* Vh, int64_t n_keys, int dh,
                   double* o, double* w)
{
    const double scale = 1.0 / sqrt((double)dh);
    double m = -INFINITY;
    for (int64_t s = 0; s < n_keys; ++s) {
        w[s] = dot(q, Kh + s * dh, dh) * scale;
        if (w[s] > m) m = w[s];
    }
    double z = 0.0;
    for (int64_t s = 0; s < n_keys; ++s) { w[s] = exp(w[s] - m); z += w[s]; }
    for (int d = 0; d < dh; ++d) o[d] = 0.0;
    for (int64_t s = 0; s < n_keys; ++s)
        for (int d = 0; d < dh; ++d) o[d] += w[s] * Vh[s * dh + d];
    for (int d = 0; d < dh; ++d) o[d] /= z;
}

/*
 * Step 8, output construction for one token ([note] §3-2 (3)-(5) and the
 * final concat; slot count kG+2 in the §3-1 table):
 *   out[g*k + j]        hard slot: o_{t,g,e} of the j-th kept expert (not averaged)
 *   mode 0: out[kG]     h_route = sum_g sum_j ptilde * o, summed g then j
 *   mode 1: out[kG + g] per-group weighted sum sum_j ptilde * o
 *   mode 2: no weighted slot
 *   mode 3: no weighted slot; hard slot g*k+j is ptilde[g*k+j] * o (ptilde
 *           then holds the group softmax p of the kept expert)
 *   out[last]           the shared head (when present)
 * o_r [G*k, dh] holds the kept-expert outputs in hard-slot order.
 */
static void assemble(const ora_desc* D, const double* o_r, const double* o_sh, const double* pt,
                     double* out)
{
    const int G = D->H_kv, k = D->k, dh = D->d_head;
    const int nroute = ora_nroute(D);
    memcpy(out, o_r, sizeof(double) * (size_t)G * k * dh);
    if (D->route_mode == 3)
        for (int h = 0; h < G * k; ++h)
            for (int d = 0; d < dh; ++d) out[h * dh + d] = pt[h] * o_r[h * dh + d];
    double* route = out + (int64_t)G * k * dh;
    for (int i = 0; i < nroute * dh; ++i) route[i] = 0.0;
    for (int g = 0; g < G && nroute; ++g)
        for (int j = 0; j < k; ++j) {
            double* dst = route + (D->route_mode ? g : 0) * dh;
            for (int d = 0; d < dh; ++d) dst[d] += pt[g * k + j] * o_r[(g * k + j) * dh + d];
        }
    if (D->n_shared) memcpy(out + ((int64_t)G * k + nroute) * dh, o_sh, sizeof(double) * dh);
}

/*
 * Steps 6-8 of the prefill forward for a list of tokens (flat ids b*T + t).
 * x [B*T, d_model]; w_q [N + n_shared, d_head, d_model]; K, V [B, H_kv, T, d_head];
 * sel / ptilde from ora_route over all B*T tokens.  out [n_list, S, d_head].
 * Kept experts of group g attend that group's KV head g (unchanged and dense,
 * [note] §1-2 (3)); the shared head attends KV head 0.
 */
void ora_prefill_rows(const ora_desc* D, const double* x, const double* w_q, const double* K,
                      const double* V, const int32_t* sel, const double* ptilde, int64_t n_list,
                      const int64_t* tok, double* out)
{
    const int G = D->H_kv, E = D->H_q / D->H_kv, k = D->k, dh = D->d_head, T = D->T;
    const int S = ora_nslots(D);
#pragma omp parallel
    {
        double* q = (double*)malloc(sizeof(double) * dh);
        double* o_r = (double*)malloc(sizeof(double) * (size_t)G * k * dh);
        double* o_sh = (double*)malloc(sizeof(double) * dh);
        double* w = (double*)malloc(sizeof(double) * (size_t)T);
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < n_list; ++i) {
            const int64_t tk = tok[i];
            const int64_t b = tk / T, t = tk % T;
            const int64_t n_keys = D->causal ? t + 1 : T;
            const double* xt = x + tk * D->d_model;
            for (int g = 0; g < G; ++g) {
                const double* Kh = K + (b * G + g) * (int64_t)T * dh;
                const double* Vh = V + (b * G + g) * (int64_t)T * dh;
                for (int j = 0; j < k; ++j) {
                    project(D, xt, w_q, g * E + sel[(tk * G + g) * k + j], q);
                    attend(q, Kh, Vh, n_keys, dh, o_r + (g * k + j) * dh, w);
                }
            }
            if (D->n_shared) {
                project(D, xt, w_q, D->H_q, q);
                attend(q, K + b * G * (int64_t)T * dh, V + b * G * (int64_t)T * dh, n_keys, dh, o_sh, w);
            }
            assemble(D, o_r, o_sh, ptilde + tk * G * k, out + i * (int64_t)S * dh);
        }
        free(q); free(o_r); free(o_sh); free(w);
    }
}

/*
 * Steps 7-8 for a list of tokens given their query rows (as ora_qproj_rows
 * returns them): q_routed [n_list, G, k, d_head], q_shared [n_list, d_head]
 * (or NULL without a shared head).  The same attention and slot assembly as
 * ora_prefill_rows, for callers whose queries were rounded (a bf16 projection
 * output) before attending.  out [n_list, S, d_head].
 */
void ora_attend_rows(const ora_desc* D, const double* q_routed, const double* q_shared, const double* K,
                     const double* V, const double* ptilde, int64_t n_list, const int64_t* tok, double* out)
{
    const int G = D->H_kv, k = D->k, dh = D->d_head, T = D->T;
    const int S = ora_nslots(D);
#pragma omp parallel
    {
        double* o_r = (double*)malloc(sizeof(double) * (size_t)G * k * dh);
        double* o_sh = (double*)malloc(sizeof(double) * dh);
        double* w = (double*)malloc(sizeof(double) * (size_t)T);
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < n_list; ++i) {
            const int64_t tk = tok[i];
            const int64_t b = tk / T, t = tk % T;
            const int64_t n_keys = D->causal ? t + 1 : T;
            for (int g = 0; g < G; ++g) {
                const double* Kh = K + (b * G + g) * (int64_t)T * dh;
                const double* Vh = V + (b * G + g) * (int64_t)T * dh;
                for (int j = 0; j < k; ++j)
                    attend(q_routed + ((i * G + g) * k + j) * dh, Kh, Vh, n_keys, dh, o_r + (g * k + j) * dh, w);
            }
            if (D->n_shared)
                attend(q_shared + i * dh, K + b * G * (int64_t)T * dh, V + b * G * (int64_t)T * dh, n_keys, dh,
                       o_sh, w);
            assemble(D, o_r, o_sh, ptilde + tk * G * k, out + i * (int64_t)S * dh);
        }
        free(o_r); free(o_sh); free(w);
    }
}

/*
 * Step 8 alone for n_list rows whose hard and shared slots are given: fills
 * the weighted slot(s) of slots [n_list, S, d_head] in place from the hard
 * slots, exactly as the prefill rows path does.  ptilde [n_list, G, k].
 */
void ora_assemble_rows(const ora_desc* D, const double* ptilde, int64_t n_list, double* slots)
{
    const int G = D->H_kv, k = D->k, dh = D->d_head;
    const int S = ora_nslots(D), nroute = ora_nroute(D);
#pragma omp parallel
    {
        double* tmp = (double*)malloc(sizeof(double) * (size_t)S * dh);
#pragma omp for schedule(static)
        for (int64_t i = 0; i < n_list; ++i) {
            double* row = slots + i * (int64_t)S * dh;
            const double* o_sh = D->n_shared ? row + ((int64_t)G * k + nroute) * dh : NULL;
            assemble(D, row, o_sh, ptilde + i * (int64_t)G * k, tmp);
            memcpy(row, tmp, sizeof(double) * (size_t)S * dh);
        }
        free(tmp);
    }
}

/*
 * Rotary position embedding of n rows of width dh in place (the pages give
 * none; the RoFormer form with rotate-half pairing is the reading taken):
 * pair (c, c + dh/2), c < dh/2, of a row at position pos[r] is rotated by
 * the angle pos * base^(-2c/dh):  (u, w) -> (u cos - w sin, w cos + u sin).
 */
void ora_rope(int64_t n, int dh, const int32_t* pos, double base, double* rowsv)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r) {
        double* x = rowsv + r * dh;
        for (int c = 0; c < dh / 2; ++c) {
            const double ang = (double)pos[r] * pow(base, -2.0 * c / dh);
            const double cs = cos(ang), sn = sin(ang);
            const double u = x[c], w = x[c + dh / 2];
            x[c] = u * cs - w * sn;
            x[c + dh / 2] = w * cs + u * sn;
        }
    }
}

/*
 * The attention output projection of n_list tokens: the S slots of a token,
 * concatenated in slot order into h_t of width S*d_head, times W_o
 * ([tut] "GQA 核心原理与计算流程", step 5: the head outputs are concatenated
 * and projected by one final linear map; [note] §3-2 (5) and (7): in GQE the
 * concatenation is of the kG+2 slots, so W_o is kG+2 slots wide).  No bias
 * (the pages name none).
 *   y[i, c] = sum_s sum_d slots[i, s, d] * w_o[c, s*d_head + d]
 * slots [n_list, S, d_head]; w_o [d_model, S*d_head]; y [n_list, d_model].
 */
void ora_out_proj_rows(const ora_desc* D, const double* slots, const double* w_o, int64_t n_list, double* y)
{
    const int64_t width = (int64_t)ora_nslots(D) * D->d_head;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n_list; ++i)
        for (int c = 0; c < D->d_model; ++c) y[i * D->d_model + c] = dot(slots + i * width, w_o + c * width, width);
}

/*
 * Decode: one new token per sequence against a KV cache that already holds
 * it.  x [B, d_model]; k_cache, v_cache [B, H_kv, L_max, d_head]; lens[b] in
 * 1..L_max counts the valid positions of sequence b.  Routing runs on the one
 * token (steps 1-4) and the kept experts attend all lens[b] cached positions
 * (decode reads the whole cache, [tut] "自回归推理中的内存带宽优势").
 * out [B, S, d_head]; sel [B, G, k], ptilde [B, G, k] and tie [B, G] are
 * filled as by ora_route (tie and ptilde may be NULL).
 */
/* Decode steps 6-8 for a given selection and p~ (the caller's routing): each
 * sequence's one new token at position lens[b]-1 attends its cache prefix. */
int ora_decode_given(const ora_desc* D, const double* x, const double* w_q, const double* k_cache,
                     const double* v_cache, int32_t L_max, const int32_t* lens, const int32_t* sel,
                     const double* pt, double* out)
{
    const int G = D->H_kv, E = D->H_q / D->H_kv, k = D->k, dh = D->d_head, B = D->B;
    const int S = ora_nslots(D);
    for (int b = 0; b < B; ++b) if (lens[b] < 1 || lens[b] > L_max) return -1;
#pragma omp parallel
    {
        double* q = (double*)malloc(sizeof(double) * dh);
        double* o_r = (double*)malloc(sizeof(double) * (size_t)G * k * dh);
        double* o_sh = (double*)malloc(sizeof(double) * dh);
        double* w = (double*)malloc(sizeof(double) * (size_t)L_max);
#pragma omp for schedule(dynamic, 1)
        for (int b = 0; b < B; ++b) {
            const double* xt = x + (int64_t)b * D->d_model;
            for (int g = 0; g < G; ++g) {
                const double* Kh = k_cache + ((int64_t)b * G + g) * L_max * dh;
                const double* Vh = v_cache + ((int64_t)b * G + g) * L_max * dh;
                for (int j = 0; j < k; ++j) {
                    project(D, xt, w_q, g * E + sel[((int64_t)b * G + g) * k + j], q);
                    attend(q, Kh, Vh, lens[b], dh, o_r + (g * k + j) * dh, w);
                }
            }
            if (D->n_shared) {
                project(D, xt, w_q, D->H_q, q);
                attend(q, k_cache + (int64_t)b * G * L_max * dh, v_cache + (int64_t)b * G * L_max * dh,
                       lens[b], dh, o_sh, w);
            }
            assemble(D, o_r, o_sh, pt + (int64_t)b * G * k, out + (int64_t)b * S * dh);
        }
        free(q); free(o_r); free(o_sh); free(w);
    }
    return 0;
}

int ora_decode(const ora_desc* D, const double* x, const double* w_router, const double* b_router,
               const double* w_q, const double* k_cache, const double* v_cache, int32_t L_max,
               const int32_t* lens, double* out, int32_t* sel, double* ptilde, uint8_t* tie)
{
    const int G = D->H_kv, k = D->k, B = D->B;
    double* pt = ptilde ? ptilde : (double*)malloc(sizeof(double) * (size_t)B * G * k);
    int rc = ora_route(D, B, x, w_router, b_router, NULL, NULL, sel, pt, tie);
    if (rc == 0) rc = ora_decode_given(D, x, w_q, k_cache, v_cache, L_max, lens, sel, pt, out);
    if (!ptilde) free(pt);
    return rc;
}
