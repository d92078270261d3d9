// Router (scores, in-group softmax, top-k, renormalisation) and the stable
// expert compaction, for gfx950.
//
// Method: GQE study note (dimensionstp.github.io) §3-2 (2) -- s_{t,g,e} =
// r_g(x_t)_e, p = softmax over the group's E experts, S = TopK(p, k) -- and
// §3-2 (4) -- p~ renormalised over the kept experts.  The compaction buckets
// the kept (token, expert) pairs by expert so the projection and attention
// touch only kept experts (ai-feeds summary, 方法/核心模块: unselected query
// heads are skipped).
//
// Kernels:
//   router_kernel   one workgroup per block of 32 tokens.  Scores come from
//                   bf16 MFMA (16x16x32, exact bf16 products) with every
//                   32-product partial sum added into a double accumulator, so
//                   the score error stays far below the 1e-6 tie margin; fp32
//                   inputs use double FMAs.  The workgroup then selects,
//                   renormalises and counts kept experts of its block in LDS.
//   scan_kernel     one workgroup per expert: exclusive scan of the per-block
//                   counts -> per-block base offsets, and the expert totals.
//   scatter_kernel  one wave per two blocks: wave ballots give each token its
//                   rank among the block's tokens that kept the expert, so
//                   rows[] is ordered by token id without atomics.
#include "gqe_device.h"
#include "gqe_launch.h"

namespace gqe {

constexpr int kRouteTok = 32;        // tokens per wave = compaction block
constexpr int kMaxExperts = 64;

// One workgroup per block of 32 tokens.  bf16: the four waves take every
// fourth 32-wide step of d_model, issue the loads of 8 steps before their
// MFMAs (the kernel is bound by load latency, not math), and add each
// 32-product partial into a double accumulator; the four partial sums are
// then added in a fixed order.  fp32: one double FMA chain per score.
template <bool BF16, int NB>
__global__ __launch_bounds__(256) void router_kernel(
    const void* __restrict__ xv, const void* __restrict__ wv, const float* __restrict__ bias,
    int32_t* __restrict__ sel, float* __restrict__ ptilde, double* __restrict__ logits_out,
    int32_t* __restrict__ blk_counts, int BT, int d_model, int G, int E, int k, int renorm)
{
    const int N = G * E;
    constexpr int nb = NB;         // 16-expert column blocks (<= 4)
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int blk = blockIdx.x;
    const int tok0 = blk * kRouteTok;
    // dynamic LDS: logits [32][N+1] doubles, then per-wave partials [4][2][nb][4][64] doubles, then counters [N]
    extern __shared__ double s_dyn[];
    double* s_lg = s_dyn;
    double* s_part = s_dyn + (size_t)kRouteTok * (N + 1);
    int* s_cnt = (int*)(s_part + (BF16 ? (size_t)4 * 2 * nb * 4 * 64 : 0));
#define LOGIT(tt, n) s_lg[(tt) * (N + 1) + (n)]
    for (int n = tid; n < N; n += 256) s_cnt[n] = 0;

    if constexpr (BF16) {
        const uint16_t* x = (const uint16_t*)xv;
        const uint16_t* w = (const uint16_t*)wv;
        double acc[2][NB][4];
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int c = 0; c < NB; ++c)
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[a][c][r] = 0.0;
        const int kq = 8 * (lane >> 4);  // k offset of this lane inside a 32-wide step
        const int t_a0 = tok0 + (lane & 15), t_a1 = tok0 + 16 + (lane & 15);
        const bool v0 = t_a0 < BT, v1 = t_a1 < BT;
        const uint16_t* xa0 = x + (size_t)(v0 ? t_a0 : 0) * d_model + kq;
        const uint16_t* xa1 = x + (size_t)(v1 ? t_a1 : 0) * d_model + kq;
        const bf16x8 zero8 = {};
        const int nsteps = d_model / 32;
        constexpr int U = NB <= 2 ? 8 : 4;
        for (int s0 = wave; s0 < nsteps; s0 += 4 * U) {
            bf16x8 a0[U], a1[U], bw[U][NB];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int st = s0 + 4 * u;
                const int k0 = st * 32;
                const bool live = st < nsteps;
                a0[u] = (v0 && live) ? ld_bf16x8(xa0 + k0) : zero8;
                a1[u] = (v1 && live) ? ld_bf16x8(xa1 + k0) : zero8;
#pragma unroll
                for (int c = 0; c < NB; ++c) {
                    const int n = c * 16 + (lane & 15);
                    bw[u][c] = (n < N && live) ? ld_bf16x8(w + (size_t)n * d_model + k0 + kq) : zero8;
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int c = 0; c < NB; ++c) {
                    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
                    const f32x4 p0 = mfma16(a0[u], bw[u][c], z);
                    const f32x4 p1 = mfma16(a1[u], bw[u][c], z);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        acc[0][c][r] += (double)p0[r];
                        acc[1][c][r] += (double)p1[r];
                    }
                }
        }
        // partials to LDS, then a fixed-order sum over the four waves
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int c = 0; c < NB; ++c)
#pragma unroll
                for (int r = 0; r < 4; ++r) s_part[(((wave * 2 + a) * nb + c) * 4 + r) * 64 + lane] = acc[a][c][r];
        __syncthreads();
        // accumulator element r of lane l: token row 4*(l/16) + r, expert column l%16
        for (int i = tid; i < 2 * nb * 4 * 64; i += 256) {
            const int l = i & 63, r = (i >> 6) & 3, c = (i >> 8) % nb, a = (i >> 8) / nb;
            const int n = c * 16 + (l & 15);
            if (n >= N) continue;
            double v = 0.0;
            for (int wv2 = 0; wv2 < 4; ++wv2) v += s_part[(((wv2 * 2 + a) * nb + c) * 4 + r) * 64 + l];
            LOGIT(a * 16 + 4 * (l >> 4) + r, n) = v + (bias ? (double)bias[n] : 0.0);
        }
    } else {
        const float* x = (const float*)xv;
        const float* w = (const float*)wv;
        for (int p = tid; p < kRouteTok * N; p += 256) {
            const int tt = p / N, n = p % N;
            const int t = tok0 + tt;
            double s = 0.0;
            if (t < BT) {
                const float* xr = x + (size_t)t * d_model;
                const float* wr = w + (size_t)n * d_model;
                for (int i = 0; i < d_model; ++i) s = fma((double)xr[i], (double)wr[i], s);
                if (bias) s += (double)bias[n];
            }
            LOGIT(tt, n) = s;
        }
    }
    __syncthreads();

    // Selection, renormalisation and counting: one (token, group) per thread.
    for (int p = tid; p < kRouteTok * G; p += 256) {
        const int tt = p / G, g = p % G;
        const int t = tok0 + tt;
        if (t >= BT) continue;
        const double* s = &LOGIT(tt, g * E);
        uint64_t chosen = 0;  // E <= 64
        int kept[8];
        for (int r = 0; r < k; ++r) {
            int best = -1;
            double bv = 0.0;
            for (int e = 0; e < E; ++e) {
                if ((chosen >> e) & 1) continue;
                if (best < 0 || s[e] > bv) { best = e; bv = s[e]; }  // strict: lowest index wins ties
            }
            chosen |= 1ull << best;
        }
        int j = 0;
        double mk = -INFINITY, ma = -INFINITY;
        for (int e = 0; e < E; ++e) {
            ma = fmax(ma, s[e]);
            if ((chosen >> e) & 1) { kept[j++] = e; mk = fmax(mk, s[e]); }
        }
        // p~ = softmax over the kept scores (renormalised), or in route mode 3
        // the group softmax p itself, p[e] = exp(s_e - max) / sum over all E
        float ex[8], den = 0.f;
        const double mref = renorm ? mk : ma;
        for (j = 0; j < k; ++j) { ex[j] = expf((float)(s[kept[j]] - mref)); den += ex[j]; }
        if (!renorm) {
            den = 0.f;
            for (int e = 0; e < E; ++e) den += expf((float)(s[e] - mref));
        }
        const size_t o = ((size_t)t * G + g) * k;
        for (j = 0; j < k; ++j) {
            sel[o + j] = kept[j];
            ptilde[o + j] = ex[j] / den;
            atomicAdd(&s_cnt[g * E + kept[j]], 1);
        }
    }
    if (logits_out) {
        for (int p = tid; p < kRouteTok * N; p += 256) {
            const int tt = p / N, n = p % N;
            if (tok0 + tt < BT) logits_out[(size_t)(tok0 + tt) * N + n] = LOGIT(tt, n);
        }
    }
    __syncthreads();
    for (int n = tid; n < N; n += 256) blk_counts[(size_t)blk * N + n] = s_cnt[n];
#undef LOGIT
}

// Exclusive scan of blk_counts[:, n] into blk_base[:, n]; counts[n] = total.
__global__ __launch_bounds__(256) void scan_kernel(const int32_t* __restrict__ blk_counts,
                                                   int32_t* __restrict__ blk_base,
                                                   int32_t* __restrict__ counts, int nblk, int N)
{
    const int n = blockIdx.x, tid = threadIdx.x;
    const int per = (nblk + 255) / 256;
    const int b0 = tid * per, b1 = min(nblk, b0 + per);
    int local = 0;
    for (int b = b0; b < b1; ++b) local += blk_counts[(size_t)b * N + n];
    __shared__ int s[256];
    s[tid] = local;
    __syncthreads();
    // Hillis-Steele inclusive scan over the 256 partial sums
    for (int o = 1; o < 256; o <<= 1) {
        int v = tid >= o ? s[tid - o] : 0;
        __syncthreads();
        s[tid] += v;
        __syncthreads();
    }
    int run = s[tid] - local;
    for (int b = b0; b < b1; ++b) {
        const int c = blk_counts[(size_t)b * N + n];
        blk_base[(size_t)b * N + n] = run;
        run += c;
    }
    if (tid == 255) counts[n] = s[255];
}

__global__ __launch_bounds__(256) void scatter_kernel(const int32_t* __restrict__ sel,
                                                      const int32_t* __restrict__ blk_base,
                                                      const int32_t* __restrict__ counts,
                                                      int32_t* __restrict__ offsets,
                                                      int32_t* __restrict__ rows, int BT, int G, int E,
                                                      int k, int nblk)
{
    const int N = G * E;
    __shared__ int s_off[kMaxExperts + 1];
    if (threadIdx.x == 0) {
        int run = 0;
        for (int n = 0; n < N; ++n) { s_off[n] = run; run += counts[n]; }
        s_off[N] = run;
    }
    __syncthreads();
    if (blockIdx.x == 0)
        for (int n = threadIdx.x; n <= N; n += blockDim.x) offsets[n] = s_off[n];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int half = lane >> 5, hl = lane & 31;
    const int blk = (blockIdx.x * 4 + wave) * 2 + half;
    const int t = blk * kRouteTok + hl;
    const bool valid = blk < nblk && t < BT;
    const uint32_t below = (1u << hl) - 1u;
    for (int g = 0; g < G; ++g) {
        int kept[8];
        for (int j = 0; j < k; ++j) kept[j] = valid ? sel[((size_t)t * G + g) * k + j] : -1;
        for (int e = 0; e < E; ++e) {
            bool has = false;
            for (int j = 0; j < k; ++j) has |= kept[j] == e;
            const uint64_t m = __ballot(has);
            if (has) {
                const uint32_t hm = (uint32_t)(m >> (32 * half));
                const int n = g * E + e;
                rows[s_off[n] + blk_base[(size_t)blk * N + n] + __popc(hm & below)] = t;
            }
        }
    }
}

// Compaction in one pass for small block tables (nblk * N <= kFusedMax):
// every workgroup reads the whole table of per-block counts (L2-resident),
// forms the expert totals, the offsets and the prefix of its own blocks, and
// scatters its blocks' tokens like scatter_kernel.  Integer sums, so the
// result is the same as the scan + scatter pair.
constexpr int kFusedMax = 1 << 14;
constexpr int kCmpWaves = 4;                       // waves per workgroup, two token blocks each

__global__ __launch_bounds__(64 * kCmpWaves) void compact_kernel(const int32_t* __restrict__ sel,
                                                                 const int32_t* __restrict__ blk_counts,
                                                                 int32_t* __restrict__ counts,
                                                                 int32_t* __restrict__ offsets,
                                                                 int32_t* __restrict__ rows, int BT, int G, int E,
                                                                 int k, int nblk)
{
    constexpr int NT = 64 * kCmpWaves, BPW = 2 * kCmpWaves;
    constexpr int SELR = 16;                     // kept entries per token staged through registers
    const int N = G * E, tid = threadIdx.x;
    const int blk0 = blockIdx.x * BPW;
    __shared__ int s_tot[NT], s_pre[NT];
    __shared__ int s_off[kMaxExperts + 1];
    __shared__ int s_base[BPW][kMaxExperts];
    __shared__ int s_sel[BPW * kRouteTok][SELR];
    // this lane's token of the scatter (lanes 0-31 and 32-63 of a wave take one block each)
    const int lane = tid & 63, wave = tid >> 6;
    const int half = lane >> 5, hl = lane & 31;
    const int bi = wave * 2 + half;
    const int blk = blk0 + bi;
    const int t = blk * kRouteTok + hl;
    const bool valid = blk < nblk && t < BT;
    const int Gk = G * k;
    const bool staged = Gk <= SELR;
    // Every global load of the kernel is issued up front: the token's kept
    // experts, its workgroup's own block counts, then the whole count table.
    int sv[SELR];
#pragma unroll
    for (int h = 0; h < SELR; ++h) sv[h] = (staged && valid) ? sel[(size_t)t * Gk + min(h, Gk - 1)] : -1;
    int own[BPW];
#pragma unroll
    for (int i = 0; i < BPW; ++i) own[i] = (tid < N && blk0 + i < nblk) ? blk_counts[(size_t)(blk0 + i) * N + tid] : 0;
    // 1. per-expert totals and the prefix before this workgroup's first block
    const int R = NT / N;                        // thread rows, one expert per column
    int tot = 0, pre = 0;
    if (tid < R * N) {
        const int n = tid % N;
        // 32 independent loads in flight per step (one step for tables up to 8192 entries)
        for (int b0 = tid / N; b0 < nblk; b0 += 32 * R) {
            int c[32];
#pragma unroll
            for (int i = 0; i < 32; ++i) {
                const int b = b0 + i * R;
                c[i] = b < nblk ? blk_counts[(size_t)b * N + n] : 0;
            }
#pragma unroll
            for (int i = 0; i < 32; ++i) {
                tot += c[i];
                pre += b0 + i * R < blk0 ? c[i] : 0;
            }
        }
    }
    s_tot[tid] = tot;
    s_pre[tid] = pre;
#pragma unroll
    for (int h = 0; h < SELR; ++h) s_sel[bi * kRouteTok + hl][h] = sv[h];
    __syncthreads();
    if (tid < N) {
        int tt = 0, q = 0;
        for (int r = 0; r < R; ++r) { tt += s_tot[r * N + tid]; q += s_pre[r * N + tid]; }
        s_tot[tid] = tt;         // row 0 of the table is only read by its own thread
        s_pre[tid] = q;
    }
    __syncthreads();
    if (tid == 0) {
        int run = 0;
        for (int n = 0; n < N; ++n) { s_off[n] = run; run += s_tot[n]; }
        s_off[N] = run;
    }
    __syncthreads();
    if (tid < N) {
        int run = s_off[tid] + s_pre[tid];
#pragma unroll
        for (int i = 0; i < BPW; ++i) {
            s_base[i][tid] = run;
            run += own[i];
        }
        if (blockIdx.x == 0) counts[tid] = s_tot[tid];
    }
    if (blockIdx.x == 0)
        for (int n = tid; n <= N; n += NT) offsets[n] = s_off[n];
    __syncthreads();
    // 2. scatter: wave ballots rank the token among its block's tokens that kept each expert
    const uint32_t below = (1u << hl) - 1u;
    const int* my_sel = s_sel[bi * kRouteTok + hl];
    if (staged) {
        // kept experts from LDS only, so no wait on global memory sits between the stores
        // (a load's wait would also wait for every store issued before it): first the token's
        // kept experts as one mask over the N <= 64 experts, then one ballot per expert, skipping
        // the experts no token of the wave kept
        uint64_t kept = 0;
        if (valid)
            for (int j = 0; j < Gk; ++j) kept |= 1ull << ((j / k) * E + my_sel[j]);
        for (int n = 0; n < N; ++n) {
            const bool has = (kept >> n) & 1;
            const uint64_t m = __ballot(has);
            if (m == 0) continue;
            if (has) rows[s_base[bi][n] + __popc((uint32_t)(m >> (32 * half)) & below)] = t;
        }
        return;
    }
    for (int g = 0; g < G; ++g) {
        int kept[8];
        for (int j = 0; j < k; ++j)
            kept[j] = !valid ? -1 : staged ? my_sel[g * k + j] : sel[((size_t)t * G + g) * k + j];
        for (int e = 0; e < E; ++e) {
            bool has = false;
            for (int j = 0; j < k; ++j) has |= kept[j] == e;
            const uint64_t m = __ballot(has);
            if (has) {
                const uint32_t hm = (uint32_t)(m >> (32 * half));
                rows[s_base[bi][g * E + e] + __popc(hm & below)] = t;
            }
        }
    }
}

__global__ void zero_i32_kernel(int32_t* __restrict__ a, int n)
{
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) a[i] = 0;
}

size_t route_workspace_bytes(int BT, int N)
{
    const size_t nblk = (size_t)(BT + kRouteTok - 1) / kRouteTok;
    return 2 * nblk * (size_t)N * sizeof(int32_t) + 256;
}

int launch_route(const RouteArgs& a, hipStream_t st)
{
    const int N = a.G * a.E;
    const int nblk = (a.BT + kRouteTok - 1) / kRouteTok;
    int32_t* blk_counts = (int32_t*)a.workspace;
    int32_t* blk_base = blk_counts + (size_t)nblk * N;
    if (a.BT == 0) {
        zero_i32_kernel<<<1, 256, 0, st>>>(a.counts, N);
        zero_i32_kernel<<<1, 256, 0, st>>>(a.offsets, N + 1);
        return hipGetLastError() == hipSuccess ? 0 : -1;
    }
    const int grid = nblk;
    const int nb = (N + 15) / 16;
    const size_t lds = (size_t)kRouteTok * (N + 1) * sizeof(double) +
                       (a.bf16 ? (size_t)4 * 2 * nb * 4 * 64 * sizeof(double) : 0) + (size_t)N * sizeof(int);
    if (a.bf16) {
#define GQE_ROUTER(NBV) router_kernel<true, NBV><<<grid, 256, lds, st>>>(a.x, a.w_router, a.b_router, a.sel, \
        a.p_tilde, a.logits, blk_counts, a.BT, a.d_model, a.G, a.E, a.k, a.renorm ? 1 : 0)
        switch (nb) {
        case 1: GQE_ROUTER(1); break;
        case 2: GQE_ROUTER(2); break;
        case 3: GQE_ROUTER(3); break;
        default: GQE_ROUTER(4); break;
        }
#undef GQE_ROUTER
    } else {
        router_kernel<false, 1><<<grid, 256, lds, st>>>(a.x, a.w_router, a.b_router, a.sel, a.p_tilde, a.logits,
                                                      blk_counts, a.BT, a.d_model, a.G, a.E, a.k, a.renorm ? 1 : 0);
    }
    if ((long long)nblk * N <= kFusedMax) {
        const int cgrid = (nblk + 2 * kCmpWaves - 1) / (2 * kCmpWaves);
        compact_kernel<<<cgrid, 64 * kCmpWaves, 0, st>>>(a.sel, blk_counts, a.counts, a.offsets, a.rows, a.BT, a.G,
                                                         a.E, a.k, nblk);
    } else {
        scan_kernel<<<N, 256, 0, st>>>(blk_counts, blk_base, a.counts, nblk, N);
        const int sgrid = (nblk + 7) / 8;
        scatter_kernel<<<sgrid, 256, 0, st>>>(a.sel, blk_base, a.counts, a.offsets, a.rows, a.BT, a.G, a.E, a.k,
                                              nblk);
    }
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace gqe
