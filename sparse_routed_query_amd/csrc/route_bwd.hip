// Backward through slot assembly and routing (gfx950): the gradient that the
// weighted slot carries back to the router -- its differentiable learning
// path (GQE study note §3-2 (4)) -- and the hard slots' share of dout.
//
// Forward being differentiated, per token t and group g (§3-2 (2), (4)):
//   s = W_router x_t + b,  p = softmax over the group's E experts,
//   p~_j = p_{S_j} / sum_i p_{S_i} over the kept set S (held fixed),
//   weighted slot(s) w = sum p~_j h_{g,j} (summed over groups in mode 0, one
//   per group in mode 1, none in mode 2), hard slots h passed through.
// Because p~ is the softmax of the kept scores alone, the score gradient is
//   ds_{S_j} = p~_j (dp~_j - sum_i p~_i dp~_i),  dp~_j = <dout_w, h_{g,j}>,
// and zero for the experts that were not kept.
//
// Kernels, all fp32 and in fixed order (so results do not depend on timing):
//   token kernel   one wave per token: d_hard, dp~ by wave reductions, ds;
//   dw kernels     dW_router and db as block partial sums over 256 tokens,
//                  then the partials added in block order;
//   dx kernel      dx = ds W_router, each column summed over n in order.
#include "gqe_device.h"
#include "gqe_launch.h"

namespace gqe {

constexpr int kRbTokBlock = 256;   // tokens per partial sum of dW_router

// one wave per token; lane l holds d = l, l + 64 (D <= 128)
template <int D>
__global__ __launch_bounds__(256) void route_bwd_token_kernel(const float* __restrict__ dout,
                                                              const float* __restrict__ out,
                                                              const float* __restrict__ p_tilde,
                                                              const int32_t* __restrict__ sel,
                                                              float* __restrict__ d_hard, float* __restrict__ d_logits,
                                                              long long BT, int G, int E, int k, int S, int mode)
{
    constexpr int ND = (D + 63) / 64;
    const long long t = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= BT) return;
    const int lane = threadIdx.x & 63;
    const int kG = G * k;
    const float* go = dout + (size_t)t * S * D;
    const float* ho = out + (size_t)t * S * D;
    float* dh = d_hard + (size_t)t * kG * D;
    const float* pt = p_tilde + (size_t)t * kG;
    const int32_t* st = sel + (size_t)t * kG;
    float* dl = d_logits + (size_t)t * G * E;
    for (int g = 0; g < G; ++g) {
        float dw[ND];
        const int wslot = mode == 0 ? kG : kG + g;
#pragma unroll
        for (int i = 0; i < ND; ++i) {
            const int d = lane + 64 * i;
            dw[i] = (mode != 2 && d < D) ? go[(size_t)wslot * D + d] : 0.f;
        }
        float dpt[8], ptg[8];
        float s = 0.f;
        for (int j = 0; j < k; ++j) {
            const int h = g * k + j;
            const float p = pt[h];
            float dot = 0.f;
#pragma unroll
            for (int i = 0; i < ND; ++i) {
                const int d = lane + 64 * i;
                if (d < D) {
                    dh[(size_t)h * D + d] = fmaf(p, dw[i], go[(size_t)h * D + d]);
                    dot = fmaf(ho[(size_t)h * D + d], dw[i], dot);
                }
            }
            dot = wave_sum(dot);
            dpt[j] = dot;
            ptg[j] = p;
            s = fmaf(p, dot, s);
        }
        // score gradient of the group's E experts: kept ones from the
        // renormalised softmax, the others zero
        if (lane < E) {
            float v = 0.f;
            for (int j = 0; j < k; ++j)
                if (st[g * k + j] == lane) v = ptg[j] * (dpt[j] - s);
            dl[g * E + lane] = v;
        }
    }
}

// partial[blk][n][c] = sum over the block's tokens of ds[t][n] x[t][c]; the
// column-chunk-0 workgroup of each block also writes partial[blk][n][C] = sum ds[t][n]
template <typename ET>
__global__ __launch_bounds__(256) void route_bwd_dw_partial_kernel(const float* __restrict__ d_logits,
                                                                   const ET* __restrict__ x, float* __restrict__ part,
                                                                   long long BT, int N, int C)
{
    constexpr int NMAX = 64, TCH = 64;   // experts, tokens per LDS chunk
    __shared__ float s_dl[TCH][NMAX];
    const long long t0 = (long long)blockIdx.x * kRbTokBlock;
    const int c = blockIdx.y * 256 + threadIdx.x;
    float acc[NMAX], db[NMAX];
#pragma unroll
    for (int n = 0; n < NMAX; ++n) acc[n] = db[n] = 0.f;
    for (int tc = 0; tc < kRbTokBlock; tc += TCH) {
        __syncthreads();
        for (int i = threadIdx.x; i < TCH * N; i += 256) {
            const long long t = t0 + tc + i / N;
            s_dl[i / N][i % N] = t < BT ? d_logits[(size_t)t * N + i % N] : 0.f;
        }
        __syncthreads();
        for (int tt = 0; tt < TCH; ++tt) {
            const long long t = t0 + tc + tt;
            if (t >= BT) break;
            float xv = 0.f;
            if (c < C) {
                if constexpr (sizeof(ET) == 2) xv = bf2f((uint16_t)x[(size_t)t * C + c]);
                else xv = (float)x[(size_t)t * C + c];
            }
#pragma unroll
            for (int n = 0; n < NMAX; ++n) {
                if (n < N) {
                    acc[n] = fmaf(s_dl[tt][n], xv, acc[n]);
                    db[n] += s_dl[tt][n];
                }
            }
        }
    }
    float* pb = part + (size_t)blockIdx.x * N * (C + 1);
    if (c < C) {
#pragma unroll
        for (int n = 0; n < NMAX; ++n)
            if (n < N) pb[(size_t)n * (C + 1) + c] = acc[n];
    }
    if (blockIdx.y == 0 && threadIdx.x == 0) {
#pragma unroll
        for (int n = 0; n < NMAX; ++n)
            if (n < N) pb[(size_t)n * (C + 1) + C] = db[n];
    }
}

// dW_router[n][c] (and db[n] at c = C) = the block partials added in block order
__global__ __launch_bounds__(256) void route_bwd_dw_final_kernel(const float* __restrict__ part, int nblk, int N,
                                                                 int C, float* __restrict__ dw, float* __restrict__ db)
{
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i >= (long long)N * (C + 1)) return;
    float s = 0.f;
    for (int b = 0; b < nblk; ++b) s += part[(size_t)b * N * (C + 1) + i];
    const int n = (int)(i / (C + 1)), c = (int)(i % (C + 1));
    if (c < C) dw[(size_t)n * C + c] = s;
    else if (db) db[n] = s;
}

// dx[t][c] = sum_n ds[t][n] W_router[n][c], n in order; four columns per thread
template <typename ET>
__global__ __launch_bounds__(256) void route_bwd_dx_kernel(const float* __restrict__ d_logits,
                                                           const ET* __restrict__ w_router, float* __restrict__ dx,
                                                           long long BT, int N, int C)
{
    const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
    const int CQ = (C + 3) / 4;
    if (gid >= BT * CQ) return;
    const long long t = gid / CQ;
    const int c0 = (int)(gid % CQ) * 4;
    const float* dl = d_logits + (size_t)t * N;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int n = 0; n < N; ++n) {
        const float a = dl[n];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int c = c0 + e;
            if (c < C) {
                float wv;
                if constexpr (sizeof(ET) == 2) wv = bf2f((uint16_t)w_router[(size_t)n * C + c]);
                else wv = (float)w_router[(size_t)n * C + c];
                acc[e] = fmaf(a, wv, acc[e]);
            }
        }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e)
        if (c0 + e < C) dx[(size_t)t * C + c0 + e] = acc[e];
}

size_t route_bwd_workspace_bytes(long long BT, int N, int C)
{
    const long long nblk = (BT + kRbTokBlock - 1) / kRbTokBlock;
    return (size_t)nblk * N * (C + 1) * sizeof(float) + 256;
}

int launch_route_bwd(const RouteBwdArgs& a, hipStream_t st)
{
    if (a.BT == 0) return 0;
    const int N = a.G * a.E, C = a.d_model;
    const unsigned tok_grid = (unsigned)((a.BT + 3) / 4);
    switch (a.d_head) {
    case 32: route_bwd_token_kernel<32><<<tok_grid, 256, 0, st>>>(a.dout, a.out, a.p_tilde, a.sel, a.d_hard,
                                                                   a.d_logits, a.BT, a.G, a.E, a.k, a.S, a.route_mode);
        break;
    case 64: route_bwd_token_kernel<64><<<tok_grid, 256, 0, st>>>(a.dout, a.out, a.p_tilde, a.sel, a.d_hard,
                                                                   a.d_logits, a.BT, a.G, a.E, a.k, a.S, a.route_mode);
        break;
    case 128: route_bwd_token_kernel<128><<<tok_grid, 256, 0, st>>>(a.dout, a.out, a.p_tilde, a.sel, a.d_hard,
                                                                     a.d_logits, a.BT, a.G, a.E, a.k, a.S,
                                                                     a.route_mode);
        break;
    default: return -2;
    }
    if (a.dw_router) {   // (db_router is only computed with it)
        const unsigned nblk = (unsigned)((a.BT + kRbTokBlock - 1) / kRbTokBlock);
        const dim3 pg(nblk, (unsigned)((C + 255) / 256));
        float* part = (float*)a.workspace;
        if (a.bf16)
            route_bwd_dw_partial_kernel<uint16_t><<<pg, 256, 0, st>>>(a.d_logits, (const uint16_t*)a.x, part, a.BT, N,
                                                                      C);
        else
            route_bwd_dw_partial_kernel<float><<<pg, 256, 0, st>>>(a.d_logits, (const float*)a.x, part, a.BT, N, C);
        const long long n_out = (long long)N * (C + 1);
        route_bwd_dw_final_kernel<<<(unsigned)((n_out + 255) / 256), 256, 0, st>>>(part, (int)nblk, N, C,
                                                                                   a.dw_router, a.db_router);
    }
    if (a.dx) {
        const long long n = a.BT * ((C + 3) / 4);
        if (a.bf16)
            route_bwd_dx_kernel<uint16_t><<<(unsigned)((n + 255) / 256), 256, 0, st>>>(
                a.d_logits, (const uint16_t*)a.w_router, a.dx, a.BT, N, C);
        else
            route_bwd_dx_kernel<float><<<(unsigned)((n + 255) / 256), 256, 0, st>>>(
                a.d_logits, (const float*)a.w_router, a.dx, a.BT, N, C);
    }
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace gqe
