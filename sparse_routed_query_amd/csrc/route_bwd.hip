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
//   token kernel   one (token, group) unit per d_head/4 lanes: d_hard, dp~ by
//                  lane-group reductions, ds;
//   dw kernels     dW_router = ds^T x (a contraction over tokens, on fp32
//                  MFMA) and db as partial sums over 256-token blocks, then
//                  the partials added in block order;
//   dx kernel      dx = ds W_router, W_router held in registers, each column
//                  summed over n in order.
#include "gqe_device.h"
#include "gqe_launch.h"

namespace gqe {

constexpr int kRbTokBlock = 256;   // tokens per partial sum of dW_router (4 waves x 64)
constexpr int kRbMaxK = 8;         // kept experts per group (the descriptor's limit)
constexpr int kRbDxTok = 32;       // tokens per dx workgroup

// sum over an aligned group of L lanes (butterfly: every lane gets the same value)
template <int L>
__device__ __forceinline__ float lanes_sum(float v)
{
#pragma unroll
    for (int o = 1; o < L; o <<= 1) v += __shfl_xor(v, o);
    return v;
}

// One (token t, group g) unit per D/4 lanes; each lane holds four elements of d_head.
template <int D>
__global__ __launch_bounds__(256) void route_bwd_token_kernel(const float* __restrict__ dout,
                                                              const float* __restrict__ out,
                                                              const float* __restrict__ p_tilde,
                                                              const int32_t* __restrict__ sel,
                                                              float* __restrict__ d_hard, float* __restrict__ d_logits,
                                                              long long BT, int G, int E, int k, int S, int mode)
{
    constexpr int L = D / 4;
    const long long u = (long long)blockIdx.x * (256 / L) + threadIdx.x / L;
    if (u >= BT * G) return;   // (whole lane groups leave together)
    const int lane = threadIdx.x % L;
    const long long t = u / G;
    const int g = (int)(u - t * G);
    const int kG = G * k;
    const float* go = dout + (size_t)t * S * D + lane * 4;
    const float* ho = out + (size_t)t * S * D + lane * 4;
    float* dh = d_hard + (size_t)t * kG * D + lane * 4;
    const float* pt = p_tilde + (size_t)t * kG + g * k;
    const int32_t* st = sel + (size_t)t * kG + g * k;
    f32x4 dw = {0.f, 0.f, 0.f, 0.f};
    if (mode != 2) dw = *(const f32x4*)(go + (size_t)(mode == 0 ? kG : kG + g) * D);
    float dpt[kRbMaxK], ptg[kRbMaxK];
    int sj[kRbMaxK];
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < kRbMaxK; ++j) {
        if (j < k) {
            const int h = g * k + j;
            const float p = pt[j];
            const f32x4 gh = *(const f32x4*)(go + (size_t)h * D);
            const f32x4 hh = *(const f32x4*)(ho + (size_t)h * D);
            f32x4 r;
            float dot = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                r[e] = fmaf(p, dw[e], gh[e]);
                dot = fmaf(hh[e], dw[e], dot);
            }
            *(f32x4*)(dh + (size_t)h * D) = r;
            dot = lanes_sum<L>(dot);
            dpt[j] = dot;
            ptg[j] = p;
            sj[j] = st[j];
            s = fmaf(p, dot, s);
        }
    }
    // score gradient of the group's E experts: kept ones from the
    // renormalised softmax, the others zero
    float* dl = d_logits + (size_t)t * G * E + (size_t)g * E;
    for (int e = lane; e < E; e += L) {
        float v = 0.f;
#pragma unroll
        for (int j = 0; j < kRbMaxK; ++j)
            if (j < k && sj[j] == e) v = ptg[j] * (dpt[j] - s);
        dl[e] = v;
    }
}

// dW_router as a contraction over tokens on v_mfma_f32_16x16x4_f32: for a
// 256-token block, A = ds^T (16 experts x 4 tokens), B = x (4 tokens x 16
// columns), so one MFMA adds four tokens to a 16 x 16 tile of dW.  Lane l
// loads x[token l/16][8 consecutive columns] (bf16) with one 16-byte load and
// feeds element j to the j-th of eight MFMAs, so MFMA j's column i is the
// workgroup's column 8i + j.  Each wave adds 64 tokens; waves 1-3 hand theirs
// to wave 0 through LDS, which adds them in wave order and writes
//   part[blk][n][c] (16-byte stores), pdb[blk][n] = sum over the block of ds[t][n].
// Rows past the end read as zero through the buffer descriptors' range check.
template <typename ET, int NB>
__global__ __launch_bounds__(256) void route_bwd_dw_partial_kernel(const float* __restrict__ d_logits,
                                                                   const ET* __restrict__ x, float* __restrict__ part,
                                                                   float* __restrict__ pdb, long long BT, int N, int C)
{
    constexpr int VE = sizeof(ET) == 2 ? 8 : 1;   // columns per lane and load
    constexpr int CW = 16 * VE;                   // columns per workgroup
    constexpr int NA = NB * VE * 4;               // accumulators per lane
    constexpr int US = 8;                         // MFMA steps (4 tokens each) per batch of loads
    __shared__ float s_red[3][NA + NB][64];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int r = lane & 15, q = lane >> 4;
    const long long tb = (long long)blockIdx.x * kRbTokBlock;
    const int rows = (int)min((long long)kRbTokBlock, BT - tb);
    const int cw0 = blockIdx.y * CW;
    const int n0 = blockIdx.z * 16 * NB;
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc((void*)(x + (size_t)tb * C), 0,
                                                                        rows * C * (int)sizeof(ET), 0x00020000);
    const __amdgpu_buffer_rsrc_t rd = __builtin_amdgcn_make_buffer_rsrc((void*)(d_logits + (size_t)tb * N), 0,
                                                                        rows * N * 4, 0x00020000);
    f32x4 acc[NB][VE];
    float dbs[NB];
#pragma unroll
    for (int nt = 0; nt < NB; ++nt) {
        dbs[nt] = 0.f;
#pragma unroll
        for (int j = 0; j < VE; ++j) acc[nt][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll 1
    for (int s0 = 0; s0 < 64; s0 += 4 * US) {
        u32x4 xv[US];
        float xs[US];
        float av[US][NB];
#pragma unroll
        for (int u = 0; u < US; ++u) {
            const int tl = wave * 64 + s0 + 4 * u + q;
            const uint32_t xoff = (uint32_t)((tl * C + cw0 + r * VE) * (int)sizeof(ET));
            if constexpr (VE == 8)
                xv[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, xoff, 0, 0));
            else
                xs[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rx, xoff, 0, 0));
#pragma unroll
            for (int nt = 0; nt < NB; ++nt) {
                const int n = n0 + nt * 16 + r;
                const uint32_t doff = n < N ? (uint32_t)((tl * N + n) * 4) : 0x7FFFFFF0u;
                av[u][nt] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rd, doff, 0, 0));
            }
        }
#pragma unroll
        for (int u = 0; u < US; ++u) {
#pragma unroll
            for (int nt = 0; nt < NB; ++nt) {
                dbs[nt] += av[u][nt];
#pragma unroll
                for (int j = 0; j < VE; ++j) {
                    float b;
                    if constexpr (VE == 8) {
                        const uint32_t wd = xv[u][j >> 1];   // (element copied out before the bit cast)
                        b = __builtin_bit_cast(float, (j & 1) ? (wd & 0xFFFF0000u) : (wd << 16));
                    } else {
                        b = xs[u];
                    }
                    acc[nt][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[u][nt], b, acc[nt][j], 0, 0, 0);
                }
            }
        }
    }
    if (wave > 0) {
#pragma unroll
        for (int nt = 0; nt < NB; ++nt) {
#pragma unroll
            for (int j = 0; j < VE; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) s_red[wave - 1][(nt * VE + j) * 4 + e][lane] = acc[nt][j][e];
            s_red[wave - 1][NA + nt][lane] = dbs[nt];
        }
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll 1
    for (int w = 0; w < 3; ++w) {
#pragma unroll
        for (int nt = 0; nt < NB; ++nt) {
#pragma unroll
            for (int j = 0; j < VE; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[nt][j][e] += s_red[w][(nt * VE + j) * 4 + e][lane];
            dbs[nt] += s_red[w][NA + nt][lane];
        }
    }
    // lane l holds dW rows n0 + 16 nt + 4 (l/16) + e, columns cw0 + VE (l%16) + j
    float* pb = part + (size_t)blockIdx.x * N * C;
    const int c = cw0 + r * VE;
#pragma unroll
    for (int nt = 0; nt < NB; ++nt) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int n = n0 + nt * 16 + 4 * q + e;
            if (n < N && c < C) {
                if constexpr (VE == 8) {
                    const f32x4 lo = {acc[nt][0][e], acc[nt][1][e], acc[nt][2][e], acc[nt][3][e]};
                    const f32x4 hi = {acc[nt][4][e], acc[nt][5][e], acc[nt][6][e], acc[nt][7][e]};
                    *(f32x4*)(pb + (size_t)n * C + c) = lo;
                    *(f32x4*)(pb + (size_t)n * C + c + 4) = hi;
                } else {
                    pb[(size_t)n * C + c] = acc[nt][0][e];
                }
            }
        }
        // db: the four lane rows (tokens l/16) added in a fixed order
        float v = dbs[nt];
        v += __shfl_xor(v, 16);
        v += __shfl_xor(v, 32);
        const int n = n0 + nt * 16 + r;
        if (blockIdx.y == 0 && q == 0 && n < N) pdb[(size_t)blockIdx.x * N + n] = v;
    }
}

// dW_router[n][c] = sum over blocks of part[b][n][c], db[n] = sum of pdb[b][n].
// A workgroup finishes 64 outputs: each wave adds a quarter of the blocks in
// block order, then wave 0 adds the four quarters in order.
__global__ __launch_bounds__(256) void route_bwd_dw_final_kernel(const float* __restrict__ part,
                                                                 const float* __restrict__ pdb, int nblk, int N, int C,
                                                                 float* __restrict__ dw, float* __restrict__ db)
{
    __shared__ float s_q[4][64];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const long long NC = (long long)N * C;
    const long long i = (long long)blockIdx.x * 64 + lane;
    const bool valid = i < NC + N, is_w = i < NC;
    const float* src = is_w ? part + i : pdb + (valid ? i - NC : 0);
    const size_t stride = is_w ? (size_t)NC : (size_t)N;
    const int per = (nblk + 3) / 4;
    const int b0 = wave * per, b1 = min(nblk, b0 + per);
    float s = 0.f;
    if (valid) {
        for (int b = b0; b < b1; b += 8) {
            float v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = src[(size_t)min(b + u, b1 - 1) * stride];
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (b + u < b1) s += v[u];
        }
    }
    s_q[wave][lane] = s;
    __syncthreads();
    if (wave == 0 && valid) {
        const float rsum = ((s_q[0][lane] + s_q[1][lane]) + s_q[2][lane]) + s_q[3][lane];
        if (is_w) dw[i] = rsum;
        else if (db) db[i - NC] = rsum;
    }
}

// dx[t][c] = sum_n ds[t][n] W_router[n][c], n in order.  Each thread keeps the
// W_router values of its CPT columns (NP rows, zero past N) in registers; a
// workgroup stages its tokens' ds rows in LDS and reads them as broadcasts.
template <typename ET, int NP>
__global__ __launch_bounds__(256) void route_bwd_dx_kernel(const float* __restrict__ d_logits,
                                                           const ET* __restrict__ w_router, float* __restrict__ dx,
                                                           long long BT, int N, int C)
{
    constexpr int CPT = 64 / NP;
    __shared__ __attribute__((aligned(16))) float s_dl[kRbDxTok][NP];
    const long long t0 = (long long)blockIdx.x * kRbDxTok;
    const int nt = (int)min((long long)kRbDxTok, BT - t0);
    for (int i = threadIdx.x; i < kRbDxTok * NP; i += 256) {
        const int tt = i / NP, n = i % NP;
        s_dl[tt][n] = (tt < nt && n < N) ? d_logits[(size_t)(t0 + tt) * N + n] : 0.f;
    }
    const int c0 = (blockIdx.y * 256 + threadIdx.x) * CPT;
    float w[NP][CPT];
#pragma unroll
    for (int n = 0; n < NP; ++n)
#pragma unroll
        for (int e = 0; e < CPT; ++e) {
            const int c = c0 + e;
            float v = 0.f;
            if (n < N && c < C) {
                if constexpr (sizeof(ET) == 2) v = bf2f((uint16_t)w_router[(size_t)n * C + c]);
                else v = (float)w_router[(size_t)n * C + c];
            }
            w[n][e] = v;
        }
    __syncthreads();
    const bool vec = (C % CPT) == 0 && c0 + CPT <= C;
    for (int tt = 0; tt < nt; ++tt) {
        float acc[CPT];
#pragma unroll
        for (int e = 0; e < CPT; ++e) acc[e] = 0.f;
#pragma unroll
        for (int n4 = 0; n4 < NP; n4 += 4) {
            const f32x4 a = *(const f32x4*)&s_dl[tt][n4];
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int e = 0; e < CPT; ++e) acc[e] = fmaf(a[m], w[n4 + m][e], acc[e]);
        }
        float* o = dx + (size_t)(t0 + tt) * C + c0;
        if (vec) {   // (streamed out: nothing reads dx back here)
            if constexpr (CPT == 4) __builtin_nontemporal_store(f32x4{acc[0], acc[1], acc[2], acc[3]}, (f32x4*)o);
            else if constexpr (CPT == 2)
                __builtin_nontemporal_store(__builtin_bit_cast(double, make_float2(acc[0], acc[1])), (double*)o);
            else __builtin_nontemporal_store(acc[0], o);
        } else {
#pragma unroll
            for (int e = 0; e < CPT; ++e)
                if (c0 + e < C) o[e] = acc[e];
        }
    }
}

// Router importance of expert n = g*E + e: sum over tokens of its in-group
// softmax probability, from the router's fp64 scores.  One workgroup per
// expert; thread i takes tokens i, i + 256, ..., in fp64, then the 256 partial
// sums are added in a fixed tree order.
__global__ __launch_bounds__(256) void route_stats_kernel(const double* __restrict__ logits, long long BT, int G,
                                                          int E, float* __restrict__ importance)
{
    __shared__ double s_red[256];
    const int n = blockIdx.x, g = n / E, e = n - g * E, N = G * E;
    double acc = 0.0;
    for (long long t = threadIdx.x; t < BT; t += 256) {
        const double* lg = logits + (size_t)t * N + (size_t)g * E;
        double m = lg[0];
        for (int i = 1; i < E; ++i) m = fmax(m, lg[i]);
        double den = 0.0;
        for (int i = 0; i < E; ++i) den += exp(lg[i] - m);
        acc += exp(lg[e] - m) / den;
    }
    s_red[threadIdx.x] = acc;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
        if ((int)threadIdx.x < o) s_red[threadIdx.x] += s_red[threadIdx.x + o];
        __syncthreads();
    }
    if (threadIdx.x == 0) importance[n] = (float)s_red[0];
}

int launch_route_stats(const double* logits, long long BT, int G, int E, float* importance, hipStream_t st)
{
    route_stats_kernel<<<(unsigned)(G * E), 256, 0, st>>>(logits, BT, G, E, importance);
    return hipGetLastError() == hipSuccess ? 0 : -1;
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
    if (a.k > kRbMaxK || N > 64 || (long long)kRbTokBlock * C * 4 >= (1ll << 31)) return -2;
    const long long units = a.BT * a.G;
    switch (a.d_head) {
    case 32: route_bwd_token_kernel<32><<<(unsigned)((units + 31) / 32), 256, 0, st>>>(
            a.dout, a.out, a.p_tilde, a.sel, a.d_hard, a.d_logits, a.BT, a.G, a.E, a.k, a.S, a.route_mode);
        break;
    case 64: route_bwd_token_kernel<64><<<(unsigned)((units + 15) / 16), 256, 0, st>>>(
            a.dout, a.out, a.p_tilde, a.sel, a.d_hard, a.d_logits, a.BT, a.G, a.E, a.k, a.S, a.route_mode);
        break;
    case 128: route_bwd_token_kernel<128><<<(unsigned)((units + 7) / 8), 256, 0, st>>>(
            a.dout, a.out, a.p_tilde, a.sel, a.d_hard, a.d_logits, a.BT, a.G, a.E, a.k, a.S, a.route_mode);
        break;
    default: return -2;
    }
    if (a.dw_router) {   // (db_router is only computed with it)
        const unsigned nblk = (unsigned)((a.BT + kRbTokBlock - 1) / kRbTokBlock);
        float* part = (float*)a.workspace;
        float* pdb = part + (size_t)nblk * N * C;
        const int nb = N <= 16 ? 1 : 2;
        const int cw = a.bf16 ? 128 : 16;
        const dim3 pg(nblk, (unsigned)((C + cw - 1) / cw), (unsigned)((N + 16 * nb - 1) / (16 * nb)));
        if (a.bf16) {
            if (nb == 1)
                route_bwd_dw_partial_kernel<uint16_t, 1><<<pg, 256, 0, st>>>(a.d_logits, (const uint16_t*)a.x, part,
                                                                            pdb, a.BT, N, C);
            else
                route_bwd_dw_partial_kernel<uint16_t, 2><<<pg, 256, 0, st>>>(a.d_logits, (const uint16_t*)a.x, part,
                                                                            pdb, a.BT, N, C);
        } else {
            if (nb == 1)
                route_bwd_dw_partial_kernel<float, 1><<<pg, 256, 0, st>>>(a.d_logits, (const float*)a.x, part, pdb,
                                                                         a.BT, N, C);
            else
                route_bwd_dw_partial_kernel<float, 2><<<pg, 256, 0, st>>>(a.d_logits, (const float*)a.x, part, pdb,
                                                                         a.BT, N, C);
        }
        const long long n_out = (long long)N * C + N;
        route_bwd_dw_final_kernel<<<(unsigned)((n_out + 63) / 64), 256, 0, st>>>(part, pdb, (int)nblk, N, C,
                                                                                 a.dw_router, a.db_router);
    }
    if (a.dx) {
        const int np = N <= 16 ? 16 : N <= 32 ? 32 : 64;
        const int cpt = 64 / np;
        const dim3 xg((unsigned)((a.BT + kRbDxTok - 1) / kRbDxTok), (unsigned)((C + 256 * cpt - 1) / (256 * cpt)));
#define RB_DX(ET, NP)                                                                                         \
    route_bwd_dx_kernel<ET, NP><<<xg, 256, 0, st>>>(a.d_logits, (const ET*)a.w_router, a.dx, a.BT, N, C)
        if (a.bf16) {
            if (np == 16) RB_DX(uint16_t, 16); else if (np == 32) RB_DX(uint16_t, 32); else RB_DX(uint16_t, 64);
        } else {
            if (np == 16) RB_DX(float, 16); else if (np == 32) RB_DX(float, 32); else RB_DX(float, 64);
        }
#undef RB_DX
    }
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace gqe
