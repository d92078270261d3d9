// Backward of the query, key and value projections (gfx950): the gradients
// that reach the layer's projection weights and its input once the attention
// backward has produced the gradients of the query rows, K and V.
//
// Forward being differentiated (GQE study note §3-2 (2), (5): each kept
// expert is its own query projection of x_t, the shared head another, and
// unselected experts are never projected; GQA tutorial, freeguideonline,
// "GQA 核心原理与计算流程" step 2: K and V are projections of x):
//   q_{t,g,j} = R_t W_q[g E + S_j] x_t,  q_sh_t = R_t W_q[N] x_t,
//   k_{t,h} = R_t W_k[h] x_t,            v_{t,h} = W_v[h] x_t,
// R_t the rotary embedding at position t when the forward used one (identity
// otherwise).  With the kept sets fixed:
//   dW_q[n] = sum over the tokens that kept n of (R_t^T dq)^T x_t, likewise
//   the shared head over every token, dW_k[h], dW_v[h] over every token;
//   dx_t = sum over the token's kept experts of W_q[n]^T R_t^T dq
//          + W_q[N]^T R_t^T dq_sh + sum_h (W_k[h]^T R_t^T dk + W_v[h]^T dv).
// Arithmetic: the incoming fp32 gradients are rotated back in fp32 and
// rounded to bf16 for bf16 MFMA products with fp32 accumulation (x and the
// weights are exact bf16); every sum runs in a fixed order and no atomics are
// used, so results are deterministic.
//
// dw kernel: one workgroup per (head, 256 columns of d_model, row chunk): a
//   chunk of the head's rows (its compacted bucket, or every token) in
//   stages of 64, both operands read across their stored rows with
//   transposing LDS reads; at d_head <= 64 the dense heads (shared, K, V)
//   go two to a workgroup, sharing each staged x tile; with a workspace the
//   rows are cut into up to 16 chunks whose partial sums a second kernel
//   adds in chunk order (so the launch has enough workgroups), else one
//   chunk writes dW directly.
// dx kernel: one workgroup per (128 tokens, 64 at d_head 128; 128 columns): the heads in turn,
//   each a stage of [tokens x D] gradient rows (zero where the token did
//   not keep the expert) against the head's [D x 128] weight slice.
#include "gqe_device.h"
#include "gqe_launch.h"

namespace gqe {

__device__ __forceinline__ int pb_kind(const ProjBwdArgs& a, int n, int& h)
{
    const int N = a.G * a.E;
    if (n < N) { h = n; return 0; }
    n -= N;
    if (n < a.ns) { h = n; return 1; }
    n -= a.ns;
    if (n < a.nkv) { h = n; return 2; }
    h = n - a.nkv;
    return 3;
}

// Gradient row of head n (kind, h) for token tok, or nullptr when tok did not
// keep the routed expert n.
__device__ __forceinline__ const float* pb_src(const ProjBwdArgs& a, int kind, int h, int n, int tok)
{
    const int b = tok / a.T, t = tok - b * a.T, D = a.D;
    if (kind == 1) return a.dq_shared + (size_t)tok * D;
    if (kind == 2) return a.dk + (((size_t)b * a.nkv + h) * a.T + t) * D;
    if (kind == 3) return a.dv + (((size_t)b * a.nkv + h) * a.T + t) * D;
    const int g = n / a.E, e = n - g * a.E;
    const int32_t* s = a.sel + ((size_t)tok * a.G + g) * a.k;
    int j = -1;
    for (int i = 0; i < a.k; ++i) j = s[i] == e ? i : j;
    return j < 0 ? nullptr : a.dq_routed + ((((size_t)b * a.G + g) * a.T + t) * a.k + j) * D;
}

// Loads the pair (d0 .. d0+3, d0+D/2 .. +3) of a gradient row, rotated back
// by the token's rotary angle when asked, as two 4-wide fp32 vectors.
__device__ __forceinline__ void pb_load_pair(const ProjBwdArgs& a, const float* src, bool rot, int pos, int d0,
                                             f32x4& u, f32x4& w)
{
    if (!src) {
        u = f32x4{0.f, 0.f, 0.f, 0.f};
        w = u;
        return;
    }
    u = *(const f32x4*)(src + d0);
    w = *(const f32x4*)(src + d0 + a.D / 2);
    if (rot) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float sn, cs;
            sincosf(rope_angle(pos, rope_freq(d0 + i, a.D, a.rope_log2_base)), &sn, &cs);
            // the transpose of the forward rotation: turn by minus the angle
            const float uu = u[i], ww = w[i];
            u[i] = uu * cs + ww * sn;
            w[i] = ww * cs - uu * sn;
        }
    }
}

// a gradient row of zeros: the row a token that did not keep a routed expert reads (at most 128 wide)
__device__ __attribute__((aligned(16))) const float pb_zero_row[128] = {};

__device__ __forceinline__ uint64_t pb_pack4(const f32x4& v)
{
    return (uint64_t)pack_bf2(v[0], v[1]) | ((uint64_t)pack_bf2(v[2], v[3]) << 32);
}

// ---------------------------------------------------------------- weights

template <int D>
struct PbDw {
    static constexpr int BN = 256;                    // d_model columns per workgroup
    static constexpr int SR = 64;                     // rows per stage
    static constexpr int PQ = D + 32, PX = BN + 32;   // LDS pitches: transposing reads free of bank conflicts
    static constexpr int MI = D / 32;                 // d blocks (every wave)
    static constexpr int NI = BN / 32 / 4;            // column blocks per wave
    static constexpr int NQ = SR * (D / 8) / 256;     // gradient pairs per thread and stage
    static constexpr int NX = SR * (BN / 8) / 256;    // x chunks per thread and stage
};

template <int D, bool ROT>
__global__ __launch_bounds__(256, D >= 64 ? 2 : 3) void pb_dw_kernel(const ProjBwdArgs a, int nchunk, float* part)
{
    using S = PbDw<D>;
    constexpr int BN = S::BN, SR = S::SR, PQ = S::PQ, PX = S::PX, MI = S::MI, NI = S::NI, NQ = S::NQ, NX = S::NX;
    const int d_model = a.d_model, BT = a.B * a.T;
    const int ncol = (d_model + BN - 1) / BN;
    const int ch = blockIdx.x % nchunk, rest = blockIdx.x / nchunk;
    const int n = rest / ncol, col0 = (rest % ncol) * BN;
    int h;
    const int kind = pb_kind(a, n, h);
    float* dw = kind <= 1 ? a.dw_q : kind == 2 ? a.dw_k : a.dw_v;
    if (!dw) return;
    const int N = a.G * a.E;
    const int Mh = kind == 0 ? a.counts[n] : BT;
    // this chunk's rows [r_lo, r_lo + M) of the head's Mh, in whole stages
    const int per = ((Mh + nchunk - 1) / nchunk + SR - 1) / SR * SR;
    const int r_lo = min(ch * per, Mh);
    const int M = min(per, Mh - r_lo);
    const int base = (kind == 0 ? a.offsets[n] : 0) + r_lo;
    const bool rot = ROT && kind <= 2;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    __shared__ __attribute__((aligned(16))) uint16_t sQ[SR * PQ];
    __shared__ __attribute__((aligned(16))) uint16_t sX[SR * PX];

    f32x4 qu[NQ], qw[NQ];
    u32x4 xr[NX];
    auto load = [&](int r0) {
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
            const int task = tid + 256 * i, rr = task / (D / 8), d0 = (task % (D / 8)) * 4;
            const int r = r0 + rr;
            const float* src = nullptr;
            int pos = 0;
            if (r < M) {
                const int tok = kind == 0 ? a.rows[base + r] : base + r;
                src = pb_src(a, kind, h, n, tok);
                pos = a.positions ? a.positions[tok] : tok % a.T;
            }
            pb_load_pair(a, src, rot, pos, d0, qu[i], qw[i]);
        }
#pragma unroll
        for (int i = 0; i < NX; ++i) {
            const int task = tid + 256 * i, rr = task / (BN / 8);
            const int r = min(r0 + rr, M - 1);
            const int tok = kind == 0 ? a.rows[base + r] : base + r;
            const int c = min(col0 + (task % (BN / 8)) * 8, d_model - 8);
            xr[i] = ld_u32x4(a.x + (size_t)tok * d_model + c);
        }
    };
    auto store = [&]() {
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
            const int task = tid + 256 * i, rr = task / (D / 8), d0 = (task % (D / 8)) * 4;
            *(uint64_t*)&sQ[rr * PQ + d0] = pb_pack4(qu[i]);
            *(uint64_t*)&sQ[rr * PQ + d0 + D / 2] = pb_pack4(qw[i]);
        }
#pragma unroll
        for (int i = 0; i < NX; ++i) {
            const int task = tid + 256 * i, rr = task / (BN / 8), c = (task % (BN / 8)) * 8;
            *(u32x4*)&sX[rr * PX + c] = xr[i];
        }
    };

    f32x16 acc[MI][NI];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[mi][ni][e] = 0.f;

    const int nst = (M + SR - 1) / SR;
    if (nst > 0) load(0);
    for (int st = 0; st < nst; ++st) {
        __syncthreads();
        store();
        __syncthreads();
        if (st + 1 < nst) load((st + 1) * SR);
#pragma unroll
        for (int c = 0; c < SR / 16; ++c) {
            bf16x8 fa[MI], fb[NI];
#pragma unroll
            for (int mi = 0; mi < MI; ++mi) fa[mi] = frag_tr(sQ, PQ, 16 * c, 32 * mi, lane);
#pragma unroll
            for (int ni = 0; ni < NI; ++ni) fb[ni] = frag_tr(sX, PX, 16 * c, 32 * (wave * NI + ni), lane);
#pragma unroll
            for (int mi = 0; mi < MI; ++mi)
#pragma unroll
                for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = mfma32(fa[mi], fb[ni], acc[mi][ni]);
        }
    }

    // one chunk: dW itself; several: this chunk's partial, added by pb_dw_reduce_kernel
    float* dst = nchunk == 1 ? dw + (size_t)(kind == 0 ? n : kind == 1 ? N + h : h) * D * d_model
                             : part + ((size_t)n * nchunk + ch) * D * d_model;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
            const int col = col0 + 32 * (wave * NI + ni) + (lane & 31);
            if (col >= d_model) continue;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int d = 32 * mi + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                dst[(size_t)d * d_model + col] = acc[mi][ni][e];
            }
        }
}

// dW of the dense heads (shared, K, V: every token is a row of each) two at a time: the two heads' gradient
// rows of a stage are staged beside one x tile, so each x fragment read feeds both heads' products and a
// stage moves 2 KB per MFMA instead of 3 KB (the kernel is bound by what its compute unit can load).
// Dense head j (0 <= j < ns + 2 nkv) is head N + j; workgroup pair p takes j = 2p, 2p + 1.
template <int D, bool ROT>
__global__ __launch_bounds__(256, 2) void pb_dw2_kernel(const ProjBwdArgs a, int nchunk, float* part)
{
    using S = PbDw<D>;
    constexpr int BN = S::BN, SR = S::SR, PQ = S::PQ, PX = S::PX, MI = S::MI, NI = S::NI, NQ = S::NQ, NX = S::NX;
    const int d_model = a.d_model, BT = a.B * a.T, N = a.G * a.E, ndense = a.ns + 2 * a.nkv;
    const int ncol = (d_model + BN - 1) / BN;
    const int ch = blockIdx.x % nchunk, rest = blockIdx.x / nchunk;
    const int pr = rest / ncol, col0 = (rest % ncol) * BN;
    const bool two = 2 * pr + 1 < ndense;
    int nh[2], kind[2], hh[2];
    float* dw[2];
    bool rot[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        nh[u] = N + min(2 * pr + u, ndense - 1);
        kind[u] = pb_kind(a, nh[u], hh[u]);
        dw[u] = kind[u] == 1 ? a.dw_q : kind[u] == 2 ? a.dw_k : a.dw_v;
        rot[u] = ROT && kind[u] <= 2;
    }
    if (!dw[0] && (!two || !dw[1])) return;
    const int per = ((BT + nchunk - 1) / nchunk + SR - 1) / SR * SR;
    const int r_lo = min(ch * per, BT);
    const int M = min(per, BT - r_lo);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    __shared__ __attribute__((aligned(16))) uint16_t sQ[2 * SR * PQ];
    __shared__ __attribute__((aligned(16))) uint16_t sX[SR * PX];

    f32x4 qu[2][NQ], qw[2][NQ];
    u32x4 xr[NX];
    auto load = [&](int r0) {
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int i = 0; i < NQ; ++i) {
                const int task = tid + 256 * i, rr = task / (D / 8), d0 = (task % (D / 8)) * 4;
                const int r = r0 + rr;
                const float* src = nullptr;
                int pos = 0;
                if (r < M) {
                    const int tok = r_lo + r;
                    src = pb_src(a, kind[u], hh[u], nh[u], tok);
                    pos = a.positions ? a.positions[tok] : tok % a.T;
                }
                pb_load_pair(a, src, rot[u], pos, d0, qu[u][i], qw[u][i]);
            }
#pragma unroll
        for (int i = 0; i < NX; ++i) {
            const int task = tid + 256 * i, rr = task / (BN / 8);
            const int tok = r_lo + min(r0 + rr, M - 1);
            const int c = min(col0 + (task % (BN / 8)) * 8, d_model - 8);
            xr[i] = ld_u32x4(a.x + (size_t)tok * d_model + c);
        }
    };
    auto store = [&]() {
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int i = 0; i < NQ; ++i) {
                const int task = tid + 256 * i, rr = task / (D / 8), d0 = (task % (D / 8)) * 4;
                *(uint64_t*)&sQ[u * SR * PQ + rr * PQ + d0] = pb_pack4(qu[u][i]);
                *(uint64_t*)&sQ[u * SR * PQ + rr * PQ + d0 + D / 2] = pb_pack4(qw[u][i]);
            }
#pragma unroll
        for (int i = 0; i < NX; ++i) {
            const int task = tid + 256 * i, rr = task / (BN / 8), c = (task % (BN / 8)) * 8;
            *(u32x4*)&sX[rr * PX + c] = xr[i];
        }
    };

    f32x16 acc[2][MI][NI];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
            for (int ni = 0; ni < NI; ++ni)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[u][mi][ni][e] = 0.f;

    const int nst = (M + SR - 1) / SR;
    if (nst > 0) load(0);
    for (int st = 0; st < nst; ++st) {
        __syncthreads();
        store();
        __syncthreads();
        if (st + 1 < nst) load((st + 1) * SR);
#pragma unroll
        for (int c = 0; c < SR / 16; ++c) {
            bf16x8 fb[NI];
#pragma unroll
            for (int ni = 0; ni < NI; ++ni) fb[ni] = frag_tr(sX, PX, 16 * c, 32 * (wave * NI + ni), lane);
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                bf16x8 fa[MI];
#pragma unroll
                for (int mi = 0; mi < MI; ++mi) fa[mi] = frag_tr(sQ + u * SR * PQ, PQ, 16 * c, 32 * mi, lane);
#pragma unroll
                for (int mi = 0; mi < MI; ++mi)
#pragma unroll
                    for (int ni = 0; ni < NI; ++ni) acc[u][mi][ni] = mfma32(fa[mi], fb[ni], acc[u][mi][ni]);
            }
        }
    }

#pragma unroll
    for (int u = 0; u < 2; ++u) {
        if (!dw[u] || (u == 1 && !two)) continue;
        float* dst = nchunk == 1 ? dw[u] + (size_t)(kind[u] == 1 ? N + hh[u] : hh[u]) * D * d_model
                                 : part + ((size_t)nh[u] * nchunk + ch) * D * d_model;
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
            for (int ni = 0; ni < NI; ++ni) {
                const int col = col0 + 32 * (wave * NI + ni) + (lane & 31);
                if (col >= d_model) continue;
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int d = 32 * mi + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                    dst[(size_t)d * d_model + col] = acc[u][mi][ni][e];
                }
            }
    }
}

// dW[head] = the sum of its nchunk partials in chunk order, four columns per thread.
__global__ __launch_bounds__(256) void pb_dw_reduce_kernel(const ProjBwdArgs a, int nchunk, const float* __restrict__ part)
{
    const int D = a.D, d_model = a.d_model, N = a.G * a.E;
    const size_t per_head = (size_t)D * d_model;
    const size_t i4 = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
    const int n_heads = N + a.ns + 2 * a.nkv;
    if (i4 >= per_head * n_heads) return;
    const int n = (int)(i4 / per_head);
    const size_t off = i4 - (size_t)n * per_head;
    int h;
    const int kind = pb_kind(a, n, h);
    float* dw = kind <= 1 ? a.dw_q : kind == 2 ? a.dw_k : a.dw_v;
    if (!dw) return;
    const float* p = part + (size_t)n * nchunk * per_head + off;
    f32x4 s = *(const f32x4*)p;
    for (int c = 1; c < nchunk; ++c) {
        const f32x4 v = *(const f32x4*)(p + (size_t)c * per_head);
        s = f32x4{s[0] + v[0], s[1] + v[1], s[2] + v[2], s[3] + v[3]};
    }
    *(f32x4*)(dw + (size_t)(kind == 0 ? n : kind == 1 ? N + h : h) * per_head + off) = s;
}

// ---------------------------------------------------------------- input

template <int D>
struct PbDx {
    static constexpr int BM = D >= 128 ? 64 : 128;    // tokens per workgroup (registers at d = 128)
    static constexpr int BN = 128;                    // d_model columns per workgroup
    static constexpr int MB = BM / 64;                // 32-token blocks per wave
    static constexpr int PA = D + 8;                  // A tile [token][d], read along d
    static constexpr int PW = BN + 32;                // weight tile [d][col], read across rows
    static constexpr int NA = BM * (D / 8) / 256;     // gradient pairs per thread and head
    static constexpr int NW = D * (BN / 8) / 256;     // weight chunks per thread and head
};

template <int D, bool ROT>
__global__ __launch_bounds__(256, 2) void pb_dx_kernel(const ProjBwdArgs a, int n_heads)
{
    using S = PbDx<D>;
    constexpr int BM = S::BM, BN = S::BN, PA = S::PA, PW = S::PW, NA = S::NA, NW = S::NW, MB = S::MB;
    const int d_model = a.d_model, BT = a.B * a.T, N = a.G * a.E;
    const int ncol = (d_model + BN - 1) / BN;
    const int tok0 = (blockIdx.x / ncol) * BM, col0 = (blockIdx.x % ncol) * BN;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;   // 2 x 2 waves of BM/2 tokens x 64 columns
    __shared__ __attribute__((aligned(16))) uint16_t sA[BM * PA];
    __shared__ __attribute__((aligned(16))) uint16_t sW[D * PW];

    f32x4 au[NA], aw[NA];
    u32x4 wr[NW];
    auto load = [&](int n) {
        int h;
        const int kind = pb_kind(a, n, h);
        const bool rot = ROT && kind <= 2;
#pragma unroll
        for (int i = 0; i < NA; ++i) {
            const int task = tid + 256 * i, m = task / (D / 8), d0 = (task % (D / 8)) * 4;
            const int tok = tok0 + m;
            const float* src = nullptr;
            int pos = 0;
            if (tok < BT) {
                src = pb_src(a, kind, h, n, tok);
                pos = a.positions ? a.positions[tok] : tok % a.T;
            }
            pb_load_pair(a, src, rot, pos, d0, au[i], aw[i]);
        }
        const uint16_t* w = (kind <= 1 ? a.w_q + (size_t)(kind == 0 ? n : N + h) * D * d_model
                                       : (kind == 2 ? a.w_k : a.w_v) + (size_t)h * D * d_model);
#pragma unroll
        for (int i = 0; i < NW; ++i) {
            const int task = tid + 256 * i, d = task / (BN / 8);
            const int c = min(col0 + (task % (BN / 8)) * 8, d_model - 8);
            wr[i] = ld_u32x4(w + (size_t)d * d_model + c);
        }
    };
    auto store = [&]() {
#pragma unroll
        for (int i = 0; i < NA; ++i) {
            const int task = tid + 256 * i, m = task / (D / 8), d0 = (task % (D / 8)) * 4;
            *(uint64_t*)&sA[m * PA + d0] = pb_pack4(au[i]);
            *(uint64_t*)&sA[m * PA + d0 + D / 2] = pb_pack4(aw[i]);
        }
#pragma unroll
        for (int i = 0; i < NW; ++i) {
            const int task = tid + 256 * i, d = task / (BN / 8), c = (task % (BN / 8)) * 8;
            *(u32x4*)&sW[d * PW + c] = wr[i];
        }
    };

    f32x16 acc[MB][2];
#pragma unroll
    for (int mi = 0; mi < MB; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[mi][ni][e] = 0.f;

    load(0);
    for (int n = 0; n < n_heads; ++n) {
        __syncthreads();
        store();
        __syncthreads();
        if (n + 1 < n_heads) load(n + 1);
#pragma unroll
        for (int c = 0; c < D / 16; ++c) {
            bf16x8 fa[MB], fb[2];
#pragma unroll
            for (int mi = 0; mi < MB; ++mi) fa[mi] = frag_perm(sA, PA, (BM / 2) * wm + 32 * mi, 16 * c, lane);
#pragma unroll
            for (int ni = 0; ni < 2; ++ni) fb[ni] = frag_tr(sW, PW, 16 * c, 64 * wn + 32 * ni, lane);
#pragma unroll
            for (int mi = 0; mi < MB; ++mi)
#pragma unroll
                for (int ni = 0; ni < 2; ++ni) acc[mi][ni] = mfma32(fa[mi], fb[ni], acc[mi][ni]);
        }
    }

#pragma unroll
    for (int mi = 0; mi < MB; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) {
            const int col = col0 + 64 * wn + 32 * ni + (lane & 31);
            if (col >= d_model) continue;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int tok = tok0 + (BM / 2) * wm + 32 * mi + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                if (tok < BT) a.dx[(size_t)tok * d_model + col] = acc[mi][ni][e];
            }
        }
}

// dx at d_head 64 with wider tiles: one workgroup of eight waves (two per SIMD) per 256 tokens x 256
// columns, so the fp32 gradient rows are read once per 256 columns (not 128) and each weight tile serves 256
// tokens; one head per stage in two LDS buffers used in turn
// (the next head is stored between the halves of the current one's products, one barrier per head); each
// wave 64 tokens x 128 columns as 2 x 4 blocks, so every fragment read from LDS feeds two or four products;
// dx leaves by buffer stores over the tile's rows.  The same products in the same order per output element
// as pb_dx_kernel.
struct PbDx64 {
    static constexpr int D = 64, BM = 256, BN = 256, NT = 512;
    static constexpr int PA = D + 8, PW = BN + 32;
    static constexpr int STG = BM * PA + D * PW;            // bf16 elements of one stage
    static constexpr int NA = BM * (D / 8) / NT;            // gradient pairs per thread and head
    static constexpr int NW = D * (BN / 8) / NT;            // weight chunks per thread and head
};

template <bool ROT>
__global__ __launch_bounds__(512, 1) void pb_dx64_kernel(const ProjBwdArgs a, int n_heads)
{
    using S = PbDx64;
    constexpr int D = S::D, BM = S::BM, BN = S::BN, NT = S::NT, PA = S::PA, PW = S::PW, STG = S::STG, NA = S::NA,
                  NW = S::NW;
    const int d_model = a.d_model, BT = a.B * a.T, N = a.G * a.E;
    const int ncol = (d_model + BN - 1) / BN, nM = (BT + BM - 1) / BM;
    // workgroup -> tile: the column tiles of a token tile get indices 8 apart, so they run on one XCD and
    // its L2 serves their shared gradient rows
    const int L = blockIdx.x, xcd = L & 7, rr = L >> 3;
    const int tm = (rr / ncol) * 8 + xcd;
    if (tm >= nM) return;
    const int tok0 = tm * BM, col0 = (rr % ncol) * BN;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave & 3, wn = wave >> 2;   // 4 x 2 waves of 64 tokens x 128 columns
    __shared__ __attribute__((aligned(16))) uint16_t sS[2 * STG];
    // the tile's kept experts (G*k <= 16 of them per token), so that a routed head's row lookup reads LDS
    // instead of waiting on a global load before the gradient load it addresses
    constexpr int KMAX = 16;
    __shared__ int8_t s_sel[BM * KMAX];   // expert indices (< 128)
    const int Gk = a.G * a.k;
    const bool staged = Gk <= KMAX;
    if (staged)
        for (int i = tid; i < BM * Gk; i += NT) {
            const int m = i / Gk, tok = min(tok0 + m, BT - 1);
            s_sel[m * KMAX + i % Gk] = a.sel[(size_t)tok * Gk + i % Gk];
        }
    __syncthreads();
    // per load task: its tile row and the parts of its gradient-row offsets that no head changes (tokens past
    // B*T use the last token: their dx rows are never stored), so a head's row address is one multiply-add
    const int T = a.T, G = a.G, k = a.k;
    int tk[NA], pos[NA];
    size_t rbase[NA], kvbase[NA];
#pragma unroll
    for (int i = 0; i < NA; ++i) {
        const int task = tid + NT * i, m = task / (D / 8);
        const int tok = min(tok0 + m, BT - 1), b = tok / T, t = tok - b * T;
        tk[i] = tok;
        rbase[i] = ((size_t)b * G * T + t) * k;      // routed row (b, g, t, j) = rbase + g T k + j
        kvbase[i] = (size_t)b * a.nkv * T + t;       // K/V row (b, h, t) = kvbase + h T
        pos[i] = ROT ? (a.positions ? a.positions[tok] : t) : 0;
    }

    f32x4 au[NA], aw[NA];
    u32x4 wr[NW];
    auto load = [&](int n) {
        int h;
        const int kind = pb_kind(a, n, h);
        const bool rot = ROT && kind <= 2;
        const int g = n / a.E, e = n - g * a.E;
#pragma unroll
        for (int i = 0; i < NA; ++i) {
            const int task = tid + NT * i, m = task / (D / 8), d0 = (task % (D / 8)) * 4;
            const float* src;
            if (kind == 0) {
                // the token's rank of expert e among its kept experts of group g (from LDS when staged); a
                // token that did not keep it reads a row of zeros
                int j = -1;
                if (staged && k == 1) {
                    j = s_sel[m * KMAX + g] == e ? 0 : -1;
                } else if (staged) {
                    for (int r = 0; r < k; ++r) j = s_sel[m * KMAX + g * k + r] == e ? r : j;
                } else {
                    const int32_t* sl = a.sel + ((size_t)tk[i] * G + g) * k;
                    for (int r = 0; r < k; ++r) j = sl[r] == e ? r : j;
                }
                src = j < 0 ? pb_zero_row : a.dq_routed + (rbase[i] + (size_t)g * T * k + j) * D;
            } else if (kind == 1) {
                src = a.dq_shared + (size_t)tk[i] * D;
            } else {
                src = (kind == 2 ? a.dk : a.dv) + (kvbase[i] + (size_t)h * T) * D;
            }
            pb_load_pair(a, src, rot, pos[i], d0, au[i], aw[i]);
        }
        const uint16_t* w = (kind <= 1 ? a.w_q + (size_t)(kind == 0 ? n : N + h) * D * d_model
                                       : (kind == 2 ? a.w_k : a.w_v) + (size_t)h * D * d_model);
#pragma unroll
        for (int i = 0; i < NW; ++i) {
            const int task = tid + NT * i, d = task / (BN / 8);
            const int c = min(col0 + (task % (BN / 8)) * 8, d_model - 8);
            wr[i] = ld_u32x4(w + (size_t)d * d_model + c);
        }
    };
    auto store = [&](uint16_t* buf) {
        uint16_t* sA = buf;
        uint16_t* sW = buf + BM * PA;
#pragma unroll
        for (int i = 0; i < NA; ++i) {
            const int task = tid + NT * i, m = task / (D / 8), d0 = (task % (D / 8)) * 4;
            *(uint64_t*)&sA[m * PA + d0] = pb_pack4(au[i]);
            *(uint64_t*)&sA[m * PA + d0 + D / 2] = pb_pack4(aw[i]);
        }
#pragma unroll
        for (int i = 0; i < NW; ++i) {
            const int task = tid + NT * i, d = task / (BN / 8), c = (task % (BN / 8)) * 8;
            *(u32x4*)&sW[d * PW + c] = wr[i];
        }
    };

    f32x16 acc[2][4];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[mi][ni][e] = 0.f;
    auto mma = [&](const uint16_t* buf, int c) {
        const uint16_t* sA = buf;
        const uint16_t* sW = buf + BM * PA;
        bf16x8 fa[2], fb[4];
#pragma unroll
        for (int mi = 0; mi < 2; ++mi) fa[mi] = frag_perm(sA, PA, 64 * wm + 32 * mi, 16 * c, lane);
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) fb[ni] = frag_tr(sW, PW, 16 * c, 128 * wn + 32 * ni, lane);
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
            for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = mfma32(fa[mi], fb[ni], acc[mi][ni]);
    };

    load(0);
    store(sS);
    if (n_heads > 1) load(1);
    __syncthreads();
    for (int n = 0; n < n_heads; ++n) {
        const uint16_t* cur = sS + (n & 1) * STG;
        mma(cur, 0);
        mma(cur, 1);
        // the next head into the other buffer (its readers passed the last barrier), then its successor's loads
        if (n + 1 < n_heads) {
            store(sS + ((n + 1) & 1) * STG);
            if (n + 2 < n_heads) load(n + 2);
        }
        mma(cur, 2);
        mma(cur, 3);
        __syncthreads();
    }

    // element e of block (mi, ni): token 64 wm + 32 mi + 8 (e / 4) + 4 (lane / 32) + e % 4,
    // column 128 wn + 32 ni + lane % 32; buffer stores over the tile's rows and columns
    const int rows = min(BM, BT - tok0);
    const __amdgpu_buffer_rsrc_t rD = __builtin_amdgcn_make_buffer_rsrc((void*)(a.dx + (size_t)tok0 * d_model), 0,
                                                                         rows * d_model * 4, 0x00020000);
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
            const int col = col0 + 128 * wn + 32 * ni + (lane & 31);
            if (col >= d_model) continue;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int r = 64 * wm + 32 * mi + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[mi][ni][e]), rD, (r * d_model + col) * 4, 0, 0);
            }
        }
}

// Row chunks of the weight gradient: enough workgroups for the chip (about
// four per compute unit), at most 16.
static int pb_nchunk(const ProjBwdArgs& a)
{
    const int n_heads = a.G * a.E + a.ns + 2 * a.nkv;
    const int ncol = (a.d_model + 255) / 256;
    const int want = (1024 + n_heads * ncol - 1) / (n_heads * ncol);
    return want < 1 ? 1 : want > 16 ? 16 : want;
}

size_t proj_bwd_workspace_bytes(const ProjBwdArgs& a)
{
    const int nc = pb_nchunk(a);
    if (nc <= 1) return 0;
    const int n_heads = a.G * a.E + a.ns + 2 * a.nkv;
    return (size_t)n_heads * nc * a.D * a.d_model * sizeof(float);
}

// dW launches: the routed experts (all heads at d_head 128) one per workgroup, then the dense-head pairs
template <int D, bool ROT>
static void pb_dw_launch(const ProjBwdArgs& a, int nc, float* part, unsigned grid1, unsigned grid2, hipStream_t st)
{
    if (grid1) pb_dw_kernel<D, ROT><<<grid1, 256, 0, st>>>(a, nc, part);
    if constexpr (D <= 64) {
        if (grid2) pb_dw2_kernel<D, ROT><<<grid2, 256, 0, st>>>(a, nc, part);
    }
}

int launch_proj_bwd(const ProjBwdArgs& a, void* workspace, size_t workspace_bytes, hipStream_t st)
{
    const int BT = a.B * a.T;
    if (BT == 0) return 0;
    const int n_heads = a.G * a.E + a.ns + 2 * a.nkv;
    // kernels without the rotary code when it is off (inlined per row, it made them several times larger)
    const bool rot = a.rope_log2_base > 0.0;
    if (a.dw_q || a.dw_k || a.dw_v) {
        const size_t need = proj_bwd_workspace_bytes(a);
        const int nc = (need > 0 && workspace && workspace_bytes >= need) ? pb_nchunk(a) : 1;
        float* part = (float*)workspace;
        const int ncol = (a.d_model + 255) / 256;
        // the routed experts one per workgroup (each over its own rows); at d_head <= 64 the dense heads two
        // per workgroup (at 128 the two heads' accumulators would not fit the registers)
        const int N = a.G * a.E, ndense = a.ns + 2 * a.nkv;
        const bool pairs = a.D <= 64;
        const unsigned grid1 = (unsigned)((pairs ? N : n_heads) * ncol * nc);
        const unsigned grid2 = pairs ? (unsigned)(((ndense + 1) / 2) * ncol * nc) : 0u;
        switch (a.D) {
        case 32: rot ? pb_dw_launch<32, true>(a, nc, part, grid1, grid2, st)
                     : pb_dw_launch<32, false>(a, nc, part, grid1, grid2, st); break;
        case 64: rot ? pb_dw_launch<64, true>(a, nc, part, grid1, grid2, st)
                     : pb_dw_launch<64, false>(a, nc, part, grid1, grid2, st); break;
        case 128: rot ? pb_dw_launch<128, true>(a, nc, part, grid1, grid2, st)
                      : pb_dw_launch<128, false>(a, nc, part, grid1, grid2, st); break;
        default: return -2;
        }
        if (nc > 1) {
            const size_t n4 = (size_t)n_heads * a.D * a.d_model / 4;
            pb_dw_reduce_kernel<<<(unsigned)((n4 + 255) / 256), 256, 0, st>>>(a, nc, part);
        }
    }
    if (a.dx && a.D == 64) {
        const int ncol = (a.d_model + PbDx64::BN - 1) / PbDx64::BN, nM = (BT + PbDx64::BM - 1) / PbDx64::BM;
        const unsigned grid = (unsigned)(8 * ((nM + 7) / 8) * ncol);
        rot ? pb_dx64_kernel<true><<<grid, PbDx64::NT, 0, st>>>(a, n_heads)
            : pb_dx64_kernel<false><<<grid, PbDx64::NT, 0, st>>>(a, n_heads);
    } else if (a.dx) {
        const int ncol = (a.d_model + 127) / 128, bm = a.D >= 128 ? 64 : 128;
        const unsigned grid = (unsigned)(((BT + bm - 1) / bm) * ncol);
        switch (a.D) {
        case 32: rot ? pb_dx_kernel<32, true><<<grid, 256, 0, st>>>(a, n_heads)
                     : pb_dx_kernel<32, false><<<grid, 256, 0, st>>>(a, n_heads); break;
        case 64: rot ? pb_dx_kernel<64, true><<<grid, 256, 0, st>>>(a, n_heads)
                     : pb_dx_kernel<64, false><<<grid, 256, 0, st>>>(a, n_heads); break;
        case 128: rot ? pb_dx_kernel<128, true><<<grid, 256, 0, st>>>(a, n_heads)
                      : pb_dx_kernel<128, false><<<grid, 256, 0, st>>>(a, n_heads); break;
        default: return -2;
        }
    }
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace gqe
