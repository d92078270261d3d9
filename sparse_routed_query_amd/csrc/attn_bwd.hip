// Backward of the routed and shared causal attention (gfx950; bf16 operands,
// fp32 accumulation): gradients of the query rows, K and V given the gradient
// of the hard and shared slots (GQE study note §3-2 (3); GQA tutorial, step 4
// of the GQA computation).
//
// Per head, with S = q K^T / sqrt(d), P = softmax(S) (masked), O = P V:
//   dV = P^T dO,   dP = dO V^T,   dS = P o (dP - Delta),  Delta_r = <dO_r, O_r>,
//   dq = dS K / sqrt(d),   dK = dS^T q / sqrt(d).
// Unless the forward kept its row statistics, the dq kernel first recomputes
// each row's log-sum-exp (base 2); it writes Delta (and the recomputed
// statistic) to the workspace for the dK/dV kernel, then forms dq.  No
// atomics: every output element is written by one workgroup, with its sums in
// a fixed order.
//
// Both kernels: 256 threads = 4 waves, tiles of 64 query rows x 64 keys,
// 32x32x16 bf16 MFMA.  Score tiles are formed transposed (S^T = K q^T), so a
// lane's accumulator column is one query row and the row statistics are one
// value per lane; wave w computes the 32 x 32 quadrant (keys 32 (w & 1),
// rows 32 (w >> 1)).  Operands are read from LDS: a fragment along a tile's
// contiguous axis is one 16-byte read, one across it two transposing reads.
//   attn_bwd_dq_kernel<D>    one 64-row tile of one head (routed or shared)
//   attn_bwd_dkdv_kernel<D>  one 64-key tile of one KV head, over every row
//                            tile that sees it: the group's routed rows and,
//                            for KV head 0, the shared rows
#include "gqe_device.h"
#include "gqe_launch.h"

#include <atomic>

namespace gqe {

namespace {

constexpr int kAbTile = 64;

// MFMA 32x32x16 bf16 fragments, lane l: A row l%32 / B column l%32, with
// k = 8 (l/32) .. +7; accumulator element i: column l%32, row
// 8 (i/4) + 4 (l/32) + i%4.
__device__ __forceinline__ bf16x8 frag_row(const uint16_t* p) { return ld_bf16x8(p); }
__device__ __forceinline__ int acc_row(int i, int lane) { return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3); }

// frag_tr (gqe_device.h) reads fragments across a row-major tile; the A
// operand read by frag_row is stored with the same k swap (kpos).

__device__ __forceinline__ uint16_t bf16_bits(float f) { return __builtin_bit_cast(uint16_t, f2bf(f)); }

// (m, l) of two partial softmax sums over disjoint keys, base 2
__device__ __forceinline__ void ml_merge(float& m, float& l, float m2, float l2)
{
    const float mm = fmaxf(m, m2);
    l = l * __builtin_amdgcn_exp2f(m - mm) + l2 * __builtin_amdgcn_exp2f(m2 - mm);
    m = mm;
}

struct RowSet {
    const uint16_t* q;     // row r at q + r * D
    const float* dO;       // token t's slot at dO + t * dO_stride, then + j * D for row t*kk + j
    const float* O;        // likewise
    long long dO_stride, O_stride;
    float* dq;             // row r at dq + r * D
    float* lse;            // row r's base-2 log-sum-exp at lse[r], Delta at delta[r]
    float* delta;
    int R, kk;
    int kshift;            // log2(kk) when kk is a power of two, else -1
};

__device__ __forceinline__ RowSet row_set(const AttnBwdArgs& a, int b, int h)
{
    const int T = a.T, D = a.d_head, G = a.G, k = a.k, S = a.S, kG = G * k;
    RowSet rs;
    const long long nrouted = (long long)a.B * G * T * k;
    if (h < G) {
        const long long base = ((long long)b * G + h) * T * k;
        rs.q = (const uint16_t*)a.q_routed + base * D;
        rs.dO = a.d_hard + ((size_t)b * T * kG + (size_t)h * k) * D;
        rs.dO_stride = (long long)kG * D;
        rs.O = a.out + ((size_t)b * T * S + (size_t)h * k) * D;
        rs.O_stride = (long long)S * D;
        rs.dq = a.dq_routed + base * D;
        rs.lse = a.lse + base;
        rs.delta = a.delta + base;
        rs.R = T * k;
        rs.kk = k;
        rs.kshift = (k & (k - 1)) == 0 ? __builtin_ctz(k) : -1;
    } else {
        const long long base = (long long)b * T;
        rs.q = (const uint16_t*)a.q_shared + base * D;
        rs.dO = a.dout + ((size_t)b * T * S + (S - 1)) * D;
        rs.dO_stride = (long long)S * D;
        rs.O = a.out + ((size_t)b * T * S + (S - 1)) * D;
        rs.O_stride = (long long)S * D;
        rs.dq = a.dq_shared + base * D;
        rs.lse = a.lse + nrouted + base;
        rs.delta = a.delta + nrouted + base;
        rs.R = T;
        rs.kk = 1;
        rs.kshift = 0;
    }
    return rs;
}

// position t of row r of a row set (r = t kk + j)
__device__ __forceinline__ int row_pos(const RowSet& rs, int r) { return rs.kshift >= 0 ? r >> rs.kshift : r / rs.kk; }

// rows r0 .. r0+63 of a row set into LDS: q (bf16) and dO (rounded to bf16);
// rows past R are zero.  With s_dp, also the partial <dO, O> of each 8-wide chunk.
template <int D>
__device__ __forceinline__ void load_rows(const RowSet& rs, int r0, uint16_t* sQ, uint16_t* sdO, float* s_dp)
{
    constexpr int P = D + 8, CPR = D / 8;
    for (int c = threadIdx.x; c < kAbTile * CPR; c += 256) {
        const int row = c / CPR, d0 = (c % CPR) * 8, r = r0 + row;
        u32x4 qv = {0u, 0u, 0u, 0u}, gv = {0u, 0u, 0u, 0u};
        float dp = 0.f;
        if (r < rs.R) {
            qv = ld_u32x4(rs.q + (size_t)r * D + d0);
            const int t = r / rs.kk, j = r - t * rs.kk;
            const float* g = rs.dO + (size_t)t * rs.dO_stride + (size_t)j * D + d0;
            const f32x4 g0 = *(const f32x4*)g, g1 = *(const f32x4*)(g + 4);
            gv = u32x4{pack_bf2(g0[0], g0[1]), pack_bf2(g0[2], g0[3]), pack_bf2(g1[0], g1[1]), pack_bf2(g1[2], g1[3])};
            if (s_dp) {
                const float* o = rs.O + (size_t)t * rs.O_stride + (size_t)j * D + d0;
                const f32x4 o0 = *(const f32x4*)o, o1 = *(const f32x4*)(o + 4);
#pragma unroll
                for (int e = 0; e < 4; ++e) dp = fmaf(g0[e], o0[e], dp);
#pragma unroll
                for (int e = 0; e < 4; ++e) dp = fmaf(g1[e], o1[e], dp);
            }
        }
        *(u32x4*)(sQ + row * P + d0) = qv;
        *(u32x4*)(sdO + row * P + d0) = gv;
        if (s_dp) s_dp[row * CPR + c % CPR] = dp;
    }
}

// keys s0 .. s0+63 of one head into LDS (bf16); keys past T are zero
template <int D>
__device__ __forceinline__ void load_keys(const uint16_t* src, int s0, int T, uint16_t* dst)
{
    constexpr int P = D + 8, CPR = D / 8;
    for (int c = threadIdx.x; c < kAbTile * CPR; c += 256) {
        const int row = c / CPR, d0 = (c % CPR) * 8, s = s0 + row;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (s < T) v = ld_u32x4(src + (size_t)s * D + d0);
        *(u32x4*)(dst + row * P + d0) = v;
    }
}

// Register stages: the next tile's global loads are issued before the
// current tile's products, and stored to LDS after them, so the loads' latency
// is hidden by the math.  Thread tid moves 16-byte chunks tid + 256 i.
template <int D>
struct KeyRegs {
    static constexpr int N = kAbTile * D / 8 / 256;
    u32x4 v[N];
};
template <int D>
__device__ __forceinline__ void keys_load(const uint16_t* src, int s0, int T, KeyRegs<D>& r)
{
    constexpr int CPR = D / 8;
#pragma unroll
    for (int i = 0; i < KeyRegs<D>::N; ++i) {
        const int c = threadIdx.x + 256 * i, row = c / CPR, d0 = (c % CPR) * 8, s = s0 + row;
        r.v[i] = s < T ? ld_u32x4(src + (size_t)s * D + d0) : u32x4{0u, 0u, 0u, 0u};
    }
}
template <int D>
__device__ __forceinline__ void keys_store(const KeyRegs<D>& r, uint16_t* dst)
{
    constexpr int P = D + 8, CPR = D / 8;
#pragma unroll
    for (int i = 0; i < KeyRegs<D>::N; ++i) {
        const int c = threadIdx.x + 256 * i;
        *(u32x4*)(dst + (c / CPR) * P + (c % CPR) * 8) = r.v[i];
    }
}
// a row tile's q (bf16), dO (fp32, rounded to bf16 when stored), log-sum-exp and Delta
template <int D>
struct RowRegs {
    static constexpr int N = kAbTile * D / 8 / 256;
    u32x4 q[N];
    f32x4 g[2 * N];
    float lse, delta;
};
template <int D>
__device__ __forceinline__ void rows_load(const RowSet& rs, int r0, RowRegs<D>& r)
{
    constexpr int CPR = D / 8;
#pragma unroll
    for (int i = 0; i < RowRegs<D>::N; ++i) {
        // rows past R read row R - 1: their log-sum-exp is +inf (below), so their P and dS are 0 and they add
        // nothing, and every load is unconditional
        const int c = threadIdx.x + 256 * i, row = c / CPR, d0 = (c % CPR) * 8, rr = min(r0 + row, rs.R - 1);
        r.q[i] = ld_u32x4(rs.q + (size_t)rr * D + d0);
        const int t = row_pos(rs, rr), j = rr - t * rs.kk;
        const float* g = rs.dO + (size_t)t * rs.dO_stride + (size_t)j * D + d0;
        r.g[2 * i] = *(const f32x4*)g;
        r.g[2 * i + 1] = *(const f32x4*)(g + 4);
    }
    const int rr = r0 + (int)threadIdx.x;
    r.lse = INFINITY;   // (rows past R weigh nothing)
    r.delta = 0.f;
    if (threadIdx.x < kAbTile && rr < rs.R) {
        r.lse = rs.lse[rr];
        r.delta = rs.delta[rr];
    }
}
template <int D>
__device__ __forceinline__ void rows_store(const RowRegs<D>& r, uint16_t* sQ, uint16_t* sdO, float* s_lse,
                                           float* s_delta)
{
    constexpr int P = D + 8, CPR = D / 8;
#pragma unroll
    for (int i = 0; i < RowRegs<D>::N; ++i) {
        const int c = threadIdx.x + 256 * i, off = (c / CPR) * P + (c % CPR) * 8;
        const f32x4 g0 = r.g[2 * i], g1 = r.g[2 * i + 1];
        *(u32x4*)(sQ + off) = r.q[i];
        *(u32x4*)(sdO + off) =
            u32x4{pack_bf2(g0[0], g0[1]), pack_bf2(g0[2], g0[3]), pack_bf2(g1[0], g1[1]), pack_bf2(g1[2], g1[3])};
    }
    if (threadIdx.x < kAbTile) {
        s_lse[threadIdx.x] = r.lse;
        s_delta[threadIdx.x] = r.delta;
    }
}

// 32 x 32 quadrant of X Y^T over d: X rows x0.., Y rows y0.. (both [64][P] bf16 tiles)
template <int D>
__device__ __forceinline__ f32x16 quad_xyT(const uint16_t* X, int x0, const uint16_t* Y, int y0, int lane)
{
    constexpr int P = D + 8;
    f32x16 c;
#pragma unroll
    for (int r = 0; r < 16; ++r) c[r] = 0.f;
    const uint16_t* xa = X + (x0 + (lane & 31)) * P + 8 * (lane >> 5);
    const uint16_t* yb = Y + (y0 + (lane & 31)) * P + 8 * (lane >> 5);
#pragma unroll
    for (int s = 0; s < D / 16; ++s) c = mfma32(frag_row(xa + 16 * s), frag_row(yb + 16 * s), c);
    return c;
}

// C[m][n] += sum over 64 k of A[m][k] Z[k][n]: A a [64][64+8] tile (row m0 + l%32)
// holding k at position kpos(k), Z a row-major [64][D+8] tile read across (columns n0 + l%32)
template <int D>
__device__ __forceinline__ f32x16 gemm_az(f32x16 c, const uint16_t* A, int m0, const uint16_t* Z, int n0, int lane)
{
    constexpr int P = D + 8, PS = kAbTile + 8;
    const uint16_t* aa = A + (m0 + (lane & 31)) * PS + 8 * (lane >> 5);
#pragma unroll
    for (int s = 0; s < kAbTile / 16; ++s) c = mfma32(frag_row(aa + 16 * s), frag_tr(Z, P, 16 * s, n0, lane), c);
    return c;
}

// C[m][n] += sum over the 64 rows k of A[k][m] Z[k][n]: A a row-major [64][64+8] tile and Z a row-major
// [64][D+8] tile, both read across (columns m0 + l%32 and n0 + l%32) in frag_tr's k order
template <int D>
__device__ __forceinline__ f32x16 gemm_tt(f32x16 c, const uint16_t* A, int m0, const uint16_t* Z, int n0, int lane)
{
    constexpr int P = D + 8, PS = kAbTile + 8;
#pragma unroll
    for (int s = 0; s < kAbTile / 16; ++s) c = mfma32(frag_tr(A, PS, 16 * s, m0, lane), frag_tr(Z, P, 16 * s, n0, lane), c);
    return c;
}

template <int D>
constexpr int ab_lds_bytes(bool dq)
{
    // dK/dV kernel: q, dO, V tiles, then P and dS (where the K tile is staged once before it is held in
    // registers), then row data.  dq kernel: dO, K, V tiles, then dS, then row data (q is staged once, in
    // the dS region or at d_head 128 the K region, before it is held in registers).
    return 3 * kAbTile * (D + 8) * 2 + (dq ? 1 : 2) * kAbTile * (kAbTile + 8) * 2 + 2 * kAbTile * 4;
}

}  // namespace

// The query tile's fragments are held in registers (each wave's 32 rows, read once); with the scratch of
// the prologue and of pass 1's end kept in regions free at those times, the kernel needs 37 KB of LDS at
// d_head 64 (four workgroups per compute unit) and 62 KB at 128 (two).
template <int D>
__global__ __launch_bounds__(256, D <= 64 ? 4 : 2) void attn_bwd_dq_kernel(const AttnBwdArgs a)
{
    constexpr int P = D + 8, PS = kAbTile + 8, CPR = D / 8, NBW = (2 * (D / 32) + 3) / 4;
    constexpr bool QS = kAbTile * P <= kAbTile * PS;   // q staged in the dS region, else in the K region
    extern __shared__ __attribute__((aligned(16))) uint16_t s_ab[];
    uint16_t* sdO = s_ab;
    uint16_t* sK = sdO + kAbTile * P;
    uint16_t* sV = sK + kAbTile * P;
    uint16_t* sS = sV + kAbTile * P;
    uint16_t* sQ = QS ? sS : sK;                                // staging, read once before K and dS are written
    float* s_dp = (float*)(QS ? sK : sV);                       // prologue only, before K and V are stored
    float* s_m = (float*)sS;                                    // [4][32], end of pass 1 only
    float* s_l = s_m + 4 * 32;                                  // [4][32]
    float* s_lse = (float*)(sS + kAbTile * PS);                 // [64]
    float* s_delta = s_lse + kAbTile;                           // [64]
    static_assert(kAbTile * CPR * 4 <= kAbTile * P * 2 && 2 * 4 * 32 * 4 <= kAbTile * PS * 2,
                  "aliased regions fit");

    const int T = a.T, G = a.G;
    const int ntr = (T * a.k + kAbTile - 1) / kAbTile, nts = (T + kAbTile - 1) / kAbTile;
    long long it = blockIdx.x;
    int b, h, tile;
    if (it < (long long)a.B * G * ntr) {
        b = (int)(it / ((long long)G * ntr));
        const int rem = (int)(it - (long long)b * G * ntr);
        h = rem / ntr;
        tile = ntr - 1 - rem % ntr;   // longest first
    } else {
        it -= (long long)a.B * G * ntr;
        b = (int)(it / nts);
        h = G;
        tile = nts - 1 - (int)(it % nts);
    }
    const RowSet rs = row_set(a, b, h);
    const int kvh = h < G ? h : 0;
    const uint16_t* Kh = (const uint16_t*)a.k_ + ((size_t)b * G + kvh) * T * D;
    const uint16_t* Vh = (const uint16_t*)a.v_ + ((size_t)b * G + kvh) * T * D;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wk = wave & 1, wr = wave >> 1;
    const int r0 = tile * kAbTile;
    const int last = min(rs.R - 1, r0 + kAbTile - 1);
    const int nkt = a.causal ? (last / rs.kk) / kAbTile + 1 : (T + kAbTile - 1) / kAbTile;
    const int row = wr * 32 + (lane & 31);          // this lane's query row in the tile
    const int rg = r0 + row;
    const int tq = rg / rs.kk;
    const float qs2 = a.qscale2;

    KeyRegs<D> rk, rv;
    keys_load<D>(Kh, 0, T, rk);
    if (a.lse_given) keys_load<D>(Vh, 0, T, rv);
    load_rows<D>(rs, r0, sQ, sdO, s_dp);
    __syncthreads();
    if (tid < kAbTile) {
        float dsum = 0.f;
        for (int c = 0; c < CPR; ++c) dsum += s_dp[tid * CPR + c];
        s_delta[tid] = dsum;
    }
    // this wave's query fragments (rows wr * 32 + l % 32), read before K, V and dS overwrite the staging
    bf16x8 qf[D / 16];
    {
        const uint16_t* yb = sQ + (wr * 32 + (lane & 31)) * P + 8 * (lane >> 5);
#pragma unroll
        for (int st = 0; st < D / 16; ++st) qf[st] = frag_row(yb + 16 * st);
    }
    __syncthreads();
    // S^T quadrant of this wave (keys wk * 32 .., rows wr * 32 ..) against the K tile in LDS
    auto scores = [&]() -> f32x16 {
        f32x16 c;
#pragma unroll
        for (int r = 0; r < 16; ++r) c[r] = 0.f;
        const uint16_t* xa = sK + (wk * 32 + (lane & 31)) * P + 8 * (lane >> 5);
#pragma unroll
        for (int st = 0; st < D / 16; ++st) c = mfma32(frag_row(xa + 16 * st), qf[st], c);
        return c;
    };
    keys_store<D>(rk, sK);
    if (a.lse_given) keys_store<D>(rv, sV);
    __syncthreads();

    if (a.lse_given) {
        // the forward's log-sum-exp of each row; only Delta goes to the workspace
        if (tid < kAbTile) {
            const int r = r0 + tid;
            s_lse[tid] = r < rs.R ? rs.lse[r] : INFINITY;   // (rows past R weigh nothing)
            if (r < rs.R) rs.delta[r] = s_delta[tid];
        }
        __syncthreads();
    } else {
    // pass 1: the rows' base-2 log-sum-exp.  Its last step fetches pass 2's first K and V tiles.
    float m = -1e30f, l = 0.f;
    for (int kt = 0; kt < nkt; ++kt) {
        const int s0 = kt * kAbTile;
        const bool more = kt + 1 < nkt;
        keys_load<D>(Kh, more ? s0 + kAbTile : 0, T, rk);
        if (!more) keys_load<D>(Vh, 0, T, rv);
        const f32x16 c = scores();
        float sv[16], mt = -INFINITY;
        if (s0 + kAbTile > T || (a.causal && s0 + kAbTile - 1 > r0 / rs.kk)) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int key = s0 + wk * 32 + acc_row(i, lane);
                const bool ok = key < T && (!a.causal || key <= tq);
                sv[i] = ok ? c[i] * qs2 : -INFINITY;
                mt = fmaxf(mt, sv[i]);
            }
        } else {   // every key of the tile is inside T and before the tile's first row's position
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                sv[i] = c[i] * qs2;
                mt = fmaxf(mt, sv[i]);
            }
        }
        const float mn = fmaxf(m, mt);
        float ls = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) ls += __builtin_amdgcn_exp2f(sv[i] - mn);
        l = l * __builtin_amdgcn_exp2f(m - mn) + ls;
        m = mn;
        __syncthreads();
        keys_store<D>(rk, sK);
        if (!more) keys_store<D>(rv, sV);
        __syncthreads();
    }
    {
        // lanes l and l^32 hold the same row over different keys; then the two key halves (waves)
        const float m2 = __shfl_xor(m, 32), l2 = __shfl_xor(l, 32);
        if (lane < 32) ml_merge(m, l, m2, l2);
        if (lane < 32) {
            s_m[wave * 32 + lane] = m;
            s_l[wave * 32 + lane] = l;
        }
        __syncthreads();
        if (wk == 0 && lane < 32) {
            float mf = s_m[(wr * 2) * 32 + lane], lf = s_l[(wr * 2) * 32 + lane];
            ml_merge(mf, lf, s_m[(wr * 2 + 1) * 32 + lane], s_l[(wr * 2 + 1) * 32 + lane]);
            const float lse = rg < rs.R ? mf + __log2f(lf) : INFINITY;   // (rows past R weigh nothing)
            s_lse[row] = lse;
            if (rg < rs.R) {
                rs.lse[rg] = lse;
                rs.delta[rg] = s_delta[row];
            }
        }
        __syncthreads();
    }
    }

    // pass 2: dq = dS K / sqrt(d)
    const float lse_r = s_lse[row], dl_r = s_delta[row];
    f32x16 acc[NBW];
#pragma unroll
    for (int j = 0; j < NBW; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
    for (int kt = 0; kt < nkt; ++kt) {
        const int s0 = kt * kAbTile;
        const bool more = kt + 1 < nkt;
        if (more) {
            keys_load<D>(Kh, s0 + kAbTile, T, rk);
            keys_load<D>(Vh, s0 + kAbTile, T, rv);
        }
        const f32x16 c = scores();
        const f32x16 dp = quad_xyT<D>(sV, wk * 32, sdO, wr * 32, lane);
        // dS[row][key] as bf16, four consecutive keys per 8-byte store; the mask (a select after an
        // unconditional exp2) only on tiles that reach past T or the row's position
        auto d_s = [&](bool masked) {
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i = 4 * i4 + e;
                    float pv = __builtin_amdgcn_exp2f(c[i] * qs2 - lse_r);
                    if (masked) {
                        const int key = s0 + wk * 32 + acc_row(i, lane);
                        pv = key < T && (!a.causal || key <= tq) ? pv : 0.f;
                    }
                    v[e] = pv * (dp[i] - dl_r);
                }
                const int k0 = wk * 32 + acc_row(4 * i4, lane);   // (kpos moves whole 4-key blocks)
                *(uint2*)(sS + row * PS + kpos(k0)) = make_uint2(pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3]));
            }
        };
        if (s0 + kAbTile > T || (a.causal && s0 + kAbTile - 1 > row_pos(rs, r0)))
            d_s(true);
        else
            d_s(false);
        __syncthreads();
#pragma unroll
        for (int j = 0; j < NBW; ++j) {
            const int blk = wave + 4 * j;
            if (blk < 2 * (D / 32)) acc[j] = gemm_az<D>(acc[j], sS, (blk & 1) * 32, sK, (blk >> 1) * 32, lane);
        }
        __syncthreads();
        if (more) {
            keys_store<D>(rk, sK);
            keys_store<D>(rv, sV);
            __syncthreads();
        }
    }
#pragma unroll
    for (int j = 0; j < NBW; ++j) {
        const int blk = wave + 4 * j;
        if (blk >= 2 * (D / 32)) continue;
        const int d = (blk >> 1) * 32 + (lane & 31);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int r = r0 + (blk & 1) * 32 + acc_row(i, lane);
            if (r < rs.R) rs.dq[(size_t)r * D + d] = acc[j][i] * a.inv_sqrt_d;
        }
    }
}

// Three workgroups per compute unit (two at d_head 128): the key tile is fixed per workgroup, so each wave
// keeps its 32 keys' K fragments in registers and K needs no LDS of its own.
template <int D>
__global__ __launch_bounds__(256, D >= 128 ? 2 : 3) void attn_bwd_dkdv_kernel(const AttnBwdArgs a)
{
    constexpr int P = D + 8, PS = kAbTile + 8, NB = D / 32;
    extern __shared__ __attribute__((aligned(16))) uint16_t s_ab[];
    uint16_t* sQ = s_ab;
    uint16_t* sdO = sQ + kAbTile * P;
    uint16_t* sV = sdO + kAbTile * P;
    uint16_t* sP = sV + kAbTile * P;          // P [row][key]; before the loop, the K tile
    uint16_t* sD = sP + kAbTile * PS;         // dS [row][key]
    float* s_lse = (float*)(sD + kAbTile * PS);
    float* s_delta = s_lse + kAbTile;
    static_assert(kAbTile * P <= 2 * kAbTile * PS, "the K tile is staged in the P and dS region");

    const int T = a.T, G = a.G;
    const int nkt = (T + kAbTile - 1) / kAbTile;
    const int kt = (int)(blockIdx.x % nkt);           // ascending: the longest first
    const int g = (int)((blockIdx.x / nkt) % G);
    const int b = (int)(blockIdx.x / ((long long)nkt * G));
    const int s0 = kt * kAbTile;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wk = wave & 1, wr = wave >> 1;
    const int row = wr * 32 + (lane & 31);

    load_keys<D>((const uint16_t*)a.k_ + ((size_t)b * G + g) * T * D, s0, T, sP);
    load_keys<D>((const uint16_t*)a.v_ + ((size_t)b * G + g) * T * D, s0, T, sV);

    // products: waves 0, 1 form dV, waves 2, 3 dK, each for keys 32 (wave & 1) .. and every d, so each
    // P^T or dS^T fragment read from LDS feeds all D / 32 blocks
    const bool is_dk = wave >= 2;
    f32x16 acc[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;

    // the row tiles that see this key tile: the group's routed rows, then (KV head 0) the shared rows
    const RowSet rs0 = row_set(a, b, g);
    const bool two = g == 0 && a.n_shared;
    const RowSet rs1 = two ? row_set(a, b, G) : rs0;
    const int n0 = (rs0.R + kAbTile - 1) / kAbTile, n1 = (rs1.R + kAbTile - 1) / kAbTile;
    const int a0 = a.causal ? (int)(((long long)s0 * rs0.kk) / kAbTile) : 0;
    const int a1 = a.causal ? (int)(((long long)s0 * rs1.kk) / kAbTile) : 0;
    const int c0 = n0 - a0, nit = c0 + (two ? n1 - a1 : 0);
    RowRegs<D> rr;
    if (nit > 0) rows_load<D>(rs0, a0 * kAbTile, rr);
    __syncthreads();
    // this wave's K fragments (keys wk * 32 + l % 32), read once; the region then holds P and dS
    bf16x8 kf[D / 16];
    {
        const uint16_t* xa = sP + (wk * 32 + (lane & 31)) * P + 8 * (lane >> 5);
#pragma unroll
        for (int st = 0; st < D / 16; ++st) kf[st] = frag_row(xa + 16 * st);
    }
    if (nit > 0) rows_store<D>(rr, sQ, sdO, s_lse, s_delta);
    __syncthreads();
    for (int it = 0; it < nit; ++it) {
        const bool in0 = it < c0;
        const RowSet& rs = in0 ? rs0 : rs1;
        const int r0 = (in0 ? a0 + it : a1 + it - c0) * kAbTile;
        const bool more = it + 1 < nit;
        if (more) {
            const bool nx0 = it + 1 < c0;
            rows_load<D>(nx0 ? rs0 : rs1, (nx0 ? a0 + it + 1 : a1 + it + 1 - c0) * kAbTile, rr);
        }
        const int tq = row_pos(rs, r0 + row);
        const float lse_r = s_lse[row], dl_r = s_delta[row];
        f32x16 c;
        {
            const uint16_t* yb = sQ + (wr * 32 + (lane & 31)) * P + 8 * (lane >> 5);
#pragma unroll
            for (int r = 0; r < 16; ++r) c[r] = 0.f;
#pragma unroll
            for (int st = 0; st < D / 16; ++st) c = mfma32(kf[st], frag_row(yb + 16 * st), c);
        }
        const f32x16 dp = quad_xyT<D>(sV, wk * 32, sdO, wr * 32, lane);
        // P and dS as bf16 in [row][key] order, four consecutive keys per 8-byte store; a tile whose keys all
        // lie inside T and before its first row's position needs no mask (the mask is a select, not a branch)
        auto p_ds = [&](bool masked) {
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                float pv[4], ds[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i = 4 * i4 + e;
                    const float ex = __builtin_amdgcn_exp2f(c[i] * a.qscale2 - lse_r);
                    if (masked) {
                        const int key = s0 + wk * 32 + acc_row(i, lane);
                        pv[e] = key < T && (!a.causal || key <= tq) ? ex : 0.f;
                    } else {
                        pv[e] = ex;
                    }
                    ds[e] = pv[e] * (dp[i] - dl_r);
                }
                const int off = row * PS + wk * 32 + acc_row(4 * i4, lane);
                *(uint2*)(sP + off) = make_uint2(pack_bf2(pv[0], pv[1]), pack_bf2(pv[2], pv[3]));
                *(uint2*)(sD + off) = make_uint2(pack_bf2(ds[0], ds[1]), pack_bf2(ds[2], ds[3]));
            }
        };
        if (s0 + kAbTile > T || (a.causal && s0 + kAbTile - 1 > row_pos(rs, r0)))
            p_ds(true);
        else
            p_ds(false);
        __syncthreads();
        {
            const uint16_t* src = is_dk ? sD : sP;   // dS^T q or P^T dO
            const uint16_t* z = is_dk ? sQ : sdO;
#pragma unroll
            for (int st = 0; st < kAbTile / 16; ++st) {
                const bf16x8 fa = frag_tr(src, PS, 16 * st, wk * 32, lane);
#pragma unroll
                for (int j = 0; j < NB; ++j) acc[j] = mfma32(fa, frag_tr(z, P, 16 * st, 32 * j, lane), acc[j]);
            }
        }
        __syncthreads();
        if (more) {
            rows_store<D>(rr, sQ, sdO, s_lse, s_delta);
            __syncthreads();
        }
    }
    float* dst = (is_dk ? a.dk : a.dv) + ((size_t)b * G + g) * T * D;
    const float scale = is_dk ? a.inv_sqrt_d : 1.f;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
        const int d = 32 * j + (lane & 31);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int key = s0 + wk * 32 + acc_row(i, lane);
            if (key < T) dst[(size_t)key * D + d] = acc[j][i] * scale;
        }
    }
}

size_t attn_bwd_workspace_bytes(int B, int T, int G, int k, int n_shared)
{
    const long long rows = (long long)B * G * T * k + (n_shared ? (long long)B * T : 0);
    return (size_t)rows * 2 * sizeof(float) + 256;
}

template <int D>
static int launch_attn_bwd_d(AttnBwdArgs a, hipStream_t st)
{
    const int ntr = (a.T * a.k + kAbTile - 1) / kAbTile, nts = (a.T + kAbTile - 1) / kAbTile;
    const long long nq = (long long)a.B * a.G * ntr + (a.n_shared ? (long long)a.B * nts : 0);
    const long long nkv = (long long)a.B * a.G * nts;
    const int lq = ab_lds_bytes<D>(true), lkv = ab_lds_bytes<D>(false);
    // LDS limits raised once per kernel (their sizes are fixed per d_head)
    static std::atomic<int> raised{0};
    if (!raised.load(std::memory_order_acquire)) {
        if (lq > 65536 && hipFuncSetAttribute((const void*)&attn_bwd_dq_kernel<D>,
                                              hipFuncAttributeMaxDynamicSharedMemorySize, lq) != hipSuccess)
            return -1;
        if (lkv > 65536 && hipFuncSetAttribute((const void*)&attn_bwd_dkdv_kernel<D>,
                                               hipFuncAttributeMaxDynamicSharedMemorySize, lkv) != hipSuccess)
            return -1;
        raised.store(1, std::memory_order_release);
    }
    attn_bwd_dq_kernel<D><<<(unsigned)nq, 256, lq, st>>>(a);
    attn_bwd_dkdv_kernel<D><<<(unsigned)nkv, 256, lkv, st>>>(a);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_attn_bwd(const AttnBwdArgs& a, hipStream_t st)
{
    if (a.B == 0 || a.T == 0) return 0;
    switch (a.d_head) {
    case 32: return launch_attn_bwd_d<32>(a, st);
    case 64: return launch_attn_bwd_d<64>(a, st);
    case 128: return launch_attn_bwd_d<128>(a, st);
    default: return -2;
    }
}

}  // namespace gqe
