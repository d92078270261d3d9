// Routed query projection as a grouped GEMM over the compacted rows, plus the
// always-on shared head (gfx950).
//
// Each kept expert is an independent query projection and unselected experts
// are never computed (ai-feeds summary of arXiv 2606.20945, 方法/核心模块;
// GQE study note §3-2 (2) last sentence, §3-2 (5)).  For expert n the rows
// rows[offsets[n] .. offsets[n+1]) are token ids; the tile computes
// Q = X[rows] W_q[n]^T ([M x d_model] x [d_model x d_head]) with bf16 MFMA
// and fp32 accumulation and scatters each row to its place in the routed
// query layout [B, G, T, k, d_head], where j is the rank of expert e among
// the token's kept experts of group g.  The shared head is expert index N
// with the identity row list.
//
// The bucket sizes stay on the device: every workgroup derives its (expert,
// tile) from the counts (qp_plan below), so the grid is sized by an upper
// bound and the few workgroups past the last tile exit at once.  The order
// keeps the k*G+1 reads of each x row inside one XCD's L2.
#include "gqe_device.h"
#include "gqe_launch.h"

namespace gqe {

constexpr int kQpBM = 128;   // rows per tile of the fp32 kernel
constexpr int kQpPad = 8;    // bf16 elements of row padding in LDS (16 bytes)

// Destination element offset of row r of expert n's bucket.  Experts n >= N
// are dense heads over every token, written as [B, H, T, d_head] with H = the
// number of dense heads (1: the shared head, [B, T, d_head]; H_kv: the K or V
// projection).
__device__ __forceinline__ size_t qp_dst(int n, int N, int n_dense, int tok, const int32_t* __restrict__ sel,
                                         int T, int G, int E, int k, int d_head)
{
    const int b = tok / T, t = tok - b * T;
    if (n >= N) return (((size_t)b * n_dense + (n - N)) * T + t) * d_head;
    const int g = n / E, e = n - g * E;
    const int32_t* s = sel + ((size_t)tok * G + g) * k;
    int j = 0;
    for (int i = 0; i < k; ++i) j = s[i] == e ? i : j;
    return ((((size_t)b * G + g) * T + t) * k + j) * d_head;
}

// Work order.  Expert n has c_n = ceil(M_n / BM) row tiles (M_N = B*T for
// the shared head).  Tiles are ordered in rounds r = 0..R-1, R = max c_n:
// expert n contributes ceil((r+1) c_n / R) - ceil(r c_n / R) tiles to round
// r, so a round covers about the same token range in every expert (buckets
// are sorted by token).  Logical item L then goes to the workgroup with
// blockIdx % 8 == L / chunk: workgroups are dealt round-robin to the eight
// XCDs, so each XCD walks a contiguous range of rounds and its L2 serves the
// k*G+1 reads of every x row.  Computed by one wave from the device-side
// counts; returns false for workgroups past the last item.
__device__ __forceinline__ int qp_before(int c, int r, int R)
{
    // ceil(r * c / R), exact: the quotient is an integer or at least 1/R away from one
    return (int)ceil((double)r * (double)c / (double)R);
}

__device__ __forceinline__ int wave_sum_i(int v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

__device__ __forceinline__ int wave_max_i(int v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o));
    return v;
}

// inclusive prefix sum over the lanes of a wave
__device__ __forceinline__ int wave_scan_i(int v, int lane)
{
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(v, o);
        if (lane >= o) v += t;
    }
    return v;
}

__device__ bool qp_plan(int bid, const int32_t* __restrict__ counts, int N, int n_exp, int BT, bool routed, int BM,
                        int lane, int& n_out, int& tile_out)
{
    auto ntiles = [&](int n) {
        if (n >= n_exp || (n < N && !routed)) return 0;
        const int M = n < N ? counts[n] : BT;
        return (M + BM - 1) / BM;
    };
    const int c0 = ntiles(lane), c1 = ntiles(lane + 64);
    const int U = wave_sum_i(c0 + c1);
    const int R = wave_max_i(max(c0, c1));
    const int chunk = (U + 7) / 8;
    const int L = (bid % 8) * chunk + bid / 8;
    if (bid / 8 >= chunk || L >= U) return false;
    auto S = [&](int r) { return wave_sum_i(qp_before(c0, r, R) + qp_before(c1, r, R)); };
    // S(r) lies in [r U / R, r U / R + n_exp): start from the estimate and walk
    int r = (int)(((long long)L * R) / U);
    while (r > 0 && S(r) > L) --r;
    while (r + 1 < R && S(r + 1) <= L) ++r;
    int rem = L - S(r);
    const int b0 = qp_before(c0, r, R), b1 = qp_before(c1, r, R);
    const int k0 = qp_before(c0, r + 1, R) - b0, k1 = qp_before(c1, r + 1, R) - b1;
    const int p0 = wave_scan_i(k0, lane);
    const int t0 = __shfl(p0, 63);
    int n, tile;
    if (rem < t0) {
        const unsigned long long m = __ballot(p0 > rem);
        const int ln = __ffsll((long long)m) - 1;
        n = ln;
        tile = __shfl(b0, ln) + rem - (__shfl(p0, ln) - __shfl(k0, ln));
    } else {
        rem -= t0;
        const int p1 = wave_scan_i(k1, lane);
        const unsigned long long m = __ballot(p1 > rem);
        const int ln = __ffsll((long long)m) - 1;
        n = ln + 64;
        tile = __shfl(b1, ln) + rem - (__shfl(p1, ln) - __shfl(k1, ln));
    }
    n_out = n;
    tile_out = tile;
    return true;
}

// Threads and rows of a bf16 tile (one 32-row block per wave): at d_head =
// 128 eight waves share a 256-row tile, so each expert's W_q slice is read
// from L2 half as often (6 % faster on the d_head = 128 workload; at d_head
// <= 64 the fewer, larger workgroups were slower).
template <int D>
struct QpNT {
    static constexpr int NT = D >= 128 ? 512 : 256;
    static constexpr int BM = NT / 2;
};
// One workgroup computes a BM-row tile of one expert: Q = X[rows] W_q[n]^T,
// each wave 32 rows.  Per stage of BK columns of d_model the x rows and the
// weight slice are loaded with 16-byte coalesced loads (16 lanes per 256-byte
// row segment) into registers while the previous stage is multiplied out of
// LDS, then stored to LDS between two barriers.  Rows past the bucket's end
// reload its last row and are not stored, so every load is unconditional.
template <int D, int BK>
__global__ __launch_bounds__(QpNT<D>::NT) void qproj_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wq, const int32_t* __restrict__ sel,
    const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets, const int32_t* __restrict__ rows,
    uint16_t* __restrict__ q_routed, uint16_t* __restrict__ q_shared, int B, int T, int d_model, int G, int E,
    int k, int n_shared)
{
    // q_routed == NULL: only the shared head; n_shared == 0: only the routed experts
    constexpr int NT = QpNT<D>::NT, BM = QpNT<D>::BM;
    const int N = G * E, BT = B * T, n_exp = N + n_shared;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    __shared__ int s_item[2];
    if (wave == 0) {
        int pn = -1, pt = 0;
        if (!qp_plan(blockIdx.x, counts, N, n_exp, BT, q_routed != nullptr, BM, lane, pn, pt)) pn = -1;
        if (lane == 0) { s_item[0] = pn; s_item[1] = pt; }
    }
    __syncthreads();
    const int n = s_item[0];
    if (n < 0) return;
    const int row0 = s_item[1] * BM;
    const int M = n < N ? counts[n] : BT;
    const int base = n < N ? offsets[n] : 0;
    constexpr int P = BK + kQpPad;
    constexpr int NB = D / 32;
    constexpr int CPR = BK / 8;                           // 16-byte chunks per row of a stage
    constexpr int ACH = BM * CPR / NT;                    // A chunks per thread
    constexpr int BCH = D * CPR / NT;                     // B chunks per thread
    __shared__ __attribute__((aligned(16))) uint16_t sA[BM * P];
    __shared__ __attribute__((aligned(16))) uint16_t sB[D * P];

    // row pointers of this thread's A chunks (rows tid / CPR + i * 256 / CPR)
    const int col = (tid % CPR) * 8;
    const uint16_t* pa[ACH];
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
        const int rr = min(row0 + tid / CPR + i * (NT / CPR), M - 1);
        const int tok = n < N ? rows[base + rr] : rr;
        pa[i] = x + (size_t)tok * d_model + col;
    }
    const uint16_t* pb = wq + (size_t)n * D * d_model + (size_t)(tid / CPR) * d_model + col;
    u32x4 ra[ACH], rb[BCH];
    auto load = [&](int k0) {
#pragma unroll
        for (int i = 0; i < ACH; ++i) ra[i] = ld_u32x4(pa[i] + k0);
#pragma unroll
        for (int i = 0; i < BCH; ++i) rb[i] = ld_u32x4(pb + (size_t)i * (NT / CPR) * d_model + k0);
    };
    const int w_off = (tid / CPR) * P + col;
    auto store = [&]() {
#pragma unroll
        for (int i = 0; i < ACH; ++i) *(u32x4*)&sA[w_off + i * (NT / CPR) * P] = ra[i];
#pragma unroll
        for (int i = 0; i < BCH; ++i) *(u32x4*)&sB[w_off + i * (NT / CPR) * P] = rb[i];
    };

    f32x16 acc[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;

    const int nst = d_model / BK;
    const int a_off = (wave * 32 + (lane & 31)) * P + 8 * (lane >> 5);
    const int b_off = (lane & 31) * P + 8 * (lane >> 5);
    load(0);
    for (int st = 0; st < nst; ++st) {
        __syncthreads();
        store();
        __syncthreads();
        if (st + 1 < nst) load((st + 1) * BK);
        if constexpr (D >= 128) {
            // all fragments of the stage first, so the reads overlap each other
            // and the MFMAs wait only for their own operands (at d = 64 the
            // extra registers cost a wave per SIMD, which costs more)
            bf16x8 fa[BK / 16], fb[BK / 16][NB];
#pragma unroll
            for (int kk = 0; kk < BK / 16; ++kk) {
                fa[kk] = ld_bf16x8(&sA[a_off + 16 * kk]);
#pragma unroll
                for (int j = 0; j < NB; ++j) fb[kk][j] = ld_bf16x8(&sB[b_off + j * 32 * P + 16 * kk]);
            }
#pragma unroll
            for (int kk = 0; kk < BK / 16; ++kk)
#pragma unroll
                for (int j = 0; j < NB; ++j) acc[j] = mfma32(fa[kk], fb[kk][j], acc[j]);
            __builtin_amdgcn_sched_group_barrier(0x100, (BK / 16) * (NB + 1), 0);   // the LDS reads
            __builtin_amdgcn_sched_group_barrier(0x008, (BK / 16) * NB, 0);         // then the MFMAs
        } else {
#pragma unroll
            for (int kk = 0; kk < BK; kk += 16) {
                const bf16x8 a = ld_bf16x8(&sA[a_off + kk]);
#pragma unroll
                for (int j = 0; j < NB; ++j) acc[j] = mfma32(a, ld_bf16x8(&sB[b_off + j * 32 * P + kk]), acc[j]);
            }
        }
    }

    // destinations of the tile's rows; rows past the bucket are not stored
    __shared__ size_t s_dst[BM];
    const int m = wave * 32 + (lane & 31);
    if (lane < 32) {
        const int r = row0 + m;
        size_t o = ~(size_t)0;
        if (r < M) o = qp_dst(n, N, n_shared, n < N ? rows[base + r] : r, sel, T, G, E, k, D);
        s_dst[m] = o;
    }
    __syncthreads();
    uint16_t* dst = n < N ? q_routed : q_shared;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const int mm = wave * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        const size_t o = s_dst[mm];
        if (o == ~(size_t)0) continue;
#pragma unroll
        for (int j = 0; j < NB; ++j) dst[o + j * 32 + (lane & 31)] = __builtin_bit_cast(uint16_t, f2bf(acc[j][e]));
    }
}

// fp32 projection: one thread per output element, fp32 FMA chain.
__global__ __launch_bounds__(256) void qproj_f32_kernel(
    const float* __restrict__ x, const float* __restrict__ wq, const int32_t* __restrict__ sel,
    const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets, const int32_t* __restrict__ rows,
    float* __restrict__ q_routed, float* __restrict__ q_shared, int B, int T, int d_model, int G, int E, int k,
    int d_head, int n_shared)
{
    const int N = G * E, BT = B * T, n_exp = N + n_shared;
    const int n = blockIdx.x % n_exp;
    if (n < N && !q_routed) return;
    const int row0 = (blockIdx.x / n_exp) * kQpBM;
    const int M = n < N ? counts[n] : BT;
    if (row0 >= M) return;
    const int base = n < N ? offsets[n] : 0;
    const float* wn = wq + (size_t)n * d_head * d_model;
    for (int idx = threadIdx.x; idx < kQpBM * d_head; idx += 256) {
        const int r = row0 + idx / d_head, d = idx % d_head;
        if (r >= M) break;
        const int tok = n < N ? rows[base + r] : r;
        const float* xr = x + (size_t)tok * d_model;
        const float* wr = wn + (size_t)d * d_model;
        float s = 0.f;
        for (int i = 0; i < d_model; ++i) s = fmaf(xr[i], wr[i], s);
        float* dst = n < N ? q_routed : q_shared;
        dst[qp_dst(n, N, n_shared, tok, sel, T, G, E, k, d_head) + d] = s;
    }
}

int launch_qproj(const QprojArgs& a, hipStream_t st)
{
    // a NULL q_shared leaves the shared head out of this call (n_shared = 0 below)
    const int ns = a.q_shared ? a.n_shared : 0;
    const bool routed = a.q_routed != nullptr;
    const int N = a.G * a.E, BT = a.B * a.T, n_exp = N + ns;
    if (BT == 0 || (!routed && ns == 0)) return 0;
    const int tiles = (BT + kQpBM - 1) / kQpBM;
    const int grid = tiles * n_exp;
    // bf16: an upper bound on the number of tiles over all buckets, rounded to the 8 XCDs
    auto grid_bf16_for = [&](int BM) {
        const long long um = (routed ? (long long)BT * a.G * a.k / BM + N : 0) + (long long)ns * ((BT + BM - 1) / BM);
        return (int)(8 * ((um + 7) / 8));
    };
    if (a.bf16) {
        const uint16_t* x = (const uint16_t*)a.x;
        const uint16_t* w = (const uint16_t*)a.w_q;
        uint16_t* qr = (uint16_t*)a.q_routed;
        uint16_t* qs = (uint16_t*)a.q_shared;
#define GQE_QP(D) qproj_bf16_kernel<D, 64><<<grid_bf16_for(QpNT<D>::BM), QpNT<D>::NT, 0, st>>>(x, w, a.sel, a.counts, a.offsets, a.rows, qr, qs, \
                                                                  a.B, a.T, a.d_model, a.G, a.E, a.k, ns)
        switch (a.d_head) {   // d_model is a multiple of the 64-wide stage (checked by the API)
        case 32: GQE_QP(32); break;
        case 64: GQE_QP(64); break;
        case 128: GQE_QP(128); break;
        default: return -2;
        }
#undef GQE_QP
    } else {
        qproj_f32_kernel<<<grid, 256, 0, st>>>((const float*)a.x, (const float*)a.w_q, a.sel, a.counts, a.offsets,
                                               a.rows, (float*)a.q_routed, (float*)a.q_shared, a.B, a.T, a.d_model,
                                               a.G, a.E, a.k, a.d_head, ns);
    }
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

// K and V projections (GQA tutorial, freeguideonline, "GQA 核心原理与计算流程"
// step 2): the same kernel with no routed experts and H_kv dense heads over
// every token, once for K and once for V, written as [B, H_kv, T, d_head].
int launch_kv_proj(const KvProjArgs& a, hipStream_t st)
{
    for (int which = 0; which < 2; ++which) {
        QprojArgs q{};
        q.x = a.x;
        q.w_q = which ? a.w_v : a.w_k;
        q.q_routed = nullptr;
        q.q_shared = which ? a.v : a.k;
        q.B = a.B; q.T = a.T; q.d_model = a.d_model; q.G = 0; q.E = 1; q.k = 1; q.d_head = a.d_head;
        q.n_shared = a.H_kv;
        q.bf16 = a.bf16;
        const int rc = launch_qproj(q, st);
        if (rc) return rc;
    }
    return 0;
}

}  // namespace gqe
