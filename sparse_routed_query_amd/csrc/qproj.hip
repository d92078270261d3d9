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
// Workgroups walk (row tile, expert) with the row tile as the major index, so
// workgroups resident at the same time read overlapping token ranges of x.
// Tiles past an expert's row count exit at once: the grid is sized for the
// largest possible bucket, and the counts never leave the device.
#include "gqe_device.h"
#include "gqe_launch.h"

namespace gqe {

constexpr int kQpBM = 128;   // rows per tile (4 waves x 32)
constexpr int kQpBK = 64;    // d_model slice per LDS stage
constexpr int kQpPad = 8;    // bf16 elements of row padding in LDS (16 bytes)

// Destination element offset of row r of expert n's bucket.
__device__ __forceinline__ size_t qp_dst(int n, int N, int tok, const int32_t* __restrict__ sel, int T, int G,
                                         int E, int k, int d_head)
{
    const int b = tok / T, t = tok - b * T;
    if (n == N) return (size_t)tok * d_head;  // shared head [B, T, d_head]
    const int g = n / E, e = n - g * E;
    const int32_t* s = sel + ((size_t)tok * G + g) * k;
    int j = 0;
    for (int i = 0; i < k; ++i) j = s[i] == e ? i : j;
    return ((((size_t)b * G + g) * T + t) * k + j) * d_head;
}

template <int D>
__global__ __launch_bounds__(256) void qproj_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wq, const int32_t* __restrict__ sel,
    const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets, const int32_t* __restrict__ rows,
    uint16_t* __restrict__ q_routed, uint16_t* __restrict__ q_shared, int B, int T, int d_model, int G, int E,
    int k, int n_shared)
{
    const int N = G * E, BT = B * T, n_exp = N + n_shared;
    const int n = blockIdx.x % n_exp;
    const int row0 = (blockIdx.x / n_exp) * kQpBM;
    const int M = n < N ? counts[n] : BT;
    if (row0 >= M) return;
    const int base = n < N ? offsets[n] : 0;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    __shared__ __attribute__((aligned(16))) uint16_t sA[kQpBM][kQpBK + kQpPad];
    __shared__ __attribute__((aligned(16))) uint16_t sB[D][kQpBK + kQpPad];
    __shared__ int s_tok[kQpBM];
    __shared__ size_t s_dst[kQpBM];

    if (tid < kQpBM) {
        const int r = row0 + tid;
        int tok = -1;
        if (r < M) tok = n < N ? rows[base + r] : r;
        s_tok[tid] = tok;
        s_dst[tid] = tok >= 0 ? qp_dst(n, N, tok, sel, T, G, E, k, D) : 0;
    }
    __syncthreads();

    // global -> register staging: A is 128 rows x 64 cols = 1024 16-byte chunks (4 per thread),
    // B is D rows x 64 cols = D*8 chunks.
    constexpr int kAch = kQpBM * kQpBK / 8 / 256;
    constexpr int kBch = D * kQpBK / 8 / 256 > 0 ? D * kQpBK / 8 / 256 : 1;
    const uint16_t* wn = wq + (size_t)n * D * d_model;
    u32x4 ra[kAch], rb[kBch];
    auto load = [&](int k0) {
#pragma unroll
        for (int i = 0; i < kAch; ++i) {
            const int c = tid + i * 256, r = c >> 3, col = (c & 7) * 8;
            const int tok = s_tok[r];
            ra[i] = tok >= 0 ? ld_u32x4(x + (size_t)tok * d_model + k0 + col) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int i = 0; i < kBch; ++i) {
            const int c = tid + i * 256, r = c >> 3, col = (c & 7) * 8;
            if (r < D) rb[i] = ld_u32x4(wn + (size_t)r * d_model + k0 + col);
        }
    };
    auto store = [&]() {
#pragma unroll
        for (int i = 0; i < kAch; ++i) {
            const int c = tid + i * 256, r = c >> 3, col = (c & 7) * 8;
            *(u32x4*)&sA[r][col] = ra[i];
        }
#pragma unroll
        for (int i = 0; i < kBch; ++i) {
            const int c = tid + i * 256, r = c >> 3, col = (c & 7) * 8;
            if (r < D) *(u32x4*)&sB[r][col] = rb[i];
        }
    };

    constexpr int NB = D / 32;
    f32x16 acc[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;

    load(0);
    for (int k0 = 0; k0 < d_model; k0 += kQpBK) {
        __syncthreads();
        store();
        __syncthreads();
        if (k0 + kQpBK < d_model) load(k0 + kQpBK);
#pragma unroll
        for (int kk = 0; kk < kQpBK; kk += 16) {
            const bf16x8 a = ld_bf16x8(&sA[wave * 32 + (lane & 31)][kk + 8 * (lane >> 5)]);
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const bf16x8 b = ld_bf16x8(&sB[j * 32 + (lane & 31)][kk + 8 * (lane >> 5)]);
                acc[j] = mfma32(a, b, acc[j]);
            }
        }
    }

    uint16_t* dst = n < N ? q_routed : q_shared;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int m = wave * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (s_tok[m] < 0) continue;
        const size_t o = s_dst[m];
#pragma unroll
        for (int j = 0; j < NB; ++j) dst[o + j * 32 + (lane & 31)] = __builtin_bit_cast(uint16_t, f2bf(acc[j][r]));
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
        dst[qp_dst(n, N, tok, sel, T, G, E, k, d_head) + d] = s;
    }
}

int launch_qproj(const QprojArgs& a, hipStream_t st)
{
    const int N = a.G * a.E, BT = a.B * a.T, n_exp = N + a.n_shared;
    if (BT == 0) return 0;
    const int tiles = (BT + kQpBM - 1) / kQpBM;
    const int grid = tiles * n_exp;
    if (a.bf16) {
        const uint16_t* x = (const uint16_t*)a.x;
        const uint16_t* w = (const uint16_t*)a.w_q;
        uint16_t* qr = (uint16_t*)a.q_routed;
        uint16_t* qs = (uint16_t*)a.q_shared;
        switch (a.d_head) {
        case 32: qproj_bf16_kernel<32><<<grid, 256, 0, st>>>(x, w, a.sel, a.counts, a.offsets, a.rows, qr, qs, a.B, a.T, a.d_model, a.G, a.E, a.k, a.n_shared); break;
        case 64: qproj_bf16_kernel<64><<<grid, 256, 0, st>>>(x, w, a.sel, a.counts, a.offsets, a.rows, qr, qs, a.B, a.T, a.d_model, a.G, a.E, a.k, a.n_shared); break;
        case 128: qproj_bf16_kernel<128><<<grid, 256, 0, st>>>(x, w, a.sel, a.counts, a.offsets, a.rows, qr, qs, a.B, a.T, a.d_model, a.G, a.E, a.k, a.n_shared); break;
        default: return -2;
        }
    } else {
        qproj_f32_kernel<<<grid, 256, 0, st>>>((const float*)a.x, (const float*)a.w_q, a.sel, a.counts, a.offsets,
                                               a.rows, (float*)a.q_routed, (float*)a.q_shared, a.B, a.T, a.d_model,
                                               a.G, a.E, a.k, a.d_head, a.n_shared);
    }
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace gqe
