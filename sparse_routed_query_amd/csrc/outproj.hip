// Attention output projection fused with slot assembly (gfx950).
//
// The head outputs of a token are concatenated and passed through one final
// linear map (GQA tutorial, freeguideonline, "GQA 核心原理与计算流程" step 5);
// in GQE that concatenation is the kG+2 slots -- hard slots, weighted slot,
// shared slot -- so the map W_o is S*d_head wide (GQE study note §3-2 (5),
// (7)).  Here y_t = W_o h_t, with W_o [d_model, S*d_head] row-major and no
// bias.
//
// The weighted slot(s) are not read from memory: they are summed from the
// hard slots while those stream through the kernel, in the same fixed order
// and fp32 arithmetic as gqe_assemble (so the values it can write back are
// the same bits).
//
// bf16 kernel: a GEMM of M = B*T tokens, N = d_model, K = S*d_head, one
// workgroup per BM x 128 tile of y (BM = 128 tokens, 64 at d_head = 128),
// four waves in a 2 x 2 grid, each holding (BM/64) x 2 blocks of 32x32x16 bf16
// MFMA with fp32 accumulation.  The K loop takes one slot per stage: the
// slot's fp32 values of the tile's tokens are loaded into registers, rounded
// to bf16 and stored to LDS next to the matching W_o columns, while the
// previous stage is multiplied.  The column tiles of a token tile run on one
// XCD, so the slots come from memory once and from that XCD's L2 after that.
#include "gqe_device.h"
#include "gqe_launch.h"

namespace gqe {

constexpr int kOpBN = 128;   // output features per tile
constexpr int kOpPad = 8;    // bf16 elements of LDS row padding (16 bytes)

// Tile shape per d_head: BM tokens, TPR threads per token, each holding AV
// fp32 values of a slot row and of the weighted sum (at d_head = 128 two
// threads per token would need 128 such registers and spill).
template <int D>
struct OpTile {
    static constexpr int BM = D >= 128 ? 64 : 128;
    static constexpr int TPR = 256 / BM;
    static constexpr int AV = D / TPR;
    static constexpr int RB = BM / 64;   // 32-row blocks per wave
};

// Slot read at K stage i (0 <= i < S).  Mode 0: slot order (hard, weighted,
// shared).  Mode 1: each group's hard slots, then that group's weighted slot,
// so the weighted sum is complete when its stage comes; the shared slot last.
__device__ __forceinline__ int op_slot(int i, int G, int k, int mode)
{
    if (mode == 0) return i;
    const int kG = G * k;
    if (i >= (k + 1) * G) return i;   // the shared slot, S - 1
    const int g = i / (k + 1), r = i - g * (k + 1);
    return r < k ? g * k + r : kG + g;
}

template <int D>
__global__ __launch_bounds__(256, 2) void out_proj_bf16_kernel(float* __restrict__ out, const float* __restrict__ p_tilde,
                                                               const uint16_t* __restrict__ w_o, float* __restrict__ y,
                                                               long long BT, int d_model, int G, int k, int n_shared,
                                                               int mode, int S, int nM, int nN, int write_weighted)
{
    constexpr int BM = OpTile<D>::BM, TPR = OpTile<D>::TPR, AV = OpTile<D>::AV, RB = OpTile<D>::RB;
    constexpr int PA = D + kOpPad;
    constexpr int BCH = kOpBN * D / 8 / 256;   // 16-byte W_o chunks per thread and stage
    __shared__ __attribute__((aligned(16))) uint16_t sA[BM * PA];
    __shared__ __attribute__((aligned(16))) uint16_t sB[kOpBN * PA];

    // workgroup -> tile: workgroups are dealt to the eight XCDs in turn, so
    // the nN column tiles of a token tile get indices 8 apart (one XCD)
    const int L = blockIdx.x, xcd = L & 7, r = L >> 3;
    const int tn = r % nN, tm = (r / nN) * 8 + xcd;
    if (tm >= nM) return;
    const long long m0 = (long long)tm * BM;
    const int n0 = tn * kOpBN;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int kG = G * k;
    const int nroute = mode ? G : 1;
    const size_t Ktot = (size_t)S * D;

    // this thread's token row and part of the slot (A side)
    const int arow = tid / TPR, acol = (tid % TPR) * AV;
    const long long tok = m0 + arow;
    const bool tok_ok = tok < BT;
    const long long tl = tok_ok ? tok : BT - 1;
    const float* arow_p = out + (size_t)tl * S * D + acol;
    const float* pt = p_tilde + (size_t)tl * kG;

    f32x4 ra[AV / 4];
    float rp = 0.f;
    u32x4 rb[BCH];
    auto load = [&](int i) {
        const int sl = op_slot(i, G, k, mode);
        if (sl < kG || sl >= kG + nroute) {
#pragma unroll
            for (int q = 0; q < AV / 4; ++q) ra[q] = *(const f32x4*)(arow_p + (size_t)sl * D + 4 * q);
            if (sl < kG) rp = pt[sl];
        }
#pragma unroll
        for (int c = 0; c < BCH; ++c) {
            const int ch = tid + 256 * c;
            const int n = min(n0 + ch / (D / 8), d_model - 1);
            rb[c] = ld_u32x4(w_o + (size_t)n * Ktot + (size_t)sl * D + (ch % (D / 8)) * 8);
        }
    };

    float wacc[AV];
#pragma unroll
    for (int v = 0; v < AV; ++v) wacc[v] = 0.f;

    // stage i into LDS: the slot as bf16 (a hard slot also adds into the
    // weighted sum; the weighted stage uses that sum and may write it back)
    auto store = [&](int i) {
        const int sl = op_slot(i, G, k, mode);
        float av[AV];
        if (sl < kG) {
#pragma unroll
            for (int q = 0; q < AV / 4; ++q)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    av[4 * q + e] = ra[q][e];
                    wacc[4 * q + e] = fmaf(rp, ra[q][e], wacc[4 * q + e]);
                }
        } else if (sl < kG + nroute) {
#pragma unroll
            for (int v = 0; v < AV; ++v) av[v] = wacc[v];
            if (write_weighted && tn == 0 && tok_ok) {
                float* dst = out + (size_t)tok * S * D + (size_t)sl * D + acol;
#pragma unroll
                for (int q = 0; q < AV / 4; ++q)
                    *(f32x4*)(dst + 4 * q) = f32x4{wacc[4 * q], wacc[4 * q + 1], wacc[4 * q + 2], wacc[4 * q + 3]};
            }
#pragma unroll
            for (int v = 0; v < AV; ++v) wacc[v] = 0.f;
        } else {
#pragma unroll
            for (int q = 0; q < AV / 4; ++q)
#pragma unroll
                for (int e = 0; e < 4; ++e) av[4 * q + e] = ra[q][e];
        }
#pragma unroll
        for (int q = 0; q < AV / 8; ++q) {
            const u32x4 pk = {pack_bf2(av[8 * q], av[8 * q + 1]), pack_bf2(av[8 * q + 2], av[8 * q + 3]),
                              pack_bf2(av[8 * q + 4], av[8 * q + 5]), pack_bf2(av[8 * q + 6], av[8 * q + 7])};
            *(u32x4*)&sA[arow * PA + acol + 8 * q] = pk;
        }
#pragma unroll
        for (int c = 0; c < BCH; ++c) {
            const int ch = tid + 256 * c;
            *(u32x4*)&sB[(ch / (D / 8)) * PA + (ch % (D / 8)) * 8] = rb[c];
        }
    };

    f32x16 acc[RB][2];
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
    const int wm = wave >> 1, wn = wave & 1;
    const int a_off = (32 * RB * wm + (lane & 31)) * PA + 8 * (lane >> 5);
    const int b_off = (64 * wn + (lane & 31)) * PA + 8 * (lane >> 5);

    load(0);
    for (int i = 0; i < S; ++i) {
        __syncthreads();
        store(i);
        __syncthreads();
        if (i + 1 < S) load(i + 1);
#pragma unroll
        for (int kk = 0; kk < D; kk += 16) {
            const bf16x8 b0 = ld_bf16x8(&sB[b_off + kk]), b1 = ld_bf16x8(&sB[b_off + 32 * PA + kk]);
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const bf16x8 a = ld_bf16x8(&sA[a_off + 32 * rb * PA + kk]);
                acc[rb][0] = mfma32(a, b0, acc[rb][0]);
                acc[rb][1] = mfma32(a, b1, acc[rb][1]);
            }
        }
    }

    // y rows: element e of block (i, j) is token 32 RB wm + 32 i + 8 (e / 4) +
    // 4 (lane / 32) + e % 4, feature 64 wn + 32 j + lane % 32
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const long long t = m0 + 32 * RB * wm + 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
            if (t >= BT) continue;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int n = n0 + 64 * wn + 32 * j + (lane & 31);
                if (n < d_model) y[(size_t)t * d_model + n] = acc[i][j][e];
            }
        }
}

// fp32: one thread per output element, fp32 FMA chain over the slots in the
// stage order above; the thread of feature 0 also writes the weighted slot(s).
__global__ __launch_bounds__(256) void out_proj_f32_kernel(float* __restrict__ out, const float* __restrict__ p_tilde,
                                                           const float* __restrict__ w_o, float* __restrict__ y,
                                                           long long BT, int d_model, int G, int k, int D, int mode,
                                                           int S, int write_weighted)
{
    const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= BT * d_model) return;
    const long long t = gid / d_model;
    const int n = (int)(gid % d_model);
    const int kG = G * k, nroute = mode ? G : 1;
    float* row = out + (size_t)t * S * D;
    const float* pt = p_tilde + (size_t)t * kG;
    const float* wr = w_o + (size_t)n * S * D;
    float s = 0.f;
    for (int d = 0; d < D; ++d) {
        float w = 0.f;
        for (int i = 0; i < S; ++i) {
            const int sl = op_slot(i, G, k, mode);
            float a;
            if (sl < kG) {
                a = row[(size_t)sl * D + d];
                w = fmaf(pt[sl], a, w);
            } else if (sl < kG + nroute) {
                a = w;
                if (write_weighted && n == 0) row[(size_t)sl * D + d] = w;
                w = 0.f;
            } else {
                a = row[(size_t)sl * D + d];
            }
            s = fmaf(a, wr[(size_t)sl * D + d], s);
        }
    }
    y[(size_t)t * d_model + n] = s;
}

int launch_out_proj(const OutProjArgs& a, hipStream_t st)
{
    if (a.BT == 0) return 0;
    if (!a.bf16) {
        const long long n = a.BT * a.d_model;
        out_proj_f32_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(a.out, a.p_tilde, (const float*)a.w_o, a.y,
                                                                           a.BT, a.d_model, a.G, a.k, a.d_head, a.route_mode,
                                                                           a.S, a.write_weighted);
        return hipGetLastError() == hipSuccess ? 0 : -1;
    }
    const int nN = (a.d_model + kOpBN - 1) / kOpBN;
#define GQE_OP(D)                                                                                                     \
    do {                                                                                                              \
        const long long nM = (a.BT + OpTile<D>::BM - 1) / OpTile<D>::BM;                                              \
        const long long grid = 8ll * ((nM + 7) / 8) * nN;                                                             \
        if (grid >= (1ll << 31)) return -2;                                                                           \
        out_proj_bf16_kernel<D><<<(unsigned)grid, 256, 0, st>>>(a.out, a.p_tilde, (const uint16_t*)a.w_o, a.y, a.BT,  \
                                                                a.d_model, a.G, a.k, a.n_shared, a.route_mode, a.S,   \
                                                                (int)nM, nN, a.write_weighted);                       \
    } while (0)
    switch (a.d_head) {
    case 32: GQE_OP(32); break;
    case 64: GQE_OP(64); break;
    case 128: GQE_OP(128); break;
    default: return -2;
    }
#undef GQE_OP
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace gqe
