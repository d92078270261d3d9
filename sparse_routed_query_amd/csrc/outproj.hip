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

#include <atomic>

namespace gqe {

constexpr int kOpBN = 128;   // output features per tile
constexpr int kOpPad = 8;    // bf16 elements of LDS row padding (16 bytes)

// Tile shape per d_head.  A slot row of a token (D fp32 values) is read by
// LPR = D/4 consecutive lanes with 16-byte loads, RPP = 256/LPR rows per
// pass, NP passes for the tile's BM tokens; a thread then holds NP x 4 values
// of the slot and of the weighted sum (BM = 64 at d_head = 128 keeps that at
// 32 registers each).
template <int D>
struct OpTile {
    static constexpr int BM = D >= 128 ? 64 : 128;
    static constexpr int LPR = D / 4;
    static constexpr int RPP = 256 / LPR;
    static constexpr int NP = BM / RPP;
    static constexpr int RB = BM / 64;   // 32-row blocks per wave
};

// Weighted slots of a route mode: one (0), one per group (1) or none (2, 3;
// mode 3's hard slots arrive already scaled, as gqe_attn_prefill leaves them).
__device__ __forceinline__ int op_nroute(int G, int mode) { return mode == 0 ? 1 : mode == 1 ? G : 0; }

// Slot read at K stage i (0 <= i < S).  Modes 0 and 2: slot order (hard,
// weighted if any, shared).  Mode 1: each group's hard slots, then that
// group's weighted slot, so the weighted sum is complete when its stage
// comes; the shared slot last.
__device__ __forceinline__ int op_slot(int i, int G, int k, int mode)
{
    if (mode != 1) return i;
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
    constexpr int BM = OpTile<D>::BM, LPR = OpTile<D>::LPR, RPP = OpTile<D>::RPP, NP = OpTile<D>::NP;
    constexpr int RB = OpTile<D>::RB;
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
    const int nroute = op_nroute(G, mode);
    const size_t Ktot = (size_t)S * D;

    // A side: this thread's rows arow0 + RPP p (p < NP), values acol .. acol+3.
    // Buffer loads over the tile's rows only: 32-bit offsets, and rows past
    // B*T fall outside the resource and read as zero (they are never stored).
    const int arow0 = tid / LPR, acol = (tid % LPR) * 4;
    const int rows = (int)(BT - m0 < BM ? BT - m0 : BM);
    const __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc((void*)(out + (size_t)m0 * S * D), 0,
                                                                         rows * S * D * 4, 0x00020000);
    const __amdgpu_buffer_rsrc_t rP = __builtin_amdgcn_make_buffer_rsrc((void*)(p_tilde + (size_t)m0 * kG), 0,
                                                                         rows * kG * 4, 0x00020000);

    f32x4 ra[NP];
    float rp[NP];
    u32x4 rb[BCH];
    auto load = [&](int i) {
        const int sl = op_slot(i, G, k, mode);
        if (sl < kG || sl >= kG + nroute) {
#pragma unroll
            for (int p = 0; p < NP; ++p)
                ra[p] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                      rA, ((arow0 + RPP * p) * S * D + sl * D + acol) * 4, 0, 0));
            if (sl < kG) {
#pragma unroll
                for (int p = 0; p < NP; ++p)
                    rp[p] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                          rP, ((arow0 + RPP * p) * kG + sl) * 4, 0, 0));
            }
        }
#pragma unroll
        for (int c = 0; c < BCH; ++c) {
            const int ch = tid + 256 * c;
            const int n = min(n0 + ch / (D / 8), d_model - 1);
            rb[c] = ld_u32x4(w_o + (size_t)n * Ktot + (size_t)sl * D + (ch % (D / 8)) * 8);
        }
    };

    f32x4 wacc[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) wacc[p] = f32x4{0.f, 0.f, 0.f, 0.f};

    // stage i into LDS: the slot as bf16 (a hard slot also adds into the
    // weighted sum; the weighted stage uses that sum and may write it back)
    auto store = [&](int i) {
        const int sl = op_slot(i, G, k, mode);
        f32x4 av[NP];
        if (sl < kG) {
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                av[p] = ra[p];
#pragma unroll
                for (int e = 0; e < 4; ++e) wacc[p][e] = fmaf(rp[p], ra[p][e], wacc[p][e]);
            }
        } else if (sl < kG + nroute) {
#pragma unroll
            for (int p = 0; p < NP; ++p) av[p] = wacc[p];
            if (write_weighted && tn == 0) {
#pragma unroll
                for (int p = 0; p < NP; ++p) {
                    const long long t = m0 + arow0 + RPP * p;
                    if (t < BT) *(f32x4*)(out + (size_t)t * S * D + (size_t)sl * D + acol) = wacc[p];
                }
            }
#pragma unroll
            for (int p = 0; p < NP; ++p) wacc[p] = f32x4{0.f, 0.f, 0.f, 0.f};
        } else {
#pragma unroll
            for (int p = 0; p < NP; ++p) av[p] = ra[p];
        }
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const uint32_t lo = pack_bf2(av[p][0], av[p][1]), hi = pack_bf2(av[p][2], av[p][3]);
            *(uint2*)&sA[(arow0 + RPP * p) * PA + acol] = make_uint2(lo, hi);
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

// Token-tile kernel for K = S*d_head small enough that a tile's whole bf16
// slot matrix fits in LDS: one workgroup of eight waves per 64 tokens, every
// output feature.  Prologue: the tile's slots are read once (fp32, several
// slots' loads in flight a thread), the weighted slot(s) formed in the fixed
// order above, everything rounded to bf16 into LDS [64][K + 8].  Then each
// wave walks its own 64-feature column tiles (tile w, w + 8, ...): 64 x 64
// outputs as 2 x 2 blocks of 32x32x16 MFMA, the W_o fragments loaded straight
// from global memory four k-steps ahead (each wave reads only its own
// features, so nothing is shared and no barrier follows the prologue), the
// slot fragments from LDS.  The slots are read from memory once instead of
// once per column tile, as bf16 from LDS thereafter.
//
// PACKED: W_o in fragment order (gqe_out_proj_pack), so that each fragment
// load of a wave is 1 KB of consecutive bytes; from the row-major W_o a load
// touches 32 rows, 32 bytes each, and the four k-steps that share a 128-byte
// line reach it at different times, so lines are fetched from L2 repeatedly.
// Packed index of W_o[64 ct + 32 cb + c][16 ks + 8 h + e] (c < 32, h < 2,
// e < 8): ((ct * K/16 + ks) * 2 + cb) * 512 + (32 h + c) * 8 + e.
constexpr int kOtM = 64;                       // tokens per workgroup
constexpr int kOtWaves = 8;
constexpr int kOtPad = 8;                      // bf16 elements of row padding
constexpr int kOtMaxLds = 160 * 1024;          // LDS of a gfx950 compute unit

__host__ __device__ constexpr int ot_lds_bytes(int K) { return kOtM * (K + kOtPad) * 2; }
bool out_proj_tile_fits(int K, int d_model) { return ot_lds_bytes(K) <= kOtMaxLds && d_model % 64 == 0; }

template <int D, bool PACKED>
__global__ __launch_bounds__(64 * kOtWaves, 1) void out_proj_tile_kernel(float* __restrict__ out,
                                                               const float* __restrict__ p_tilde,
                                                               const uint16_t* __restrict__ w_o,
                                                               float* __restrict__ y, long long BT, int d_model,
                                                               int G, int k, int mode, int S, int write_weighted)
{
    extern __shared__ __attribute__((aligned(16))) uint16_t sA[];
    constexpr int LPR = D / 4, RPP = 64 * kOtWaves / LPR, NP = kOtM / RPP;
    constexpr int SB = D == 32 ? 4 : NP >= 10 ? 1 : 10 / NP;   // slots whose loads are in flight together
    const int K = S * D, PA = K + kOtPad;
    const long long m0 = (long long)blockIdx.x * kOtM;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int kG = G * k, nroute = op_nroute(G, mode);

    // ---- prologue: slots -> bf16 LDS tile (rows past B*T read as zero and are never stored)
    const int arow0 = tid / LPR, acol = (tid % LPR) * 4;
    const int rows = (int)(BT - m0 < kOtM ? BT - m0 : kOtM);
    const __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc((void*)(out + (size_t)m0 * S * D), 0,
                                                                         rows * S * D * 4, 0x00020000);
    const __amdgpu_buffer_rsrc_t rP = __builtin_amdgcn_make_buffer_rsrc((void*)(p_tilde + (size_t)m0 * kG), 0,
                                                                         rows * kG * 4, 0x00020000);
    f32x4 wacc[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) wacc[p] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int i0 = 0; i0 < S; i0 += SB) {
        f32x4 ra[SB][NP];
        float rp[SB][NP];
#pragma unroll
        for (int u = 0; u < SB; ++u) {
            const int sl = i0 + u < S ? op_slot(i0 + u, G, k, mode) : kG;   // past S: a weighted-like no-load
            const bool data = i0 + u < S && (sl < kG || sl >= kG + nroute);
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                ra[u][p] = data ? __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                      rA, ((arow0 + RPP * p) * S * D + sl * D + acol) * 4, 0, 0))
                                : f32x4{0.f, 0.f, 0.f, 0.f};
                rp[u][p] = (data && sl < kG) ? __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                   rP, ((arow0 + RPP * p) * kG + sl) * 4, 0, 0))
                                             : 0.f;
            }
        }
#pragma unroll
        for (int u = 0; u < SB; ++u) {
            if (i0 + u >= S) break;
            const int sl = op_slot(i0 + u, G, k, mode);
            f32x4 av[NP];
            if (sl < kG) {
#pragma unroll
                for (int p = 0; p < NP; ++p) {
                    av[p] = ra[u][p];
#pragma unroll
                    for (int e = 0; e < 4; ++e) wacc[p][e] = fmaf(rp[u][p], ra[u][p][e], wacc[p][e]);
                }
            } else if (sl < kG + nroute) {
#pragma unroll
                for (int p = 0; p < NP; ++p) av[p] = wacc[p];
                if (write_weighted) {
#pragma unroll
                    for (int p = 0; p < NP; ++p) {
                        const long long t = m0 + arow0 + RPP * p;
                        if (t < BT) *(f32x4*)(out + (size_t)t * S * D + (size_t)sl * D + acol) = wacc[p];
                    }
                }
#pragma unroll
                for (int p = 0; p < NP; ++p) wacc[p] = f32x4{0.f, 0.f, 0.f, 0.f};
            } else {
#pragma unroll
                for (int p = 0; p < NP; ++p) av[p] = ra[u][p];
            }
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                const uint32_t lo = pack_bf2(av[p][0], av[p][1]), hi = pack_bf2(av[p][2], av[p][3]);
                *(uint2*)&sA[(arow0 + RPP * p) * PA + sl * D + acol] = make_uint2(lo, hi);
            }
        }
    }
    __syncthreads();

    // ---- each wave: its 64-feature column tiles over the whole K
    constexpr int KC = 4;                      // k-steps of W_o fragments loaded ahead
    constexpr int BSTEP = PACKED ? 1024 : 16;  // elements between a lane's fragments of consecutive k-steps
    const int NT = d_model / 64, KS = K / 16;
    const __amdgpu_buffer_rsrc_t rY = __builtin_amdgcn_make_buffer_rsrc((void*)(y + (size_t)m0 * d_model), 0,
                                                                         rows * d_model * 4, 0x00020000);
    const uint16_t* a0p = sA + (lane & 31) * PA + 8 * (lane >> 5);
    const uint16_t* a1p = a0p + 32 * PA;
    for (int ct = wave; ct < NT; ct += kOtWaves) {
        const int n0 = ct * 64;
        const uint16_t* b0p = PACKED ? w_o + (size_t)n0 * K + lane * 8
                                     : w_o + (size_t)(n0 + (lane & 31)) * K + 8 * (lane >> 5);
        const uint16_t* b1p = PACKED ? b0p + 512 : b0p + (size_t)32 * K;
        f32x16 acc[2][2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
        // W_o fragments in two register sets used in turn: the loads of the next chunk of KC k-steps
        // are issued before the current chunk's products
        u32x4 bA[KC][2], bB[KC][2];
        auto load_b = [&](u32x4 (&b)[KC][2], int c0) {
#pragma unroll
            for (int u = 0; u < KC; ++u) {
                const int ks = min(c0 + u, KS - 1);
                b[u][0] = ld_u32x4(b0p + BSTEP * ks);
                b[u][1] = ld_u32x4(b1p + BSTEP * ks);
            }
        };
        auto mma = [&](const u32x4 (&b)[KC][2], int c0) {
            if (c0 + KC <= KS) {
                // a whole chunk: no per-step test, so the slot fragments' LDS reads are issued ahead
                bf16x8 a0[KC], a1[KC];
#pragma unroll
                for (int u = 0; u < KC; ++u) {
                    a0[u] = ld_bf16x8(a0p + 16 * (c0 + u));
                    a1[u] = ld_bf16x8(a1p + 16 * (c0 + u));
                }
#pragma unroll
                for (int u = 0; u < KC; ++u) {
                    const bf16x8 b0 = __builtin_bit_cast(bf16x8, b[u][0]), b1 = __builtin_bit_cast(bf16x8, b[u][1]);
                    acc[0][0] = mfma32(a0[u], b0, acc[0][0]);
                    acc[0][1] = mfma32(a0[u], b1, acc[0][1]);
                    acc[1][0] = mfma32(a1[u], b0, acc[1][0]);
                    acc[1][1] = mfma32(a1[u], b1, acc[1][1]);
                }
            } else {
#pragma unroll
                for (int u = 0; u < KC; ++u) {
                    const int ks = c0 + u;
                    if (ks < KS) {
                        const bf16x8 a0 = ld_bf16x8(a0p + 16 * ks), a1 = ld_bf16x8(a1p + 16 * ks);
                        const bf16x8 b0 = __builtin_bit_cast(bf16x8, b[u][0]), b1 = __builtin_bit_cast(bf16x8, b[u][1]);
                        acc[0][0] = mfma32(a0, b0, acc[0][0]);
                        acc[0][1] = mfma32(a0, b1, acc[0][1]);
                        acc[1][0] = mfma32(a1, b0, acc[1][0]);
                        acc[1][1] = mfma32(a1, b1, acc[1][1]);
                    }
                }
            }
        };
        // (loads past the last k-step repeat it, in bounds, and are not used)
        load_b(bA, 0);
        for (int c0 = 0; c0 < KS; c0 += 2 * KC) {
            load_b(bB, c0 + KC);
            mma(bA, c0);
            load_b(bA, c0 + 2 * KC);
            mma(bB, c0 + KC);
        }
        // element e of block (i, j): token 32 i + 8 (e / 4) + 4 (lane / 32) + e % 4, feature 32 j + lane % 32;
        // buffer stores over the tile's rows, so rows past B*T are dropped without a branch (the value goes
        // through __float_as_uint: this compiler's __builtin_bit_cast of a vector element reads element 0)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e)
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int r = 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[i][j][e]), rY,
                                                          (r * d_model + n0 + 32 * j + (lane & 31)) * 4, 0, 0);
                }
    }
}

// W_o [d_model, K] bf16 -> fragment order (see PACKED above): one thread per 16-byte chunk.
__global__ __launch_bounds__(256) void out_proj_pack_kernel(const uint16_t* __restrict__ w_o, uint16_t* __restrict__ wp,
                                                            int d_model, int K)
{
    const long long q = (long long)blockIdx.x * 256 + threadIdx.x;   // destination chunk
    const int KS = K / 16;
    if (q >= (long long)d_model * KS * 2) return;
    const int l = (int)(q & 63);
    const long long blk = q >> 6;                                    // (ct * KS + ks) * 2 + cb
    const int cb = (int)(blk & 1);
    const long long cs = blk >> 1;
    const int ks = (int)(cs % KS), ct = (int)(cs / KS);
    const int n = 64 * ct + 32 * cb + (l & 31);
    *(u32x4*)(wp + q * 8) = ld_u32x4(w_o + (size_t)n * K + 16 * ks + 8 * (l >> 5));
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
    const int kG = G * k, nroute = op_nroute(G, mode);
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

int launch_out_proj_pack(const void* w_o, void* w_packed, int d_model, int K, hipStream_t st)
{
    if (!out_proj_tile_fits(K, d_model) || K % 16) return -2;
    const long long chunks = (long long)d_model * (K / 16) * 2;
    if (chunks == 0) return 0;
    out_proj_pack_kernel<<<(unsigned)((chunks + 255) / 256), 256, 0, st>>>((const uint16_t*)w_o, (uint16_t*)w_packed,
                                                                           d_model, K);
    return hipGetLastError() == hipSuccess ? 0 : -1;
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
    // packed weights: the token-tile kernel (row-major W_o stays on the kernel below, which reads it
    // through LDS with coalesced loads: 54 against 58 us for the tile kernel on main_250m)
    const int K = a.S * a.d_head;
    if (a.w_packed) {
        if (!out_proj_tile_fits(K, a.d_model)) return -2;
        const long long grid = (a.BT + kOtM - 1) / kOtM;
        if (grid >= (1ll << 31)) return -2;
        const int lds = ot_lds_bytes(K);
        // the LDS limit is raised once per kernel to the largest tile that fits (setting it per call
        // costs host time comparable to the kernel's)
#define GQE_OT(D, PK)                                                                                                 \
    do {                                                                                                              \
        static std::atomic<int> raised{0};                                                                            \
        if (lds > 65536 && !raised.load(std::memory_order_acquire)) {                                                 \
            if (hipFuncSetAttribute((const void*)&out_proj_tile_kernel<D, PK>,                                         \
                                    hipFuncAttributeMaxDynamicSharedMemorySize, kOtMaxLds) != hipSuccess)             \
                return -1;                                                                                            \
            raised.store(1, std::memory_order_release);                                                               \
        }                                                                                                             \
        out_proj_tile_kernel<D, PK><<<(unsigned)grid, 64 * kOtWaves, lds, st>>>(                                      \
            a.out, a.p_tilde, (const uint16_t*)(PK ? a.w_packed : a.w_o), a.y, a.BT, a.d_model, a.G, a.k,            \
            a.route_mode, a.S, a.write_weighted);                                                                     \
    } while (0)
#define GQE_OT2(D) GQE_OT(D, true)
        switch (a.d_head) {
        case 32: GQE_OT2(32); break;
        case 64: GQE_OT2(64); break;
        case 128: GQE_OT2(128); break;
        default: return -2;
        }
#undef GQE_OT2
#undef GQE_OT
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
