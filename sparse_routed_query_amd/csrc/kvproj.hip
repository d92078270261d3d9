// The K and V projections as one dense GEMM (gfx950, bf16 MFMA, fp32
// accumulation): k[b,h,t] = R_t W_k[h] x_t and v[b,h,t] = W_v[h] x_t for every
// token, R_t the optional rotary embedding at the token's position (GQA
// tutorial, freeguideonline, "GQA 核心原理与计算流程" step 2: the input is
// projected to K and V, split into KV heads as wide as a query head).
//
// Unlike the query rows, K and V have no routing: every token needs all
// 2 * H_kv * d_head output features, so the product is a plain
// [B*T, d_model] x [d_model, 2 H_kv d_head] GEMM and takes large tiles: one
// workgroup of eight waves per 256 tokens x 256 features, stages of 64 along
// d_model staged through LDS (x rows and weight rows both read as 128-byte
// lines), each wave 64 tokens x 128 features as 2 x 4 blocks of 32x32x16
// MFMA, so every fragment read from LDS feeds two or four products.  x is
// read once per 256 features (four times at 1024), the weights once per 256
// tokens.  The column tiles of a token tile run on one XCD, so x comes from
// HBM once and from that XCD's L2 after that.  Results leave through LDS in
// fp32, where the rotary pairs (c, c + d/2) of a K head are rotated before the
// one bf16 rounding (the same angle arithmetic as the query rows), so every
// global store is 16 bytes of one output row.
#include "gqe_device.h"
#include "gqe_launch.h"

namespace gqe {

constexpr int kKvTM = 256, kKvTN = 256, kKvSK = 64, kKvPad = 8;
constexpr int kKvPitch = kKvSK + kKvPad;   // LDS row pitch in bf16 elements

template <int D>
__global__ __launch_bounds__(512, 1) void kv_dense_kernel(const KvDenseArgs a)
{
    const int BT = a.B * a.T, H = a.H, HD = H * D, NC = 2 * HD, dm = a.d_model;
    const int nM = (BT + kKvTM - 1) / kKvTM, nN = (NC + kKvTN - 1) / kKvTN;
    // workgroup -> tile: the nN column tiles of a token tile get indices 8 apart (one XCD)
    const int L = blockIdx.x, xcd = L & 7, r = L >> 3;
    const int tn = r % nN, tm = (r / nN) * 8 + xcd;
    if (tm >= nM) return;
    const int m0 = tm * kKvTM, n0 = tn * kKvTN;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave & 3, wn = wave >> 2;   // 4 x 2 waves of 64 tokens x 128 features

    // two LDS stages (x rows, then weight rows), used in turn: one barrier per stage
    constexpr int STAGE = (kKvTM + kKvTN) * kKvPitch;
    __shared__ __attribute__((aligned(16))) uint16_t sS[2 * STAGE];

    // this thread's 16-byte chunks of a stage: row tid / 8 + 64 i, columns 8 (tid % 8) .. +7
    const int crow = tid >> 3, ccol = (tid & 7) * 8;
    const uint16_t* xs[4];
    const uint16_t* ws[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int tok = min(m0 + crow + 64 * i, BT - 1);   // rows past B*T repeat the last one, never stored
        xs[i] = a.x + (size_t)tok * dm + ccol;
        const int c = min(n0 + crow + 64 * i, NC - 1);
        const int kv = c >= HD, rem = c - kv * HD;          // weight row rem of W_k or W_v, [H*D, d_model]
        ws[i] = (kv ? a.w_v : a.w_k) + (size_t)rem * dm + ccol;
    }
    u32x4 ra[4], rb[4];
    auto load = [&](int k0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            ra[i] = ld_u32x4(xs[i] + k0);
            rb[i] = ld_u32x4(ws[i] + k0);
        }
    };
    auto store = [&](uint16_t* buf) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            *(u32x4*)&buf[(crow + 64 * i) * kKvPitch + ccol] = ra[i];
            *(u32x4*)&buf[(kKvTM + crow + 64 * i) * kKvPitch + ccol] = rb[i];
        }
    };

    f32x16 acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    const int a_off = (64 * wm + (lane & 31)) * kKvPitch + 8 * (lane >> 5);
    const int b_off = (kKvTM + 128 * wn + (lane & 31)) * kKvPitch + 8 * (lane >> 5);
    auto mma = [&](const uint16_t* buf, int kk) {
        bf16x8 fa[2], fb[4];
#pragma unroll
        for (int i = 0; i < 2; ++i) fa[i] = ld_bf16x8(buf + a_off + 32 * i * kKvPitch + kk);
#pragma unroll
        for (int j = 0; j < 4; ++j) fb[j] = ld_bf16x8(buf + b_off + 32 * j * kKvPitch + kk);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = mfma32(fa[i], fb[j], acc[i][j]);
    };
    const int nst = dm / kKvSK;   // d_model is a multiple of 64 (checked by the API)
    load(0);
    store(sS);
    if (nst > 1) load(kKvSK);
    __syncthreads();
    for (int st = 0; st < nst; ++st) {
        const uint16_t* cur = sS + (st & 1) * STAGE;
        mma(cur, 0);
        mma(cur, 16);
        // the next stage into the other buffer (its readers passed the last barrier), then its successor's loads
        if (st + 1 < nst) {
            store(sS + ((st + 1) & 1) * STAGE);
            if (st + 2 < nst) load((st + 2) * kKvSK);
        }
        mma(cur, 32);
        mma(cur, 48);
        __syncthreads();
    }

    // element e of block (i, j): token 64 wm + 32 i + 8 (e / 4) + 4 (lane / 32) + e % 4,
    // feature 128 wn + 32 j + lane % 32 of the tile.  The results leave through the wave's own LDS region,
    // 32 tokens x 128 features in fp32 at a time: the rotary pairs of K are formed there (fp32, before the
    // one bf16 rounding), and every global store is 16 bytes of one output row.
    const int cw = n0 + 128 * wn;                       // first feature of this wave's span (a multiple of 128)
    constexpr int RP = 128 + 4;                         // region pitch in floats
    float* regf = (float*)sS + wave * 32 * RP;          // 16.5 KB per wave
    // a lane's chunk: features f0 .. f0+7 of the span (the same chunk for all its rows)
    const int f0 = 8 * (lane & 15), c = cw + f0;
    const bool live_c = c < NC;
    const int kv = c >= HD, rem = c - kv * HD, h = rem / D, d0 = rem - h * D;
    const bool rot = a.rope_log2_base > 0.0 && live_c && kv == 0;
    // rotary: feature d < D/2 pairs with d + D/2 (the partner chunk, D/2 features on in the same span);
    // the lane holding the first half of a pair writes both
    double freq[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) freq[u] = (rot && d0 < D / 2) ? rope_freq(d0 + u, D, a.rope_log2_base) : 0.0;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                regf[(8 * (e >> 2) + 4 * (lane >> 5) + (e & 3)) * RP + 32 * j + (lane & 31)] = acc[i][j][e];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        for (int q = 0; q < 8; ++q) {
            const int rl = (lane >> 4) + 4 * q;          // row of the 32
            const int row = m0 + 64 * wm + 32 * i + rl;
            const f32x4 v0 = *(const f32x4*)&regf[rl * RP + f0], v1 = *(const f32x4*)&regf[rl * RP + f0 + 4];
            if (row >= BT || !live_c) continue;
            const int b = row / a.T, t = row - b * a.T;
            uint16_t* dst = (uint16_t*)(kv ? a.v_out : a.k_out);
            uint16_t* o = dst + (((size_t)b * H + h) * a.T + t) * D + d0;
            if (!rot) {
                *(u32x4*)o = u32x4{pack_bf2(v0[0], v0[1]), pack_bf2(v0[2], v0[3]), pack_bf2(v1[0], v1[1]),
                                   pack_bf2(v1[2], v1[3])};
            } else if (d0 < D / 2) {
                // the lane of the first half turns the pair: (x1, x2) -> (x1 cos - x2 sin, x2 cos + x1 sin)
                const f32x4 p0 = *(const f32x4*)&regf[rl * RP + f0 + D / 2];
                const f32x4 p1 = *(const f32x4*)&regf[rl * RP + f0 + D / 2 + 4];
                const int pos = a.positions ? a.positions[row] : t;
                float r1[8], r2[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    float sn, cs;
                    sincosf(rope_angle(pos, freq[u]), &sn, &cs);
                    const float x1 = u < 4 ? v0[u] : v1[u - 4], x2 = u < 4 ? p0[u] : p1[u - 4];
                    r1[u] = x1 * cs - x2 * sn;
                    r2[u] = x2 * cs + x1 * sn;
                }
                *(u32x4*)o = u32x4{pack_bf2(r1[0], r1[1]), pack_bf2(r1[2], r1[3]), pack_bf2(r1[4], r1[5]),
                                   pack_bf2(r1[6], r1[7])};
                *(u32x4*)(o + D / 2) = u32x4{pack_bf2(r2[0], r2[1]), pack_bf2(r2[2], r2[3]), pack_bf2(r2[4], r2[5]),
                                             pack_bf2(r2[6], r2[7])};
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
}

int launch_kv_dense(const KvDenseArgs& a, hipStream_t st)
{
    const long long BT = (long long)a.B * a.T;
    if (BT == 0 || a.H == 0) return 0;
    if (a.d_model % kKvSK) return -2;
    const long long nM = (BT + kKvTM - 1) / kKvTM, nN = (2ll * a.H * a.d_head + kKvTN - 1) / kKvTN;
    const long long grid = 8 * ((nM + 7) / 8) * nN;
    if (grid >= (1ll << 31) || BT >= (1ll << 31)) return -2;
    switch (a.d_head) {
    case 32: kv_dense_kernel<32><<<(unsigned)grid, 512, 0, st>>>(a); break;
    case 64: kv_dense_kernel<64><<<(unsigned)grid, 512, 0, st>>>(a); break;
    case 128: kv_dense_kernel<128><<<(unsigned)grid, 512, 0, st>>>(a); break;
    default: return -2;
    }
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace gqe
