// The decode step's routing and query projection in one launch (gfx950): for
// one new token per sequence, the router scores of each group, the in-group
// softmax, the top-k with lower-index ties and the renormalised weights (GQE
// study note §3-2 (2), (4)), then the projections of only the kept experts
// and the shared head (§3-2 (2) last sentence, (5)), with the optional rotary
// embedding of the queries at the token's position.
//
// One workgroup per (sequence, group) and one more per sequence for the
// shared head.  bf16 scores are exact products summed in double in a fixed
// order (fp32: one fp64 FMA chain per score in index order, as gqe_route
// does); the top k is picked in parallel by rank.  Each weight row is read by
// 32 lanes with 16-byte loads, about 16 of them in flight a lane, and reduced
// across those lanes in a fixed order.  With this launch a decode step is
// route+project, then the attention: no compaction (decode needs none).
#include "gqe_device.h"
#include "gqe_launch.h"

namespace gqe {

constexpr int kDpMaxE = 64;   // experts per group (the descriptor's H_q limit)

template <typename ET>
__device__ __forceinline__ float dp_elem(const u32x4& v, int i);
template <>
__device__ __forceinline__ float dp_elem<uint16_t>(const u32x4& v, int i)
{
    const uint32_t w = v[i >> 1];
    return __builtin_bit_cast(float, (i & 1) ? (w & 0xffff0000u) : (w << 16));
}
template <>
__device__ __forceinline__ float dp_elem<float>(const u32x4& v, int i)
{
    return __uint_as_float(v[i]);
}

__device__ __forceinline__ float elem_f32(float v) { return v; }
__device__ __forceinline__ float elem_f32(uint16_t v) { return bf2f(v); }

template <typename ET, int D>
__global__ __launch_bounds__(256) void decode_preamble_kernel(const DecodePreArgs a)
{
    constexpr int VEC = 16 / sizeof(ET);          // elements per 16-byte load
    const int b = blockIdx.x, gg = blockIdx.y;
    const int G = a.G, E = a.E, k = a.k, N = G * E, dm = a.d_model;
    const bool shared = gg == G;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const ET* xb = (const ET*)a.x + (size_t)b * dm;
    __shared__ double s_sc[kDpMaxE];
    __shared__ int s_sel[8];
    __shared__ float s_q[8][D];

    int nsel = 0;   // kept rows this workgroup projects
    if (!shared) {
        // ---- scores of the group's E experts
        if constexpr (sizeof(ET) == 4) {
            // fp32: one fp64 FMA chain per score, in index order (bit for bit gqe_route's)
            if (tid < E) {
                const float* xr = (const float*)xb;
                const float* wr = (const float*)a.w_router + (size_t)(gg * E + tid) * dm;
                double s = 0.0;
                for (int i = 0; i < dm; ++i) s = fma((double)xr[i], (double)wr[i], s);
                s_sc[tid] = s;
            }
        } else {
            // bf16: four experts per wave at a time, each lane over 8-element chunks (d_model is a
            // multiple of 64); exact products added in double, then the lanes in a fixed tree
            const uint16_t* wq0 = (const uint16_t*)a.w_router + (size_t)gg * E * dm;
            for (int e0 = 4 * wave; e0 < E; e0 += 16) {
                double acc[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll 2
                for (int col = 8 * lane; col < dm; col += 512) {
                    const u32x4 xv = ld_u32x4(xb + col);
                    u32x4 wv[4];
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        wv[c] = e0 + c < E ? ld_u32x4(wq0 + (size_t)(e0 + c) * dm + col) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
                    for (int c = 0; c < 4; ++c)
#pragma unroll
                        for (int i = 0; i < 8; ++i)
                            acc[c] += (double)(dp_elem<uint16_t>(xv, i) * dp_elem<uint16_t>(wv[c], i));
                }
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    double v = acc[c];
#pragma unroll
                    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
                    if (lane == 0 && e0 + c < E) s_sc[e0 + c] = v;
                }
            }
        }
        __syncthreads();
        // ---- bias, logits, then the selection in parallel (wave 0, one expert a lane): expert e is kept
        // when fewer than k experts rank above it (higher score, or equal score and lower index), which is
        // the k largest with lower-index ties; the kept ones are numbered in ascending index.
        if (wave == 0) {
            const bool live = lane < E;
            double se = 0.0;
            if (live) {
                se = s_sc[lane] + (a.b_router ? (double)a.b_router[gg * E + lane] : 0.0);
                if (a.logits) a.logits[(size_t)b * N + gg * E + lane] = se;
            }
            // every lane's score, with the bias, from its owner lane
            int rank = 0;
            for (int f = 0; f < E; ++f) {
                const double sf = __shfl(se, f);
                rank += (sf > se) || (sf == se && f < lane);
            }
            const bool kept = live && rank < k;
            const uint64_t mask = __ballot(kept);
            double mk = kept ? se : -INFINITY, ma = live ? se : -INFINITY;
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) {
                mk = fmax(mk, __shfl_xor(mk, o));
                ma = fmax(ma, __shfl_xor(ma, o));
            }
            const double mref = a.renorm ? mk : ma;
            const float ex = live ? expf((float)(se - mref)) : 0.f;
            // the denominator in ascending index, the same in every lane: the kept terms (or, not
            // renormalised, all E)
            float den = 0.f;
            for (int e = 0; e < E; ++e) {
                const float v = __shfl(ex, e);
                if (!a.renorm || ((mask >> e) & 1)) den += v;
            }
            if (kept) {
                const int j = __popcll(mask & ((1ull << lane) - 1));
                const size_t o = ((size_t)b * G + gg) * k + j;
                a.sel[o] = lane;
                a.p_tilde[o] = ex / den;
                s_sel[j] = gg * E + lane;
            }
        }
        __syncthreads();
        nsel = k;
    } else {
        if (tid == 0) s_sel[0] = N;
        __syncthreads();
        nsel = 1;
    }

    // ---- projections: each 32-lane group owns rows grp, grp + 8, ... of the d_head rows of each kept
    // expert (or the shared head); a sweep loads U column chunks of 16 bytes of each of its rows at once
    // (about 16 loads in flight a lane), x's chunks alongside.  16-byte loads when d_model is a
    // multiple of VEC (always for bf16, whose d_model is a multiple of 64): a lane's chunk is then wholly
    // inside or past the row; else one element a lane.
    constexpr int RPG = D / 8;                     // rows per 32-lane group
    constexpr int U = RPG >= 16 ? 1 : 16 / RPG;    // column chunks per sweep
    constexpr int PER = 32 * VEC;                  // columns one chunk of the 32 lanes covers
    const int sub = tid & 31, grp = tid >> 5;
    const bool vec = dm % VEC == 0;
    for (int j = 0; j < nsel; ++j) {
        const ET* w = (const ET*)a.w_q + ((size_t)s_sel[j] * D + grp) * dm;
        float acc[RPG];
#pragma unroll
        for (int i = 0; i < RPG; ++i) acc[i] = 0.f;
        if (vec) {
            for (int c0 = sub * VEC; c0 < dm; c0 += U * PER) {
                u32x4 xv[U], wv[U][RPG];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int col = c0 + u * PER;
                    const bool in = col < dm;
                    xv[u] = in ? ld_u32x4(xb + col) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
                    for (int i = 0; i < RPG; ++i)
                        wv[u][i] = in ? ld_u32x4(w + (size_t)(8 * i) * dm + col) : u32x4{0u, 0u, 0u, 0u};
                }
#pragma unroll
                for (int u = 0; u < U; ++u)
#pragma unroll
                    for (int i = 0; i < RPG; ++i)
#pragma unroll
                        for (int e = 0; e < VEC; ++e)
                            acc[i] = fmaf(dp_elem<ET>(xv[u], e), dp_elem<ET>(wv[u][i], e), acc[i]);
            }
        } else {
            for (int col = sub; col < dm; col += 32) {
                const float xv = elem_f32(xb[col]);
#pragma unroll
                for (int i = 0; i < RPG; ++i) acc[i] = fmaf(xv, elem_f32(w[(size_t)(8 * i) * dm + col]), acc[i]);
            }
        }
#pragma unroll
        for (int i = 0; i < RPG; ++i) {
            float v = acc[i];
#pragma unroll
            for (int o = 16; o > 0; o >>= 1) v += __shfl_xor(v, o);
            if (sub == 0) s_q[j][grp + 8 * i] = v;
        }
    }
    __syncthreads();
    // ---- rotary embedding (fp32, before the one rounding) and stores
    const bool rot = a.rope_log2_base > 0.0;
    const int pos = rot ? (a.positions ? a.positions[b] : 0) : 0;
    for (int i = tid; i < nsel * (D / 2); i += 256) {
        const int j = i / (D / 2), c = i % (D / 2);
        float u = s_q[j][c], w = s_q[j][c + D / 2];
        if (rot) {
            float sn, cs;
            sincosf(rope_angle(pos, rope_freq(c, D, a.rope_log2_base)), &sn, &cs);
            const float uu = u;
            u = uu * cs - w * sn;
            w = w * cs + uu * sn;
        }
        ET* dst = shared ? (ET*)a.q_shared + (size_t)b * D : (ET*)a.q_routed + (((size_t)b * G + gg) * k + j) * D;
        if constexpr (sizeof(ET) == 4) {
            dst[c] = u;
            dst[c + D / 2] = w;
        } else {
            dst[c] = __builtin_bit_cast(uint16_t, f2bf(u));
            dst[c + D / 2] = __builtin_bit_cast(uint16_t, f2bf(w));
        }
    }
}

int launch_decode_preamble(const DecodePreArgs& a, hipStream_t st)
{
    if (a.B == 0) return 0;
    if (a.E > kDpMaxE || a.k > 8) return -2;
    const dim3 grid(a.B, a.G + (a.q_shared ? 1 : 0));
#define GQE_DP(ET, D) decode_preamble_kernel<ET, D><<<grid, 256, 0, st>>>(a)
    if (a.bf16) {
        switch (a.d_head) {
        case 32: GQE_DP(uint16_t, 32); break;
        case 64: GQE_DP(uint16_t, 64); break;
        case 128: GQE_DP(uint16_t, 128); break;
        default: return -2;
        }
    } else {
        switch (a.d_head) {
        case 32: GQE_DP(float, 32); break;
        case 64: GQE_DP(float, 64); break;
        case 128: GQE_DP(float, 128); break;
        default: return -2;
        }
    }
#undef GQE_DP
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace gqe
