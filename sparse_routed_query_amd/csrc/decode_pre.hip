// The decode step's routing and query projection in one launch (gfx950): for
// one new token per sequence, the router scores of each group, the in-group
// softmax, the top-k with lower-index ties and the renormalised weights (GQE
// study note §3-2 (2), (4)), then the projections of only the kept experts
// and the shared head (§3-2 (2) last sentence, (5)), with the optional rotary
// embedding of the queries at the token's position.
//
// One workgroup per (sequence, group) and one more per sequence for the
// shared head.  The token's x row is read once into registers; scores are
// exact products summed in double (fp32 inputs: one fp64 FMA chain per score
// in index order, as gqe_route does); each kept expert's d_head x d_model
// weight rows are read with 16-byte loads, 32 lanes per row, and reduced
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
    constexpr int PER = 32 * VEC;                 // elements of a row one 32-lane group covers per pass
    const int b = blockIdx.x, gg = blockIdx.y;
    const int G = a.G, E = a.E, k = a.k, N = G * E, dm = a.d_model;
    const bool shared = gg == G;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int sub = tid & 31, grp = tid >> 5;     // 8 groups of 32 lanes
    const ET* xb = (const ET*)a.x + (size_t)b * dm;
    __shared__ double s_red[4][kDpMaxE];
    __shared__ int s_sel[8];
    __shared__ float s_q[8 + 1][D];

    int nsel = 0;   // kept rows this workgroup projects
    if (!shared) {
        // ---- scores of the group's E experts
        const float* bias = a.b_router ? a.b_router + gg * E : nullptr;
        if constexpr (sizeof(ET) == 4) {
            // fp32: one fp64 FMA chain per score, in index order (bit for bit gqe_route's)
            if (tid < E) {
                const float* xr = (const float*)xb;
                const float* wr = (const float*)a.w_router + (size_t)(gg * E + tid) * dm;
                double s = 0.0;
                for (int i = 0; i < dm; ++i) s = fma((double)xr[i], (double)wr[i], s);
                s_red[0][tid] = s;
            }
        } else {
            // bf16: exact products added in double, each wave over a quarter of d_model,
            // then the lanes and the waves in a fixed order
            for (int e0 = 0; e0 < E; e0 += 4) {
                double p[4] = {0.0, 0.0, 0.0, 0.0};
                for (int i = tid; i < dm; i += 256) {
                    const float xv = bf2f(((const uint16_t*)xb)[i]);
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        if (e0 + c < E)
                            p[c] += (double)(xv * bf2f(((const uint16_t*)a.w_router)[(size_t)(gg * E + e0 + c) * dm + i]));
                }
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    double v = p[c];
#pragma unroll
                    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
                    if (lane == 0 && e0 + c < E) s_red[wave][e0 + c] = v;
                }
            }
            __syncthreads();
            if (tid < E) s_red[0][tid] = ((s_red[0][tid] + s_red[1][tid]) + s_red[2][tid]) + s_red[3][tid];
        }
        // the bias and the logits output, one expert a thread
        if (tid < E) {
            const double v = s_red[0][tid] + (bias ? (double)bias[tid] : 0.0);
            s_red[0][tid] = v;
            if (a.logits) a.logits[(size_t)b * N + gg * E + tid] = v;
        }
        __syncthreads();
        // ---- softmax, top-k (lower index wins ties), weights: one thread, scores read from LDS
        if (tid == 0) {
            const double* s = s_red[0];
            uint64_t chosen = 0;
            double mk = -INFINITY, ma = -INFINITY;
            for (int r = 0; r < k; ++r) {
                int best = -1;
                double bv = 0.0;
                for (int e = 0; e < E; ++e) {
                    if ((chosen >> e) & 1) continue;
                    if (best < 0 || s[e] > bv) { best = e; bv = s[e]; }
                }
                chosen |= 1ull << best;
                mk = fmax(mk, bv);
            }
            for (int e = 0; e < E; ++e) ma = fmax(ma, s[e]);
            const double mref = a.renorm ? mk : ma;
            float den = 0.f;
            if (a.renorm) {
                for (int e = 0; e < E; ++e)
                    if ((chosen >> e) & 1) den += expf((float)(s[e] - mref));
            } else {
                for (int e = 0; e < E; ++e) den += expf((float)(s[e] - mref));
            }
            const size_t o = ((size_t)b * G + gg) * k;
            int j = 0;
            for (int e = 0; e < E; ++e) {
                if (!((chosen >> e) & 1)) continue;
                a.sel[o + j] = e;
                a.p_tilde[o + j] = expf((float)(s[e] - mref)) / den;
                s_sel[j] = gg * E + e;
                ++j;
            }
        }
        __syncthreads();
        nsel = k;
    } else {
        if (tid == 0) s_sel[0] = N;
        __syncthreads();
        nsel = 1;
    }

    // ---- projections: each 32-lane group one weight row per pass, 8 rows at a time.
    // 16-byte loads when d_model is a multiple of VEC (always for bf16, whose d_model is a
    // multiple of 64): a lane's chunk is then wholly inside or past the row; else one element a lane.
    const bool vec = dm % VEC == 0;
    const int passes = (dm + PER - 1) / PER;
    for (int j = 0; j < nsel; ++j) {
        const ET* w = (const ET*)a.w_q + (size_t)s_sel[j] * D * dm;
        for (int d0 = 0; d0 < D; d0 += 8) {
            const int d = d0 + grp;
            float acc = 0.f;
            if (vec) {
                const ET* wr = w + (size_t)d * dm + sub * VEC;
                for (int p = 0; p < passes; ++p) {
                    if (sub * VEC + p * PER >= dm) break;
                    const u32x4 wv = ld_u32x4(wr + p * PER);
                    const u32x4 xv = ld_u32x4(xb + sub * VEC + p * PER);
#pragma unroll
                    for (int i = 0; i < VEC; ++i) acc = fmaf(dp_elem<ET>(xv, i), dp_elem<ET>(wv, i), acc);
                }
            } else {
                const ET* wr = w + (size_t)d * dm;
                for (int i = sub; i < dm; i += 32) acc = fmaf(elem_f32(xb[i]), elem_f32(wr[i]), acc);
            }
#pragma unroll
            for (int o = 16; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
            if (sub == 0) s_q[j][d] = acc;
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
