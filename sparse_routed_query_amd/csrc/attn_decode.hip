// Decode attention: one new token per sequence against a dense KV cache
// (gfx950).  Decode reads the whole cache for every step, so it is bound by
// memory bandwidth (GQA tutorial, freeguideonline, "自回归推理中的内存带宽优势");
// GQE leaves the KV path unchanged, so every KV head is read (GQE study note
// §1-2 (3), §5-3 (2)).  Only kept experts (and the shared head, on KV head 0)
// attend.
//
// split kernel:   grid (key chunk, group, sequence).  A workgroup streams one
//                 chunk of K and V of one (b, g) with 16-byte loads issued all
//                 at once, then serves every query row of that group from
//                 registers (k kept rows, plus the shared row on group 0), so
//                 each cached byte is read once.  It writes (max, sum, o) of
//                 the chunk in base-2 units.
// merge kernel:   one workgroup per sequence merges each row's chunks in
//                 chunk order (deterministic) into its hard or shared slot
//                 and then forms the weighted slot(s) from those hard slots.
#include "gqe_device.h"
#include "gqe_launch.h"

namespace gqe {

constexpr int kDcPasses = 8;   // 16-byte loads per thread for each of K and V

template <typename ET, int D>
struct DcShape {
    static constexpr int VEC = 16 / sizeof(ET);    // elements per 16-byte load
    static constexpr int LPP = D / VEC;            // lanes per key position
    static constexpr int PPP = 256 / LPP;          // positions per pass
    static constexpr int CH = PPP * kDcPasses;     // keys per chunk
};

__device__ __forceinline__ float elem(const u32x4& v, int i, const uint16_t*)
{
    const uint32_t w = v[i >> 1];
    return bf2f((uint16_t)((i & 1) ? (w >> 16) : (w & 0xffff)));
}
__device__ __forceinline__ float elem(const u32x4& v, int i, const float*) { return __uint_as_float(v[i]); }

template <typename ET, int D>
__global__ __launch_bounds__(256) void decode_split_kernel(const ET* __restrict__ q_routed,
                                                           const ET* __restrict__ q_shared,
                                                           const ET* __restrict__ kc, const ET* __restrict__ vc,
                                                           const int32_t* __restrict__ lens, float* __restrict__ part,
                                                           int G, int k, int n_shared, int L_max, int nch,
                                                           float qscale)
{
    using SH = DcShape<ET, D>;
    constexpr int VEC = SH::VEC, LPP = SH::LPP, PPP = SH::PPP, CH = SH::CH;
    const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int L = min(max(lens[b], 0), L_max);   // never read outside the cache
    const int c0 = c * CH;
    if (c0 >= L) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int dq = (tid % LPP) * VEC;
    const int pp = tid / LPP;
    const ET* K = kc + ((size_t)b * G + g) * (size_t)L_max * D;
    const ET* V = vc + ((size_t)b * G + g) * (size_t)L_max * D;

    u32x4 kr[kDcPasses], vr[kDcPasses];
#pragma unroll
    for (int i = 0; i < kDcPasses; ++i) {
        const int pos = c0 + i * PPP + pp;
        if (pos < L) {
            // the cache is read once per step: non-temporal loads keep it from
            // displacing other data in the caches
            kr[i] = __builtin_nontemporal_load((const u32x4*)(K + (size_t)pos * D + dq));
            vr[i] = __builtin_nontemporal_load((const u32x4*)(V + (size_t)pos * D + dq));
        } else {
            kr[i] = u32x4{0, 0, 0, 0};
            vr[i] = u32x4{0, 0, 0, 0};
        }
    }

    __shared__ float s_red[4][D + 2];
    const int RG = k + n_shared;
    const int nrows = k + ((g == 0 && n_shared) ? 1 : 0);
    for (int row = 0; row < nrows; ++row) {
        const ET* q = row < k ? q_routed + (((size_t)b * G + g) * k + row) * D : q_shared + (size_t)b * D;
        float qv[VEC];
        {
            const u32x4 raw = ld_u32x4(q + dq);
#pragma unroll
            for (int v = 0; v < VEC; ++v) qv[v] = elem(raw, v, (const ET*)nullptr) * qscale;
        }
        float sc[kDcPasses];
        float m = -INFINITY;
#pragma unroll
        for (int i = 0; i < kDcPasses; ++i) {
            float dot = 0.f;
#pragma unroll
            for (int v = 0; v < VEC; ++v) dot = fmaf(qv[v], elem(kr[i], v, (const ET*)nullptr), dot);
#pragma unroll
            for (int o = 1; o < LPP; o <<= 1) dot += __shfl_xor(dot, o);
            const int pos = c0 + i * PPP + pp;
            sc[i] = pos < L ? dot : -INFINITY;
            m = fmaxf(m, sc[i]);
        }
#pragma unroll
        for (int o = LPP; o < 64; o <<= 1) m = fmaxf(m, __shfl_xor(m, o));
        if (lane == 0) s_red[wave][D] = m;
        __syncthreads();
        m = fmaxf(fmaxf(s_red[0][D], s_red[1][D]), fmaxf(s_red[2][D], s_red[3][D]));
        float l = 0.f, acc[VEC];
#pragma unroll
        for (int v = 0; v < VEC; ++v) acc[v] = 0.f;
#pragma unroll
        for (int i = 0; i < kDcPasses; ++i) {
            const float p = __builtin_amdgcn_exp2f(sc[i] - m);
            l += p;
#pragma unroll
            for (int v = 0; v < VEC; ++v) acc[v] = fmaf(p, elem(vr[i], v, (const ET*)nullptr), acc[v]);
        }
#pragma unroll
        for (int o = LPP; o < 64; o <<= 1) {
            l += __shfl_xor(l, o);
#pragma unroll
            for (int v = 0; v < VEC; ++v) acc[v] += __shfl_xor(acc[v], o);
        }
        if (lane < LPP) {
#pragma unroll
            for (int v = 0; v < VEC; ++v) s_red[wave][dq + v] = acc[v];
        }
        if (lane == 0) s_red[wave][D + 1] = l;
        __syncthreads();
        float* dst = part + ((((size_t)b * G + g) * RG + row) * nch + c) * (D + 2);
        if (tid < D) dst[2 + tid] = s_red[0][tid] + s_red[1][tid] + s_red[2][tid] + s_red[3][tid];
        if (tid == 0) {
            dst[0] = m;
            dst[1] = s_red[0][D + 1] + s_red[1][D + 1] + s_red[2][D + 1] + s_red[3][D + 1];
        }
        __syncthreads();
    }
}

// One workgroup per sequence: each wave merges the chunk partials of some of
// the sequence's query rows (in chunk order, so the result does not depend on
// timing) into their hard or shared slot, keeping the hard slots in LDS; the
// weighted slot(s) are then summed from LDS in fixed g-then-j order, exactly
// as the slot-assembly kernel does from memory.
constexpr int kDcMergeWaves = 16;
constexpr int kDcMergeRegs = 32;          // value registers per lane for merging a row from registers

template <int D>
__global__ __launch_bounds__(64 * kDcMergeWaves) void decode_merge_kernel(
    const float* __restrict__ part, const int32_t* __restrict__ lens, const float* __restrict__ p_tilde,
    float* __restrict__ out, int G, int k, int n_shared, int S, int route_mode, int nch, int CH)
{
    extern __shared__ float s_hard[];       // [k*G][D]
    const int b = blockIdx.x, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int kG = G * k;
    const int RG = k + n_shared;
    const int L = min(max(lens[b], 0), nch * CH);
    const int nc = (L + CH - 1) / CH;
    for (int row = wave; row < kG + n_shared; row += kDcMergeWaves) {
        const int g = row < kG ? row / k : 0;
        const int r = row < kG ? row % k : k;
        const float* pp = part + (((size_t)b * G + g) * RG + r) * (size_t)nch * (D + 2);
        constexpr int ND = (D + 63) / 64;          // value columns per lane
        constexpr int FAST = kDcMergeRegs / ND;    // rows with at most this many chunks merge from registers
        float Ls = 0.f;
        float O[ND];
#pragma unroll
        for (int i = 0; i < ND; ++i) O[i] = 0.f;
        if (nc <= FAST) {
            // every partial of the row is loaded at once (one memory round trip):
            // lane c holds chunk c's (max, sum); value rows of every chunk are
            // held per lane (chunks past nc repeat chunk nc-1 and are not used)
            float m = -INFINITY, l = 0.f;
            if (lane < nc) {
                m = pp[(size_t)lane * (D + 2)];
                l = pp[(size_t)lane * (D + 2) + 1];
            }
            float ov[FAST][ND];
#pragma unroll
            for (int c = 0; c < FAST; ++c)
#pragma unroll
                for (int i = 0; i < ND; ++i) {
                    const int d = min(64 * i + lane, D - 1);
                    ov[c][i] = pp[(size_t)min(c, nc - 1) * (D + 2) + 2 + d];
                }
            const float M = wave_max(m);
            const float wgt = lane < nc ? __builtin_amdgcn_exp2f(m - M) : 0.f;
            Ls = l * wgt;
#pragma unroll
            for (int c = 0; c < FAST; ++c) {
                if (c >= nc) break;
                const float wi = __shfl(wgt, c);
#pragma unroll
                for (int i = 0; i < ND; ++i) O[i] = fmaf(ov[c][i], wi, O[i]);
            }
        } else {
            // pass 1: the largest chunk maximum
            float M = -INFINITY;
            for (int c = lane; c < nc; c += 64) M = fmaxf(M, pp[(size_t)c * (D + 2)]);
            M = wave_max(M);
            // pass 2, 64 chunks at a time: lane c forms chunk c's weight; the
            // weighted value rows are added in chunk order
            for (int c0 = 0; c0 < nc; c0 += 64) {
                const int c = c0 + lane;
                float wgt = 0.f;
                if (c < nc) {
                    wgt = __builtin_amdgcn_exp2f(pp[(size_t)c * (D + 2)] - M);
                    Ls += pp[(size_t)c * (D + 2) + 1] * wgt;
                }
                const int n = min(64, nc - c0);
                for (int i = 0; i < n; ++i) {
                    const float wi = __shfl(wgt, i);
                    const float* q = pp + (size_t)(c0 + i) * (D + 2) + 2;
#pragma unroll
                    for (int d0 = 0; d0 < D; d0 += 64)
                        if (d0 + lane < D) O[d0 / 64] = fmaf(q[d0 + lane], wi, O[d0 / 64]);
                }
            }
        }
        Ls = wave_sum(Ls);
        const float inv = 1.f / Ls;
        float* dst = out + ((size_t)b * S + (row < kG ? row : S - 1)) * D;
#pragma unroll
        for (int d0 = 0; d0 < D; d0 += 64) {
            const int d = d0 + lane;
            if (d < D) {
                const float v = O[d0 / 64] * inv;
                dst[d] = v;
                if (row < kG) s_hard[row * D + d] = v;
            }
        }
    }
    __syncthreads();
    // weighted slot(s)
    const float* pt = p_tilde + (size_t)b * kG;
    float* orow = out + (size_t)b * S * D;
    for (int d = threadIdx.x; d < D; d += 64 * kDcMergeWaves) {
        if (route_mode == 0) {
            float acc = 0.f;
            for (int h = 0; h < kG; ++h) acc = fmaf(pt[h], s_hard[h * D + d], acc);
            orow[(size_t)kG * D + d] = acc;
        } else {
            for (int g = 0; g < G; ++g) {
                float acc = 0.f;
                for (int j = 0; j < k; ++j) acc = fmaf(pt[g * k + j], s_hard[(g * k + j) * D + d], acc);
                orow[(size_t)(kG + g) * D + d] = acc;
            }
        }
    }
}

template <typename ET, int D>
static int decode_chunk()
{
    return DcShape<ET, D>::CH;
}

static int decode_chunk_for(int d_head, bool bf16)
{
    if (bf16) return d_head == 32 ? decode_chunk<uint16_t, 32>() : d_head == 64 ? decode_chunk<uint16_t, 64>() : decode_chunk<uint16_t, 128>();
    return d_head == 32 ? decode_chunk<float, 32>() : d_head == 64 ? decode_chunk<float, 64>() : decode_chunk<float, 128>();
}

size_t decode_workspace_bytes(int B, int G, int k, int n_shared, int d_head, int L_max, bool bf16)
{
    const int CH = decode_chunk_for(d_head, bf16);
    const size_t nch = (size_t)(L_max + CH - 1) / CH;
    return (size_t)B * G * (k + n_shared) * nch * (d_head + 2) * sizeof(float) + 256;
}

template <typename ET, int D>
static void launch_decode_t(const DecodeArgs& a, hipStream_t st)
{
    constexpr int CH = DcShape<ET, D>::CH;
    const int nch = (a.L_max + CH - 1) / CH;
    const float qscale = 1.4426950408889634f / sqrtf((float)D);
    dim3 grid(nch, a.G, a.B);
    decode_split_kernel<ET, D><<<grid, 256, 0, st>>>((const ET*)a.q_routed, (const ET*)a.q_shared, (const ET*)a.k_cache,
                                                     (const ET*)a.v_cache, a.lens, (float*)a.workspace, a.G, a.k,
                                                     a.n_shared, a.L_max, nch, qscale);
    const size_t lds = (size_t)a.G * a.k * D * sizeof(float);
    decode_merge_kernel<D><<<a.B, 64 * kDcMergeWaves, lds, st>>>((const float*)a.workspace, a.lens, a.p_tilde, a.out,
                                                                 a.G, a.k, a.n_shared, a.S, a.route_mode, nch, CH);
}

int launch_decode(const DecodeArgs& a, hipStream_t st)
{
    if (a.B == 0) return 0;
    if (a.bf16) {
        switch (a.d_head) {
        case 32: launch_decode_t<uint16_t, 32>(a, st); break;
        case 64: launch_decode_t<uint16_t, 64>(a, st); break;
        case 128: launch_decode_t<uint16_t, 128>(a, st); break;
        default: return -2;
        }
    } else {
        switch (a.d_head) {
        case 32: launch_decode_t<float, 32>(a, st); break;
        case 64: launch_decode_t<float, 64>(a, st); break;
        case 128: launch_decode_t<float, 128>(a, st); break;
        default: return -2;
        }
    }
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace gqe
