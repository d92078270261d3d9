// Prefill attention of the routed and shared query rows against each group's
// dense KV head, and slot assembly (gfx950).
//
// Attention(Q,K,V) = softmax(QK^T / sqrt(d)) V (GQE study note §1-1), causal
// (key s visible to query t iff s <= t).  Kept experts of group g attend the
// group's single, unchanged KV head (study note §1-2 (3), §3-2 (2)); the
// always-on shared head attends KV head 0 (§3-2 (5)).  Output slots follow
// §3-2 (3)-(5): hard slots, the router-weighted sum, the shared slot.
//
// bf16 kernel design (one workgroup = 4 waves = 128 query rows of one
// (b, head); key tiles of 64):
//   * Within a group the routed queries are a dense [T*k, d] matrix whose row
//     r sits at position r / k, so all k kept rows of a position share every
//     K/V tile staged in LDS -- each K/V tile is loaded once per 128 rows.
//   * The wave computes S^T = K Q^T (32 keys x 32 queries per MFMA block), so a
//     lane owns one query column: the row max and row sum need one exchange
//     with lane l^32 and no LDS.  Q is pre-scaled by log2(e)/sqrt(d), so the
//     softmax is a bare exp2.
//   * P^T feeds O^T = V^T P^T straight from the S^T accumulators.  The order
//     of keys inside a 16-key MFMA step is permuted to match the accumulator
//     layout; V^T is written to LDS in that permuted order, so no shuffle of P
//     is needed.  O^T columns are again owned per lane, so the online-softmax
//     rescale needs no exchange either.
//   * Workgroups are issued longest-first (causal work grows with the query
//     tile) over both the routed tiles (k rows per position) and the shared
//     tiles (one row per position).
#include "gqe_device.h"
#include "gqe_launch.h"

namespace gqe {

constexpr int kPfBM = 128;   // query rows per workgroup (4 waves x 32)
constexpr int kPfBN = 64;    // keys per iteration
constexpr int kPfPad = 8;    // LDS row padding in bf16 elements

struct PfWork {
    int b, h, tile;          // h == G means the shared head
};

// Key tiles needed by query tile i of a head with kk rows per position.
__device__ __forceinline__ int pf_nkv(int i, int kk, int R, int T, int causal)
{
    if (!causal) return (T + kPfBN - 1) / kPfBN;
    const int last_row = min(R - 1, (i + 1) * kPfBM - 1);
    const int t_hi = last_row / kk;
    return t_hi / kPfBN + 1;
}

// Map a workgroup id to (b, head, tile), ordering tiles by decreasing work.
// Routed tiles (B*G of them per tile index) and shared tiles (B per index)
// are merged like two sorted lists.
__device__ __forceinline__ PfWork pf_map(int id, int B, int T, int G, int k, int n_shared, int causal)
{
    const int Rr = T * k, Rs = T;
    int ir = (Rr + kPfBM - 1) / kPfBM - 1;
    int is = n_shared ? (Rs + kPfBM - 1) / kPfBM - 1 : -1;
    PfWork w{0, 0, 0};
    while (true) {
        const int cr = ir >= 0 ? pf_nkv(ir, k, Rr, T, causal) : -1;
        const int cs = is >= 0 ? pf_nkv(is, 1, Rs, T, causal) : -1;
        if (cr >= cs) {
            const int n = B * G;
            if (id < n) { w.b = id / G; w.h = id % G; w.tile = ir; return w; }
            id -= n; --ir;
        } else {
            if (id < B) { w.b = id; w.h = G; w.tile = is; return w; }
            id -= B; --is;
        }
    }
}

__device__ __forceinline__ int swap_bits23(int s) { return (s & ~12) | ((s & 4) << 1) | ((s & 8) >> 1); }

template <int D>
__global__ __launch_bounds__(256) void prefill_bf16_kernel(
    const uint16_t* __restrict__ q_routed, const uint16_t* __restrict__ q_shared, const uint16_t* __restrict__ kg,
    const uint16_t* __restrict__ vg, float* __restrict__ out, int B, int T, int G, int k, int n_shared, int causal,
    int S, float qscale)
{
    const PfWork w = pf_map(blockIdx.x, B, T, G, k, n_shared, causal);
    const bool shared = w.h == G;
    const int kk = shared ? 1 : k;
    const int R = T * kk;
    const int kvh = shared ? 0 : w.h;
    const uint16_t* Q = shared ? q_shared + (size_t)w.b * T * D : q_routed + ((size_t)w.b * G + w.h) * (size_t)R * D;
    const uint16_t* K = kg + ((size_t)w.b * G + kvh) * (size_t)T * D;
    const uint16_t* V = vg + ((size_t)w.b * G + kvh) * (size_t)T * D;
    const int slot0 = shared ? S - 1 : w.h * k;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 31, lh = lane >> 5;
    const int r0 = w.tile * kPfBM;
    const int nkv = pf_nkv(w.tile, kk, R, T, causal);

    // this lane's query row / position
    const int qrow = r0 + wave * 32 + lr;
    const bool qvalid = qrow < R;
    const int tq = qvalid ? qrow / kk : 0;
    // key tiles this wave needs (waves of the first rows of a diagonal tile need fewer)
    const int wrow_hi = min(R - 1, r0 + wave * 32 + 31);
    const int nkv_w = causal ? (wrow_hi / kk) / kPfBN + 1 : nkv;
    const int t_lo_w = (r0 + wave * 32) / kk;

    __shared__ __attribute__((aligned(16))) uint16_t sK[kPfBN][D + kPfPad];
    __shared__ __attribute__((aligned(16))) uint16_t sV[D][kPfBN + kPfPad];

    // Q^T operand: lane holds query column lr, d = 16c + 8*lh .. +8, scaled.
    bf16x8 qf[D / 16];
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
        if (qvalid) {
            const u32x4 raw = ld_u32x4(Q + (size_t)qrow * D + 16 * c + 8 * lh);
            bf16x8 v;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                v[2 * i] = f2bf(bf2f((uint16_t)(raw[i] & 0xffff)) * qscale);
                v[2 * i + 1] = f2bf(bf2f((uint16_t)(raw[i] >> 16)) * qscale);
            }
            qf[c] = v;
        } else {
            qf[c] = bf16x8{};
        }
    }

    constexpr int NCH = kPfBN * D / 8 / 256;  // 16-byte chunks per thread for one K or V tile
    u32x4 rk[NCH], rv[NCH];
    auto load = [&](int kt) {
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            const int c = tid + i * 256, s = c / (D / 8), d0 = (c % (D / 8)) * 8;
            const int pos = kt * kPfBN + s;
            if (pos < T) {
                rk[i] = ld_u32x4(K + (size_t)pos * D + d0);
                rv[i] = ld_u32x4(V + (size_t)pos * D + d0);
            } else {
                rk[i] = u32x4{0, 0, 0, 0};
                rv[i] = u32x4{0, 0, 0, 0};
            }
        }
    };
    auto store = [&]() {
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            const int c = tid + i * 256, s = c / (D / 8), d0 = (c % (D / 8)) * 8;
            *(u32x4*)&sK[s][d0] = rk[i];
            const int sp = swap_bits23(s);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                sV[d0 + 2 * e][sp] = (uint16_t)(rv[i][e] & 0xffff);
                sV[d0 + 2 * e + 1][sp] = (uint16_t)(rv[i][e] >> 16);
            }
        }
    };

    constexpr int NDB = D / 32;
    f32x16 o[NDB];
#pragma unroll
    for (int j = 0; j < NDB; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[j][r] = 0.f;
    float m_run = -INFINITY, l_half = 0.f;

    load(0);
    for (int kt = 0; kt < nkv; ++kt) {
        __syncthreads();
        store();
        __syncthreads();
        if (kt + 1 < nkv) load(kt + 1);
        if (kt >= nkv_w) continue;

        // S^T = K Q^T for two 32-key blocks
        f32x16 s[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
            for (int c = 0; c < D / 16; ++c) {
                const bf16x8 a = ld_bf16x8(&sK[kb * 32 + lr][16 * c + 8 * lh]);
                s[kb] = mfma32(a, qf[c], s[kb]);
            }
        }
        // mask: keys past the causal edge, or past T
        const int s0 = kt * kPfBN;
        const bool need_mask = causal ? (s0 + kPfBN - 1 > t_lo_w) : (s0 + kPfBN > T);
        if (need_mask) {
            const int lim = causal ? tq : T - 1;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = s0 + kb * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
                    if (key > lim) s[kb][r] = -INFINITY;
                }
        }
        float mt = s[0][0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mt = fmaxf(mt, s[0][r]);
#pragma unroll
        for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[1][r]);
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        const float m_new = fmaxf(m_run, mt);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        float ls = 0.f;
        bf16x8 pb[4];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p = __builtin_amdgcn_exp2f(s[kb][r] - m_new);
                ls += p;
                pb[kb * 2 + (r >> 3)][r & 7] = f2bf(p);
            }
        l_half = l_half * alpha + ls;
#pragma unroll
        for (int j = 0; j < NDB; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[j][r] *= alpha;
        // O^T += V^T P^T over the four 16-key steps
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int j = 0; j < NDB; ++j) {
                const bf16x8 a = ld_bf16x8(&sV[j * 32 + lr][16 * c + 8 * lh]);
                o[j] = mfma32(a, pb[c], o[j]);
            }
    }

    if (!qvalid) return;
    const float l = l_half + __shfl_xor(l_half, 32);
    const float inv = 1.f / l;
    const int t = qrow / kk, jj = qrow - t * kk;
    float* dst = out + (((size_t)w.b * T + t) * S + slot0 + jj) * D;
#pragma unroll
    for (int j = 0; j < NDB; ++j)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            const int d = j * 32 + 8 * g4 + 4 * lh;
            f32x4 v = {o[j][4 * g4] * inv, o[j][4 * g4 + 1] * inv, o[j][4 * g4 + 2] * inv, o[j][4 * g4 + 3] * inv};
            *(f32x4*)(dst + d) = v;
        }
}

// fp32 path: one thread per query row, online softmax in fp32.
template <int D>
__global__ __launch_bounds__(128) void prefill_f32_kernel(const float* __restrict__ q_routed,
                                                          const float* __restrict__ q_shared,
                                                          const float* __restrict__ kg, const float* __restrict__ vg,
                                                          float* __restrict__ out, int B, int T, int G, int k,
                                                          int n_shared, int causal, int S)
{
    const int Rr = T * k;
    const long long per_b = (long long)G * Rr + (long long)n_shared * T;
    const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= per_b * B) return;
    const int b = (int)(gid / per_b);
    long long r = gid % per_b;
    const float* q;
    int h, kk, slot, t;
    if (r < (long long)G * Rr) {
        h = (int)(r / Rr);
        const int rr = (int)(r % Rr);
        kk = k; t = rr / k;
        slot = h * k + rr % k;
        q = q_routed + (((size_t)b * G + h) * Rr + rr) * D;
    } else {
        h = 0; kk = 1; t = (int)(r - (long long)G * Rr);
        slot = S - 1;
        q = q_shared + ((size_t)b * T + t) * D;
    }
    (void)kk;
    const float* K = kg + ((size_t)b * G + h) * (size_t)T * D;
    const float* V = vg + ((size_t)b * G + h) * (size_t)T * D;
    const float scale = 1.f / sqrtf((float)D);
    float qv[D], acc[D];
    for (int d = 0; d < D; ++d) { qv[d] = q[d]; acc[d] = 0.f; }
    float m = -INFINITY, l = 0.f;
    const int n_keys = causal ? t + 1 : T;
    for (int s = 0; s < n_keys; ++s) {
        float dot = 0.f;
        for (int d = 0; d < D; ++d) dot = fmaf(qv[d], K[(size_t)s * D + d], dot);
        dot *= scale;
        const float m_new = fmaxf(m, dot);
        const float a = expf(m - m_new), p = expf(dot - m_new);
        l = l * a + p;
        for (int d = 0; d < D; ++d) acc[d] = acc[d] * a + p * V[(size_t)s * D + d];
        m = m_new;
    }
    float* dst = out + (((size_t)b * T + t) * S + slot) * D;
    for (int d = 0; d < D; ++d) dst[d] = acc[d] / l;
}

// Weighted slot(s): sum over g then j of p~ times the hard slots, fp32.
__global__ __launch_bounds__(256) void assemble_kernel(const float* __restrict__ p_tilde, float* __restrict__ out,
                                                       long long n_tok, int G, int k, int D, int S, int route_mode)
{
    const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= n_tok * D) return;
    const long long tok = gid / D;
    const int d = (int)(gid % D);
    float* row = out + (size_t)tok * S * D;
    const float* pt = p_tilde + (size_t)tok * G * k;
    const int kG = k * G;
    if (route_mode == 0) {
        float acc = 0.f;
        for (int g = 0; g < G; ++g)
            for (int j = 0; j < k; ++j) acc = fmaf(pt[g * k + j], row[(size_t)(g * k + j) * D + d], acc);
        row[(size_t)kG * D + d] = acc;
    } else {
        for (int g = 0; g < G; ++g) {
            float acc = 0.f;
            for (int j = 0; j < k; ++j) acc = fmaf(pt[g * k + j], row[(size_t)(g * k + j) * D + d], acc);
            row[(size_t)(kG + g) * D + d] = acc;
        }
    }
}

int launch_assemble(const float* p_tilde, float* out, long long n_tok, int G, int k, int D, int S, int route_mode,
                    hipStream_t st)
{
    const long long n = n_tok * D;
    if (n == 0) return 0;
    assemble_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(p_tilde, out, n_tok, G, k, D, S, route_mode);
    return 0;
}

int launch_prefill(const PrefillArgs& a, hipStream_t st)
{
    const long long BT = (long long)a.B * a.T;
    if (BT == 0) return 0;
    if (a.bf16) {
        const int ntr = (a.T * a.k + kPfBM - 1) / kPfBM;
        const int nts = a.n_shared ? (a.T + kPfBM - 1) / kPfBM : 0;
        const int grid = a.B * (a.G * ntr + nts);
        const float qscale = 1.4426950408889634f / sqrtf((float)a.d_head);
        const uint16_t* qr = (const uint16_t*)a.q_routed;
        const uint16_t* qs = (const uint16_t*)a.q_shared;
        const uint16_t* k = (const uint16_t*)a.kmat;
        const uint16_t* v = (const uint16_t*)a.vmat;
        switch (a.d_head) {
        case 32: prefill_bf16_kernel<32><<<grid, 256, 0, st>>>(qr, qs, k, v, a.out, a.B, a.T, a.G, a.k, a.n_shared, a.causal, a.S, qscale); break;
        case 64: prefill_bf16_kernel<64><<<grid, 256, 0, st>>>(qr, qs, k, v, a.out, a.B, a.T, a.G, a.k, a.n_shared, a.causal, a.S, qscale); break;
        case 128: prefill_bf16_kernel<128><<<grid, 256, 0, st>>>(qr, qs, k, v, a.out, a.B, a.T, a.G, a.k, a.n_shared, a.causal, a.S, qscale); break;
        default: return -2;
        }
    } else {
        const long long rows = BT * ((long long)a.G * a.k + a.n_shared);
        const unsigned grid = (unsigned)((rows + 127) / 128);
        const float* qr = (const float*)a.q_routed;
        const float* qs = (const float*)a.q_shared;
        const float* k = (const float*)a.kmat;
        const float* v = (const float*)a.vmat;
        switch (a.d_head) {
        case 32: prefill_f32_kernel<32><<<grid, 128, 0, st>>>(qr, qs, k, v, a.out, a.B, a.T, a.G, a.k, a.n_shared, a.causal, a.S); break;
        case 64: prefill_f32_kernel<64><<<grid, 128, 0, st>>>(qr, qs, k, v, a.out, a.B, a.T, a.G, a.k, a.n_shared, a.causal, a.S); break;
        case 128: prefill_f32_kernel<128><<<grid, 128, 0, st>>>(qr, qs, k, v, a.out, a.B, a.T, a.G, a.k, a.n_shared, a.causal, a.S); break;
        default: return -2;
        }
    }
    if (hipGetLastError() != hipSuccess) return -1;
    launch_assemble(a.p_tilde, a.out, BT, a.G, a.k, a.d_head, a.S, a.route_mode, st);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace gqe
