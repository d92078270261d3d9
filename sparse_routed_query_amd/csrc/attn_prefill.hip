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
__device__ __forceinline__ int pf_nkv(int i, int kk, int R, int T, int causal, int bn = kPfBN)
{
    if (!causal) return (T + bn - 1) / bn;
    const int last_row = min(R - 1, (i + 1) * kPfBM - 1);
    const int t_hi = last_row / kk;
    return t_hi / bn + 1;
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

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two transposing LDS reads give the V^T operand of a 32x32x16 MFMA.  Within
// each 16-lane group, lane i of ds_read_b64_tr_b16 receives element (i % 4) of
// the 8-byte chunk addressed by lane 4*j + i/4, as its element j.  Source lane
// s = 4*j + q therefore points at V[key_j][d0 + 4q .. 4q+3] so that lane i ends
// up holding V[key_0..3][d0 + i].  The caller folds the per-lane part of that
// address into `off`.
__device__ __forceinline__ bf16x8 load_vt(const uint16_t* base, int off, int pitch8)
{
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + off));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + off + pitch8));
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
}

// Lanes l and l^32 own the same query column.  (v_permlane32_swap would avoid
// the LDS round trip, but inside this loop it returned stale values on gfx950
// with this compiler, so the exchange goes through ds_bpermute.)
__device__ __forceinline__ float half_max(float v) { return fmaxf(v, __shfl_xor(v, 32)); }
__device__ __forceinline__ float half_sum(float v) { return v + __shfl_xor(v, 32); }

__device__ __forceinline__ uint32_t pk_bf16(float a, float b)
{
    const f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Softmax reference threshold: the running reference m_ref only moves when a
// tile's scores exceed it by more than 2^8, so probabilities stay <= 256 and
// most tiles need neither a subtraction nor a rescale of the accumulators.
constexpr float kPfRescale = 8.0f;
constexpr float kPfRescaleSum = 256.0f;   // 2^kPfRescale

template <int D>
__global__ __launch_bounds__(256) void prefill_bf16_kernel(
    const uint16_t* __restrict__ q_routed, const uint16_t* __restrict__ q_shared, const uint16_t* __restrict__ kg,
    const uint16_t* __restrict__ vg, float* __restrict__ out, int B, int T, int G, int k, int n_shared, int causal,
    int S, float qscale)
{
    constexpr int P = D + kPfPad;           // LDS row pitch (elements)
    constexpr int NDB = D / 32;
    constexpr int NCH = kPfBN * D / 8 / 256; // 16-byte chunks per thread for one K or V tile
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

    const int qrow = r0 + wave * 32 + lr;
    const bool qvalid = qrow < R;
    const int tq = qvalid ? qrow / kk : 0;   // invalid rows see key 0 only, so they stay finite
    const int wrow_hi = min(R - 1, r0 + wave * 32 + 31);
    const int nkv_w = causal ? (wrow_hi / kk) / kPfBN + 1 : nkv;
    const int t_lo_w = (r0 + wave * 32) / kk;

    // V rows get 32 elements of padding: the transposing reads are then free of
    // bank conflicts (16 for K rows, read with 16-byte loads).
    constexpr int PV = D + 32;
    __shared__ __attribute__((aligned(16))) uint16_t sK[2][kPfBN * P];
    __shared__ __attribute__((aligned(16))) uint16_t sV[2][kPfBN * PV];

    // Q loads (rows past R read row R-1 and are zeroed) are issued together
    // with the first K/V tile's, so the prologue waits for memory once
    u32x4 qraw[D / 16];
    {
        const uint16_t* qsrc = Q + (size_t)min(qrow, R - 1) * D + 8 * lh;
#pragma unroll
        for (int c = 0; c < D / 16; ++c) qraw[c] = ld_u32x4(qsrc + 16 * c);
    }

    u32x4 rk[NCH], rv[NCH];
    // Keys past T are loaded from row T-1 instead: their scores are masked, so
    // their probabilities are exactly 0 and the (finite) values never count.
    auto load = [&](int kt) {
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            const int c = tid + i * 256, s = c / (D / 8), d0 = (c % (D / 8)) * 8;
            const int pos = min(kt * kPfBN + s, T - 1);
            rk[i] = ld_u32x4(K + (size_t)pos * D + d0);
            rv[i] = ld_u32x4(V + (size_t)pos * D + d0);
        }
    };
    auto store = [&](int buf) {
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            const int c = tid + i * 256, s = c / (D / 8), d0 = (c % (D / 8)) * 8;
            *(u32x4*)&sK[buf][s * P + d0] = rk[i];
            *(u32x4*)&sV[buf][s * PV + d0] = rv[i];
        }
    };
    // per-lane parts of the LDS addresses
    const int k_off = lr * P + 8 * lh;                                       // K row lr, d half lh
    const int s16 = lane & 15;
    const int v_off = (4 * lh + (s16 >> 2)) * PV + 16 * ((lane >> 4) & 1) + 4 * (s16 & 3);

    f32x16 o[NDB];
#pragma unroll
    for (int j = 0; j < NDB; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[j][r] = 0.f;
    float m_ref = 0.f, l_half = 0.f;
    f32x16 cneg;
#pragma unroll
    for (int r = 0; r < 16; ++r) cneg[r] = 0.f;

    load(0);
    bf16x8 qf[D / 16];
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
        bf16x8 v = {};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = f2bf(bf2f((uint16_t)(qraw[c][i] & 0xffff)) * qscale);
            v[2 * i + 1] = f2bf(bf2f((uint16_t)(qraw[c][i] >> 16)) * qscale);
        }
        qf[c] = qvalid ? v : bf16x8{};
        // pin the Q fragments here, ahead of the first tile's store: the Q loads
        // are then in flight together with the tile loads, not issued after them
        asm volatile("" ::"v"(qf[c]));
    }
    store(0);
    __syncthreads();
    for (int kt = 0; kt < nkv; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nkv) load(kt + 1);
        if (kt < nkv_w) {
            const uint16_t* bK = sK[buf];
            const uint16_t* bV = sV[buf];
            // S^T - m_ref = K Q^T + cneg for two 32-key blocks
            f32x16 s[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                s[kb] = mfma32(ld_bf16x8(bK + k_off + kb * 32 * P), qf[0], cneg);
#pragma unroll
                for (int c = 1; c < D / 16; ++c) s[kb] = mfma32(ld_bf16x8(bK + k_off + kb * 32 * P + 16 * c), qf[c], s[kb]);
            }
            const int s0 = kt * kPfBN;
            const bool need_mask = causal ? (s0 + kPfBN - 1 > t_lo_w) : (s0 + kPfBN > T);
            if (need_mask) {
                // key of element r in block kb is s0 + 4*lh + (kb*32 + 8*(r/4) + r%4)
                const int lim = (causal ? tq : T - 1) - s0 - 4 * lh;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        s[kb][r] = (kb * 32 + 8 * (r >> 2) + (r & 3)) > lim ? -INFINITY : s[kb][r];
            }
            // P = exp2(S - m_ref), packed to bf16; the row sum uses the rounded values.
            // If no lane's partial row sum exceeds 2^8, no probability does, so the
            // reference stays and the row max is never computed.  The first tile,
            // and any tile whose sum trips that check, take the exact path: row
            // max, move the reference if it jumped by more than 2^8, recompute.
            uint32_t pw[16];
            const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};
            auto probs = [&]() {
                float ls = 0.f;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; r += 2)
                        pw[kb * 8 + r / 2] = pk_bf16(__builtin_amdgcn_exp2f(s[kb][r]), __builtin_amdgcn_exp2f(s[kb][r + 1]));
#pragma unroll
                for (int i = 0; i < 16; ++i) ls = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pw[i]), ones, ls, false);
                return ls;
            };
            bool exact = kt == 0;
            if (!exact) {
                const float ls = probs();
                exact = __ballot(!(ls <= kPfRescaleSum)) != 0;
                if (!exact) l_half += ls;
            }
            if (exact) {
                // chained form so the compiler emits v_max3_f32
                float mt = s[0][0];
#pragma unroll
                for (int r = 1; r < 15; r += 2) mt = fmaxf(fmaxf(mt, s[0][r]), s[0][r + 1]);
                mt = fmaxf(fmaxf(mt, s[0][15]), s[1][0]);
#pragma unroll
                for (int r = 1; r < 15; r += 2) mt = fmaxf(fmaxf(mt, s[1][r]), s[1][r + 1]);
                mt = fmaxf(mt, s[1][15]);
                mt = half_max(mt);
                // first tile: set the reference; later tiles: move it only on a large jump
                const bool move = kt == 0 ? true : mt > kPfRescale;
                if (__ballot(move)) {
                    const float shift = move ? mt : 0.f;
                    const float alpha = kt == 0 ? 0.f : __builtin_amdgcn_exp2f(-shift);
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                        for (int r = 0; r < 16; ++r) s[kb][r] -= shift;
#pragma unroll
                    for (int j = 0; j < NDB; ++j)
#pragma unroll
                        for (int r = 0; r < 16; ++r) o[j][r] *= alpha;
                    l_half *= alpha;
                    m_ref += shift;
#pragma unroll
                    for (int r = 0; r < 16; ++r) cneg[r] = -m_ref;
                }
                l_half += probs();
            }
            // O^T += V^T P^T over the four 16-key steps
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const u32x4 pv = {pw[4 * c], pw[4 * c + 1], pw[4 * c + 2], pw[4 * c + 3]};
                const bf16x8 pb = __builtin_bit_cast(bf16x8, pv);
#pragma unroll
                for (int j = 0; j < NDB; ++j) o[j] = mfma32(load_vt(bV, v_off + 16 * c * PV + 32 * j, 8 * PV), pb, o[j]);
            }
        }
        if (kt + 1 < nkv) store(buf ^ 1);
        __syncthreads();
    }

    if (!qvalid) return;
    const float l = half_sum(l_half);
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
    int h, slot, t;
    if (r < (long long)G * Rr) {
        h = (int)(r / Rr);
        const int rr = (int)(r % Rr);
        t = rr / k;
        slot = h * k + rr % k;
        q = q_routed + (((size_t)b * G + h) * Rr + rr) * D;
    } else {
        h = 0; t = (int)(r - (long long)G * Rr);
        slot = S - 1;
        q = q_shared + ((size_t)b * T + t) * D;
    }
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

// Weighted slot(s): sum over g then j of p~ times the hard slots, fp32, in
// that fixed order.  One thread per 4 consecutive d of a token (16-byte
// accesses); the loads of up to 8 hard slots are issued before their FMAs.
__global__ __launch_bounds__(256) void assemble_kernel(const float* __restrict__ p_tilde, float* __restrict__ out,
                                                       long long n_tok, int G, int k, int D, int S, int route_mode)
{
    const int DQ = D / 4;
    const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= n_tok * DQ) return;
    const long long tok = gid / DQ;
    const int d = (int)(gid % DQ) * 4;
    float* row = out + (size_t)tok * S * D + d;
    const float* pt = p_tilde + (size_t)tok * G * k;
    const int kG = k * G;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int h0 = 0; h0 < kG; h0 += 8) {
        f32x4 v[8];
        float w[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int h = min(h0 + i, kG - 1);
            v[i] = *(const f32x4*)(row + (size_t)h * D);
            w[i] = pt[h];
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int h = h0 + i;
            if (h >= kG) break;
            acc[0] = fmaf(w[i], v[i][0], acc[0]);
            acc[1] = fmaf(w[i], v[i][1], acc[1]);
            acc[2] = fmaf(w[i], v[i][2], acc[2]);
            acc[3] = fmaf(w[i], v[i][3], acc[3]);
            if (route_mode == 1 && (h + 1) % k == 0) {    // end of group h / k
                *(f32x4*)(row + (size_t)(kG + h / k) * D) = acc;
                acc = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
    }
    if (route_mode == 0) *(f32x4*)(row + (size_t)kG * D) = acc;
}

int launch_assemble(const float* p_tilde, float* out, long long n_tok, int G, int k, int D, int S, int route_mode,
                    hipStream_t st)
{
    const long long n = n_tok * (D / 4);
    if (n == 0) return 0;
    assemble_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(p_tilde, out, n_tok, G, k, D, S, route_mode);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_prefill_heads(const PrefillArgs& a, hipStream_t st)
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
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_prefill(const PrefillArgs& a, hipStream_t st)
{
    const int rc = launch_prefill_heads(a, st);
    if (rc != 0) return rc;
    return launch_assemble(a.p_tilde, a.out, (long long)a.B * a.T, a.G, a.k, a.d_head, a.S, a.route_mode, st);
}

}  // namespace gqe
