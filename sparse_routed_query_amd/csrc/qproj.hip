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

// Projections of one launch.  Expert indices: [0, N) the routed experts
// (W_q rows n, compacted rows), then ns shared heads (W_q row block N), then
// nkv K heads and nkv V heads (W_k, W_v), the dense ones over every token.
struct QpArgs {
    const uint16_t* x;            // bf16 kernel; the fp32 kernel reads xf etc.
    const void* w_q;
    const void* w_k;
    const void* w_v;
    const int32_t* sel;
    const int32_t* counts;
    const int32_t* offsets;
    const int32_t* rows;
    void* q_routed;               // NULL: the routed experts are left out
    void* q_shared;               // [B, T, d_head]
    void* k_out;                  // [B, nkv, T, d_head]
    void* v_out;
    const int32_t* positions;     // [B*T] rotary positions, NULL: t
    int B, T, d_model, G, E, k, ns, nkv;
    double rope_log2_base;        // > 0: rotate q (routed, shared) and K by the rotary embedding
};

__host__ __device__ __forceinline__ int qp_n_exp(const QpArgs& a) { return a.G * a.E + a.ns + 2 * a.nkv; }

// Kind of expert n: 0 routed, 1 shared, 2 K head, 3 V head; h = the head within its kind.
__device__ __forceinline__ int qp_kind(const QpArgs& a, int n, int& h)
{
    const int N = a.G * a.E;
    if (n < N) { h = n; return 0; }
    n -= N;
    if (n < a.ns) { h = n; return 1; }
    n -= a.ns;
    if (n < a.nkv) { h = n; return 2; }
    h = n - a.nkv;
    return 3;
}

// Destination element offset of row r of expert n's bucket (token tok).
__device__ __forceinline__ size_t qp_dst(const QpArgs& a, int kind, int h, int n, int tok, int d_head)
{
    const int b = tok / a.T, t = tok - b * a.T;
    if (kind == 1) return ((size_t)b * a.T + t) * d_head;
    if (kind >= 2) return (((size_t)b * a.nkv + h) * a.T + t) * d_head;
    const int g = n / a.E, e = n - g * a.E;
    const int32_t* s = a.sel + ((size_t)tok * a.G + g) * a.k;
    int j = 0;
    for (int i = 0; i < a.k; ++i) j = s[i] == e ? i : j;
    return ((((size_t)b * a.G + g) * a.T + t) * a.k + j) * d_head;
}

__device__ __forceinline__ double qp_rope_freq(int i, int d_head, double log2_base)
{
    return rope_freq(i, d_head, log2_base);
}
__device__ __forceinline__ float qp_rope_angle(int pos, double freq) { return rope_angle(pos, freq); }

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

__device__ bool qp_plan(int bid, const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets, int N,
                        int n_exp, int BT, bool routed, int BM, int lane, int& n_out, int& tile_out, int& m_out,
                        int& base_out)
{
    // n_exp <= 128: two candidate experts per lane, with their row counts and bucket starts (loaded together,
    // so the chosen expert's need no second round trip)
    auto rows_of = [&](int n) { return n >= n_exp || (n < N && !routed) ? 0 : n < N ? counts[n] : BT; };
    auto start_of = [&](int n) { return n < N && routed ? offsets[n] : 0; };
    const int m0 = rows_of(lane), m1 = rows_of(lane + 64);
    const int s0 = start_of(lane), s1 = start_of(lane + 64);
    const int c0 = (m0 + BM - 1) / BM, c1 = (m1 + BM - 1) / BM;
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
        m_out = __shfl(m0, ln);
        base_out = __shfl(s0, ln);
    } else {
        rem -= t0;
        const int p1 = wave_scan_i(k1, lane);
        const unsigned long long m = __ballot(p1 > rem);
        const int ln = __ffsll((long long)m) - 1;
        n = ln + 64;
        tile = __shfl(b1, ln) + rem - (__shfl(p1, ln) - __shfl(k1, ln));
        m_out = __shfl(m1, ln);
        base_out = __shfl(s1, ln);
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
// weight slice are loaded with 16-byte coalesced loads (8 lanes per 128-byte
// row segment) into registers while the previous stage is multiplied out of
// LDS, then stored to LDS (d_head <= 64: one buffer between two barriers;
// 128: the other of two buffers, mid-stage, one barrier).  Rows past the
// bucket's end reload its last row and are not stored, so every load is
// unconditional.  The epilogue applies the rotary embedding in fp32 where
// asked (pairs (c, c + D/2) of a row, which a lane holds in blocks j and
// j + NB/2, or at D = 32 in lanes l and l ^ 16), rounds once to bf16 and
// writes each row through LDS as 16-byte stores.
template <int D, int BK>
__global__ __launch_bounds__(QpNT<D>::NT) void qproj_bf16_kernel(const QpArgs a)
{
    constexpr int NT = QpNT<D>::NT, BM = QpNT<D>::BM;
    const int N = a.G * a.E, BT = a.B * a.T, n_exp = qp_n_exp(a), d_model = a.d_model;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    __shared__ int s_item[4];
    if (wave == 0) {
        int pn = -1, pt = 0, pm = 0, pb = 0;
        if (!qp_plan(blockIdx.x, a.counts, a.offsets, N, n_exp, BT, a.q_routed != nullptr, BM, lane, pn, pt, pm, pb))
            pn = -1;
        if (lane == 0) { s_item[0] = pn; s_item[1] = pt; s_item[2] = pm; s_item[3] = pb; }
    }
    __syncthreads();
    const int n = s_item[0];
    if (n < 0) return;
    int h;
    const int kind = qp_kind(a, n, h);
    const int row0 = s_item[1] * BM, M = s_item[2], base = s_item[3];
    const uint16_t* wsrc = kind <= 1 ? (const uint16_t*)a.w_q + (size_t)(kind == 0 ? n : N + h) * D * d_model
                                     : (const uint16_t*)(kind == 2 ? a.w_k : a.w_v) + (size_t)h * D * d_model;
    constexpr int P = BK + kQpPad;
    constexpr int NB = D / 32;
    constexpr int CPR = BK / 8;                           // 16-byte chunks per row of a stage
    constexpr int ACH = BM * CPR / NT;                    // A chunks per thread
    constexpr int BCH = D * CPR / NT;                     // B chunks per thread
    // the stages of x rows and weight rows in LDS: at d_head 128 two, used in turn with one barrier per
    // stage (one workgroup of eight waves per compute unit); below, one stage between two barriers, which
    // keeps more workgroups on a compute unit (two buffers cost 10 % at d_head 64 and gain 17 % at 128)
    constexpr bool DB = D >= 128;
    constexpr int STG = (BM + D) * P;
    __shared__ __attribute__((aligned(16))) uint16_t sS[(DB ? 2 : 1) * STG];
    uint16_t* const sA = sS;   // stage 0's x rows; the epilogue's regions

    // row pointers of this thread's A chunks (rows tid / CPR + i * 256 / CPR)
    const int col = (tid % CPR) * 8;
    const uint16_t* pa[ACH];
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
        const int rr = min(row0 + tid / CPR + i * (NT / CPR), M - 1);
        const int tok = kind == 0 ? a.rows[base + rr] : rr;
        pa[i] = a.x + (size_t)tok * d_model + col;
    }
    const uint16_t* pb = wsrc + (size_t)(tid / CPR) * d_model + col;
    u32x4 ra[ACH], rb[BCH];
    auto load = [&](int k0) {
#pragma unroll
        for (int i = 0; i < ACH; ++i) ra[i] = ld_u32x4(pa[i] + k0);
#pragma unroll
        for (int i = 0; i < BCH; ++i) rb[i] = ld_u32x4(pb + (size_t)i * (NT / CPR) * d_model + k0);
    };
    const int w_off = (tid / CPR) * P + col;
    auto store = [&](uint16_t* buf) {
#pragma unroll
        for (int i = 0; i < ACH; ++i) *(u32x4*)&buf[w_off + i * (NT / CPR) * P] = ra[i];
#pragma unroll
        for (int i = 0; i < BCH; ++i) *(u32x4*)&buf[BM * P + w_off + i * (NT / CPR) * P] = rb[i];
    };

    f32x16 acc[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;

    const int nst = d_model / BK;
    const int a_off = (wave * 32 + (lane & 31)) * P + 8 * (lane >> 5);
    const int b_off = (lane & 31) * P + 8 * (lane >> 5);
    auto mma = [&](const uint16_t* buf, int kk) {
        const uint16_t* bA = buf;
        const uint16_t* bB = buf + BM * P;
        const bf16x8 fa = ld_bf16x8(&bA[a_off + kk]);
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[j] = mfma32(fa, ld_bf16x8(&bB[b_off + j * 32 * P + kk]), acc[j]);
    };
    // destinations (and rotary positions) of the tile's rows, looked up while the first stage loads (the
    // barriers of the stage loop publish them); rows past the bucket are not stored
    __shared__ size_t s_dst[BM];
    __shared__ int s_pos[BM];
    auto lookup = [&]() {
        for (int m = tid; m < BM; m += NT) {
            const int r = row0 + m;
            size_t o = ~(size_t)0;
            int pos = 0;
            if (r < M) {
                const int tok = kind == 0 ? a.rows[base + r] : r;
                o = qp_dst(a, kind, h, n, tok, D);
                pos = a.positions ? a.positions[tok] : tok % a.T;
            }
            s_dst[m] = o;
            s_pos[m] = pos;
        }
    };
    if constexpr (DB) {
        load(0);
        lookup();
        store(sS);
        if (nst > 1) load(BK);
        __syncthreads();
        for (int st = 0; st < nst; ++st) {
            const uint16_t* cur = sS + (st & 1) * STG;
#pragma unroll
            for (int kk = 0; kk < BK / 2; kk += 16) mma(cur, kk);
            // the next stage into the other buffer (its readers passed the last barrier), then its successor's
            // loads
            if (st + 1 < nst) {
                store(sS + ((st + 1) & 1) * STG);
                if (st + 2 < nst) load((st + 2) * BK);
            }
#pragma unroll
            for (int kk = BK / 2; kk < BK; kk += 16) mma(cur, kk);
            __syncthreads();
        }
    } else {
        load(0);
        lookup();
        for (int st = 0; st < nst; ++st) {
            __syncthreads();
            store(sS);
            __syncthreads();
            if (st + 1 < nst) load((st + 1) * BK);
#pragma unroll
            for (int kk = 0; kk < BK; kk += 16) mma(sS, kk);
        }
    }

    // every wave is past its last read of the stage buffers before they hold the results
    __syncthreads();
    uint16_t* dst = (uint16_t*)(kind == 0 ? a.q_routed : kind == 1 ? a.q_shared : kind == 2 ? a.k_out : a.v_out);
    const bool rope = a.rope_log2_base > 0.0 && kind <= 2;
    const int c0 = lane & 31;
    // this lane's pair frequencies (pair 32 j + c0, or c0 mod 16 at D = 32)
    double freq[NB > 1 ? NB / 2 : 1];
    if (rope) {
#pragma unroll
        for (int j = 0; j < (NB > 1 ? NB / 2 : 1); ++j)
            freq[j] = qp_rope_freq(NB > 1 ? 32 * j + c0 : (c0 & 15), D, a.rope_log2_base);
    }
    // results leave through the wave's own LDS region, 16 rows at a time, so every global store is 16 bytes
    // of one output row (the stage buffers are free: every wave passed the barrier above)
    constexpr int RPC = D + 8;                          // region pitch (bf16)
    constexpr int CH = D / 8;                           // 16-byte chunks per row
    uint16_t* reg = sA + wave * 16 * RPC;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
#pragma unroll
        for (int e = 8 * p; e < 8 * p + 8; ++e) {
            const int mm = wave * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
            float v[NB];
#pragma unroll
            for (int j = 0; j < NB; ++j) v[j] = acc[j][e];
            if (rope) {
                const int pos = s_pos[mm];
                if constexpr (NB == 1) {
                    // D = 32: column c pairs with c ^ 16, held by lane l ^ 16
                    const float other = __shfl_xor(v[0], 16);
                    float sn, cs;
                    sincosf(qp_rope_angle(pos, freq[0]), &sn, &cs);
                    v[0] = c0 < 16 ? v[0] * cs - other * sn : v[0] * cs + other * sn;
                } else {
#pragma unroll
                    for (int j = 0; j < NB / 2; ++j) {
                        float sn, cs;
                        sincosf(qp_rope_angle(pos, freq[j]), &sn, &cs);
                        const float x1 = v[j], x2 = v[j + NB / 2];
                        v[j] = x1 * cs - x2 * sn;
                        v[j + NB / 2] = x2 * cs + x1 * sn;
                    }
                }
            }
            const int rl = 8 * ((e >> 2) & 1) + 4 * (lane >> 5) + (e & 3);   // row within the 16
#pragma unroll
            for (int j = 0; j < NB; ++j) reg[rl * RPC + j * 32 + c0] = __builtin_bit_cast(uint16_t, f2bf(v[j]));
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int q = 0; q < 16 * CH / 64; ++q) {
            const int idx = lane + 64 * q, rl = idx / CH, ch = idx % CH;
            const size_t o = s_dst[wave * 32 + 16 * p + rl];
            if (o != ~(size_t)0) *(u32x4*)&dst[o + 8 * ch] = *(const u32x4*)&reg[rl * RPC + 8 * ch];
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
}

// fp32 projection: one thread per output element, fp32 FMA chain (two chains
// where the rotary embedding needs the partner element of the pair).
__global__ __launch_bounds__(256) void qproj_f32_kernel(const QpArgs a, const float* __restrict__ x, int d_head)
{
    const int N = a.G * a.E, BT = a.B * a.T, n_exp = qp_n_exp(a);
    const int n = blockIdx.x % n_exp;
    int h;
    const int kind = qp_kind(a, n, h);
    if (kind == 0 && !a.q_routed) return;
    const int row0 = (blockIdx.x / n_exp) * kQpBM;
    const int M = kind == 0 ? a.counts[n] : BT;
    if (row0 >= M) return;
    const int base = kind == 0 ? a.offsets[n] : 0;
    const int d_model = a.d_model;
    const float* wn = kind <= 1 ? (const float*)a.w_q + (size_t)(kind == 0 ? n : N + h) * d_head * d_model
                                : (const float*)(kind == 2 ? a.w_k : a.w_v) + (size_t)h * d_head * d_model;
    float* dst = (float*)(kind == 0 ? a.q_routed : kind == 1 ? a.q_shared : kind == 2 ? a.k_out : a.v_out);
    const bool rope = a.rope_log2_base > 0.0 && kind <= 2;
    const int half = d_head / 2;
    for (int idx = threadIdx.x; idx < kQpBM * d_head; idx += 256) {
        const int r = row0 + idx / d_head, d = idx % d_head;
        if (r >= M) break;
        const int tok = kind == 0 ? a.rows[base + r] : r;
        const float* xr = x + (size_t)tok * d_model;
        auto dotw = [&](int dd) {
            const float* wr = wn + (size_t)dd * d_model;
            float s = 0.f;
            for (int i = 0; i < d_model; ++i) s = fmaf(xr[i], wr[i], s);
            return s;
        };
        float s = dotw(d);
        if (rope) {
            const int pos = a.positions ? a.positions[tok] : tok % a.T;
            const float other = dotw(d < half ? d + half : d - half);
            float sn, cs;
            sincosf(qp_rope_angle(pos, qp_rope_freq(d % half, d_head, a.rope_log2_base)), &sn, &cs);
            s = d < half ? s * cs - other * sn : s * cs + other * sn;
        }
        dst[qp_dst(a, kind, h, n, tok, d_head) + d] = s;
    }
}

static int launch_qp(const QpArgs& q, int d_head, bool bf16, hipStream_t st)
{
    const int N = q.G * q.E, BT = q.B * q.T, n_exp = qp_n_exp(q);
    const bool routed = q.q_routed != nullptr;
    if (BT == 0 || (!routed && q.ns + q.nkv == 0)) return 0;
    if (n_exp > 128) return -2;
    if (bf16) {
        // an upper bound on the number of tiles over all buckets, rounded to the 8 XCDs
        auto grid_for = [&](int BM) {
            const long long um = (routed ? (long long)BT * q.G * q.k / BM + N : 0) +
                                 (long long)(q.ns + 2 * q.nkv) * ((BT + BM - 1) / BM);
            return (int)(8 * ((um + 7) / 8));
        };
        switch (d_head) {   // d_model is a multiple of the 64-wide stage (checked by the API)
        case 32: qproj_bf16_kernel<32, 64><<<grid_for(QpNT<32>::BM), QpNT<32>::NT, 0, st>>>(q); break;
        case 64: qproj_bf16_kernel<64, 64><<<grid_for(QpNT<64>::BM), QpNT<64>::NT, 0, st>>>(q); break;
        case 128: qproj_bf16_kernel<128, 64><<<grid_for(QpNT<128>::BM), QpNT<128>::NT, 0, st>>>(q); break;
        default: return -2;
        }
    } else {
        const int tiles = (BT + kQpBM - 1) / kQpBM;
        qproj_f32_kernel<<<tiles * n_exp, 256, 0, st>>>(q, (const float*)q.x, d_head);
    }
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

static QpArgs qp_args(const void* x, int B, int T, int d_model, int G, int E, int k)
{
    QpArgs q{};
    q.x = (const uint16_t*)x;
    q.B = B; q.T = T; q.d_model = d_model; q.G = G; q.E = E; q.k = k;
    return q;
}

int launch_qproj(const QprojArgs& a, hipStream_t st)
{
    // a NULL q_shared leaves the shared head out of this call
    QpArgs q = qp_args(a.x, a.B, a.T, a.d_model, a.G, a.E, a.k);
    q.w_q = a.w_q; q.sel = a.sel; q.counts = a.counts; q.offsets = a.offsets; q.rows = a.rows;
    q.q_routed = a.q_routed; q.q_shared = a.q_shared;
    q.ns = a.q_shared ? a.n_shared : 0;
    return launch_qp(q, a.d_head, a.bf16, st);
}

// K and V projections (GQA tutorial, freeguideonline, "GQA 核心原理与计算流程"
// step 2): the same kernel with no routed experts and 2 H_kv dense heads over
// every token in one launch, written as [B, H_kv, T, d_head].
static KvDenseArgs kv_dense_args(const void* x, const void* w_k, const void* w_v, void* k, void* v,
                                 const int32_t* positions, int B, int T, int d_model, int H, int d_head,
                                 double rope_log2_base)
{
    KvDenseArgs d{};
    d.x = (const uint16_t*)x; d.w_k = (const uint16_t*)w_k; d.w_v = (const uint16_t*)w_v; d.k_out = k; d.v_out = v;
    d.positions = positions; d.B = B; d.T = T; d.d_model = d_model; d.H = H; d.d_head = d_head;
    d.rope_log2_base = rope_log2_base;
    return d;
}

int launch_kv_proj(const KvProjArgs& a, hipStream_t st)
{
    // bf16: one dense GEMM over every token (kvproj.hip)
    if (a.bf16)
        return launch_kv_dense(kv_dense_args(a.x, a.w_k, a.w_v, a.k, a.v, nullptr, a.B, a.T, a.d_model, a.H_kv,
                                             a.d_head, 0.0), st);
    QpArgs q = qp_args(a.x, a.B, a.T, a.d_model, 0, 1, 1);
    q.w_k = a.w_k; q.w_v = a.w_v; q.k_out = a.k; q.v_out = a.v;
    q.nkv = a.H_kv;   // at most 64 (the descriptor's limit), so one plan covers both
    return launch_qp(q, a.d_head, a.bf16, st);
}

// The whole Q/K/V preamble from one read of x: the routed experts over their
// compacted rows, the shared head, and the K and V heads in one launch, so
// the k*G + 1 + 2*H_kv projections of every x row are served from one XCD's
// L2; the rotary embedding, when asked, is applied to q and K in fp32 before
// the one bf16 rounding.
int launch_qkv_proj(const QkvProjArgs& a, hipStream_t st)
{
    QpArgs q = qp_args(a.x, a.B, a.T, a.d_model, a.G, a.E, a.k_);
    q.w_q = a.w_q; q.w_k = a.w_k; q.w_v = a.w_v;
    q.sel = a.sel; q.counts = a.counts; q.offsets = a.offsets; q.rows = a.rows;
    q.q_routed = a.q_routed; q.q_shared = a.n_shared ? a.q_shared : nullptr; q.k_out = a.k; q.v_out = a.v;
    q.ns = a.n_shared ? 1 : 0;
    q.nkv = a.H_kv;
    q.positions = a.positions;
    q.rope_log2_base = a.rope_base > 0.f ? log2((double)a.rope_base) : 0.0;
    if (a.bf16) {
        // the queries over their compacted rows, then K and V as one dense GEMM
        QpArgs qq = q;
        qq.nkv = 0;
        const int rc = launch_qp(qq, a.d_head, true, st);
        return rc ? rc : launch_kv_dense(kv_dense_args(a.x, a.w_k, a.w_v, a.k, a.v, a.positions, a.B, a.T,
                                                       a.d_model, a.H_kv, a.d_head, q.rope_log2_base), st);
    }
    if (qp_n_exp(q) <= 128) return launch_qp(q, a.d_head, a.bf16, st);
    // more experts than one plan covers: the queries, then K and V
    QpArgs qq = q, qkv = q;
    qq.nkv = 0;
    qkv.q_routed = nullptr; qkv.ns = 0; qkv.G = 0; qkv.E = 1;
    const int rc = launch_qp(qq, a.d_head, a.bf16, st);
    return rc ? rc : launch_qp(qkv, a.d_head, a.bf16, st);
}

}  // namespace gqe
