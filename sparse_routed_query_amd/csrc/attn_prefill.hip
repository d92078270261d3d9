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
// (b, head), at d_head 128 8 waves = 256 rows; key tiles of 64):
//   * Within a group the routed queries are a dense [T*k, d] matrix whose row
//     r sits at position r / k, so all k kept rows of a position share every
//     K/V tile staged in LDS -- each K/V tile is loaded once per 128 (256) rows.
//   * The wave computes S^T = K Q^T (32 keys x 32 queries per MFMA block), so a
//     lane owns one query column: the row max and row sum need one exchange
//     with lane l^32 and no LDS.  Q enters the product exactly as the
//     projection stored it; the scale log2(e)/sqrt(d) is applied in fp32 to
//     the scores, fused with the subtraction of the row's reference, so the
//     softmax is one fma and one exp2 per score and q is rounded only once.
//   * P^T feeds O^T = V^T P^T straight from the S^T accumulators.  The order
//     of keys inside a 16-key MFMA step is permuted to match the accumulator
//     layout; V^T is written to LDS in that permuted order, so no shuffle of P
//     is needed.  O^T columns are again owned per lane, so the online-softmax
//     rescale needs no exchange either.
//   * Workgroups are issued longest-first (causal work grows with the query
//     tile) over both the routed tiles (k rows per position) and the shared
//     tiles (one row per position).  With a workspace, the causal tiles that
//     need more than a threshold of key tiles are cut into two work items
//     over the two halves of their key range, so that no workgroup is much
//     longer than the average load of a workgroup slot; both halves write
//     their partial softmax state (reference, row sum, unnormalised output),
//     and the one that finishes second merges the two (no waiting).
#include "gqe_device.h"
#include "gqe_launch.h"

namespace gqe {

// Query rows per workgroup (waves of 32 rows): 256 at d_head 128, where the
// registers allow two waves per SIMD either way and eight waves of one tile
// halve the K/V tile loads per query row; 128 otherwise (three workgroups of
// four waves per compute unit).
__host__ __device__ constexpr int pf_bm(int d_head) { return d_head == 128 ? 256 : 128; }
constexpr int kPfBN = 64;    // keys per iteration
constexpr int kPfPad = 8;    // LDS row padding in bf16 elements

// Key tiles needed by query tile i of a head with kk rows per position.
__host__ __device__ __forceinline__ int pf_nkv(int i, int kk, int R, int T, int causal, int bm)
{
    if (!causal) return (T + kPfBN - 1) / kPfBN;
    const int last_row = min(R - 1, (i + 1) * bm - 1);
    return (last_row / kk) / kPfBN + 1;
}

// Work schedule of one launch.  A routed head has ntr query tiles (k rows per
// position), the shared head nts (one row per position).  Tiles i >= isr
// (routed) and i >= iss (shared) are split: part 0 takes key tiles [0, h),
// part 1 [h, nkv), h = nkv / 2.  Work items are ordered by decreasing size
// (key tiles of the item; for a split tile, the larger part), then routed
// before shared, split before whole, by decreasing tile index, and split
// tiles by part, then head.
struct PfSched {
    int B, T, G, k, n_shared, causal;
    int bm;         // query rows per tile (pf_bm)
    int ntr, nts;   // query tiles per routed / shared head
    int isr, iss;   // first split tile (== ntr / nts: none)
    int nkv_max;    // key tiles of the longest tile
    int routed, shared;   // which heads this launch computes (the split and the
                          // pair numbering always follow the whole shape)
};

__host__ __device__ __forceinline__ long long pf_heads(const PfSched& p, int l)
{
    return l ? ((p.n_shared && p.shared) ? p.B : 0) : (p.routed ? (long long)p.B * p.G : 0);
}
struct PfItem {
    int b, h, tile;   // h == G means the shared head
    int part;         // -1: whole tile; 0, 1: first / second half of its keys
    int pair;         // split tiles: index of the (part 0, part 1) pair; else -1
};

// Smallest tile index in [0, nt] whose key-tile count is at least n
// (nkv is non-decreasing in the tile index).
__host__ __device__ __forceinline__ int pf_first_ge(int n, int kk, int R, int nt, int T, int causal, int bm)
{
    if (!causal) return n <= (T + kPfBN - 1) / kPfBN ? 0 : nt;
    if (n <= 1) return 0;
    // nkv(i) >= n  <=>  min(R - 1, bm i + bm - 1) >= 64 kk (n - 1)
    const long long need = (long long)kPfBN * kk * (n - 1);
    if (need > R - 1) return nt;
    return (int)min((long long)nt, need / bm);
}

// Number of work items whose size is at least s.
__host__ __device__ __forceinline__ long long pf_count_ge(const PfSched& p, int s)
{
    long long n = 0;
#pragma unroll
    for (int l = 0; l < 2; ++l) {
        const int kk = l ? 1 : p.k, nt = l ? p.nts : p.ntr, is = l ? p.iss : p.isr;
        const long long cnt = pf_heads(p, l);
        const int R = p.T * kk;
        const int whole = max(0, is - pf_first_ge(s, kk, R, nt, p.T, p.causal, p.bm));
        const int split = max(0, nt - max(is, pf_first_ge(2 * s - 1, kk, R, nt, p.T, p.causal, p.bm)));
        n += (whole + 2ll * split) * cnt;
    }
    return n;
}

// The id-th work item, given the size s of that item: the largest s with
// pf_count_ge(p, s) > id.
__host__ __device__ __forceinline__ PfItem pf_item_of_size(const PfSched& p, long long id, int s)
{
    const long long gid = id;
    id -= pf_count_ge(p, s + 1);
    PfItem w{0, 0, 0, -1, -1};
    for (int l = 0; l < 2; ++l) {
        const int kk = l ? 1 : p.k, nt = l ? p.nts : p.ntr, is = l ? p.iss : p.isr;
        const long long cnt = pf_heads(p, l);
        const int R = p.T * kk;
        for (int sp = 1; sp >= 0; --sp) {
            // tiles of this group whose item size is exactly s: [a, e)
            int a, e;
            if (sp) {
                a = max(is, pf_first_ge(2 * s - 1, kk, R, nt, p.T, p.causal, p.bm));
                e = max(is, pf_first_ge(2 * s + 1, kk, R, nt, p.T, p.causal, p.bm));
            } else {
                a = min(is, pf_first_ge(s, kk, R, nt, p.T, p.causal, p.bm));
                e = min(is, pf_first_ge(s + 1, kk, R, nt, p.T, p.causal, p.bm));
            }
            const long long per = cnt * (sp ? 2 : 1);
            const long long n = (long long)max(0, e - a) * per;
            if (id < n) {
                const int i = e - 1 - (int)(id / per);
                const int rem = (int)(id % per);
                // a tile's items come as runs of cnt consecutive workgroups, one
                // per head (split tiles part-major: all part 0s, then all part
                // 1s).  Workgroup j runs on XCD j mod 8, so when cnt is a
                // multiple of 8 the run's workgroup j takes head
                // 8 floor(r / 8) + j mod 8 (r its rank in the run): every item
                // of a head, whole or either half, then runs on XCD head mod 8,
                // whose L2 serves the head's K/V to all of them
                const int r = sp ? rem % (int)cnt : rem;
                const int bh = cnt % 8 == 0 ? (r & ~7) | (int)(gid & 7) : r;
                w.tile = i;
                w.part = sp ? rem / (int)cnt : -1;
                if (l == 0) {
                    w.b = bh / p.G; w.h = bh % p.G;
                } else {
                    w.b = bh; w.h = p.G;
                }
                w.pair = !sp ? -1 : l == 0 ? (i - is) * p.B * p.G + bh
                                           : (p.ntr - p.isr) * p.B * p.G + (i - is) * p.B + bh;
                return w;
            }
            id -= n;
        }
    }
    return w;   // not reached for id < pf_count_ge(p, 1)
}

// The id-th work item (0 <= id < pf_count_ge(p, 1)), by binary search.
__host__ __device__ __forceinline__ PfItem pf_item(const PfSched& p, long long id)
{
    int lo = 1, hi = p.nkv_max;
    while (lo < hi) {
        const int mid = (lo + hi + 1) / 2;
        if (pf_count_ge(p, mid) > id) lo = mid; else hi = mid - 1;
    }
    return pf_item_of_size(p, id, lo);
}

// The same on the GPU, by the 64 lanes of a wave at once: lane l tests a
// candidate size, and since pf_count_ge is non-increasing in s the lanes that
// pass form a prefix.  Two rounds (stride, then within the stride) cover up
// to 4096 key tiles.  Keeps the search off the scalar unit, which all waves
// of a compute unit share.
__device__ __forceinline__ PfItem pf_item_wave(const PfSched& p, long long id, int lane)
{
    const int stride = (p.nkv_max + 63) / 64;
    const int s1 = 1 + lane * stride;
    const bool ok1 = s1 <= p.nkv_max && pf_count_ge(p, s1) > id;
    int s = 1 + (__popcll(__ballot(ok1)) - 1) * stride;
    if (stride > 1) {
        const int s2 = s + lane;
        const bool ok2 = lane < stride && s2 <= p.nkv_max && pf_count_ge(p, s2) > id;
        s += __popcll(__ballot(ok2)) - 1;
    }
    return pf_item_of_size(p, id, s);
}

// Floats of one part's partial state: per thread, the output accumulators
// (D / 2) and (reference, half row sum).
template <int D>
__host__ __device__ constexpr int pf_part_floats() { return 2 * pf_bm(D) * (D / 2 + 2); }

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

struct PfParams {
    const uint16_t* q_routed;
    const uint16_t* q_shared;
    const uint16_t* kg;
    const uint16_t* vg;
    float* out;
    int* ctr;      // one counter per split pair (even before a launch, even after)
    float* part;   // pf_part_floats<D>() floats per part of each split pair
    float* lse;    // NULL, or each row's base-2 log-sum-exp: routed rows [B, G, T*k], then shared rows [B, T]
    int S;
    float qscale;  // log2(e) / sqrt(d)
    PfSched sc;
};

// One work item: attention of a query tile over its key tiles [kt0, kt1).
template <int D>
__device__ __forceinline__ void pf_item_run(const PfParams& p, const PfItem w)
{
    constexpr int BM = pf_bm(D), NT = 2 * BM; // query rows and threads of the workgroup
    constexpr int P = D + kPfPad;           // LDS row pitch (elements)
    constexpr int NDB = D / 32;
    constexpr int NCH = kPfBN * D / 8 / NT;  // 16-byte chunks per thread for one K or V tile
    const int T = p.sc.T, G = p.sc.G, k = p.sc.k, causal = p.sc.causal, S = p.S;
    const float qscale = p.qscale;
    const uint16_t* __restrict__ q_routed = p.q_routed;
    const uint16_t* __restrict__ q_shared = p.q_shared;
    const uint16_t* __restrict__ kg = p.kg;
    const uint16_t* __restrict__ vg = p.vg;
    float* __restrict__ out = p.out;
    const bool shared = w.h == G;
    const int kk = shared ? 1 : k;
    const int R = T * kk;
    const int kvh = shared ? 0 : w.h;
    const uint16_t* Q = shared ? q_shared + (size_t)w.b * T * D : q_routed + ((size_t)w.b * G + w.h) * (size_t)R * D;
    const uint16_t* K = kg + ((size_t)w.b * G + kvh) * (size_t)T * D;
    const uint16_t* V = vg + ((size_t)w.b * G + kvh) * (size_t)T * D;
    const int slot0 = shared ? S - 1 : w.h * k;

    const int tid = threadIdx.x, lane = tid & 63;
    // wave-uniform, so that the per-wave tile limits and mask tests stay scalar
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 31, lh = lane >> 5;
    const int r0 = w.tile * BM;
    const int nkv = pf_nkv(w.tile, kk, R, T, causal, BM);
    // key tiles of this work item: [kt0, kt1)
    const int kt0 = w.part == 1 ? nkv / 2 : 0;
    const int kt1 = w.part == 0 ? nkv / 2 : nkv;

    const int qrow = r0 + wave * 32 + lr;
    const bool qvalid = qrow < R;
    const int tq = qvalid ? qrow / kk : T - 1;   // rows past R see every key, so they stay finite
    const int wrow_hi = min(R - 1, r0 + wave * 32 + 31);
    const int nkv_w = __builtin_amdgcn_readfirstlane(causal ? (wrow_hi / kk) / kPfBN + 1 : nkv);
    const int t_lo_w = __builtin_amdgcn_readfirstlane((r0 + wave * 32) / kk);
    // key tiles starting after this position need a mask: some key is past
    // the wave's first row (causal) or past T
    const int mask_after = causal ? t_lo_w - kPfBN + 1 : T - kPfBN;

    // V rows get 32 elements of padding: the transposing reads are then free of
    // bank conflicts (16 for K rows, read with 16-byte loads).
    constexpr int PV = D + 32;
    constexpr int KVSZ = kPfBN * (P + PV);   // one stage: K rows, then V rows
    __shared__ __attribute__((aligned(16))) uint16_t sKV[2 * KVSZ];

    // Q loads (rows past R read row R-1 and are zeroed) are issued together
    // with the first K/V tile's, so the prologue waits for memory once
    u32x4 qraw[D / 16];
    {
        const uint16_t* qsrc = Q + (size_t)min(qrow, R - 1) * D + 8 * lh;
#pragma unroll
        for (int c = 0; c < D / 16; ++c) qraw[c] = ld_u32x4(qsrc + 16 * c);
    }

    u32x4 rk[NCH], rv[NCH];
    // Thread tid moves 16-byte chunks tid + NT i of a tile: key row
    // srow + i * RPP, elements scol .. scol + 7.  A tile is contiguous in
    // memory, so its chunks sit at tid * 8 + i * NT * 8 from the tile start.
    constexpr int RPP = NT / (D / 8);        // key rows per NT chunks
    const int srow = tid / (D / 8), scol = (tid % (D / 8)) * 8;
    // Buffer loads: the resource starts at the tile and covers the rest of the
    // head, so rows past T fall outside it and read as zero (their scores are
    // masked, so their probabilities are exactly 0).
    auto load = [&](int kt) {
        const int p0 = kt * kPfBN;
        const int bytes = (T - p0) * D * 2;
        const __amdgpu_buffer_rsrc_t rK = __builtin_amdgcn_make_buffer_rsrc((void*)(K + (size_t)p0 * D), 0, bytes, 0x00020000);
        const __amdgpu_buffer_rsrc_t rV = __builtin_amdgcn_make_buffer_rsrc((void*)(V + (size_t)p0 * D), 0, bytes, 0x00020000);
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            rk[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rK, tid * 16 + i * NT * 16, 0, 0));
            rv[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rV, tid * 16 + i * NT * 16, 0, 0));
        }
    };
    const int k_st = srow * P + scol, v_st = kPfBN * P + srow * PV + scol;   // store offsets in a stage
    auto store = [&](int buf) {
        uint16_t* stage = sKV + buf * KVSZ;
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            *(u32x4*)(stage + k_st + i * RPP * P) = rk[i];
            *(u32x4*)(stage + v_st + i * RPP * PV) = rv[i];
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
    float negm = 0.f;   // -m_ref, the fma addend of every exponent
    f32x16 zero16;
#pragma unroll
    for (int r = 0; r < 16; ++r) zero16[r] = 0.f;

    load(kt0);
    bf16x8 qf[D / 16];
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
        const u32x4 v = qvalid ? qraw[c] : u32x4{0, 0, 0, 0};
        qf[c] = __builtin_bit_cast(bf16x8, v);
        // pin the Q fragments here, ahead of the first tile's store: the Q loads
        // are then in flight together with the tile loads, not issued after them
        asm volatile("" ::"v"(qf[c]));
    }
    store(0);
    __syncthreads();
    for (int kt = kt0; kt < kt1; ++kt) {
        const int buf = (kt - kt0) & 1;
        if (kt + 1 < kt1) load(kt + 1);
        if (kt < nkv_w) {
            const uint16_t* bK = sKV + buf * KVSZ;
            const uint16_t* bV = bK + kPfBN * P;
            const int s0 = kt * kPfBN;
            const bool need_mask = s0 > mask_after;
            bool done = false;
            if (!need_mask && kt != kt0) {
                // Fast path, per 32-key block: block 0's probabilities are formed
                // while block 1's scores are in the matrix cores, and block 1's
                // while block 0's PV is.  A block whose row sums could exceed 2^8
                // falls back: block 0 to the general path below (nothing has been
                // accumulated yet), block 1 to moving the reference on its own
                // (which rescales what block 0 already added).
                f32x16 sb0, sb1;
                sb0 = mfma32(ld_bf16x8(bK + k_off), qf[0], zero16);
#pragma unroll
                for (int c = 1; c < D / 16; ++c) sb0 = mfma32(ld_bf16x8(bK + k_off + 16 * c), qf[c], sb0);
                sb1 = mfma32(ld_bf16x8(bK + k_off + 32 * P), qf[0], zero16);
#pragma unroll
                for (int c = 1; c < D / 16; ++c) sb1 = mfma32(ld_bf16x8(bK + k_off + 32 * P + 16 * c), qf[c], sb1);
                uint32_t pb0[8], pb1[8];
                auto probs_block = [&](const f32x16& sv, uint32_t (&pw8)[8]) {
                    float la = 0.f, lb = 0.f;
#pragma unroll
                    for (int r = 0; r < 16; r += 2) {
                        const float e0 = __builtin_amdgcn_exp2f(fmaf(sv[r], qscale, negm));
                        const float e1 = __builtin_amdgcn_exp2f(fmaf(sv[r + 1], qscale, negm));
                        pw8[r / 2] = pk_bf16(e0, e1);
                        la += e0;
                        lb += e1;
                    }
                    return la + lb;
                };
                // O^T += V^T P^T over 16-key steps c0, c0 + 1
                auto pv_steps = [&](const uint32_t (&pw8)[8], int c0) {
#pragma unroll
                    for (int c = 0; c < 2; ++c) {
                        const u32x4 pv = {pw8[4 * c], pw8[4 * c + 1], pw8[4 * c + 2], pw8[4 * c + 3]};
                        const bf16x8 pbv = __builtin_bit_cast(bf16x8, pv);
#pragma unroll
                        for (int j = 0; j < NDB; ++j)
                            o[j] = mfma32(load_vt(bV, v_off + 16 * (c0 + c) * PV + 32 * j, 8 * PV), pbv, o[j]);
                    }
                };
                const float ls0 = probs_block(sb0, pb0);
                if (__ballot(!(ls0 <= kPfRescaleSum)) == 0) {
                    l_half += ls0;
                    pv_steps(pb0, 0);
                    float ls1 = probs_block(sb1, pb1);
                    if (__ballot(!(ls1 <= kPfRescaleSum)) != 0) {
                        float mt = sb1[0];
#pragma unroll
                        for (int r = 1; r < 15; r += 2) mt = fmaxf(fmaxf(mt, sb1[r]), sb1[r + 1]);
                        // (fma by a positive scale is monotone: the scaled maximum is the
                        // maximum of the scaled scores)
                        mt = half_max(fmaf(fmaxf(mt, sb1[15]), qscale, negm));
                        const float shift = mt > kPfRescale ? mt : 0.f;
                        const float alpha = __builtin_amdgcn_exp2f(-shift);
#pragma unroll
                        for (int j = 0; j < NDB; ++j)
#pragma unroll
                            for (int r = 0; r < 16; ++r) o[j][r] *= alpha;
                        l_half *= alpha;
                        m_ref += shift;
                        negm = -m_ref;
                        ls1 = probs_block(sb1, pb1);
                    }
                    l_half += ls1;
                    pv_steps(pb1, 2);
                    done = true;
                }
            }
            if (!done) {
                // General path: the first tile of the item, tiles that need a
                // mask, and tiles whose first block failed the check above.
                // S^T = K Q^T for two 32-key blocks (unscaled)
                f32x16 s[2];
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    s[kb] = mfma32(ld_bf16x8(bK + k_off + kb * 32 * P), qf[0], zero16);
#pragma unroll
                    for (int c = 1; c < D / 16; ++c) s[kb] = mfma32(ld_bf16x8(bK + k_off + kb * 32 * P + 16 * c), qf[c], s[kb]);
                }
                if (need_mask) {
                    // key of element r in block kb is s0 + 4*lh + (kb*32 + 8*(r/4) + r%4)
                    const int lim = (causal ? tq : T - 1) - s0 - 4 * lh;
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                        for (int r = 0; r < 16; ++r)
                            s[kb][r] = (kb * 32 + 8 * (r >> 2) + (r & 3)) > lim ? -INFINITY : s[kb][r];
                }
                // P = exp2(S * log2(e)/sqrt(d) - m_ref), packed to bf16 for the PV product.  The row sum
                // adds the fp32 values with plain adds (v_dot2 on the packed values
                // does not run alongside other waves' MFMAs; adds do).
                // If no lane's partial row sum exceeds 2^8, no probability does, so the
                // reference stays and the row max is never computed.  The first tile,
                // and any tile whose sum trips that check, take the exact path: row
                // max, move the reference if it jumped by more than 2^8, recompute.
                uint32_t pw[16];
                auto probs = [&]() {
                    float la = 0.f, lb = 0.f;
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                        for (int r = 0; r < 16; r += 2) {
                            const float e0 = __builtin_amdgcn_exp2f(fmaf(s[kb][r], qscale, negm));
                            const float e1 = __builtin_amdgcn_exp2f(fmaf(s[kb][r + 1], qscale, negm));
                            pw[kb * 8 + r / 2] = pk_bf16(e0, e1);
                            la += e0;
                            lb += e1;
                        }
                    return la + lb;
                };
                bool exact = kt == kt0;
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
                    mt = half_max(fmaf(mt, qscale, negm));
                    // first tile: set the reference; later tiles: move it only on a large jump
                    const bool move = kt == kt0 ? true : mt > kPfRescale;
                    if (__ballot(move)) {
                        const float shift = move ? mt : 0.f;
                        const float alpha = kt == kt0 ? 0.f : __builtin_amdgcn_exp2f(-shift);
#pragma unroll
                        for (int j = 0; j < NDB; ++j)
#pragma unroll
                            for (int r = 0; r < 16; ++r) o[j][r] *= alpha;
                        l_half *= alpha;
                        m_ref += shift;
                        negm = -m_ref;
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
        }
        if (kt + 1 < kt1) store(buf ^ 1);
        __syncthreads();
    }

    if (w.part >= 0) {
        // Split tile: publish this part's state, then take a ticket; the part
        // that draws the second ticket merges, the first one is done.
        // Ordering, argued at the instruction level (the atomics are relaxed,
        // so the HIP memory model alone does not give it): the agent-scope
        // stores and loads are emitted with the device-scope cache bit (sc1),
        // so a store is acknowledged only once it is visible device-wide and
        // a load is served from the device-coherent level, never from a stale
        // line of this XCD's L2; vmcnt counts stores on CDNA, so the wait
        // below returns only after every state store of the wave has been
        // acknowledged, and the barrier makes that true of all the waves
        // before thread 0's ticket atomic is issued; the merging part issues
        // its loads only after its own ticket has returned (through LDS and a
        // barrier), i.e. after the other part's ticket and so after its
        // acknowledged stores.  Release/acquire would add an L2 write-back
        // and invalidate to every split tile (measured 3.5x slower).
        __shared__ int s_ticket;
        typedef unsigned long long u64;
        constexpr int NQ = D / 4;   // 8-byte words of output accumulators per thread
        auto word = [&](int c) {    // accumulators 2c, 2c+1 of this thread
            const f32x2 v = {o[(2 * c) >> 4][(2 * c) & 15], o[(2 * c) >> 4][(2 * c + 1) & 15]};
            return __builtin_bit_cast(u64, v);
        };
        u64* mine = (u64*)(p.part + ((size_t)w.pair * 2 + w.part) * pf_part_floats<D>());
#pragma unroll
        for (int c = 0; c < NQ; ++c)
            __hip_atomic_store(mine + c * NT + tid, word(c), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(mine + NQ * NT + tid, __builtin_bit_cast(u64, f32x2{m_ref, l_half}), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (tid == 0) s_ticket = __hip_atomic_fetch_add(p.ctr + w.pair, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        if ((s_ticket & 1) == 0) return;
        const u64* other = (const u64*)(p.part + ((size_t)w.pair * 2 + (w.part ^ 1)) * pf_part_floats<D>());
        u64 ov[NQ + 1];
#pragma unroll
        for (int c = 0; c <= NQ; ++c)
            ov[c] = __hip_atomic_load(other + c * NT + tid, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        // part 0's term first, whichever part merges, so the result does not
        // depend on which part finished last
        const f32x2 ml = __builtin_bit_cast(f32x2, ov[NQ]);
        const float m_o = ml[0], l_o = ml[1];
        const float mm = fmaxf(m_ref, m_o);
        const float a_me = __builtin_amdgcn_exp2f(m_ref - mm), a_o = __builtin_amdgcn_exp2f(m_o - mm);
        const bool first = w.part == 0;
        const float a0 = first ? a_me : a_o, a1 = first ? a_o : a_me;
        l_half = fmaf(first ? l_half : l_o, a0, (first ? l_o : l_half) * a1);
        m_ref = mm;
#pragma unroll
        for (int c = 0; c < NQ; ++c) {
            const f32x2 y = __builtin_bit_cast(f32x2, ov[c]);
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int f = 2 * c + e;
                const float x = o[f >> 4][f & 15];
                o[f >> 4][f & 15] = fmaf(first ? x : y[e], a0, (first ? y[e] : x) * a1);
            }
        }
        if (tid == 0) __hip_atomic_store(p.ctr + w.pair, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    if (!qvalid) return;
    const float l = half_sum(l_half);
    const float inv = 1.f / l;
    if (p.lse && lh == 0) {
        // log2 of the row's sum of 2^(s log2(e)/sqrt(d)): the reference plus log2 of the sum
        const size_t ri = shared ? (size_t)p.sc.B * G * T * k + (size_t)w.b * T + qrow
                                 : ((size_t)w.b * G + w.h) * (size_t)R + qrow;
        p.lse[ri] = m_ref + log2f(l);
    }
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

// At most 168 VGPRs for d <= 64 keeps three waves on each SIMD (the LDS of
// three workgroups fits a compute unit); d = 128 runs two (one workgroup of
// eight waves).
template <int D>
__global__ __launch_bounds__(2 * pf_bm(D), D <= 64 ? 3 : 1) void prefill_bf16_kernel(const PfParams p)
{
    pf_item_run<D>(p, pf_item_wave(p.sc, blockIdx.x, threadIdx.x & 63));
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
        if (!q_routed) return;
        h = (int)(r / Rr);
        const int rr = (int)(r % Rr);
        t = rr / k;
        slot = h * k + rr % k;
        q = q_routed + (((size_t)b * G + h) * Rr + rr) * D;
    } else {
        if (!q_shared) return;
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
    if (route_mode == 3) {
        // weighted concatenation: every hard slot times its kept expert's
        // (not renormalised) group softmax probability, in place
        for (int h = 0; h < kG; ++h) {
            f32x4 v = *(const f32x4*)(row + (size_t)h * D);
            const float w = pt[h];
            v = f32x4{v[0] * w, v[1] * w, v[2] * w, v[3] * w};
            *(f32x4*)(row + (size_t)h * D) = v;
        }
        return;
    }
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
    if (n == 0 || route_mode == 2) return 0;   // mode 2 has no weighted slot
    assemble_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(p_tilde, out, n_tok, G, k, D, S, route_mode);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

// Causal query tiles that need more than this many key tiles are split in two
// when a workspace is given ...
constexpr int kPfSplitTiles = 32;
// ... and the longest tile needs more key tiles than the average load of a
// workgroup slot (3 resident workgroups on each of the 256 compute units);
// otherwise longest-first order alone balances the launch.
constexpr int kPfSlots = 3 * 256;

// First split tile of a head: the split tiles are the suffix of tiles that
// need more than kPfSplitTiles key tiles and whose first row sees the first
// key of part 1 (so both parts start from a finite reference).
static int pf_split_start(int nt, int kk, int T, int causal, int bm)
{
    if (!causal) return nt;
    const int R = T * kk;
    int i = nt;
    while (i > 0) {
        const int j = i - 1, n = pf_nkv(j, kk, R, T, causal, bm);
        const long long t0 = (long long)j * bm / kk;
        if (n > kPfSplitTiles && (long long)kPfBN * (n / 2) <= t0) i = j; else break;
    }
    return i;
}

static PfSched pf_sched(int B, int T, int G, int k, int n_shared, int causal, bool split, int bm,
                        bool routed = true, bool shared = true)
{
    PfSched sc;
    sc.bm = bm;
    sc.B = B; sc.T = T; sc.G = G; sc.k = k; sc.n_shared = n_shared; sc.causal = causal;
    sc.routed = routed; sc.shared = shared;
    sc.ntr = (T * k + bm - 1) / bm;
    sc.nts = n_shared ? (T + bm - 1) / bm : 0;
    if (split && causal) {
        long long units = 0;   // key tiles over all query tiles
        for (int i = 0; i < sc.ntr; ++i) units += (long long)pf_nkv(i, k, T * k, T, causal, bm) * B * G;
        for (int i = 0; i < sc.nts; ++i) units += (long long)pf_nkv(i, 1, T, T, causal, bm) * B;
        // (slots counted in 128-row tiles)
        split = (long long)((T + kPfBN - 1) / kPfBN) * kPfSlots * 128 / bm > units;
    }
    sc.isr = split ? pf_split_start(sc.ntr, k, T, causal, bm) : sc.ntr;
    sc.iss = split ? pf_split_start(sc.nts, 1, T, causal, bm) : sc.nts;
    sc.nkv_max = (T + kPfBN - 1) / kPfBN;
    return sc;
}

static long long pf_pairs(const PfSched& sc)
{
    return (long long)(sc.ntr - sc.isr) * sc.B * sc.G + (long long)(sc.nts - sc.iss) * sc.B;
}

// One counter per split pair.
static size_t pf_ctr_bytes(long long pairs) { return (size_t)((pairs * 4 + 255) / 256 * 256); }

size_t prefill_workspace_bytes(int B, int T, int G, int k, int d_head, int n_shared, int causal, bool bf16)
{
    if (!bf16 || (long long)B * T == 0) return 0;
    const long long pairs = pf_pairs(pf_sched(B, T, G, k, n_shared, causal, true, pf_bm(d_head)));
    if (pairs == 0) return 0;
    const int pf = d_head == 32 ? pf_part_floats<32>() : d_head == 64 ? pf_part_floats<64>() : pf_part_floats<128>();
    return pf_ctr_bytes(pairs) + (size_t)pairs * 2 * pf * sizeof(float);
}

long long prefill_plan(int B, int T, int G, int k, int d_head, int n_shared, int causal, bool split, int32_t* items,
                       long long max_items)
{
    const PfSched sc = pf_sched(B, T, G, k, n_shared, causal, split, pf_bm(d_head));
    const long long n = (long long)B * T == 0 ? 0 : pf_count_ge(sc, 1);
    for (long long i = 0; items && i < n && i < max_items; ++i) {
        const PfItem w = pf_item(sc, i);
        const int32_t v[5] = {w.b, w.h, w.tile, w.part, w.pair};
        for (int j = 0; j < 5; ++j) items[i * 5 + j] = v[j];
    }
    return n;
}

int launch_prefill_heads(const PrefillArgs& a, hipStream_t st)
{
    const long long BT = (long long)a.B * a.T;
    if (BT == 0) return 0;
    if (a.lse && !a.bf16) return -2;
    if (a.bf16) {
        const bool split = a.workspace != nullptr &&
                           prefill_workspace_bytes(a.B, a.T, a.G, a.k, a.d_head, a.n_shared, a.causal, true) > 0;
        PfParams prm;
        prm.q_routed = (const uint16_t*)a.q_routed;
        prm.q_shared = (const uint16_t*)a.q_shared;
        prm.kg = (const uint16_t*)a.kmat;
        prm.vg = (const uint16_t*)a.vmat;
        prm.out = a.out;
        prm.sc = pf_sched(a.B, a.T, a.G, a.k, a.n_shared, a.causal, split, pf_bm(a.d_head), a.q_routed != nullptr,
                          a.q_shared != nullptr);
        prm.ctr = split ? (int*)a.workspace : nullptr;
        prm.part = split ? (float*)((char*)a.workspace + pf_ctr_bytes(pf_pairs(prm.sc))) : nullptr;
        prm.lse = a.lse;
        prm.S = a.S;
        prm.qscale = 1.4426950408889634f / sqrtf((float)a.d_head);
        const long long items = pf_count_ge(prm.sc, 1);
        if (items >= (1ll << 31)) return -2;
        if (items == 0) return 0;
        const int grid = (int)items;
        switch (a.d_head) {
        case 32: prefill_bf16_kernel<32><<<grid, 2 * pf_bm(32), 0, st>>>(prm); break;
        case 64: prefill_bf16_kernel<64><<<grid, 2 * pf_bm(64), 0, st>>>(prm); break;
        case 128: prefill_bf16_kernel<128><<<grid, 2 * pf_bm(128), 0, st>>>(prm); break;
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
