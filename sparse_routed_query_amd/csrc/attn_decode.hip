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

#include <mutex>

// Split-KV partials of gqe_attn_decode_noalloc: a fixed device array instead
// of a caller's workspace, for callers that cannot allocate.  Each GPU holds
// its own copy for the life of the process.  In host code the name is only a
// symbol: kernels get the device address hipGetSymbolAddress returns for it.
static __device__ __align__(256) unsigned char scratch[gqe::kDecodeScratchBytes];

namespace gqe {

constexpr int kDcPasses = 12;  // 16-byte loads per thread for each of K and V

template <typename ET, int D>
struct DcShape {
    static constexpr int VEC = 16 / sizeof(ET);    // elements per 16-byte load
    static constexpr int LPP = D / VEC;            // lanes per key position (4 .. 32)
    static constexpr int PPW = 64 / LPP;           // positions per wave and pass
    static constexpr int PPP = 4 * PPW;            // positions per pass
    static constexpr int CH = PPP * kDcPasses;     // keys per chunk
};

typedef __bf16 dc_bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float elem(const u32x4& v, int i, const uint16_t*)
{
    const uint32_t w = v[i >> 1];
    return __builtin_bit_cast(float, (i & 1) ? (w & 0xffff0000u) : (w << 16));
}
__device__ __forceinline__ float elem(const u32x4& v, int i, const float*) { return __uint_as_float(v[i]); }

// q . k over one 16-byte slice: bf16 pairs through the two-term dot product
// with fp32 accumulation, fp32 through fused multiply-adds
__device__ __forceinline__ float slice_dot(const u32x4& q, const u32x4& k, const uint16_t*)
{
    // (elements are copied out before the bit cast: a bit cast of a vector
    // element in place reads element 0 with this compiler)
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t qj = q[j], kj = k[j];
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(dc_bf16x2, qj), __builtin_bit_cast(dc_bf16x2, kj), acc,
                                              false);
    }
    return acc;
}
__device__ __forceinline__ float slice_dot(const u32x4& q, const u32x4& k, const float*)
{
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) acc = fmaf(__uint_as_float(q[j]), __uint_as_float(k[j]), acc);
    return acc;
}

// Value of the lane whose index differs in bit O (O a power of two); below 16
// through DPP (quad permutes, then the 8- and 16-lane mirrors).  The mirrors
// pair lane i with 7-i (15-i), which is an exchange across bit 2 (bit 3) for
// values already equal within groups of 4 (8) lanes, as they are in the
// butterflies below, which take the bits in increasing order.
template <int O>
__device__ __forceinline__ float lane_partner(float v)
{
    const int x = __builtin_bit_cast(int, v);
    if constexpr (O == 1) return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, true));
    else if constexpr (O == 2) return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, true));
    else if constexpr (O == 4) return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, true));
    else if constexpr (O == 8) return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(x, 0x140, 0xF, 0xF, true));
    else return __shfl_xor(v, O);
}
// sum / max over the lanes that differ in bits FROM..TO-1 (values already
// equal within groups of FROM lanes); every lane gets the same result
template <int FROM, int TO>
__device__ __forceinline__ float lanes_sum(float v)
{
    if constexpr (FROM < TO) return lanes_sum<FROM * 2, TO>(v + lane_partner<FROM>(v));
    else return v;
}
template <int FROM, int TO>
__device__ __forceinline__ float lanes_max(float v)
{
    if constexpr (FROM < TO) return lanes_max<FROM * 2, TO>(fmaxf(v, lane_partner<FROM>(v)));
    else return v;
}

// PAGED != 0: the cache is [num_pages, G, page_size, D] and position pos of
// sequence b is row pos % page_size of page block_table[b][pos / page_size]
// (page ids outside 0 .. num_pages-1 are clamped, so a bad table reads wrong
// data but never outside the pages); PAGED == 0: dense [B, G, L_max, D].
// PAGED == 1 when a page holds at least the PPW positions a wave reads per
// pass, 2 otherwise (see row_of below).
template <typename ET, int D, int PAGED>
__global__ __launch_bounds__(256) void decode_split_kernel(const ET* __restrict__ q_routed,
                                                           const ET* __restrict__ q_shared,
                                                           const ET* __restrict__ kc, const ET* __restrict__ vc,
                                                           const int32_t* __restrict__ lens, float* __restrict__ part,
                                                           int G, int k, int n_shared, int L_max, int nch,
                                                           float qscale, const int32_t* __restrict__ block_table,
                                                           int page_shift, int max_pages, int num_pages)
{
    using SH = DcShape<ET, D>;
    constexpr int VEC = SH::VEC, LPP = SH::LPP, PPW = SH::PPW, PPP = SH::PPP, CH = SH::CH;
    const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int c0 = c * CH;
    const int L = min(max(lens[b], 0), L_max);   // never read outside the cache
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int dq = (lane % LPP) * VEC;
    const int pp = tid / LPP;                    // = wave * PPW + position slot in the wave
    // Paged: a wave's PPW positions of a pass start at a multiple of PPW, so
    // when pages hold at least PPW positions (PAGED == 1) they lie in one page
    // and the wave looks its page up once, with a scalar load.  Those loads
    // take the table column clamped to its width (a pass past the end uses
    // no page), not a bound from the sequence's length, so they are all
    // issued at once, together with the length's load, without branches.
    // Smaller pages (PAGED == 2) are looked up per lane.
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const int32_t* bt = PAGED ? block_table + (size_t)b * max_pages : nullptr;
    int wpage[kDcPasses];
    if constexpr (PAGED == 1) {
#pragma unroll
        for (int i = 0; i < kDcPasses; ++i) {
            const int pos_w = c0 + i * PPP + wave_u * PPW;
            wpage[i] = bt[min(pos_w >> page_shift, max_pages - 1)];
        }
        // keep the lookups here: left to itself the compiler moves each into
        // its pass's branch below and waits for it there, one pass at a time
#pragma unroll
        for (int i = 0; i < kDcPasses; ++i) asm volatile("" : "+s"(wpage[i]));
    }
    if (c0 >= L) return;
    auto row_of = [&](int i, int pos) -> size_t {   // element offset of position pos's row (pass i)
        if constexpr (PAGED != 0) {
            int id;
            if constexpr (PAGED == 1) {
                id = wpage[i];
            } else {
                id = bt[pos >> page_shift];
            }
            const int pg = min(max(id, 0), num_pages - 1);
            return (((size_t)pg * G + g) << page_shift) + (pos & ((1 << page_shift) - 1));
        } else {
            return ((size_t)b * G + g) * (size_t)L_max + pos;
        }
    };

    u32x4 kr[kDcPasses], vr[kDcPasses];
#pragma unroll
    for (int i = 0; i < kDcPasses; ++i) {
        const int pos = c0 + i * PPP + pp;
        if (pos < L) {
            // the cache is read once per step: non-temporal loads keep it from
            // displacing other data in the caches
            const size_t r = row_of(i, pos) * D + dq;
            kr[i] = __builtin_nontemporal_load((const u32x4*)(kc + r));
            vr[i] = __builtin_nontemporal_load((const u32x4*)(vc + r));
        } else {
            kr[i] = u32x4{0, 0, 0, 0};
            vr[i] = u32x4{0, 0, 0, 0};
        }
    }

    // Each wave forms (max, sum, o) over its own positions; after one barrier
    // per row, D threads rescale the four waves' terms to the chunk maximum and
    // add them in wave order.  Rows alternate between two LDS buffers: the
    // barrier of row r+1 is passed only after every thread has finished
    // combining row r, so row r+2 may overwrite row r's buffer.
    __shared__ __attribute__((aligned(16))) float s_acc[2][4 * PPW * D];
    __shared__ float s_ml[2][8];
    const int RG = k + n_shared;
    const int nrows = k + ((g == 0 && n_shared) ? 1 : 0);
    for (int row = 0; row < nrows; ++row) {
        const int buf = row & 1;
        const ET* q = row < k ? q_routed + (((size_t)b * G + g) * k + row) * D : q_shared + (size_t)b * D;
        const u32x4 qr = ld_u32x4(q + dq);
        // most workgroups serve one row: keep the unpacking of V inside the
        // row loop rather than holding every unpacked value in registers
#pragma unroll
        for (int i = 0; i < kDcPasses; ++i) asm volatile("" : "+v"(vr[i]));
        float sc[kDcPasses];
        float m = -INFINITY;
#pragma unroll
        for (int i = 0; i < kDcPasses; ++i) {
            const float dot = lanes_sum<1, LPP>(slice_dot(qr, kr[i], (const ET*)nullptr)) * qscale;
            sc[i] = c0 + i * PPP + pp < L ? dot : -INFINITY;
            m = fmaxf(m, sc[i]);
        }
        m = lanes_max<LPP, 64>(m);
        const float mu = m == -INFINITY ? 0.f : m;   // a wave past the end of the cache adds nothing
        float l = 0.f, acc[VEC];
#pragma unroll
        for (int v = 0; v < VEC; ++v) acc[v] = 0.f;
#pragma unroll
        for (int i = 0; i < kDcPasses; ++i) {
            const float p = __builtin_amdgcn_exp2f(sc[i] - mu);
            l += p;
#pragma unroll
            for (int v = 0; v < VEC; ++v) acc[v] = fmaf(p, elem(vr[i], v, (const ET*)nullptr), acc[v]);
        }
        l = lanes_sum<LPP, 64>(l);
        float* sa = &s_acc[buf][pp * D + dq];
#pragma unroll
        for (int v = 0; v < VEC; v += 4) *(f32x4*)(sa + v) = f32x4{acc[v], acc[v + 1], acc[v + 2], acc[v + 3]};
        if (lane == 0) {
            s_ml[buf][wave] = m;
            s_ml[buf][4 + wave] = l;
        }
        __syncthreads();
        if (tid < D) {
            const float* ml = s_ml[buf];
            const float M = fmaxf(fmaxf(ml[0], ml[1]), fmaxf(ml[2], ml[3]));
            float o = 0.f, ls = 0.f;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const float f = __builtin_amdgcn_exp2f(ml[w] - M);
                float ow = 0.f;
#pragma unroll
                for (int s = 0; s < PPW; ++s) ow += s_acc[buf][(w * PPW + s) * D + tid];
                o = fmaf(f, ow, o);
                ls = fmaf(f, ml[4 + w], ls);
            }
            float* dst = part + ((((size_t)b * G + g) * RG + row) * nch + c) * (D + 2);
            dst[2 + tid] = o;
            if (tid == 0) {
                dst[0] = M;
                dst[1] = ls;
            }
        }
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
                    ov[c][i] = pp[(size_t)min(c, max(nc - 1, 0)) * (D + 2) + 2 + d];
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
        // a length below 1 (outside the documented range) has no chunk: its slots are NaN;
        // route mode 3 scales each hard slot by its kept expert's group softmax probability
        const float scale = (route_mode == 3 && row < kG) ? p_tilde[(size_t)b * kG + row] : 1.f;
        const float inv = nc > 0 ? scale / Ls : __builtin_nanf("");
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
        } else if (route_mode == 1) {
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
    if (a.block_table && (1 << a.page_shift) >= DcShape<ET, D>::PPW)
        decode_split_kernel<ET, D, 1><<<grid, 256, 0, st>>>(
            (const ET*)a.q_routed, (const ET*)a.q_shared, (const ET*)a.k_cache, (const ET*)a.v_cache, a.lens,
            (float*)a.workspace, a.G, a.k, a.n_shared, a.L_max, nch, qscale, a.block_table, a.page_shift, a.max_pages,
            a.num_pages);
    else if (a.block_table)
        decode_split_kernel<ET, D, 2><<<grid, 256, 0, st>>>(
            (const ET*)a.q_routed, (const ET*)a.q_shared, (const ET*)a.k_cache, (const ET*)a.v_cache, a.lens,
            (float*)a.workspace, a.G, a.k, a.n_shared, a.L_max, nch, qscale, a.block_table, a.page_shift, a.max_pages,
            a.num_pages);
    else
        decode_split_kernel<ET, D, 0><<<grid, 256, 0, st>>>(
            (const ET*)a.q_routed, (const ET*)a.q_shared, (const ET*)a.k_cache, (const ET*)a.v_cache, a.lens,
            (float*)a.workspace, a.G, a.k, a.n_shared, a.L_max, nch, qscale, nullptr, 0, 0, 0);
    const size_t lds = (size_t)a.G * a.k * D * sizeof(float);
    decode_merge_kernel<D><<<a.B, 64 * kDcMergeWaves, lds, st>>>((const float*)a.workspace, a.lens, a.p_tilde, a.out,
                                                                 a.G, a.k, a.n_shared, a.S, a.route_mode, nch, CH);
}

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};
}  // namespace

// Device address of the current device's copy of `scratch`, looked up once
// per device (with that device current) and kept.
int decode_scratch(void** ptr)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return -1;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return -1;
        g_scratch[dev] = p;
    }
    *ptr = g_scratch[dev];
    return 0;
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

// Precondition audit for decode inputs: counts lens[b] outside 1 .. L_max
// into bad[0] and, for a paged cache, the block-table entries a sequence uses
// (its first ceil(lens[b] / page_size) columns) whose page id is outside
// 0 .. num_pages-1 into bad[1].  One workgroup; bad is written, not added to.
__global__ __launch_bounds__(256) void decode_check_kernel(const int32_t* __restrict__ lens, int B, int L_max,
                                                           const int32_t* __restrict__ block_table, int page_size,
                                                           int max_pages, int num_pages, int32_t* __restrict__ bad)
{
    __shared__ int s_bad[2];
    if (threadIdx.x < 2) s_bad[threadIdx.x] = 0;
    __syncthreads();
    int nl = 0, np = 0;
    for (int b = threadIdx.x; b < B; b += 256) {
        const int L = lens[b];
        nl += (L < 1 || L > L_max) ? 1 : 0;
        if (block_table) {
            const int used = min(max(L, 0), max_pages * page_size);
            const int cols = (used + page_size - 1) / page_size;
            for (int j = 0; j < cols; ++j) {
                const int id = block_table[(size_t)b * max_pages + j];
                np += (id < 0 || id >= num_pages) ? 1 : 0;
            }
        }
    }
    atomicAdd(&s_bad[0], nl);
    atomicAdd(&s_bad[1], np);
    __syncthreads();
    if (threadIdx.x < 2) bad[threadIdx.x] = s_bad[threadIdx.x];
}

int launch_decode_check(const int32_t* lens, int B, int L_max, const int32_t* block_table, int page_size,
                        int max_pages, int num_pages, int32_t* bad, hipStream_t st)
{
    decode_check_kernel<<<1, 256, 0, st>>>(lens, B, L_max, block_table, page_size, max_pages, num_pages, bad);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace gqe
