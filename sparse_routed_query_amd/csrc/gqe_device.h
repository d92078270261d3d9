// Device-side helpers shared by the GQE HIP kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqe {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf2f(uint16_t u) { return __builtin_bit_cast(float, (uint32_t)u << 16); }
__device__ __forceinline__ float bf2f(bf16 b) { return bf2f(__builtin_bit_cast(uint16_t, b)); }
// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ bf16 f2bf(float f) { return (bf16)f; }
// two floats rounded to bf16 (nearest even, as f2bf), lo in the low half: one v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi)
{
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ bf16x8 ld_bf16x8(const void* p) { return __builtin_bit_cast(bf16x8, *(const u32x4*)p); }
__device__ __forceinline__ u32x4 ld_u32x4(const void* p) { return *(const u32x4*)p; }

// D = A(32x16) * B(16x32) + C on bf16 MFMA.  Lane l holds row/column l%32 of
// A/B with the k-half l/32; accumulator element r of lane l is
// (row 8*(r/4) + 4*(l/32) + r%4, column l%32).
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// D = A(16x32) * B(32x16) + C.  Lane l holds row/column l%16 with k-quarter
// l/16; accumulator element r of lane l is (row 4*(l/16) + r, column l%16).
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// MFMA fragment read across a row-major LDS tile M[k][n] (pitch in elements)
// with two transposing reads.  Within each 16-lane group, lane i of
// ds_read_b64_tr_b16 receives, as its element j, element i % 4 of the 8 bytes
// that lane 4 j + i / 4 addresses; pointing lane 4 j + q at
// M[k0 + 4 (l/32) + j][n + 4 q .. +3] gives lane l column n0 + l%32 and rows
// k0 + 4 (l/32) + 0..3, then (second read) 8 rows further.  In the MFMA's k
// order, rows 4-7 and 8-11 of each 16-row block are therefore swapped; an
// operand read along k from a [n][k] tile must take the same swap (kpos, or
// frag_perm below), so the products are unchanged.
typedef short tr_s16x4 __attribute__((ext_vector_type(4)));
typedef short tr_s16x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ bf16x8 frag_tr(const uint16_t* M, int pitch, int k0, int n0, int lane)
{
    typedef __attribute__((address_space(3))) tr_s16x4 lds_s16x4;
    const int s16 = lane & 15;
    const uint16_t* p = M + (k0 + 4 * (lane >> 5) + (s16 >> 2)) * pitch + n0 + 16 * ((lane >> 4) & 1) + 4 * (s16 & 3);
    const tr_s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
    const tr_s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 8 * pitch));
    const tr_s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
}
// storage position of contraction index k (0..63) in an A-operand tile read by frag_row
__device__ __forceinline__ int kpos(int k)
{
    const int b = k & 12;
    return b == 4 ? k + 4 : b == 8 ? k - 4 : k;
}
// A fragment from a row-major LDS tile M[m][k] in frag_tr's k order: lane l
// takes row m0 + l%32, elements k0 + 4 (l/32) + 0..3 and 8 further.
__device__ __forceinline__ bf16x8 frag_perm(const uint16_t* M, int pitch, int m0, int k0, int lane)
{
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const uint16_t* p = M + (m0 + (lane & 31)) * pitch + k0 + 4 * (lane >> 5);
    const u32x2 lo = *(const u32x2*)p, hi = *(const u32x2*)(p + 8);
    const u32x4 v = {lo[0], lo[1], hi[0], hi[1]};
    return __builtin_bit_cast(bf16x8, v);
}

// Rotary embedding: frequency of pair i of a d-wide row, base^(-2i/d), in
// double (a float exponent would move the angle of a far position by ~1e-3),
// and the angle pos * freq reduced to [-pi, pi] in double, so that fp32 sin
// and cos keep full accuracy at any position.
__device__ __forceinline__ double rope_freq(int i, int d, double log2_base)
{
    return exp2(-(double)(2 * i) / (double)d * log2_base);
}
__device__ __forceinline__ float rope_angle(int pos, double freq)
{
    const double a = (double)pos * freq;
    const double two_pi = 6.283185307179586476925;
    return (float)(a - two_pi * rint(a * (1.0 / two_pi)));
}

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}
__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

}  // namespace gqe
