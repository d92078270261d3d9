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
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi)
{
    return (uint32_t)__builtin_bit_cast(uint16_t, f2bf(lo)) | ((uint32_t)__builtin_bit_cast(uint16_t, f2bf(hi)) << 16);
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
