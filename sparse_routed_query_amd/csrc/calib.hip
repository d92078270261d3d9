// Calibration kernels for the measurements (gfx950): what this chip reaches
// under sustained load with nothing but dense bf16 MFMAs, and with nothing but
// streaming reads from HBM.  They compute nothing of the method; the
// benchmark reports them beside the kernels' fractions of the published
// peaks (MI355X: 2516.6 TFLOP/s dense bf16, 8 TB/s HBM3E).
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef float calib_f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 calib_bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t calib_u32x4 __attribute__((ext_vector_type(4)));

// Every wave runs `iters` rounds of four independent chains of
// v_mfma_f32_32x32x16_bf16 (32768 FLOP each), so the matrix core never waits
// on a result.  Wave 0 of workgroup 0 records the shader-clock counter
// (s_memtime) and the 100 MHz reference counter (s_memrealtime) at its start
// and end: their ratio is the clock the loop ran at.
__global__ __launch_bounds__(256) void calib_mfma_kernel(float* __restrict__ sink, uint64_t* __restrict__ clk, int iters)
{
    calib_bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(0.001f * (threadIdx.x + i));
        b[i] = (__bf16)(0.002f * (i + 1));
    }
    calib_f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    const bool rec = blockIdx.x == 0 && threadIdx.x == 0;
    uint64_t t0 = 0, r0 = 0;
    if (rec) {
        t0 = __builtin_amdgcn_s_memtime();
        r0 = __builtin_amdgcn_s_memrealtime();
    }
    for (int it = 0; it < iters; ++it) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, b, c3, 0, 0, 0);
    }
    if (rec) {
        const uint64_t t1 = __builtin_amdgcn_s_memtime();
        const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
        clk[0] = t1 - t0;
        clk[1] = r1 - r0;
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
    // never true for these inputs; keeps the chains from being removed
    if (s == -1.f) sink[blockIdx.x * 256 + threadIdx.x] = s;
}

// Streaming read of `n16` 16-byte words with non-temporal loads, each
// workgroup one contiguous chunk with eight loads per lane in flight; one
// partial xor per workgroup is written so the loads are kept.
__global__ __launch_bounds__(256) void calib_read_kernel(const calib_u32x4* __restrict__ src, long long n16,
                                                         uint32_t* __restrict__ sink)
{
    const long long per = (n16 + gridDim.x - 1) / gridDim.x;
    const long long lo = (long long)blockIdx.x * per, hi = lo + per < n16 ? lo + per : n16;
    uint32_t acc = 0;
    for (long long i = lo + threadIdx.x; i < hi; i += 256 * 8) {
        calib_u32x4 v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const long long k = i + (long long)j * 256;
            v[j] = k < hi ? __builtin_nontemporal_load(src + k) : calib_u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) acc ^= v[j][0] ^ v[j][1] ^ v[j][2] ^ v[j][3];
    }
    __shared__ uint32_t s_acc[256];
    s_acc[threadIdx.x] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t t = 0;
        for (int i = 0; i < 256; ++i) t ^= s_acc[i];
        sink[blockIdx.x] = t;
    }
}

extern "C" {

// Dense bf16 MFMA loop: `blocks` workgroups of 4 waves, each wave 4 * iters
// MFMAs of 32768 FLOP.  sink: blocks * 256 floats (device, never written for
// these inputs); clk: 2 uint64 (device): shader-clock ticks and 100 MHz ticks
// of wave 0 of workgroup 0.  Returns 0 or -1 (launch failure).
int gqe_calib_mfma(float* sink, uint64_t* clk, int blocks, int iters, void* stream)
{
    if (!sink || !clk || blocks < 1 || iters < 1) return -1;
    calib_mfma_kernel<<<blocks, 256, 0, (hipStream_t)stream>>>(sink, clk, iters);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

// Streaming read of `bytes` (a multiple of 16; src 16-byte aligned, device)
// by `blocks` workgroups; sink: blocks uint32 (device).  Returns 0 or -1.
int gqe_calib_read(const void* src, long long bytes, uint32_t* sink, int blocks, void* stream)
{
    if (!src || !sink || bytes < 16 || (bytes & 15) || blocks < 1 || ((uintptr_t)src & 15)) return -1;
    calib_read_kernel<<<blocks, 256, 0, (hipStream_t)stream>>>((const calib_u32x4*)src, bytes / 16, sink);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // extern "C"
