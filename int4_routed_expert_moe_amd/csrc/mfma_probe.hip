// Matrix-core rate probe for the benchmark's context figures (not part of the
// layer or its C ABI; linked into libmoe_probe.so beside the HBM read probe).
//
// Every wave runs `iters` rounds of independent accumulation chains of one
// matrix-core shape on register operands (no memory traffic in the loop), then
// folds its accumulators into one value per lane and stores it, so the work
// stays live.  The figure is what the part's matrix cores reach under a pure
// matrix-core load at the clock they then run at: the practical ceiling the
// MFMA-bound kernels are compared with beside the nominal peak.  Measured on
// MI355X: the 32x32x16 shape fills the pipe from 8 chains at one wave per
// SIMD; the 16x16x32 shape needs about 16 chains per SIMD in flight (8 chains
// at one wave per SIMD reach about 40% of what 16 chains at two waves do).
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// SHAPE 0: v_mfma_f32_32x32x16_bf16, 8 chains; SHAPE 1: v_mfma_f32_16x16x32_f16, 16 chains.
template <int SHAPE>
__global__ __launch_bounds__(256) void k_mfma_probe(float* __restrict__ out, int iters, float seed) {
    constexpr int kChains = SHAPE == 0 ? 8 : 16;
    const int lane = threadIdx.x & 63;
    float s = 0.0f;
    if constexpr (SHAPE == 0) {
        bf16x8_t a, b;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            a[i] = (__bf16)(seed * (float)(lane + i));
            b[i] = (__bf16)(seed * (float)(i - lane));
        }
        f32x16_t acc[kChains];
#pragma unroll
        for (int c = 0; c < kChains; ++c)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[c][i] = 0.0f;
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
        }
#pragma unroll
        for (int c = 0; c < kChains; ++c)
#pragma unroll
            for (int i = 0; i < 16; ++i) s += acc[c][i];
    } else {
        half8_t a, b;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            a[i] = (_Float16)(seed * (float)(lane + i));
            b[i] = (_Float16)(seed * (float)(i - lane));
        }
        f32x4_t acc[kChains];
#pragma unroll
        for (int c = 0; c < kChains; ++c) acc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[c], 0, 0, 0);
        }
#pragma unroll
        for (int c = 0; c < kChains; ++c)
#pragma unroll
            for (int i = 0; i < 4; ++i) s += acc[c][i];
    }
    out[(size_t)blockIdx.x * 256 + threadIdx.x] = s;
}

// Runs `blocks` workgroups of 4 waves, each wave `iters` rounds of 8 products
// of shape 0 (32x32x16 bf16, 32768 flops each) or 16 of shape 1 (16x16x32 f16,
// 16384 flops each); `out` must hold blocks * 256 floats.  Returns 0, or -1 on bad
// arguments or a failed launch.
extern "C" int moe_probe_mfma(int shape, float* out, int blocks, int iters, void* stream) {
    if (!out || blocks <= 0 || iters <= 0 || (shape != 0 && shape != 1)) return -1;
    const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (shape == 0) hipLaunchKernelGGL(k_mfma_probe<0>, dim3((unsigned)blocks), dim3(256), 0, st, out, iters, 1e-3f);
    else hipLaunchKernelGGL(k_mfma_probe<1>, dim3((unsigned)blocks), dim3(256), 0, st, out, iters, 1e-3f);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}
