// Shared host/device helpers of the gfx950 MoE library (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe_int4.h"

#define MOE_WAVE 64

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// host side: status reporting (status.cpp)
// ---------------------------------------------------------------------------
namespace moe {
int fail(int status, const char* fmt, ...);
int launch_status(const char* what);  // MOE_OK, or MOE_ERR_LAUNCH after a failed launch
bool aligned16(const void* p);
inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }
// Blocks of a 1-D grid are dealt to the 8 XCDs round robin; this many blocks
// per XCD cover `n` logical blocks.
inline int per_xcd(long n) { return (int)((n + 7) / 8); }
}  // namespace moe

// ---------------------------------------------------------------------------
// device side
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// Round a finite fp32 value to bf16 (nearest, ties to even).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// Map a logical block id onto the launched 1-D grid so that consecutive
// logical ids run on the same XCD (and share its L2).  The grid has
// 8 * per_xcd blocks; ids >= n_logical are surplus and must exit.
__device__ __forceinline__ long xcd_logical_block(int per_xcd) {
    long b = blockIdx.x;
    return (b & 7) * (long)per_xcd + (b >> 3);
}

// e^t for the router's sigmoid and SiLU: Cody-Waite reduction t = n ln2 + r
// with n = rint(t log2 e) and a two-part ln2, the degree-7 Taylor polynomial
// of e^r by Horner's rule with fused multiply-adds, then scaling by 2^n
// (W. J. Cody, W. Waite, Software Manual for the Elementary Functions, 1980).
// Each constant is the binary32 value nearest to the stated real number.
// Compiled with contraction off: the only fused operations are the explicit fmaf.
__device__ __forceinline__ float moe_exp(float t) {
    const float kLog2e = 0x1.715476p+0f;   // log2(e)
    const float kLn2Hi = 0x1.62e430p-1f;   // ln 2
    const float kLn2Lo = -0x1.05c610p-29f; // ln 2 - kLn2Hi
    float n = __builtin_rintf(t * kLog2e);
    float r = __builtin_fmaf(-n, kLn2Hi, t);
    r = __builtin_fmaf(-n, kLn2Lo, r);
    float p = 0x1.a01a02p-13f;             // 1/7!
    p = __builtin_fmaf(p, r, 0x1.6c16c2p-10f); // 1/6!
    p = __builtin_fmaf(p, r, 0x1.111112p-7f);  // 1/5!
    p = __builtin_fmaf(p, r, 0x1.555556p-5f);  // 1/4!
    p = __builtin_fmaf(p, r, 0x1.555556p-3f);  // 1/3!
    p = __builtin_fmaf(p, r, 0x1.000000p-1f);  // 1/2!
    p = __builtin_fmaf(p, r, 1.0f);            // 1/1!
    p = __builtin_fmaf(p, r, 1.0f);            // 1/0!
    return __builtin_ldexpf(p, (int)n);
}

// Logistic function with the argument clamped to [-80, 80] (keeps e^-z normal).
__device__ __forceinline__ float moe_sigmoid(float z) {
    float zc = z < -80.0f ? -80.0f : (z > 80.0f ? 80.0f : z);
    return 1.0f / (1.0f + moe_exp(-zc));
}

__device__ __forceinline__ float moe_silu(float z) { return z * moe_sigmoid(z); }

// Symmetric int8 quantisation of one value given the group scale s = amax/127.
__device__ __forceinline__ int32_t moe_quant_i8(float v, float s) {
    if (s == 0.0f) return 0;
    float r = __builtin_rintf(v / s);
    r = r > 127.0f ? 127.0f : (r < -127.0f ? -127.0f : r);
    return (int32_t)r;
}

// The same quantiser for 16-bit codes: clamp to +-32767.
__device__ __forceinline__ int32_t moe_quant_i16(float v, float s) {
    if (s == 0.0f) return 0;
    float r = __builtin_rintf(v / s);
    r = r > 32767.0f ? 32767.0f : (r < -32767.0f ? -32767.0f : r);
    return (int32_t)r;
}

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (MOE_WAVE - 1)); }
