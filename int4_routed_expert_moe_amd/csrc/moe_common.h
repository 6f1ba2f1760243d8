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

// Descriptor for raw buffer loads from `bytes` bytes at p (gfx9 family: the
// fourth word selects the 32-bit data format).  Offsets are 32-bit, and loads
// past the end return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
// The same for an address and size that are wave-uniform but computed from
// values the compiler cannot prove uniform: both are read from the first lane
// (a descriptor it took for divergent would be used through a loop over lanes).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc_uniform(const void* p, uint32_t bytes) {
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
    const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
    return buffer_rsrc(reinterpret_cast<const void*>(lo | (hi << 32)), (uint32_t)__builtin_amdgcn_readfirstlane((int)bytes));
}

// Workgroup barrier for LDS traffic only: waits for this wave's LDS operations
// (lgkmcnt) but not for its global loads, so prefetched weights and the next
// activation chunk stay in flight across it (a full __syncthreads also drains
// every outstanding global load).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// One 16-byte buffer load per lane written straight to LDS: lane l's bytes go
// to lds + 16 l (lds wave-uniform).  The builtin exists for the device pass
// only; the host pass compiles the kernels' launch stubs.
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t rsrc, void* lds, uint32_t voffset,
                                                  uint32_t soffset) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)lds, 16,
                                             voffset, soffset, 0, 0);
#else
    (void)rsrc, (void)lds, (void)voffset, (void)soffset;
#endif
}

// Wait until at most N vector-memory operations of this wave are outstanding
// (they complete in issue order).  Used where the compiler cannot see the wait:
// LDS written by global-to-LDS loads, read by other waves after a barrier.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    if constexpr (N == 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
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
