// Exact int4 x int8 group sums on the int8 matrix cores ("Kimi exact-generator
// adaptation", "Sources & provenance": ExactLinear / PackedInt4Linear compute
// the int4 multiply-accumulate exactly).  One wave per 16x16 output block;
// each v_mfma_i32_16x16x32_i8 covers exactly one 32-element scale group, so its
// int32 result is that group's exact dot product.
#include "moe_common.h"

namespace {

// 8 int4 (one packed dword) -> 8 sign-extended int8 in element order.
__device__ __forceinline__ long unpack_i4_to_i8(uint32_t w) {
    uint64_t r = 0;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        const int q = (int)((w >> (4 * p)) & 0xFu);
        const int v = (q ^ 8) - 8;
        r |= (uint64_t)(uint8_t)(int8_t)v << (8 * p);
    }
    return (long)r;
}

__global__ __launch_bounds__(64) void k_group_sums(const int8_t* __restrict__ qx, const uint8_t* __restrict__ packed,
                                                   int N, int K, int32_t* __restrict__ G) {
    const int lane = lane_id();
    const int r = lane & 15, j = lane >> 4;
    const int m0 = blockIdx.x * 16, n0 = blockIdx.y * 16;
    const int NG = K / 32;
    const int8_t* arow = qx + (size_t)(m0 + r) * K;
    const uint8_t* brow = packed + (size_t)(n0 + r) * (K / 2);
    for (int g = 0; g < NG; ++g) {
        const long av = *reinterpret_cast<const long*>(arow + 32 * g + 8 * j);
        const long bv = unpack_i4_to_i8(*reinterpret_cast<const uint32_t*>(brow + 16 * g + 4 * j));
        const i32x4_t d = __builtin_amdgcn_mfma_i32_16x16x32_i8(av, bv, i32x4_t{0, 0, 0, 0}, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) G[((size_t)(m0 + 4 * j + i) * N + n0 + r) * NG + g] = d[i];
    }
}

}  // namespace

extern "C" int moe_int4_group_sums_i32(const int8_t* q_x, const uint8_t* packed, int M, int N, int K,
                                       int32_t* G, void* stream) {
    using namespace moe;
    const char* what = "moe_int4_group_sums_i32";
    if (M < 0 || N <= 0 || K <= 0) return fail(MOE_ERR_INVALID_ARG, "%s: bad sizes", what);
    if (M % 16 || N % 16 || K % 32) return fail(MOE_ERR_UNSUPPORTED, "%s: M,N multiples of 16, K of 32", what);
    if (M == 0) return MOE_OK;
    if (!q_x || !packed || !G) return fail(MOE_ERR_INVALID_ARG, "%s: null pointer", what);
    if (!aligned16(q_x) || !aligned16(packed)) return fail(MOE_ERR_INVALID_ARG, "%s: inputs must be 16-byte aligned", what);
    hipLaunchKernelGGL(k_group_sums, dim3(M / 16, N / 16), dim3(64), 0, as_stream(stream), q_x, packed, N, K, G);
    return launch_status(what);
}
