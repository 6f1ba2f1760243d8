// ExactLinear with 8-bit weights ("Kimi exact-generator adaptation", "The
// proposed substitution": ExactLinear.from_weight with bits 4 or 8 and group
// size 32; the class body is not on the pages).  y[m][n] = sum over groups g
// (ascending, from 0) of fma(fl32(s_w[n][g] * (float)G), s_x[m][g], acc), with
// G the exact int32 dot product of the int8 codes of row m and weight row n
// over group g.  Weights are quantised like the activations (moe_quant_act_int8
// applied to the weight rows).
//
// Matrix cores: v_mfma_i32_32x32x32_i8 multiplies one whole group (32 K) per
// operation, so its int32 result is G itself.  Lane l = c + 32 kb supplies row
// (or column) c and bytes [16 kb, 16 kb + 16) of the group for both operands;
// result element i of lane l is row 8(i/4) + 4 kb + i%4, column c.  The fold is
// three VALU operations per result and group (convert, scale, fma), so the
// kernel is VALU-bound; it stages 64x128 tiles of both operands and their
// scales in LDS, one chunk at a time.
#include "moe_common.h"

namespace {

typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));
typedef int32_t i32x16_t __attribute__((ext_vector_type(16)));

constexpr int kXKC = 128;      // K per chunk (4 groups)
constexpr int kXStride = 144;  // bytes per LDS row (128 + 16 pad: conflict-free 16-byte reads)

// 64 x 64 output tile per workgroup; wave w owns rows 32 (w & 1) .. +32 and
// columns 32 (w >> 1) .. +32 of it.
__global__ __launch_bounds__(256) void k_exact_linear_i8w(const int8_t* __restrict__ qx, const float* __restrict__ sx,
                                                          const int8_t* __restrict__ qw, const float* __restrict__ sw,
                                                          int M, int N, int K, float* __restrict__ y) {
    __shared__ __attribute__((aligned(16))) int8_t Ax[64][kXStride];
    __shared__ __attribute__((aligned(16))) int8_t Bw[64][kXStride];
    __shared__ float SX[64][4];
    __shared__ float SW[64][4];

    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wave = tid >> 6;
    const int c32 = lane & 31;
    const int kb = lane >> 5;
    const int m0 = blockIdx.y * 64;
    const int n0 = blockIdx.x * 64;
    const int rb = wave & 1, cbk = wave >> 1;
    const int ng = K / 32;
    const int nch = K / kXKC;

    i32x16_t zero;
#pragma unroll
    for (int i = 0; i < 16; ++i) zero[i] = 0;
    float acc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.0f;

    for (int c = 0; c < nch; ++c) {
        // stage: 512 pieces of 16 bytes per operand (2 per thread); rows past the
        // matrix stage zeros (their results are never stored)
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int p = it * 256 + tid;
            const int row = p >> 3, piece = p & 7;
            const int mr = m0 + row, nr = n0 + row;
            i32x4_t va = {0, 0, 0, 0}, vb = {0, 0, 0, 0};
            if (mr < M) va = *reinterpret_cast<const i32x4_t*>(qx + (size_t)mr * K + c * kXKC + piece * 16);
            if (nr < N) vb = *reinterpret_cast<const i32x4_t*>(qw + (size_t)nr * K + c * kXKC + piece * 16);
            *reinterpret_cast<i32x4_t*>(&Ax[row][piece * 16]) = va;
            *reinterpret_cast<i32x4_t*>(&Bw[row][piece * 16]) = vb;
        }
        {
            const int row = tid >> 2, g = tid & 3;
            const int mr = m0 + row, nr = n0 + row;
            SX[row][g] = mr < M ? sx[(size_t)mr * ng + 4 * c + g] : 0.0f;
            SW[row][g] = nr < N ? sw[(size_t)nr * ng + 4 * c + g] : 0.0f;
        }
        __syncthreads();
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const i32x4_t a = *reinterpret_cast<const i32x4_t*>(&Ax[32 * rb + c32][32 * g + 16 * kb]);
            const i32x4_t b = *reinterpret_cast<const i32x4_t*>(&Bw[32 * cbk + c32][32 * g + 16 * kb]);
            const i32x16_t d = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, zero, 0, 0, 0);
            const float s_w = SW[32 * cbk + c32][g];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float s_x = SX[32 * rb + 8 * (i >> 2) + 4 * kb + (i & 3)][g];
                const float cw = s_w * (float)d[i];  // fl32(s_w * G); G < 2^20 converts exactly
                acc[i] = __builtin_fmaf(cw, s_x, acc[i]);
            }
        }
        __syncthreads();
    }

    const int col = n0 + 32 * cbk + c32;
    if (col < N) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int row = m0 + 32 * rb + 8 * (i >> 2) + 4 * kb + (i & 3);
            if (row < M) y[(size_t)row * N + col] = acc[i];
        }
    }
}

}  // namespace

extern "C" int moe_exact_linear_i8w(const int8_t* qx, const float* sx, const int8_t* qw, const float* sw, int M, int N,
                                    int K, float* y, void* stream) {
    using namespace moe;
    const char* what = "moe_exact_linear_i8w";
    if (M < 0 || N <= 0 || K <= 0) return fail(MOE_ERR_INVALID_ARG, "%s: bad sizes M=%d N=%d K=%d", what, M, N, K);
    if (K % kXKC != 0) return fail(MOE_ERR_UNSUPPORTED, "%s: K=%d (multiple of %d)", what, K, kXKC);
    if (M == 0) return MOE_OK;
    if (!qx || !sx || !qw || !sw || !y) return fail(MOE_ERR_INVALID_ARG, "%s: null pointer", what);
    if (!aligned16(qx) || !aligned16(qw)) return fail(MOE_ERR_INVALID_ARG, "%s: codes must be 16-byte aligned", what);
    const dim3 grid((unsigned)((N + 63) / 64), (unsigned)((M + 63) / 64));
    hipLaunchKernelGGL(k_exact_linear_i8w, grid, dim3(256), 0, as_stream(stream), qx, sx, qw, sw, M, N, K, y);
    return launch_status(what);
}
