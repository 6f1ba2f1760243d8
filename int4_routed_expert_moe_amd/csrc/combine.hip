// Weighted combine of the selected experts' outputs back into token order
// ("Kimi K2.5 donor reference", records "Sum the selected expert outputs with
// their routing weights" and "Add an always-active shared expert"; "Kimi-K3
// latent MoE" page, Code: moe_infer scatters the outputs back by the sort
// index, multiplies by topk_weight in the weight dtype and sums over the k
// slots, then casts back), and the exact-mode activation quantiser ("Kimi
// exact-generator adaptation", "The proposed substitution": ExactLinear with
// group size 32).
#include "moe_common.h"

namespace {

// Grid (token, 2048-column block); each thread owns 8 consecutive columns.  The
// KMAX slot rows are gathered through slot_pos with every load issued before
// the sum; slots past k repeat the last slot with weight 0 (adding w*y = +-0 to
// a sum that starts at +0 changes no bit).  fp32 multiply then add, slots in
// ascending order.
template <int MODE, int KMAX>
__global__ __launch_bounds__(256) void k_combine(const void* __restrict__ y, const int32_t* __restrict__ slot_pos,
                                                 const float* __restrict__ topk_w,
                                                 const uint16_t* __restrict__ shared, int k, int H,
                                                 void* __restrict__ out) {
    const int t = blockIdx.x;
    const int c = (blockIdx.y * blockDim.x + threadIdx.x) * 8;
    if (c >= H) return;
    int pj[KMAX];
    float wj[KMAX];
#pragma unroll
    for (int jj = 0; jj < KMAX; ++jj) {
        const int js = min(jj, k - 1);
        pj[jj] = slot_pos[(size_t)t * k + js];
        const float w = topk_w[(size_t)t * k + js];
        wj[jj] = jj < k ? w : 0.0f;
    }
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
    if (MODE == MOE_MODE_BF16) {
        u32x4_t v[KMAX];
#pragma unroll
        for (int jj = 0; jj < KMAX; ++jj)
            v[jj] = *reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(y) + (size_t)pj[jj] * H + c);
#pragma unroll
        for (int jj = 0; jj < KMAX; ++jj)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                acc[2 * q] = acc[2 * q] + wj[jj] * __uint_as_float(v[jj][q] << 16);
                acc[2 * q + 1] = acc[2 * q + 1] + wj[jj] * __uint_as_float(v[jj][q] & 0xFFFF0000u);
            }
        u32x4_t o;
        u32x4_t sh = {0u, 0u, 0u, 0u};
        if (shared) sh = *reinterpret_cast<const u32x4_t*>(shared + (size_t)t * H + c);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            uint32_t lo = f32_to_bf16_bits(acc[2 * q]);
            uint32_t hi = f32_to_bf16_bits(acc[2 * q + 1]);
            if (shared) {
                lo = f32_to_bf16_bits(bf16_bits_to_f32(lo) + __uint_as_float(sh[q] << 16));
                hi = f32_to_bf16_bits(bf16_bits_to_f32(hi) + __uint_as_float(sh[q] & 0xFFFF0000u));
            }
            o[q] = lo | (hi << 16);
        }
        *reinterpret_cast<u32x4_t*>(static_cast<uint16_t*>(out) + (size_t)t * H + c) = o;
    } else {
        f32x4_t v0[KMAX], v1[KMAX];
#pragma unroll
        for (int jj = 0; jj < KMAX; ++jj) {
            const float* yr = static_cast<const float*>(y) + (size_t)pj[jj] * H + c;
            v0[jj] = *reinterpret_cast<const f32x4_t*>(yr);
            v1[jj] = *reinterpret_cast<const f32x4_t*>(yr + 4);
        }
#pragma unroll
        for (int jj = 0; jj < KMAX; ++jj)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                acc[q] = acc[q] + wj[jj] * v0[jj][q];
                acc[4 + q] = acc[4 + q] + wj[jj] * v1[jj][q];
            }
        float* orow = static_cast<float*>(out) + (size_t)t * H + c;
        *reinterpret_cast<f32x4_t*>(orow) = f32x4_t{acc[0], acc[1], acc[2], acc[3]};
        *reinterpret_cast<f32x4_t*>(orow + 4) = f32x4_t{acc[4], acc[5], acc[6], acc[7]};
    }
}

// One thread per (row, group of 32): amax, s = amax/127, q = clamp(rint(x/s)).
__global__ __launch_bounds__(256) void k_quant_act(const uint16_t* __restrict__ x, long groups, int K,
                                                   int8_t* __restrict__ q, float* __restrict__ s) {
    const long gidx = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (gidx >= groups) return;
    const long row = gidx / (K / 32);
    const int g = (int)(gidx % (K / 32));
    const uint16_t* src = x + (size_t)row * K + (size_t)g * 32;
    float v[32];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const u32x4_t d = *reinterpret_cast<const u32x4_t*>(src + 8 * p);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[8 * p + 2 * i] = __uint_as_float(d[i] << 16);
            v[8 * p + 2 * i + 1] = __uint_as_float(d[i] & 0xFFFF0000u);
        }
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
    const float sc = amax == 0.0f ? 0.0f : amax / 127.0f;
    uint32_t packed[8];
#pragma unroll
    for (int w = 0; w < 8; ++w) {
        uint32_t acc = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) acc |= ((uint32_t)(moe_quant_i8(v[4 * w + b], sc) & 0xFF)) << (8 * b);
        packed[w] = acc;
    }
    int8_t* dst = q + (size_t)row * K + (size_t)g * 32;
    *reinterpret_cast<u32x4_t*>(dst) = u32x4_t{packed[0], packed[1], packed[2], packed[3]};
    *reinterpret_cast<u32x4_t*>(dst + 16) = u32x4_t{packed[4], packed[5], packed[6], packed[7]};
    s[gidx] = sc;
}

}  // namespace

extern "C" int moe_combine(int mode, const void* y, const int32_t* slot_pos, const float* topk_w,
                           const uint16_t* shared, int T, int k, int H, void* out, void* stream) {
    using namespace moe;
    const char* what = "moe_combine";
    if (mode != MOE_MODE_BF16 && mode != MOE_MODE_EXACT_I8) return fail(MOE_ERR_INVALID_ARG, "%s: mode %d", what, mode);
    if (T < 0 || k <= 0 || H <= 0) return fail(MOE_ERR_INVALID_ARG, "%s: bad sizes", what);
    if (k > 16 || H % 8) return fail(MOE_ERR_UNSUPPORTED, "%s: k=%d H=%d", what, k, H);
    if (T == 0) return MOE_OK;
    if (!y || !slot_pos || !topk_w || !out) return fail(MOE_ERR_INVALID_ARG, "%s: null pointer", what);
    if (mode == MOE_MODE_EXACT_I8 && shared) return fail(MOE_ERR_INVALID_ARG, "%s: exact mode takes no shared input", what);
    if (!aligned16(y) || !aligned16(out) || (shared && !aligned16(shared)))
        return fail(MOE_ERR_INVALID_ARG, "%s: y, out, shared must be 16-byte aligned", what);
    hipStream_t st = as_stream(stream);
    const dim3 grid((unsigned)T, (unsigned)((H / 8 + 255) / 256));
    if (mode == MOE_MODE_BF16) {
        if (k <= 8) hipLaunchKernelGGL((k_combine<MOE_MODE_BF16, 8>), grid, dim3(256), 0, st, y, slot_pos, topk_w, shared, k, H, out);
        else hipLaunchKernelGGL((k_combine<MOE_MODE_BF16, 16>), grid, dim3(256), 0, st, y, slot_pos, topk_w, shared, k, H, out);
    } else {
        if (k <= 8) hipLaunchKernelGGL((k_combine<MOE_MODE_EXACT_I8, 8>), grid, dim3(256), 0, st, y, slot_pos, topk_w, nullptr, k, H, out);
        else hipLaunchKernelGGL((k_combine<MOE_MODE_EXACT_I8, 16>), grid, dim3(256), 0, st, y, slot_pos, topk_w, nullptr, k, H, out);
    }
    return launch_status(what);
}

// 16-bit activation codes (exact mode with act_bits = 16): one group of 32 per
// thread, s = amax / 32767, codes clamped to +-32767.
__global__ __launch_bounds__(256) void k_quant_act16(const uint16_t* __restrict__ x, long groups, int K,
                                                     int16_t* __restrict__ q, float* __restrict__ s) {
    const long gidx = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (gidx >= groups) return;
    const long row = gidx / (K / 32);
    const int g = (int)(gidx % (K / 32));
    const uint16_t* src = x + (size_t)row * K + (size_t)g * 32;
    float v[32];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const u32x4_t d = *reinterpret_cast<const u32x4_t*>(src + 8 * p);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[8 * p + 2 * i] = __uint_as_float(d[i] << 16);
            v[8 * p + 2 * i + 1] = __uint_as_float(d[i] & 0xFFFF0000u);
        }
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
    const float sc = amax == 0.0f ? 0.0f : amax / 32767.0f;
    uint32_t packed[16];
#pragma unroll
    for (int w = 0; w < 16; ++w)
        packed[w] = ((uint32_t)moe_quant_i16(v[2 * w], sc) & 0xFFFFu) |
                    (((uint32_t)moe_quant_i16(v[2 * w + 1], sc) & 0xFFFFu) << 16);
    int16_t* dst = q + (size_t)row * K + (size_t)g * 32;
#pragma unroll
    for (int p = 0; p < 4; ++p)
        *reinterpret_cast<u32x4_t*>(dst + 8 * p) =
            u32x4_t{packed[4 * p], packed[4 * p + 1], packed[4 * p + 2], packed[4 * p + 3]};
    s[gidx] = sc;
}

extern "C" int moe_quant_act_int16(const uint16_t* x, int M, int K, int16_t* q, float* s, void* stream) {
    using namespace moe;
    const char* what = "moe_quant_act_int16";
    if (M < 0 || K <= 0) return fail(MOE_ERR_INVALID_ARG, "%s: bad sizes", what);
    if (K % 32) return fail(MOE_ERR_UNSUPPORTED, "%s: K=%d not a multiple of 32", what, K);
    if (M == 0) return MOE_OK;
    if (!x || !q || !s) return fail(MOE_ERR_INVALID_ARG, "%s: null pointer", what);
    if (!aligned16(x) || !aligned16(q)) return fail(MOE_ERR_INVALID_ARG, "%s: x, q must be 16-byte aligned", what);
    const long groups = (long)M * (K / 32);
    hipLaunchKernelGGL(k_quant_act16, dim3((unsigned)((groups + 255) / 256)), dim3(256), 0, as_stream(stream), x,
                       groups, K, q, s);
    return launch_status(what);
}

extern "C" int moe_quant_act_int8(const uint16_t* x, int M, int K, int8_t* q, float* s, void* stream) {
    using namespace moe;
    const char* what = "moe_quant_act_int8";
    if (M < 0 || K <= 0) return fail(MOE_ERR_INVALID_ARG, "%s: bad sizes", what);
    if (K % 32) return fail(MOE_ERR_UNSUPPORTED, "%s: K=%d not a multiple of 32", what, K);
    if (M == 0) return MOE_OK;
    if (!x || !q || !s) return fail(MOE_ERR_INVALID_ARG, "%s: null pointer", what);
    if (!aligned16(x) || !aligned16(q)) return fail(MOE_ERR_INVALID_ARG, "%s: x, q must be 16-byte aligned", what);
    const long groups = (long)M * (K / 32);
    hipLaunchKernelGGL(k_quant_act, dim3((unsigned)((groups + 255) / 256)), dim3(256), 0, as_stream(stream), x, groups,
                       K, q, s);
    return launch_status(what);
}
