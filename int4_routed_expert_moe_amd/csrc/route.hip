// Router: fp32 logits in a fixed order, sigmoid scores, bias-corrected top-k
// selection and renormalisation ("Kimi K2.5 donor reference", records
// "MoEGate.forward: logits", "Independent sigmoid scores for the router",
// "Bias the choice of experts while retaining original affinities",
// "MoEGate.forward: ( , topk idx)" and "Normalize the selected routing
// affinities").
//
// The selected indices must be reproducible bit for bit, so every logit is
// one fp32 chain summed in ascending hidden index from 0 (no split, no
// matrix cores: their internal summation order is unspecified).  Lanes are
// tokens and each wave runs EPW such chains (one per expert) side by side;
// the expert rows are wave-uniform LDS reads (broadcasts).
#include "moe_common.h"

namespace {

constexpr int kRouteTok = 64;   // tokens per block (one per lane)
constexpr int kRouteKC = 64;    // hidden elements staged per LDS chunk
constexpr int kRouteWaves = 4;

// Logits of 64 tokens x (4 * EPW) experts.  Lanes are tokens; wave w runs the
// EPW chains of experts e0 + w*EPW + q side by side.  The x tile and the
// router rows of each 64-wide hidden chunk are staged in LDS as fp32, double
// buffered: the loads of chunk c+1 are in flight while chunk c is consumed,
// and one barrier per chunk orders the buffers.  Each chain adds its products
// in ascending hidden index, one fused multiply-add per element (the product
// of two bf16 values is exact in fp32, so this equals a multiply then an add).
template <int EPW>
__global__ __launch_bounds__(256) void k_router_logits(const uint16_t* __restrict__ x,
                                                       const uint16_t* __restrict__ w, int T, int H,
                                                       int E, float* __restrict__ logits) {
    constexpr int NE = kRouteWaves * EPW;                     // experts per block
    constexpr int XPIECES = kRouteTok * (kRouteKC / 8);       // 16-byte pieces of the x tile
    constexpr int WPIECES = NE * (kRouteKC / 8);              // 16-byte pieces of the w tile
    constexpr int XITER = (XPIECES + 255) / 256;
    constexpr int WITER = (WPIECES + 255) / 256;
    __shared__ __attribute__((aligned(16))) float xs[2][kRouteTok][kRouteKC + 4];
    __shared__ __attribute__((aligned(16))) float wsm[2][NE][kRouteKC];
    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wave = tid >> 6;
    const int t0 = blockIdx.x * kRouteTok;
    const int eb = blockIdx.y * NE;  // first expert of the block

    u32x4_t xq[XITER], wq[WITER];
    auto load = [&](int c) {
#pragma unroll
        for (int it = 0; it < XITER; ++it) {
            const int p = it * 256 + tid;
            const int row = p / (kRouteKC / 8), piece = p % (kRouteKC / 8);
            // out-of-range rows load row 0 and are zeroed by a select (no load under a branch)
            const bool ok = p < XPIECES && t0 + row < T;
            const u32x4_t v = *reinterpret_cast<const u32x4_t*>(x + (size_t)(ok ? t0 + row : 0) * H + c + (ok ? piece : 0) * 8);
            xq[it] = ok ? v : u32x4_t{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int it = 0; it < WITER; ++it) {
            const int p = it * 256 + tid;
            const int row = p / (kRouteKC / 8), piece = p % (kRouteKC / 8);
            const bool ok = p < WPIECES && eb + row < E;
            const u32x4_t v = *reinterpret_cast<const u32x4_t*>(w + (size_t)(ok ? eb + row : 0) * H + c + (ok ? piece : 0) * 8);
            wq[it] = ok ? v : u32x4_t{0u, 0u, 0u, 0u};
        }
    };
    auto store = [&](int buf) {
#pragma unroll
        for (int it = 0; it < XITER; ++it) {
            const int p = it * 256 + tid;
            if (p < XPIECES) {
                const int row = p / (kRouteKC / 8), piece = p % (kRouteKC / 8);
                float* dst = &xs[buf][row][piece * 8];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    dst[2 * j] = __uint_as_float(xq[it][j] << 16);
                    dst[2 * j + 1] = __uint_as_float(xq[it][j] & 0xFFFF0000u);
                }
            }
        }
#pragma unroll
        for (int it = 0; it < WITER; ++it) {
            const int p = it * 256 + tid;
            if (p < WPIECES) {
                const int row = p / (kRouteKC / 8), piece = p % (kRouteKC / 8);
                float* dst = &wsm[buf][row][piece * 8];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    dst[2 * j] = __uint_as_float(wq[it][j] << 16);
                    dst[2 * j + 1] = __uint_as_float(wq[it][j] & 0xFFFF0000u);
                }
            }
        }
    };

    float acc[EPW];
#pragma unroll
    for (int q = 0; q < EPW; ++q) acc[q] = 0.0f;
    const int nch = H / kRouteKC;
    load(0);
    store(0);
    __syncthreads();
    for (int c = 0; c < nch; ++c) {
        const int buf = c & 1;
        if (c + 1 < nch) load((c + 1) * kRouteKC);
#pragma unroll
        for (int i = 0; i < kRouteKC; i += 4) {
            const f32x4_t xv = *reinterpret_cast<const f32x4_t*>(&xs[buf][lane][i]);
#pragma unroll
            for (int q = 0; q < EPW; ++q) {
                const f32x4_t wv = *reinterpret_cast<const f32x4_t*>(&wsm[buf][wave * EPW + q][i]);
                float a = acc[q];
                a = __builtin_fmaf(xv[0], wv[0], a);
                a = __builtin_fmaf(xv[1], wv[1], a);
                a = __builtin_fmaf(xv[2], wv[2], a);
                a = __builtin_fmaf(xv[3], wv[3], a);
                acc[q] = a;
            }
        }
        if (c + 1 < nch) store(buf ^ 1);
        __syncthreads();
    }
    const int t = t0 + lane;
    if (t < T) {
#pragma unroll
        for (int q = 0; q < EPW; ++q) {
            const int e = eb + wave * EPW + q;
            if (e < E) logits[(size_t)t * E + e] = acc[q];
        }
    }
}

// One wave per token: scores, biased ranking keys, k rounds of a wave-wide
// arg-max (larger key, then lower expert index), renormalisation in rank order.
template <int NQ>
__global__ __launch_bounds__(256) void k_route_topk(const float* __restrict__ logits,
                                                    const float* __restrict__ bias, int T, int E,
                                                    int k, int renormalize,
                                                    int32_t* __restrict__ topk_idx,
                                                    float* __restrict__ topk_w) {
    const int lane = lane_id();
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    float s[NQ], key[NQ];
    uint32_t taken = 0;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const int e = lane + MOE_WAVE * q;
        if (e < E) {
            s[q] = moe_sigmoid(logits[(size_t)t * E + e]);
            key[q] = s[q] + bias[e];
        } else {
            s[q] = 0.0f;
            key[q] = -__builtin_huge_valf();
            taken |= 1u << q;
        }
    }
    int sel_e = 0;
    float sel_s = 0.0f;
    float denom = 0.0f;
    for (int j = 0; j < k; ++j) {
        float bk = -__builtin_huge_valf(), bs = 0.0f;
        int be = 0x7FFFFFFF;
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            if (!((taken >> q) & 1u) && (key[q] > bk || be == 0x7FFFFFFF)) {
                bk = key[q];
                bs = s[q];
                be = lane + MOE_WAVE * q;
            }
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            const float ok = __shfl_xor(bk, off);
            const float os = __shfl_xor(bs, off);
            const int oe = __shfl_xor(be, off);
            if (oe != 0x7FFFFFFF && (be == 0x7FFFFFFF || ok > bk || (ok == bk && oe < be))) {
                bk = ok;
                bs = os;
                be = oe;
            }
        }
        if ((be & (MOE_WAVE - 1)) == lane) taken |= 1u << (be / MOE_WAVE);
        denom = denom + bs;  // rank order, as the selection produced them
        if (lane == j) {
            sel_e = be;
            sel_s = bs;
        }
    }
    denom = denom + 1e-20f;
    if (lane < k) {
        topk_idx[(size_t)t * k + lane] = sel_e;
        topk_w[(size_t)t * k + lane] = renormalize ? sel_s / denom : sel_s;
    }
}

template <int NQ>
void launch_topk(const float* logits, const float* bias, int T, int E, int k, int renorm,
                 int32_t* idx, float* w, hipStream_t st) {
    hipLaunchKernelGGL(k_route_topk<NQ>, dim3((T + 3) / 4), dim3(256), 0, st, logits, bias, T, E, k,
                       renorm, idx, w);
}

}  // namespace

extern "C" size_t moe_route_workspace_bytes(int T, int E) {
    if (T <= 0 || E <= 0) return 0;
    return (size_t)T * (size_t)E * sizeof(float);
}

extern "C" int moe_route(const uint16_t* x, const uint16_t* w_router, const float* bias, int T,
                         int H, int E, int k, int renormalize, int32_t* topk_idx, float* topk_w,
                         void* ws, size_t ws_bytes, void* stream) {
    using namespace moe;
    if (T < 0 || H <= 0 || E <= 0 || k <= 0)
        return fail(MOE_ERR_INVALID_ARG, "moe_route: bad sizes T=%d H=%d E=%d k=%d", T, H, E, k);
    if (E > 1024 || k > 16 || k > E)
        return fail(MOE_ERR_UNSUPPORTED, "moe_route: need k <= min(E,16), E <= 1024 (E=%d k=%d)", E, k);
    if (H % kRouteKC != 0)
        return fail(MOE_ERR_UNSUPPORTED, "moe_route: H=%d must be a multiple of %d", H, kRouteKC);
    if (T == 0) return MOE_OK;
    if (!x || !w_router || !bias || !topk_idx || !topk_w)
        return fail(MOE_ERR_INVALID_ARG, "moe_route: null pointer");
    if (!aligned16(x) || !aligned16(w_router))
        return fail(MOE_ERR_INVALID_ARG, "moe_route: x and w_router must be 16-byte aligned");
    if (!ws || ws_bytes < moe_route_workspace_bytes(T, E))
        return fail(MOE_ERR_WORKSPACE, "moe_route: workspace %zu < %zu bytes", ws_bytes,
                    moe_route_workspace_bytes(T, E));
    hipStream_t st = as_stream(stream);
    float* logits = static_cast<float*>(ws);
    const int tb = (T + kRouteTok - 1) / kRouteTok;
    if (T <= 256) {
        dim3 grid(tb, (E + kRouteWaves - 1) / kRouteWaves);
        hipLaunchKernelGGL(k_router_logits<1>, grid, dim3(256), 0, st, x, w_router, T, H, E, logits);
    } else {
        dim3 grid(tb, (E + kRouteWaves * 8 - 1) / (kRouteWaves * 8));
        hipLaunchKernelGGL(k_router_logits<8>, grid, dim3(256), 0, st, x, w_router, T, H, E, logits);
    }
    int rc = launch_status("moe_route logits");
    if (rc) return rc;
    const int nq = (E + MOE_WAVE - 1) / MOE_WAVE;
    if (nq <= 1) launch_topk<1>(logits, bias, T, E, k, renormalize, topk_idx, topk_w, st);
    else if (nq <= 2) launch_topk<2>(logits, bias, T, E, k, renormalize, topk_idx, topk_w, st);
    else if (nq <= 4) launch_topk<4>(logits, bias, T, E, k, renormalize, topk_idx, topk_w, st);
    else if (nq <= 8) launch_topk<8>(logits, bias, T, E, k, renormalize, topk_idx, topk_w, st);
    else launch_topk<16>(logits, bias, T, E, k, renormalize, topk_idx, topk_w, st);
    return launch_status("moe_route topk");
}
