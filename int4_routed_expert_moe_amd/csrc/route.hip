// Router: fp32 logits in a fixed order, sigmoid scores, bias-corrected top-k
// selection and renormalisation ("Kimi K2.5 donor reference", records
// "MoEGate.forward: logits", "Independent sigmoid scores for the router",
// "Bias the choice of experts while retaining original affinities",
// "MoEGate.forward: ( , topk idx)" and "Normalize the selected routing
// affinities").
//
// The selected indices must be reproducible bit for bit, so every logit is
// summed in one fixed fp32 order: each 64-element hidden block from 0 in
// ascending index, then the block sums from 0 in ascending block order.  Few
// tokens: fma chains on the VALU; many: the fp32 matrix-core shape with K = 1,
// which adds one product per step with one rounding (no multi-term sums).
#include "moe_common.h"

#include <algorithm>

namespace {

constexpr int kRouteTok = 64;   // tokens per block
constexpr int kRouteKC = 64;    // hidden elements per block sum (one LDS chunk)
constexpr int kRouterWaves = 4; // waves (16 experts each) per many-token logits workgroup
// grids of up to this many workgroups (one per CU) take the two-chain logits kernel
constexpr long kRouterPairMaxTiles = 256;

// Stage 64 rows x 64 hidden elements of a bf16 matrix as fp32, transposed to
// [i][row]; rows at or past `limit` are zero.  Two 16-byte pieces per thread.
struct TileLoad {
    u32x4_t v[2];
};
__device__ __forceinline__ void tile_load(TileLoad& tl, const uint16_t* __restrict__ m, int row0, int limit, int H,
                                          int col0) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        // 512 pieces of 8 elements; consecutive lanes take consecutive rows of one
        // piece, so the transposed LDS stores below hit 64 distinct banks
        const int p = it * 256 + tid;
        const int row = p & 63, piece = p >> 6;
        const bool ok = row0 + row < limit;
        tl.v[it] = *reinterpret_cast<const u32x4_t*>(m + (size_t)(ok ? row0 + row : 0) * H + col0 + piece * 8);
        if (!ok) tl.v[it] = u32x4_t{0u, 0u, 0u, 0u};
    }
}
__device__ __forceinline__ void tile_store(const TileLoad& tl, float (*dst)[64 + 4]) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const int p = it * 256 + tid;
        const int row = p & 63, piece = p >> 6;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            dst[piece * 8 + 2 * j][row] = __uint_as_float(tl.v[it][j] << 16);
            dst[piece * 8 + 2 * j + 1][row] = __uint_as_float(tl.v[it][j] & 0xFFFF0000u);
        }
    }
}

// One 64-long ascending chain per (token, expert) of a 4x4 register tile.
__device__ __forceinline__ void block_chain(const float (*xs)[64 + 4], const float (*ws)[64 + 4], int tt, int te,
                                            float (&acc)[4][4]) {
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[a][c] = 0.0f;
#pragma unroll 4
    for (int i = 0; i < kRouteKC; ++i) {
        const f32x4_t xv = *reinterpret_cast<const f32x4_t*>(&xs[i][4 * tt]);
        const f32x4_t wv = *reinterpret_cast<const f32x4_t*>(&ws[i][4 * te]);
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[a][c] = __builtin_fmaf(xv[a], wv[c], acc[a][c]);
    }
}

// Logits on the matrix cores.  The fp32 16x16x1 shape adds one product to
// each output per instruction with a single rounding, the same as an fma
// (products of bf16 values are exact in fp32), so a run of them in ascending
// hidden index is exactly the block chain; the block sums are then added to the
// running totals in ascending block order on the VALU.  A workgroup of NW waves
// owns 64 tokens x 16 NW experts; wave w multiplies all 64 tokens (four blocks
// of 16) by experts e0 + 16w .. e0 + 16w + 15.  Per 64-wide hidden block the
// token and router tiles go straight from memory to LDS by buffer loads as
// 16-byte pieces of 8 elements, laid out [piece][row] (tokens: 64 rows; router:
// 16 NW rows), so that the operand reads are 16 bytes per lane, conflict free.
// Three tile buffers: block b+2 loads while block b is multiplied, and each wave
// waits for its own loads of block b+1 before the barrier that ends step b.
// Lane l feeds token t0 + l and expert e0 + 16w + l mod 16; element i of its
// result is token t0 + 16(i/4) + 4(l/16) + i mod 4.  Rows past T or E load a
// valid row and are not stored.  The expert tiles of one token tile run on one
// XCD.
template <int NW>
__global__ __launch_bounds__(64 * NW) void k_router_mfma(const uint16_t* __restrict__ x,
                                                         const uint16_t* __restrict__ w, int T, int H, int E,
                                                         float* __restrict__ logits, int n_et, int per_xcd) {
    constexpr int RW = 16 * NW;           // router rows per tile
    constexpr int NI = 8 + RW / 8;        // 1-KB load instructions per block (token tile: 8)
    static_assert(NI % NW == 0, "load instructions shared evenly by the waves");
    constexpr int PER = NI / NW;          // this wave's load instructions per block
    __shared__ __attribute__((aligned(16))) uint16_t X0[8][64][8], X1[8][64][8], X2[8][64][8];
    __shared__ __attribute__((aligned(16))) uint16_t W0[8][RW][8], W1[8][RW][8], W2[8][RW][8];
    auto xt = [&](auto bc) -> uint16_t(&)[8][64][8] {
        if constexpr (decltype(bc)::value == 0) return X0;
        else if constexpr (decltype(bc)::value == 1) return X1;
        else return X2;
    };
    auto wt = [&](auto bc) -> uint16_t(&)[8][RW][8] {
        if constexpr (decltype(bc)::value == 0) return W0;
        else if constexpr (decltype(bc)::value == 1) return W1;
        else return W2;
    };

    const long L = xcd_logical_block(per_xcd);
    const long n_tt = (T + kRouteTok - 1) / kRouteTok;
    if (L >= n_tt * n_et) return;
    const int t0 = (int)(L / n_et) * kRouteTok;
    const int e0 = (int)(L % n_et) * RW;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int NB = H / kRouteKC;

    // this wave's load instructions j = wave + NW m: j < 8 is piece j of the
    // token tile (lane l: row l); j >= 8 covers router slots 64 (j - 8) + l of
    // the [piece][row] layout
    const __amdgpu_buffer_rsrc_t xr = buffer_rsrc(x, (uint32_t)((size_t)T * H * 2));
    const __amdgpu_buffer_rsrc_t wr = buffer_rsrc(w, (uint32_t)((size_t)E * H * 2));
    uint32_t voff[PER];
#pragma unroll
    for (int m = 0; m < PER; ++m) {
        const int j = wave + NW * m;
        if (j < 8) {
            voff[m] = ((uint32_t)min(t0 + lane, T - 1) * (uint32_t)H + 8u * (uint32_t)j) * 2u;
        } else {
            const int s = 64 * (j - 8) + lane;
            voff[m] = ((uint32_t)min(e0 + s % RW, E - 1) * (uint32_t)H + 8u * (uint32_t)(s / RW)) * 2u;
        }
    }
    auto load_block = [&](int b, auto bc) __attribute__((always_inline)) {
#pragma unroll
        for (int m = 0; m < PER; ++m) {
            const int j = wave + NW * m;
            if (j < 8) buffer_load_lds16(xr, &xt(bc)[j][0][0], voff[m], (uint32_t)b * (kRouteKC * 2));
            else buffer_load_lds16(wr, &wt(bc)[0][0][0] + 64 * 8 * (j - 8), voff[m], (uint32_t)b * (kRouteKC * 2));
        }
    };
    auto elem = [](const u32x4_t& v, int q) __attribute__((always_inline)) {
        return __uint_as_float((q & 1) ? (v[q >> 1] & 0xFFFF0000u) : (v[q >> 1] << 16));
    };
    f32x16_t tot = {};
    // one block: 64 dependent steps from zero, then the block sum into the total
    auto block = [&](auto bc) __attribute__((always_inline)) {
        f32x16_t part = {};
#pragma unroll
        for (int g = 0; g < 8; ++g) {
            const u32x4_t xa = *reinterpret_cast<const u32x4_t*>(&xt(bc)[g][lane][0]);
            const u32x4_t wa = *reinterpret_cast<const u32x4_t*>(&wt(bc)[g][16 * wave + (lane & 15)][0]);
#pragma unroll
            for (int q = 0; q < 8; ++q)
                part = __builtin_amdgcn_mfma_f32_16x16x1f32(elem(xa, q), elem(wa, q), part, 0, 0, 0);
        }
        tot = tot + part;
    };
    auto step = [&](auto bc, int b) __attribute__((always_inline)) {
        constexpr std::integral_constant<int, (decltype(bc)::value + 2) % 3> bn{};
        load_block(min(b + 2, NB - 1), bn);  // past the end: a redundant in-bounds load, never used
        block(bc);
        wait_vmcnt<PER>();  // this wave's loads of block b+1 have landed
        lds_barrier();
    };
    constexpr std::integral_constant<int, 0> B0{};
    constexpr std::integral_constant<int, 1> B1{};
    constexpr std::integral_constant<int, 2> B2{};
    load_block(0, B0);
    load_block(min(1, NB - 1), B1);
    wait_vmcnt<PER>();
    lds_barrier();
    int b = 0;
    for (; b + 3 <= NB; b += 3) {
        step(B0, b);
        step(B1, b + 1);
        step(B2, b + 2);
    }
    if (b < NB) step(B0, b);
    if (b + 1 < NB) step(B1, b + 1);
    wait_vmcnt<0>();  // the trailing redundant loads land before the workgroup ends

    const int ex = e0 + 16 * wave + (lane & 15);
    if (ex >= E) return;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int tok = t0 + 16 * (i >> 2) + 4 * (lane >> 4) + (i & 3);
        if (tok < T) logits[(size_t)tok * E + ex] = tot[i];
    }
}

// k_router_mfma for grids of at most one workgroup per CU (2048 tokens at 384
// experts: 192 workgroups): each wave then runs alone on its SIMD, and its one
// chain of dependent matrix-core steps leaves the pipe idle between steps.
// Here a wave multiplies two consecutive hidden blocks at once, as two
// independent chains whose steps alternate; the two block sums still enter the
// total in block order, so the results are those of k_router_mfma.  Tiles go
// through four LDS buffers in two pairs (64 KB, two workgroups per CU at most,
// which is why larger grids keep the three-buffer kernel).
template <int NW>
__global__ __launch_bounds__(64 * NW) void k_router_mfma_pair(const uint16_t* __restrict__ x,
                                                              const uint16_t* __restrict__ w, int T, int H, int E,
                                                              float* __restrict__ logits, int n_et,
                                                              int per_xcd) {
    constexpr int RW = 16 * NW;           // router rows per tile
    constexpr int NI = 8 + RW / 8;        // 1-KB load instructions per block (token tile: 8)
    static_assert(NI % NW == 0, "load instructions shared evenly by the waves");
    constexpr int PER = NI / NW;          // this wave's load instructions per block
    // four tile buffers in two pairs: a step multiplies the two blocks of one pair
    // while the next two blocks load into the other (separate LDS objects, so that
    // the compiler can tell a read of one buffer from the loads into another)
    __shared__ __attribute__((aligned(16))) uint16_t X0[8][64][8], X1[8][64][8], X2[8][64][8], X3[8][64][8];
    __shared__ __attribute__((aligned(16))) uint16_t W0[8][RW][8], W1[8][RW][8], W2[8][RW][8], W3[8][RW][8];
    auto xt = [&](auto bc) -> uint16_t(&)[8][64][8] {
        if constexpr (decltype(bc)::value == 0) return X0;
        else if constexpr (decltype(bc)::value == 1) return X1;
        else if constexpr (decltype(bc)::value == 2) return X2;
        else return X3;
    };
    auto wt = [&](auto bc) -> uint16_t(&)[8][RW][8] {
        if constexpr (decltype(bc)::value == 0) return W0;
        else if constexpr (decltype(bc)::value == 1) return W1;
        else if constexpr (decltype(bc)::value == 2) return W2;
        else return W3;
    };

    const long L = xcd_logical_block(per_xcd);
    const long n_tt = (T + kRouteTok - 1) / kRouteTok;
    if (L >= n_tt * n_et) return;
    const int t0 = (int)(L / n_et) * kRouteTok;
    const int e0 = (int)(L % n_et) * RW;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int NB = H / kRouteKC;

    // this wave's load instructions j = wave + NW m: j < 8 is piece j of the
    // token tile (lane l: row l); j >= 8 covers router slots 64 (j - 8) + l of
    // the [piece][row] layout
    const __amdgpu_buffer_rsrc_t xr = buffer_rsrc(x, (uint32_t)((size_t)T * H * 2));
    const __amdgpu_buffer_rsrc_t wr = buffer_rsrc(w, (uint32_t)((size_t)E * H * 2));
    uint32_t voff[PER];
#pragma unroll
    for (int m = 0; m < PER; ++m) {
        const int j = wave + NW * m;
        if (j < 8) {
            voff[m] = ((uint32_t)min(t0 + lane, T - 1) * (uint32_t)H + 8u * (uint32_t)j) * 2u;
        } else {
            const int s = 64 * (j - 8) + lane;
            voff[m] = ((uint32_t)min(e0 + s % RW, E - 1) * (uint32_t)H + 8u * (uint32_t)(s / RW)) * 2u;
        }
    }
    auto load_block = [&](int b, auto bc) __attribute__((always_inline)) {
#pragma unroll
        for (int m = 0; m < PER; ++m) {
            const int j = wave + NW * m;
            if (j < 8) buffer_load_lds16(xr, &xt(bc)[j][0][0], voff[m], (uint32_t)b * (kRouteKC * 2));
            else buffer_load_lds16(wr, &wt(bc)[0][0][0] + 64 * 8 * (j - 8), voff[m], (uint32_t)b * (kRouteKC * 2));
        }
    };
    auto elem = [](const u32x4_t& v, int q) __attribute__((always_inline)) {
        return __uint_as_float((q & 1) ? (v[q >> 1] & 0xFFFF0000u) : (v[q >> 1] << 16));
    };
    f32x16_t tot = {};
    // two consecutive blocks as two independent 64-step chains from zero, their
    // steps interleaved (one chain's latency hides behind the other's), then the
    // two block sums into the total in block order
    auto block2 = [&](auto bc0, auto bc1) __attribute__((always_inline)) {
        f32x16_t p0 = {}, p1 = {};
#pragma unroll
        for (int g = 0; g < 8; ++g) {
            const u32x4_t xa0 = *reinterpret_cast<const u32x4_t*>(&xt(bc0)[g][lane][0]);
            const u32x4_t wa0 = *reinterpret_cast<const u32x4_t*>(&wt(bc0)[g][16 * wave + (lane & 15)][0]);
            const u32x4_t xa1 = *reinterpret_cast<const u32x4_t*>(&xt(bc1)[g][lane][0]);
            const u32x4_t wa1 = *reinterpret_cast<const u32x4_t*>(&wt(bc1)[g][16 * wave + (lane & 15)][0]);
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                p0 = __builtin_amdgcn_mfma_f32_16x16x1f32(elem(xa0, q), elem(wa0, q), p0, 0, 0, 0);
                p1 = __builtin_amdgcn_mfma_f32_16x16x1f32(elem(xa1, q), elem(wa1, q), p1, 0, 0, 0);
            }
        }
        tot = tot + p0;
        tot = tot + p1;
    };
    // one block: 64 dependent steps from zero, then the block sum into the total
    auto block1 = [&](auto bc) __attribute__((always_inline)) {
        f32x16_t part = {};
#pragma unroll
        for (int g = 0; g < 8; ++g) {
            const u32x4_t xa = *reinterpret_cast<const u32x4_t*>(&xt(bc)[g][lane][0]);
            const u32x4_t wa = *reinterpret_cast<const u32x4_t*>(&wt(bc)[g][16 * wave + (lane & 15)][0]);
#pragma unroll
            for (int q = 0; q < 8; ++q)
                part = __builtin_amdgcn_mfma_f32_16x16x1f32(elem(xa, q), elem(wa, q), part, 0, 0, 0);
        }
        tot = tot + part;
    };
    // step over blocks b, b+1 in pair P (buffers 2P, 2P+1): blocks b+2, b+3 load
    // into the other pair (read last in the previous step, before its barrier)
    auto step2 = [&](auto pc, int b) __attribute__((always_inline)) {
        constexpr int P = decltype(pc)::value;
        load_block(min(b + 2, NB - 1), std::integral_constant<int, 2 * (1 - P)>{});
        load_block(min(b + 3, NB - 1), std::integral_constant<int, 2 * (1 - P) + 1>{});
        block2(std::integral_constant<int, 2 * P>{}, std::integral_constant<int, 2 * P + 1>{});
        wait_vmcnt<0>();  // this wave's loads of blocks b+2, b+3 have landed
        lds_barrier();
    };
    constexpr std::integral_constant<int, 0> P0{};
    constexpr std::integral_constant<int, 1> P1{};
    load_block(0, std::integral_constant<int, 0>{});
    load_block(min(1, NB - 1), std::integral_constant<int, 1>{});
    wait_vmcnt<0>();
    lds_barrier();
    int b = 0;
    for (; b + 4 <= NB; b += 4) {
        step2(P0, b);
        step2(P1, b + 2);
    }
    // 0..3 blocks left, the next two (if any) in buffers 0 and 1
    if (NB - b >= 2) {
        step2(P0, b);
        if (NB - b == 3) block1(std::integral_constant<int, 2>{});
    } else if (NB - b == 1) {
        block1(std::integral_constant<int, 0>{});
    }

    const int ex = e0 + 16 * wave + (lane & 15);
    if (ex >= E) return;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int tok = t0 + 16 * (i >> 2) + 4 * (lane >> 4) + (i & 3);
        if (tok < T) logits[(size_t)tok * E + ex] = tot[i];
    }
}

// Block sums of the logits for few tokens: P[t][b][e] = sum over the 64-wide
// hidden block b in ascending index.  Every (token, expert, block) is an
// independent 64-long chain, so all of them run in parallel; the top-k kernel
// adds the block sums of each logit in ascending block order.
// Grid: (H/64, ceil(E/64), ceil(T/64)); each thread owns 4 tokens x 4 experts.
__global__ __launch_bounds__(256) void k_router_partials(const uint16_t* __restrict__ x,
                                                         const uint16_t* __restrict__ w, int T, int H,
                                                         int E, float* __restrict__ P) {
    __shared__ __attribute__((aligned(16))) float xs[kRouteKC][64 + 4];  // [i][t]
    __shared__ __attribute__((aligned(16))) float ws[kRouteKC][64 + 4];  // [i][e]
    const int tid = threadIdx.x;
    const int b = blockIdx.x;
    const int e0 = blockIdx.y * 64;
    const int t0 = blockIdx.z * 64;
    const int NB = H / kRouteKC;
    TileLoad lx, lw;
    tile_load(lx, x, t0, T, H, b * kRouteKC);
    tile_load(lw, w, e0, E, H, b * kRouteKC);
    tile_store(lx, xs);
    tile_store(lw, ws);
    __syncthreads();
    const int tt = tid >> 4, te = tid & 15;
    float acc[4][4];
    block_chain(xs, ws, tt, te, acc);
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        const int t = t0 + 4 * tt + a;
        if (t >= T) continue;
        float* dst = P + ((size_t)t * NB + b) * E + e0 + 4 * te;
        if (e0 + 4 * te + 3 < E) {
            *reinterpret_cast<f32x4_t*>(dst) = f32x4_t{acc[a][0], acc[a][1], acc[a][2], acc[a][3]};
        } else {
#pragma unroll
            for (int c = 0; c < 4; ++c)
                if (e0 + 4 * te + c < E) dst[c] = acc[a][c];
        }
    }
}

// logits[t][e] = sum of the block sums P[t][b][e] in ascending b, one thread
// per (token, expert); the loads of 16 blocks are issued before their adds.
__global__ __launch_bounds__(256) void k_router_blocksum(const float* __restrict__ P, int T, int NB, int E,
                                                         float* __restrict__ logits) {
    const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (long)T * E) return;
    const long t = idx / E;
    const int e = (int)(idx % E);
    const float* src = P + (size_t)t * NB * E + e;
    float total = 0.0f;
    constexpr int BB = 16;
    int b = 0;
    for (; b + BB <= NB; b += BB) {
        float v[BB];
#pragma unroll
        for (int u = 0; u < BB; ++u) v[u] = src[(size_t)(b + u) * E];
#pragma unroll
        for (int u = 0; u < BB; ++u) total = total + v[u];
    }
    for (; b < NB; ++b) total = total + src[(size_t)b * E];
    logits[idx] = total;
}

// One wave per token: scores, biased ranking keys, k rounds of a wave-wide
// arg-max (larger key, then lower expert index), renormalisation in rank order.
template <int NQ>
__global__ __launch_bounds__(256) void k_route_topk(const float* __restrict__ logits,
                                                    const float* __restrict__ bias, int T, int E,
                                                    int k, int renormalize, int n_group, int topk_group,
                                                    float scale, int32_t* __restrict__ topk_idx,
                                                    float* __restrict__ topk_w) {
    const int lane = lane_id();
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    float s[NQ], key[NQ];
    uint32_t taken = 0;
    float lg[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) lg[q] = logits[(size_t)t * E + min(lane + MOE_WAVE * q, E - 1)];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const int e = lane + MOE_WAVE * q;
        if (e < E) {
            s[q] = moe_sigmoid(lg[q]);
            key[q] = s[q] + bias[e];
        } else {
            s[q] = 0.0f;
            key[q] = -__builtin_huge_valf();
            taken |= 1u << q;
        }
    }
    // Group-limited selection ("Kimi K2.5 donor reference", MoEGate.forward
    // records: group scores, group idx, score mask): a group of E/n_group
    // consecutive experts scores the sum of its two largest biased scores; the
    // topk_group best groups are kept (ties to the lower group); experts of the
    // other groups are marked taken, so the selection below never picks them.
    if (n_group > 1) {
        const int G = E / n_group;
        float gsc = -__builtin_huge_valf();  // lane g holds group g's score
        for (int g = 0; g < n_group; ++g) {
            float m1 = -__builtin_huge_valf(), m2 = -__builtin_huge_valf();
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                const int e = lane + MOE_WAVE * q;
                if (e < E && e / G == g) {
                    if (key[q] > m1) {
                        m2 = m1;
                        m1 = key[q];
                    } else if (key[q] > m2) {
                        m2 = key[q];
                    }
                }
            }
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) {  // merge two (largest, second) pairs
                const float o1 = __shfl_xor(m1, off), o2 = __shfl_xor(m2, off);
                const float n2 = fmaxf(fminf(m1, o1), fmaxf(m2, o2));
                m1 = fmaxf(m1, o1);
                m2 = n2;
            }
            if (lane == g) gsc = m1 + m2;
        }
        uint64_t keep = 0;
        for (int j = 0; j < topk_group; ++j) {
            float bv = (lane < n_group && !((keep >> lane) & 1ull)) ? gsc : -__builtin_huge_valf();
            int bg = (lane < n_group && !((keep >> lane) & 1ull)) ? lane : 0x7FFFFFFF;
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) {
                const float ov = __shfl_xor(bv, off);
                const int og = __shfl_xor(bg, off);
                if (og != 0x7FFFFFFF && (bg == 0x7FFFFFFF || ov > bv || (ov == bv && og < bg))) {
                    bv = ov;
                    bg = og;
                }
            }
            keep |= 1ull << bg;
        }
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const int e = lane + MOE_WAVE * q;
            if (e < E && !((keep >> (e / G)) & 1ull)) taken |= 1u << q;
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
        topk_w[(size_t)t * k + lane] = (renormalize ? sel_s / denom : sel_s) * scale;  // routed scaling factor
    }
}

template <int NQ>
void launch_topk(const float* logits, const float* bias, int T, int E, int k, int renorm, int n_group,
                 int topk_group, float scale, int32_t* idx, float* w, hipStream_t st) {
    hipLaunchKernelGGL(k_route_topk<NQ>, dim3((T + 3) / 4), dim3(256), 0, st, logits, bias, T, E,
                       k, renorm, n_group, topk_group, scale, idx, w);
}

// Few tokens: all (token, expert, block) sums in parallel, summed in the top-k
// kernel.  Many tokens: one fused pass keeps each logit's running total.
constexpr int kPartialsMaxT = 256;

}  // namespace

// Logits [T, E] fp32 (256-byte aligned), and for few tokens the block sums
// [T, H/64, E] fp32 after them.
static size_t logits_bytes(int T, int E) { return (((size_t)T * (size_t)E * sizeof(float)) + 255) & ~(size_t)255; }

extern "C" size_t moe_route_workspace_bytes(int T, int H, int E) {
    if (T <= 0 || E <= 0 || H <= 0) return 0;
    if (T <= kPartialsMaxT) return logits_bytes(T, E) + (size_t)T * (size_t)(H / kRouteKC) * (size_t)E * sizeof(float);
    return (size_t)T * (size_t)E * sizeof(float);
}

namespace {
int route_impl(const uint16_t* x, const uint16_t* w_router, const float* bias, int T, int H, int E, int k,
               int renormalize, int n_group, int topk_group, float scale, int32_t* topk_idx, float* topk_w,
               void* ws, size_t ws_bytes, void* stream) {
    using namespace moe;
    if (T < 0 || H <= 0 || E <= 0 || k <= 0)
        return fail(MOE_ERR_INVALID_ARG, "moe_route: bad sizes T=%d H=%d E=%d k=%d", T, H, E, k);
    if (E > 1024 || k > 16 || k > E)
        return fail(MOE_ERR_UNSUPPORTED, "moe_route: need k <= min(E,16), E <= 1024 (E=%d k=%d)", E, k);
    if (H % kRouteKC != 0)
        return fail(MOE_ERR_UNSUPPORTED, "moe_route: H=%d must be a multiple of %d", H, kRouteKC);
    if ((size_t)E * (size_t)H * 2 >= ((size_t)1 << 32))
        return fail(MOE_ERR_UNSUPPORTED, "moe_route: the router matrix (E=%d, H=%d) must stay below 4 GiB", E, H);
    if (T == 0) return MOE_OK;
    if (!x || !w_router || !bias || !topk_idx || !topk_w)
        return fail(MOE_ERR_INVALID_ARG, "moe_route: null pointer");
    if (!aligned16(x) || !aligned16(w_router))
        return fail(MOE_ERR_INVALID_ARG, "moe_route: x and w_router must be 16-byte aligned");
    if (!ws || ws_bytes < moe_route_workspace_bytes(T, H, E))
        return fail(MOE_ERR_WORKSPACE, "moe_route: workspace %zu < %zu bytes", ws_bytes,
                    moe_route_workspace_bytes(T, H, E));
    if (!aligned16(ws)) return fail(MOE_ERR_INVALID_ARG, "moe_route: workspace must be 16-byte aligned");
    hipStream_t st = as_stream(stream);
    float* logits = static_cast<float*>(ws);
    const int tb = (T + kRouteTok - 1) / kRouteTok;
    if (T <= kPartialsMaxT) {
        const int NB = H / kRouteKC;
        float* P = reinterpret_cast<float*>(static_cast<char*>(ws) + logits_bytes(T, E));
        dim3 grid(NB, (E + 63) / 64, tb);
        hipLaunchKernelGGL(k_router_partials, grid, dim3(256), 0, st, x, w_router, T, H, E, P);
        if (int rc = launch_status("moe_route block sums")) return rc;
        const long n = (long)T * E;
        hipLaunchKernelGGL(k_router_blocksum, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, P, T, NB, E, logits);
    } else {
        // chunks of tokens whose rows stay below 2 GiB (the kernel's buffer
        // offsets are 32-bit); 64 experts per workgroup
        constexpr int NW = kRouterWaves;
        const long tc = (((1L << 31) - 1) / ((long)H * 2)) / kRouteTok * kRouteTok;
        const int n_et = (E + 16 * NW - 1) / (16 * NW);
        for (long c0 = 0; c0 < T; c0 += tc) {
            const int Tc = (int)std::min<long>(tc, (long)T - c0);
            const long tiles = (long)n_et * ((Tc + kRouteTok - 1) / kRouteTok);
            const int per_xcd = moe::per_xcd(tiles);
            if (tiles <= kRouterPairMaxTiles)
                hipLaunchKernelGGL(k_router_mfma_pair<NW>, dim3(8 * per_xcd), dim3(64 * NW), 0, st,
                                   x + (size_t)c0 * H, w_router, Tc, H, E, logits + (size_t)c0 * E, n_et, per_xcd);
            else
                hipLaunchKernelGGL(k_router_mfma<NW>, dim3(8 * per_xcd), dim3(64 * NW), 0, st, x + (size_t)c0 * H,
                                   w_router, Tc, H, E, logits + (size_t)c0 * E, n_et, per_xcd);
        }
    }
    int rc = launch_status("moe_route logits");
    if (rc) return rc;
    const int nq = (E + MOE_WAVE - 1) / MOE_WAVE;
    if (nq <= 1) launch_topk<1>(logits, bias, T, E, k, renormalize, n_group, topk_group, scale, topk_idx, topk_w, st);
    else if (nq <= 2) launch_topk<2>(logits, bias, T, E, k, renormalize, n_group, topk_group, scale, topk_idx, topk_w, st);
    else if (nq <= 4) launch_topk<4>(logits, bias, T, E, k, renormalize, n_group, topk_group, scale, topk_idx, topk_w, st);
    else if (nq <= 8) launch_topk<8>(logits, bias, T, E, k, renormalize, n_group, topk_group, scale, topk_idx, topk_w, st);
    else launch_topk<16>(logits, bias, T, E, k, renormalize, n_group, topk_group, scale, topk_idx, topk_w, st);
    return launch_status("moe_route topk");
}
}  // namespace

extern "C" int moe_route(const uint16_t* x, const uint16_t* w_router, const float* bias, int T,
                         int H, int E, int k, int renormalize, int32_t* topk_idx, float* topk_w,
                         void* ws, size_t ws_bytes, void* stream) {
    return route_impl(x, w_router, bias, T, H, E, k, renormalize, 1, 1, 1.0f, topk_idx, topk_w, ws, ws_bytes,
                      stream);
}

extern "C" int moe_route_grouped(const uint16_t* x, const uint16_t* w_router, const float* bias, int T, int H,
                                 int E, int k, int renormalize, int n_group, int topk_group, float routed_scale,
                                 int32_t* topk_idx, float* topk_w, void* ws, size_t ws_bytes, void* stream) {
    using namespace moe;
    if (n_group < 1 || topk_group < 1 || topk_group > n_group)
        return fail(MOE_ERR_INVALID_ARG, "moe_route_grouped: n_group=%d topk_group=%d", n_group, topk_group);
    if (!(routed_scale == routed_scale) || routed_scale == __builtin_huge_valf() ||
        routed_scale == -__builtin_huge_valf())
        return fail(MOE_ERR_INVALID_ARG, "moe_route_grouped: routed_scale must be finite");
    if (E > 0 && (n_group > 64 || E % n_group != 0 || (n_group > 1 && E / n_group < 2) ||
                  k > topk_group * (E / n_group)))
        return fail(MOE_ERR_UNSUPPORTED,
                    "moe_route_grouped: need n_group <= 64 dividing E into groups of 2+ and k <= topk_group*E/n_group "
                    "(E=%d n_group=%d topk_group=%d k=%d)", E, n_group, topk_group, k);
    return route_impl(x, w_router, bias, T, H, E, k, renormalize, n_group, topk_group, routed_scale, topk_idx,
                      topk_w, ws, ws_bytes, stream);
}
