// Dense bf16 pieces around the routed experts: the shared expert (a bf16
// SwiGLU MLP on the full-width input) and the Kimi-K3 latent down/up
// projections ("Kimi exact-generator adaptation", "The proposed
// substitution": shared experts keep ordinary bf16 linear layers; "Kimi-K3
// latent MoE", Parameters table: weights held [out, in], no bias; "Kimi K2.5
// donor reference", record "Add an always-active shared expert"), plus the
// RMSNorm before the latent up-projection (records "RMSNorm mean square",
// "Normalize by the root mean square", "Apply learned per-feature RMSNorm
// gains").
//
// GEMM C = A W^T with A [M,K], W [N,K] both K-contiguous: the natural operand
// layout of v_mfma_f32_16x16x32_bf16 (each lane holds 8 consecutive k of one
// row / one weight row).  A workgroup of 4 waves stages a 16*MB-row A tile in
// LDS per 128-wide K chunk; each wave streams its own 16*CB weight rows
// straight from global memory (16 bytes per lane) into a register ring.
// Decode-shaped problems (few rows) split K over the grid and write fp32
// partials that a second kernel sums in a fixed order (deterministic), then
// applies the epilogue.  From 256 rows the 32x32x16 shape takes over, on tiles
// of 128, 192 or 256 rows (k_dense32, k_dense32_dma below).
#include <utility>

#include "moe_common.h"

namespace {

constexpr int kDKC = 128;
constexpr int kDense32MinM = 256;   // rows from which the 32x32 tile kernel runs
constexpr int kDense32TallM = 6144; // rows from which it takes 192-row tiles
constexpr int kDense256MinTiles = 192;  // 256-row tiles from this many workgroups
// 32-bit byte offsets within a 256-row tile; longer rows take the 16x16 kernel
constexpr int kDense32MaxK = 1 << 22;
constexpr int kDAStride = 136;  // bf16 per LDS row

enum { EPI_LINEAR = 0, EPI_SWIGLU = 1 };

struct DenseArgs {
    const uint16_t* x;   // [M,K]
    const uint16_t* w0;  // [N0,K]  (linear: W; swiglu: W_gate)
    const uint16_t* w1;  // swiglu: W_up [N0,K]
    const uint16_t* add; // linear: optional [M,N0]
    uint16_t* y;         // [M,N0]
    float* part;         // split-K partials [ks][M][Ntot]
    int M, N0, K;
    int Ntot;            // N0 (linear) or 2*N0 (swiglu)
    int tiles_m, n_chunks, ksplit;
    long n_logical;
    int per_xcd;
};

__device__ __forceinline__ uint32_t silu_mul_bits(float g, float u) {
    const uint32_t gb = f32_to_bf16_bits(g);
    const uint32_t ub = f32_to_bf16_bits(u);
    const uint32_t ab = f32_to_bf16_bits(moe_silu(bf16_bits_to_f32(gb)));
    return f32_to_bf16_bits(bf16_bits_to_f32(ab) * bf16_bits_to_f32(ub));
}

__device__ __forceinline__ uint32_t add_bits(uint32_t yb, uint16_t addv) {
    return f32_to_bf16_bits(bf16_bits_to_f32(yb) + bf16_bits_to_f32(addv));
}

// Column layout of a wave (CB blocks of 16 columns):
//   linear: output columns n0 + 16 cb + r, n0 = chunk * 64 CB + wave * 16 CB
//   swiglu: blocks [0, CB/2) gate, [CB/2, CB) up, same output columns
//           n0 + 16 (cb mod CB/2) + r with n0 = chunk * 32 CB + wave * 8 CB
// The A tile is double-buffered in LDS (one LDS-only barrier per chunk); each
// wave's weight rows run D-1 chunks ahead in a ring of D register slots.
template <int MB, int CB, int EPI, bool SPLIT>
__global__ __launch_bounds__(256) void k_dense(DenseArgs a) {
    constexpr int BM = 16 * MB;
    constexpr int HALF = CB / 2;
    constexpr int D = CB == 2 ? 3 : 2;
    __shared__ __attribute__((aligned(16))) uint16_t As[2][BM][kDAStride];

    const long L = xcd_logical_block(a.per_xcd);
    if (L >= a.n_logical) return;
    const int ks = (int)(L % a.ksplit);
    const long rest = L / a.ksplit;
    const int nc = (int)(rest % a.n_chunks);
    const int tm = (int)(rest / a.n_chunks);

    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wave = tid >> 6;
    const int r = lane & 15;
    const int j = lane >> 4;
    const int K = a.K;
    const int m0 = tm * BM;
    const int rows = min(BM, a.M - m0);
    const int nch = K / kDKC;
    const int c_beg = (int)((long)nch * ks / a.ksplit);
    const int c_end = (int)((long)nch * (ks + 1) / a.ksplit);
    const int nloc = c_end - c_beg;  // >= 1 (the planner keeps at least two chunks per split)

    // weight rows past N read the last row (never stored)
    int n0;
    const uint16_t* wrow[CB];
    if (EPI == EPI_SWIGLU) {
        n0 = nc * 32 * CB + wave * 8 * CB;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
            const int n = min(n0 + 16 * (cb % HALF) + r, a.N0 - 1);
            wrow[cb] = (cb < HALF ? a.w0 : a.w1) + (size_t)n * K + 8 * j;
        }
    } else {
        n0 = nc * 64 * CB + wave * 16 * CB;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
            const int n = min(n0 + 16 * cb + r, a.N0 - 1);
            wrow[cb] = a.w0 + (size_t)n * K + 8 * j;
        }
    }
    const int active_mb = (rows + 15) >> 4;

    // A staging: each load instruction of a wave reads 4 whole row chunks (16 lanes
    // x 16 contiguous bytes); wave w moves rows 4*A_ITERS*w + 4*it + lane/16 (rows
    // past the tile read the tile's first row; their products are never stored)
    constexpr int A_ITERS = BM * 16 / 256;
    static_assert(BM * 16 % 256 == 0 && A_ITERS * 16 == BM, "A staging");
    auto srow_of = [&](int it) { return 4 * A_ITERS * wave + 4 * it + (lane >> 4); };
    const uint16_t* aptr[A_ITERS];
#pragma unroll
    for (int it = 0; it < A_ITERS; ++it)
        aptr[it] = a.x + (size_t)(m0 + (srow_of(it) < rows ? srow_of(it) : 0)) * K + (lane & 15) * 8;
    u32x4_t Aq[A_ITERS];
    auto load_A = [&](int c) __attribute__((always_inline)) {
#pragma unroll
        for (int it = 0; it < A_ITERS; ++it)
            Aq[it] = *reinterpret_cast<const u32x4_t*>(aptr[it] + (size_t)c * kDKC);
    };
    auto store_A = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int it = 0; it < A_ITERS; ++it)
            *reinterpret_cast<u32x4_t*>(&As[buf][srow_of(it)][(lane & 15) * 8]) = Aq[it];
    };

    struct Slot {
        u32x4_t B[CB][4];  // per column block and group step: 8 bf16 of the lane's weight row
    };
    auto load_B = [&](int c, Slot& sl) __attribute__((always_inline)) {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int g = 0; g < 4; ++g)
                sl.B[cb][g] = *reinterpret_cast<const u32x4_t*>(wrow[cb] + (size_t)c * kDKC + 32 * g);
    };

    f32x4_t acc[MB][CB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) acc[mb][cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](int buf, const Slot& sl) __attribute__((always_inline)) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                if (mb < active_mb) {
                    const bf16x8_t af = __builtin_bit_cast(
                        bf16x8_t, *reinterpret_cast<const u32x4_t*>(&As[buf][16 * mb + r][32 * g + 8 * j]));
#pragma unroll
                    for (int cb = 0; cb < CB; ++cb)
                        acc[mb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            af, __builtin_bit_cast(bf16x8_t, sl.B[cb][g]), acc[mb][cb], 0, 0, 0);
                }
            }
        }
    };

    // local chunk i = c_beg + i lives in slot i % D; indices past the split are
    // clamped (redundant in-bounds loads, a staged buffer nobody reads)
    Slot sl[D];
    load_A(c_beg);
#pragma unroll
    for (int i = 0; i < D; ++i) load_B(c_beg + min(i, nloc - 1), sl[i]);
    store_A(0);
    lds_barrier();
    auto step = [&](int i, Slot& cur) __attribute__((always_inline)) {
        load_A(c_beg + min(i + 1, nloc - 1));
        __builtin_amdgcn_sched_barrier(0);
        compute(i & 1, cur);
        __builtin_amdgcn_sched_barrier(0);
        load_B(c_beg + min(i + D, nloc - 1), cur);
        __builtin_amdgcn_sched_barrier(0);
        store_A((i + 1) & 1);
        lds_barrier();
    };
    int i = 0;
    for (; i + D <= nloc; i += D) {
#pragma unroll
        for (int q = 0; q < D; ++q) step(i + q, sl[q]);
    }
#pragma unroll
    for (int q = 0; q < D - 1; ++q)
        if (i + q < nloc) step(i + q, sl[q]);

#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        if (mb >= active_mb) continue;
        // the block's addends are loaded before its first store (a store in
        // between would make each later load wait for it: y may alias add); rows
        // and columns past the matrix read a clamped in-bounds element, never used
        uint32_t addv[4][CB];
        if (!SPLIT && EPI == EPI_LINEAR && a.add) {
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                const int rl = min(16 * mb + 4 * j + ii, rows - 1);
#pragma unroll
                for (int cb = 0; cb < CB; ++cb)
                    addv[ii][cb] = a.add[(size_t)(m0 + rl) * a.N0 + min(n0 + 16 * cb + r, a.N0 - 1)];
            }
        }
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            const int rl = 16 * mb + 4 * j + ii;
            if (rl >= rows) continue;
            const size_t m = (size_t)(m0 + rl);
            if (SPLIT) {
                float* prow = a.part + ((size_t)ks * a.M + m) * a.Ntot;
#pragma unroll
                for (int cb = 0; cb < CB; ++cb) {
                    int col;
                    if (EPI == EPI_SWIGLU) col = (cb < HALF ? 0 : a.N0) + n0 + 16 * (cb % HALF) + r;
                    else col = n0 + 16 * cb + r;
                    if ((EPI == EPI_SWIGLU ? n0 + 16 * (cb % HALF) + r : col) < a.N0) prow[col] = acc[mb][cb][ii];
                }
            } else if (EPI == EPI_SWIGLU) {
#pragma unroll
                for (int p = 0; p < HALF; ++p) {
                    const int col = n0 + 16 * p + r;
                    if (col < a.N0) a.y[m * a.N0 + col] = (uint16_t)silu_mul_bits(acc[mb][p][ii], acc[mb][HALF + p][ii]);
                }
            } else {
#pragma unroll
                for (int cb = 0; cb < CB; ++cb) {
                    const int col = n0 + 16 * cb + r;
                    if (col < a.N0) {
                        uint32_t yb = f32_to_bf16_bits(acc[mb][cb][ii]);
                        if (a.add) yb = add_bits(yb, (uint16_t)addv[ii][cb]);
                        a.y[m * a.N0 + col] = (uint16_t)yb;
                    }
                }
            }
        }
    }
}

// f(integral_constant<int, i>) for i = 0 .. N-1, unrolled whatever the body's size.
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Epilogue of the 32x32 dense kernels: element i of lane (c32, kb) in row
// block mb is tile row 32 mb + 8(i/4) + 4 kb + i%4, column n0 + 32 cb + c32
// (linear) or n0 + c32 (swiglu: block 0 gate, block 1 up).
template <int M32, int EPI>
__device__ __forceinline__ void dense32_epilogue(const DenseArgs& a, const f32x16_t (&acc)[M32][2], int m0,
                                                 int rows, int n0, int c32, int kb) {
    // In batches of MBB row blocks.  A batch's addend loads are all
    // issued before its first store (a store in between would make each later
    // load wait for it: y may alias add); rows and columns past the matrix read a
    // clamped in-bounds element, never used.  Tiles of more than 128 rows take
    // two batches, which keeps the addends out of scratch.
    constexpr int MBB = M32 > 4 ? M32 / 2 : M32;
    static_assert(M32 % MBB == 0, "epilogue batches");
#pragma unroll
    for (int mb0 = 0; mb0 < M32; mb0 += MBB) {
        uint32_t addv[MBB][16][2];
        if (EPI == EPI_LINEAR && a.add) {
#pragma unroll
            for (int b = 0; b < MBB; ++b)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int rl = min(32 * (mb0 + b) + 8 * (i >> 2) + 4 * kb + (i & 3), rows - 1);
#pragma unroll
                    for (int cb = 0; cb < 2; ++cb) {
                        const int col = min(n0 + 32 * cb + c32, a.N0 - 1);
                        addv[b][i][cb] = a.add[(size_t)(m0 + rl) * a.N0 + col];
                    }
                }
        }
#pragma unroll
        for (int b = 0; b < MBB; ++b) {
            const int mb = mb0 + b;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int rl = 32 * mb + 8 * (i >> 2) + 4 * kb + (i & 3);
                if (rl >= rows) continue;
                const size_t m = (size_t)(m0 + rl);
                if (EPI == EPI_SWIGLU) {
                    const int col = n0 + c32;
                    if (col < a.N0) a.y[m * a.N0 + col] = (uint16_t)silu_mul_bits(acc[mb][0][i], acc[mb][1][i]);
                } else {
#pragma unroll
                    for (int cb = 0; cb < 2; ++cb) {
                        const int col = n0 + 32 * cb + c32;
                        if (col < a.N0) {
                            uint32_t yb = f32_to_bf16_bits(acc[mb][cb][i]);
                            if (a.add) yb = add_bits(yb, (uint16_t)addv[b][i][cb]);
                            a.y[m * a.N0 + col] = (uint16_t)yb;
                        }
                    }
                }
            }
        }
    }
}

// Row tiles of 32*M32 rows on v_mfma_f32_32x32x16_bf16 (one wave per SIMD
// drives that shape near its peak; the 16x16x32 shape above stops near 1.4 PF
// at this occupancy).  A workgroup is 4 waves; each wave owns two 32-column
// blocks (linear: 64 output columns; swiglu: 32 gate and the same 32 up
// columns) and all tile rows.  Within a 128-wide K chunk lane (c, kb) holds K
// elements [64 kb, 64 kb + 64) of its row or column in 8 steps of 8 (both
// operands use the same order, so each step still multiplies matching K):
// every weight load then reads whole 128-byte lines, and the A-fragment reads
// from LDS (272-byte rows) are free of bank conflicts.  The A tile is staged in
// LDS one chunk ahead, a piece every 4 products; weights run R-1 chunks ahead
// in an R-slot register ring; one LDS-only barrier per chunk.  Accumulator
// element i of lane l is row 8(i/4) + 4 kb + i%4, column c.
template <int M32, int EPI, int R>
__global__ __launch_bounds__(256) void k_dense32(DenseArgs a) {
    constexpr int BM = 32 * M32;
    constexpr int A_ITERS = BM * 16 / 256;  // 16-byte pieces per lane per chunk
    constexpr int NS = 8 * M32;             // (K step, row block) products per chunk
    static_assert(NS == 4 * A_ITERS, "staging: one piece every 4 products");
    __shared__ __attribute__((aligned(16))) uint16_t As[2][BM][kDAStride];

    const long L = xcd_logical_block(a.per_xcd);
    if (L >= a.n_logical) return;
    const int nc = (int)(L % a.n_chunks);
    const int tm = (int)(L / a.n_chunks);

    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wave = tid >> 6;
    const int c32 = lane & 31;
    const int kb = lane >> 5;
    const int K = a.K;
    const int m0 = tm * BM;
    const int rows = min(BM, a.M - m0);
    const int nch = K / kDKC;

    // weight rows past N read the last row (never stored)
    const int n0 = EPI == EPI_SWIGLU ? nc * 128 + wave * 32 : nc * 256 + wave * 64;
    const uint16_t* wrow[2];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
        const int n = min(EPI == EPI_SWIGLU ? n0 + c32 : n0 + 32 * cb + c32, a.N0 - 1);
        wrow[cb] = (EPI == EPI_SWIGLU && cb == 1 ? a.w1 : a.w0) + (size_t)n * K + 64 * kb;
    }

    // A staging: each wave load instruction reads 4 whole row chunks (16 lanes x
    // 16 contiguous bytes); wave w moves rows 4*A_ITERS*w + 4*it + lane/16 (rows
    // past the tile read the tile's first row; their products are never stored)
    auto srow_of = [&](int it) { return 4 * A_ITERS * wave + 4 * it + (lane >> 4); };
    const uint16_t* xt = a.x + (size_t)m0 * K;  // the tile's first row
    uint32_t aoff[A_ITERS];                       // element offsets within the tile
#pragma unroll
    for (int it = 0; it < A_ITERS; ++it)
        aoff[it] = (uint32_t)(srow_of(it) < rows ? srow_of(it) : 0) * (uint32_t)K + (uint32_t)(lane & 15) * 8u;
    u32x4_t Aq[A_ITERS];
    auto load_piece = [&](int it, int c) __attribute__((always_inline)) {
        Aq[it] = *reinterpret_cast<const u32x4_t*>(xt + aoff[it] + (size_t)c * kDKC);
    };
    auto store_piece = [&](int it, int buf) __attribute__((always_inline)) {
        *reinterpret_cast<u32x4_t*>(&As[buf][srow_of(it)][(lane & 15) * 8]) = Aq[it];
    };

    struct Slot {
        u32x4_t B[2][8];  // per column block and step: 8 bf16 of the lane's weight row
    };
    auto load_B = [&](int c, Slot& sl) __attribute__((always_inline)) {
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
            for (int q = 0; q < 8; ++q)
                sl.B[cb][q] = *reinterpret_cast<const u32x4_t*>(wrow[cb] + (size_t)c * kDKC + 8 * q);
    };

    f32x16_t acc[M32][2];
#pragma unroll
    for (int mb = 0; mb < M32; ++mb)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[mb][cb][i] = 0.0f;

    auto compute = [&](int c, const Slot& sl) __attribute__((always_inline)) {
        const int buf = c & 1;
        constexpr int PF = 4;
        auto frag = [&](int p) __attribute__((always_inline)) {
            return __builtin_bit_cast(
                bf16x8_t, *reinterpret_cast<const u32x4_t*>(&As[buf][32 * (p % M32) + c32][64 * kb + 8 * (p / M32)]));
        };
        bf16x8_t afr[NS];
#pragma unroll
        for (int q = 0; q < PF; ++q) afr[q] = frag(q);
        static_for<NS>([&](auto pc) __attribute__((always_inline)) {
            constexpr int p = decltype(pc)::value;
            constexpr int st = p / M32;
            constexpr int mb = p % M32;
            if constexpr (p + PF < NS) afr[p + PF] = frag(p + PF);
            if constexpr (p % 4 == 2) {
                store_piece(p / 4, (c + 1) & 1);
                load_piece(p / 4, min(c + 2, nch - 1));
            }
#pragma unroll
            for (int cb = 0; cb < 2; ++cb)
                acc[mb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    afr[p], __builtin_bit_cast(bf16x8_t, sl.B[cb][st]), acc[mb][cb], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0x0002);
        });
    };

    // prologue: the loads in flight at each step's start are, in issue order,
    // weights c, activations c+1, weights c+1 .. c+R-1 (chunk c+i in slot
    // (c+i) mod R; indices past the end are clamped, redundant in-bounds loads)
    static_assert(R == 2 || R == 3, "ring depth");
    Slot sl[R];
#pragma unroll
    for (int it = 0; it < A_ITERS; ++it) load_piece(it, 0);
    load_B(0, sl[0]);
#pragma unroll
    for (int it = 0; it < A_ITERS; ++it) store_piece(it, 0);
#pragma unroll
    for (int it = 0; it < A_ITERS; ++it) load_piece(it, min(1, nch - 1));
#pragma unroll
    for (int q = 1; q < R; ++q) load_B(min(q, nch - 1), sl[q]);
    lds_barrier();
    auto step = [&](int c, Slot& cur) __attribute__((always_inline)) {
        compute(c, cur);
        __builtin_amdgcn_sched_barrier(0);
        load_B(min(c + R, nch - 1), cur);
        lds_barrier();
    };
    int c = 0;
    for (; c + R <= nch; c += R) {
#pragma unroll
        for (int q = 0; q < R; ++q) step(c + q, sl[q]);
    }
#pragma unroll
    for (int q = 0; q < R - 1; ++q)
        if (c + q < nch) step(c + q, sl[q]);

    dense32_epilogue<M32, EPI>(a, acc, m0, rows, n0, c32, kb);
}

// The 32x32 dense kernel for 256-row tiles (M32 = 8).  The same products and
// order as k_dense32, but the A tile is staged by buffer-to-LDS loads, so that
// no registers hold it in flight: two LDS buffers of 256 unpadded 256-byte rows
// whose 16-byte units are XOR-swizzled by the row (unit u of row r at u ^ (r mod
// 16)), so that the fragment reads stay free of bank conflicts.  Chunk c+1 is
// loaded into the other buffer while chunk c is multiplied (its last readers
// finished before the previous barrier).  Taller tiles read each weight line
// for twice the rows of the 128-row ones.
template <int M32, int EPI, int R>
__global__ __launch_bounds__(256) void k_dense32_dma(DenseArgs a) {
    constexpr int BM = 32 * M32;
    constexpr int A_ITERS = BM / 16;  // staging instructions per wave per chunk (4 rows each)
    constexpr int NS = 8 * M32;       // (K step, row block) products per chunk
    static_assert(A_ITERS * 4 * 4 == BM && 2 * A_ITERS <= NS, "staging: 4 rows per wave instruction");
    // two separate LDS objects, so that the compiler can tell a fragment read of
    // one buffer from the loads into the other
    __shared__ __attribute__((aligned(16))) uint16_t As0[BM][kDKC];
    __shared__ __attribute__((aligned(16))) uint16_t As1[BM][kDKC];
    auto tile = [&](auto bc) -> uint16_t(&)[BM][kDKC] {
        if constexpr (decltype(bc)::value == 0) return As0;
        else return As1;
    };

    const long L = xcd_logical_block(a.per_xcd);
    if (L >= a.n_logical) return;
    const int nc = (int)(L % a.n_chunks);
    const int tm = (int)(L / a.n_chunks);

    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c32 = lane & 31;
    const int kb = lane >> 5;
    const int K = a.K;
    const int m0 = tm * BM;
    const int rows = min(BM, a.M - m0);
    const int nch = K / kDKC;

    // weight rows past N read the last row (never stored)
    const int n0 = EPI == EPI_SWIGLU ? nc * 128 + wave * 32 : nc * 256 + wave * 64;
    const uint16_t* wrow[2];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
        const int n = min(EPI == EPI_SWIGLU ? n0 + c32 : n0 + 32 * cb + c32, a.N0 - 1);
        wrow[cb] = (EPI == EPI_SWIGLU && cb == 1 ? a.w1 : a.w0) + (size_t)n * K + 64 * kb;
    }

    // staging instruction it of this wave writes tile rows 4 A_ITERS wave + 4 it
    // .. +3 (lane l: row + l/16, physical unit l mod 16, which holds logical unit
    // (l mod 16) ^ (row mod 16)), read through a descriptor over the tile's rows;
    // rows past the matrix read the tile's first row (their products are never
    // stored)
    const __amdgpu_buffer_rsrc_t ra =
        buffer_rsrc(a.x + (size_t)m0 * K, (uint32_t)rows * (uint32_t)K * 2u);
    uint32_t aoff[A_ITERS];
#pragma unroll
    for (int it = 0; it < A_ITERS; ++it) {
        const int row = 4 * A_ITERS * wave + 4 * it + (lane >> 4);
        const uint32_t unit = (uint32_t)((lane & 15) ^ (row & 15));
        aoff[it] = ((uint32_t)(row < rows ? row : 0) * (uint32_t)K + unit * 8u) * 2u;
    }
    auto dma_piece = [&](int it, int c, auto bc) __attribute__((always_inline)) {
        buffer_load_lds16(ra, &tile(bc)[4 * A_ITERS * wave + 4 * it][0], aoff[it], (uint32_t)c * (kDKC * 2));
    };

    struct Slot {
        u32x4_t B[2][8];  // per column block and step: 8 bf16 of the lane's weight row
    };
    auto load_B = [&](int c, Slot& sl) __attribute__((always_inline)) {
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
            for (int q = 0; q < 8; ++q)
                sl.B[cb][q] = *reinterpret_cast<const u32x4_t*>(wrow[cb] + (size_t)c * kDKC + 8 * q);
    };

    f32x16_t acc[M32][2];
#pragma unroll
    for (int mb = 0; mb < M32; ++mb)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[mb][cb][i] = 0.0f;

    // products of chunk c from buffer BUF; the staging loads of chunk c+1 into
    // the other buffer spread over the first half
    auto compute = [&](auto bc, int c, const Slot& sl) __attribute__((always_inline)) {
        constexpr int BUF = decltype(bc)::value;
        constexpr int PF = 4;
        const int swz = c32 & 15;
        auto frag = [&](int p) __attribute__((always_inline)) {
            const int unit = (8 * kb + p / M32) ^ swz;
            return __builtin_bit_cast(bf16x8_t,
                                      *reinterpret_cast<const u32x4_t*>(&tile(bc)[32 * (p % M32) + c32][8 * unit]));
        };
        bf16x8_t afr[NS];
#pragma unroll
        for (int q = 0; q < PF; ++q) afr[q] = frag(q);
        const int cs = min(c + 1, nch - 1);
        static_for<NS>([&](auto pc) __attribute__((always_inline)) {
            constexpr int p = decltype(pc)::value;
            constexpr int st = p / M32;
            constexpr int mb = p % M32;
            if constexpr (p + PF < NS) afr[p + PF] = frag(p + PF);
            static_for<A_ITERS>([&](auto ic) __attribute__((always_inline)) {
                constexpr int i = decltype(ic)::value;
                if constexpr (i * NS / (2 * A_ITERS) == p)
                    dma_piece(i, cs, std::integral_constant<int, 1 - BUF>{});
            });
#pragma unroll
            for (int cb = 0; cb < 2; ++cb)
                acc[mb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    afr[p], __builtin_bit_cast(bf16x8_t, sl.B[cb][st]), acc[mb][cb], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0x0002);
        });
    };

    // Loads issued, in order: weights of chunks 0 .. R-2, staging 0, weights R-1 |
    // step c: staging c+1 (first half of the products), weights c+R (16 per lane)
    // | staging c+1 has landed once at most 16 younger loads are outstanding (the
    // weights of c+R), and in the prologue staging 0 too (weights R-1).  Chunk
    // indices past the end are clamped: redundant in-bounds loads, never read.
    static_assert(R == 2 || R == 3, "ring depth");
    Slot sl[R];
#pragma unroll
    for (int q = 0; q < R - 1; ++q) load_B(min(q, nch - 1), sl[q]);
#pragma unroll
    for (int it = 0; it < A_ITERS; ++it) dma_piece(it, 0, std::integral_constant<int, 0>{});
    load_B(min(R - 1, nch - 1), sl[R - 1]);
    wait_vmcnt<16>();
    lds_barrier();
    auto step = [&](auto bc, int c, Slot& cur) __attribute__((always_inline)) {
        compute(bc, c, cur);
        __builtin_amdgcn_sched_barrier(0);
        load_B(min(c + R, nch - 1), cur);
        wait_vmcnt<16>();
        lds_barrier();
    };
    // unrolled by lcm(2, R): buffers and slots stay compile-time choices
    constexpr int U = R == 2 ? 2 : 6;
    int c = 0;
    for (; c + U <= nch; c += U) {
        static_for<U>([&](auto qc) __attribute__((always_inline)) {
            constexpr int q = decltype(qc)::value;
            step(std::integral_constant<int, q % 2>{}, c + q, sl[q % R]);
        });
    }
    static_for<U - 1>([&](auto qc) __attribute__((always_inline)) {
        constexpr int q = decltype(qc)::value;
        if (c + q < nch) step(std::integral_constant<int, q % 2>{}, c + q, sl[q % R]);
    });
    wait_vmcnt<0>();  // the trailing (redundant) staging loads land before the wave ends

    dense32_epilogue<M32, EPI>(a, acc, m0, rows, n0, c32, kb);
}

// Sum the split-K partials in ascending split order, then the epilogue.
template <int EPI>
__global__ __launch_bounds__(256) void k_dense_reduce(const float* __restrict__ part, int ksplit, int M,
                                                      int N0, int Ntot, const uint16_t* __restrict__ add,
                                                      uint16_t* __restrict__ y) {
    const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (long)M * N0) return;
    const long m = idx / N0;
    const int n = (int)(idx % N0);
    if (EPI == EPI_SWIGLU) {
        float g = 0.0f, u = 0.0f;
        for (int s = 0; s < ksplit; ++s) {
            const float* prow = part + ((size_t)s * M + m) * Ntot;
            g = g + prow[n];
            u = u + prow[N0 + n];
        }
        y[idx] = (uint16_t)silu_mul_bits(g, u);
    } else {
        float v = 0.0f;
        for (int s = 0; s < ksplit; ++s) v = v + part[((size_t)s * M + m) * Ntot + n];
        uint32_t yb = f32_to_bf16_bits(v);
        if (add) yb = add_bits(yb, add[idx]);
        y[idx] = (uint16_t)yb;
    }
}

struct Plan {
    int mb, cb, ksplit, tiles_m, n_chunks;
};

// Tile shape and split: wide tiles for many rows, narrow tiles plus a K split
// for few rows (the weights then stream once and ~256+ workgroups fill the GPU).
Plan plan_dense(int M, int Ntot_cols, int K, bool swiglu) {
    Plan p{};
    const int nch = K / kDKC;
    if (M <= 64) {
        p.mb = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
        p.cb = 2;
    } else {
        p.mb = M <= 512 ? 4 : 8;
        p.cb = 4;
    }
    const int cols_per_wg = swiglu ? 4 * 8 * p.cb : 4 * 16 * p.cb;  // output columns per workgroup
    const int N0 = swiglu ? Ntot_cols / 2 : Ntot_cols;
    p.tiles_m = (M + 16 * p.mb - 1) / (16 * p.mb);
    p.n_chunks = (N0 + cols_per_wg - 1) / cols_per_wg;
    p.ksplit = 1;
    const long blocks = (long)p.tiles_m * p.n_chunks;
    if (M <= 64) {
        while (p.ksplit < 8 && blocks * p.ksplit < 256 && nch / (p.ksplit * 2) >= 2) p.ksplit *= 2;
    }
    return p;
}

template <int EPI, bool SPLIT>
void launch_dense_mb_cb(const Plan& p, DenseArgs& a, hipStream_t st) {
    const dim3 grid(8 * a.per_xcd), block(256);
#define MOE_DENSE_CASE(MBv, CBv)                                                                 \
    if (p.mb == MBv && p.cb == CBv) {                                                            \
        hipLaunchKernelGGL((k_dense<MBv, CBv, EPI, SPLIT>), grid, block, 0, st, a);              \
        return;                                                                                  \
    }
    MOE_DENSE_CASE(1, 2)
    MOE_DENSE_CASE(2, 2)
    MOE_DENSE_CASE(4, 2)
    MOE_DENSE_CASE(4, 4)
    MOE_DENSE_CASE(8, 4)
#undef MOE_DENSE_CASE
}

int run_dense(int epi, const uint16_t* x, const uint16_t* w0, const uint16_t* w1, const uint16_t* add,
              uint16_t* y, int M, int N0, int K, void* ws, size_t ws_bytes, hipStream_t st,
              const char* what) {
    const bool sw = epi == EPI_SWIGLU;
    const int Ntot = sw ? 2 * N0 : N0;
    const Plan p = plan_dense(M, Ntot, K, sw);
    DenseArgs a{};
    a.x = x;
    a.w0 = w0;
    a.w1 = w1;
    a.add = add;
    a.y = y;
    a.M = M;
    a.N0 = N0;
    a.K = K;
    a.Ntot = Ntot;
    a.tiles_m = p.tiles_m;
    a.n_chunks = p.n_chunks;
    a.ksplit = p.ksplit;
    a.n_logical = (long)p.tiles_m * p.n_chunks * p.ksplit;
    a.per_xcd = moe::per_xcd(a.n_logical);
    if (p.ksplit > 1) {
        const size_t need = (size_t)p.ksplit * M * Ntot * sizeof(float);
        if (!ws || ws_bytes < need)
            return moe::fail(MOE_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", what, ws_bytes, need);
        a.part = static_cast<float*>(ws);
        if (sw) launch_dense_mb_cb<EPI_SWIGLU, true>(p, a, st);
        else launch_dense_mb_cb<EPI_LINEAR, true>(p, a, st);
        if (int rc = moe::launch_status(what)) return rc;
        const long n = (long)M * N0;
        const dim3 g((unsigned)((n + 255) / 256));
        if (sw) hipLaunchKernelGGL(k_dense_reduce<EPI_SWIGLU>, g, dim3(256), 0, st, a.part, p.ksplit, M, N0, Ntot, nullptr, y);
        else hipLaunchKernelGGL(k_dense_reduce<EPI_LINEAR>, g, dim3(256), 0, st, a.part, p.ksplit, M, N0, Ntot, add, y);
        return moe::launch_status(what);
    }
    if (M >= kDense32MinM && K <= kDense32MaxK) {
        const int cols = sw ? 128 : 256;
        const int n_chunks = (N0 + cols - 1) / cols;
        if ((long)((M + 255) / 256) * n_chunks >= kDense256MinTiles) {
            // 256-row tiles wherever they still give most CUs a workgroup
            a.n_chunks = n_chunks;
            a.tiles_m = (M + 255) / 256;
            a.n_logical = (long)a.tiles_m * a.n_chunks;
            a.per_xcd = moe::per_xcd(a.n_logical);
            const dim3 grid(8 * a.per_xcd), block(256);
            if (sw) hipLaunchKernelGGL((k_dense32_dma<8, EPI_SWIGLU, 2>), grid, block, 0, st, a);
            else hipLaunchKernelGGL((k_dense32_dma<8, EPI_LINEAR, 2>), grid, block, 0, st, a);
            return moe::launch_status(what);
        }
        // 32x32 tiles of 128 rows, or 192 from kDense32TallM rows (the weights,
        // read from L2 once per row tile, dominate a tile's operand traffic:
        // taller tiles re-read them less often).  The 128-row tiles keep a
        // 3-slot weight ring; the 192-row tiles' accumulators leave room for 2
        // slots only (3 spill).  Measured on 2048 rows, 192-row tiles left too
        // few workgroups (0.18 -> 0.22 ms); on 8192 rows they gained 10%.
        a.n_chunks = n_chunks;
        const int m32 = M >= kDense32TallM ? 6 : 4;
        a.tiles_m = (M + 32 * m32 - 1) / (32 * m32);
        a.n_logical = (long)a.tiles_m * a.n_chunks;
        a.per_xcd = moe::per_xcd(a.n_logical);
        const dim3 grid(8 * a.per_xcd), block(256);
        if (m32 == 6) {
            if (sw) hipLaunchKernelGGL((k_dense32<6, EPI_SWIGLU, 2>), grid, block, 0, st, a);
            else hipLaunchKernelGGL((k_dense32<6, EPI_LINEAR, 2>), grid, block, 0, st, a);
        } else {
            if (sw) hipLaunchKernelGGL((k_dense32<4, EPI_SWIGLU, 3>), grid, block, 0, st, a);
            else hipLaunchKernelGGL((k_dense32<4, EPI_LINEAR, 3>), grid, block, 0, st, a);
        }
        return moe::launch_status(what);
    }
    if (sw) launch_dense_mb_cb<EPI_SWIGLU, false>(p, a, st);
    else launch_dense_mb_cb<EPI_LINEAR, false>(p, a, st);
    return moe::launch_status(what);
}

__global__ __launch_bounds__(256) void k_silu_mul(const uint16_t* __restrict__ g, const uint16_t* __restrict__ u,
                                                  uint16_t* __restrict__ h, long n) {
    const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const uint32_t ab = f32_to_bf16_bits(moe_silu(bf16_bits_to_f32(g[i])));
    h[i] = (uint16_t)f32_to_bf16_bits(bf16_bits_to_f32(ab) * bf16_bits_to_f32(u[i]));
}

// One workgroup per row: fp32 mean square (tree order), r = 1/sqrt(ms + eps),
// y = bf16(bf16(x r) * gain).
__global__ __launch_bounds__(256) void k_rmsnorm(const uint16_t* __restrict__ x, const uint16_t* __restrict__ gain,
                                                 float eps, uint16_t* __restrict__ y, int N) {
    __shared__ float red[4];
    const uint16_t* xr = x + (size_t)blockIdx.x * N;
    float ss = 0.0f;
    for (int i = threadIdx.x; i < N; i += blockDim.x) {
        const float v = bf16_bits_to_f32(xr[i]);
        ss = ss + v * v;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) ss = ss + __shfl_xor(ss, off);
    if (lane_id() == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    const float tot = (red[0] + red[1]) + (red[2] + red[3]);
    const float rr = 1.0f / __builtin_sqrtf(tot / (float)N + eps);
    uint16_t* yr = y + (size_t)blockIdx.x * N;
    for (int i = threadIdx.x; i < N; i += blockDim.x) {
        const uint32_t nb = f32_to_bf16_bits(bf16_bits_to_f32(xr[i]) * rr);
        yr[i] = (uint16_t)f32_to_bf16_bits(bf16_bits_to_f32(nb) * bf16_bits_to_f32(gain[i]));
    }
}

}  // namespace

extern "C" size_t moe_dense_workspace_bytes(int M, int N_total, int K) {
    if (M <= 0 || N_total <= 0 || K <= 0 || K % kDKC) return 0;
    // both epilogues share the plan shape rules; take the larger split
    const Plan pl = plan_dense(M, N_total, K, false);
    const Plan ps = plan_dense(M, N_total, K, true);
    const int ks = pl.ksplit > ps.ksplit ? pl.ksplit : ps.ksplit;
    return ks > 1 ? (size_t)ks * M * N_total * sizeof(float) : 0;
}

extern "C" int moe_linear_bf16(const uint16_t* x, const uint16_t* w, const uint16_t* add, uint16_t* y,
                               int M, int N, int K, void* ws, size_t ws_bytes, void* stream) {
    using namespace moe;
    const char* what = "moe_linear_bf16";
    if (M < 0 || N <= 0 || K <= 0) return fail(MOE_ERR_INVALID_ARG, "%s: bad sizes", what);
    if (N % 64 || K % kDKC) return fail(MOE_ERR_UNSUPPORTED, "%s: N=%d (x64) K=%d (x128)", what, N, K);
    if (M == 0) return MOE_OK;
    if (!x || !w || !y) return fail(MOE_ERR_INVALID_ARG, "%s: null pointer", what);
    if (!aligned16(x) || !aligned16(w)) return fail(MOE_ERR_INVALID_ARG, "%s: x, w must be 16-byte aligned", what);
    return run_dense(EPI_LINEAR, x, w, nullptr, add, y, M, N, K, ws, ws_bytes, as_stream(stream), what);
}

extern "C" int moe_dense_swiglu_bf16(const uint16_t* x, const uint16_t* w_gate, const uint16_t* w_up,
                                     uint16_t* h, int M, int H, int I, void* ws, size_t ws_bytes,
                                     void* stream) {
    using namespace moe;
    const char* what = "moe_dense_swiglu_bf16";
    if (M < 0 || H <= 0 || I <= 0) return fail(MOE_ERR_INVALID_ARG, "%s: bad sizes", what);
    if (I % 64 || H % kDKC) return fail(MOE_ERR_UNSUPPORTED, "%s: I=%d (x64) H=%d (x128)", what, I, H);
    if (M == 0) return MOE_OK;
    if (!x || !w_gate || !w_up || !h) return fail(MOE_ERR_INVALID_ARG, "%s: null pointer", what);
    if (!aligned16(x) || !aligned16(w_gate) || !aligned16(w_up))
        return fail(MOE_ERR_INVALID_ARG, "%s: x and weights must be 16-byte aligned", what);
    return run_dense(EPI_SWIGLU, x, w_gate, w_up, nullptr, h, M, I, H, ws, ws_bytes, as_stream(stream), what);
}

extern "C" int moe_silu_mul_bf16(const uint16_t* g, const uint16_t* u, uint16_t* h, int64_t n, void* stream) {
    using namespace moe;
    if (n < 0) return fail(MOE_ERR_INVALID_ARG, "moe_silu_mul_bf16: n=%lld", (long long)n);
    if (n == 0) return MOE_OK;
    if (!g || !u || !h) return fail(MOE_ERR_INVALID_ARG, "moe_silu_mul_bf16: null pointer");
    hipLaunchKernelGGL(k_silu_mul, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, as_stream(stream), g, u, h, (long)n);
    return launch_status("moe_silu_mul_bf16");
}

extern "C" int moe_rmsnorm_bf16(const uint16_t* x, const uint16_t* gain, float eps, uint16_t* y, int M, int N,
                                void* stream) {
    using namespace moe;
    if (M < 0 || N <= 0 || !(eps >= 0.0f)) return fail(MOE_ERR_INVALID_ARG, "moe_rmsnorm_bf16: bad sizes/eps");
    if (M == 0) return MOE_OK;
    if (!x || !gain || !y) return fail(MOE_ERR_INVALID_ARG, "moe_rmsnorm_bf16: null pointer");
    hipLaunchKernelGGL(k_rmsnorm, dim3(M), dim3(256), 0, as_stream(stream), x, gain, eps, y, N);
    return launch_status("moe_rmsnorm_bf16");
}
