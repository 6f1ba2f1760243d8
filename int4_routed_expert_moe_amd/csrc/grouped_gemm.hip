// Grouped int4 expert GEMMs over the ragged expert segments ("Kimi
// exact-generator adaptation": routed gate/up/down as packed int4 with group-32
// scales, "The preserved forward form"; "Kimi K2.5 donor reference", record
// "SwiGLU-style gated feed-forward projection"; "Kimi-K3 latent MoE" page,
// Code: the per-expert loop of moe_infer, here one launch for all experts).
//
// Work item = (tile, column chunk).  A tile is up to 16*MB consecutive rows of
// one expert's segment of the permuted slot list; its expert and first row
// come from the device-side offsets (no host synchronisation; the grid is
// sized for the worst case and surplus blocks exit).  A workgroup is 4 waves;
// each wave owns a few column blocks of weight rows and all tile rows.  Three
// kernels by tile height: k_grouped_skinny (at most 16 rows, decode),
// k_grouped / k_grouped_exact (16*MB rows, 16x16x32 shape) and k_grouped32
// (32*M32 rows, 32x32x16 shape, bf16 prefill).
//
// Matrix cores: v_mfma_f32_16x16x32_f16 (and 32x32x16).  Weights are dequantised in
// registers to fp16 q*s: a nibble is moved to bits 6..9 of a half, its sign
// bit flipped and an exponent OR-ed in (the half is then 16 + q + 8), and one
// packed fma with (s, -24 s) gives q*s exactly (q*s has at most 11 significant
// bits; s and 24 s are exact in fp16 for scales in [2^-14, 2^9]).  Two weights
// per packed op; the half pairs hold elements (p, p+4) of an 8-element block,
// and the activation tile in LDS is stored with the same in-block order.
//
// Weights are read in a fragment-major layout made once by moe_int4_prepack
// (an exact byte permutation of the checkpoint layout: int4 stays int4, the
// scales stay bf16).  For expert e, 16-row group n16 and 128-wide K chunk c,
// one 1 KB weight fragment holds, for lane l = r + 16 j, the 16 bytes
// [dword of group 4c+g covering K 128c+32g+8j .. +7, g = 0..3] of row
// 16 n16 + r; the matching 128-byte scale fragment holds the 4 group scales of
// each of the 16 rows.  Each wave-wide load is then one contiguous 1 KB (or
// 128 B) piece: every fetched cache line is used whole, at once.
//
// Each matrix-core step covers exactly one scale group (lane j supplies its
// K sub-block j).  bf16 mode: activations are converted to fp16 (exact for
// |x| < 65504 away from fp16 subnormals) and all of K accumulates in one fp32
// accumulator.  Exact mode: int8 activations are exact fp16 integers, so a
// step's result is s_w * G with G the exact int32 group sum (every partial sum
// is an integer multiple of the scale's last-bit weight below 2^24, hence
// exact in fp32); it is folded into the row's accumulator as
// fma(s_w*G, s_x, acc), groups ascending.  With 16-bit activation codes the
// high and low bytes are two exact fp16 operand planes and two steps per group
// give s_w*G_hi and s_w*G_lo, joined exactly as fma(s_w*G_hi, 256, s_w*G_lo).
#include <algorithm>
#include <type_traits>

#include "moe_common.h"

namespace {

constexpr int kKC = 128;        // K elements per chunk (4 scale groups)
constexpr int kAStride = 136;   // halves per LDS activation row (128 + 8 pad)
constexpr int kFragBytes = 1024;  // weight fragment: 16 rows x 128 K
constexpr int kFragScales = 64;   // scale fragment: 16 rows x 4 groups (bf16)

struct GroupedArgs {
    const void* act;        // bf16 or int8 [rows][K]
    const float* act_scale; // exact: [rows][K/32]
    const uint8_t* w0;      // gate (gate/up) or down, prepacked
    const uint16_t* s0;
    const uint8_t* w1;      // up (gate/up only), prepacked
    const uint16_t* s1;
    const int32_t* offsets;
    const int32_t* sorted_slot;
    int k;
    int E;
    int K;
    int N;          // output columns per matrix
    int n_chunks;   // column chunks per tile
    void* out;
    float* out_scale;
    uint32_t act_bytes;  // size of act in bytes, when under 4 GiB (32x32 kernel's loads)
};

struct TileInfo {
    int e;
    int row0;   // first sorted position of the tile
    int rows;   // rows in the tile (1..16*MB)
};

// Work items are (tile, column chunk) pairs: ceil(count_e / bm) tiles per expert
// of ceil(count_e / tiles) consecutive sorted rows (the last may be shorter),
// n_chunks column chunks per tile.  The
// grid is sized on the host for the worst case; here every wave derives the
// real item count from the offsets (each lane owns a run of up to 16 experts,
// so all offset loads are issued at once) and spreads the real items over the
// 8 XCDs in equal contiguous runs (the items of one tile, which share its
// activation rows, stay on one XCD).  Blocks past the real count return
// false.  The result is wave-uniform.
__device__ bool locate_item(const int32_t* __restrict__ offsets, int E, int bm, int n_chunks, TileInfo& ti,
                            int& nc) {
    const int lane = lane_id();
    const int per = (E + MOE_WAVE - 1) / MOE_WAVE;  // experts per lane (E <= 1024)
    const int e0 = min(lane * per, E);
    int bound[17];  // offsets[e0 .. e0+per], clamped to the last expert
#pragma unroll
    for (int i = 0; i <= 16; ++i)
        if (i <= per) bound[i] = offsets[min(e0 + i, E)];
    int mine_tiles = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i)
        if (i < per) mine_tiles += (bound[i + 1] - bound[i] + bm - 1) / bm;
    int incl = mine_tiles;
#pragma unroll
    for (int d = 1; d < MOE_WAVE; d <<= 1) {
        const int v = __shfl_up(incl, d);
        if (lane >= d) incl += v;
    }
    const long n_real = (long)__shfl(incl, MOE_WAVE - 1) * n_chunks;
    const long per_xcd = (n_real + 7) / 8;
    const long q = (long)(blockIdx.x >> 3);
    if (q >= per_xcd) return false;
    const long L = (long)(blockIdx.x & 7) * per_xcd + q;
    if (L >= n_real) return false;
    const long tile = L / n_chunks;
    nc = (int)(L % n_chunks);
    const int excl = incl - mine_tiles;
    const uint64_t m = __ballot(tile >= excl && tile < incl);
    const int src = __ffsll((unsigned long long)m) - 1;
    int fe = 0, frow0 = 0, frows = 0;
    if (lane == src) {
        int t = (int)(tile - excl);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            if (i < per && frows == 0) {
                const int cnt = bound[i + 1] - bound[i];
                const int nt = (cnt + bm - 1) / bm;
                if (t < nt) {
                    const int rpt = (cnt + nt - 1) / nt;  // balanced: the tiles differ by at most one row
                    fe = e0 + i;
                    frow0 = bound[i] + t * rpt;
                    frows = min(rpt, cnt - t * rpt);
                }
                t -= nt;
            }
        }
    }
    // wave-uniform by construction; reading them through readfirstlane puts them
    // (and the fragment bases derived from them) in scalar registers
    ti.e = __builtin_amdgcn_readfirstlane(__shfl(fe, src));
    ti.row0 = __builtin_amdgcn_readfirstlane(__shfl(frow0, src));
    ti.rows = __builtin_amdgcn_readfirstlane(__shfl(frows, src));
    nc = __builtin_amdgcn_readfirstlane(nc);
    return true;
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

// First fragment (chunk 0) of 16-row group n16 of expert e in a prepacked
// matrix with N rows per expert and nch chunks per row.
__device__ __forceinline__ size_t frag_index(int e, int n16, int N, int nch) {
    return ((size_t)e * (size_t)(N / 16) + (size_t)n16) * (size_t)nch;
}

// 8 int4 weights of one packed dword (element p in nibble p) -> fp16 q*s,
// ordered (e0, e4, e1, e5, e2, e6, e3, e7).
__device__ __forceinline__ half8_t dequant8(uint32_t w, half2_t s2, half2_t c2) {
    const uint32_t M = 0x03C003C0u;  // bits 6..9 of each half
    const uint32_t X = 0x4E004E00u;  // flips the nibble's sign bit, sets the exponent of 16
    const uint32_t t0 = ((w << 6) & M) ^ X;
    const uint32_t t1 = ((w << 2) & M) ^ X;
    const uint32_t t2 = ((w >> 2) & M) ^ X;
    const uint32_t t3 = ((w >> 6) & M) ^ X;
    const half2_t h0 = __builtin_elementwise_fma(__builtin_bit_cast(half2_t, t0), s2, c2);
    const half2_t h1 = __builtin_elementwise_fma(__builtin_bit_cast(half2_t, t1), s2, c2);
    const half2_t h2 = __builtin_elementwise_fma(__builtin_bit_cast(half2_t, t2), s2, c2);
    const half2_t h3 = __builtin_elementwise_fma(__builtin_bit_cast(half2_t, t3), s2, c2);
    half8_t r;
    r[0] = h0[0]; r[1] = h0[1];
    r[2] = h1[0]; r[3] = h1[1];
    r[4] = h2[0]; r[5] = h2[1];
    r[6] = h3[0]; r[7] = h3[1];
    return r;
}

// Pair Q (0..3) of dequant8: elements (Q, Q+4) of dword w, the same three
// operations, so that a caller can spread one dword's conversion over several
// matrix-core operations.
template <int Q>
__device__ __forceinline__ uint32_t dequant_pair(uint32_t w, half2_t s2, half2_t c2) {
    const uint32_t M = 0x03C003C0u;
    const uint32_t X = 0x4E004E00u;
    const uint32_t sh = Q == 0 ? (w << 6) : Q == 1 ? (w << 2) : Q == 2 ? (w >> 2) : (w >> 6);
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(__builtin_bit_cast(half2_t, (sh & M) ^ X), s2, c2));
}

// Group scale (fp16 bits, as moe_int4_prepack stores it) -> (s, s) and
// (-24 s, -24 s) in fp16; -24 s is exact for scales in the supported range.
__device__ __forceinline__ void scale_pair(uint32_t sbits, half2_t& s2, half2_t& c2) {
    const uint32_t b = sbits & 0xFFFFu;
    s2 = __builtin_bit_cast(half2_t, b | (b << 16));
    c2 = s2 * half2_t{(_Float16)-24.0f, (_Float16)-24.0f};
}
// 8 bf16 (4 dwords, elements in order) -> 8 fp16 in the (p, p+4) pair order.
__device__ __forceinline__ u32x4_t bf16x8_to_f16_perm(u32x4_t d) {
    const float f0 = __uint_as_float(d[0] << 16), f1 = __uint_as_float(d[0] & 0xFFFF0000u);
    const float f2 = __uint_as_float(d[1] << 16), f3 = __uint_as_float(d[1] & 0xFFFF0000u);
    const float f4 = __uint_as_float(d[2] << 16), f5 = __uint_as_float(d[2] & 0xFFFF0000u);
    const float f6 = __uint_as_float(d[3] << 16), f7 = __uint_as_float(d[3] & 0xFFFF0000u);
    u32x4_t r;
    r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(f0, f4));
    r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(f1, f5));
    r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(f2, f6));
    r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(f3, f7));
    return r;
}

// The fp16 staging format of activations (moe_act_f16p, mode
// MOE_MODE_BF16_F16P): each 8-element block stored as e0,e4,e1,e5,e2,e6,e3,e7,
// the pair order above.  Position of element `col` of a row in that format.
__device__ __forceinline__ int f16p_col(int col) {
    const int e = col & 7;
    return (col & ~7) | (e < 4 ? 2 * e : 2 * e - 7);
}

// bf16 bits -> fp16 bits, rounding toward zero as the staging conversion does
// (exact for bf16 values in the fp16 normal range).
__device__ __forceinline__ uint16_t bf16_to_f16_bits(uint32_t b) {
    return (uint16_t)(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(bf16_bits_to_f32(b), 0.0f)) & 0xFFFFu);
}

// Store of a gate/up output element h (bf16 bits hb) at row-major index
// row_base + col: bf16 as is, or in the fp16 staging format.
template <bool F16P>
__device__ __forceinline__ void store_h(void* out, size_t row_base, int col, uint32_t hb) {
    if constexpr (F16P)
        static_cast<uint16_t*>(out)[row_base + f16p_col(col)] = bf16_to_f16_bits(hb);
    else
        static_cast<uint16_t*>(out)[row_base + col] = (uint16_t)hb;
}

// bf16 path helpers (its outputs are compared within a tolerance; the exact
// path keeps the pinned moe_silu).  SiLU on the hardware exp2 and reciprocal,
// a few fp32 ulps, far below a bf16 step; and the gfx950 packed conversion of
// two fp32 values to bf16, round to nearest even like f32_to_bf16_bits.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float silu_fast(float z) {
    const float e = __builtin_amdgcn_exp2f(-z * 1.44269504088896341f);
    return z * __builtin_amdgcn_rcpf(1.0f + e);
}
__device__ __forceinline__ uint32_t bf16x2_bits(float lo, float hi) {
    const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// 8 int8 (2 dwords, elements in order) -> 8 exact fp16 integers in pair order.
__device__ __forceinline__ u32x4_t i8x8_to_f16_perm(uint32_t d0, uint32_t d1) {
    u32x4_t r;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const uint32_t sel = 0x0C000C00u | ((uint32_t)(4 + p) << 16) | (uint32_t)p;
        uint32_t t = __builtin_amdgcn_perm(d1, d0, sel);       // (e_p, e_{p+4}) in the low bytes
        t = (t ^ 0x00800080u) | 0x64006400u;                    // fp16 1024 + (q + 128)
        const half2_t h = __builtin_bit_cast(half2_t, t) + half2_t{(_Float16)-1152.0f, (_Float16)-1152.0f};
        r[p] = __builtin_bit_cast(uint32_t, h);
    }
    return r;
}

// 8 int16 (4 dwords, elements in order) -> their high bytes (signed) and low
// bytes (unsigned) as exact fp16 integers in pair order, q = 256 * hi + lo.
__device__ __forceinline__ void i16x8_to_f16_hilo(u32x4_t d, u32x4_t& hi, u32x4_t& lo) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const uint32_t A = d[p >> 1], B = d[2 + (p >> 1)];  // elements p and p + 4
        const uint32_t hb = 2 * (p & 1) + 1, lb = 2 * (p & 1);
        uint32_t th = __builtin_amdgcn_perm(B, A, 0x0C000C00u | ((4 + hb) << 16) | hb);
        uint32_t tl = __builtin_amdgcn_perm(B, A, 0x0C000C00u | ((4 + lb) << 16) | lb);
        th = (th ^ 0x00800080u) | 0x64006400u;  // fp16 1024 + (hi + 128)
        tl = tl | 0x64006400u;                  // fp16 1024 + lo
        hi[p] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, th) +
                                                 half2_t{(_Float16)-1152.0f, (_Float16)-1152.0f});
        lo[p] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, tl) +
                                                 half2_t{(_Float16)-1024.0f, (_Float16)-1024.0f});
    }
}

// Tiles of up to 16*MB rows on the 16x16x32 shape: bf16 tiles of 2, 4 or 6 row
// blocks (mid-size batches) and every exact-mode tile (2 or 4 row blocks).  A
// workgroup is 4 waves; each wave owns CB column blocks of 16 weight rows and
// all tile rows, so a dequantised weight fragment feeds up to MB matrix-core
// steps.  The tile's activation rows are gathered, converted to fp16 (unless
// already in the fp16 staging format) and staged in LDS one 128-wide K chunk
// ahead (double buffer, one LDS-only barrier per chunk); weights and scales run
// in a register ring of RING slots.  Rows past the tile's count read a valid
// row and are never written out (an output row depends only on its own
// activation row).
template <int MODE, int OP, int MB, int CB>
__device__ __forceinline__ void grouped_tile(const GroupedArgs& a) {
    static_assert(CB == 2 || CB == 4, "column blocks per wave");
    static_assert(CB == 4 || MODE != MOE_MODE_EXACT_I8, "exact mode quantises 32 output columns per wave");
    constexpr int BM = 16 * MB;
    constexpr bool EXACT = MODE == MOE_MODE_EXACT_I8 || MODE == MOE_MODE_EXACT_I16;
    constexpr bool ACT16 = MODE == MOE_MODE_EXACT_I16;  // 16-bit activation codes: two fp16 planes
    constexpr bool F16P = MODE == MOE_MODE_BF16_F16P;  // activations already in the fp16 staging format
    constexpr bool GATEUP = OP == 0;
    // activation staging: a bf16 row chunk is 16 pieces of 16 B, an int8 row chunk 8
    constexpr int PIECES = (EXACT && !ACT16) ? 8 : 16;
    constexpr int A_ITERS = BM * PIECES / 256;
    static_assert(BM * PIECES % 256 == 0 && A_ITERS * (64 / PIECES) * 4 == BM, "staging pieces must tile the workgroup");

    __shared__ __attribute__((aligned(16))) _Float16 As[2][BM][kAStride];
    // 16-bit activations: As holds the high-byte plane, As2 the low-byte plane
    __shared__ __attribute__((aligned(16))) _Float16 As2[ACT16 ? 2 : 1][ACT16 ? BM : 1][kAStride];
    __shared__ __attribute__((aligned(16))) float SXs[2][4][EXACT ? BM : 1];
    __shared__ int32_t rowsrc[BM];

    TileInfo ti;
    int nc;
    if (!locate_item(a.offsets, a.E, BM, a.n_chunks, ti, nc)) return;

    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15;   // row/column within a 16-block
    const int j = lane >> 4;   // k-block of the lane (0..3)
    const int K = a.K;
    const int N = a.N;
    const int nch = K / kKC;

    if (tid < BM) {
        int src = -1;
        if (tid < ti.rows) src = GATEUP ? a.sorted_slot[ti.row0 + tid] / a.k : ti.row0 + tid;
        rowsrc[tid] = src;
    }

    // this wave's weight fragments, per column block (16 rows each): gate/up
    // waves own 8*CB output columns (CB/2 gate blocks, then the matching up
    // blocks), down waves 16*CB
    // Weights and scales are read through buffer descriptors over the tile
    // expert's fragments (the host bounds an expert's matrix below 2 GiB), with
    // each column block's fragment offset in a scalar register and one lane
    // offset shared by all blocks.
    const int n0 = GATEUP ? (nc * 4 + wave) * (8 * CB) : (nc * 4 + wave) * (16 * CB);
    const uint32_t w_bytes = (uint32_t)(N / 16) * (uint32_t)nch * kFragBytes;
    const uint32_t s_bytes = (uint32_t)(N / 16) * (uint32_t)nch * kFragScales * 2;
    const __amdgpu_buffer_rsrc_t rw0 = buffer_rsrc_uniform(a.w0 + (size_t)ti.e * w_bytes, w_bytes);
    const __amdgpu_buffer_rsrc_t rs0 = buffer_rsrc_uniform(a.s0 + (size_t)ti.e * (s_bytes / 2), s_bytes);
    const __amdgpu_buffer_rsrc_t rw1 = GATEUP ? buffer_rsrc_uniform(a.w1 + (size_t)ti.e * w_bytes, w_bytes) : rw0;
    const __amdgpu_buffer_rsrc_t rs1 = GATEUP ? buffer_rsrc_uniform(a.s1 + (size_t)ti.e * (s_bytes / 2), s_bytes) : rs0;
    int woff[CB], soff[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
        const int n16 = (n0 >> 4) + (GATEUP ? (cb % (CB / 2)) : cb);
        woff[cb] = __builtin_amdgcn_readfirstlane(n16 * nch * kFragBytes);
        soff[cb] = __builtin_amdgcn_readfirstlane(n16 * nch * (kFragScales * 2));
    }
    const uint32_t lane_w = (uint32_t)lane * 16u, lane_s = (uint32_t)r * 8u;
    lds_barrier();  // rowsrc visible

    // staging: each load instruction of a wave reads RPI whole row chunks (PIECES
    // lanes x 16 contiguous bytes per row), so every cache line it touches is used
    // whole; wave w moves rows A_ITERS*RPI*w + RPI*it + lane/PIECES.  Rows past the
    // tile take the tile's first row.
    constexpr int PIECE_ELEMS = (EXACT && !ACT16) ? 16 : 8;
    constexpr int RPI = 64 / PIECES;
    auto srow_of = [&](int it) { return A_ITERS * RPI * wave + RPI * it + lane / PIECES; };
    int aoff[A_ITERS];
#pragma unroll
    for (int it = 0; it < A_ITERS; ++it) {
        const int src = rowsrc[srow_of(it)];
        aoff[it] = (src >= 0 ? src : rowsrc[0]) * K + (lane % PIECES) * PIECE_ELEMS;
    }
    int sxrow = 0;
    if (EXACT && tid < BM) sxrow = rowsrc[tid] >= 0 ? rowsrc[tid] : rowsrc[0];

    const int active_mb = (ti.rows + 15) >> 4;

    struct Slot {
        u32x4_t B[CB];   // dwords of groups 0..3 (K sub-block j), per column block
        u32x2_t S[CB];   // 4 bf16 scales of the lane's row, per column block
    };
    auto load_B = [&](int c, Slot& sl) __attribute__((always_inline)) {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
            const bool second = GATEUP && cb >= CB / 2;
            sl.B[cb] = __builtin_amdgcn_raw_buffer_load_b128(second ? rw1 : rw0, lane_w, woff[cb] + c * kFragBytes, 0);
            sl.S[cb] = __builtin_amdgcn_raw_buffer_load_b64(second ? rs1 : rs0, lane_s, soff[cb] + c * (kFragScales * 2), 0);
        }
    };
    // activation chunks in flight in registers: bf16 loads chunk c+2 while chunk c
    // is multiplied (the gathered rows come from L2 or HBM, whose latency one
    // chunk of products does not cover); exact mode, whose chunks are long
    // (VALU folds) and registers tight, chunk c+1
    constexpr int ADEPTH = EXACT ? 1 : 2;
    u32x4_t Aq[ADEPTH][A_ITERS];
    f32x4_t SXq = {0.f, 0.f, 0.f, 0.f};
    // With NACT > 0 active row blocks known at compile time, staging instructions
    // whose rows all lie past them are skipped (wave-uniform branches): their
    // rows are never read.
    auto staged = [&](auto nact, int it) __attribute__((always_inline)) {
        constexpr int NACT = decltype(nact)::value;
        return NACT == 0 || A_ITERS * RPI * wave + RPI * it < 16 * NACT;
    };
    auto load_A = [&](int c, auto nact, auto slotc) __attribute__((always_inline)) {
        constexpr int NACT = decltype(nact)::value;
        constexpr int SL = decltype(slotc)::value;
#pragma unroll
        for (int it = 0; it < A_ITERS; ++it) {
            if (!staged(nact, it)) continue;
            if (!EXACT || ACT16)
                Aq[SL][it] = *reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(a.act) + aoff[it] + c * kKC);
            else
                Aq[SL][it] = *reinterpret_cast<const u32x4_t*>(static_cast<const int8_t*>(a.act) + aoff[it] + c * kKC);
        }
        if (EXACT && tid < (NACT > 0 ? 16 * NACT : BM))
            SXq = *reinterpret_cast<const f32x4_t*>(a.act_scale + (size_t)sxrow * (K / 32) + c * 4);
    };
    auto store_A = [&](int buf, auto nact, auto slotc) __attribute__((always_inline)) {
        constexpr int NACT = decltype(nact)::value;
        constexpr int SL = decltype(slotc)::value;
#pragma unroll
        for (int it = 0; it < A_ITERS; ++it) {
            if (!staged(nact, it)) continue;
            const int row = srow_of(it);
            const int piece = lane % PIECES;
            const u32x4_t q = Aq[SL][it];
            if (ACT16) {
                u32x4_t hi, lo;
                i16x8_to_f16_hilo(q, hi, lo);
                *reinterpret_cast<u32x4_t*>(&As[buf][row][piece * 8]) = hi;
                *reinterpret_cast<u32x4_t*>(&As2[ACT16 ? buf : 0][ACT16 ? row : 0][piece * 8]) = lo;
            } else if (!EXACT) {
                *reinterpret_cast<u32x4_t*>(&As[buf][row][piece * 8]) = F16P ? q : bf16x8_to_f16_perm(q);
            } else {
                *reinterpret_cast<u32x4_t*>(&As[buf][row][piece * 16]) = i8x8_to_f16_perm(q[0], q[1]);
                *reinterpret_cast<u32x4_t*>(&As[buf][row][piece * 16 + 8]) = i8x8_to_f16_perm(q[2], q[3]);
            }
        }
        if (EXACT && tid < (NACT > 0 ? 16 * NACT : BM)) {
#pragma unroll
            for (int g = 0; g < 4; ++g) SXs[buf][g][tid] = SXq[g];
        }
    };

    f32x4_t acc[MB][CB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) acc[mb][cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    auto dequant_step = [&](const Slot& sl, int g, half8_t (&bf)[CB]) __attribute__((always_inline)) {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
            half2_t s2, c2;
            scale_pair(sl.S[cb][g >> 1] >> (16 * (g & 1)), s2, c2);
            bf[cb] = dequant8(sl.B[cb][g], s2, c2);
        }
    };
    // NACT > 0 (exact mode): one stream of 4*NACT (group step, row block)
    // products over the tile's NACT active row blocks (blocks wholly past its
    // rows are skipped; one branch-free instance per count).  Fragment and s_x
    // reads run PF products ahead.  A product's results are folded one product
    // later, so each fold reads matrix-core results issued four operations
    // earlier instead of waiting on the newest one; per row, groups still fold
    // in ascending order.  NACT == 0 (bf16): the row blocks under uniform
    // branches.
    auto compute = [&](auto nact, int c, const Slot& sl) __attribute__((always_inline)) {
        constexpr int NACT = decltype(nact)::value;
        if constexpr (NACT == 0) {
            // bf16: all MB row blocks, each under a uniform branch on the tile's
            // active count (fewer registers than the instances: this kernel
            // serves HBM-bound batches, where two waves per SIMD matter more).
            // One stream of 4 MB (group, row block) products.  Fragment reads run
            // two products ahead, unconditionally (inactive rows are staged too),
            // so that no product waits on its own LDS read; the next group's
            // weights are dequantised while the current group's products run.
            const int buf = c & 1;
            constexpr int NS = 4 * MB;
            constexpr int PFA = 2;
            auto frag = [&](int st) __attribute__((always_inline)) {
                return *reinterpret_cast<const half8_t*>(&As[buf][16 * (st % MB) + r][32 * (st / MB) + 8 * j]);
            };
            half8_t afr[NS];
#pragma unroll
            for (int q = 0; q < PFA; ++q) afr[q] = frag(q);
            half8_t bfa[CB], bfb[CB];
            dequant_step(sl, 0, bfa);
            static_for<NS>([&](auto sc) __attribute__((always_inline)) {
                constexpr int st = decltype(sc)::value;
                constexpr int g = st / MB;
                constexpr int mb = st % MB;
                if constexpr (st + PFA < NS) afr[st + PFA] = frag(st + PFA);
                half8_t(&cur)[CB] = (g & 1) ? bfb : bfa;
                half8_t(&nxt)[CB] = (g & 1) ? bfa : bfb;
                if (mb == 0 || mb < active_mb) {
#pragma unroll
                    for (int cb = 0; cb < CB; ++cb)
                        acc[mb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(afr[st], cur[cb], acc[mb][cb], 0, 0, 0);
                }
                // column blocks of group g+1 dequantised after product (g, mb)
                if constexpr (g < 3) {
#pragma unroll
                    for (int cb = 0; cb < CB; ++cb) {
                        if (cb * MB / CB == mb) {
                            half2_t s2, c2;
                            scale_pair(sl.S[cb][(g + 1) >> 1] >> (16 * ((g + 1) & 1)), s2, c2);
                            nxt[cb] = dequant8(sl.B[cb][g + 1], s2, c2);
                        }
                    }
                }
            });
        } else {
        constexpr int NS = 4 * NACT;
        constexpr int PF = EXACT ? 2 : 4;
        const int buf = c & 1;
        auto frag = [&](int st) __attribute__((always_inline)) {
            return *reinterpret_cast<const half8_t*>(&As[buf][16 * (st % NACT) + r][32 * (st / NACT) + 8 * j]);
        };
        auto sxv = [&](int st) __attribute__((always_inline)) {
            return *reinterpret_cast<const f32x4_t*>(&SXs[buf][st / NACT][16 * (st % NACT) + 4 * j]);
        };
        auto frag2 = [&](int st) __attribute__((always_inline)) {
            return *reinterpret_cast<const half8_t*>(&As2[ACT16 ? buf : 0][ACT16 ? 16 * (st % NACT) + r : 0]
                                                         [ACT16 ? 32 * (st / NACT) + 8 * j : 0]);
        };
        half8_t afr[NS], afr2[ACT16 ? NS : 1];
        f32x4_t sxr[NS];
#pragma unroll
        for (int q = 0; q < PF && q < NS; ++q) {
            afr[q] = frag(q);
            if constexpr (ACT16) afr2[q] = frag2(q);
            if constexpr (EXACT) sxr[q] = sxv(q);
        }
        half8_t bfa[CB], bfb[CB];
        dequant_step(sl, 0, bfa);
        f32x4_t d[2][CB];
        f32x4_t d2[ACT16 ? 2 : 1][CB];  // 16-bit activations: the low-byte plane's results
        auto fold = [&](auto sc) __attribute__((always_inline)) {
            constexpr int st = decltype(sc)::value;
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    // s_w * G: exact for 8-bit codes; for 16-bit codes the two planes'
                    // exact results combine with one rounding, 256 * hi + lo
                    float sg = d[st & 1][cb][i];
                    if constexpr (ACT16) sg = __builtin_fmaf(sg, 256.0f, d2[st & 1][cb][i]);
                    acc[st % NACT][cb][i] = __builtin_fmaf(sg, sxr[st][i], acc[st % NACT][cb][i]);
                }
                // an empty statement that reads and writes the sums keeps the folds
                // here, between the products, instead of all at the chunk's end
                asm volatile("" : "+v"(acc[st % NACT][cb]));
            }
        };
        static_for<NS>([&](auto sc) __attribute__((always_inline)) {
            constexpr int st = decltype(sc)::value;
            constexpr int g = st / NACT;
            constexpr int mb = st % NACT;
            if constexpr (st + PF < NS) {
                afr[st + PF] = frag(st + PF);
                if constexpr (ACT16) afr2[st + PF] = frag2(st + PF);
                if constexpr (EXACT) sxr[st + PF] = sxv(st + PF);
            }
            if constexpr (mb == 0 && g < 3) dequant_step(sl, g + 1, (g & 1) ? bfa : bfb);
            half8_t(&cur)[CB] = (g & 1) ? bfb : bfa;
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
                if constexpr (!EXACT)
                    acc[mb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(afr[st], cur[cb], acc[mb][cb], 0, 0, 0);
                else {
                    d[st & 1][cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(afr[st], cur[cb],
                                                                           f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                    if constexpr (ACT16)
                        d2[st & 1][cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                            afr2[st], cur[cb], f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                }
            }
            if constexpr (EXACT && st > 0) fold(std::integral_constant<int, st - 1>{});
            // bf16: VALU work may move across products; exact: nothing does (the
            // folds would otherwise sink past later products and hold their
            // matrix-core results)
            __builtin_amdgcn_sched_barrier(EXACT ? 0 : 0x0002);
        });
        if constexpr (EXACT) fold(std::integral_constant<int, NS - 1>{});
        }
    };

    // One chunk: stage the next activation chunk's loads, multiply the current
    // one, refill this weight slot RING chunks ahead, then write the staged
    // chunk to the other LDS buffer (whose last readers finished before the
    // previous barrier).  Indices past the end are clamped: redundant in-bounds
    // loads, and a staged buffer nobody reads.  Each instance issues its own
    // prologue (weights of the first RING chunks in flight, activation chunk 0
    // staged).  bf16 keeps three weight chunks in flight; exact mode, whose
    // chunks are long (VALU folds), two, which keeps its registers within two
    // waves per SIMD.
    constexpr int RING = EXACT ? 2 : 3;
    constexpr int UNROLL = RING * ADEPTH / (RING % ADEPTH == 0 ? ADEPTH : 1);  // lcm(RING, ADEPTH), ADEPTH <= 2
    auto main_loop = [&](auto nact) __attribute__((always_inline)) {
        Slot sl[RING];
        load_A(0, nact, std::integral_constant<int, 0>{});
#pragma unroll
        for (int i = 0; i < RING; ++i) load_B(min(i, nch - 1), sl[i]);
        if constexpr (ADEPTH == 2) load_A(min(1, nch - 1), nact, std::integral_constant<int, 1>{});
        store_A(0, nact, std::integral_constant<int, 0>{});
        lds_barrier();
        // step c: load chunk c+ADEPTH into the register slot chunk c left (it is in
        // LDS already), multiply chunk c, refill the weight slot, write chunk c+1
        // (loaded ADEPTH-1 steps ago) to the other LDS buffer
        auto step = [&](int c, auto ic) __attribute__((always_inline)) {
            constexpr int I = decltype(ic)::value;
            load_A(min(c + ADEPTH, nch - 1), nact, std::integral_constant<int, I % ADEPTH>{});
            __builtin_amdgcn_sched_barrier(0);
            compute(nact, c, sl[I % RING]);
            __builtin_amdgcn_sched_barrier(0);
            load_B(min(c + RING, nch - 1), sl[I % RING]);
            __builtin_amdgcn_sched_barrier(0);
            store_A((c + 1) & 1, nact, std::integral_constant<int, (I + 1) % ADEPTH>{});
            lds_barrier();
        };
        int c = 0;
        for (; c + UNROLL <= nch; c += UNROLL)
            static_for<UNROLL>([&](auto ic) __attribute__((always_inline)) { step(c + decltype(ic)::value, ic); });
        static_for<UNROLL - 1>([&](auto ic) __attribute__((always_inline)) {
            if (c + decltype(ic)::value < nch) step(c + decltype(ic)::value, ic);
        });
    };
    if constexpr (EXACT) {
        static_for<MB>([&](auto ic) __attribute__((always_inline)) {
            constexpr int n = decltype(ic)::value + 1;
            if (active_mb == n) main_loop(std::integral_constant<int, n>{});
        });
    } else {
        main_loop(std::integral_constant<int, 0>{});
    }

    // ---- epilogue ----
    if (GATEUP) {
        const int grp = n0 / 32;  // this wave's 32 output columns form one scale group
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            if (mb >= active_mb) continue;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int rl = 16 * mb + 4 * j + i;
                const bool ok = rl < ti.rows;
                const size_t orow = (size_t)(ti.row0 + rl);
                if (!EXACT) {
#pragma unroll
                    for (int p = 0; p < CB / 2; ++p) {
                        // g and u rounded to bf16 by one packed conversion, SiLU on the
                        // hardware exp2 and reciprocal (bf16 path)
                        const uint32_t v = bf16x2_bits(acc[mb][p][i], acc[mb][CB / 2 + p][i]);
                        const float g = __uint_as_float(v << 16), u = __uint_as_float(v & 0xFFFF0000u);
                        const uint32_t ab = bf16x2_bits(silu_fast(g), 0.0f) & 0xFFFFu;
                        const uint32_t hb = bf16x2_bits(__uint_as_float(ab << 16) * u, 0.0f) & 0xFFFFu;
                        if (ok) store_h<F16P>(a.out, orow * N, n0 + 16 * p + r, hb);
                    }
                } else {
                    const float h0 = moe_silu(acc[mb][0][i]) * acc[mb][CB / 2][i];
                    const float h1 = moe_silu(acc[mb][1][i]) * acc[mb][CB - 1][i];
                    float amax = fmaxf(fabsf(h0), fabsf(h1));
#pragma unroll
                    for (int off = 1; off < 16; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
                    const float s = (amax == 0.0f) ? 0.0f : amax / (ACT16 ? 32767.0f : 127.0f);
                    if (ok) {
                        if constexpr (ACT16) {
                            int16_t* o = static_cast<int16_t*>(a.out) + orow * N + n0 + r;
                            o[0] = (int16_t)moe_quant_i16(h0, s);
                            o[16] = (int16_t)moe_quant_i16(h1, s);
                        } else {
                            int8_t* o = static_cast<int8_t*>(a.out) + orow * N + n0 + r;
                            o[0] = (int8_t)moe_quant_i8(h0, s);
                            o[16] = (int8_t)moe_quant_i8(h1, s);
                        }
                        if (r == 0) a.out_scale[orow * (N / 32) + grp] = s;
                    }
                }
            }
        }
    } else {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            if (mb >= active_mb) continue;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int rl = 16 * mb + 4 * j + i;
                if (rl >= ti.rows) continue;
                const size_t orow = (size_t)(ti.row0 + rl);
#pragma unroll
                for (int cb = 0; cb < CB; ++cb) {
                    const int col = n0 + 16 * cb + r;
                    if (!EXACT)
                        static_cast<uint16_t*>(a.out)[orow * N + col] = (uint16_t)f32_to_bf16_bits(acc[mb][cb][i]);
                    else
                        static_cast<float*>(a.out)[orow * N + col] = acc[mb][cb][i];
                }
            }
        }
    }
}

template <int MODE, int OP, int MB, int CB>
__global__ __launch_bounds__(256) void k_grouped(GroupedArgs a) {
    grouped_tile<MODE, OP, MB, CB>(a);
}

// Exact mode: register use capped at two waves per SIMD.  Under that cap the
// compiler writes matrix-core results to ordinary VGPRs, where the VALU folds
// read them (otherwise each fold first copies its operand out of an AGPR).
template <int MODE, int OP, int MB, int CB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_grouped_exact(GroupedArgs a) {
    grouped_tile<MODE, OP, MB, CB>(a);
}

// Epilogue of the 32x32 tile kernels: element i of lane l is tile row
// 32 mb + 8(i/4) + 4 kb + i%4, column c32 of each column block.  Gate/up:
// h = bf16(bf16(silu(g)) * u) from g = bf16(gate sum), u = bf16(up sum)
// (both converted by one packed instruction), stored as bf16 or in the fp16
// staging format; down: the two column blocks' sums as bf16.
template <bool GATEUP, bool F16P, int M32>
__device__ __forceinline__ void epilogue32(const GroupedArgs& a, const TileInfo& ti, int n0, int c32, int kb,
                                           const f32x16_t (&acc)[M32][2]) {
    const int N = a.N;
    uint16_t* out = static_cast<uint16_t*>(a.out) + (size_t)ti.row0 * (size_t)N +
                    (GATEUP && F16P ? f16p_col(n0 + c32) : n0 + c32);
#pragma unroll
    for (int mb = 0; mb < M32; ++mb) {
        if (32 * mb >= ti.rows) break;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int rl = 32 * mb + 8 * (i >> 2) + 4 * kb + (i & 3);
            if (rl >= ti.rows) continue;
            uint16_t* o = out + (size_t)rl * (size_t)N;
            const uint32_t v = bf16x2_bits(acc[mb][0][i], acc[mb][1][i]);
            if constexpr (GATEUP) {
                const float g = __uint_as_float(v << 16), u = __uint_as_float(v & 0xFFFF0000u);
                const uint32_t ab = bf16x2_bits(silu_fast(g), 0.0f) & 0xFFFFu;
                const uint32_t hb = bf16x2_bits(__uint_as_float(ab << 16) * u, 0.0f) & 0xFFFFu;
                o[0] = F16P ? bf16_to_f16_bits(hb) : (uint16_t)hb;
            } else {
                o[0] = (uint16_t)(v & 0xFFFFu);
                o[32] = (uint16_t)(v >> 16);
            }
        }
    }
}

// Large bf16 tiles on the 32x32x16 matrix-core shape (one wave per SIMD drives
// it at close to the peak rate; the 16x16x32 shape needs two).  Tiles of
// 32*M32 rows; each wave owns two 32-row column blocks (gate/up: 32 gate rows
// and the matching 32 up rows; down: 64 output columns) and all tile rows.
// Operands: lane l = c + 32 kb holds row/column c of a 32-block and K
// sub-block kb of each 16-wide K step.  From the fragment layout a lane takes
// the 16-byte pieces of 16-row lanes (c mod 16, kb) and (c mod 16, kb + 2):
// dword g of the first holds K step 2g, of the second step 2g + 1.  The
// accumulator element i of lane l is row 8(i/4) + 4 kb + i%4, column c.
// Staging, barrier and weight ring as in k_grouped.
template <int OP, int M32, bool F16P>
__global__ __launch_bounds__(256) void k_grouped32(GroupedArgs a) {
    constexpr int BM = 32 * M32;
    constexpr bool GATEUP = OP == 0;
    constexpr int PIECES = 16;
    constexpr int A_ITERS = BM * PIECES / 256;
    constexpr int AST = 144;  // halves per LDS row (128 + 16 pad)
    static_assert(BM % 16 == 0 && A_ITERS * 4 * 4 == BM, "staging: 4 rows per wave instruction");

    __shared__ __attribute__((aligned(16))) _Float16 As[2][BM][AST];
    __shared__ int32_t rowsrc[BM];

    TileInfo ti;
    int nc;
    if (!locate_item(a.offsets, a.E, BM, a.n_chunks, ti, nc)) return;

    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wave = tid >> 6;
    const int c32 = lane & 31;  // row (A) / column (B, D) within a 32-block
    const int kb = lane >> 5;   // K sub-block within a 16-wide step
    const int K = a.K;
    const int N = a.N;
    const int nch = K / kKC;

    if (tid < BM) {
        int src = -1;
        if (tid < ti.rows) src = GATEUP ? a.sorted_slot[ti.row0 + tid] / a.k : ti.row0 + tid;
        rowsrc[tid] = src;
    }

    // this wave's two 32-row column blocks: first 16-row group of each, its fragment pointers
    const int n0 = GATEUP ? (nc * 4 + wave) * 32 : (nc * 4 + wave) * 64;
    const uint8_t* wf[2];
    const uint16_t* sf[2];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
        const int n16 = (GATEUP ? n0 : n0 + 32 * cb) / 16 + (c32 >> 4);
        const bool second = GATEUP && cb == 1;
        const size_t f = frag_index(ti.e, n16, N, nch);
        wf[cb] = (second ? a.w1 : a.w0) + f * kFragBytes + ((c32 & 15) + 16 * kb) * 16;
        sf[cb] = (second ? a.s1 : a.s0) + f * kFragScales + 4 * (c32 & 15);
    }
    lds_barrier();  // rowsrc visible

    // staging: each load instruction of a wave reads 4 whole row chunks (16 lanes x
    // 16 contiguous bytes per row), so every cache line it touches is used whole;
    // wave w moves rows A_ITERS*4*w + 4*it + lane/16.  Rows past the tile take the
    // tile's first row.  The loads are raw buffer loads with 32-bit byte offsets
    // (the host launches this kernel only for activations under 4 GiB): one
    // offset register per load, the chunk offset in a scalar register.
    uint32_t aoff[A_ITERS];
#pragma unroll
    for (int it = 0; it < A_ITERS; ++it) {
        const int src = rowsrc[A_ITERS * 4 * wave + 4 * it + (lane >> 4)];
        aoff[it] = ((uint32_t)(src >= 0 ? src : rowsrc[0]) * (uint32_t)K + (uint32_t)(lane & 15) * 8u) * 2u;
    }

    struct Slot {
        u32x4_t B[2][2];  // per column block: pieces (kb) and (kb + 2)
        u32x2_t S[2];     // per column block: 4 bf16 group scales of the lane's column
    };
    auto load_B = [&](int c, Slot& sl) __attribute__((always_inline)) {
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
            sl.B[cb][0] = *reinterpret_cast<const u32x4_t*>(wf[cb] + (size_t)c * kFragBytes);
            sl.B[cb][1] = *reinterpret_cast<const u32x4_t*>(wf[cb] + (size_t)c * kFragBytes + 512);
            sl.S[cb] = *reinterpret_cast<const u32x2_t*>(sf[cb] + (size_t)c * kFragScales);
        }
    };
    u32x4_t Aq[A_ITERS];
    const __amdgpu_buffer_rsrc_t act_rsrc = buffer_rsrc(a.act, a.act_bytes);
    auto load_piece = [&](int it, int c) __attribute__((always_inline)) {
        Aq[it] = __builtin_amdgcn_raw_buffer_load_b128(act_rsrc, aoff[it], c * (kKC * 2), 0);
    };
    auto store_piece = [&](int it, int buf) __attribute__((always_inline)) {
        *reinterpret_cast<u32x4_t*>(&As[buf][A_ITERS * 4 * wave + 4 * it + (lane >> 4)][(lane & 15) * 8]) =
            F16P ? Aq[it] : bf16x8_to_f16_perm(Aq[it]);
    };
    auto load_A = [&](int c) __attribute__((always_inline)) {
#pragma unroll
        for (int it = 0; it < A_ITERS; ++it) load_piece(it, c);
    };
    auto store_A = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int it = 0; it < A_ITERS; ++it) store_piece(it, buf);
    };

    f32x16_t acc[M32][2];
#pragma unroll
    for (int mb = 0; mb < M32; ++mb)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[mb][cb][i] = 0.0f;

    // dequantised operands of K step s (column blocks 0, 1)
    // Piece J (0..7) of K step st's dequantised operands: column block J/4, pair
    // J%4 (three VALU operations); the group's scale pair is converted at the
    // block's first piece of the group's first step and kept for its second.
    auto dq_piece = [&](const Slot& sl, int st, auto jc, half2_t (&s2)[2], half2_t (&c2)[2],
                        u32x4_t (&bf)[2]) __attribute__((always_inline)) {
        constexpr int J = decltype(jc)::value;
        constexpr int cb = J >> 2, q = J & 3;
        const int g = st >> 1;
        if (q == 0 && (st & 1) == 0) scale_pair(sl.S[cb][g >> 1] >> (16 * (g & 1)), s2[cb], c2[cb]);
        bf[cb][q] = dequant_pair<q>(sl.B[cb][st & 1][g], s2[cb], c2[cb]);
    };
    // One stream of 8*NACT (K step, row block) products over the tile's NACT
    // active row blocks (blocks wholly past its rows are skipped); fragment
    // reads run PF products ahead; only VALU work (the next step's
    // dequantisation, the staged chunk's conversion) may move across products.
    // The next activation chunk is staged piece by piece, the A_ITERS pieces
    // spread evenly over the products: piece i, loaded at the same point of the
    // previous chunk, is converted and written to the other LDS buffer (whose
    // last readers finished before the previous barrier), and the same piece of
    // the chunk after is loaded into the freed registers.  Loads retire in issue
    // order, so each piece's wait leaves the younger pieces and the newest
    // weight slot in flight: it covers only loads issued a whole chunk earlier,
    // and the conversion work is spread among the products instead of stalling
    // them at one point.
    auto compute = [&](auto nact, int c, const Slot& sl) __attribute__((always_inline)) {
        constexpr int NACT = decltype(nact)::value;
        constexpr int NS = 8 * NACT;
        constexpr int PF = 4;
        const int buf = c & 1;
        auto frag = [&](int p) __attribute__((always_inline)) {
            return *reinterpret_cast<const half8_t*>(&As[buf][32 * (p % NACT) + c32][16 * (p / NACT) + 8 * kb]);
        };
        half8_t afr[NS];
#pragma unroll
        for (int q = 0; q < PF; ++q) afr[q] = frag(q);
        // the next step's operands are converted in 8 pieces spread evenly over
        // this step's products (piece J at product J*NACT/8): a clump of all 8 at
        // one product outlasts the matrix-core operations around it
        u32x4_t bfa[2], bfb[2];
        half2_t s2[2], c2[2];
        static_for<8>([&](auto jc) __attribute__((always_inline)) { dq_piece(sl, 0, jc, s2, c2, bfa); });
        static_for<NS>([&](auto pc) __attribute__((always_inline)) {
            constexpr int p = decltype(pc)::value;
            constexpr int st = p / NACT;
            constexpr int mb = p % NACT;
            if constexpr (p + PF < NS) afr[p + PF] = frag(p + PF);
            static_for<A_ITERS>([&](auto ic) __attribute__((always_inline)) {
                constexpr int i = decltype(ic)::value;
                if constexpr ((2 * i + 1) * NS / (2 * A_ITERS) == p) {  // piece i at the middle of its share
                    store_piece(i, (c + 1) & 1);
                    load_piece(i, min(c + 2, nch - 1));
                }
            });
            if constexpr (st < 7) {
                static_for<8>([&](auto jc) __attribute__((always_inline)) {
                    constexpr int J = decltype(jc)::value;
                    if constexpr (J * NACT / 8 == mb) dq_piece(sl, st + 1, jc, s2, c2, (st & 1) ? bfa : bfb);
                });
            }
            u32x4_t(&cur)[2] = (st & 1) ? bfb : bfa;
#pragma unroll
            for (int cb = 0; cb < 2; ++cb)
                acc[mb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(afr[p], __builtin_bit_cast(half8_t, cur[cb]),
                                                                      acc[mb][cb], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        });
    };

    // prologue: the loads in flight at each step's start are, in issue order,
    // weights c, weights c+1, activations c+1, weights c+2 (so a piece's wait
    // leaves weights c+2 in flight), in the first step as in every later one
    auto main_loop = [&](auto nact) __attribute__((always_inline)) {
        Slot s0, s1, s2;
        load_A(0);
        load_B(0, s0);
        load_B(min(1, nch - 1), s1);
        store_A(0);
        load_A(min(1, nch - 1));
        load_B(min(2, nch - 1), s2);
        lds_barrier();
        auto step = [&](int c, Slot& cur) __attribute__((always_inline)) {
            compute(nact, c, cur);
            __builtin_amdgcn_sched_barrier(0);
            load_B(min(c + 3, nch - 1), cur);
            lds_barrier();
        };
        int c = 0;
        for (; c + 3 <= nch; c += 3) {
            step(c, s0);
            step(c + 1, s1);
            step(c + 2, s2);
        }
        if (c < nch) step(c, s0);
        if (c + 1 < nch) step(c + 1, s1);
    };
    // one branch-free instance of the loop per active row-block count
    const int nact = (ti.rows + 31) >> 5;
    static_for<M32>([&](auto ic) __attribute__((always_inline)) {
        constexpr int n = decltype(ic)::value + 1;
        if (nact == n) main_loop(std::integral_constant<int, n>{});
    });

    epilogue32<GATEUP, F16P, M32>(a, ti, n0, c32, kb, acc);
}

// k_grouped32 for activations already in the fp16 staging format, with the
// activation tile staged by global-to-LDS buffer loads: the data goes straight
// from memory into LDS, with no VGPRs, no LDS store instructions and no waits
// in the product stream.  Such a load writes 16 bytes per lane at consecutive
// LDS addresses (1 KB per wave instruction), so a tile row is 128 halves
// unpadded and its 16-byte units are XOR-swizzled by the row's low four bits:
// lane l of the instruction for rows R..R+3 writes physical unit l mod 16 of
// row R + l/16 and fetches logical unit (l mod 16) ^ (row mod 16) for it; a
// fragment read of 16 consecutive rows then touches every bank once.  Three
// tile buffers: chunk c+2 is loaded while chunk c is multiplied, and a wave
// waits for its own loads of chunk c+1 (issued a whole chunk earlier) before
// the barrier that ends step c.  Same products and results as k_grouped32.
template <int OP, int M32>
__device__ __forceinline__ void grouped32_dma_tile(const GroupedArgs& a) {
    constexpr int BM = 32 * M32;
    constexpr bool GATEUP = OP == 0;
    constexpr int A_ITERS = BM / 16;  // staging instructions per wave per chunk (4 rows each)
    static_assert(A_ITERS * 4 * 4 == BM, "staging: 4 rows per wave instruction");

    // three separate LDS objects, so that the compiler can tell a read of one
    // buffer from the loads into another (it waits for those only on overlap)
    __shared__ __attribute__((aligned(16))) _Float16 As0[BM][kKC];
    __shared__ __attribute__((aligned(16))) _Float16 As1[BM][kKC];
    __shared__ __attribute__((aligned(16))) _Float16 As2[BM][kKC];
    __shared__ int32_t rowsrc[BM];
    auto tile = [&](auto bufc) -> _Float16(&)[BM][kKC] {
        if constexpr (decltype(bufc)::value == 0) return As0;
        else if constexpr (decltype(bufc)::value == 1) return As1;
        else return As2;
    };

    TileInfo ti;
    int nc;
    if (!locate_item(a.offsets, a.E, BM, a.n_chunks, ti, nc)) return;

    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wave = tid >> 6;
    const int c32 = lane & 31;
    const int kb = lane >> 5;
    const int K = a.K;
    const int N = a.N;
    const int nch = K / kKC;

    const int n0 = GATEUP ? (nc * 4 + wave) * 32 : (nc * 4 + wave) * 64;
    const uint8_t* wf[2];
    const uint16_t* sf[2];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
        const int n16 = (GATEUP ? n0 : n0 + 32 * cb) / 16 + (c32 >> 4);
        const bool second = GATEUP && cb == 1;
        const size_t f = frag_index(ti.e, n16, N, nch);
        wf[cb] = (second ? a.w1 : a.w0) + f * kFragBytes + ((c32 & 15) + 16 * kb) * 16;
        sf[cb] = (second ? a.s1 : a.s0) + f * kFragScales + 4 * (c32 & 15);
    }

    struct Slot {
        u32x4_t B[2][2];
        u32x2_t S[2];
    };
    auto load_B = [&](int c, Slot& sl) __attribute__((always_inline)) {
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
            sl.B[cb][0] = *reinterpret_cast<const u32x4_t*>(wf[cb] + (size_t)c * kFragBytes);
            sl.B[cb][1] = *reinterpret_cast<const u32x4_t*>(wf[cb] + (size_t)c * kFragBytes + 512);
            sl.S[cb] = *reinterpret_cast<const u32x2_t*>(sf[cb] + (size_t)c * kFragScales);
        }
    };
    // the first three weight chunks depend only on the tile's expert: they go out
    // before the activation rows are gathered, so the two latencies overlap
    Slot s0, s1, s2;
    load_B(0, s0);
    load_B(min(1, nch - 1), s1);
    load_B(min(2, nch - 1), s2);

    if (tid < BM) {
        int src = -1;
        if (tid < ti.rows) src = GATEUP ? a.sorted_slot[ti.row0 + tid] / a.k : ti.row0 + tid;
        rowsrc[tid] = src;
    }
    lds_barrier();  // rowsrc visible

    // staging instruction it of this wave: tile rows R = A_ITERS*4*wave + 4*it .. R+3
    // (rows past the tile take the tile's first row)
    uint32_t aoff[A_ITERS];
#pragma unroll
    for (int it = 0; it < A_ITERS; ++it) {
        const int row = A_ITERS * 4 * wave + 4 * it + (lane >> 4);
        const int src = rowsrc[row];
        const uint32_t unit = (uint32_t)((lane & 15) ^ (row & 15));
        aoff[it] = ((uint32_t)(src >= 0 ? src : rowsrc[0]) * (uint32_t)K + unit * 8u) * 2u;
    }
    const __amdgpu_buffer_rsrc_t act_rsrc = buffer_rsrc(a.act, a.act_bytes);
    auto dma_piece = [&](int it, int c, auto bufc) __attribute__((always_inline)) {
        buffer_load_lds16(act_rsrc, &tile(bufc)[A_ITERS * 4 * wave + 4 * it][0], aoff[it], (uint32_t)c * (kKC * 2));
    };

    f32x16_t acc[M32][2];
#pragma unroll
    for (int mb = 0; mb < M32; ++mb)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[mb][cb][i] = 0.0f;

    // Piece J (0..7) of K step st's dequantised operands: column block J/4, pair
    // J%4 (three VALU operations); the group's scale pair is converted at the
    // block's first piece of the group's first step and kept for its second.
    auto dq_piece = [&](const Slot& sl, int st, auto jc, half2_t (&s2)[2], half2_t (&c2)[2],
                        u32x4_t (&bf)[2]) __attribute__((always_inline)) {
        constexpr int J = decltype(jc)::value;
        constexpr int cb = J >> 2, q = J & 3;
        const int g = st >> 1;
        if (q == 0 && (st & 1) == 0) scale_pair(sl.S[cb][g >> 1] >> (16 * (g & 1)), s2[cb], c2[cb]);
        bf[cb][q] = dequant_pair<q>(sl.B[cb][st & 1][g], s2[cb], c2[cb]);
    };
    // One stream of 8*NACT (K step, row block) products reading tile buffer BUF;
    // the staging loads of chunk c+2 into buffer (BUF+2) mod 3 are spread over
    // its first half (the barrier that ends the step waits for all of this wave's
    // staging loads: the LDS release there covers them).
    auto compute = [&](auto nact, auto bufc, int c, const Slot& sl) __attribute__((always_inline)) {
        constexpr int NACT = decltype(nact)::value;
        constexpr int BUF = decltype(bufc)::value;
        constexpr int NS = 8 * NACT;
        constexpr int PF = 4;
        const int swz = c32 & 15;
        auto frag = [&](int p) __attribute__((always_inline)) {
            const int unit = (2 * (p / NACT) + kb) ^ swz;
            return *reinterpret_cast<const half8_t*>(&tile(bufc)[32 * (p % NACT) + c32][8 * unit]);
        };
        half8_t afr[NS];
#pragma unroll
        for (int q = 0; q < PF; ++q) afr[q] = frag(q);
        // the next step's operands in 8 pieces spread over this step's products,
        // as in k_grouped32
        u32x4_t bfa[2], bfb[2];
        half2_t s2[2], c2[2];
        static_for<8>([&](auto jc) __attribute__((always_inline)) { dq_piece(sl, 0, jc, s2, c2, bfa); });
        const int cs = min(c + 2, nch - 1);
        static_for<NS>([&](auto pc) __attribute__((always_inline)) {
            constexpr int p = decltype(pc)::value;
            constexpr int st = p / NACT;
            constexpr int mb = p % NACT;
            if constexpr (p + PF < NS) afr[p + PF] = frag(p + PF);
            static_for<A_ITERS>([&](auto ic) __attribute__((always_inline)) {
                constexpr int i = decltype(ic)::value;
                if constexpr (i * NS / (2 * A_ITERS) == p)
                    dma_piece(i, cs, std::integral_constant<int, (BUF + 2) % 3>{});
            });
            if constexpr (st < 7) {
                static_for<8>([&](auto jc) __attribute__((always_inline)) {
                    constexpr int J = decltype(jc)::value;
                    if constexpr (J * NACT / 8 == mb) dq_piece(sl, st + 1, jc, s2, c2, (st & 1) ? bfa : bfb);
                });
            }
            u32x4_t(&cur)[2] = (st & 1) ? bfb : bfa;
#pragma unroll
            for (int cb = 0; cb < 2; ++cb)
                acc[mb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(afr[p], __builtin_bit_cast(half8_t, cur[cb]),
                                                                      acc[mb][cb], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        });
    };

    // Loads issued, in order: weights 0, 1, 2 (above), staging 0, staging 1 |
    // step c: staging c+2 (A_ITERS pieces, first half of the step), weights c+3
    // (6) | wait: staging c+1 done when at most 6 + A_ITERS younger loads are
    // outstanding (the release before the barrier then also waits for staging
    // c+2).  The prologue waits for staging 0 with staging 1 still in flight.
    auto main_loop = [&](auto nact) __attribute__((always_inline)) {
#pragma unroll
        for (int it = 0; it < A_ITERS; ++it) dma_piece(it, 0, std::integral_constant<int, 0>{});
#pragma unroll
        for (int it = 0; it < A_ITERS; ++it) dma_piece(it, min(1, nch - 1), std::integral_constant<int, 1>{});
        wait_vmcnt<A_ITERS>();
        lds_barrier();
        auto step = [&](auto bufc, int c, Slot& cur) __attribute__((always_inline)) {
            compute(nact, bufc, c, cur);
            __builtin_amdgcn_sched_barrier(0);
            load_B(min(c + 3, nch - 1), cur);
            wait_vmcnt<6 + A_ITERS>();
            lds_barrier();
        };
        int c = 0;
        for (; c + 3 <= nch; c += 3) {
            step(std::integral_constant<int, 0>{}, c, s0);
            step(std::integral_constant<int, 1>{}, c + 1, s1);
            step(std::integral_constant<int, 2>{}, c + 2, s2);
        }
        if (c < nch) step(std::integral_constant<int, 0>{}, c, s0);
        if (c + 1 < nch) step(std::integral_constant<int, 1>{}, c + 1, s1);
    };
    const int nact = (ti.rows + 31) >> 5;
    static_for<M32>([&](auto ic) __attribute__((always_inline)) {
        constexpr int n = decltype(ic)::value + 1;
        if (nact == n) main_loop(std::integral_constant<int, n>{});
    });
    wait_vmcnt<0>();  // the trailing (redundant) staging loads land before the wave ends
    epilogue32<GATEUP, true, M32>(a, ti, n0, c32, kb, acc);
}

template <int OP, int M32>
__global__ __launch_bounds__(256) void k_grouped32_dma(GroupedArgs a) {
    grouped32_dma_tile<OP, M32>(a);
}

// Tiles of at most 16 rows (decode): the weights dominate the bytes, so each
// wave streams its 64 weight rows (4 fragments per chunk) independently, with
// no workgroup barrier and no LDS.  Bytes in flight set the speed here: the
// loads of the next D-1 chunks (weights, scales and the tile's activation rows)
// are in flight while the current chunk is converted and multiplied.  Chunk
// indices past the end are clamped (redundant in-bounds loads) rather than
// skipped, so every step issues the same unconditional loads and the
// outstanding-load counts stay exact; rows past the tile's count read row 0
// and are zeroed at use.  Same arithmetic as k_grouped.
template <int MODE, int OP, int D>
__global__ __launch_bounds__(256) void k_grouped_skinny(GroupedArgs a) {
    constexpr bool EXACT = MODE == MOE_MODE_EXACT_I8;
    constexpr bool F16P = MODE == MOE_MODE_BF16_F16P;  // activations already in the fp16 staging format
    constexpr bool GATEUP = OP == 0;

    TileInfo ti;
    int nc;
    if (!locate_item(a.offsets, a.E, 16, a.n_chunks, ti, nc)) return;

    const int lane = lane_id();
    const int wave = threadIdx.x >> 6;
    const int r = lane & 15;
    const int j = lane >> 4;
    const int K = a.K;
    const int N = a.N;
    const int nch = K / kKC;

    auto src_of = [&](int row) -> int {
        if (row >= ti.rows) return -1;
        return GATEUP ? a.sorted_slot[ti.row0 + row] / a.k : ti.row0 + row;
    };
    const int asrc = src_of(r);
    const bool avalid = asrc >= 0;
    const int arow = avalid ? asrc : 0;
    int dsrc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) dsrc[i] = EXACT ? src_of(4 * j + i) : -1;

    const int n0 = GATEUP ? nc * 128 + wave * 32 : nc * 256 + wave * 64;
    const uint8_t* wf[4];
    const uint16_t* sf[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
        const int n16 = (n0 >> 4) + (GATEUP ? (cb & 1) : cb);
        const bool second = GATEUP && cb >= 2;
        const size_t f = frag_index(ti.e, n16, N, nch);
        wf[cb] = (second ? a.w1 : a.w0) + f * kFragBytes + lane * 16;
        sf[cb] = (second ? a.s1 : a.s0) + f * kFragScales + 4 * r;
    }

    struct Slot {
        u32x4_t B[4];    // dwords of groups 0..3 (K sub-block j), per column block
        u32x2_t S[4];    // 4 bf16 scales of the lane's row, per column block
        u32x4_t A[4];    // per group: 8 bf16 (bf16 mode) or 8 int8 in A[g][0..1] (exact)
        f32x4_t SX[4];   // exact: s_x of result rows 4j+i for groups 0..3
    };
    auto load = [&](int c, Slot& sl) {
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
            // weights and scales are read once per launch: non-temporal loads keep
            // them from displacing the activation rows in the caches (measured 4-5%
            // faster for gate/up and about 2% for down, which then fetches 10% more
            // bytes than the plain loads did)
            sl.B[cb] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(wf[cb] + (size_t)c * kFragBytes));
            sl.S[cb] = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(sf[cb] + (size_t)c * kFragScales));
        }
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            if (!EXACT) {
                sl.A[g] = *reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(a.act) + (size_t)arow * K +
                                                             c * kKC + 32 * g + 8 * j);
            } else {
                const u32x2_t q = *reinterpret_cast<const u32x2_t*>(static_cast<const int8_t*>(a.act) +
                                                                     (size_t)arow * K + c * kKC + 32 * g + 8 * j);
                sl.A[g] = u32x4_t{q[0], q[1], 0u, 0u};
            }
        }
        if (EXACT) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                sl.SX[i] = *reinterpret_cast<const f32x4_t*>(a.act_scale + (size_t)max(dsrc[i], 0) * (K / 32) + c * 4);
        }
    };

    f32x4_t acc[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) acc[cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](const Slot& sl) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            half8_t af;
            f32x4_t sx;
            if (!EXACT) {
                const u32x4_t av = avalid ? sl.A[g] : u32x4_t{0u, 0u, 0u, 0u};
                af = __builtin_bit_cast(half8_t, F16P ? av : bf16x8_to_f16_perm(av));
            } else {
                af = __builtin_bit_cast(half8_t, i8x8_to_f16_perm(avalid ? sl.A[g][0] : 0u, avalid ? sl.A[g][1] : 0u));
#pragma unroll
                for (int i = 0; i < 4; ++i) sx[i] = dsrc[i] >= 0 ? sl.SX[i][g] : 0.0f;
            }
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) {
                half2_t s2, c2;
                scale_pair(sl.S[cb][g >> 1] >> (16 * (g & 1)), s2, c2);
                const half8_t bf = dequant8(sl.B[cb][g], s2, c2);
                if (!EXACT) {
                    acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bf, acc[cb], 0, 0, 0);
                } else {
                    const f32x4_t d = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bf, f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[cb][i] = __builtin_fmaf(d[i], sx[i], acc[cb][i]);
                }
            }
        }
    };

    // D chunk slots: chunk c+i lives in slot i of the iteration starting at c.
    Slot sl[D];
#pragma unroll
    for (int i = 0; i < D - 1; ++i) load(min(i, nch - 1), sl[i]);
    __builtin_amdgcn_sched_barrier(0);
    int c = 0;
    for (; c + D <= nch; c += D) {
#pragma unroll
        for (int i = 0; i < D; ++i) {
            load(min(c + i + D - 1, nch - 1), sl[(i + D - 1) % D]);
            __builtin_amdgcn_sched_barrier(0);
            compute(sl[i]);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#pragma unroll
    for (int i = 0; i < D - 1; ++i)
        if (c + i < nch) compute(sl[i]);

    // epilogue (rows 4j+i of the lane)
    if (GATEUP) {
        const int grp = n0 / 32;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int rl = 4 * j + i;
            const bool ok = rl < ti.rows;
            const size_t orow = (size_t)(ti.row0 + rl);
            if (!EXACT) {
#pragma unroll
                for (int p = 0; p < 2; ++p) {
                    const uint32_t v = bf16x2_bits(acc[p][i], acc[2 + p][i]);
                    const float g = __uint_as_float(v << 16), u = __uint_as_float(v & 0xFFFF0000u);
                    const uint32_t ab = bf16x2_bits(silu_fast(g), 0.0f) & 0xFFFFu;
                    const uint32_t hb = bf16x2_bits(__uint_as_float(ab << 16) * u, 0.0f) & 0xFFFFu;
                    if (ok) store_h<F16P>(a.out, orow * N, n0 + 16 * p + r, hb);
                }
            } else {
                const float h0 = moe_silu(acc[0][i]) * acc[2][i];
                const float h1 = moe_silu(acc[1][i]) * acc[3][i];
                float amax = fmaxf(fabsf(h0), fabsf(h1));
#pragma unroll
                for (int off = 1; off < 16; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
                const float s = (amax == 0.0f) ? 0.0f : amax / 127.0f;
                if (ok) {
                    int8_t* o = static_cast<int8_t*>(a.out) + orow * N + n0 + r;
                    o[0] = (int8_t)moe_quant_i8(h0, s);
                    o[16] = (int8_t)moe_quant_i8(h1, s);
                    if (r == 0) a.out_scale[orow * (N / 32) + grp] = s;
                }
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int rl = 4 * j + i;
            if (rl >= ti.rows) continue;
            const size_t orow = (size_t)(ti.row0 + rl);
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) {
                const int col = n0 + 16 * cb + r;
                if (!EXACT)
                    static_cast<uint16_t*>(a.out)[orow * N + col] = (uint16_t)f32_to_bf16_bits(acc[cb][i]);
                else
                    static_cast<float*>(a.out)[orow * N + col] = acc[cb][i];
            }
        }
    }
}

// Checkpoint layout -> fragment layout.  One thread per 16-byte lane piece of
// a weight fragment (fragment = (row group, chunk) in row-group-major order;
// 16 row groups of consecutive rows per expert, experts consecutive).
__global__ __launch_bounds__(256) void k_prepack_w(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                                  long pieces, int K) {
    const long t = (long)blockIdx.x * 256 + threadIdx.x;
    if (t >= pieces) return;
    const int nch = K / kKC;
    const int l = (int)(t & 63);
    const long fid = t >> 6;
    const long rg = fid / nch;
    const int c = (int)(fid % nch);
    const int r = l & 15, j = l >> 4;
    const uint8_t* row = src + (size_t)(rg * 16 + r) * (size_t)(K / 2) + 64 * c + 4 * j;
    u32x4_t v;
#pragma unroll
    for (int g = 0; g < 4; ++g) v[g] = *reinterpret_cast<const uint32_t*>(row + 16 * g);
    *reinterpret_cast<u32x4_t*>(dst + (size_t)t * 16) = v;
}

// One thread per (fragment, row): the row's 4 group scales of the chunk, converted
// to fp16 (the operand format of the dequantisation).
__global__ __launch_bounds__(256) void k_prepack_s(const uint16_t* __restrict__ src, uint16_t* __restrict__ dst,
                                                  long pieces, int K) {
    const long t = (long)blockIdx.x * 256 + threadIdx.x;
    if (t >= pieces) return;
    const int nch = K / kKC;
    const int r = (int)(t & 15);
    const long fid = t >> 4;
    const long rg = fid / nch;
    const int c = (int)(fid % nch);
    const u32x2_t v = *reinterpret_cast<const u32x2_t*>(src + (size_t)(rg * 16 + r) * (size_t)(K / 32) + 4 * c);
    // bf16 -> fp16 (round to nearest even; exact for the scales moe_int4_check_scales accepts)
    u32x2_t o;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const _Float16 lo = (_Float16)bf16_bits_to_f32(v[h] & 0xFFFFu);
        const _Float16 hi = (_Float16)bf16_bits_to_f32(v[h] >> 16);
        o[h] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
    }
    *reinterpret_cast<u32x2_t*>(dst + (size_t)t * 4) = o;
}

// Scale range check: a bf16 scale keeps the fp16 dequantisation exact when it
// is zero or its magnitude lies in [2^-14, 2^9] (bf16 bits 0x3880..0x4400).
__device__ __forceinline__ bool scale_in_range(uint32_t bits) {
    const uint32_t a = bits & 0x7FFFu;
    return a == 0 || (a >= 0x3880u && a <= 0x4400u);
}

__global__ __launch_bounds__(64) void k_zero_count(int32_t* __restrict__ count) {
    if (threadIdx.x == 0) count[0] = 0;
}

// Counts the out-of-range scales: one ballot per wave and step, one atomic add
// per wave at the end.
__global__ __launch_bounds__(256) void k_count_bad_scales(const uint16_t* __restrict__ scale, long n,
                                                         int32_t* __restrict__ count) {
    const long stride = (long)gridDim.x * 256;
    int bad = 0;
    for (long i = (long)blockIdx.x * 256 + threadIdx.x; i - threadIdx.x % MOE_WAVE < n; i += stride) {
        const bool b = i < n && !scale_in_range(scale[i]);
        bad += __popcll(__ballot(b));
    }
    if (lane_id() == 0 && bad) atomicAdd(count, bad);
}

// Activations into the fp16 staging format: one 8-element block per thread.
__global__ __launch_bounds__(256) void k_act_f16p(const u32x4_t* __restrict__ x, u32x4_t* __restrict__ out, long blocks) {
    const long i = (long)blockIdx.x * 256 + threadIdx.x;
    if (i < blocks) out[i] = bf16x8_to_f16_perm(x[i]);
}

// chunk slots of the decode kernel (D-1 chunks in flight): with the
// non-temporal weight loads, more waves per SIMD beat a deeper ring per wave
// (measured: 4 slots, two waves per SIMD < 3 slots, three < 2 slots)
constexpr int kSkinnyDepth = 2;
constexpr int kSkinnyDepthExact = 3;  // exact mode carries the activation scales too

// Rows per tile: the smallest tile that holds an average expert segment with
// some margin (segments split into balanced tiles, so most tiles run full).
int pick_mb(int S, int E) {
    const double avg = (double)S / (double)E;
    if (avg <= 12.0) return 1;
    const double need = 1.15 * avg;
    if (need <= 32.0) return 2;
    if (need <= 64.0) return 4;
    if (need <= 96.0) return 6;
    if (need <= 128.0) return 8;
    return 12;
}

// Column blocks per wave of the bf16 tile kernel: 2 for the 6-block tiles, whose
// accumulators then leave room for more than one workgroup per CU, else 4.
constexpr int pick_cb(int mb) { return mb == 6 ? 2 : 4; }

template <int MODE, int OP, int MB, int CB>
void launch_tiles(GroupedArgs a, int S, hipStream_t st) {
    a.n_chunks = OP == 0 ? a.N / (32 * CB) : a.N / (64 * CB);
    const long tiles = ((long)S + (long)a.E * (16 * MB - 1)) / (16 * MB) + 1;
    const dim3 grid(8 * moe::per_xcd(tiles * a.n_chunks));
    if constexpr (MODE == MOE_MODE_EXACT_I8 || MODE == MOE_MODE_EXACT_I16)
        hipLaunchKernelGGL((k_grouped_exact<MODE, OP, MB, CB>), grid, dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL((k_grouped<MODE, OP, MB, CB>), grid, dim3(256), 0, st, a);
}

template <int MODE, int OP, int M32>
void launch_tiles32(GroupedArgs a, int S, hipStream_t st) {
    a.n_chunks = OP == 0 ? a.N / 128 : a.N / 256;
    const long tiles = ((long)S + (long)a.E * (32 * M32 - 1)) / (32 * M32) + 1;
    const dim3 grid(8 * moe::per_xcd(tiles * a.n_chunks));
    if constexpr (MODE == MOE_MODE_BF16_F16P)
        hipLaunchKernelGGL((k_grouped32_dma<OP, M32>), grid, dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL((k_grouped32<OP, M32, false>), grid, dim3(256), 0, st, a);
}

template <int MODE, int OP>
int launch_grouped(GroupedArgs& a, int S, hipStream_t st, const char* what) {
    // exact mode keeps its accumulators in VGPRs (the group folds are VALU work)
    // and carries the s_x tile: at most 4 row blocks; with 16-bit activations
    // (two operand planes) always 2, whatever the batch
    if constexpr (MODE == MOE_MODE_EXACT_I16) {
        launch_tiles<MODE, OP, 2, 4>(a, S, st);
    } else {
        constexpr bool EXACT = MODE == MOE_MODE_EXACT_I8;
        const int mb = EXACT ? min(pick_mb(S, a.E), 4) : pick_mb(S, a.E);
        if (mb == 1) {
            a.n_chunks = OP == 0 ? a.N / 128 : a.N / 256;
            const long tiles = ((long)S + (long)a.E * 15) / 16 + 1;
            hipLaunchKernelGGL((k_grouped_skinny<MODE, OP, EXACT ? kSkinnyDepthExact : kSkinnyDepth>),
                               dim3(8 * moe::per_xcd(tiles * a.n_chunks)), dim3(256), 0, st, a);
            return moe::launch_status(what);
        }
        if constexpr (EXACT) {
            if (mb == 2) launch_tiles<MODE, OP, 2, 4>(a, S, st);
            else launch_tiles<MODE, OP, 4, 4>(a, S, st);
        } else {
            switch (mb) {
            case 2: launch_tiles<MODE, OP, 2, pick_cb(2)>(a, S, st); break;
            case 4: launch_tiles<MODE, OP, 4, pick_cb(4)>(a, S, st); break;
            case 6: launch_tiles<MODE, OP, 6, pick_cb(6)>(a, S, st); break;
            default: {
                // the 32x32 kernel addresses activation rows with 32-bit byte offsets
                const size_t act_rows = OP == 0 ? (size_t)S / (size_t)a.k : (size_t)S;
                const size_t act_bytes = act_rows * (size_t)a.K * 2;
                a.act_bytes = (uint32_t)act_bytes;
                if (act_bytes >= ((size_t)1 << 32)) launch_tiles<MODE, OP, 6, pick_cb(6)>(a, S, st);
                else if (mb == 8) launch_tiles32<MODE, OP, 4>(a, S, st);
                else launch_tiles32<MODE, OP, 6>(a, S, st);
                break;
            }
            }
        }
    }
    return moe::launch_status(what);
}

// The kernels address one expert's packed matrix (N x K/2 bytes) with 32-bit
// byte counts and int offsets: it must stay below 2 GiB.
bool expert_fits_offsets(int N, int K) { return (size_t)N * (size_t)(K / 2) < ((size_t)1 << 31); }

int check_common(const char* what, int mode, int T, int k, int E) {
    using namespace moe;
    if (mode != MOE_MODE_BF16 && mode != MOE_MODE_EXACT_I8 && mode != MOE_MODE_BF16_F16P &&
        mode != MOE_MODE_EXACT_I16)
        return fail(MOE_ERR_INVALID_ARG, "%s: mode %d", what, mode);
    if (T < 0 || k <= 0 || E <= 0) return fail(MOE_ERR_INVALID_ARG, "%s: bad sizes", what);
    if (E > 1024 || k > 16 || k > E || (long)T * k >= (1L << 31))
        return fail(MOE_ERR_UNSUPPORTED, "%s: E=%d k=%d T=%d outside limits", what, E, k, T);
    return MOE_OK;
}

}  // namespace

extern "C" int moe_int4_grouped_swiglu(int mode, const void* act, const float* act_scale,
                                       const uint8_t* gate_packed, const uint16_t* gate_scale,
                                       const uint8_t* up_packed, const uint16_t* up_scale,
                                       const int32_t* offsets, const int32_t* sorted_slot, int T,
                                       int k, int E, int H, int I, void* h, float* h_scale,
                                       void* stream) {
    using namespace moe;
    const char* what = "moe_int4_grouped_swiglu";
    if (int rc = check_common(what, mode, T, k, E)) return rc;
    if (H <= 0 || I <= 0 || H % kKC != 0 || I % 128 != 0)
        return fail(MOE_ERR_UNSUPPORTED, "%s: H=%d (multiple of 128) I=%d (multiple of 128)", what, H, I);
    if (!expert_fits_offsets(I, H))
        return fail(MOE_ERR_UNSUPPORTED, "%s: one expert's %d x %d matrix is 2 GiB or more", what, I, H);
    if (T == 0) return MOE_OK;
    if (!act || !gate_packed || !gate_scale || !up_packed || !up_scale || !offsets || !sorted_slot || !h)
        return fail(MOE_ERR_INVALID_ARG, "%s: null pointer", what);
    const bool exact = mode == MOE_MODE_EXACT_I8 || mode == MOE_MODE_EXACT_I16;
    if (exact && (!act_scale || !h_scale))
        return fail(MOE_ERR_INVALID_ARG, "%s: exact mode needs act_scale and h_scale", what);
    if (!exact && (act_scale || h_scale))
        return fail(MOE_ERR_INVALID_ARG, "%s: bf16 mode takes no scales", what);
    if (!aligned16(act) || !aligned16(gate_packed) || !aligned16(up_packed) ||
        (exact && !aligned16(act_scale)))
        return fail(MOE_ERR_INVALID_ARG, "%s: activations and packed weights must be 16-byte aligned", what);
    GroupedArgs a{};
    a.act = act;
    a.act_scale = act_scale;
    a.w0 = gate_packed;
    a.s0 = gate_scale;
    a.w1 = up_packed;
    a.s1 = up_scale;
    a.offsets = offsets;
    a.sorted_slot = sorted_slot;
    a.k = k;
    a.E = E;
    a.K = H;
    a.N = I;
    a.out = h;
    a.out_scale = h_scale;
    hipStream_t st = as_stream(stream);
    if (mode == MOE_MODE_EXACT_I16) return launch_grouped<MOE_MODE_EXACT_I16, 0>(a, T * k, st, what);
    if (exact) return launch_grouped<MOE_MODE_EXACT_I8, 0>(a, T * k, st, what);
    if (mode == MOE_MODE_BF16_F16P) return launch_grouped<MOE_MODE_BF16_F16P, 0>(a, T * k, st, what);
    return launch_grouped<MOE_MODE_BF16, 0>(a, T * k, st, what);
}

extern "C" int moe_int4_grouped_down(int mode, const void* h, const float* h_scale,
                                     const uint8_t* down_packed, const uint16_t* down_scale,
                                     const int32_t* offsets, int T, int k, int E, int I, int H,
                                     void* y, void* stream) {
    using namespace moe;
    const char* what = "moe_int4_grouped_down";
    if (int rc = check_common(what, mode, T, k, E)) return rc;
    if (H <= 0 || I <= 0 || I % kKC != 0 || H % 256 != 0)
        return fail(MOE_ERR_UNSUPPORTED, "%s: I=%d (multiple of 128) H=%d (multiple of 256)", what, I, H);
    if (!expert_fits_offsets(H, I))
        return fail(MOE_ERR_UNSUPPORTED, "%s: one expert's %d x %d matrix is 2 GiB or more", what, H, I);
    if (T == 0) return MOE_OK;
    if (!h || !down_packed || !down_scale || !offsets || !y)
        return fail(MOE_ERR_INVALID_ARG, "%s: null pointer", what);
    const bool exact = mode == MOE_MODE_EXACT_I8 || mode == MOE_MODE_EXACT_I16;
    if (exact && !h_scale) return fail(MOE_ERR_INVALID_ARG, "%s: exact mode needs h_scale", what);
    if (!exact && h_scale) return fail(MOE_ERR_INVALID_ARG, "%s: bf16 mode takes no scales", what);
    if (!aligned16(h) || !aligned16(down_packed) || (exact && !aligned16(h_scale)))
        return fail(MOE_ERR_INVALID_ARG, "%s: activations and packed weights must be 16-byte aligned", what);
    GroupedArgs a{};
    a.act = h;
    a.act_scale = h_scale;
    a.w0 = down_packed;
    a.s0 = down_scale;
    a.offsets = offsets;
    a.k = k;
    a.E = E;
    a.K = I;
    a.N = H;
    a.out = y;
    hipStream_t st = as_stream(stream);
    if (mode == MOE_MODE_EXACT_I16) return launch_grouped<MOE_MODE_EXACT_I16, 1>(a, T * k, st, what);
    if (exact) return launch_grouped<MOE_MODE_EXACT_I8, 1>(a, T * k, st, what);
    if (mode == MOE_MODE_BF16_F16P) return launch_grouped<MOE_MODE_BF16_F16P, 1>(a, T * k, st, what);
    return launch_grouped<MOE_MODE_BF16, 1>(a, T * k, st, what);
}

extern "C" int moe_act_f16p(const uint16_t* x, int rows, int K, uint16_t* out, void* stream) {
    using namespace moe;
    const char* what = "moe_act_f16p";
    if (rows < 0 || K <= 0) return fail(MOE_ERR_INVALID_ARG, "%s: bad sizes rows=%d K=%d", what, rows, K);
    if (K % 8 != 0) return fail(MOE_ERR_UNSUPPORTED, "%s: K=%d (multiple of 8)", what, K);
    if (rows == 0) return MOE_OK;
    if (!x || !out) return fail(MOE_ERR_INVALID_ARG, "%s: null pointer", what);
    if (!aligned16(x) || !aligned16(out)) return fail(MOE_ERR_INVALID_ARG, "%s: buffers must be 16-byte aligned", what);
    const char* xb = reinterpret_cast<const char*>(x);
    const char* ob = reinterpret_cast<const char*>(out);
    const size_t bytes = (size_t)rows * (size_t)K * 2;
    if (xb < ob + bytes && ob < xb + bytes) return fail(MOE_ERR_INVALID_ARG, "%s: input and output overlap", what);
    const long blocks = (long)rows * (K / 8);
    hipLaunchKernelGGL(k_act_f16p, dim3((unsigned)((blocks + 255) / 256)), dim3(256), 0, as_stream(stream),
                       reinterpret_cast<const u32x4_t*>(x), reinterpret_cast<u32x4_t*>(out), blocks);
    return launch_status(what);
}

extern "C" int moe_int4_check_scales(const uint16_t* scale, size_t n, int32_t* count, void* stream) {
    using namespace moe;
    const char* what = "moe_int4_check_scales";
    if (n == 0) return MOE_OK;
    if (!scale || !count) return fail(MOE_ERR_INVALID_ARG, "%s: null pointer", what);
    if ((reinterpret_cast<uintptr_t>(scale) & 1) || (reinterpret_cast<uintptr_t>(count) & 3))
        return fail(MOE_ERR_INVALID_ARG, "%s: misaligned pointer", what);
    hipStream_t st = as_stream(stream);
    hipLaunchKernelGGL(k_zero_count, dim3(1), dim3(64), 0, st, count);
    if (int rc = launch_status(what)) return rc;
    const long blocks = std::min<long>(2048, ((long)n + 255) / 256);
    hipLaunchKernelGGL(k_count_bad_scales, dim3((unsigned)blocks), dim3(256), 0, st, scale, (long)n, count);
    if (int rc = launch_status(what)) return rc;
    int32_t host = 0;
    hipError_t e = hipMemcpyAsync(&host, count, sizeof host, hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return fail(MOE_ERR_LAUNCH, "%s: %s", what, hipGetErrorString(e));
    if (host != 0)
        return fail(MOE_ERR_UNSUPPORTED, "%s: %d of %zu scales are neither 0 nor of magnitude in [2^-14, 2^9]", what,
                    host, n);
    return MOE_OK;
}

extern "C" int moe_int4_prepack(const uint8_t* packed, const uint16_t* scale, int E, int N, int K,
                                uint8_t* packed_out, uint16_t* scale_out, void* stream) {
    using namespace moe;
    const char* what = "moe_int4_prepack";
    if (E < 0 || N <= 0 || K <= 0) return fail(MOE_ERR_INVALID_ARG, "%s: bad sizes E=%d N=%d K=%d", what, E, N, K);
    if (N % 16 != 0 || K % kKC != 0)
        return fail(MOE_ERR_UNSUPPORTED, "%s: N=%d (multiple of 16) K=%d (multiple of 128)", what, N, K);
    if (E == 0) return MOE_OK;
    if (!packed || !scale || !packed_out || !scale_out) return fail(MOE_ERR_INVALID_ARG, "%s: null pointer", what);
    if (!aligned16(packed) || !aligned16(packed_out) || (reinterpret_cast<uintptr_t>(scale) & 7) ||
        (reinterpret_cast<uintptr_t>(scale_out) & 7))
        return fail(MOE_ERR_INVALID_ARG, "%s: packed buffers 16-byte, scale buffers 8-byte aligned", what);
    const size_t wbytes = (size_t)E * N * (K / 2), sbytes = (size_t)E * N * (K / 32) * 2;
    const uintptr_t pi = reinterpret_cast<uintptr_t>(packed), po = reinterpret_cast<uintptr_t>(packed_out);
    const uintptr_t si = reinterpret_cast<uintptr_t>(scale), so = reinterpret_cast<uintptr_t>(scale_out);
    if ((pi < po + wbytes && po < pi + wbytes) || (si < so + sbytes && so < si + sbytes))
        return fail(MOE_ERR_INVALID_ARG, "%s: output overlaps input (the permutation is out of place)", what);
    hipStream_t st = as_stream(stream);
    const long wp = (long)(wbytes / 16), sp = (long)(sbytes / 8);
    hipLaunchKernelGGL(k_prepack_w, dim3((unsigned)((wp + 255) / 256)), dim3(256), 0, st, packed, packed_out, wp, K);
    if (int rc = launch_status(what)) return rc;
    hipLaunchKernelGGL(k_prepack_s, dim3((unsigned)((sp + 255) / 256)), dim3(256), 0, st, scale, scale_out, sp, K);
    return launch_status(what);
}
