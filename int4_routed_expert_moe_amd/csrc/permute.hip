// Stable permutation of the (token, slot) pairs by expert ("Kimi-K3 latent
// MoE" page, Code: moe_infer counts assignments per expert, argsorts the
// flattened expert ids and walks the experts with start/end indices; "Kimi
// K2.5 donor reference", records "DeepSeek MoE.moe_infer: tokens per
// expert", "sorted tokens", "start idx").
//
// A stable counting sort replaces the host-side count/argsort/.cpu() walk.
// The slot list is cut into contiguous ranges; every range counts its experts
// (LDS atomics: counts are order-free), each range's first position per
// expert is offsets[e] plus the counts of the ranges before it, and each wave
// then walks its range 64 slots at a time in slot order: lanes with equal
// experts find each other with ballots over the expert id bits, so a slot's
// position is its range's base + the number of earlier equal lanes, and the
// order inside an expert is the slot order (stable, deterministic).
//
// Few slots: one workgroup of 16 waves, one range per wave.  Many slots
// (kPermBlocksMinS and up): blocks of kPermBlock slots, three launches:
//   1. k_perm_block_counts: per block, the expert counts -> hist[b][e];
//   2. k_perm_scan: counts, offsets, and hist[b][e] turned into the block's
//      first position per expert (one workgroup; blocks in order per expert);
//   3. k_perm_block_scatter: per block, 4 waves with the single-workgroup
//      scheme inside the block, starting from the block's first positions.
#include <mutex>

#include "moe_common.h"

// Per-block count buffer of moe_permute_noalloc: a fixed device array (every
// GPU the library runs on holds its own copy until the process ends).  Host
// code reaches it only through the address hipGetSymbolAddress returns for
// the current device; the array's name on the host is not a device address.
constexpr long kNoAllocHistInts = 1L << 18;  // 1 MiB: blocks x E <= 262144
static __device__ __align__(256) int32_t scratch[kNoAllocHistInts];

namespace {

constexpr int kPermWaves = 16;             // single-workgroup path
constexpr int kPermMaxE = 1024;
constexpr int kPermBlock = 1024;           // slots per block of the multi-block path
constexpr int kPermBlockWaves = 4;         // waves per block
constexpr long kPermBlocksMinS = 16384;    // slots from which the multi-block path runs

__device__ __forceinline__ int expert_bits(int E) {
    int nbits = 0;
    while ((1 << nbits) < E) ++nbits;
    return nbits;
}

// This wave's slots [r0, r1) counted into its LDS row.
__device__ __forceinline__ void count_range(const int32_t* __restrict__ topk_idx, int r0, int r1, int32_t* cnt_row) {
    for (int f = r0 + lane_id(); f < r1; f += MOE_WAVE) atomicAdd(&cnt_row[topk_idx[f]], 1);
}

// Stable scatter of this wave's slots [r0, r1), 64 at a time in slot order;
// base_row[e] (LDS, this wave's own row) is the next position of expert e and
// is advanced in place.
__device__ __forceinline__ void scatter_range(const int32_t* __restrict__ topk_idx, int r0, int r1, int nbits,
                                              int32_t* base_row, int32_t* __restrict__ sorted_slot,
                                              int32_t* __restrict__ slot_pos) {
    const int lane = lane_id();
    for (int f0 = r0; f0 < r1; f0 += MOE_WAVE) {
        const int f = f0 + lane;
        const bool valid = f < r1;
        const int e = valid ? topk_idx[f] : 0;
        uint64_t same = __ballot(valid);
        for (int b = 0; b < nbits; ++b) {
            const uint64_t ones = __ballot(valid && ((e >> b) & 1));
            same &= ((e >> b) & 1) ? ones : ~ones;
        }
        const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (MOE_WAVE - lane));
        const int rank = __popcll(same & below);
        const int grp = __popcll(same);
        int pos = 0;
        if (valid) {
            pos = base_row[e] + rank;
            sorted_slot[pos] = f;
            slot_pos[f] = pos;
        }
        // every lane has read its base; the last lane of each group advances it
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
        if (valid && rank == grp - 1) base_row[e] = pos + 1;
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
    }
}

// Exclusive scan of v over the threads of a 1024-thread workgroup (Hillis-Steele
// in LDS); every thread calls it.
__device__ __forceinline__ int block_exclusive_scan(int v, int32_t* scan) {
    const int tid = threadIdx.x;
    scan[tid] = v;
    __syncthreads();
    for (int d = 1; d < kPermMaxE; d <<= 1) {
        const int u = (tid >= d) ? scan[tid - d] : 0;
        __syncthreads();
        scan[tid] += u;
        __syncthreads();
    }
    return scan[tid] - v;
}

__global__ __launch_bounds__(1024) void k_permute(const int32_t* __restrict__ topk_idx, int S, int E,
                                                  int32_t* __restrict__ counts,
                                                  int32_t* __restrict__ offsets,
                                                  int32_t* __restrict__ sorted_slot,
                                                  int32_t* __restrict__ slot_pos) {
    __shared__ int32_t cnt[kPermWaves][kPermMaxE];
    __shared__ int32_t scan[kPermMaxE];
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int per_wave = (S + kPermWaves - 1) / kPermWaves;
    const int r0 = min(S, wave * per_wave);
    const int r1 = min(S, r0 + per_wave);

    for (int i = tid; i < kPermWaves * kPermMaxE; i += blockDim.x) (&cnt[0][0])[i] = 0;
    __syncthreads();
    count_range(topk_idx, r0, r1, cnt[wave]);
    __syncthreads();

    // per expert e = tid: totals and the per-wave running prefix
    int total = 0;
    if (tid < E) {
        for (int w = 0; w < kPermWaves; ++w) {
            const int c = cnt[w][tid];
            cnt[w][tid] = total;  // exclusive prefix over waves
            total += c;
        }
        counts[tid] = total;
    }
    const int excl = block_exclusive_scan(tid < E ? total : 0, scan);
    if (tid < E) {
        offsets[tid] = excl;
        for (int w = 0; w < kPermWaves; ++w) cnt[w][tid] += excl;
    }
    if (tid == 0) offsets[E] = S;
    __syncthreads();

    scatter_range(topk_idx, r0, r1, expert_bits(E), cnt[wave], sorted_slot, slot_pos);
}

// 1. hist[b][e] = number of slots of block b routed to expert e.
__global__ __launch_bounds__(256) void k_perm_block_counts(const int32_t* __restrict__ topk_idx, int S, int E,
                                                           int32_t* __restrict__ hist) {
    __shared__ int32_t cnt[kPermMaxE];
    const int tid = threadIdx.x;
    const int b = blockIdx.x;
    const int r0 = b * kPermBlock, r1 = min(S, r0 + kPermBlock);
    for (int e = tid; e < E; e += blockDim.x) cnt[e] = 0;
    __syncthreads();
    for (int f = r0 + tid; f < r1; f += blockDim.x) atomicAdd(&cnt[topk_idx[f]], 1);
    __syncthreads();
    for (int e = tid; e < E; e += blockDim.x) hist[(size_t)b * E + e] = cnt[e];
}

// 2. counts[e] = sum over blocks; offsets = exclusive scan over experts;
//    hist[b][e] <- offsets[e] + sum_{b' < b} hist[b'][e] (thread e walks the
//    blocks in order).
__global__ __launch_bounds__(1024) void k_perm_scan(int32_t* __restrict__ hist, int nb, int S, int E,
                                                    int32_t* __restrict__ counts, int32_t* __restrict__ offsets) {
    __shared__ int32_t scan[kPermMaxE];
    const int e = threadIdx.x;
    int total = 0;
    if (e < E) {
        for (int b = 0; b < nb; ++b) {
            const int c = hist[(size_t)b * E + e];
            hist[(size_t)b * E + e] = total;
            total += c;
        }
        counts[e] = total;
    }
    const int excl = block_exclusive_scan(e < E ? total : 0, scan);
    if (e < E) {
        offsets[e] = excl;
        for (int b = 0; b < nb; ++b) hist[(size_t)b * E + e] += excl;
    }
    if (e == 0) offsets[E] = S;
}

// 3. Block b's slots in 4 contiguous wave ranges, each wave's first position per
//    expert = the block's (hist[b][e]) + the counts of the block's earlier waves.
__global__ __launch_bounds__(256) void k_perm_block_scatter(const int32_t* __restrict__ topk_idx, int S, int E,
                                                            const int32_t* __restrict__ hist,
                                                            int32_t* __restrict__ sorted_slot,
                                                            int32_t* __restrict__ slot_pos) {
    __shared__ int32_t cnt[kPermBlockWaves][kPermMaxE];
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int b = blockIdx.x;
    const int b0 = b * kPermBlock, b1 = min(S, b0 + kPermBlock);
    const int per_wave = (b1 - b0 + kPermBlockWaves - 1) / kPermBlockWaves;
    const int r0 = min(b1, b0 + wave * per_wave);
    const int r1 = min(b1, r0 + per_wave);
    for (int i = tid; i < kPermBlockWaves * kPermMaxE; i += blockDim.x) (&cnt[0][0])[i] = 0;
    __syncthreads();
    count_range(topk_idx, r0, r1, cnt[wave]);
    __syncthreads();
    for (int e = tid; e < E; e += blockDim.x) {
        int running = hist[(size_t)b * E + e];
        for (int w = 0; w < kPermBlockWaves; ++w) {
            const int c = cnt[w][e];
            cnt[w][e] = running;
            running += c;
        }
    }
    __syncthreads();
    scatter_range(topk_idx, r0, r1, expert_bits(E), cnt[wave], sorted_slot, slot_pos);
}

long perm_blocks(long S) { return S >= kPermBlocksMinS ? (S + kPermBlock - 1) / kPermBlock : 0; }

// Host-side checks shared by both permutation entry points.
int check_permute(const char* what, const int32_t* topk_idx, int T, int k, int E, const int32_t* counts,
                  const int32_t* offsets, const int32_t* sorted_slot, const int32_t* slot_pos) {
    using namespace moe;
    if (T < 0 || k <= 0 || E <= 0) return fail(MOE_ERR_INVALID_ARG, "%s: bad sizes T=%d k=%d E=%d", what, T, k, E);
    if (E > kPermMaxE || k > 16 || (long)T * k >= (1L << 31))
        return fail(MOE_ERR_UNSUPPORTED, "%s: E=%d k=%d T=%d outside limits", what, E, k, T);
    if (!counts || !offsets) return fail(MOE_ERR_INVALID_ARG, "%s: null pointer", what);
    if (T > 0 && (!topk_idx || !sorted_slot || !slot_pos)) return fail(MOE_ERR_INVALID_ARG, "%s: null pointer", what);
    return MOE_OK;
}

// The launches of both entry points; hist is the per-block count buffer
// (unused below kPermBlocksMinS slots).
int launch_permute(const char* what, const int32_t* topk_idx, int S, int E, int32_t* counts, int32_t* offsets,
                   int32_t* sorted_slot, int32_t* slot_pos, int32_t* hist, hipStream_t st) {
    using namespace moe;
    const long nb = perm_blocks(S);
    if (nb == 0) {
        hipLaunchKernelGGL(k_permute, dim3(1), dim3(1024), 0, st, topk_idx, S, E, counts, offsets, sorted_slot,
                           slot_pos);
        return launch_status(what);
    }
    hipLaunchKernelGGL(k_perm_block_counts, dim3((unsigned)nb), dim3(256), 0, st, topk_idx, S, E, hist);
    if (int rc = launch_status(what)) return rc;
    hipLaunchKernelGGL(k_perm_scan, dim3(1), dim3(1024), 0, st, hist, (int)nb, S, E, counts, offsets);
    if (int rc = launch_status(what)) return rc;
    hipLaunchKernelGGL(k_perm_block_scatter, dim3((unsigned)nb), dim3(256), 0, st, topk_idx, S, E, hist, sorted_slot,
                       slot_pos);
    return launch_status(what);
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
int32_t* g_scratch_dev[kMaxDevices] = {};

// The current device's copy of `scratch`, looked up once per device.
int scratch_for_current_device(const char* what, int32_t** out) {
    using namespace moe;
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(MOE_ERR_LAUNCH, "%s: hipGetDevice: %s", what, hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(MOE_ERR_UNSUPPORTED, "%s: device %d", what, dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(MOE_ERR_LAUNCH, "%s: hipGetSymbolAddress: %s", what, hipGetErrorString(e));
        g_scratch_dev[dev] = static_cast<int32_t*>(p);
    }
    *out = g_scratch_dev[dev];
    return MOE_OK;
}

}  // namespace

extern "C" size_t moe_permute_workspace_bytes(int T, int k, int E) {
    if (T <= 0 || k <= 0 || E <= 0) return 0;
    return (size_t)perm_blocks((long)T * k) * (size_t)E * sizeof(int32_t);
}

extern "C" int moe_permute(const int32_t* topk_idx, int T, int k, int E, int32_t* counts,
                           int32_t* offsets, int32_t* sorted_slot, int32_t* slot_pos, void* ws,
                           size_t ws_bytes, void* stream) {
    using namespace moe;
    const char* what = "moe_permute";
    if (int rc = check_permute(what, topk_idx, T, k, E, counts, offsets, sorted_slot, slot_pos)) return rc;
    const int S = T * k;
    if (perm_blocks(S) > 0) {
        const size_t need = moe_permute_workspace_bytes(T, k, E);
        if (!ws || ws_bytes < need)
            return fail(MOE_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", what, ws_bytes, need);
        if (!aligned16(ws)) return fail(MOE_ERR_INVALID_ARG, "%s: workspace must be 16-byte aligned", what);
    }
    return launch_permute(what, topk_idx, S, E, counts, offsets, sorted_slot, slot_pos, static_cast<int32_t*>(ws),
                          as_stream(stream));
}

extern "C" int moe_permute_noalloc(const int32_t* topk_idx, int T, int k, int E, int32_t* counts,
                                   int32_t* offsets, int32_t* sorted_slot, int32_t* slot_pos, void* stream) {
    using namespace moe;
    const char* what = "moe_permute_noalloc";
    if (int rc = check_permute(what, topk_idx, T, k, E, counts, offsets, sorted_slot, slot_pos)) return rc;
    const int S = T * k;
    const long nb = perm_blocks(S);
    if (nb * (long)E > kNoAllocHistInts)
        return fail(MOE_ERR_UNSUPPORTED, "%s: %d slots over %d experts need %ld count entries, more than the fixed %ld",
                    what, S, E, nb * (long)E, kNoAllocHistInts);
    int32_t* hist = nullptr;
    if (nb > 0) {
        if (int rc = scratch_for_current_device(what, &hist)) return rc;
    }
    return launch_permute(what, topk_idx, S, E, counts, offsets, sorted_slot, slot_pos, hist, as_stream(stream));
}
