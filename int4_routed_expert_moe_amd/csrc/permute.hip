// Stable permutation of the (token, slot) pairs by expert ("Kimi-K3 latent
// MoE" page, Code: moe_infer counts assignments per expert, argsorts the
// flattened expert ids and walks the experts with start/end indices; "Kimi
// K2.5 donor reference", records "DeepSeek MoE.moe_infer: tokens per
// expert", "sorted tokens", "start idx").
//
// One workgroup of 16 waves replaces the host-side count/argsort/.cpu() walk:
//   1. wave w owns the contiguous slot range R_w and counts its experts into
//      its own LDS row cnt[w][*] (LDS atomics: the counts are order-free);
//   2. per expert: counts, the exclusive scan over experts (offsets), and each
//      wave's first position base[w][e] = offsets[e] + sum_{w' < w} cnt[w'][e];
//   3. each wave walks its range 64 slots at a time in slot order; lanes with
//      equal experts find each other with ballots over the expert id bits, so
//      a slot's position is base + (number of earlier equal lanes) and the
//      order inside an expert is the slot order (stable, deterministic).
#include "moe_common.h"

namespace {

constexpr int kPermWaves = 16;
constexpr int kPermMaxE = 1024;

__global__ __launch_bounds__(1024) void k_permute(const int32_t* __restrict__ topk_idx, int S, int E,
                                                  int32_t* __restrict__ counts,
                                                  int32_t* __restrict__ offsets,
                                                  int32_t* __restrict__ sorted_slot,
                                                  int32_t* __restrict__ slot_pos) {
    __shared__ int32_t cnt[kPermWaves][kPermMaxE];
    __shared__ int32_t scan[kPermMaxE];
    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wave = tid >> 6;
    const int per_wave = (S + kPermWaves - 1) / kPermWaves;
    const int r0 = min(S, wave * per_wave);
    const int r1 = min(S, r0 + per_wave);

    for (int i = tid; i < kPermWaves * kPermMaxE; i += blockDim.x) (&cnt[0][0])[i] = 0;
    __syncthreads();
    for (int f = r0 + lane; f < r1; f += MOE_WAVE) atomicAdd(&cnt[wave][topk_idx[f]], 1);
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
    // exclusive scan of totals over experts (Hillis-Steele in LDS)
    scan[tid] = (tid < E) ? total : 0;
    __syncthreads();
    for (int d = 1; d < kPermMaxE; d <<= 1) {
        const int v = (tid >= d) ? scan[tid - d] : 0;
        __syncthreads();
        scan[tid] += v;
        __syncthreads();
    }
    const int incl = scan[tid];
    const int excl = incl - ((tid < E) ? total : 0);
    if (tid < E) {
        offsets[tid] = excl;
        for (int w = 0; w < kPermWaves; ++w) cnt[w][tid] += excl;
    }
    if (tid == 0) offsets[E] = S;
    __syncthreads();

    // stable scatter
    int nbits = 0;
    while ((1 << nbits) < E) ++nbits;
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
            pos = cnt[wave][e] + rank;
            sorted_slot[pos] = f;
            slot_pos[f] = pos;
        }
        // every lane has read its base; the last lane of each group advances it
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
        if (valid && rank == grp - 1) cnt[wave][e] = pos + 1;
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
    }
}

}  // namespace

extern "C" int moe_permute(const int32_t* topk_idx, int T, int k, int E, int32_t* counts,
                           int32_t* offsets, int32_t* sorted_slot, int32_t* slot_pos, void* stream) {
    using namespace moe;
    if (T < 0 || k <= 0 || E <= 0)
        return fail(MOE_ERR_INVALID_ARG, "moe_permute: bad sizes T=%d k=%d E=%d", T, k, E);
    if (E > kPermMaxE || k > 16 || (long)T * k >= (1L << 31))
        return fail(MOE_ERR_UNSUPPORTED, "moe_permute: E=%d k=%d T=%d outside limits", E, k, T);
    if (!counts || !offsets) return fail(MOE_ERR_INVALID_ARG, "moe_permute: null pointer");
    if (T > 0 && (!topk_idx || !sorted_slot || !slot_pos))
        return fail(MOE_ERR_INVALID_ARG, "moe_permute: null pointer");
    hipLaunchKernelGGL(k_permute, dim3(1), dim3(1024), 0, as_stream(stream), topk_idx, T * k, E, counts,
                       offsets, sorted_slot, slot_pos);
    return launch_status("moe_permute");
}
