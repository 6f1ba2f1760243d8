/*
 * moe_int4.h -- C ABI of the MI355X (gfx950) int4 routed-expert MoE layer.
 *
 * The layer: sigmoid top-k routing with an fp32 correction bias, a stable
 * permutation of (token, slot) pairs by expert, per-expert SwiGLU MLPs whose
 * gate/up/down projections are packed signed int4 with one bf16 scale per 32
 * input elements, and a routing-weighted combine back into token order, plus
 * the dense pieces around it (bf16 shared expert, Kimi-K3 latent down/up
 * projections and RMSNorm).  Sources: "Kimi exact-generator adaptation"
 * (routed experts as PackedInt4Linear / ExactLinear, group size 32, shared
 * expert kept bf16), "Kimi K2.5 donor reference" (router records, moe_infer
 * records, SwiGLU, RMSNorm, shared expert) and "Kimi-K3 latent MoE: latent
 * up-projection" (moe_infer code, latent block, Parameters table).
 *
 * Conventions shared by every call
 *  - Every pointer argument is a DEVICE pointer unless stated otherwise, to a
 *    row-major contiguous array, aligned to 16 bytes.  bf16 tensors are passed
 *    as uint16_t bit patterns.  `stream` is a hipStream_t cast to void* (NULL =
 *    the default stream).  The caller owns every buffer; the library allocates
 *    no device memory, keeps no state between calls and never synchronises
 *    with the host.  Calls are asynchronous: they validate their arguments on
 *    the host, enqueue kernels on `stream` and return.
 *  - Return value: MOE_OK (0) or a negative moe_status.  A non-OK return
 *    enqueues nothing.  moe_status_string() gives static text and
 *    moe_last_error_detail() a thread-local description of the last failure
 *    on the calling thread.  Nothing is printed and no exception crosses the
 *    ABI.  A size of zero tokens/rows is a no-op returning MOE_OK.
 *  - Packed int4 weight of a [N, K] projection: `packed` is uint8 [N][K/2];
 *    byte b of row n holds element 2b in its low nibble and element 2b+1 in
 *    its high nibble; each nibble is a two's-complement integer in [-8, 7].
 *    `scale` is bf16 [N][K/32]; the weight is q * scale[n][i/32] (symmetric,
 *    no zero point).  A routed expert set stacks E such matrices:
 *    gate/up [E][I][H/2] + [E][I][H/32], down [E][H][I/2] + [E][H][I/32].
 *    This is the checkpoint layout.  The grouped expert GEMMs read the same
 *    bytes in the fragment layout made once by moe_int4_prepack (below).
 *  - Numerics of the routed GEMMs: operands are fp16 on the matrix cores.
 *    bf16 activations are converted rounding toward zero: magnitudes in
 *    [2^-14, 65504] convert exactly, smaller ones become fp16 subnormals
 *    (absolute error below 2^-24) and larger ones saturate to 65504; with
 *    the fp16 staging format (MOE_MODE_BF16_F16P) the same holds for h.
 *    bf16 scales must be 0 or of magnitude in [2^-14, 2^9], where q * s is
 *    exact in fp16; moe_int4_check_scales checks a scale tensor once at
 *    weight load.
 *  - Shape limits (else MOE_ERR_UNSUPPORTED): 1 <= k <= min(E, 16), E <= 1024,
 *    T*k < 2^31; H and I multiples of 128; expert-output widths (I for
 *    gate/up, H for down) multiples of 128 and 256 respectively; dense
 *    linear N a multiple of 64 and K a multiple of 128.
 */
#ifndef MOE_INT4_H
#define MOE_INT4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = -1, /* null pointer, misaligned pointer, negative size, bad mode */
    MOE_ERR_UNSUPPORTED = -2, /* shape outside the limits listed above */
    MOE_ERR_WORKSPACE = -3,   /* workspace missing or smaller than the *_workspace_bytes query */
    MOE_ERR_LAUNCH = -4,      /* the HIP runtime rejected a kernel launch */
} moe_status;

enum { MOE_MODE_BF16 = 0, MOE_MODE_EXACT_I8 = 1, MOE_MODE_BF16_F16P = 2, MOE_MODE_EXACT_I16 = 3 };

/* Version of this ABI (incremented on any signature change). */
int moe_abi_version(void);
/* Static text for a status code; never NULL. */
const char* moe_status_string(int status);
/* Thread-local detail of the last non-OK return on this thread ("" if none). */
const char* moe_last_error_detail(void);

/* ---------------------------------------------------------------------------
 * Routing.  "Kimi K2.5 donor reference", records "MoEGate.forward: logits",
 * "Independent sigmoid scores for the router", "Bias the choice of experts
 * while retaining original affinities", "MoEGate.forward: ( , topk idx)" and
 * "Normalize the selected routing affinities".
 *   l[t,e] = sum over 64-wide hidden blocks b (ascending, from 0) of
 *            the block sums (fp32, ascending index within the block, from 0)
 *   s = 1 / (1 + exp(-l))                   fp32, exp by the pinned
 *                                           Cody-Waite/Taylor-7 algorithm
 *   selection: the k largest s[t,e] + bias[e], ties to the lower e, in rank order
 *   topk_w[t,j] = s_sel / (sum_j s_sel + 1e-20)  (renormalize != 0; else s_sel)
 * x [T,H] bf16; w_router [E,H] bf16; bias [E] fp32;
 * out: topk_idx [T,k] int32, topk_w [T,k] fp32.
 * H a multiple of 64, k <= min(E, 16), E <= 1024, E*H*2 bytes below 4 GiB
 * (else MOE_ERR_UNSUPPORTED).
 * ws: device workspace of at least moe_route_workspace_bytes(T, H, E) bytes,
 * 16-byte aligned (it holds the fp32 logits and, for up to 256 tokens, the
 * 64-wide block sums).
 * Results are bit-exact and deterministic. */
size_t moe_route_workspace_bytes(int T, int H, int E);
int moe_route(const uint16_t* x, const uint16_t* w_router, const float* bias, int T, int H, int E,
              int k, int renormalize, int32_t* topk_idx, float* topk_w, void* ws, size_t ws_bytes,
              void* stream);

/* Group-limited routing ("Kimi K2.5 donor reference", MoEGate.forward records
 * "group scores", "group idx", "score mask", "( , topk idx)", "denominator";
 * the records name those steps without their code, so the reading is stated):
 * as moe_route, except that the E experts form n_group groups of E/n_group
 * consecutive indices; a group scores the sum of its two largest biased scores
 * s + bias (one fp32 add); the topk_group best groups are kept, ties to the
 * lower group; the k experts are selected among the kept groups only; and
 * each weight is multiplied by routed_scale (fp32, after the renormalisation).
 * n_group = 1 (or topk_group = n_group) with routed_scale = 1 is moe_route.
 * Requires n_group <= 64 dividing E into groups of at least 2 (when n_group >
 * 1), 1 <= topk_group <= n_group, k <= topk_group * E / n_group, routed_scale
 * finite.  Same workspace as moe_route.  Bit-exact and deterministic. */
int moe_route_grouped(const uint16_t* x, const uint16_t* w_router, const float* bias, int T, int H, int E,
                      int k, int renormalize, int n_group, int topk_group, float routed_scale,
                      int32_t* topk_idx, float* topk_w, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Permutation ("Kimi-K3 latent MoE" page, Code: moe_infer's per-expert counts,
 * argsort of the flattened expert ids and start/end walk; "Kimi K2.5 donor
 * reference", records "DeepSeek MoE.moe_infer: tokens per expert", "sorted
 * tokens", "start idx").  Slot f = t*k + j.
 *   counts[e]   = #{f : topk_idx[f] == e}
 *   offsets[e]  = sum_{e' < e} counts[e'],  offsets[E] = T*k
 *   sorted_slot = the slots ordered by expert, stable in f
 *   slot_pos[f] = position of f in sorted_slot (its inverse)
 * Requires every topk_idx value in [0, E).  Bit-exact and deterministic; no
 * host synchronisation.  Up to 16383 slots (T*k) one workgroup does it all
 * and ws may be NULL; from 16384 slots the slots are cut into blocks of 1024
 * and ws (device, 16-byte aligned, at least moe_permute_workspace_bytes(T, k,
 * E) bytes, 0 below that size) holds per-block expert counts between three
 * launches; the result is the same either way. */
size_t moe_permute_workspace_bytes(int T, int k, int E);
int moe_permute(const int32_t* topk_idx, int T, int k, int E, int32_t* counts, int32_t* offsets,
                int32_t* sorted_slot, int32_t* slot_pos, void* ws, size_t ws_bytes, void* stream);

/* moe_permute for callers that cannot allocate device memory (code under HIP
 * graph capture, serving loops and harnesses that forbid allocation): the same
 * arguments and results without the workspace.  From 16384 slots the
 * per-block expert counts live in a fixed 1 MiB device array inside the
 * library (one copy per GPU, held until the process ends), so the call
 * supports ceil(T*k / 1024) * E <= 262144 there (at E = 384: up to 696,320
 * slots) and returns MOE_ERR_UNSUPPORTED beyond it.  Every count entry is
 * written before it is read, so nothing carries over from an earlier call.
 * All calls on one GPU share that array: calls that overlap in time on one
 * GPU (other streams, other host threads) race and must be serialised by the
 * caller.  Allocates nothing; the first call on a device looks up the array's
 * address for that device. */
int moe_permute_noalloc(const int32_t* topk_idx, int T, int k, int E, int32_t* counts, int32_t* offsets,
                        int32_t* sorted_slot, int32_t* slot_pos, void* stream);

/* ---------------------------------------------------------------------------
 * Exact-mode activation quantiser ("Kimi exact-generator adaptation", "The
 * proposed substitution": ExactLinear with group size 32 and an activation
 * width).  Per row and group of 32: amax = max|x|; s = amax / 127 (fp32);
 * q = clamp(rint(x / s), -127, 127), ties to even; amax == 0 gives s = 0, q = 0.
 * x [M,K] bf16 -> q [M,K] int8, s [M,K/32] fp32.  Bit-exact. */
int moe_quant_act_int8(const uint16_t* x, int M, int K, int8_t* q, float* s, void* stream);
/* ExactLinear with 8-bit weights ("Kimi exact-generator adaptation", "The
 * proposed substitution": ExactLinear.from_weight with bits 4 or 8, group size
 * 32; the class body is not on the pages, so the reading is stated):
 *   y[m][n] = fold over groups g ascending of
 *             acc = fmaf(fl32(sw[n][g] * (float)G), sx[m][g], acc),  acc from 0,
 *   G = sum over the group of qx[m][i] * qw[n][i] (exact int32).
 * qx [M,K] int8 with sx [M,K/32] fp32 (moe_quant_act_int8 of the input);
 * qw [N,K] int8 with sw [N,K/32] fp32 (moe_quant_act_int8 of the bf16 weight
 * rows); y [M,N] fp32.  K a multiple of 128; qx, qw 16-byte aligned.
 * Bit-exact. */
int moe_exact_linear_i8w(const int8_t* qx, const float* sx, const int8_t* qw, const float* sw, int M, int N, int K,
                         float* y, void* stream);

/* The same with 16-bit codes (exact mode with act_bits = 16, the adaptation's
 * default activation width): s = amax / 32767, q = clamp(rint(x / s), +-32767)
 * -> q [M,K] int16, s [M,K/32] fp32.  Bit-exact. */
int moe_quant_act_int16(const uint16_t* x, int M, int K, int16_t* q, float* s, void* stream);

/* ---------------------------------------------------------------------------
 * Weight fragment layout for the grouped GEMMs (a layout step of this library,
 * not of the method: the checkpoint buffers of "Kimi exact-generator
 * adaptation", "The proposed substitution", load without any arithmetic
 * conversion; this reorders their bytes once, exactly, and stores the scales
 * as fp16, the operand format of the dequantisation, which is exact for the
 * scales moe_int4_check_scales accepts).
 * Input: a stacked expert matrix in the checkpoint layout, packed [E][N][K/2],
 * scale [E][N][K/32] bf16.  Output (same sizes, out of place): with
 * nch = K/128, row group R = e*(N/16) + n/16 and chunk c,
 *   packed_out[((R*nch + c)*64 + l)*16 + 4g + b] = packed[row 16(R%(N/16))+r of
 *       expert e][64c + 16g + 4j + b],  lane l = r + 16j (r < 16, j < 4),
 *       g < 4, b < 4   (1 KB per (R, c): 16 rows x 128 K, lane-major)
 *   scale_out[((R*nch + c)*16 + r)*4 + g] = fp16(scale[row ...][4c + g])
 *       (fp16 bits; bf16 -> fp16 rounds to nearest even)
 * Nibble order inside each byte is unchanged.  N a multiple of 16, K of 128;
 * packed buffers 16-byte and scale buffers 8-byte aligned; input and output
 * must not overlap.  E == 0 is a no-op. */
int moe_int4_prepack(const uint8_t* packed, const uint16_t* scale, int E, int N, int K,
                     uint8_t* packed_out, uint16_t* scale_out, void* stream);

/* Load-time check of a scale tensor for the routed GEMMs (the checkpoint's
 * weight_scale of "Kimi exact-generator adaptation", "Sources & provenance",
 * loaded without conversion): counts the bf16 scales that are neither zero
 * nor of magnitude in [2^-14, 2^9] (NaN and infinity included) into *count
 * (device int32, 4-byte aligned, overwritten) and returns MOE_ERR_UNSUPPORTED
 * with the count in the error detail when there is any, else MOE_OK.  scale
 * is n bf16 values (2-byte aligned), in either layout.  Unlike every other
 * call it synchronises `stream` to return its result: a weight-load step,
 * not for the forward path.  n == 0 returns MOE_OK. */
int moe_int4_check_scales(const uint16_t* scale, size_t n, int32_t* count, void* stream);

/* ---------------------------------------------------------------------------
 * fp16 staging format of activations (an implementation layout, not from the
 * pages: the routed GEMMs run their operands as fp16 on the matrix cores, and
 * their dequantised weights pair elements (p, p+4) of each 8-element block).
 * out [rows, K] fp16 bits: for every row and block of 8 elements e0..e7 of x
 * [rows, K] bf16, the block is stored as e0,e4,e1,e5,e2,e6,e3,e7, each
 * converted bf16 -> fp16 rounding toward zero (exact in the fp16 normal
 * range; larger magnitudes saturate to the largest finite fp16, as in the
 * kernels' own conversion).  K a multiple of 8; buffers 16-byte aligned and
 * not overlapping.  rows == 0 is a no-op. */
int moe_act_f16p(const uint16_t* x, int rows, int K, uint16_t* out, void* stream);

/* ---------------------------------------------------------------------------
 * Grouped gate/up projections + SwiGLU over the ragged expert segments
 * ("Kimi exact-generator adaptation", "The preserved forward form";
 * "Kimi K2.5 donor reference", record "SwiGLU-style gated feed-forward
 * projection").  Row p of the output (sorted position p, expert e with
 * offsets[e] <= p < offsets[e+1]) uses token t = sorted_slot[p] / k:
 *   mode MOE_MODE_BF16: act = x [T,H] bf16, act_scale = NULL;
 *     g = bf16(x_t . Wg[e]), u = bf16(x_t . Wu[e]), a = bf16(silu(g)),
 *     h[p] = bf16(a * u)  ->  h [T*k, I] bf16, h_scale = NULL.
 *   mode MOE_MODE_EXACT_I8: act = q_x [T,H] int8, act_scale = s_x [T,H/32];
 *     g, u = sum over groups (ascending) of fma(s_w * G, s_x, acc) in fp32,
 *     G the exact int32 group dot product; h = silu(g) * u (fp32), quantised
 *     per row and group of 32 like moe_quant_act_int8 -> h = q_h [T*k, I]
 *     int8, h_scale = s_h [T*k, I/32] fp32.  Bit-exact.
 *   mode MOE_MODE_EXACT_I16 (act_bits = 16): as MOE_MODE_EXACT_I8 with int16
 *     codes: act = q_x [T,H] int16 (moe_quant_act_int16), G the exact int4 x
 *     int16 group sum (|G| < 2^23), the fold fma(fl32(s_w * G), s_x, acc) with
 *     the product rounded once to fp32 (exact for 8-bit codes); h quantised
 *     to int16 codes (amax/32767) -> h = q_h [T*k, I] int16, h_scale fp32.
 *     Bit-exact.
 *   mode MOE_MODE_BF16_F16P: the arithmetic of MOE_MODE_BF16 with the
 *     activations already in the fp16 staging format of moe_act_f16p:
 *     act = moe_act_f16p(x) [T,H], and h is written in that format (the
 *     staging format of the bf16 h that MOE_MODE_BF16 writes).  Results are
 *     bit-identical to MOE_MODE_BF16; the kernels skip the per-tile
 *     conversion of the activations.
 * gate/up weights and their fp16 scales in the fragment layout of moe_int4_prepack.
 * Empty experts are skipped; rows of absent experts are not written. */
int moe_int4_grouped_swiglu(int mode, const void* act, const float* act_scale,
                            const uint8_t* gate_packed, const uint16_t* gate_scale,
                            const uint8_t* up_packed, const uint16_t* up_scale,
                            const int32_t* offsets, const int32_t* sorted_slot, int T, int k, int E,
                            int H, int I, void* h, float* h_scale, void* stream);

/* ---------------------------------------------------------------------------
 * Grouped down projection: y[p] = h[p] . Wd[e]^T for every sorted row p.
 *   MOE_MODE_BF16: h [T*k, I] bf16 -> y [T*k, H] bf16 (= bf16 of the fp32 sum).
 *   MOE_MODE_EXACT_I8: h = q_h int8 with h_scale = s_h -> y [T*k, H] fp32,
 *     the fixed-order group combine as above.  Bit-exact.
 *   MOE_MODE_EXACT_I16: h = q_h int16 with h_scale = s_h -> y [T*k, H] fp32
 *     (the 16-bit fold above).  Bit-exact.
 *   MOE_MODE_BF16_F16P: h in the fp16 staging format (as written by
 *     moe_int4_grouped_swiglu in that mode) -> y [T*k, H] bf16, bit-identical
 *     to MOE_MODE_BF16 on the bf16 h. 
 * down weights and their fp16 scales in the fragment layout of moe_int4_prepack. */
int moe_int4_grouped_down(int mode, const void* h, const float* h_scale, const uint8_t* down_packed,
                          const uint16_t* down_scale, const int32_t* offsets, int T, int k, int E,
                          int I, int H, void* y, void* stream);

/* ---------------------------------------------------------------------------
 * Combine ("Kimi K2.5 donor reference", records "Sum the selected expert
 * outputs with their routing weights" and "Add an always-active shared
 * expert"; "Kimi-K3 latent MoE" page, Code: moe_infer's weighted sum over
 * the k slots in the weight dtype, then the cast back).
 *   acc = sum_{j ascending} topk_w[t,j] * y[slot_pos[t*k+j]]  (fp32 mul, fp32 add)
 *   MOE_MODE_BF16: y bf16; out[t] = bf16(acc); if shared != NULL,
 *     out[t] = bf16(out[t] + shared[t]).  out [T,H] bf16.
 *   MOE_MODE_EXACT_I8: y fp32; out [T,H] fp32 = acc (shared must be NULL). */
int moe_combine(int mode, const void* y, const int32_t* slot_pos, const float* topk_w,
                const uint16_t* shared, int T, int k, int H, void* out, void* stream);

/* ---------------------------------------------------------------------------
 * Dense bf16 pieces (shared expert and the K3 latent projections are plain
 * bf16 linear layers with [out, in] weights and no bias: "Kimi exact-generator
 * adaptation", "The proposed substitution"; "Kimi-K3 latent MoE", Parameters
 * table).  fp32 accumulation on the matrix cores.
 *   moe_linear_bf16: y = bf16(x w^T); if add != NULL, y = bf16(y + add).
 *     x [M,K], w [N,K], add/y [M,N].
 *   moe_dense_swiglu_bf16: h = bf16(bf16(silu(bf16(x wg^T))) * bf16(x wu^T)),
 *     x [M,H], wg/wu [I,H], h [M,I].
 * ws: device workspace of at least moe_dense_workspace_bytes(M, N_total, K)
 * bytes (N_total = N for linear, 2*I for swiglu); may be NULL when that is 0. */
size_t moe_dense_workspace_bytes(int M, int N_total, int K);
int moe_linear_bf16(const uint16_t* x, const uint16_t* w, const uint16_t* add, uint16_t* y, int M,
                    int N, int K, void* ws, size_t ws_bytes, void* stream);
int moe_dense_swiglu_bf16(const uint16_t* x, const uint16_t* w_gate, const uint16_t* w_up,
                          uint16_t* h, int M, int H, int I, void* ws, size_t ws_bytes, void* stream);
/* h[i] = bf16(bf16(silu(g[i])) * u[i]) elementwise, n elements. */
int moe_silu_mul_bf16(const uint16_t* g, const uint16_t* u, uint16_t* h, int64_t n, void* stream);

/* RMSNorm ("Kimi K2.5 donor reference", records "RMSNorm mean square",
 * "Normalize by the root mean square", "Apply learned per-feature RMSNorm
 * gains"): r = 1/sqrt(mean_fp32(x^2) + eps); y = bf16(bf16(x r) * gain).
 * x, y [M,N] bf16; gain [N] bf16. */
int moe_rmsnorm_bf16(const uint16_t* x, const uint16_t* gain, float eps, uint16_t* y, int M, int N,
                     void* stream);

/* ---------------------------------------------------------------------------
 * Exact int4 x int8 group sums on the int8 matrix cores ("Kimi exact-generator
 * adaptation", "Sources & provenance": the exact int4 multiply-accumulate):
 *   G[m][n][g] = sum_{i in [32g, 32g+32)} q_x[m][i] * q_w[n][i]   (int32)
 * q_x [M,K] int8, packed [N][K/2] -> G [M][N][K/32] int32.  Bit-exact.
 * M, N multiples of 16; K a multiple of 32. */
int moe_int4_group_sums_i32(const int8_t* q_x, const uint8_t* packed, int M, int N, int K,
                            int32_t* G, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_INT4_H */
