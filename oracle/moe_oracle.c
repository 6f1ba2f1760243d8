/*
 * moe_oracle.c -- plain, slow, CPU reference for the int4 routed-expert MoE layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link or
 * call this file: only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark use it.  It shares no code, header, table or constant with the
 * HIP library; every routine below is written from the pages' description of
 * the method (cited per function); where the pages leave a step open, the
 * reading taken is stated at the function.
 *
 * Conventions
 *   bf16 values travel as uint16_t bit patterns.
 *   Packed int4 weights: row n of a [N, K] matrix is K/2 bytes; byte b holds
 *   element 2b in its low nibble and element 2b+1 in its high nibble; a nibble
 *   is a two's-complement integer in [-8, 7].  One bf16 scale per 32
 *   consecutive elements of a row: scale[n][i/32].  Dequantised weight is
 *   q * s (no zero point).
 *   Precision: the parts the method fixes to fp32 (router logits, sigmoid,
 *   selection, exact mode) are computed in fp32 in the stated order; the parts
 *   compared within a tolerance (the bf16 path) accumulate in fp64 and round to
 *   bf16 at the points where a bf16 PyTorch module would.
 *
 * Build: gcc -O2 -std=c11 -fopenmp -ffp-contract=off -fno-fast-math -fPIC -shared
 * (contraction off: every a*b+c below is a rounded multiply then a rounded add
 * unless fmaf() is written).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------- */
/* bf16 <-> binary32 / binary64                                              */
/* ------------------------------------------------------------------------- */

static float bf16_to_f32(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Round a finite binary32 value to the nearest bf16, ties to even. */
static uint16_t f32_to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    return (uint16_t)(u >> 16);
}

/* Round a finite binary64 value directly to the nearest bf16 (8 significant
 * bits), ties to even, with no intermediate rounding to binary32.  Values in
 * the bf16 subnormal range go through binary32 (never reached by the layer's
 * data, kept only so the function is total). */
static uint16_t f64_to_bf16(double d) {
    if (d == 0.0) return signbit(d) ? 0x8000u : 0u;
    if (fabs(d) < 0x1p-126) return f32_to_bf16((float)d);
    int e;
    double m = frexp(d, &e);            /* |m| in [0.5, 1) */
    double r = nearbyint(ldexp(m, 8));  /* 8 significant bits, ties-to-even */
    float f = (float)ldexp(r, e - 8);   /* exact: r has at most 9 bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);         /* low half is zero by construction */
}

uint16_t oracle_f32_to_bf16(float f) { return f32_to_bf16(f); }
uint16_t oracle_f64_to_bf16(double d) { return f64_to_bf16(d); }

/* ------------------------------------------------------------------------- */
/* exp_ref / sigmoid_ref / silu_ref                                          */
/*                                                                           */
/* The router's score is the logistic function 1/(1+e^-z) of each logit      */
/* (Kimi K2.5 donor reference, record "Independent sigmoid scores for the    */
/* router").  Its selection must be reproduced bit for bit, so e^t is pinned */
/* to one fp32 algorithm: Cody-Waite reduction t = n ln2 + r with           */
/* n = rint(t log2 e), a two-part ln2, and the degree-7 Taylor polynomial of */
/* e^r evaluated by Horner's rule with fused multiply-adds, then scaling by  */
/* 2^n (W. J. Cody and W. Waite, Software Manual for the Elementary          */
/* Functions, 1980).  Each constant is the binary32 value nearest to the     */
/* stated real number (checked by the tests against high-precision values). */
/* ------------------------------------------------------------------------- */

static const float ORC_LOG2E  = 0x1.715476p+0f;   /* log2(e)               */
static const float ORC_LN2_HI = 0x1.62e430p-1f;   /* ln 2                  */
static const float ORC_LN2_LO = -0x1.05c610p-29f; /* ln 2 - ORC_LN2_HI     */
static const float ORC_INV_FACT[8] = {
    0x1.000000p+0f,  /* 1/0! */
    0x1.000000p+0f,  /* 1/1! */
    0x1.000000p-1f,  /* 1/2! */
    0x1.555556p-3f,  /* 1/3! */
    0x1.555556p-5f,  /* 1/4! */
    0x1.111112p-7f,  /* 1/5! */
    0x1.6c16c2p-10f, /* 1/6! */
    0x1.a01a02p-13f, /* 1/7! */
};

float oracle_const(int which) {
    switch (which) {
    case 0: return ORC_LOG2E;
    case 1: return ORC_LN2_HI;
    case 2: return ORC_LN2_LO;
    default: return (which >= 3 && which < 11) ? ORC_INV_FACT[which - 3] : 0.0f;
    }
}

float oracle_exp_ref(float t) {
    float n = rintf(t * ORC_LOG2E);
    float r = fmaf(-n, ORC_LN2_HI, t);
    r = fmaf(-n, ORC_LN2_LO, r);
    float p = ORC_INV_FACT[7];
    for (int m = 6; m >= 0; --m) p = fmaf(p, r, ORC_INV_FACT[m]);
    return ldexpf(p, (int)n);
}

float oracle_sigmoid_ref(float z) {
    float zc = z < -80.0f ? -80.0f : (z > 80.0f ? 80.0f : z);
    return 1.0f / (1.0f + oracle_exp_ref(-zc));
}

float oracle_silu_ref(float z) { return z * oracle_sigmoid_ref(z); }

/* SiLU in fp64 for the tolerance (bf16) path. */
static double silu_f64(double z) { return z / (1.0 + exp(-z)); }

/* ------------------------------------------------------------------------- */
/* int4 access                                                               */
/* ------------------------------------------------------------------------- */

static int q4_at(const uint8_t* row, int i) {
    uint8_t b = row[i >> 1];
    int nib = (i & 1) ? (b >> 4) : (b & 0x0F);
    return nib >= 8 ? nib - 16 : nib;
}

/* Dequantised weight W[n][i] = q * s, exact in binary64 (and in binary32). */
static double w4_at(const uint8_t* packed, const uint16_t* scale, int K, int n, int i) {
    const uint8_t* row = packed + (size_t)n * (size_t)(K / 2);
    double s = (double)bf16_to_f32(scale[(size_t)n * (size_t)(K / 32) + (size_t)(i / 32)]);
    return (double)q4_at(row, i) * s;
}

void oracle_unpack_int4(const uint8_t* packed, int N, int K, int8_t* q_out) {
    for (int n = 0; n < N; ++n)
        for (int i = 0; i < K; ++i)
            q_out[(size_t)n * K + i] = (int8_t)q4_at(packed + (size_t)n * (K / 2), i);
}

/* ------------------------------------------------------------------------- */
/* Router: logits, sigmoid scores, biased selection, renormalisation.        */
/*                                                                           */
/* Kimi K2.5 donor reference, records "MoEGate.forward: logits" (a           */
/* contraction of the hidden state with the router weight), "Independent     */
/* sigmoid scores for the router", "Bias the choice of experts while         */
/* retaining original affinities" (bias added for ranking only),             */
/* "MoEGate.forward: ( , topk idx)" and "Normalize the selected routing      */
/* affinities" (divide by the sum of the selected affinities plus 1e-20).    */
/* Readings: logits in fp32 in a fixed two-level order: each block of 64    */
/* consecutive hidden elements is summed from 0 in ascending index, and the  */
/* block sums are added from 0 in ascending block order (H is a multiple of  */
/* 64); ties in the biased score go to the lower expert index; slots are in  */
/* rank order; routed scaling factor 1; one expert group.                    */
/* ------------------------------------------------------------------------- */

#define ORC_LOGIT_BLOCK 64

void oracle_router_logits(const uint16_t* x, const uint16_t* wr, int T, int H, int E,
                          float* logits /* [T,E] */) {
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        const uint16_t* xr = x + (size_t)t * H;
        for (int e = 0; e < E; ++e) {
            const uint16_t* wrow = wr + (size_t)e * H;
            float total = 0.0f;
            for (int b = 0; b < H; b += ORC_LOGIT_BLOCK) {
                float part = 0.0f;
                for (int i = b; i < b + ORC_LOGIT_BLOCK; ++i)
                    part = part + bf16_to_f32(xr[i]) * bf16_to_f32(wrow[i]);
                total = total + part;
            }
            logits[(size_t)t * E + e] = total;
        }
    }
}

/* Selection and weights from given sigmoid scores s[T,E]. */
void oracle_topk_from_scores(const float* scores, const float* bias, int T, int E, int k,
                             int renormalize, int32_t* topk_idx, float* topk_w) {
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        const float* s = scores + (size_t)t * E;
        float* c = (float*)malloc(sizeof(float) * (size_t)E);
        char* taken = (char*)calloc((size_t)E, 1);
        for (int e = 0; e < E; ++e) c[e] = s[e] + bias[e];
        for (int j = 0; j < k; ++j) {
            int best = -1;
            for (int e = 0; e < E; ++e) {
                if (taken[e]) continue;
                if (best < 0 || c[e] > c[best]) best = e; /* strict: ties keep lower e */
            }
            taken[best] = 1;
            topk_idx[(size_t)t * k + j] = best;
        }
        if (renormalize) {
            float d = 0.0f;
            for (int j = 0; j < k; ++j) d = d + s[topk_idx[(size_t)t * k + j]];
            d = d + 1e-20f;
            for (int j = 0; j < k; ++j) topk_w[(size_t)t * k + j] = s[topk_idx[(size_t)t * k + j]] / d;
        } else {
            for (int j = 0; j < k; ++j) topk_w[(size_t)t * k + j] = s[topk_idx[(size_t)t * k + j]];
        }
        free(c);
        free(taken);
    }
}

/* Group-limited selection ("Kimi K2.5 donor reference", MoEGate.forward
 * records: group scores, group idx, score mask, topk idx, denominator; the
 * records name these statements without their code).  Readings taken:
 *   - the E experts form n_group groups of E/n_group consecutive indices;
 *   - a group's score is the sum of its two largest biased scores c = s + b
 *     (largest + second largest, one fp32 add);
 *   - the topk_group groups with the largest scores are kept, ties to the
 *     lower group index;
 *   - experts outside the kept groups cannot be selected; the top k of c is
 *     taken among the rest, ties to the lower expert index;
 *   - weights: as oracle_topk_from_scores, then each multiplied by the routed
 *     scaling factor (fp32): w = (s / d) * scale.
 * n_group = 1 (or topk_group = n_group) is the ungrouped selection. */
void oracle_topk_grouped_from_scores(const float* scores, const float* bias, int T, int E, int k, int n_group,
                                     int topk_group, int renormalize, float scale, int32_t* topk_idx,
                                     float* topk_w) {
    const int G = E / n_group;
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        const float* s = scores + (size_t)t * E;
        float* c = (float*)malloc(sizeof(float) * (size_t)E);
        float* gs = (float*)malloc(sizeof(float) * (size_t)n_group);
        char* keep = (char*)calloc((size_t)n_group, 1);
        char* taken = (char*)calloc((size_t)E, 1);
        for (int e = 0; e < E; ++e) c[e] = s[e] + bias[e];
        for (int g = 0; g < n_group; ++g) {
            int b1 = -1, b2 = -1;
            for (int e = g * G; e < (g + 1) * G; ++e) {
                if (b1 < 0 || c[e] > c[b1]) { b2 = b1; b1 = e; }
                else if (b2 < 0 || c[e] > c[b2]) b2 = e;
            }
            gs[g] = (G >= 2) ? c[b1] + c[b2] : c[b1];
        }
        for (int j = 0; j < topk_group; ++j) {
            int best = -1;
            for (int g = 0; g < n_group; ++g) {
                if (keep[g]) continue;
                if (best < 0 || gs[g] > gs[best]) best = g;
            }
            keep[best] = 1;
        }
        for (int j = 0; j < k; ++j) {
            int best = -1;
            for (int e = 0; e < E; ++e) {
                if (taken[e] || !keep[e / G]) continue;
                if (best < 0 || c[e] > c[best]) best = e;
            }
            taken[best] = 1;
            topk_idx[(size_t)t * k + j] = best;
        }
        float d = 0.0f;
        for (int j = 0; j < k; ++j) d = d + s[topk_idx[(size_t)t * k + j]];
        d = d + 1e-20f;
        for (int j = 0; j < k; ++j) {
            const float v = s[topk_idx[(size_t)t * k + j]];
            topk_w[(size_t)t * k + j] = (renormalize ? v / d : v) * scale;
        }
        free(c);
        free(gs);
        free(keep);
        free(taken);
    }
}

void oracle_route(const uint16_t* x, const uint16_t* wr, const float* bias, int T, int H, int E,
                  int k, int renormalize, int32_t* topk_idx, float* topk_w,
                  float* logits_out /* [T,E] or NULL */, float* scores_out /* [T,E] or NULL */) {
    float* logits = logits_out ? logits_out : (float*)malloc(sizeof(float) * (size_t)T * E);
    float* scores = scores_out ? scores_out : (float*)malloc(sizeof(float) * (size_t)T * E);
    oracle_router_logits(x, wr, T, H, E, logits);
    for (size_t i = 0; i < (size_t)T * E; ++i) scores[i] = oracle_sigmoid_ref(logits[i]);
    oracle_topk_from_scores(scores, bias, T, E, k, renormalize, topk_idx, topk_w);
    if (!logits_out) free(logits);
    if (!scores_out) free(scores);
}

/* ------------------------------------------------------------------------- */
/* Permutation: tokens per expert, start offsets, sorted slots.              */
/* Kimi-K3 latent MoE page, Code (moe_infer): count assignments per expert,  */
/* argsort the flattened expert ids, walk experts with start/end indices,    */
/* scatter outputs back by the sort index.  Reading: the sort is stable in   */
/* the flattened slot index f = t*k + j.                                     */
/* ------------------------------------------------------------------------- */

void oracle_permute(const int32_t* topk_idx, int T, int k, int E, int32_t* counts,
                    int32_t* offsets /* [E+1] */, int32_t* sorted_slot, int32_t* slot_pos) {
    int S = T * k;
    for (int e = 0; e < E; ++e) counts[e] = 0;
    for (int f = 0; f < S; ++f) counts[topk_idx[f]] += 1;
    offsets[0] = 0;
    for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
    int32_t* next = (int32_t*)malloc(sizeof(int32_t) * (size_t)(E > 0 ? E : 1));
    for (int e = 0; e < E; ++e) next[e] = offsets[e];
    for (int f = 0; f < S; ++f) {
        int e = topk_idx[f];
        sorted_slot[next[e]] = f;
        slot_pos[f] = next[e];
        next[e] += 1;
    }
    free(next);
}

/* ------------------------------------------------------------------------- */
/* bf16 path of one routed expert (tolerance part).                          */
/* SwiGLU form down(silu(gate x) * up x) (Kimi exact-generator adaptation,   */
/* "The preserved forward form"; Kimi K2.5 donor reference, record           */
/* "SwiGLU-style gated feed-forward projection"), with packed int4 gate, up  */
/* and down projections (adaptation page, "The proposed substitution").      */
/* Rounding points mirror bf16 modules: g, u, silu(g), h and y are bf16.     */
/* ------------------------------------------------------------------------- */

/* rows: P activation rows [P,H] (bf16); experts: expert id per row.
 * Weights: gate/up packed [E][I][H/2] with scales [E][I][H/32]; down packed
 * [E][H][I/2] with scales [E][H][I/32].  Outputs (any may be NULL):
 * g,u [P,I] bf16, h [P,I] bf16, y [P,H] bf16. */
void oracle_experts_bf16(const uint16_t* rows, const int32_t* experts, int P, int H, int I,
                         const uint8_t* wg, const uint16_t* sg, const uint8_t* wu,
                         const uint16_t* su, const uint8_t* wd, const uint16_t* sd,
                         uint16_t* g_out, uint16_t* u_out, uint16_t* h_out, uint16_t* y_out) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int p = 0; p < P; ++p) {
        const uint16_t* xr = rows + (size_t)p * H;
        int e = experts[p];
        const uint8_t* wge = wg + (size_t)e * I * (H / 2);
        const uint16_t* sge = sg + (size_t)e * I * (H / 32);
        const uint8_t* wue = wu + (size_t)e * I * (H / 2);
        const uint16_t* sue = su + (size_t)e * I * (H / 32);
        const uint8_t* wde = wd + (size_t)e * H * (I / 2);
        const uint16_t* sde = sd + (size_t)e * H * (I / 32);
        double* xd = (double*)malloc(sizeof(double) * (size_t)H);
        double* hd = (double*)malloc(sizeof(double) * (size_t)I);
        for (int i = 0; i < H; ++i) xd[i] = (double)bf16_to_f32(xr[i]);
        for (int n = 0; n < I; ++n) {
            double ag = 0.0, au = 0.0;
            for (int i = 0; i < H; ++i) {
                ag += xd[i] * w4_at(wge, sge, H, n, i);
                au += xd[i] * w4_at(wue, sue, H, n, i);
            }
            uint16_t gb = f64_to_bf16(ag), ub = f64_to_bf16(au);
            uint16_t ab = f64_to_bf16(silu_f64((double)bf16_to_f32(gb)));
            uint16_t hb = f64_to_bf16((double)bf16_to_f32(ab) * (double)bf16_to_f32(ub));
            if (g_out) g_out[(size_t)p * I + n] = gb;
            if (u_out) u_out[(size_t)p * I + n] = ub;
            if (h_out) h_out[(size_t)p * I + n] = hb;
            hd[n] = (double)bf16_to_f32(hb);
        }
        if (y_out) {
            for (int m = 0; m < H; ++m) {
                double acc = 0.0;
                for (int n = 0; n < I; ++n) acc += hd[n] * w4_at(wde, sde, I, m, n);
                y_out[(size_t)p * H + m] = f64_to_bf16(acc);
            }
        }
        free(xd);
        free(hd);
    }
}

/* The SwiGLU join alone on given bf16 g and u (the same rounding chain as in
 * oracle_experts_bf16): h = bf16(bf16(silu(g)) * u), n elements. */
void oracle_silu_mul_bf16(const uint16_t* g, const uint16_t* u, long n, uint16_t* h) {
#pragma omp parallel for schedule(static)
    for (long i = 0; i < n; ++i) {
        uint16_t ab = f64_to_bf16(silu_f64((double)bf16_to_f32(g[i])));
        h[i] = f64_to_bf16((double)bf16_to_f32(ab) * (double)bf16_to_f32(u[i]));
    }
}

/* Weighted sum of the selected expert outputs (Kimi K2.5 donor reference,
 * record "Sum the selected expert outputs with their routing weights";
 * Kimi-K3 latent MoE page, Code: moe_infer multiplies the scattered outputs
 * by topk_weight and sums over the k slots), then the optional shared-expert
 * add (record "Add an always-active shared expert"), each rounded to bf16.
 * y: [T, k, H] bf16 in slot order; w: [T, k]; shared: [T, H] bf16 or NULL. */
void oracle_combine_bf16(const uint16_t* y, const float* w, const uint16_t* shared, int T, int k,
                         int H, uint16_t* out) {
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        for (int m = 0; m < H; ++m) {
            double acc = 0.0;
            for (int j = 0; j < k; ++j)
                acc += (double)w[(size_t)t * k + j] * (double)bf16_to_f32(y[((size_t)t * k + j) * H + m]);
            uint16_t ob = f64_to_bf16(acc);
            if (shared)
                ob = f64_to_bf16((double)bf16_to_f32(ob) + (double)bf16_to_f32(shared[(size_t)t * H + m]));
            out[(size_t)t * H + m] = ob;
        }
    }
}

/* Dense bf16 linear y = bf16(x W^T), W in [out, in] layout, fp64 accumulation
 * (the shared expert and the latent projections are ordinary bf16 linear
 * layers: adaptation page, "The proposed substitution"; Kimi-K3 latent MoE
 * page, Parameters table: weight held [out, in], no bias).
 * add: optional [M,N] bf16 added after rounding (y = bf16(bf16(xW^T) + add)). */
void oracle_linear_bf16(const uint16_t* x, const uint16_t* w, const uint16_t* add, int M, int N,
                        int K, uint16_t* y) {
#pragma omp parallel for schedule(static)
    for (int m = 0; m < M; ++m) {
        const uint16_t* xr = x + (size_t)m * K;
        for (int n = 0; n < N; ++n) {
            const uint16_t* wr = w + (size_t)n * K;
            double acc = 0.0;
            for (int i = 0; i < K; ++i) acc += (double)bf16_to_f32(xr[i]) * (double)bf16_to_f32(wr[i]);
            uint16_t r = f64_to_bf16(acc);
            if (add) r = f64_to_bf16((double)bf16_to_f32(r) + (double)bf16_to_f32(add[(size_t)m * N + n]));
            y[(size_t)m * N + n] = r;
        }
    }
}

/* Shared expert: the same SwiGLU flow with dense bf16 weights
 * wg, wu [I,H], wd [H,I].  Outputs h [M,I] (may be NULL) and y [M,H]. */
void oracle_dense_swiglu_bf16(const uint16_t* x, const uint16_t* wg, const uint16_t* wu,
                              const uint16_t* wd, int M, int H, int I, uint16_t* h_out,
                              uint16_t* y) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int m = 0; m < M; ++m) {
        const uint16_t* xr = x + (size_t)m * H;
        double* hd = (double*)malloc(sizeof(double) * (size_t)I);
        for (int n = 0; n < I; ++n) {
            double ag = 0.0, au = 0.0;
            for (int i = 0; i < H; ++i) {
                double xv = (double)bf16_to_f32(xr[i]);
                ag += xv * (double)bf16_to_f32(wg[(size_t)n * H + i]);
                au += xv * (double)bf16_to_f32(wu[(size_t)n * H + i]);
            }
            uint16_t gb = f64_to_bf16(ag), ub = f64_to_bf16(au);
            uint16_t ab = f64_to_bf16(silu_f64((double)bf16_to_f32(gb)));
            uint16_t hb = f64_to_bf16((double)bf16_to_f32(ab) * (double)bf16_to_f32(ub));
            if (h_out) h_out[(size_t)m * I + n] = hb;
            hd[n] = (double)bf16_to_f32(hb);
        }
        for (int j = 0; j < H; ++j) {
            double acc = 0.0;
            for (int n = 0; n < I; ++n) acc += hd[n] * (double)bf16_to_f32(wd[(size_t)j * I + n]);
            y[(size_t)m * H + j] = f64_to_bf16(acc);
        }
        free(hd);
    }
}

/* RMSNorm (Kimi K2.5 donor reference, records "RMSNorm mean square",
 * "Normalize by the root mean square", "Apply learned per-feature RMSNorm
 * gains"): r = 1/sqrt(mean(x^2) + eps); nrm = bf16(x r); out = bf16(nrm * gain).
 * Reading: the bf16 cast of the normalised value comes before the gain. */
void oracle_rmsnorm_bf16(const uint16_t* x, const uint16_t* gain, float eps, int M, int N,
                         uint16_t* y) {
#pragma omp parallel for schedule(static)
    for (int m = 0; m < M; ++m) {
        const uint16_t* xr = x + (size_t)m * N;
        double ss = 0.0;
        for (int i = 0; i < N; ++i) {
            double v = (double)bf16_to_f32(xr[i]);
            ss += v * v;
        }
        double r = 1.0 / sqrt(ss / (double)N + (double)eps);
        for (int i = 0; i < N; ++i) {
            uint16_t nb = f64_to_bf16((double)bf16_to_f32(xr[i]) * r);
            y[(size_t)m * N + i] = f64_to_bf16((double)bf16_to_f32(nb) * (double)bf16_to_f32(gain[i]));
        }
    }
}

/* ------------------------------------------------------------------------- */
/* Exact mode (bit-exact part).                                              */
/* Adaptation page, "The proposed substitution" and "Sources & provenance":  */
/* routed experts become PackedInt4Linear / ExactLinear (group size 32) with */
/* an exact integer multiply-accumulate and a configurable activation width. */
/* Readings: activations are quantised per row and per group of 32 to int8   */
/* with an fp32 scale amax/127, round-half-even, clamped to +-127, all-zero  */
/* group -> scale 0; each group's int4 x int8 dot product is an exact int32; */
/* groups are combined in fp32 in ascending order as                         */
/*   acc = fmaf(f32(s_w) * (float)G, s_x, acc)   (the product is exact),     */
/* starting from acc = 0.                                                    */
/* ------------------------------------------------------------------------- */

static void quant_group_f32(const float* v, int n, int8_t* q, float* s) {
    float amax = 0.0f;
    for (int i = 0; i < n; ++i) {
        float a = fabsf(v[i]);
        if (a > amax) amax = a;
    }
    if (amax == 0.0f) {
        for (int i = 0; i < n; ++i) q[i] = 0;
        *s = 0.0f;
        return;
    }
    float sc = amax / 127.0f;
    for (int i = 0; i < n; ++i) {
        float r = rintf(v[i] / sc);
        if (r > 127.0f) r = 127.0f;
        if (r < -127.0f) r = -127.0f;
        q[i] = (int8_t)r;
    }
    *s = sc;
}

/* x: [M, K] fp32 -> q [M, K] int8, s [M, K/32] fp32. */
void oracle_quant_f32_int8(const float* x, int M, int K, int8_t* q, float* s) {
#pragma omp parallel for schedule(static)
    for (int m = 0; m < M; ++m)
        for (int g = 0; g < K / 32; ++g)
            quant_group_f32(x + (size_t)m * K + (size_t)g * 32, 32, q + (size_t)m * K + (size_t)g * 32,
                            s + (size_t)m * (K / 32) + g);
}

/* x: [M, K] bf16 -> q, s as above. */
void oracle_quant_act_int8(const uint16_t* x, int M, int K, int8_t* q, float* s) {
#pragma omp parallel for schedule(static)
    for (int m = 0; m < M; ++m) {
        float v[32];
        for (int g = 0; g < K / 32; ++g) {
            for (int i = 0; i < 32; ++i) v[i] = bf16_to_f32(x[(size_t)m * K + (size_t)g * 32 + i]);
            quant_group_f32(v, 32, q + (size_t)m * K + (size_t)g * 32, s + (size_t)m * (K / 32) + g);
        }
    }
}

/* Exact group sums G[m][n][g] = sum_{i in group g} qw[n][i] * qx[m][i] (int32),
 * and the same sums in int64 (for the bound check). */
void oracle_group_sums(const int8_t* qx, const uint8_t* packed, int M, int N, int K,
                       int32_t* G32, int64_t* G64 /* may be NULL */) {
    int NG = K / 32;
#pragma omp parallel for schedule(static)
    for (int m = 0; m < M; ++m)
        for (int n = 0; n < N; ++n) {
            const uint8_t* row = packed + (size_t)n * (K / 2);
            for (int g = 0; g < NG; ++g) {
                int32_t a32 = 0;
                int64_t a64 = 0;
                for (int i = g * 32; i < g * 32 + 32; ++i) {
                    int prod = q4_at(row, i) * (int)qx[(size_t)m * K + i];
                    a32 += prod;
                    a64 += prod;
                }
                G32[((size_t)m * N + n) * NG + g] = a32;
                if (G64) G64[((size_t)m * N + n) * NG + g] = a64;
            }
        }
}

static float exact_dot(const int8_t* qx, const float* sx, const uint8_t* wrow, const uint16_t* srow,
                       int K) {
    float acc = 0.0f;
    for (int g = 0; g < K / 32; ++g) {
        int32_t G = 0;
        for (int i = g * 32; i < g * 32 + 32; ++i) G += q4_at(wrow, i) * (int)qx[i];
        float cw = bf16_to_f32(srow[g]) * (float)G;
        acc = fmaf(cw, sx[g], acc);
    }
    return acc;
}

/* Exact linear y[m][n] = exact_dot(row m, weight row n), fp32 output. */
void oracle_exact_linear(const int8_t* qx, const float* sx, const uint8_t* packed,
                         const uint16_t* scale, int M, int N, int K, float* y) {
#pragma omp parallel for schedule(static)
    for (int m = 0; m < M; ++m)
        for (int n = 0; n < N; ++n)
            y[(size_t)m * N + n] = exact_dot(qx + (size_t)m * K, sx + (size_t)m * (K / 32),
                                             packed + (size_t)n * (K / 2),
                                             scale + (size_t)n * (K / 32), K);
}

/* Exact-mode routed expert for P rows: g,u = exact linear (fp32);
 * h = silu_ref(g) * u (fp32); (q_h, s_h) = quantise h per group of 32;
 * y = exact linear of (q_h, s_h) with the down projection (fp32).
 * Outputs may be NULL except y. */
void oracle_experts_exact(const int8_t* qx, const float* sx, const int32_t* experts, int P, int H,
                          int I, const uint8_t* wg, const uint16_t* sg, const uint8_t* wu,
                          const uint16_t* su, const uint8_t* wd, const uint16_t* sd, float* g_out,
                          float* u_out, int8_t* qh_out, float* sh_out, float* y_out) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int p = 0; p < P; ++p) {
        int e = experts[p];
        const int8_t* xq = qx + (size_t)p * H;
        const float* xs = sx + (size_t)p * (H / 32);
        const uint8_t* wge = wg + (size_t)e * I * (H / 2);
        const uint16_t* sge = sg + (size_t)e * I * (H / 32);
        const uint8_t* wue = wu + (size_t)e * I * (H / 2);
        const uint16_t* sue = su + (size_t)e * I * (H / 32);
        const uint8_t* wde = wd + (size_t)e * H * (I / 2);
        const uint16_t* sde = sd + (size_t)e * H * (I / 32);
        float* h = (float*)malloc(sizeof(float) * (size_t)I);
        int8_t* qh = (int8_t*)malloc((size_t)I);
        float* sh = (float*)malloc(sizeof(float) * (size_t)(I / 32));
        for (int n = 0; n < I; ++n) {
            float g = exact_dot(xq, xs, wge + (size_t)n * (H / 2), sge + (size_t)n * (H / 32), H);
            float u = exact_dot(xq, xs, wue + (size_t)n * (H / 2), sue + (size_t)n * (H / 32), H);
            if (g_out) g_out[(size_t)p * I + n] = g;
            if (u_out) u_out[(size_t)p * I + n] = u;
            h[n] = oracle_silu_ref(g) * u;
        }
        for (int gi = 0; gi < I / 32; ++gi) quant_group_f32(h + gi * 32, 32, qh + gi * 32, sh + gi);
        if (qh_out) memcpy(qh_out + (size_t)p * I, qh, (size_t)I);
        if (sh_out) memcpy(sh_out + (size_t)p * (I / 32), sh, sizeof(float) * (size_t)(I / 32));
        for (int m = 0; m < H; ++m)
            y_out[(size_t)p * H + m] =
                exact_dot(qh, sh, wde + (size_t)m * (I / 2), sde + (size_t)m * (I / 32), I);
        free(h);
        free(qh);
        free(sh);
    }
}

/* ------------------------------------------------------------------------- */
/* Exact mode with 16-bit activations (the adaptation's act_bits, whose       */
/* default the K2.5 source passes as 16).  Readings: the quantiser of the     */
/* 8-bit mode with 32767 for 127 (scale amax/32767, round-half-even, clamp to */
/* +-32767, zero group -> scale 0); the int4 x int16 group sums are exact     */
/* (|G| <= 32 * 8 * 32767 < 2^23); the fold is the 8-bit one,                 */
/*   acc = fmaf(f32(s_w) * (float)G, s_x, acc),                              */
/* where the product is now rounded once to fp32 (it is exact for 8 bits).   */
/* ------------------------------------------------------------------------- */

static void quant_group_f32_i16(const float* v, int n, int16_t* q, float* s) {
    float amax = 0.0f;
    for (int i = 0; i < n; ++i) {
        float a = fabsf(v[i]);
        if (a > amax) amax = a;
    }
    if (amax == 0.0f) {
        for (int i = 0; i < n; ++i) q[i] = 0;
        *s = 0.0f;
        return;
    }
    float sc = amax / 32767.0f;
    for (int i = 0; i < n; ++i) {
        float r = rintf(v[i] / sc);
        if (r > 32767.0f) r = 32767.0f;
        if (r < -32767.0f) r = -32767.0f;
        q[i] = (int16_t)r;
    }
    *s = sc;
}

/* x: [M, K] bf16 -> q [M, K] int16, s [M, K/32] fp32. */
void oracle_quant_act_int16(const uint16_t* x, int M, int K, int16_t* q, float* s) {
#pragma omp parallel for schedule(static)
    for (int m = 0; m < M; ++m) {
        float v[32];
        for (int g = 0; g < K / 32; ++g) {
            for (int i = 0; i < 32; ++i) v[i] = bf16_to_f32(x[(size_t)m * K + (size_t)g * 32 + i]);
            quant_group_f32_i16(v, 32, q + (size_t)m * K + (size_t)g * 32, s + (size_t)m * (K / 32) + g);
        }
    }
}

/* Group sums of int4 weights with int16 activations (int32 and int64). */
void oracle_group_sums16(const int16_t* qx, const uint8_t* packed, int M, int N, int K, int32_t* G32,
                         int64_t* G64 /* may be NULL */) {
    int NG = K / 32;
#pragma omp parallel for schedule(static)
    for (int m = 0; m < M; ++m)
        for (int n = 0; n < N; ++n) {
            const uint8_t* row = packed + (size_t)n * (K / 2);
            for (int g = 0; g < NG; ++g) {
                int32_t a32 = 0;
                int64_t a64 = 0;
                for (int i = g * 32; i < g * 32 + 32; ++i) {
                    int prod = q4_at(row, i) * (int)qx[(size_t)m * K + i];
                    a32 += prod;
                    a64 += prod;
                }
                G32[((size_t)m * N + n) * NG + g] = a32;
                if (G64) G64[((size_t)m * N + n) * NG + g] = a64;
            }
        }
}

static float exact_dot16(const int16_t* qx, const float* sx, const uint8_t* wrow, const uint16_t* srow, int K) {
    float acc = 0.0f;
    for (int g = 0; g < K / 32; ++g) {
        int32_t G = 0;
        for (int i = g * 32; i < g * 32 + 32; ++i) G += q4_at(wrow, i) * (int)qx[i];
        float cw = bf16_to_f32(srow[g]) * (float)G;
        acc = fmaf(cw, sx[g], acc);
    }
    return acc;
}

void oracle_exact_linear16(const int16_t* qx, const float* sx, const uint8_t* packed, const uint16_t* scale, int M,
                           int N, int K, float* y) {
#pragma omp parallel for schedule(static)
    for (int m = 0; m < M; ++m)
        for (int n = 0; n < N; ++n)
            y[(size_t)m * N + n] = exact_dot16(qx + (size_t)m * K, sx + (size_t)m * (K / 32),
                                               packed + (size_t)n * (K / 2), scale + (size_t)n * (K / 32), K);
}

/* The expert chain of oracle_experts_exact with 16-bit activations and h. */
void oracle_experts_exact16(const int16_t* qx, const float* sx, const int32_t* experts, int P, int H, int I,
                            const uint8_t* wg, const uint16_t* sg, const uint8_t* wu, const uint16_t* su,
                            const uint8_t* wd, const uint16_t* sd, float* g_out, float* u_out, int16_t* qh_out,
                            float* sh_out, float* y_out) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int p = 0; p < P; ++p) {
        int e = experts[p];
        const int16_t* xq = qx + (size_t)p * H;
        const float* xs = sx + (size_t)p * (H / 32);
        const uint8_t* wge = wg + (size_t)e * I * (H / 2);
        const uint16_t* sge = sg + (size_t)e * I * (H / 32);
        const uint8_t* wue = wu + (size_t)e * I * (H / 2);
        const uint16_t* sue = su + (size_t)e * I * (H / 32);
        const uint8_t* wde = wd + (size_t)e * H * (I / 2);
        const uint16_t* sde = sd + (size_t)e * H * (I / 32);
        float* h = (float*)malloc(sizeof(float) * (size_t)I);
        int16_t* qh = (int16_t*)malloc(sizeof(int16_t) * (size_t)I);
        float* sh = (float*)malloc(sizeof(float) * (size_t)(I / 32));
        for (int n = 0; n < I; ++n) {
            float g = exact_dot16(xq, xs, wge + (size_t)n * (H / 2), sge + (size_t)n * (H / 32), H);
            float u = exact_dot16(xq, xs, wue + (size_t)n * (H / 2), sue + (size_t)n * (H / 32), H);
            if (g_out) g_out[(size_t)p * I + n] = g;
            if (u_out) u_out[(size_t)p * I + n] = u;
            h[n] = oracle_silu_ref(g) * u;
        }
        for (int gi = 0; gi < I / 32; ++gi) quant_group_f32_i16(h + gi * 32, 32, qh + gi * 32, sh + gi);
        if (qh_out) memcpy(qh_out + (size_t)p * I, qh, sizeof(int16_t) * (size_t)I);
        if (sh_out) memcpy(sh_out + (size_t)p * (I / 32), sh, sizeof(float) * (size_t)(I / 32));
        for (int m = 0; m < H; ++m)
            y_out[(size_t)p * H + m] = exact_dot16(qh, sh, wde + (size_t)m * (I / 2), sde + (size_t)m * (I / 32), I);
        free(h);
        free(qh);
        free(sh);
    }
}

/* ------------------------------------------------------------------------- */
/* ExactLinear with 8-bit weights (adaptation page, "The proposed            */
/* substitution": ExactLinear.from_weight with bits 4 or 8 and group size 32; */
/* the class body is not on the pages).  Readings: the weights are quantised  */
/* like the activations, per row and group of 32 with an fp32 scale amax/127  */
/* and codes clamped to +-127; each group's int8 x int8 dot product is an     */
/* exact int32 (|G| <= 32 * 127 * 127); the fold is the exact mode's,         */
/*   acc = fmaf(fl32(s_w * (float)G), s_x, acc), groups ascending, from 0.    */
/* y [M, N] fp32.                                                             */
/* ------------------------------------------------------------------------- */
void oracle_exact_linear_i8w(const int8_t* qx, const float* sx, const int8_t* qw, const float* sw, int M, int N,
                             int K, float* y) {
#pragma omp parallel for schedule(static)
    for (int m = 0; m < M; ++m)
        for (int n = 0; n < N; ++n) {
            const int8_t* xr = qx + (size_t)m * K;
            const int8_t* wr = qw + (size_t)n * K;
            float acc = 0.0f;
            for (int g = 0; g < K / 32; ++g) {
                int32_t G = 0;
                for (int i = g * 32; i < g * 32 + 32; ++i) G += (int)wr[i] * (int)xr[i];
                const float cw = sw[(size_t)n * (K / 32) + g] * (float)G;
                acc = fmaf(cw, sx[(size_t)m * (K / 32) + g], acc);
            }
            y[(size_t)m * N + n] = acc;
        }
}

/* Exact-mode combine: out[t][m] = sum_j w[t][j] * y[t][j][m] in fp32, j ascending,
 * each product rounded then added (fp32 output, no bf16 cast). */
void oracle_combine_f32(const float* y, const float* w, int T, int k, int H, float* out) {
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t)
        for (int m = 0; m < H; ++m) {
            float acc = 0.0f;
            for (int j = 0; j < k; ++j) acc = acc + w[(size_t)t * k + j] * y[((size_t)t * k + j) * H + m];
            out[(size_t)t * H + m] = acc;
        }
}

/* Vector forms of the scalar references (for sweeps in the tests). */
void oracle_exp_ref_n(const float* t, int n, float* out) {
    for (int i = 0; i < n; ++i) out[i] = oracle_exp_ref(t[i]);
}
void oracle_sigmoid_ref_n(const float* z, int n, float* out) {
    for (int i = 0; i < n; ++i) out[i] = oracle_sigmoid_ref(z[i]);
}
void oracle_silu_ref_n(const float* z, int n, float* out) {
    for (int i = 0; i < n; ++i) out[i] = oracle_silu_ref(z[i]);
}
void oracle_f64_to_bf16_n(const double* d, int n, uint16_t* out) {
    for (int i = 0; i < n; ++i) out[i] = f64_to_bf16(d[i]);
}
void oracle_f32_to_bf16_n(const float* f, int n, uint16_t* out) {
    for (int i = 0; i < n; ++i) out[i] = f32_to_bf16(f[i]);
}

#ifdef _OPENMP
#include <omp.h>
#endif
/* Number of threads the oracle's parallel loops use. */
int oracle_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
