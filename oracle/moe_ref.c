/*
 * moe_ref.c -- plain, slow CPU oracle of the sparse MoE layer forward.
 *
 * TEST INFRASTRUCTURE ONLY (see moe_ref.h).  Written for a reader to check by
 * eye against the pages; there is no blocking, fusion or reordering beyond what
 * the definitions below state.  fp64 throughout.  The only parallelism is an
 * OpenMP "parallel for" over independent output rows inside one FFN, which
 * changes no result.
 *
 * Citations:
 *   [R] "MoE 路由与专家流式加载" (colibri-analysis 07), §1.1-§1.4
 *   [Q] "colibrì 深度拆解：1300行纯C代码驱动7440亿参数大模型", §5.2
 *   [C] "colibri 开发演进实录：从 CHANGELOG 看多引擎 MoE 推理框架的工程迭代脉络", §2.1, §2.2,
 *       §五 and §六 (fp4 / MXFP4 experts), §8.3 (int3-g64)
 */
#include "moe_ref.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#define REF_EINVAL (-1)

/* ------------------------------------------------------------------------- */
/* int4 codec                                                                  */
/* ------------------------------------------------------------------------- */

/* [Q] §5.2: two signed int4 values share a byte, the first in the low nibble;
 * each is stored as its low four two's-complement bits. */
uint8_t moe_ref_pack_int4(int32_t lo, int32_t hi) {
    return (uint8_t)((lo & 0x0F) | ((hi & 0x0F) << 4));
}

/* [Q] §5.2: unpack takes each nibble and sign-extends bit 3. */
void moe_ref_unpack_int4(uint8_t b, int32_t *lo, int32_t *hi) {
    int32_t a = b & 0x0F;
    int32_t c = (b >> 4) & 0x0F;
    if (a & 0x08) a -= 16;
    if (c & 0x08) c -= 16;
    *lo = a;
    *hi = c;
}

/* Element k of a packed row (even k: low nibble, odd k: high nibble). */
static int32_t ref_code(const uint8_t *row_q, int64_t k) {
    int32_t lo, hi;
    moe_ref_unpack_int4(row_q[k / 2], &lo, &hi);
    return (k % 2 == 0) ? lo : hi;
}

/* Dequantised weight W[n][k] of an int4-gs64 matrix with K columns, in fp64.
 * The product of a code in [-8,7] and an fp32 scale is exact in fp64. */
static double ref_weight(const uint8_t *q, const float *s, int64_t K, int64_t n, int64_t k) {
    const uint8_t *row_q = q + n * (K / 2);
    const float *row_s = s + n * (K / 64);
    return (double)ref_code(row_q, k) * (double)row_s[k / 64];
}

/* One scale per 64 consecutive weights along K ([C] §2.1, "int4-gs64").  The
 * pages give no quantiser rule; the reading used here is symmetric absmax. */
int moe_ref_quantize_gs64(const float *w, int64_t N, int64_t K, uint8_t *q, float *s) {
    if (!w || !q || !s || N < 0 || K <= 0 || K % 64 != 0) return REF_EINVAL;
    for (int64_t n = 0; n < N; n++) {
        for (int64_t g = 0; g < K / 64; g++) {
            const float *wg = w + n * K + g * 64;
            float amax = 0.0f;
            for (int i = 0; i < 64; i++) {
                float a = fabsf(wg[i]);
                if (a > amax) amax = a;
            }
            float scale = amax / 7.0f;
            s[n * (K / 64) + g] = scale;
            int32_t code[64];
            for (int i = 0; i < 64; i++) {
                int32_t c = 0;
                if (scale > 0.0f) {
                    float r = nearbyintf(wg[i] / scale); /* round half to even */
                    if (r > 7.0f) r = 7.0f;
                    if (r < -8.0f) r = -8.0f;
                    c = (int32_t)r;
                }
                code[i] = c;
            }
            for (int i = 0; i < 64; i += 2)
                q[n * (K / 2) + g * 32 + i / 2] = moe_ref_pack_int4(code[i], code[i + 1]);
        }
    }
    return 0;
}

int moe_ref_dequantize_gs64(const uint8_t *q, const float *s, int64_t N, int64_t K, double *w) {
    if (!q || !s || !w || N < 0 || K <= 0 || K % 64 != 0) return REF_EINVAL;
    for (int64_t n = 0; n < N; n++)
        for (int64_t k = 0; k < K; k++) w[n * K + k] = ref_weight(q, s, K, n, k);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* The other expert formats (moe_ref.h)                                        */
/* ------------------------------------------------------------------------- */

/* [C] §五/§六 name fp4 experts with UE8M0 block scales and MXFP4 experts; the reading
 * is the OCP Microscaling FP4 element: sign, a two-bit exponent with bias 1 and one
 * mantissa bit.  Exponent 0 is subnormal: 0 or one half. */
double moe_ref_e2m1(uint8_t code) {
    const int sgn = (code >> 3) & 1;
    const int ex = (code >> 1) & 3;
    const int man = code & 1;
    double mag;
    if (ex == 0)
        mag = 0.5 * man;
    else
        mag = ldexp(1.0 + 0.5 * man, ex - 1);
    return sgn ? -mag : mag;
}

/* UE8M0: an unsigned biased exponent and nothing else; the all-ones byte is NaN. */
double moe_ref_ue8m0(uint8_t e) {
    if (e == 255) return NAN;
    return ldexp(1.0, (int)e - 127);
}

/* [C] §8.3 (fmt=5): 3-bit codes, one scale per 64.  Bit planes as moe_ref.h states. */
int32_t moe_ref_int3_code(const uint8_t *row_q, int64_t K, int64_t k) {
    const int64_t G = k / 64;
    const int i = (int)(k % 64);
    /* i = 16d + 8a + 2b + o for the low-bit plane */
    const int d = i / 16, a = (i / 8) % 2, b = (i / 2) % 4, o = i % 2;
    const int low = (row_q[16 * G + 4 * d + b] >> (2 * (2 * a + o))) & 3;
    /* i = 32h + 8m + 2b + o for the sign plane */
    const int h = i / 32, m = (i / 8) % 4;
    const int sign = (row_q[K / 4 + 8 * G + 4 * h + b] >> (2 * m + o)) & 1;
    return low - 4 * sign;
}

int64_t moe_ref_code_bytes(int32_t fmt, int64_t K) { return fmt == MOE_REF_FMT_INT3 ? 3 * K / 8 : K / 2; }

int64_t moe_ref_scale_bytes(int32_t fmt, int64_t K) {
    return fmt == MOE_REF_FMT_MXFP4 ? K / 32 : 4 * (K / 64);
}

/* W[n][k] of a matrix in format fmt, fp64.  Every product here is exact in fp64: a
 * code of at most 4 bits times an fp32 scale or a power of two. */
static double ref_weight_fmt(int32_t fmt, const uint8_t *q, const void *s, int64_t K, int64_t n,
                             int64_t k) {
    const uint8_t *row_q = q + n * moe_ref_code_bytes(fmt, K);
    if (fmt == MOE_REF_FMT_MXFP4) {
        const uint8_t *row_e = (const uint8_t *)s + n * (K / 32);
        const uint8_t byte = row_q[k / 2];
        const uint8_t code = (k % 2 == 0) ? (byte & 15) : (byte >> 4);
        return moe_ref_e2m1(code) * moe_ref_ue8m0(row_e[k / 32]);
    }
    const float *row_s = (const float *)s + n * (K / 64);
    const int32_t c = fmt == MOE_REF_FMT_INT3 ? moe_ref_int3_code(row_q, K, k) : ref_code(row_q, k);
    return (double)c * (double)row_s[k / 64];
}

static int ref_fmt_ok(int32_t fmt) {
    return fmt == MOE_REF_FMT_INT4 || fmt == MOE_REF_FMT_MXFP4 || fmt == MOE_REF_FMT_INT3;
}

int moe_ref_dequantize(int32_t fmt, const uint8_t *q, const void *s, int64_t N, int64_t K, double *w) {
    if (!ref_fmt_ok(fmt) || !q || !s || !w || N < 0 || K <= 0 || K % 64 != 0) return REF_EINVAL;
    for (int64_t n = 0; n < N; n++)
        for (int64_t k = 0; k < K; k++) w[n * K + k] = ref_weight_fmt(fmt, q, s, K, n, k);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Steps 1-2: router logits and noaux_tc selection ([R] §1.1, §1.2)            */
/* ------------------------------------------------------------------------- */

static int ref_layer_ok(const moe_ref_layer *L) {
    if (!L) return 0;
    if (L->hidden <= 0 || L->hidden % 64 != 0) return 0;
    if (L->n_experts <= 0 || L->ffn <= 0 || L->ffn % 64 != 0) return 0;
    if (L->shared_ffn < 0 || L->shared_ffn % 64 != 0) return 0;
    if (L->top_k < 1 || L->top_k > L->n_experts || L->top_k > 64) return 0;
    if (!(L->top_p >= 0.0f && L->top_p <= 1.0f)) return 0;
    if (L->n_group < 0) return 0;
    if (L->act_bits != 0 && L->act_bits != 16 && L->act_bits != 8) return 0;
    if (L->act_bits == 8 && L->act_block <= 0) return 0;
    if (!ref_fmt_ok(L->fmt)) return 0;
    if (L->n_group > 256) return 0;
    if (L->n_group > 1) { /* equal groups of at least two experts, enough experts kept */
        if (L->n_experts % L->n_group != 0 || L->n_experts / L->n_group < 2) return 0;
        if (L->topk_group < 1 || L->topk_group > L->n_group) return 0;
        if ((int64_t)L->topk_group * (L->n_experts / L->n_group) < L->top_k) return 0;
    }
    if (!L->router_w) return 0;
    return 1;
}

/* [R] §1.1: each position's logit for expert e is the router row dotted with x. */
int moe_ref_logits(const moe_ref_layer *L, const float *x, int32_t T, double *logits) {
    if (!ref_layer_ok(L) || (T > 0 && (!x || !logits)) || T < 0) return REF_EINVAL;
    const int32_t H = L->hidden, E = L->n_experts;
    for (int32_t t = 0; t < T; t++)
        for (int32_t e = 0; e < E; e++) {
            double acc = 0.0;
            for (int32_t h = 0; h < H; h++)
                acc += (double)x[(int64_t)t * H + h] * (double)L->router_w[(int64_t)e * H + h];
            logits[(int64_t)t * E + e] = acc;
        }
    return 0;
}

static double ref_sigmoid(double z) { return 1.0 / (1.0 + exp(-z)); }

/* One token's selection.  [R] §1.1: sig = sigmoid(logit); the choice score adds
 * the per-expert bias; the applied gate is the unbiased sig of the chosen expert.
 * [R] §1.2: k rounds of argmax over choice, excluding experts already taken;
 * optional adaptive top-p over the chosen gates sorted descending; norm_topk
 * renormalises the kept gates to sum 1; routed_scale multiplies them. */
static void ref_select_one(const moe_ref_layer *L, const double *logit,
                           int32_t *ids, float *w, int32_t *keff_out) {
    const int32_t E = L->n_experts, k = L->top_k;
    double *sig = (double *)malloc(sizeof(double) * (size_t)E);
    double *choice = (double *)malloc(sizeof(double) * (size_t)E);
    char *taken = (char *)calloc((size_t)E, 1);
    int32_t pick[64];
    double pick_sig[64];

    for (int32_t e = 0; e < E; e++) {
        sig[e] = ref_sigmoid(logit[e]);
        double b = L->router_bias ? (double)L->router_bias[e] : 0.0;
        choice[e] = sig[e] + b;
    }
    /* Group-limited routing (n_group > 1).  The pages' engine has n_group == 1 and
     * asserts it ([R] §1.2); for more groups this follows DeepSeek-V3's noaux_tc, the
     * routing the page is modelled on: experts form n_group equal groups of consecutive
     * ids; a group's score is the sum of its two largest choice scores (a repeated
     * maximum counts twice); the topk_group groups with the largest scores are kept
     * (iterative argmax, equal scores to the lower group id); experts of the other
     * groups take no part in the top-k below. */
    if (L->n_group > 1) {
        const int32_t G = L->n_group, gsz = E / G;
        double gscore[256];
        char gkeep[256];
        for (int32_t g = 0; g < G; g++) {
            double m1 = -INFINITY, m2 = -INFINITY;
            for (int32_t j = 0; j < gsz; j++) {
                double c = choice[g * gsz + j];
                if (c > m1) {
                    m2 = m1;
                    m1 = c;
                } else if (c > m2) {
                    m2 = c;
                }
            }
            gscore[g] = m1 + m2;
            gkeep[g] = 0;
        }
        for (int32_t r = 0; r < L->topk_group; r++) {
            int32_t best = -1;
            for (int32_t g = 0; g < G; g++) {
                if (gkeep[g]) continue;
                if (best < 0 || gscore[g] > gscore[best]) best = g;
            }
            gkeep[best] = 1;
        }
        for (int32_t e = 0; e < E; e++)
            if (!gkeep[e / gsz]) taken[e] = 1; /* never a candidate */
    }
    /* Iterative argmax; a strictly greater score replaces the best so far, so
     * equal scores go to the lowest expert id. */
    for (int32_t j = 0; j < k; j++) {
        int32_t best = -1;
        for (int32_t e = 0; e < E; e++) {
            if (taken[e]) continue;
            if (best < 0 || choice[e] > choice[best]) best = e;
        }
        taken[best] = 1;
        pick[j] = best;
        pick_sig[j] = sig[best];
    }

    /* Adaptive top-p: order the k chosen gates by sig descending (equal gates keep
     * slot order), keep the shortest prefix whose running sum reaches p * total. */
    char keep[64];
    for (int32_t j = 0; j < k; j++) keep[j] = 1;
    int32_t keff = k;
    if (L->top_p > 0.0f && L->top_p < 1.0f) {
        int32_t ord[64];
        for (int32_t j = 0; j < k; j++) ord[j] = j;
        for (int32_t a = 1; a < k; a++) { /* stable insertion sort, descending */
            int32_t v = ord[a], b = a - 1;
            while (b >= 0 && pick_sig[ord[b]] < pick_sig[v]) {
                ord[b + 1] = ord[b];
                b--;
            }
            ord[b + 1] = v;
        }
        double tot = 0.0;
        for (int32_t a = 0; a < k; a++) tot += pick_sig[ord[a]];
        double thr = (double)L->top_p * tot;
        double cum = 0.0;
        int32_t m = k;
        for (int32_t a = 0; a < k; a++) {
            cum += pick_sig[ord[a]];
            if (cum >= thr) {
                m = a + 1;
                break;
            }
        }
        for (int32_t j = 0; j < k; j++) keep[j] = 0;
        for (int32_t a = 0; a < m; a++) keep[ord[a]] = 1;
        keff = m;
    }

    /* Kept picks, compacted in selection order. */
    int32_t kid[64];
    double ksig[64];
    int32_t n = 0;
    for (int32_t j = 0; j < k; j++)
        if (keep[j]) {
            kid[n] = pick[j];
            ksig[n] = pick_sig[j];
            n++;
        }
    double denom = 0.0;
    for (int32_t j = 0; j < n; j++) denom += ksig[j];
    for (int32_t j = 0; j < k; j++) {
        if (j < n) {
            double g = ksig[j];
            if (L->norm_topk) g = g / denom;
            g = g * (double)L->routed_scale;
            ids[j] = kid[j];
            w[j] = (float)g;
        } else {
            ids[j] = -1;
            w[j] = 0.0f;
        }
    }
    *keff_out = keff;
    free(sig);
    free(choice);
    free(taken);
}

int moe_ref_select(const moe_ref_layer *L, const double *logits, int32_t T,
                   int32_t *ids, float *w, int32_t *keff) {
    if (!ref_layer_ok(L) || T < 0) return REF_EINVAL;
    if (T > 0 && (!logits || !ids || !w || !keff)) return REF_EINVAL;
    for (int32_t t = 0; t < T; t++)
        ref_select_one(L, logits + (int64_t)t * L->n_experts, ids + (int64_t)t * L->top_k,
                       w + (int64_t)t * L->top_k, keff + t);
    return 0;
}

int moe_ref_route(const moe_ref_layer *L, const float *x, int32_t T,
                  int32_t *ids, float *w, int32_t *keff) {
    if (!ref_layer_ok(L) || T < 0) return REF_EINVAL;
    if (T == 0) return 0;
    double *logits = (double *)malloc(sizeof(double) * (size_t)T * (size_t)L->n_experts);
    if (!logits) return REF_EINVAL;
    int rc = moe_ref_logits(L, x, T, logits);
    if (rc == 0) rc = moe_ref_select(L, logits, T, ids, w, keff);
    free(logits);
    return rc;
}

/* ------------------------------------------------------------------------- */
/* Step 3: batch union ([R] §1.3)                                             */
/* ------------------------------------------------------------------------- */

/* The experts chosen by any position of the batch, deduplicated, each listed
 * once; the rows of an expert are the tokens routed to it, in token order. */
int moe_ref_union(int32_t E, int32_t k, const int32_t *ids, const int32_t *keff, int32_t T,
                  int32_t *n_uniq, int32_t *uniq, int32_t *off, int32_t *row_tok,
                  int32_t *pick_row) {
    if (E <= 0 || k <= 0 || T < 0 || !n_uniq || !uniq || !off) return REF_EINVAL;
    if (T > 0 && (!ids || !keff || !row_tok || !pick_row)) return REF_EINVAL;
    for (int32_t t = 0; t < T; t++) {
        if (keff[t] < 0 || keff[t] > k) return REF_EINVAL;
        for (int32_t j = 0; j < keff[t]; j++)
            if (ids[(int64_t)t * k + j] < 0 || ids[(int64_t)t * k + j] >= E) return REF_EINVAL;
    }
    /* count[e] by brute force over every kept pick */
    int32_t nu = 0;
    off[0] = 0;
    for (int32_t e = 0; e < E; e++) {
        int32_t c = 0;
        for (int32_t t = 0; t < T; t++)
            for (int32_t j = 0; j < keff[t]; j++)
                if (ids[(int64_t)t * k + j] == e) c++;
        off[e + 1] = off[e] + c;
        if (c > 0) uniq[nu++] = e;
    }
    for (int32_t i = nu; i < E; i++) uniq[i] = -1;
    *n_uniq = nu;
    for (int64_t i = 0; i < (int64_t)T * k; i++) {
        row_tok[i] = -1;
        pick_row[i] = -1;
    }
    /* rows ordered by (expert ascending, token ascending) */
    for (int32_t e = 0; e < E; e++) {
        int32_t r = off[e];
        for (int32_t t = 0; t < T; t++)
            for (int32_t j = 0; j < keff[t]; j++)
                if (ids[(int64_t)t * k + j] == e) {
                    row_tok[r] = t;
                    pick_row[(int64_t)t * k + j] = r;
                    r++;
                }
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Opt-in 8-bit activations ([C] §2.2)                                         */
/* ------------------------------------------------------------------------- */

/* The pages' integer (IDOT) path quantises the activations to int8 once per layer and
 * is opt-in because it changes the results ([C] §2.2).  They give no quantiser; the
 * reading here: symmetric, one power-of-two step per block of consecutive values, the
 * largest step exponent that keeps the block's largest magnitude within 127. */
void moe_ref_quant_act8(const double *v, int32_t K, int32_t block, double *out) {
    for (int32_t b0 = 0; b0 < K; b0 += block) {
        const int32_t b1 = b0 + block < K ? b0 + block : K;
        double amax = 0.0;
        for (int32_t i = b0; i < b1; i++)
            if (fabs(v[i]) > amax) amax = fabs(v[i]);
        if (amax == 0.0) {
            for (int32_t i = b0; i < b1; i++) out[i] = 0.0;
            continue;
        }
        int n = 149; /* the largest n <= 149 with amax * 2^n <= 127 */
        while (ldexp(amax, n) > 127.0) n--;
        for (int32_t i = b0; i < b1; i++) out[i] = ldexp(nearbyint(ldexp(v[i], n)), -n);
    }
}

/* ------------------------------------------------------------------------- */
/* Step 4: expert FFN ([R] §1.3: gate, up, SiLU, down)                        */
/* ------------------------------------------------------------------------- */

/* act_block > 0: the opt-in 8-bit activations, x and the SwiGLU output quantised per
 * act_block values before their products. */
static int ref_swiglu_q(int32_t fmt, const uint8_t *gq, const void *gs, const uint8_t *uq,
                        const void *us, const uint8_t *dq, const void *ds, int32_t H, int32_t F,
                        const float *x, double *y, int32_t act_block) {
    if (!gq || !gs || !uq || !us || !dq || !ds || !x || !y) return REF_EINVAL;
    if (!ref_fmt_ok(fmt)) return REF_EINVAL;
    if (H <= 0 || F <= 0 || H % 64 != 0 || F % 64 != 0 || act_block < 0) return REF_EINVAL;
    double *hbuf = (double *)malloc(sizeof(double) * (size_t)F);
    double *xin = (double *)malloc(sizeof(double) * (size_t)H);
    if (!hbuf || !xin) {
        free(hbuf);
        free(xin);
        return REF_EINVAL;
    }
    for (int32_t h = 0; h < H; h++) xin[h] = (double)x[h];
    if (act_block > 0) moe_ref_quant_act8(xin, H, act_block, xin);
#pragma omp parallel for schedule(static)
    for (int32_t f = 0; f < F; f++) {
        double g = 0.0, u = 0.0;
        for (int32_t h = 0; h < H; h++) {
            g += ref_weight_fmt(fmt, gq, gs, H, f, h) * xin[h];
            u += ref_weight_fmt(fmt, uq, us, H, f, h) * xin[h];
        }
        double silu = g / (1.0 + exp(-g)); /* SiLU(g) = g * sigmoid(g) */
        hbuf[f] = silu * u;
    }
    if (act_block > 0) moe_ref_quant_act8(hbuf, F, act_block, hbuf);
#pragma omp parallel for schedule(static)
    for (int32_t n = 0; n < H; n++) {
        double acc = 0.0;
        for (int32_t f = 0; f < F; f++) acc += ref_weight_fmt(fmt, dq, ds, F, n, f) * hbuf[f];
        y[n] = acc;
    }
    free(hbuf);
    free(xin);
    return 0;
}

int moe_ref_swiglu(const uint8_t *gq, const float *gs, const uint8_t *uq, const float *us,
                   const uint8_t *dq, const float *ds, int32_t H, int32_t F,
                   const float *x, double *y) {
    return ref_swiglu_q(MOE_REF_FMT_INT4, gq, gs, uq, us, dq, ds, H, F, x, y, 0);
}

int moe_ref_swiglu_fmt(int32_t fmt, const uint8_t *gq, const void *gs, const uint8_t *uq,
                       const void *us, const uint8_t *dq, const void *ds, int32_t H, int32_t F,
                       const float *x, double *y) {
    return ref_swiglu_q(fmt, gq, gs, uq, us, dq, ds, H, F, x, y, 0);
}

/* the activation block of a layer: act_block values when the 8-bit path is on, else 0 */
static int32_t ref_act_block(const moe_ref_layer *L) { return L->act_bits == 8 ? L->act_block : 0; }

/* Expert e's tensors inside the stacked arrays. */
static void ref_expert_ptrs(const moe_ref_layer *L, int32_t e, const uint8_t **gq,
                            const void **gs, const uint8_t **uq, const void **us,
                            const uint8_t **dq, const void **ds) {
    const int64_t H = L->hidden, F = L->ffn;
    const int32_t fmt = L->fmt;
    const int64_t gu_q = F * moe_ref_code_bytes(fmt, H), gu_s = F * moe_ref_scale_bytes(fmt, H);
    const int64_t d_q = H * moe_ref_code_bytes(fmt, F), d_s = H * moe_ref_scale_bytes(fmt, F);
    *gq = L->gate_q + (int64_t)e * gu_q;
    *gs = (const uint8_t *)L->gate_s + (int64_t)e * gu_s;
    *uq = L->up_q + (int64_t)e * gu_q;
    *us = (const uint8_t *)L->up_s + (int64_t)e * gu_s;
    *dq = L->down_q + (int64_t)e * d_q;
    *ds = (const uint8_t *)L->down_s + (int64_t)e * d_s;
}

int moe_ref_expert_ffn(const moe_ref_layer *L, const float *x, int32_t T,
                       const int32_t *off, const int32_t *row_tok, double *y_rows) {
    if (!ref_layer_ok(L) || T < 0 || !off) return REF_EINVAL;
    const int32_t H = L->hidden, E = L->n_experts;
    for (int32_t e = 0; e < E; e++) {
        for (int32_t r = off[e]; r < off[e + 1]; r++) {
            const uint8_t *gq, *uq, *dq;
            const void *gs, *us, *ds;
            ref_expert_ptrs(L, e, &gq, &gs, &uq, &us, &dq, &ds);
            int32_t t = row_tok[r];
            if (t < 0 || t >= T) return REF_EINVAL;
            int rc = ref_swiglu_q(L->fmt, gq, gs, uq, us, dq, ds, H, L->ffn, x + (int64_t)t * H,
                                  y_rows + (int64_t)r * H, ref_act_block(L));
            if (rc) return rc;
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Steps 1-5: the layer ([R] §1: moe(x[S,hidden]); §1.4: shared expert added)  */
/* ------------------------------------------------------------------------- */

int moe_ref_layer_forward(const moe_ref_layer *L, const float *x, int32_t T,
                          const int32_t *toks, int32_t n_toks, double *out) {
    if (!ref_layer_ok(L) || T < 0 || (T > 0 && (!x || !out))) return REF_EINVAL;
    const int32_t H = L->hidden, E = L->n_experts;
    int32_t n_out = toks ? n_toks : T;
    if (n_out < 0) return REF_EINVAL;
    double *logit = (double *)malloc(sizeof(double) * (size_t)E);
    double *y = (double *)malloc(sizeof(double) * (size_t)H);
    int32_t ids[64];
    float w[64];
    int32_t keff = 0;
    int rc = 0;
    for (int32_t i = 0; i < n_out && rc == 0; i++) {
        int32_t t = toks ? toks[i] : i;
        if (t < 0 || t >= T) {
            rc = REF_EINVAL;
            break;
        }
        const float *xt = x + (int64_t)t * H;
        double *ot = out + (int64_t)i * H;
        rc = moe_ref_logits(L, xt, 1, logit);
        if (rc) break;
        ref_select_one(L, logit, ids, w, &keff);
        for (int32_t h = 0; h < H; h++) ot[h] = 0.0;
        /* weighted sum over the kept picks, in slot order */
        for (int32_t j = 0; j < keff && rc == 0; j++) {
            const uint8_t *gq, *uq, *dq;
            const void *gs, *us, *ds;
            ref_expert_ptrs(L, ids[j], &gq, &gs, &uq, &us, &dq, &ds);
            rc = ref_swiglu_q(L->fmt, gq, gs, uq, us, dq, ds, H, L->ffn, xt, y, ref_act_block(L));
            if (rc) break;
            for (int32_t h = 0; h < H; h++) ot[h] += (double)w[j] * y[h];
        }
        /* the shared expert: every token, weight 1, not scaled */
        if (rc == 0 && L->shared_ffn > 0) {
            rc = ref_swiglu_q(L->fmt, L->sh_gate_q, L->sh_gate_s, L->sh_up_q, L->sh_up_s,
                              L->sh_down_q, L->sh_down_s, H, L->shared_ffn, xt, y, ref_act_block(L));
            if (rc) break;
            for (int32_t h = 0; h < H; h++) ot[h] += y[h];
        }
    }
    free(logit);
    free(y);
    return rc;
}

/* [R] §1.5: the first layers are a plain MLP (dense_mlp), the same SwiGLU as an
 * expert applied to every token. */
int moe_ref_dense_mlp(const uint8_t *gq, const float *gs, const uint8_t *uq, const float *us,
                      const uint8_t *dq, const float *ds, int32_t H, int32_t F,
                      const float *x, int32_t T, double *out) {
    if (T < 0 || (T > 0 && (!x || !out))) return REF_EINVAL;
    for (int32_t t = 0; t < T; t++) {
        int rc = moe_ref_swiglu(gq, gs, uq, us, dq, ds, H, F, x + (int64_t)t * H, out + (int64_t)t * H);
        if (rc) return rc;
    }
    return 0;
}

int moe_ref_rmsnorm(const float *h, int32_t T, int32_t H, double eps, float *y) {
    if (!h || !y || T < 0 || H <= 0) return REF_EINVAL;
    for (int32_t t = 0; t < T; t++) {
        double ss = 0.0;
        for (int32_t i = 0; i < H; i++) ss += (double)h[(int64_t)t * H + i] * h[(int64_t)t * H + i];
        double r = 1.0 / sqrt(ss / H + eps);
        for (int32_t i = 0; i < H; i++) y[(int64_t)t * H + i] = (float)((double)h[(int64_t)t * H + i] * r);
    }
    return 0;
}
