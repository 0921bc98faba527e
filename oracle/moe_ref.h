/*
 * moe_ref.h -- plain CPU oracle of the sparse MoE layer forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or calls
 * this library; only the tests, the smoke check and the CPU-baseline leg of the
 * benchmark do.  It shares no source with the HIP library.
 *
 * It follows the colibrì MoE forward as described in
 *   [R] "MoE 路由与专家流式加载" (colibri-analysis 07, blog.chen3feng.top), §1.1-§1.4
 *   [Q] "colibrì 深度拆解：1300行纯C代码驱动7440亿参数大模型" (chenxutan.com), §5.2
 *   [C] "colibri 开发演进实录：从 CHANGELOG 看多引擎 MoE 推理框架的工程迭代脉络"
 *       (framerc.cn), §2.1 (int4-gs64 container) and §2.2 (K1 offset identity)
 *
 * All arithmetic is fp64 unless stated.  All pointers are host pointers owned
 * by the caller.  Functions returning int return 0 on success and a negative
 * value on an invalid argument; they never allocate caller-visible memory.
 *
 * Weight format (int4-gs64): a matrix W[N][K] (y = W x, K contiguous) is
 *   q : uint8 [N][K/2], element 2j in the low nibble of byte j, 2j+1 in the
 *       high nibble, two's complement ([Q] §5.2 pack/unpack);
 *   s : fp32  [N][K/64], one scale per 64 consecutive K ([C] §2.1);
 *   W[n][k] = q(n,k) * s[n][k/64].
 * Routed experts are stacked by expert id: gate/up [E][F][H/2] (+ [E][F][H/64]),
 * down [E][H][F/2] (+ [E][H][F/64]).
 *
 * Other expert formats (moe_ref_layer.fmt; one format for the routed and the shared
 * experts), W[N][K] with K a multiple of 64:
 *   MOE_REF_FMT_MXFP4 -- fp4 experts with UE8M0 block scales ([C] §五; the MXFP4
 *       experts of [C] §六): OCP MX FP4, i.e. E2M1 codes (bit 3 sign, bits 2-1 exponent
 *       with bias 1, bit 0 mantissa) packed two per byte like int4 (element 2j in the
 *       low nibble), q : uint8 [N][K/2]; s : uint8 [N][K/32], one UE8M0 exponent per
 *       32 consecutive elements; W[n][k] = e2m1(q(n,k)) * 2^(s[n][k/32] - 127), and an
 *       exponent byte of 255 is NaN.
 *   MOE_REF_FMT_INT3 -- int3-g64 ([C] §8.3, fmt=5: 3-bit weights with one scale per 64):
 *       codes c in [-4, 3], W[n][k] = c * s[n][k/64], s : fp32 [N][K/64];
 *       q : uint8 [N][3K/8], per row two bit planes: bytes [0, K/4) the codes' low two
 *       bits, bytes [K/4, 3K/8) their sign bits (c = low - 4 sign).  For element
 *       i = 16d + 8a + 2b + o (d < 4, a < 2, b < 4, o < 2) of 64-group G, its low bits
 *       are bits 2(2a+o) and 2(2a+o)+1 of byte 16G + 4d + b, and writing the same
 *       i = 32h + 8m + 2b + o (h < 2, m < 4), its sign bit is bit 2m+o of byte
 *       K/4 + 8G + 4h + b.  (The pages fix no bit layout; this one is the library's.)
 * The scale pointers are untyped for that reason (fp32 or uint8 elements).
 */
#ifndef MOE_REF_H
#define MOE_REF_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
    int32_t hidden;       /* H */
    int32_t n_experts;    /* E */
    int32_t ffn;          /* F: routed expert FFN width */
    int32_t shared_ffn;   /* Fs: shared expert FFN width, 0 = no shared expert */
    int32_t top_k;        /* k */
    float top_p;          /* 0 = off, else (0,1]; 1 keeps all k */
    int32_t norm_topk;    /* 0/1 */
    float routed_scale;
    const float *router_w;     /* [E][H] */
    const float *router_bias;  /* [E] or NULL (= 0) */
    const uint8_t *gate_q; const void *gate_s;   /* int4: [E][F][H/2], [E][F][H/64] */
    const uint8_t *up_q;   const void *up_s;     /* int4: [E][F][H/2], [E][F][H/64] */
    const uint8_t *down_q; const void *down_s;   /* int4: [E][H][F/2], [E][H][F/64] */
    const uint8_t *sh_gate_q; const void *sh_gate_s;  /* int4: [Fs][H/2], [Fs][H/64] */
    const uint8_t *sh_up_q;   const void *sh_up_s;
    const uint8_t *sh_down_q; const void *sh_down_s;  /* int4: [H][Fs/2], [H][Fs/64] */
    int32_t n_group;      /* expert groups for group-limited routing; 0 or 1 = none */
    int32_t topk_group;   /* groups kept when n_group > 1 */
    int32_t act_bits;     /* 8: the opt-in 8-bit activations (below); 0 = exact */
    int32_t act_block;    /* values per activation block when act_bits == 8 */
    int32_t fmt;          /* expert weight format, MOE_REF_FMT_* (0 = int4-gs64) */
} moe_ref_layer;

enum { MOE_REF_FMT_INT4 = 0, MOE_REF_FMT_MXFP4 = 1, MOE_REF_FMT_INT3 = 2 };

/* ---- int4 codec ([Q] §5.2) ------------------------------------------------ */
uint8_t moe_ref_pack_int4(int32_t lo, int32_t hi);
void moe_ref_unpack_int4(uint8_t b, int32_t *lo, int32_t *hi);
/* Symmetric absmax int4-gs64 quantiser: s = max|w_g|/7 (fp32), q = clamp(rint(w/s),-8,7),
 * all-zero group -> s = 0, q = 0.  K must be a multiple of 64. */
int moe_ref_quantize_gs64(const float *w, int64_t N, int64_t K, uint8_t *q, float *s);
/* W[n][k] = q*s in fp64 (exact). */
int moe_ref_dequantize_gs64(const uint8_t *q, const float *s, int64_t N, int64_t K, double *w);

/* ---- the other expert formats (above) -------------------------------------- */
/* Value of an E2M1 code (low four bits of `code`): 0, 0.5, 1, 1.5, 2, 3, 4, 6, signed. */
double moe_ref_e2m1(uint8_t code);
/* UE8M0 exponent byte: 2^(e - 127), NaN for 255. */
double moe_ref_ue8m0(uint8_t e);
/* Code of element k (0 <= k < K) of one int3-g64 row (3K/8 bytes), in [-4, 3]. */
int32_t moe_ref_int3_code(const uint8_t *row_q, int64_t K, int64_t k);
/* Row bytes of the codes and of the scales of one row of K elements in format fmt. */
int64_t moe_ref_code_bytes(int32_t fmt, int64_t K);
int64_t moe_ref_scale_bytes(int32_t fmt, int64_t K);
/* W[n][k] in fp64 (exact: a code times a power of two or an fp32 scale) for any format. */
int moe_ref_dequantize(int32_t fmt, const uint8_t *q, const void *s, int64_t N, int64_t K, double *w);

/* ---- steps 1-2: routing ([R] §1.1-§1.2) ---------------------------------- */
/* logits[t][e] = sum_h x[t][h] * Wr[e][h] in fp64 (products of fp32 exact). */
int moe_ref_logits(const moe_ref_layer *L, const float *x, int32_t T, double *logits);
/* noaux_tc selection from logits: ids [T][k] (selection order, -1 padding past keff),
 * w [T][k] fp32 (0 padding), keff [T]. */
int moe_ref_select(const moe_ref_layer *L, const double *logits, int32_t T,
                   int32_t *ids, float *w, int32_t *keff);
int moe_ref_route(const moe_ref_layer *L, const float *x, int32_t T,
                  int32_t *ids, float *w, int32_t *keff);

/* ---- step 3: batch union and token permutation ([R] §1.3) ---------------- */
/* n_uniq[1]; uniq [E] ascending (first n_uniq valid, rest -1); off [E+1] exclusive
 * prefix of per-expert counts; row_tok [T*k] (first off[E] valid, rest -1), rows ordered
 * by (expert, token) ascending; pick_row [T*k] row of pick (t,j) or -1. */
int moe_ref_union(int32_t E, int32_t k, const int32_t *ids, const int32_t *keff, int32_t T,
                  int32_t *n_uniq, int32_t *uniq, int32_t *off, int32_t *row_tok,
                  int32_t *pick_row);

/* ---- opt-in 8-bit activations ([C] §2.2) --------------------------------- */
/* Each block of `block` consecutive values of v[K] (the last one may be shorter) is
 * replaced by c * 2^-n with n the largest integer (at most 149) for which
 * max|v_block| * 2^n <= 127 and c = rint(v * 2^n) (round half to even), in [-127, 127];
 * an all-zero block stays zero.  out may alias v. */
void moe_ref_quant_act8(const double *v, int32_t K, int32_t block, double *out);

/* ---- step 4: one expert's SwiGLU FFN on one token ([R] §1.3) ------------- */
/* y[H] = Wd * (silu(Wg x) .* (Wu x)); Wg/Wu [F][H], Wd [H][F] (int4-gs64). */
int moe_ref_swiglu(const uint8_t *gq, const float *gs, const uint8_t *uq, const float *us,
                   const uint8_t *dq, const float *ds, int32_t H, int32_t F,
                   const float *x, double *y);
/* The same in any format (scale arrays as described above). */
int moe_ref_swiglu_fmt(int32_t fmt, const uint8_t *gq, const void *gs, const uint8_t *uq,
                       const void *us, const uint8_t *dq, const void *ds, int32_t H, int32_t F,
                       const float *x, double *y);
/* y_rows[r][H] = FFN_{e(r)}(x[row_tok[r]]) for every row r < off[E] of the union
 * (unweighted); the rows past off[E] are left untouched. */
int moe_ref_expert_ffn(const moe_ref_layer *L, const float *x, int32_t T,
                       const int32_t *off, const int32_t *row_tok, double *y_rows);

/* ---- steps 1-5: the layer, token by token ([R] §1, §1.4) ----------------- */
/* out[t][h] = sum_{j<keff_t} w_tj * FFN_{e_tj}(x_t) + FFN_shared(x_t), in fp64.
 * When toks != NULL only the n_toks listed tokens are computed and out is
 * [n_toks][H] in list order; otherwise out is [T][H]. */
int moe_ref_layer_forward(const moe_ref_layer *L, const float *x, int32_t T,
                          const int32_t *toks, int32_t n_toks, double *out);

/* ---- first-dense layers ([R] §1.5) ---------------------------------------- */
/* out[t] = Wd (silu(Wg x_t) .* (Wu x_t)) for every token: the plain SwiGLU MLP of the
 * first layers; Wg/Wu [F][H], Wd [H][F] int4-gs64; out [T][H] fp64. */
int moe_ref_dense_mlp(const uint8_t *gq, const float *gs, const uint8_t *uq, const float *us,
                      const uint8_t *dq, const float *ds, int32_t H, int32_t F,
                      const float *x, int32_t T, double *out);

/* RMSNorm (gamma = 1): y = h / sqrt(mean(h^2) + eps), fp64 internally, fp32 out. */
int moe_ref_rmsnorm(const float *h, int32_t T, int32_t H, double eps, float *y);

#ifdef __cplusplus
}
#endif
#endif
