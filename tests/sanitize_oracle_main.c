/* Drives every entry point of the C oracle (oracle/moe_ref.c) on a small synthetic
 * layer, valid and invalid arguments, for a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_sanitizers.py compiles and runs it).  Exits
 * 0 when every call returns what it should; a sanitizer report aborts the run. */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../oracle/moe_ref.h"

static unsigned long long rng = 0x9E3779B97F4A7C15ull;
static float unif(void) { /* xorshift64*, uniform in [-1, 1) */
    rng ^= rng >> 12; rng ^= rng << 25; rng ^= rng >> 27;
    return (float)((double)((rng * 2685821657736338717ull) >> 11) / 9007199254740992.0 * 2.0 - 1.0);
}
static int fails = 0;
#define EXPECT(c) do { if (!(c)) { fprintf(stderr, "FAILED: %s (line %d)\n", #c, __LINE__); fails++; } } while (0)

static void quantized(int64_t N, int64_t K, float amp, uint8_t **q, float **s) {
    float *w = malloc(sizeof(float) * N * K);
    for (int64_t i = 0; i < N * K; i++) w[i] = amp * unif();
    *q = malloc(N * K / 2);
    *s = malloc(sizeof(float) * N * K / 64);
    EXPECT(moe_ref_quantize_gs64(w, N, K, *q, *s) == 0);
    double *d = malloc(sizeof(double) * N * K);
    EXPECT(moe_ref_dequantize_gs64(*q, *s, N, K, d) == 0);
    free(d);
    free(w);
}

int main(void) {
    enum { H = 128, E = 8, F = 64, FS = 64, K = 3, T = 7 };
    for (int lo = -8; lo < 8; lo++)
        for (int hi = -8; hi < 8; hi++) {
            int32_t a, b;
            moe_ref_unpack_int4(moe_ref_pack_int4(lo, hi), &a, &b);
            EXPECT(a == lo && b == hi);
        }
    moe_ref_layer L;
    memset(&L, 0, sizeof L);
    L.hidden = H; L.n_experts = E; L.ffn = F; L.shared_ffn = FS; L.top_k = K;
    L.top_p = 0.8f; L.norm_topk = 1; L.routed_scale = 2.5f;
    float *rw = malloc(sizeof(float) * E * H), *rb = malloc(sizeof(float) * E);
    for (int i = 0; i < E * H; i++) rw[i] = 0.1f * unif();
    for (int i = 0; i < E; i++) rb[i] = 0.1f * unif();
    L.router_w = rw; L.router_bias = rb;
    uint8_t *gq, *uq, *dq, *sgq, *suq, *sdq;
    float *gs, *us, *ds, *sgs, *sus, *sds;
    quantized((int64_t)E * F, H, 0.05f, &gq, &gs);
    quantized((int64_t)E * F, H, 0.05f, &uq, &us);
    quantized((int64_t)E * H, F, 0.05f, &dq, &ds);
    quantized(FS, H, 0.05f, &sgq, &sgs);
    quantized(FS, H, 0.05f, &suq, &sus);
    quantized(H, FS, 0.05f, &sdq, &sds);
    L.gate_q = gq; L.gate_s = gs; L.up_q = uq; L.up_s = us; L.down_q = dq; L.down_s = ds;
    L.sh_gate_q = sgq; L.sh_gate_s = sgs; L.sh_up_q = suq; L.sh_up_s = sus;
    L.sh_down_q = sdq; L.sh_down_s = sds;

    float *x = malloc(sizeof(float) * T * H);
    for (int i = 0; i < T * H; i++) x[i] = unif();
    double *lg = malloc(sizeof(double) * T * E);
    int32_t ids[T * K], keff[T], ids2[T * K], keff2[T];
    float w[T * K], w2[T * K];
    EXPECT(moe_ref_logits(&L, x, T, lg) == 0);
    EXPECT(moe_ref_select(&L, lg, T, ids, w, keff) == 0);
    EXPECT(moe_ref_route(&L, x, T, ids2, w2, keff2) == 0);
    EXPECT(memcmp(ids, ids2, sizeof ids) == 0 && memcmp(keff, keff2, sizeof keff) == 0);
    int32_t n_uniq, uniq[E], off[E + 1], row_tok[T * K], pick_row[T * K];
    EXPECT(moe_ref_union(E, K, ids, keff, T, &n_uniq, uniq, off, row_tok, pick_row) == 0);
    EXPECT(n_uniq >= 1 && n_uniq <= E && off[E] <= T * K);
    double *yr = malloc(sizeof(double) * T * K * H), *y1 = malloc(sizeof(double) * H);
    EXPECT(moe_ref_expert_ffn(&L, x, T, off, row_tok, yr) == 0);
    EXPECT(moe_ref_swiglu(gq, gs, uq, us, dq, ds, H, F, x, y1) == 0);
    double *out = malloc(sizeof(double) * T * H);
    EXPECT(moe_ref_layer_forward(&L, x, T, NULL, 0, out) == 0);
    for (int i = 0; i < T * H; i++) EXPECT(isfinite(out[i]));
    const int32_t toks[2] = {0, T - 1};
    EXPECT(moe_ref_layer_forward(&L, x, T, toks, 2, out) == 0);
    float *nrm = malloc(sizeof(float) * T * H);
    EXPECT(moe_ref_rmsnorm(x, T, H, 1e-6, nrm) == 0);
    /* no shared expert, no top-p, no norm */
    L.shared_ffn = 0; L.top_p = 0.0f; L.norm_topk = 0;
    EXPECT(moe_ref_layer_forward(&L, x, T, NULL, 0, out) == 0);
    /* empty batch */
    EXPECT(moe_ref_union(E, K, ids, keff, 0, &n_uniq, uniq, off, row_tok, pick_row) == 0);
    EXPECT(n_uniq == 0);
    /* invalid arguments are rejected, not dereferenced */
    EXPECT(moe_ref_logits(NULL, x, T, lg) != 0);
    EXPECT(moe_ref_route(&L, NULL, T, ids, w, keff) != 0);
    EXPECT(moe_ref_quantize_gs64(x, 1, 63, gq, gs) != 0);
    EXPECT(moe_ref_dequantize_gs64(NULL, gs, 1, 64, lg) != 0);
    L.top_k = E + 1;
    EXPECT(moe_ref_route(&L, x, T, ids, w, keff) != 0);

    free(rw); free(rb); free(gq); free(gs); free(uq); free(us); free(dq); free(ds);
    free(sgq); free(sgs); free(suq); free(sus); free(sdq); free(sds);
    free(x); free(lg); free(yr); free(y1); free(out); free(nrm);
    if (fails) return 1;
    printf("oracle sanitizer run ok\n");
    return 0;
}
