/*
 * gen.c -- seeded synthetic inputs for the MoE layer (weights, biases, tokens).
 *
 * This module holds no step of the MoE forward.  It is the one source of inputs
 * for both the HIP library's tests/benchmark and the CPU oracle.
 *
 * Random numbers: a counter-based SplitMix64.  Element i of a stream with key K
 * is mix(K + (i + 1) * 0x9E3779B97F4A7C15), where mix is SplitMix64's output
 * function (Steele, Lea, Flood, "Fast splittable pseudorandom number
 * generators", OOPSLA 2014).  Uniforms in (0,1) use the top 53 bits plus half an
 * ulp; a normal is the standard normal quantile of the uniform at the same
 * counter (Acklam's approximation, below), in fp64.  Every element is a pure function of
 * (key, index), so any slice can be regenerated on its own and the generation
 * parallelises without changing a value.
 *
 * Expert weights are drawn in fp32 and turned into the int4-gs64 container by a
 * symmetric absmax quantiser (one fp32 scale per 64 consecutive K, scale =
 * max|w|/7, code = clamp(rint(w/scale), -8, 7), two codes per byte with the
 * even element in the low nibble) -- the offline conversion that produces the
 * weights the layer consumes, not a step of the layer.  The other expert formats
 * are produced the same way from the same fp32 draws:
 *  - int3-g64: scale = max|w|/3 per 64, code = clamp(rint(w/scale), -4, 3), the codes'
 *    low two bits and sign bits written into the two bit planes of the library's layout;
 *  - MXFP4 (OCP Microscaling): per 32 consecutive K the shared exponent
 *    X = floor(log2(max|w|)) - 2 (2 = the largest E2M1 exponent), stored as X + 127,
 *    and each element the E2M1 value nearest to w / 2^X (ties to the even mantissa),
 *    saturated at 6.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

uint64_t synth_key(uint64_t seed, uint64_t stream) {
    return mix64(mix64(seed + GOLDEN) ^ (stream * 0xD1B54A32D192ED03ULL + 1));
}

static inline uint64_t bits_at(uint64_t key, uint64_t i) { return mix64(key + (i + 1) * GOLDEN); }

static inline double u01_at(uint64_t key, uint64_t i) {
    return ((double)(bits_at(key, i) >> 11) + 0.5) * (1.0 / 9007199254740992.0);
}

/* Standard normal quantile by P. J. Acklam's rational approximation ("An
 * algorithm for computing the inverse normal cumulative distribution
 * function", 2003; relative error below 1.2e-9): a rational function of
 * (u - 1/2)^2 in the central region, of sqrt(-2 log u) in the tails. */
static inline double inv_normal(double u) {
    static const double a[6] = {-3.969683028665376e+01, 2.209460984245205e+02,
                                -2.759285104469687e+02, 1.383577518672690e+02,
                                -3.066479806614716e+01, 2.506628277459239e+00};
    static const double b[5] = {-5.447609879822406e+01, 1.615858368580409e+02,
                                -1.556989798598866e+02, 6.680131188771972e+01,
                                -1.328068155288572e+01};
    static const double c[6] = {-7.784894002430293e-03, -3.223964580411365e-01,
                                -2.400758277161838e+00, -2.549732539343734e+00,
                                4.374664141464968e+00, 2.938163982698783e+00};
    static const double d[4] = {7.784695709041462e-03, 3.224671290700398e-01,
                                2.445134137142996e+00, 3.754408661907416e+00};
    const double lo = 0.02425;
    if (u < lo || u > 1.0 - lo) {
        double q = sqrt(-2.0 * log(u < lo ? u : 1.0 - u));
        double v = (((((c[0] * q + c[1]) * q + c[2]) * q + c[3]) * q + c[4]) * q + c[5]) /
                   ((((d[0] * q + d[1]) * q + d[2]) * q + d[3]) * q + 1.0);
        return u < lo ? v : -v;
    }
    double q = u - 0.5, r = q * q;
    return (((((a[0] * r + a[1]) * r + a[2]) * r + a[3]) * r + a[4]) * r + a[5]) * q /
           (((((b[0] * r + b[1]) * r + b[2]) * r + b[3]) * r + b[4]) * r + 1.0);
}

static inline double normal_at(uint64_t key, uint64_t i) { return inv_normal(u01_at(key, i)); }

double synth_inv_normal(double u) { return inv_normal(u); }

void synth_u64(uint64_t key, int64_t n, uint64_t *out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) out[i] = bits_at(key, (uint64_t)i);
}

void synth_uniform_f64(uint64_t key, int64_t n, double lo, double hi, double *out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) out[i] = lo + (hi - lo) * u01_at(key, (uint64_t)i);
}

void synth_normal_f64(uint64_t key, int64_t n, double mean, double std, double *out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) out[i] = mean + std * normal_at(key, (uint64_t)i);
}

void synth_normal_f32(uint64_t key, int64_t n, double mean, double std, float *out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) out[i] = (float)(mean + std * normal_at(key, (uint64_t)i));
}

/* Quantise one group of 64 fp32 weights into 32 packed bytes and a scale. */
static void quant_group(const float *w, uint8_t *q, float *s) {
    float amax = 0.0f;
    for (int i = 0; i < 64; i++) {
        float a = fabsf(w[i]);
        amax = a > amax ? a : amax;
    }
    float sc = amax / 7.0f;
    *s = sc;
    for (int i = 0; i < 64; i += 2) {
        int c[2] = {0, 0};
        for (int h = 0; h < 2; h++) {
            if (sc > 0.0f) {
                float r = rintf(w[i + h] / sc);
                r = r > 7.0f ? 7.0f : (r < -8.0f ? -8.0f : r);
                c[h] = (int)r;
            }
        }
        q[i / 2] = (uint8_t)((c[0] & 15) | ((c[1] & 15) << 4));
    }
}

void synth_quantize_gs64(const float *w, int64_t N, int64_t K, uint8_t *q, float *s) {
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; n++)
        for (int64_t g = 0; g < K / 64; g++)
            quant_group(w + n * K + g * 64, q + n * (K / 2) + g * 32, s + n * (K / 64) + g);
}

/* W[N][K] ~ N(0, std^2) in fp32 (element n*K+k of the stream), quantised to
 * int4-gs64 without materialising the fp32 matrix. */
void synth_q4_normal(uint64_t key, int64_t N, int64_t K, double std, uint8_t *q, float *s) {
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; n++) {
        float w[64];
        for (int64_t g = 0; g < K / 64; g++) {
            for (int i = 0; i < 64; i++)
                w[i] = (float)(std * normal_at(key, (uint64_t)(n * K + g * 64 + i)));
            quant_group(w, q + n * (K / 2) + g * 32, s + n * (K / 64) + g);
        }
    }
}

/* ---- int3-g64 ---------------------------------------------------------------
 * Element i = 16d + 8a + 2b + o of a 64-group: low two bits at bits 2(2a+o).. of byte
 * 16G + 4d + b of the low plane; i = 32h + 8m + 2b + o: sign at bit 2m+o of byte
 * 8G + 4h + b of the sign plane (which starts K/4 bytes into the row). */
static void quant_group3(const float *w, uint8_t *lowp, uint8_t *signp, float *s) {
    float amax = 0.0f;
    for (int i = 0; i < 64; i++) {
        float a = fabsf(w[i]);
        amax = a > amax ? a : amax;
    }
    float sc = amax / 3.0f;
    *s = sc;
    memset(lowp, 0, 16);
    memset(signp, 0, 8);
    for (int d = 0; d < 4; d++)
        for (int a = 0; a < 2; a++)
            for (int b = 0; b < 4; b++)
                for (int o = 0; o < 2; o++) {
                    const int i = 16 * d + 8 * a + 2 * b + o;
                    int c = 0;
                    if (sc > 0.0f) {
                        float r = rintf(w[i] / sc);
                        r = r > 3.0f ? 3.0f : (r < -4.0f ? -4.0f : r);
                        c = (int)r;
                    }
                    const int bits = c & 7; /* 3-bit two's complement */
                    lowp[4 * d + b] |= (uint8_t)((bits & 3) << (2 * (2 * a + o)));
                    const int h = i / 32, m = (i / 8) % 4;
                    signp[4 * h + b] |= (uint8_t)(((bits >> 2) & 1) << (2 * m + o));
                }
}

void synth_q3_normal(uint64_t key, int64_t N, int64_t K, double std, uint8_t *q, float *s) {
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; n++) {
        float w[64];
        uint8_t *row = q + n * (3 * K / 8);
        for (int64_t g = 0; g < K / 64; g++) {
            for (int i = 0; i < 64; i++)
                w[i] = (float)(std * normal_at(key, (uint64_t)(n * K + g * 64 + i)));
            quant_group3(w, row + 16 * g, row + K / 4 + 8 * g, s + n * (K / 64) + g);
        }
    }
}

/* ---- MXFP4 ------------------------------------------------------------------ */
static const float kE2M1[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};

static void quant_block_fp4(const float *w, uint8_t *q, uint8_t *e) {
    float amax = 0.0f;
    for (int i = 0; i < 32; i++) {
        float a = fabsf(w[i]);
        amax = a > amax ? a : amax;
    }
    int X = -127;
    if (amax > 0.0f) {
        int ex;
        frexpf(amax, &ex); /* amax = f * 2^ex, f in [0.5, 1): floor(log2 amax) = ex - 1 */
        X = ex - 1 - 2;
        if (X < -127) X = -127;
        if (X > 127) X = 127;
    }
    *e = (uint8_t)(X + 127);
    for (int i = 0; i < 32; i += 2) {
        int c[2];
        for (int h = 0; h < 2; h++) {
            const double v = ldexp((double)w[i + h], -X);
            const double a = fabs(v);
            int best = 0;
            for (int m = 1; m < 8; m++) {
                const double dm = fabs(a - kE2M1[m]), db = fabs(a - kE2M1[best]);
                if (dm < db || (dm == db && (m & 1) == 0)) best = m;
            }
            c[h] = best | (v < 0.0 && best != 0 ? 8 : 0);
        }
        q[i / 2] = (uint8_t)(c[0] | (c[1] << 4));
    }
}

void synth_f4_normal(uint64_t key, int64_t N, int64_t K, double std, uint8_t *q, uint8_t *e) {
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; n++) {
        float w[32];
        for (int64_t b = 0; b < K / 32; b++) {
            for (int i = 0; i < 32; i++)
                w[i] = (float)(std * normal_at(key, (uint64_t)(n * K + b * 32 + i)));
            quant_block_fp4(w, q + n * (K / 2) + b * 16, e + n * (K / 32) + b);
        }
    }
}
