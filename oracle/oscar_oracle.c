/*
 * CPU oracle for the OSCAR three-segment INT2 KV pool: the per-token codec.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the test-suite, the smoke check and the benchmark's
 * CPU-baseline leg do.  It shares no code, header or constant table with the
 * HIP library: it is written from the description of the method, plainly
 * and slowly, so that a reader can check it against that description.
 *
 * Source of the method: the news article on OSCAR ("Beyond TurboQuant:
 * Together AI brings 2-bit KV Cache to real serving", sanyangsrq.com),
 * section "From offline calibration to online inference": the oldest recent
 * token is rotated, clipped, quantized and packed, four 2-bit values to a
 * byte; section "Not better vector compression but protecting attention":
 * 2-bit integers give four discrete levels; the decode kernel dequantizes
 * with a scale and a zero point.
 *
 * Readings where the article is silent:
 *   - the rotation acts on row vectors, y = x R, evaluated per output
 *     channel j as a fused-multiply-add chain over i = 0..d-1 in fp32,
 *     starting from +0;
 *   - clipping is symmetric per rotated channel: y <- min(max(y, -c), c);
 *   - quantization is asymmetric min/max per group of G consecutive rotated
 *     channels: s = fp16((max - min) / 3), z = fp16(min), both rounded to
 *     nearest even; codes use the fp16-rounded s and z:
 *     code = clamp(rint((y - z) / s), 0, 3), rint rounding half to even;
 *     s == 0 gives code 0 everywhere; a zero range or minimum is stored as
 *     +0 whatever the sign of the zeros it came from;
 *   - four codes of consecutive channels share a byte, first channel in the
 *     least significant bits.
 * All fp32 operations are IEEE binary32 with correctly rounded results
 * (fmaf, subtraction, division, rintf); build without -ffast-math and with
 * -ffp-contract=off.
 *
 * Parity pins (tests/test_oracle_codec.py): binary16 conversion against
 * numpy on ties and sub-normals, pack/unpack over all 256 bytes, a hand
 * worked FMA-chain rounding case, grid round trip, ties to even, constant
 * groups, the closed-form reconstruction bound.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* ---- number formats ---------------------------------------------------- */

/* bf16 is the upper half of a binary32 pattern, so widening is exact. */
static float bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Value of a binary16 bit pattern (exact in binary32). */
float oracle_f16_to_f32(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);                 /* zero or sub-normal */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25);     /* (1 + m/1024) 2^(e-15) */
    return (float)(sign ? -v : v);
}

/* Nearest binary16 (ties to even) of a binary32 value.  The value is first
 * divided by the binary16 quantum of its binade (a power of two, so exact),
 * rounded to an integer half-to-even, then re-encoded. */
uint16_t oracle_f32_to_f16(float f)
{
    uint16_t sign = signbit(f) ? 0x8000 : 0;
    double a = fabs((double)f);
    if (isnan(f))
        return 0x7e00;
    /* 65504 is the largest finite value; the midpoint to the next binade
     * (65520) and everything above round to infinity. */
    if (a >= 65520.0)
        return sign | 0x7c00;
    int e;                              /* a = frac * 2^e, frac in [0.5, 1) */
    frexp(a, &e);
    int unbiased = e - 1;               /* a in [2^unbiased, 2^(unbiased+1)) */
    if (a == 0.0 || unbiased < -14)
        unbiased = -14;                 /* sub-normal binade shares 2^-24 quantum */
    double quantum = ldexp(1.0, unbiased - 10);
    double n = nearbyint(a / quantum); /* default rounding mode: half to even */
    double r = n * quantum;
    if (r < ldexp(1.0, -14))           /* zero or sub-normal: mantissa = r / 2^-24 */
        return sign | (uint16_t)(r / ldexp(1.0, -24));
    frexp(r, &e);
    int be = e - 1;                     /* r may have carried into the next binade */
    uint16_t mant = (uint16_t)(r / ldexp(1.0, be - 10) - 1024.0);
    return sign | (uint16_t)((be + 15) << 10) | mant;
}

/* ---- per-token codec ---------------------------------------------------- */

/* y = x R for one bf16 row vector x[d]; R is row-major fp32 [d][d]. */
void oracle_rotate(const uint16_t *x, const float *R, int d, float *y)
{
    for (int j = 0; j < d; ++j) {
        float acc = 0.0f;
        for (int i = 0; i < d; ++i)
            acc = fmaf(bf16_to_f32(x[i]), R[(size_t)i * d + j], acc);
        y[j] = acc;
    }
}

/* Symmetric per-channel clip. */
void oracle_clip(float *y, const float *c, int d)
{
    for (int j = 0; j < d; ++j)
        y[j] = fminf(fmaxf(y[j], -c[j]), c[j]);
}

/* Asymmetric 4-level quantization of y[d] in groups of G channels.
 * codes[d] receive values 0..3; scale16/zero16[d/G] the fp16 parameters. */
void oracle_quantize(const float *y, int d, int G, uint8_t *codes,
                     uint16_t *scale16, uint16_t *zero16)
{
    for (int g = 0; g < d / G; ++g) {
        const float *v = y + g * G;
        float mn = v[0], mx = v[0];
        for (int k = 1; k < G; ++k) {
            mn = fminf(mn, v[k]);
            mx = fmaxf(mx, v[k]);
        }
        /* "+ 0.0f" maps a zero of either sign to +0, so an exactly zero
         * range or minimum is always stored as the +0 pattern */
        float range = (mx - mn) + 0.0f;
        uint16_t s16 = oracle_f32_to_f16(range / 3.0f);
        uint16_t z16 = oracle_f32_to_f16(mn + 0.0f);
        float s = oracle_f16_to_f32(s16);
        float z = oracle_f16_to_f32(z16);
        for (int k = 0; k < G; ++k) {
            float q = 0.0f;
            if (s != 0.0f) {
                q = rintf((v[k] - z) / s);
                q = fminf(fmaxf(q, 0.0f), 3.0f);
            }
            codes[g * G + k] = (uint8_t)q;
        }
        scale16[g] = s16;
        zero16[g] = z16;
    }
}

/* Four 2-bit codes per byte, first code in the low bits. */
void oracle_pack(const uint8_t *codes, int n, uint8_t *bytes)
{
    for (int b = 0; b < n / 4; ++b)
        bytes[b] = (uint8_t)(codes[4 * b] | (codes[4 * b + 1] << 2) |
                             (codes[4 * b + 2] << 4) | (codes[4 * b + 3] << 6));
}

void oracle_unpack(const uint8_t *bytes, int n, uint8_t *codes)
{
    for (int i = 0; i < n; ++i)
        codes[i] = (bytes[i / 4] >> (2 * (i % 4))) & 3;
}

/* Encode N bf16 vectors: rotate, clip, quantize, pack.
 * x: [N][d] bf16; packed: [N][d/4]; scale16, zero16: [N][d/G]. */
void oracle_encode(const uint16_t *x, long N, int d, int G, const float *R,
                   const float *clip, uint8_t *packed, uint16_t *scale16,
                   uint16_t *zero16)
{
    float y[512];
    uint8_t codes[512];
    for (long t = 0; t < N; ++t) {
        oracle_rotate(x + t * d, R, d, y);
        oracle_clip(y, clip, d);
        oracle_quantize(y, d, G, codes, scale16 + t * (d / G), zero16 + t * (d / G));
        oracle_pack(codes, d, packed + t * (d / 4));
    }
}

/* Rotate N vectors without clipping (used by clip calibration). */
void oracle_rotate_many(const uint16_t *x, long N, int d, const float *R, float *y)
{
    for (long t = 0; t < N; ++t)
        oracle_rotate(x + t * d, R, d, y + t * d);
}

/* ---- Lloyd-Max codebook variant -----------------------------------------
 * Reading of the article's section "Why this matters for long-context
 * agents" (the OSCAR code combines the rotation with a Lloyd-Max codebook):
 * a group keeps its fp16 scale s and zero point z, but its four levels are
 * z + (L_k / 64) s for a codebook L_0 <= L_1 <= L_2 <= L_3 of integers in
 * 0..255 (one per kv head and K|V, fitted offline), instead of z + k s.  A
 * channel takes the nearest level: with u = (y - z) / s (fp32, correctly
 * rounded), code = [u > t_0] + [u > t_1] + [u > t_2], t_k = (L_k + L_{k+1})
 * / 128 (exact in fp32), so a value midway between two levels takes the
 * lower one; s == 0 gives code 0.
 */

/* u = (y - z) / s of every channel of y[d] (slightly negative for a group's
 * minimum when fp16 rounds z above it); channels of a group with s == 0 get
 * NaN (they carry no information for a codebook fit). */
void oracle_normalized(const float *y, int d, int G, float *u)
{
    uint8_t codes[512];
    uint16_t s16[512], z16[512];
    oracle_quantize(y, d, G, codes, s16, z16); /* the group's s and z */
    for (int g = 0; g < d / G; ++g) {
        float s = oracle_f16_to_f32(s16[g]);
        float z = oracle_f16_to_f32(z16[g]);
        for (int k = 0; k < G; ++k)
            u[g * G + k] = s != 0.0f ? (y[g * G + k] - z) / s : NAN;
    }
}

/* Quantization of y[d] with codebook L[4]: codes 0..3, fp16 s and z. */
void oracle_quantize_lut(const float *y, int d, int G, const uint8_t *L,
                         uint8_t *codes, uint16_t *scale16, uint16_t *zero16)
{
    float t[3];
    for (int k = 0; k < 3; ++k)
        t[k] = (float)(L[k] + L[k + 1]) / 128.0f;
    oracle_quantize(y, d, G, codes, scale16, zero16); /* the group's s and z */
    for (int g = 0; g < d / G; ++g) {
        float s = oracle_f16_to_f32(scale16[g]);
        float z = oracle_f16_to_f32(zero16[g]);
        for (int k = 0; k < G; ++k) {
            int c = 0;
            if (s != 0.0f) {
                float u = (y[g * G + k] - z) / s;
                c = (u > t[0]) + (u > t[1]) + (u > t[2]);
            }
            codes[g * G + k] = (uint8_t)c;
        }
    }
}

/* Encode N bf16 vectors with codebook L: rotate, clip, quantize, pack. */
void oracle_encode_lut(const uint16_t *x, long N, int d, int G, const float *R,
                       const float *clip, const uint8_t *L, uint8_t *packed,
                       uint16_t *scale16, uint16_t *zero16)
{
    float y[512];
    uint8_t codes[512];
    for (long t = 0; t < N; ++t) {
        oracle_rotate(x + t * d, R, d, y);
        oracle_clip(y, clip, d);
        oracle_quantize_lut(y, d, G, L, codes, scale16 + t * (d / G), zero16 + t * (d / G));
        oracle_pack(codes, d, packed + t * (d / 4));
    }
}

/* Normalised values u[N][d] of N bf16 vectors (rotate, clip, then u). */
void oracle_normalized_many(const uint16_t *x, long N, int d, int G, const float *R,
                            const float *clip, float *u)
{
    float y[512];
    for (long t = 0; t < N; ++t) {
        oracle_rotate(x + t * d, R, d, y);
        oracle_clip(y, clip, d);
        oracle_normalized(y, d, G, u + t * d);
    }
}
