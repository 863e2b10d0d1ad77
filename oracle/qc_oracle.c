/*
 * qc_oracle.c -- CPU oracle for the quantized-communication codec.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke
 * check and the CPU-baseline leg of the benchmark may load this library.
 * It shares no source with the GPU library.
 *
 * Build: gcc -std=c11 -O2 -ffp-contract=off -fno-fast-math -fPIC -shared
 *        qc_oracle.c -lm
 * Every fp32 expression below is evaluated as written: one rounding per
 * operation, round-to-nearest-even, no fused multiply-add, denormals kept.
 *
 * Page abbreviations are defined in qc_oracle.h.
 */
#include "qc_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* small helpers                                                       */
/* ------------------------------------------------------------------ */

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

static uint32_t f32_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float    f32_from(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

static void put_word(uint8_t* p, int64_t w, uint32_t v)
{
    p[4 * w + 0] = (uint8_t)(v);
    p[4 * w + 1] = (uint8_t)(v >> 8);
    p[4 * w + 2] = (uint8_t)(v >> 16);
    p[4 * w + 3] = (uint8_t)(v >> 24);
}

static uint32_t get_word(const uint8_t* p, int64_t w)
{
    return (uint32_t)p[4 * w] | ((uint32_t)p[4 * w + 1] << 8) |
           ((uint32_t)p[4 * w + 2] << 16) | ((uint32_t)p[4 * w + 3] << 24);
}

/* 4-bit code of element i (least significant nibble first in each word). */
static uint32_t get_nibble(const uint8_t* p, int64_t i)
{
    return (get_word(p, i / 8) >> (4 * (i % 8))) & 0xFu;
}

static void or_nibble(uint8_t* p, int64_t i, uint32_t code)
{
    put_word(p, i / 8, get_word(p, i / 8) | (code << (4 * (i % 8))));
}

/* 2-bit code of element i (least significant pair first in each word). */
static uint32_t get_crumb(const uint8_t* p, int64_t i)
{
    return (get_word(p, i / 16) >> (2 * (i % 16))) & 0x3u;
}

static void or_crumb(uint8_t* p, int64_t i, uint32_t code)
{
    put_word(p, i / 16, get_word(p, i / 16) | (code << (2 * (i % 16))));
}

static uint32_t get_bit(const uint8_t* p, int64_t i)
{
    return (get_word(p, i / 32) >> (i % 32)) & 1u;
}

static void or_bit(uint8_t* p, int64_t i, uint32_t b)
{
    put_word(p, i / 32, get_word(p, i / 32) | (b << (i % 32)));
}

int64_t qco_payload_bytes(int32_t fmt, int64_t n, int32_t bits)
{
    int64_t code_bytes;
    if (fmt == QCO_SIGN)
        code_bytes = 4 * ceil_div(n, 32);
    else if (fmt == QCO_TERNARY || (fmt == QCO_UNIFORM && bits == 2))
        code_bytes = 4 * ceil_div(n, 16);
    else if (fmt == QCO_QSGD || (fmt == QCO_UNIFORM && bits == 4))
        code_bytes = 4 * ceil_div(n, 8);
    else
        code_bytes = n; /* one byte per element: INT8 and FP8 */
    return ceil_div(code_bytes, 16) * 16;
}

/* A uniform draw in [0, 1) for global element index g: the top 24 bits of
 * word g%4 of Philox4x32-10 with key = seed (low word first) and counter =
 * (g/4 low word, g/4 high word, 0, 0), scaled by 2^-24 (exact). */
static float uniform_draw(uint64_t seed, uint64_t g)
{
    const uint32_t key[2] = { (uint32_t)seed, (uint32_t)(seed >> 32) };
    const uint64_t blk = g >> 2;
    const uint32_t ctr[4] = { (uint32_t)blk, (uint32_t)(blk >> 32), 0u, 0u };
    uint32_t r[4];
    qco_philox4x32_10(ctr, key, r);
    return (float)(r[g & 3u] >> 8) * 0x1p-24f;
}

/* ------------------------------------------------------------------ */
/* contiguous pairwise summation                                        */
/* ------------------------------------------------------------------ */
/* The pages do not fix a summation order for the bucket statistics; the
 * reading taken is the contiguous pairwise tree: the sum of a block of
 * 2^k terms is the sum of its first half plus the sum of its second half.
 * A short bucket is padded with +0 up to the full power of two. */

static float pair_sum(const float* a, int64_t len)
{
    if (len == 1)
        return a[0];
    float left = pair_sum(a, len / 2);
    float right = pair_sum(a + len / 2, len / 2);
    return left + right;
}

float qco_tree_sum(const float* terms, int64_t len, int64_t pow2len)
{
    float* padded = (float*)malloc((size_t)pow2len * sizeof(float));
    for (int64_t i = 0; i < pow2len; ++i)
        padded[i] = (i < len) ? terms[i] : 0.0f;
    float s = pair_sum(padded, pow2len);
    free(padded);
    return s;
}

/* ------------------------------------------------------------------ */
/* Philox4x32-10                                                        */
/* ------------------------------------------------------------------ */
/* Counter-based generator of Salmon, Moraes, Dror and Shaw ("Parallel
 * random numbers: as easy as 1, 2, 3", SC'11).  One round multiplies
 * counter words 0 and 2 by two fixed odd constants, keeps both halves of
 * each 64-bit product, and mixes the high halves with the other two
 * counter words and the key; the key advances by two Weyl constants
 * between rounds.  Ten rounds. */

void qco_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4])
{
    const uint32_t mult0 = 0xD2511F53u, mult1 = 0xCD9E8D57u;
    const uint32_t weyl0 = 0x9E3779B9u, weyl1 = 0xBB67AE85u;
    uint32_t x0 = ctr[0], x1 = ctr[1], x2 = ctr[2], x3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += weyl0;
            k1 += weyl1;
        }
        uint64_t p0 = (uint64_t)mult0 * x0;
        uint64_t p1 = (uint64_t)mult1 * x2;
        uint32_t y0 = (uint32_t)(p1 >> 32) ^ x1 ^ k0;
        uint32_t y1 = (uint32_t)p1;
        uint32_t y2 = (uint32_t)(p0 >> 32) ^ x3 ^ k1;
        uint32_t y3 = (uint32_t)p0;
        x0 = y0; x1 = y1; x2 = y2; x3 = y3;
    }
    out[0] = x0; out[1] = x1; out[2] = x2; out[3] = x3;
}

/* ------------------------------------------------------------------ */
/* OCP FP8 E4M3FN                                                       */
/* ------------------------------------------------------------------ */
/* 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits; no infinities;
 * largest finite magnitude 448 (code 0x7E); codes 0x7F/0xFF are NaN and
 * are never produced here.  Exponent field 0 holds subnormals m * 2^-9. */

uint8_t qco_e4m3_from_f32(float y)
{
    uint8_t sign = (f32_bits(y) >> 31) ? 0x80 : 0x00;
    double a = fabs((double)y);          /* exact */
    if (a < ldexp(1.0, -6)) {
        /* subnormal range: nearest multiple of 2^-9, ties to even.  A
         * result of 8 is the smallest normal, 2^-6, whose code is also 8. */
        double m = rint(a * 512.0);      /* a*512 is exact */
        return (uint8_t)(sign | (uint8_t)m);
    }
    int e2;
    double frac = frexp(a, &e2);         /* a = frac * 2^e2, frac in [0.5,1) */
    int e = e2 - 1;                      /* a = s * 2^e, s in [1,2) */
    double s = frac * 2.0;
    double m = rint((s - 1.0) * 8.0);    /* 3 fraction bits, ties to even */
    if (m == 8.0) {                      /* rounded up to the next binade */
        m = 0.0;
        e += 1;
    }
    return (uint8_t)(sign | (uint8_t)((e + 7) << 3) | (uint8_t)m);
}

void qco_e4m3_from_f32_n(const float* y, int64_t n, uint8_t* out)
{
    for (int64_t i = 0; i < n; ++i) {
        float v = y[i];
        if (v > 448.0f) v = 448.0f;
        if (v < -448.0f) v = -448.0f;
        out[i] = qco_e4m3_from_f32(v);
    }
}

float qco_e4m3_to_f32(uint8_t c)
{
    int e = (c >> 3) & 0xF;
    int m = c & 0x7;
    double mag = (e == 0) ? ldexp((double)m, -9) : ldexp(8.0 + m, e - 10);
    float v = (float)mag;                /* exact: at most 4 significant bits */
    return (c & 0x80) ? -v : v;
}

/* ------------------------------------------------------------------ */
/* uniform affine quantization  [QCD, "Quantization Schemes": uniform]  */
/* ------------------------------------------------------------------ */
/* For a bucket with extremes mn, mx and L = 2^bits - 1 levels:
 *   scale = (mx - mn) / L,  q = round((v - mn) / scale),  DQ = q*scale + mn.
 * With error feedback [QCD, "Error Feedback for Quantization": the
 * implementation steps; GCQC, "Error feedback is the component that makes
 * it work"]: v = e + g; q = Q(v); e = v - DQ(q).
 * Readings: round is round-half-to-even; mn and mx are made +0 if they are
 * -0; a bucket with mx == mn has scale 0 and all codes 0 (DQ = mn). */

static float uniform_dq(uint32_t q, float scale, float zero)
{
    float p = (float)q * scale;
    return p + zero;
}

/* Uniform codes of 8, 4 or 2 bits: byte i, nibble i, or 2-bit field i. */
static void put_uniform_code(uint8_t* payload, int64_t i, int32_t bits, uint32_t q)
{
    if (bits == 8)
        payload[i] = (uint8_t)q;
    else if (bits == 4)
        or_nibble(payload, i, q);
    else
        or_crumb(payload, i, q);
}

static uint32_t get_uniform_code(const uint8_t* payload, int64_t i, int32_t bits)
{
    if (bits == 8)
        return payload[i];
    return bits == 4 ? get_nibble(payload, i) : get_crumb(payload, i);
}

/* The affine grid of one bucket, then one code per element: nearest level
 * (round half to even) or, when `stochastic`, the lower level plus one with
 * probability equal to the fractional part [QCD, "Quantization Schemes":
 * stochastic quantization; GQC, "Quantization Schemes"], the draw for
 * element i being uniform_draw(seed, elem_offset + i). */
static void encode_uniform_any(const float* x, float* ef, int64_t n, int32_t bucket, int32_t bits,
                               int stochastic, uint64_t seed, uint64_t elem_offset,
                               uint8_t* payload, float* scale, float* zero)
{
    const uint32_t L = (1u << bits) - 1u;
    const int64_t nb = ceil_div(n, bucket);
    memset(payload, 0, (size_t)qco_payload_bytes(QCO_UNIFORM, n, bits));
    float* v = (float*)malloc((size_t)bucket * sizeof(float));

    for (int64_t k = 0; k < nb; ++k) {
        const int64_t lo = k * bucket;
        const int64_t cnt = (lo + bucket <= n) ? bucket : n - lo;

        for (int64_t j = 0; j < cnt; ++j)
            v[j] = ef ? ef[lo + j] + x[lo + j] : x[lo + j];

        float mn = v[0], mx = v[0];
        for (int64_t j = 1; j < cnt; ++j) {
            if (v[j] < mn) mn = v[j];
            if (v[j] > mx) mx = v[j];
        }
        mn = mn + 0.0f; /* -0 -> +0 */
        mx = mx + 0.0f;

        const float sc = (mx - mn) / (float)L;
        for (int64_t j = 0; j < cnt; ++j) {
            const int64_t i = lo + j;
            uint32_t q = 0;
            if (sc != 0.0f) {
                float t = (v[j] - mn) / sc;
                float r;
                if (stochastic) {
                    float fl = floorf(t);
                    float frac = t - fl; /* exact */
                    r = fl + (uniform_draw(seed, elem_offset + (uint64_t)i) < frac ? 1.0f : 0.0f);
                } else {
                    r = rintf(t);
                }
                if (r < 0.0f) r = 0.0f;
                if (r > (float)L) r = (float)L;
                q = (uint32_t)r;
            }
            put_uniform_code(payload, i, bits, q);
            if (ef)
                ef[i] = v[j] - uniform_dq(q, sc, mn);
        }
        scale[k] = sc;
        zero[k] = mn;
    }
    free(v);
}

void qco_encode_uniform(const float* x, float* ef, int64_t n, int32_t bucket,
                        int32_t bits, uint8_t* payload, float* scale, float* zero)
{
    encode_uniform_any(x, ef, n, bucket, bits, 0, 0, 0, payload, scale, zero);
}

void qco_encode_uniform_stochastic(const float* x, float* ef, int64_t n, int32_t bucket,
                                   int32_t bits, uint64_t seed, uint64_t elem_offset,
                                   uint8_t* payload, float* scale, float* zero)
{
    encode_uniform_any(x, ef, n, bucket, bits, 1, seed, elem_offset, payload, scale, zero);
}

void qco_decode_uniform(const uint8_t* payload, const float* scale, const float* zero,
                        int64_t n, int32_t bucket, int32_t bits, float* out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = uniform_dq(get_uniform_code(payload, i, bits), scale[i / bucket], zero[i / bucket]);
}

/* ------------------------------------------------------------------ */
/* rowwise FP8  [QCDT, "Numeric Example" and "Pinterest QComms Example"] */
/* ------------------------------------------------------------------ */
/* Each embedding row is sent as one E4M3 byte per value plus one fp32
 * scale.  Reading: scale = amax/448 so the largest |value| lands on the
 * largest finite code; y = x/scale is rounded to fp32 first, clamped to
 * [-448, 448], then rounded to E4M3 (ties to even).  amax == 0 gives
 * scale 0 and all codes 0.  DQ = E4M3(c) * scale. */

void qco_encode_fp8_rowwise(const float* x, int64_t rows, int32_t dim,
                            uint8_t* payload, float* scale)
{
    memset(payload, 0, (size_t)qco_payload_bytes(QCO_FP8_ROWWISE, rows * dim, 8));
    for (int64_t r = 0; r < rows; ++r) {
        const float* row = x + r * dim;
        float amax = 0.0f;
        for (int32_t j = 0; j < dim; ++j) {
            float a = fabsf(row[j]);
            if (a > amax) amax = a;
        }
        const float sc = amax / 448.0f;
        for (int32_t j = 0; j < dim; ++j) {
            uint8_t c = 0;
            if (sc != 0.0f) {
                float y = row[j] / sc;
                if (y > 448.0f) y = 448.0f;
                if (y < -448.0f) y = -448.0f;
                c = qco_e4m3_from_f32(y);
            }
            payload[r * dim + j] = c;
        }
        scale[r] = sc;
    }
}

void qco_decode_fp8_rowwise(const uint8_t* payload, const float* scale,
                            int64_t rows, int32_t dim, float* out)
{
    for (int64_t r = 0; r < rows; ++r)
        for (int32_t j = 0; j < dim; ++j)
            out[r * dim + j] = qco_e4m3_to_f32(payload[r * dim + j]) * scale[r];
}

/* ------------------------------------------------------------------ */
/* QSGD  [QCD, "Quantized SGD Algorithms"; QCD, "Quantization Schemes":  */
/*        stochastic; GCQC, "Why sparsification fights the all-reduce"]  */
/* ------------------------------------------------------------------ */
/* s = 16 codes per element (4 bits, so 32/log2(16) = 8x smaller than
 * fp32).  Reading: a code is a sign bit (bit 3) and a level l in 0..7
 * (bits 0-2); level l stands for l * d with d = ||v||_2 / 7 over the
 * bucket.  |v| / d is rounded down or up at random with P(up) equal to its
 * fractional part, which makes DQ unbiased: the element with global index
 * g rounds up iff uniform_draw(seed, g) < frac.  A level-0 code is always 0
 * (no negative zero); DQ of code 0 is +0. */

static float qsgd_dq(uint32_t code, float d)
{
    uint32_t level = code & 7u;
    if (level == 0)
        return 0.0f;
    float mag = (float)level * d;
    return (code & 8u) ? -mag : mag;
}

void qco_encode_qsgd(const float* x, float* ef, int64_t n, int32_t bucket,
                     uint64_t seed, uint64_t elem_offset,
                     uint8_t* payload, float* norm)
{
    const int64_t nb = ceil_div(n, bucket);
    memset(payload, 0, (size_t)qco_payload_bytes(QCO_QSGD, n, 4));
    float* v = (float*)malloc((size_t)bucket * sizeof(float));
    float* sq = (float*)malloc((size_t)bucket * sizeof(float));

    for (int64_t k = 0; k < nb; ++k) {
        const int64_t lo = k * bucket;
        const int64_t cnt = (lo + bucket <= n) ? bucket : n - lo;

        for (int64_t j = 0; j < cnt; ++j) {
            v[j] = ef ? ef[lo + j] + x[lo + j] : x[lo + j];
            sq[j] = v[j] * v[j];
        }
        const float nrm = sqrtf(qco_tree_sum(sq, cnt, bucket));
        const float d = nrm / 7.0f;

        for (int64_t j = 0; j < cnt; ++j) {
            const int64_t i = lo + j;
            uint32_t code = 0;
            if (d != 0.0f) {
                float t = fabsf(v[j]) / d;
                float fl = floorf(t);
                float frac = t - fl; /* exact */
                float u = uniform_draw(seed, elem_offset + (uint64_t)i);
                uint32_t level = (uint32_t)fl + (u < frac ? 1u : 0u);
                if (level > 7u) level = 7u;
                if (level != 0u)
                    code = ((v[j] < 0.0f) ? 8u : 0u) | level;
            }
            or_nibble(payload, i, code);
            if (ef)
                ef[i] = v[j] - qsgd_dq(code, d);
        }
        norm[k] = nrm;
    }
    free(v);
    free(sq);
}

void qco_decode_qsgd(const uint8_t* payload, const float* norm, int64_t n,
                     int32_t bucket, float* out)
{
    for (int64_t i = 0; i < n; ++i) {
        float d = norm[i / bucket] / 7.0f;
        out[i] = qsgd_dq(get_nibble(payload, i), d);
    }
}

/* ------------------------------------------------------------------ */
/* TernGrad  [QCD, "Quantized SGD Algorithms": TernGrad]                */
/* ------------------------------------------------------------------ */
/* Three levels {-1, 0, +1} times a scale.  Readings: the scale is
 * s = max |v| over the bucket (the pages give one scale per layer; a bucket
 * plays that role here, as for the other codecs); element v becomes sign(v)
 * with probability |v|/s and 0 otherwise, so E[DQ] = v: it is nonzero iff
 * uniform_draw(seed, g) < fl(|v| / s).  A 2-bit code holds "nonzero" in
 * bit 0 and "negative" in bit 1 (0 = zero, 1 = +s, 3 = -s; 2 never
 * occurs).  s == 0 gives all codes 0.  DQ = code ? (code & 2 ? -s : s) : +0. */

static float ternary_dq(uint32_t code, float s)
{
    if ((code & 1u) == 0u)
        return 0.0f;
    return (code & 2u) ? -s : s;
}

void qco_encode_ternary(const float* x, float* ef, int64_t n, int32_t bucket,
                        uint64_t seed, uint64_t elem_offset,
                        uint8_t* payload, float* scale)
{
    const int64_t nb = ceil_div(n, bucket);
    memset(payload, 0, (size_t)qco_payload_bytes(QCO_TERNARY, n, 2));
    float* v = (float*)malloc((size_t)bucket * sizeof(float));

    for (int64_t k = 0; k < nb; ++k) {
        const int64_t lo = k * bucket;
        const int64_t cnt = (lo + bucket <= n) ? bucket : n - lo;

        float s = 0.0f;
        for (int64_t j = 0; j < cnt; ++j) {
            v[j] = ef ? ef[lo + j] + x[lo + j] : x[lo + j];
            if (fabsf(v[j]) > s) s = fabsf(v[j]);
        }

        for (int64_t j = 0; j < cnt; ++j) {
            const int64_t i = lo + j;
            uint32_t code = 0;
            if (s != 0.0f) {
                float p = fabsf(v[j]) / s;
                if (uniform_draw(seed, elem_offset + (uint64_t)i) < p)
                    code = (v[j] < 0.0f) ? 3u : 1u;
            }
            or_crumb(payload, i, code);
            if (ef)
                ef[i] = v[j] - ternary_dq(code, s);
        }
        scale[k] = s;
    }
    free(v);
}

void qco_decode_ternary(const uint8_t* payload, const float* scale, int64_t n,
                        int32_t bucket, float* out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = ternary_dq(get_crumb(payload, i), scale[i / bucket]);
}

/* ------------------------------------------------------------------ */
/* 1-bit sign  [QCD, "Bit-Width Selection" and "Quantized SGD           */
/*              Algorithms": SignSGD; GCQC, "Why sparsification fights  */
/*              the all-reduce": one bit]                                */
/* ------------------------------------------------------------------ */
/* Reading: bit = (v < 0); a bucket's scale is the mean of |v| over its
 * valid elements (sum in the contiguous pairwise tree, then divided by the
 * count); DQ = -scale for bit 1 and +scale for bit 0.  bf16 inputs are
 * widened exactly (bits << 16). */

void qco_encode_sign(const void* x, int32_t x_bf16, float* ef, int64_t n,
                     int32_t bucket, uint8_t* payload, float* scale)
{
    const int64_t nb = ceil_div(n, bucket);
    memset(payload, 0, (size_t)qco_payload_bytes(QCO_SIGN, n, 1));
    float* v = (float*)malloc((size_t)bucket * sizeof(float));
    float* av = (float*)malloc((size_t)bucket * sizeof(float));

    for (int64_t k = 0; k < nb; ++k) {
        const int64_t lo = k * bucket;
        const int64_t cnt = (lo + bucket <= n) ? bucket : n - lo;

        for (int64_t j = 0; j < cnt; ++j) {
            float g = x_bf16 ? f32_from((uint32_t)((const uint16_t*)x)[lo + j] << 16)
                             : ((const float*)x)[lo + j];
            v[j] = ef ? ef[lo + j] + g : g;
            av[j] = fabsf(v[j]);
        }
        const float sc = qco_tree_sum(av, cnt, bucket) / (float)cnt;

        for (int64_t j = 0; j < cnt; ++j) {
            const int64_t i = lo + j;
            uint32_t b = (v[j] < 0.0f) ? 1u : 0u;
            or_bit(payload, i, b);
            if (ef)
                ef[i] = v[j] - (b ? -sc : sc);
        }
        scale[k] = sc;
    }
    free(v);
    free(av);
}

void qco_decode_sign(const uint8_t* payload, const float* scale, int64_t n,
                     int32_t bucket, float* out)
{
    for (int64_t i = 0; i < n; ++i) {
        float sc = scale[i / bucket];
        out[i] = get_bit(payload, i) ? -sc : sc;
    }
}

/* ------------------------------------------------------------------ */
/* receive side                                                          */
/* ------------------------------------------------------------------ */

/* ------------------------------------------------------------------ */
/* shared-scale INT8  [QCD, "Quantization-Aware All-Reduce": local and  */
/*   distributed quantization; QCD, "Practical Considerations":         */
/*   synchronization of scale and zero point; GCQC, "Why sparsification */
/*   fights the all-reduce": compressed forms that can be summed]       */
/* ------------------------------------------------------------------ */
/* Readings: the ranks agree one scale per bucket before they encode: the
 * largest |v| that any rank holds in the bucket (each rank's local maximum,
 * combined with max, as an all-reduce would).  Codes are symmetric signed
 * INT8 in [-127, 127] with no zero point, so a sum of codes is an exact
 * integer and the receiver dequantizes it once (quantize locally, reduce the
 * quantized data, dequantize after the reduction).  scale = amax/127;
 * code = rint(v/scale) clamped to [-127, 127]; scale 0 gives code 0;
 * DQ = code * scale; ef = v - DQ. */

void qco_bucket_absmax(const float* x, const float* ef, int64_t n, int32_t bucket, float* amax)
{
    const int64_t nb = ceil_div(n, bucket);
    for (int64_t k = 0; k < nb; ++k) {
        const int64_t lo = k * bucket;
        const int64_t hi = (lo + bucket <= n) ? lo + bucket : n;
        float m = 0.0f;
        for (int64_t i = lo; i < hi; ++i) {
            const float v = ef ? ef[i] + x[i] : x[i];
            if (fabsf(v) > m)
                m = fabsf(v);
        }
        amax[k] = m;
    }
}

void qco_absmax_combine(const float* amax, int32_t m, int64_t nb, float* out)
{
    for (int64_t k = 0; k < nb; ++k) {
        float r = amax[k];
        for (int32_t w = 1; w < m; ++w)
            if (amax[(int64_t)w * nb + k] > r)
                r = amax[(int64_t)w * nb + k];
        out[k] = r;
    }
}

void qco_encode_int8_shared(const float* x, float* ef, int64_t n, int32_t bucket,
                            const float* amax, uint8_t* payload, float* scale)
{
    const int64_t nb = ceil_div(n, bucket);
    memset(payload, 0, (size_t)qco_payload_bytes(QCO_INT8_SHARED, n, 8));
    for (int64_t k = 0; k < nb; ++k) {
        const float sc = amax[k] / 127.0f;
        const int64_t lo = k * bucket;
        const int64_t hi = (lo + bucket <= n) ? lo + bucket : n;
        for (int64_t i = lo; i < hi; ++i) {
            const float v = ef ? ef[i] + x[i] : x[i];
            int32_t q = 0;
            if (sc != 0.0f) {
                float r = rintf(v / sc);
                if (r > 127.0f) r = 127.0f;
                if (r < -127.0f) r = -127.0f;
                q = (int32_t)r;
            }
            payload[i] = (uint8_t)(int8_t)q;
            if (ef)
                ef[i] = v - (float)q * sc;
        }
        scale[k] = sc;
    }
}

void qco_decode_int8_shared(const uint8_t* payload, const float* scale, int64_t n,
                            int32_t bucket, float* out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = (float)(int8_t)payload[i] * scale[i / bucket];
}

void qco_sum_int8_shared(const uint8_t* payloads, int32_t m, int64_t n, int32_t bucket,
                         const float* scale, int32_t* isum, int32_t accumulate, float* out)
{
    const int64_t pb = qco_payload_bytes(QCO_INT8_SHARED, n, 8);
    for (int64_t i = 0; i < n; ++i) {
        int64_t t = (accumulate && isum) ? isum[i] : 0;
        for (int32_t w = 0; w < m; ++w)
            t += (int8_t)payloads[(int64_t)w * pb + i];
        if (isum)
            isum[i] = (int32_t)t;
        if (out)
            out[i] = (float)(int32_t)t * scale[i / bucket];
    }
}

/* ------------------------------------------------------------------ */
/* top-k sparsification  [GQC, "Quantization Schemes": Top-K             */
/*   sparsification; GCQC, opening section: only the largest-magnitude  */
/*   coordinates; GCQC, "Why sparsification fights the all-reduce":     */
/*   index-value pairs; GCQC, "Error feedback is the component that     */
/*   makes it work"]                                                    */
/* ------------------------------------------------------------------ */
/* Readings: the selection is made per bucket, like every other statistic
 * here; a bucket sends k_b = min(k, count) coordinates, those of largest
 * |v| (v = x + ef), comparing the fp32 magnitude (the bit pattern with the
 * sign cleared); equal magnitudes go to the smaller index, so the chosen set
 * is unique.  Each chosen coordinate travels as (index inside the bucket,
 * fp32 value), in ascending index order; the residual is v - sent, i.e. v
 * for unsent coordinates and 0 for sent ones.  The receiver's sum of
 * several workers' pairs is a sparse sum: each pair is added to the dense
 * accumulator in worker order (elements no pair touches are left as they
 * are). */

typedef struct { uint32_t key; uint32_t idx; } topk_item;

static int topk_order(const void* a, const void* b)
{
    const topk_item* p = (const topk_item*)a;
    const topk_item* q = (const topk_item*)b;
    if (p->key != q->key)
        return p->key > q->key ? -1 : 1;   /* larger magnitude first */
    return p->idx < q->idx ? -1 : (p->idx > q->idx ? 1 : 0);  /* then smaller index */
}

void qco_encode_topk(const float* x, float* ef, int64_t n, int32_t bucket, int32_t k,
                     float* values, uint32_t* indices)
{
    const int64_t nb = ceil_div(n, bucket);
    float* v = (float*)malloc((size_t)bucket * sizeof(float));
    topk_item* items = (topk_item*)malloc((size_t)bucket * sizeof(topk_item));
    uint8_t* chosen = (uint8_t*)malloc((size_t)bucket);
    for (int64_t b = 0; b < nb; ++b) {
        const int64_t lo = b * bucket;
        const int64_t cnt = (lo + bucket <= n) ? bucket : n - lo;
        const int64_t kb = k < cnt ? k : cnt;
        for (int64_t j = 0; j < cnt; ++j) {
            v[j] = ef ? ef[lo + j] + x[lo + j] : x[lo + j];
            items[j].key = f32_bits(v[j]) & 0x7FFFFFFFu;
            items[j].idx = (uint32_t)j;
            chosen[j] = 0;
        }
        qsort(items, (size_t)cnt, sizeof(topk_item), topk_order);
        for (int64_t r = 0; r < kb; ++r)
            chosen[items[r].idx] = 1;
        int64_t slot = b * (int64_t)k;
        for (int64_t j = 0; j < cnt; ++j) {
            if (chosen[j]) {
                values[slot] = v[j];
                indices[slot] = (uint32_t)j;
                ++slot;
            }
            if (ef)
                ef[lo + j] = v[j] - (chosen[j] ? v[j] : 0.0f);
        }
        for (; slot < (b + 1) * (int64_t)k; ++slot) {
            values[slot] = 0.0f;
            indices[slot] = 0xFFFFFFFFu;
        }
    }
    free(v);
    free(items);
    free(chosen);
}

void qco_decode_topk(const float* values, const uint32_t* indices, int64_t n, int32_t bucket,
                     int32_t k, float* out)
{
    const int64_t nb = ceil_div(n, bucket);
    for (int64_t i = 0; i < n; ++i)
        out[i] = 0.0f;
    for (int64_t b = 0; b < nb; ++b) {
        const int64_t cnt = (b * bucket + bucket <= n) ? bucket : n - b * bucket;
        for (int64_t j = 0; j < k; ++j) {
            const uint32_t idx = indices[b * k + j];
            if ((int64_t)idx < cnt)
                out[b * bucket + idx] = values[b * k + j];
        }
    }
}

void qco_topk_accumulate(const float* values, const uint32_t* indices, int32_t m, int64_t n,
                         int32_t bucket, int32_t k, float* acc, int32_t accumulate)
{
    const int64_t nb = ceil_div(n, bucket);
    if (!accumulate)
        for (int64_t i = 0; i < n; ++i)
            acc[i] = 0.0f;
    for (int32_t w = 0; w < m; ++w) {
        const float* vw = values + (int64_t)w * nb * k;
        const uint32_t* iw = indices + (int64_t)w * nb * k;
        for (int64_t b = 0; b < nb; ++b) {
            const int64_t cnt = (b * bucket + bucket <= n) ? bucket : n - b * bucket;
            for (int64_t j = 0; j < k; ++j) {
                const uint32_t idx = iw[b * k + j];
                if ((int64_t)idx < cnt)
                    acc[b * bucket + idx] = acc[b * bucket + idx] + vw[b * k + j];
            }
        }
    }
}

float qco_decode_one(int32_t fmt, const uint8_t* payload, const float* scale,
                     const float* zero, int64_t i, int32_t group, int32_t bits)
{
    const int64_t k = i / group;
    switch (fmt) {
    case QCO_UNIFORM:
        return uniform_dq(get_uniform_code(payload, i, bits), scale[k], zero[k]);
    case QCO_FP8_ROWWISE:
        return qco_e4m3_to_f32(payload[i]) * scale[k];
    case QCO_QSGD:
        return qsgd_dq(get_nibble(payload, i), scale[k] / 7.0f);
    case QCO_TERNARY:
        return ternary_dq(get_crumb(payload, i), scale[k]);
    case QCO_INT8_SHARED:
        return (float)(int8_t)payload[i] * scale[k];
    default: /* QCO_SIGN */
        return get_bit(payload, i) ? -scale[k] : scale[k];
    }
}

/* Quantized accumulation in fp32 [QCD, "Quantization-Aware All-Reduce":
 * quantized accumulation; GQC, "How Gradient Quantization Works":
 * dequantize, then aggregate].  Reading: the aggregate is a sum (not a
 * mean), taken in worker order 0..m-1. */
void qco_dequant_accumulate(int32_t fmt, const uint8_t* payloads, const float* scale,
                            const float* zero, int32_t m, int64_t n, int32_t group,
                            int32_t bits, float* acc, int32_t accumulate)
{
    const int64_t pb = qco_payload_bytes(fmt, n, bits);
    const int64_t nb = ceil_div(n, group);
    for (int64_t i = 0; i < n; ++i) {
        float a = accumulate ? acc[i] : 0.0f;
        for (int32_t w = 0; w < m; ++w) {
            float dq = qco_decode_one(fmt, payloads + (int64_t)w * pb, scale + (int64_t)w * nb,
                                      zero ? zero + (int64_t)w * nb : NULL, i, group, bits);
            a = a + dq;
        }
        acc[i] = a;
    }
}

/* signSGD aggregation by majority vote [QCD, "Quantized SGD Algorithms":
 * SignSGD; GCQC, "Why sparsification fights the all-reduce": one bit].
 * Reading: a strict majority of set bits ("negative") is needed, so a tie
 * at even m gives 0 ("positive"), matching sign(0) = + in the encoder. */
void qco_majority_vote(const uint8_t* payloads, int32_t m, int64_t n, uint8_t* out)
{
    const int64_t pb = qco_payload_bytes(QCO_SIGN, n, 1);
    memset(out, 0, (size_t)pb);
    for (int64_t p = 0; p < n; ++p) {
        int64_t c = 0;
        for (int32_t w = 0; w < m; ++w)
            c += get_bit(payloads + (int64_t)w * pb, p);
        if (2 * c > m)
            or_bit(out, p, 1u);
    }
}
