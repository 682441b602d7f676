/*
 * zero_oracle.c -- CPU oracle for one rank's share of a ZeRO mixed-precision
 * training step.  TEST INFRASTRUCTURE ONLY: the test-suite, the smoke check and
 * the benchmark's CPU-baseline leg are the only users.  It shares no code,
 * header, table or constant with the GPU library and must never be on the
 * product path.
 *
 * Everything here is plain scalar C, built with -O2 -ffp-contract=off
 * -fno-fast-math, one element at a time, in the order the method states it.
 *
 * What the method computes (sources):
 *   - gradient reduction to the owner of a partition ("reduce-scatter":
 *     results of all GPUs are merged, then each keeps only the part it is
 *     responsible for) -- ZeRO mind-map page (paperbridge.wiki), glossary entry
 *     for reduce-scatter and the section on how a GPU holding a quarter computes;
 *   - the optimizer state of mixed-precision Adam: low-precision parameters,
 *     an fp32 master copy and the first and second moments -- ZeRO concept
 *     page (papers.lqhl.me), section "why it is needed";
 *   - the Adam recurrence itself is not printed on the pages; the oracle uses
 *     the textbook rule of Kingma & Ba (2015), Algorithm 1: bias-corrected
 *     moments, epsilon added outside the square root, no weight decay.
 *
 * Precision: the pages fix the optimizer state as fp32 (master weights and
 * both moments) and the parameters and gradients as 16-bit, so the oracle
 * computes the update in fp32, one IEEE-rounded operation per statement,
 * with the operation order written out below.  An fp64 version of the same
 * recurrence (orc_adam_f64) is provided to bound its accuracy.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

enum { ORC_F32 = 0, ORC_F16 = 1, ORC_BF16 = 2 };

static float orc_from_bits(uint32_t b) { float f; memcpy(&f, &b, sizeof f); return f; }
static uint32_t orc_to_bits(float f) { uint32_t b; memcpy(&b, &f, sizeof b); return b; }

/* ------------------------------------------------------------------ */
/* 16-bit formats, decoded and encoded from their IEEE-754 definitions */
/* ------------------------------------------------------------------ */

/* binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
double orc_f16_value(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double mag;
    if (e == 0x1f) mag = f ? NAN : INFINITY;
    else if (e == 0) mag = ldexp((double)f, -24);            /* subnormal: f * 2^-24 */
    else mag = ldexp((double)(1024 + f), e - 25);            /* (1 + f/1024) * 2^(e-15) */
    return sign ? -mag : mag;
}

/* bfloat16: 1 sign, 8 exponent (bias 127), 7 fraction bits. */
double orc_bf16_value(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 7) & 0xff;
    int f = h & 0x7f;
    double mag;
    if (e == 0xff) mag = f ? NAN : INFINITY;
    else if (e == 0) mag = ldexp((double)f, -133);           /* f * 2^(-126-7) */
    else mag = ldexp((double)(128 + f), e - 134);            /* (1 + f/128) * 2^(e-127) */
    return sign ? -mag : mag;
}

/*
 * Round x to the nearest value of a binary format with p fraction bits,
 * minimum normal exponent emin and maximum finite magnitude maxval, ties to
 * the even significand.  Returns the rounded magnitude (may be +inf) -- an
 * arithmetic formulation: scale by the quantum of x's binade, round to an
 * integer with rint (round-half-even in the default rounding mode), scale
 * back.  All steps are exact in double for fp32 inputs.
 */
static double orc_round_magnitude(double ax, int p, int emin, double maxval)
{
    int E;
    frexp(ax, &E);                 /* ax = fr * 2^E, fr in [0.5, 1) */
    int e = E - 1;                 /* ax in [2^e, 2^(e+1)) */
    if (e < emin) e = emin;        /* subnormal range shares the smallest quantum */
    double quantum = ldexp(1.0, e - p);
    double r = rint(ax / quantum) * quantum;
    /* Overflow: anything at or above the midpoint between maxval and the next
     * power of two (which the format cannot hold) becomes infinity; at the
     * midpoint itself the even neighbour is that power of two. */
    if (r > maxval) return INFINITY;
    return r;
}

static uint16_t orc_encode16(double r, int sign, int p, int emin, int ebias)
{
    uint32_t s = (uint32_t)sign << 15;
    int expbits = 15 - p;          /* 5 for fp16, 8 for bf16 */
    uint32_t emax_field = (1u << expbits) - 1;
    if (isinf(r)) return (uint16_t)(s | (emax_field << p));
    if (r == 0.0) return (uint16_t)s;
    int E;
    frexp(r, &E);
    int e = E - 1;
    if (e < emin) {                /* subnormal: fraction = r / 2^(emin-p) */
        uint32_t f = (uint32_t)ldexp(r, p - emin);
        return (uint16_t)(s | f);
    }
    uint32_t f = (uint32_t)(ldexp(r, p - e) - ldexp(1.0, p));
    return (uint16_t)(s | ((uint32_t)(e + ebias) << p) | f);
}

/* fp32 -> binary16, round to nearest even; NaN -> quiet NaN (sign kept). */
uint16_t orc_f32_to_f16(float x)
{
    double d = (double)x;
    int sign = signbit(d) ? 1 : 0;
    if (isnan(d)) return (uint16_t)((sign << 15) | 0x7e00);
    double maxval = 65504.0;       /* (2 - 2^-10) * 2^15 */
    double r = isinf(d) ? INFINITY : orc_round_magnitude(fabs(d), 10, -14, maxval);
    return orc_encode16(r, sign, 10, -14, 15);
}

/* fp32 -> bfloat16, round to nearest even; NaN -> quiet NaN (sign kept). */
uint16_t orc_f32_to_bf16(float x)
{
    double d = (double)x;
    int sign = signbit(d) ? 1 : 0;
    if (isnan(d)) return (uint16_t)((sign << 15) | 0x7fc0);
    double maxval = ldexp(255.0, 120);   /* (2 - 2^-7) * 2^127 */
    double r = isinf(d) ? INFINITY : orc_round_magnitude(fabs(d), 7, -126, maxval);
    return orc_encode16(r, sign, 7, -126, 127);
}

/* Batch forms, for exhaustive checks from Python. */
void orc_cast_f32_to_16(const float* x, uint16_t* out, int64_t n, int dt)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = dt == ORC_F16 ? orc_f32_to_f16(x[i]) : orc_f32_to_bf16(x[i]);
}

void orc_cast_bits_range_to_16(uint32_t first, int64_t n, uint16_t* out, int dt)
{
    for (int64_t i = 0; i < n; ++i) {
        float x = orc_from_bits(first + (uint32_t)i);
        out[i] = dt == ORC_F16 ? orc_f32_to_f16(x) : orc_f32_to_bf16(x);
    }
}

/* Widen a stored 16-bit gradient element to fp32 (exact). */
static float orc_widen(const void* base, int dt, int64_t j)
{
    const uint16_t h = ((const uint16_t*)base)[j];
    if (dt == ORC_F16) return (float)orc_f16_value(h);
    return (float)orc_bf16_value(h);
}

/* ------------------------------------------------------------------ */
/* Adam constants                                                      */
/* ------------------------------------------------------------------ */

/*
 * The nine fp32 constants of step t, each computed in fp64 from the decimal
 * hyper-parameters and rounded once to fp32:
 *   [0] beta1  [1] 1-beta1  [2] beta2  [3] 1-beta2
 *   [4] 1-beta1^t  [5] 1-beta2^t  (bias corrections)
 *   [6] lr  [7] eps  [8] grad_scale
 */
void orc_adam_consts(double lr, double beta1, double beta2, double eps,
                     double grad_scale, int64_t t, float out[9])
{
    out[0] = (float)beta1;
    out[1] = (float)(1.0 - beta1);
    out[2] = (float)beta2;
    out[3] = (float)(1.0 - beta2);
    out[4] = (float)(1.0 - pow(beta1, (double)t));
    out[5] = (float)(1.0 - pow(beta2, (double)t));
    out[6] = (float)lr;
    out[7] = (float)eps;
    out[8] = (float)grad_scale;
}

/* ------------------------------------------------------------------ */
/* Reduction of the owner's partition                                   */
/* ------------------------------------------------------------------ */

/*
 * out[j] = ((g_0[j] + g_1[j]) + ... + g_{n-1}[j]) * grad_scale, in fp32,
 * ranks folded in the fixed order 0..n-1 whatever rank owns the partition.
 * slices[q] points at the first element of rank q's contribution.
 */
void orc_reduce(int32_t n_ranks, const void* const* slices, int dt, int64_t count,
                float grad_scale, float* out)
{
    for (int64_t j = 0; j < count; ++j) {
        float acc = orc_widen(slices[0], dt, j);
        for (int32_t q = 1; q < n_ranks; ++q) {
            float gq = orc_widen(slices[q], dt, j);
            acc = acc + gq;
        }
        float g = acc * grad_scale;
        out[j] = g;
    }
}

/* ------------------------------------------------------------------ */
/* Mixed-precision Adam on the shard                                    */
/* ------------------------------------------------------------------ */

/*
 * One Adam step on count elements, in place on fp32 w (master), m, v, with
 * the reduced gradient g; writes the rounded 16-bit parameter to p.
 * Each statement is exactly one fp32 operation.
 */
void orc_adam(int64_t count, const float* gr, float* w, float* m, float* v,
              const float c[9], uint16_t* p, int pdt)
{
    const float b1 = c[0], c1 = c[1], b2 = c[2], c2 = c[3];
    const float bc1 = c[4], bc2 = c[5], lr = c[6], eps = c[7];
    for (int64_t j = 0; j < count; ++j) {
        float g = gr[j];
        float m_keep = b1 * m[j];
        float m_new_part = c1 * g;
        float mn = m_keep + m_new_part;
        float gsq = g * g;
        float v_keep = b2 * v[j];
        float v_new_part = c2 * gsq;
        float vn = v_keep + v_new_part;
        float mhat = mn / bc1;
        float vhat = vn / bc2;
        float root = sqrtf(vhat);
        float den = root + eps;
        float ratio = mhat / den;
        float delta = lr * ratio;
        float wn = w[j] - delta;
        m[j] = mn;
        v[j] = vn;
        w[j] = wn;
        if (p) p[j] = pdt == ORC_F16 ? orc_f32_to_f16(wn) : orc_f32_to_bf16(wn);
    }
}

/* The same recurrence carried in fp64 throughout (accuracy bound only). */
void orc_adam_f64(int64_t count, const double* g, double* w, double* m, double* v,
                  double lr, double beta1, double beta2, double eps, int64_t t)
{
    double bc1 = 1.0 - pow(beta1, (double)t);
    double bc2 = 1.0 - pow(beta2, (double)t);
    for (int64_t j = 0; j < count; ++j) {
        m[j] = beta1 * m[j] + (1.0 - beta1) * g[j];
        v[j] = beta2 * v[j] + (1.0 - beta2) * g[j] * g[j];
        double mhat = m[j] / bc1;
        double vhat = v[j] / bc2;
        w[j] = w[j] - lr * mhat / (sqrt(vhat) + eps);
    }
}

/* The sum of fp32 values in fp64 (for the reduction error bound). */
void orc_widen_to_f64(const void* src, int dt, int64_t count, double* out)
{
    for (int64_t j = 0; j < count; ++j)
        out[j] = dt == ORC_F16 ? orc_f16_value(((const uint16_t*)src)[j])
                               : orc_bf16_value(((const uint16_t*)src)[j]);
}

/* Bits helpers exported for tests that walk bit patterns. */
uint32_t orc_f32_bits(float x) { return orc_to_bits(x); }
float orc_bits_f32(uint32_t b) { return orc_from_bits(b); }
