/*
 * CPU oracle for the FP8 (OCP e4m3fn) weight-only linear layer.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may link, load or call
 * this file: only the test suite, the package smoke check and the benchmark's
 * CPU-baseline leg use it. It shares no code, header, table or constant
 * generator with the HIP library.
 *
 * Plain and slow on purpose: every function follows one passage of the pages
 * and does the arithmetic in the order that passage states. fp32 steps that the
 * method fixes (the scale and the quotient) are done in IEEE single precision;
 * everything else is fp64.
 *
 * Sources (page title, section):
 *   [FP8W]  "FP8 weight-only (precision: fp8_weights)" (kernel-agent skill page),
 *           section "The contract".
 *   [B04]   "B04 - Precision & Quantization", sections "The numbers, derived
 *           rather than tabulated" (format formulas, the E4M3 table row and its
 *           footnote) and "Hardware support, and where the vendors diverge"
 *           (OCP versus FNUZ encodings).
 *   [WFK]   "Skill: Write an FP8 Kernel", sections "Required reasoning process"
 *           step 2 (amax -> scale -> cast of x/scale) and step 7 (scale = 0);
 *           steps 4-5 and "Correctness requirements" for W8A8.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------- */
/* e4m3fn decode: [B04] "The numbers, derived rather than tabulated".        */
/* Fields: sign s (1 bit), exponent e (4 bits, bias 7), mantissa m (3 bits).  */
/* e == 0 is the subnormal binade: value m * 2^(1-7-3). The top pattern       */
/* e == 15, m == 7 is the format's only NaN (no infinities), which is what    */
/* lets e == 15 carry finite values up to 1.75 * 2^8 = 448.                   */
/* ------------------------------------------------------------------------- */
double o_e4m3_decode(uint8_t c)
{
    const int s = (c >> 7) & 1;
    const int e = (c >> 3) & 15;
    const int m = c & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m, 1 - 7 - 3);            /* subnormal: m * 2^-9 */
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7);    /* normal: 1.m * 2^(e-7) */
    return s ? -v : v;
}

/* ------------------------------------------------------------------------- */
/* Encoder 1: round-to-nearest-even onto the e4m3 grid, working on the       */
/* integer significand of the fp32 input, saturating to +-448 ([FP8W] "codes */
/* round(w / scale) in e4m3 (round to nearest even, clamped to +-448)").     */
/* ------------------------------------------------------------------------- */

/* Shift `sig` right by `sh` bits with round-half-to-even on the dropped bits. */
static uint32_t rne_shift(uint32_t sig, int sh)
{
    uint32_t kept, rem, half;
    if (sh <= 0)
        return sig;
    if (sh >= 32)
        return 0;
    kept = sig >> sh;
    rem = sig & ((1u << sh) - 1u);
    half = 1u << (sh - 1);
    if (rem > half || (rem == half && (kept & 1u)))
        kept += 1u;
    return kept;
}

uint8_t o_e4m3_encode(float t)
{
    uint32_t u;
    memcpy(&u, &t, sizeof u);
    const uint8_t sign = (uint8_t)((u >> 31) << 7);
    const uint32_t mag = u & 0x7fffffffu;
    if (mag > 0x7f800000u)
        return (uint8_t)(sign | 0x7f);              /* NaN in, NaN out (unit tests only) */
    if (fabsf(t) >= 448.0f)
        return (uint8_t)(sign | 0x7e);              /* saturate, infinities included */

    const int bexp = (int)(mag >> 23);
    if (bexp == 0)
        return sign;                                /* fp32 zero/subnormal: far below 2^-10 */
    const int e = bexp - 127;                       /* unbiased exponent of |t| */
    const uint32_t sig = (1u << 23) | (mag & 0x7fffffu); /* |t| = sig * 2^(e-23) */

    if (e < -6) {
        /* e4m3 subnormal binade: count quanta of 2^-9, i.e. sig * 2^(e-23+9). */
        const uint32_t q = rne_shift(sig, 14 - e);  /* 0..8; 8 is the smallest normal */
        return (uint8_t)(sign | q);                 /* the magnitude code equals q here */
    }
    /* normal: keep 1 implicit + 3 mantissa bits of the 24-bit significand */
    const uint32_t q4 = rne_shift(sig, 20);          /* 8..16; 16 carries into e+1 */
    uint32_t code = (uint32_t)(e + 7) * 8u + (q4 - 8u);
    if (code > 0x7eu)
        code = 0x7eu;
    return (uint8_t)(sign | code);
}

/* ------------------------------------------------------------------------- */
/* Encoder 2 (cross-check only, written independently of encoder 1): search  */
/* the ordered table of positive finite values for the two neighbours of |t| */
/* and pick the nearer one, the even code on an exact tie. Every midpoint     */
/* between neighbours has at most 5 significant bits, so comparing it with    */
/* the fp32 input in double precision is exact.                               */
/* ------------------------------------------------------------------------- */
static double g_positive[0x7f];                      /* value(c) for c = 0x00..0x7e */
static int g_positive_ready = 0;

static void positive_table_init(void)
{
    if (g_positive_ready)
        return;
    for (int c = 0; c < 0x7f; ++c)
        g_positive[c] = o_e4m3_decode((uint8_t)c);
    g_positive_ready = 1;
}

uint8_t o_e4m3_encode_search(float t)
{
    positive_table_init();
    const uint8_t sign = signbit(t) ? 0x80 : 0x00;
    if (isnan(t))
        return (uint8_t)(sign | 0x7f);
    const double a = fabs((double)t);
    if (a >= g_positive[0x7e])
        return (uint8_t)(sign | 0x7e);
    /* largest lo in [0, 0x7e) with value(lo) <= a; value is increasing in the code */
    int lo = 0, hi = 0x7e;                           /* invariant: v(lo) <= a < v(hi) */
    while (hi - lo > 1) {
        const int mid = (lo + hi) / 2;
        if (g_positive[mid] <= a)
            lo = mid;
        else
            hi = mid;
    }
    const double vlo = g_positive[lo];
    const double vhi = g_positive[hi];
    const double midpoint = 0.5 * (vlo + vhi);
    int pick;
    if (a < midpoint)
        pick = lo;
    else if (a > midpoint)
        pick = hi;
    else
        pick = (lo % 2 == 0) ? lo : hi;              /* tie: the code with an even mantissa */
    return (uint8_t)(sign | pick);
}

/* ------------------------------------------------------------------------- */
/* Exhaustive agreement of the two encoders over fp32 bit patterns           */
/* [first, first+count). NaN patterns are skipped. Returns the number of     */
/* disagreements and the first disagreeing pattern in *first_bad.            */
/* ------------------------------------------------------------------------- */
int64_t o_encoders_compare(uint64_t first, uint64_t count, uint64_t *first_bad)
{
    int64_t bad = 0;
    uint64_t fb = UINT64_MAX;
    positive_table_init();                           /* before the threads read it */
#pragma omp parallel for reduction(+ : bad) schedule(static)
    for (int64_t i = 0; i < (int64_t)count; ++i) {
        const uint32_t u = (uint32_t)(first + (uint64_t)i);
        if ((u & 0x7fffffffu) > 0x7f800000u)
            continue;
        float t;
        memcpy(&t, &u, sizeof t);
        if (o_e4m3_encode(t) != o_e4m3_encode_search(t)) {
            bad += 1;
#pragma omp critical
            if ((uint64_t)u < fb)
                fb = (uint64_t)u;
        }
    }
    if (first_bad)
        *first_bad = fb;
    return bad;
}

/* Encode an array (scale 1), used to compare the encoder with the pages' */
/* worked values and with the GPU on wide sweeps.                           */
void o_e4m3_encode_array(const float *t, int64_t n, uint8_t *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = o_e4m3_encode(t[i]);
}

/* ------------------------------------------------------------------------- */
/* Build-time per-output-channel quantizer ([FP8W] "The contract"; [WFK]     */
/* step 2 "compute amax -> scale = amax / fp8_max -> cast(x / scale)";       */
/* [WFK] step 7 for the all-zero row).                                       */
/*   amax[n]  = max_k |W[n,k]|                                               */
/*   scale[n] = fl32(amax[n] / 448)                                          */
/*   q[n,k]   = E(fl32(W[n,k] / scale[n]))     (0x00 for every k if scale=0)*/
/* Returns 0, or 3 when any weight is NaN or infinite (outputs then hold    */
/* whatever was computed).                                                   */
/* ------------------------------------------------------------------------- */
int o_quantize_rows(const float *w, int64_t n, int64_t k, uint8_t *q, float *scale)
{
    int nonfinite = 0;
#pragma omp parallel for reduction(| : nonfinite) schedule(static)
    for (int64_t r = 0; r < n; ++r) {
        const float *row = w + r * k;
        float amax = 0.0f;
        for (int64_t j = 0; j < k; ++j) {
            const float a = fabsf(row[j]);
            if (!isfinite(a))
                nonfinite = 1;
            else if (a > amax)
                amax = a;
        }
        const float s = amax / 448.0f;
        scale[r] = s;
        for (int64_t j = 0; j < k; ++j)
            q[r * k + j] = (s == 0.0f) ? 0x00 : o_e4m3_encode(row[j] / s);
    }
    return nonfinite ? 3 : 0;
}

/* max_k |W[n,k]| per row (the amax used by the tolerance gate). */
void o_row_amax(const float *w, int64_t n, int64_t k, double *amax)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r) {
        double a = 0.0;
        for (int64_t j = 0; j < k; ++j) {
            const double v = fabs((double)w[r * k + j]);
            if (v > a)
                a = v;
        }
        amax[r] = a;
    }
}

/* ------------------------------------------------------------------------- */
/* The linear layer in fp64 ([FP8W] "The contract"):                         */
/*   y[m,n] = scale[n] * sum_k x[m,k] * value(q[n,k]) + bias[n]             */
/* x and bias are the exact activation-dtype values, passed as doubles; bias */
/* may be NULL. Every product is exact in fp64 (8-bit x 4-bit significands   */
/* into 53 bits), so the only rounding is the fp64 accumulation.             */
/* ------------------------------------------------------------------------- */
void o_linear_f64(const double *x, int64_t m, int64_t k, const uint8_t *q, const float *scale,
                  const double *bias, int64_t n, double *y)
{
    double lut[256];
    for (int c = 0; c < 256; ++c)
        lut[c] = o_e4m3_decode((uint8_t)c);
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < n; ++c) {
        const uint8_t *qr = q + c * k;
        for (int64_t r = 0; r < m; ++r) {
            const double *xr = x + r * k;
            double acc = 0.0;
            for (int64_t j = 0; j < k; ++j)
                acc += xr[j] * lut[qr[j]];
            y[r * n + c] = (double)scale[c] * acc + (bias ? bias[c] : 0.0);
        }
    }
}

/* Same as o_linear_f64 but only for the listed (row, channel) pairs. */
void o_linear_f64_sampled(const double *x, int64_t k, const uint8_t *q, const float *scale,
                          const double *bias, const int64_t *rows, const int64_t *cols,
                          int64_t count, double *y)
{
    double lut[256];
    for (int c = 0; c < 256; ++c)
        lut[c] = o_e4m3_decode((uint8_t)c);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i) {
        const double *xr = x + rows[i] * k;
        const uint8_t *qr = q + cols[i] * k;
        double acc = 0.0;
        for (int64_t j = 0; j < k; ++j)
            acc += xr[j] * lut[qr[j]];
        y[i] = (double)scale[cols[i]] * acc + (bias ? bias[cols[i]] : 0.0);
    }
}

/* ------------------------------------------------------------------------- */
/* Dequantised weight, [FP8W] "Fallback": value(q[n,k]) * scale[n], in fp64 */
/* (scale == NULL gives the unscaled decode).                                */
/* ------------------------------------------------------------------------- */
void o_dequantize_f64(const uint8_t *q, const float *scale, int64_t n, int64_t k, double *out)
{
    double lut[256];
    for (int c = 0; c < 256; ++c)
        lut[c] = o_e4m3_decode((uint8_t)c);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r)
        for (int64_t j = 0; j < k; ++j)
            out[r * k + j] = lut[q[r * k + j]] * (scale ? (double)scale[r] : 1.0);
}

/* ------------------------------------------------------------------------- */
/* Weight error report named by [FP8W] "The contract" (rel_l2,               */
/* worst_channel_rel_l2, underflow, crest). The page names the figures but   */
/* not their formulas; the readings used here:                               */
/*   rel_l2      = ||What - W||_F / ||W||_F,   What = value(q) * scale       */
/*   channel[n]  = ||What[n] - W[n]||_2 / ||W[n]||_2   (0 for a zero row)    */
/*   underflow   = #{W != 0 and value(q) == 0} / #{W != 0}                   */
/*   crest[n]    = max|W[n]| / rms(W[n])           (0 for a zero row)        */
/* out[0] = rel_l2, out[1] = worst channel, out[2] = underflow fraction.     */
/* ------------------------------------------------------------------------- */
void o_weight_error(const float *w, const uint8_t *q, const float *scale, int64_t n, int64_t k,
                    double *out, double *channel_rel_l2, double *crest)
{
    double lut[256];
    for (int c = 0; c < 256; ++c)
        lut[c] = o_e4m3_decode((uint8_t)c);
    double err2 = 0.0, ref2 = 0.0, worst = 0.0;
    int64_t nz = 0, under = 0;
#pragma omp parallel for reduction(+ : err2, ref2, nz, under) reduction(max : worst) schedule(static)
    for (int64_t r = 0; r < n; ++r) {
        double e2 = 0.0, w2 = 0.0, amax = 0.0;
        for (int64_t j = 0; j < k; ++j) {
            const double wv = (double)w[r * k + j];
            const double v = lut[q[r * k + j]];
            const double d = v * (double)scale[r] - wv;
            e2 += d * d;
            w2 += wv * wv;
            if (fabs(wv) > amax)
                amax = fabs(wv);
            if (wv != 0.0) {
                nz += 1;
                if (v == 0.0)
                    under += 1;
            }
        }
        err2 += e2;
        ref2 += w2;
        const double ch = (w2 > 0.0) ? sqrt(e2 / w2) : 0.0;
        if (channel_rel_l2)
            channel_rel_l2[r] = ch;
        if (crest)
            crest[r] = (w2 > 0.0) ? amax / sqrt(w2 / (double)k) : 0.0;
        if (ch > worst)
            worst = ch;
    }
    out[0] = (ref2 > 0.0) ? sqrt(err2 / ref2) : 0.0;
    out[1] = worst;
    out[2] = (nz > 0) ? (double)under / (double)nz : 0.0;
}

/* ========================================================================= */
/* Group-wise scales along k.                                                 */
/*   [B04] "Post-training quantization versus quantization-aware training"   */
/*   (granularity table: one scale per run of g weights in a row, g = 32, 64 */
/*   or 128) and "The one that matters: quantization is a quality decision"  */
/*   (raise the granularity from per-channel to per-group); the Day-98 lab   */
/*   page's storage census ("FP8 e4m3, one scale per 32": the block's max    */
/*   |w| / 448 as an fp32 scale, the cast of w / scale as the code).          */
/* Each run of g weights of a row is quantized exactly as [FP8W]'s contract   */
/* quantizes a whole row:                                                     */
/*   scale[n, j] = fl32(max_{i < g} |W[n, j*g + i]| / 448)                    */
/*   q[n, k]     = E(fl32(W[n, k] / scale[n, k / g]))   (0x00 if scale is 0) */
/* scale is [n, k / g] row-major; k % g == 0.                                 */
/* ========================================================================= */
int o_quantize_groups(const float *w, int64_t n, int64_t k, int64_t g, uint8_t *q, float *scale)
{
    const int64_t ng = k / g;
    int nonfinite = 0;
#pragma omp parallel for reduction(| : nonfinite) schedule(static)
    for (int64_t r = 0; r < n; ++r) {
        for (int64_t j = 0; j < ng; ++j) {
            const float *grp = w + r * k + j * g;
            float amax = 0.0f;
            for (int64_t i = 0; i < g; ++i) {
                const float a = fabsf(grp[i]);
                if (!isfinite(a))
                    nonfinite = 1;
                else if (a > amax)
                    amax = a;
            }
            const float s = amax / 448.0f;
            scale[r * ng + j] = s;
            for (int64_t i = 0; i < g; ++i)
                q[r * k + j * g + i] = (s == 0.0f) ? 0x00 : o_e4m3_encode(grp[i] / s);
        }
    }
    return nonfinite ? 3 : 0;
}

/* The linear layer with group scales, in fp64:                              */
/*   y[m,n] = sum_j scale[n,j] * (sum_{i<g} x[m,jg+i] * value(q[n,jg+i]))     */
/*            + bias[n]                                                       */
/* Each product x * value(q) is exact in fp64; the group sums, their scaling */
/* and the sum over groups round in fp64 only.                                */
void o_linear_f64_groups(const double *x, int64_t m, int64_t k, const uint8_t *q, const float *scale,
                         int64_t g, const double *bias, int64_t n, double *y)
{
    double lut[256];
    for (int c = 0; c < 256; ++c)
        lut[c] = o_e4m3_decode((uint8_t)c);
    const int64_t ng = k / g;
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < n; ++c) {
        const uint8_t *qr = q + c * k;
        for (int64_t r = 0; r < m; ++r) {
            const double *xr = x + r * k;
            double acc = 0.0;
            for (int64_t j = 0; j < ng; ++j) {
                double part = 0.0;
                for (int64_t i = 0; i < g; ++i)
                    part += xr[j * g + i] * lut[qr[j * g + i]];
                acc += (double)scale[c * ng + j] * part;
            }
            y[r * n + c] = acc + (bias ? bias[c] : 0.0);
        }
    }
}

/* The same for the listed (row, channel) pairs only. */
void o_linear_f64_groups_sampled(const double *x, int64_t k, const uint8_t *q, const float *scale, int64_t g,
                                 const double *bias, const int64_t *rows, const int64_t *cols, int64_t count,
                                 double *y)
{
    double lut[256];
    for (int c = 0; c < 256; ++c)
        lut[c] = o_e4m3_decode((uint8_t)c);
    const int64_t ng = k / g;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < count; ++t) {
        const double *xr = x + rows[t] * k;
        const uint8_t *qr = q + cols[t] * k;
        double acc = 0.0;
        for (int64_t j = 0; j < ng; ++j) {
            double part = 0.0;
            for (int64_t i = 0; i < g; ++i)
                part += xr[j * g + i] * lut[qr[j * g + i]];
            acc += (double)scale[cols[t] * ng + j] * part;
        }
        y[t] = acc + (bias ? bias[cols[t]] : 0.0);
    }
}

/* Dequantised weight with group scales: value(q[n,k]) * scale[n, k / g]. */
void o_dequantize_groups_f64(const uint8_t *q, const float *scale, int64_t g, int64_t n, int64_t k, double *out)
{
    double lut[256];
    for (int c = 0; c < 256; ++c)
        lut[c] = o_e4m3_decode((uint8_t)c);
    const int64_t ng = k / g;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r)
        for (int64_t j = 0; j < k; ++j)
            out[r * k + j] = lut[q[r * k + j]] * (double)scale[r * ng + j / g];
}

/* The error report of o_weight_error with group scales: What[n,k] =        */
/* value(q[n,k]) * scale[n, k / g]. The figures are defined as there.         */
void o_weight_error_groups(const float *w, const uint8_t *q, const float *scale, int64_t g, int64_t n,
                           int64_t k, double *out, double *channel_rel_l2, double *crest)
{
    double lut[256];
    for (int c = 0; c < 256; ++c)
        lut[c] = o_e4m3_decode((uint8_t)c);
    const int64_t ng = k / g;
    double err2 = 0.0, ref2 = 0.0, worst = 0.0;
    int64_t nz = 0, under = 0;
#pragma omp parallel for reduction(+ : err2, ref2, nz, under) reduction(max : worst) schedule(static)
    for (int64_t r = 0; r < n; ++r) {
        double e2 = 0.0, w2 = 0.0, amax = 0.0;
        for (int64_t j = 0; j < k; ++j) {
            const double wv = (double)w[r * k + j];
            const double v = lut[q[r * k + j]];
            const double d = v * (double)scale[r * ng + j / g] - wv;
            e2 += d * d;
            w2 += wv * wv;
            if (fabs(wv) > amax)
                amax = fabs(wv);
            if (wv != 0.0) {
                nz += 1;
                if (v == 0.0)
                    under += 1;
            }
        }
        err2 += e2;
        ref2 += w2;
        const double ch = (w2 > 0.0) ? sqrt(e2 / w2) : 0.0;
        if (channel_rel_l2)
            channel_rel_l2[r] = ch;
        if (crest)
            crest[r] = (w2 > 0.0) ? amax / sqrt(w2 / (double)k) : 0.0;
        if (ch > worst)
            worst = ch;
    }
    out[0] = (ref2 > 0.0) ? sqrt(err2 / ref2) : 0.0;
    out[1] = worst;
    out[2] = (nz > 0) ? (double)under / (double)nz : 0.0;
}

/* ========================================================================= */
/* W8A8 (both operands e4m3), [WFK] "Required reasoning process" steps 2, 4   */
/* and 5 and its correctness requirements: activations quantized per token   */
/* (row of x) exactly as weights are per channel (o_quantize_rows on x),      */
/* fp32 accumulation of the e4m3 x e4m3 products, and the epilogue           */
/*   y[m,n] = acc[m,n] * scale_x[m] * scale_w[n] + bias[n],                  */
/* with scale_x indexed by the row, scale_w by the column. In fp64 here:     */
/* every product of two e4m3 values is exact, so only the sum rounds.         */
/* ========================================================================= */
void o_linear_w8a8_f64(const uint8_t *qx, const float *sx, int64_t m, int64_t k, const uint8_t *qw,
                       const float *sw, const double *bias, int64_t n, double *y)
{
    double lut[256];
    for (int c = 0; c < 256; ++c)
        lut[c] = o_e4m3_decode((uint8_t)c);
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < n; ++c) {
        const uint8_t *wr = qw + c * k;
        for (int64_t r = 0; r < m; ++r) {
            const uint8_t *xr = qx + r * k;
            double acc = 0.0;
            for (int64_t j = 0; j < k; ++j)
                acc += lut[xr[j]] * lut[wr[j]];
            y[r * n + c] = acc * (double)sx[r] * (double)sw[c] + (bias ? bias[c] : 0.0);
        }
    }
}

/* ========================================================================= */
/* The other e4m3: E4M3FNUZ ([B04] "The numbers, derived rather than         */
/* tabulated", its table row and footnote; "Hardware support, and where the   */
/* vendors diverge"; the "values 2x off" trap). Fields as OCP e4m3 but bias 8, */
/* no infinities, no negative zero, and one NaN: 0x80. Every other pattern is */
/* finite, the top exponent included (maximum 1.875 * 2^7 = 240).            */
/* ========================================================================= */
double o_fnuz_decode(uint8_t c)
{
    if (c == 0x80)
        return NAN;
    const int s = (c >> 7) & 1;
    const int e = (c >> 3) & 15;
    const int m = c & 7;
    double v;
    if (e == 0)
        v = ldexp((double)m, 1 - 8 - 3);            /* subnormal: m * 2^-10 */
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 8);    /* normal: 1.m * 2^(e-8) */
    return s ? -v : v;
}

/* An FNUZ-coded weight carried over to OCP codes with its scales unchanged:  */
/* each code becomes the OCP code of the same value, by the encoder above     */
/* (round to nearest even; every FNUZ value is within the OCP range). NaN     */
/* stays NaN (0x7F).                                                           */
void o_fnuz_to_ocp(const uint8_t *src, int64_t count, uint8_t *dst)
{
    uint8_t table[256];
    for (int c = 0; c < 256; ++c) {
        const double v = o_fnuz_decode((uint8_t)c);
        table[c] = isnan(v) ? 0x7F : o_e4m3_encode((float)v);
    }
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i)
        dst[i] = table[src[i]];
}

/* Number of OpenMP threads the oracle runs with (1 without OpenMP). */
int o_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void o_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}
