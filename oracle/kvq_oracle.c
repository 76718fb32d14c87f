/*
 * kvq_oracle.c -- CPU oracle for the paged quantized KV-cache decode path.
 *
 * TEST INFRASTRUCTURE ONLY (see kvq_oracle.h).  Plain, slow, obviously
 * correct: every number format is built from its definition with exact
 * double arithmetic, the quantizers follow the pages' pipeline step by step,
 * and attention is the softmax definition evaluated in fp64.
 *
 * Build: gcc -O2 -std=c99 -fopenmp -ffp-contract=off -fno-fast-math -fPIC -shared
 * (no contraction, so every float32 operation below is one IEEE operation).
 */
#include "kvq_oracle.h"

#include <float.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>

static uint32_t f32_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float bits_f32(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

/* ======================================================================= *
 * bfloat16: the upper half of an IEEE binary32.                            *
 * ======================================================================= */
float kvqo_bf16_value(uint16_t bits) { return bits_f32((uint32_t)bits << 16); }

/* Truncation toward zero keeps the upper 16 bits; the other bracketing bf16
 * value is one unit further from zero.                                      */
static uint16_t bf16_trunc(float f) { return (uint16_t)(f32_bits(f) >> 16); }

uint16_t kvqo_bf16_up(float f)
{
    if (isnan(f)) return 0x7FC0;
    uint16_t t = bf16_trunc(f);
    if ((double)kvqo_bf16_value(t) == (double)f) return t;
    return f > 0.0f ? (uint16_t)(t + 1) : t;          /* t + 1 grows |value|  */
}

uint16_t kvqo_bf16_down(float f)
{
    if (isnan(f)) return 0x7FC0;
    uint16_t t = bf16_trunc(f);
    if ((double)kvqo_bf16_value(t) == (double)f) return t;
    return f < 0.0f ? (uint16_t)(t + 1) : t;
}

uint16_t kvqo_bf16_rne(float f)
{
    if (isnan(f)) return 0x7FC0;
    uint16_t t = bf16_trunc(f);
    double a = kvqo_bf16_value(t);
    if (a == (double)f) return t;
    uint16_t u = (uint16_t)(t + 1);
    /* value of the next representable point (as if the exponent continued) */
    double b = ((u & 0x7FFF) == 0x7F80) ? copysign(ldexp(1.0, 128), a) : (double)kvqo_bf16_value(u);
    double da = fabs((double)f - a), db = fabs(b - (double)f);
    if (da < db) return t;
    if (db < da) return u;
    return (t & 1) ? u : t;                            /* tie: even mantissa  */
}

/* ======================================================================= *
 * IEEE binary16 (KIVI residual window only).                               *
 * ======================================================================= */
double kvqo_f16_value(uint16_t h)
{
    int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
    double v;
    if (e == 31) v = m ? NAN : INFINITY;
    else if (e == 0) v = ldexp((double)m, -24);
    else v = ldexp((double)(1024 + m), e - 25);
    return s ? -v : v;
}

uint16_t kvqo_f16_rne(double x)
{
    if (isnan(x)) return 0x7E00;
    uint16_t sg = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (a >= 65520.0) return sg | 0x7C00;              /* rounds past 65504   */
    if (a < ldexp(1.0, -14)) {                          /* subnormal binade    */
        double m = nearbyint(a * ldexp(1.0, 24));       /* 0 .. 1024           */
        return sg | (uint16_t)m;                        /* 1024 = min normal   */
    }
    int ex;
    frexp(a, &ex);
    int e = ex - 1;                                     /* a in [2^e, 2^e+1)   */
    double m = nearbyint((ldexp(a, -e) - 1.0) * 1024.0);
    if (m == 1024.0) { e += 1; m = 0.0; }
    if (e + 15 >= 31) return sg | 0x7C00;
    return sg | (uint16_t)(((e + 15) << 10) | (int)m);
}

void kvqo_bf16_to_f16_array(const uint16_t* bf16, int64_t n, uint16_t* f16)
{
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) f16[i] = kvqo_f16_rne((double)kvqo_bf16_value(bf16[i]));
}

/* ======================================================================= *
 * OCP FP8 E4M3 (the "FN" variant: no infinities, one NaN pattern per sign). *
 * 4 exponent bits (bias 7), 3 mantissa bits; largest finite 448 = 0x7E.     *
 * The pages name E4M3 as 4 exponent / 3 mantissa bits ([molayo] formats     *
 * notes; [ryotta] §3.1).  [ryotta] §3.1 also quotes a +-240 range, which is  *
 * the FNUZ variant's; the OCP encoding, max 448, is the one used here.      *
 * ======================================================================= */
double kvqo_e4m3_value(uint8_t c)
{
    int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    if (e == 15 && m == 7) return NAN;
    double v = (e == 0) ? ldexp((double)m, -9)          /* m * 2^-9            */
                        : ldexp((double)(8 + m), e - 10); /* (1+m/8) 2^(e-7)   */
    return s ? -v : v;
}

/* Round to the nearest E4M3 value, ties to the even mantissa, saturating at
 * +-448; the sign of zero is kept (-0 and negatives that round to 0 give 0x80).
 * The rule is applied to the exact value y (float32 inputs convert exactly). */
uint8_t kvqo_e4m3_encode_f64(double y)
{
    if (isnan(y)) return 0x7F;
    uint8_t sg = signbit(y) ? 0x80 : 0x00;
    double a = fabs(y);
    if (a >= 448.0) return sg | 0x7E;
    if (a < ldexp(1.0, -6)) {                           /* subnormal binade    */
        double m = nearbyint(a * ldexp(1.0, 9));        /* 0 .. 8; 8 = 2^-6    */
        return sg | (uint8_t)m;
    }
    int ex;
    frexp(a, &ex);
    int e = ex - 1;                                     /* -6 .. 8             */
    double m = nearbyint((ldexp(a, -e) - 1.0) * 8.0);   /* 0 .. 8              */
    if (m == 8.0) { e += 1; m = 0.0; }
    return sg | (uint8_t)(((e + 7) << 3) | (int)m);
}

uint8_t kvqo_e4m3_encode(float y) { return kvqo_e4m3_encode_f64((double)y); }

void kvqo_e4m3_encode_range(uint32_t first_bits, uint32_t count, uint8_t* codes)
{
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < (int64_t)count; ++i)
        codes[i] = kvqo_e4m3_encode(bits_f32(first_bits + (uint32_t)i));
}

void kvqo_e4m3_encode_array(const float* y, int64_t n, uint8_t* codes)
{
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) codes[i] = kvqo_e4m3_encode(y[i]);
}

/* ======================================================================= *
 * OCP FP8 E5M2: 5 exponent bits (bias 15), 2 mantissa bits, with IEEE-style *
 * specials: exponent 31 holds +-inf (mantissa 0) and NaN (mantissa != 0).  *
 * Largest finite 57344 = 0x7B; subnormals m * 2^-16.  The pages name E5M2  *
 * as the wider-range, lower-precision FP8 format and list it among the KV  *
 * cache dtypes ([molayo] formats notes and the serving-flag values;        *
 * [ryotta] §3.1).                                                          *
 * ======================================================================= */
double kvqo_e5m2_value(uint8_t c)
{
    int s = c >> 7, e = (c >> 2) & 31, m = c & 3;
    double v;
    if (e == 31) v = (m == 0) ? INFINITY : NAN;
    else if (e == 0) v = ldexp((double)m, -16);               /* m * 2^-16          */
    else v = ldexp((double)(4 + m), e - 17);                  /* (1+m/4) 2^(e-15)   */
    return s ? -v : v;
}

/* Round to the nearest E5M2 value, ties to the even mantissa, saturating at
 * +-57344 (the same rule as E4M3: no infinities are produced); NaN -> 0x7F;
 * the sign of zero is kept. */
uint8_t kvqo_e5m2_encode(float y)
{
    if (isnan(y)) return 0x7F;
    uint8_t sg = signbit(y) ? 0x80 : 0x00;
    double a = fabs((double)y);
    if (a >= 57344.0) return sg | 0x7B;
    if (a < ldexp(1.0, -14)) {                          /* subnormal binade    */
        double m = nearbyint(a * ldexp(1.0, 16));       /* 0 .. 4; 4 = 2^-14   */
        return sg | (uint8_t)m;
    }
    int ex;
    frexp(a, &ex);
    int e = ex - 1;                                     /* -14 .. 15           */
    double m = nearbyint((ldexp(a, -e) - 1.0) * 4.0);   /* 0 .. 4              */
    if (m == 4.0) { e += 1; m = 0.0; }
    return sg | (uint8_t)(((e + 15) << 2) | (int)m);
}

void kvqo_e5m2_encode_range(uint32_t first_bits, uint32_t count, uint8_t* codes)
{
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < (int64_t)count; ++i)
        codes[i] = kvqo_e5m2_encode(bits_f32(first_bits + (uint32_t)i));
}

void kvqo_e5m2_encode_array(const float* y, int64_t n, uint8_t* codes)
{
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) codes[i] = kvqo_e5m2_encode(y[i]);
}

/* ======================================================================= *
 * Quantizers.  Quantization happens once, when a token's K/V row is stored, *
 * from the full-precision values, with a per-(token, head) scale kept in     *
 * BF16 next to the codes ([molayo] "what it is"; [ryotta] §5.1 and §6.3).    *
 * The scale maps the row's extreme(s) onto the end(s) of the code range and  *
 * is rounded outward to BF16 so that no element saturates; codes use         *
 * round-half-to-even.                                                        *
 * ======================================================================= */
void kvqo_fp8_row(const uint16_t* x, int n, uint8_t* codes, uint16_t* scale)
{
    float amax = 0.0f;
    for (int i = 0; i < n; ++i) {
        float a = fabsf(kvqo_bf16_value(x[i]));
        if (a > amax) amax = a;
    }
    float s32 = amax / 448.0f;                           /* one IEEE division   */
    uint16_t s = kvqo_bf16_up(s32);
    float sf = kvqo_bf16_value(s);
    *scale = s;
    for (int i = 0; i < n; ++i)
        codes[i] = (sf == 0.0f) ? 0x00 : kvqo_e4m3_encode(kvqo_bf16_value(x[i]) / sf);
}

void kvqo_fp8_row_static(const uint16_t* x, int n, uint16_t scale, uint8_t* codes)
{
    float sf = kvqo_bf16_value(scale);
    for (int i = 0; i < n; ++i)
        codes[i] = (sf == 0.0f) ? 0x00 : kvqo_e4m3_encode(kvqo_bf16_value(x[i]) / sf);
}

/* The same two FP8 quantizers with the E5M2 code: the per-(token, head) scale
 * maps the row's largest magnitude onto 57344. */
void kvqo_e5m2_row(const uint16_t* x, int n, uint8_t* codes, uint16_t* scale)
{
    float amax = 0.0f;
    for (int i = 0; i < n; ++i) {
        float a = fabsf(kvqo_bf16_value(x[i]));
        if (a > amax) amax = a;
    }
    float s32 = amax / 57344.0f;                         /* one IEEE division   */
    uint16_t s = kvqo_bf16_up(s32);
    float sf = kvqo_bf16_value(s);
    *scale = s;
    for (int i = 0; i < n; ++i)
        codes[i] = (sf == 0.0f) ? 0x00 : kvqo_e5m2_encode(kvqo_bf16_value(x[i]) / sf);
}

void kvqo_e5m2_row_static(const uint16_t* x, int n, uint16_t scale, uint8_t* codes)
{
    float sf = kvqo_bf16_value(scale);
    for (int i = 0; i < n; ++i)
        codes[i] = (sf == 0.0f) ? 0x00 : kvqo_e5m2_encode(kvqo_bf16_value(x[i]) / sf);
}

/* Asymmetric unsigned quantizer with `levels` steps ([molayo] formats notes:
 * a (scale, zero_point) pair per token; [ryotta] §3.1 KIVI):
 *   z = bf16 floor of min,  s = bf16 ceil of (max - z) / levels,
 *   code = clamp(rne((x - z) / s), 0, levels),  x^ = code * s + z.          */
void kvqo_uint_asym(const float* x, int n, int stride, int levels,
                    uint8_t* codes, int code_stride, uint16_t* scale, uint16_t* zero)
{
    float lo = INFINITY, hi = -INFINITY;
    for (int i = 0; i < n; ++i) {
        float v = x[(int64_t)i * stride];
        if (v < lo) lo = v;
        if (v > hi) hi = v;
    }
    uint16_t z = kvqo_bf16_down(lo);
    float zf = kvqo_bf16_value(z);
    float range = hi - zf;                               /* float32 difference  */
    uint16_t s = kvqo_bf16_up(range / (float)levels);
    float sf = kvqo_bf16_value(s);
    *scale = s;
    *zero = z;
    for (int i = 0; i < n; ++i) {
        uint8_t c = 0;
        if (sf != 0.0f) {
            float t = (x[(int64_t)i * stride] - zf) / sf;
            double r = nearbyint((double)t);
            if (r < 0.0) r = 0.0;
            if (r > (double)levels) r = (double)levels;
            c = (uint8_t)r;
        }
        codes[(int64_t)i * code_stride] = c;
    }
}

void kvqo_int8_row(const uint16_t* x, int n, uint8_t* codes, uint16_t* scale, uint16_t* zero)
{
    float buf[n];
    for (int i = 0; i < n; ++i) buf[i] = kvqo_bf16_value(x[i]);
    kvqo_uint_asym(buf, n, 1, 255, codes, 1, scale, zero);
}

void kvqo_quantize_rows(int dtype, int mode, const uint16_t* x, int64_t rows, int n,
                        const uint16_t* static_scale, uint8_t* codes, uint16_t* scale,
                        uint16_t* zero)
{
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const uint16_t* xr = x + r * n;
        uint8_t* cr = codes + r * n;
        if (dtype == 1 && mode == 2) kvqo_fp8_row(xr, n, cr, &scale[r]);
        else if (dtype == 1) { kvqo_fp8_row_static(xr, n, static_scale[r], cr); if (scale) scale[r] = static_scale[r]; }
        else if (dtype == 4 && mode == 2) kvqo_e5m2_row(xr, n, cr, &scale[r]);
        else if (dtype == 4) { kvqo_e5m2_row_static(xr, n, static_scale[r], cr); if (scale) scale[r] = static_scale[r]; }
        else kvqo_int8_row(xr, n, cr, &scale[r], &zero[r]);
    }
}

void kvqo_dequantize_rows(int dtype, int mode, const uint8_t* codes, int64_t rows, int n,
                          const uint16_t* scale, const uint16_t* zero, double* out)
{
    (void)mode;
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        double s = kvqo_bf16_value(scale[r]);
        double z = (dtype == 2) ? (double)kvqo_bf16_value(zero[r]) : 0.0;
        for (int i = 0; i < n; ++i) {
            uint8_t c = codes[r * n + i];
            out[r * n + i] = (dtype == 1) ? s * kvqo_e4m3_value(c)
                           : (dtype == 4) ? s * kvqo_e5m2_value(c)
                                          : (double)c * s + z;
        }
    }
}

/* ======================================================================= *
 * KIVI-style b-bit ([ryotta] §3.1 KIVI: asymmetric 2-bit; [molayo] formats *
 * notes on mixed 4-bit): K per channel, V per token, the most recent       *
 * tokens kept in full precision.  Tokens leave the fp16 window in whole    *
 * groups, oldest first, once the window holds more than `resid` tokens.    *
 * b = 4 or 2: 2^b - 1 steps of the asymmetric quantizer above.             *
 * ======================================================================= */
int64_t kvqo_kivi_quantized_count(int64_t T, int resid, int group)
{
    int64_t over = T - resid;
    if (over <= 0) return 0;
    return (over / group) * group;
}

void kvqo_kivi_k(const uint16_t* x16, int64_t nq, int n, int group, int bits,
                 uint8_t* codes, uint16_t* s, uint16_t* z)
{
    int64_t ng = nq / group;
    int levels = (1 << bits) - 1;
    #pragma omp parallel for schedule(static)
    for (int64_t gi = 0; gi < ng; ++gi) {
        float buf[group * n];
        for (int t = 0; t < group; ++t)
            for (int c = 0; c < n; ++c)
                buf[t * n + c] = (float)kvqo_f16_value(x16[(gi * group + t) * n + c]);
        for (int c = 0; c < n; ++c)
            kvqo_uint_asym(buf + c, group, n, levels, codes + gi * group * n + c, n,
                           &s[gi * n + c], &z[gi * n + c]);
    }
}

void kvqo_kivi_v(const uint16_t* x16, int64_t nq, int n, int bits, uint8_t* codes, uint16_t* s, uint16_t* z)
{
    int levels = (1 << bits) - 1;
    #pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < nq; ++t) {
        float buf[n];
        for (int c = 0; c < n; ++c) buf[c] = (float)kvqo_f16_value(x16[t * n + c]);
        kvqo_uint_asym(buf, n, 1, levels, codes + t * n, 1, &s[t], &z[t]);
    }
}

/* ======================================================================= *
 * Attention: softmax(q . k^T * scale) . v per query head, every cached      *
 * token attended, in fp64.  GQA: query head h reads KV head h / (n_q/n_kv). *
 * ======================================================================= */
void kvqo_attention(const double* q, const double* k, const double* v, int64_t T,
                    int n_q, int n_kv, int d, double softmax_scale, double* out, double* lse)
{
    int grp = n_q / n_kv;
    #pragma omp parallel for schedule(static)
    for (int h = 0; h < n_q; ++h) {
        int g = h / grp;
        double* o = out + (int64_t)h * d;
        for (int i = 0; i < d; ++i) o[i] = 0.0;
        if (T == 0) { if (lse) lse[h] = -INFINITY; continue; }
        double mx = -INFINITY;
        for (int64_t t = 0; t < T; ++t) {
            const double* kt = k + (t * n_kv + g) * d;
            double sdot = 0.0;
            for (int i = 0; i < d; ++i) sdot += q[(int64_t)h * d + i] * kt[i];
            double sc = softmax_scale * sdot;
            if (sc > mx) mx = sc;
        }
        double z = 0.0;
        for (int64_t t = 0; t < T; ++t) {
            const double* kt = k + (t * n_kv + g) * d;
            const double* vt = v + (t * n_kv + g) * d;
            double sdot = 0.0;
            for (int i = 0; i < d; ++i) sdot += q[(int64_t)h * d + i] * kt[i];
            double w = exp(softmax_scale * sdot - mx);
            z += w;
            for (int i = 0; i < d; ++i) o[i] += w * vt[i];
        }
        for (int i = 0; i < d; ++i) o[i] /= z;
        if (lse) lse[h] = mx + log(z);
    }
}

/* ======================================================================= *
 * Attention with the score-V product in the FP8 domain.  Some backends run   *
 * QK and the score-V product themselves in FP8 ([daewooki] core concept 3);  *
 * the pages give no rule for the probabilities, so this reading fixes one:   *
 *  - scores as above; lambda_t = score_t / ln 2 (log2 units);               *
 *  - the context is cut into blocks of `block` tokens from token 0; block    *
 *    c takes the reference mu_c = ceil(max_{t in c} lambda_t) (an integer);  *
 *  - P_t = 2^(lambda_t - mu_c) * vs_t, the weight of token t relative to its *
 *    block times the token's V scale (the V row is x^ = vs_t * vcode_t);    *
 *  - S_c = 2^E_c, the smallest power of two with max_{t in c} P_t <= 448 S_c;*
 *  - pi_t = E4M3 code of P_t / S_c (nearest-even; never saturates);          *
 *  - out = sum_t 2^(mu_c - M) S_c e4m3(pi_t) vcode_t / sum_t 2^(lambda_t - M)*
 *    for any M (the largest mu_c here): the exact attention with each       *
 *    P_t replaced by its E4M3 value.  lse is the exact one.                  *
 * vcode: decoded V codes without their scale [T][n_kv][d]; vs [T][n_kv].    *
 * allowance [n_q][d]: for every token whose P_t / S_c lies within a relative *
 * a_t of an E4M3 rounding boundary, one code step times its weight and       *
 * |vcode|, where a_t = 2^-18 + score_rel * softmax_scale * sum_i |q_i k_ti|: *
 * an evaluation whose scores are off by up to score_rel of that sum (and     *
 * whose P is otherwise float32) may take the neighbouring code.  Where the   *
 * block maximum lies that close to a power-of-two boundary of S_c, the       *
 * block's subnormal-range codes count one subnormal step of 2 S_c too.      *
 * All divided by the softmax denominator, like out.                          *
 * ======================================================================= */
static int e4m3_neighbour_steps(double y, double* lo_step, double* hi_step, double* lo_mid, double* hi_mid)
{
    uint8_t c = kvqo_e4m3_encode_f64(y);              /* y >= 0 here        */
    double v = kvqo_e4m3_value(c);
    double vl = c > 0 ? kvqo_e4m3_value((uint8_t)(c - 1)) : v;
    double vh = c < 0x7E ? kvqo_e4m3_value((uint8_t)(c + 1)) : v;
    *lo_step = v - vl;
    *hi_step = vh - v;
    *lo_mid = 0.5 * (v + vl);
    *hi_mid = 0.5 * (v + vh);
    return c;
}

void kvqo_attention_fp8pv(const double* q, const double* k, const double* vcode, const double* vs,
                          int64_t T, int n_q, int n_kv, int d, double softmax_scale, int block,
                          double score_rel, double* out, double* lse, double* allowance)
{
    int grp = n_q / n_kv;
    #pragma omp parallel for schedule(static)
    for (int h = 0; h < n_q; ++h) {
        int g = h / grp;
        double* o = out + (int64_t)h * d;
        double* al = allowance + (int64_t)h * d;
        for (int i = 0; i < d; ++i) { o[i] = 0.0; al[i] = 0.0; }
        if (T == 0) { if (lse) lse[h] = -INFINITY; continue; }
        double* lam = (double*)malloc(sizeof(double) * (size_t)T);
        double* amb = (double*)malloc(sizeof(double) * (size_t)T);
        for (int64_t t = 0; t < T; ++t) {
            const double* kt = k + (t * n_kv + g) * d;
            double sdot = 0.0, sabs = 0.0;
            for (int i = 0; i < d; ++i) {
                sdot += q[(int64_t)h * d + i] * kt[i];
                sabs += fabs(q[(int64_t)h * d + i] * kt[i]);
            }
            lam[t] = softmax_scale * sdot / M_LN2;
            amb[t] = ldexp(1.0, -18) + score_rel * softmax_scale * sabs;
        }
        /* M = the largest block reference; L = sum_t 2^(lambda_t - M) */
        double M = -INFINITY;
        for (int64_t t = 0; t < T; ++t) if (ceil(lam[t]) > M) M = ceil(lam[t]);
        double L = 0.0;
        for (int64_t t = 0; t < T; ++t) L += exp2(lam[t] - M);
        for (int64_t b0 = 0; b0 < T; b0 += block) {
            int64_t b1 = b0 + block < T ? b0 + block : T;
            double mx = -INFINITY;
            for (int64_t t = b0; t < b1; ++t) if (lam[t] > mx) mx = lam[t];
            double mu = ceil(mx);
            double pmax = 0.0, amax_amb = 0.0;
            for (int64_t t = b0; t < b1; ++t) {
                double P = exp2(lam[t] - mu) * vs[t * n_kv + g];
                if (P > pmax) { pmax = P; amax_amb = amb[t]; }
            }
            if (pmax == 0.0) continue;
            /* smallest E with pmax <= 448 * 2^E (exact comparisons) */
            int E = ilogb(pmax) - 8;
            while (pmax > ldexp(448.0, E)) ++E;
            while (pmax <= ldexp(448.0, E - 1)) --E;
            double S = ldexp(1.0, E);
            int s_edge = fabs(pmax - ldexp(448.0, E - 1)) <= amax_amb * pmax;   /* S or 2 S */
            double wgt = S * exp2(mu - M);
            for (int64_t t = b0; t < b1; ++t) {
                double y = exp2(lam[t] - mu) * vs[t * n_kv + g] / S;       /* exact division */
                double ls, hs, lm, hm;
                uint8_t c = (uint8_t)e4m3_neighbour_steps(y, &ls, &hs, &lm, &hm);
                double w = kvqo_e4m3_value(c) * wgt;
                double step = 0.0;
                if (fabs(y - lm) <= amb[t] * y && ls > 0.0) step = ls;
                if (fabs(y - hm) <= amb[t] * y && hs > step) step = hs;
                if (s_edge && y < ldexp(1.0, -5)) step += ldexp(1.0, -8);
                const double* vt = vcode + (t * n_kv + g) * d;
                for (int i = 0; i < d; ++i) {
                    o[i] += w * vt[i];
                    al[i] += step * wgt * fabs(vt[i]);
                }
            }
        }
        for (int i = 0; i < d; ++i) { o[i] /= L; al[i] /= L; }
        if (lse) lse[h] = M * M_LN2 + log(L);
        free(lam);
        free(amb);
    }
}

/* Merging the softmax results of disjoint token ranges: each part i is
 * (o_i, lse_i); weights exp(lse_i - L) with L = max lse_i.                 */
void kvqo_lse_merge(const double* o, const double* lse, int P, int d, double* out, double* lse_out)
{
    double L = -INFINITY;
    for (int i = 0; i < P; ++i) if (lse[i] > L) L = lse[i];
    for (int c = 0; c < d; ++c) out[c] = 0.0;
    if (L == -INFINITY) { if (lse_out) *lse_out = -INFINITY; return; }
    double wsum = 0.0;
    for (int i = 0; i < P; ++i) {
        double w = exp(lse[i] - L);
        wsum += w;
        for (int c = 0; c < d; ++c) out[c] += w * o[(int64_t)i * d + c];
    }
    for (int c = 0; c < d; ++c) out[c] /= wsum;
    if (lse_out) *lse_out = L + log(wsum);
}

/* ======================================================================= *
 * KV bytes = 2 (K and V) x layers x kv heads x head_dim x seq x batch x     *
 * bytes per element ([ryotta] §1; [molayo] TL;DR; [story] §2).              *
 * ======================================================================= */
double kvqo_kv_bytes(double layers, double n_kv_heads, double head_dim, double seq_len,
                     double batch, double bytes_per_elem)
{
    return 2.0 * layers * n_kv_heads * head_dim * seq_len * batch * bytes_per_elem;
}
