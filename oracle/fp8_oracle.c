/*
 * fp8_oracle.c -- plain CPU oracle (test infrastructure only; see fp8_oracle.h).
 *
 * Built with gcc, -O2 -fno-fast-math -ffp-contract=off, so that every fp32
 * operation below is one correctly rounded IEEE operation and no FMA is
 * formed behind our back.  fp64 is used where the definition is a real-valued
 * sum (the GEMM) or a real-valued rounding (the FP8 grid, bf16 output).
 */
#include "fp8_oracle.h"

#include <float.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------- formats
 * Bit splits from "How to Enable FP8 Training in NanoChat", section "FP8
 * Training Modes Explained" (e4m3: 4+3, e5m2: 5+2).  Encodings: the OCP
 * E4M3FN / E5M2 forms, the only ones whose largest finite values are the
 * 448 and 57344 printed in "FP8 stability guardrails", section "Why FP8 is
 * tempting and why it is fragile".
 *   E4M3: bias 7, no Inf, S.1111.111 is NaN.
 *   E5M2: bias 15, exponent 31 holds Inf (mantissa 0) and NaN (mantissa != 0).
 */
static int mbits(int fmt) { return fmt == ORC_E4M3 ? 3 : 2; }
static int ebits(int fmt) { return fmt == ORC_E4M3 ? 4 : 5; }
static int ebias(int fmt) { return fmt == ORC_E4M3 ? 7 : 15; }
/* exponent of the smallest normal number: 1 - bias */
static int emin(int fmt) { return 1 - ebias(fmt); }

int orc_mant_bits(int fmt) { return mbits(fmt); }
int orc_exp_bits(int fmt) { return ebits(fmt); }

double orc_decode(int fmt, uint8_t code)
{
    const int mb = mbits(fmt);
    const int sign = code >> 7;
    const int e = (code >> mb) & ((1 << ebits(fmt)) - 1);
    const int m = code & ((1 << mb) - 1);
    double v;
    if (fmt == ORC_E4M3) {
        if (e == 15 && m == 7) return NAN;
    } else {
        if (e == 31) {
            if (m != 0) return NAN;
            return sign ? -INFINITY : INFINITY;
        }
    }
    if (e == 0)
        v = ldexp((double)m, emin(fmt) - mb);                  /* subnormal: m * 2^(emin-mb) */
    else
        v = ldexp(1.0 + (double)m / (double)(1 << mb), e - ebias(fmt));
    return sign ? -v : v;
}

/* Largest finite value: exponent field all ones minus one step (E4M3 keeps
 * the top exponent but loses mantissa 111 to NaN). */
double orc_fmax(int fmt)
{
    return fmt == ORC_E4M3 ? orc_decode(fmt, 0x7E) : orc_decode(fmt, 0x7B);
}

static uint8_t max_code(int fmt) { return fmt == ORC_E4M3 ? 0x7E : 0x7B; }

/* ---------------------------------------------------------------- encode
 * v is already fl32(x/s).  Round |v| to the nearest point of the grid
 *   { j * 2^(E - mb) : j integer },  E = max(floor(log2|v|), emin)
 * which is the format's grid extended without an upper exponent bound;
 * nearbyint() in the default rounding mode breaks ties to even j, which is
 * the even-mantissa rule.  Then: above fmax saturates ("overflow ... or
 * saturate"), zero from a non-zero source is an underflow ("underflow to
 * zero"), NaN maps to the all-ones code with the sign kept. */
uint8_t orc_encode(int fmt, float v, int src_nonzero, int* event)
{
    const int mb = mbits(fmt);
    const double fmax = orc_fmax(fmt);
    const uint8_t sign = signbit(v) ? 0x80 : 0x00;
    *event = ORC_EV_NONE;

    if (isnan(v)) {
        *event = ORC_EV_NAN;
        return sign | 0x7F;
    }
    const double a = fabs((double)v);
    if (isinf(a)) {
        *event = ORC_EV_SATURATED;
        return sign | max_code(fmt);
    }
    int E = emin(fmt);
    if (a > 0.0) {
        int fe;
        frexp(a, &fe);            /* a = f * 2^fe, f in [0.5, 1) */
        if (fe - 1 > E) E = fe - 1;
    }
    const double quantum = ldexp(1.0, E - mb);
    const double r = nearbyint(a / quantum) * quantum;   /* a/quantum is exact in fp64 */

    if (r > fmax) {
        *event = ORC_EV_SATURATED;
        return sign | max_code(fmt);
    }
    if (r == 0.0) {
        if (src_nonzero) *event = ORC_EV_UNDERFLOW;
        return sign;
    }
    /* r is exactly representable: write its fields */
    int re;
    frexp(r, &re);
    re -= 1;                                   /* r in [2^re, 2^(re+1)) */
    unsigned efield, mfield;
    if (re < emin(fmt)) {
        efield = 0;
        mfield = (unsigned)(r / ldexp(1.0, emin(fmt) - mb));
    } else {
        efield = (unsigned)(re + ebias(fmt));
        mfield = (unsigned)(r / ldexp(1.0, re - mb)) - (1u << mb);
    }
    return (uint8_t)(sign | (efield << mb) | mfield);
}

static void count_event(orc_counters* c, int ev)
{
    if (!c) return;
    if (ev == ORC_EV_SATURATED) c->saturated++;
    else if (ev == ORC_EV_UNDERFLOW) c->underflow++;
    else if (ev == ORC_EV_NAN) c->nan++;
}

/* Division by the scale comes before the FP8 cast (#84 lab card, section
 * "Explanation"); the quotient is the IEEE fp32 one. */
uint8_t orc_cast_one(int fmt, float x, float s, orc_counters* ctr)
{
    volatile float v = x / s;   /* one correctly rounded fp32 division */
    int ev;
    uint8_t c = orc_encode(fmt, v, x != 0.0f, &ev);
    /* IEEE 754 leaves the sign of a NaN result unspecified; the NaN code takes
     * the sign the quotient would have, sign(x) xor sign(s). */
    if (ev == ORC_EV_NAN) c = (uint8_t)(((signbit(x) != 0) != (signbit(s) != 0) ? 0x80 : 0) | 0x7F);
    count_event(ctr, ev);
    return c;
}

/* ---------------------------------------------------------------- inputs */
float orc_load(const void* x, int dtype, int64_t idx)
{
    if (dtype == ORC_BF16) {
        /* bf16 is the upper half of an fp32 word */
        uint32_t w = (uint32_t)((const uint16_t*)x)[idx] << 16;
        float f;
        memcpy(&f, &w, sizeof f);
        return f;
    }
    return ((const float*)x)[idx];
}

/* ---------------------------------------------------------------- amax/scale */
float orc_amax_rect(const void* x, int dtype, int64_t ld,
                    int64_t r0, int64_t r1, int64_t c0, int64_t c1)
{
    float best = 0.0f;
    for (int64_t r = r0; r < r1; ++r)
        for (int64_t c = c0; c < c1; ++c) {
            float v = fabsf(orc_load(x, dtype, r * ld + c));
            if (isfinite(v) && v > best) best = v;
        }
    return best;
}

float orc_scale_from_amax(int fmt, float amax)
{
    if (amax == 0.0f) return 1.0f;
    volatile float s = amax / (float)orc_fmax(fmt);   /* fp32 division, RNE */
    if (s < FLT_MIN) s = FLT_MIN;
    return s;
}

static int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

int64_t orc_scale_count(int gran, int64_t rows, int64_t cols)
{
    if (gran == ORC_TENSOR) return 1;
    if (gran == ORC_ROW_1x128) return rows * cdiv(cols, 128);
    return cdiv(rows, 128) * cdiv(cols, 128);
}

/* Scaling group g of a granularity as a rectangle. */
static void group_rect(int gran, int64_t rows, int64_t cols, int64_t g,
                       int64_t* r0, int64_t* r1, int64_t* c0, int64_t* c1)
{
    if (gran == ORC_TENSOR) {
        *r0 = 0; *r1 = rows; *c0 = 0; *c1 = cols;
    } else if (gran == ORC_ROW_1x128) {
        const int64_t nt = cdiv(cols, 128);
        *r0 = g / nt; *r1 = *r0 + 1;
        *c0 = (g % nt) * 128; *c1 = *c0 + 128 < cols ? *c0 + 128 : cols;
    } else {
        const int64_t nt = cdiv(cols, 128);
        *r0 = (g / nt) * 128; *r1 = *r0 + 128 < rows ? *r0 + 128 : rows;
        *c0 = (g % nt) * 128; *c1 = *c0 + 128 < cols ? *c0 + 128 : cols;
    }
}

void orc_amax(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld,
              int gran, float* out)
{
    const int64_t ng = orc_scale_count(gran, rows, cols);
    if (gran == ORC_TENSOR) {
        /* per-row maxima in parallel, then the max of those */
        float best = 0.0f;
        #pragma omp parallel for reduction(max:best) schedule(static)
        for (int64_t r = 0; r < rows; ++r) {
            float v = orc_amax_rect(x, dtype, ld, r, r + 1, 0, cols);
            if (v > best) best = v;
        }
        out[0] = best;
        return;
    }
    #pragma omp parallel for schedule(static)
    for (int64_t g = 0; g < ng; ++g) {
        int64_t r0, r1, c0, c1;
        group_rect(gran, rows, cols, g, &r0, &r1, &c0, &c1);
        out[g] = orc_amax_rect(x, dtype, ld, r0, r1, c0, c1);
    }
}

/* ---------------------------------------------------------------- quantize */
int orc_quantize(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld,
                 int fmt, int gran, int mode, float* scale,
                 uint8_t* q, int64_t ldq, uint8_t* qt, int64_t ldqt,
                 orc_counters* ctr)
{
    if (rows < 0 || cols < 0 || ld < cols || ldq < cols) return -1;
    if (qt && (gran == ORC_ROW_1x128 || ldqt < rows)) return -1;
    const int64_t ng = orc_scale_count(gran, rows, cols);

    if (mode == ORC_FROM_AMAX) {
        /* an empty tensor has amax 0 and therefore scale 1 */
        orc_amax(x, dtype, rows, cols, ld, gran, scale);
        for (int64_t g = 0; g < ng; ++g) scale[g] = orc_scale_from_amax(fmt, scale[g]);
    }
    if (rows == 0 || cols == 0) return 0;

    uint64_t sat = 0, und = 0, nan_ = 0;
    #pragma omp parallel for reduction(+:sat,und,nan_) schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        orc_counters local = {0, 0, 0, 0};
        for (int64_t c = 0; c < cols; ++c) {
            int64_t g;
            if (gran == ORC_TENSOR) g = 0;
            else if (gran == ORC_ROW_1x128) g = r * cdiv(cols, 128) + c / 128;
            else g = (r / 128) * cdiv(cols, 128) + c / 128;
            const uint8_t code = orc_cast_one(fmt, orc_load(x, dtype, r * ld + c), scale[g], &local);
            q[r * ldq + c] = code;
            if (qt) qt[c * ldqt + r] = code;
        }
        sat += local.saturated;
        und += local.underflow;
        nan_ += local.nan;
    }
    if (ctr) {
        ctr->saturated += sat;
        ctr->underflow += und;
        ctr->nan += nan_;
    }
    return 0;
}

/* ---------------------------------------------------------------- GEMM
 * "_scaled_mm(x, w_fp8, scale_a, scale_b)" (#84 lab card, code excerpt and
 * "Explanation"): y = (s_a * A_q)(s_b * B_q)^T, B given K-contiguous (the
 * column-major operand _scaled_mm expects).  Fine-grained form (DeepSeek-V3,
 * "Real products" in the guardrails explainer): each 128-wide K block
 * carries its own pair of scales. */
static int gemm_args_ok(int ga, int gb, int64_t k)
{
    if (ga == ORC_TENSOR && gb == ORC_TENSOR) return 1;
    if (ga == ORC_ROW_1x128 && gb == ORC_BLOCK_128x128) return k % 128 == 0;
    return 0;
}

static double gemm_one(const uint8_t* a, const double* da, int64_t lda, const float* sa, int ga,
                       const uint8_t* b, const double* db, int64_t ldb, const float* sb,
                       int64_t k, int64_t i, int64_t j)
{
    const uint8_t* ar = a + i * lda;
    const uint8_t* br = b + j * ldb;
    if (ga == ORC_TENSOR) {
        double d = 0.0;
        for (int64_t kk = 0; kk < k; ++kk) d += da[ar[kk]] * db[br[kk]];
        return (double)sa[0] * (double)sb[0] * d;
    }
    const int64_t nkb = k / 128;
    double y = 0.0;
    for (int64_t kb = 0; kb < nkb; ++kb) {
        double d = 0.0;
        for (int64_t kk = kb * 128; kk < kb * 128 + 128; ++kk) d += da[ar[kk]] * db[br[kk]];
        y += (double)sa[i * nkb + kb] * (double)sb[(j / 128) * nkb + kb] * d;
    }
    return y;
}

int orc_gemm(const uint8_t* a, int fa, int64_t lda, const float* sa, int ga,
             const uint8_t* b, int fb, int64_t ldb, const float* sb, int gb,
             int64_t m, int64_t n, int64_t k, double* y, int64_t ldy)
{
    if (!gemm_args_ok(ga, gb, k)) return -1;
    double da[256], db[256];
    for (int c = 0; c < 256; ++c) {
        da[c] = orc_decode(fa, (uint8_t)c);
        db[c] = orc_decode(fb, (uint8_t)c);
    }
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < m; ++i)
        for (int64_t j = 0; j < n; ++j)
            y[i * ldy + j] = gemm_one(a, da, lda, sa, ga, b, db, ldb, sb, k, i, j);
    return 0;
}

int orc_gemm_points(const uint8_t* a, int fa, int64_t lda, const float* sa, int ga,
                    const uint8_t* b, int fb, int64_t ldb, const float* sb, int gb,
                    int64_t m, int64_t n, int64_t k,
                    const int64_t* pm, const int64_t* pn, int64_t npts, double* out)
{
    if (!gemm_args_ok(ga, gb, k)) return -1;
    for (int64_t p = 0; p < npts; ++p)
        if (pm[p] < 0 || pm[p] >= m || pn[p] < 0 || pn[p] >= n) return -1;
    double da[256], db[256];
    for (int c = 0; c < 256; ++c) {
        da[c] = orc_decode(fa, (uint8_t)c);
        db[c] = orc_decode(fb, (uint8_t)c);
    }
    #pragma omp parallel for schedule(dynamic, 16)
    for (int64_t p = 0; p < npts; ++p)
        out[p] = gemm_one(a, da, lda, sa, ga, b, db, ldb, sb, k, pm[p], pn[p]);
    return 0;
}

/* ---------------------------------------------------------------- bf16 out
 * bf16 keeps fp32's 8 exponent bits and 7 stored mantissa bits ("#84",
 * section "Hardware precision"): round the real value to 8 significant bits,
 * ties to even, overflow to Inf when the rounded value leaves the range. */
uint16_t orc_bf16_rne(double y)
{
    if (isnan(y)) return 0x7FC0;
    const uint16_t sign = signbit(y) ? 0x8000 : 0;
    double a = fabs(y);
    if (isinf(a)) return sign | 0x7F80;
    const int emin_b = -126;              /* smallest normal exponent */
    int E = emin_b;
    if (a > 0.0) {
        int fe;
        frexp(a, &fe);
        if (fe - 1 > E) E = fe - 1;
    }
    const double quantum = ldexp(1.0, E - 7);
    const double r = nearbyint(a / quantum) * quantum;
    const double bmax = ldexp(255.0 / 128.0, 127);   /* 0x7F7F */
    if (r > bmax) return sign | 0x7F80;
    /* r is a bf16 value: its fp32 encoding has 16 zero low bits */
    float f = (float)r;
    uint32_t w;
    memcpy(&w, &f, sizeof w);
    return sign | (uint16_t)(w >> 16);
}

uint64_t orc_count_nonfinite_bf16(const double* y, int64_t count)
{
    uint64_t n = 0;
    for (int64_t i = 0; i < count; ++i) {
        uint16_t h = orc_bf16_rne(y[i]);
        if ((h & 0x7F80) == 0x7F80) n++;
    }
    return n;
}

int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
