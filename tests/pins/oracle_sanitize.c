/*
 * Memory and undefined-behaviour check of the CPU oracle (not a parity pin):
 * built together with oracle/fp8_oracle.c under gcc's AddressSanitizer and
 * UndefinedBehaviorSanitizer (no recovery), it drives every exported function
 * over small and edge-case shapes: empty, single element, ragged tails of the
 * 128-wide groups, leading dimensions wider than the row, both input types,
 * every granularity and scale mode, both formats, the transposed copy, the
 * GEMM in both scale modes and at sampled points, and every special value of
 * the bf16 rounding.  Each buffer is allocated with exactly the bytes its
 * shape needs, so a read or write past a row end or a matrix end is caught.
 * A few plain invariants are checked on the way (codes decode to values on
 * the format grid, a zero matrix quantizes to zero codes with scale 1).
 * Exit 0 and "OK <n>" on success, where n counts the calls made.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "fp8_oracle.h"

static uint64_t g_state = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(void)
{
    /* xorshift64*: input data only */
    g_state ^= g_state >> 12;
    g_state ^= g_state << 25;
    g_state ^= g_state >> 27;
    return (uint32_t)((g_state * 0x2545F4914F6CDD1Dull) >> 32);
}

static long g_calls = 0;

/* exactly n bytes (an empty shape still gets a distinct pointer) */
static void* alloc_exact(size_t n) { return malloc(n ? n : 1); }

static void fail(const char* what)
{
    printf("FAIL %s\n", what);
    exit(1);
}

/* A bf16 or fp32 matrix of rows x ld elements with random finite values,
 * a few outliers, and (if special) Inf, NaN, -0 and subnormals. */
static void* make_input(int dtype, int64_t rows, int64_t cols, int64_t ld, int special)
{
    const size_t n = rows > 0 ? (size_t)((rows - 1) * ld + cols) : 0;
    const size_t eb = dtype == ORC_BF16 ? 2 : 4;
    void* x = alloc_exact(n * eb);
    for (size_t i = 0; i < n; ++i) {
        float v = ((float)(rnd() % 20001) - 10000.0f) * 1e-4f;
        if (rnd() % 97 == 0) v *= 3000.0f;
        if (special) {
            const uint32_t r = rnd() % 211;
            if (r == 0) v = INFINITY;
            if (r == 1) v = -INFINITY;
            if (r == 2) v = NAN;
            if (r == 3) v = -0.0f;
            if (r == 4) v = 1e-40f;
        }
        if (dtype == ORC_BF16) {
            uint32_t b;
            memcpy(&b, &v, 4);
            ((uint16_t*)x)[i] = (uint16_t)(b >> 16);
        } else {
            ((float*)x)[i] = v;
        }
    }
    return x;
}

static void check_codes(int fmt, const uint8_t* q, int64_t rows, int64_t cols, int64_t ldq)
{
    const double fmax = orc_fmax(fmt);
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) {
            const double v = orc_decode(fmt, q[r * ldq + c]);
            if (!isnan(v) && fabs(v) > fmax) fail("decoded code above fmax");
        }
}

static void one_quantize(int dtype, int64_t rows, int64_t cols, int64_t ld, int fmt, int gran, int mode,
                         int want_t, int special)
{
    void* x = make_input(dtype, rows, cols, ld, special);
    const int64_t ns = orc_scale_count(gran, rows, cols);
    float* amax = alloc_exact((size_t)ns * 4);
    float* scale = alloc_exact((size_t)ns * 4);
    const int64_t ldq = cols + (ld > cols ? 3 : 0), ldqt = rows + (ld > cols ? 5 : 0);
    const size_t nq = rows > 0 ? (size_t)((rows - 1) * ldq + cols) : 0;
    const size_t nqt = cols > 0 ? (size_t)((cols - 1) * ldqt + rows) : 0;
    uint8_t* q = alloc_exact(nq);
    uint8_t* qt = want_t ? alloc_exact(nqt) : NULL;
    orc_amax(x, dtype, rows, cols, ld, gran, amax);
    ++g_calls;
    for (int64_t i = 0; i < ns; ++i) scale[i] = mode == ORC_GIVEN ? 0.001f * (float)(1 + i % 7) : 0.0f;
    orc_counters ctr = {0, 0, 0, 0};
    if (orc_quantize(x, dtype, rows, cols, ld, fmt, gran, mode, scale, q, ldq, qt, ldqt, &ctr) != 0)
        fail("orc_quantize rejected valid arguments");
    ++g_calls;
    check_codes(fmt, q, rows, cols, ldq);
    if (qt)
        for (int64_t r = 0; r < rows; ++r)
            for (int64_t c = 0; c < cols; ++c)
                if (qt[c * ldqt + r] != q[r * ldq + c]) fail("transposed copy differs");
    for (int64_t r = 0; r < rows && r < 3; ++r)
        for (int64_t c = 0; c < cols && c < 3; ++c) {
            (void)orc_load(x, dtype, r * ld + c);
            (void)orc_amax_rect(x, dtype, ld, r, r + 1, c, cols);
            g_calls += 2;
        }
    free(x);
    free(amax);
    free(scale);
    free(q);
    free(qt);
}

static void one_gemm(int64_t m, int64_t n, int64_t k, int blocks)
{
    const int64_t lda = k + 16, ldb = k + 32, ldy = n + 1;
    const int ga = blocks ? ORC_ROW_1x128 : ORC_TENSOR, gb = blocks ? ORC_BLOCK_128x128 : ORC_TENSOR;
    const size_t na = m > 0 ? (size_t)((m - 1) * lda + k) : 0, nb = n > 0 ? (size_t)((n - 1) * ldb + k) : 0;
    uint8_t* a = alloc_exact(na);
    uint8_t* b = alloc_exact(nb);
    for (size_t i = 0; i < na; ++i) a[i] = (uint8_t)(rnd() & 0xFF);
    for (size_t i = 0; i < nb; ++i) b[i] = (uint8_t)(rnd() & 0xFF);
    const int64_t nsa = orc_scale_count(ga, m, k), nsb = orc_scale_count(gb, n, k);
    float* sa = alloc_exact((size_t)nsa * 4);
    float* sb = alloc_exact((size_t)nsb * 4);
    for (int64_t i = 0; i < nsa; ++i) sa[i] = 0.01f * (float)(1 + i % 5);
    for (int64_t i = 0; i < nsb; ++i) sb[i] = 0.02f * (float)(1 + i % 3);
    const size_t ny = m > 0 ? (size_t)((m - 1) * ldy + n) : 0;
    double* y = alloc_exact(ny * 8);
    for (int fa = 0; fa < 2; ++fa)
        for (int fb = 0; fb < 2; ++fb) {
            if (orc_gemm(a, fa, lda, sa, ga, b, fb, ldb, sb, gb, m, n, k, y, ldy) != 0) fail("orc_gemm rejected");
            ++g_calls;
            int64_t pm[4] = {0, m - 1, m / 2, 0}, pn[4] = {0, n - 1, n / 2, n - 1};
            double pts[4];
            const int64_t np = (m > 0 && n > 0) ? 4 : 0;
            if (orc_gemm_points(a, fa, lda, sa, ga, b, fb, ldb, sb, gb, m, n, k, pm, pn, np, pts) != 0)
                fail("orc_gemm_points rejected");
            ++g_calls;
            for (int64_t i = 0; i < np; ++i) {
                const double ref = y[pm[i] * ldy + pn[i]];
                if (!(pts[i] == ref || (isnan(pts[i]) && isnan(ref)))) fail("points differ from the full GEMM");
            }
            if (m > 0 && n > 0) {
                uint64_t nf = 0;
                for (int64_t r = 0; r < m; ++r) nf += orc_count_nonfinite_bf16(y + r * ldy, n);
                (void)nf;
                g_calls += m;
            }
        }
    /* unsupported pairs are rejected, not run */
    if (orc_gemm(a, 0, lda, sa, ORC_BLOCK_128x128, b, 0, ldb, sb, ORC_ROW_1x128, m, n, k, y, ldy) != -1)
        fail("orc_gemm accepted an unsupported granularity pair");
    ++g_calls;
    free(a);
    free(b);
    free(sa);
    free(sb);
    free(y);
}

int main(void)
{
    /* codec: every code, and the encoder over a sweep of fp32 values */
    for (int fmt = 0; fmt < 2; ++fmt) {
        for (int c = 0; c < 256; ++c) {
            (void)orc_decode(fmt, (uint8_t)c);
            ++g_calls;
        }
        for (int i = 0; i < 200000; ++i) {
            const uint32_t bits = rnd();
            float v;
            memcpy(&v, &bits, 4);
            int ev = -1;
            const uint8_t code = orc_encode(fmt, v, 1, &ev);
            if (ev < ORC_EV_NONE || ev > ORC_EV_NAN) fail("encode event out of range");
            orc_counters ctr = {0, 0, 0, 0};
            (void)orc_cast_one(fmt, v, 0.37f, &ctr);
            (void)code;
            g_calls += 2;
        }
        (void)orc_mant_bits(fmt);
        (void)orc_exp_bits(fmt);
        (void)orc_scale_from_amax(fmt, 0.0f);
        (void)orc_scale_from_amax(fmt, 1e-38f);
        (void)orc_scale_from_amax(fmt, 3e38f);
        g_calls += 5;
    }
    /* bf16 rounding: specials and a sweep */
    const double sp[] = {0.0, -0.0, 1.0, -1.0, 3.3895313892515355e38, 3.4e38, -3.4e38, 1e-45, INFINITY, -INFINITY, NAN};
    for (size_t i = 0; i < sizeof sp / sizeof sp[0]; ++i) {
        (void)orc_bf16_rne(sp[i]);
        ++g_calls;
    }
    for (int i = 0; i < 100000; ++i) {
        (void)orc_bf16_rne(((double)rnd() - 2147483648.0) * 1e-5);
        ++g_calls;
    }

    /* quantize: shapes x dtypes x formats x granularities x modes */
    const int64_t shapes[][3] = {{0, 0, 1},   {0, 64, 64},   {5, 0, 1},     {1, 1, 1},     {1, 5, 9},
                                 {3, 130, 130}, {129, 127, 140}, {128, 128, 128}, {257, 300, 301}, {130, 256, 256}};
    for (size_t s = 0; s < sizeof shapes / sizeof shapes[0]; ++s)
        for (int dtype = 0; dtype < 2; ++dtype)
            for (int fmt = 0; fmt < 2; ++fmt)
                for (int gran = 0; gran < 3; ++gran)
                    for (int mode = 0; mode < 2; ++mode)
                        for (int want_t = 0; want_t < (gran == ORC_ROW_1x128 ? 1 : 2); ++want_t)
                            one_quantize(dtype, shapes[s][0], shapes[s][1], shapes[s][2], fmt, gran, mode, want_t,
                                         (int)(s & 1));

    /* an all-zero matrix: zero codes and scale 1 */
    {
        uint16_t z[4 * 130];
        memset(z, 0, sizeof z);
        uint8_t q[4 * 130];
        float sc[4 * 2];
        if (orc_quantize(z, ORC_BF16, 4, 130, 130, ORC_E4M3, ORC_ROW_1x128, ORC_FROM_AMAX, sc, q, 130, NULL, 0,
                         NULL) != 0)
            fail("zero matrix rejected");
        for (int i = 0; i < 4 * 130; ++i)
            if (q[i] != 0) fail("zero matrix gave a non-zero code");
        for (int i = 0; i < 8; ++i)
            if (sc[i] != 1.0f) fail("zero matrix gave a scale other than 1");
        ++g_calls;
    }
    /* bad arguments are rejected, not run */
    {
        uint16_t x1[4] = {0, 0, 0, 0};
        uint8_t q1[4];
        float s1[1];
        if (orc_quantize(x1, ORC_BF16, 2, 2, 1, ORC_E4M3, ORC_TENSOR, ORC_FROM_AMAX, s1, q1, 2, NULL, 0, NULL) != -1)
            fail("a leading dimension below the row length was accepted");
        if (orc_quantize(x1, ORC_BF16, 2, 2, 2, ORC_E4M3, ORC_ROW_1x128, ORC_FROM_AMAX, s1, q1, 2, q1, 2, NULL) != -1)
            fail("a transposed copy of 1x128 tiles was accepted");
        ++g_calls;
    }

    /* GEMM: ragged m and n, K of one and several 128-wide blocks, both scale modes */
    const int64_t gs[][3] = {{0, 4, 128}, {4, 0, 128}, {1, 1, 128}, {3, 5, 256}, {17, 130, 384}, {130, 129, 128}};
    for (size_t s = 0; s < sizeof gs / sizeof gs[0]; ++s)
        for (int blocks = 0; blocks < 2; ++blocks) one_gemm(gs[s][0], gs[s][1], gs[s][2], blocks);
    one_gemm(5, 7, 100, 0);   /* per-tensor scales take any K */

    printf("OK %ld\n", g_calls);
    return 0;
}
