/*
 * Design check for the HIP cast kernels (not an oracle pin): when the scale
 * comes from a bf16 amax, s = fl32(amax / fmax) (raised to FLT_MIN), the
 * kernels form the quotient with one multiply and two FMAs,
 *     r = fl32(1/s);  q0 = fl32(x*r);  e = fma(-q0, s, x);  v = copysign(fma(e, r, q0), x),
 * (P. Markstein's correction step, "IA-64 and Elementary Functions", 2000)
 * instead of a full IEEE division (s > 0, so the quotient has x's sign; the
 * copysign keeps -0 and negative underflows negative, which the FMA loses).  This program proves that v == fl32(x/s)
 * bit for bit for EVERY finite bf16 x with |x| <= amax and EVERY such s, for
 * both formats (every bf16 amax from the smallest subnormal to the largest
 * finite value).  That is the whole domain the kernels use it on: amax is
 * the largest finite |x| of the group, and +-Inf / NaN inputs take a
 * separate branch.  (For |x| > amax the quotient can overflow and the
 * correction step yields NaN instead of Inf; the kernels never get there.)
 * Scales below 2^-64 are excluded: the kernels take a full IEEE division
 * for such groups (a branch that is uniform over the group).  For s >= 2^-64
 * the only inexact cases are |x| below about 2^-102, whose residual underflows; their
 * quotients are below 2^-38, far under half the smallest E5M2 subnormal
 * (2^-17), so both values encode to the same signed zero.  The property
 * checked is therefore: v == fl32(x/s) bit for bit, or both have magnitude
 * below 2^-20 and the same sign (same FP8 code and same counter events).
 * The same check runs over every power-of-two scale the fast path can see
 * (s = 2^e, -64 <= e <= 121) and every finite bf16 x with |x| <= fmax s,
 * where it must hold bit for bit with no exception (1/s is exact, so x r is
 * already the correctly rounded quotient and the correction leaves it).
 * The bf16 fast path of the kernels drops the copysign and ORs the input's
 * sign bit into the code byte instead; both loops also check that without
 * the copysign the value is bit-identical for every x != 0 and is a zero
 * for x = +-0, so that form yields the same codes.
 *
 * Given scales (any fp32 s in [2^-64, 2^64], no amax to bound x): the
 * kernels take the corrected quotient for the elements whose |x| is at most
 * a limit L(s), the largest bf16 magnitude whose IEEE quotient is <= fmax,
 * and IEEE division for the others.  L(s) starts from fl32(fmax s) cut to
 * bf16 and takes at most one step up or down (given_limit below, the same
 * steps as the kernels).  Third check: for x and s both in [1, 2) (every
 * one of the 2^7 bf16 and 2^23 fp32 significands) v == fl32(x/s) bit for
 * bit.  Each step (1/s, x r, the FMA residual, the corrected sum) commutes
 * with scaling x by 2^a and s by 2^b as long as no intermediate leaves the
 * normal range, so this covers every pair whose r, q0, residual and
 * quotient are normal: with s in [2^-64, 2^64], r is normal; the residual
 * is exact for |x| >= 2^-102 (its lowest bit is 2^-47 of x's binade); the
 * quotient is normal down to 2^-125.  Below those bounds both values are
 * under 2^-20 in magnitude with the sign of x (the same signed zero code).
 * Fourth check, stated directly: s = m 2^e for -64 <= e <= 63 and 24
 * significands m (1, 1 + 2^-23, 2 - 2^-23, 1.5, and 20 seeded ones), both
 * formats, and the scales next to B / fmax for 1024 bf16 magnitudes B
 * (fl32(B / fmax) and its two fp32 neighbours, where fmax s lands within
 * an fp32 step of B and the step up or down is taken):
 * L(s) equals the limit found by scanning every bf16 magnitude,
 * and for every bf16 x with |x| <= L(s), v and fl32(x/s) give the same code
 * (bit-identical, or both below 2^-20 with the same sign), and the
 * no-copysign form agrees as above.
 * Exit 0 and "OK <n>" on success.
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float f_of(uint32_t w) { float f; memcpy(&f, &w, 4); return f; }
static uint32_t w_of(float f) { uint32_t w; memcpy(&w, &f, 4); return w; }

/* L(s) as the kernels compute it (s in [2^-64, 2^64]). */
static int given_ok(uint32_t b, float s, float fm) { volatile float q = f_of(b << 16) / s; return q <= fm; }
static uint32_t given_limit(float s, float fm)
{
    volatile float p = fm * s;
    uint32_t c = w_of(p) >> 16;
    if (c > 0x7F7Fu) c = 0x7F7Fu;
    if (c < 0x7F7Fu && given_ok(c + 1, s, fm)) ++c;
    else if (!given_ok(c, s, fm)) --c;
    return c;
}

int main(void)
{
    const float fmaxv[2] = {448.0f, 57344.0f};
    uint64_t bad = 0, n = 0;
    for (int fmt = 0; fmt < 2; ++fmt) {
        #pragma omp parallel for schedule(dynamic, 64) reduction(+:bad, n)
        for (uint32_t ab = 1; ab < 0x7F80; ++ab) {          /* positive finite bf16 amax */
            volatile float amax = f_of(ab << 16);
            volatile float s = amax / fmaxv[fmt];
            if (s < FLT_MIN) s = FLT_MIN;
            if (s < 0x1p-64f) continue;                          /* full-division branch */
            volatile float r = 1.0f / s;
            for (uint32_t xb = 0; xb < 0x10000; ++xb) {
                if ((xb & 0x7F80) == 0x7F80) continue;         /* Inf / NaN: other branch */
                if ((xb & 0x7FFF) > ab) continue;              /* |x| > amax: not in a group with this amax */
                float x = f_of(xb << 16);
                volatile float q0 = x * r;
                float e = fmaf(-q0, s, x);
                float vn = fmaf(e, r, q0);
                float v = copysignf(vn, x);
                volatile float ref = x / s;
                n++;
                if ((xb & 0x7FFF) ? w_of(vn) != w_of(v) : vn != 0.0f) {
                    if (bad < 5) printf("no-copysign fmt %d amax %a x %a: %a vs %a\n", fmt, amax, x, vn, v);
                    bad++;
                }
                int same = w_of(v) == w_of(ref);
                if (!same && fabsf(v) < 0x1p-20f && fabsf(ref) < 0x1p-20f &&
                    signbit(v) == signbit(ref))
                    same = 1;                                  /* same signed zero code */
                if (!same) {
                    if (bad < 5) printf("fmt %d amax %a x %a: %a vs %a\n", fmt, amax, x, v, ref);
                    bad++;
                }
            }
        }
    }
    /* Power-of-two scales (the FROM_AMAX_POW2 rule): every s = 2^e the fast
     * path can see (2^-64 .. 2^121) and every finite bf16 x with |x| <= fmax s
     * (a group whose power-of-two scale is s has amax <= fmax s). */
    for (int fmt = 0; fmt < 2; ++fmt) {
        #pragma omp parallel for schedule(dynamic, 4) reduction(+:bad, n)
        for (int e = -64; e <= 121; ++e) {
            volatile float s = ldexpf(1.0f, e);
            volatile float r = 1.0f / s;
            const double lim = (double)fmaxv[fmt] * (double)s;
            for (uint32_t xb = 0; xb < 0x10000; ++xb) {
                if ((xb & 0x7F80) == 0x7F80) continue;
                float x = f_of(xb << 16);
                if (fabs((double)x) > lim) continue;
                volatile float q0 = x * r;
                float ee = fmaf(-q0, s, x);
                float vn = fmaf(ee, r, q0);
                float v = copysignf(vn, x);
                volatile float ref = x / s;
                n++;
                if ((xb & 0x7FFF) ? w_of(vn) != w_of(v) : vn != 0.0f) {
                    if (bad < 5) printf("no-copysign pow2 fmt %d s 2^%d x %a: %a vs %a\n", fmt, e, x, vn, v);
                    bad++;
                }
                if (w_of(v) != w_of(ref)) {
                    if (bad < 5) printf("pow2 fmt %d s 2^%d x %a: %a vs %a\n", fmt, e, x, v, ref);
                    bad++;
                }
            }
        }
    }
    /* Given scales, significands: x, s in [1, 2). */
    #pragma omp parallel for schedule(dynamic, 4096) reduction(+:bad, n)
    for (uint32_t ms = 0; ms < (1u << 23); ++ms) {
        volatile float s = f_of(0x3F800000u | ms);
        volatile float r = 1.0f / s;
        for (uint32_t mx = 0; mx < 128; ++mx) {
            float x = f_of(0x3F800000u | (mx << 16));
            volatile float q0 = x * r;
            float v = fmaf(fmaf(-q0, s, x), r, q0);
            volatile float ref = x / s;
            n++;
            if (w_of(v) != w_of(ref)) {
                if (bad < 5) printf("given significands x %a s %a: %a vs %a\n", x, s, v, ref);
                bad++;
            }
        }
    }
    /* Given scales, every finite bf16 x over the whole exponent range. */
    uint32_t sig[24] = {0, 1, 0x7FFFFF, 0x400000};
    uint32_t lcg = 12345u;
    for (int i = 4; i < 24; ++i) {
        lcg = lcg * 1664525u + 1013904223u;
        sig[i] = lcg >> 9;
    }
    for (int fmt = 0; fmt < 2; ++fmt) {
        #pragma omp parallel for schedule(dynamic, 1) reduction(+:bad, n)
        for (int si = 0; si < 128 * 24 + 3 * 1024; ++si) {
                volatile float s;
                if (si < 128 * 24) {
                    s = ldexpf(f_of(0x3F800000u | sig[si % 24]), si / 24 - 64);
                } else {
                    /* bf16 magnitudes B spread over the binades fmax s can reach */
                    const int j = (si - 128 * 24) / 3, k = (si - 128 * 24) % 3;
                    const uint32_t eb = (uint32_t)(127 - 64 + 16 + (j * 7) % 112), mb = (uint32_t)(j * 37) & 0x7F;
                    const float B = f_of((eb << 23) | (mb << 16));
                    float sc = (float)((double)B / (double)fmaxv[fmt]);
                    if (k == 1) sc = nextafterf(sc, 0.0f);
                    if (k == 2) sc = nextafterf(sc, INFINITY);
                    if (!(sc >= 0x1p-64f && sc <= 0x1p64f)) continue;
                    s = sc;
                }
                volatile float r = 1.0f / s;
                const uint32_t lim = given_limit(s, fmaxv[fmt]);
                uint32_t scan = 0;
                while (scan < 0x7F7Fu && given_ok(scan + 1, s, fmaxv[fmt])) ++scan;
                if (lim != scan) {
                    if (bad < 5) printf("given limit fmt %d s %a: %#x vs scan %#x\n", fmt, s, lim, scan);
                    bad++;
                }
                for (uint32_t xb = 0; xb < 0x10000; ++xb) {
                    if ((xb & 0x7FFF) > lim) continue;               /* IEEE division */
                    float x = f_of(xb << 16);
                    volatile float q0 = x * r;
                    float vn = fmaf(fmaf(-q0, s, x), r, q0);
                    float v = copysignf(vn, x);
                    volatile float ref = x / s;
                    n++;
                    if ((xb & 0x7FFF) ? w_of(vn) != w_of(v) : vn != 0.0f) {
                        if (bad < 5) printf("no-copysign given fmt %d s %a x %a: %a vs %a\n", fmt, s, x, vn, v);
                        bad++;
                    }
                    int same = w_of(v) == w_of(ref);
                    if (!same && fabsf(v) < 0x1p-20f && fabsf(ref) < 0x1p-20f && signbit(v) == signbit(ref))
                        same = 1;
                    if (!same) {
                        if (bad < 5) printf("given fmt %d s %a x %a: %a vs %a\n", fmt, s, x, v, ref);
                        bad++;
                    }
                }
        }
    }
    if (bad) { printf("FAIL %llu of %llu\n", (unsigned long long)bad, (unsigned long long)n); return 1; }
    printf("OK %llu\n", (unsigned long long)n);
    return 0;
}
