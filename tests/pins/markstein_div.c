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
 * Exit 0 and "OK <n>" on success.
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float f_of(uint32_t w) { float f; memcpy(&f, &w, 4); return f; }
static uint32_t w_of(float f) { uint32_t w; memcpy(&w, &f, 4); return w; }

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
    if (bad) { printf("FAIL %llu of %llu\n", (unsigned long long)bad, (unsigned long long)n); return 1; }
    printf("OK %llu\n", (unsigned long long)n);
    return 0;
}
