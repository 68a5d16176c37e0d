/*
 * Pin for the oracle's FP8 encoder: compare orc_encode() with a brute-force
 * nearest-value encoder on EVERY fp32 bit pattern (2^32 inputs per format).
 *
 * The brute-force side shares nothing with the oracle.  It builds the sorted
 * list of the non-negative finite FP8 values by construction from the bit
 * split (E4M3: 4+3 bits, E5M2: 5+2 bits, as in "How to Enable FP8 Training in
 * NanoChat", section "FP8 Training Modes Explained"), checks that its largest
 * entry is the page's maximum (448 / 57344, "FP8 stability guardrails",
 * section "Why FP8 is tempting and why it is fragile"), and then encodes v as
 * the nearest list entry, a tie going to the even code, with one extra grid
 * point past the maximum standing for "overflow" (saturated).
 *
 * Usage: exhaustive_encode <fmt 0|1> [stride]   (stride 1 = all 2^32)
 * Prints "OK <checked>" or the first mismatches, exit status 0/1.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../oracle/fp8_oracle.h"

#define MAXV 160
static double tab[MAXV];   /* tab[c] = value of positive code c; tab[n] = virtual overflow point */
static int ntab;           /* number of finite non-negative codes */

static void build_table(int fmt)
{
    int mb = fmt == 0 ? 3 : 2;
    int eb = fmt == 0 ? 4 : 5;
    int bias = (1 << (eb - 1)) - 1;
    int n = 0;
    /* subnormals (and zero): j * 2^(1 - bias - mb) */
    for (int j = 0; j < (1 << mb); ++j) tab[n++] = ldexp((double)j, 1 - bias - mb);
    /* normals: ((1<<mb) + j) * 2^(E - mb), E = 1-bias ... (top exponent) */
    int etop = fmt == 0 ? (1 << eb) - 1 - bias : (1 << eb) - 2 - bias;
    for (int E = 1 - bias; E <= etop; ++E)
        for (int j = 0; j < (1 << mb); ++j) tab[n++] = ldexp((double)((1 << mb) + j), E - mb);
    if (fmt == 0) n -= 1;          /* E4M3: the top code of the top exponent is NaN */
    ntab = n;
    /* virtual next grid point above the maximum (same exponent step) */
    double step = fmt == 0 ? ldexp(1.0, 8 - 3) : ldexp(1.0, 15 - 2);
    tab[n] = tab[n - 1] + step;
}

/* returns code for |v| (no sign), and *sat / *und flags */
static int brute(double a, int* sat, int* und)
{
    *sat = 0;
    *und = 0;
    if (isinf(a) || a > tab[ntab]) { *sat = 1; return ntab - 1; }
    int lo = 0, hi = ntab;                  /* tab[lo] <= a < tab[hi] invariant */
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (tab[mid] <= a) lo = mid; else hi = mid;
    }
    int pick;
    if (a == tab[lo]) pick = lo;
    else {
        double midp = (tab[lo] + tab[hi]) / 2.0;   /* exact: few significant bits */
        if (a < midp) pick = lo;
        else if (a > midp) pick = hi;
        else pick = (lo % 2 == 0) ? lo : hi;       /* tie: even code */
    }
    if (pick == ntab) { *sat = 1; return ntab - 1; }
    if (pick == 0 && a != 0.0) *und = 1;
    return pick;
}

int main(int argc, char** argv)
{
    int fmt = argc > 1 ? atoi(argv[1]) : 0;
    uint64_t stride = argc > 2 ? strtoull(argv[2], 0, 10) : 1;
    build_table(fmt);
    const double want_max = fmt == 0 ? 448.0 : 57344.0;
    if (tab[ntab - 1] != want_max || ntab != (fmt == 0 ? 127 : 124)) {
        printf("table mismatch: max %g count %d\n", tab[ntab - 1], ntab);
        return 1;
    }
    uint64_t bad = 0, checked = 0;
    #pragma omp parallel for schedule(dynamic, 65536) reduction(+:bad, checked)
    for (uint64_t i = 0; i < (1ull << 32); i += stride) {
        uint32_t w = (uint32_t)i;
        float v;
        memcpy(&v, &w, 4);
        int ev;
        uint8_t got = orc_encode(fmt, v, v != 0.0f, &ev);
        uint8_t want;
        int want_ev;
        if (isnan(v)) {
            want = (uint8_t)((w >> 31 ? 0x80 : 0) | 0x7F);
            want_ev = ORC_EV_NAN;
        } else {
            int sat, und;
            int c = brute(fabs((double)v), &sat, &und);
            want = (uint8_t)((w >> 31 ? 0x80 : 0) | c);
            want_ev = sat ? ORC_EV_SATURATED : (und ? ORC_EV_UNDERFLOW : ORC_EV_NONE);
        }
        checked++;
        if (got != want || ev != want_ev) {
            if (bad < 8) {
                #pragma omp critical
                printf("mismatch fmt=%d bits=0x%08x v=%.9g got=0x%02x/%d want=0x%02x/%d\n",
                       fmt, w, (double)v, got, ev, want, want_ev);
            }
            bad++;
        }
    }
    if (bad) {
        printf("FAIL %llu of %llu\n", (unsigned long long)bad, (unsigned long long)checked);
        return 1;
    }
    printf("OK %llu\n", (unsigned long long)checked);
    return 0;
}
