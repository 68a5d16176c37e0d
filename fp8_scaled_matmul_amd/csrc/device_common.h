// Device-side helpers shared by the quantizer kernels: FP8 format traits, the
// scaled quotient, the saturating cast to OCP E4M3 / E5M2 and counter
// reduction.  gfx950 only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp8mi.h"

namespace fp8mi {

// OCP E4M3 (max 448) and E5M2 (max 57344): the maxima printed in "FP8
// stability guardrails", section "Why FP8 is tempting and why it is fragile".
template <int FMT> struct Fmt;
template <> struct Fmt<0> {
    static constexpr float fmax = 448.0f;
    static constexpr int fmax_exp = 8;          // 448 = 1.75 * 2^8
    static constexpr uint32_t maxcode = 0x7E;
    // Round-to-nearest-even with no upper exponent bound sends |v| <= 464 to
    // 448 (464 is the tie between 448 and 480, 448 has the even mantissa) and
    // anything larger past the range: that is a saturation event.
    __device__ static bool saturates(float a) { return a > 464.0f; }
    // Largest |v| that rounds to zero: half the smallest subnormal 2^-9,
    // which ties to the even code 0.
    static constexpr float zero_below_eq = 0x1p-10f;
};
template <> struct Fmt<1> {
    static constexpr float fmax = 57344.0f;
    static constexpr int fmax_exp = 15;         // 57344 = 1.75 * 2^15
    static constexpr uint32_t maxcode = 0x7B;
    // 61440 ties 57344 (odd mantissa) and 65536 (even): rounds up, saturates.
    __device__ static bool saturates(float a) { return a >= 61440.0f; }
    static constexpr float zero_below_eq = 0x1p-17f;
};

// Scales at or above this use the multiply + correction quotient; smaller
// ones take a full IEEE division (see quot_corrected).
constexpr float kCorrectedQuotMinScale = 0x1p-64f;
// A given scale (no amax bounds x) takes the corrected quotient only up to
// this (1/s stays a normal number), and only for |x| <= given_limit(s).
constexpr float kCorrectedQuotMaxScale = 0x1p64f;

// Dequantization scale from an amax: s = fl32(amax / fmax), 1 for amax 0,
// raised to FLT_MIN when smaller (so no result depends on denormal scales).
template <int FMT>
__device__ inline float scale_from_amax(float amax)
{
    if (amax == 0.0f) return 1.0f;
    float s = amax / Fmt<FMT>::fmax;            // correctly rounded fp32 division
    return s < 0x1p-126f ? 0x1p-126f : s;
}

// Power-of-two scale: the smallest 2^e with amax / 2^e <= fmax on the real
// quotient.  With fmax = 1.75 * 2^E and a normal amax = m * 2^ea (m in
// [1, 2)), that is e = ea - E, plus one when m > 1.75 (fraction bits above
// 0x600000).  1 for amax 0; e is raised to -126 (amax below FLT_MIN always
// lands there), so s is a normal number whose exponent field is its E8M0 code.
template <int FMT>
__device__ inline float scale_pow2(float amax)
{
    if (amax == 0.0f) return 1.0f;
    if (amax < 0x1p-126f) return 0x1p-126f;
    const uint32_t b = __builtin_bit_cast(uint32_t, amax);
    int e = (int)(b >> 23) - 127 - Fmt<FMT>::fmax_exp + ((b & 0x7FFFFFu) > 0x600000u ? 1 : 0);
    e = e < -126 ? -126 : e;
    return __builtin_bit_cast(float, (uint32_t)(e + 127) << 23);
}

// The scale rule of a FROM_AMAX quantization: fl32(amax / fmax), or the
// power-of-two rule.
template <int FMT>
__device__ inline float scale_rule(float amax, int pow2)
{
    return pow2 ? scale_pow2<FMT>(amax) : scale_from_amax<FMT>(amax);
}

// v = fl32(x / s) for |x| <= amax of the group and s >= 2^-64, from the
// correctly rounded reciprocal r = fl32(1/s): q0 = x r, residual
// e = x - q0 s (exact by FMA), v = q0 + e r (P. Markstein, "IA-64 and
// Elementary Functions", 2000).  The copysign restores the sign of zero
// quotients.  Checked exhaustively on the CPU over every finite bf16 x and
// every scale a bf16 amax can produce: the FP8 code and counter events equal
// those of the IEEE quotient in every case.
__device__ inline float quot_corrected(float x, float s, float r)
{
    float q0 = x * r;
    float e = __builtin_fmaf(-q0, s, x);
    float v = __builtin_fmaf(e, r, q0);
    return __builtin_copysignf(v, x);
}

// Given scale s: the largest bf16 magnitude pattern L (0 .. 0x7F7F) whose
// IEEE quotient L / s is at most fmax; for s outside [2^-64, 2^64], 0.  Every
// bf16 x with |x| <= L then has a finite quotient within +-fmax, on which
// the corrected quotient gives the IEEE quotient's code and events (checked
// on the CPU over every x and s significand, and against a scan of every
// magnitude for over 6000 scales), and nothing saturates.  Elements above L
// (saturating, Inf, NaN) take IEEE division.  L starts from fl32(fmax s) cut
// to bf16 and moves at most one step: up when the next magnitude's quotient
// still rounds to fmax or below, else down when its own does not (the one
// below is then always within: a bf16 step is 2^-8 of it, fl32(fmax s) is
// within 2^-24 of fmax s).  Every returned L has been checked with a
// division, except after a step down, which is safe by that margin.
template <int FMT>
__device__ inline uint32_t given_limit(float s)
{
    if (!(s >= kCorrectedQuotMinScale && s <= kCorrectedQuotMaxScale)) return 0;
    constexpr float fm = Fmt<FMT>::fmax;
    uint32_t c = __builtin_bit_cast(uint32_t, fm * s) >> 16;
    c = c > 0x7F7Fu ? 0x7F7Fu : c;
    auto within = [&](uint32_t b) { return __builtin_bit_cast(float, b << 16) / s <= fm; };
    if (c < 0x7F7Fu && within(c + 1))
        ++c;
    else if (!within(c))
        --c;
    return c;
}

// Two fp32 values (already clamped to +-fmax) to two FP8 bytes; hi selects
// bytes 2-3 of `old`.  The hardware conversion rounds to nearest even.
template <int FMT, bool HI>
__device__ inline int cvt_pk(float a, float b, int old)
{
    if constexpr (FMT == 0)
        return __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, HI);
    else
        return __builtin_amdgcn_cvt_pk_bf8_f32(a, b, old, HI);
}

template <int FMT>
__device__ inline float clamp_fmax(float v)
{
    return __builtin_amdgcn_fmed3f(v, -Fmt<FMT>::fmax, Fmt<FMT>::fmax);
}

// Unpack bf16 pairs to fp32.
__device__ inline float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

// Four quotients (finite, |v| bounded by about fmax) to four codes, plus the
// count of underflows (non-zero x whose code is +-0).
template <int FMT>
__device__ inline uint32_t encode4_fast(const float v[4], const float x[4], uint32_t& und)
{
    int w = cvt_pk<FMT, false>(clamp_fmax<FMT>(v[0]), clamp_fmax<FMT>(v[1]), 0);
    w = cvt_pk<FMT, true>(clamp_fmax<FMT>(v[2]), clamp_fmax<FMT>(v[3]), w);
#pragma unroll
    for (int i = 0; i < 4; ++i)
        und += (__builtin_fabsf(v[i]) <= Fmt<FMT>::zero_below_eq) & (x[i] != 0.0f);
    return (uint32_t)w;
}

// Underflows among four codes (byte i holds element i) of the bf16 inputs in
// xw0 (elements 0, 1) and xw1 (elements 2, 3): non-zero inputs whose code has
// magnitude 0.  Byte-parallel: adding 0x7F to a 7-bit magnitude sets bit 7
// exactly when the magnitude is non-zero (no carry leaves the byte); adding
// 0x7FFF does the same for each bf16 half, whose high bytes v_perm gathers
// into code byte order.
__device__ inline uint32_t underflows4_bf16(uint32_t code, uint32_t xw0, uint32_t xw1)
{
    const uint32_t cnz = (code & 0x7F7F7F7Fu) + 0x7F7F7F7Fu;
    const uint32_t x0 = (xw0 & 0x7FFF7FFFu) + 0x7FFF7FFFu;
    const uint32_t x1 = (xw1 & 0x7FFF7FFFu) + 0x7FFF7FFFu;
    const uint32_t xnz = __builtin_amdgcn_perm(x1, x0, 0x07050301u);   // bytes 1, 3 of x0, then of x1
    return (uint32_t)__builtin_popcount(xnz & ~cnz & 0x80808080u);
}

// Eight bf16 inputs (four packed words) to eight codes on the fast path
// (every quotient finite, scale >= 2^-64): corrected quotient, clamp, packed
// conversion, and the underflow count taken on the packed words.  A code of
// magnitude 0 is exactly a quotient with |v| <= half the smallest subnormal
// (round to nearest even), so this counts what encode4_fast counts.
// The quotient is taken without quot_corrected's copysign: for x != 0 the
// corrected quotient already has the sign of x (q0 = fl(x r) has it, the
// correction is smaller than one ulp of q0, and a result that rounds to zero
// keeps its sign), so only x = -0 comes out as +0; OR-ing the input sign bits
// into the code bytes restores it and changes no other code.  No clamp: with
// |x| <= amax and s = fl32(amax / fmax) (or a power of two >= amax / fmax),
// |v| <= fmax (1 + 2^-23), below the midpoint between fmax and the next
// binade step (464 for E4M3, 61440 for E5M2), so the conversion's round to
// nearest even already gives +-fmax.
template <int FMT>
__device__ inline uint2 cast8_bf16_fast(const uint32_t ws[4], float s, float r, uint32_t& und)
{
    float v[8];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const float x = e ? bf16_hi(ws[h]) : bf16_lo(ws[h]);
            const float q0 = x * r;
            v[2 * h + e] = __builtin_fmaf(__builtin_fmaf(-q0, s, x), r, q0);
        }
    }
    int w0 = cvt_pk<FMT, false>(v[0], v[1], 0);
    w0 = cvt_pk<FMT, true>(v[2], v[3], w0);
    int w1 = cvt_pk<FMT, false>(v[4], v[5], 0);
    w1 = cvt_pk<FMT, true>(v[6], v[7], w1);
    // input sign bits (bit 15 and 31 of each word) into code byte order
    const uint32_t sg0 = __builtin_amdgcn_perm(ws[1], ws[0], 0x07050301u) & 0x80808080u;
    const uint32_t sg1 = __builtin_amdgcn_perm(ws[3], ws[2], 0x07050301u) & 0x80808080u;
    const uint32_t c0 = (uint32_t)w0 | sg0, c1 = (uint32_t)w1 | sg1;
    und += underflows4_bf16(c0, ws[0], ws[1]) + underflows4_bf16(c1, ws[2], ws[3]);
    return uint2{c0, c1};
}

// General per-element encode for any quotient (NaN, Inf, out of range), with
// all three counters.  NaN quotients get 0x7F with sign(x) xor sign(s).
template <int FMT>
__device__ inline uint32_t encode4_general(const float v[4], const float x[4], float s,
                                           uint32_t& sat, uint32_t& und, uint32_t& nan)
{
    int w = cvt_pk<FMT, false>(clamp_fmax<FMT>(v[0]), clamp_fmax<FMT>(v[1]), 0);
    w = cvt_pk<FMT, true>(clamp_fmax<FMT>(v[2]), clamp_fmax<FMT>(v[3]), w);
    uint32_t out = (uint32_t)w;
    const uint32_t ssign = __builtin_bit_cast(uint32_t, s) >> 31;
    // Branch-free: with a branch per element the compiler merges the three
    // counter updates through a pointer select, which moves the counters
    // into scratch memory (and every update then waits on vector memory).
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float a = __builtin_fabsf(v[i]);
        const uint32_t isnan = v[i] != v[i];
        const uint32_t sg = (__builtin_bit_cast(uint32_t, x[i]) >> 31) ^ ssign;
        const uint32_t nan_code = (out & ~(0xFFu << (8 * i))) | (((sg << 7) | 0x7Fu) << (8 * i));
        out = isnan ? nan_code : out;
        nan += isnan;
        sat += (isnan ^ 1u) & (uint32_t)Fmt<FMT>::saturates(a);
        und += (isnan ^ 1u) & (uint32_t)(a <= Fmt<FMT>::zero_below_eq) & (uint32_t)(x[i] != 0.0f);
    }
    return out;
}

__device__ inline uint32_t wave_sum(uint32_t v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

__device__ inline uint32_t wave_max(uint32_t v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        uint32_t o = __shfl_xor(v, off, 64);
        v = o > v ? o : v;
    }
    return v;
}

// Adds per-thread counts to the device counters: one atomic per wave and
// counter, skipped when the wave's count is zero.
__device__ inline void flush_counters(fp8_counters* ctr, uint32_t sat, uint32_t und, uint32_t nan,
                                      uint32_t nonfinite = 0)
{
    if (!ctr) return;
    sat = wave_sum(sat);
    und = wave_sum(und);
    nan = wave_sum(nan);
    nonfinite = wave_sum(nonfinite);
    if ((threadIdx.x & 63) == 0) {
        if (sat) atomicAdd((unsigned long long*)&ctr->saturated, (unsigned long long)sat);
        if (und) atomicAdd((unsigned long long*)&ctr->underflow, (unsigned long long)und);
        if (nan) atomicAdd((unsigned long long*)&ctr->nan, (unsigned long long)nan);
        if (nonfinite) atomicAdd((unsigned long long*)&ctr->nonfinite_out, (unsigned long long)nonfinite);
    }
}

// The same for a whole workgroup (every thread must call it): the waves'
// sums meet in LDS and one thread adds them, so a workgroup issues at most
// one atomic per counter.  Many waves adding to the same 64-bit counter
// serialize in the L2 (measured: about 5 ns each).
__device__ inline void flush_counters_block(fp8_counters* ctr, uint32_t sat, uint32_t und, uint32_t nan)
{
    __shared__ uint32_t sh[3][16];
    if (!ctr) return;
    sat = wave_sum(sat);
    und = wave_sum(und);
    nan = wave_sum(nan);
    const int w = threadIdx.x >> 6, nw = (blockDim.x + 63) >> 6;
    if ((threadIdx.x & 63) == 0) {
        sh[0][w] = sat;
        sh[1][w] = und;
        sh[2][w] = nan;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t a = 0, b = 0, c = 0;
        for (int i = 0; i < nw; ++i) {
            a += sh[0][i];
            b += sh[1][i];
            c += sh[2][i];
        }
        if (a) atomicAdd((unsigned long long*)&ctr->saturated, (unsigned long long)a);
        if (b) atomicAdd((unsigned long long*)&ctr->underflow, (unsigned long long)b);
        if (c) atomicAdd((unsigned long long*)&ctr->nan, (unsigned long long)c);
    }
}

// |x| as an ordered integer key for finite x, 0 for Inf/NaN (amax ignores
// them); bit 31 flags a non-finite element.
__device__ inline uint32_t absbits_bf16(uint32_t h)
{
    const uint32_t a = h & 0x7FFFu;
    return a < 0x7F80u ? (a << 16) : 0x80000000u;
}
__device__ inline uint32_t absbits_f32(uint32_t w)
{
    const uint32_t a = w & 0x7FFFFFFFu;
    return a < 0x7F800000u ? a : 0x80000000u;
}
// Combine two keys: max of the magnitudes, OR of the non-finite flags.
__device__ inline uint32_t key_merge(uint32_t p, uint32_t q)
{
    const uint32_t m = max(p & 0x7FFFFFFFu, q & 0x7FFFFFFFu);
    return m | ((p | q) & 0x80000000u);
}
__device__ inline float key_amax(uint32_t k) { return __builtin_bit_cast(float, k & 0x7FFFFFFFu); }
__device__ inline bool key_special(uint32_t k) { return (k >> 31) != 0; }

__device__ inline uint32_t wave_key_merge(uint32_t v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = key_merge(v, __shfl_xor(v, off, 64));
    return v;
}


}  // namespace fp8mi
