// Division of 32-bit unsigned integers below 2^31 by a runtime-invariant
// divisor with one multiply-high, one add and one shift (T. Granlund and P.
// Montgomery, "Division by invariant integers using multiplication", PLDI
// 1994, the round-up variant with an (N+1)-bit multiplier).
#pragma once

#include <stdint.h>

#ifdef __HIPCC__
#define FP8MI_HD __host__ __device__
#else
#define FP8MI_HD
#endif

namespace fp8mi {

struct FastDiv {
    uint32_t d = 1, mul = 0, shift = 0;

    FastDiv() = default;
    explicit FastDiv(uint32_t divisor) : d(divisor)
    {
        uint32_t l = 0;
        while ((1ull << l) < divisor) ++l;        // l = ceil(log2 d)
        shift = l;
        // mul = floor(2^32 (2^l - d) / d) + 1
        mul = (uint32_t)(((1ull << 32) * ((1ull << l) - divisor)) / divisor + 1);
    }

    // Valid for n < 2^31 (so that mulhi(n) + n cannot wrap).
    FP8MI_HD uint32_t div(uint32_t n) const
    {
#ifdef __HIP_DEVICE_COMPILE__
        const uint32_t t = __umulhi(n, mul);
#else
        const uint32_t t = (uint32_t)(((uint64_t)n * mul) >> 32);
#endif
        return (t + n) >> shift;
    }
};

}  // namespace fp8mi
