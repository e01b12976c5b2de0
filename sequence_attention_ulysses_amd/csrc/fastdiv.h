// Division by a run-time invariant 32-bit divisor, shared by the host plan
// builder and the gfx950 kernels.  Kept free of HIP headers so the host
// compiler alone can test it.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define ULY_HD __host__ __device__ __forceinline__
#else
#define ULY_HD inline
#endif

namespace uly {

// Unsigned 32-bit division with one multiply-high, an add and a shift
// (Granlund & Montgomery, "Division by Invariant Integers using
// Multiplication", PLDI 1994, the round-up method with an N+1-bit
// multiplier): with s = ceil(log2 d) and m = floor(2^32 * (2^s - d) / d) + 1,
// floor(n / d) = (mulhi(n, m) + n) >> s for every 32-bit n.  The sum is formed
// in 64 bits so it cannot wrap.
struct FastDiv {
    uint32_t d;
    uint32_t m;
    uint32_t s;
    uint32_t pad;

    static FastDiv make(uint32_t divisor) {
        FastDiv f{};
        f.d = divisor ? divisor : 1;
        uint32_t s = 0;
        while ((uint64_t(1) << s) < f.d) ++s;
        f.s = s;
        f.m = uint32_t(((uint64_t(1) << 32) * ((uint64_t(1) << s) - f.d)) / f.d + 1);
        return f;
    }

    ULY_HD uint32_t div(uint32_t n) const {
#if defined(__HIP_DEVICE_COMPILE__)
        const uint32_t hi = __umulhi(n, m);
#else
        const uint32_t hi = uint32_t((uint64_t(n) * m) >> 32);
#endif
        return uint32_t((uint64_t(hi) + n) >> s);
    }

    ULY_HD void divmod(uint32_t n, uint32_t &q, uint32_t &r) const {
        q = div(n);
        r = n - q * d;
    }
};

}  // namespace uly
