// Unsigned division by a divisor fixed for a launch (the GQA group, the
// split plan's chunk length): a multiply-high by m = floor((2^32 - 1) / d)
// and at most two corrections, exact for every 32-bit dividend (m * x / 2^32
// lies in (x / d - 2, x / d]).  The split plan divides per lane before its
// first K/V load; the compiler's general sequence there (a reciprocal, a
// multiply-high and two corrections, with the reciprocal rebuilt for every
// division) sits on that path.  Host-compilable, so the host checks can
// compare it with the division operator.
#pragma once

#include <cstdint>

#if defined(__HIPCC__)
#define DIFFKV_HOST_DEVICE __host__ __device__
#else
#define DIFFKV_HOST_DEVICE
#endif

namespace diffkv {

struct FastDiv {
  uint32_t d, m;
  DIFFKV_HOST_DEVICE explicit FastDiv(uint32_t divisor) : d(divisor), m(0xffffffffu / divisor) {}
  DIFFKV_HOST_DEVICE uint32_t div(uint32_t x) const {
    uint32_t q = (uint32_t)(((uint64_t)x * m) >> 32);
    uint32_t r = x - q * d;
    if (r >= d) {
      ++q;
      r -= d;
    }
    if (r >= d) ++q;
    return q;
  }
  DIFFKV_HOST_DEVICE int value() const { return (int)d; }
};

}  // namespace diffkv
