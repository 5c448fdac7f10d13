// Unsigned 32-bit division by a runtime-constant divisor via a multiply-high:
// the round-up method of Granlund and Montgomery ("Division by invariant
// integers using multiplication", PLDI 1994).  q = (mulhi(n, magic) + n) >> shift
// with the sum taken in 64 bits is exact for every 32-bit n and d >= 1.
// Plain C++ so that the host self-test can build it without HIP.
#pragma once

#include <cstdint>

namespace sp {

struct FastDiv {
  uint32_t d;
  uint32_t magic;
  uint32_t shift;
};

inline FastDiv make_fastdiv(uint32_t d) {
  FastDiv f;
  f.d = d;
  uint32_t s = 0;
  while (s < 32 && (uint64_t(1) << s) < d) ++s;
  f.shift = s;
  f.magic = uint32_t(((uint64_t(1) << 32) * ((uint64_t(1) << s) - d)) / d + 1);
  return f;
}

inline uint32_t fdiv_host(uint32_t n, const FastDiv& f) {
  uint64_t hi = (uint64_t(n) * f.magic) >> 32;
  return uint32_t((hi + n) >> f.shift);
}

}  // namespace sp
