// Packing of mask bytes into visibility bits: bit j of the result is set iff
// byte j of x is not zero, four bytes at a time.  Adding 0x7f to the low 7
// bits of a byte carries into its top bit iff they are not all zero (and
// never out of the byte); OR-ing the byte itself adds its own top bit.  The
// multiply by 0x10204080 then moves the top bits of bytes 0..3 (at bits 0, 8,
// 16, 24 after the shift) to bits 28..31: the other partial products land
// below bit 28 at distinct positions (no carries reach bit 28) or above bit 31.
// Plain C++ (constexpr, so also callable from device code) so that the host
// self-test can build it without HIP.
#pragma once

#include <cstdint>

namespace sp {

constexpr uint32_t nonzero_bytes_to_bits4(uint32_t x) {
  return ((((((x & 0x7f7f7f7fu) + 0x7f7f7f7fu) | x) & 0x80808080u) >> 7) * 0x10204080u) >> 28;
}

constexpr uint32_t nonzero_bytes_to_bits8(uint64_t x) {
  return nonzero_bytes_to_bits4(uint32_t(x)) | (nonzero_bytes_to_bits4(uint32_t(x >> 32)) << 4);
}

}  // namespace sp
