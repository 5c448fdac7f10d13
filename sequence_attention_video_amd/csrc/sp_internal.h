// Internal helpers shared by the libspattn.so translation units.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "sp.h"
#include "sp_fastdiv.h"

namespace sp {

constexpr int kThreads = 256;   // every kernel here runs 4 waves of 64 lanes

inline int64_t elem_bytes(sp_dtype dt) { return dt == SP_F32 ? 4 : 2; }
inline bool dtype_ok(int dt) { return dt == SP_F32 || dt == SP_BF16; }

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Launch status after a kernel launch.
inline sp_status launch_status() {
  return hipGetLastError() == hipSuccess ? SP_OK : SP_ERR_HIP;
}

// Device form of fdiv_host (same arithmetic).
__device__ __forceinline__ uint32_t fdiv(uint32_t n, const FastDiv& f) {
  uint64_t hi = __umulhi(n, f.magic);
  return uint32_t((hi + n) >> f.shift);
}

}  // namespace sp
