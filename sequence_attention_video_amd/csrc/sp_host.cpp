// Host-only entry points: status names, version and the sequence partition.
// Nothing here touches the GPU.

#include <cstdint>

#include "sp.h"

extern "C" const char* sp_status_string(sp_status status) {
  switch (status) {
    case SP_OK: return "SP_OK";
    case SP_ERR_NOT_DIVISIBLE: return "SP_ERR_NOT_DIVISIBLE: token count not divisible by world size";
    case SP_ERR_INVALID_ARG: return "SP_ERR_INVALID_ARG: invalid argument";
    case SP_ERR_UNSUPPORTED: return "SP_ERR_UNSUPPORTED: outside the supported set";
    case SP_ERR_HIP: return "SP_ERR_HIP: HIP runtime error at launch";
  }
  return "SP_ERR_UNKNOWN";
}

extern "C" int32_t sp_version(void) { return 100; }  // 0.1.0

// compute_sequence_partition: page "LTX-2 序列并行拆解：token 切分、all2all 换头与
// runner 接入全链路", section "token 切片、换头、gather 还原", step 切分 -- equal
// shards, and a total that does not divide by the world size is an error.
extern "C" sp_status sp_partition(int64_t total_tokens, int32_t world_size, int64_t* offsets,
                                  int64_t* lengths) {
  if (world_size < 1 || total_tokens < 0) return SP_ERR_INVALID_ARG;
  if (total_tokens % world_size != 0) return SP_ERR_NOT_DIVISIBLE;
  const int64_t ts = total_tokens / world_size;
  for (int32_t r = 0; r < world_size; ++r) {
    if (offsets) offsets[r] = int64_t(r) * ts;
    if (lengths) lengths[r] = ts;
  }
  return SP_OK;
}
