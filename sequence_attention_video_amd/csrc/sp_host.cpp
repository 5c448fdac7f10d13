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
    case SP_ERR_SCRATCH:
      return "SP_ERR_SCRATCH: the call needs more workspace than the no-allocation entry point's fixed "
             "scratch (SP_NOALLOC_SCRATCH_BYTES)";
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

// get_optimal_split: page "LongCat-Video上下文并行技术如何实现高效的多GPU推理",
// section 智能张量拆分策略 -- the split of the height x width grid over the
// ranks whose ratio is closest to a square; an uneven split is not offered.
extern "C" sp_status sp_optimal_split(int32_t n_ranks, int64_t height, int64_t width, int32_t* split_h,
                                      int32_t* split_w) {
  if (n_ranks < 1 || height < 1 || width < 1) return SP_ERR_INVALID_ARG;
  int32_t best_a = 0;
  int64_t best_k0 = 0, best_k1 = 0;
  for (int32_t a = 1; a <= n_ranks; ++a) {
    if (n_ranks % a != 0) continue;
    const int32_t b = n_ranks / a;
    if (height % a != 0 || width % b != 0) continue;
    const int64_t k0 = a > b ? a - b : b - a;                       // ranks closest to square
    const int64_t th = height / a, tw = width / b;
    const int64_t k1 = th > tw ? th - tw : tw - th;                 // then tiles closest to square
    if (best_a == 0 || k0 < best_k0 || (k0 == best_k0 && k1 < best_k1)) {   // ties keep the smaller a
      best_a = a;
      best_k0 = k0;
      best_k1 = k1;
    }
  }
  if (best_a == 0) return SP_ERR_NOT_DIVISIBLE;
  if (split_h) *split_h = best_a;
  if (split_w) *split_w = n_ranks / best_a;
  return SP_OK;
}
