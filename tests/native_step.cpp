// A native consumer of libspattn.so: the whole sequence-parallel path (pad,
// partition, send_recv_heads, masked attention on every rank's local heads,
// gather_heads, gather_output_tokens) through the C ABI alone, with device
// buffers from hipMalloc and a stream of its own; no Python, no torch.
//
// Usage: native_step DIR B T W H D
//   reads DIR/q.bin, DIR/k.bin, DIR/v.bin: (B, T, H, D) float32, and writes
//   DIR/out.bin: (B, T, H, D) float32.  Exit status 0 on success; any failed
//   call prints its status and exits 1.
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <string>
#include <vector>

#include "sp.h"

#define HIP_OK(x)                                                              \
  do {                                                                         \
    hipError_t e_ = (x);                                                       \
    if (e_ != hipSuccess) {                                                    \
      std::fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));      \
      std::exit(1);                                                            \
    }                                                                          \
  } while (0)
#define SP_OK_(x)                                                              \
  do {                                                                         \
    sp_status s_ = (x);                                                        \
    if (s_ != SP_OK) {                                                         \
      std::fprintf(stderr, "%s failed: %s\n", #x, sp_status_string(s_));       \
      std::exit(1);                                                            \
    }                                                                          \
  } while (0)

static std::vector<float> read_all(const std::string& path, size_t n) {
  std::vector<float> v(n);
  FILE* f = std::fopen(path.c_str(), "rb");
  if (!f || std::fread(v.data(), sizeof(float), n, f) != n) {
    std::fprintf(stderr, "cannot read %s\n", path.c_str());
    std::exit(1);
  }
  std::fclose(f);
  return v;
}

int main(int argc, char** argv) {
  if (argc != 7) {
    std::fprintf(stderr, "usage: %s DIR B T W H D\n", argv[0]);
    return 2;
  }
  const std::string dir = argv[1];
  const int64_t B = std::atoll(argv[2]), T = std::atoll(argv[3]);
  const int32_t W = std::atoi(argv[4]), H = std::atoi(argv[5]), D = std::atoi(argv[6]);
  const int64_t T_pad = W * ((T + W - 1) / W), Ts = T_pad / W, Hl = H / W, C = int64_t(H) * D;
  std::vector<int64_t> offsets(W), lengths(W);
  SP_OK_(sp_partition(T_pad, W, offsets.data(), lengths.data()));

  hipStream_t stream;
  HIP_OK(hipStreamCreate(&stream));
  const size_t in_b = size_t(B * T * C) * 4, pad_b = size_t(B * T_pad * C) * 4;
  void *x[3], *xp[3], *xh[3], *oh, *ot, *out;
  const char* names[3] = {"q", "k", "v"};
  for (int i = 0; i < 3; ++i) {
    std::vector<float> h = read_all(dir + "/" + names[i] + ".bin", size_t(B * T * C));
    HIP_OK(hipMalloc(&x[i], in_b));
    HIP_OK(hipMalloc(&xp[i], pad_b));
    HIP_OK(hipMalloc(&xh[i], pad_b));
    HIP_OK(hipMemcpy(x[i], h.data(), in_b, hipMemcpyHostToDevice));
  }
  HIP_OK(hipMalloc(&oh, pad_b));
  HIP_OK(hipMalloc(&ot, pad_b));
  HIP_OK(hipMalloc(&out, in_b));

  // pad each of Q, K, V to T_pad tokens (tail zero bytes)
  for (int i = 0; i < 3; ++i) SP_OK_(sp_pad(x[i], T * C, xp[i], B, T, T_pad, C, SP_F32, nullptr, nullptr, stream));
  // send_recv_heads: rank s's token shard is rows s*Ts.. of the padded tensor
  const sp_shard_strides tok_in = {Ts * C, T_pad * C};
  const sp_shard_strides head = {B * T_pad * Hl * D, T_pad * Hl * D};
  SP_OK_(sp_relayout_heads(xp, xh, 3, W, B, T_pad, H, D, SP_F32, SP_TOKENS_TO_HEADS, tok_in, head, stream));
  // attention over every rank's local heads, key-only padding mask
  const sp_attn_strides hs = {B * T_pad * Hl * D, T_pad * Hl * D, Hl * D, D};
  const size_t ws = sp_masked_attention_workspace_size(W, B, T_pad, T_pad, Hl, D, SP_F32, 0, 0);
  void* workspace = nullptr;
  if (ws) HIP_OK(hipMalloc(&workspace, ws));
  SP_OK_(sp_masked_attention(xh[0], hs, xh[1], hs, xh[2], hs, oh, hs, W, B, T_pad, T_pad, int32_t(Hl), D, SP_F32, T,
                             nullptr, 0, float(1.0 / std::sqrt(double(D))), workspace, ws, stream));
  // gather_heads into the stacked per-rank token layout, then gather/unpad
  const sp_shard_strides tok_out = {B * Ts * C, Ts * C};
  SP_OK_(sp_relayout_heads(&oh, &ot, 1, W, B, T_pad, H, D, SP_F32, SP_HEADS_TO_TOKENS, tok_out, head, stream));
  SP_OK_(sp_gather_unpad(ot, tok_out, out, W, B, Ts, C, lengths.data(), T, SP_F32, stream));
  HIP_OK(hipStreamSynchronize(stream));

  std::vector<float> h(size_t(B * T * C));
  HIP_OK(hipMemcpy(h.data(), out, in_b, hipMemcpyDeviceToHost));
  FILE* f = std::fopen((dir + "/out.bin").c_str(), "wb");
  if (!f || std::fwrite(h.data(), sizeof(float), h.size(), f) != h.size()) return 1;
  std::fclose(f);
  for (int i = 0; i < 3; ++i) {
    HIP_OK(hipFree(x[i]));
    HIP_OK(hipFree(xp[i]));
    HIP_OK(hipFree(xh[i]));
  }
  HIP_OK(hipFree(oh));
  HIP_OK(hipFree(ot));
  HIP_OK(hipFree(out));
  if (workspace) HIP_OK(hipFree(workspace));
  HIP_OK(hipStreamDestroy(stream));
  std::printf("native step ok\n");
  return 0;
}
