// Data-movement kernels of the sequence-parallel path: pad (with the user-mask
// extension), the token<->head relayout of the virtual ranks, and
// gather/unpad.  All three are HBM-bound byte moves: every thread moves 16-byte
// vectors, a wave covers 1 KiB of contiguous destination per instruction, and
// no value is ever converted, so results are bit-exact by construction.  Loads
// and stores are non-temporal (each byte is touched once, so keeping it in the
// caches only evicts useful lines): measured +15 % on the Q/K/V relayout.
//
// Sources: page "LTX-2 序列并行拆解：token 切分、all2all 换头与 runner 接入全链路",
// section "token 切片、换头、gather 还原", steps 补齐 (pad), 换头 (head swap) and
// 还原 (restore).

#include "sp_internal.h"

namespace sp {
namespace {

constexpr int kUnroll = 4;                        // 16-byte vectors per thread
constexpr int64_t kChunk = int64_t(kThreads) * kUnroll;
constexpr int kMaxWorld = 128;                     // ranks per gather_unpad launch
constexpr int kMaxGridY = 65535;

typedef unsigned int vec16 __attribute__((ext_vector_type(4)));   // one 16-byte vector

__device__ __forceinline__ vec16 load16(const char* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const vec16*>(p));
}
__device__ __forceinline__ void store16(char* p, vec16 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<vec16*>(p));
}

// One thread's kUnroll vectors f0 + u*kThreads (u < kUnroll) of a range of n.
// at(f, so, dof) sets vector f's source and destination byte offsets and
// returns whether it is read (false: written as a zero vector).  With `full`
// (uniform over the workgroup) the caller has checked that all of the
// workgroup's vectors are below n and read: the loads then carry no
// per-vector test and issue back to back, where guarded ones each wait for
// the load before them (measured +4 to +7 % on 100 MB to 1 GB moves).
template <typename Idx, typename At>
__device__ __forceinline__ void move_vectors(const char* src, char* dst, Idx f0, Idx n, bool full, At at) {
  vec16 buf[kUnroll];
  int64_t so[kUnroll], dof[kUnroll];
  if (full) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      at(f0 + Idx(u) * kThreads, so[u], dof[u]);
      buf[u] = load16(src + so[u]);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) store16(dst + dof[u], buf[u]);
    return;
  }
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const Idx f = f0 + Idx(u) * kThreads;
    buf[u] = vec16{0, 0, 0, 0};
    if (f < n && at(f, so[u], dof[u])) buf[u] = load16(src + so[u]);
  }
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    if (f0 + Idx(u) * kThreads < n) store16(dst + dof[u], buf[u]);
  }
}

// ------------------------------------------------------------------ relayout

struct RelayoutArgs {
  const char* src[3];
  char* dst[3];
  int64_t B;
  int64_t tok_rank_b, tok_batch_b, tok_row_b;   // token side (bytes)
  int64_t head_rank_b, head_batch_b;            // head side (bytes)
  int64_t run_b;                                 // Hl*D*eb: one head group of one token
  int64_t seg_b;                                 // Ts*run_b: one source rank's rows on the head side
  uint32_t V;                                    // 16-byte vectors per run
  FastDiv fdV;
  uint32_t n_per_seg;                            // Ts*V vectors per (tensor, r, b, s)
  uint32_t chunks;                               // workgroups per segment
  int to_heads;                                  // 1: token side -> head side
  int64_t Ts;                                    // tokens per rank shard
  int64_t valid;                                 // to heads: token rows s*Ts + t >= valid are zero
};

// One workgroup per (tensor, head-group rank r, batch b, source-token rank s,
// chunk).  On the head side the segment (r, b, s) is one contiguous block of
// Ts runs; on the token side each run sits inside a token row at offset
// r*run_b.  Flat vector f of the segment is token t = f/V, vector f%V of the
// run.  Toward the head side, token rows at or past `valid` (the pad rows of
// 补齐) are written as zero bytes and never read, so an unpadded token tensor
// is padded and exchanged in the same move.
//
// Dispatch order (the workgroup index blockIdx.y * gridDim.x + blockIdx.x,
// then the tensor; the grid is W * chunks by W * B by tensors): toward the
// head side r is fastest, then chunk, s and b, so the W workgroups
// that read the W runs of the same token rows run together and every token
// row is read whole within a short window (with r slowest each row was read a
// run at a time, W times over the launch: 5.70 -> 6.25 TB/s on long_hires's
// 3.2 GB, unchanged on video_self's 302 MB).  Toward the token side chunk is
// fastest, then s, r and b.
__global__ __launch_bounds__(kThreads) void relayout_kernel(RelayoutArgs a) {
  const uint32_t W = gridDim.x / a.chunks;
  uint32_t s, chunk;
  int64_t r, b;
  if (a.to_heads) {
    const uint64_t L = uint64_t(blockIdx.y) * gridDim.x + blockIdx.x;
    r = int64_t(L % W);
    const uint64_t rest = L / W;
    chunk = uint32_t(rest % a.chunks);
    const uint64_t sb = rest / a.chunks;
    s = uint32_t(sb % W);
    b = int64_t(sb / W);
  } else {
    s = blockIdx.x / a.chunks;
    chunk = blockIdx.x - s * a.chunks;
    r = blockIdx.y / a.B;
    b = blockIdx.y - r * a.B;
  }
  const int n = blockIdx.z;
  const char* src = a.src[n];
  char* dst = a.dst[n];
  const int64_t tok_off = s * a.tok_rank_b + b * a.tok_batch_b + r * a.run_b;
  const int64_t head_off = r * a.head_rank_b + b * a.head_batch_b + int64_t(s) * a.seg_b;
  const uint32_t end = (chunk + 1) * uint32_t(kChunk);
  const bool full = end <= a.n_per_seg && (!a.to_heads || int64_t(s) * a.Ts + fdiv(end - 1, a.fdV) < a.valid);
  move_vectors(src, dst, chunk * uint32_t(kChunk) + threadIdx.x, a.n_per_seg, full,
               [&](uint32_t f, int64_t& so, int64_t& dof) {
                 const uint32_t t = fdiv(f, a.fdV);
                 const uint32_t v = f - t * a.V;
                 const int64_t tok = tok_off + int64_t(t) * a.tok_row_b + int64_t(v) * 16;
                 const int64_t head = head_off + int64_t(f) * 16;
                 so = a.to_heads ? tok : head;
                 dof = a.to_heads ? head : tok;
                 return !a.to_heads || int64_t(s) * a.Ts + t < a.valid;
               });
}

// gather_heads walks the token side instead: every workgroup writes whole
// token rows (the rows of one rank's shard are contiguous), and each 1 KiB
// wave store is fed by one run of one head-side rank.  Walking the head side
// here (contiguous reads, stores scattered in runs at the token-row stride)
// measured 5.0 TB/s on 100 MB against 6.0 for the send direction, whose
// scattered side is the reads.
struct GatherHeadsArgs {
  const char* src[3];
  char* dst[3];
  int64_t tok_rank_b, tok_batch_b;    // token side (bytes); rows of W runs packed
  int64_t head_rank_b, head_batch_b;  // head side (bytes)
  int64_t run_b;                      // Hl*D*eb
  int64_t seg_b;                      // Ts*run_b
  uint32_t V;                         // 16-byte vectors per run
  FastDiv fdV, fdRow;                 // by V and by W*V (vectors per token row)
  uint32_t n_per_shard;               // Ts*W*V vectors per (tensor, s, b)
  uint32_t chunks;                    // workgroups per shard
};

// blockIdx.x = (token-side rank s, chunk), blockIdx.y = batch b, blockIdx.z =
// tensor.  Flat vector f of shard (s, b) is token t = f / (W*V), head-group
// rank r = (f % (W*V)) / V, vector v = f % V of the run; it comes from rank
// r's head side at token s*Ts + t.
__global__ __launch_bounds__(kThreads) void gather_heads_kernel(GatherHeadsArgs a) {
  const uint32_t s = blockIdx.x / a.chunks;
  const uint32_t chunk = blockIdx.x - s * a.chunks;
  const int64_t b = blockIdx.y;
  const int n = blockIdx.z;
  const char* src = a.src[n] + b * a.head_batch_b + int64_t(s) * a.seg_b;
  char* dst = a.dst[n] + int64_t(s) * a.tok_rank_b + b * a.tok_batch_b;
  const bool full = (chunk + 1) * uint32_t(kChunk) <= a.n_per_shard;
  move_vectors(src, dst, chunk * uint32_t(kChunk) + threadIdx.x, a.n_per_shard, full,
               [&](uint32_t f, int64_t& so, int64_t& dof) {
                 const uint32_t t = fdiv(f, a.fdRow);
                 const uint32_t rem = f - t * a.fdRow.d;
                 const uint32_t r = fdiv(rem, a.fdV);
                 const uint32_t v = rem - r * a.V;
                 so = int64_t(r) * a.head_rank_b + int64_t(t) * a.run_b + int64_t(v) * 16;
                 dof = int64_t(f) * 16;
                 return true;
               });
}

// gather_heads followed by gather_output_tokens as one move: rank s's token
// rows after the swap back, trimmed to its first counts[s] rows, land at row
// cum[s] of the output (B, T, H, D), and rows from T on are dropped.  Walked
// from the output side like gather_heads_kernel (whole output rows per
// workgroup, 1 KiB wave stores each fed by one run of one head-side rank).
constexpr int kMaxWorldFused = 128;
struct GatherHeadsUnpadArgs {
  const char* src[3];
  char* dst[3];
  int64_t head_rank_b, head_batch_b;  // head side (bytes)
  int64_t run_b;                      // Hl*D*eb
  int64_t seg_b;                      // Ts*run_b
  int64_t out_batch_b, row_b;         // output: T*H*D*eb per batch, H*D*eb per row
  uint32_t V;
  FastDiv fdV, fdRow;                 // by V and by W*V
  uint32_t chunks;                    // workgroups per rank (for the longest kept piece)
  int32_t n_tensors;
  int64_t cum[kMaxWorldFused + 1];    // output row of each rank's first kept row
  uint32_t n_vec[kMaxWorldFused];     // kept rows * W*V of each rank (after the unpad)
};

// blockIdx.x = chunk, blockIdx.y = rank s, blockIdx.z = batch b; the
// workgroup moves the same vectors of each tensor in turn.  The rank and
// batch come straight from the grid, so the per-rank table loads do not wait
// on a division (each workgroup moves 16 KiB per tensor, so the latency of
// its first loads weighs).
template <int U>
__global__ __launch_bounds__(kThreads) void gather_heads_unpad_kernel(GatherHeadsUnpadArgs a) {
  constexpr uint32_t kVec = uint32_t(kThreads) * U;   // vectors per workgroup and tensor
  const uint32_t chunk = blockIdx.x;
  const uint32_t s = blockIdx.y;
  const int64_t b = blockIdx.z;
  const uint32_t nv = a.n_vec[s];
  const uint32_t f0 = chunk * kVec + threadIdx.x;
  if (chunk * kVec >= nv) return;
  const int64_t src_off = b * a.head_batch_b + int64_t(s) * a.seg_b;
  const int64_t dst_off = b * a.out_batch_b + a.cum[s] * a.row_b;
  int64_t raddr[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint32_t f = f0 + u * kThreads;
    const uint32_t t = fdiv(f, a.fdRow);
    const uint32_t rem = f - t * a.fdRow.d;
    const uint32_t r = fdiv(rem, a.fdV);
    const uint32_t v = rem - r * a.V;
    raddr[u] = src_off + int64_t(r) * a.head_rank_b + int64_t(t) * a.run_b + int64_t(v) * 16;
  }
  // A workgroup whose vectors are all in range (all but the last of each
  // rank) moves them with no per-vector test, so its loads issue back to
  // back; guarded, each load would wait for the one before it.
  const bool full = (chunk + 1) * kVec <= nv;
  for (int n = 0; n < a.n_tensors; ++n) {
    const char* src = a.src[n];
    char* dst = a.dst[n] + dst_off;
    vec16 buf[U];
    if (full) {
#pragma unroll
      for (int u = 0; u < U; ++u) buf[u] = load16(src + raddr[u]);
#pragma unroll
      for (int u = 0; u < U; ++u) store16(dst + int64_t(f0 + u * kThreads) * 16, buf[u]);
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t f = f0 + u * kThreads;
        if (f < nv) buf[u] = load16(src + raddr[u]);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t f = f0 + u * kThreads;
        if (f < nv) store16(dst + int64_t(f) * 16, buf[u]);
      }
    }
  }
}

// ------------------------------------------------------------------ 2-D tiles

struct Tile2dArgs {
  const char* src;
  char* dst;
  int64_t B;
  int64_t grid_batch_b, row_b;        // grid side (bytes)
  int64_t tile_rank_b, tile_batch_b;  // tile side (bytes)
  int64_t height, width, th, tw;
  int32_t split_w;
  uint32_t runV;                      // 16-byte vectors of one tile row run (tw tokens)
  FastDiv fd_runV, fd_th;
  uint32_t n_per_rb;                  // F*th*runV vectors per (rank, batch)
  uint32_t chunks;                    // workgroups per (rank, batch)
  int to_tiles;                       // 1: grid -> tiles
};

// blockIdx.x = chunk, blockIdx.y = (rank r, batch b).  On the tile side the
// block (r, b) is contiguous; on the grid side it is F*th runs of tw whole
// token rows (one frame row of the tile), each contiguous.  Flat vector f of
// the block is run f / runV (frame f_ = run / th, tile row y = run % th),
// vector f % runV of the run.
__global__ __launch_bounds__(kThreads) void tile_2d_kernel(Tile2dArgs a) {
  const int64_t r = blockIdx.y / a.B;
  const int64_t b = blockIdx.y - r * a.B;
  const int64_t i = r / a.split_w, j = r - (r / a.split_w) * a.split_w;
  const int64_t tile_off = r * a.tile_rank_b + b * a.tile_batch_b;
  const int64_t grid_off = b * a.grid_batch_b + (i * a.th * a.width + j * a.tw) * a.row_b;
  const bool full = (blockIdx.x + 1) * uint32_t(kChunk) <= a.n_per_rb;
  move_vectors(a.src, a.dst, blockIdx.x * uint32_t(kChunk) + threadIdx.x, a.n_per_rb, full,
               [&](uint32_t f, int64_t& so, int64_t& dof) {
                 const uint32_t run = fdiv(f, a.fd_runV);
                 const uint32_t v = f - run * a.runV;
                 const uint32_t fr = fdiv(run, a.fd_th);
                 const uint32_t y = run - fr * uint32_t(a.th);
                 const int64_t g = grid_off + ((int64_t(fr) * a.height + y) * a.width) * a.row_b + int64_t(v) * 16;
                 const int64_t t = tile_off + int64_t(f) * 16;
                 so = a.to_tiles ? g : t;
                 dof = a.to_tiles ? t : g;
                 return true;
               });
}

// ------------------------------------------------------------------ 2-D split + head exchange

// The 2-D split (split_cp_2d) followed by the head exchange (send_recv_heads)
// is one permutation of token rows and head groups, and so is its inverse:
// rank r's head side holds, at row s*Tt + t, head group r of grid token
// g(s, t) = (fr*height + i*th + y)*width + j*tw + x, where rank s = i*split_w
// + j and its tile token t = (fr*th + y)*tw + x.  Moving the bytes once per
// direction skips the tile-side copy.  Both kernels walk their destination
// contiguously (1 KiB wave stores; sources in whole runs).
struct Tile2dHeadsArgs {
  const char* src[3];
  char* dst[3];
  int64_t B;
  int64_t grid_batch_b, grid_row_b;   // grid side (bytes); rows of W runs packed
  int64_t head_rank_b, head_batch_b;  // head side (bytes)
  int64_t run_b;                      // Hl*D*eb
  int64_t height, width, th, tw, Tt;  // grid and tile sizes (tokens)
  int32_t split_w;
  uint32_t V;                         // 16-byte vectors per run
  FastDiv fdV, fd_tw, fd_th;          // to heads: t -> (fr, y, x)
  FastDiv fd_row, fd_width, fd_height;  // to grid: f -> grid token -> (fr, y_, x_)
  uint32_t n_per;                     // vectors per workgroup-row of the grid: Tt*V or T*W*V
  uint32_t chunks;
};

// One workgroup per (tensor, head-group rank r, batch b, source rank s,
// chunk), in the dispatch order of relayout_kernel toward the head side (r
// fastest, so that the W runs of a grid token row are read together; the
// grid is W * chunks by W * B by tensors).  Flat vector f of the head-side
// segment (r, b, s) is tile token t = f / V, vector f % V of its run.
__global__ __launch_bounds__(kThreads) void tile_2d_to_heads_kernel(Tile2dHeadsArgs a) {
  const uint32_t W = gridDim.x / a.chunks;
  const uint64_t L = uint64_t(blockIdx.y) * gridDim.x + blockIdx.x;
  const int64_t r = int64_t(L % W);
  const uint64_t rest = L / W;
  const uint32_t chunk = uint32_t(rest % a.chunks);
  const uint64_t sb = rest / a.chunks;
  const uint32_t s = uint32_t(sb % W);
  const int64_t b = int64_t(sb / W);
  const int n = blockIdx.z;
  const int64_t i = s / uint32_t(a.split_w), j = s - (s / uint32_t(a.split_w)) * uint32_t(a.split_w);
  const char* src = a.src[n] + b * a.grid_batch_b + r * a.run_b;
  char* dst = a.dst[n] + r * a.head_rank_b + b * a.head_batch_b + int64_t(s) * a.Tt * a.run_b;
  const int64_t row0 = i * a.th * a.width + j * a.tw;   // grid token of the tile's first token
  const bool full = (chunk + 1) * uint32_t(kChunk) <= a.n_per;
  move_vectors(src, dst, chunk * uint32_t(kChunk) + threadIdx.x, a.n_per, full,
               [&](uint32_t f, int64_t& so, int64_t& dof) {
                 const uint32_t t = fdiv(f, a.fdV);
                 const uint32_t v = f - t * a.V;
                 const uint32_t q = fdiv(t, a.fd_tw);
                 const uint32_t x = t - q * uint32_t(a.tw);
                 const uint32_t fr = fdiv(q, a.fd_th);
                 const uint32_t y = q - fr * uint32_t(a.th);
                 const int64_t g = row0 + (int64_t(fr) * a.height + y) * a.width + x;
                 so = g * a.grid_row_b + int64_t(v) * 16;
                 dof = int64_t(f) * 16;
                 return true;
               });
}

// blockIdx.x = chunk, blockIdx.y = batch b, blockIdx.z = tensor.  Flat
// vector f of batch b's grid is grid token g = f / (W*V), head-group rank
// r = (f % (W*V)) / V, vector f % V of the run; it comes from rank r's head
// side at the row of g's tile token.
__global__ __launch_bounds__(kThreads) void tile_2d_from_heads_kernel(Tile2dHeadsArgs a) {
  const int64_t b = blockIdx.y;
  const int n = blockIdx.z;
  const char* src = a.src[n] + b * a.head_batch_b;
  char* dst = a.dst[n] + b * a.grid_batch_b;
  const bool full = (blockIdx.x + 1) * uint32_t(kChunk) <= a.n_per;
  move_vectors(src, dst, blockIdx.x * uint32_t(kChunk) + threadIdx.x, a.n_per, full,
               [&](uint32_t f, int64_t& so, int64_t& dof) {
                 const uint32_t g = fdiv(f, a.fd_row);
                 const uint32_t rem = f - g * a.fd_row.d;
                 const uint32_t r = fdiv(rem, a.fdV);
                 const uint32_t v = rem - r * a.V;
                 const uint32_t q = fdiv(g, a.fd_width);
                 const uint32_t x_ = g - q * uint32_t(a.width);
                 const uint32_t fr = fdiv(q, a.fd_height);
                 const uint32_t y_ = q - fr * uint32_t(a.height);
                 const uint32_t i = fdiv(y_, a.fd_th), j = fdiv(x_, a.fd_tw);
                 const uint32_t y = y_ - i * uint32_t(a.th), x = x_ - j * uint32_t(a.tw);
                 const int64_t s = int64_t(i) * a.split_w + j;
                 const int64_t t = (int64_t(fr) * a.th + y) * a.tw + x;
                 so = int64_t(r) * a.head_rank_b + (s * a.Tt + t) * a.run_b + int64_t(v) * 16;
                 dof = int64_t(f) * 16;
                 return true;
               });
}

// ------------------------------------------------------------------ pad

struct PadArgs {
  const char* x;
  char* y;
  int64_t x_batch_b, y_batch_b;
  int64_t copy_vecs;     // T*C*eb/16: vectors copied from x per batch
  int64_t start_vec;     // first vector written (copy_vecs when padding in place)
  int64_t end_vec;       // T_pad*C*eb/16
};

// blockIdx.y = batch.  Vectors below copy_vecs come from x, the rest are zero.
__global__ __launch_bounds__(kThreads) void pad_tokens_kernel(PadArgs a) {
  const int64_t b = blockIdx.y;
  const char* x = a.x + b * a.x_batch_b;
  char* y = a.y + b * a.y_batch_b;
  const int64_t first = a.start_vec + int64_t(blockIdx.x) * kChunk;
  const bool full = first + kChunk <= a.copy_vecs;
  move_vectors(x, y, first + threadIdx.x, a.end_vec, full, [&](int64_t f, int64_t& so, int64_t& dof) {
    so = f * 16;
    dof = f * 16;
    return f < a.copy_vecs;
  });
}

struct MaskPadArgs {
  const uint8_t* in;   // (B, T, T)
  uint8_t* out;        // (B, Tp, Tp)
  int64_t T, Tp;
  int64_t total;       // B*Tp*Tp
  int64_t in_bytes;    // B*T*T
};

typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u32x4_a16 __attribute__((ext_vector_type(4)));

// Each thread writes 16 consecutive output bytes (flat order).  Output byte
// (b, i, j): i < T and j < T -> in[b, i, j]; i >= T and j < T -> 1 (a pad query
// row sees every real key); j >= T -> 0 (pad keys are hidden from every row).
// Inside the copied block (the common case) the 16 source bytes are
// contiguous at any byte alignment: they come from five aligned dwords (one
// 4-aligned dwordx4 load and one dword load) and a byte shift; chunks that
// cross a row end, the pad rows and the buffer's last bytes go byte by byte.
__global__ __launch_bounds__(kThreads) void pad_mask_kernel(MaskPadArgs a) {
  const int64_t p0 = (int64_t(blockIdx.x) * kThreads + threadIdx.x) * 16;
  if (p0 >= a.total) return;
  const int64_t plane = a.Tp * a.Tp;
  int64_t b = p0 / plane;
  int64_t rem = p0 - b * plane;
  int64_t i = rem / a.Tp;
  int64_t j = rem - i * a.Tp;
  if (i < a.T && j + 16 <= a.T && p0 + 16 <= a.total) {
    const uintptr_t addr = reinterpret_cast<uintptr_t>(a.in) + uintptr_t((b * a.T + i) * a.T + j);
    const uintptr_t base = addr & ~uintptr_t(3);
    // dwords past the last one holding a mask byte are never read
    const uintptr_t lim = (reinterpret_cast<uintptr_t>(a.in) + uintptr_t(a.in_bytes) + 3) & ~uintptr_t(3);
    if (base + 20 <= lim) {
      const u32x4_a4 lo = *reinterpret_cast<const u32x4_a4*>(base);
      const uint32_t hi = *reinterpret_cast<const uint32_t*>(base + 16);
      const uint32_t sh = uint32_t(addr & 3);
      u32x4_a16 w;
      w.x = __builtin_amdgcn_alignbyte(lo.y, lo.x, sh);
      w.y = __builtin_amdgcn_alignbyte(lo.z, lo.y, sh);
      w.z = __builtin_amdgcn_alignbyte(lo.w, lo.z, sh);
      w.w = __builtin_amdgcn_alignbyte(hi, lo.w, sh);
      *reinterpret_cast<u32x4_a16*>(a.out + p0) = w;
      return;
    }
  }
  uint8_t v[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    uint8_t val = 0;
    if (p0 + e < a.total && j < a.T) {
      val = i < a.T ? a.in[(b * a.T + i) * a.T + j] : uint8_t(1);
    }
    v[e] = val;
    if (++j == a.Tp) {
      j = 0;
      if (++i == a.Tp) { i = 0; ++b; }
    }
  }
  if (p0 + 16 <= a.total) {
    uint4 w;
    w.x = v[0] | (v[1] << 8) | (v[2] << 16) | (uint32_t(v[3]) << 24);
    w.y = v[4] | (v[5] << 8) | (v[6] << 16) | (uint32_t(v[7]) << 24);
    w.z = v[8] | (v[9] << 8) | (v[10] << 16) | (uint32_t(v[11]) << 24);
    w.w = v[12] | (v[13] << 8) | (v[14] << 16) | (uint32_t(v[15]) << 24);
    *reinterpret_cast<uint4*>(a.out + p0) = w;
  } else {
    for (int e = 0; p0 + e < a.total; ++e) a.out[p0 + e] = v[e];
  }
}

// ------------------------------------------------------------------ gather/unpad

struct GatherArgs {
  const char* in;
  char* out;
  int64_t rank_b, batch_b;   // input strides (bytes)
  int64_t row_b;             // C*eb
  int64_t T;
  int32_t W;
  int64_t cum[kMaxWorld + 1];  // prefix sums of the kept counts
};

// blockIdx.y = (batch b, rank r).  Rank r's kept rows are one contiguous block
// of its shard and land as one contiguous block of the output at row cum[r].
__global__ __launch_bounds__(kThreads) void gather_unpad_kernel(GatherArgs a) {
  const int64_t b = blockIdx.y / a.W;
  const int r = int(blockIdx.y - b * a.W);
  const int64_t first = a.cum[r];
  int64_t kept = a.cum[r + 1] - first;
  if (first + kept > a.T) kept = a.T - first;
  if (kept <= 0) return;
  const int64_t nvec = kept * a.row_b / 16;
  const char* src = a.in + r * a.rank_b + b * a.batch_b;
  char* dst = a.out + (b * a.T + first) * a.row_b;
  const int64_t f_first = int64_t(blockIdx.x) * kChunk;
  move_vectors(src, dst, f_first + threadIdx.x, nvec, f_first + kChunk <= nvec,
               [&](int64_t f, int64_t& so, int64_t& dof) {
                 so = f * 16;
                 dof = f * 16;
                 return true;
               });
}

int64_t div_up(int64_t a, int64_t b) { return (a + b - 1) / b; }

// The W*B blocks of `len` elements at r*rs + b*bs (r < W, b < B) are pairwise
// disjoint if the layout is rank-major (bs >= len, rs >= (B-1)*bs + len) or
// batch-major (rs >= len, bs >= (W-1)*rs + len).
bool disjoint_blocks(int64_t rs, int64_t bs, int64_t W, int64_t B, int64_t len) {
  if (rs < 0 || bs < 0) return false;
  const bool ranks = W <= 1, batches = B <= 1;
  const bool rank_major = (batches || bs >= len) && (ranks || rs >= (B - 1) * bs + len);
  const bool batch_major = (ranks || rs >= len) && (batches || bs >= (W - 1) * rs + len);
  return rank_major || batch_major;
}

}  // namespace
}  // namespace sp

using namespace sp;

extern "C" sp_status sp_pad(const void* x, int64_t x_batch_stride, void* y, int64_t B, int64_t T,
                            int64_t T_pad, int64_t C, sp_dtype dtype, const uint8_t* mask_in,
                            uint8_t* mask_out, void* stream) {
  if (!dtype_ok(dtype)) return SP_ERR_INVALID_ARG;
  if (B < 0 || T < 0 || C < 0 || T_pad < T) return SP_ERR_INVALID_ARG;
  if (x != nullptr && y == nullptr) return SP_ERR_INVALID_ARG;
  if ((mask_in == nullptr) != (mask_out == nullptr)) return SP_ERR_INVALID_ARG;
  const int64_t eb = elem_bytes(dtype);
  const bool tokens = y != nullptr;           // x may be null only when there are no rows to copy
  if (tokens && x == nullptr && B > 0 && T > 0 && C > 0) return SP_ERR_INVALID_ARG;
  const bool in_place = tokens && x == y;
  if (tokens) {
    if ((C * eb) % 16 != 0) return SP_ERR_UNSUPPORTED;
    if (x_batch_stride < T * C || x_batch_stride < 0) return SP_ERR_INVALID_ARG;
    if (in_place && x_batch_stride != T_pad * C) return SP_ERR_INVALID_ARG;
    if ((x != nullptr && !aligned16(x)) || !aligned16(y) || (x_batch_stride * eb) % 16 != 0) return SP_ERR_INVALID_ARG;
    if (B > kMaxGridY) return SP_ERR_UNSUPPORTED;
    if (!in_place && x != nullptr) {
      const char* xs = static_cast<const char*>(x);
      const char* ys = static_cast<const char*>(y);
      const char* xe = xs + ((B > 0 ? B - 1 : 0) * x_batch_stride + T * C) * eb;
      const char* ye = ys + B * T_pad * C * eb;
      if (B > 0 && T * C > 0 && xs < ye && ys < xe) return SP_ERR_INVALID_ARG;
    }
  }
  if (mask_in != nullptr) {
    const uint8_t* ie = mask_in + B * T * T;
    const uint8_t* oe = mask_out + B * T_pad * T_pad;
    if (B > 0 && T > 0 && mask_in < oe && mask_out < ie) return SP_ERR_INVALID_ARG;
    // the mask kernel reads the input as 4-byte words (a word holding the
    // mask's first byte starts at mask_in itself)
    if (!aligned16(mask_out) || (reinterpret_cast<uintptr_t>(mask_in) & 3u) != 0) return SP_ERR_INVALID_ARG;
  }
  hipStream_t s = as_stream(stream);
  if (tokens && B > 0 && T_pad * C > 0) {
    PadArgs a;
    a.x = static_cast<const char*>(x);
    a.y = static_cast<char*>(y);
    a.x_batch_b = x_batch_stride * eb;
    a.y_batch_b = T_pad * C * eb;
    a.copy_vecs = x != nullptr ? T * C * eb / 16 : 0;
    a.end_vec = T_pad * C * eb / 16;
    a.start_vec = in_place ? a.copy_vecs : 0;
    const int64_t n = a.end_vec - a.start_vec;
    if (n > 0) {
      dim3 grid(unsigned(div_up(n, kChunk)), unsigned(B));
      hipLaunchKernelGGL(pad_tokens_kernel, grid, dim3(kThreads), 0, s, a);
      if (launch_status() != SP_OK) return SP_ERR_HIP;
    }
  }
  if (mask_in != nullptr && B > 0 && T_pad > 0) {
    MaskPadArgs m;
    m.in = mask_in;
    m.out = mask_out;
    m.T = T;
    m.Tp = T_pad;
    m.total = B * T_pad * T_pad;
    m.in_bytes = B * T * T;
    const int64_t threads = div_up(m.total, 16);
    hipLaunchKernelGGL(pad_mask_kernel, dim3(unsigned(div_up(threads, kThreads))), dim3(kThreads), 0, s, m);
    if (launch_status() != SP_OK) return SP_ERR_HIP;
  }
  return SP_OK;
}

extern "C" sp_status sp_relayout_heads(const void* const* src, void* const* dst, int32_t n_tensors, int32_t W,
                                       int64_t B, int64_t T_pad, int32_t H, int32_t D, sp_dtype dtype,
                                       sp_dir dir, sp_shard_strides tok, sp_shard_strides head,
                                       void* stream) {
  if (!dtype_ok(dtype) || (dir != SP_TOKENS_TO_HEADS && dir != SP_HEADS_TO_TOKENS)) return SP_ERR_INVALID_ARG;
  if (W < 1 || B < 0 || T_pad < 0 || H < 1 || D < 1) return SP_ERR_INVALID_ARG;
  if (T_pad % W != 0) return SP_ERR_NOT_DIVISIBLE;
  if (H % W != 0) return SP_ERR_INVALID_ARG;
  if (n_tensors < 1 || n_tensors > 3 || src == nullptr || dst == nullptr) return SP_ERR_INVALID_ARG;
  const int64_t eb = elem_bytes(dtype);
  const int64_t Hl = H / W, Ts = T_pad / W;
  const int64_t run = Hl * D;              // elements per (token, head group)
  if ((run * eb) % 16 != 0) return SP_ERR_UNSUPPORTED;
  // the (rank, batch) blocks of each side must not overlap each other
  if (!disjoint_blocks(tok.rank, tok.batch, W, B, Ts * H * D) ||
      !disjoint_blocks(head.rank, head.batch, W, B, T_pad * run))
    return SP_ERR_INVALID_ARG;
  const int64_t tok_shard = B > 0 ? (B - 1) * tok.batch + Ts * H * D : 0;
  const int64_t head_shard = B > 0 ? (B - 1) * head.batch + T_pad * run : 0;
  if (((tok.rank | tok.batch | head.rank | head.batch) * eb) % 16 != 0) return SP_ERR_INVALID_ARG;
  const int64_t tok_span = (W - 1) * tok.rank + tok_shard;
  const int64_t head_span = (W - 1) * head.rank + head_shard;
  const int64_t s_span = (dir == SP_TOKENS_TO_HEADS ? tok_span : head_span) * eb;
  const int64_t d_span = (dir == SP_TOKENS_TO_HEADS ? head_span : tok_span) * eb;
  for (int i = 0; i < n_tensors; ++i) {
    if (src[i] == nullptr || dst[i] == nullptr || !aligned16(src[i]) || !aligned16(dst[i])) return SP_ERR_INVALID_ARG;
  }
  // no destination may overlap any source or another destination
  for (int i = 0; i < n_tensors && B > 0 && Ts > 0; ++i) {
    const char* d0 = static_cast<const char*>(dst[i]);
    for (int j = 0; j < n_tensors; ++j) {
      const char* s0 = static_cast<const char*>(src[j]);
      if (s0 < d0 + d_span && d0 < s0 + s_span) return SP_ERR_INVALID_ARG;
      const char* d1 = static_cast<const char*>(dst[j]);
      if (j != i && d1 < d0 + d_span && d0 < d1 + d_span) return SP_ERR_INVALID_ARG;
    }
  }
  if (B == 0 || Ts == 0) return SP_OK;
  const int64_t V = run * eb / 16;
  if (Ts * V >= (int64_t(1) << 32) - kChunk) return SP_ERR_UNSUPPORTED;
  if (int64_t(W) * B > kMaxGridY) return SP_ERR_UNSUPPORTED;
  if (dir == SP_HEADS_TO_TOKENS && Ts * V * W < (int64_t(1) << 32) - kChunk &&
      div_up(Ts * V * W, kChunk) * W < (int64_t(1) << 31)) {
    GatherHeadsArgs g;
    for (int i = 0; i < 3; ++i) {
      g.src[i] = static_cast<const char*>(src[i < n_tensors ? i : 0]);
      g.dst[i] = static_cast<char*>(dst[i < n_tensors ? i : 0]);
    }
    g.tok_rank_b = tok.rank * eb;
    g.tok_batch_b = tok.batch * eb;
    g.head_rank_b = head.rank * eb;
    g.head_batch_b = head.batch * eb;
    g.run_b = run * eb;
    g.seg_b = Ts * run * eb;
    g.V = uint32_t(V);
    g.fdV = make_fastdiv(uint32_t(V));
    g.fdRow = make_fastdiv(uint32_t(V * W));
    g.n_per_shard = uint32_t(Ts * V * W);
    g.chunks = uint32_t(div_up(Ts * V * W, kChunk));
    dim3 grid(unsigned(int64_t(g.chunks) * W), unsigned(B), unsigned(n_tensors));
    hipLaunchKernelGGL(gather_heads_kernel, grid, dim3(kThreads), 0, as_stream(stream), g);
    return launch_status();
  }
  RelayoutArgs a;
  for (int i = 0; i < 3; ++i) {
    a.src[i] = static_cast<const char*>(src[i < n_tensors ? i : 0]);
    a.dst[i] = static_cast<char*>(dst[i < n_tensors ? i : 0]);
  }
  a.B = B;
  a.tok_rank_b = tok.rank * eb;
  a.tok_batch_b = tok.batch * eb;
  a.tok_row_b = int64_t(H) * D * eb;
  a.head_rank_b = head.rank * eb;
  a.head_batch_b = head.batch * eb;
  a.run_b = run * eb;
  a.seg_b = Ts * run * eb;
  a.V = uint32_t(V);
  a.fdV = make_fastdiv(uint32_t(V));
  a.n_per_seg = uint32_t(Ts * V);
  a.chunks = uint32_t(div_up(Ts * V, kChunk));
  a.to_heads = dir == SP_TOKENS_TO_HEADS;
  a.Ts = Ts;
  a.valid = T_pad;
  const int64_t gx = int64_t(a.chunks) * W;
  if (gx >= (int64_t(1) << 31)) return SP_ERR_UNSUPPORTED;
  dim3 grid(unsigned(gx), unsigned(W * B), unsigned(n_tensors));
  hipLaunchKernelGGL(relayout_kernel, grid, dim3(kThreads), 0, as_stream(stream), a);
  return launch_status();
}

// Host checks shared by the two fused moves: the tensor lists, and that no
// destination overlaps a source or another destination (spans in bytes).
static sp_status check_tensor_lists(const void* const* src, void* const* dst, int32_t n_tensors, int64_t s_span,
                                    int64_t d_span) {
  if (n_tensors < 1 || n_tensors > 3 || src == nullptr || dst == nullptr) return SP_ERR_INVALID_ARG;
  for (int i = 0; i < n_tensors; ++i) {
    if (src[i] == nullptr || dst[i] == nullptr || !aligned16(src[i]) || !aligned16(dst[i])) return SP_ERR_INVALID_ARG;
  }
  for (int i = 0; i < n_tensors && s_span > 0 && d_span > 0; ++i) {
    const char* d0 = static_cast<const char*>(dst[i]);
    for (int j = 0; j < n_tensors; ++j) {
      const char* s0 = static_cast<const char*>(src[j]);
      if (s0 < d0 + d_span && d0 < s0 + s_span) return SP_ERR_INVALID_ARG;
      const char* d1 = static_cast<const char*>(dst[j]);
      if (j != i && d1 < d0 + d_span && d0 < d1 + d_span) return SP_ERR_INVALID_ARG;
    }
  }
  return SP_OK;
}

extern "C" sp_status sp_pad_relayout_heads(const void* const* src, void* const* dst, int32_t n_tensors, int32_t W,
                                           int64_t B, int64_t T, int64_t T_pad, int32_t H, int32_t D,
                                           sp_dtype dtype, int64_t src_batch_stride, sp_shard_strides head,
                                           void* stream) {
  if (!dtype_ok(dtype)) return SP_ERR_INVALID_ARG;
  if (W < 1 || B < 0 || T < 0 || T_pad < T || H < 1 || D < 1) return SP_ERR_INVALID_ARG;
  if (T_pad % W != 0) return SP_ERR_NOT_DIVISIBLE;
  if (H % W != 0) return SP_ERR_INVALID_ARG;
  const int64_t eb = elem_bytes(dtype);
  const int64_t Hl = H / W, Ts = T_pad / W, run = Hl * D, row = int64_t(H) * D;
  if ((run * eb) % 16 != 0) return SP_ERR_UNSUPPORTED;
  if (src_batch_stride < T * row || (src_batch_stride * eb) % 16 != 0) return SP_ERR_INVALID_ARG;
  if (!disjoint_blocks(head.rank, head.batch, W, B, T_pad * run)) return SP_ERR_INVALID_ARG;
  if (((head.rank | head.batch) * eb) % 16 != 0) return SP_ERR_INVALID_ARG;
  const int64_t s_span = B > 0 && T > 0 ? ((B - 1) * src_batch_stride + T * row) * eb : 0;
  const int64_t d_span = B > 0 && T_pad > 0 ? ((W - 1) * head.rank + (B - 1) * head.batch + T_pad * run) * eb : 0;
  const sp_status st = check_tensor_lists(src, dst, n_tensors, s_span, d_span);
  if (st != SP_OK) return st;
  if (B == 0 || Ts == 0) return SP_OK;
  const int64_t V = run * eb / 16;
  if (Ts * V >= (int64_t(1) << 32) - kChunk) return SP_ERR_UNSUPPORTED;
  if (int64_t(W) * B > kMaxGridY) return SP_ERR_UNSUPPORTED;
  RelayoutArgs a;
  for (int i = 0; i < 3; ++i) {
    a.src[i] = static_cast<const char*>(src[i < n_tensors ? i : 0]);
    a.dst[i] = static_cast<char*>(dst[i < n_tensors ? i : 0]);
  }
  a.B = B;
  a.tok_rank_b = Ts * row * eb;            // rank s's shard of the padded sequence
  a.tok_batch_b = src_batch_stride * eb;
  a.tok_row_b = row * eb;
  a.head_rank_b = head.rank * eb;
  a.head_batch_b = head.batch * eb;
  a.run_b = run * eb;
  a.seg_b = Ts * run * eb;
  a.V = uint32_t(V);
  a.fdV = make_fastdiv(uint32_t(V));
  a.n_per_seg = uint32_t(Ts * V);
  a.chunks = uint32_t(div_up(Ts * V, kChunk));
  a.to_heads = 1;
  a.Ts = Ts;
  a.valid = T;
  const int64_t gx = int64_t(a.chunks) * W;
  if (gx >= (int64_t(1) << 31)) return SP_ERR_UNSUPPORTED;
  dim3 grid(unsigned(gx), unsigned(W * B), unsigned(n_tensors));
  hipLaunchKernelGGL(relayout_kernel, grid, dim3(kThreads), 0, as_stream(stream), a);
  return launch_status();
}

extern "C" sp_status sp_gather_heads_unpad(const void* const* src, void* const* dst, int32_t n_tensors, int32_t W,
                                           int64_t B, int64_t T_pad, int32_t H, int32_t D, sp_dtype dtype,
                                           sp_shard_strides head, const int64_t* counts, int64_t T, void* stream) {
  if (!dtype_ok(dtype)) return SP_ERR_INVALID_ARG;
  if (W < 1 || B < 0 || T_pad < 0 || T < 0 || H < 1 || D < 1) return SP_ERR_INVALID_ARG;
  if (T_pad % W != 0) return SP_ERR_NOT_DIVISIBLE;
  if (H % W != 0) return SP_ERR_INVALID_ARG;
  if (W > kMaxWorldFused) return SP_ERR_UNSUPPORTED;
  const int64_t eb = elem_bytes(dtype);
  const int64_t Hl = H / W, Ts = T_pad / W, run = Hl * D, row = int64_t(H) * D;
  if ((run * eb) % 16 != 0) return SP_ERR_UNSUPPORTED;
  GatherHeadsUnpadArgs a;
  a.cum[0] = 0;
  for (int r = 0; r < W; ++r) {
    const int64_t c = counts ? counts[r] : Ts;
    if (c < 0 || c > Ts) return SP_ERR_INVALID_ARG;
    a.cum[r + 1] = a.cum[r] + c;
  }
  if (a.cum[W] < T) return SP_ERR_INVALID_ARG;
  if (!disjoint_blocks(head.rank, head.batch, W, B, T_pad * run)) return SP_ERR_INVALID_ARG;
  if (((head.rank | head.batch) * eb) % 16 != 0) return SP_ERR_INVALID_ARG;
  const int64_t s_span = B > 0 && T_pad > 0 ? ((W - 1) * head.rank + (B - 1) * head.batch + T_pad * run) * eb : 0;
  const int64_t d_span = B * T * row * eb;
  const sp_status st = check_tensor_lists(src, dst, n_tensors, s_span, d_span);
  if (st != SP_OK) return st;
  if (B == 0 || T == 0) return SP_OK;
  const int64_t V = run * eb / 16;
  if (Ts * V * W >= (int64_t(1) << 32) - kChunk) return SP_ERR_UNSUPPORTED;
  if (B > kMaxGridY) return SP_ERR_UNSUPPORTED;
  int64_t max_vec = 0;
  for (int r = 0; r < W; ++r) {
    int64_t kept = a.cum[r + 1] - a.cum[r];
    if (a.cum[r] + kept > T) kept = T - a.cum[r];
    if (kept < 0) kept = 0;
    a.n_vec[r] = uint32_t(kept * W * V);
    if (kept * W * V > max_vec) max_vec = kept * W * V;
  }
  for (int i = 0; i < 3; ++i) {
    a.src[i] = static_cast<const char*>(src[i < n_tensors ? i : 0]);
    a.dst[i] = static_cast<char*>(dst[i < n_tensors ? i : 0]);
  }
  a.head_rank_b = head.rank * eb;
  a.head_batch_b = head.batch * eb;
  a.run_b = run * eb;
  a.seg_b = Ts * run * eb;
  a.out_batch_b = T * row * eb;
  a.row_b = row * eb;
  a.V = uint32_t(V);
  a.fdV = make_fastdiv(uint32_t(V));
  a.fdRow = make_fastdiv(uint32_t(V * W));
  a.chunks = uint32_t(div_up(max_vec, kChunk));
  a.n_tensors = n_tensors;
  if (a.chunks == 0) return SP_OK;
  hipLaunchKernelGGL(gather_heads_unpad_kernel<kUnroll>, dim3(a.chunks, unsigned(W), unsigned(B)), dim3(kThreads), 0,
                     as_stream(stream), a);
  return launch_status();
}

extern "C" sp_status sp_gather_unpad(const void* in, sp_shard_strides in_strides, void* out, int32_t W,
                                     int64_t B, int64_t Ts, int64_t C, const int64_t* counts, int64_t T,
                                     sp_dtype dtype, void* stream) {
  if (!dtype_ok(dtype)) return SP_ERR_INVALID_ARG;
  if (W < 1 || B < 0 || Ts < 0 || C < 0 || T < 0) return SP_ERR_INVALID_ARG;
  if (W > kMaxWorld) return SP_ERR_UNSUPPORTED;
  const int64_t eb = elem_bytes(dtype);
  if ((C * eb) % 16 != 0) return SP_ERR_UNSUPPORTED;
  GatherArgs a;
  a.cum[0] = 0;
  for (int r = 0; r < W; ++r) {
    const int64_t c = counts ? counts[r] : Ts;
    if (c < 0 || c > Ts) return SP_ERR_INVALID_ARG;
    a.cum[r + 1] = a.cum[r] + c;
  }
  if (a.cum[W] < T) return SP_ERR_INVALID_ARG;
  if (B == 0 || T == 0 || C == 0) return SP_OK;
  if (in == nullptr || out == nullptr || !aligned16(in) || !aligned16(out)) return SP_ERR_INVALID_ARG;
  if (!disjoint_blocks(in_strides.rank, in_strides.batch, W, B, Ts * C)) return SP_ERR_INVALID_ARG;
  const int64_t shard = (B - 1) * in_strides.batch + Ts * C;
  if (((in_strides.rank | in_strides.batch) * eb) % 16 != 0) return SP_ERR_INVALID_ARG;
  {
    const char* i0 = static_cast<const char*>(in);
    const char* o0 = static_cast<const char*>(out);
    const int64_t ispan = ((W - 1) * in_strides.rank + shard) * eb;
    const int64_t ospan = B * T * C * eb;
    if (i0 < o0 + ospan && o0 < i0 + ispan) return SP_ERR_INVALID_ARG;
  }
  if (int64_t(W) * B > kMaxGridY) return SP_ERR_UNSUPPORTED;
  a.in = static_cast<const char*>(in);
  a.out = static_cast<char*>(out);
  a.rank_b = in_strides.rank * eb;
  a.batch_b = in_strides.batch * eb;
  a.row_b = C * eb;
  a.T = T;
  a.W = W;
  int64_t max_vec = 0;
  for (int r = 0; r < W; ++r) {
    int64_t kept = a.cum[r + 1] - a.cum[r];
    if (a.cum[r] + kept > T) kept = T - a.cum[r];
    if (kept > 0 && kept * a.row_b / 16 > max_vec) max_vec = kept * a.row_b / 16;
  }
  dim3 grid(unsigned(div_up(max_vec, kChunk)), unsigned(W * B));
  hipLaunchKernelGGL(gather_unpad_kernel, grid, dim3(kThreads), 0, as_stream(stream), a);
  return launch_status();
}

extern "C" sp_status sp_tile_2d(const void* src, void* dst, int32_t split_h, int32_t split_w, int64_t B, int64_t F,
                                int64_t height, int64_t width, int64_t C, sp_dtype dtype, sp_tile_dir dir,
                                sp_shard_strides tiles, int64_t grid_batch_stride, void* stream) {
  if (!dtype_ok(dtype) || (dir != SP_GRID_TO_TILES && dir != SP_TILES_TO_GRID)) return SP_ERR_INVALID_ARG;
  if (split_h < 1 || split_w < 1 || B < 0 || F < 0 || height < 0 || width < 0 || C < 0) return SP_ERR_INVALID_ARG;
  if (height % split_h != 0 || width % split_w != 0) return SP_ERR_NOT_DIVISIBLE;
  const int64_t eb = elem_bytes(dtype);
  if ((C * eb) % 16 != 0) return SP_ERR_UNSUPPORTED;
  const int64_t N = int64_t(split_h) * split_w;
  const int64_t th = height / split_h, tw = width / split_w;
  const int64_t T = F * height * width, Tt = F * th * tw;
  if (B == 0 || T == 0 || C == 0) return SP_OK;
  if (src == nullptr || dst == nullptr || src == dst) return SP_ERR_INVALID_ARG;
  if (!aligned16(src) || !aligned16(dst)) return SP_ERR_INVALID_ARG;
  if (grid_batch_stride < T * C || (grid_batch_stride * eb) % 16 != 0) return SP_ERR_INVALID_ARG;
  if ((tiles.rank * eb) % 16 != 0 || (tiles.batch * eb) % 16 != 0) return SP_ERR_INVALID_ARG;
  if (!disjoint_blocks(tiles.rank, tiles.batch, N, B, Tt * C)) return SP_ERR_INVALID_ARG;
  // the two sides must not overlap
  const void* grid = dir == SP_GRID_TO_TILES ? src : dst;
  const void* tl = dir == SP_GRID_TO_TILES ? dst : src;
  const char* gs = static_cast<const char*>(grid);
  const char* ts = static_cast<const char*>(tl);
  const char* ge = gs + ((B - 1) * grid_batch_stride + T * C) * eb;
  const char* te = ts + ((N - 1) * tiles.rank + (B - 1) * tiles.batch + Tt * C) * eb;
  if (gs < te && ts < ge) return SP_ERR_INVALID_ARG;
  if (N * B > kMaxGridY) return SP_ERR_UNSUPPORTED;
  const int64_t runV = tw * C * eb / 16;
  const int64_t n_per_rb = F * th * runV;
  if (n_per_rb >= (int64_t(1) << 32) - kChunk) return SP_ERR_UNSUPPORTED;
  Tile2dArgs a;
  a.src = static_cast<const char*>(src);
  a.dst = static_cast<char*>(dst);
  a.B = B;
  a.grid_batch_b = grid_batch_stride * eb;
  a.row_b = C * eb;
  a.tile_rank_b = tiles.rank * eb;
  a.tile_batch_b = tiles.batch * eb;
  a.height = height; a.width = width; a.th = th; a.tw = tw;
  a.split_w = split_w;
  a.runV = uint32_t(runV);
  a.fd_runV = make_fastdiv(uint32_t(runV));
  a.fd_th = make_fastdiv(uint32_t(th));
  a.n_per_rb = uint32_t(n_per_rb);
  a.chunks = uint32_t(div_up(n_per_rb, kChunk));
  a.to_tiles = dir == SP_GRID_TO_TILES;
  hipLaunchKernelGGL(tile_2d_kernel, dim3(a.chunks, unsigned(N * B)), dim3(kThreads), 0, as_stream(stream), a);
  return launch_status();
}

extern "C" sp_status sp_tile_2d_relayout_heads(const void* const* src, void* const* dst, int32_t n_tensors,
                                               int32_t split_h, int32_t split_w, int64_t B, int64_t F,
                                               int64_t height, int64_t width, int32_t H, int32_t D, sp_dtype dtype,
                                               sp_dir dir, int64_t grid_batch_stride, sp_shard_strides head,
                                               void* stream) {
  if (!dtype_ok(dtype) || (dir != SP_TOKENS_TO_HEADS && dir != SP_HEADS_TO_TOKENS)) return SP_ERR_INVALID_ARG;
  if (split_h < 1 || split_w < 1 || B < 0 || F < 0 || height < 0 || width < 0 || H < 1 || D < 1)
    return SP_ERR_INVALID_ARG;
  if (height % split_h != 0 || width % split_w != 0) return SP_ERR_NOT_DIVISIBLE;
  const int64_t W = int64_t(split_h) * split_w;
  if (H % W != 0) return SP_ERR_INVALID_ARG;
  if (n_tensors < 1 || n_tensors > 3 || src == nullptr || dst == nullptr) return SP_ERR_INVALID_ARG;
  const int64_t eb = elem_bytes(dtype);
  const int64_t Hl = H / W, run = Hl * D;
  if ((run * eb) % 16 != 0) return SP_ERR_UNSUPPORTED;
  const int64_t th = height / split_h, tw = width / split_w;
  const int64_t T = F * height * width, Tt = F * th * tw;
  if (grid_batch_stride < T * H * D || (grid_batch_stride * eb) % 16 != 0) return SP_ERR_INVALID_ARG;
  if (((head.rank | head.batch) * eb) % 16 != 0) return SP_ERR_INVALID_ARG;
  if (!disjoint_blocks(head.rank, head.batch, W, B, T * run)) return SP_ERR_INVALID_ARG;
  for (int i = 0; i < n_tensors; ++i) {
    if (src[i] == nullptr || dst[i] == nullptr || !aligned16(src[i]) || !aligned16(dst[i])) return SP_ERR_INVALID_ARG;
  }
  const int64_t grid_span = B > 0 ? ((B - 1) * grid_batch_stride + T * H * D) * eb : 0;
  const int64_t head_span = B > 0 ? ((W - 1) * head.rank + (B - 1) * head.batch + T * run) * eb : 0;
  const int64_t s_span = dir == SP_TOKENS_TO_HEADS ? grid_span : head_span;
  const int64_t d_span = dir == SP_TOKENS_TO_HEADS ? head_span : grid_span;
  // no destination may overlap any source or another destination
  for (int i = 0; i < n_tensors && B > 0 && T > 0; ++i) {
    const char* d0 = static_cast<const char*>(dst[i]);
    for (int j = 0; j < n_tensors; ++j) {
      const char* s0 = static_cast<const char*>(src[j]);
      if (s0 < d0 + d_span && d0 < s0 + s_span) return SP_ERR_INVALID_ARG;
      const char* d1 = static_cast<const char*>(dst[j]);
      if (j != i && d1 < d0 + d_span && d0 < d1 + d_span) return SP_ERR_INVALID_ARG;
    }
  }
  if (B == 0 || T == 0) return SP_OK;
  const int64_t V = run * eb / 16;
  const int64_t n_per = dir == SP_TOKENS_TO_HEADS ? Tt * V : T * W * V;
  if (n_per >= (int64_t(1) << 32) - kChunk || T >= (int64_t(1) << 31)) return SP_ERR_UNSUPPORTED;
  if (W * B > kMaxGridY) return SP_ERR_UNSUPPORTED;
  Tile2dHeadsArgs a;
  for (int i = 0; i < 3; ++i) {
    a.src[i] = static_cast<const char*>(src[i < n_tensors ? i : 0]);
    a.dst[i] = static_cast<char*>(dst[i < n_tensors ? i : 0]);
  }
  a.B = B;
  a.grid_batch_b = grid_batch_stride * eb;
  a.grid_row_b = int64_t(H) * D * eb;
  a.head_rank_b = head.rank * eb;
  a.head_batch_b = head.batch * eb;
  a.run_b = run * eb;
  a.height = height; a.width = width; a.th = th; a.tw = tw; a.Tt = Tt;
  a.split_w = split_w;
  a.V = uint32_t(V);
  a.fdV = make_fastdiv(uint32_t(V));
  a.fd_tw = make_fastdiv(uint32_t(tw));
  a.fd_th = make_fastdiv(uint32_t(th));
  a.fd_row = make_fastdiv(uint32_t(W * V));
  a.fd_width = make_fastdiv(uint32_t(width));
  a.fd_height = make_fastdiv(uint32_t(height));
  a.n_per = uint32_t(n_per);
  a.chunks = uint32_t(div_up(n_per, kChunk));
  if (dir == SP_TOKENS_TO_HEADS) {
    const int64_t gx = int64_t(a.chunks) * W;
    if (gx >= (int64_t(1) << 31)) return SP_ERR_UNSUPPORTED;
    hipLaunchKernelGGL(tile_2d_to_heads_kernel, dim3(unsigned(gx), unsigned(W * B), unsigned(n_tensors)),
                       dim3(kThreads), 0, as_stream(stream), a);
  } else {
    hipLaunchKernelGGL(tile_2d_from_heads_kernel, dim3(a.chunks, unsigned(B), unsigned(n_tensors)), dim3(kThreads),
                       0, as_stream(stream), a);
  }
  return launch_status();
}
