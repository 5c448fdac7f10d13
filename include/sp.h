/*
 * sp.h -- C ABI of libspattn.so: the Ulysses-style sequence-parallel attention
 * hot path for audio-video diffusion transformers, on one AMD MI355X (gfx950).
 *
 * Sources (page title, then the section on it):
 *   [SP] "LTX-2 序列并行拆解：token 切分、all2all 换头与 runner 接入全链路",
 *        section "token 切片、换头、gather 还原" and its steps 补齐 (pad),
 *        切分 (partition), 换头 (head swap), 还原 (restore); section
 *        "全局注意力没有变，只是分布方式变了" (invariants).
 *   [MG] "Multi-GPU Inference" (LTX-2 multigpu README), table "Capabilities".
 *
 * One GPU holds all W ranks ("virtual ranks"): rank r's buffers are slices of
 * one allocation, addressed through a rank stride.  The exchange between ranks
 * becomes an on-device relayout.
 *
 * Conventions for every entry point:
 *   - Pointers named as device pointers are device memory owned by the caller;
 *     arrays named as host arrays are host memory owned by the caller.  The
 *     library allocates nothing, frees nothing and keeps no state between
 *     calls.
 *   - All GPU work is enqueued on `stream` (a hipStream_t; NULL = the null
 *     stream) and returns without synchronising.  A device fault surfaces at
 *     the caller's next synchronisation.
 *   - Arguments are validated on the host before anything is launched.  On
 *     any error status nothing is written and nothing is launched.
 *   - Strides and sizes are in elements, not bytes, unless named *_bytes.
 *   - Element types: SP_F32 (4-byte float) and SP_BF16 (bfloat16 stored as 2
 *     bytes).  Copies (pad, relayout, gather) move bytes and never round.
 *   - Source and destination buffers of one call must not overlap, except
 *     where an entry point says otherwise.
 */
#ifndef SP_H
#define SP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SP_OK = 0,
  SP_ERR_NOT_DIVISIBLE = 1, /* a token count does not divide by the world size ([SP] 切分) */
  SP_ERR_INVALID_ARG = 2,   /* null pointer, bad size, bad stride, inconsistent counts */
  SP_ERR_UNSUPPORTED = 3,   /* valid request outside the built set (head dim, dtype) */
  SP_ERR_HIP = 4,           /* the HIP runtime refused a launch */
  SP_ERR_SCRATCH = 5        /* sp_masked_attention_noalloc: workspace beyond its fixed scratch */
} sp_status;

typedef enum { SP_F32 = 0, SP_BF16 = 1 } sp_dtype;

typedef enum {
  SP_TOKENS_TO_HEADS = 0, /* send_recv_heads ([SP] 换头) */
  SP_HEADS_TO_TOKENS = 1  /* gather_heads   ([SP] 换头, the swap back) */
} sp_dir;

/* Where the W rank shards of one tensor sit in memory: rank r, batch b start
 * at base + r*rank + b*batch (elements).  Token rows inside a shard are packed. */
typedef struct {
  int64_t rank;
  int64_t batch;
} sp_shard_strides;

/* Strides of a (rank, batch, token, head, d) view; d is contiguous. */
typedef struct {
  int64_t rank;
  int64_t batch;
  int64_t token;
  int64_t head;
} sp_attn_strides;

/* Human-readable name of a status (static storage; never NULL). */
const char* sp_status_string(sp_status status);

/* Version of the library, as major*10000 + minor*100 + patch. */
int32_t sp_version(void);

/*
 * sp_partition -- compute_sequence_partition ([SP] 切分).
 * Splits `total_tokens` into `world_size` equal shards.  The total must divide
 * evenly: otherwise SP_ERR_NOT_DIVISIBLE (the page's ValueError) and nothing is
 * written.  world_size < 1 or total_tokens < 0 -> SP_ERR_INVALID_ARG.
 * offsets, lengths: host arrays of world_size entries, or NULL to skip.
 * Host only: launches nothing and needs no GPU.
 */
sp_status sp_partition(int64_t total_tokens, int32_t world_size, int64_t* offsets, int64_t* lengths);

/*
 * sp_pad -- pad_modality_for_uniform_sharding ([SP] 补齐).
 * Tokens: y[b, t, :] = x[b, t, :] for t < T and zero bytes for T <= t < T_pad,
 *   with x (B, T, C) at batch stride x_batch_stride (>= T*C) and y (B, T_pad,
 *   C) packed.  x == y with x_batch_stride == T_pad*C pads in place (only the
 *   tail rows are written).  x and y may both be NULL (mask only); x may be
 *   NULL alone when T == 0 (y is then all zero bytes).
 * User mask (optional; mask_in and mask_out both NULL or both non-NULL):
 *   mask_in (B, T, T) uint8, 1 = may attend, packed, 4-byte aligned;
 *   mask_out (B, T_pad, T_pad), 16-byte aligned: the T x T block is copied,
 *   pad key columns are 0 for every row, and pad query rows see every real
 *   key and no pad key, so no row is left with nothing visible.  With no user
 *   mask the caller uses the key-only mask instead, i.e. kv_valid_len = T in
 *   sp_masked_attention.  The mask has the same B as the tokens: to extend
 *   one mask shared by every batch, call with x = y = NULL and B = 1.
 * T_pad >= T is required (any value; divisibility is sp_partition's check).
 * Errors: SP_ERR_INVALID_ARG for negative sizes, T_pad < T, a bad stride, an
 * unpaired pointer, a misaligned or overlapping mask buffer;
 * SP_ERR_UNSUPPORTED if C * element size is not a multiple of 16 bytes.
 */
sp_status sp_pad(const void* x, int64_t x_batch_stride, void* y, int64_t B, int64_t T, int64_t T_pad,
                 int64_t C, sp_dtype dtype, const uint8_t* mask_in, uint8_t* mask_out, void* stream);

/*
 * sp_relayout_heads -- send_recv_heads / gather_heads ([SP] 换头).
 * Token side of rank s: (B, Ts, H, D) with Ts = T_pad / W, at
 *   base + s*tok.rank + b*tok.batch, rows of H*D packed.
 * Head side of rank r: (B, T_pad, Hl, D) with Hl = H / W, at
 *   base + r*head.rank + b*head.batch, rows of Hl*D packed.
 * The map is head_r[b, s*Ts + t, j, :] = tok_s[b, t, r*Hl + j, :]: every rank
 * ends up with every token of its Hl local heads.  SP_TOKENS_TO_HEADS reads the
 * token side (src) and writes the head side (dst); SP_HEADS_TO_TOKENS is the
 * exact inverse.  The round trip returns the input byte for byte.
 * src, dst: host arrays of n_tensors device pointers (1..3 tensors, e.g. Q, K,
 * V in one launch), all with the same shapes and strides.
 * Errors: T_pad % W != 0 -> SP_ERR_NOT_DIVISIBLE; H % W != 0, n_tensors out of
 * 1..3, W < 1, null or equal src/dst pointers, strides that make shards
 * overlap -> SP_ERR_INVALID_ARG; Hl*D*element size not a multiple of 16 bytes
 * -> SP_ERR_UNSUPPORTED.
 */
sp_status sp_relayout_heads(const void* const* src, void* const* dst, int32_t n_tensors, int32_t W,
                            int64_t B, int64_t T_pad, int32_t H, int32_t D, sp_dtype dtype, sp_dir dir,
                            sp_shard_strides tok, sp_shard_strides head, void* stream);

/*
 * sp_pad_relayout_heads -- pad_modality_for_uniform_sharding ([SP] 补齐)
 * followed by send_recv_heads ([SP] 换头), as one move.
 * src: n_tensors unpadded token tensors (B, T, H, D), batch b at base +
 *   b*src_batch_stride (>= T*H*D), rows of H*D packed.
 * dst: the head side of every rank, as in sp_relayout_heads: rank r, batch b
 *   at base + r*head.rank + b*head.batch, (T_pad, Hl, D) packed.
 * The bytes written are those of sp_pad (tail rows T..T_pad-1 zero) into a
 * (B, T_pad, H, D) buffer, then sp_relayout_heads(SP_TOKENS_TO_HEADS) with
 * rank s's token shard at rows s*Ts.. of that buffer (Ts = T_pad / W): head
 * side row s*Ts + t of rank r holds head group r of token s*Ts + t, and zero
 * bytes where s*Ts + t >= T.  The padded token tensor is never written.
 * Errors: T_pad % W != 0 -> SP_ERR_NOT_DIVISIBLE; T_pad < T, H % W != 0,
 * n_tensors out of 1..3, W < 1, negative sizes, null, misaligned (16 bytes)
 * or overlapping pointers, head blocks that overlap, a bad batch stride ->
 * SP_ERR_INVALID_ARG; Hl*D*element size not a multiple of 16 bytes, more than
 * 65535 rank x batch blocks -> SP_ERR_UNSUPPORTED.
 */
sp_status sp_pad_relayout_heads(const void* const* src, void* const* dst, int32_t n_tensors, int32_t W,
                                int64_t B, int64_t T, int64_t T_pad, int32_t H, int32_t D, sp_dtype dtype,
                                int64_t src_batch_stride, sp_shard_strides head, void* stream);

/*
 * sp_gather_heads_unpad -- gather_heads ([SP] 换头, the swap back) followed by
 * gather_output_tokens ([SP] 还原), as one move.
 * src: the head side of every rank (B, T_pad, Hl, D) at base + r*head.rank +
 *   b*head.batch (as sp_relayout_heads writes it).
 * dst: out (B, T, H, D), packed.
 * The bytes written are those of sp_relayout_heads(SP_HEADS_TO_TOKENS) into a
 * stacked token side (W, B, Ts, H, D), then sp_gather_unpad with the same
 * counts: rank s keeps its first counts[s] token rows (counts: host array of
 * W entries, or NULL for Ts each), the kept rows are concatenated in rank
 * order and the first T form out.  The token side is never written.
 * Errors: T_pad % W != 0 -> SP_ERR_NOT_DIVISIBLE; H % W != 0, counts[s]
 * outside 0..Ts, sum(counts) < T, n_tensors out of 1..3, negative sizes, null,
 * misaligned (16 bytes) or overlapping pointers, head blocks that overlap ->
 * SP_ERR_INVALID_ARG; W > 128, Hl*D*element size not a multiple of 16 bytes,
 * B > 65535 -> SP_ERR_UNSUPPORTED.
 */
sp_status sp_gather_heads_unpad(const void* const* src, void* const* dst, int32_t n_tensors, int32_t W,
                                int64_t B, int64_t T_pad, int32_t H, int32_t D, sp_dtype dtype,
                                sp_shard_strides head, const int64_t* counts, int64_t T, void* stream);

/*
 * sp_masked_attention -- attention on the local heads ([SP] 换头, computed in
 * place on each rank; masks as defined in [SP] 补齐).
 * For R rank shares, B batches, Hl heads: query i attends key j iff
 *   j < kv_valid_len, and, if mask != NULL, mask[b, i, j] != 0.
 * o = softmax(scale * q k^T) v over the visible keys, accumulated in float32;
 * a query row with no visible key gets 0 (never NaN).  scale must be a
 * positive, finite, normal float whose product with log2(e) is normal too
 * (the path passes 1/sqrt(D)): the kernels hide a key by giving its raw
 * score -inf and take the row maximum of raw scores, which both need a
 * positive factor.  Scores are assumed finite.
 * q: (R, B, Tq, Hl, D) with strides qs; k, v: (R, B, Tk, Hl, D) with ks, vs;
 * o: (R, B, Tq, Hl, D) with os (o must not overlap q, k or v).  d is
 * contiguous for all four.  Base pointers and strides must keep every 16-byte
 * group of d aligned (bf16: multiples of 8 elements; f32: of 4).
 * mask: device (B, Tq, Tk) uint8, rows packed (row stride Tk), batch stride
 * mask_batch_stride (0 = one mask for every batch), or NULL for the key-only
 * padding mask.  The mask is shared by every rank and head.
 * workspace: device scratch of sp_masked_attention_workspace_size() bytes,
 * 256-byte aligned, rewritten by every call; may be NULL when that size is 0.
 * With a mask it holds per-tile mask classes and bit-packed mask rows and is
 * required.  For bf16 it may also hold, after that part, the partial results
 * of a split launch (per query row, O/l rounded once to bf16 and the running
 * max and sum in float32): when the query tiles do not spread evenly over the
 * GPU (one rank's share of a few heads, or a count a little above a multiple
 * of the compute units), the query tiles of whole rounds of the GPU run
 * unsplit, the key tiles of the others are cut into one equal range per
 * compute unit, and a second kernel merges the partial results.  Without room
 * for them (NULL or a smaller workspace) the same call runs unsplit: the same
 * result up to float32 summation order and that one extra rounding (at most
 * 2^-9 of |O|), slower on such shapes.
 * Supported: D in {16, 64, 128} for both types.  SP_BF16 at D = 64 and 128
 * runs bf16 MFMA with float32 softmax and accumulation; SP_BF16 at D = 16
 * widens the bf16 values exactly to float32 and runs float32 MFMA; SP_F32
 * runs float32 MFMA throughout.  bf16 outputs are rounded to nearest even.
 * Errors: sizes < 0, null tensors, kv_valid_len < 0, scale outside the range
 * above, a mask without a large enough workspace -> SP_ERR_INVALID_ARG;
 * other D, or (bf16, D = 64 or 128) a K or V token
 * stride above 8 million elements (its 32-bit tile offsets), or (bf16) a user
 * mask with Tk above 4096 * 64 keys (the per-row tile classes it keeps in
 * LDS), or a user mask with B above 65535 or Tq above 65535 query tiles
 * (tiles of 256 rows for bf16 at D = 64, else 384) -> SP_ERR_UNSUPPORTED.
 */
size_t sp_masked_attention_workspace_size(int32_t R, int64_t B, int64_t Tq, int64_t Tk, int32_t Hl, int32_t D,
                                          sp_dtype dtype, int32_t has_mask, int64_t mask_batch_stride);

sp_status sp_masked_attention(const void* q, sp_attn_strides qs, const void* k, sp_attn_strides ks,
                              const void* v, sp_attn_strides vs, void* o, sp_attn_strides os, int32_t R,
                              int64_t B, int64_t Tq, int64_t Tk, int32_t Hl, int32_t D, sp_dtype dtype,
                              int64_t kv_valid_len, const uint8_t* mask, int64_t mask_batch_stride, float scale,
                              void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of the fixed device scratch behind sp_masked_attention_noalloc. */
#define SP_NOALLOC_SCRATCH_BYTES (128u * 1024u * 1024u)

/*
 * sp_masked_attention_noalloc -- sp_masked_attention for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, result and errors as
 * sp_masked_attention, without the workspace: the library uses a fixed
 * scratch array of SP_NOALLOC_SCRATCH_BYTES in device memory, one per GPU,
 * loaded with the library and held until the process ends.  The call makes
 * no allocation and no free.  It uses exactly the workspace bytes that
 * sp_masked_attention_workspace_size() reports for the same arguments, so
 * its launches are the ones sp_masked_attention makes with a workspace of
 * that size (the same bytes out).
 * Every call on one GPU shares that GPU's scratch: calls that may overlap on
 * one GPU (on different streams, or from several host threads) race on it
 * and must be ordered by the caller.  Nothing in the scratch needs clearing
 * between calls.
 * Errors: those of sp_masked_attention; a call whose workspace size exceeds
 * SP_NOALLOC_SCRATCH_BYTES (for example a user mask over very long
 * sequences) -> SP_ERR_SCRATCH, with nothing launched; no HIP device ->
 * SP_ERR_HIP.
 */
sp_status sp_masked_attention_noalloc(const void* q, sp_attn_strides qs, const void* k, sp_attn_strides ks,
                                      const void* v, sp_attn_strides vs, void* o, sp_attn_strides os, int32_t R,
                                      int64_t B, int64_t Tq, int64_t Tk, int32_t Hl, int32_t D, sp_dtype dtype,
                                      int64_t kv_valid_len, const uint8_t* mask, int64_t mask_batch_stride,
                                      float scale, void* stream);

/*
 * sp_gather_unpad -- gather_output_tokens ([SP] 还原).
 * in: rank r's local output (B, Ts, C) at in + r*in_strides.rank +
 *   b*in_strides.batch, rows of C packed.  Rank r keeps its first counts[r]
 *   rows; the kept rows are concatenated in rank order and the first T of them
 *   form out (B, T, C), packed.  With equal shards all ranks are already at the
 *   longest length, so padding to it is a no-op.
 * counts: host array of W entries, or NULL for Ts each.
 * Errors: counts[r] outside 0..Ts, sum(counts) < T, negative sizes, null
 * pointers -> SP_ERR_INVALID_ARG; C * element size not a multiple of 16 bytes
 * -> SP_ERR_UNSUPPORTED.
 */
sp_status sp_gather_unpad(const void* in, sp_shard_strides in_strides, void* out, int32_t W, int64_t B,
                          int64_t Ts, int64_t C, const int64_t* counts, int64_t T, sp_dtype dtype,
                          void* stream);

/* Direction of sp_tile_2d. */
typedef enum {
  SP_GRID_TO_TILES = 0, /* split_cp_2d: the token grid -> every rank's tile */
  SP_TILES_TO_GRID = 1  /* gather_cp_2d: the inverse */
} sp_tile_dir;

/*
 * sp_optimal_split -- the rank grid of the 2-D (height x width) split
 * ([LC] "LongCat-Video上下文并行技术如何实现高效的多GPU推理", section
 * 智能张量拆分策略: the split ratio closest to a square).  Host only.
 * Among factor pairs split_h * split_w = n_ranks with height % split_h == 0
 * and width % split_w == 0: the pair closest to square (smallest
 * |split_h - split_w|), then the orientation whose tiles are closer to square
 * (smallest |height/split_h - width/split_w|), then the smaller split_h.
 * split_h, split_w: host outputs (either may be NULL).
 * Errors: n_ranks < 1, height or width < 1 -> SP_ERR_INVALID_ARG; no even
 * split -> SP_ERR_NOT_DIVISIBLE.
 */
sp_status sp_optimal_split(int32_t n_ranks, int64_t height, int64_t width, int32_t* split_h, int32_t* split_w);

/*
 * sp_tile_2d -- the 2-D split of a token grid over split_h x split_w ranks and
 * its inverse ([LC] 智能张量拆分策略: split_tensor_in_cp_2d splits along height
 * then width; gather_cp_2d puts the pieces back).  A bit copy.
 * grid: (B, F, height, width, C) tokens in raster order (token f*height*width
 *   + y*width + x), batch b at grid + b*grid_batch_stride, rows of C packed.
 * tiles: rank r = i*split_w + j, batch b at tiles + r*tiles.rank +
 *   b*tiles.batch: F*th*tw rows of C packed (th = height/split_h, tw =
 *   width/split_w): rows i*th.., columns j*tw.. of every frame, in raster
 *   order within the tile.
 * SP_GRID_TO_TILES reads grid (src) and writes tiles (dst); SP_TILES_TO_GRID
 * the reverse.  All strides in elements; the round trip returns the input
 * byte for byte.
 * Errors: height % split_h or width % split_w != 0 -> SP_ERR_NOT_DIVISIBLE;
 * negative sizes, split < 1, null, misaligned (16 bytes) or overlapping
 * pointers, tile blocks that overlap, grid_batch_stride < F*height*width*C ->
 * SP_ERR_INVALID_ARG; C * element size not a multiple of 16 bytes, more than
 * 65535 rank x batch blocks -> SP_ERR_UNSUPPORTED.
 */
sp_status sp_tile_2d(const void* src, void* dst, int32_t split_h, int32_t split_w, int64_t B, int64_t F,
                     int64_t height, int64_t width, int64_t C, sp_dtype dtype, sp_tile_dir dir,
                     sp_shard_strides tiles, int64_t grid_batch_stride, void* stream);

/*
 * sp_tile_2d_relayout_heads -- the 2-D split and the head exchange as one
 * move ([LC] 智能张量拆分策略: split_tensor_in_cp_2d, then [SP] 换头
 * send_recv_heads on the tiles; the inverse is [SP] gather_heads, then [LC]
 * gather_cp_2d).  A bit copy.  W = split_h * split_w ranks, rank s = i*split_w
 * + j holding tile (i, j) of every frame (th = height/split_h, tw =
 * width/split_w, Tt = F*th*tw tokens, raster order inside the tile).
 * grid: (B, T, H, D) tokens in raster order, T = F*height*width, batch b at
 *   base + b*grid_batch_stride, rows of H*D packed (as in sp_tile_2d).
 * head side of rank r: (B, T, Hl, D) with Hl = H / W at base + r*head.rank +
 *   b*head.batch, rows of Hl*D packed; row s*Tt + t holds head group r of rank
 *   s's tile token t (as sp_relayout_heads leaves it after sp_tile_2d).
 * SP_TOKENS_TO_HEADS reads the grid (src) and writes the head side (dst): the
 * same bytes as sp_tile_2d(SP_GRID_TO_TILES) followed by
 * sp_relayout_heads(SP_TOKENS_TO_HEADS) on stacked tiles (W, B, Tt, H, D);
 * SP_HEADS_TO_TOKENS is the exact inverse (sp_relayout_heads(
 * SP_HEADS_TO_TOKENS), then sp_tile_2d(SP_TILES_TO_GRID)).
 * src, dst: host arrays of n_tensors device pointers (1..3), same shapes and
 * strides.  Strides in elements.
 * Errors: height % split_h or width % split_w != 0 -> SP_ERR_NOT_DIVISIBLE;
 * H % W != 0, n_tensors out of 1..3, negative sizes, split < 1, null,
 * misaligned (16 bytes) or overlapping pointers, head blocks that overlap,
 * grid_batch_stride < T*H*D -> SP_ERR_INVALID_ARG; Hl*D*element size not a
 * multiple of 16 bytes, more than 65535 rank x batch blocks, T of 2^31 tokens
 * or more, or more than 2^32 - 1024 16-byte vectors in one head-side segment
 * (Tt*Hl*D elements) for SP_TOKENS_TO_HEADS or in one batch of the grid
 * (T*H*D elements) for SP_HEADS_TO_TOKENS -> SP_ERR_UNSUPPORTED.
 */
sp_status sp_tile_2d_relayout_heads(const void* const* src, void* const* dst, int32_t n_tensors, int32_t split_h,
                                    int32_t split_w, int64_t B, int64_t F, int64_t height, int64_t width, int32_t H,
                                    int32_t D, sp_dtype dtype, sp_dir dir, int64_t grid_batch_stride,
                                    sp_shard_strides head, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SP_H */
