// Masked attention on the local heads of every virtual rank, as one flash-style
// kernel per dtype for gfx950 (CDNA4).
//
// Source: page "LTX-2 序列并行拆解：token 切分、all2all 换头与 runner 接入全链路",
// section "token 切片、换头、gather 还原": step 换头 (after the swap each rank runs
// full-sequence attention over its local heads) and step 补齐 (the key-only
// padding mask, and the extended user mask in which pad query rows keep the real
// keys visible).
//
// Design (bf16):
//   * one workgroup = 12 waves = 384 query rows of one (rank, batch, head)
//     at D = 128 (8 waves = 256 rows at D = 64, two workgroups per CU); each
//     wave owns 32 query rows for the whole key loop, and three (four) waves
//     share each SIMD, so one wave's softmax (VALU) runs while another's MFMAs
//     do.  The kernel is templated on query blocks per wave (QB); two blocks
//     per wave would let every LDS operand feed two MFMAs, but at D = 128 the
//     registers then only allow one wave per SIMD, which measured slower;
//   * key tiles of KT = 128 are fetched with 16-byte MUBUF loads straight into
//     LDS (double buffer, one barrier per tile; the next tile's loads overlap
//     this tile's compute); the tile is stored as padded 1 KiB key groups (see
//     Bf16Tile) so that the MFMA operand reads are bank-conflict free and their
//     addresses are a lane base plus immediates;
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (Q stays in registers as the B
//     operand).  In the 32x32 accumulator layout a lane holds 16 keys of ONE
//     query, so the row max/sum are in-lane plus one swap with lane^32, and the
//     same registers, rounded to bf16, are directly the B operand of
//     O^T += V^T P^T, whose accumulator again gives each lane one query: the
//     softmax rescale is a per-lane scalar.  The V^T operand is read from the
//     row-major V tile with the LDS transpose read ds_read_b64_tr_b16;
//   * each tile is processed in parts of 32 keys, software pipelined: one
//     scheduling block holds PV of part k-1, QK^T of part k+1 and the softmax
//     of part k;
//   * softmax in float32 with exp2 (scale*log2 e folded into one FMA); the
//     running max is raised lazily: only when some lane's sum of a part's p
//     exceeds 256 (every p of the part is below that sum), so p stays <= 256
//     between rescales; row sums add the bf16-rounded p with v_dot2;
//   * user masks are classified once per call into empty/full/partial tiles:
//     empty tiles are skipped, full tiles read no mask bytes, partial tiles one
//     64-bit visibility word per row and 64 keys (direct loads into LDS with
//     the tile's K/V; the tile classes of a query tile's row sit in LDS too);
//   * without a user mask, workgroup ids are remapped so that the 8 XCDs each
//     take a contiguous run of (rank, batch, head) groups: the q-tiles sharing
//     one head's K/V run on the same XCD and share its L2; with a user mask
//     the work is uneven and query tiles go longest first over the whole GPU;
//   * launches with too few query tiles to fill the GPU (one rank's share)
//     split the key range over all compute units and merge partial results
//     (attn_combine_kernel).

#include "sp_bits.h"
#include "sp_internal.h"

#include <cmath>
#include <mutex>
#include <type_traits>

namespace sp {
namespace {

constexpr int QB = 1;                // 32-row query blocks per wave of the bf16 kernel
// Waves per bf16 workgroup, by head dim.  D = 128: 12 waves, three per SIMD,
// one workgroup per CU (its K/V buffers take 136 KiB of LDS; measured +4-6 %
// over 8 waves).  D = 64: 8 waves, and the buffers take 68 KiB, so two
// workgroups share a CU at four waves per SIMD (128 VGPRs): one workgroup's
// prologue and epilogue overlap the other's tiles (measured +3 % on long key
// ranges, +10-20 % on the 1024-key cross-attention launches).  At three waves
// the D = 128 kernels sit at the 168-VGPR limit; the plain kernel has no
// scratch access and the others a few reloads outside the per-part work.
// After any change, check that no scratch access lands in the per-tile path
// (the tile loop's load issue and compute blocks): a reload there waits for
// every load in flight and costs 5-12 %.
template <int D>
constexpr int kWaves = D == 64 ? 8 : 12;
template <int D>
constexpr int kWavesPerSimd = D == 64 ? 4 : 3;
// D = 64 launches whose items would leave at least half of the GPU's
// workgroup slots empty run 4-wave workgroups of 128 query rows instead (no
// user mask, unsplit): twice the workgroups over the same work, two per CU
// (cross_v2a's share, 96 query tiles of 256 rows: 25.4 -> 20.6 us; the
// all-ranks launch, which fills the GPU, measured 11 % slower so).
constexpr int kNarrowWaves64 = 4;
// query rows per bf16 workgroup, and the height of the mask-class tiles of
// bf16 launches
template <int D>
constexpr int kRows = 32 * QB * kWaves<D>;
constexpr int BM32 = 128;            // query rows per fp32 workgroup
constexpr int kClsRowsF32 = 384;     // mask-class tile height of fp32 launches (a multiple of BM32)
constexpr int BN = 64;               // keys per tile (all kernels, and the mask-class tile width)
constexpr int KT = 128;              // keys per LDS tile of the bf16 kernel (a multiple of BN)
constexpr int NBUF = 2;              // LDS tile buffers of the bf16 kernel (pipeline depth)
static_assert(kClsRowsF32 % BM32 == 0, "an fp32 query tile lies inside one class tile");
constexpr float kRescaleSlack = 8.0f;  // log2 units: p <= 2^8 between rescales (fp32 kernel)
constexpr int kMaxClassTiles = 4096;   // BN-key class tiles per mask row the bf16 kernel supports (even)
static_assert(kMaxClassTiles % 2 == 0, "class rows are padded to even length in place");
constexpr float kSumLimit = 256.0f;    // bf16 kernel: p <= (sum of a lane's part) <= 256 between rescales

enum : uint8_t { kTileEmpty = 0, kTileFull = 1, kTilePartial = 2 };

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  int64_t qs[4], ks[4], vs[4], os[4];   // rank, batch, token, head strides (elements)
  int64_t B, Tq, Tk;
  int32_t Hl;
  int64_t kv_end;                        // keys >= kv_end are never visible
  const uint8_t* mask;                   // (B, Tq, Tk) or null
  int64_t mask_bs;                       // batch stride of mask (0 = shared)
  const uint8_t* cls;                    // tile classes (Bm, nqt_cls, nkt) of class-tile rows x BN keys
  const uint64_t* bits;                  // visibility words (Bm, nkt, ldw): bit j = key BN*kt + j
  int64_t ldw;                           // rows per class tile of bits: Tq rounded up to even
  int32_t nqt, nkt;                      // query tiles of this kernel, key tiles of BN
  int32_t nqt_cls;                       // query tiles of the class map
  float c;                               // scale * log2(e)
  uint32_t nwg;
  // split launches (bf16): items [0, n_direct) run whole, one workgroup
  // each, as in a plain launch; the key tiles of the others, item after
  // item, are cut into ranges
  int64_t units;                         // nwg * nku (balanced split: unused, planned on the device)
  int64_t upw;                           // units per range
  int32_t nku;                           // key tiles of KT per item
  uint32_t n_direct;                     // items run whole before the ranges (0 with a user mask)
  char* part;                            // partial records, two per workgroup (RecordLayout)
  // balanced split of a masked launch (see attn_bf16_kernel): workgroups of
  // the launch, and the plan written by logical workgroup 0 for the merge
  int32_t split_wgs;
  int32_t* plan_nnz;                     // non-empty key tiles of each query block, in dispatch order
  int64_t* plan_s;                       // first unit of each query block; plan_s[nqt] = all units
  int64_t* plan_start;                   // per logical workgroup: first unit, end unit, block, item << 32 | tile
};

// Query blocks a balanced split plans for (its per-block counts sit in LDS).
constexpr int kMaxPlanBlocks = 512;
// Units a balanced split charges for the start of an item's segment, on top
// of its non-empty key tiles: a segment's Q load, first-tile wait and output
// or record store take two to three tile-times at D = 128 (per-workgroup
// timestamps on MI355X: ~6.5 us to the first tile and ~7 us of stores against
// ~5.5 us per tile).  Without it the workgroups whose range meets two items
// set the critical path (1.21x the average workgroup time on a block-causal
// share); the uneven-mask share's split launch measured 102.6 / 96.8 / 94.1
// / 95.2 us at 0 / 2 / 3 / 4 units.
constexpr int kSegmentCost = 3;

// One partial record of a split launch: for BM query rows, O/l of the
// segment rounded once to bf16 (rows of D), then m (running max, log2 units)
// and l (sum of p) per row in float32.  The merge recombines the segments'
// O/l with weights 2^(m_s - M) l_s, so each record costs half the bytes of
// unnormalised float32 rows; the one extra bf16 rounding of O/l adds at most
// 2^-9 of |O/l| (a convex combination of V rows) to the result, below the
// output's own bf16 rounding of the same size.
template <int D>
struct RecordLayout {
  static constexpr int64_t BM = kRows<D>;
  static constexpr int64_t kO = 0;                      // bf16 [BM][D]
  static constexpr int64_t kM = BM * D * 2;             // float [BM]
  static constexpr int64_t kL = kM + BM * 4;            // float [BM]
  static constexpr int64_t kBytes = kL + BM * 4;
  static_assert(kBytes % 256 == 0, "records stay 256-byte aligned");
};

// Workgroup i runs on XCD i % 8.  Give XCD x a contiguous range of logical
// tiles so that neighbouring q-tiles of one head share that XCD's L2.
__device__ __forceinline__ uint32_t xcd_remap(uint32_t i, uint32_t n) {
  const uint32_t x = i & 7u, j = i >> 3;
  const uint32_t q = n >> 3, rr = n & 7u;
  return x < rr ? x * (q + 1) + j : rr * (q + 1) + (x - rr) * q + j;
}

struct TileCoord {
  int64_t r, b;
  int32_t head, qt;
};

// Item i: one query tile of one (rank, batch, head).  Without a user mask
// every item costs the same: query tile fastest, then head, batch, rank, and
// workgroups are remapped so that each XCD takes a contiguous run (the query
// tiles of a head share that XCD's L2).  With a user mask the later query
// tiles usually see more keys (causal-like masks): items are ordered by
// query tile, last tile first, with (rank, batch, head) fastest, and
// dispatched in that order (longest first over the whole GPU); the hardware's
// round-robin over the 8 XCDs still keeps each head on one XCD when the
// number of heads is a multiple of 8.
template <bool MASK>
__device__ __forceinline__ TileCoord decode_item(const AttnArgs& a, uint32_t item) {
  TileCoord t;
  uint32_t qi, rest;
  if (MASK) {
    const uint32_t nrbh = a.nwg / uint32_t(a.nqt);
    qi = item / nrbh;
    rest = item - qi * nrbh;
  } else {
    qi = item % uint32_t(a.nqt);
    rest = item / uint32_t(a.nqt);
  }
  t.head = int32_t(rest % uint32_t(a.Hl));
  rest /= uint32_t(a.Hl);
  t.b = int64_t(rest % uint64_t(a.B));
  t.r = int64_t(rest / uint64_t(a.B));
  t.qt = MASK ? a.nqt - 1 - int32_t(qi) : int32_t(qi);
  return t;
}

// A wave-uniform value moved to scalar registers (the compiler cannot tell
// that values loaded from LDS or derived from them are uniform, and would
// keep them in vector registers).
__device__ __forceinline__ int32_t uniform(int32_t x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ int64_t uniform(int64_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(uint64_t(x)));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(uint64_t(x) >> 32));
  return int64_t((uint64_t(hi) << 32) | lo);
}

// max of x over the lane pair (l, l ^ 32): one v_permlane32_swap (no LDS trip)
__device__ __forceinline__ float wave_max_pair(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// ---------------------------------------------------------------- bf16 kernel

// LDS layout of one K or V tile (KT keys x D dims, bf16).  The tile is cut
// into groups of KPG keys whose rows make exactly 1 KiB (KPG = 4 at D = 128,
// 8 at D = 64); one 16-byte direct load of a wave (64 lanes) fills one group,
// reading KPG whole rows.  Groups sit GROUP_BYTES apart (1 KiB + 64 B of
// padding, which shifts consecutive groups by 16 banks).  Inside a group,
// chunk c (dims 8c .. 8c+7) of key n sits at c*KPG*16 + pos*16 with pos the
// key's index in the group, XOR 4 on odd chunks when KPG = 8.  With this
// layout the 8 lanes of each ds_read_b128 phase (8 keys, one chunk) and the
// 16 lanes of each transpose read (4 keys x 2 adjacent chunks) touch 32
// different banks, and every read address is a per-lane base plus a
// compile-time offset.
template <int D>
struct Bf16Tile {
  static constexpr int KPG = 512 / D;               // keys per 1 KiB group
  static constexpr int NG = KT / KPG;               // groups per tile = direct loads per tile
  static constexpr int GROUP_BYTES = 1024 + 64;
  static constexpr int TILE_BYTES = NG * GROUP_BYTES;
  static constexpr int NKS = D / 16;                // k-steps of QK^T
  static constexpr int NDB = D / 32;                // 32-row blocks of O^T
  static_assert(D == 64 || D == 128, "bf16 tiles are built for D = 64 and 128");
  static_assert(2 * NBUF * TILE_BYTES <= 160 * 1024, "K and V buffers must fit the 160 KiB LDS");

  static __host__ __device__ constexpr int pos(int n, int c) {
    return KPG == 8 ? ((n % KPG) ^ (4 * (c & 1))) : (n % KPG);
  }
  // byte offset of chunk c of key n inside the tile
  static __host__ __device__ constexpr int offset(int n, int c) {
    return (n / KPG) * GROUP_BYTES + c * KPG * 16 + pos(n, c) * 16;
  }
};

// s_waitcnt with vmcnt = n and expcnt / lgkmcnt left at their maximum.
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00);
}

template <int D, bool MASK, bool SPLIT, bool BAL = false, int WAVES = kWaves<D>>
__global__ __launch_bounds__(64 * WAVES)
__attribute__((amdgpu_waves_per_eu(WAVES == kWaves<D> ? kWavesPerSimd<D> : kWavesPerSimd<D> * WAVES / kWaves<D>)))
void attn_bf16_kernel(AttnArgs a) {
  static_assert(!BAL || (MASK && SPLIT), "the balanced split is a split of masked launches");
  // (class tiles and partial records are kRows<D> rows high)
  static_assert(WAVES == kWaves<D> || (!MASK && !SPLIT), "narrow workgroups only for plain launches");
  constexpr int THREADS = 64 * WAVES, BM = 32 * QB * WAVES;
  using T = Bf16Tile<D>;
  constexpr int NKS = T::NKS, NDB = T::NDB, KPG = T::KPG, NG = T::NG;
  constexpr int NLD = (NG + WAVES - 1) / WAVES;   // direct loads per wave per tile and tensor (at most)
  constexpr int LOADS = 2 * NLD;   // direct loads per wave per tile (K and V)
  // Each buffer is its own LDS object, so that the compiler can tell which
  // buffer a direct load writes and never waits on it before reading another.
  __shared__ __attribute__((aligned(1024))) char k_lds0[T::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char v_lds0[T::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char k_lds1[T::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char v_lds1[T::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char k_lds2[NBUF > 2 ? T::TILE_BYTES : 16];
  __shared__ __attribute__((aligned(1024))) char v_lds2[NBUF > 2 ? T::TILE_BYTES : 16];
  // class bytes of this query tile's row of the class map (user masks): read
  // from LDS, so that looking up a tile's class never waits on global memory
  // (a wait for a global load would also wait for the K/V tile in flight)
  // (padded with one kTileEmpty byte to even length, so that a key tile
  // always reads both of its class bytes as one 16-bit word; kMaxClassTiles
  // is even, and the array is sized to keep two D = 64 workgroups in LDS)
  __shared__ __attribute__((aligned(4))) uint8_t cls_lds[MASK ? kMaxClassTiles : 4];
  // visibility words of the key tiles in flight (partial tiles only): buffer i
  // holds, for each BN-key class tile c of its key tile, the words of this
  // workgroup's BM rows at [c * BM + row]; filled by direct loads with K/V
  __shared__ __attribute__((aligned(16))) uint64_t mw_lds[MASK ? NBUF * (KT / BN) * BM : 2];
  auto kbuf = [&](auto i) __attribute__((always_inline)) -> char* {
    constexpr int I = decltype(i)::value;
    return I == 0 ? k_lds0 : (I == 1 ? k_lds1 : k_lds2);
  };
  auto vbuf = [&](auto i) __attribute__((always_inline)) -> char* {
    constexpr int I = decltype(i)::value;
    return I == 0 ? v_lds0 : (I == 1 ? v_lds1 : v_lds2);
  };
  using I0 = std::integral_constant<int, 0>;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, h = lane >> 5;

  // Work split.  Without SPLIT a workgroup runs one item over all of its key
  // tiles.  With SPLIT (launches whose items do not divide evenly over the
  // GPU) the key tiles of all items, item after item, form one sequence of
  // units.  The first n_direct workgroups run items [0, n_direct) whole, one
  // each (whole rounds of the GPU, dispatched first, as in a plain launch);
  // after them logical range g (workgroup n_direct + g before the remap)
  // runs units n_direct*nku + [g*upw, (g+1)*upw), one segment per item it
  // meets.  A segment that covers a whole item ends like an unsplit one; only
  // the first and the last segment of a range can be partial, and each of
  // those ends in a partial record (O/l rows, running max and sum) that
  // attn_combine_kernel merges into O.  So the dispatcher fills the last,
  // partly filled round of a plain launch with ranges of equal work.
  const bool run_whole = SPLIT && !MASK && blockIdx.x < a.n_direct;
  const uint32_t gl = !SPLIT || run_whole ? 0u
                      : BAL              ? xcd_remap(blockIdx.x, gridDim.x)
                                         : xcd_remap(blockIdx.x - a.n_direct, gridDim.x - a.n_direct);
  int64_t u_next = 0, u_end = 0;
  if constexpr (SPLIT && !BAL) {
    if (run_whole) {
      u_next = uniform(int64_t(xcd_remap(blockIdx.x, a.n_direct)) * a.nku);
      u_end = u_next + a.nku;
    } else {
      u_next = uniform(int64_t(a.n_direct) * a.nku + int64_t(gl) * a.upw);
      u_end = uniform(a.units < u_next + a.upw ? a.units : u_next + a.upw);
    }
  }
  // Balanced split (masked launches whose items all share one mask): the
  // units are the non-empty key tiles of every item, after kSegmentCost
  // units for the item's start, so each workgroup's range holds the same
  // work, where counting empty tiles too (above) leaves the ranges over long
  // query tiles with several times the work of the others.  Items come query
  // block by query block (block qi is query tile nqt-1-qi), (rank, batch,
  // head) fastest, so every item of a block has the block's count of
  // non-empty tiles (a.plan_nnz).  plan_balanced_split_kernel has written
  // where this workgroup's range starts: block qi_cur, item p_cur of the
  // block, unit k_cur of the item.  (Planned in a kernel of its own: the same
  // planning inside this kernel pushed Q fragments out to scratch in the tile
  // loop.)
  int32_t qi_cur = 0, p_cur = 0, k_cur = 0;
  const int32_t nrbh = int32_t(a.nwg / uint32_t(a.nqt));          // items per query block
  const int32_t nku_b = int32_t((a.kv_end + KT - 1) / KT);          // key tiles below kv_end
  if constexpr (BAL) {
    const int64_t* st = a.plan_start + 4 * int64_t(gl);
    u_next = uniform(st[0]);
    u_end = uniform(st[1]);
    qi_cur = int32_t(uniform(st[2]));
    const int64_t pk = uniform(st[3]);
    p_cur = int32_t(pk >> 32);
    k_cur = int32_t(pk & 0xffffffff);
  }
  for (int seg = 0;; ++seg) {
  uint32_t item;
  int kt_first = 0, kt_stop = 0;
  int32_t k_first = 0, k_stop = 0, nnz_seg = 0;   // (BAL) this segment's non-empty tiles of its item
  bool whole = false;                              // (BAL) the segment covers its whole item
  if constexpr (BAL) {
    if (u_next >= u_end) break;
    while (uniform(a.plan_nnz[qi_cur]) == 0) {   // blocks with no visible key tile: the merge writes their zeros
      ++qi_cur;
      p_cur = 0;
      k_cur = 0;
    }
    item = uint32_t(qi_cur * nrbh + p_cur);
    nnz_seg = uniform(a.plan_nnz[qi_cur]);
    // an item's units: kSegmentCost units for its start, then its non-empty
    // tiles; k_first, k_stop count them, and the segment runs tiles
    // [k_first - kSegmentCost, k_stop - kSegmentCost) (clamped at 0)
    const int32_t nu = nnz_seg + kSegmentCost;
    k_first = k_cur;
    k_stop = int64_t(nu - k_first) < u_end - u_next ? nu : k_first + int32_t(u_end - u_next);
    whole = k_first <= kSegmentCost && k_stop == nu;
    u_next += k_stop - k_first;
    if (k_stop == nu) {
      k_cur = 0;
      if (++p_cur == nrbh) {
        p_cur = 0;
        ++qi_cur;
      }
    } else {
      k_cur = k_stop;
    }
    // (no range ends inside an item's start units: the plan ends it at the
    // item's first unit instead, so every segment has tiles)
    k_first = k_first > kSegmentCost ? k_first - kSegmentCost : 0;
    k_stop -= kSegmentCost;
    if (seg > 0) __syncthreads();   // every wave is done with the previous segment's LDS tiles
  } else if constexpr (SPLIT) {
    if (u_next >= u_end) break;
    item = uint32_t(uniform(int32_t(u_next / a.nku)));
    kt_first = uniform(int32_t(u_next - int64_t(item) * a.nku));
    kt_stop = uniform(int32_t(a.nku - kt_first < u_end - u_next ? a.nku : kt_first + (u_end - u_next)));
    u_next = uniform(u_next + (kt_stop - kt_first));
    if (seg > 0) __syncthreads();   // every wave is done with the previous segment's LDS tiles
  } else {
    item = MASK ? blockIdx.x : xcd_remap(blockIdx.x, a.nwg);
  }
  // (the decode divides by runtime values in vector instructions; its results
  // are uniform and kept in scalar registers, which leaves the vector
  // registers to the tile loop)
  TileCoord tc = decode_item<MASK>(a, item);
  tc.r = uniform(tc.r);
  tc.b = uniform(tc.b);
  tc.head = uniform(tc.head);
  tc.qt = uniform(tc.qt);

  const uint16_t* qp = static_cast<const uint16_t*>(a.q) + tc.r * a.qs[0] + tc.b * a.qs[1] + tc.head * a.qs[3];
  const uint16_t* kp = static_cast<const uint16_t*>(a.k) + tc.r * a.ks[0] + tc.b * a.ks[1] + tc.head * a.ks[3];
  const uint16_t* vp = static_cast<const uint16_t*>(a.v) + tc.r * a.vs[0] + tc.b * a.vs[1] + tc.head * a.vs[3];
  uint16_t* op = static_cast<uint16_t*>(a.o) + tc.r * a.os[0] + tc.b * a.os[1] + tc.head * a.os[3];

  // query rows of this lane: block qb covers rows 32*QB*w + 32*qb .. +31 of the tile
  int64_t qrow[QB];
  bool qvalid[QB];
  bf16x8 qf[QB][NKS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    qrow[qb] = int64_t(tc.qt) * BM + 32 * QB * w + 32 * qb + l32;
    qvalid[qb] = qrow[qb] < a.Tq;
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      qf[qb][s] = bf16x8{};
      if (qvalid[qb]) qf[qb][s] = *reinterpret_cast<const bf16x8*>(qp + qrow[qb] * a.qs[2] + 16 * s + 8 * h);
    }
  }

  f32x16 oacc[QB][NDB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int d = 0; d < NDB; ++d) oacc[qb][d] = f32x16{};
  float m_run[QB], l_run[QB];   // running max per query (log2 units); this lane's share of the sum
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = -1e30f;
    l_run[qb] = 0.f;
  }

  const uint8_t* cls_row = nullptr;
  const uint64_t* wbase = nullptr;   // visibility words of this batch's mask, class tile 0
  if (MASK) {
    const int64_t bm = a.mask_bs ? tc.b : 0;
    cls_row = a.cls + (bm * a.nqt_cls + tc.qt) * int64_t(a.nkt);
    wbase = a.bits + bm * a.nkt * a.ldw;
    // (the split kernel instead masks the byte past an odd-length row where
    // it reads it: with the padding copy its register allocation moved Q
    // fragments to scratch inside the tile loop)
    if constexpr (SPLIT) {
      for (int i = tid; i < a.nkt; i += THREADS) cls_lds[i] = cls_row[i];
    } else {
      for (int i = tid; i < a.nkt + (a.nkt & 1); i += THREADS) cls_lds[i] = i < a.nkt ? cls_row[i] : uint8_t(kTileEmpty);
    }
    __syncthreads();
  }
  if constexpr (BAL) {
    // key tile of the k-th non-empty key tile of this item's class row (nku_b
    // when k is the count): each wave scans 64 tiles at a time with a ballot
    auto nth_tile = [&](int32_t k) -> int {
      for (int c0 = 0; c0 < nku_b; c0 += 64) {
        const int kt = c0 + lane;
        bool ne = false;
        if (kt < nku_b) {
          uint32_t c = cls_lds[2 * kt];
          if (2 * kt + 1 < a.nkt) c |= cls_lds[2 * kt + 1];
          ne = c != kTileEmpty;
        }
        const uint64_t m = __ballot(ne);
        const int cnt = __popcll(m);
        if (k < cnt) {
          const uint32_t below = __builtin_amdgcn_mbcnt_hi(uint32_t(m >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(m), 0u));
          return c0 + __ffsll((unsigned long long)__ballot(ne && int(below) == k)) - 1;
        }
        k -= cnt;
      }
      return nku_b;
    };
    kt_first = uniform(nth_tile(k_first));
    kt_stop = k_stop == nnz_seg ? nku_b : uniform(nth_tile(k_stop));
  }
  // Key tiles of KT keys; with a user mask a tile's class combines the classes
  // of its BN-key class tiles, and empty tiles are skipped.  This segment runs
  // tiles [kt_first, nkt_eff).
  const int nkt_eff = SPLIT ? kt_stop : int((a.kv_end + KT - 1) / KT);
  // The class of a key tile is read once, when the tile enters the pipeline
  // (right after the barrier, with no operand reads in flight), and carried
  // with it: each class read is an LDS round trip that the wave waits for
  // (-3 % on fully masked launches with the carry).  The split kernel, with
  // its segment state, reads the class again where it is used: there the
  // carried values push the Q fragments out to scratch (+3.5 %).
  constexpr bool kCarryClass = !SPLIT;
  static_assert(KT / BN == 2 && kTileEmpty == 0 && kTileFull == 1, "two class bytes per key tile");
  auto tile_class = [&](int kt) __attribute__((always_inline)) -> uint8_t {
    if (!MASK) return kTileFull;
    // uniform over the workgroup: kept in scalar registers
    uint32_t pair = __builtin_amdgcn_readfirstlane(*reinterpret_cast<const uint16_t*>(cls_lds + 2 * kt));
    if (SPLIT && 2 * kt + 1 >= a.nkt) pair &= 0xffu;
    return pair == 0 ? kTileEmpty : (pair == 0x0101u ? kTileFull : kTilePartial);
  };
  // next tile after kt that is not empty (nkt_eff or more if none), and its class
  auto next_tile = [&](int kt, uint8_t& c) __attribute__((always_inline)) {
    ++kt;
    c = kTileFull;
    if (MASK)
      for (; kt < nkt_eff; ++kt) {
        c = tile_class(kt);
        if (c != kTileEmpty) break;
      }
    return kt;
  };

  // Direct loads: per tile and tensor, wave w fills groups w, w + WAVES, ...
  // Lane i of a load writes LDS byte 16*i of its group, which holds chunk
  // c = i / KPG of the key whose pos() is i % KPG.  Keys past kv_end read row
  // kv_end-1 instead (in bounds and finite); their scores are masked to -inf,
  // so their weight is exactly 0.
  //
  // The loads are MUBUF buffer loads into LDS through a descriptor based at
  // the tile's first key (rebuilt per tile, 32-bit offsets inside it, bounds
  // checked by the descriptor).  The FLAT-encoded global_load_lds would do
  // the same copy, but while one of those is in flight the compiler cannot
  // count LDS reads precisely and waits for all of them before every MFMA.
  //
  // The lane offsets are recomputed from the lane index at every issue (a few
  // VALU ops per tile): kept live across the tile loop they are the first
  // values the register allocator spills at three waves per SIMD, and a
  // reload before each load then waits for every load in flight.
  const int wu = __builtin_amdgcn_readfirstlane(w);          // wave index, as a scalar
  // Waves whose query rows all lie past Tq (in the last query tile of a
  // ragged Tq) still share the loads and barriers but skip the compute.
  const bool wave_has_rows = int64_t(tc.qt) * BM + 32 * QB * wu < a.Tq;
  const int32_t kst = int32_t(a.ks[2]) * 2, vst = int32_t(a.vs[2]) * 2;   // token strides in bytes (host-checked)
  const int32_t k_nrec = (KT - 1) * kst + 2 * D, v_nrec = (KT - 1) * vst + 2 * D;
  constexpr int32_t kRsrcWord3 = 0x00020000;   // raw 32-bit data format, no swizzle
  auto issue = [&](int kt, char* kdst, char* vdst) __attribute__((always_inline)) {
    int ln = lane;
    asm volatile("" : "+v"(ln));   // opaque: not hoisted out of the tile loop
    const int ld_c = ln / KPG;
    const int ld_n = (KPG == 8 ? ((ln % KPG) ^ (4 * (ld_c & 1))) : (ln % KPG));
    const int32_t k_lane = ld_n * kst + 16 * ld_c;
    const int32_t v_lane = ld_n * vst + 16 * ld_c;
    const int64_t key0 = int64_t(kt) * KT;
    const __amdgpu_buffer_rsrc_t krs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(kp + key0 * a.ks[2]), 0, k_nrec, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t vrs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(vp + key0 * a.vs[2]), 0, v_nrec, kRsrcWord3);
    if (key0 + KT <= a.kv_end) {
#pragma unroll
      for (int j = 0; j < NLD; ++j) {
        const int grp = j * WAVES + wu;
        if (NG % WAVES != 0 && grp >= NG) break;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_void*)(kdst + grp * T::GROUP_BYTES), 16, k_lane,
                                                 grp * KPG * kst, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_void*)(vdst + grp * T::GROUP_BYTES), 16, v_lane,
                                                 grp * KPG * vst, 0, 0);
      }
    } else {
#pragma unroll
      for (int j = 0; j < NLD; ++j) {
        const int grp = j * WAVES + wu;
        if (NG % WAVES != 0 && grp >= NG) break;
        int32_t n = grp * KPG + ld_n;                       // key - key0
        if (key0 + n >= a.kv_end) n = int32_t(a.kv_end - 1 - key0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_void*)(kdst + grp * T::GROUP_BYTES), 16,
                                                 n * kst + 16 * ld_c, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_void*)(vdst + grp * T::GROUP_BYTES), 16,
                                                 n * vst + 16 * ld_c, 0, 0, 0);
      }
    }
  };

  // per-lane LDS bases: K fragment (key l32, chunk h); V transpose source
  // (key 4*h + s16/4, chunk 2*dh + (s16%4)/2, byte 8*(s16%2))
  const int g = lane >> 4, s16 = lane & 15, dh = g & 1;
  const int k_base = T::offset(l32, h);
  const int v_base = T::offset(4 * h + (s16 >> 2), 2 * dh + ((s16 & 3) >> 1)) + 8 * (s16 & 1);

  // One key tile on LDS buffers (kb_, vb_), in parts of 32 keys, software
  // pipelined inside the wave: for part k the program issues PV(k-1) and the
  // QK^T MFMAs of part k+1 while computing the exponentials of part k, so the
  // MFMA unit has independent work while the VALU runs the softmax; the rare
  // rescale branch comes after.
  // Visibility words of the workgroup's rows for the BN-key class tiles of a
  // partial tile kt: one 16-byte direct load per wave for the first WLOADS
  // waves (two rows per lane), issued with that tile's K/V loads into the same
  // pipeline stage, so the same wait and barrier cover them.  The rows of a
  // class tile are ldw (even) words apart, so every 16-byte unit holds two
  // rows of one class tile; the descriptor ends at the tile's last class
  // tile, and rows past Tq (never stored) read another tile's words or zero.
  constexpr int WROWS = 2 * 64;                       // rows per wave-wide load
  constexpr int WLOADS = (KT / BN) * (BM / WROWS);
  static_assert(BM % WROWS == 0 && WLOADS <= WAVES, "one word load per wave");
  auto issue_words = [&](int kt, uint8_t cls, uint64_t* dst) __attribute__((always_inline)) {
    if (!MASK || kt >= nkt_eff || wu >= WLOADS || cls != kTilePartial) return;
    const int c = wu / (BM / WROWS), r0 = (wu % (BM / WROWS)) * WROWS;
    const int ncls = a.nkt - kt * (KT / BN) < KT / BN ? a.nkt - kt * (KT / BN) : KT / BN;
    if (c >= ncls) return;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint64_t*>(wbase + int64_t(kt) * (KT / BN) * a.ldw), 0, int32_t(ncls * a.ldw * 8), kRsrcWord3);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(dst + c * BM + r0), 16, 16 * lane,
                                             int32_t((c * a.ldw + int64_t(tc.qt) * BM + r0) * 8), 0, 0);
  };
  auto compute = [&](int kt, uint8_t cls, const char* kb_, const char* vb_, const uint64_t* mwl)
                     __attribute__((always_inline)) {
    constexpr int NP = KT / 32;   // parts per tile
    const int64_t key0 = int64_t(kt) * KT;
    const bool edge = (MASK && cls == kTilePartial) || key0 + KT > a.kv_end;
    // visibility words of this lane's rows for the BN-key class tiles of this tile
    // S^T of part kb (keys x queries).  The K fragment (key 32*kb + l32,
    // chunk 2*ks + h) feeds every query block.  Lane (l32, h), register v then
    // holds key 32*kb + 8*(v/4) + 4*h + v%4 of query l32.
    auto load_k = [&](int kb, bf16x8 (&kx)[NKS]) __attribute__((always_inline)) {
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        // offset(32*kb + l32, 2*ks + h) - offset(l32, h) is lane-independent
        kx[ks] = *reinterpret_cast<const bf16x8*>(kb_ + k_base + (T::offset(32 * kb, 2 * ks) - T::offset(0, 0)));
    };
    auto qk_f = [&](const bf16x8 (&kx)[NKS], f32x16 (&sx)[QB]) __attribute__((always_inline)) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) sx[qb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          sx[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kx[ks], qf[qb][ks], sx[qb], 0, 0, 0);
    };
    auto qk = [&](int kb, f32x16 (&sx)[QB]) __attribute__((always_inline)) {
      bf16x8 kx[NKS];
      load_k(kb, kx);
      qk_f(kx, sx);
    };
    // O^T += V^T P^T for part kb.  B element e of lane half h is key
    // 16*j2 + 8*(e/4) + 4*h + e%4 of the part.  The V^T operand takes the same
    // keys through two transpose reads: in each 16-lane group, source lane s
    // addresses key k0 + s/4 at dims n0 + 4*(s%4) .. +3, and lane j receives
    // dim n0 + j of keys k0 .. k0+3 (k0 = 32*kb + 16*j2 + 4*h (+8), n0 = 32*d + 16*dh).
    auto load_v = [&](int kb, bf16x8 (&vx)[NDB][2]) __attribute__((always_inline)) {
#pragma unroll
      for (int d = 0; d < NDB; ++d) {
#pragma unroll
        for (int j2 = 0; j2 < 2; ++j2) {
          constexpr int z = T::offset(0, 0);
          const int o0 = T::offset(32 * kb + 16 * j2, 4 * d) - z;
          const int o1 = T::offset(32 * kb + 16 * j2 + 8, 4 * d) - z;
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vb_ + v_base + o0));
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vb_ + v_base + o1));
          vx[d][j2] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
      }
    };
    auto pv_f = [&](const bf16x8 (&vx)[NDB][2], const bf16x8 (&px)[QB][2]) __attribute__((always_inline)) {
#pragma unroll
      for (int d = 0; d < NDB; ++d)
#pragma unroll
        for (int j2 = 0; j2 < 2; ++j2)
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            oacc[qb][d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vx[d][j2], px[qb][j2], oacc[qb][d], 0, 0, 0);
    };
    auto pv = [&](int kb, const bf16x8 (&px)[QB][2]) __attribute__((always_inline)) {
      bf16x8 vx[NDB][2];
      load_v(kb, vx);
      pv_f(vx, px);
    };

    // p = 2^(c*s - m) for the 32 keys of one lane pair's part, as bf16 B
    // operands; returns this lane's sum of the rounded p (v_dot2 with ones)
    auto exp_part = [&](const f32x16& sx, float m, bf16x8 (&px)[2]) __attribute__((always_inline)) -> float {
      const float nm = -m;
      float sum = 0.f;
#pragma unroll
      for (int j2 = 0; j2 < 2; ++j2) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          px[j2][e] = static_cast<__bf16>(__builtin_amdgcn_exp2f(__builtin_fmaf(sx[8 * j2 + e], a.c, nm)));
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const bf16x2 pair = {px[j2][e], px[j2][e + 1]};
          sum = __builtin_amdgcn_fdot2_f32_bf16(pair, bf16x2{(__bf16)1.0f, (__bf16)1.0f}, sum, false);
        }
      }
      return sum;
    };
    f32x16 s_cur[QB], s_nxt[QB];
    bf16x8 p_prev[QB][2], p_cur[QB][2];
    qk(0, s_cur);
#pragma unroll
    for (int kb = 0; kb < NP; ++kb) {
      if (edge) {
        // visible iff key < kv_end (and its mask bit is set on partial tiles)
        const int room = int(a.kv_end - key0) - 4 * h - 32 * kb;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          // bit 8*(v/4) + v%4 of wsh is register v's key
          const uint32_t wsh =
              MASK ? uint32_t(mwl[(kb / 2) * BM + 32 * QB * w + 32 * qb + l32] >> (32 * (kb & 1) + 4 * h)) : 0u;
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int kofs = 8 * (v >> 2) + (v & 3);
            bool vis = kofs < room;
            if (MASK && cls == kTilePartial) vis = vis && ((wsh >> kofs) & 1u);
            if (!vis) s_cur[qb][v] = -INFINITY;
          }
        }
      }
      // One basic block for the scheduler: PV of the previous part and QK^T of
      // the next part (independent MFMA chains) around the exponentials of this
      // part.  p of this part is computed against the running max and rounded
      // to bf16 (the B operands of PV).
      if (kb > 0) pv(kb - 1, p_prev);
      if (kb + 1 < NP) qk(kb + 1, s_nxt);
      float part[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) part[qb] = exp_part(s_cur[qb], m_run[qb], p_cur[qb]);
      // Every p is <= this lane's sum of the part, so a sum <= kSumLimit proves
      // that no p exceeds it and the running max may stay; otherwise (rare: the
      // first visible keys of a row, or a score far above the running max) raise
      // the max to the part's, rescale what is accumulated (which includes
      // PV of the previous part, issued above), and recompute.
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        if (__ballot(!(part[qb] <= kSumLimit)) != 0) {
          float mx = -INFINITY;
#pragma unroll
          for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s_cur[qb][v]);
          const float m_new = fmaxf(m_run[qb], wave_max_pair(mx) * a.c);
          const float alpha = __builtin_amdgcn_exp2f(m_run[qb] - m_new);
          l_run[qb] *= alpha;
#pragma unroll
          for (int d = 0; d < NDB; ++d) oacc[qb][d] *= alpha;
          m_run[qb] = m_new;
          part[qb] = exp_part(s_cur[qb], m_run[qb], p_cur[qb]);
        }
        l_run[qb] += part[qb];
#pragma unroll
        for (int j2 = 0; j2 < 2; ++j2) p_prev[qb][j2] = p_cur[qb][j2];
        if (kb + 1 < NP) s_cur[qb] = s_nxt[qb];
      }
    }
    pv(NP - 1, p_prev);
  };

  // NBUF-stage pipeline over the tiles, unrolled by NBUF so that every LDS
  // buffer is a constant index (the compiler then knows which buffer each
  // direct load writes and does not wait on them before unrelated LDS reads).
  // Iteration i: wait for tile i's loads, barrier (tile i visible to all waves;
  // every wave done with tile i-1), issue tile i+NBUF-1 into tile i-1's
  // buffer, compute tile i.
  int ahead[NBUF];       // tiles i .. i+NBUF-1
  uint8_t acls[NBUF];    // and their classes
  ahead[0] = next_tile(kt_first - 1, acls[0]);
#pragma unroll
  for (int j = 1; j < NBUF; ++j) ahead[j] = next_tile(ahead[j - 1] < nkt_eff ? ahead[j - 1] : nkt_eff, acls[j]);
  constexpr int MWB = (KT / BN) * BM;   // words per mask-word buffer
  if (ahead[0] < nkt_eff) issue(ahead[0], kbuf(I0{}), vbuf(I0{}));
  issue_words(ahead[0], acls[0], mw_lds);
  if constexpr (NBUF > 2) {
    if (ahead[1] < nkt_eff) issue(ahead[1], kbuf(std::integral_constant<int, 1>{}), vbuf(std::integral_constant<int, 1>{}));
    issue_words(ahead[1], acls[1], mw_lds + MWB);
  }
  auto stage = [&](auto sidx) __attribute__((always_inline)) -> bool {
    constexpr int S = decltype(sidx)::value;
    const int kt = ahead[0];
    const uint8_t cls = kCarryClass ? acls[0] : uint8_t(0);
    if (kt >= nkt_eff) return false;
    // loads still allowed in flight: those of the tiles issued after tile i
    int later = 0;
#pragma unroll
    for (int j = 1; j < NBUF - 1; ++j) later += ahead[j] < nkt_eff;
    if (later == NBUF - 2) wait_vmem<LOADS * (NBUF - 2)>();
    else wait_vmem<0>();
    __syncthreads();
#pragma unroll
    for (int j = 0; j < NBUF - 1; ++j) {
      ahead[j] = ahead[j + 1];
      acls[j] = acls[j + 1];
    }
    ahead[NBUF - 1] = next_tile(ahead[NBUF - 2] < nkt_eff ? ahead[NBUF - 2] : nkt_eff, acls[NBUF - 1]);
    using NX = std::integral_constant<int, (S + NBUF - 1) % NBUF>;
    if (ahead[NBUF - 2] < nkt_eff) issue(ahead[NBUF - 2], kbuf(NX{}), vbuf(NX{}));
    issue_words(ahead[NBUF - 2], kCarryClass ? acls[NBUF - 2] : tile_class(ahead[NBUF - 2]),
                mw_lds + NX::value * MWB);
    if (wave_has_rows) compute(kt, kCarryClass ? cls : tile_class(kt), kbuf(sidx), vbuf(sidx), mw_lds + S * MWB);
    return true;
  };
  for (;;) {
    if (!stage(std::integral_constant<int, 0>{})) break;
    if (!stage(std::integral_constant<int, 1>{})) break;
    if constexpr (NBUF > 2) {
      if (!stage(std::integral_constant<int, 2>{})) break;
    }
  }

  // O^T accumulator: lane (l32, h), register v of block d is dim 32*d + 8*(v/4) + 4*h + v%4.
  // A segment that covers its whole item writes O; a partial one (split
  // launches) writes a record, in slot 2*g if it is the workgroup's first
  // segment, else (it is then the last) in slot 2*g + 1.
  const bool direct = !SPLIT || (BAL ? whole : kt_first == 0 && kt_stop == a.nku);
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lt = l_run[qb] + __shfl_xor(l_run[qb], 32);
    if (!direct) {
      // partial record: O/l rows (bf16), then m and l per row (float32)
      using RL = RecordLayout<D>;
      const int row = 32 * QB * w + 32 * qb + l32;
      char* rec = a.part + int64_t(2 * gl + (seg > 0 ? 1 : 0)) * RL::kBytes;
      if (qvalid[qb]) {
        const float inv = lt > 0.f ? 1.0f / lt : 0.f;
        uint16_t* ro = reinterpret_cast<uint16_t*>(rec + RL::kO) + row * D;
#pragma unroll
        for (int d = 0; d < NDB; ++d)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            bf16x4 ov;
#pragma unroll
            for (int i = 0; i < 4; ++i) ov[i] = static_cast<__bf16>(oacc[qb][d][4 * g4 + i] * inv);
            *reinterpret_cast<bf16x4*>(ro + 32 * d + 8 * g4 + 4 * h) = ov;
          }
        if (h == 0) {
          reinterpret_cast<float*>(rec + RL::kM)[row] = m_run[qb];
          reinterpret_cast<float*>(rec + RL::kL)[row] = lt;
        }
      }
    } else {
      const float inv = lt > 0.f ? 1.0f / lt : 0.f;
      if (qvalid[qb]) {
        uint16_t* orow = op + qrow[qb] * a.os[2];
#pragma unroll
        for (int d = 0; d < NDB; ++d) {
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            bf16x4 ov;
#pragma unroll
            for (int i = 0; i < 4; ++i) ov[i] = static_cast<__bf16>(oacc[qb][d][4 * g4 + i] * inv);
            *reinterpret_cast<bf16x4*>(orow + 32 * d + 8 * g4 + 4 * h) = ov;
          }
        }
      }
    }
  }
  if constexpr (!SPLIT) break;
  }   // segments
}

// Merges the partial records of split launches: for every row of every item
// the ranges ran (items n_direct and on), O = sum_s w_s (O/l)_s / sum_s w_s
// with w_s = 2^(m_s - M) l_s and M = max_s m_s (the running rescale's
// algebra, applied once), 0 where no key was visible.  One workgroup per
// (item, 32 rows); kMergeTpr threads per row, each D / kMergeTpr dims.  The
// records' m values are read first, then each record's weight and O/l, their
// loads independent of the running sums.
constexpr int kMergeTpr = 8;
constexpr int kMergeRows = kThreads / kMergeTpr;   // rows per merge workgroup

template <int D, bool MASK, bool BAL = false>
__global__ __launch_bounds__(kThreads) void attn_combine_kernel(AttnArgs a) {
  using RL = RecordLayout<D>;
  constexpr int BM = kRows<D>;
  constexpr int DPT = D / kMergeTpr;   // dims per thread (16 or 8: two or one 16-byte loads)
  static_assert(DPT % 8 == 0, "whole 16-byte groups of bf16 per thread");
  const uint32_t item = (BAL ? 0u : a.n_direct) + blockIdx.x;
  const int row = blockIdx.y * kMergeRows + int(threadIdx.x) / kMergeTpr;
  const int d0 = (int(threadIdx.x) % kMergeTpr) * DPT;
  const TileCoord tc = decode_item<MASK>(a, item);
  const int64_t qrow = int64_t(tc.qt) * BM + row;
  if (qrow >= a.Tq) return;
  uint16_t* orow = static_cast<uint16_t*>(a.o) + tc.r * a.os[0] + tc.b * a.os[1] + tc.head * a.os[3] + qrow * a.os[2];
  // this item's units [u0, u1) and the units per workgroup; workgroups whose
  // unit ranges meet the item, and the slot of each; an item inside one
  // range was written whole by its workgroup
  int64_t u0, u1, upw;
  if constexpr (BAL) {
    // the balanced split's plan: an item of query block qi has plan_nnz[qi]
    // units; a block without any visible key tile was run by no workgroup,
    // and its rows are 0
    const int32_t nrbh = int32_t(a.nwg / uint32_t(a.nqt));
    const int32_t qi = int32_t(item) / nrbh;
    const int32_t n = a.plan_nnz[qi];
    if (n == 0) {
#pragma unroll
      for (int i = 0; i < DPT; i += 4) *reinterpret_cast<bf16x4*>(orow + d0 + i) = bf16x4{};
      return;
    }
    u0 = a.plan_s[qi] + int64_t(int32_t(item) - qi * nrbh) * (n + kSegmentCost);
    u1 = u0 + n + kSegmentCost;
    upw = 0;
  } else {
    // (units counted from the first range's, n_direct * nku)
    u0 = int64_t(item - a.n_direct) * a.nku;
    u1 = u0 + a.nku;
    upw = a.upw;
  }
  // the workgroup whose range holds unit x, and the first unit of range g
  // (the balanced split's ranges: q = total / W units each, one more for the
  // first rem = total % W)
  const int64_t total = BAL ? a.plan_s[a.nqt] : 0, W = a.split_wgs;
  const int64_t q = BAL ? total / W : upw, rem = BAL ? total - q * W : 0;
  auto wg_of = [&](int64_t x) -> int64_t { return x < rem * (q + 1) ? x / (q + 1) : rem + (x - rem * (q + 1)) / q; };
  auto start_of = [&](int64_t g) -> int64_t { return g * q + (g < rem ? g : rem); };
  // (with the balanced split, the workgroups that ran tiles of the item: a
  // range that ends inside the item's start units ran none)
  const int64_t g_first = wg_of(BAL ? u0 + kSegmentCost : u0), g_last = wg_of(u1 - 1);
  if (g_first == g_last) return;
  auto rec_of = [&](int64_t g) -> const char* {
    const int64_t slot = 2 * g + (start_of(g) < u0 ? 1 : 0);
    return a.part + slot * RL::kBytes;
  };
  float mx = -INFINITY;
  for (int64_t g = g_first; g <= g_last; ++g)
    mx = fmaxf(mx, reinterpret_cast<const float*>(rec_of(g) + RL::kM)[row]);
  float acc[DPT] = {};
  float lsum = 0.f;
#pragma unroll 4
  for (int64_t g = g_first; g <= g_last; ++g) {
    const char* rec = rec_of(g);
    const float wgt = __builtin_amdgcn_exp2f(reinterpret_cast<const float*>(rec + RL::kM)[row] - mx) *
                      reinterpret_cast<const float*>(rec + RL::kL)[row];
    lsum += wgt;
    const uint16_t* ro = reinterpret_cast<const uint16_t*>(rec + RL::kO) + int64_t(row) * D + d0;
#pragma unroll
    for (int i = 0; i < DPT; i += 8) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(ro + i);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[i + 2 * j] += wgt * __uint_as_float(v[j] << 16);
        acc[i + 2 * j + 1] += wgt * __uint_as_float(v[j] & 0xffff0000u);
      }
    }
  }
  const float inv = lsum > 0.f ? 1.0f / lsum : 0.f;
#pragma unroll
  for (int i = 0; i < DPT; i += 4) {
    bf16x4 ov;
#pragma unroll
    for (int j = 0; j < 4; ++j) ov[j] = static_cast<__bf16>(acc[i + j] * inv);
    *reinterpret_cast<bf16x4*>(orow + d0 + i) = ov;
  }
}

// ---------------------------------------------------------------- fp32 kernel

// Element access of the fp32-MFMA kernel: float storage, or bfloat16 storage
// (E = uint16_t bit patterns) widened exactly to float on load and rounded to
// nearest even on store.  The bf16 form serves the head dims the bf16 MFMA
// kernel is not built for (D = 16).
__device__ __forceinline__ float widen(float x) { return x; }
__device__ __forceinline__ float widen(uint16_t x) { return __uint_as_float(uint32_t(x) << 16); }
__device__ __forceinline__ void narrow_store(float* p, float x) { *p = x; }
__device__ __forceinline__ void narrow_store(uint16_t* p, float x) {
  *reinterpret_cast<__bf16*>(p) = static_cast<__bf16>(x);
}
// four consecutive elements (16-byte aligned for float, 8-byte for bf16)
__device__ __forceinline__ void load4(const float* p, float (&o)[4]) {
  const u32x4 v = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = __uint_as_float(v[i]);
}
__device__ __forceinline__ void load4(const uint16_t* p, float (&o)[4]) {
  const uint2 v = *reinterpret_cast<const uint2*>(p);
  o[0] = __uint_as_float(v.x << 16);
  o[1] = __uint_as_float(v.x & 0xffff0000u);
  o[2] = __uint_as_float(v.y << 16);
  o[3] = __uint_as_float(v.y & 0xffff0000u);
}

// Same structure with v_mfma_f32_32x32x2f32: each k-step contracts two values,
// one per lane half.  V needs no transpose (one element per lane per step).
template <int D, bool MASK, typename E>
__global__ __launch_bounds__(kThreads) void attn_f32_kernel(AttnArgs a) {
  static_assert(D % 16 == 0, "f32 path needs D divisible by 16");
  constexpr int KST = D + 1;                 // odd stride: column reads hit distinct banks
  constexpr int VST = D + 4;
  constexpr int NDB = (D + 31) / 32;
  __shared__ float k_lds[BN * KST];
  __shared__ float v_lds[BN * VST];

  const TileCoord tc = decode_item<MASK>(a, MASK ? blockIdx.x : xcd_remap(blockIdx.x, a.nwg));
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, h = lane >> 5;

  const E* qp = static_cast<const E*>(a.q) + tc.r * a.qs[0] + tc.b * a.qs[1] + tc.head * a.qs[3];
  const E* kp = static_cast<const E*>(a.k) + tc.r * a.ks[0] + tc.b * a.ks[1] + tc.head * a.ks[3];
  const E* vp = static_cast<const E*>(a.v) + tc.r * a.vs[0] + tc.b * a.vs[1] + tc.head * a.vs[3];
  E* op = static_cast<E*>(a.o) + tc.r * a.os[0] + tc.b * a.os[1] + tc.head * a.os[3];

  const int64_t qrow = int64_t(tc.qt) * BM32 + w * 32 + l32;
  const bool qvalid = qrow < a.Tq;
  float qf[D / 2];
#pragma unroll
  for (int s = 0; s < D / 2; ++s) qf[s] = qvalid ? widen(qp[qrow * a.qs[2] + 2 * s + h]) : 0.f;

  f32x16 oacc[NDB];
#pragma unroll
  for (int d = 0; d < NDB; ++d) oacc[d] = f32x16{};
  float m_run = -1e30f, l_run = 0.f;

  const uint8_t* cls_row = nullptr;
  const uint8_t* mrow = nullptr;
  if (MASK) {
    const int64_t bm = a.mask_bs ? tc.b : 0;
    // a class tile is kClsRowsF32 rows high: it holds this workgroup's BM32 rows
    cls_row = a.cls + (bm * a.nqt_cls + tc.qt * BM32 / kClsRowsF32) * int64_t(a.nkt);
    mrow = a.mask + tc.b * a.mask_bs + qrow * a.Tk;
  }

  const int nkt_eff = int((a.kv_end + BN - 1) / BN);
  for (int kt = 0; kt < nkt_eff; ++kt) {
    uint8_t cls = kTileFull;
    if (MASK) {
      cls = cls_row[kt];
      if (cls == kTileEmpty) continue;
    }
    const int64_t key0 = int64_t(kt) * BN;
    __syncthreads();
    for (int c = tid; c < BN * D / 4; c += kThreads) {
      const int n = c / (D / 4), dc = c % (D / 4);
      float kv[4] = {0.f, 0.f, 0.f, 0.f}, vv[4] = {0.f, 0.f, 0.f, 0.f};
      if (key0 + n < a.Tk) {
        load4(kp + (key0 + n) * a.ks[2] + 4 * dc, kv);
        load4(vp + (key0 + n) * a.vs[2] + 4 * dc, vv);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        k_lds[n * KST + 4 * dc + i] = kv[i];
        v_lds[n * VST + 4 * dc + i] = vv[i];
      }
    }
    __syncthreads();

    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < D / 2; ++ks)
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x2f32(k_lds[(32 * kb + l32) * KST + 2 * ks + h], qf[ks], s[kb], 0, 0, 0);
    }
    if ((MASK && cls == kTilePartial) || key0 + BN > a.kv_end) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int64_t key = key0 + 32 * kb + 8 * (v >> 2) + 4 * h + (v & 3);
          bool vis = key < a.kv_end;
          if (MASK && cls == kTilePartial && vis) vis = qvalid && mrow[key] != 0;
          if (!vis) s[kb][v] = -INFINITY;
        }
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[kb][v]);
    const float mxc = wave_max_pair(mx) * a.c;
    if (__ballot(mxc > m_run + kRescaleSlack) != 0) {
      const float m_new = fmaxf(m_run, mxc);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int d = 0; d < NDB; ++d) oacc[d] *= alpha;
      m_run = m_new;
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][v], a.c, -m_run));
        l_run += p;
        s[kb][v] = p;
      }
    }
    // O^T += V^T P^T, one key per lane half per step: step (kb, v) contracts key
    // 32*kb + 8*(v/4) + 4*h + v%4 of lane half h.
#pragma unroll
    for (int d = 0; d < NDB; ++d) {
      const int dim = 32 * d + l32;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = 32 * kb + 8 * (v >> 2) + 4 * h + (v & 3);
          const float vval = dim < D ? v_lds[key * VST + dim] : 0.f;
          oacc[d] = __builtin_amdgcn_mfma_f32_32x32x2f32(vval, s[kb][v], oacc[d], 0, 0, 0);
        }
      }
    }
  }

  const float lt = l_run + __shfl_xor(l_run, 32);
  const float inv = lt > 0.f ? 1.0f / lt : 0.f;
  if (qvalid) {
    E* orow = op + qrow * a.os[2];
#pragma unroll
    for (int d = 0; d < NDB; ++d) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dim = 32 * d + 8 * g + 4 * h;
        if (dim < D) {
#pragma unroll
          for (int i = 0; i < 4; ++i) narrow_store(orow + dim + i, oacc[d][4 * g + i] * inv);
        }
      }
    }
  }
}

// ---------------------------------------------------------------- balanced split plan

// Plans a balanced split (see attn_bf16_kernel) from the class map of the
// one mask every item shares: per query block (dispatch order, block qi =
// query tile nqt-1-qi) the count of non-empty key tiles below kv_end, the
// prefix sums of units over the items (an item's units: kSegmentCost, then
// one per non-empty tile), and for each of the split_wgs logical workgroups
// its range of units [u, u_end) with the block, the item of the block and the
// unit of the item that unit u falls on.  One
// workgroup; nqt <= kMaxPlanBlocks <= its threads.
constexpr int kPlanThreads = 512;
static_assert(kMaxPlanBlocks <= kPlanThreads, "one query block per thread in the prefix sum");

__global__ __launch_bounds__(kPlanThreads) void plan_balanced_split_kernel(AttnArgs a) {
  __shared__ int32_t nnz[kMaxPlanBlocks];
  __shared__ int64_t pre[kMaxPlanBlocks];   // inclusive prefix sums of units over the blocks
  const int tid = threadIdx.x;
  const int32_t nqt = a.nqt;
  const int32_t nrbh = int32_t(a.nwg / uint32_t(nqt));
  const int32_t nku = int32_t((a.kv_end + KT - 1) / KT);
  for (int i = tid; i < nqt; i += kPlanThreads) nnz[i] = 0;
  __syncthreads();
  for (int i = tid; i < nqt * nku; i += kPlanThreads) {
    const int qi = i / nku, j = i - qi * nku;
    const uint8_t* row = a.cls + int64_t(nqt - 1 - qi) * a.nkt;
    uint32_t c = row[2 * j];
    if (2 * j + 1 < a.nkt) c |= row[2 * j + 1];
    if (c != kTileEmpty) atomicAdd(&nnz[qi], 1);
  }
  __syncthreads();
  // units of an item: its non-empty tiles plus kSegmentCost for its start
  // (none for an item without a visible tile, which no workgroup runs)
  auto units = [&](int qi) -> int64_t { return nnz[qi] ? nnz[qi] + kSegmentCost : 0; };
  if (tid < nqt) pre[tid] = units(tid) * nrbh;
  __syncthreads();
  for (int off = 1; off < nqt; off *= 2) {
    const int64_t add = tid < nqt && tid >= off ? pre[tid - off] : 0;
    __syncthreads();
    if (tid < nqt) pre[tid] += add;
    __syncthreads();
  }
  const int64_t total = pre[nqt - 1];
  for (int i = tid; i < nqt; i += kPlanThreads) {
    a.plan_nnz[i] = nnz[i];
    a.plan_s[i] = i == 0 ? 0 : pre[i - 1];
  }
  if (tid == 0) a.plan_s[nqt] = total;
  // the first block whose inclusive sum exceeds unit x (it has units, so x
  // lies inside one of its items), the item of the block and x's unit in it
  auto locate = [&](int64_t x, int& blk, int64_t& p, int64_t& k) {
    int lo = 0, hi = nqt - 1;
    while (lo < hi) {
      const int mid = (lo + hi) / 2;
      if (pre[mid] > x) hi = mid; else lo = mid + 1;
    }
    const int64_t within = x - (lo == 0 ? 0 : pre[lo - 1]);
    blk = lo;
    p = within / units(lo);
    k = within - p * units(lo);
  };
  // workgroup g's range: q = total / W units, one more for the first
  // total % W workgroups (W = split_wgs): every workgroup has work when there
  // are W units or more, and any empty ranges come after all units
  for (int g = tid; g < a.split_wgs; g += kPlanThreads) {
    const int64_t q = total / a.split_wgs, rem = total - q * a.split_wgs;
    const int64_t u = g * q + (g < rem ? g : rem);
    int64_t u_end = (g + 1) * q + (g + 1 < rem ? g + 1 : rem);
    int64_t* st = a.plan_start + 4 * int64_t(g);
    int blk;
    int64_t p, k;
    // a range whose last unit is one of an item's start units ends at the
    // item's first unit instead (the next range runs the item)
    if (u < u_end) {
      locate(u_end - 1, blk, p, k);
      if (k < kSegmentCost) u_end = u_end - 1 - k > u ? u_end - 1 - k : u;
    }
    st[0] = u;
    st[1] = u_end;
    st[2] = 0;
    st[3] = 0;
    if (u >= u_end) continue;
    locate(u, blk, p, k);
    st[2] = blk;
    st[3] = (p << 32) | k;
  }
}

// ---------------------------------------------------------------- mask tiles

// One workgroup (16 waves) per (batch, block of `rows` mask rows, kClsSpan
// class tiles of BN keys).  Wave w takes rows w, w + 16, ..., kClsUnroll rows
// at a time (their loads in flight together); on a row, lane l reads the 8
// mask bytes of keys 8l .. 8l+7 of the span (the wave reads 512 contiguous
// bytes of the row) and stores their 8 visibility bits as byte l % 8 of the
// row's word of class tile l / 8 in LDS (bit j of a word = key BN*kt + j).
// The words then go out class tile by class tile, rows contiguous, and a
// class tile is empty, full or partial by the OR / AND of its words (keys
// past Tk count as absent).  Reading whole 512-byte row pieces keeps every
// fetched line in one workgroup: one workgroup per 64-byte class tile made
// neighbouring workgroups (often on other XCDs) fetch the same lines, 2.9x the
// mask bytes from HBM.
constexpr int kClsSpan = 8;          // class tiles per classifier workgroup
constexpr int kClsMaxRows = 384;     // largest class-tile height
constexpr int kClsThreads = 1024;    // classifier workgroup
constexpr int kClsUnroll = 4;        // rows per wave whose loads are in flight together
static_assert(kRows<64> <= kClsMaxRows && kRows<128> <= kClsMaxRows && kClsRowsF32 <= kClsMaxRows,
              "every class-tile height fits the classifier's row stage");

__global__ __launch_bounds__(kClsThreads) void classify_mask_kernel(const uint8_t* mask, int64_t mask_bs, int64_t Tq,
                                                                  int64_t Tk, int32_t nqt, int32_t nkt, uint8_t* cls,
                                                                  uint64_t* bits, int64_t ldw, int32_t rows) {
  static_assert(BN == 64, "one 64-bit word per row and class tile");
  constexpr int kWavesC = kClsThreads / 64;
  __shared__ uint64_t words[kClsSpan * kClsMaxRows];   // [class tile][row]
  __shared__ int any_w[kWavesC], all_w[kWavesC];         // per wave: some word non-zero, every word full
  const int span = blockIdx.x, qt = blockIdx.y;
  const int64_t b = blockIdx.z;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c = lane >> 3;                                   // this lane's class tile in the span
  const int64_t key = (int64_t(span) * kClsSpan + c) * BN + 8 * (lane & 7);   // first of its 8 keys
  const int nv = int(Tk - key <= 0 ? 0 : (Tk - key < 8 ? Tk - key : 8));
  const bool aligned8 = ((reinterpret_cast<uintptr_t>(mask) | uintptr_t(mask_bs) | uintptr_t(Tk)) & 7) == 0;
  const int64_t left = Tq - int64_t(qt) * rows;
  const int nrows = int(left < rows ? left : rows);
  uint8_t* wbytes = reinterpret_cast<uint8_t*>(words);
  const uint8_t* base = mask + b * mask_bs + int64_t(qt) * rows * Tk + key;
  for (int r0 = w; r0 < nrows; r0 += kWavesC * kClsUnroll) {
    uint64_t x[kClsUnroll];
#pragma unroll
    for (int u = 0; u < kClsUnroll; ++u) {
      const int r = r0 + u * kWavesC;
      x[u] = 0;
      if (r < nrows) {
        const uint8_t* p = base + int64_t(r) * Tk;
        if (nv == 8 && aligned8) {
          x[u] = *reinterpret_cast<const uint64_t*>(p);
        } else {
          for (int i = 0; i < nv; ++i) x[u] |= uint64_t(p[i]) << (8 * i);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kClsUnroll; ++u) {
      const int r = r0 + u * kWavesC;
      if (r < nrows) wbytes[(c * kClsMaxRows + r) * 8 + (lane & 7)] = uint8_t(nonzero_bytes_to_bits8(x[u]));
    }
  }
  __syncthreads();
  // Words out, rows contiguous per class tile: waves kWavesPerTile*ci ..
  // take class tile ci, each wave 64 consecutive rows per store (512
  // contiguous bytes), and fold its words into the tile's class with two
  // ballots (a per-thread row index divided by nrows, and a flag store from
  // every lane, had made this phase longer than reading the mask).
  constexpr int kWavesPerTile = kWavesC / kClsSpan;
  static_assert(kWavesC % kClsSpan == 0, "whole waves per class tile");
  {
    const int ci = w / kWavesPerTile;
    const int cti = span * kClsSpan + ci;
    bool any = false, all = true;
    if (cti < nkt) {
      const int64_t n = Tk - int64_t(cti) * BN < BN ? Tk - int64_t(cti) * BN : BN;   // in-range keys
      const uint64_t full = n >= 64 ? ~0ull : ((1ull << n) - 1);
      uint64_t* dst = bits + (b * nkt + cti) * ldw + int64_t(qt) * rows;
      for (int r = (w % kWavesPerTile) * 64 + lane; r < nrows; r += 64 * kWavesPerTile) {
        const uint64_t word = words[ci * kClsMaxRows + r];
        dst[r] = word;
        any = any || word != 0;
        all = all && word == full;
      }
    }
    const bool wave_any = __ballot(any) != 0, wave_all = __ballot(!all) == 0;
    if (lane == 0) {
      any_w[w] = wave_any;
      all_w[w] = wave_all;
    }
  }
  __syncthreads();
  if (threadIdx.x < kClsSpan && span * kClsSpan + int(threadIdx.x) < nkt) {
    bool any = false, all = true;
#pragma unroll
    for (int j = 0; j < kWavesPerTile; ++j) {
      any = any || any_w[threadIdx.x * kWavesPerTile + j];
      all = all && all_w[threadIdx.x * kWavesPerTile + j];
    }
    cls[(b * nqt + qt) * int64_t(nkt) + span * kClsSpan + threadIdx.x] =
        !any ? kTileEmpty : (all ? kTileFull : kTilePartial);
  }
}

int64_t div_up(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool nonneg(const sp_attn_strides& s) { return s.rank >= 0 && s.batch >= 0 && s.token >= 0 && s.head >= 0; }

bool multiple_of(const sp_attn_strides& s, int64_t m) {
  return s.rank % m == 0 && s.batch % m == 0 && s.token % m == 0 && s.head % m == 0;
}

// Byte extent [base, base + span) reached through a strided view.
int64_t span_bytes(const sp_attn_strides& s, int64_t R, int64_t B, int64_t T, int64_t H, int64_t D, int64_t eb) {
  return ((R - 1) * s.rank + (B - 1) * s.batch + (T - 1) * s.token + (H - 1) * s.head + D) * eb;
}

bool overlap(const void* a, int64_t na, const void* b, int64_t nb) {
  const char* x = static_cast<const char*>(a);
  const char* y = static_cast<const char*>(b);
  return x < y + nb && y < x + na;
}

// The bf16 MFMA kernel is built for D = 64 and 128; bf16 at D = 16 runs the
// fp32-MFMA kernel on widened values (exact products, float32 accumulation).
bool bf16_mfma_kernel(sp_dtype dt, int32_t D) { return dt == SP_BF16 && (D == 64 || D == 128); }

template <int D, bool MASK>
void launch_attn(const AttnArgs& a, sp_dtype dt, bool narrow, hipStream_t s) {
  if (bf16_mfma_kernel(dt, D)) {
    if constexpr (D % 32 == 0) {
      if (a.part && a.split_wgs > 0) {
        if constexpr (MASK && D == 128) {
          hipLaunchKernelGGL(plan_balanced_split_kernel, dim3(1), dim3(kPlanThreads), 0, s, a);
          hipLaunchKernelGGL((attn_bf16_kernel<D, true, true, true>), dim3(unsigned(a.split_wgs)),
                             dim3(64 * kWaves<D>), 0, s, a);
          hipLaunchKernelGGL((attn_combine_kernel<D, true, true>), dim3(a.nwg, kRows<D> / kMergeRows), dim3(kThreads),
                             0, s, a);
        }
      } else if (a.part) {
        hipLaunchKernelGGL((attn_bf16_kernel<D, MASK, true>),
                           dim3(a.n_direct + unsigned((a.units - int64_t(a.n_direct) * a.nku + a.upw - 1) / a.upw)),
                           dim3(64 * kWaves<D>), 0, s, a);
        hipLaunchKernelGGL((attn_combine_kernel<D, MASK>), dim3(a.nwg - a.n_direct, kRows<D> / kMergeRows),
                           dim3(kThreads), 0, s, a);
      } else if (narrow) {
        if constexpr (D == 64 && !MASK)
          hipLaunchKernelGGL((attn_bf16_kernel<D, false, false, false, kNarrowWaves64>), dim3(a.nwg),
                             dim3(64 * kNarrowWaves64), 0, s, a);
      } else {
        hipLaunchKernelGGL((attn_bf16_kernel<D, MASK, false>), dim3(a.nwg), dim3(64 * kWaves<D>), 0, s, a);
      }
    }
  } else if (dt == SP_BF16) {
    hipLaunchKernelGGL((attn_f32_kernel<D, MASK, uint16_t>), dim3(a.nwg), dim3(kThreads), 0, s, a);
  } else {
    hipLaunchKernelGGL((attn_f32_kernel<D, MASK, float>), dim3(a.nwg), dim3(kThreads), 0, s, a);
  }
}

template <bool MASK>
sp_status dispatch_d(int D, const AttnArgs& a, sp_dtype dt, bool narrow, hipStream_t s) {
  switch (D) {
    case 16: launch_attn<16, MASK>(a, dt, narrow, s); break;
    case 64: launch_attn<64, MASK>(a, dt, narrow, s); break;
    case 128: launch_attn<128, MASK>(a, dt, narrow, s); break;
    default: return SP_ERR_UNSUPPORTED;
  }
  return launch_status();
}

}  // namespace
}  // namespace sp

using namespace sp;

// Compute units of the current device (256 on MI355X; also the default when no
// device can be queried).
int64_t device_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      n <= 0) {
    (void)hipGetLastError();
    return 256;
  }
  return n;
}

// Split decision for the bf16 kernel, per CU, with `items` query tiles of
// nku key tiles each.  Without a user mask the whole rounds of a plain
// launch, floor(items / ncu) * ncu items, run as they would there (dispatched
// first, one workgroup per item), and only the rest, `tail` items, can be
// split: a plain launch runs them in one more round of nku tile-times, a
// split in ranges of upw = ceil(tail * nku / ncu) key tiles plus a fixed
// cost for the partial records and the merge launch, about 4 tile-times at
// D = 128 and twice that at D = 64 (a tile costs half as much; measured on
// MI355X: ~4-5 us per tile-time at D = 128, ~15 us of fixed cost).  With a
// user mask the units differ in cost (empty tiles are free): no items run
// whole, and ranges stay shorter than an item (at most two segments), where
// the split still bounds the critical path.  The split runs when it pays by
// 1.1x: the model overprices a plain launch's partly filled round (its CUs
// then run faster).
struct SplitPlan {
  int64_t upw = 0;        // key tiles per range; 0: no split
  int64_t n_direct = 0;   // items run whole before the ranges
};
SplitPlan split_plan(int64_t items, int64_t nku, int64_t ncu, int32_t D, bool masked) {
  SplitPlan p;
  if (items <= 0 || nku < 2 || ncu <= 0) return p;
  const int64_t nd = masked ? 0 : items / ncu * ncu;
  const int64_t tail = items - nd;
  if (tail == 0) return p;
  const int64_t upw = div_up(tail * nku, ncu);
  if (masked && upw >= nku) return p;
  const int64_t plain = div_up(tail, ncu) * nku;
  const int64_t fixed = 4 * 128 / D;
  if (plain * 10 >= (upw + fixed) * 11) {
    p.upw = upw;
    p.n_direct = nd;
  }
  return p;
}

// query rows per workgroup of the bf16 kernel for head dim D (64 or 128)
int64_t bf16_rows(int32_t D) { return D == 64 ? kRows<64> : kRows<128>; }

// query rows per workgroup of the kernel a launch runs
int64_t kernel_rows(sp_dtype dtype, int32_t D) { return bf16_mfma_kernel(dtype, D) ? bf16_rows(D) : BM32; }

// height of the mask-class tiles of a launch: the bf16 kernel's query tile,
// or kClsRowsF32 for the fp32-MFMA kernel
int64_t cls_rows(sp_dtype dtype, int32_t D) { return bf16_mfma_kernel(dtype, D) ? bf16_rows(D) : kClsRowsF32; }

// bytes of partial records of a split launch: two slots per workgroup
int64_t split_bytes(int64_t ncu, int32_t D) {
  return 2 * ncu * (D == 64 ? RecordLayout<64>::kBytes : RecordLayout<128>::kBytes);
}

// bytes of the class part of the workspace: one class byte per (class tile
// rows x BN) tile, padded to 256 bytes
int64_t cls_ws_bytes(int64_t bm, int64_t Tq, int64_t Tk, int64_t rows) {
  return (bm * div_up(Tq, rows) * div_up(Tk, BN) + 255) / 256 * 256;
}

// Bytes of the mask part of the workspace (class bytes, then one 64-bit
// visibility word per mask row (Tq rounded up to even) and BN-key tile); 0
// without a mask.
int64_t mask_ws_bytes(int64_t B, int64_t Tq, int64_t Tk, bool has_mask, int64_t mask_batch_stride, int64_t rows) {
  if (!has_mask) return 0;
  const int64_t bm = mask_batch_stride ? B : 1;
  return cls_ws_bytes(bm, Tq, Tk, rows) + bm * div_up(Tq, 2) * 2 * div_up(Tk, BN) * 8;
}

// A masked split launch cuts its ranges in non-empty key tiles (the balanced
// split) when the kernel can plan them: D = 128, one mask for every batch (or
// one batch), at most kMaxPlanBlocks query blocks.
bool balanced_split(bool has_mask, int32_t D, int64_t mask_batch_stride, int64_t B, int64_t nqt) {
  return has_mask && D == 128 && (mask_batch_stride == 0 || B == 1) && nqt <= kMaxPlanBlocks;
}

// The balanced split's plan: prefix sums (nqt + 1 int64), counts (nqt int32),
// then four int64 per workgroup (its start); 256-byte aligned in all.
int64_t plan_counts_at(int64_t nqt) { return (nqt + 1) * 8; }
int64_t plan_starts_at(int64_t nqt) { return (plan_counts_at(nqt) + nqt * 4 + 7) / 8 * 8; }
int64_t plan_bytes(int64_t nqt, int64_t wgs) { return (plan_starts_at(nqt) + wgs * 32 + 255) / 256 * 256; }

extern "C" size_t sp_masked_attention_workspace_size(int32_t R, int64_t B, int64_t Tq, int64_t Tk, int32_t Hl,
                                                     int32_t D, sp_dtype dtype, int32_t has_mask,
                                                     int64_t mask_batch_stride) {
  if (R <= 0 || B <= 0 || Tq <= 0 || Tk <= 0 || Hl <= 0) return 0;
  // [mask classes and words][a balanced split's plan][partial records of a
  // split launch], each part 256-byte aligned; the split part is sized for
  // kv_valid_len = Tk (a shorter key range needs no more)
  const int64_t mask_bytes = mask_ws_bytes(B, Tq, Tk, has_mask != 0, mask_batch_stride, cls_rows(dtype, D));
  int64_t split = 0;
  if (bf16_mfma_kernel(dtype, D)) {
    const int64_t ncu = device_cus();
    const int64_t nqt = div_up(Tq, bf16_rows(D));
    const int64_t items = nqt * Hl * B * R;
    if (split_plan(items, div_up(Tk, KT), ncu, D, has_mask != 0).upw) {
      split = split_bytes(ncu, D);
      if (balanced_split(has_mask != 0, D, mask_batch_stride, B, nqt)) split += plan_bytes(nqt, ncu);
    }
  }
  return size_t(split ? (mask_bytes + 255) / 256 * 256 + split : mask_bytes);
}

namespace {

// One attention call after the host-side checks: the launch arguments and
// what the launch needs from the workspace.  Built without any HIP call.
struct AttnCall {
  AttnArgs a;
  sp_dtype dtype;
  int32_t D;
  bool empty;          // nothing to compute (a size is 0)
  bool has_mask;
  int64_t mask_bytes;  // class bytes and visibility words (0 without a mask)
  int64_t crows;       // class-tile height
  int64_t nqt_cls, nkt, nwg;
  int64_t bm;          // masks in the workspace: B per-batch masks, or 1 shared
};

// Every check of sp_masked_attention that does not concern the workspace.
sp_status attn_check(const void* q, sp_attn_strides qs, const void* k, sp_attn_strides ks, const void* v,
                     sp_attn_strides vs, void* o, sp_attn_strides os, int32_t R, int64_t B, int64_t Tq, int64_t Tk,
                     int32_t Hl, int32_t D, sp_dtype dtype, int64_t kv_valid_len, const uint8_t* mask,
                     int64_t mask_batch_stride, float scale, AttnCall& c) {
  if (!dtype_ok(dtype)) return SP_ERR_INVALID_ARG;
  if (R < 0 || B < 0 || Tq < 0 || Tk < 0 || Hl < 0 || kv_valid_len < 0 || mask_batch_stride < 0)
    return SP_ERR_INVALID_ARG;
  if (!(D == 16 || D == 64 || D == 128)) return SP_ERR_UNSUPPORTED;
  // The kernels hide a key by setting its raw score q.k to -inf and take the
  // row maximum of raw scores before multiplying by scale * log2(e): both are
  // right only for a positive factor, and a zero or denormal factor would turn
  // -inf * 0 into NaN.  The softmax scale of the path is 1/sqrt(D).
  const float c2 = scale * 1.4426950408889634f;
  if (!std::isfinite(scale) || !(scale > 0.f) || !std::isnormal(c2) || !std::isnormal(scale)) return SP_ERR_INVALID_ARG;
  c.empty = R == 0 || B == 0 || Tq == 0 || Hl == 0;
  if (c.empty) return SP_OK;
  if (!q || !k || !v || !o) return SP_ERR_INVALID_ARG;
  if (!nonneg(qs) || !nonneg(ks) || !nonneg(vs) || !nonneg(os)) return SP_ERR_INVALID_ARG;
  const int64_t eb = elem_bytes(dtype);
  const int64_t vec = 16 / eb;   // elements per 16-byte group
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return SP_ERR_INVALID_ARG;
  if (!multiple_of(qs, vec) || !multiple_of(ks, vec) || !multiple_of(vs, vec) || !multiple_of(os, vec))
    return SP_ERR_INVALID_ARG;
  const int64_t tk1 = Tk > 0 ? Tk : 1;
  const int64_t on = span_bytes(os, R, B, Tq, Hl, D, eb);
  if (overlap(o, on, q, span_bytes(qs, R, B, Tq, Hl, D, eb)) || overlap(o, on, k, span_bytes(ks, R, B, tk1, Hl, D, eb)) ||
      overlap(o, on, v, span_bytes(vs, R, B, tk1, Hl, D, eb)))
    return SP_ERR_INVALID_ARG;
  const bool mfma16 = bf16_mfma_kernel(dtype, D);
  const int64_t crows = cls_rows(dtype, D);
  const int64_t nqt = div_up(Tq, kernel_rows(dtype, D)), nkt = div_up(Tk, BN);
  const int64_t nqt_cls = div_up(Tq, crows);
  const int64_t nwg = nqt * Hl * B * R;
  if (nwg >= (int64_t(1) << 31) || nkt >= (int64_t(1) << 31)) return SP_ERR_UNSUPPORTED;
  // the bf16 kernel addresses one key tile of K and of V with 32-bit byte offsets
  if (mfma16 && ((KT - 1) * (ks.token > vs.token ? ks.token : vs.token) + D) * eb >= (int64_t(1) << 31))
    return SP_ERR_UNSUPPORTED;
  const bool has_mask = mask != nullptr && Tk > 0;
  if (mfma16 && has_mask && nkt > kMaxClassTiles) return SP_ERR_UNSUPPORTED;
  // (grid limits; nqt_cls also keeps the visibility-word offsets, below
  // 2 * 8 * ldw bytes, inside 32 bits)
  if (has_mask && (B > 65535 || nqt_cls > 65535)) return SP_ERR_UNSUPPORTED;

  AttnArgs& a = c.a;
  a.q = q; a.k = k; a.v = v; a.o = o;
  const sp_attn_strides* src[4] = {&qs, &ks, &vs, &os};
  int64_t* dst[4] = {a.qs, a.ks, a.vs, a.os};
  for (int i = 0; i < 4; ++i) {
    dst[i][0] = src[i]->rank; dst[i][1] = src[i]->batch; dst[i][2] = src[i]->token; dst[i][3] = src[i]->head;
  }
  a.B = B; a.Tq = Tq; a.Tk = Tk; a.Hl = Hl;
  a.kv_end = kv_valid_len < Tk ? kv_valid_len : Tk;
  a.mask = mask; a.mask_bs = mask_batch_stride;
  a.cls = nullptr; a.bits = nullptr;
  a.ldw = div_up(Tq, 2) * 2;
  a.nqt = int32_t(nqt); a.nkt = int32_t(nkt); a.nqt_cls = int32_t(nqt_cls);
  a.c = c2;
  a.nwg = uint32_t(nwg);
  a.units = 0; a.upw = 0; a.nku = 0; a.n_direct = 0; a.part = nullptr;
  a.split_wgs = 0; a.plan_nnz = nullptr; a.plan_s = nullptr; a.plan_start = nullptr;
  c.dtype = dtype;
  c.D = D;
  c.has_mask = has_mask;
  c.crows = crows;
  c.nqt_cls = nqt_cls;
  c.nkt = nkt;
  c.nwg = nwg;
  c.bm = mask_batch_stride ? B : 1;
  c.mask_bytes = mask_ws_bytes(B, Tq, Tk, has_mask, mask_batch_stride, crows);
  return SP_OK;
}

// Checks the workspace, decides the split and launches: the mask classifier
// (with a user mask), then the attention kernel (and the merge of a split
// launch).
sp_status attn_run(AttnCall& c, void* workspace, size_t workspace_bytes, hipStream_t s) {
  AttnArgs& a = c.a;
  if (c.has_mask && (workspace == nullptr || workspace_bytes < size_t(c.mask_bytes))) return SP_ERR_INVALID_ARG;
  if (c.has_mask && (reinterpret_cast<uintptr_t>(workspace) & 255) != 0) return SP_ERR_INVALID_ARG;
  a.cls = static_cast<const uint8_t*>(workspace);
  a.bits = c.has_mask ? reinterpret_cast<const uint64_t*>(static_cast<const char*>(workspace) +
                                                          cls_ws_bytes(c.bm, a.Tq, a.Tk, c.crows))
                      : nullptr;
  bool narrow = false;
  if (bf16_mfma_kernel(c.dtype, c.D)) {
    const int64_t ncu = device_cus();
    const int64_t nku = div_up(a.kv_end, KT);
    const SplitPlan sp = split_plan(c.nwg, nku, ncu, c.D, c.has_mask);
    const int64_t upw = sp.upw;
    // the split runs only with room for its partial records after the mask
    // part (as sized by sp_masked_attention_workspace_size); otherwise the
    // plain launch runs
    const bool bal = balanced_split(c.has_mask, c.D, a.mask_bs, a.B, a.nqt);
    const int64_t plan_at = (c.mask_bytes + 255) / 256 * 256;
    const int64_t part_at = plan_at + (bal ? plan_bytes(a.nqt, ncu) : 0);
    if (upw && workspace && workspace_bytes >= size_t(part_at + split_bytes(ncu, c.D)) &&
        (reinterpret_cast<uintptr_t>(workspace) & 255) == 0) {
      a.n_direct = uint32_t(sp.n_direct);
      a.units = c.nwg * nku; a.upw = upw; a.nku = int32_t(nku);
      a.part = static_cast<char*>(workspace) + part_at;
      if (bal) {
        // one range of non-empty key tiles per compute unit, planned on the device
        a.split_wgs = int32_t(ncu);
        char* plan = static_cast<char*>(workspace) + plan_at;
        a.plan_s = reinterpret_cast<int64_t*>(plan);
        a.plan_nnz = reinterpret_cast<int32_t*>(plan + plan_counts_at(a.nqt));
        a.plan_start = reinterpret_cast<int64_t*>(plan + plan_starts_at(a.nqt));
      }
    }
    // an unsplit D = 64 launch without a user mask whose items fill at most
    // one of each CU's two workgroup slots: 4-wave workgroups of 128 rows
    if (c.D == 64 && !c.has_mask && a.part == nullptr && c.nwg <= ncu) {
      narrow = true;
      const int64_t per_tile = c.nwg / a.nqt;   // items per query tile: R * B * Hl
      a.nqt = int32_t(div_up(a.Tq, 32 * QB * kNarrowWaves64));
      a.nwg = uint32_t(per_tile * a.nqt);
    }
  }
  if (c.has_mask) {
    hipLaunchKernelGGL(classify_mask_kernel, dim3(unsigned(div_up(c.nkt, kClsSpan)), unsigned(c.nqt_cls), unsigned(c.bm)),
                       dim3(kClsThreads), 0,
                       s, a.mask, a.mask_bs, a.Tq, a.Tk, int32_t(c.nqt_cls), int32_t(c.nkt),
                       static_cast<uint8_t*>(workspace), const_cast<uint64_t*>(a.bits), a.ldw, int32_t(c.crows));
    if (launch_status() != SP_OK) return SP_ERR_HIP;
    return dispatch_d<true>(c.D, a, c.dtype, narrow, s);
  }
  return dispatch_d<false>(c.D, a, c.dtype, narrow, s);
}

}  // namespace

extern "C" sp_status sp_masked_attention(const void* q, sp_attn_strides qs, const void* k, sp_attn_strides ks,
                                         const void* v, sp_attn_strides vs, void* o, sp_attn_strides os,
                                         int32_t R, int64_t B, int64_t Tq, int64_t Tk, int32_t Hl, int32_t D,
                                         sp_dtype dtype, int64_t kv_valid_len, const uint8_t* mask,
                                         int64_t mask_batch_stride, float scale, void* workspace,
                                         size_t workspace_bytes, void* stream) {
  AttnCall c;
  const sp_status st = attn_check(q, qs, k, ks, v, vs, o, os, R, B, Tq, Tk, Hl, D, dtype, kv_valid_len, mask,
                                  mask_batch_stride, scale, c);
  if (st != SP_OK || c.empty) return st;
  return attn_run(c, workspace, workspace_bytes, as_stream(stream));
}

// ---------------------------------------------------------------- no-allocation entry point

// The workspace of sp_masked_attention_noalloc: a fixed array in device
// memory, one per GPU (each device that loads the library holds its own copy
// until the process ends).  In host code `scratch` names a host-side stand-in,
// not device memory: its device address comes from hipGetSymbolAddress, taken
// once per device with that device current, and only that address is ever
// handed to a kernel.  Nothing in it needs to start at zero: the mask
// classifier writes every class byte and visibility word a launch reads, and
// a split launch writes every partial record its merge reads.
static __device__ __align__(256) unsigned char scratch[SP_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of the current device's scratch array.
sp_status scratch_ptr(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return SP_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return SP_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return SP_ERR_HIP;
    }
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return SP_OK;
}
}  // namespace

extern "C" sp_status sp_masked_attention_noalloc(const void* q, sp_attn_strides qs, const void* k, sp_attn_strides ks,
                                                 const void* v, sp_attn_strides vs, void* o, sp_attn_strides os,
                                                 int32_t R, int64_t B, int64_t Tq, int64_t Tk, int32_t Hl, int32_t D,
                                                 sp_dtype dtype, int64_t kv_valid_len, const uint8_t* mask,
                                                 int64_t mask_batch_stride, float scale, void* stream) {
  AttnCall c;
  const sp_status st = attn_check(q, qs, k, ks, v, vs, o, os, R, B, Tq, Tk, Hl, D, dtype, kv_valid_len, mask,
                                  mask_batch_stride, scale, c);
  if (st != SP_OK || c.empty) return st;
  // the same workspace as sp_masked_attention would be given (the size query's
  // bytes), so both entry points take the same launch decisions
  const size_t need = sp_masked_attention_workspace_size(R, B, Tq, Tk, Hl, D, dtype, mask != nullptr ? 1 : 0,
                                                         mask_batch_stride);
  if (need > size_t(SP_NOALLOC_SCRATCH_BYTES)) return SP_ERR_SCRATCH;
  void* ws = nullptr;
  if (need > 0) {
    const sp_status sst = scratch_ptr(&ws);
    if (sst != SP_OK) return sst;
  }
  return attn_run(c, ws, need, as_stream(stream));
}
