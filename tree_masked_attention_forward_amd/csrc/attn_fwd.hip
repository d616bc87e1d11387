// Tree attention forward on gfx950, bf16 inputs, head size 128.
//
// What is computed ("Tree Attention", inferensys.com glossary, Modified Causal
// Attention Mask and Speculative KV Cache Reuse; "Tree Attention",
// zhongzhoutan-coder.github.io, How It Works): node i of sequence b, query
// head h, attends to all L_b prefix keys of KV head g = h / G, to itself and
// to its ancestors; softmax(scale * q.k) weights the matching values.
//
// Layout of the work.  For one (sequence, KV head) the N_b nodes times the G
// query heads that share the KV head form a dense block of N_b*G query rows
// (row = node*G + j), so every key/value row fetched from HBM is used by all
// of them and the key scan is a dense contraction on MFMA.  A sequence's key
// axis is [prefix, padded to 32 | tree nodes] in 32-key tiles; prefix tiles
// need no mask; a tree tile tests the row node's ancestor bits (one uint64
// word per 64 nodes); tiles past a row tile's last node are never visited
// because nodes are topologically ordered.
//
// Workgroup = RG row groups x KG key groups of one wave each.  A wave owns 32
// query rows; the KG waves that share those rows take alternate tiles of the
// workgroup's key range, and are merged through LDS at the end.  Grid items
// are (sequence, key split, KV head, row tile), row tile fastest; splits cut
// the tile range in balanced pieces (the tree tiles ride with the last prefix
// tiles).  Each XCD runs a contiguous run of item ids: the row tiles that
// share a KV chunk read it once from HBM and once from that XCD's L2, and the
// XCD streams whole key rows (all KV heads) of one key range.  Ragged batches
// (one row tile, at most 64 sequences) instead cut every sequence into pieces
// of about equal length that workgroups take longest first, so the XCDs get
// equal shares (lpt_piece).
//
// Per 32-key tile and wave:
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (A = K rows from LDS, B = Q^T
//     held in registers for the whole kernel): each lane holds 16 keys of ONE
//     query row and lane^32 holds the other 16, so the row max is one
//     cross-lane step (v_permlane32_swap) and the output rescale is one
//     factor per lane;
//   * online softmax in fp32 in the log2 domain (scale*log2(e) folded into one
//     FMA before v_exp_f32); the running max is lazy (it moves only when a
//     tile exceeds it by 2^8), so the 64-register rescale of O is rare;
//   * O^T += V^T P^T on the same MFMA: B = P^T comes straight from the score
//     registers (rounded to bf16), A = V^T is read from the row-major V tile
//     with ds_read_b64_tr_b16, whose 16-lane 4x16 transpose hands each lane
//     four consecutive keys of one head dimension.
// K and V tiles (and, ahead of the first stage, the query rows) are staged
// through LDS with direct 16-byte global->LDS loads in a three-stage ring, one
// barrier per stage.  Items with one split write bf16 output (and lse)
// directly; otherwise each leaves its normalised O (bf16) and running max and
// sum (fp32) in the workspace, in the MFMA register layout so every store is
// coalesced, and the splits are combined by log-sum-exp: by merge workgroups
// at the end of the same grid when there are few groups (see
// merge_in_kernel; items then run head-major, so a group's splits share an
// XCD), else by a separate merge kernel.
//
// Mask bits: a tree tile's 32-bit mask half per lane rides in the stage, or,
// for trees of up to 128 nodes (MR), each lane keeps its node's whole row in
// registers.  With MR the kernel can also build those rows itself from the
// parent array (tree_attn_mask_and_forward: the node and its parent chain,
// the same relation as the separate mask builder) while its first tiles load.
// A sequence's prefix is the range prefix_offsets[b] .. [b+1], or the first
// prefix_lens[b] rows of it when the prefix is a cache slot.
#include "internal.h"

#include <math.h>

#include <algorithm>
#include <type_traits>

namespace ta {

// Timeline build (TA_TIMELINE defined: libtreeattn_timeline.so, a measurement
// tool that `bench.py --timeline` loads; the product library has no trace
// code).  Thread 0 of each workgroup of the forward kernel stamps
// s_memrealtime (a 100 MHz counter) into 16 slots per workgroup:
//   0 start, 1 offsets decoded, 2 first stage in LDS, 3 key loop done,
//   4 arrival issued (split) or group seen complete (merge), 5 end,
//   6 kind (1 split, 2 merge) | XCD << 8, 7 partial stores issued,
//   14 key tiles walked | sequence << 16 | KV head << 24 | split << 32,
//   15 HW_REG_HW_ID.
#ifdef TA_TIMELINE
__device__ unsigned long long* g_timeline = nullptr;
__device__ long long g_timeline_cap = 0;
#define TA_TL(slot, value)                                                              \
  do {                                                                                \
    if (g_timeline && threadIdx.x == 0 && (long long)blockIdx.x < g_timeline_cap)     \
      g_timeline[(long long)blockIdx.x * 16 + (slot)] = (unsigned long long)(value);  \
  } while (0)
#define TA_TL_NOW() __builtin_amdgcn_s_memrealtime()
#else
#define TA_TL(slot, value) ((void)0)
#endif

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));

constexpr int kD = 128;                       // head size of the MFMA path
constexpr int kKT = 32;                       // keys per tile
constexpr int kRow = kD * 2;                  // LDS bytes per K or V row (unpadded, chunks swizzled)
constexpr int kTileKV = kKT * kRow;           // 8192: one K or one V tile
constexpr int kTileBytes = 2 * kTileKV;       // K tile then V tile
constexpr int kLdsMax = 160 * 1024;           // LDS per workgroup on gfx950
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_inff();
constexpr float kLazyLog2 = 8.f;              // running-max slack: probabilities stay <= 256
// Split partials are stored in fp16 scaled by a power of two per row, chosen
// so that the row's largest possible value lies in [2^kPartialExp, 2^(kPartialExp+1)):
// 11 significant bits (rounding error at most 2^-11 of the value) and a
// factor of four below fp16's largest finite value.
constexpr int kPartialExp = 13;

struct KParams {
  const uint16_t* q;
  const uint16_t* k_tree;
  const uint16_t* v_tree;
  const uint16_t* k_prefix;
  const uint16_t* v_prefix;
  const int64_t* prefix_offsets;
  const int64_t* prefix_lens;   // nullable: rows in use of each prefix slot
  const int32_t* node_offsets;
  const uint64_t* mask;      // ancestor rows (null when the kernel builds them)
  uint16_t* out;
  float* lse;
  // Mask built in the kernel (tree_attn_mask_and_forward): parents in, rows,
  // depths and per-sequence status out.
  const int32_t* parents;
  uint64_t* mask_out;
  int32_t* depth_out;
  int32_t* status_out;
  int build;
  u32x2_t* ws_o;   // [n_items][RG][16][64] 4 x fp16: 2^k O / l in register layout
  float2* ws_ml;   // [n_items][rows_wg]   running max (score units), sum carrying k
  // In-kernel merge: per (sequence, KV head, row tile) group, four words
  // (arrivals, arrival tags, epoch, merge workgroups done; see
  // merge_in_kernel), and the call status word; null when a separate merge
  // kernel combines the splits.
  unsigned long long* cnt;
  unsigned int* merge_status;
  long long total_prefix, max_prefix, n_items;
  long long n_split_blocks;   // workgroups [0, n_split_blocks) run splits
  int merge_wpg;              // merge workgroups per group (in-kernel merge)
  long long groups;           // B * Hkv * R (sequence, KV head, row tile) groups
  int head_major;             // item order: (b, g, s, r) if set, else (b, s, g, r)
  int piece;                  // > 0: a sequence takes ceil(T / piece) splits (ragged batches)
  int lpt;                    // workgroups take the pieces longest first (see lpt_piece)
  int total_nodes, max_nodes;
  int B, Hq, Hkv, G, W;
  int rows_wg, R, S, tmax;
  float scale, scale_log2;
};

// One sequence's extents, every offset checked against the host sizes so a
// malformed offset array can never send a load out of bounds.
struct Seq {
  int n0, nn, L;
  long long p0;
};

__device__ inline bool decode_seq(const KParams& P, int b, Seq& s) {
  const int n0 = P.node_offsets[b];
  const int n1 = P.node_offsets[b + 1];
  const long long p0 = P.prefix_offsets[b];
  const long long pe = P.prefix_offsets[b + 1];
  const long long p1 = P.prefix_lens ? p0 + P.prefix_lens[b] : pe;
  if (n0 < 0 || n1 <= n0 || n1 - n0 > P.max_nodes || n1 > P.total_nodes) return false;
  if (p0 < 0 || p1 < p0 || p1 > pe || p1 - p0 > P.max_prefix || pe > P.total_prefix) return false;
  s.n0 = n0;
  s.nn = n1 - n0;
  s.p0 = p0;
  s.L = (int)(p1 - p0);
  return true;
}

// Tile range of one (sequence, row tile): prefix tiles then tree tiles up to
// the row tile's last node, and how many splits it gets (in proportion to the
// longest possible range, so equal-length sequences split identically).
struct Range {
  int rows_here, n_hi, Lt, T, Sb;
};

__device__ inline bool row_tile_range(const KParams& P, const Seq& sq, int r, Range& g) {
  const int rows_b = sq.nn * P.G;
  const int row0 = r * P.rows_wg;
  if (row0 >= rows_b) return false;
  g.rows_here = min(P.rows_wg, rows_b - row0);
  g.n_hi = (row0 + g.rows_here - 1) / P.G;
  g.Lt = (sq.L + kKT - 1) / kKT;
  // Every tree tile of the sequence: in a reranked tree an ancestor may be
  // listed after its descendant, so the row tile's own nodes do not bound
  // the keys it sees (the mask drops the rest).
  g.T = g.Lt + (sq.nn + kKT - 1) / kKT;
  const int sb = P.piece > 0 ? (g.T + P.piece - 1) / P.piece
                             : (int)(((long long)P.S * g.T + P.tmax - 1) / P.tmax);
  g.Sb = max(1, min(sb, min(P.S, g.T)));
  return true;
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Lanes l and l^32 hold the two halves of one query row.  v_permlane32_swap
// exchanges the wave's two 32-lane halves in the VALU (no LDS round trip), so
// each lane sees both values of its row.
__device__ inline float2 row_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return make_float2(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float row_max(float x) {
  const float2 h = row_halves(x);
  return fmaxf(h.x, h.y);
}
__device__ inline float row_sum(float x) {
  const float2 h = row_halves(x);
  return h.x + h.y;
}

// Grid item of (sequence b, KV head g, split s, row tile r).  Split-major
// order (b, s, g, r) lets one XCD stream whole key rows of a key range; the
// in-kernel merge uses head-major order (b, g, s, r) so that every split of a
// (sequence, KV head) lands on one XCD, next to its merge workgroups.
__device__ inline long long item_index(const KParams& P, int b, int g, int s, int r) {
  return P.head_major ? (((long long)b * P.Hkv + g) * P.S + s) * P.R + r
                      : (((long long)b * P.S + s) * P.Hkv + g) * P.R + r;
}

// Longest-piece-first order for ragged batches (one row tile, B <= 64).
// Sequences are cut into pieces of about `piece` tiles; the pieces of all
// (sequence, split, KV head) units are ordered by length, longest first (ties:
// lower sequence, then split, then head), and workgroup k takes piece k.
// Workgroup ids are dealt round-robin over the XCDs and each XCD starts its
// workgroups in id order, so every XCD gets an equal share of the work and
// starts its longest pieces first.  Every wave computes the same answer from
// the offsets (lane b holds sequence b).  A sequence whose offsets do not
// decode keeps one piece per KV head, ordered last, so its workgroups still
// report it.  Returns false when k is past the last piece.
__device__ inline bool lpt_piece(const KParams& P, long long k, int& b, int& g, int& s) {
  const int lane = threadIdx.x & 63;
  int key = 0, cnt = 0;   // piece length (tiles) and pieces of sequence `lane`
  if (lane < P.B) {
    Seq sq;
    Range rg;
    if (decode_seq(P, lane, sq) && row_tile_range(P, sq, 0, rg)) {
      key = (rg.T + rg.Sb - 1) / rg.Sb;
      cnt = rg.Sb * P.Hkv;
    } else {
      cnt = P.Hkv;
    }
  }
  // Pieces of the sequences ahead of this one in the order.
  long long off = 0;
  for (int j = 0; j < P.B; ++j) {
    const int kj = __builtin_amdgcn_readlane(key, j);
    const int cj = __builtin_amdgcn_readlane(cnt, j);
    if (kj > key || (kj == key && j < lane)) off += cj;
  }
  const unsigned long long hit = __ballot(lane < P.B && k >= off && k < off + cnt);
  if (!hit) return false;
  b = __builtin_ctzll(hit);
  const long long idx = k - __shfl(off, b);
  s = (int)(idx / P.Hkv);
  g = (int)(idx % P.Hkv);
  return true;
}

// Hardware id of the XCD this wave runs on (HW_REG_XCC_ID, bits 3:0).
__device__ inline int xcc_id() { return __builtin_amdgcn_s_getreg(20 | (0 << 6) | (3 << 11)) & 15; }

// Counter block of the in-kernel merge at the start of the workspace: the
// call status word (uint32 at byte 0), then from byte kGroupBase four 64-bit
// words per (sequence, KV head, row tile) group: arrivals, epoch, merge
// workgroups done, unused.
constexpr int kGroupBase = 64;
constexpr int kGroupBytes = 32;

// Arrival word of one split: bits 0..5 count the splits that stored their
// partial, 6 bits per XCD (from bit 6) count them per XCD, so the merge can
// check that every split ran on its own XCD, and bits 54..63 add up the
// splits' tags (2E + 1 for the group's epoch E, modulo 2^10), so arrivals of
// another call never complete this call's sum.  At most 32 splits per group.
__device__ inline unsigned long long arrival_word(int xcc, unsigned long long epoch) {
  return 1ull + (1ull << (6 + 6 * xcc)) + (((2ull * epoch + 1ull) & 1023ull) << 54);
}

// Sum of the arrival words of `sb` splits on XCD `xcc` in epoch `epoch`.
__device__ inline unsigned long long group_complete(int sb, int xcc, unsigned long long epoch) {
  const unsigned long long n = (unsigned long long)sb;
  return n + (n << (6 + 6 * xcc)) + (((n * (2ull * epoch + 1ull)) & 1023ull) << 54);
}

__device__ inline unsigned long long load_agent(const unsigned long long* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Loads of other workgroups' partials in the in-kernel merge: agent scope,
// past the CU's L1 (plain loads measured the same).
__device__ inline unsigned long long load_part(const unsigned long long* p) {
  return load_agent(p);
}

// Stored partial of one row (split epilogue): 4 x fp16 per 8 bytes, each the
// normalised value times 2^k, and the row's running max m and sum l, whose
// low 8 mantissa bits hold k + 128 (a relative change of l below 2^-15).
__device__ inline f32x4_t unpack_f16x4(u32x2_t v) {
  return __builtin_convertvector(__builtin_bit_cast(f16x4_t, v), f32x4_t);
}
__device__ inline float partial_sum(float2 m_l) {
  return __uint_as_float(__float_as_uint(m_l.y) & ~255u);
}
// 2^-k, the factor that undoes the row's scale.
__device__ inline float partial_unscale(float2 m_l) {
  const int k = (int)(__float_as_uint(m_l.y) & 255u) - 128;
  return __uint_as_float((uint32_t)(127 - k) << 23);
}

// Log-sum-exp merge of the splits of one (sequence, KV head, row tile, row
// group, 32-dim block e, 8-dim slice j): split s left its normalised output
// O_s, its running max m_s and sum l_s; with M = max_s m_s and
// w_s = l_s * exp(scale*(m_s - M)),
//   out = sum_s w_s O_s / sum_s w_s,  lse = scale*M + log(sum_s w_s).
// Splits that saw no visible key carry m = -inf and weigh nothing.  Lane
// owns dims 32e + 8j + 4*(lane/32) .. +3 of row lane%32 of the row group.
struct MergeAcc {
  float M = kNegInf;
  float lsum = 0.f;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  __device__ void add(float2 m_l, u32x2_t hv, float c2) {
    const float l = partial_sum(m_l);
    const float m_new = fmaxf(M, m_l.x);
    const float mu = (m_new == kNegInf) ? 0.f : m_new;
    const float a = fast_exp2((M - mu) * c2);
    const float w = fast_exp2((m_l.x - mu) * c2) * l;
    acc = acc * a + (w * partial_unscale(m_l)) * unpack_f16x4(hv);
    lsum = lsum * a + w;
    M = m_new;
  }
};

// s_waitcnt immediate that waits for vmcnt <= N and nothing else (gfx9
// encoding: vmcnt[3:0] in bits 3:0, vmcnt[5:4] in bits 15:14, expcnt and
// lgkmcnt at their maxima).
template <int N>
constexpr int vmcnt_imm() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  return (N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8);
}

// Direct global -> LDS loads, issued through inline asm so that the only
// waits on them are the explicit vmcnt waits of the pipeline (the compiler
// would otherwise wait for every pending load before each LDS read).  The
// LDS base goes to M0 and must be wave-uniform; lane i's data lands at
// base + i * size.
__device__ inline uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)((const __attribute__((address_space(3))) void*)p);
}
__device__ inline void dma_b128(const void* g, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(lds_base), "v"(g)
               : "memory", "m0");
}
__device__ inline void dma_b32(const void* g, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off"
               :
               : "s"(lds_base), "v"(g)
               : "memory", "m0");
}

__device__ inline i16x4_t lds_read_tr16(const unsigned char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4_t*)(p));
}

__device__ inline void store_merged(const KParams& P, const Seq& sq, int g, int r, int rl, int e,
                                    int j, int hh, const MergeAcc& ma) {
  const int my_row = r * P.rows_wg + rl;
  const int node = my_row / P.G;
  const int head = g * P.G + my_row % P.G;
  const float inv = ma.lsum > 0.f ? 1.f / ma.lsum : 0.f;
  const bf16x4_t h4 = __builtin_convertvector(ma.acc * inv, bf16x4_t);
  *reinterpret_cast<u32x2_t*>(P.out + ((size_t)(sq.n0 + node) * P.Hq + head) * kD + 32 * e + 8 * j +
                              4 * hh) = __builtin_bit_cast(u32x2_t, h4);
  if (P.lse && e == 0 && j == 0 && hh == 0)
    P.lse[(size_t)(sq.n0 + node) * P.Hq + head] =
        ma.lsum > 0.f ? ma.M * P.scale + logf(ma.lsum) : kNegInf;
}

// In-kernel merge, used when few (sequence, KV head, row tile) groups carry
// the splits.  Merge workgroups follow the split workgroups in the grid and
// never hold up a split (a split never waits).  Workgroups are dealt to the
// 8 XCDs round-robin by id, and the item order puts all splits of a
// (sequence, KV head) on one XCD; merge workgroup m also runs on XCD m % 8 and
// takes groups of that XCD.  Partials then stay in that XCD's L2, which is
// coherent for all its CUs, so no L2 write-back or invalidate is needed.
//
// Protocol.  Every workgroup of a group reads the group's epoch E at its
// start; E only changes once all of them have read it (below).  A split
// stores its partial, waits for the stores to be acknowledged, and adds its
// arrival word (count, per-XCD count, tag of E) to the group's arrivals.  A
// merge workgroup polls the arrivals until the count reaches the group's
// split count Sb; the partials are this call's and coherent in its L2 iff the
// arrivals then equal group_complete(Sb, its XCD, E): every split ran on its
// own XCD and every arrival carries this epoch's tag.  Then it merges RG*16/NW
// (row group, 32-dim block, 8-dim slice) units, one per wave, and counts
// itself done; the last one of a group returns arrivals and done count to
// zero and advances E, so the next call's tags differ from this call's.
// When the check fails it writes NaN instead of a possibly stale result and
// sets a bit in the call status word (kMergeStatus*, the caller's way to
// tell).  The wait is bounded (2^18 polls, under a second), so counters that
// were not zero at entry cannot hang a call: a merge workgroup that times out
// writes NaN, zeroes the group's words and advances E itself.  A split of a
// timed-out call that arrives after that reset carries the old tag, so the
// next call fails its check loudly instead of merging its stale partial, and
// that call's last merge workgroup zeroes the words again.
constexpr int kSpinMax = 1 << 18;
constexpr unsigned kMergeStatusPlacement = TA_MERGE_PLACEMENT;
constexpr unsigned kMergeStatusTimeout = TA_MERGE_TIMEOUT;
constexpr unsigned kMergeStatusStale = TA_MERGE_STALE;

template <int RG, int NW>
__device__ void merge_in_kernel(const KParams& P, long long m) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const long long groups_per_xcd = P.groups / 8;
  const long long i = m >> 3;
  const long long gi = (m & 7) * groups_per_xcd + i / P.merge_wpg;
  const int unit = (int)(i % P.merge_wpg) * NW + wave;   // (rg, e, j) of this wave
  const int r = (int)(gi % P.R);
  const int g = (int)((gi / P.R) % P.Hkv);
  const int b = (int)(gi / ((long long)P.R * P.Hkv));
  Seq sq;
  Range rgn;
  if (!decode_seq(P, b, sq) || !row_tile_range(P, sq, r, rgn) || rgn.Sb <= 1) return;
  // arrivals, epoch, done
  unsigned long long* word = P.cnt + (kGroupBase + kGroupBytes * gi) / 8;
  __shared__ unsigned long long seen_word, seen_epoch;
  __shared__ int timed_out;
  if (tid == 0) {
    // Poll with relaxed agent-scope atomic loads (coherent with the splits'
    // agent-scope adds, never a cached copy); they return sooner than an
    // atomic add of zero would.
    const unsigned long long ep = load_agent(word + 1);
    unsigned long long seen = 0;
    int n = 0;
    for (; n < kSpinMax; ++n) {
      seen = load_agent(word);
      if ((seen & 63) == (unsigned long long)rgn.Sb) break;
      __builtin_amdgcn_s_sleep(4);
    }
    seen_word = seen;
    seen_epoch = ep;
    timed_out = n == kSpinMax;
  }
  __syncthreads();
  TA_TL(4, TA_TL_NOW());
  const int xcc = xcc_id();
  const bool coherent = !timed_out && seen_word == group_complete(rgn.Sb, xcc, seen_epoch);
  // Every merge workgroup counts itself done as soon as it has seen its group
  // complete (its round trip then overlaps the partial loads below); once all
  // of a group's merge workgroups have, nothing reads the group's words in
  // this call, so the last of them resets them for the next call.
  unsigned long long done = 0ull;
  if (tid == 0) {
    if (!timed_out)
      done = __hip_atomic_fetch_add(word + 2, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (!coherent) {
      // Which check failed: a count beyond the splits' own (per XCD) means
      // another call's arrivals; a count on another XCD, a placement failure.
      // Placement: the per-XCD counts account for every arrival but not all
      // on this XCD.  Otherwise the words hold arrivals of another call.
      int per_xcd = 0;
#pragma unroll
      for (int x = 0; x < 8; ++x) per_xcd += (int)((seen_word >> (6 + 6 * x)) & 63ull);
      const bool all_here = (int)((seen_word >> (6 + 6 * xcc)) & 63ull) == rgn.Sb;
      const unsigned bits = timed_out ? kMergeStatusTimeout
                            : (per_xcd == rgn.Sb && !all_here) ? kMergeStatusPlacement
                                                               : kMergeStatusStale;
      __hip_atomic_fetch_or(P.merge_status, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }

  const int rg = unit >> 4;   // the same for every wave of the workgroup (NW divides 16)
  const int e = (unit >> 2) & 3;
  const int j = unit & 3;
  const int hh = lane >> 5;
  const int rl = rg * 32 + (lane & 31);
  const long long item0 = item_index(P, b, g, 0, r);
  const long long split_stride = item_index(P, b, g, 1, r) - item0;
  const bool row_here = rl < rgn.rows_here;
  // The first kBatch splits: their (m, l) for the row group's 32 rows are
  // loaded once per workgroup and shared through LDS (every wave needs the
  // same rows), their partials are all requested before any is used, so the
  // merge waits on one round trip instead of one per split.  Slots past the
  // split count re-read split 0 and are ignored.
  constexpr int kBatch = 16;
  __shared__ unsigned long long ml_s[kBatch][32];
  unsigned long long ov[kBatch];
  auto o_ptr = [&](long long it) {
    return reinterpret_cast<const unsigned long long*>(
        P.ws_o + (((size_t)it * RG + rg) * 16 + 4 * e + j) * 64 + lane);
  };
  auto ml_ptr = [&](long long it, int row) {
    return reinterpret_cast<const unsigned long long*>(P.ws_ml + (size_t)it * P.rows_wg + row);
  };
  if (coherent) {
    for (int q = tid; q < kBatch * 32; q += NW * 64) {
      const int s = q >> 5;
      const int row = rg * 32 + (q & 31);
      if (s < rgn.Sb && row < rgn.rows_here)
        ml_s[s][q & 31] = load_part(ml_ptr(item0 + s * split_stride, row));
    }
    if (row_here) {
#pragma unroll
      for (int s = 0; s < kBatch; ++s)
        ov[s] = load_part(o_ptr(item0 + (s < rgn.Sb ? s : 0) * split_stride));
    }
  }
  __syncthreads();
  if (row_here) {
    MergeAcc ma;
    if (coherent) {
#pragma unroll
      for (int s = 0; s < kBatch; ++s)
        if (s < rgn.Sb)
          ma.add(__builtin_bit_cast(float2, ml_s[s][lane & 31]),
                 __builtin_bit_cast(u32x2_t, ov[s]), P.scale_log2);
      // Splits past the first kBatch (at most 32 in all): requested together
      // too, then folded in.
      if (rgn.Sb > kBatch) {
        unsigned long long mv[kBatch];
#pragma unroll
        for (int s = 0; s < kBatch; ++s) {
          const long long it = item0 + (kBatch + s < rgn.Sb ? kBatch + s : 0) * split_stride;
          mv[s] = load_part(ml_ptr(it, rl));
          ov[s] = load_part(o_ptr(it));
        }
#pragma unroll
        for (int s = 0; s < kBatch; ++s)
          if (kBatch + s < rgn.Sb)
            ma.add(__builtin_bit_cast(float2, mv[s]), __builtin_bit_cast(u32x2_t, ov[s]),
                   P.scale_log2);
      }
    } else {
      ma.M = __builtin_nanf("");
      ma.lsum = 1.f;
      ma.acc = f32x4_t{ma.M, ma.M, ma.M, ma.M};
    }
    store_merged(P, sq, g, r, rl, e, j, hh, ma);
  }
  if (tid == 0) {
    if (timed_out || done + 1 == (unsigned long long)P.merge_wpg) {
      __hip_atomic_store(word, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(word + 2, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(word + 1, seen_epoch + 1ull, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// LDS map of one workgroup: a ring of NS stages, each KG*TPW x (K tile,
// V tile), followed (when the mask rows are not held in registers, MR false)
// by TPW mask dwords per lane per wave; the workgroup's query rows (32*RG
// rows, laid out like a K tile); and, with MR, a small block for the lanes'
// mask words or the sequence's parents.  The query block sits after the ring
// when it fits, otherwise over the last ring slot, which is first written
// only after every wave has copied its rows to registers.
template <int RG, int KG, int TPW, int NS, bool MR>
struct LdsMap {
  static constexpr int kMaskOff = KG * TPW * kTileBytes;
  static constexpr int kStage = kMaskOff + (MR ? 0 : RG * KG * TPW * 256);
  static constexpr int kRing = NS * kStage;
  static constexpr int kQBytes = RG * 32 * kRow;
  static constexpr int kAuxBytes = MR ? RG * KG * 1024 : 0;   // 4 dwords per lane per wave
  static constexpr bool kQAlias = kRing + kQBytes + kAuxBytes > kLdsMax;
  static constexpr int kQOff = kQAlias ? (NS - 1) * kStage : kRing;
  static constexpr int kQEnd = kQOff + kQBytes > kRing ? kQOff + kQBytes : kRing;
  static constexpr int kAuxOff = kQEnd;
  static constexpr int kBytes = kQEnd + kAuxBytes;
  static_assert(kBytes <= kLdsMax, "LDS budget");
};

// At most two waves per SIMD (eight waves per workgroup, and the LDS holds one
// workgroup per CU): telling the compiler so lets it schedule for latency
// instead of trying to fit more waves.
// SKIP (mask rows from memory only): drop the tree tiles no row of the
// workgroup sees, for trees whose tiles are a good part of the key range.
template <int RG, int KG, int TPW, int NS, bool MR, bool SKIP>
__global__ __launch_bounds__(RG * KG * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_bf16_kernel(KParams P) {
  static_assert(NS >= 3 && NS <= 4, "ring depth");
  constexpr int kDepth = NS - 1;   // stages requested ahead of the one in use
  constexpr int NW = RG * KG;
  constexpr int NT = NW * 64;
  constexpr int kTilesPerStage = KG * TPW;
  using Map = LdsMap<RG, KG, TPW, NS, MR>;
  constexpr int kMaskOff = Map::kMaskOff;
  constexpr int kStage = Map::kStage;
  extern __shared__ __align__(16) unsigned char lds[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // Wave-uniform values live in scalar registers, so tile-type tests below
  // are uniform branches (the masking code is skipped on prefix tiles).
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kg = wave / RG;
  const int rg = wave % RG;
  const int hh = lane >> 5;   // lane half: which 8 of each 16 contraction elements
  const int l32 = lane & 31;

  TA_TL(0, TA_TL_NOW());
  TA_TL(15, (unsigned)__builtin_amdgcn_s_getreg(4 | (0 << 6) | (31 << 11)));
  TA_TL(6, (unsigned)xcc_id() << 8);
  if (blockIdx.x >= P.n_split_blocks) {
    TA_TL(6, 2u | ((unsigned)xcc_id() << 8));
    merge_in_kernel<RG, NW>(P, (long long)blockIdx.x - P.n_split_blocks);
    TA_TL(5, TA_TL_NOW());
    return;
  }

  // Workgroup ids are dealt round-robin over the 8 XCDs; remap so that
  // consecutive items (same sequence and KV head, same key split, different
  // row tiles) run on one XCD.
  int g, s, b, r;
  long long item;
  if (P.lpt) {
    if (!lpt_piece(P, blockIdx.x, b, g, s)) return;
    r = 0;
    item = item_index(P, b, g, s, 0);
  } else {
  const long long nb = P.n_split_blocks;
  item = (long long)(blockIdx.x & 7) * (nb >> 3) + (blockIdx.x >> 3);
  if (item >= P.n_items) return;
  r = (int)(item % P.R);
  long long t = item / P.R;
  if (P.head_major) {
    s = (int)(t % P.S);
    t /= P.S;
    g = (int)(t % P.Hkv);
    b = (int)(t / P.Hkv);
  } else {
    g = (int)(t % P.Hkv);
    t /= P.Hkv;
    s = (int)(t % P.S);
    b = (int)(t / P.S);
  }
  }
  // The item is the same for every lane, but the longest-first decode moves
  // values through lane shuffles, after which the compiler can no longer
  // prove it: without this, everything derived from it (offsets, tile
  // ranges, the key loop's trip count and addresses) would be computed per
  // lane, and the key loop would run as a divergent loop under exec masks.
  b = __builtin_amdgcn_readfirstlane(b);
  g = __builtin_amdgcn_readfirstlane(g);
  s = __builtin_amdgcn_readfirstlane(s);
  r = __builtin_amdgcn_readfirstlane(r);
  item = ((long long)__builtin_amdgcn_readfirstlane((int)(item >> 32)) << 32) |
         (unsigned)__builtin_amdgcn_readfirstlane((int)item);

  Seq sq;
  if (!decode_seq(P, b, sq)) {
    // A sequence without nodes is valid (nothing to compute or write), as the
    // mask builder has it; any other offset that does not decode is reported.
    if (P.build && P.status_out && g == 0 && s == 0 && r == 0 && tid == 0) {
      const int n0 = P.node_offsets[b];
      const int n1 = P.node_offsets[b + 1];
      P.status_out[b] = (n0 >= 0 && n1 == n0 && n1 <= P.total_nodes) ? 0 : TA_ERR_INVALID_ARG;
    }
    return;
  }
  Range rgn;
  if (!row_tile_range(P, sq, r, rgn)) return;
  if (s >= rgn.Sb) return;
  TA_TL(1, TA_TL_NOW());
  TA_TL(6, 1u | ((unsigned)xcc_id() << 8));
  // In-kernel merge: this group's words, and its epoch, read now so that the
  // arrival after the key loop does not wait for it.
  unsigned long long* grp_word = nullptr;
  unsigned long long epoch = 0ull;
  if (P.cnt && rgn.Sb > 1) {
    grp_word = P.cnt + (kGroupBase + kGroupBytes * (((long long)b * P.Hkv + g) * P.R + r)) / 8;
    epoch = load_agent(grp_word + 1);
  }
  const int t_lo = (int)((long long)s * rgn.T / rgn.Sb);
  const int t_hi = (int)((long long)(s + 1) * rgn.T / rgn.Sb);
  const int L = sq.L;
  const int Lt = rgn.Lt;
  const int row0 = r * P.rows_wg;

  // Sparse tree keys (SKIP: above 128 nodes, mask rows read from memory).
  // A split's tree keys are those of its dense tree tiles; it needs only the
  // ones some row of the workgroup sees: the union of those rows' ancestor
  // sets.  Gather mode lists that union in LDS (s_keys, ascending) and walks
  // it in 32-key tiles whose K/V rows are loaded through the list, with each
  // row's visibility bits for each gathered tile precomputed in LDS
  // (s_gbits); when the union or the bits would not fit, the split keeps
  // instead the dense tree tiles in which some row sees a key (tile
  // compaction, s_tt).  The split's bounds stay those of the dense tile range
  // (every split of a row tile, and the merge, agree on them without reading
  // the mask); its loop walks its prefix tiles, then the gathered or kept
  // tiles.  A split left with no tile still runs one (masked) iteration, so
  // its query and stage loads are waited for before it ends.
  constexpr int kGatherMaxKeys = 2048;
  constexpr int kGatherBitWords = 2048;
  constexpr int kGath = 1 << 24;   // gathered tile t is walked as "tile" kGath + t
  __shared__ int s_tt[TA_MAX_NODES / kKT];
  __shared__ unsigned char s_act[TA_MAX_NODES / kKT];
  __shared__ int s_nact;
  __shared__ unsigned long long s_u[TA_MAX_NODES / 64];
  __shared__ int s_ust[TA_MAX_NODES / 64];
  __shared__ int16_t s_keys[kGatherMaxKeys];
  __shared__ uint32_t s_gbits[kGatherBitWords];
  __shared__ int s_ng;
  int n_pre = t_hi - t_lo;   // tiles walked in order from t_lo
  int n_act = 0;             // kept tree tiles after them (compact mode)
  int n_gt = 0;              // gathered tiles after them (gather mode)
  int n_g = 0;               // gathered keys
  int g_lo = 0;              // the workgroup's first node (rows of s_gbits)
  bool compact = false, gather = false;
  const bool sparse_tree = SKIP && !MR && sq.nn > 128 && t_hi > Lt;
  if (sparse_tree) n_pre = max(0, min(t_hi, Lt) - t_lo);
  // Run below: after the first stages are requested when those are all
  // prefix tiles (their loads then overlap the mask reads), else before.
  auto gather_setup = [&]() {
  if constexpr (SKIP && !MR) {
    {
      const int ta0 = max(t_lo, Lt) - Lt;   // the split's tree tiles: [ta0, ta0 + nt)
      const int nt = t_hi - Lt - ta0;
      const int n_lo = row0 / P.G;
      const int nodes = rgn.n_hi - n_lo + 1;
      const uint64_t* mrows = P.mask + (size_t)(sq.n0 + n_lo) * P.W;
      // Keys [k_lo, k_hi) of those tiles lie in mask words [w_lo, w_lo + nw).
      const int k_lo = ta0 * kKT;
      const int k_hi = min(sq.nn, (ta0 + nt) * kKT);
      const int w_lo = k_lo / 64;
      const int nw = (k_hi + 63) / 64 - w_lo;
      for (int w = tid; w < nw; w += NT) s_u[w] = 0ull;
      __syncthreads();
      // Union of the rows' words.  When they fit (at most kHeld per thread,
      // e.g. 64 nodes x 64 words) each thread loads its words once, all in
      // flight together, and keeps them for the visibility bits below;
      // otherwise two passes over memory, four loads in flight per thread.
      const int total = nodes * nw;
      auto word_at = [&](int q) { return mrows[(size_t)(q / nw) * P.W + w_lo + q % nw]; };
      constexpr int kHeld = 8;
      const bool held = total <= NT * kHeld;
      uint64_t vh[kHeld];
      if (held) {
#pragma unroll
        for (int u = 0; u < kHeld; ++u) {
          const int q = u * NT + tid;
          vh[u] = q < total ? word_at(q) : 0ull;
        }
#pragma unroll
        for (int u = 0; u < kHeld; ++u)
          if (vh[u]) atomicOr(&s_u[(u * NT + tid) % nw], (unsigned long long)vh[u]);
      } else {
        for (int q0 = 0; q0 < total; q0 += NT * 4) {
          uint64_t v[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) v[u] = word_at(min(q0 + u * NT + tid, total - 1));
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int q = q0 + u * NT + tid;
            if (q < total && v[u]) atomicOr(&s_u[q % nw], (unsigned long long)v[u]);
          }
        }
      }
      __syncthreads();
      // Clip to [k_lo, k_hi); key positions: an exclusive scan of popcounts.
      if (wave == 0) {
        int base = 0;
        for (int w0 = 0; w0 < nw; w0 += 64) {
          const int w = w0 + lane;
          uint64_t v = 0ull;
          if (w < nw) {
            v = s_u[w];
            const int lo = 64 * (w_lo + w);
            if (lo < k_lo) v &= ~0ull << (k_lo - lo);
            if (k_hi - lo < 64) v &= (1ull << (k_hi - lo)) - 1ull;
            s_u[w] = v;
          }
          const int c = __popcll(v);
          int incl = c;
          for (int o = 1; o < 64; o <<= 1) {
            const int t = __shfl_up(incl, o);
            if (lane >= o) incl += t;
          }
          if (w < nw) s_ust[w] = base + incl - c;
          base += __shfl(incl, 63);
        }
        if (lane == 0) s_ng = base;
      }
      __syncthreads();
      n_g = __builtin_amdgcn_readfirstlane(s_ng);
      n_gt = (n_g + kKT - 1) / kKT;
      gather = n_g <= kGatherMaxKeys && nodes * n_gt <= kGatherBitWords;
      if (gather) {
        g_lo = n_lo;
        // The key list: a wave per word, a lane per bit.
        for (int w = wave; w < nw; w += NW) {
          const uint64_t v = s_u[w];
          if ((v >> lane) & 1ull)
            s_keys[s_ust[w] + __popcll(v & ((1ull << lane) - 1ull))] =
                (int16_t)(64 * (w_lo + w) + lane);
        }
        for (int q = tid; q < nodes * n_gt; q += NT) s_gbits[q] = 0u;
        __syncthreads();
        // Visibility bits: for each (row node, word) pair, each key the node
        // sees in the word (a node sees few keys, so few steps) set at its
        // position in the list: the word's start plus the union's bits below.
        auto set_bits = [&](int q, uint64_t v) {
          const int nd = q / nw;
          const int w = q % nw;
          const uint64_t uu = s_u[w];
          uint64_t vv = v & uu;
          while (vv) {
            const int b = __builtin_ctzll(vv);
            vv &= vv - 1ull;
            const int pos = s_ust[w] + __popcll(uu & ((1ull << b) - 1ull));
            atomicOr(&s_gbits[nd * n_gt + (pos >> 5)], 1u << (pos & 31));
          }
        };
        if (held) {
#pragma unroll
          for (int u = 0; u < kHeld; ++u)
            if (vh[u]) set_bits(u * NT + tid, vh[u]);
        } else {
          for (int q0 = 0; q0 < total; q0 += NT * 4) {
            uint64_t v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) v[u] = word_at(min(q0 + u * NT + tid, total - 1));
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const int q = q0 + u * NT + tid;
              if (q < total) set_bits(q, v[u]);
            }
          }
        }
        __syncthreads();
      } else {
        compact = true;
        for (int k = tid; k < nt; k += NT) s_act[k] = 0;
        __syncthreads();
        const int per = NT / nt;   // threads per tile (nt <= 128 <= NT)
        if (tid < per * nt) {
          const int k = tid % nt;
          uint32_t acc = 0u;
#pragma unroll 8
          for (int n = n_lo + tid / nt; n <= rgn.n_hi; n += per)
            acc |= reinterpret_cast<const uint32_t*>(P.mask + (size_t)(sq.n0 + n) * P.W)[ta0 + k];
          if (acc) s_act[k] = 1;
        }
        __syncthreads();
        if (wave == 0) {
          int base = 0;
          for (int k0 = 0; k0 < nt; k0 += 64) {
            const int k = k0 + lane;
            const bool act = k < nt && s_act[k] != 0;
            const uint64_t bal = __ballot(act);
            if (act) s_tt[base + __popcll(bal & ((1ull << lane) - 1ull))] = ta0 + k;
            base += __popcll(bal);
          }
          if (lane == 0) s_nact = base;
        }
        __syncthreads();
        n_act = __builtin_amdgcn_readfirstlane(s_nact);
      }
    }
  }
  };
  // Tile of the split's li-th step: prefix tiles in order, then the gathered
  // or kept tree tiles; past the end, t_hi (loaded in bounds, masked as
  // inactive).
  auto phys = [&](int li) -> int {
    if (!SKIP || (!compact && !gather) || li < n_pre) return t_lo + li;
    if (gather) return li < n_pre + n_gt ? kGath + (li - n_pre) : t_hi;
    if (li < n_pre + n_act) return __builtin_amdgcn_readfirstlane(Lt + s_tt[li - n_pre]);
    return t_hi;
  };
  auto is_active = [&](int tile) { return tile < t_hi || (SKIP && tile >= kGath); };

  // This lane's query row.
  const int my_row = row0 + rg * 32 + l32;
  const bool row_ok = my_row < row0 + rgn.rows_here;
  const bool group_active = rg * 32 < rgn.rows_here;
  const int node = row_ok ? my_row / P.G : 0;
  const int head = g * P.G + (row_ok ? my_row % P.G : 0);

  bf16x8_t qf[8];

  const size_t kv_row = (size_t)P.Hkv * kD;   // elements between consecutive key rows
  const uint16_t* kp = P.k_prefix + ((size_t)sq.p0 * P.Hkv + g) * kD;
  const uint16_t* vp = P.v_prefix + ((size_t)sq.p0 * P.Hkv + g) * kD;
  const uint16_t* kt = P.k_tree + ((size_t)sq.n0 * P.Hkv + g) * kD;
  const uint16_t* vt = P.v_tree + ((size_t)sq.n0 * P.Hkv + g) * kD;

  // Query rows go to LDS with the same direct loads, ahead of stage 0, so
  // they arrive in the same round trip as the first K/V tiles.  Block u of
  // wave w is rows 4(w + NW*u) .. +3 of the workgroup, swizzled like a K
  // tile; rows past the tile's end read the tile's first row (in bounds,
  // finite) and their outputs are never written.
  static_assert((RG * 8) % NW == 0, "query blocks must split evenly over the waves");
  auto issue_q = [&]() {
#pragma unroll
    for (int u = 0; u < RG * 8 / NW; ++u) {
      const int blk = wave + NW * u;
      const int qr = 4 * blk + (lane >> 4);
      const int mr = row0 + qr < row0 + rgn.rows_here ? row0 + qr : row0;
      const uint16_t* src = P.q + ((size_t)(sq.n0 + mr / P.G) * P.Hq + g * P.G + mr % P.G) * kD +
                            (((lane & 15) ^ (qr & 15)) << 3);
      dma_b128(src, lds_addr(lds + Map::kQOff + blk * 1024));
    }
  };

  // Stage loader: direct global -> LDS loads (no staging registers).  For each
  // tile of the stage and each of K, V, wave w writes rows 4w + 4*NW*u ..
  // +3 (1 KB) per instruction; lane i lands at byte 16*i of that block, i.e.
  // row 4w + 4*NW*u + i/16, 16-byte slot i%16.  The slot holds logical chunk
  // (i%16) ^ swz(row): K uses swz = row%16 and V uses swz = 4*(row%4), which
  // keeps the K b128 reads and the V transpose reads free of bank conflicts.
  // Padding keys, past-the-end tree nodes and tiles beyond the split read tree
  // row 0 (in bounds, finite); the mask turns their scores into -inf, so they
  // contribute exactly zero.  Each thread issues the same number of loads per
  // stage (kLoads), so stage it is complete when vmcnt <= kLoads * (stages
  // issued after it).
  constexpr int kRowsPerPass = NT / 16;
  constexpr int kPasses = kKT / kRowsPerPass;   // per tile and per K/V
  static_assert(kPasses * kRowsPerPass == kKT, "tile rows must split evenly");
  constexpr int kLoads = kTilesPerStage * 2 * kPasses + (MR ? 0 : TPW);
  static_assert(kLoads <= 63, "vmcnt range");
  const int ld_key = tid >> 4;
  const int ld_slot = tid & 15;
  // Loop-invariant per-lane source pointers: this lane's row of K and V
  // (chunk already swizzled) at tile 0 of the prefix and of the tree, and
  // its mask row.  A plain prefix tile then costs one uniform 64-bit add per
  // load; only the boundary tile and the tree tiles take the general path.
  const size_t tile_stride = (size_t)kKT * kv_row;    // elements per 32 key rows
  const uint16_t* pk[kPasses];
  const uint16_t* pv[kPasses];
#pragma unroll
  for (int u = 0; u < kPasses; ++u) {
    const int row = ld_key + kRowsPerPass * u;
    pk[u] = kp + (size_t)row * kv_row + ((ld_slot ^ (row & 15)) << 3);
    pv[u] = vp + (size_t)row * kv_row + ((ld_slot ^ ((row & 3) << 2)) << 3);
  }
  const int L_full = L / kKT;                         // tiles entirely inside the prefix
  const uint32_t* mrow_dw =
      P.mask ? reinterpret_cast<const uint32_t*>(P.mask + (size_t)(sq.n0 + (row_ok ? node : 0)) * P.W)
             : nullptr;
  auto issue_stage = [&](int it) {
    unsigned char* st = lds + (it % NS) * kStage;
#pragma unroll
    for (int tk = 0; tk < kTilesPerStage; ++tk) {
      const int tile = phys(it * kTilesPerStage + tk);
#pragma unroll
      for (int u = 0; u < kPasses; ++u) {
        const uint16_t* gk;
        const uint16_t* gv;
        if (SKIP && tile >= kGath) {
          // Gathered tile: row `row` holds listed key 32 * (tile - kGath) + row
          // (node 0 past the list's end; its scores are masked).
          const int row = ld_key + kRowsPerPass * u;
          const int idx = kKT * (tile - kGath) + row;
          const size_t off = (size_t)(idx < n_g ? (int)s_keys[idx] : 0) * kv_row;
          gk = kt + off + ((ld_slot ^ (row & 15)) << 3);
          gv = vt + off + ((ld_slot ^ ((row & 3) << 2)) << 3);
        } else if (tile < L_full) {
          gk = pk[u] + (size_t)tile * tile_stride;
          gv = pv[u] + (size_t)tile * tile_stride;
        } else {
          const int row = ld_key + kRowsPerPass * u;
          const int kk = tile * kKT + row;
          const int tn = kk - Lt * kKT;
          const bool in_prefix = kk < L;
          const bool in_tree = tile >= Lt && tn < sq.nn;
          const size_t off = (size_t)(in_prefix ? kk : (in_tree ? tn : 0)) * kv_row;
          gk = (in_prefix ? kp : kt) + off + ((ld_slot ^ (row & 15)) << 3);
          gv = (in_prefix ? vp : vt) + off + ((ld_slot ^ ((row & 3) << 2)) << 3);
        }
        const uint32_t dk = lds_addr(st + tk * kTileBytes + (4 * wave + kRowsPerPass * u) * kRow);
        dma_b128(gk, dk);
        dma_b128(gv, dk + kTileKV);
      }
    }
    // The 32-bit half of this lane's mask word that covers each of its
    // wave's tiles (any in-bounds word for prefix tiles and idle rows).
    if constexpr (!MR) {
#pragma unroll
      for (int j = 0; j < TPW; ++j) {
        const int my_tile = phys((it * KG + kg) * TPW + j);
        const int dw = (my_tile >= Lt && my_tile < t_hi) ? my_tile - Lt : 0;
        dma_b32(mrow_dw + dw, lds_addr(st + kMaskOff + (wave * TPW + j) * 256));
      }
    }
  };

  // MR: the whole mask row of this lane's node (at most 128 nodes, 4 dwords)
  // lives in registers.  Ahead of the query rows, each wave copies its lanes'
  // mask dwords to LDS, or, when the kernel builds the mask, wave 0 copies
  // the sequence's parents; both are retired by the first stage wait.
  unsigned char* aux = lds + Map::kAuxOff;
  auto issue_aux = [&]() {
    if constexpr (MR) {
      if (P.build) {
        if (wave == 0) {
          for (int h = 0; h * 64 < sq.nn; ++h) {
            const int k = h * 64 + lane;
            dma_b32(P.parents + sq.n0 + (k < sq.nn ? k : 0), lds_addr(aux + h * 256));
          }
        }
      } else {
        for (int d = 0; d < 2 * P.W; ++d)
          dma_b32(mrow_dw + d, lds_addr(aux + wave * 1024 + d * 256));
      }
    }
  };
  // Stage it is in LDS for every wave once each has retired its own loads up
  // to stage it and all have passed the barrier.  The barrier carries no
  // memory fence (a fence would wait for the stages still in flight); the
  // empty asm statements keep the compiler from moving LDS accesses across.
  // Stages issued after stage it: min(kDepth - 1, n_iter - 1 - it).
  static_assert((kDepth - 1) * kLoads <= 63, "vmcnt range");
  auto wait_stage = [&](int it, int n_iter) {
    const int later = min(kDepth - 1, n_iter - 1 - it);
    if (kDepth > 2 && later >= 2)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm<2 * kLoads>());
    else if (later >= 1)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm<kLoads>());
    else
      __builtin_amdgcn_s_waitcnt(vmcnt_imm<0>());
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  f32x16_t oacc[4];
#pragma unroll
  for (int e = 0; e < 4; ++e)
#pragma unroll
    for (int v = 0; v < 16; ++v) oacc[e][v] = 0.f;
  float m_run = kNegInf;
  float l_run = 0.f;
  const float c2 = P.scale_log2;

  // Per-lane LDS offsets (swizzled rows, see the loader).  K: chunk 2i+hh of
  // key row l32.  V transpose reads: a 16-lane group reads a 4-key x 16-dim
  // block, lane i of the group gets dim (base + i) of keys key0 .. key0+3;
  // with r = (lane%16)/4 the physical chunk of dim block e is 4*(e^r) + clo.
  uint32_t koff[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) koff[i] = l32 * kRow + (((2 * i + hh) ^ (l32 & 15)) << 4);
  uint32_t voff[4];
  {
    const int r = (lane & 15) >> 2;
    const int clo = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      voff[e] = (4 * hh + r) * kRow + (((4 * (e ^ r)) + clo) << 4) + 8 * (lane & 1);
  }


  // S^T = K Q^T for one tile's 32 keys x this wave's 32 rows.  Accumulator v
  // of this lane holds key 8*(v/4) + 4*hh + v%4 of the tile.
  auto qk = [&](const unsigned char* kb) {
    f32x16_t sacc;
#pragma unroll
    for (int v = 0; v < 16; ++v) sacc[v] = 0.f;
    // All eight K fragments are requested before the MFMA chain starts, so
    // the chain waits for the LDS once instead of before every MFMA.
    u32x4_t kf[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) kf[i] = *reinterpret_cast<const u32x4_t*>(kb + koff[i]);
    asm volatile("" ::: "memory");
#pragma unroll
    for (int i = 0; i < 8; ++i)
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, kf[i]), qf[i],
                                                     sacc, 0, 0, 0);
    return sacc;
  };

  // Masking of one tile's scores: an idle tile (beyond the split, or an idle
  // row group) is all -inf; a tree tile keeps the row node's ancestors; the
  // prefix's partial last tile drops the keys past the prefix.
  // One uniform branch that edits the scores in place: full prefix tiles (all
  // but a few) skip it, and no per-case copies of the scores are made.
  auto mask_tile = [&](f32x16_t& sacc, int tile, uint32_t mbits, bool active) {
    const bool tree = tile >= Lt;
    const bool tail = !tree && (tile + 1) * kKT > L;
    if (!active || tree || tail) {
      // Bit k of keep: key k of the tile stays visible.
      uint32_t keep;
      if (!active)
        keep = 0u;
      else if (tree)
        keep = row_ok ? mbits : 0u;
      else
        keep = (1u << (L - tile * kKT)) - 1u;   // 1 <= L - 32*tile <= 31 keys left
      const uint32_t kh = keep >> (4 * hh);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int key = 8 * (v >> 2) + (v & 3);
        sacc[v] = (kh & (1u << key)) ? sacc[v] : kNegInf;
      }
    }
  };

  // Online softmax and O^T += V^T P^T over the wave's TPW tiles of a stage,
  // taken as one block of keys: one max, one lazy-reference decision and at
  // most one rescale per stage, and the exponentials of one tile can overlap
  // the PV MFMAs of the other.
  auto softmax_pv = [&](f32x16_t (&sc)[TPW], const unsigned char* const (&vb)[TPW]) {
    float mt = sc[0][0];
#pragma unroll
    for (int j = 0; j < TPW; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) mt = fmaxf(mt, sc[j][v]);
    mt = row_max(mt);
    // Lazy running max: the reference moves only when the block's max exceeds
    // it by more than kLazyLog2 (log2 units), so after the first tiles the
    // output is almost never rescaled; probabilities stay below 2^kLazyLog2
    // and numerator and denominator share the reference, so the result is
    // unchanged.  Lanes l and l^32 hold the same row and take the same
    // decision.
    const bool move = (mt - m_run) * c2 > kLazyLog2;   // also true when m_run = -inf
    const float m_old = m_run;
    if (move) m_run = mt;
    const float m_use = (m_run == kNegInf) ? 0.f : m_run;
    const float alpha = move ? fast_exp2((m_old - m_use) * c2) : 1.f;
    const float mc = m_use * c2;
    if (__ballot(move)) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int v = 0; v < 16; ++v) oacc[e][v] *= alpha;
    }
    float ps = 0.f;
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      f32x16_t p;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        p[v] = fast_exp2(fmaf(sc[j][v], c2, -mc));
        ps += p[v];
      }
      // Two 16-key steps x four 32-dim blocks; one address add per dim block,
      // the key offsets are immediates.
      bf16x8_t pb[2];
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        f32x8_t pf;
#pragma unroll
        for (int q = 0; q < 8; ++q) pf[q] = p[8 * cc + q];
        pb[cc] = __builtin_convertvector(pf, bf16x8_t);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const unsigned char* ve = vb[j] + voff[e];
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          // slots 0-3: keys 16cc+4hh+0..3, slots 4-7: keys 16cc+8+4hh+0..3
          const i16x4_t lo = lds_read_tr16(ve + 16 * cc * kRow);
          const i16x4_t hi = lds_read_tr16(ve + (16 * cc + 8) * kRow);
          const i16x8_t a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          oacc[e] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                            pb[cc], oacc[e], 0, 0, 0);
        }
      }
    }
    l_run = fmaf(l_run, alpha, ps);
  };

  // Pipeline: stage it is computed while stages it+1 .. it+NS-2 are in
  // flight; stage it+NS-1 goes to slot (it-1) % NS, which every wave finished
  // reading before the barrier of stage it.  Each wave takes TPW consecutive
  // tiles per stage: all their scores first, then one softmax over them and
  // the PV of each, in one basic block, so the scheduler can fill the MFMA
  // chains of one tile with the VALU work of the other.
  // The query (and mask) loads precede stage 0, so the first stage wait
  // retires them.
  uint32_t mw[4] = {0u, 0u, 0u, 0u};   // MR: this lane's mask row, 32 nodes per dword
  bool tree_bad = false;               // built mask: the sequence's parents are invalid
  const bool early = sparse_tree && n_pre >= kDepth * kTilesPerStage;
  if (early) {
    issue_aux();
    issue_q();
#pragma unroll
    for (int k = 0; k < kDepth; ++k) issue_stage(k);
  }
  if (sparse_tree) gather_setup();
  const int n_log = max(1, n_pre + (gather ? n_gt : n_act));
  const int n_iter = (n_log + kTilesPerStage - 1) / kTilesPerStage;
  TA_TL(14, (unsigned long long)n_log | ((unsigned long long)b << 16) |
                ((unsigned long long)g << 24) | ((unsigned long long)s << 32));
  if (!early) {
    issue_aux();
    issue_q();
#pragma unroll
    for (int k = 0; k < kDepth; ++k)
      if (k < n_iter) issue_stage(k);
  }
  if constexpr (MR) {
    if (P.build) {
      // Wave 0's parent loads were issued first: wait for them alone (the
      // query and stage loads issued after them stay in flight), share them
      // through the barrier, and build the rows while the first stages load.
      constexpr int kQLoads = RG * 8 / NW;
      const int staged = n_iter < kDepth ? n_iter : kDepth;   // stages issued so far
      if (staged >= 2)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm<kQLoads + 2 * kLoads>());
      else if (staged == 1)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm<kQLoads + kLoads>());
      else
        __builtin_amdgcn_s_waitcnt(vmcnt_imm<kQLoads>());
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      // Ancestor rows from the parents (scope of tree_attn_build_mask):
      // node i sees itself and every node on its path to the root, in
      // whatever order the nodes are listed.  A tree is valid iff every
      // parent is -1 or another node of the sequence and no chain of
      // parents is longer than the sequence (no cycle); each wave checks
      // the whole sequence, so all agree.  An invalid tree gets all-zero
      // rows, depth -1 and status 2.
      const int32_t* par = reinterpret_cast<const int32_t*>(aux);
      bool bad = false;
      for (int h = 0; h * 64 < sq.nn; ++h) {
        const int k = h * 64 + lane;
        if (k < sq.nn) {
          const int p = par[k];
          bad = bad || p < -1 || p >= sq.nn || p == k;
        }
      }
      bad = __ballot(bad) != 0;
      if (!bad) {
        for (int h = 0; h * 64 < sq.nn; ++h) {
          const int k = h * 64 + lane;
          int steps = 0;
          for (int cur = k < sq.nn ? par[k] : -1; cur >= 0 && steps <= sq.nn; cur = par[cur])
            ++steps;
          bad = bad || steps > sq.nn;
        }
        bad = __ballot(bad) != 0;
      }
      uint64_t lo = 0, hi = 0;
      if (!bad) {
        for (int cur = node; cur >= 0; cur = par[cur]) {   // ends: the parents form a forest
          if (cur < 64)
            lo |= 1ull << cur;
          else
            hi |= 1ull << (cur - 64);
        }
      }
      mw[0] = (uint32_t)lo;
      mw[1] = (uint32_t)(lo >> 32);
      mw[2] = (uint32_t)hi;
      mw[3] = (uint32_t)(hi >> 32);
      tree_bad = bad;
    }
  }
  int slot = 0;   // it % NS, kept in a scalar register
  for (int it = 0; it < n_iter; ++it) {
    wait_stage(it, n_iter);
    if (it == 0) TA_TL(2, TA_TL_NOW());
    if (it == 0) {
      const unsigned char* qb = lds + Map::kQOff + rg * 32 * kRow;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        qf[i] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(qb + koff[i]));
      if constexpr (MR) {
        if (!P.build) {
#pragma unroll
          for (int d = 0; d < 4; ++d)
            mw[d] = d < 2 * P.W ? *reinterpret_cast<const uint32_t*>(aux + wave * 1024 + d * 256 +
                                                                     lane * 4)
                                : 0u;
        }
      }
      if (Map::kQAlias) {
        // The last ring slot holds the query block: every wave has its rows
        // in registers before stage NS-1 is issued over it.
        __builtin_amdgcn_s_waitcnt((63 & 15) | ((63 >> 4) << 14) | (7 << 4));   // lgkmcnt(0)
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
      }
    }
    if (it + kDepth < n_iter) issue_stage(it + kDepth);
    // Stage base as one uniform value, so each LDS read needs one add.
    const unsigned char* st = lds + __builtin_amdgcn_readfirstlane(slot * kStage);
    slot = (slot + 1 == NS) ? 0 : slot + 1;
    f32x16_t sc[TPW];
    int tl[TPW];
    bool ac[TPW];
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      tl[j] = phys((it * KG + kg) * TPW + j);
      ac[j] = group_active && is_active(tl[j]);
      // Unconditional, so the MFMA chains of the wave's tiles share one basic
      // block (an idle tile's scores come from in-bounds rows and are dropped).
      sc[j] = qk(st + (kg * TPW + j) * kTileBytes);
    }
    bool any = false;
    const unsigned char* vbs[TPW];
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      any = any || ac[j];
      uint32_t mbits;
      if constexpr (MR) {
        const int d = tl[j] - Lt;   // uniform; only tree tiles (d >= 0) use the bits
        mbits = d <= 0 ? mw[0] : d == 1 ? mw[1] : d == 2 ? mw[2] : mw[3];
      } else if (SKIP && tl[j] >= kGath) {
        mbits = row_ok ? s_gbits[(node - g_lo) * n_gt + (tl[j] - kGath)] : 0u;
      } else {
        mbits = *reinterpret_cast<const uint32_t*>(st + kMaskOff + (wave * TPW + j) * 256 +
                                                   lane * 4);
      }
      mask_tile(sc[j], tl[j], mbits, ac[j]);
      vbs[j] = st + (kg * TPW + j) * kTileBytes + kTileKV;
    }
    if (any) softmax_pv(sc, vbs);
  }
  TA_TL(3, TA_TL_NOW());
  if (MR && P.build && g == 0 && s == 0) {
    // One writer per node: the workgroups of KV head 0 and split 0, the lane
    // holding the node's first query head.  An invalid tree's rows are zero,
    // so its depths come out as -1.
    if (row_ok && my_row % P.G == 0) {
      uint64_t* mo = P.mask_out + (size_t)(sq.n0 + node) * P.W;
      const uint64_t lo = (uint64_t)mw[1] << 32 | mw[0];
      const uint64_t hi = (uint64_t)mw[3] << 32 | mw[2];
      mo[0] = lo;
      if (P.W > 1) mo[1] = hi;
      if (P.depth_out) P.depth_out[sq.n0 + node] = __popcll(lo) + __popcll(hi) - 1;
    }
    if (r == 0 && tid == 0 && P.status_out)
      P.status_out[b] = tree_bad ? TA_ERR_INVALID_TREE : 0;
  }
  // Split partials: this lane's largest |O| (un-normalised), for the scale
  // of its row's stored partial (see the partial stores below).
  float mx = 0.f;
  if (rgn.Sb > 1) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, fabsf(oacc[e][v]));
  }
  __syncthreads();

  // Dim blocks (32 dims each) this wave combines and stores.
  bool keep_lo = true, keep_hi = true;
  // Split partials: a bound on the row's normalised |O| (no smaller than any
  // of its values), from which the row's scale is taken.
  auto ratio = [&](float mxl, float ll) {
    const float lr = row_sum(ll);
    return lr > 0.f ? row_max(mxl) * __builtin_amdgcn_rcpf(lr) : 0.f;
  };
  float bound = 0.f;
  if constexpr (KG == 1) {
    if (rgn.Sb > 1) bound = ratio(mx, l_run);
  }
  if constexpr (KG > 1) {
    // The two key groups of a row group swap halves through LDS (the stage
    // buffers are free now): wave kg keeps dim blocks 2kg, 2kg+1, hands the
    // other two to its partner with its running max and sum, and both
    // combine and store half of the rows' dims.  Layout [rg][kg][v][lane].
    static_assert(KG == 2, "key groups are merged in pairs");
    // Each lane's 32 values sit in one row of 9 float4 (32 values and 4
    // pad floats): 16-byte accesses, and consecutive lanes start on distinct
    // banks.
    constexpr int kRowF4 = 9;
    f32x4_t* xo = reinterpret_cast<f32x4_t*>(lds);
    float* xm = reinterpret_cast<float*>(xo + RG * 2 * 64 * kRowF4);
    float* xl = xm + RG * 2 * 64;
    float* xx = xl + RG * 2 * 64;
    const int mine = rg * 2 + kg;
    const int other = rg * 2 + (kg ^ 1);
    // Register arrays are only ever indexed with constants (a runtime index
    // would move them to scratch memory), hence the per-key-group branches.
    auto put4 = [&](int e2, int q, const f32x16_t& src) {
      xo[(mine * 64 + lane) * kRowF4 + 4 * e2 + q] =
          f32x4_t{src[4 * q], src[4 * q + 1], src[4 * q + 2], src[4 * q + 3]};
    };
    if (group_active) {
      if (kg == 0) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          put4(0, q, oacc[2]);
          put4(1, q, oacc[3]);
        }
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          put4(0, q, oacc[0]);
          put4(1, q, oacc[1]);
        }
      }
      xm[mine * 64 + lane] = m_run;
      xl[mine * 64 + lane] = l_run;
      xx[mine * 64 + lane] = mx;
    }
    __syncthreads();
    const float m1 = xm[other * 64 + lane];
    const float l1 = xl[other * 64 + lane];
    // The combined row is a convex combination of the two key groups'
    // normalised rows, so the larger of their bounds bounds it.
    if (rgn.Sb > 1) bound = fmaxf(ratio(mx, l_run), ratio(xx[other * 64 + lane], l1));
    const float mm = fmaxf(m_run, m1);
    const float mu = (mm == kNegInf) ? 0.f : mm;
    const float a0 = fast_exp2((m_run - mu) * c2);
    const float a1 = fast_exp2((m1 - mu) * c2);
    auto get4 = [&](int e2, int q, f32x16_t& dst) {
      const f32x4_t t = xo[(other * 64 + lane) * kRowF4 + 4 * e2 + q];
#pragma unroll
      for (int x = 0; x < 4; ++x) dst[4 * q + x] = dst[4 * q + x] * a0 + t[x] * a1;
    };
    if (!group_active) {
      // idle row group: nothing to combine (its outputs are never written)
    } else if (kg == 0) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        get4(0, q, oacc[0]);
        get4(1, q, oacc[1]);
      }
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        get4(0, q, oacc[2]);
        get4(1, q, oacc[3]);
      }
    }
    l_run = l_run * a0 + l1 * a1;
    m_run = mm;
    keep_lo = kg == 0;
    keep_hi = kg == 1;
  }

  // No wave leaves early from here on: with the in-kernel merge every wave
  // takes part in the arrival barrier below.
  const float l_tot = row_sum(l_run);
  if (!(group_active && row_ok)) keep_lo = keep_hi = false;
  // Accumulator v of oacc[e] holds dim 32e + 8*(v/4) + 4*hh + v%4 of this row.
  if (rgn.Sb == 1) {
    const float inv = 1.f / l_tot;
    uint16_t* orow = P.out + ((size_t)(sq.n0 + node) * P.Hq + head) * kD;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (!(e < 2 ? keep_lo : keep_hi)) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f32x4_t f;
#pragma unroll
        for (int x = 0; x < 4; ++x) f[x] = oacc[e][4 * j + x] * inv;
        const bf16x4_t h4 = __builtin_convertvector(f, bf16x4_t);
        *reinterpret_cast<u32x2_t*>(orow + 32 * e + 8 * j + 4 * hh) = __builtin_bit_cast(u32x2_t, h4);
      }
    }
    if (P.lse && hh == 0 && keep_lo)
      P.lse[(size_t)(sq.n0 + node) * P.Hq + head] = m_run * P.scale + logf(l_tot);
  } else {
    // Normalised partial O (the merge reweights by l), lane-major so each
    // store instruction writes 512 contiguous bytes, in fp16 times 2^k, the
    // row's scale: k puts the row's bound in [2^kPartialExp, 2^(kPartialExp+1)),
    // so no value overflows and each keeps 11 significant bits (a split over a
    // few keys averages a few value rows, up to ~4 in size, where a bf16
    // rounding would already cost 0.0078).  k + 128 rides in the low 8 bits
    // of the stored sum.  Streaming stores: the partials are read once (by
    // the merge), so they should not sit dirty in L2 when this kernel ends.
    const int eb = (int)((__float_as_uint(bound) >> 23) & 255u);
    const int k = min(126, max(-126, 127 + kPartialExp - eb));
    const float inv =
        l_tot > 0.f ? __uint_as_float((uint32_t)(127 + k) << 23) / l_tot : 0.f;
    auto put = [&](u32x2_t* p, u32x2_t v) { __builtin_nontemporal_store(v, p); };
    u32x2_t* wo = P.ws_o + ((size_t)item * RG + rg) * 16 * 64 + lane;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (!(e < 2 ? keep_lo : keep_hi)) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f32x4_t f;
#pragma unroll
        for (int x = 0; x < 4; ++x) f[x] = oacc[e][4 * j + x] * inv;
        put(&wo[(4 * e + j) * 64], __builtin_bit_cast(u32x2_t, __builtin_convertvector(f, f16x4_t)));
      }
    }
    if (hh == 0 && keep_lo) {
      const float l_k = __uint_as_float((__float_as_uint(l_tot) & ~255u) | (uint32_t)(k + 128));
      put(reinterpret_cast<u32x2_t*>(P.ws_ml + (size_t)item * P.rows_wg + rg * 32 + l32),
          __builtin_bit_cast(u32x2_t, make_float2(m_run, l_k)));
    }
    if (grp_word) {
      // Arrival: every thread's partial is in this XCD's L2 (its stores are
      // acknowledged) before the group's counter moves.
      TA_TL(7, TA_TL_NOW());
      __builtin_amdgcn_s_waitcnt(vmcnt_imm<0>());
      __syncthreads();
      // The epoch was requested before the key loop; the empty asm keeps the
      // compiler from computing the tag (and so waiting for the load) there.
      asm volatile("" : "+v"(epoch));
      if (tid == 0)
        __hip_atomic_fetch_add(grp_word, arrival_word(xcc_id(), epoch), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
      TA_TL(4, TA_TL_NOW());
    }
  }
  TA_TL(5, TA_TL_NOW());
}

// Separate merge kernel: one workgroup per (sequence, KV head, row tile, row
// group); wave j takes the 8-dim slice j of each of the four 32-dim blocks, so
// every thread has four partial loads per split in flight.
template <int RG>
__global__ __launch_bounds__(256) void merge_bf16_kernel(KParams P) {
  long long t = blockIdx.x;
  const int rg = (int)(t % RG);
  t /= RG;
  const int r = (int)(t % P.R);
  t /= P.R;
  const int g = (int)(t % P.Hkv);
  const int b = (int)(t / P.Hkv);
  const int lane = threadIdx.x & 63;
  const int j = threadIdx.x >> 6;
  const int hh = lane >> 5;
  const int rl = rg * 32 + (lane & 31);
  const long long item0 = item_index(P, b, g, 0, r);
  const long long split_stride = item_index(P, b, g, 1, r) - item0;

  // The partial slots do not depend on the offsets: with equal prefix
  // lengths (every group split alike) issue the loads of the first kPre
  // splits before decoding the sequence, so both round trips overlap.  Slots
  // past this row tile's split count are never written by this call and are
  // ignored below.  A ragged batch leaves many groups whole (nothing to
  // merge), so there the loads wait for the decode instead of fetching slots
  // no one wrote.
  constexpr int kPre = 8;
  float2 ml[kPre];
  u32x2_t h[kPre][4];
  auto oslot = [&](long long it, int e) {
    return (((size_t)it * RG + rg) * 16 + 4 * e + j) * 64 + lane;
  };
  auto load_first = [&](int n) {
#pragma unroll
    for (int k = 0; k < kPre; ++k) {
      if (k < n) {
        const long long it = item0 + k * split_stride;
        ml[k] = P.ws_ml[(size_t)it * P.rows_wg + rl];
#pragma unroll
        for (int e = 0; e < 4; ++e) h[k][e] = P.ws_o[oslot(it, e)];
      }
    }
  };
  const bool early = P.piece == 0;
  if (early) load_first(P.S);

  Seq sq;
  if (!decode_seq(P, b, sq)) return;
  Range rgn;
  if (!row_tile_range(P, sq, r, rgn)) return;
  if (rgn.Sb <= 1 || rl >= rgn.rows_here) return;
  const float c2 = P.scale_log2;
  const int Sb = rgn.Sb;
  if (!early) load_first(Sb);

  MergeAcc ma[4];
#pragma unroll
  for (int k = 0; k < kPre; ++k)
    if (k < Sb)
#pragma unroll
      for (int e = 0; e < 4; ++e) ma[e].add(ml[k], h[k][e], c2);
  // The rest kPre splits at a time, each batch requested before it is used.
  for (int s0 = kPre; s0 < Sb; s0 += kPre) {
#pragma unroll
    for (int k = 0; k < kPre; ++k) {
      if (s0 + k < Sb) {
        const long long it = item0 + (s0 + k) * split_stride;
        ml[k] = P.ws_ml[(size_t)it * P.rows_wg + rl];
#pragma unroll
        for (int e = 0; e < 4; ++e) h[k][e] = P.ws_o[oslot(it, e)];
      }
    }
#pragma unroll
    for (int k = 0; k < kPre; ++k)
      if (s0 + k < Sb)
#pragma unroll
        for (int e = 0; e < 4; ++e) ma[e].add(ml[k], h[k][e], c2);
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) store_merged(P, sq, g, r, rl, e, j, hh, ma[e]);
}

template <int RG, int KG, int TPW, int NS, bool MR, bool SKIP = false>
hipError_t launch_shape(const KParams& kp, long long grid, long long merge_grid, hipStream_t stream) {
  const size_t lds = LdsMap<RG, KG, TPW, NS, MR>::kBytes;
  if (lds > 64 * 1024) {
    hipError_t e = raise_dynamic_lds(
        reinterpret_cast<const void*>(&fwd_bf16_kernel<RG, KG, TPW, NS, MR, SKIP>), (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((fwd_bf16_kernel<RG, KG, TPW, NS, MR, SKIP>), dim3((unsigned)grid),
                     dim3(RG * KG * 64), lds, stream, kp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || merge_grid == 0) return e;
  hipLaunchKernelGGL((merge_bf16_kernel<RG>), dim3((unsigned)merge_grid), dim3(256), 0, stream, kp);
  return hipGetLastError();
}

// Largest in-kernel merge grid: half of MI355X's 256 CUs (checked against the
// device's CU count at launch).
constexpr long long kMaxMergeBlocks = 128;
// Bytes of the counter block at the start of a workspace that holds partials
// (status word and per-group words of the in-kernel merge).
constexpr size_t kCounterBytes = kFwdCounterBytes;

// Pieces per CU for ragged batches (see plan_forward_bf16); measured on the
// 32-sequence batch: 1 beats 2, 3 and 4 (each piece pays its own first-data
// latency and partial).
constexpr long long kItemsPerCU = 1;

int pow2_ceil(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

}  // namespace

FwdPlan plan_forward_bf16(int B, int total_nodes, int max_nodes, int Hq, int Hkv,
                          long long total_prefix, long long max_prefix) {
  (void)total_nodes;
  FwdPlan p{};
  const int G = Hq / Hkv;
  const long long rows_max = (long long)max_nodes * G;
  if (rows_max <= 128) {
    p.rg = pow2_ceil((int)((rows_max + 31) / 32));
    p.kg = 2;
  } else {
    // Many row tiles already fill the chip: one key group, 256-row tiles.
    // Few: 128-row tiles with two key groups halve the split partials.
    const long long units8 = (long long)B * Hkv * ((rows_max + 255) / 256);
    p.rg = units8 >= 128 ? 8 : 4;
    p.kg = units8 >= 128 ? 1 : 2;
  }
  p.nwaves = p.rg * p.kg;
  p.rows_wg = 32 * p.rg;
  p.R = (int)((rows_max + p.rows_wg - 1) / p.rows_wg);
  p.tmax = (int)((max_prefix + kKT - 1) / kKT + (max_nodes + kKT - 1) / kKT);
  // Splits.  Equal prefix lengths: aim for one full round of workgroups
  // (MI355X's 256 CUs), every sequence split alike.  Ragged prefix lengths:
  // cut every sequence into pieces of about the same number of tiles, sized
  // so the whole workload makes about kItemsPerCU pieces per CU; with one row
  // tile and at most 64 sequences the workgroups then take the pieces
  // longest first (lpt_piece), which balances the XCDs and keeps the long
  // pieces from starting last.  Keep at least two iterations per split.
  const long long units = (long long)B * Hkv * p.R;
  const bool ragged = max_prefix * B > total_prefix + total_prefix / 4;
  long long S;
  p.piece = 0;
  if (ragged) {
    const long long tiles = (total_prefix + (long long)B * (kKT - 1)) / kKT +
                            (long long)B * ((max_nodes + kKT - 1) / kKT);   // all sequences
    const long long pieces = 256LL * kItemsPerCU;
    const long long piece = std::max<long long>(
        2 * p.kg, (tiles * Hkv * p.R + pieces - 1) / pieces);
    p.piece = (int)std::min<long long>(piece, p.tmax);
    S = (p.tmax + p.piece - 1) / p.piece;
  } else {
    S = (256 + units - 1) / units;
  }
  S = std::min<long long>(S, std::max(1, p.tmax / (2 * p.kg)));
  p.S = (int)std::max<long long>(1, S);
  p.n_items = units * p.S;
  p.groups = units;
  p.merge_wpg = 16 / p.kg;   // RG*16 (row group, dim block, slice) units over RG*KG waves
  // Merge in the same kernel when the merge workgroups are few: they then
  // never occupy more than half of the CUs, so the splits they wait for
  // always find room to run.
  // Each XCD must hold whole (sequence, KV head) blocks of items, and the
  // arrival word counts at most 127 splits per XCD.
  p.merge_in_kernel = p.S > 1 && p.S <= 32 && p.groups * p.merge_wpg <= kMaxMergeBlocks &&
                      ((long long)B * Hkv) % 8 == 0 &&
                      kGroupBase + p.groups * kGroupBytes <= (long long)kCounterBytes;
  p.lpt = p.piece > 0 && p.R == 1 && B <= 64 && !p.merge_in_kernel;
  p.ws_bytes = 0;
  if (p.S > 1) {
    // [counter block | O partials | max and sum partials].
    // The counter block (status word, per-group words) leads every
    // workspace that holds partials, whichever merge runs, so a buffer
    // shared by calls of different shapes never has partials written over
    // the counters (every completed call leaves the arrival and done words
    // at zero; an epoch word is only ever compared with itself).
    p.ws_bytes = kCounterBytes + (size_t)p.n_items * p.rows_wg * (kD * 2 + 8);
  }
  return p;
}

hipError_t launch_forward_bf16(const FwdArgs& a, const FwdPlan& p, hipStream_t stream) {
  KParams kp{};
  kp.q = static_cast<const uint16_t*>(a.q);
  kp.k_tree = static_cast<const uint16_t*>(a.k_tree);
  kp.v_tree = static_cast<const uint16_t*>(a.v_tree);
  kp.k_prefix = static_cast<const uint16_t*>(a.k_prefix);
  kp.v_prefix = static_cast<const uint16_t*>(a.v_prefix);
  kp.prefix_offsets = a.prefix_offsets;
  kp.prefix_lens = a.prefix_lens;
  kp.node_offsets = a.node_offsets;
  kp.mask = a.mask;
  kp.out = static_cast<uint16_t*>(a.out);
  kp.lse = a.lse;
  kp.parents = a.parents;
  kp.mask_out = a.mask_out;
  kp.depth_out = a.depth_out;
  kp.status_out = a.status_out;
  kp.build = a.build_mask ? 1 : 0;
  // Mask rows in registers: required when the rows are built here; for a
  // given mask they pay off only on the eight-row-block shape (measured: a
  // few per cent faster there, slower on the smaller shapes, whose extra
  // scalar spills cost more than the mask DMA they save).
  if (a.build_mask && a.W > 2) return hipErrorInvalidValue;
  const bool mr = a.build_mask || (a.W <= 2 && p.rg == 8);
  long long merge_blocks = 0;
  if (p.S > 1) {
    unsigned char* ws = static_cast<unsigned char*>(a.workspace);
    kp.ws_o = reinterpret_cast<u32x2_t*>(ws + kCounterBytes);
    kp.ws_ml = reinterpret_cast<float2*>(ws + kCounterBytes +
                                         (size_t)p.n_items * p.rows_wg * kD * 2);
    // The in-kernel merge relies on the 8-XCD round-robin dealing of
    // MI355X (256 CUs); elsewhere the separate merge kernel runs.
    if (p.merge_in_kernel && device_cu_count() == 256) {
      kp.cnt = reinterpret_cast<unsigned long long*>(ws);
      kp.merge_status = a.merge_status ? a.merge_status : reinterpret_cast<unsigned int*>(ws);
      merge_blocks = p.groups * p.merge_wpg;
      kp.head_major = 1;
    }
  }
  kp.merge_wpg = p.merge_wpg;
  kp.piece = p.piece;
  // The in-kernel merge needs its own item placement; lpt never comes with it.
  kp.lpt = p.lpt && !kp.head_major ? 1 : 0;
  kp.B = a.B;
  kp.groups = p.groups;
  kp.total_prefix = a.total_prefix;
  kp.max_prefix = a.max_prefix;
  kp.n_items = p.n_items;
  kp.total_nodes = a.total_nodes;
  kp.max_nodes = a.max_nodes;
  kp.Hq = a.Hq;
  kp.Hkv = a.Hkv;
  kp.G = a.Hq / a.Hkv;
  kp.W = a.W;
  kp.rows_wg = p.rows_wg;
  kp.R = p.R;
  kp.S = p.S;
  kp.tmax = p.tmax;
  kp.scale = a.scale;
  kp.scale_log2 = a.scale * kLog2e;
  kp.n_split_blocks = (p.n_items + 7) / 8 * 8;
  const long long grid = kp.n_split_blocks + merge_blocks;
  const long long merge_grid =
      (p.S > 1 && merge_blocks == 0) ? (long long)a.B * a.Hkv * p.R * p.rg : 0;
  // Tile skipping where tree tiles are at least an eighth of the key tiles
  // (measured: on 512-node trees over 16K-key prefixes, 3% tree tiles, the
  // skipping variant of the loop ran 5% slower, on 4096-node trees over 1K
  // keys 24% faster).
  const int tree_tiles = (a.max_nodes + kKT - 1) / kKT;
  const bool skip = !mr && a.max_nodes > 128 && 8LL * tree_tiles >= p.tmax;
  switch (p.rg * 16 + p.kg) {
    // A three-stage ring measured as fast as four on every shape here.  With
    // MR the mask rows (at most 128 nodes) sit in registers.
    case 1 * 16 + 2: return mr   ? launch_shape<1, 2, 1, 3, true>(kp, grid, merge_grid, stream)
                           : skip ? launch_shape<1, 2, 1, 3, false, true>(kp, grid, merge_grid, stream)
                                  : launch_shape<1, 2, 1, 3, false>(kp, grid, merge_grid, stream);
    case 2 * 16 + 2: return mr   ? launch_shape<2, 2, 1, 3, true>(kp, grid, merge_grid, stream)
                           : skip ? launch_shape<2, 2, 1, 3, false, true>(kp, grid, merge_grid, stream)
                                  : launch_shape<2, 2, 1, 3, false>(kp, grid, merge_grid, stream);
    case 4 * 16 + 2: return mr   ? launch_shape<4, 2, 1, 3, true>(kp, grid, merge_grid, stream)
                           : skip ? launch_shape<4, 2, 1, 3, false, true>(kp, grid, merge_grid, stream)
                                  : launch_shape<4, 2, 1, 3, false>(kp, grid, merge_grid, stream);
    case 8 * 16 + 1: return mr   ? launch_shape<8, 1, 2, 3, true>(kp, grid, merge_grid, stream)
                           : skip ? launch_shape<8, 1, 2, 3, false, true>(kp, grid, merge_grid, stream)
                                  : launch_shape<8, 1, 2, 3, false>(kp, grid, merge_grid, stream);
    default: return hipErrorInvalidValue;
  }
}

#ifdef TA_TIMELINE
// Points the timeline at `buf` (cap workgroups of 16 uint64 slots), or turns
// it off (buf null).  Synchronous; returns 0 or the HIP error.
extern "C" __attribute__((visibility("default"))) int ta_timeline_set(unsigned long long* buf,
                                                                      long long cap) {
  hipError_t e = hipMemcpyToSymbol(HIP_SYMBOL(g_timeline), &buf, sizeof(buf));
  if (e == hipSuccess) e = hipMemcpyToSymbol(HIP_SYMBOL(g_timeline_cap), &cap, sizeof(cap));
  return (int)e;
}
#endif

}  // namespace ta
