// Greedy tree verification.
//
// Follows "Tree Attention" (inferensys.com glossary), Multi-Token Acceptance &
// Rollback and Integration with Speculative Decoding: after the verification
// pass, the longest branch from the root whose draft tokens the target agrees
// with is accepted.  The premlal listing (verify_candidate_tree) takes the
// target's argmax per position and compares it with the draft token; it scans
// the flattened order, which is a root path only for a chain.  Here every node
// is tested on its own root path instead.
//
// Two kernels:
//   argmax_partial_kernel  streams the [sum_N][V] logits once (the only large
//       input; bound by HBM bandwidth).  Each workgroup scans one vocabulary
//       chunk of one row with 16-byte loads and leaves (max value, lowest index
//       holding it).  Values are compared as floats, so -0 and +0 tie.
//   path_select_kernel  one workgroup per sequence: merges the chunk results
//       (ties -> lowest index), forms the match bit set with wavefront ballots,
//       accepts node i iff mask[i] is a subset of the match set (every node on
//       its root path matches), and picks the accepted node with the most mask
//       bits (the longest path), lowest index on ties.  The accepted path is
//       the set bits of that node's mask, each placed at its depth (the
//       popcount of its own row minus one), so root to leaf in whatever order
//       the nodes are listed.
//
// Next-token rows (tree_verify_greedy_next): row i holds the target's
// distribution of the token that follows node i, and one more row per
// sequence that of the token after the prefix.  A node's draft token is then
// checked against the prediction of its parent's row (a root's against the
// prefix row); the parent is the deepest of the node's proper ancestors.  The prediction after the accepted leaf (after the prefix
// when nothing is accepted) is the bonus token the step emits on top.
#include "internal.h"

#include <algorithm>

namespace ta {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr float kNegInf = -__builtin_inff();

__device__ inline bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

// One step of the wave reduction with a DPP lane move inside each row of 16
// lanes (CTRL: a DPP control code whose pairing covers the row).
template <int CTRL>
__device__ inline void best_dpp(float& bv, int& bi) {
  const float ov = __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(bv), CTRL, 0xf, 0xf, false));
  const int oi = __builtin_amdgcn_update_dpp(0, bi, CTRL, 0xf, 0xf, false);
  if (better(ov, oi, bv, bi)) {
    bv = ov;
    bi = oi;
  }
}

// Best (value, index) over aligned segments of cpr lanes (cpr a power of two,
// at most 64), in every lane of the segment: a butterfly over lane ^ o; the
// swaps by 1 and 2 are DPP quad moves, wider ones LDS permutes.
__device__ inline void seg_best(float& bv, int& bi, int cpr) {
  for (int o = cpr >> 1; o > 0; o >>= 1) {
    if (o == 1) {
      best_dpp<0xB1>(bv, bi);   // quad_perm [1,0,3,2] = lane ^ 1
    } else if (o == 2) {
      best_dpp<0x4E>(bv, bi);   // quad_perm [2,3,0,1] = lane ^ 2
    } else {
      const float ov = __shfl_xor(bv, o);
      const int oi = __shfl_xor(bi, o);
      if (better(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
  }
}

// Best (value, index) of the wave, in every lane.  "Larger value, then lower
// index" is a strict order, so any pairing gives the same winner: lane moves
// within each row of 16 (quad swaps by 1 and 2, then the 8- and 16-lane
// mirrors), then the four rows' winners read as uniform values.
__device__ inline void wave_best(float& bv, int& bi) {
  best_dpp<0xB1>(bv, bi);    // quad_perm [1,0,3,2]
  best_dpp<0x4E>(bv, bi);    // quad_perm [2,3,0,1]
  best_dpp<0x141>(bv, bi);   // row_half_mirror
  best_dpp<0x140>(bv, bi);   // row_mirror
  float v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bv), 0));
  int i = __builtin_amdgcn_readlane(bi, 0);
#pragma unroll
  for (int row = 1; row < 4; ++row) {
    const float rv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bv), 16 * row));
    const int ri = __builtin_amdgcn_readlane(bi, 16 * row);
    if (better(rv, ri, v, i)) {
      v = rv;
      i = ri;
    }
  }
  bv = v;
  bi = i;
}

// VEC: elements per 16-byte load (8 for bf16, 4 for fp32), or 1 for scalar
// loads when rows are not 16-byte aligned.  Each thread keeps kUnroll loads
// in flight before comparing, so one workgroup streams a whole chunk
// (kUnroll * 256 * VEC elements per pass) at full memory-level parallelism.
constexpr int kUnroll = 16;   // measured: 8 and 32 are slower on a 128256-entry row

// Rows [0, rows1) come from `logits1`, the rest from `logits2`; partial
// results go to ws[row][chunk] over both.
template <bool BF16, int VEC>
__global__ __launch_bounds__(kThreads) void argmax_partial_kernel(const void* __restrict__ logits1,
                                                                  const void* __restrict__ logits2,
                                                                  long long rows1, int V, int cpr,
                                                                  int chunk,
                                                                  float2* __restrict__ ws) {
  const long long out_row = blockIdx.x / cpr;
  const bool first = out_row < rows1;
  const void* logits = first ? logits1 : logits2;
  const long long row = first ? out_row : out_row - rows1;
  const int c = blockIdx.x % cpr;
  const int lo = c * chunk;
  const int hi = min(V, lo + chunk);
  // In-thread scans visit increasing indices, so a strict '>' keeps the
  // lowest index of equal values; starting from this thread's first index
  // with -inf keeps it for a range of -inf as well.
  float bv = kNegInf;
  int bi = 0x7fffffff;
  if (VEC > 1) {
    const int first = lo + threadIdx.x * VEC;
    if (first < hi) bi = first;
    for (int base = lo; base < hi; base += kThreads * VEC * kUnroll) {
      // Every load is issued (no branch around it), so they retire in order
      // and each compare waits only for its own load.  Past the chunk's end a
      // lane reads the chunk's last full vector again instead: those values
      // are copies of elements of this chunk under higher indices, so they
      // never change the maximum nor become the lowest index holding it.
      // (Vector rows hold a multiple of VEC elements, so hi - VEC >= lo.)
      u32x4_t u[kUnroll];
#pragma unroll
      for (int k = 0; k < kUnroll; ++k) {
        const int e = base + (k * kThreads + threadIdx.x) * VEC;
        const int ec = e < hi ? e : hi - VEC;
        if (BF16)
          u[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(
              static_cast<const uint16_t*>(logits) + row * V + ec));
        else
          u[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(
              static_cast<const float*>(logits) + row * V + ec));
      }
#pragma unroll
      for (int k = 0; k < kUnroll; ++k) {
        const int e = base + (k * kThreads + threadIdx.x) * VEC;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (BF16) {
            const float a = __uint_as_float(u[k][j] << 16);
            const float b = __uint_as_float(u[k][j] & 0xffff0000u);
            if (a > bv) { bv = a; bi = e + 2 * j; }
            if (b > bv) { bv = b; bi = e + 2 * j + 1; }
          } else {
            const float a = __uint_as_float(u[k][j]);
            if (a > bv) { bv = a; bi = e + j; }
          }
        }
      }
    }
  } else {
    if (lo + (int)threadIdx.x < hi) bi = lo + threadIdx.x;
    for (int e = lo + threadIdx.x; e < hi; e += kThreads) {
      float a;
      if (BF16)
        a = __uint_as_float((uint32_t)static_cast<const uint16_t*>(logits)[row * V + e] << 16);
      else
        a = static_cast<const float*>(logits)[row * V + e];
      if (a > bv) { bv = a; bi = e; }
    }
  }
  // Ties (including -0 == +0 and rows of -inf) resolve to the lower index at
  // every level: in-thread, across lanes, across waves, across chunks.
  wave_best(bv, bi);
  __shared__ float sv[kThreads / 64];
  __shared__ int si[kThreads / 64];
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    sv[wave] = bv;
    si[wave] = bi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kThreads / 64; ++w)
      if (better(sv[w], si[w], bv, bi)) {
        bv = sv[w];
        bi = si[w];
      }
    ws[out_row * cpr + c] = make_float2(bv, __int_as_float(bi));
  }
}

// One step of a wave's 64-bit maximum with a DPP lane move inside each row.
template <int CTRL>
__device__ inline unsigned long long max_dpp(unsigned long long x) {
  const uint32_t lo = __builtin_amdgcn_update_dpp(0, (uint32_t)x, CTRL, 0xf, 0xf, false);
  const uint32_t hi = __builtin_amdgcn_update_dpp(0, (uint32_t)(x >> 32), CTRL, 0xf, 0xf, false);
  const unsigned long long o = ((unsigned long long)hi << 32) | lo;
  return o > x ? o : x;
}

// Maximum over the wave, in every lane: the same pairings as wave_best.
__device__ inline unsigned long long wave_max_u64(unsigned long long x) {
  x = max_dpp<0xB1>(x);
  x = max_dpp<0x4E>(x);
  x = max_dpp<0x141>(x);
  x = max_dpp<0x140>(x);
  unsigned long long m = 0ull;
#pragma unroll
  for (int row = 0; row < 4; ++row) {
    const unsigned long long r =
        ((unsigned long long)(uint32_t)__builtin_amdgcn_readlane((int)(x >> 32), 16 * row) << 32) |
        (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)x, 16 * row);
    m = r > m ? r : m;
  }
  return m;
}

// Sum and maximum over each Wp-lane segment of the wave (Wp = 32 or 64), in
// every lane of the segment: DPP moves inside each 16-lane row (the pairings
// of wave_best), then the rows' results read as scalars.  No LDS permutes.
template <int CTRL>
__device__ inline int dpp_i(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xf, 0xf, false);
}
__device__ inline int seg_sum(int x, int Wp) {
  x += dpp_i<0xB1>(x);
  x += dpp_i<0x4E>(x);
  x += dpp_i<0x141>(x);
  x += dpp_i<0x140>(x);
  const int r0 = __builtin_amdgcn_readlane(x, 0), r1 = __builtin_amdgcn_readlane(x, 16);
  const int r2 = __builtin_amdgcn_readlane(x, 32), r3 = __builtin_amdgcn_readlane(x, 48);
  if (Wp == 64) return r0 + r1 + r2 + r3;
  return (threadIdx.x & 32) ? r2 + r3 : r0 + r1;
}
__device__ inline int seg_max(int x, int Wp) {
  x = max(x, dpp_i<0xB1>(x));
  x = max(x, dpp_i<0x4E>(x));
  x = max(x, dpp_i<0x141>(x));
  x = max(x, dpp_i<0x140>(x));
  const int r0 = __builtin_amdgcn_readlane(x, 0), r1 = __builtin_amdgcn_readlane(x, 16);
  const int r2 = __builtin_amdgcn_readlane(x, 32), r3 = __builtin_amdgcn_readlane(x, 48);
  if (Wp == 64) return max(max(r0, r1), max(r2, r3));
  return (threadIdx.x & 32) ? max(r2, r3) : max(r0, r1);
}
// Any lane of the segment set?
__device__ inline bool seg_any(bool b, int Wp) {
  const uint64_t bb = __ballot(b);
  if (Wp == 64) return bb != 0ull;
  return ((threadIdx.x & 32) ? (bb >> 32) : (bb & 0xffffffffull)) != 0ull;
}

// Inputs of one sequence that path_select_kernel keeps in registers: slot k
// of thread t holds item t + 256k of the chunk results, of the draft tokens
// and of the mask words.  Items past kSpec slots are read where they are used.
constexpr int kSpec = 4;

struct SeqRegs {
  float2 x[kSpec];
  int32_t d[kSpec];
  uint64_t m[kSpec];
};

__device__ inline void load_seq_regs(SeqRegs& r, const float2* ws, const int32_t* draft,
                                     const uint64_t* mask, int cpr, int W, int base, int cnt) {
#pragma unroll
  for (int k = 0; k < kSpec; ++k) {
    const int q = threadIdx.x + k * kThreads;
    if (q < cnt * cpr) r.x[k] = ws[(size_t)base * cpr + q];
    if (q < cnt) r.d[k] = draft[base + q];
    if (q < cnt * W) r.m[k] = mask[(size_t)base * W + q];
  }
}

template <bool NEXT>
__global__ __launch_bounds__(kThreads) void path_select_kernel(
    const float2* __restrict__ ws, int cpr, const int32_t* __restrict__ draft,
    const uint64_t* __restrict__ mask, const int32_t* __restrict__ node_offsets,
    int total_nodes, int max_nodes, int W, int32_t* __restrict__ target_argmax,
    int32_t* __restrict__ accept_len, int32_t* __restrict__ accept_nodes,
    int32_t* __restrict__ accept_tokens, const float2* __restrict__ ws_root,
    int32_t* __restrict__ bonus_token) {
  extern __shared__ uint64_t rows[];   // [nn][W] mask rows of the sequence
  __shared__ int32_t tgt[kLdsTreeMaxNodes];
  __shared__ uint64_t match_w[(kLdsTreeMaxNodes + 63) / 64];
  __shared__ unsigned long long red[kThreads / 64];
  __shared__ int32_t root_pred;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  // Sequence 0 starts at node 0 whenever its offsets are well formed: its
  // inputs are requested together with the offsets, so the whole kernel
  // waits on one memory round trip.
  SeqRegs r;
  if (b == 0) load_seq_regs(r, ws, draft, mask, cpr, W, 0, min(max_nodes, total_nodes));
  const int n0 = node_offsets[b];
  const int n1 = node_offsets[b + 1];
  int nn = n1 - n0;
  if (n0 < 0 || nn < 0 || nn > max_nodes || n1 > total_nodes) nn = 0;   // nothing accepted
  if (b != 0 || n0 != 0) load_seq_regs(r, ws, draft, mask, cpr, W, n0, nn);

  const int words = nn * W;
#pragma unroll
  for (int k = 0; k < kSpec; ++k) {
    const int q = tid + k * kThreads;
    if (q < words) rows[q] = r.m[k];
  }
  for (int q = tid + kSpec * kThreads; q < words; q += kThreads) rows[q] = mask[(size_t)n0 * W + q];

  // Target argmax per node: the cpr chunk results of one node sit in cpr
  // consecutive lanes of one wave (cpr is a power of two <= 64); a segmented
  // butterfly leaves the winner in the node's first lane.
  const int pairs = nn * cpr;
  auto reduce_pass = [&](int pidx, float2 x) {
    float bv = kNegInf;
    int bi = 0x7fffffff;
    if (pidx < pairs) {
      bv = x.x;
      bi = __float_as_int(x.y);
    }
    seg_best(bv, bi, cpr);
    if (pidx < pairs && (pidx & (cpr - 1)) == 0) {
      const int i = pidx / cpr;
      tgt[i] = bi;
      if (target_argmax) target_argmax[n0 + i] = bi;
    }
  };
#pragma unroll
  for (int k = 0; k < kSpec; ++k)
    if (k * kThreads < pairs) reduce_pass(tid + k * kThreads, r.x[k]);
  for (int p0 = kSpec * kThreads; p0 < pairs; p0 += kThreads) {
    const int pidx = p0 + tid;
    reduce_pass(pidx, pidx < pairs ? ws[(size_t)n0 * cpr + pidx] : make_float2(0.f, 0.f));
  }
  if (NEXT && wave == 0) {
    // The prefix row's chunks (cpr <= 64 of them) in the first wave.
    float bv = kNegInf;
    int bi = 0x7fffffff;
    if (lane < cpr) {
      const float2 x = ws_root[(size_t)b * cpr + lane];
      bv = x.x;
      bi = __float_as_int(x.y);
    }
    wave_best(bv, bi);
    if (lane == 0) root_pred = bi;
  }
  __syncthreads();

  // Match set: node i matches iff its draft token is the target's argmax.
  // Thread t, slot k holds node t + 256k, so wave w's ballot is word 4k + w.
  // Depth of node j: its row holds itself and its ancestors.
  auto depth_of = [&](int j) {
    int c = 0;
    for (int w = 0; w < W; ++w) c += __popcll(rows[j * W + w]);
    return c - 1;
  };
  auto expected = [&](int i) {
    if constexpr (NEXT) {
      // parent = the deepest proper ancestor (in whatever order the nodes
      // are listed)
      int par = -1, par_d = -1;
      for (int w = 0; w < W; ++w) {
        uint64_t mw = rows[i * W + w];
        if (w == (i >> 6)) mw &= ~(1ull << (i & 63));
        while (mw) {
          const int j = 64 * w + __builtin_ctzll(mw);
          mw &= mw - 1ull;
          const int d = depth_of(j);
          if (d > par_d) {
            par_d = d;
            par = j;
          }
        }
      }
      return par >= 0 ? tgt[par] : root_pred;
    } else {
      return tgt[i];
    }
  };
  auto match_pass = [&](int i, int32_t d) {
    const bool m = i < nn && d == expected(i < nn ? i : 0);
    const uint64_t bits = __ballot(m);
    if (lane == 0 && 64 * (i >> 6) < nn) match_w[i >> 6] = bits;
  };
#pragma unroll
  for (int k = 0; k < kSpec; ++k)
    if (k * kThreads < nn) match_pass(tid + k * kThreads, r.d[k]);
  for (int i0 = kSpec * kThreads; i0 < nn; i0 += kThreads) {
    const int i = i0 + tid;
    match_pass(i, i < nn ? draft[n0 + i] : -1);
  }
  __syncthreads();

  // Node i is accepted iff its whole root path matches (mask row within the
  // match set); the longest accepted path wins, lowest index on ties.
  unsigned long long key = 0ull;
  for (int i = tid; i < nn; i += kThreads) {
    bool ok = true;
    int len = 0;
    for (int w = 0; w < W; ++w) {
      uint64_t mw = rows[i * W + w];
      const int base = 64 * w;
      if (base >= nn) mw = 0ull;
      else if (nn - base < 64) mw &= (1ull << (nn - base)) - 1ull;
      len += __popcll(mw);
      if (mw & ~match_w[w]) ok = false;
    }
    if (ok && len > 0) {
      const unsigned long long k = ((unsigned long long)len << 32) | (0xffffffffu - (uint32_t)i);
      key = k > key ? k : key;
    }
  }
  key = wave_max_u64(key);
  if (lane == 0) red[wave] = key;
  __syncthreads();
  key = red[0];
  for (int w = 1; w < kThreads / 64; ++w) key = red[w] > key ? red[w] : key;
  const int len = (int)(key >> 32);
  const int best = (int)(0xffffffffu - (uint32_t)(key & 0xffffffffull));

  // The accepted path is the set bits of the best node's row, placed root
  // to leaf by depth (each node's depth is its position on the path, in
  // whatever order the nodes are listed) by the thread that holds its draft
  // token.
  int32_t* an = accept_nodes + (size_t)b * max_nodes;
  int32_t* at = accept_tokens + (size_t)b * max_nodes;
  for (int pos = tid; pos < max_nodes; pos += kThreads)
    if (pos >= len) {
      an[pos] = -1;
      at[pos] = -1;
    }
  if (len > 0) {
    const uint64_t* brow = rows + (size_t)best * W;
    auto place = [&](int j, int32_t d) {
      if (j >= nn) return;
      if (!((brow[j >> 6] >> (j & 63)) & 1ull)) return;
      const int pos = depth_of(j);
      an[pos] = j;
      at[pos] = d;
    };
#pragma unroll
    for (int k = 0; k < kSpec; ++k)
      if (k * kThreads < nn) place(tid + k * kThreads, r.d[k]);
    for (int j0 = kSpec * kThreads; j0 < nn; j0 += kThreads) {
      const int j = j0 + tid;
      place(j, j < nn ? draft[n0 + j] : -1);
    }
  }
  if (tid == 0) {
    accept_len[b] = len;
    if (NEXT) bonus_token[b] = len > 0 ? tgt[best] : root_pred;
  }
}

// Trees above 1024 nodes (up to TA_MAX_NODES): the path selection is spread
// over many workgroups, each taking 64 rows of one sequence (Wp lanes per row,
// Wp = the row's W words rounded up to a power of two, 32 or 64), with the
// steps and tie rules of path_select_kernel:
//   large_rows_kernel     per node: target argmax from its chunk results,
//                         depth (row popcount minus one) and, for same-row
//                         predictions, the match bit; a ballot packs each
//                         64 nodes' bits into one word of the match set.
//   large_parents_kernel  next-token rows only: per node the parent (its
//                         deepest proper ancestor, depths from LDS) and the
//                         match bit against the parent's (or the prefix's)
//                         prediction.
//   large_accept_kernel   per node: accepted iff its row lies inside the
//                         match set; (length, lowest index) keys, one atomic
//                         maximum per workgroup into the sequence's key.
//   large_place_kernel    per sequence: the best node's row, each node placed
//                         at its depth, and the outputs.
// Scratch (node-indexed, so disjoint sequences never share an entry):
// predictions, depths, match words (sequence word w of the sequence starting
// at node n0 is stored at n0 + 64w) and keys (the sequence's at n0).
constexpr int kLargeThreads = 1024;
constexpr int kLargeRows = 64;   // rows per workgroup

struct LargeScratch {
  int32_t* tgt;
  int32_t* dep;
  uint64_t* match;
  unsigned long long* key;
};

// Sequence b's first node and node count; nn = 0 when its offsets do not
// decode (nothing accepted, as in path_select_kernel).
__device__ inline void seq_range(const int32_t* node_offsets, int b, int total_nodes,
                                 int max_nodes, int& n0, int& nn) {
  n0 = node_offsets[b];
  const int n1 = node_offsets[b + 1];
  nn = n1 - n0;
  if (n0 < 0 || nn < 0 || nn > max_nodes || n1 > total_nodes || max_nodes > TA_MAX_NODES) {
    n0 = 0;
    nn = 0;
  }
}

// The match bits of the workgroup's 64 rows (flags in LDS), packed by wave 0
// into the sequence's word c.
__device__ inline void pack_match(const unsigned char* flag, uint64_t* match, int n0, int c,
                                  int nn) {
  if (threadIdx.x < 64) {
    const int i = kLargeRows * c + (int)threadIdx.x;
    const uint64_t bits = __ballot(i < nn && flag[threadIdx.x] != 0);
    if (threadIdx.x == 0) match[n0 + kLargeRows * c] = bits;
  }
}

template <bool NEXT>
__global__ __launch_bounds__(kLargeThreads) void large_rows_kernel(
    const float2* __restrict__ ws, int cpr, const int32_t* __restrict__ draft,
    const uint64_t* __restrict__ mask, const int32_t* __restrict__ node_offsets,
    int total_nodes, int max_nodes, int W, int Wp, int chunks, int32_t* __restrict__ target_argmax,
    LargeScratch sc) {
  __shared__ unsigned char flag[kLargeRows];
  const int b = blockIdx.x / chunks;
  const int c = blockIdx.x % chunks;
  int n0, nn;
  seq_range(node_offsets, b, total_nodes, max_nodes, n0, nn);
  if (kLargeRows * c >= nn) return;
  const int tid = threadIdx.x;
  const int w = tid & (Wp - 1);
  const int rpp = kLargeThreads / Wp;   // rows per pass
  const int passes = kLargeRows / rpp;  // 2 or 4
  constexpr int kMaxPasses = 4;
  // Every load first: the rows' mask words, each lane's chunk results (lane w
  // takes chunks w and w + Wp), and the draft token; rows past the sequence
  // re-read its last row and are dropped below.
  uint64_t mw[kMaxPasses];
  float2 x0[kMaxPasses], x1[kMaxPasses];
  int32_t d[kMaxPasses];
#pragma unroll
  for (int u = 0; u < kMaxPasses; ++u) {
    if (u >= passes) break;
    const int i = min(kLargeRows * c + u * rpp + tid / Wp, nn - 1);
    mw[u] = mask[(size_t)(n0 + i) * W + (w < W ? w : 0)];
    const float2* xr = ws + (size_t)(n0 + i) * cpr;
    x0[u] = xr[w < cpr ? w : 0];
    x1[u] = xr[w + Wp < cpr ? w + Wp : 0];
    d[u] = draft[n0 + i];
  }
  const uint64_t keep =
      64 * w + 64 <= nn ? ~0ull : (64 * w < nn ? (1ull << (nn - 64 * w)) - 1ull : 0ull);
#pragma unroll
  for (int u = 0; u < kMaxPasses; ++u) {
    if (u >= passes) break;
    const int i = kLargeRows * c + u * rpp + tid / Wp;
    const int len = seg_sum(__popcll(w < W ? (mw[u] & keep) : 0ull), Wp);
    float bv = kNegInf;
    int bi = 0x7fffffff;
    if (w < cpr) {
      bv = x0[u].x;
      bi = __float_as_int(x0[u].y);
    }
    if (w + Wp < cpr && better(x1[u].x, __float_as_int(x1[u].y), bv, bi)) {
      bv = x1[u].x;
      bi = __float_as_int(x1[u].y);
    }
    seg_best(bv, bi, Wp);
    if (w == 0 && i < nn) {
      sc.dep[n0 + i] = len - 1;
      sc.tgt[n0 + i] = bi;
      if (target_argmax) target_argmax[n0 + i] = bi;
      flag[i - kLargeRows * c] = !NEXT && d[u] == bi;
    }
  }
  if (c == 0 && tid == 0) sc.key[n0] = 0ull;
  if constexpr (!NEXT) {
    __syncthreads();
    pack_match(flag, sc.match, n0, c, nn);
  }
}

__device__ inline void large_root_pred(const float2* ws_root, int b, int cpr, int32_t* out) {
  // Wave 0: the prefix row's prediction (its chunk results, ties -> lowest
  // index) into *out.
  if (threadIdx.x < 64) {
    float bv = kNegInf;
    int bi = 0x7fffffff;
    if ((int)threadIdx.x < cpr) {
      const float2 x = ws_root[(size_t)b * cpr + threadIdx.x];
      bv = x.x;
      bi = __float_as_int(x.y);
    }
    wave_best(bv, bi);
    if (threadIdx.x == 0) *out = bi;
  }
}

__global__ __launch_bounds__(kLargeThreads) void large_parents_kernel(
    const int32_t* __restrict__ draft, const uint64_t* __restrict__ mask,
    const int32_t* __restrict__ node_offsets, int total_nodes, int max_nodes, int W, int Wp,
    int chunks, const float2* __restrict__ ws_root, int cpr, LargeScratch sc) {
  __shared__ int32_t dep[TA_MAX_NODES];
  __shared__ unsigned char flag[kLargeRows];
  __shared__ int32_t root_pred;
  const int b = blockIdx.x / chunks;
  const int c = blockIdx.x % chunks;
  int n0, nn;
  seq_range(node_offsets, b, total_nodes, max_nodes, n0, nn);
  if (kLargeRows * c >= nn) return;
  const int tid = threadIdx.x;
  for (int j = tid; j < nn; j += kLargeThreads) dep[j] = sc.dep[n0 + j];
  large_root_pred(ws_root, b, cpr, &root_pred);
  const int w = tid & (Wp - 1);
  const int rpp = kLargeThreads / Wp;
  const int passes = kLargeRows / rpp;
  constexpr int kMaxPasses = 4;
  uint64_t mw[kMaxPasses];
  int32_t d[kMaxPasses];
#pragma unroll
  for (int u = 0; u < kMaxPasses; ++u) {
    if (u >= passes) break;
    const int i = min(kLargeRows * c + u * rpp + tid / Wp, nn - 1);
    mw[u] = mask[(size_t)(n0 + i) * W + (w < W ? w : 0)];
    d[u] = draft[n0 + i];
  }
  const uint64_t keep =
      64 * w + 64 <= nn ? ~0ull : (64 * w < nn ? (1ull << (nn - 64 * w)) - 1ull : 0ull);
  __syncthreads();
#pragma unroll
  for (int u = 0; u < kMaxPasses; ++u) {
    if (u >= passes) break;
    const int i = kLargeRows * c + u * rpp + tid / Wp;
    // The deepest proper ancestor, as (depth, index) packed for one maximum.
    uint64_t m = w < W ? (mw[u] & keep) : 0ull;
    if ((i >> 6) == w) m &= ~(1ull << (i & 63));
    int best = -1;
    while (m) {
      const int j = 64 * w + __builtin_ctzll(m);
      m &= m - 1ull;
      best = max(best, (dep[j] << 16) | j);
    }
    best = seg_max(best, Wp);
    if (w == 0 && i < nn) {
      const int e = best >= 0 ? sc.tgt[n0 + (best & 0xffff)] : root_pred;
      flag[i - kLargeRows * c] = d[u] == e;
    }
  }
  __syncthreads();
  pack_match(flag, sc.match, n0, c, nn);
}

__global__ __launch_bounds__(kLargeThreads) void large_accept_kernel(
    const uint64_t* __restrict__ mask, const int32_t* __restrict__ node_offsets, int total_nodes,
    int max_nodes, int W, int Wp, int chunks, LargeScratch sc) {
  __shared__ uint64_t match_w[TA_MAX_NODES / 64];
  __shared__ unsigned long long red[kLargeThreads / 64];
  const int b = blockIdx.x / chunks;
  const int c = blockIdx.x % chunks;
  int n0, nn;
  seq_range(node_offsets, b, total_nodes, max_nodes, n0, nn);
  if (kLargeRows * c >= nn) return;
  const int tid = threadIdx.x;
  if (tid < W && 64 * tid < nn) match_w[tid] = sc.match[n0 + 64 * tid];
  const int w = tid & (Wp - 1);
  const int rpp = kLargeThreads / Wp;
  const int passes = kLargeRows / rpp;
  constexpr int kMaxPasses = 4;
  uint64_t mw[kMaxPasses];
#pragma unroll
  for (int u = 0; u < kMaxPasses; ++u) {
    if (u >= passes) break;
    const int i = min(kLargeRows * c + u * rpp + tid / Wp, nn - 1);
    mw[u] = mask[(size_t)(n0 + i) * W + (w < W ? w : 0)];
  }
  const uint64_t keep =
      64 * w + 64 <= nn ? ~0ull : (64 * w < nn ? (1ull << (nn - 64 * w)) - 1ull : 0ull);
  __syncthreads();
  // Accepted iff the row (cut at nn) lies inside the match set; the longest
  // accepted path wins, lowest index on ties.
  unsigned long long key = 0ull;
#pragma unroll
  for (int u = 0; u < kMaxPasses; ++u) {
    if (u >= passes) break;
    const int i = kLargeRows * c + u * rpp + tid / Wp;
    const uint64_t m = w < W ? (mw[u] & keep) : 0ull;
    const bool bad = seg_any((m & ~(m ? match_w[w] : 0ull)) != 0ull, Wp);
    const int len = seg_sum(__popcll(m), Wp);
    if (i < nn && w == 0 && !bad && len > 0) {
      const unsigned long long k = ((unsigned long long)len << 32) | (0xffffffffu - (uint32_t)i);
      key = k > key ? k : key;
    }
  }
  key = wave_max_u64(key);
  if ((tid & 63) == 0) red[tid >> 6] = key;
  __syncthreads();
  if (tid == 0) {
    for (int k = 1; k < kLargeThreads / 64; ++k) key = red[k] > key ? red[k] : key;
    if (key) atomicMax(sc.key + n0, key);
  }
}

template <bool NEXT>
__global__ __launch_bounds__(kLargeThreads) void large_place_kernel(
    const int32_t* __restrict__ draft, const uint64_t* __restrict__ mask,
    const int32_t* __restrict__ node_offsets, int total_nodes, int max_nodes, int W,
    int32_t* __restrict__ accept_len, int32_t* __restrict__ accept_nodes,
    int32_t* __restrict__ accept_tokens, const float2* __restrict__ ws_root, int cpr,
    int32_t* __restrict__ bonus_token, LargeScratch sc) {
  __shared__ uint64_t brow[TA_MAX_NODES / 64];
  __shared__ int32_t root_pred;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  int n0, nn;
  seq_range(node_offsets, b, total_nodes, max_nodes, n0, nn);
  if (NEXT) large_root_pred(ws_root, b, cpr, &root_pred);
  const unsigned long long key = nn > 0 ? sc.key[n0] : 0ull;
  const int len = (int)(key >> 32);
  const int best = (int)(0xffffffffu - (uint32_t)(key & 0xffffffffull));
  int32_t* an = accept_nodes + (size_t)b * max_nodes;
  int32_t* at = accept_tokens + (size_t)b * max_nodes;
  for (int pos = len + tid; pos < max_nodes; pos += kLargeThreads) {
    an[pos] = -1;
    at[pos] = -1;
  }
  if (len > 0) {
    // The accepted path: the best row's bits, each node placed at its depth
    // (its position on the path, in whatever order the nodes are listed).
    if (tid < W) {
      uint64_t m = 64 * tid < nn ? mask[(size_t)(n0 + best) * W + tid] : 0ull;
      if (64 * tid < nn && nn - 64 * tid < 64) m &= (1ull << (nn - 64 * tid)) - 1ull;
      brow[tid] = m;
    }
    __syncthreads();
    for (int j = tid; j < nn; j += kLargeThreads) {
      if ((brow[j >> 6] >> (j & 63)) & 1ull) {
        const int pos = sc.dep[n0 + j];
        an[pos] = j;
        at[pos] = draft[n0 + j];
      }
    }
  }
  __syncthreads();
  if (tid == 0) {
    accept_len[b] = len;
    if (NEXT) bonus_token[b] = len > 0 ? sc.tgt[n0 + best] : root_pred;
  }
}

}  // namespace

VerifyPlan plan_verify(int rows, int V, int max_nodes) {
  VerifyPlan p{};
  // One chunk is one pass of the unrolled scan (32768 entries for bf16 or
  // fp32), so each workgroup streams 64 or 128 KB; chunks per row are a power
  // of two (at most 64) for the in-wave reduction in path_select_kernel.
  const int target = kThreads * 8 * kUnroll;
  int cpr = 1;
  while (cpr < 64 && (long long)cpr * target < V) cpr <<= 1;
  int chunk = (V + cpr - 1) / cpr;
  chunk = (chunk + 7) / 8 * 8;
  p.cpr = cpr;
  p.chunk = chunk;
  p.ws_bytes = (size_t)rows * p.cpr * sizeof(float2);
  p.large = max_nodes > kLdsTreeMaxNodes;
  if (p.large) {
    // Scratch of the many-workgroup path selection, per row: prediction and
    // depth (int32), match word and key (64 bits), each array 256-aligned.
    const auto a256 = [](size_t x) { return (x + 255) & ~(size_t)255; };
    p.scratch_off = a256(p.ws_bytes);
    p.ws_bytes = p.scratch_off + 2 * a256((size_t)rows * 4) + 2 * a256((size_t)rows * 8);
  }
  return p;
}

namespace {

hipError_t launch_argmax(bool bf16, const void* logits1, long long rows1,
                         const void* logits2, long long rows2, int V, const VerifyPlan& p,
                         float2* ws, hipStream_t stream) {
  const long long rows = rows1 + rows2;
  if (rows <= 0) return hipSuccess;
  const dim3 grid((unsigned)(rows * p.cpr));
  const auto al = [](const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15) == 0; };
  const bool aligned = al(logits1) && (rows2 == 0 || al(logits2));
  if (bf16) {
    if (aligned && V % 8 == 0)
      hipLaunchKernelGGL((argmax_partial_kernel<true, 8>), grid, dim3(kThreads), 0, stream,
                         logits1, logits2, rows1, V, p.cpr, p.chunk, ws);
    else
      hipLaunchKernelGGL((argmax_partial_kernel<true, 1>), grid, dim3(kThreads), 0, stream,
                         logits1, logits2, rows1, V, p.cpr, p.chunk, ws);
  } else {
    if (aligned && V % 4 == 0)
      hipLaunchKernelGGL((argmax_partial_kernel<false, 4>), grid, dim3(kThreads), 0, stream,
                         logits1, logits2, rows1, V, p.cpr, p.chunk, ws);
    else
      hipLaunchKernelGGL((argmax_partial_kernel<false, 1>), grid, dim3(kThreads), 0, stream,
                         logits1, logits2, rows1, V, p.cpr, p.chunk, ws);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_verify(bool bf16, const void* logits, const int32_t* draft,
                         const uint64_t* mask, const int32_t* node_offsets, int B,
                         int total_nodes, int max_nodes, int V, int32_t* target_argmax,
                         int32_t* accept_len, int32_t* accept_nodes, int32_t* accept_tokens,
                         void* workspace, const VerifyPlan& p, hipStream_t stream,
                         const void* root_logits, int32_t* bonus_token) {
  float2* ws = static_cast<float2*>(workspace);
  float2* ws_root = ws + (size_t)total_nodes * p.cpr;
  const int W = (max_nodes + 63) / 64;
  // One launch over the node rows and, for next-token rows, the prefix rows.
  hipError_t e = launch_argmax(bf16, logits, total_nodes, root_logits, root_logits ? B : 0, V, p,
                               ws, stream);
  if (e != hipSuccess) return e;
  if (p.large) {
    int Wp = 1;
    while (Wp < W) Wp <<= 1;
    // Scratch laid out as plan_verify sized it, for `rows` rows (node rows,
    // and the prefix rows of next-token verification).
    const int rows = total_nodes + (root_logits ? B : 0);
    const auto a256 = [](size_t x) { return (x + 255) & ~(size_t)255; };
    unsigned char* base = static_cast<unsigned char*>(workspace) + p.scratch_off;
    LargeScratch sc;
    sc.tgt = reinterpret_cast<int32_t*>(base);
    sc.dep = reinterpret_cast<int32_t*>(base + a256((size_t)rows * 4));
    sc.match = reinterpret_cast<uint64_t*>(base + 2 * a256((size_t)rows * 4));
    sc.key = reinterpret_cast<unsigned long long*>(base + 2 * a256((size_t)rows * 4) +
                                                   a256((size_t)rows * 8));
    const int chunks = (max_nodes + kLargeRows - 1) / kLargeRows;
    const dim3 grid((unsigned)((long long)B * chunks));
    if (root_logits) {
      hipLaunchKernelGGL(large_rows_kernel<true>, grid, dim3(kLargeThreads), 0, stream, ws, p.cpr,
                         draft, mask, node_offsets, total_nodes, max_nodes, W, Wp, chunks,
                         target_argmax, sc);
      hipLaunchKernelGGL(large_parents_kernel, grid, dim3(kLargeThreads), 0, stream, draft, mask,
                         node_offsets, total_nodes, max_nodes, W, Wp, chunks, ws_root, p.cpr, sc);
    } else {
      hipLaunchKernelGGL(large_rows_kernel<false>, grid, dim3(kLargeThreads), 0, stream, ws,
                         p.cpr, draft, mask, node_offsets, total_nodes, max_nodes, W, Wp, chunks,
                         target_argmax, sc);
    }
    hipLaunchKernelGGL(large_accept_kernel, grid, dim3(kLargeThreads), 0, stream, mask,
                       node_offsets, total_nodes, max_nodes, W, Wp, chunks, sc);
    if (root_logits)
      hipLaunchKernelGGL(large_place_kernel<true>, dim3(B), dim3(kLargeThreads), 0, stream, draft,
                         mask, node_offsets, total_nodes, max_nodes, W, accept_len, accept_nodes,
                         accept_tokens, ws_root, p.cpr, bonus_token, sc);
    else
      hipLaunchKernelGGL(large_place_kernel<false>, dim3(B), dim3(kLargeThreads), 0, stream, draft,
                         mask, node_offsets, total_nodes, max_nodes, W, accept_len, accept_nodes,
                         accept_tokens, nullptr, p.cpr, nullptr, sc);
    return hipGetLastError();
  }
  const size_t lds = (size_t)max_nodes * W * sizeof(uint64_t);
  const void* kern = root_logits ? reinterpret_cast<const void*>(&path_select_kernel<true>)
                                 : reinterpret_cast<const void*>(&path_select_kernel<false>);
  if (lds > 32 * 1024) {
    e = raise_dynamic_lds(kern, (int)lds);
    if (e != hipSuccess) return e;
  }
  if (root_logits)
    hipLaunchKernelGGL(path_select_kernel<true>, dim3(B), dim3(kThreads), lds, stream, ws,
                       p.cpr, draft, mask, node_offsets, total_nodes, max_nodes, W,
                       target_argmax, accept_len, accept_nodes, accept_tokens, ws_root,
                       bonus_token);
  else
    hipLaunchKernelGGL(path_select_kernel<false>, dim3(B), dim3(kThreads), lds, stream, ws,
                       p.cpr, draft, mask, node_offsets, total_nodes, max_nodes, W,
                       target_argmax, accept_len, accept_nodes, accept_tokens, nullptr,
                       nullptr);
  return hipGetLastError();
}

}  // namespace ta
