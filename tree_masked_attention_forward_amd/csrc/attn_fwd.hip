// Tree attention forward on gfx950.
//
// What is computed ("Tree Attention", inferensys.com glossary, Modified Causal
// Attention Mask and Speculative KV Cache Reuse; "Tree Attention",
// zhongzhoutan-coder.github.io, How It Works): node i of sequence b, query
// head h, attends to all L_b prefix keys of KV head g = h / G, to itself and
// to its ancestors; softmax(scale * q.k) weights the matching values.
//
// bf16 path (D = 128).  For one (sequence, KV head) the N_b nodes times the G
// query heads that share the KV head form a dense block of N_b*G query rows
// (row = node*G + j), so every key/value row fetched from HBM is used by all
// of them: the key scan is a dense contraction on MFMA.  The work is cut into
// items (sequence, KV head, key split, row tile):
//
//   * each wave owns 32 query rows; the workgroup (up to 8 waves) shares one
//     32-key K tile and the matching V tile, staged through LDS from 16-byte
//     coalesced global loads (double buffered, one barrier per tile);
//   * scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16 (A = K from LDS, B = Q^T held in registers), so
//     each lane holds 16 keys of ONE query row and the other 16 keys of that
//     row sit in lane ^ 32: the row max needs one cross-lane step and the
//     rescale of the output accumulator is one factor per lane;
//   * online softmax in fp32 in the log2 domain (scale * log2(e) folded into
//     one FMA before v_exp_f32), probabilities rounded to bf16;
//   * O^T += V^T P^T on the same MFMA (A = V^T from LDS, stored transposed
//     when the tile is staged; B = P^T straight from the score registers);
//   * the key axis of a sequence is [prefix (padded to 32) | tree nodes]; a
//     prefix tile needs no mask; a tree tile tests bit (key) of the row's
//     node mask word (one uint64 word per 64 nodes, built by
//     tree_attn_build_mask); tiles past the row tile's last node are never
//     visited because nodes are topologically ordered;
//   * each item leaves a partial (unnormalised O, running max m, sum l); a
//     second kernel merges the partials of a row by log-sum-exp.  With a
//     single split the item writes the final output directly.
//
// fp32 path: one wave per (node, head), exact-fp32 dot products reduced
// across lanes, online softmax with expf.  A plain correctness path.
#include "internal.h"

#include <math.h>

#include <algorithm>

namespace ta {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kD = 128;                        // head size of the MFMA path
constexpr int kKT = 32;                        // keys per tile
constexpr int kKStride = kD * 2 + 16;          // LDS bytes per K row (padded: no bank conflicts)
constexpr int kVStride = kKT * 2 + 16;         // LDS bytes per V^T row
constexpr int kKTileBytes = kKT * kKStride;    // 8704
constexpr int kVTileBytes = kD * kVStride;     // 10240
constexpr int kStageBytes = kKTileBytes + kVTileBytes;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_inff();

struct KParams {
  const uint16_t* q;
  const uint16_t* k_tree;
  const uint16_t* v_tree;
  const uint16_t* k_prefix;
  const uint16_t* v_prefix;
  const int64_t* prefix_offsets;
  const int32_t* node_offsets;
  const uint64_t* mask;
  uint16_t* out;
  float* lse;
  float* ws_o;   // [n_items][rows_wg][128] unnormalised partial outputs
  float* ws_ml;  // [n_items][rows_wg][2]   (running max in score units, sum)
  long long total_prefix, max_prefix, n_items;
  int total_nodes, max_nodes;
  int Hq, Hkv, G, W;
  int rows_wg, R, S, chunk;
  float scale, scale_log2;
};

// One sequence's extents, with every offset checked against the host sizes
// so that a malformed offset array can never send a load out of bounds.
struct Seq {
  int n0, nn, L;
  long long p0;
};

__device__ inline bool decode_seq(const KParams& P, int b, Seq& s) {
  const int n0 = P.node_offsets[b];
  const int n1 = P.node_offsets[b + 1];
  const long long p0 = P.prefix_offsets[b];
  const long long p1 = P.prefix_offsets[b + 1];
  if (n0 < 0 || n1 <= n0 || n1 - n0 > P.max_nodes || n1 > P.total_nodes) return false;
  if (p0 < 0 || p1 < p0 || p1 - p0 > P.max_prefix || p1 > P.total_prefix) return false;
  s.n0 = n0;
  s.nn = n1 - n0;
  s.p0 = p0;
  s.L = (int)(p1 - p0);
  return true;
}

// Position of key k (0..31 in a tile) inside a transposed V row: within each
// 16-key group the middle two quads swap, so that the 8 keys one MFMA lane
// needs for P^T (keys 4h..4h+3 and 8+4h..8+4h+3 of the group) are contiguous.
__device__ inline int vt_pos(int k) {
  const int quad = (k >> 2) & 3;
  const int nq = (quad == 1) ? 2 : (quad == 2) ? 1 : quad;
  return (k & 16) | (nq << 2) | (k & 3);
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <int NW>
struct TileRegs {
  static constexpr int NT = NW * 64;
  static constexpr int KC = (kKT * 16 + NT - 1) / NT;  // 16-byte K chunks per thread
  static constexpr int VU = (kKT * 8 + NT - 1) / NT;   // (key pair, 8-d chunk) units per thread
  u32x4_t k[KC];
  u32x4_t v[2 * VU];
};

template <int NW>
__global__ __launch_bounds__(NW * 64) void fwd_bf16_kernel(KParams P) {
  extern __shared__ __align__(16) unsigned char lds[];
  constexpr int NT = NW * 64;
  using Regs = TileRegs<NW>;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hh = lane >> 5;   // lane half: which 8 of each 16 contraction elements
  const int l32 = lane & 31;

  // Consecutive items (same sequence and KV head) go to the same XCD: the
  // hardware deals workgroup ids round-robin over the 8 XCDs.
  const long long nb = gridDim.x;
  const long long item = (long long)(blockIdx.x & 7) * (nb >> 3) + (blockIdx.x >> 3);
  if (item >= P.n_items) return;
  const int r = (int)(item % P.R);
  long long t = item / P.R;
  const int s = (int)(t % P.S);
  t /= P.S;
  const int g = (int)(t % P.Hkv);
  const int b = (int)(t / P.Hkv);

  Seq sq;
  if (!decode_seq(P, b, sq)) return;
  const int G = P.G;
  const int rows_b = sq.nn * G;
  const int row0 = r * P.rows_wg;
  if (row0 >= rows_b) return;
  const int rows_here = min(P.rows_wg, rows_b - row0);
  const int n_hi = (row0 + rows_here - 1) / G;          // last node of this row tile
  const int L = sq.L;
  const int Lpad = (L + kKT - 1) & ~(kKT - 1);
  const int keys_total = Lpad + n_hi + 1;
  const int n_splits = (keys_total + P.chunk - 1) / P.chunk;
  if (s >= n_splits) return;
  const int k_begin = s * P.chunk;
  const int k_end = min(k_begin + P.chunk, keys_total);

  // This lane's query row.
  const int my_row = row0 + wave * 32 + l32;
  const bool row_ok = my_row < row0 + rows_here;
  const bool wave_active = wave * 32 < rows_here;
  const int node = row_ok ? my_row / G : 0;
  const int head = g * G + (row_ok ? my_row % G : 0);

  bf16x8_t qf[8];
  {
    const uint16_t* qrow = P.q + ((size_t)(sq.n0 + node) * P.Hq + head) * kD + 8 * hh;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (row_ok) v = *reinterpret_cast<const u32x4_t*>(qrow + 16 * i);
      qf[i] = __builtin_bit_cast(bf16x8_t, v);
    }
  }
  const uint64_t* mrow = P.mask + (size_t)(sq.n0 + node) * P.W;

  const size_t kv_row = (size_t)P.Hkv * kD;   // elements between consecutive key rows
  const uint16_t* kp = P.k_prefix + ((size_t)sq.p0 * P.Hkv + g) * kD;
  const uint16_t* vp = P.v_prefix + ((size_t)sq.p0 * P.Hkv + g) * kD;
  const uint16_t* kt = P.k_tree + ((size_t)sq.n0 * P.Hkv + g) * kD;
  const uint16_t* vt = P.v_tree + ((size_t)sq.n0 * P.Hkv + g) * kD;

  // Global source row of virtual key kk, or null for padding / past the end.
  auto src_row = [&](const uint16_t* pre, const uint16_t* tre, int kk) -> const uint16_t* {
    if (kk < L) return pre + (size_t)kk * kv_row;
    if (kk >= Lpad && kk < k_end) return tre + (size_t)(kk - Lpad) * kv_row;
    return nullptr;
  };

  auto load_tile = [&](int kt0, Regs& rg) {
#pragma unroll
    for (int j = 0; j < Regs::KC; ++j) {
      const int c = tid + j * NT;
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (c < kKT * 16) {
        const uint16_t* p = src_row(kp, kt, kt0 + (c >> 4));
        if (p) v = *reinterpret_cast<const u32x4_t*>(p + (c & 15) * 8);
      }
      rg.k[j] = v;
    }
#pragma unroll
    for (int j = 0; j < Regs::VU; ++j) {
      const int u = tid + j * NT;
      u32x4_t a = {0u, 0u, 0u, 0u}, c2 = {0u, 0u, 0u, 0u};
      if (u < kKT * 8) {
        const int key = 2 * (u >> 4);
        const int dc = (u & 15) * 8;
        const uint16_t* p0 = src_row(vp, vt, kt0 + key);
        const uint16_t* p1 = src_row(vp, vt, kt0 + key + 1);
        if (p0) a = *reinterpret_cast<const u32x4_t*>(p0 + dc);
        if (p1) c2 = *reinterpret_cast<const u32x4_t*>(p1 + dc);
      }
      rg.v[2 * j] = a;
      rg.v[2 * j + 1] = c2;
    }
  };

  auto store_tile = [&](unsigned char* stage, const Regs& rg) {
#pragma unroll
    for (int j = 0; j < Regs::KC; ++j) {
      const int c = tid + j * NT;
      if (c < kKT * 16)
        *reinterpret_cast<u32x4_t*>(stage + (c >> 4) * kKStride + (c & 15) * 16) = rg.k[j];
    }
    unsigned char* vs = stage + kKTileBytes;
#pragma unroll
    for (int j = 0; j < Regs::VU; ++j) {
      const int u = tid + j * NT;
      if (u < kKT * 8) {
        const int key = 2 * (u >> 4);
        const int dc = (u & 15) * 8;
        const int pos = vt_pos(key);   // key and key+1 stay adjacent
        const u32x4_t a = rg.v[2 * j];
        const u32x4_t c2 = rg.v[2 * j + 1];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t lo = (a[e] & 0xffffu) | (c2[e] << 16);
          const uint32_t hi = (a[e] >> 16) | (c2[e] & 0xffff0000u);
          *reinterpret_cast<uint32_t*>(vs + (dc + 2 * e) * kVStride + pos * 2) = lo;
          *reinterpret_cast<uint32_t*>(vs + (dc + 2 * e + 1) * kVStride + pos * 2) = hi;
        }
      }
    }
  };

  f32x16_t oacc[4];
#pragma unroll
  for (int e = 0; e < 4; ++e)
#pragma unroll
    for (int v = 0; v < 16; ++v) oacc[e][v] = 0.f;
  float m_run = kNegInf;
  float l_run = 0.f;
  const float c2 = P.scale_log2;

  const int n_tiles = (k_end - k_begin + kKT - 1) / kKT;
  Regs rg;
  load_tile(k_begin, rg);
  store_tile(lds, rg);
  __syncthreads();

  for (int it = 0; it < n_tiles; ++it) {
    const int kt0 = k_begin + it * kKT;
    unsigned char* cur = lds + (it & 1) * kStageBytes;
    unsigned char* nxt = lds + ((it + 1) & 1) * kStageBytes;
    const bool more = it + 1 < n_tiles;
    if (more) load_tile(kt0 + kKT, rg);

    if (wave_active) {
      // S^T = K Q^T for 32 keys x this wave's 32 rows.
      f32x16_t sacc;
#pragma unroll
      for (int v = 0; v < 16; ++v) sacc[v] = 0.f;
      const unsigned char* krow = cur + l32 * kKStride + 16 * hh;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const u32x4_t kv = *reinterpret_cast<const u32x4_t*>(krow + 32 * i);
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, kv), qf[i],
                                                       sacc, 0, 0, 0);
      }
      // Accumulator v of this lane holds key 8*(v/4) + 4*hh + v%4 of the tile.
      if (kt0 >= Lpad) {
        const int t0 = kt0 - Lpad;   // multiple of 32
        const uint64_t word = row_ok ? mrow[t0 >> 6] : 0ull;
        const uint32_t bits = (uint32_t)(word >> (t0 & 63));
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = 8 * (v >> 2) + 4 * hh + (v & 3);
          if (!((bits >> key) & 1u)) sacc[v] = kNegInf;
        }
      } else if (kt0 + kKT > L) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = 8 * (v >> 2) + 4 * hh + (v & 3);
          if (kt0 + key >= L) sacc[v] = kNegInf;
        }
      }
      float mt = sacc[0];
#pragma unroll
      for (int v = 1; v < 16; ++v) mt = fmaxf(mt, sacc[v]);
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      const float m_new = fmaxf(m_run, mt);
      const float m_use = (m_new == kNegInf) ? 0.f : m_new;
      const float alpha = fast_exp2((m_run - m_use) * c2);
      const float mc = m_use * c2;
      float ps = 0.f;
      f32x16_t p;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        p[v] = fast_exp2(fmaf(sacc[v], c2, -mc));
        ps += p[v];
      }
      l_run = fmaf(l_run, alpha, ps);
      m_run = m_new;
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int v = 0; v < 16; ++v) oacc[e][v] *= alpha;

      // O^T += V^T P^T, two 16-key steps.
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        f32x8_t pf;
#pragma unroll
        for (int j = 0; j < 8; ++j) pf[j] = p[8 * cc + j];
        const bf16x8_t pb = __builtin_convertvector(pf, bf16x8_t);
        const unsigned char* vrow = cur + kKTileBytes + l32 * kVStride + (16 * cc + 8 * hh) * 2;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const u32x4_t vv = *reinterpret_cast<const u32x4_t*>(vrow + 32 * e * kVStride);
          oacc[e] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, vv), pb,
                                                            oacc[e], 0, 0, 0);
        }
      }
    }
    if (more) store_tile(nxt, rg);
    __syncthreads();
  }

  if (!row_ok) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  // Accumulator v of oacc[e] holds d = 32e + 8*(v/4) + 4*hh + v%4 of this row.
  if (n_splits == 1) {
    const float inv = 1.f / l_tot;
    uint16_t* orow = P.out + ((size_t)(sq.n0 + node) * P.Hq + head) * kD;
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f32x4_t f;
#pragma unroll
        for (int x = 0; x < 4; ++x) f[x] = oacc[e][4 * j + x] * inv;
        typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
        const bf16x4_t h4 = __builtin_convertvector(f, bf16x4_t);
        *reinterpret_cast<u32x2_t*>(orow + 32 * e + 8 * j + 4 * hh) = __builtin_bit_cast(u32x2_t, h4);
      }
    if (P.lse && hh == 0) P.lse[(size_t)(sq.n0 + node) * P.Hq + head] = m_run * P.scale + logf(l_tot);
  } else {
    const size_t prow = (size_t)item * P.rows_wg + (my_row - row0);
    float* wo = P.ws_o + prow * kD;
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f32x4_t f;
#pragma unroll
        for (int x = 0; x < 4; ++x) f[x] = oacc[e][4 * j + x];
        *reinterpret_cast<f32x4_t*>(wo + 32 * e + 8 * j + 4 * hh) = f;
      }
    if (hh == 0) {
      P.ws_ml[2 * prow] = m_run;
      P.ws_ml[2 * prow + 1] = l_tot;
    }
  }
}

// Log-sum-exp merge of the split partials of one (sequence, KV head, row
// tile): with M = max_s m_s and w_s = exp(scale * (m_s - M)),
//   out = sum_s w_s O_s / sum_s w_s l_s,  lse = scale * M + log(sum_s w_s l_s).
// Splits that saw no visible key carry m = -inf and weigh nothing.
__global__ __launch_bounds__(256) void merge_bf16_kernel(KParams P) {
  const int grp = blockIdx.x;
  const int r = grp % P.R;
  const int g = (grp / P.R) % P.Hkv;
  const int b = grp / (P.R * P.Hkv);
  Seq sq;
  if (!decode_seq(P, b, sq)) return;
  const int G = P.G;
  const int rows_b = sq.nn * G;
  const int row0 = r * P.rows_wg;
  if (row0 >= rows_b) return;
  const int rows_here = min(P.rows_wg, rows_b - row0);
  const int n_hi = (row0 + rows_here - 1) / G;
  const int Lpad = (sq.L + kKT - 1) & ~(kKT - 1);
  const int n_splits = (Lpad + n_hi + 1 + P.chunk - 1) / P.chunk;
  if (n_splits <= 1) return;
  const float c2 = P.scale_log2;
  const long long item0 = ((long long)(b * P.Hkv + g) * P.S) * P.R + r;   // split s adds s*R

  for (int idx = threadIdx.x; idx < rows_here * 32; idx += blockDim.x) {
    const int rl = idx >> 5;
    const int d0 = (idx & 31) * 4;
    float M = kNegInf;
    for (int s = 0; s < n_splits; ++s) {
      const size_t prow = (size_t)(item0 + (long long)s * P.R) * P.rows_wg + rl;
      M = fmaxf(M, P.ws_ml[2 * prow]);
    }
    float lsum = 0.f;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    if (M != kNegInf) {
      for (int s = 0; s < n_splits; ++s) {
        const size_t prow = (size_t)(item0 + (long long)s * P.R) * P.rows_wg + rl;
        const float w = fast_exp2((P.ws_ml[2 * prow] - M) * c2);
        lsum = fmaf(w, P.ws_ml[2 * prow + 1], lsum);
        const f32x4_t o = *reinterpret_cast<const f32x4_t*>(P.ws_o + prow * kD + d0);
        acc += w * o;
      }
    }
    const int my_row = row0 + rl;
    const int node = my_row / G;
    const int head = g * G + my_row % G;
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
    const bf16x4_t h4 = __builtin_convertvector(acc * inv, bf16x4_t);
    *reinterpret_cast<u32x2_t*>(P.out + ((size_t)(sq.n0 + node) * P.Hq + head) * kD + d0) =
        __builtin_bit_cast(u32x2_t, h4);
    if (P.lse && d0 == 0)
      P.lse[(size_t)(sq.n0 + node) * P.Hq + head] =
          lsum > 0.f ? M * P.scale + logf(lsum) : kNegInf;
  }
}

// ------------------------------------------------------------------ fp32 path

struct F32Params {
  const float* q;
  const float* k_tree;
  const float* v_tree;
  const float* k_prefix;
  const float* v_prefix;
  const int64_t* prefix_offsets;
  const int32_t* node_offsets;
  const uint64_t* mask;
  float* out;
  float* lse;
  long long total_prefix, max_prefix;
  int B, total_nodes, max_nodes, Hq, Hkv, G, D, W;
  float scale;
};

__device__ inline float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

__global__ __launch_bounds__(256) void fwd_f32_kernel(F32Params P) {
  const int lane = threadIdx.x & 63;
  const long long wid = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wid >= (long long)P.total_nodes * P.Hq) return;
  const int gnode = (int)(wid / P.Hq);
  const int head = (int)(wid % P.Hq);
  const int g = head / P.G;
  // Sequence of this node: last b with node_offsets[b] <= gnode.
  int lo = 0, hi = P.B;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (P.node_offsets[mid] <= gnode) lo = mid; else hi = mid;
  }
  const int b = lo;
  const int n0 = P.node_offsets[b], n1 = P.node_offsets[b + 1];
  const long long p0 = P.prefix_offsets[b], p1 = P.prefix_offsets[b + 1];
  if (n0 < 0 || n1 <= n0 || n1 - n0 > P.max_nodes || n1 > P.total_nodes) return;
  if (gnode < n0 || gnode >= n1) return;
  if (p0 < 0 || p1 < p0 || p1 - p0 > P.max_prefix || p1 > P.total_prefix) return;
  const int nn = n1 - n0;
  const int D = P.D;
  float qv[4], acc[4];
  const float* qrow = P.q + ((size_t)gnode * P.Hq + head) * D;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int d = lane + 64 * j;
    qv[j] = d < D ? qrow[d] : 0.f;
    acc[j] = 0.f;
  }
  float m = kNegInf, l = 0.f;
  auto step = [&](const float* krow, const float* vrow) {
    float part = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d = lane + 64 * j;
      if (d < D) part = fmaf(qv[j], krow[d], part);
    }
    const float sc = wave_sum(part) * P.scale;
    const float m_new = fmaxf(m, sc);
    const float alpha = expf(m - m_new);
    const float p = expf(sc - m_new);
    l = l * alpha + p;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d = lane + 64 * j;
      acc[j] = acc[j] * alpha + (d < D ? p * vrow[d] : 0.f);
    }
    m = m_new;
  };
  const size_t kv_row = (size_t)P.Hkv * D;
  for (long long k = 0; k < p1 - p0; ++k)
    step(P.k_prefix + (size_t)(p0 + k) * kv_row + (size_t)g * D,
         P.v_prefix + (size_t)(p0 + k) * kv_row + (size_t)g * D);
  const uint64_t* mrow = P.mask + (size_t)gnode * P.W;
  for (int w = 0; w < P.W; ++w) {
    uint64_t bits = mrow[w];
    while (bits) {
      const int tn = 64 * w + __builtin_ctzll(bits);
      bits &= bits - 1;
      if (tn >= nn) break;
      step(P.k_tree + (size_t)(n0 + tn) * kv_row + (size_t)g * D,
           P.v_tree + (size_t)(n0 + tn) * kv_row + (size_t)g * D);
    }
  }
  float* orow = P.out + ((size_t)gnode * P.Hq + head) * D;
  const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int d = lane + 64 * j;
    if (d < D) orow[d] = acc[j] * inv;
  }
  if (P.lse && lane == 0) P.lse[(size_t)gnode * P.Hq + head] = l > 0.f ? m + logf(l) : kNegInf;
}

template <int NW>
hipError_t launch_nw(const KParams& kp, long long grid, hipStream_t stream) {
  hipLaunchKernelGGL(fwd_bf16_kernel<NW>, dim3((unsigned)grid), dim3(NW * 64), 2 * kStageBytes,
                     stream, kp);
  return hipGetLastError();
}

}  // namespace

FwdPlan plan_forward_bf16(int B, int total_nodes, int max_nodes, int Hq, int Hkv,
                          long long total_prefix, long long max_prefix) {
  FwdPlan p{};
  const int G = Hq / Hkv;
  const long long rows_max = (long long)max_nodes * G;
  p.nwaves = (int)std::min<long long>(8, (rows_max + 31) / 32);
  if (p.nwaves == 3) p.nwaves = 4;
  if (p.nwaves >= 5) p.nwaves = 8;
  p.rows_wg = 32 * p.nwaves;
  p.R = (int)((rows_max + p.rows_wg - 1) / p.rows_wg);
  const long long keys_max = ((max_prefix + kKT - 1) / kKT) * kKT + max_nodes;
  // Aim for about two workgroups per compute unit over the whole call; never
  // split below 4 tiles, never above the longest sequence.
  const long long total_keys = total_prefix + (long long)kKT * B + total_nodes;
  const long long target_items = 512;
  long long chunk = (total_keys * Hkv * p.R + target_items - 1) / target_items;
  chunk = ((chunk + kKT - 1) / kKT) * kKT;
  chunk = std::max<long long>(chunk, 4 * kKT);
  chunk = std::min<long long>(chunk, ((keys_max + kKT - 1) / kKT) * kKT);
  p.chunk = (int)chunk;
  p.S = (int)((keys_max + chunk - 1) / chunk);
  p.n_items = (long long)B * Hkv * p.S * p.R;
  p.ws_bytes = p.S > 1 ? (size_t)p.n_items * p.rows_wg * (kD + 2) * sizeof(float) : 0;
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
  kp.node_offsets = a.node_offsets;
  kp.mask = a.mask;
  kp.out = static_cast<uint16_t*>(a.out);
  kp.lse = a.lse;
  if (p.S > 1) {
    kp.ws_o = static_cast<float*>(a.workspace);
    kp.ws_ml = kp.ws_o + (size_t)p.n_items * p.rows_wg * kD;
  }
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
  kp.chunk = p.chunk;
  kp.scale = a.scale;
  kp.scale_log2 = a.scale * kLog2e;
  const long long grid = (p.n_items + 7) / 8 * 8;
  hipError_t e;
  switch (p.nwaves) {
    case 1: e = launch_nw<1>(kp, grid, stream); break;
    case 2: e = launch_nw<2>(kp, grid, stream); break;
    case 4: e = launch_nw<4>(kp, grid, stream); break;
    default: e = launch_nw<8>(kp, grid, stream); break;
  }
  if (e != hipSuccess || p.S <= 1) return e;
  const long long groups = (long long)a.B * a.Hkv * p.R;
  hipLaunchKernelGGL(merge_bf16_kernel, dim3((unsigned)groups), dim3(256), 0, stream, kp);
  return hipGetLastError();
}

hipError_t launch_forward_f32(const FwdArgs& a, hipStream_t stream) {
  F32Params fp{};
  fp.q = static_cast<const float*>(a.q);
  fp.k_tree = static_cast<const float*>(a.k_tree);
  fp.v_tree = static_cast<const float*>(a.v_tree);
  fp.k_prefix = static_cast<const float*>(a.k_prefix);
  fp.v_prefix = static_cast<const float*>(a.v_prefix);
  fp.prefix_offsets = a.prefix_offsets;
  fp.node_offsets = a.node_offsets;
  fp.mask = a.mask;
  fp.out = static_cast<float*>(a.out);
  fp.lse = a.lse;
  fp.total_prefix = a.total_prefix;
  fp.max_prefix = a.max_prefix;
  fp.B = a.B;
  fp.total_nodes = a.total_nodes;
  fp.max_nodes = a.max_nodes;
  fp.Hq = a.Hq;
  fp.Hkv = a.Hkv;
  fp.G = a.Hq / a.Hkv;
  fp.D = a.D;
  fp.W = a.W;
  fp.scale = a.scale;
  const long long waves = (long long)a.total_nodes * a.Hq;
  hipLaunchKernelGGL(fwd_f32_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, stream, fp);
  return hipGetLastError();
}

}  // namespace ta
