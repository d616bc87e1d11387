// Stochastic tree verification (rejection sampling down the tree).
//
// "Speculative Tree Attention" (news.premlal.in), Production Inference
// Runtimes: a speculative step leaves the target model's output distribution
// unchanged.  The pages give no rule; this is the published one that makes it
// so: speculative sampling's accept test and residual (Leviathan et al. 2023;
// Chen et al. 2023) walked child by child down the tree, as in SpecInfer's
// multi-step speculative sampling (Miao et al. 2024).
//
// Two kernels.  softmax_stats_kernel (four workgroups per logits row, all rows
// at once) leaves, for every row, the softmax statistics of each vocabulary
// segment: (max, sum of exp2 relative to it) in log2 units at the given
// temperature.  spec_sample_kernel (one workgroup per sequence) then walks the
// tree: the current distribution P is either a target row's softmax, kept
// implicit (its row, max and sum, merged from the segment statistics without
// touching the row), or an explicit residual in a per-sequence scratch row;
// LDS keeps P's mass per segment.  Testing child c with draft token x reads
// P(x) and the draft probability Q(x) and accepts iff u_c * Q(x) < P(x).  An
// accepted child becomes the current node (its statistics merged); a rejected
// one turns P into max(0, P - Q) renormalised (one pass over the vocabulary,
// written to the other scratch row so that P survives when the residual is
// all zero).  The bonus token is drawn from P by inversion: the segment
// holding u_final * sum(P) from the segment masses, then one wave scans that
// segment.  The walk's decisions are uniform: every thread takes them from
// values in LDS.
//
// Vocabulary layout shared by both kernels: thread t of a 1024-thread
// workgroup owns the run [t*C, t*C + C), C = ceil(V / 1024) rounded up to 8;
// a segment is four consecutive runs (4C entries), so V has at most 256
// segments and a segment's statistics combine four neighbouring lanes.
#include "internal.h"

namespace ta {
namespace {

constexpr int kSThreads = 1024;
constexpr int kSWaves = kSThreads / 64;
constexpr int kRunsPerSeg = 4;
constexpr int kMaxSeg = kSThreads / kRunsPerSeg;   // 256
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInfS = -__builtin_inff();

__device__ inline float wave_sum_f(float x) {
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}
__device__ inline float wave_max_f(float x) {
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

// Workgroup-wide sum (every thread gets the result).
__device__ inline float block_sum(float x, float* red) {
  x = wave_sum_f(x);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int w = 0; w < kSWaves; ++w) s += red[w];
  return s;
}
template <bool BF16>
__device__ inline float logit(const void* row, int v) {
  if constexpr (BF16) {
    const uint16_t h = static_cast<const uint16_t*>(row)[v];
    return __uint_as_float((uint32_t)h << 16);
  } else {
    return static_cast<const float*>(row)[v];
  }
}

// The current distribution: P(v) = exp2(s_v - m) / Z with s_v = logit * kc
// (implicit), or P(v) = R[v] / Z (explicit).
struct Dist {
  const void* row;   // logits row (implicit) or nullptr
  const float* R;    // residual row (explicit)
  float m, Z;
};

template <bool BF16>
__device__ inline float dist_at(const Dist& d, int v, float kc) {
  if (d.row) return __builtin_amdgcn_exp2f(logit<BF16>(d.row, v) * kc - d.m);
  return d.R[v];
}

typedef uint32_t u32x4s_t __attribute__((ext_vector_type(4)));
typedef float f32x4s_t __attribute__((ext_vector_type(4)));

// Eight entries v .. v+7 of a row (entries past V read as `pad`).  VEC: the
// row is 16-byte aligned and V % 8 == 0, so a whole group is one (bf16) or
// two (fp32) 16-byte loads.
template <bool BF16, bool VEC>
__device__ inline void load8_logits(const void* row, int v, int V, float (&x)[8]) {
  if (VEC && v + 8 <= V) {
    if constexpr (BF16) {
      const u32x4s_t w = *reinterpret_cast<const u32x4s_t*>(static_cast<const uint16_t*>(row) + v);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        x[2 * k] = __uint_as_float(w[k] << 16);
        x[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
      }
    } else {
      const f32x4s_t a = *reinterpret_cast<const f32x4s_t*>(static_cast<const float*>(row) + v);
      const f32x4s_t c = *reinterpret_cast<const f32x4s_t*>(static_cast<const float*>(row) + v + 4);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        x[k] = a[k];
        x[4 + k] = c[k];
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] = v + k < V ? logit<BF16>(row, v + k) : kNegInfS;
  }
}
template <bool VEC>
__device__ inline void load8_f32(const float* row, int v, int V, float (&x)[8]) {
  if (VEC && v + 8 <= V) {
    const f32x4s_t a = *reinterpret_cast<const f32x4s_t*>(row + v);
    const f32x4s_t c = *reinterpret_cast<const f32x4s_t*>(row + v + 4);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x[k] = a[k];
      x[4 + k] = c[k];
    }
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] = v + k < V ? row[v + k] : 0.f;
  }
}
template <bool VEC>
__device__ inline void store8_f32(float* row, int v, int V, const float (&x)[8]) {
  if (VEC && v + 8 <= V) {
    *reinterpret_cast<f32x4s_t*>(row + v) = f32x4s_t{x[0], x[1], x[2], x[3]};
    *reinterpret_cast<f32x4s_t*>(row + v + 4) = f32x4s_t{x[4], x[5], x[6], x[7]};
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (v + k < V) row[v + k] = x[k];
  }
}

// Unnormalised P over eight entries: exp2(logit * kc - m), or the residual row.
template <bool BF16, bool VEC>
__device__ inline void dist8(const Dist& d, int v, int V, float kc, float (&x)[8]) {
  if (d.row) {
    load8_logits<BF16, VEC>(d.row, v, V, x);
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] = __builtin_amdgcn_exp2f(x[k] * kc - d.m);
  } else {
    load8_f32<VEC>(d.R, v, V, x);
  }
}

// (max, sum of exp2(x - max)) pairs merged: the larger max, the other sum
// rescaled to it.
__device__ inline void merge_ms(float& m, float& s, float m2, float s2) {
  const float mm = fmaxf(m, m2);
  if (mm == kNegInfS) return;
  s = s * __builtin_amdgcn_exp2f(m - mm) + s2 * __builtin_amdgcn_exp2f(m2 - mm);
  m = mm;
}

// Running (max, sum of exp2(x - max)) over this thread's run of a logits row
// (x = logit * kc): a bf16 row with aligned 16-byte groups in one batch of raw
// loads (4 registers per group, unpacked one at a time), anything else in
// batches of four groups.
template <bool BF16, bool VEC>
__device__ inline void run_stats(const void* row, int r0, int r1, int V, float kc, float& m,
                                 float& s) {
  m = kNegInfS;
  s = 0.f;
  auto absorb = [&](float (&x)[8]) {
    float cm = kNegInfS;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      x[k] *= kc;
      cm = fmaxf(cm, x[k]);
    }
    if (cm > m) {
      s = m == kNegInfS ? 0.f : s * __builtin_amdgcn_exp2f(m - cm);
      m = cm;
    }
    if (m != kNegInfS) {
#pragma unroll
      for (int k = 0; k < 8; ++k) s += __builtin_amdgcn_exp2f(x[k] - m);
    }
  };
  if constexpr (BF16 && VEC) {
    constexpr int kB = 16;
    for (int v0 = r0; v0 < r1; v0 += 8 * kB) {
      u32x4s_t w[kB];
#pragma unroll
      for (int j = 0; j < kB; ++j)
        w[j] = *reinterpret_cast<const u32x4s_t*>(static_cast<const uint16_t*>(row) +
                                                  min(v0 + 8 * j, V - 8));
#pragma unroll
      for (int j = 0; j < kB; ++j) {
        if (v0 + 8 * j >= r1) break;
        float x[8];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          x[2 * k] = __uint_as_float(w[j][k] << 16);
          x[2 * k + 1] = __uint_as_float(w[j][k] & 0xffff0000u);
        }
        absorb(x);
      }
    }
  } else {
    constexpr int kB = 4;
    for (int v0 = r0; v0 < r1; v0 += 8 * kB) {
      float x[kB][8];
#pragma unroll
      for (int j = 0; j < kB; ++j) load8_logits<BF16, VEC>(row, min(v0 + 8 * j, V), V, x[j]);
#pragma unroll
      for (int j = 0; j < kB; ++j) {
        if (v0 + 8 * j >= r1) break;
        absorb(x[j]);
      }
    }
  }
}

__device__ inline int run_len(int V) { return ((V + kSThreads - 1) / kSThreads + 7) / 8 * 8; }

// Segment statistics of every logits row: row r < total_nodes is node row r,
// the rest are the prefix rows.  stats[r][k] = (max, sum) of segment k.  Four
// 256-thread workgroups per row, workgroup q taking runs 256q .. 256q + 255
// (segments 64q .. 64q + 63), so a row's exponentials spread over four CUs.
constexpr int kStatsThreads = 256;
constexpr int kStatsSplit = kSThreads / kStatsThreads;

template <bool BF16, bool VEC>
__global__ __launch_bounds__(kStatsThreads) void softmax_stats_kernel(
    const void* __restrict__ logits, const void* __restrict__ root_logits, int total_nodes,
    int V, float kc, float2* __restrict__ stats, float2* __restrict__ wgstats) {
  __shared__ float2 wred[kStatsThreads / 64];
  const int r = blockIdx.x / kStatsSplit;
  const int t = (blockIdx.x % kStatsSplit) * kStatsThreads + threadIdx.x;   // run index
  const size_t esz = BF16 ? 2 : 4;
  const void* row = r < total_nodes
                        ? static_cast<const void*>(static_cast<const unsigned char*>(logits) +
                                                   (size_t)r * V * esz)
                        : static_cast<const void*>(static_cast<const unsigned char*>(root_logits) +
                                                   (size_t)(r - total_nodes) * V * esz);
  const int C = run_len(V);
  const int r0 = t * C;
  const int r1 = min(V, r0 + C);
  float m, s;
  run_stats<BF16, VEC>(row, r0, r1, V, kc, m, s);
  // the four runs of a segment sit in lanes 4k .. 4k+3 of one wave
  for (int o = 1; o < kRunsPerSeg; o <<= 1) {
    const float m2 = __shfl_xor(m, o), s2 = __shfl_xor(s, o);
    merge_ms(m, s, m2, s2);
  }
  const int nseg = (V + kRunsPerSeg * C - 1) / (kRunsPerSeg * C);
  if ((t & (kRunsPerSeg - 1)) == 0 && t / kRunsPerSeg < nseg)
    stats[(size_t)r * kMaxSeg + t / kRunsPerSeg] = make_float2(m, s);
  // and this workgroup's quarter of the row as one pair (wgstats[r][q])
  for (int o = kRunsPerSeg; o < 64; o <<= 1) {
    const float m2 = __shfl_xor(m, o), s2 = __shfl_xor(s, o);
    merge_ms(m, s, m2, s2);
  }
  if ((threadIdx.x & 63) == 0) wred[threadIdx.x >> 6] = make_float2(m, s);
  __syncthreads();
  if (threadIdx.x == 0) {
    float bm = wred[0].x, bs = wred[0].y;
    for (int w = 1; w < kStatsThreads / 64; ++w) merge_ms(bm, bs, wred[w].x, wred[w].y);
    wgstats[(size_t)r * kStatsSplit + blockIdx.x % kStatsSplit] = make_float2(bm, bs);
  }
}

// A row's (max, sum) from its four quarters.
__device__ inline float2 row_stats(const float2* wgstats, size_t r) {
  float m = kNegInfS, s = 0.f;
#pragma unroll
  for (int q = 0; q < kStatsSplit; ++q) {
    const float2 p = wgstats[r * kStatsSplit + q];
    merge_ms(m, s, p.x, p.y);
  }
  return make_float2(m, s);
}

template <bool BF16, bool VEC>
__global__ __launch_bounds__(kSThreads) void spec_sample_kernel(
    const void* __restrict__ logits, const void* __restrict__ root_logits,
    const float* __restrict__ qp, const float* __restrict__ root_qp,
    const int32_t* __restrict__ draft, const int32_t* __restrict__ parents,
    const int32_t* __restrict__ node_offsets, int total_nodes, int max_nodes, int V, float kc,
    const float* __restrict__ u_accept, const float* __restrict__ u_final,
    int32_t* __restrict__ accept_len, int32_t* __restrict__ accept_nodes,
    int32_t* __restrict__ accept_tokens, int32_t* __restrict__ bonus_token,
    float* __restrict__ scratch, const float2* __restrict__ stats,
    const float2* __restrict__ wgstats) {
  __shared__ int32_t par[TA_MAX_NODES];
  __shared__ int32_t jmp[TA_MAX_NODES];
  __shared__ int32_t s_tok[TA_MAX_NODES];   // the sequence's draft tokens
  __shared__ float s_u[TA_MAX_NODES];       // and its uniforms
  __shared__ float s_qx[TA_MAX_NODES];      // Q(x_i) and logit(x_i) in node i's parent's rows
  __shared__ float s_lx[TA_MAX_NODES];
  __shared__ float s_rm[TA_MAX_NODES];      // node i's own row: softmax max and sum
  __shared__ float s_rz[TA_MAX_NODES];
  __shared__ float segm[2][kMaxSeg];   // P's mass per segment (two copies, see sel)
  __shared__ float red[kSWaves];
  __shared__ float red2[kSWaves];
  __shared__ int ired[kSWaves];
  __shared__ int s_bad;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const size_t esz = BF16 ? 2 : 4;
  int n0 = node_offsets[b];
  const int n1 = node_offsets[b + 1];
  int nn = n1 - n0;
  if (n0 < 0 || nn < 0 || nn > max_nodes || n1 > total_nodes || max_nodes > TA_MAX_NODES) {
    n0 = 0;
    nn = 0;
  }

  // Tree check (as the oracle): every parent -1 or another node of the
  // sequence, and every parent chain reaching -1 (pointer jumping: after
  // ceil(log2 nn) + 1 doublings a chain of length < nn has ended).  An
  // invalid tree is walked as an empty one.
  if (tid == 0) s_bad = 0;
  __syncthreads();
  for (int i = tid; i < nn; i += kSThreads) {
    const int p = parents[n0 + i];
    par[i] = p;
    jmp[i] = p;
    const int x = draft[n0 + i];
    s_tok[i] = x;
    s_u[i] = u_accept[n0 + i];
    // Each node is tested at most once, against its parent's rows: the two
    // values its test reads come in one round trip for the whole tree.
    float qx = 0.f, lx = kNegInfS;
    if (x >= 0 && x < V && p >= -1 && p < nn) {
      const size_t rowi = p < 0 ? (size_t)b : (size_t)(n0 + p);
      qx = (p < 0 ? root_qp : qp)[rowi * V + x];
      lx = logit<BF16>(static_cast<const unsigned char*>(p < 0 ? root_logits : logits) +
                           rowi * V * esz, x);
    }
    s_qx[i] = qx;
    s_lx[i] = lx;
    // and node i's own row statistics, for when it is accepted
    const float2 rs = row_stats(wgstats, (size_t)(n0 + i));
    s_rm[i] = rs.x;
    s_rz[i] = rs.y;
    if (p < -1 || p >= nn || p == i) s_bad = 1;
  }
  __syncthreads();
  if (!s_bad) {
    for (int span = 1; span < 2 * nn; span <<= 1) {
      int nj[TA_MAX_NODES / kSThreads];
#pragma unroll
      for (int k = 0; k < TA_MAX_NODES / kSThreads; ++k) {
        const int i = tid + k * kSThreads;
        nj[k] = (i < nn && jmp[i] >= 0) ? jmp[jmp[i]] : (i < nn ? jmp[i] : -1);
      }
      __syncthreads();
#pragma unroll
      for (int k = 0; k < TA_MAX_NODES / kSThreads; ++k) {
        const int i = tid + k * kSThreads;
        if (i < nn) jmp[i] = nj[k];
      }
      __syncthreads();
    }
    for (int i = tid; i < nn; i += kSThreads)
      if (jmp[i] != -1) s_bad = 1;
    __syncthreads();
  }
  if (s_bad) nn = 0;

  // Two scratch rows per sequence; rsel: the one holding an explicit P.
  float* const rows2 = scratch + (size_t)b * 2 * V;
  int rsel = 0;
  int sel = 0;   // segm[sel]: the current P's segment masses
  const int C = run_len(V);
  const int SEG = kRunsPerSeg * C;
  const int nseg = (V + SEG - 1) / SEG;
  const int r0 = tid * C;
  const int r1 = min(V, r0 + C);
  constexpr int kBatch = 4;   // groups of 8 per batch in the residual pass
  // Rejections since P's base (an implicit softmax row or an explicit
  // residual row) are kept as a chain of normalisers rather than written out:
  // P(v) = base(v) / Z_base, then max(0, p - Q(v)) * izc[i] for each of the
  // `chain` steps, all with the current node's Q.  The rejection after
  // kChain steps writes the residual out as a new explicit base instead.
  constexpr int kChain = 8;
  int chain = 0;
  float izc[kChain];
#pragma unroll
  for (int i = 0; i < kChain; ++i) izc[i] = 0.f;
  // Normalised P after `steps` chain steps, from the base's unnormalised value.
  auto pchain = [&](float bv, float q, float invb, int steps) {
    float p = bv * invb;
#pragma unroll
    for (int i = 0; i < kChain; ++i)
      if (i < steps) p = fmaxf(p - q, 0.f) * izc[i];
    return p;
  };

  // Implicit softmax of logits row r: max and sum merged from its segment
  // statistics, and the segment masses relative to that max.
  // Implicit softmax of a logits row from its (max, sum).  Its segment masses
  // (segm) are filled only when the bonus is drawn from it (seg_fresh).
  auto softmax_of = [&](const void* row, float m, float z) {
    Dist d;
    d.row = row;
    d.R = nullptr;
    d.m = m;
    d.Z = z;
    return d;
  };
  bool seg_fresh = false;   // segm[sel] holds the masses of P
  const float2 rootst = row_stats(wgstats, (size_t)(total_nodes + b));
  Dist P = softmax_of(static_cast<const unsigned char*>(root_logits) + (size_t)b * V * esz,
                      rootst.x, rootst.y);
  int prow = total_nodes + b;   // logits row of P's implicit base
  const float* Q = root_qp + (size_t)b * V;
  int cur = -1;     // current node (-1: above the roots)
  int after = -1;   // children of cur with index <= after are done
  int len = 0;
  int32_t* an = accept_nodes + (size_t)b * max_nodes;
  int32_t* at = accept_tokens + (size_t)b * max_nodes;
  for (;;) {
    // Next child of cur: the lowest index above `after` whose parent is cur.
    int c = 0x7fffffff;
    for (int i = after + 1 + tid; i < nn; i += kSThreads)
      if (par[i] == cur) {
        c = i;
        break;
      }
    for (int o = 32; o > 0; o >>= 1) c = min(c, __shfl_xor(c, o));
    __syncthreads();
    if (lane == 0) ired[wave] = c;
    __syncthreads();
    c = ired[0];
#pragma unroll
    for (int w = 1; w < kSWaves; ++w) c = min(c, ired[w]);
    if (c >= nn) break;
    after = c;
    // The test's loads and, in the same round trip, the child's statistics
    // (used if it is accepted).
    const int x = s_tok[c];
    const bool xin = x >= 0 && x < V;
    const float qx = s_qx[c];
    // base(x): from the prefetched logit while P's base is the current node's
    // row, read from the written-out residual otherwise
    const float bx = !xin ? 0.f
                     : P.row ? __builtin_amdgcn_exp2f(s_lx[c] * kc - P.m) : P.R[x];
    const bool take = xin && s_u[c] * qx < pchain(bx, qx, 1.f / P.Z, chain);
    if (take) {
      if (tid == 0) {
        an[len] = c;
        at[len] = x;
      }
      ++len;
      cur = c;
      after = -1;
      chain = 0;
      P = softmax_of(static_cast<const unsigned char*>(logits) + (size_t)(n0 + c) * V * esz,
                     s_rm[c], s_rz[c]);
      prow = n0 + c;
      seg_fresh = false;
      Q = qp + (size_t)(n0 + c) * V;
    } else {
      // Residual max(0, P - Q): its sum and segment masses (into the other
      // copy of segm); written out to the other scratch row only when the
      // chain is full.
      const bool spill = chain == kChain;
      float* out = rows2 + (size_t)(rsel ^ 1) * V;
      const float invb = 1.f / P.Z;
      float s = 0.f;
      for (int v0 = r0; v0 < r1; v0 += 8 * kBatch) {
        float xv[kBatch][8], q[kBatch][8];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
          dist8<BF16, VEC>(P, min(v0 + 8 * j, V), V, kc, xv[j]);
          load8_f32<VEC>(Q, min(v0 + 8 * j, V), V, q[j]);
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
          if (v0 + 8 * j >= r1) break;
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            xv[j][k] = fmaxf(pchain(xv[j][k], q[j][k], invb, chain) - q[j][k], 0.f);
            if (v0 + 8 * j + k < r1) s += xv[j][k];
          }
          if (spill) store8_f32<VEC>(out, v0 + 8 * j, V, xv[j]);
        }
      }
      float seg = s;
      for (int o = 1; o < kRunsPerSeg; o <<= 1) seg += __shfl_xor(seg, o);
      if ((tid & (kRunsPerSeg - 1)) == 0) segm[sel ^ 1][tid / kRunsPerSeg] = seg;
      const float z = block_sum(s, red);   // its barriers also order the row's writes
      if (z > 0.f) {
        sel ^= 1;
        seg_fresh = true;
        if (spill) {
          rsel ^= 1;
          P.row = nullptr;
          P.R = out;
          P.m = 0.f;
          P.Z = z;
          chain = 0;
        } else {
#pragma unroll
          for (int i = 0; i < kChain; ++i)
            if (i == chain) izc[i] = 1.f / z;
          ++chain;
        }
      }
    }
  }

  // Bonus token by inversion: the lowest v with sum_{w<=v} P(w) > u * Z.
  // The segment holding the threshold from an exclusive scan of the segment
  // masses (intervals [start_k, start_{k+1}) tile [0, total) exactly, so at
  // most one segment holds it), then wave 0 scans that segment 512 entries at
  // a time (8 per lane).  If rounding leaves the threshold at or past the
  // total, or inside the segment past its recomputed entries, the last entry
  // with mass of the last segment with mass is taken.
  __shared__ int s_seg;
  if (!seg_fresh) {
    // P is a row's softmax: its segment masses relative to the row's max
    float mass0 = 0.f;
    if (tid < nseg) {
      const float2 st = stats[(size_t)prow * kMaxSeg + tid];
      if (st.x != kNegInfS) mass0 = st.y * __builtin_amdgcn_exp2f(st.x - P.m);
    }
    if (tid < kMaxSeg) segm[sel][tid] = mass0;
    __syncthreads();
  }
  float mass = tid < nseg ? segm[sel][tid] : 0.f;
  float incl = mass;
  for (int o = 1; o < 64; o <<= 1) {
    const float t = __shfl_up(incl, o);
    if (lane >= o) incl += t;
  }
  __syncthreads();
  if (lane == 63) red[wave] = incl;
  if (tid == 0) s_seg = -1;
  __syncthreads();
  float before = 0.f, total = 0.f;
  for (int w = 0; w < kSWaves; ++w) {
    if (w < wave) before += red[w];
    total += red[w];
  }
  const float start = before + (incl - mass);
  float end = __shfl_down(start, 1);
  if (lane == 63) end = wave + 1 < kSWaves ? before + red[wave] : total;
  const float thr = u_final[b] * total;
  if (tid < nseg && start <= thr && thr < end) s_seg = tid;
  // the last segment with mass, for the rounding case
  int lastm = (tid < nseg && mass > 0.f) ? tid : -1;
  for (int o = 32; o > 0; o >>= 1) lastm = max(lastm, __shfl_xor(lastm, o));
  if (lane == 0) ired[wave] = lastm;
  __syncthreads();
  int kseg = s_seg;
  const bool exact = kseg >= 0;
  if (!exact) {
    for (int w = 0; w < kSWaves; ++w) kseg = max(kseg, ired[w]);
  }
  int pick = -1;
  __syncthreads();
  if (exact && tid == kseg) red[1] = start;   // the mass before the segment
  __syncthreads();
  if (wave == 0 && kseg >= 0) {
    float run = exact ? red[1] : 0.f;
    const int e0 = kseg * SEG;
    const int e1 = min(V, e0 + SEG);
    int lastnz = -1;
    const float invb = 1.f / P.Z;
    for (int v0 = e0; v0 < e1; v0 += 512) {
      const int v = v0 + 8 * lane;
      float xv[8];
      dist8<BF16, VEC>(P, min(v, V), V, kc, xv);
      if (chain > 0) {
        // the segment masses are those of the last residual, max(0, P' - Q)
        float q[8];
        load8_f32<VEC>(Q, min(v, V), V, q);
#pragma unroll
        for (int k = 0; k < 8; ++k) xv[k] = fmaxf(pchain(xv[k], q[k], invb, chain - 1) - q[k], 0.f);
      }
      float ls = 0.f;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        if (v + k >= e1) xv[k] = 0.f;
        ls += xv[k];
        if (xv[k] > 0.f) lastnz = max(lastnz, v + k);
      }
      float li = ls;   // inclusive scan over the lanes, in lane order
      for (int o = 1; o < 64; o <<= 1) {
        const float t = __shfl_up(li, o);
        if (lane >= o) li += t;
      }
      if (exact && pick < 0) {
        const uint64_t hit = __ballot(run + li > thr);
        if (hit) {
          const int hl = __builtin_ctzll(hit);
          if (lane == hl) {
            float r = run + li - ls;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
              r += xv[k];
              if (pick < 0 && r > thr) pick = v + k;
            }
            if (pick < 0) pick = v + 7 < e1 ? v + 7 : e1 - 1;
          }
          pick = __shfl(pick, hl);
        }
      }
      run += __shfl(li, 63);
    }
    for (int o = 32; o > 0; o >>= 1) lastnz = max(lastnz, __shfl_xor(lastnz, o));
    if (pick < 0) pick = lastnz >= 0 ? lastnz : e1 - 1;
    if (lane == 0) ired[0] = pick;
  }
  __syncthreads();
  pick = kseg >= 0 ? ired[0] : V - 1;
  for (int pos = len + tid; pos < max_nodes; pos += kSThreads) {
    an[pos] = -1;
    at[pos] = -1;
  }
  if (tid == 0) {
    accept_len[b] = len;
    bonus_token[b] = pick;
  }
}

}  // namespace

size_t verify_sample_workspace_bytes(int B, int total_nodes, int V) {
  const size_t rows = ((size_t)B * 2 * V * sizeof(float) + 255) & ~(size_t)255;
  return rows + ((size_t)total_nodes + B) * (kMaxSeg + kStatsSplit) * sizeof(float2);
}

hipError_t launch_verify_sample(bool bf16, const void* logits, const void* root_logits,
                                const float* draft_probs, const float* root_draft_probs,
                                const int32_t* draft, const int32_t* parents,
                                const int32_t* node_offsets, int B, int total_nodes,
                                int max_nodes, int V, float temperature, const float* u_accept,
                                const float* u_final, int32_t* accept_len, int32_t* accept_nodes,
                                int32_t* accept_tokens, int32_t* bonus_token, void* workspace,
                                hipStream_t stream) {
  const float kc = kLog2e / temperature;
  // [two residual rows per sequence | segment statistics per logits row]
  float* scratch = static_cast<float*>(workspace);
  float2* stats = reinterpret_cast<float2*>(
      static_cast<unsigned char*>(workspace) +
      (((size_t)B * 2 * V * sizeof(float) + 255) & ~(size_t)255));
  float2* wgstats = stats + ((size_t)total_nodes + B) * kMaxSeg;
  const auto a16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
  const bool vec = V % 8 == 0 && a16(logits) && a16(root_logits) && a16(draft_probs) &&
                   a16(root_draft_probs) && a16(workspace);
  const unsigned rows = (unsigned)(total_nodes + B);
#define TA_SAMPLE_LAUNCH(BF, VC)                                                                \
  do {                                                                                         \
    hipLaunchKernelGGL((softmax_stats_kernel<BF, VC>), dim3(rows * kStatsSplit),              \
                       dim3(kStatsThreads), 0, stream,                                         \
                       logits, root_logits, total_nodes, V, kc, stats, wgstats);               \
    hipLaunchKernelGGL((spec_sample_kernel<BF, VC>), dim3(B), dim3(kSThreads), 0, stream,      \
                       logits, root_logits, draft_probs, root_draft_probs, draft, parents,     \
                       node_offsets, total_nodes, max_nodes, V, kc, u_accept, u_final,         \
                       accept_len, accept_nodes, accept_tokens, bonus_token, scratch, stats,   \
                       wgstats);                                                               \
  } while (0)
  if (bf16) {
    if (vec) TA_SAMPLE_LAUNCH(true, true);
    else TA_SAMPLE_LAUNCH(true, false);
  } else {
    if (vec) TA_SAMPLE_LAUNCH(false, true);
    else TA_SAMPLE_LAUNCH(false, false);
  }
#undef TA_SAMPLE_LAUNCH
  return hipGetLastError();
}

}  // namespace ta
