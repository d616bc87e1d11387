// Tree attention forward, fp32 path: one wave per (node, query head).
//
// Follows "Tree Attention" (inferensys.com glossary), Modified Causal
// Attention Mask, and "Tree Attention" (zhongzhoutan-coder.github.io), How It
// Works: the node's query is scored against every prefix key of its KV head and
// against the tree keys whose bit is set in the node's ancestor mask (itself and
// its ancestors); online softmax with expf, exact fp32 products reduced across
// the 64 lanes (lane j holds dimensions j, j+64, j+128, j+192).  A plain
// correctness path for fp32 inputs, head sizes up to 256.
#include "internal.h"

#include <math.h>

namespace ta {
namespace {

constexpr float kNegInf = -__builtin_inff();

// ------------------------------------------------------------------ fp32 path

struct F32Params {
  const float* q;
  const float* k_tree;
  const float* v_tree;
  const float* k_prefix;
  const float* v_prefix;
  const int64_t* prefix_offsets;
  const int64_t* prefix_lens;   // nullable: rows in use of each prefix slot
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
  const long long p0 = P.prefix_offsets[b], pe = P.prefix_offsets[b + 1];
  const long long p1 = P.prefix_lens ? p0 + P.prefix_lens[b] : pe;
  if (n0 < 0 || n1 <= n0 || n1 - n0 > P.max_nodes || n1 > P.total_nodes) return;
  if (gnode < n0 || gnode >= n1) return;
  if (p0 < 0 || p1 < p0 || p1 > pe || p1 - p0 > P.max_prefix || pe > P.total_prefix) return;
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

}  // namespace

hipError_t launch_forward_f32(const FwdArgs& a, hipStream_t stream) {
  F32Params fp{};
  fp.q = static_cast<const float*>(a.q);
  fp.k_tree = static_cast<const float*>(a.k_tree);
  fp.v_tree = static_cast<const float*>(a.v_tree);
  fp.k_prefix = static_cast<const float*>(a.k_prefix);
  fp.v_prefix = static_cast<const float*>(a.v_prefix);
  fp.prefix_offsets = a.prefix_offsets;
  fp.prefix_lens = a.prefix_lens;
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
