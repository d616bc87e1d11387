// Ancestor bitmask builder.
//
// Follows "Tree Attention" (inferensys.com glossary), Modified Causal
// Attention Mask: a node sees itself and every node on its path back to the
// root, never a sibling branch.  The premlal listing (build_tree_attention_mask)
// builds the same relation as a dense N x N boolean matrix by walking parent
// pointers; here it is packed to one bit per node (64 nodes per uint64 word)
// and built level by level on the GPU:
//
//   row(root) = bit(root);   row(i) = row(parent(i)) | bit(i)
//
// Nodes are topologically ordered (parent < child), so after round d every
// node of depth <= d holds its final row.  One workgroup per sequence keeps
// the rows in LDS (max_nodes * W * 8 bytes, 128 KiB at the 1024-node limit),
// then writes them out coalesced.  Rounds = tree depth + 1.
#include "internal.h"

namespace ta {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void build_mask_kernel(
    const int32_t* __restrict__ parents, const int32_t* __restrict__ node_offsets,
    int total_nodes, int max_nodes, int W, uint64_t* __restrict__ mask,
    int32_t* __restrict__ depth, int32_t* __restrict__ status) {
  extern __shared__ uint64_t smem[];
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int n0 = node_offsets[b];
  const int n1 = node_offsets[b + 1];
  const int n = n1 - n0;
  if (n0 < 0 || n < 0 || n > max_nodes || n1 > total_nodes) {
    if (tid == 0 && status) status[b] = 1;  // TA_ERR_INVALID_ARG
    return;
  }
  uint64_t* rows = smem;                                          // [n][W]
  int32_t* par = reinterpret_cast<int32_t*>(smem + (size_t)max_nodes * W);  // [n]
  int32_t* dep = par + max_nodes;                                 // [n]

  int bad = 0;
  for (int i = tid; i < n; i += kThreads) {
    const int p = parents[n0 + i];
    if (p < -1 || p >= i) bad = 1;
    par[i] = p;
    dep[i] = (p == -1) ? 0 : -1;
    for (int w = 0; w < W; ++w)
      rows[i * W + w] = (p == -1 && (i >> 6) == w) ? (1ull << (i & 63)) : 0ull;
  }
  bad = __syncthreads_or(bad);
  if (bad) {
    for (int i = tid; i < n; i += kThreads) {
      for (int w = 0; w < W; ++w) mask[(size_t)(n0 + i) * W + w] = 0ull;
      if (depth) depth[n0 + i] = -1;
    }
    if (tid == 0 && status) status[b] = 2;  // TA_ERR_INVALID_TREE
    return;
  }

  // Level rounds: a node whose parent reached depth d-1 in the previous round
  // takes depth d and its row.  Rows written in round d are read only in
  // later rounds, so one barrier per round suffices.
  for (int d = 1; d <= n; ++d) {
    int changed = 0;
    for (int i = tid; i < n; i += kThreads) {
      if (dep[i] >= 0) continue;
      const int p = par[i];
      if (dep[p] != d - 1) continue;
      for (int w = 0; w < W; ++w) {
        uint64_t v = rows[p * W + w];
        if ((i >> 6) == w) v |= 1ull << (i & 63);
        rows[i * W + w] = v;
      }
      dep[i] = d;
      changed = 1;
    }
    if (!__syncthreads_or(changed)) break;
  }

  for (int idx = tid; idx < n * W; idx += kThreads)
    mask[(size_t)n0 * W + idx] = rows[idx];
  if (depth)
    for (int i = tid; i < n; i += kThreads) depth[n0 + i] = dep[i];
  if (tid == 0 && status) status[b] = 0;
}

}  // namespace

hipError_t launch_build_mask(const int32_t* parents, const int32_t* node_offsets, int B,
                             int total_nodes, int max_nodes, uint64_t* mask, int32_t* depth,
                             int32_t* status, hipStream_t stream) {
  const int W = (max_nodes + 63) / 64;
  const size_t lds = (size_t)max_nodes * W * sizeof(uint64_t) + 2 * (size_t)max_nodes * sizeof(int32_t);
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&build_mask_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(build_mask_kernel, dim3(B), dim3(kThreads), lds, stream, parents,
                     node_offsets, total_nodes, max_nodes, W, mask, depth, status);
  return hipGetLastError();
}

}  // namespace ta
