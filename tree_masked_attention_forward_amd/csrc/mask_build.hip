// Ancestor bitmask builder.
//
// Follows "Tree Attention" (inferensys.com glossary), Modified Causal
// Attention Mask: a node sees itself and every node on its path back to the
// root, never a sibling branch.  The premlal article builds the same relation
// as a dense N x N boolean matrix by walking parent pointers; here it is
// packed to one bit per node (64 nodes per uint64 word) and built on the GPU
// by pointer jumping, one workgroup per sequence with the rows in LDS
// (max_nodes * W * 8 bytes, 128 KiB at the 1024-node limit):
//
//   R(i) = {i},  J(i) = parent(i)                          (round 0)
//   R(i) |= R(J(i)),  J(i) = J(J(i))   while some J(i) >= 0
//
// After round k, R(i) holds every ancestor of i closer than 2^(k+1) and J(i)
// is the ancestor exactly 2^(k+1) steps up (or -1), so a tree of depth d
// needs ceil(log2(d + 1)) rounds.  R is updated in place: a row read while
// its owner is extending it is still a subset of that node's ancestors, and
// J is double buffered, so the covered distance never falls behind J.  The
// depth of i is |R(i)| - 1.  Nothing here depends on the order in which the
// nodes are listed: a reranked tree may list a child before its parent ("Tree
// Attention", zhongzhoutan-coder.github.io, Where It Appears: EAGLE-2 builds
// the mask after reranking).  A parent out of range or equal to its node is
// invalid, and so is a cycle, found as a jump still pending after the
// ceil(log2(n + 1)) rounds any forest of n nodes needs.
//
// Trees above 1024 nodes (up to TA_MAX_NODES): the rows no longer fit in LDS.
// build_mask_large_kernel spreads a sequence over several workgroups; each
// keeps the whole parent array in LDS (4 bytes per node), validates it, and
// writes the rows of its own block of nodes straight to global memory.  Lane
// (row i, word w) follows the parent chain of i and sets the bits of the
// ancestors inside word w, stopping as soon as the chain drops below the word
// when the order is
// topological (every parent before its child: the chain's indices fall), and
// following it to the root otherwise.  A row's depth is the popcount summed
// over its lanes, minus one.  The walk costs up to depth + 1 LDS steps per
// lane: fast for bushy trees, linear in N for a long chain.  Cycles are found
// first, by pointer jumping over the parent array in LDS.
#include "internal.h"

namespace ta {
namespace {

// Threads per workgroup: 256, or 1024 for trees whose rows span more than
// 2048 (node, word) pairs (e.g. 512 nodes of 8 words), so every pointer-
// jumping round takes a few steps per thread.
constexpr int kThreads = 256;
constexpr int kThreadsWide = 1024;
constexpr int kWideFrom = 2048;

__device__ inline uint64_t lds_load(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ inline void lds_store(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

template <int NT>
__global__ __launch_bounds__(NT) void build_mask_kernel(
    const int32_t* __restrict__ parents, const int32_t* __restrict__ node_offsets,
    int total_nodes, int max_nodes, int W, uint64_t* __restrict__ mask,
    int32_t* __restrict__ depth, int32_t* __restrict__ status) {
  constexpr int kPerThread = (kLdsTreeMaxNodes + NT - 1) / NT;
  extern __shared__ uint64_t smem[];
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  // Sequence 0 starts at node 0 whenever its offsets are well formed, so its
  // parent loads go out together with the offset loads.
  const int spec_n = min(max_nodes, total_nodes);
  int pv[kPerThread];
#pragma unroll
  for (int k = 0; k < kPerThread; ++k) {
    const int i = tid + k * NT;
    pv[k] = (b == 0 && i < spec_n) ? parents[i] : -1;
  }
  const int n0 = node_offsets[b];
  const int n1 = node_offsets[b + 1];
  const int n = n1 - n0;
  if (n0 < 0 || n < 0 || n > max_nodes || n1 > total_nodes) {
    if (tid == 0 && status) status[b] = 1;  // TA_ERR_INVALID_ARG
    return;
  }
  if (b != 0 || n0 != 0) {
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
      const int i = tid + k * NT;
      pv[k] = i < n ? parents[n0 + i] : -1;
    }
  }
  uint64_t* rows = smem;                                                    // [n][W]
  int32_t* jmp0 = reinterpret_cast<int32_t*>(smem + (size_t)max_nodes * W);  // [n]
  int32_t* jmp1 = jmp0 + max_nodes;                                          // [n]

  int bad = 0;
  int any = 0;
#pragma unroll
  for (int k = 0; k < kPerThread; ++k) {
    const int i = tid + k * NT;
    if (i < n) {
      const int p = pv[k];
      bad |= (p < -1 || p >= n || p == i);
      any |= (p >= 0);
      jmp0[i] = p;
      for (int w = 0; w < W; ++w) rows[i * W + w] = (i >> 6) == w ? 1ull << (i & 63) : 0ull;
    }
  }
  bad = __syncthreads_or(bad);
  auto invalid = [&]() {
    for (int i = tid; i < n; i += NT) {
      for (int w = 0; w < W; ++w) mask[(size_t)(n0 + i) * W + w] = 0ull;
      if (depth) depth[n0 + i] = -1;
    }
    if (tid == 0 && status) status[b] = 2;  // TA_ERR_INVALID_TREE
  };
  if (bad) {
    invalid();
    return;
  }
  any = __syncthreads_or(any);

  // Rounds any forest of n nodes needs (2^rounds > n > depth); a jump still
  // pending after them lies on a cycle.
  int rounds = 1;
  while ((1 << rounds) <= n) ++rounds;
  int32_t* jcur = jmp0;
  int32_t* jnext = jmp1;
  for (int round = 0; any; ++round) {
    if (round == rounds) {
      invalid();
      return;
    }
    for (int idx = tid; idx < n * W; idx += NT) {
      const int i = idx / W;
      const int j = jcur[i];
      if (j >= 0) {
        const int w = idx - i * W;
        lds_store(&rows[idx], lds_load(&rows[idx]) | lds_load(&rows[j * W + w]));
      }
    }
    int more = 0;
    for (int i = tid; i < n; i += NT) {
      const int j = jcur[i];
      const int jj = j >= 0 ? jcur[j] : -1;
      jnext[i] = jj;
      more |= (jj >= 0);
    }
    any = __syncthreads_or(more);
    int32_t* t = jcur;
    jcur = jnext;
    jnext = t;
  }

  for (int idx = tid; idx < n * W; idx += NT) mask[(size_t)n0 * W + idx] = rows[idx];
  if (depth)
    for (int i = tid; i < n; i += NT) {
      int c = 0;
      for (int w = 0; w < W; ++w) c += __popcll(rows[i * W + w]);
      depth[n0 + i] = c - 1;
    }
  if (tid == 0 && status) status[b] = 0;
}

constexpr int kLargeThreads = 1024;
constexpr int kLargeRows = 64;   // node rows per workgroup

// Grid B x nblk workgroups, nblk row blocks per sequence.  Wp = W rounded up to a power of two (32 or 64 here):
// Wp consecutive lanes hold one row, so a wave covers 64 / Wp rows per pass.
__global__ __launch_bounds__(kLargeThreads) void build_mask_large_kernel(
    const int32_t* __restrict__ parents, const int32_t* __restrict__ node_offsets,
    int total_nodes, int max_nodes, int W, int Wp, int nblk, uint64_t* __restrict__ mask,
    int32_t* __restrict__ depth, int32_t* __restrict__ status) {
  __shared__ int32_t par[TA_MAX_NODES];
  const int b = blockIdx.x / nblk;
  const int blk = blockIdx.x % nblk;
  const int r0 = blk * kLargeRows;
  const int tid = threadIdx.x;
  const int n0 = node_offsets[b];
  const int n1 = node_offsets[b + 1];
  const int n = n1 - n0;
  if (n0 < 0 || n < 0 || n > max_nodes || n1 > total_nodes || max_nodes > TA_MAX_NODES) {
    if (blk == 0 && tid == 0 && status) status[b] = 1;  // TA_ERR_INVALID_ARG
    return;
  }
  // Every workgroup checks the whole parent array, so all of them agree on
  // whether the tree is valid.
  __shared__ int32_t jmp[2][TA_MAX_NODES];
  int bad = 0;
  int later = 0;   // some parent after its child: walk whole chains below
  for (int i = tid; i < n; i += kLargeThreads) {
    const int p = parents[n0 + i];
    bad |= (p < -1 || p >= n || p == i);
    later |= p > i;
    par[i] = p;
    jmp[0][i] = p;
  }
  bad = __syncthreads_or(bad);
  later = __syncthreads_or(later);
  if (!bad && later) {
    // Cycle check by pointer jumping: after k rounds jmp holds the ancestor
    // 2^k steps up; in a forest of n nodes every one is -1 once 2^k > n.
    int cur = 0;
    for (int k = 0; (1 << k) <= n; ++k) {
      for (int i = tid; i < n; i += kLargeThreads) {
        const int j = jmp[cur][i];
        jmp[cur ^ 1][i] = j >= 0 ? jmp[cur][j] : -1;
      }
      __syncthreads();
      cur ^= 1;
    }
    int cyc = 0;
    for (int i = tid; i < n; i += kLargeThreads) cyc |= jmp[cur][i] >= 0;
    bad = __syncthreads_or(cyc);
  }
  const int r1 = min(n, r0 + kLargeRows);
  if (bad) {
    for (int idx = tid; idx < (r1 - r0) * W; idx += kLargeThreads)
      mask[(size_t)(n0 + r0) * W + idx] = 0ull;
    if (depth)
      for (int i = r0 + tid; i < r1; i += kLargeThreads) depth[n0 + i] = -1;
    if (blk == 0 && tid == 0 && status) status[b] = 2;  // TA_ERR_INVALID_TREE
    return;
  }
  const int w = tid & (Wp - 1);
  const int rows_per_pass = kLargeThreads / Wp;
  // Uniform trip count: the row lanes of one wave reduce together below.
  for (int base = r0; base < r1; base += rows_per_pass) {
    const int i = base + tid / Wp;
    uint64_t word = 0ull;
    if (i < r1 && w < W) {
      const int lo = 64 * w;
      const int stop = later ? 0 : lo;   // topological: the chain's indices fall
      int x = i;
      while (x >= stop) {   // ends at -1: the tree is a forest
        if (x >= lo && x < lo + 64) word |= 1ull << (x - lo);
        x = par[x];
      }
      mask[(size_t)(n0 + i) * W + w] = word;
    }
    int c = __popcll(word);
    for (int o = Wp >> 1; o > 0; o >>= 1) c += __shfl_xor(c, o);
    if (depth && i < r1 && w == 0) depth[n0 + i] = c - 1;
  }
  if (blk == 0 && tid == 0 && status) status[b] = 0;
}

}  // namespace

hipError_t launch_build_mask(const int32_t* parents, const int32_t* node_offsets, int B,
                             int total_nodes, int max_nodes, uint64_t* mask, int32_t* depth,
                             int32_t* status, hipStream_t stream) {
  const int W = (max_nodes + 63) / 64;
  if (max_nodes > kLdsTreeMaxNodes) {
    int Wp = 1;
    while (Wp < W) Wp <<= 1;
    const int nblk = (max_nodes + kLargeRows - 1) / kLargeRows;
    hipLaunchKernelGGL(build_mask_large_kernel, dim3((unsigned)((long long)B * nblk)),
                       dim3(kLargeThreads), 0, stream, parents, node_offsets, total_nodes,
                       max_nodes, W, Wp, nblk, mask, depth, status);
    return hipGetLastError();
  }
  const size_t lds = (size_t)max_nodes * W * sizeof(uint64_t) + 2 * (size_t)max_nodes * sizeof(int32_t);
  auto launch = [&](auto kernel, int threads) -> hipError_t {
    if (lds > 64 * 1024) {
      hipError_t e = raise_dynamic_lds(reinterpret_cast<const void*>(kernel), (int)lds);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kernel, dim3(B), dim3(threads), lds, stream, parents, node_offsets,
                       total_nodes, max_nodes, W, mask, depth, status);
    return hipGetLastError();
  };
  if ((long long)max_nodes * W > kWideFrom)
    return launch(&build_mask_kernel<kThreadsWide>, kThreadsWide);
  return launch(&build_mask_kernel<kThreads>, kThreads);
}

}  // namespace ta
