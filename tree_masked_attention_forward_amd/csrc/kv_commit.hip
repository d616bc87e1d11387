// Commit of the accepted path to the KV cache.
//
// Follows "Tree Attention" (inferensys.com glossary), Multi-Token Acceptance &
// Rollback and Speculative KV Cache Reuse: once the target has accepted a
// root-to-node path, that path's K/V rows, already computed for the
// verification pass, join the sequence's cache in path order, and the rows of
// every rejected node are dropped (rollback is simply not copying them).
//
// One workgroup per sequence.  Sequence b's cache is a slot of rows
// [cache_offsets[b], cache_offsets[b+1]) of which cache_lens[b] are in use;
// accepted node accept_nodes[b][t] (local index, root first) lands at slot row
// cache_lens[b] + t, i.e. at position L_b + t of the sequence.  Everything is
// checked before the first store: offsets, lengths, node indices and room in
// the slot; a sequence that fails any check is left untouched and reported.
// The copy moves whole rows (Hkv * D elements) with 16-byte accesses when the
// row size and the buffers allow, else 2-byte ones.
#include "internal.h"

namespace ta {
namespace {

constexpr int kThreads = 256;

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

template <bool VEC16>
__global__ __launch_bounds__(kThreads) void kv_commit_kernel(
    const unsigned char* __restrict__ k_tree, const unsigned char* __restrict__ v_tree,
    const int32_t* __restrict__ node_offsets, const int32_t* __restrict__ accept_len,
    const int32_t* __restrict__ accept_nodes, int total_nodes, int max_nodes, long long row_bytes,
    unsigned char* __restrict__ k_cache, unsigned char* __restrict__ v_cache,
    const int64_t* __restrict__ cache_offsets, int64_t* __restrict__ cache_lens,
    long long total_cache, int32_t* __restrict__ status) {
  __shared__ int32_t src[TA_MAX_NODES];
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int n0 = node_offsets[b];
  const int n1 = node_offsets[b + 1];
  const long long c0 = cache_offsets[b];
  const long long c1 = cache_offsets[b + 1];
  const long long len0 = cache_lens[b];
  const int n = accept_len[b];
  const int nn = n1 - n0;
  bool bad = n0 < 0 || nn < 0 || nn > max_nodes || n1 > total_nodes || c0 < 0 || c1 < c0 ||
             c1 > total_cache || len0 < 0 || n < 0 || n > nn || len0 + n > c1 - c0;
  if (!bad) {
    for (int t = tid; t < n; t += kThreads) {
      const int j = accept_nodes[(size_t)b * max_nodes + t];
      bad = bad || j < 0 || j >= nn;
      src[t] = n0 + (j >= 0 && j < nn ? j : 0);
    }
  }
  // Every thread has read cache_lens[b] before thread 0 may overwrite it.
  if (__syncthreads_or(bad)) {
    if (tid == 0 && status) status[b] = TA_ERR_INVALID_ARG;
    return;
  }
  const long long dst0 = c0 + len0;
  if (VEC16) {
    const long long per_row = row_bytes / 16;
    for (long long i = tid; i < (long long)n * per_row; i += kThreads) {
      const int t = (int)(i / per_row);
      const long long c = i - t * per_row;
      const size_t so = (size_t)src[t] * row_bytes + c * 16;
      const size_t d = (size_t)(dst0 + t) * row_bytes + c * 16;
      *reinterpret_cast<u32x4_t*>(k_cache + d) = *reinterpret_cast<const u32x4_t*>(k_tree + so);
      *reinterpret_cast<u32x4_t*>(v_cache + d) = *reinterpret_cast<const u32x4_t*>(v_tree + so);
    }
  } else {
    const long long per_row = row_bytes / 2;
    for (long long i = tid; i < (long long)n * per_row; i += kThreads) {
      const int t = (int)(i / per_row);
      const long long c = i - t * per_row;
      const size_t so = (size_t)src[t] * row_bytes + c * 2;
      const size_t d = (size_t)(dst0 + t) * row_bytes + c * 2;
      *reinterpret_cast<uint16_t*>(k_cache + d) = *reinterpret_cast<const uint16_t*>(k_tree + so);
      *reinterpret_cast<uint16_t*>(v_cache + d) = *reinterpret_cast<const uint16_t*>(v_tree + so);
    }
  }
  if (tid == 0) {
    cache_lens[b] = len0 + n;
    if (status) status[b] = TA_OK;
  }
}

}  // namespace

hipError_t launch_kv_commit(const void* k_tree, const void* v_tree, const int32_t* node_offsets,
                            const int32_t* accept_len, const int32_t* accept_nodes, int B,
                            int total_nodes, int max_nodes, long long row_bytes, void* k_cache,
                            void* v_cache, const int64_t* cache_offsets, int64_t* cache_lens,
                            long long total_cache, int32_t* status, hipStream_t stream) {
  const auto aligned = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
  const bool vec16 = row_bytes % 16 == 0 && aligned(k_tree) && aligned(v_tree) &&
                     aligned(k_cache) && aligned(v_cache);
  const auto* kt = static_cast<const unsigned char*>(k_tree);
  const auto* vt = static_cast<const unsigned char*>(v_tree);
  auto* kc = static_cast<unsigned char*>(k_cache);
  auto* vc = static_cast<unsigned char*>(v_cache);
  if (vec16)
    hipLaunchKernelGGL(kv_commit_kernel<true>, dim3(B), dim3(kThreads), 0, stream, kt, vt,
                       node_offsets, accept_len, accept_nodes, total_nodes, max_nodes, row_bytes,
                       kc, vc, cache_offsets, cache_lens, total_cache, status);
  else
    hipLaunchKernelGGL(kv_commit_kernel<false>, dim3(B), dim3(kThreads), 0, stream, kt, vt,
                       node_offsets, accept_len, accept_nodes, total_nodes, max_nodes, row_bytes,
                       kc, vc, cache_offsets, cache_lens, total_cache, status);
  return hipGetLastError();
}

}  // namespace ta
