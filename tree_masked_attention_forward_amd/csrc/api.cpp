// Host side of the C ABI declared in include/tree_attn.h: argument checks that
// need no GPU, workspace sizing, and kernel launches on the caller's stream.
// Every check runs before the first HIP call, so a rejected call enqueues
// nothing and touches no device state.
#include <math.h>

#include <mutex>
#include <vector>

#include "internal.h"

namespace ta {

hipError_t raise_dynamic_lds(const void* kernel, int bytes) {
  struct Entry {
    const void* kernel;
    int device;
    int bytes;
  };
  static std::mutex mu;
  static std::vector<Entry> done;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  for (const Entry& x : done)
    if (x.kernel == kernel && x.device == dev && x.bytes >= bytes) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess) done.push_back(Entry{kernel, dev, bytes});
  return e;
}

int device_cu_count() {
  static std::mutex mu;
  static std::vector<int> cus;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  std::lock_guard<std::mutex> lock(mu);
  if ((int)cus.size() <= dev) cus.resize(dev + 1, -1);
  if (cus[dev] < 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) n = 0;
    cus[dev] = n;
  }
  return cus[dev];
}

}  // namespace ta

namespace {

constexpr int kMaxF32HeadDim = 256;

bool misaligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) != 0; }

// Whether the byte ranges [a, a + na) and [b, b + nb) share a byte.
bool overlaps(const void* a, unsigned long long na, const void* b, unsigned long long nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a);
  const uintptr_t y = reinterpret_cast<uintptr_t>(b);
  return na > 0 && nb > 0 && x < y + nb && y < x + na;
}

int hip_status(hipError_t e) { return e == hipSuccess ? TA_OK : TA_ERR_HIP; }

}  // namespace

extern "C" {

const char* tree_attn_status_string(int status) {
  switch (status) {
    case TA_OK: return "ok";
    case TA_ERR_INVALID_ARG: return "invalid argument";
    case TA_ERR_INVALID_TREE: return "invalid tree (a parent is not -1 or an earlier node)";
    case TA_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case TA_ERR_WORKSPACE: return "workspace missing or too small";
    case TA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int tree_attn_build_mask(const int32_t* parents, const int32_t* node_offsets, int32_t B,
                         int32_t total_nodes, int32_t max_nodes, uint64_t* mask,
                         int32_t* depth, int32_t* tree_status, void* stream) {
  if (B <= 0 || total_nodes < 0 || max_nodes < 1 || !node_offsets) return TA_ERR_INVALID_ARG;
  if (max_nodes > TA_MAX_NODES) return TA_ERR_UNSUPPORTED;
  if (total_nodes > 0 && (!parents || !mask)) return TA_ERR_INVALID_ARG;
  return hip_status(ta::launch_build_mask(parents, node_offsets, B, total_nodes, max_nodes, mask,
                                          depth, tree_status,
                                          static_cast<hipStream_t>(stream)));
}

size_t tree_attn_forward_workspace_size(int dtype, int32_t B, int32_t total_nodes,
                                        int32_t max_nodes, int32_t Hq, int32_t Hkv, int32_t D,
                                        int64_t total_prefix, int64_t max_prefix) {
  if (dtype != TA_BF16 || B <= 0 || total_nodes <= 0 || max_nodes < 1 || Hq <= 0 ||
      Hkv <= 0 || Hq % Hkv != 0 || D != 128 || total_prefix < 0 || max_prefix < 0)
    return 0;
  return ta::plan_forward_bf16(B, total_nodes, max_nodes, Hq, Hkv, total_prefix, max_prefix)
      .ws_bytes;
}

}  // extern "C"

namespace {

// Host checks shared by tree_attn_forward and tree_attn_mask_and_forward.
// Returns TA_OK with `a` filled (mask left null), or the status to return.
// `empty` is set when there is nothing to compute (total_nodes == 0).
int check_forward(int dtype, const void* q, const void* k_tree, const void* v_tree,
                  const void* k_prefix, const void* v_prefix, const int64_t* prefix_offsets,
                  const int64_t* prefix_lens, const int32_t* node_offsets, int32_t B,
                  int32_t total_nodes, int32_t max_nodes,
                  int64_t total_prefix, int64_t max_prefix, int32_t Hq, int32_t Hkv, int32_t D,
                  float scale, void* out, float* lse, void* workspace, ta::FwdArgs& a,
                  bool& empty) {
  empty = false;
  if (dtype != TA_BF16 && dtype != TA_F32) return TA_ERR_UNSUPPORTED;
  if (B <= 0 || total_nodes < 0 || max_nodes < 1 || Hq <= 0 || Hkv <= 0 || D <= 0 ||
      total_prefix < 0 || max_prefix < 0 || max_prefix > total_prefix)
    return TA_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return TA_ERR_INVALID_ARG;
  if (!isfinite(scale)) return TA_ERR_INVALID_ARG;
  if (max_nodes > TA_MAX_NODES) return TA_ERR_UNSUPPORTED;
  if (dtype == TA_BF16 && D != 128) return TA_ERR_UNSUPPORTED;
  if (dtype == TA_F32 && D > kMaxF32HeadDim) return TA_ERR_UNSUPPORTED;
  if (!prefix_offsets || !node_offsets) return TA_ERR_INVALID_ARG;
  if (total_nodes == 0) {
    empty = true;
    return TA_OK;
  }
  if (!q || !k_tree || !v_tree || !out) return TA_ERR_INVALID_ARG;
  if (total_prefix > 0 && (!k_prefix || !v_prefix)) return TA_ERR_INVALID_ARG;
  if (dtype == TA_BF16 &&
      (misaligned16(q) || misaligned16(k_tree) || misaligned16(v_tree) ||
       misaligned16(k_prefix) || misaligned16(v_prefix) || misaligned16(out)))
    return TA_ERR_INVALID_ARG;
  // Element offsets must fit the kernels' 64-bit index arithmetic comfortably
  // and row counts their 32-bit node/row indices.
  if ((long long)max_nodes * (Hq / Hkv) > (1LL << 30) || total_prefix > (1LL << 40))
    return TA_ERR_UNSUPPORTED;
  a = ta::FwdArgs{};
  a.q = q;
  a.k_tree = k_tree;
  a.v_tree = v_tree;
  a.k_prefix = k_prefix;
  a.v_prefix = v_prefix;
  a.prefix_offsets = prefix_offsets;
  a.prefix_lens = prefix_lens;
  a.node_offsets = node_offsets;
  a.B = B;
  a.total_nodes = total_nodes;
  a.max_nodes = max_nodes;
  a.total_prefix = total_prefix;
  a.max_prefix = max_prefix;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.D = D;
  a.W = (max_nodes + 63) / 64;
  a.scale = scale;
  a.out = out;
  a.lse = lse;
  a.workspace = workspace;
  return TA_OK;
}

int run_forward(int dtype, const ta::FwdArgs& a, size_t workspace_bytes, hipStream_t s) {
  if (dtype == TA_F32) return hip_status(ta::launch_forward_f32(a, s));
  const ta::FwdPlan p = ta::plan_forward_bf16(a.B, a.total_nodes, a.max_nodes, a.Hq, a.Hkv,
                                              a.total_prefix, a.max_prefix);
  if (p.ws_bytes > 0 &&
      (!a.workspace || workspace_bytes < p.ws_bytes || misaligned16(a.workspace)))
    return TA_ERR_WORKSPACE;
  return hip_status(ta::launch_forward_bf16(a, p, s));
}

// ---------------------------------------------------------------------------
// Scratch for tree_attn_forward_noalloc: the split partials and the in-kernel
// merge's counters live in this file-scope device array instead of a caller
// workspace.  Each GPU the library runs on holds its own copy until the
// process ends.  In host code `scratch` only names the symbol; its device
// address comes from hipGetSymbolAddress, once per device, and only that
// address is ever passed to a kernel.
constexpr size_t kNoAllocBytes = (size_t)TA_NOALLOC_MAX_WORKSPACE;
static __device__ __align__(256) unsigned char scratch[kNoAllocBytes];

// Zeroes n 64-bit words (the counter block, once per device).
__global__ void clear_words_kernel(unsigned long long* p, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0ull;
}

// Device address of this device's scratch (null on failure).  The first call
// on a device also enqueues, on `stream`, the zeroing of the counter block
// that the in-kernel merge needs at its first use.
void* noalloc_scratch(hipStream_t stream, hipError_t& err) {
  static std::mutex mu;
  static std::vector<void*> ptrs;
  int dev = 0;
  err = hipGetDevice(&dev);
  if (err != hipSuccess || dev < 0) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if ((int)ptrs.size() <= dev) ptrs.resize(dev + 1, nullptr);
  if (!ptrs[dev]) {
    void* ptr = nullptr;
    err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (err != hipSuccess || !ptr) return nullptr;
    hipLaunchKernelGGL(clear_words_kernel, dim3(1), dim3(256), 0, stream,
                       static_cast<unsigned long long*>(ptr), (int)(ta::kFwdCounterBytes / 8));
    err = hipGetLastError();
    if (err != hipSuccess) return nullptr;
    ptrs[dev] = ptr;
  }
  return ptrs[dev];
}

// Largest tree the forward kernel builds its own mask for (rows in registers).
constexpr int kFusedMaskMaxNodes = 128;

}  // namespace

extern "C" {

int tree_attn_forward(int dtype, const void* q, const void* k_tree, const void* v_tree,
                      const void* k_prefix, const void* v_prefix,
                      const int64_t* prefix_offsets, const int64_t* prefix_lens,
                      const int32_t* node_offsets, const uint64_t* mask, int32_t B,
                      int32_t total_nodes, int32_t max_nodes,
                      int64_t total_prefix, int64_t max_prefix, int32_t Hq, int32_t Hkv,
                      int32_t D, float scale, void* out, float* lse, void* workspace,
                      size_t workspace_bytes, void* stream) {
  ta::FwdArgs a;
  bool empty = false;
  const int st = check_forward(dtype, q, k_tree, v_tree, k_prefix, v_prefix, prefix_offsets,
                               prefix_lens, node_offsets, B, total_nodes, max_nodes, total_prefix,
                               max_prefix, Hq, Hkv, D, scale, out, lse, workspace, a, empty);
  if (st != TA_OK || empty) return st;
  if (!mask) return TA_ERR_INVALID_ARG;
  a.mask = mask;
  return run_forward(dtype, a, workspace_bytes, static_cast<hipStream_t>(stream));
}

int tree_attn_forward_noalloc(int dtype, const void* q, const void* k_tree, const void* v_tree,
                              const void* k_prefix, const void* v_prefix,
                              const int64_t* prefix_offsets, const int64_t* prefix_lens,
                              const int32_t* node_offsets, const uint64_t* mask, int32_t B,
                              int32_t total_nodes, int32_t max_nodes, int64_t total_prefix,
                              int64_t max_prefix, int32_t Hq, int32_t Hkv, int32_t D, float scale,
                              void* out, float* lse, uint32_t* merge_status, void* stream) {
  ta::FwdArgs a;
  bool empty = false;
  const int st = check_forward(dtype, q, k_tree, v_tree, k_prefix, v_prefix, prefix_offsets,
                               prefix_lens, node_offsets, B, total_nodes, max_nodes, total_prefix,
                               max_prefix, Hq, Hkv, D, scale, out, lse, nullptr, a, empty);
  if (st != TA_OK || empty) return st;
  if (!mask) return TA_ERR_INVALID_ARG;
  a.mask = mask;
  a.merge_status = merge_status;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == TA_F32) return hip_status(ta::launch_forward_f32(a, s));
  const ta::FwdPlan p = ta::plan_forward_bf16(a.B, a.total_nodes, a.max_nodes, a.Hq, a.Hkv,
                                              a.total_prefix, a.max_prefix);
  if (p.ws_bytes > kNoAllocBytes) return TA_ERR_WORKSPACE;
  if (p.ws_bytes > 0) {
    hipError_t e = hipSuccess;
    a.workspace = noalloc_scratch(s, e);
    if (!a.workspace) return TA_ERR_HIP;
  }
  return hip_status(ta::launch_forward_bf16(a, p, s));
}

int tree_attn_mask_and_forward(int dtype, const int32_t* parents, const void* q,
                               const void* k_tree, const void* v_tree, const void* k_prefix,
                               const void* v_prefix, const int64_t* prefix_offsets,
                               const int64_t* prefix_lens, const int32_t* node_offsets,
                               int32_t B, int32_t total_nodes,
                               int32_t max_nodes, int64_t total_prefix, int64_t max_prefix,
                               int32_t Hq, int32_t Hkv, int32_t D, float scale, uint64_t* mask,
                               int32_t* depth, int32_t* tree_status, void* out, float* lse,
                               void* workspace, size_t workspace_bytes, void* stream) {
  ta::FwdArgs a;
  bool empty = false;
  const int st = check_forward(dtype, q, k_tree, v_tree, k_prefix, v_prefix, prefix_offsets,
                               prefix_lens, node_offsets, B, total_nodes, max_nodes, total_prefix,
                               max_prefix, Hq, Hkv, D, scale, out, lse, workspace, a, empty);
  if (st != TA_OK) return st;
  if (empty) {
    if (tree_status && B > 0)   // same as tree_attn_build_mask on zero nodes
      return hip_status(ta::launch_build_mask(parents, node_offsets, B, total_nodes, max_nodes,
                                              mask, depth, tree_status,
                                              static_cast<hipStream_t>(stream)));
    return TA_OK;
  }
  if (!parents || !mask) return TA_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == TA_BF16 && max_nodes <= kFusedMaskMaxNodes) {
    a.build_mask = true;
    a.parents = parents;
    a.mask_out = mask;
    a.depth_out = depth;
    a.status_out = tree_status;
    return run_forward(dtype, a, workspace_bytes, s);
  }
  // Larger trees (or fp32): the mask builder, then the forward.
  const ta::FwdPlan p = ta::plan_forward_bf16(B, total_nodes, max_nodes, Hq, Hkv, total_prefix,
                                              max_prefix);
  if (dtype == TA_BF16 && p.ws_bytes > 0 &&
      (!workspace || workspace_bytes < p.ws_bytes || misaligned16(workspace)))
    return TA_ERR_WORKSPACE;
  const int ms = hip_status(ta::launch_build_mask(parents, node_offsets, B, total_nodes,
                                                  max_nodes, mask, depth, tree_status, s));
  if (ms != TA_OK) return ms;
  a.mask = mask;
  return run_forward(dtype, a, workspace_bytes, s);
}

size_t tree_verify_greedy_workspace_size(int32_t total_nodes, int32_t max_nodes, int32_t V) {
  if (total_nodes <= 0 || V <= 0 || max_nodes < 1) return 0;
  return ta::plan_verify(total_nodes, V, max_nodes).ws_bytes;
}

int tree_verify_greedy(int logits_dtype, const void* logits, const int32_t* draft_tokens,
                       const uint64_t* mask, const int32_t* node_offsets, int32_t B,
                       int32_t total_nodes, int32_t max_nodes, int32_t V,
                       int32_t* target_argmax, int32_t* accept_len, int32_t* accept_nodes,
                       int32_t* accept_tokens, void* workspace, size_t workspace_bytes,
                       void* stream) {
  if (logits_dtype != TA_BF16 && logits_dtype != TA_F32) return TA_ERR_UNSUPPORTED;
  if (B <= 0 || total_nodes < 0 || max_nodes < 1 || V <= 0) return TA_ERR_INVALID_ARG;
  if (max_nodes > TA_MAX_NODES) return TA_ERR_UNSUPPORTED;
  if (!node_offsets || !accept_len || !accept_nodes || !accept_tokens) return TA_ERR_INVALID_ARG;
  if (total_nodes > 0 && (!logits || !draft_tokens || !mask)) return TA_ERR_INVALID_ARG;
  const ta::VerifyPlan p = ta::plan_verify(total_nodes, V, max_nodes);
  if (total_nodes > 0 && (!workspace || workspace_bytes < p.ws_bytes || misaligned16(workspace)))
    return TA_ERR_WORKSPACE;
  return hip_status(ta::launch_verify(logits_dtype == TA_BF16, logits, draft_tokens, mask,
                                      node_offsets, B, total_nodes, max_nodes, V, target_argmax,
                                      accept_len, accept_nodes, accept_tokens, workspace, p,
                                      static_cast<hipStream_t>(stream)));
}

int tree_verify_greedy_next(int logits_dtype, const void* logits, const void* root_logits,
                            const int32_t* draft_tokens, const uint64_t* mask,
                            const int32_t* node_offsets, int32_t B, int32_t total_nodes,
                            int32_t max_nodes, int32_t V, int32_t* target_argmax,
                            int32_t* accept_len, int32_t* accept_nodes, int32_t* accept_tokens,
                            int32_t* bonus_token, void* workspace, size_t workspace_bytes,
                            void* stream) {
  if (logits_dtype != TA_BF16 && logits_dtype != TA_F32) return TA_ERR_UNSUPPORTED;
  if (B <= 0 || total_nodes < 0 || max_nodes < 1 || V <= 0) return TA_ERR_INVALID_ARG;
  if (max_nodes > TA_MAX_NODES) return TA_ERR_UNSUPPORTED;
  if (!node_offsets || !accept_len || !accept_nodes || !accept_tokens || !bonus_token ||
      !root_logits)
    return TA_ERR_INVALID_ARG;
  if (total_nodes > 0 && (!logits || !draft_tokens || !mask)) return TA_ERR_INVALID_ARG;
  const ta::VerifyPlan p = ta::plan_verify(total_nodes + B, V, max_nodes);
  if (!workspace || workspace_bytes < p.ws_bytes || misaligned16(workspace))
    return TA_ERR_WORKSPACE;
  return hip_status(ta::launch_verify(logits_dtype == TA_BF16, logits, draft_tokens, mask,
                                      node_offsets, B, total_nodes, max_nodes, V, target_argmax,
                                      accept_len, accept_nodes, accept_tokens, workspace, p,
                                      static_cast<hipStream_t>(stream), root_logits,
                                      bonus_token));
}

int tree_kv_commit(int dtype, const void* k_tree, const void* v_tree,
                   const int32_t* node_offsets, const int32_t* accept_len,
                   const int32_t* accept_nodes, int32_t B, int32_t total_nodes,
                   int32_t max_nodes, int32_t Hkv, int32_t D, void* k_cache, void* v_cache,
                   const int64_t* cache_offsets, int64_t* cache_lens, int64_t total_cache,
                   int32_t* commit_status, void* stream) {
  if (dtype != TA_BF16 && dtype != TA_F32) return TA_ERR_UNSUPPORTED;
  if (B <= 0 || total_nodes < 0 || max_nodes < 1 || Hkv <= 0 || D <= 0 || total_cache < 0)
    return TA_ERR_INVALID_ARG;
  if (max_nodes > TA_MAX_NODES) return TA_ERR_UNSUPPORTED;
  if (!node_offsets || !accept_len || !accept_nodes || !cache_offsets || !cache_lens)
    return TA_ERR_INVALID_ARG;
  if (total_nodes > 0 && (!k_tree || !v_tree)) return TA_ERR_INVALID_ARG;
  if (total_cache > 0 && (!k_cache || !v_cache)) return TA_ERR_INVALID_ARG;
  const long long row_bytes = (long long)Hkv * D * (dtype == TA_BF16 ? 2 : 4);
  if (row_bytes > (1LL << 30) || total_cache > (1LL << 40)) return TA_ERR_UNSUPPORTED;
  // The rows are copied in parallel, so a tree buffer inside a cache buffer
  // (draft K/V appended after the prefix in the same allocation) could be
  // overwritten before it is read: such calls are refused.
  if (total_nodes > 0 && total_cache > 0) {
    const unsigned long long tree_len = (unsigned long long)total_nodes * row_bytes;
    const unsigned long long cache_len = (unsigned long long)total_cache * row_bytes;
    const void* trees[2] = {k_tree, v_tree};
    const void* caches[2] = {k_cache, v_cache};
    for (const void* t : trees)
      for (const void* c : caches)
        if (overlaps(t, tree_len, c, cache_len)) return TA_ERR_INVALID_ARG;
  }
  return hip_status(ta::launch_kv_commit(k_tree, v_tree, node_offsets, accept_len, accept_nodes,
                                         B, total_nodes, max_nodes, row_bytes, k_cache, v_cache,
                                         cache_offsets, cache_lens, total_cache, commit_status,
                                         static_cast<hipStream_t>(stream)));
}

size_t tree_verify_sample_workspace_size(int32_t B, int32_t total_nodes, int32_t V) {
  if (B <= 0 || total_nodes < 0 || V <= 0) return 0;
  return ta::verify_sample_workspace_bytes(B, total_nodes, V);
}

int tree_verify_sample(int logits_dtype, const void* logits, const void* root_logits,
                       const float* draft_probs, const float* root_draft_probs,
                       const int32_t* draft_tokens, const int32_t* parents,
                       const int32_t* node_offsets, int32_t B, int32_t total_nodes,
                       int32_t max_nodes, int32_t V, float temperature, const float* u_accept,
                       const float* u_final, int32_t* accept_len, int32_t* accept_nodes,
                       int32_t* accept_tokens, int32_t* bonus_token, void* workspace,
                       size_t workspace_bytes, void* stream) {
  if (logits_dtype != TA_BF16 && logits_dtype != TA_F32) return TA_ERR_UNSUPPORTED;
  if (B <= 0 || total_nodes < 0 || max_nodes < 1 || V <= 0) return TA_ERR_INVALID_ARG;
  if (!(temperature > 0.f) || temperature > 3.0e38f) return TA_ERR_INVALID_ARG;
  if (max_nodes > TA_MAX_NODES) return TA_ERR_UNSUPPORTED;
  if (!root_logits || !root_draft_probs || !u_final || !node_offsets || !accept_len ||
      !accept_nodes || !accept_tokens || !bonus_token)
    return TA_ERR_INVALID_ARG;
  if (total_nodes > 0 && (!logits || !draft_probs || !draft_tokens || !parents || !u_accept))
    return TA_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < tree_verify_sample_workspace_size(B, total_nodes, V) ||
      misaligned16(workspace))
    return TA_ERR_WORKSPACE;
  return hip_status(ta::launch_verify_sample(
      logits_dtype == TA_BF16, logits, root_logits, draft_probs, root_draft_probs, draft_tokens,
      parents, node_offsets, B, total_nodes, max_nodes, V, temperature, u_accept, u_final,
      accept_len, accept_nodes, accept_tokens, bonus_token, workspace,
      static_cast<hipStream_t>(stream)));
}

}  // extern "C"
