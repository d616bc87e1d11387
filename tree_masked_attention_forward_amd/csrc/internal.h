// Internal declarations shared by the host API (api.cpp) and the kernel
// translation units.  Not part of the public ABI (include/tree_attn.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "tree_attn.h"

namespace ta {

// Trees of up to this many nodes per sequence have their mask rows built and
// scanned in LDS (max_nodes * W * 8 bytes, 128 KiB here); larger ones, up to
// TA_MAX_NODES, take kernels that keep only per-node scalars in LDS and read
// the rows from global memory.
constexpr int kLdsTreeMaxNodes = 1024;

// Work decomposition of one tree_attn_forward call on the bf16 MFMA path.
// Derived from host scalars only, so the workspace query and the call agree.
struct FwdPlan {
  int rg;          // row groups per workgroup (one wave = 32 query rows each)
  int kg;          // key groups per workgroup (waves sharing rows, alternate tiles)
  int nwaves;      // rg * kg
  int rows_wg;     // query rows per workgroup = 32 * rg
  int R;           // row tiles per (sequence, KV head) = ceil(max_nodes*G / rows_wg)
  int S;           // key splits for the longest possible tile range
  int tmax;        // that longest range, in 32-key tiles
  long long n_items;   // B * Hkv * S * R
  long long groups;    // B * Hkv * R (sequence, KV head, row tile) groups
  int merge_wpg;       // merge workgroups per group when the merge runs in-kernel
  bool merge_in_kernel;  // splits merged by trailing workgroups of the same grid
  int piece;           // > 0: ragged batch, a sequence takes ceil(tiles / piece) splits
  bool lpt;            // split workgroups take the pieces longest first
  size_t ws_bytes;     // partial (O, m, l) storage [+ counters]; 0 when S == 1
};

struct FwdArgs {
  const void* q;
  const void* k_tree;
  const void* v_tree;
  const void* k_prefix;
  const void* v_prefix;
  const int64_t* prefix_offsets;
  const int64_t* prefix_lens;   // nullable: rows in use of each prefix slot
  const int32_t* node_offsets;
  const uint64_t* mask;
  int B, total_nodes, max_nodes;
  long long total_prefix, max_prefix;
  int Hq, Hkv, D, W;
  float scale;
  void* out;
  float* lse;
  void* workspace;
  // Mask built inside the forward kernel (tree_attn_mask_and_forward; bf16,
  // at most 128 nodes per sequence): parents in, mask rows, depths and
  // per-sequence status out, `mask` unused.
  bool build_mask;
  const int32_t* parents;
  uint64_t* mask_out;
  int32_t* depth_out;
  int32_t* status_out;
  // Where the in-kernel merge reports failures (TA_MERGE_* bits, by OR);
  // null: the status word at byte 0 of the workspace.
  uint32_t* merge_status;
};

// Raises a kernel's dynamic LDS limit to at least `bytes` on the current
// device.  The attribute is set once per (kernel, device) and cached, so
// launches after the first make no runtime call here (safe under stream
// capture once the kernel has run eagerly).
hipError_t raise_dynamic_lds(const void* kernel, int bytes);

// Compute units of the current device (cached per device; 0 if unknown).
int device_cu_count();

// Bytes of workspace at the start of every forward workspace that the
// in-kernel merge's counters and status word occupy (zero before first use).
constexpr size_t kFwdCounterBytes = 2048;

FwdPlan plan_forward_bf16(int B, int total_nodes, int max_nodes, int Hq, int Hkv,
                          long long total_prefix, long long max_prefix);

hipError_t launch_build_mask(const int32_t* parents, const int32_t* node_offsets, int B,
                             int total_nodes, int max_nodes, uint64_t* mask, int32_t* depth,
                             int32_t* status, hipStream_t stream);

hipError_t launch_forward_bf16(const FwdArgs& a, const FwdPlan& p, hipStream_t stream);
hipError_t launch_forward_f32(const FwdArgs& a, hipStream_t stream);

struct VerifyPlan {
  int cpr;             // vocabulary chunks per logits row
  int chunk;           // vocabulary entries per chunk (multiple of 8)
  bool large;          // trees above kLdsTreeMaxNodes: many-workgroup path selection
  size_t scratch_off;  // its scratch, after the chunk results (large only)
  size_t ws_bytes;     // one (value, index) pair per (row, chunk), then the scratch
};

// rows: logits rows (the node rows, plus one prefix row per sequence for
// next-token verification).
VerifyPlan plan_verify(int rows, int V, int max_nodes);

hipError_t launch_verify(bool bf16, const void* logits, const int32_t* draft,
                         const uint64_t* mask, const int32_t* node_offsets, int B,
                         int total_nodes, int max_nodes, int V, int32_t* target_argmax,
                         int32_t* accept_len, int32_t* accept_nodes, int32_t* accept_tokens,
                         void* workspace, const VerifyPlan& p, hipStream_t stream,
                         const void* root_logits = nullptr, int32_t* bonus_token = nullptr);

// Appends each sequence's accepted path (rows of row_bytes bytes) to its
// cache slot and advances cache_lens; see tree_kv_commit.
hipError_t launch_kv_commit(const void* k_tree, const void* v_tree, const int32_t* node_offsets,
                            const int32_t* accept_len, const int32_t* accept_nodes, int B,
                            int total_nodes, int max_nodes, long long row_bytes, void* k_cache,
                            void* v_cache, const int64_t* cache_offsets, int64_t* cache_lens,
                            long long total_cache, int32_t* status, hipStream_t stream);

// Stochastic verification (tree_verify_sample): segment statistics of every
// logits row, then one workgroup per sequence; workspace = two fp32 rows of V
// per sequence, then 256 + 4 (max, sum) pairs per logits row.
size_t verify_sample_workspace_bytes(int B, int total_nodes, int V);
hipError_t launch_verify_sample(bool bf16, const void* logits, const void* root_logits,
                                const float* draft_probs, const float* root_draft_probs,
                                const int32_t* draft, const int32_t* parents,
                                const int32_t* node_offsets, int B, int total_nodes,
                                int max_nodes, int V, float temperature, const float* u_accept,
                                const float* u_final, int32_t* accept_len, int32_t* accept_nodes,
                                int32_t* accept_tokens, int32_t* bonus_token, void* workspace,
                                hipStream_t stream);

}  // namespace ta
