/*
 * tree_attn.h - C ABI of libtreeattn.so: tree attention and greedy tree
 * verification on AMD Instinct MI355X (gfx950).
 *
 * What the library computes (the pages it follows):
 *   - "Tree Attention", inferensys.com glossary, section "Key Mechanisms of
 *     Tree Attention" (Modified Causal Attention Mask; Speculative KV Cache
 *     Reuse; Multi-Token Acceptance & Rollback).
 *   - "Tree Attention", zhongzhoutan-coder.github.io glossary term, sections
 *     "How It Works" and "Common Confusions".
 *   - "Speculative Tree Attention: How Multi-Candidate Draft Models and
 *     Parallel Verification Deliver 4x LLM Speedups", news.premlal.in, its
 *     code listing (build_tree_attention_mask, verify_candidate_tree).
 *
 * A draft tree is flattened into one token sequence: in sequence b, node i
 * (local index 0..N_b-1) has parent[i] = -1 (a root; more than one root makes
 * a forest) or the local index of another node of the sequence, and the
 * parent links form a forest (no cycle).  The order is free: a tree reranked
 * after drafting may list a child before its parent (zhongzhoutan-coder
 * "Tree Attention", Where It Appears: EAGLE-2 builds the ancestry mask after
 * reranking).  Every node attends to the sequence's whole verified prefix
 * (the KV cache), to itself and to its ancestors, and to nothing else: no
 * sibling, no node of another branch or another tree.
 *
 * Conventions shared by every call:
 *   - Array arguments are DEVICE pointers unless marked [host].  Every buffer is
 *     allocated and owned by the caller; the library allocates nothing and
 *     never synchronises the stream.  Its only state between calls is a
 *     record, per device, of the kernels whose dynamic-LDS limit it has raised
 *     and of the device's compute-unit count (so later launches make no such
 *     runtime call and can be captured in a HIP graph).
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     All work is enqueued on it; the call returns before the work finishes.
 *   - Return value: TA_OK, or an error code for anything the host can check
 *     (null pointers, bad sizes, unsupported shapes, short workspace).  On an
 *     error nothing is enqueued.  Problems only visible in device data (a
 *     malformed parent array, offsets that do not fit the stated sizes) are
 *     reported per sequence in `tree_status` by tree_attn_build_mask; the other
 *     kernels clamp such offsets so that they never read or write out of
 *     bounds, and skip the sequence.
 *   - Tensors are contiguous, row-major in the layouts given, 16-byte aligned.
 *   - sum_N = total_nodes = node_offsets[B]; sum_L = total_prefix =
 *     prefix_offsets[B]; W = ceil(max_nodes / 64) mask words per node.
 *   - Limits: 1 <= max_nodes <= TA_MAX_NODES (4096 nodes per sequence, W <= 64
 *     mask words per row); bf16 attention needs D == 128;
 *     fp32 attention needs 1 <= D <= 256; Hq % Hkv == 0.
 */
#ifndef TREE_ATTN_H
#define TREE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TA_MAX_NODES 4096

#if defined(__GNUC__) || defined(__clang__)
#define TA_API __attribute__((visibility("default")))
#else
#define TA_API
#endif

typedef enum {
  TA_OK = 0,
  TA_ERR_INVALID_ARG = 1,   /* null pointer, non-positive size, bad offsets */
  TA_ERR_INVALID_TREE = 2,  /* parent array is not a forest (out of range, cycle) */
  TA_ERR_UNSUPPORTED = 3,   /* head size / dtype / node count outside the limits */
  TA_ERR_WORKSPACE = 4,     /* workspace missing or smaller than the size query */
  TA_ERR_HIP = 5            /* a HIP runtime call failed */
} ta_status;

typedef enum { TA_F32 = 0, TA_BF16 = 1 } ta_dtype;

/* Bits of the merge status word at byte 0 of a forward workspace (see
 * tree_attn_forward). */
#define TA_MERGE_PLACEMENT 1u
#define TA_MERGE_TIMEOUT 2u
#define TA_MERGE_STALE 4u

/*
 * Ancestor bitmask and depth from a parent array.
 *
 * Follows: inferensys "Tree Attention", Modified Causal Attention Mask (a node
 * sees its ancestral path and itself, never a sibling branch); premlal listing,
 * build_tree_attention_mask (mark self, then walk parent pointers to the root),
 * here packed to bits instead of a dense N x N boolean matrix.
 *
 *   parents       int32 [sum_N]   local parent index, -1 for a root.
 *   node_offsets  int32 [B+1]     sequence b owns nodes node_offsets[b] ..
 *                                 node_offsets[b+1]-1; node_offsets[0] == 0.
 *   B, total_nodes, max_nodes [host]; every N_b <= max_nodes.
 *   mask   out uint64 [sum_N][W]: bit t (LSB = 0) of word w of node i's row is
 *          set iff local node 64*w + t is i or an ancestor of i; unused high
 *          bits are 0.
 *   depth  out int32 [sum_N], nullable: root = 0.
 *   tree_status out int32 [B], nullable: per sequence TA_OK;
 *          TA_ERR_INVALID_TREE if some parent is outside {-1} U [0, N_b), is
 *          the node itself, or the parents form a cycle (then the
 *          sequence's mask rows are 0 and its depths -1); TA_ERR_INVALID_ARG if
 *          its offsets are decreasing, exceed max_nodes or total_nodes (then
 *          its rows are not written).
 * The mask is computed once per verification step and reused by every layer.
 * Up to 1024 nodes one workgroup per sequence builds the rows in LDS by
 * pointer jumping; larger trees are split over workgroups of 64 rows, each
 * walking its rows' parent chains (time grows with the tree's depth, and
 * with the tree's size too when a child is listed before its parent).
 */
TA_API int tree_attn_build_mask(const int32_t* parents, const int32_t* node_offsets, int32_t B,
                         int32_t total_nodes, int32_t max_nodes, uint64_t* mask,
                         int32_t* depth, int32_t* tree_status, void* stream);

/*
 * Bytes of device workspace tree_attn_forward needs for these host sizes
 * (0 is a valid answer).  Pure host arithmetic; calls no HIP function.
 */
TA_API size_t tree_attn_forward_workspace_size(int dtype, int32_t B, int32_t total_nodes,
                                        int32_t max_nodes, int32_t Hq, int32_t Hkv, int32_t D,
                                        int64_t total_prefix, int64_t max_prefix);

/*
 * Tree attention forward: for every node i of sequence b and query head h,
 *   keys(i)   = prefix rows of b (all of them) + tree rows of i's ancestors and i,
 *   out[i][h] = softmax(scale * q[i][h] . keys(i)) @ values(i),
 *   lse[i][h] = log(sum(exp(scale * q[i][h] . keys(i))))   (natural log),
 * with KV head g = h / (Hq / Hkv).
 *
 * Follows: inferensys "Tree Attention", Modified Causal Attention Mask and
 * Speculative KV Cache Reuse (the tree's own K/V rows are inputs, reused from
 * the draft or recomputed by the caller); zhongzhoutan "Tree Attention", How It
 * Works (every node also sees the verified prefix).
 *
 *   dtype          TA_BF16 (q/k/v/out bf16, fp32 accumulation; D == 128) or
 *                  TA_F32 (everything fp32; 1 <= D <= 256).
 *   q              [sum_N][Hq][D]   queries of the tree nodes (already rotated).
 *   k_tree, v_tree [sum_N][Hkv][D]  keys/values of the tree nodes.
 *   k_prefix, v_prefix [sum_L][Hkv][D] verified-prefix KV cache, sequences
 *                  packed back to back.
 *   prefix_offsets int64 [B+1]  sequence b's prefix rows are
 *                  prefix_offsets[b] .. prefix_offsets[b+1]-1 (L_b may be 0).
 *   prefix_lens    int64 [B], nullable: when given, sequence b's prefix is
 *                  only the first prefix_lens[b] rows of that range (a cache
 *                  slot with room to grow, as tree_kv_commit appends to; the
 *                  rows past the length are never read).  max_prefix bounds
 *                  the lengths, total_prefix = prefix_offsets[B] the slots.
 *   node_offsets   int32 [B+1]  as for tree_attn_build_mask.
 *   mask           uint64 [sum_N][W] from tree_attn_build_mask.
 *   B, total_nodes, max_nodes, total_prefix, max_prefix, Hq, Hkv, D, scale [host].
 *   out            out [sum_N][Hq][D], dtype as the inputs.
 *   lse            out fp32 [sum_N][Hq], nullable.
 *   workspace      device buffer of at least tree_attn_forward_workspace_size()
 *                  bytes (may be NULL when that size is 0), 16-byte aligned.
 *                  It must be zero-filled before its first use.  Its first
 *                  2 KiB are a counter block, used when the splits of the key
 *                  range are merged inside the same kernel: a status word
 *                  (below) and per-group arrival, epoch and done words; every
 *                  call that runs to completion leaves it ready for the next
 *                  call, whatever its shape, and the rest is scratch, so one
 *                  buffer (of the largest size needed) serves calls of any
 *                  shapes.  Calls sharing one workspace must be ordered on one
 *                  stream.
 *
 * Merge status.  The uint32 at byte 0 of the workspace collects, by bitwise
 * OR, the failures of the in-kernel merge; the library sets bits and never
 * clears them (zero the word before a call whose status you want to read).
 * Whenever one is set, the outputs (out, lse) of the affected rows are NaN,
 * never a plausible wrong value; no call hangs (every wait is bounded: 2^18
 * polls, under a second), and the counters are reset for the next call.
 *   TA_MERGE_PLACEMENT  the key splits of a row group did not all run on the
 *                       XCD of the workgroup merging them (the hardware did not
 *                       deal workgroups round-robin over its 8 XCDs, e.g. on a
 *                       compute-unit-masked queue);
 *   TA_MERGE_TIMEOUT    a merge workgroup gave up waiting for its splits (the
 *                       counters held non-zero values at entry, e.g. a workspace
 *                       that was never zero-filled);
 *   TA_MERGE_STALE      the counters held an arrival of another call (likewise).
 */
TA_API int tree_attn_forward(int dtype, const void* q, const void* k_tree, const void* v_tree,
                      const void* k_prefix, const void* v_prefix,
                      const int64_t* prefix_offsets, const int64_t* prefix_lens,
                      const int32_t* node_offsets, const uint64_t* mask, int32_t B,
                      int32_t total_nodes, int32_t max_nodes,
                      int64_t total_prefix, int64_t max_prefix, int32_t Hq, int32_t Hkv,
                      int32_t D, float scale, void* out, float* lse, void* workspace,
                      size_t workspace_bytes, void* stream);

/*
 * tree_attn_forward without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments, results and errors as
 * tree_attn_forward, minus workspace and workspace_bytes, plus merge_status.
 *
 * The split partials and merge counters live in a static device array of
 * TA_NOALLOC_MAX_WORKSPACE bytes (64 MiB) that the library holds on every GPU
 * it runs on until the process ends; the call allocates nothing.  A call that
 * would need more scratch than that (tree_attn_forward_workspace_size above
 * the limit) returns TA_ERR_WORKSPACE and enqueues nothing; the 8B-shaped
 * layer (B=1, Hq=32, Hkv=8, L=4096, N=64) needs 8.25 MiB, the 32-sequence
 * batch of up to 8192 keys each 33 MiB.  The first call on a device also
 * enqueues a small kernel that zeroes the array's counter block.
 *
 * All calls on one GPU share that GPU's array, which keeps the last call's
 * contents: calls that may overlap on one GPU (different streams without
 * ordering, different host threads) race and must not be made; ordered calls
 * are safe.
 *
 *   merge_status   uint32 [1], device, nullable: the in-kernel merge ORs its
 *                  failure bits (TA_MERGE_*) into it, as into the workspace's
 *                  status word of tree_attn_forward (zero it before the call).
 */
#define TA_NOALLOC_MAX_WORKSPACE (64u << 20)
TA_API int tree_attn_forward_noalloc(int dtype, const void* q, const void* k_tree,
                                     const void* v_tree, const void* k_prefix,
                                     const void* v_prefix, const int64_t* prefix_offsets,
                                     const int64_t* prefix_lens, const int32_t* node_offsets,
                                     const uint64_t* mask, int32_t B, int32_t total_nodes,
                                     int32_t max_nodes, int64_t total_prefix, int64_t max_prefix,
                                     int32_t Hq, int32_t Hkv, int32_t D, float scale, void* out,
                                     float* lse, uint32_t* merge_status, void* stream);

/*
 * Ancestor mask and tree attention in one call: the same results as
 * tree_attn_build_mask(parents, node_offsets, B, total_nodes, max_nodes, mask,
 * depth, tree_status) followed by tree_attn_forward(..., mask, ...) with the
 * other arguments unchanged.  For bf16 inputs and max_nodes <= 128 it is one
 * kernel launch: each forward workgroup builds the ancestor rows of its own
 * nodes from the parents (while its first K/V tiles load) and keeps them in
 * registers, and one workgroup per row tile writes mask, depth and status for
 * tree_verify_greedy; otherwise it runs the two calls in order.
 *
 * Follows: inferensys "Tree Attention", Modified Causal Attention Mask (the
 * mask is the ancestor relation of the parent array) and Batched Parallel
 * Verification (one pass scores every node).
 *
 *   parents        int32 [sum_N], as for tree_attn_build_mask.
 *   mask           out uint64 [sum_N][W], W = ceil(max_nodes / 64).
 *   depth          out int32 [sum_N], nullable.
 *   tree_status    out int32 [B], nullable: 0 ok (also for a sequence without
 *                  nodes), 1 offsets out of range, 2 invalid parent (that
 *                  sequence's rows are all zero).
 *   everything else as for tree_attn_forward (workspace: the same size query,
 *                  the same zero-filled requirement).
 * Returns the first non-OK status of the checks of either call.
 */
TA_API int tree_attn_mask_and_forward(int dtype, const int32_t* parents, const void* q,
                                      const void* k_tree, const void* v_tree,
                                      const void* k_prefix, const void* v_prefix,
                                      const int64_t* prefix_offsets, const int64_t* prefix_lens,
                                      const int32_t* node_offsets, int32_t B,
                                      int32_t total_nodes, int32_t max_nodes,
                                      int64_t total_prefix, int64_t max_prefix, int32_t Hq,
                                      int32_t Hkv, int32_t D, float scale, uint64_t* mask,
                                      int32_t* depth, int32_t* tree_status, void* out,
                                      float* lse, void* workspace, size_t workspace_bytes,
                                      void* stream);

/*
 * Bytes of device workspace tree_verify_greedy needs.  Pure host arithmetic.
 * total_nodes: the logits rows (sum_N; sum_N + B for tree_verify_greedy_next);
 * max_nodes: as passed to the call (above 1024 the size includes the
 * many-workgroup path selection's scratch).  0 for no rows.
 */
TA_API size_t tree_verify_greedy_workspace_size(int32_t total_nodes, int32_t max_nodes, int32_t V);

/*
 * Greedy tree verification: target argmax per node, then the longest
 * root-to-node path whose draft tokens all equal the target's argmax.
 *
 * Follows: inferensys "Tree Attention", Multi-Token Acceptance & Rollback and
 * Integration with Speculative Decoding (accept the longest verified branch
 * from the root); premlal listing, verify_candidate_tree (argmax of the target
 * logits, draft compared with prediction node by node), walked along tree
 * paths instead of the flat order, which coincide on a chain.
 *
 *   logits_dtype   TA_BF16 or TA_F32.
 *   logits         [sum_N][V]; row i is the target's distribution for the
 *                  token at node i (the caller gathers it from the target
 *                  output at the node's parent, or at the prefix's last
 *                  position for a root).
 *   draft_tokens   int32 [sum_N].
 *   mask           uint64 [sum_N][W] from tree_attn_build_mask.
 *   node_offsets   int32 [B+1].
 *   B, total_nodes, max_nodes, V [host].
 *   target_argmax  out int32 [sum_N], nullable: lowest index of the row max
 *                  (values compared exactly; -0 equals +0).
 *   accept_len     out int32 [B]: nodes on the accepted path (0 if the root
 *                  itself is rejected).  Among accepted paths of equal length
 *                  the one ending at the lowest node index wins.
 *   accept_nodes   out int32 [B][max_nodes]: local node ids, root first, padded
 *                  with -1.
 *   accept_tokens  out int32 [B][max_nodes]: their draft tokens, padded with -1.
 *   workspace      at least tree_verify_greedy_workspace_size() bytes (it
 *                  grows by 24 bytes per node when max_nodes > 1024, where the
 *                  path selection runs over many workgroups and keeps
 *                  per-node scratch there).
 * Sequences must not overlap (node_offsets non-decreasing); a sequence whose
 * offsets do not decode is treated as empty (accept_len 0).
 */
TA_API int tree_verify_greedy(int logits_dtype, const void* logits, const int32_t* draft_tokens,
                       const uint64_t* mask, const int32_t* node_offsets, int32_t B,
                       int32_t total_nodes, int32_t max_nodes, int32_t V,
                       int32_t* target_argmax, int32_t* accept_len, int32_t* accept_nodes,
                       int32_t* accept_tokens, void* workspace, size_t workspace_bytes,
                       void* stream);

/*
 * Greedy tree verification on next-token rows: the same acceptance rule as
 * tree_verify_greedy, with the target's outputs given as they come out of the
 * verification pass, one row per position for the token that FOLLOWS it.
 *
 * Follows: inferensys "Tree Attention", comparison table (the target yields
 * next-token logits at every node) and Multi-Token Acceptance & Rollback;
 * premlal listing, verify_candidate_tree (argmax of the target, draft compared
 * with prediction) and its final step, which counts one more token than the
 * accepted ones: the target's own prediction after the accepted path.
 *
 *   logits         [sum_N][V]; row i: the target's distribution of the token
 *                  after node i.
 *   root_logits    [B][V]; row b: the distribution of the token after the
 *                  prefix of sequence b (what the roots are checked against).
 *   draft_tokens, mask, node_offsets, B, total_nodes, max_nodes, V,
 *   accept_len, accept_nodes, accept_tokens: as for tree_verify_greedy.
 *   target_argmax  out int32 [sum_N], nullable: argmax of each node's row.
 *   bonus_token    out int32 [B]: argmax of the accepted leaf's row, or of the
 *                  prefix row when nothing is accepted (the token the step
 *                  emits after its accepted ones).
 *   workspace      at least tree_verify_greedy_workspace_size(total_nodes + B,
 *                  max_nodes, V) bytes.
 * Node c matches iff draft_tokens[c] equals the argmax of its parent's row (of
 * the prefix row for a root); ties and the longest-path rule are those of
 * tree_verify_greedy.  Equivalent to tree_verify_greedy on the rows gathered
 * so that row c is its parent's (the prefix's for a root).
 */
TA_API int tree_verify_greedy_next(int logits_dtype, const void* logits, const void* root_logits,
                                   const int32_t* draft_tokens, const uint64_t* mask,
                                   const int32_t* node_offsets, int32_t B, int32_t total_nodes,
                                   int32_t max_nodes, int32_t V, int32_t* target_argmax,
                                   int32_t* accept_len, int32_t* accept_nodes,
                                   int32_t* accept_tokens, int32_t* bonus_token, void* workspace,
                                   size_t workspace_bytes, void* stream);

/*
 * Commit of the accepted path to the KV cache (and rollback of the rest).
 *
 * Follows: inferensys "Tree Attention", Multi-Token Acceptance & Rollback (the
 * accepted branch's entries stay in the cache, the rejected branches' are
 * discarded) and Speculative KV Cache Reuse (the K/V rows the verification
 * pass computed for the tree are reused, not recomputed).
 *
 *   dtype          TA_BF16 or TA_F32: element type of the four K/V buffers.
 *   k_tree, v_tree [sum_N][Hkv][D]   the tree's K/V rows (as for
 *                  tree_attn_forward).
 *   node_offsets   int32 [B+1], as for tree_attn_build_mask.
 *   accept_len     int32 [B], accept_nodes int32 [B][max_nodes]: the accepted
 *                  paths, local node ids root first (tree_verify_greedy's
 *                  outputs).
 *   k_cache, v_cache [total_cache][Hkv][D] in/out: sequence b's cache slot is
 *                  rows cache_offsets[b] .. cache_offsets[b+1]-1, of which the
 *                  first cache_lens[b] are in use.
 *   cache_offsets  int64 [B+1], non-decreasing slots within total_cache.
 *   cache_lens     int64 [B] in/out.
 *   B, total_nodes, max_nodes, Hkv, D, total_cache [host].
 *   commit_status  out int32 [B], nullable.
 * Effect per sequence b, with n = accept_len[b] and c = cache_lens[b] on
 * entry: slot row c + t (t < n) of k_cache and v_cache receives the row of
 * node accept_nodes[b][t] of k_tree and v_tree, and cache_lens[b] becomes
 * c + n; no row of a rejected node is copied and no other cache row changes.
 * Status TA_OK, or TA_ERR_INVALID_ARG when the offsets, lengths or node ids
 * are out of range or the slot lacks room for n more rows; such a sequence is
 * left untouched (cache rows and cache_lens).  The tree buffers must not
 * overlap the cache buffers (rows are copied in parallel, so a source row in
 * the cache could be overwritten before it is read): the call returns
 * TA_ERR_INVALID_ARG, enqueuing nothing, when [k_tree or v_tree, + sum_N rows)
 * and [k_cache or v_cache, + total_cache rows) share a byte.  The next step reads the cache
 * with tree_attn_forward(..., prefix_offsets = cache_offsets,
 * prefix_lens = cache_lens, ...).  Calls on one cache must be ordered on one
 * stream (the lengths are read and written on the device).
 */
TA_API int tree_kv_commit(int dtype, const void* k_tree, const void* v_tree,
                          const int32_t* node_offsets, const int32_t* accept_len,
                          const int32_t* accept_nodes, int32_t B, int32_t total_nodes,
                          int32_t max_nodes, int32_t Hkv, int32_t D, void* k_cache,
                          void* v_cache, const int64_t* cache_offsets, int64_t* cache_lens,
                          int64_t total_cache, int32_t* commit_status, void* stream);

/*
 * Bytes of device workspace tree_verify_sample needs: two fp32 rows of V per
 * sequence, then 260 (max, sum) float pairs per logits row (sum_N + B rows).
 * Pure host arithmetic.
 */
TA_API size_t tree_verify_sample_workspace_size(int32_t B, int32_t total_nodes, int32_t V);

/*
 * Stochastic verification: rejection sampling down the tree, which keeps the
 * emitted tokens distributed as the target model's own samples would be.
 *
 * Follows: premlal "Speculative Tree Attention", Production Inference
 * Runtimes (the speculative step leaves the output distribution unchanged);
 * the pages give no rule, so the published one is taken: speculative
 * sampling's accept test and residual (Leviathan et al. 2023; Chen et al.
 * 2023) applied child by child down the tree (SpecInfer's multi-step
 * speculative sampling, Miao et al. 2024).  Lossless when the children of
 * each node were drawn independently from that node's draft distribution.
 *
 *   logits_dtype   TA_BF16 or TA_F32 (the logits; draft probabilities are
 *                  always fp32).
 *   logits         [sum_N][V]: row i, the target's logits for the token after
 *                  node i (as tree_verify_greedy_next).
 *   root_logits    [B][V]: the target's logits after sequence b's prefix.
 *   draft_probs    fp32 [sum_N][V]: row i, the draft distribution node i's
 *                  children were drawn from.
 *   root_draft_probs fp32 [B][V]: the one sequence b's roots were drawn from.
 *   draft_tokens   int32 [sum_N].
 *   parents        int32 [sum_N]: local parent ids, -1 for a root (any node
 *                  order, as tree_attn_build_mask).
 *   node_offsets   int32 [B+1], non-decreasing.
 *   B, total_nodes, max_nodes, V [host]; temperature [host] > 0: the target
 *                  distribution is softmax(logits / temperature).
 *   u_accept       fp32 [sum_N] uniforms in [0, 1), one per node (read only
 *                  when the node is tested); u_final fp32 [B], one per sequence.
 *   accept_len     out int32 [B]; accept_nodes, accept_tokens out int32
 *                  [B][max_nodes]: the accepted path, local ids root first,
 *                  and its draft tokens, -1 padded.
 *   bonus_token    out int32 [B]: the token drawn after the accepted path.
 *   workspace      at least tree_verify_sample_workspace_size(B, sum_N, V)
 *                  bytes, 16-byte aligned, any content.
 * The walk: with P the target's and Q the draft's distribution above the
 * roots, the children of the current node are tested in increasing index
 * order; child c with token x is accepted iff u_accept[c] * Q(x) < P(x) and
 * becomes the current node (P, Q from its rows); a rejection turns P into
 * max(0, P - Q) renormalised (kept when that is all zero).  When no child is
 * left, the bonus is the lowest token whose cumulative P exceeds u_final[b].
 * Computed in fp32 (an fp64 evaluation can decide differently only where the
 * two sides of a test, or u_final and a cumulative boundary, are within
 * rounding of each other).  A tree with an out-of-range parent or a cycle,
 * or a sequence whose offsets do not decode, is walked as empty.  Asynchronous
 * on `stream`: four workgroups per logits row compute its softmax statistics
 * per vocabulary segment, then one workgroup per sequence walks the tree.
 */
TA_API int tree_verify_sample(int logits_dtype, const void* logits, const void* root_logits,
                              const float* draft_probs, const float* root_draft_probs,
                              const int32_t* draft_tokens, const int32_t* parents,
                              const int32_t* node_offsets, int32_t B, int32_t total_nodes,
                              int32_t max_nodes, int32_t V, float temperature,
                              const float* u_accept, const float* u_final, int32_t* accept_len,
                              int32_t* accept_nodes, int32_t* accept_tokens,
                              int32_t* bonus_token, void* workspace, size_t workspace_bytes,
                              void* stream);

/* Static text for a status code; never NULL. */
TA_API const char* tree_attn_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* TREE_ATTN_H */
