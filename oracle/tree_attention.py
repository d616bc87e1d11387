"""fp64 oracle: the plain definitions, written out node by node.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Nothing here is tuned:
each node's attention is computed by rebuilding that node's literal token
sequence (verified prefix followed by its root-to-node path) and running
ordinary causal attention over it; acceptance is a literal enumeration over
nodes.  Inputs are the exact values a device would receive (bf16 or fp32),
upcast to float64.

Readings of the pages taken here (where they are silent or disagree):
  * visibility: a node sees the whole verified prefix, itself and its
    ancestors, never a sibling or another branch ([IS] Modified Causal
    Attention Mask; [ZT] How It Works, Common Confusions).  The comparison
    table's remark that attention crosses branches at equal depth contradicts
    both pages and is not followed.
  * a tree is a parent array over the sequence's nodes: parent[i] is -1 (a
    root; several roots make a forest) or the index of another node of the
    same sequence, and following parents from any node reaches a root.  The
    flattened order is free: a reranked draft ([ZT] Where It Appears: EAGLE-2
    builds the ancestry mask after reranking its tree) may list a child before
    its parent.  An out-of-range parent or a cycle makes the whole sequence
    invalid.
  * query head h reads KV head h // (Hq // Hkv).
  * softmax is natural-base with a caller-given scale; lse is natural log.
  * greedy acceptance: row i of the logits is the target's distribution for
    the token at node i; the predicted token is the lowest index holding the
    row maximum; a node is accepted when every node on its root path matches;
    the longest accepted path wins, ties going to the lowest terminal index
    ([IS] Multi-Token Acceptance & Rollback; [PL] verify_candidate_tree, whose
    flat scan is read as this tree walk: the two coincide on a chain).
"""
from __future__ import annotations

from typing import List, Optional, Sequence, Tuple

import numpy as np

STATUS_OK = 0
STATUS_INVALID_ARG = 1
STATUS_INVALID_TREE = 2


def _f64(x) -> np.ndarray:
    """Exact upcast of a CPU torch tensor (fp32/bf16) or array to float64."""
    try:
        import torch  # local import: the oracle itself needs only numpy
        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu").to(torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float64)


# ---------------------------------------------------------------------------
# Mask ([IS] Modified Causal Attention Mask; [PL] build_tree_attention_mask)
# ---------------------------------------------------------------------------

def tree_is_valid(parents: Sequence[int]) -> bool:
    """Every parent is -1 or another node of the same sequence, and the parent
    pointers form a forest: walking them from any node reaches -1 within n
    steps (a longer walk has entered a cycle)."""
    par = [int(x) for x in parents]
    n = len(par)
    if any(not (p == -1 or (0 <= p < n and p != i)) for i, p in enumerate(par)):
        return False
    for i in range(n):
        p, steps = par[i], 0
        while p != -1:
            steps += 1
            if steps > n:
                return False
            p = par[p]
    return True


def root_path(parents: Sequence[int], i: int) -> List[int]:
    """Nodes from the root down to node i, found by walking parent pointers."""
    path = [i]
    p = int(parents[i])
    while p != -1:
        path.append(p)
        p = int(parents[p])
    path.reverse()
    return path


def ancestor_mask_dense(parents: Sequence[int]) -> np.ndarray:
    """Dense N x N visibility: M[i, j] is True iff j is i or an ancestor of i.

    For each node: mark itself, then walk its parent pointers to the root,
    marking every node met on the way.
    """
    n = len(parents)
    m = np.zeros((n, n), dtype=bool)
    for i in range(n):
        m[i, i] = True
        p = int(parents[i])
        while p != -1:
            m[i, p] = True
            p = int(parents[p])
    return m


def pack_mask_words(dense: np.ndarray, words: int) -> np.ndarray:
    """Bit t (LSB first) of word w in row i is dense[i, 64 * w + t]."""
    n = dense.shape[0]
    out = np.zeros((n, words), dtype=np.uint64)
    for i in range(n):
        for j in np.flatnonzero(dense[i]):
            out[i, j // 64] |= np.uint64(1) << np.uint64(j % 64)
    return out


def build_mask(parents: np.ndarray, node_offsets: np.ndarray, max_nodes: int
               ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Packed ancestor-or-self bitmask, depth and per-sequence status.

    Returns (mask uint64 [sum_N][W], depth int32 [sum_N], status int32 [B])
    with W = ceil(max_nodes / 64).  A sequence whose offsets are malformed gets
    STATUS_INVALID_ARG and its rows are left untouched (zero); a sequence whose
    parent array is not a forest (a parent out of range, a cycle) gets
    STATUS_INVALID_TREE, all-zero mask rows and depth -1.
    """
    parents = np.asarray(parents, dtype=np.int64)
    node_offsets = np.asarray(node_offsets, dtype=np.int64)
    B = len(node_offsets) - 1
    W = max(1, -(-max_nodes // 64))
    total = len(parents)
    mask = np.zeros((total, W), dtype=np.uint64)
    depth = np.zeros(total, dtype=np.int32)
    status = np.zeros(B, dtype=np.int32)
    for b in range(B):
        lo, hi = int(node_offsets[b]), int(node_offsets[b + 1])
        if lo < 0 or hi < lo or hi - lo > max_nodes or hi > total:
            status[b] = STATUS_INVALID_ARG
            continue
        par = parents[lo:hi]
        if not tree_is_valid(par):
            status[b] = STATUS_INVALID_TREE
            depth[lo:hi] = -1
            continue
        dense = ancestor_mask_dense(par)
        mask[lo:hi] = pack_mask_words(dense, W)
        for i in range(hi - lo):
            depth[lo + i] = len(root_path(par, i)) - 1
    return mask, depth, status


# ---------------------------------------------------------------------------
# Attention ([IS] Modified Causal Attention Mask, Speculative KV Cache Reuse;
#            [ZT] How It Works)
# ---------------------------------------------------------------------------

def path_causal_attention(q_path: np.ndarray, k_prefix: np.ndarray, v_prefix: np.ndarray,
                          k_path: np.ndarray, v_path: np.ndarray, scale: float,
                          ) -> Tuple[np.ndarray, np.ndarray]:
    """Ordinary causal attention over the token sequence prefix || path.

    q_path [P][G][D] are the queries of the path's P nodes (root first) for the
    G query heads that share one KV head; k_prefix/v_prefix [L][D] and
    k_path/v_path [P][D].  Query r sits at position L + r and sees positions
    0 .. L + r.  Returns (out [P][G][D], lse [P][G]).
    """
    L = k_prefix.shape[0]
    P = k_path.shape[0]
    keys = np.concatenate([k_prefix, k_path], axis=0)      # [L+P][D]
    vals = np.concatenate([v_prefix, v_path], axis=0)
    Pq, G, D = q_path.shape
    scores = scale * (q_path.reshape(Pq * G, D) @ keys.T)  # [P*G][L+P]
    scores = scores.reshape(Pq, G, L + P)
    for r in range(P):
        scores[r, :, L + r + 1:] = -np.inf                  # causal: later positions hidden
    mx = scores.max(axis=2, keepdims=True)
    e = np.exp(scores - mx)
    z = e.sum(axis=2, keepdims=True)
    out = ((e / z).reshape(Pq * G, L + P) @ vals).reshape(Pq, G, D)
    lse = (mx + np.log(z))[..., 0]
    return out, lse


def tree_attention(q, k_tree, v_tree, k_prefix, v_prefix, parents, node_offsets,
                   prefix_offsets, scale: float, nodes: Optional[Sequence[int]] = None,
                   return_path_rows: bool = False, prefix_lens=None):
    """Tree attention output for every node (or for the global node ids given).

    q [sum_N][Hq][D]; k_tree, v_tree [sum_N][Hkv][D]; k_prefix, v_prefix
    [sum_L][Hkv][D]; parents are local to each sequence.  For node i of
    sequence b the keys/values are the sequence's prefix followed by the tree
    rows of path(i); the queries of the whole path are run causally and the
    last row is node i's result.  Returns (out [n][Hq][D], lse [n][Hq]) in
    float64 for the requested nodes (all nodes when ``nodes`` is None), plus,
    if asked, the per-node list of all path rows (the causal outputs of the
    ancestors as seen from node i's sequence).  With ``prefix_lens`` the
    prefix of sequence b is only the first prefix_lens[b] rows of its range
    (a cache slot with room to grow).
    """
    q = _f64(q)
    kt, vt = _f64(k_tree), _f64(v_tree)
    kp, vp = _f64(k_prefix), _f64(v_prefix)
    parents = np.asarray(parents, dtype=np.int64)
    node_offsets = np.asarray(node_offsets, dtype=np.int64)
    prefix_offsets = np.asarray(prefix_offsets, dtype=np.int64)
    total, Hq, D = q.shape
    Hkv = kt.shape[1]
    G = Hq // Hkv
    if nodes is None:
        nodes = range(total)
    nodes = list(nodes)
    seq_of = np.searchsorted(node_offsets, np.arange(total), side="right") - 1
    out = np.zeros((len(nodes), Hq, D))
    lse = np.zeros((len(nodes), Hq))
    rows = []
    for n_idx, gi in enumerate(nodes):
        b = int(seq_of[gi])
        n0 = int(node_offsets[b])
        p0, p1 = int(prefix_offsets[b]), int(prefix_offsets[b + 1])
        if prefix_lens is not None:
            p1 = p0 + int(prefix_lens[b])
        path = [n0 + j for j in root_path(parents[n0:int(node_offsets[b + 1])], gi - n0)]
        seq_rows = np.zeros((len(path), Hq, D))
        for g in range(Hkv):
            heads = slice(g * G, (g + 1) * G)
            o, l = path_causal_attention(q[path][:, heads, :], kp[p0:p1, g, :], vp[p0:p1, g, :],
                                         kt[path, g, :], vt[path, g, :], scale)
            out[n_idx, heads, :] = o[-1]
            lse[n_idx, heads] = l[-1]
            seq_rows[:, heads, :] = o
        rows.append((path, seq_rows))
    if return_path_rows:
        return out, lse, rows
    return out, lse


# ---------------------------------------------------------------------------
# Greedy verification ([IS] Multi-Token Acceptance & Rollback;
#                      [PL] verify_candidate_tree)
# ---------------------------------------------------------------------------

def target_argmax(logits) -> np.ndarray:
    """Lowest vocabulary index holding each row's maximum (exact comparison)."""
    lg = _f64(logits)
    out = np.zeros(lg.shape[0], dtype=np.int32)
    for i in range(lg.shape[0]):
        row = lg[i]
        out[i] = int(np.flatnonzero(row == row.max())[0])
    return out


def verify_greedy(logits, draft, parents, node_offsets, max_nodes: int):
    """Longest root-to-node path whose draft tokens all equal the target's.

    Returns (pred int32 [sum_N], accept_len int32 [B], accept_nodes int32
    [B][max_nodes], accept_tokens int32 [B][max_nodes]); node lists run root to
    leaf in local indices and are padded with -1.  No accepted node gives
    length 0.
    """
    pred = target_argmax(logits)
    draft = np.asarray(draft, dtype=np.int64)
    parents = np.asarray(parents, dtype=np.int64)
    node_offsets = np.asarray(node_offsets, dtype=np.int64)
    B = len(node_offsets) - 1
    acc_len = np.zeros(B, dtype=np.int32)
    acc_nodes = np.full((B, max_nodes), -1, dtype=np.int32)
    acc_tok = np.full((B, max_nodes), -1, dtype=np.int32)
    for b in range(B):
        lo, hi = int(node_offsets[b]), int(node_offsets[b + 1])
        par = parents[lo:hi]
        match = [bool(draft[lo + i] == pred[lo + i]) for i in range(hi - lo)]
        best, best_path = -1, []
        for i in range(hi - lo):
            path = root_path(par, i)
            if all(match[j] for j in path) and len(path) > len(best_path):
                best, best_path = i, path
        acc_len[b] = len(best_path)
        for k, j in enumerate(best_path):
            acc_nodes[b, k] = j
            acc_tok[b, k] = int(draft[lo + j])
    return pred, acc_len, acc_nodes, acc_tok


def verify_greedy_next(logits, root_logits, draft, parents, node_offsets, max_nodes: int):
    """Greedy acceptance on next-token rows, plus the bonus token.

    Row i of ``logits`` is the target's distribution of the token that
    follows node i; row b of ``root_logits`` that of the token after sequence
    b's prefix.  A node's draft token must equal the prediction made where the
    node's token is produced: at its parent (at the prefix for a root).  The
    longest path of matching nodes from a root wins (lowest terminal index on
    ties), and the step also emits the target's prediction after the accepted
    leaf (after the prefix when nothing is accepted).  Returns (pred
    [sum_N], accept_len [B], accept_nodes [B][max_nodes], accept_tokens
    [B][max_nodes], bonus [B]).
    """
    pred = target_argmax(logits)
    root_pred = target_argmax(root_logits)
    draft = np.asarray(draft, dtype=np.int64)
    parents = np.asarray(parents, dtype=np.int64)
    node_offsets = np.asarray(node_offsets, dtype=np.int64)
    B = len(node_offsets) - 1
    acc_len = np.zeros(B, dtype=np.int32)
    acc_nodes = np.full((B, max_nodes), -1, dtype=np.int32)
    acc_tok = np.full((B, max_nodes), -1, dtype=np.int32)
    bonus = np.zeros(B, dtype=np.int32)
    for b in range(B):
        lo, hi = int(node_offsets[b]), int(node_offsets[b + 1])
        par = parents[lo:hi]

        def expected(i):
            return int(root_pred[b]) if par[i] < 0 else int(pred[lo + int(par[i])])

        match = [bool(draft[lo + i] == expected(i)) for i in range(hi - lo)]
        best, best_path = -1, []
        for i in range(hi - lo):
            path = root_path(par, i)
            if all(match[j] for j in path) and len(path) > len(best_path):
                best, best_path = i, path
        acc_len[b] = len(best_path)
        for k, j in enumerate(best_path):
            acc_nodes[b, k] = j
            acc_tok[b, k] = int(draft[lo + j])
        bonus[b] = int(pred[lo + best]) if best_path else int(root_pred[b])
    return pred, acc_len, acc_nodes, acc_tok, bonus


# ---------------------------------------------------------------------------
# Commit of the accepted path ([IS] Multi-Token Acceptance & Rollback,
#                              Speculative KV Cache Reuse)
# ---------------------------------------------------------------------------

def kv_commit(k_tree, v_tree, node_offsets, accept_len, accept_nodes, k_cache, v_cache,
              cache_offsets, cache_lens, max_nodes: int):
    """Append each sequence's accepted path to its cache slot.

    The accepted branch keeps its K/V entries, in root-to-leaf order, right
    after the rows already in the sequence's cache; the rejected nodes' rows
    are dropped.  Sequence b's slot is rows cache_offsets[b] ..
    cache_offsets[b+1]-1 of k_cache/v_cache, the first cache_lens[b] in use.
    Works on CPU torch tensors (any dtype; rows are copied, never converted).
    Returns (k_cache', v_cache', cache_lens', status) as new objects; a
    sequence whose offsets, lengths or node ids are out of range, or whose
    slot has no room, is left as it was with status STATUS_INVALID_ARG.
    """
    kc, vc = k_cache.clone(), v_cache.clone()
    node_offsets = np.asarray(node_offsets, dtype=np.int64)
    accept_len = np.asarray(accept_len, dtype=np.int64)
    accept_nodes = np.asarray(accept_nodes, dtype=np.int64)
    cache_offsets = np.asarray(cache_offsets, dtype=np.int64)
    lens = np.asarray(cache_lens, dtype=np.int64).copy()
    B = len(node_offsets) - 1
    total_nodes, total_cache = k_tree.shape[0], k_cache.shape[0]
    status = np.zeros(B, dtype=np.int32)
    for b in range(B):
        n0, n1 = int(node_offsets[b]), int(node_offsets[b + 1])
        c0, c1 = int(cache_offsets[b]), int(cache_offsets[b + 1])
        n, c = int(accept_len[b]), int(lens[b])
        nodes = [int(accept_nodes[b, t]) for t in range(max(0, min(n, max_nodes)))]
        ok = (0 <= n0 <= n1 <= total_nodes and n1 - n0 <= max_nodes and
              0 <= c0 <= c1 <= total_cache and c >= 0 and 0 <= n <= n1 - n0 and
              c + n <= c1 - c0 and all(0 <= j < n1 - n0 for j in nodes))
        if not ok:
            status[b] = STATUS_INVALID_ARG
            continue
        for t, j in enumerate(nodes):
            kc[c0 + c + t] = k_tree[n0 + j]
            vc[c0 + c + t] = v_tree[n0 + j]
        lens[b] = c + n
    return kc, vc, lens, status
