"""fp64 oracle: stochastic (rejection-sampling) verification of a draft tree.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages claim that a speculative tree step leaves the target model's output
distribution unchanged ([PL] Production Inference Runtimes) but give no
acceptance rule; greedy acceptance ([IS] Multi-Token Acceptance & Rollback)
is the deterministic special case.  The rule taken here is the published one
that makes the claim true: speculative sampling's accept test and residual
(Leviathan, Kalman and Matias 2023; Chen et al. 2023), walked down the tree
child by child as in SpecInfer's multi-step speculative sampling (Miao et al.
2024).  It is lossless when the children of each node were drawn
independently from the draft distribution given for that node.

Readings (the pages are silent on all of these):
  * rows: next-token convention, as in verify_greedy_next: row i of
    ``logits`` is the target's logits after node i, row b of ``root_logits``
    after sequence b's prefix; ``draft_probs`` / ``root_draft_probs`` hold,
    in the same rows, the draft distribution the node's children (the
    sequence's roots) were drawn from.  The target distribution is
    softmax(logits / temperature).
  * the walk: starting above the roots with P the target's and Q the draft's
    distribution there, the children of the current node are tested in
    increasing index order.  Child c with draft token x is accepted iff
    u_accept[c] * Q(x) < P(x) (the test u < min(1, P(x)/Q(x)) without a
    division; a token neither model gives any mass is rejected).  An accepted
    child becomes the current node (P, Q from its rows); a rejected one turns
    P into the residual max(0, P - Q) renormalised (left as it is when the
    residual is all zero).  When the current node has no child left, the
    step emits a bonus token drawn from P by inversion with u_final[b]: the
    lowest token whose cumulative probability exceeds u_final[b].
  * random numbers are inputs: one uniform in [0, 1) per node (used only if
    the node is tested) and one per sequence.
  * an invalid tree (a parent out of range, or a cycle) is treated as empty:
    nothing accepted, the bonus drawn from the prefix row.
"""
from __future__ import annotations

from typing import List, Optional

import numpy as np

from .tree_attention import _f64, tree_is_valid


def softmax_t(logits_row, temperature: float) -> np.ndarray:
    """softmax(row / temperature) in float64 (max subtracted first)."""
    z = _f64(logits_row) / float(temperature)
    z = z - np.max(z)
    e = np.exp(z)
    return e / e.sum()


def sample_inverse_cdf(p: np.ndarray, u: float):
    """Lowest index whose cumulative probability exceeds u, and the distance
    of u from the nearest cumulative boundary (how far rounding would have to
    move it to change the draw).  If rounding leaves the total at or below u,
    the last index with mass is taken."""
    cdf = np.cumsum(p)
    v = int(np.searchsorted(cdf, u, side="right"))
    if v >= len(p):
        nz = np.nonzero(p > 0)[0]
        v = int(nz[-1]) if len(nz) else len(p) - 1
        return v, 0.0
    below = cdf[v - 1] if v > 0 else 0.0
    return v, float(min(u - below, cdf[v] - u))


def residual(P: np.ndarray, Q: np.ndarray) -> np.ndarray:
    """The distribution after a rejection: max(0, P - Q) renormalised, or P
    itself when that is all zero."""
    R = np.maximum(P - Q, 0.0)
    Z = R.sum()
    return R / Z if Z > 0 else P


def speculative_sample(logits, root_logits, draft_probs, root_draft_probs, draft, parents,
                       node_offsets, temperature: float, u_accept, u_final, max_nodes: int,
                       final_p: Optional[list] = None):
    """Stochastic verification of every sequence's tree.

    Returns (accept_len [B], accept_nodes [B][max_nodes], accept_tokens
    [B][max_nodes], bonus [B], margin [B]).  accept_nodes lists the accepted
    path root first (local node ids, -1 padded).  margin[b] is the smallest
    relative distance, over sequence b's accept tests, between the two sides
    u * Q(x) and P(x), relative to the size of the operands P(x) was computed
    from (after residuals, P - Q before cancellation): an implementation
    whose relative rounding stays below it takes the same accept decisions
    (inf when nothing was tested).  If ``final_p`` is a list, the
    distribution the bonus was drawn from is appended per sequence.
    """
    draft = np.asarray(draft, dtype=np.int64)
    parents = np.asarray(parents, dtype=np.int64)
    node_offsets = np.asarray(node_offsets, dtype=np.int64)
    u_accept = np.asarray(u_accept, dtype=np.float64)
    u_final = np.asarray(u_final, dtype=np.float64)
    B = len(node_offsets) - 1
    acc_len = np.zeros(B, dtype=np.int32)
    acc_nodes = np.full((B, max_nodes), -1, dtype=np.int32)
    acc_tok = np.full((B, max_nodes), -1, dtype=np.int32)
    bonus = np.zeros(B, dtype=np.int32)
    margin = np.full(B, np.inf)
    for b in range(B):
        lo, hi = int(node_offsets[b]), int(node_offsets[b + 1])
        par = parents[lo:hi].tolist()
        nn = hi - lo if tree_is_valid(par) else 0
        P = softmax_t(root_logits[b], temperature)
        E = P                       # operand size behind each P(v), for the margin
        Q = _f64(root_draft_probs[b])
        cur = -1
        path: List[int] = []
        while True:
            taken = None
            for c in (i for i in range(nn) if par[i] == cur):
                x = int(draft[lo + c])
                lhs, rhs = u_accept[lo + c] * Q[x], P[x]
                size = max(E[x], lhs)
                if size > 0:
                    margin[b] = min(margin[b], abs(lhs - rhs) / size)
                if lhs < rhs:
                    taken = c
                    break
                R = np.maximum(P - Q, 0.0)
                Z = R.sum()
                P = residual(P, Q)
                if Z > 0:
                    E = (E + Q) / Z
            if taken is None:
                break
            path.append(taken)
            cur = taken
            P = softmax_t(logits[lo + cur], temperature)
            E = P
            Q = _f64(draft_probs[lo + cur])
        v, _ = sample_inverse_cdf(P, float(u_final[b]))
        if final_p is not None:
            final_p.append(P)
        acc_len[b] = len(path)
        for k, j in enumerate(path):
            acc_nodes[b, k] = j
            acc_tok[b, k] = int(draft[lo + j])
        bonus[b] = v
    return acc_len, acc_nodes, acc_tok, bonus, margin
