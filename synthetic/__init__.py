"""Seeded synthetic inputs for tree attention and greedy tree verification.

This module only draws inputs: random draft trees (as parent arrays), Gaussian
q/k/v tensors, Gaussian vocabulary logits and draft tokens.  It holds none of
the method's arithmetic (no ancestor masks, no attention, no path acceptance),
so both the fp64 oracle side and the HIP side can be fed from it without
sharing any computation.

Recipe (the same for every consumer):
  * trees: ``numpy.random.default_rng(seed)``; roots are nodes ``0..R-1``; every
    later node ``i`` picks its parent uniformly among the existing nodes whose
    depth is below the depth cap and whose child count is below the branching
    cap, so ``parent[i] < i`` always holds (a topologically ordered, flattened
    tree as the pages lay it out);
  * tensors: ``torch.Generator('cpu').manual_seed(seed)``, ``randn`` in fp32,
    then round-to-nearest-even to bf16 (fp32 configs keep fp32);
  * logits: the same torch generator, ``randn`` fp32 then bf16; each draft
    token equals the row's target argmax (``torch.argmax``, a library call)
    with probability ``p_match``, else it is uniform over the vocabulary.
  * stochastic verification (make_sampling_case): target logits
    ``scale * randn`` (bf16 or fp32) from ``default_rng(seed)``; the draft
    distribution of each row is ``softmax((logits + noise * randn) / T)``
    (a stand-in draft model close to the target), in fp32; each node's draft
    token is drawn from its parent's draft row (the prefix row for a root);
    uniforms in [0, 1) in fp32.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np
import torch

__all__ = [
    "CONFIGS",
    "TreeAttnCase",
    "random_tree",
    "rerank_tree",
    "make_case",
    "make_config_case",
    "SamplingCase",
    "make_sampling_case",
    "EXAMPLE_PARENTS",
    "EXAMPLE_TOKENS",
]

# The 5-node mock tree of the premlal article's code listing (__main__ block):
# a root with two children, each child with one child of its own.
EXAMPLE_PARENTS = [-1, 0, 0, 1, 2]
EXAMPLE_TOKENS = [1204, 3401, 892, 451, 9872]


def random_tree(rng: np.random.Generator, n_nodes: int, n_roots: int = 1,
                max_depth: Optional[int] = None,
                max_children: Optional[int] = None) -> np.ndarray:
    """Draw one flattened tree (or forest) as a parent array.

    Nodes ``0..n_roots-1`` are roots (parent -1, depth 0).  Node ``i`` then
    picks a parent uniformly among nodes ``j < i`` with ``depth[j] <
    max_depth`` and fewer than ``max_children`` children.  ``max_depth`` is
    the largest node depth allowed (root depth 0), so a root-to-node path holds
    at most ``max_depth + 1`` nodes.
    """
    if n_nodes < 0 or n_roots < 0 or (n_nodes > 0 and n_roots == 0):
        raise ValueError("need at least one root for a non-empty tree")
    n_roots = min(n_roots, n_nodes)
    parents = np.full(n_nodes, -1, dtype=np.int32)
    depth = np.zeros(n_nodes, dtype=np.int64)
    kids = np.zeros(n_nodes, dtype=np.int64)
    for i in range(n_roots, n_nodes):
        ok = np.ones(i, dtype=bool)
        if max_depth is not None:
            ok &= depth[:i] < max_depth
        if max_children is not None:
            ok &= kids[:i] < max_children
        cand = np.flatnonzero(ok)
        if cand.size == 0:
            raise ValueError("depth/branching caps leave no parent for node %d" % i)
        p = int(cand[rng.integers(cand.size)])
        parents[i] = p
        depth[i] = depth[p] + 1
        kids[p] += 1
    return parents


def rerank_tree(parents: Sequence[int], perm: Sequence[int]) -> np.ndarray:
    """The same tree listed in another order: node k of the result is node
    perm[k] of `parents` (perm is a permutation of range(n)).  Parent links
    follow their nodes, so a child may now come before its parent, as in a
    draft tree reordered by score."""
    par = np.asarray(parents, dtype=np.int64)
    perm = np.asarray(perm, dtype=np.int64)
    inv = np.empty_like(perm)
    inv[perm] = np.arange(len(perm))
    old = par[perm]
    return np.where(old < 0, -1, inv[np.maximum(old, 0)]).astype(np.int32)


@dataclass
class TreeAttnCase:
    """One batch of inputs, all on the CPU.

    Layouts (row-major, contiguous):
      parents        int32 [sum_N]            local parent index, -1 for a root
      node_offsets   int32 [B+1]
      prefix_offsets int64 [B+1]
      q              [sum_N][Hq][D]
      k_tree, v_tree [sum_N][Hkv][D]
      k_prefix, v_prefix [sum_L][Hkv][D]
      logits         [sum_N][V]   (optional)
      draft          int32 [sum_N] (optional)
    """
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    dtype: torch.dtype
    parents: np.ndarray
    node_offsets: np.ndarray
    prefix_offsets: np.ndarray
    q: torch.Tensor
    k_tree: torch.Tensor
    v_tree: torch.Tensor
    k_prefix: torch.Tensor
    v_prefix: torch.Tensor
    scale: float
    logits: Optional[torch.Tensor] = None
    draft: Optional[np.ndarray] = None
    seed: int = 0
    notes: dict = field(default_factory=dict)

    @property
    def n_nodes(self) -> List[int]:
        return [int(self.node_offsets[b + 1] - self.node_offsets[b]) for b in range(self.B)]

    @property
    def prefix_lens(self) -> List[int]:
        return [int(self.prefix_offsets[b + 1] - self.prefix_offsets[b]) for b in range(self.B)]

    @property
    def total_nodes(self) -> int:
        return int(self.node_offsets[-1])

    @property
    def total_prefix(self) -> int:
        return int(self.prefix_offsets[-1])

    @property
    def max_nodes(self) -> int:
        return max(self.n_nodes) if self.B else 0

    @property
    def max_prefix(self) -> int:
        return max(self.prefix_lens) if self.B else 0

    @property
    def vocab(self) -> int:
        return 0 if self.logits is None else int(self.logits.shape[1])


def _randn(gen: torch.Generator, shape, dtype: torch.dtype) -> torch.Tensor:
    x = torch.randn(*shape, generator=gen, dtype=torch.float32)
    return x if dtype == torch.float32 else x.to(dtype)


def make_case(name: str, *, prefix_lens: Sequence[int], trees: Sequence[Sequence[int]],
              Hq: int, Hkv: int, D: int, dtype: torch.dtype = torch.bfloat16,
              seed: int = 0, scale: Optional[float] = None, vocab: int = 0,
              p_match: float = 0.6, draft: Optional[Sequence[int]] = None) -> TreeAttnCase:
    """Build a batch from explicit prefix lengths and parent arrays.

    Tensors are drawn in a fixed order (q, k_prefix, v_prefix, k_tree, v_tree,
    logits) from one torch CPU generator seeded with ``seed``; the draft-token
    coin flips use ``numpy.random.default_rng(seed + 1)``.
    """
    B = len(prefix_lens)
    assert len(trees) == B
    n = [len(t) for t in trees]
    node_offsets = np.zeros(B + 1, dtype=np.int32)
    node_offsets[1:] = np.cumsum(n)
    prefix_offsets = np.zeros(B + 1, dtype=np.int64)
    prefix_offsets[1:] = np.cumsum(np.asarray(prefix_lens, dtype=np.int64))
    parents = (np.concatenate([np.asarray(t, dtype=np.int32) for t in trees])
               if B else np.zeros(0, np.int32))
    sum_n, sum_l = int(node_offsets[-1]), int(prefix_offsets[-1])
    gen = torch.Generator("cpu").manual_seed(seed)
    q = _randn(gen, (sum_n, Hq, D), dtype)
    k_prefix = _randn(gen, (sum_l, Hkv, D), dtype)
    v_prefix = _randn(gen, (sum_l, Hkv, D), dtype)
    k_tree = _randn(gen, (sum_n, Hkv, D), dtype)
    v_tree = _randn(gen, (sum_n, Hkv, D), dtype)
    logits = None
    draft_arr = None
    if vocab:
        logits = _randn(gen, (sum_n, vocab), dtype)
        if draft is not None:
            draft_arr = np.asarray(draft, dtype=np.int32)
        else:
            rng = np.random.default_rng(seed + 1)
            target = torch.argmax(logits, dim=1).numpy().astype(np.int32)
            coin = rng.random(sum_n) < p_match
            other = rng.integers(0, vocab, size=sum_n).astype(np.int32)
            draft_arr = np.where(coin, target, other).astype(np.int32)
    return TreeAttnCase(
        name=name, B=B, Hq=Hq, Hkv=Hkv, D=D, dtype=dtype, parents=parents,
        node_offsets=node_offsets, prefix_offsets=prefix_offsets, q=q,
        k_tree=k_tree, v_tree=v_tree, k_prefix=k_prefix, v_prefix=v_prefix,
        scale=(1.0 / math.sqrt(D)) if scale is None else float(scale),
        logits=logits, draft=draft_arr, seed=seed)


# The five workloads.  ``tree`` holds (nodes, roots, depth cap, branching cap).
CONFIGS = {
    "tiny": dict(B=1, Hq=1, Hkv=1, D=64, L=16, dtype="f32", example=True,
                 vocab=16384, seed=1),
    "llama3_8b": dict(B=1, Hq=32, Hkv=8, D=128, L=4096, tree=(64, 1, 6, 4),
                      dtype="bf16", vocab=128256, seed=2),
    "batched": dict(B=32, Hq=32, Hkv=8, D=128, L=(512, 8192), tree=(64, 1, 6, 4),
                    dtype="bf16", vocab=0, seed=3),
    "llama3_70b": dict(B=4, Hq=64, Hkv=8, D=128, L=32768, tree=(128, 1, 8, 6),
                       dtype="bf16", vocab=0, seed=4),
    "forest": dict(B=8, Hq=32, Hkv=8, D=128, L=16384, tree=(512, 8, 16, None),
                   dtype="bf16", vocab=128256, seed=5),
    # The 8B layer with a one-node tree: the denominator of the cost ratio of
    # 64 candidates against one at the same prefix.
    "llama3_8b_n1": dict(B=1, Hq=32, Hkv=8, D=128, L=4096, tree=(1, 1, 6, 4),
                         dtype="bf16", vocab=128256, seed=2),
    # A tree-heavy layer: 4096 draft nodes over a 1024-token prefix, a random
    # recursive forest of 16 roots (no depth or branching cap: deep and bushy).
    "tree_4096": dict(B=1, Hq=32, Hkv=8, D=128, L=1024, tree=(4096, 16, None, None),
                      dtype="bf16", vocab=128256, seed=6),
}


def make_config_case(name: str, *, with_logits: Optional[bool] = None,
                     seed: Optional[int] = None) -> TreeAttnCase:
    """Inputs of one of the named workloads.

    Each sequence draws its own tree from ``default_rng(seed * 1000 + b)``;
    ragged prefix lengths (the batched workload) come from
    ``default_rng(seed).integers(lo, hi + 1, B)``.
    """
    cfg = CONFIGS[name]
    seed = cfg["seed"] if seed is None else seed
    B = cfg["B"]
    dtype = torch.float32 if cfg["dtype"] == "f32" else torch.bfloat16
    if isinstance(cfg["L"], tuple):
        lo, hi = cfg["L"]
        lens = [int(x) for x in np.random.default_rng(seed).integers(lo, hi + 1, size=B)]
    else:
        lens = [cfg["L"]] * B
    if cfg.get("example"):
        trees = [list(EXAMPLE_PARENTS)] * B
    else:
        n, roots, dmax, cmax = cfg["tree"]
        trees = [random_tree(np.random.default_rng(seed * 1000 + b), n, roots, dmax, cmax)
                 for b in range(B)]
    vocab = cfg["vocab"] if (with_logits is None or with_logits) else 0
    if with_logits and not vocab:
        vocab = 128256
    draft = None
    if cfg.get("example") and vocab:
        draft = list(EXAMPLE_TOKENS) * B
    case = make_case(name, prefix_lens=lens, trees=trees, Hq=cfg["Hq"], Hkv=cfg["Hkv"],
                     D=cfg["D"], dtype=dtype, seed=seed, vocab=vocab, draft=draft)
    if cfg.get("example") and vocab:
        # Plant the target's preference so that the branch 0 -> 1 -> 3 matches
        # and node 2 (the sibling branch) does not: a large logit at the draft
        # token of nodes 0, 1 and 3, and at another token for nodes 2 and 4.
        lg = case.logits
        for b in range(B):
            base = int(case.node_offsets[b])
            for i, tok in enumerate(EXAMPLE_TOKENS):
                want = tok if i in (0, 1, 3) else (tok + 1) % vocab
                lg[base + i, want] = 8.0
    return case


@dataclass
class SamplingCase:
    """Inputs of one tree_verify_sample call (host arrays / CPU tensors)."""
    parents: np.ndarray          # int32 [sum_N]
    node_offsets: np.ndarray     # int32 [B+1]
    logits: torch.Tensor         # [sum_N][V] bf16 or fp32
    root_logits: torch.Tensor    # [B][V]
    draft_probs: np.ndarray      # fp32 [sum_N][V]
    root_draft_probs: np.ndarray  # fp32 [B][V]
    draft: np.ndarray            # int32 [sum_N]
    u_accept: np.ndarray         # fp32 [sum_N]
    u_final: np.ndarray          # fp32 [B]
    temperature: float
    max_nodes: int


def _softmax_rows(z: np.ndarray) -> np.ndarray:
    z = z - z.max(axis=1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=1, keepdims=True)


def make_sampling_case(trees: Sequence[Sequence[int]], V: int, *, dtype=torch.bfloat16,
                       seed: int = 0, temperature: float = 1.0, scale: float = 2.0,
                       noise: float = 0.5, max_nodes: Optional[int] = None) -> SamplingCase:
    """Seeded inputs for stochastic verification over the given parent arrays
    (recipe in the module docstring).  Parents that are not a valid tree are
    kept as given (their nodes draw from the prefix row)."""
    rng = np.random.default_rng(seed)
    sizes = [len(t) for t in trees]
    B = len(trees)
    offs = np.zeros(B + 1, dtype=np.int32)
    offs[1:] = np.cumsum(sizes)
    total = int(offs[-1])
    parents = np.array([p for t in trees for p in t], dtype=np.int32)
    lg = (scale * rng.standard_normal((total + B, V))).astype(np.float32)
    lt = torch.from_numpy(lg).to(dtype)
    lg_exact = lt.to(torch.float64).numpy()
    q = _softmax_rows((lg_exact + noise * rng.standard_normal((total + B, V))) / temperature)
    q = q.astype(np.float32)
    draft = np.zeros(total, dtype=np.int32)
    for b in range(B):
        lo = int(offs[b])
        for i, p in enumerate(trees[b]):
            row = q[total + b] if not (0 <= p < sizes[b]) else q[lo + p]
            pr = row.astype(np.float64)
            draft[lo + i] = int(rng.choice(V, p=pr / pr.sum()))
    return SamplingCase(
        parents=parents, node_offsets=offs, logits=lt[:total].contiguous(),
        root_logits=lt[total:].contiguous(), draft_probs=q[:total].copy(),
        root_draft_probs=q[total:].copy(), draft=draft,
        u_accept=rng.random(total).astype(np.float32), u_final=rng.random(B).astype(np.float32),
        temperature=float(temperature),
        max_nodes=int(max_nodes if max_nodes is not None else max(1, max(sizes, default=1))))
