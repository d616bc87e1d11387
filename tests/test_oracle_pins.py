"""Pins of the fp64 oracle against facts fixed outside the oracle's own code.

Each test ties one oracle function to something the pages or the mathematics
fix: the pages' worked example, brute force on tiny inputs computed another
way, textbook special cases checked with a library routine (PyTorch's
scaled_dot_product_attention in float64), closed forms and invariants.  Each
plausible slip in the oracle (a dropped term, a wrong index, a sibling leak, a
transposed operand, the wrong KV head) fails at least one of them.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import synthetic

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _example():
    with open(os.path.join(GOLDEN, "example_tree.json")) as f:
        return json.load(f)


def _all_topological_parent_arrays(n):
    """Every parent array with parent[i] in {-1} U [0, i): n! of them."""
    choices = [range(-1, i) for i in range(n)]
    for combo in itertools.product(*choices):
        yield list(combo)


def _closure_by_matrix_powers(parents):
    """Ancestor-or-self relation as the reflexive-transitive closure of the
    child->parent adjacency matrix, via repeated boolean matrix products."""
    n = len(parents)
    a = np.zeros((n, n), dtype=np.int64)
    for i, p in enumerate(parents):
        if p >= 0:
            a[i, p] = 1
    reach = np.eye(n, dtype=np.int64)
    power = np.eye(n, dtype=np.int64)
    for _ in range(n):
        power = (power @ a > 0).astype(np.int64)
        reach = ((reach + power) > 0).astype(np.int64)
    return reach.astype(bool)


def _pack_with_numpy(dense, words):
    """Little-endian bit packing by numpy.packbits, viewed as uint64 words."""
    n = dense.shape[0]
    padded = np.zeros((n, words * 64), dtype=bool)
    padded[:, :dense.shape[1]] = dense
    by = np.packbits(padded, axis=1, bitorder="little")
    return by.view("<u8").reshape(n, words)


# ----------------------------------------------------------------- mask pins

def test_example_tree_mask_matches_worked_example():
    ex = _example()
    parents = ex["parents"]
    dense = oracle.ancestor_mask_dense(parents)
    assert dense.astype(int).tolist() == ex["mask_rows"]
    mask, depth, status = oracle.build_mask(np.array(parents, np.int32),
                                            np.array([0, 5], np.int32), 5)
    assert status.tolist() == [0]
    assert mask[:, 0].astype(np.int64).tolist() == ex["mask_words"]
    assert depth.tolist() == ex["depth"]
    assert abs((~dense).mean() - ex["hidden_fraction"]) < 1e-12
    # siblings 1 and 2 never see each other; the grandchildren see only their own branch
    assert not dense[1, 2] and not dense[2, 1] and not dense[3, 2] and not dense[4, 1]


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 6])
def test_mask_equals_transitive_closure_for_every_tiny_tree(n):
    for parents in _all_topological_parent_arrays(n):
        dense = oracle.ancestor_mask_dense(parents)
        np.testing.assert_array_equal(dense, _closure_by_matrix_powers(parents))


def test_mask_brute_force_n7_packing_and_depth():
    W = 1
    for parents in _all_topological_parent_arrays(7):
        mask, depth, status = oracle.build_mask(np.array(parents, np.int32),
                                                np.array([0, 7], np.int32), 7)
        closure = _closure_by_matrix_powers(parents)
        np.testing.assert_array_equal(mask, _pack_with_numpy(closure, W))
        np.testing.assert_array_equal(depth, closure.sum(axis=1) - 1)


def test_mask_multiword_packing_and_invariants():
    rng = np.random.default_rng(7)
    parents = synthetic.random_tree(rng, 300, n_roots=3, max_depth=40, max_children=None)
    mask, depth, status = oracle.build_mask(parents, np.array([0, 300], np.int32), 300)
    W = 5
    assert mask.shape == (300, W)
    dense = _closure_by_matrix_powers(parents.tolist())
    np.testing.assert_array_equal(mask, _pack_with_numpy(dense, W))
    for i, p in enumerate(parents):
        bit = np.zeros(W, np.uint64)
        bit[i // 64] = np.uint64(1) << np.uint64(i % 64)
        if p >= 0:
            np.testing.assert_array_equal(mask[i], mask[p] | bit)   # mask[i] = mask[p] | self
        assert dense[i, :i + 1].sum() == dense[i].sum()             # only earlier nodes
        assert int(sum(bin(int(w)).count("1") for w in mask[i])) == depth[i] + 1


def test_mask_rejects_invalid_trees_and_offsets():
    off = np.array([0, 3, 6, 9, 12, 15], np.int32)
    parents = np.array([-1, 0, 1,    -1, 2, 0,    -1, 0, 3,    -1, 1, 1,    1, 2, 0], np.int32)
    mask, depth, status = oracle.build_mask(parents, off, 3)
    # a later parent is fine (a reranked tree: 0 <- 2 <- 1); a parent out of
    # range, a self-parent and a cycle (0 -> 1 -> 2 -> 0, no root) are not
    assert status.tolist() == [0, 0, 2, 2, 2]
    assert mask[3:6, 0].tolist() == [0b001, 0b111, 0b101] and depth[3:6].tolist() == [0, 2, 1]
    assert (mask[6:] == 0).all() and (depth[6:] == -1).all()
    mask, depth, status = oracle.build_mask(parents[:6], np.array([0, 3, 6], np.int32), 2)
    assert status.tolist() == [1, 1]              # more nodes than max_nodes


def _all_parent_arrays(n):
    """Every array with entries in {-1} U [0, n): (n + 1)^n of them, in any
    order, with cycles and self-parents among them."""
    return itertools.product(range(-1, n), repeat=n)


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
def test_validity_is_acyclicity_for_every_tiny_parent_array(n):
    """A parent array is a forest iff its child -> parent adjacency matrix is
    nilpotent (no walk of length n exists: the n-th boolean power is zero);
    valid ones, in whatever order, get the transitive closure as their mask."""
    for parents in _all_parent_arrays(n):
        a = np.zeros((n, n), dtype=np.int64)
        for i, p in enumerate(parents):
            if p >= 0:
                a[i, p] = 1
        nilpotent = not np.linalg.matrix_power(a, n).any()
        self_free = all(p != i for i, p in enumerate(parents))
        assert oracle.tree_is_valid(parents) == (nilpotent and self_free), parents
        if nilpotent:
            np.testing.assert_array_equal(oracle.ancestor_mask_dense(list(parents)),
                                          _closure_by_matrix_powers(list(parents)))


def _perm_matrix_check(parents, perm):
    """Mask of the reranked tree = P M P^T: row k, column k' of the reranked
    mask is row perm[k], column perm[k'] of the original one."""
    re = synthetic.rerank_tree(parents, perm)
    d0 = oracle.ancestor_mask_dense(parents)
    d1 = oracle.ancestor_mask_dense(re)
    np.testing.assert_array_equal(d1, d0[np.ix_(perm, perm)])
    return re


def test_reranked_tree_mask_and_depth_follow_the_permutation():
    rng = np.random.default_rng(23)
    for n, roots in ((9, 1), (70, 3), (200, 5)):
        parents = synthetic.random_tree(rng, n, n_roots=roots)
        perm = rng.permutation(n)
        re = _perm_matrix_check(parents, perm)
        W = -(-n // 64)
        m0, d0, s0 = oracle.build_mask(parents, np.array([0, n], np.int32), n)
        m1, d1, s1 = oracle.build_mask(re, np.array([0, n], np.int32), n)
        assert s1.tolist() == [0]
        np.testing.assert_array_equal(d1, d0[perm])
        assert any(re[k] > k for k in range(n)), "the reranked order should not be topological"
        np.testing.assert_array_equal(m1, _pack_with_numpy(_closure_by_matrix_powers(re.tolist()),
                                                           W))


# ------------------------------------------------------------ attention pins

def _sdpa(q, k, v, mask, scale):
    """float64 CPU scaled_dot_product_attention; q [H][Lq][D], k/v [H][Lk][D]."""
    out = F.scaled_dot_product_attention(q[None], k[None], v[None], attn_mask=mask, scale=scale)
    return out[0]


def _case(prefix, trees, Hq=2, Hkv=1, D=16, seed=0, dtype=torch.float32):
    return synthetic.make_case("pin", prefix_lens=prefix, trees=trees, Hq=Hq, Hkv=Hkv, D=D,
                               dtype=dtype, seed=seed)


def _run(c, nodes=None, **kw):
    return oracle.tree_attention(c.q, c.k_tree, c.v_tree, c.k_prefix, c.v_prefix, c.parents,
                                 c.node_offsets, c.prefix_offsets, c.scale, nodes=nodes, **kw)


@pytest.mark.parametrize("L,N", [(0, 1), (0, 6), (9, 5), (33, 12)])
def test_chain_tree_equals_causal_attention(L, N):
    """A chain is an ordinary sequence: tree attention must equal bottom-right
    aligned causal attention over prefix + chain."""
    c = _case([L], [[-1] + list(range(N - 1))], Hq=3, Hkv=3, D=8, seed=L + N)
    out, lse = _run(c)
    q = c.q.double().permute(1, 0, 2)                          # [H][N][D]
    k = torch.cat([c.k_prefix, c.k_tree]).double().permute(1, 0, 2)
    v = torch.cat([c.v_prefix, c.v_tree]).double().permute(1, 0, 2)
    allow = torch.ones(N, L + N, dtype=torch.bool).tril(diagonal=L)
    ref = _sdpa(q, k, v, allow, c.scale).permute(1, 0, 2).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)
    # lse against the explicit log-sum-exp of the same causal scores
    s = (q @ k.transpose(1, 2)) * c.scale
    s = s.masked_fill(~allow, float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=2).T.numpy(), rtol=1e-12, atol=1e-12)


def test_single_node_equals_decode_attention():
    c = _case([50], [[-1]], Hq=4, Hkv=4, D=32, seed=3)
    out, _ = _run(c)
    q = c.q.double().permute(1, 0, 2)
    k = torch.cat([c.k_prefix, c.k_tree]).double().permute(1, 0, 2)
    v = torch.cat([c.v_prefix, c.v_tree]).double().permute(1, 0, 2)
    ref = _sdpa(q, k, v, None, c.scale).permute(1, 0, 2).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_empty_prefix_root_returns_its_value_row_exactly():
    c = _case([0, 0], [[-1, 0, 0], [-1, -1]], Hq=2, Hkv=1, D=8, seed=4)
    out, lse = _run(c)
    for gi in (0, 3, 4):                                  # the roots
        np.testing.assert_array_equal(out[gi], np.repeat(c.v_tree[gi].double().numpy(), 2, 0))
        np.testing.assert_allclose(lse[gi], c.scale * (c.q[gi].double() @ c.k_tree[gi, 0].double()).numpy(),
                                   rtol=1e-12)


def test_equal_keys_give_mean_of_visible_values():
    c = _case([7], [synthetic.EXAMPLE_PARENTS], Hq=2, Hkv=1, D=8, seed=5)
    c.k_prefix[:] = 0.5
    c.k_tree[:] = 0.5
    out, _ = _run(c)
    vis = oracle.ancestor_mask_dense(synthetic.EXAMPLE_PARENTS)
    for i in range(5):
        rows = torch.cat([c.v_prefix[:, 0], c.v_tree[torch.from_numpy(np.flatnonzero(vis[i])), 0]])
        np.testing.assert_allclose(out[i, 0], rows.double().mean(0).numpy(), rtol=1e-12, atol=1e-13)


def test_example_tree_matches_sdpa_with_tree_mask():
    """The worked-example tree through the library routine with the explicit
    prefix-plus-ancestors visibility matrix of the golden fixture."""
    ex = _example()
    c = _case([11], [ex["parents"]], Hq=2, Hkv=2, D=16, seed=6)
    out, _ = _run(c)
    allow = torch.cat([torch.ones(5, 11, dtype=torch.bool),
                       torch.tensor(ex["mask_rows"], dtype=torch.bool)], dim=1)
    q = c.q.double().permute(1, 0, 2)
    k = torch.cat([c.k_prefix, c.k_tree]).double().permute(1, 0, 2)
    v = torch.cat([c.v_prefix, c.v_tree]).double().permute(1, 0, 2)
    ref = _sdpa(q, k, v, allow, c.scale).permute(1, 0, 2).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_gqa_equals_mha_on_repeated_kv():
    trees = [synthetic.random_tree(np.random.default_rng(9), 10, 1, 3, 3).tolist()]
    c = _case([20], trees, Hq=6, Hkv=2, D=8, seed=9)
    out, lse = _run(c)
    m = _case([20], trees, Hq=6, Hkv=6, D=8, seed=9)
    for name in ("k_tree", "v_tree", "k_prefix", "v_prefix"):
        setattr(m, name, getattr(c, name).repeat_interleave(3, dim=1))
    m.q = c.q
    out2, lse2 = _run(m)
    np.testing.assert_allclose(out, out2, rtol=1e-12, atol=1e-14)   # BLAS blocking may differ
    np.testing.assert_allclose(lse, lse2, rtol=1e-12, atol=1e-14)


def test_non_ancestor_rows_do_not_matter():
    parents = synthetic.random_tree(np.random.default_rng(11), 24, 2, 5, 3)
    c = _case([6], [parents.tolist()], Hq=2, Hkv=1, D=8, seed=11)
    out, lse = _run(c)
    vis = oracle.ancestor_mask_dense(parents)
    for i in (5, 17, 23):
        hidden = np.flatnonzero(~vis[i])
        d = _case([6], [parents.tolist()], Hq=2, Hkv=1, D=8, seed=11)
        d.k_tree[hidden] += 3.0
        d.v_tree[hidden] -= 7.0
        o2, l2 = _run(d, nodes=[i])
        np.testing.assert_array_equal(o2[0], out[i])
        np.testing.assert_array_equal(l2[0], lse[i])
        if hidden.size:   # and the rows it does see do matter
            e = _case([6], [parents.tolist()], Hq=2, Hkv=1, D=8, seed=11)
            e.v_tree[i] += 1.0
            assert not np.array_equal(_run(e, nodes=[i])[0][0], out[i])


def test_path_rows_are_the_ancestors_outputs():
    parents = synthetic.random_tree(np.random.default_rng(12), 30, 1, 6, 4)
    c = _case([13], [parents.tolist()], Hq=4, Hkv=2, D=8, seed=12)
    out, lse, rows = _run(c, return_path_rows=True)
    for path, seq_rows in rows:
        for k, node in enumerate(path):
            np.testing.assert_allclose(seq_rows[k], out[node], rtol=1e-12, atol=1e-13)


def test_lse_consistent_with_an_extra_key():
    """Prepending one prefix key with score s0 and value v0 must give
    (e^lse o + e^s0 v0) / (e^lse + e^s0): pins lse and out together."""
    parents = [-1, 0, 1, 0]
    a = _case([5], [parents], Hq=1, Hkv=1, D=8, seed=13)
    b = _case([6], [parents], Hq=1, Hkv=1, D=8, seed=13)
    b.q, b.k_tree, b.v_tree = a.q, a.k_tree, a.v_tree
    k0 = torch.full((1, 1, 8), 0.25)
    v0 = torch.arange(8, dtype=torch.float32).reshape(1, 1, 8)
    b.k_prefix = torch.cat([k0, a.k_prefix])
    b.v_prefix = torch.cat([v0, a.v_prefix])
    o1, l1 = _run(a)
    o2, l2 = _run(b)
    s0 = a.scale * (a.q[:, 0].double() @ k0[0, 0].double()).numpy()
    w1, w0 = np.exp(l1[:, 0]), np.exp(s0)
    expect = (w1[:, None] * o1[:, 0] + w0[:, None] * v0[0, 0].double().numpy()) / (w1 + w0)[:, None]
    np.testing.assert_allclose(o2[:, 0], expect, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l2[:, 0], np.log(w1 + w0), rtol=1e-12)


def test_forest_trees_do_not_see_each_other_and_sequences_are_independent():
    trees = [[-1, 0, -1, 2, 1], [-1, 0]]
    c = _case([4, 3], trees, Hq=2, Hkv=1, D=8, seed=14)
    out, _ = _run(c)
    alone = _case([3], [[-1, 0]], Hq=2, Hkv=1, D=8, seed=99)
    for name in ("q", "k_tree", "v_tree"):
        setattr(alone, name, getattr(c, name)[5:7].clone())
    alone.k_prefix, alone.v_prefix = c.k_prefix[4:7].clone(), c.v_prefix[4:7].clone()
    np.testing.assert_array_equal(_run(alone)[0], out[5:7])
    d = _case([4, 3], trees, Hq=2, Hkv=1, D=8, seed=14)
    d.k_tree[[0, 1, 4]] *= -2.0                   # first tree of the forest
    np.testing.assert_array_equal(_run(d, nodes=[2, 3])[0], out[2:4])


# ---------------------------------------------------------- verifier pins

def test_argmax_matches_library_routines_with_forced_ties():
    g = torch.Generator().manual_seed(21)
    lg = torch.randn(40, 300, generator=g).to(torch.bfloat16)
    lg[3, 10] = lg[3, 200] = 9.0                  # tie: lowest index wins
    lg[4, :] = 0.0
    lg[5, 7] = -0.0
    lg[5, :] = -1.0
    lg[5, 7] = -0.0
    lg[5, 8] = 0.0                               # -0 == +0: index 7
    pred = oracle.target_argmax(lg)
    np.testing.assert_array_equal(pred, np.argmax(lg.float().numpy(), axis=1))
    np.testing.assert_array_equal(pred, torch.argmax(lg.float(), dim=1).numpy())
    assert pred[3] == 10 and pred[4] == 0 and pred[5] == 7


def _children(parents):
    ch = {i: [] for i in range(len(parents))}
    for i, p in enumerate(parents):
        if p >= 0:
            ch[p].append(i)
    return ch


def _best_path_by_dfs(parents, match):
    """Enumerate every root-to-node path top-down; keep the longest fully
    matching one, lowest terminal index on ties."""
    ch = _children(parents)
    best = []
    stack = [[r] for r in range(len(parents)) if parents[r] == -1]
    while stack:
        path = stack.pop()
        if not all(match[j] for j in path):
            continue
        if len(path) > len(best) or (len(path) == len(best) and path[-1] < best[-1]):
            best = path
        for c in ch[path[-1]]:
            stack.append(path + [c])
    return best


def _logits_for(pred, V, rng):
    lg = rng.standard_normal((len(pred), V)).astype(np.float32)
    lg[np.arange(len(pred)), pred] = 10.0
    return torch.from_numpy(lg)


@pytest.mark.parametrize("seed", range(12))
def test_verify_matches_dfs_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    trees = [synthetic.random_tree(rng, int(rng.integers(1, 40)), int(rng.integers(1, 4)), 6, 3)
             for _ in range(3)]
    parents = np.concatenate(trees).astype(np.int32)
    off = np.zeros(4, np.int32)
    off[1:] = np.cumsum([len(t) for t in trees])
    V = 50
    pred = rng.integers(0, V, len(parents))
    draft = np.where(rng.random(len(parents)) < 0.75, pred, rng.integers(0, V, len(parents)))
    lg = _logits_for(pred, V, rng)
    maxn = max(len(t) for t in trees)
    p, alen, anodes, atok = oracle.verify_greedy(lg, draft, parents, off, maxn)
    np.testing.assert_array_equal(p, pred)
    for b, t in enumerate(trees):
        lo = off[b]
        match = [draft[lo + i] == pred[lo + i] for i in range(len(t))]
        best = _best_path_by_dfs(t.tolist(), match)
        assert alen[b] == len(best)
        assert anodes[b, :len(best)].tolist() == best
        assert (anodes[b, len(best):] == -1).all()
        assert atok[b, :len(best)].tolist() == [int(draft[lo + j]) for j in best]


@pytest.mark.parametrize("seed", range(8))
def test_verify_reranked_matches_dfs_brute_force(seed):
    """Trees listed in a random order (children before parents): the DFS over
    children lists does not use the order, so it pins the oracle there too."""
    rng = np.random.default_rng(200 + seed)
    trees = []
    for _ in range(3):
        t = synthetic.random_tree(rng, int(rng.integers(1, 40)), int(rng.integers(1, 4)), 6, 3)
        trees.append(synthetic.rerank_tree(t, rng.permutation(len(t))))
    parents = np.concatenate(trees).astype(np.int32)
    off = np.zeros(4, np.int32)
    off[1:] = np.cumsum([len(t) for t in trees])
    V = 50
    pred = rng.integers(0, V, len(parents))
    draft = np.where(rng.random(len(parents)) < 0.8, pred, rng.integers(0, V, len(parents)))
    lg = _logits_for(pred, V, rng)
    maxn = max(len(t) for t in trees)
    p, alen, anodes, atok = oracle.verify_greedy(lg, draft, parents, off, maxn)
    for b, t in enumerate(trees):
        lo = off[b]
        match = [draft[lo + i] == pred[lo + i] for i in range(len(t))]
        best = _best_path_by_dfs(t.tolist(), match)
        assert alen[b] == len(best)
        assert anodes[b, :len(best)].tolist() == best
        assert atok[b, :len(best)].tolist() == [int(draft[lo + j]) for j in best]


def test_reranked_tree_attention_is_the_permuted_attention():
    """Listing the nodes of a tree in another order (their rows and parent
    links moved along) permutes the outputs and changes nothing else: every
    node's visible set is the same set of rows."""
    rng = np.random.default_rng(41)
    n = 37
    parents = synthetic.random_tree(rng, n, n_roots=2, max_depth=7)
    c0 = _case([11], [parents.tolist()], Hq=4, Hkv=2, D=16, seed=41)
    perm = rng.permutation(n)
    c1 = _case([11], [synthetic.rerank_tree(parents, perm).tolist()], Hq=4, Hkv=2, D=16, seed=41)
    c1.q, c1.k_tree, c1.v_tree = c0.q[perm], c0.k_tree[perm], c0.v_tree[perm]
    c1.k_prefix, c1.v_prefix = c0.k_prefix, c0.v_prefix
    o0, l0 = _run(c0)
    o1, l1 = _run(c1)
    np.testing.assert_array_equal(o1, o0[perm])
    np.testing.assert_array_equal(l1, l0[perm])


def test_verify_on_chain_equals_flat_scan():
    """On a chain the flattened order is the path order, so the code listing's
    flat scan (stop at the first mismatch) is exact there."""
    rng = np.random.default_rng(31)
    for trial in range(20):
        n = int(rng.integers(1, 30))
        parents = np.array([-1] + list(range(n - 1)), np.int32)
        pred = rng.integers(0, 20, n)
        draft = np.where(rng.random(n) < 0.8, pred, (pred + 1) % 20)
        lg = _logits_for(pred, 20, rng)
        _, alen, anodes, atok = oracle.verify_greedy(lg, draft, parents, np.array([0, n], np.int32), n)
        flat = []
        for i in range(n):
            if draft[i] == pred[i]:
                flat.append(int(draft[i]))
            else:
                break
        assert alen[0] == len(flat)
        assert atok[0, :len(flat)].tolist() == flat


def test_verify_example_and_degenerate_cases():
    ex = _example()
    parents = np.array(ex["parents"], np.int32)
    toks = np.array(ex["tokens"], np.int32)
    off = np.array([0, 5], np.int32)
    rng = np.random.default_rng(41)
    # all match: deepest node, lowest index among equal depth -> path 0,1,3
    _, alen, anodes, atok = oracle.verify_greedy(_logits_for(toks, 10000, rng), toks, parents, off, 5)
    assert alen[0] == 3 and anodes[0].tolist() == [0, 1, 3, -1, -1]
    assert atok[0, :3].tolist() == [1204, 3401, 451]
    # node 1 rejected: the other branch wins
    pred = toks.copy()
    pred[1] += 1
    _, alen, anodes, _ = oracle.verify_greedy(_logits_for(pred, 10000, rng), toks, parents, off, 5)
    assert alen[0] == 3 and anodes[0, :3].tolist() == [0, 2, 4]
    # root rejected: nothing accepted
    pred = toks.copy()
    pred[0] += 1
    _, alen, anodes, atok = oracle.verify_greedy(_logits_for(pred, 10000, rng), toks, parents, off, 5)
    assert alen[0] == 0 and (anodes == -1).all() and (atok == -1).all()
