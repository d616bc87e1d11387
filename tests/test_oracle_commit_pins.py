"""Pins of the oracle's commit of the accepted path (and of its reading of a
prefix held in a cache slot) against facts fixed outside that code: closed
forms on chains, rows that carry their own identity, and the identity that
makes commit correct at all — after committing a node's ancestors, ordinary
decode attention of the node over the cache (PyTorch's
scaled_dot_product_attention in float64) equals that node's tree attention.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import synthetic


def _tagged_tree_rows(n, Hkv, D):
    """K/V rows whose every entry names the row: k = row + 0.25, v = -row."""
    k = torch.arange(n, dtype=torch.float32)[:, None, None].expand(n, Hkv, D) + 0.25
    return k.contiguous(), (-k + 0.25).contiguous()


def _slots(caps, lens, Hkv, D, fill=1e6):
    offs = np.concatenate([[0], np.cumsum(caps)]).astype(np.int64)
    total = int(offs[-1])
    kc = torch.full((total, Hkv, D), fill, dtype=torch.float32)
    vc = torch.full((total, Hkv, D), -fill, dtype=torch.float32)
    return kc, vc, offs, np.asarray(lens, dtype=np.int64)


def test_chain_fully_accepted_appends_rows_in_order():
    n, Hkv, D = 6, 2, 4
    kt, vt = _tagged_tree_rows(n, Hkv, D)
    kc, vc, offs, lens = _slots([10], [3], Hkv, D)
    nodes = np.full((1, 8), -1, dtype=np.int32)
    nodes[0, :n] = np.arange(n)
    kc2, vc2, lens2, st = oracle.kv_commit(kt, vt, [0, n], [n], nodes, kc, vc, offs, lens, 8)
    assert st.tolist() == [0] and lens2.tolist() == [3 + n]
    assert torch.equal(kc2[3:3 + n], kt) and torch.equal(vc2[3:3 + n], vt)
    assert torch.equal(kc2[:3], kc[:3]) and torch.equal(kc2[3 + n:], kc[3 + n:])


def test_rejected_rows_never_reach_the_cache():
    """Only the accepted path's rows, root first, land after the rows in use."""
    rng = np.random.default_rng(7)
    parents = synthetic.random_tree(rng, 40, 1, 6, 4)
    n, Hkv, D = len(parents), 2, 3
    kt, vt = _tagged_tree_rows(n, Hkv, D)
    leaf = int(np.argmax([len(oracle.root_path(parents, i)) for i in range(n)]))
    path = oracle.root_path(parents, leaf)
    nodes = np.full((1, 64), -1, dtype=np.int32)
    nodes[0, :len(path)] = path
    kc, vc, offs, lens = _slots([20], [5], Hkv, D)
    kc2, vc2, lens2, st = oracle.kv_commit(kt, vt, [0, n], [len(path)], nodes, kc, vc, offs,
                                           lens, 64)
    assert st.tolist() == [0] and lens2.tolist() == [5 + len(path)]
    got = kc2[5:5 + len(path), 0, 0].numpy() - 0.25
    np.testing.assert_array_equal(got, np.asarray(path, dtype=np.float32))
    assert torch.equal(vc2[5:5 + len(path)], vt[path])
    rejected = sorted(set(range(n)) - set(path))
    present = set((kc2[:, 0, 0] - 0.25).round().to(torch.int64).tolist())
    assert not present.intersection(rejected)


def test_empty_no_room_and_bad_ids_leave_the_sequence_untouched():
    Hkv, D = 1, 2
    kt, vt = _tagged_tree_rows(9, Hkv, D)
    node_offsets = [0, 3, 6, 9]
    kc, vc, offs, lens = _slots([4, 4, 6], [0, 3, 1], Hkv, D)
    nodes = np.full((3, 4), -1, dtype=np.int32)
    nodes[1, :2] = [0, 1]          # two rows, one free row in the slot: no room
    nodes[2, :2] = [0, 7]          # node 7 is outside a 3-node sequence
    kc2, vc2, lens2, st = oracle.kv_commit(kt, vt, node_offsets, [0, 2, 2], nodes, kc, vc, offs,
                                           lens, 4)
    assert st.tolist() == [0, oracle.STATUS_INVALID_ARG, oracle.STATUS_INVALID_ARG]
    assert lens2.tolist() == [0, 3, 1]
    assert torch.equal(kc2, kc) and torch.equal(vc2, vc)


def test_prefix_in_a_slot_reads_only_the_rows_in_use():
    """Decode attention of one root over a slot whose tail holds huge values:
    only the rows in use may count (checked with SDPA over those rows)."""
    c = synthetic.make_case("slot", prefix_lens=[9], trees=[[-1]], Hq=2, Hkv=1, D=8,
                            dtype=torch.float32, seed=11)
    kp = torch.cat([c.k_prefix, torch.full((5, 1, 8), 30.0)])
    vp = torch.cat([c.v_prefix, torch.full((5, 1, 8), -50.0)])
    out, _ = oracle.tree_attention(c.q, c.k_tree, c.v_tree, kp, vp, c.parents, c.node_offsets,
                                   [0, 14], c.scale, prefix_lens=[9])
    q = c.q.double().permute(1, 0, 2)
    k = torch.cat([c.k_prefix, c.k_tree]).double().permute(1, 0, 2).expand(2, -1, -1)
    v = torch.cat([c.v_prefix, c.v_tree]).double().permute(1, 0, 2).expand(2, -1, -1)
    ref = F.scaled_dot_product_attention(q[None], k[None], v[None], scale=c.scale)[0]
    np.testing.assert_allclose(out, ref.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_committed_ancestors_then_decode_equals_tree_attention(seed):
    """Commit path(i) minus i, then attend from node i as a new one-node step
    over the cache: the result is node i's tree attention, and both equal
    SDPA over the cache rows in use plus node i's own K/V."""
    rng = np.random.default_rng(100 + seed)
    trees = [synthetic.random_tree(rng, 12, 1, 4, 3).tolist() for _ in range(2)]
    L = [7, 0]
    Hq, Hkv, D = 4, 2, 8
    c = synthetic.make_case("commit", prefix_lens=L, trees=trees, Hq=Hq, Hkv=Hkv, D=D,
                            dtype=torch.float32, seed=seed)
    full, _ = oracle.tree_attention(c.q, c.k_tree, c.v_tree, c.k_prefix, c.v_prefix, c.parents,
                                    c.node_offsets, c.prefix_offsets, c.scale)
    caps = [L[0] + 8, L[1] + 8]
    offs = np.concatenate([[0], np.cumsum(caps)]).astype(np.int64)
    for local in (rng.integers(12), rng.integers(12)):
        local = int(local)
        kc = torch.zeros((int(offs[-1]), Hkv, D))
        vc = torch.zeros_like(kc)
        for b in range(2):                       # each slot starts with the sequence's prefix
            p0 = int(c.prefix_offsets[b])
            kc[offs[b]:offs[b] + L[b]] = c.k_prefix[p0:p0 + L[b]]
            vc[offs[b]:offs[b] + L[b]] = c.v_prefix[p0:p0 + L[b]]
        nodes = np.full((2, 12), -1, dtype=np.int32)
        acc = np.zeros(2, dtype=np.int32)
        for b in range(2):
            n0, n1 = int(c.node_offsets[b]), int(c.node_offsets[b + 1])
            anc = oracle.root_path(c.parents[n0:n1], local)[:-1]
            nodes[b, :len(anc)] = anc
            acc[b] = len(anc)
        kc2, vc2, lens2, st = oracle.kv_commit(c.k_tree, c.v_tree, c.node_offsets, acc, nodes,
                                               kc, vc, offs, np.asarray(L), 12)
        assert st.tolist() == [0, 0]
        # the next step: one root per sequence, node `local` of each tree
        g = [int(c.node_offsets[b]) + local for b in range(2)]
        out, _ = oracle.tree_attention(c.q[g], c.k_tree[g], c.v_tree[g], kc2, vc2, [-1, -1],
                                       [0, 1, 2], offs, c.scale, prefix_lens=lens2)
        np.testing.assert_allclose(out, full[g], rtol=1e-11, atol=1e-12)
        for b in range(2):
            rows = slice(int(offs[b]), int(offs[b] + lens2[b]))
            k = torch.cat([kc2[rows], c.k_tree[g[b]:g[b] + 1]]).double()
            v = torch.cat([vc2[rows], c.v_tree[g[b]:g[b] + 1]]).double()
            G = Hq // Hkv
            k = k.permute(1, 0, 2).repeat_interleave(G, 0)
            v = v.permute(1, 0, 2).repeat_interleave(G, 0)
            q = c.q[g[b]:g[b] + 1].double().permute(1, 0, 2)
            ref = F.scaled_dot_product_attention(q[None], k[None], v[None], scale=c.scale)[0]
            np.testing.assert_allclose(full[g[b]], ref[:, 0].numpy(), rtol=1e-11, atol=1e-12)
