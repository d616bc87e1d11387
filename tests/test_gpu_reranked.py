"""GPU parity on trees listed in a reranked order (a child may come before its
parent), against the fp64 oracle.

"Tree Attention" (zhongzhoutan-coder.github.io), Where It Appears: EAGLE-2
reranks its draft tree and then builds the ancestry mask, so the flattened
order need not be topological.  Each tree here is a random tree listed in a
random order (synthetic.rerank_tree).  Checked: masks, depths and statuses
bit for bit (the LDS builder up to 1024 nodes, the global one above, cycles
rejected by both and by the in-kernel builder), attention at the parity bars
(rows built in the forward kernel, a given mask, key splits merged in the
kernel and by the merge kernel, fp32), both verifiers bit for bit (the
accepted path placed root first by depth), and the commit of the accepted
path.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from helpers import DevCase, check_attention, gpu_forward, gpu_mask, lib

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ta():
    return lib()


def _reranked(rng, n, roots=1, depth=None, kids=None):
    t = synthetic.random_tree(rng, n, roots, depth, kids)
    return synthetic.rerank_tree(t, rng.permutation(n)).tolist()


def _check_mask(ta, c):
    dc = DevCase(c)
    mask, depth, status = gpu_mask(ta, dc)
    rm, rd, rs = oracle.build_mask(c.parents, c.node_offsets, dc.max_nodes)
    np.testing.assert_array_equal(status.cpu().numpy(), rs)
    np.testing.assert_array_equal(mask.cpu().numpy(), rm)
    np.testing.assert_array_equal(depth.cpu().numpy(), rd)
    return dc, mask


def _oracle(c, nodes=None):
    return oracle.tree_attention(c.q, c.k_tree, c.v_tree, c.k_prefix, c.v_prefix, c.parents,
                                 c.node_offsets, c.prefix_offsets, c.scale, nodes=nodes)


@pytest.mark.parametrize("sizes", [[1, 9, 64, 128], [300, 1024], [1500, 4096], [2000]])
def test_reranked_masks_bit_exact(ta, sizes):
    rng = np.random.default_rng(sum(sizes))
    trees = [_reranked(rng, n, 1 + n // 500) for n in sizes]
    if sizes == [2000]:
        # the deepest case: a chain listed leaf first (every parent after its child)
        trees = [list(range(1, 2000)) + [-1]]
    c = synthetic.make_case("rmask", prefix_lens=[0] * len(trees), trees=trees, Hq=1, Hkv=1,
                            D=8, dtype=torch.float32, seed=len(sizes))
    assert any(p > i for t in trees for i, p in enumerate(t)), "expected a parent after its child"
    print(f"[reranked mask] sizes={[len(t) for t in trees]}", flush=True)
    _check_mask(ta, c)


@pytest.mark.parametrize("n", [5, 700, 3000])
def test_cycles_are_invalid_trees(ta, n):
    """A cycle through the root (no path reaches -1), next to a valid reranked
    tree: status 2, rows zero and depth -1 for the cyclic sequence only."""
    rng = np.random.default_rng(n)
    cyc = synthetic.random_tree(rng, n, 1).tolist()
    cyc[0] = n - 1          # the root under its own descendant
    good = _reranked(rng, n)
    c = synthetic.make_case("rcyc", prefix_lens=[0, 0], trees=[cyc, good], Hq=1, Hkv=1, D=8,
                            dtype=torch.float32, seed=n)
    dc = DevCase(c)
    mask, depth, status = gpu_mask(ta, dc)
    assert status.cpu().tolist() == [oracle.STATUS_INVALID_TREE, 0]
    _check_mask(ta, c)


@pytest.mark.parametrize("entry", ["forward", "mask_and_forward"])
def test_reranked_forward_small_trees_bf16(ta, entry):
    """Trees up to 128 nodes (the forward builds their rows itself in
    mask_and_forward) over prefixes long enough to split the keys."""
    rng = np.random.default_rng(7)
    trees = [_reranked(rng, n, r) for n, r in ((64, 1), (128, 3), (17, 2), (100, 1))]
    # a cycle in the last sequence: its status is 2 and its rows stay zero
    trees.append([1, 2, 0])
    c = synthetic.make_case("rfwd", prefix_lens=[3000, 700, 0, 1500, 64], trees=trees, Hq=8,
                            Hkv=2, D=128, seed=7)
    dc = DevCase(c)
    rm, rd, rs = oracle.build_mask(c.parents, c.node_offsets, dc.max_nodes)
    if entry == "forward":
        mask, _, status = gpu_mask(ta, dc)
        np.testing.assert_array_equal(mask.cpu().numpy(), rm)
        out, lse = gpu_forward(ta, dc, mask)
    else:
        out, lse, fm, fd, fs = ta.mask_and_forward(
            dc.parents, dc.q, dc.k_tree, dc.v_tree, dc.k_prefix, dc.v_prefix, dc.prefix_offsets,
            dc.node_offsets, dc.max_nodes, dc.max_prefix, c.scale, return_lse=True)
        np.testing.assert_array_equal(fm.cpu().numpy(), rm)
        np.testing.assert_array_equal(fd.cpu().numpy(), rd)
        np.testing.assert_array_equal(fs.cpu().numpy(), rs)
    assert rs.tolist() == [0, 0, 0, 0, oracle.STATUS_INVALID_TREE]
    good = int(c.node_offsets[4])
    ro, rl = _oracle(c, nodes=list(range(good)))
    check_attention(out[:good], lse[:good], ro, rl, fp32=False, what=f"reranked {entry}")


def test_reranked_forward_8b_layer_shape(ta):
    """The 8B-shaped layer (one 64-node tree, L=4096, in-kernel merge of 16
    key splits per row tile) with its tree reranked: every node."""
    rng = np.random.default_rng(11)
    c = synthetic.make_case("r8b", prefix_lens=[4096], trees=[_reranked(rng, 64, 1, 6, 4)],
                            Hq=32, Hkv=8, D=128, seed=11)
    for entry in ("forward", "mask_and_forward"):
        dc = DevCase(c)
        if entry == "forward":
            mask, _, _ = gpu_mask(ta, dc)
            out, lse = gpu_forward(ta, dc, mask)
        else:
            out, lse, *_ = ta.mask_and_forward(
                dc.parents, dc.q, dc.k_tree, dc.v_tree, dc.k_prefix, dc.v_prefix,
                dc.prefix_offsets, dc.node_offsets, dc.max_nodes, dc.max_prefix, c.scale,
                return_lse=True)
        ro, rl = _oracle(c)
        check_attention(out, lse, ro, rl, fp32=False, what=f"reranked 8B layer, {entry}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_reranked_forward_large_trees(ta, dtype):
    """512- and 1500-node reranked trees (rows from the builder, tree keys
    anywhere in the sequence), every node."""
    D = 128 if dtype == torch.bfloat16 else 64
    rng = np.random.default_rng(13)
    trees = [_reranked(rng, 512, 8, 16), _reranked(rng, 1500, 6, 20)]
    c = synthetic.make_case("rlarge", prefix_lens=[96, 64], trees=trees, Hq=8, Hkv=2, D=D,
                            dtype=dtype, seed=13)
    dc, mask = _check_mask(ta, c)
    out, lse = gpu_forward(ta, dc, mask)
    ro, rl = _oracle(c)
    check_attention(out, lse, ro, rl, fp32=dtype == torch.float32, what=f"reranked {dtype}")


def _same(got, ref, names):
    for n, a, r in zip(names, got, ref):
        np.testing.assert_array_equal(a.cpu().numpy(), r, err_msg=n)


@pytest.mark.parametrize("sizes,V", [([1, 30, 200, 64], 50000), ([1500, 3000], 1000)])
def test_reranked_verify_bit_exact(ta, sizes, V):
    rng = np.random.default_rng(V + len(sizes))
    trees = [_reranked(rng, n, 1 + n // 400, 8) for n in sizes]
    c = synthetic.make_case("rver", prefix_lens=[0] * len(trees), trees=trees, Hq=1, Hkv=1, D=8,
                            dtype=torch.bfloat16, seed=V, vocab=V, p_match=0.92)
    dc, mask = _check_mask(ta, c)
    got = ta.verify_greedy(dc.logits, dc.draft, mask, dc.node_offsets, dc.max_nodes)
    ref = oracle.verify_greedy(c.logits, c.draft, c.parents, c.node_offsets, dc.max_nodes)
    _same(got, ref, ("target_argmax", "accept_len", "accept_nodes", "accept_tokens"))
    print(f"[reranked verify] accept_len={ref[1].tolist()}", flush=True)
    # next-token rows: drafts that follow the parent's prediction mostly
    root = torch.randn((c.B, V), generator=torch.Generator().manual_seed(V)).to(torch.bfloat16)
    pred = np.argmax(c.logits.double().numpy(), axis=1)
    rpred = np.argmax(root.double().numpy(), axis=1)
    draft = np.array(c.draft)
    for b in range(c.B):
        lo, hi = int(c.node_offsets[b]), int(c.node_offsets[b + 1])
        for i in range(hi - lo):
            p = int(c.parents[lo + i])
            if rng.random() < 0.9:
                draft[lo + i] = rpred[b] if p < 0 else pred[lo + p]
    d = torch.from_numpy(draft.astype(np.int32)).cuda()
    got = ta.verify_greedy_next(dc.logits, root.cuda(), d, mask, dc.node_offsets, dc.max_nodes)
    ref = oracle.verify_greedy_next(c.logits, root, draft, c.parents, c.node_offsets,
                                    dc.max_nodes)
    _same(got, ref, ("target_argmax", "accept_len", "accept_nodes", "accept_tokens",
                     "bonus_token"))
    assert max(ref[1]) >= 3, "the drafts should give paths of several nodes"


def test_reranked_commit_appends_the_path_root_first(ta):
    """Verify a reranked tree, commit its accepted path: the cache rows are the
    accepted nodes' K/V rows in root-to-leaf order (oracle commit)."""
    rng = np.random.default_rng(17)
    trees = [_reranked(rng, 40, 1, 8), _reranked(rng, 90, 2, 10)]
    c = synthetic.make_case("rcommit", prefix_lens=[5, 9], trees=trees, Hq=2, Hkv=1, D=64,
                            seed=17, vocab=500, p_match=0.95)
    dc, mask = _check_mask(ta, c)
    _, alen, anodes, _ = ta.verify_greedy(dc.logits, dc.draft, mask, dc.node_offsets,
                                          dc.max_nodes)
    L = [5, 9]
    room = [dc.max_nodes, dc.max_nodes]
    offs = np.zeros(3, np.int64)
    offs[1:] = np.cumsum(np.array(L) + np.array(room))
    kc = torch.zeros((int(offs[-1]), 1, 64), dtype=torch.bfloat16)
    vc = torch.zeros_like(kc)
    lens = torch.tensor(L, dtype=torch.int64)
    rk, rv, rlens, rst = oracle.kv_commit(c.k_tree, c.v_tree, c.node_offsets,
                                          alen.cpu().numpy(), anodes.cpu().numpy(), kc.clone(),
                                          vc.clone(), offs, lens.clone(), dc.max_nodes)
    kd, vd = kc.cuda(), vc.cuda()
    ld = lens.cuda()
    st = ta.kv_commit(dc.k_tree, dc.v_tree, dc.node_offsets, alen, anodes, kd, vd,
                      torch.from_numpy(offs).cuda(), ld)
    assert st.cpu().tolist() == list(rst) == [0, 0]
    assert torch.equal(kd.cpu(), rk) and torch.equal(vd.cpu(), rv)
    assert ld.cpu().tolist() == list(rlens)
    assert int(alen.sum()) >= 2
