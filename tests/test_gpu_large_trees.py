"""GPU parity for trees above 1024 nodes (up to the 4096-node limit), where
the mask builder and the path selection leave LDS for global memory: masks,
depths and statuses bit for bit against the oracle (and the closed form of a
chain at the limit), attention against the oracle at the bf16 and fp32 bars
on every node or on sampled nodes, both verifiers and the commit bit for bit,
and the two-call mask-and-forward path against separate calls."""
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


def _trees(seed, spec):
    rng = np.random.default_rng(seed)
    return [synthetic.random_tree(rng, n, r, d, c).tolist() for n, r, d, c in spec]


def _check_mask(ta, c):
    dc = DevCase(c)
    mask, depth, status = gpu_mask(ta, dc)
    rm, rd, rs = oracle.build_mask(c.parents, c.node_offsets, dc.max_nodes)
    np.testing.assert_array_equal(status.cpu().numpy(), rs)
    np.testing.assert_array_equal(mask.cpu().numpy(), rm)
    np.testing.assert_array_equal(depth.cpu().numpy(), rd)
    return dc, mask


def test_large_masks_bit_exact(ta):
    trees = _trees(1, [(4096, 1, 16, 4), (2000, 8, 40, None), (1100, 1, 6, None)])
    trees += [[-1] + list(range(1499)), [-1]]
    c = synthetic.make_case("lmask", prefix_lens=[0] * 5, trees=trees, Hq=1, Hkv=1, D=8,
                            dtype=torch.float32, seed=1)
    print(f"[large mask] sizes={[len(t) for t in trees]}", flush=True)
    _check_mask(ta, c)


def test_large_mask_invalid_tree_and_chain_at_the_limit(ta):
    bad = _trees(2, [(1500, 1, 12, None)])[0]
    bad[0] = 900                                     # the root under a descendant: a cycle
    chain = [-1] + list(range(4095))
    c = synthetic.make_case("lbad", prefix_lens=[0] * 3, trees=[bad, chain, [-1, 0]], Hq=1,
                            Hkv=1, D=8, dtype=torch.float32, seed=2)
    dc = DevCase(c)
    mask, depth, status = gpu_mask(ta, dc)
    assert status.cpu().tolist() == [oracle.STATUS_INVALID_TREE, 0, 0]
    m = mask.cpu().numpy()
    d = depth.cpu().numpy()
    assert (m[:1500] == 0).all() and (d[:1500] == -1).all()
    # Chain closed form: row i holds bits 0..i, depth i.
    rows = m[1500:5596]
    i = np.arange(4096)
    full_words = i[:, None] // 64 > np.arange(64)[None, :]
    part = (i[:, None] // 64 == np.arange(64)[None, :])
    want = np.where(full_words, np.uint64(0xFFFFFFFFFFFFFFFF), np.uint64(0))
    tail = ((np.uint64(1) << (i % 64 + 1).astype(np.uint64)) - np.uint64(1)).astype(np.uint64)
    tail = np.where(i % 64 == 63, np.uint64(0xFFFFFFFFFFFFFFFF), tail)
    want = np.where(part, tail[:, None], want)
    np.testing.assert_array_equal(rows, want)
    np.testing.assert_array_equal(d[1500:5596], i)
    assert m[5596, 0] == 1 and m[5597, 0] == 3 and d[5596:].tolist() == [0, 1]


def test_large_forward_bf16_sampled_at_the_limit(ta):
    trees = _trees(3, [(4096, 1, 16, 4)])
    c = synthetic.make_case("lfwd", prefix_lens=[100], trees=trees, Hq=4, Hkv=1, D=128, seed=3)
    dc, mask = _check_mask(ta, c)
    out, lse = gpu_forward(ta, dc, mask)
    rng = np.random.default_rng(4)
    nodes = sorted(set(range(48)) | set(range(4096 - 48, 4096)) |
                   set(rng.choice(4096, 160, replace=False).tolist()))
    ref_o, ref_l = oracle.tree_attention(c.q, c.k_tree, c.v_tree, c.k_prefix, c.v_prefix,
                                         c.parents, c.node_offsets, c.prefix_offsets, c.scale,
                                         nodes=nodes)
    check_attention(out[nodes], lse[nodes], ref_o, ref_l, fp32=False, what="bf16 N=4096 sampled")


@pytest.mark.parametrize("order", ["root_first", "leaf_first"])
@pytest.mark.parametrize("Hkv", [1, 2])
def test_large_forward_chain_gathered_and_dense_splits(ta, order, Hkv):
    """A 4096-node chain: a workgroup's rows near the root see few tree keys
    (listed and gathered), those near the leaf see thousands (more than the
    key list holds, so the split walks the dense tree tiles that hold a
    visible key); both kinds of split in one call, on the 128-row two-key-
    group shape (one KV head) and the 256-row shape (two).  Leaf first lists
    every parent after its child."""
    n = 4096
    chain = [-1] + list(range(n - 1)) if order == "root_first" else list(range(1, n)) + [-1]
    c = synthetic.make_case("lchainf", prefix_lens=[100], trees=[chain], Hq=4 * Hkv, Hkv=Hkv,
                            D=128, seed=8 + Hkv)
    dc, mask = _check_mask(ta, c)
    out, lse = gpu_forward(ta, dc, mask)
    rng = np.random.default_rng(9)
    nodes = sorted(set(range(40)) | set(range(n - 40, n)) | set(range(2000, 2100)) |
                   set(rng.choice(n, 120, replace=False).tolist()))
    ref_o, ref_l = oracle.tree_attention(c.q, c.k_tree, c.v_tree, c.k_prefix, c.v_prefix,
                                         c.parents, c.node_offsets, c.prefix_offsets, c.scale,
                                         nodes=nodes)
    check_attention(out[nodes], lse[nodes], ref_o, ref_l, fp32=False,
                    what=f"bf16 chain {order} Hkv={Hkv}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_large_forward_full(ta, dtype):
    D = 128 if dtype == torch.bfloat16 else 64
    # Prefixes of 96 and 64 keys keep the outputs at the magnitude the bf16
    # bar is set for (a tree-only row averages a few V rows, and bf16 alone
    # rounds an output above 2 by up to 0.008).
    trees = _trees(5, [(1500, 6, 20, None), (600, 1, 8, 3)])
    c = synthetic.make_case("lfull", prefix_lens=[96, 64], trees=trees, Hq=8, Hkv=2, D=D,
                            dtype=dtype, seed=5)
    dc, mask = _check_mask(ta, c)
    out, lse = gpu_forward(ta, dc, mask)
    ref_o, ref_l = oracle.tree_attention(c.q, c.k_tree, c.v_tree, c.k_prefix, c.v_prefix,
                                         c.parents, c.node_offsets, c.prefix_offsets, c.scale)
    check_attention(out, lse, ref_o, ref_l, fp32=dtype == torch.float32,
                    what=f"{dtype} N=1500+600")


def test_large_mask_and_forward_matches_separate_calls(ta):
    trees = _trees(6, [(1300, 2, 12, None)])
    c = synthetic.make_case("lmf", prefix_lens=[64], trees=trees, Hq=4, Hkv=1, D=128, seed=6)
    dc = DevCase(c)
    mask, depth, status = gpu_mask(ta, dc)
    out, lse = gpu_forward(ta, dc, mask)
    o2, l2, m2, d2, s2 = ta.mask_and_forward(dc.parents, dc.q, dc.k_tree, dc.v_tree,
                                             dc.k_prefix, dc.v_prefix, dc.prefix_offsets,
                                             dc.node_offsets, dc.max_nodes, dc.max_prefix,
                                             c.scale, return_lse=True)
    assert torch.equal(m2, mask) and torch.equal(d2, depth) and torch.equal(s2, status)
    assert torch.equal(o2, out) and torch.equal(l2, lse)


def _draft_same_row(c, rng, p):
    pred = np.argmax(c.logits.double().numpy(), axis=1)
    flip = rng.random(c.total_nodes) < p
    return np.where(flip, pred, rng.integers(c.vocab, size=c.total_nodes)).astype(np.int32)


@pytest.mark.parametrize("dtype,V", [(torch.float32, 300), (torch.bfloat16, 1000)])
def test_large_verify_bit_exact(ta, dtype, V):
    trees = _trees(7, [(4096, 1, 16, 4), (1800, 9, 30, None)])
    c = synthetic.make_case("lver", prefix_lens=[0, 0], trees=trees, Hq=1, Hkv=1, D=8,
                            dtype=dtype, seed=7, vocab=V)
    rng = np.random.default_rng(8)
    draft = _draft_same_row(c, rng, 0.97)
    dc = DevCase(c)
    mask, _, _ = gpu_mask(ta, dc)
    got = ta.verify_greedy(dc.logits, torch.from_numpy(draft).cuda(), mask, dc.node_offsets,
                           dc.max_nodes)
    ref = oracle.verify_greedy(c.logits, draft, c.parents, c.node_offsets, dc.max_nodes)
    for n, a, r in zip(("target_argmax", "accept_len", "accept_nodes", "accept_tokens"), got, ref):
        np.testing.assert_array_equal(a.cpu().numpy(), r, err_msg=n)
    print(f"[large verify] accept_len={ref[1].tolist()}", flush=True)


def test_large_verify_next_bit_exact(ta):
    trees = _trees(9, [(3000, 1, 16, 4), (1200, 4, 12, None)])
    V = 500
    c = synthetic.make_case("lvn", prefix_lens=[0, 0], trees=trees, Hq=1, Hkv=1, D=8,
                            dtype=torch.bfloat16, seed=9, vocab=V)
    root = torch.randn((2, V), generator=torch.Generator().manual_seed(10)).to(torch.bfloat16)
    pred = np.argmax(c.logits.double().numpy(), axis=1)
    rpred = np.argmax(root.double().numpy(), axis=1)
    rng = np.random.default_rng(11)
    draft = np.zeros(c.total_nodes, dtype=np.int32)
    for b in range(2):
        lo, hi = int(c.node_offsets[b]), int(c.node_offsets[b + 1])
        for i in range(hi - lo):
            par = int(c.parents[lo + i])
            want = rpred[b] if par < 0 else pred[lo + par]
            draft[lo + i] = want if rng.random() < 0.97 else int(rng.integers(V))
    dc = DevCase(c)
    mask, _, _ = gpu_mask(ta, dc)
    got = ta.verify_greedy_next(dc.logits, root.cuda(), torch.from_numpy(draft).cuda(), mask,
                                dc.node_offsets, dc.max_nodes)
    ref = oracle.verify_greedy_next(c.logits, root, draft, c.parents, c.node_offsets,
                                    dc.max_nodes)
    names = ("target_argmax", "accept_len", "accept_nodes", "accept_tokens", "bonus_token")
    for n, a, r in zip(names, got, ref):
        np.testing.assert_array_equal(a.cpu().numpy(), r, err_msg=n)
    print(f"[large verify next] accept_len={ref[1].tolist()}", flush=True)


def test_large_chain_accepted_whole_and_committed(ta):
    """A 4096-node chain whose every draft token matches: the path is the
    whole chain (64 mask words placed in order), and the commit appends all
    4096 rows in order."""
    n, V = 4096, 64
    c = synthetic.make_case("lchain", prefix_lens=[0], trees=[[-1] + list(range(n - 1))], Hq=1,
                            Hkv=2, D=16, dtype=torch.float32, seed=12, vocab=V)
    draft = np.argmax(c.logits.double().numpy(), axis=1).astype(np.int32)
    dc = DevCase(c)
    mask, _, _ = gpu_mask(ta, dc)
    _, alen, anodes, atok = ta.verify_greedy(dc.logits, torch.from_numpy(draft).cuda(), mask,
                                             dc.node_offsets, n)
    assert alen.cpu().tolist() == [n]
    np.testing.assert_array_equal(anodes.cpu().numpy()[0], np.arange(n))
    np.testing.assert_array_equal(atok.cpu().numpy()[0], draft)
    cap = n + 10
    kc = torch.zeros((cap, 2, 16), device="cuda")
    vc = torch.zeros_like(kc)
    co = torch.tensor([0, cap], dtype=torch.int64, device="cuda")
    cl = torch.tensor([7], dtype=torch.int64, device="cuda")
    st = ta.kv_commit(dc.k_tree, dc.v_tree, dc.node_offsets, alen, anodes, kc, vc, co, cl)
    assert st.cpu().tolist() == [0] and cl.cpu().tolist() == [7 + n]
    assert torch.equal(kc[7:7 + n], dc.k_tree) and torch.equal(vc[7:7 + n], dc.v_tree)
    assert (kc[:7] == 0).all() and (kc[7 + n:] == 0).all()
