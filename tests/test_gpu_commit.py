"""GPU parity of the commit of the accepted path (tree_kv_commit) and of the
forward reading its prefix from cache slots (prefix_lens), through the C ABI,
against the fp64 oracle: the cache rows, lengths and statuses bit for bit; the
attention at the usual bars; and the whole loop — verify, commit, next step —
agreeing with the tree attention it continues."""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from helpers import DevCase, check_attention, lib

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ta():
    return lib()


def _slotted_cache(c, extra, fill_seed, dtype):
    """Copy each sequence's prefix to the start of a slot with `extra[b]` spare
    rows; the spare rows hold large finite values that must never be read."""
    g = torch.Generator().manual_seed(fill_seed)
    L = np.diff(c.prefix_offsets)
    caps = [int(L[b]) + int(extra[b]) for b in range(c.B)]
    offs = np.concatenate([[0], np.cumsum(caps)]).astype(np.int64)
    Hkv, D = c.k_prefix.shape[1], c.k_prefix.shape[2]
    kc = (torch.randn((int(offs[-1]), Hkv, D), generator=g) * 40).to(dtype)
    vc = (torch.randn((int(offs[-1]), Hkv, D), generator=g) * 40 + 60).to(dtype)
    for b in range(c.B):
        p0, n = int(c.prefix_offsets[b]), int(L[b])
        kc[offs[b]:offs[b] + n] = c.k_prefix[p0:p0 + n]
        vc[offs[b]:offs[b] + n] = c.v_prefix[p0:p0 + n]
    return kc, vc, offs, L.astype(np.int64)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_commit_bit_exact_with_bad_cases(ta, dtype):
    rng = np.random.default_rng(4)
    ns = [9, 1, 30, 12, 5]
    trees = [synthetic.random_tree(rng, n, 1, 5, 3).tolist() for n in ns]
    # bf16 rows of 2 KiB take the 16-byte copy; fp32 rows of 228 bytes the 2-byte one
    Hkv, D = (8, 128) if dtype == torch.bfloat16 else (3, 19)
    c = synthetic.make_case("commit", prefix_lens=[4, 0, 17, 3, 8], trees=trees, Hq=Hkv, Hkv=Hkv,
                            D=D, dtype=dtype, seed=4)
    max_nodes = 32
    kc, vc, offs, lens = _slotted_cache(c, [6, 3, 40, 2, 9], 5, dtype)
    acc = np.zeros(c.B, dtype=np.int32)
    nodes = np.full((c.B, max_nodes), -1, dtype=np.int32)
    for b in range(c.B):
        n0, n1 = int(c.node_offsets[b]), int(c.node_offsets[b + 1])
        leaf = int(rng.integers(n1 - n0))
        path = oracle.root_path(c.parents[n0:n1], leaf)
        nodes[b, :len(path)] = path
        acc[b] = len(path)
    acc[1] = 0                                   # nothing accepted
    acc[3] = 3                                   # more rows than the slot's 2 spare ones
    nodes[4, 0] = 77                             # a node id outside the sequence
    acc[4] = max(acc[4], 1)
    ref = oracle.kv_commit(c.k_tree, c.v_tree, c.node_offsets, acc, nodes, kc, vc, offs, lens,
                           max_nodes)
    d = torch.device("cuda")
    kc_d, vc_d = kc.to(d), vc.to(d)
    lens_d = torch.from_numpy(lens).to(d)
    st = ta.kv_commit(c.k_tree.to(d), c.v_tree.to(d), torch.from_numpy(c.node_offsets).to(d),
                      torch.from_numpy(acc).to(d), torch.from_numpy(nodes).to(d), kc_d, vc_d,
                      torch.from_numpy(offs).to(d), lens_d)
    torch.cuda.synchronize()
    assert st.cpu().tolist() == ref[3].tolist() == [0, 0, 0, 1, 1]
    assert lens_d.cpu().tolist() == ref[2].tolist()
    assert torch.equal(kc_d.cpu(), ref[0]) and torch.equal(vc_d.cpu(), ref[1])


@pytest.mark.parametrize("shape", [([300, 0, 77], [20, 3, 64], 8, 2),   # separate merge kernel
                                   ([3000], [64], 32, 8)],              # merge inside the kernel
                         ids=["three-seqs", "one-seq"])
def test_forward_reads_only_the_rows_in_use_of_each_slot(ta, shape):
    lens, ns, Hq, Hkv = shape
    rng = np.random.default_rng(sum(lens))
    trees = [synthetic.random_tree(rng, n, 1, 6, 4).tolist() for n in ns]
    c = synthetic.make_case("slot", prefix_lens=lens, trees=trees, Hq=Hq, Hkv=Hkv, D=128, seed=6)
    kc, vc, offs, L = _slotted_cache(c, [50] * c.B, 7, torch.bfloat16)
    ro, rl = oracle.tree_attention(c.q, c.k_tree, c.v_tree, c.k_prefix, c.v_prefix, c.parents,
                                   c.node_offsets, c.prefix_offsets, c.scale)
    dc = DevCase(c)
    mask, _, _ = ta.build_mask(dc.parents, dc.node_offsets, dc.max_nodes)
    d = torch.device("cuda")
    out, lse = ta.forward(dc.q, dc.k_tree, dc.v_tree, kc.to(d), vc.to(d),
                          torch.from_numpy(offs).to(d), dc.node_offsets, mask, dc.max_nodes,
                          int(L.max()), c.scale, return_lse=True,
                          prefix_lens=torch.from_numpy(L).to(d))
    check_attention(out, lse, ro, rl, fp32=False, what=f"slotted prefix {lens}")
    out2 = ta.mask_and_forward(dc.parents, dc.q, dc.k_tree, dc.v_tree, kc.to(d), vc.to(d),
                               torch.from_numpy(offs).to(d), dc.node_offsets, dc.max_nodes,
                               int(L.max()), c.scale, prefix_lens=torch.from_numpy(L).to(d))[0]
    assert torch.equal(out2, out)


def test_verify_commit_next_step_continues_the_tree(ta):
    """Verify a tree, commit the accepted path minus its last node, then run
    that last node alone as the next step over the updated cache: its output
    is the tree attention of that node (oracle), within the bf16 bar."""
    rng = np.random.default_rng(12)
    trees = [synthetic.random_tree(rng, 64, 1, 6, 4).tolist() for _ in range(2)]
    c = synthetic.make_case("loop", prefix_lens=[500, 90], trees=trees, Hq=32, Hkv=8, D=128,
                            seed=12, vocab=3000, p_match=1.0)
    dc = DevCase(c)
    mask, _, _ = ta.build_mask(dc.parents, dc.node_offsets, dc.max_nodes)
    _, alen, anodes, _ = ta.verify_greedy(dc.logits, dc.draft, mask, dc.node_offsets,
                                          dc.max_nodes)
    alen_h = alen.cpu().numpy()
    assert (alen_h >= 2).all(), alen_h           # the seeds give a real path to continue
    kc, vc, offs, L = _slotted_cache(c, [20, 20], 13, torch.bfloat16)
    d = torch.device("cuda")
    kc_d, vc_d = kc.to(d), vc.to(d)
    lens_d = torch.from_numpy(L).to(d)
    offs_d = torch.from_numpy(offs).to(d)
    st = ta.kv_commit(dc.k_tree, dc.v_tree, dc.node_offsets, (alen - 1).contiguous(), anodes,
                      kc_d, vc_d, offs_d, lens_d)
    assert st.cpu().tolist() == [0, 0]
    assert lens_d.cpu().tolist() == (L + alen_h - 1).tolist()
    leaf = [int(c.node_offsets[b]) + int(anodes[b, alen_h[b] - 1]) for b in range(2)]
    one = torch.tensor([-1, -1], dtype=torch.int32, device=d)
    offs1 = torch.tensor([0, 1, 2], dtype=torch.int32, device=d)
    m1, _, _ = ta.build_mask(one, offs1, 1)
    out, lse = ta.forward(dc.q[leaf].contiguous(), dc.k_tree[leaf].contiguous(),
                          dc.v_tree[leaf].contiguous(), kc_d, vc_d, offs_d, offs1, m1, 1,
                          int(lens_d.max()), c.scale, return_lse=True, prefix_lens=lens_d)
    ro, rl = oracle.tree_attention(c.q, c.k_tree, c.v_tree, c.k_prefix, c.v_prefix, c.parents,
                                   c.node_offsets, c.prefix_offsets, c.scale, nodes=leaf)
    check_attention(out, lse, ro, rl, fp32=False, what="next step after commit")


def test_commit_replayed_from_a_graph_appends_each_time(ta):
    """The commit keeps its lengths on the device, so a captured graph can
    replay it: each replay appends the accepted path once more, after the
    rows the previous replays appended."""
    rng = np.random.default_rng(40)
    trees = [synthetic.random_tree(rng, 20, 1, 5, 3).tolist() for _ in range(2)]
    c = synthetic.make_case("gcommit", prefix_lens=[10, 3], trees=trees, Hq=8, Hkv=8, D=128,
                            seed=40)
    reps = 4
    kc, vc, offs, L = _slotted_cache(c, [reps * 8, reps * 8], 41, torch.bfloat16)
    acc = np.zeros(2, dtype=np.int32)
    nodes = np.full((2, 20), -1, dtype=np.int32)
    for b in range(2):
        n0, n1 = int(c.node_offsets[b]), int(c.node_offsets[b + 1])
        path = oracle.root_path(c.parents[n0:n1], int(rng.integers(n1 - n0)))
        nodes[b, :len(path)] = path
        acc[b] = len(path)
    d = torch.device("cuda")
    args = [c.k_tree.to(d), c.v_tree.to(d), torch.from_numpy(c.node_offsets).to(d),
            torch.from_numpy(acc).to(d), torch.from_numpy(nodes).to(d)]
    kc_d, vc_d = kc.to(d), vc.to(d)
    offs_d, lens_d = torch.from_numpy(offs).to(d), torch.from_numpy(L).to(d)
    status = torch.empty(2, dtype=torch.int32, device=d)
    ta.kv_commit(*args, kc_d, vc_d, offs_d, lens_d, status=status)   # eager once
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ta.kv_commit(*args, kc_d, vc_d, offs_d, lens_d, status=status)
    ref_k, ref_v, ref_len = kc, vc, L
    for _ in range(reps):   # the eager call, then reps - 1 replays
        ref_k, ref_v, ref_len, st = oracle.kv_commit(c.k_tree, c.v_tree, c.node_offsets, acc,
                                                     nodes, ref_k, ref_v, offs, ref_len, 20)
    for _ in range(reps - 1):
        g.replay()
        torch.cuda.synchronize()
    assert status.cpu().tolist() == [0, 0]
    assert lens_d.cpu().tolist() == ref_len.tolist() == (L + reps * acc).tolist()
    assert torch.equal(kc_d.cpu(), ref_k) and torch.equal(vc_d.cpu(), ref_v)


def test_fp32_forward_reads_only_the_rows_in_use_of_each_slot(ta):
    rng = np.random.default_rng(50)
    trees = [synthetic.random_tree(rng, n, 1, 5, 3).tolist() for n in (6, 19)]
    c = synthetic.make_case("slot32", prefix_lens=[40, 0], trees=trees, Hq=6, Hkv=2, D=72,
                            dtype=torch.float32, seed=50)
    kc, vc, offs, L = _slotted_cache(c, [9, 4], 51, torch.float32)
    ro, rl = oracle.tree_attention(c.q, c.k_tree, c.v_tree, c.k_prefix, c.v_prefix, c.parents,
                                   c.node_offsets, c.prefix_offsets, c.scale)
    dc = DevCase(c)
    mask, _, _ = ta.build_mask(dc.parents, dc.node_offsets, dc.max_nodes)
    d = torch.device("cuda")
    out, lse = ta.forward(dc.q, dc.k_tree, dc.v_tree, kc.to(d), vc.to(d),
                          torch.from_numpy(offs).to(d), dc.node_offsets, mask, dc.max_nodes,
                          int(L.max()), c.scale, return_lse=True,
                          prefix_lens=torch.from_numpy(L).to(d))
    check_attention(out, lse, ro, rl, fp32=True, what="fp32 slotted prefix")


def test_commit_longest_path_at_the_node_limit(ta):
    """A 1024-node chain accepted whole: every source index slot is used."""
    n = 1024
    c = synthetic.make_case("chain", prefix_lens=[5], trees=[[-1] + list(range(n - 1))], Hq=2,
                            Hkv=2, D=16, dtype=torch.float32, seed=60)
    kc, vc, offs, L = _slotted_cache(c, [n + 3], 61, torch.float32)
    acc = np.array([n], dtype=np.int32)
    nodes = np.arange(n, dtype=np.int32)[None, :]
    ref = oracle.kv_commit(c.k_tree, c.v_tree, c.node_offsets, acc, nodes, kc, vc, offs, L, n)
    d = torch.device("cuda")
    kc_d, vc_d, lens_d = kc.to(d), vc.to(d), torch.from_numpy(L).to(d)
    st = ta.kv_commit(c.k_tree.to(d), c.v_tree.to(d), torch.from_numpy(c.node_offsets).to(d),
                      torch.from_numpy(acc).to(d), torch.from_numpy(nodes).to(d), kc_d, vc_d,
                      torch.from_numpy(offs).to(d), lens_d)
    assert st.cpu().tolist() == [0] and lens_d.cpu().tolist() == ref[2].tolist() == [5 + n]
    assert torch.equal(kc_d.cpu(), ref[0]) and torch.equal(vc_d.cpu(), ref[1])
