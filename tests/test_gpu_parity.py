"""GPU parity: the HIP library, called through its C ABI, against the fp64
oracle on the same seeded inputs.

Masks, depths, statuses, argmax and accepted paths must be bit-exact; bf16
attention must meet max-abs <= 1e-2 and relative RMS <= 5e-3, fp32 attention
max-abs <= 2e-5 and relative RMS <= 1e-5.  Small cases are checked in full
(several 32-key tiles, ragged tails, several row tiles); the full-size
workloads are checked on every node where the oracle is quick (the 8B-shaped
layer) and on sampled nodes elsewhere.
"""
import itertools

import numpy as np
import pytest
import torch

import oracle
import synthetic
from helpers import DevCase, check_attention, config_case, gpu_forward, gpu_mask, lib

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ta():
    return lib()


def _oracle_attn(c, nodes=None):
    return oracle.tree_attention(c.q, c.k_tree, c.v_tree, c.k_prefix, c.v_prefix, c.parents,
                                 c.node_offsets, c.prefix_offsets, c.scale, nodes=nodes)


def _check_mask(ta, c):
    dc = DevCase(c)
    mask, depth, status = gpu_mask(ta, dc)
    rm, rd, rs = oracle.build_mask(c.parents, c.node_offsets, dc.max_nodes)
    np.testing.assert_array_equal(status.cpu().numpy(), rs)
    np.testing.assert_array_equal(mask.cpu().numpy(), rm)
    np.testing.assert_array_equal(depth.cpu().numpy(), rd)
    return dc, mask


# ------------------------------------------------------------------- masks

@pytest.mark.parametrize("name", list(synthetic.CONFIGS))
def test_mask_configs_bit_exact(ta, name):
    print(f"[mask] config={name}", flush=True)
    c = config_case(name)
    _check_mask(ta, c)


def test_mask_every_tiny_tree(ta):
    trees = []
    for n in range(1, 7):
        trees += [list(p) for p in itertools.product(*[range(-1, i) for i in range(n)])]
    c = synthetic.make_case("alltrees", prefix_lens=[0] * len(trees), trees=trees, Hq=1, Hkv=1,
                            D=8, dtype=torch.float32, seed=0)
    _check_mask(ta, c)


def test_mask_max_size_chain_and_forest(ta):
    rng = np.random.default_rng(5)
    trees = [[-1] + list(range(1023)),
             synthetic.random_tree(rng, 1024, 7, None, None).tolist(),
             synthetic.random_tree(rng, 700, 1, 20, 3).tolist(), [-1]]
    c = synthetic.make_case("big", prefix_lens=[0] * 4, trees=trees, Hq=1, Hkv=1, D=8,
                            dtype=torch.float32, seed=1)
    _check_mask(ta, c)


def test_mask_invalid_trees_and_offsets(ta):
    trees = [[-1, 0, 1], [-1, 2, 0], [-1, 0, 3], [0, -1], [-1, -2]]
    c = synthetic.make_case("bad", prefix_lens=[0] * 5, trees=trees, Hq=1, Hkv=1, D=8,
                            dtype=torch.float32, seed=2)
    _check_mask(ta, c)
    dc = DevCase(c)
    # node_offsets that exceed max_nodes: status INVALID_ARG, nothing written
    mask, depth, status = ta.build_mask(dc.parents, dc.node_offsets, 2)
    assert status.cpu().tolist() == [1, 1, 1, 2, 2]


# ------------------------------------------------------------- attention

def test_forward_tiny_fp32(ta):
    c = synthetic.make_config_case("tiny", with_logits=False)
    dc, mask = _check_mask(ta, c)
    out, lse = gpu_forward(ta, dc, mask)
    ro, rl = _oracle_attn(c)
    check_attention(out, lse, ro, rl, fp32=True, what="tiny fp32")


def test_forward_fp32_ragged_gqa(ta):
    rng = np.random.default_rng(3)
    trees = [synthetic.random_tree(rng, n, 1, 5, 3).tolist() for n in (1, 9, 40)]
    c = synthetic.make_case("f32", prefix_lens=[0, 33, 150], trees=trees, Hq=6, Hkv=2, D=96,
                            dtype=torch.float32, seed=3)
    dc, mask = _check_mask(ta, c)
    out, lse = gpu_forward(ta, dc, mask)
    check_attention(out, lse, *_oracle_attn(c), fp32=True, what="f32 ragged")


BF16_SHAPES = [
    # (prefix lengths, node counts, roots, Hq, Hkv)
    ([0], [1], 1, 8, 2),
    ([5], [3], 1, 4, 4),
    ([37, 0, 300], [17, 1, 70], 1, 8, 2),      # ragged tails, L=0, two row tiles
    ([64], [64], 1, 32, 8),                   # exact tile multiples
    ([1000], [9], 2, 16, 2),                  # G = 8, forest of 2
    ([129, 2049], [130, 33], 3, 4, 1),         # G = 4, Hkv = 1, 3 row tiles
]


@pytest.mark.parametrize("shape", BF16_SHAPES, ids=lambda s: f"L{s[0]}-N{s[1]}-G{s[3]//s[4]}")
def test_forward_bf16_small_full_check(ta, shape):
    lens, ns, roots, Hq, Hkv = shape
    rng = np.random.default_rng(sum(lens) + sum(ns))
    trees = [synthetic.random_tree(rng, n, min(roots, n), 6, 4).tolist() for n in ns]
    c = synthetic.make_case("bf16", prefix_lens=lens, trees=trees, Hq=Hq, Hkv=Hkv, D=128,
                            seed=len(lens) * 7 + Hq)
    print(f"[fwd bf16] lens={lens} ns={ns} Hq={Hq} Hkv={Hkv}", flush=True)
    dc, mask = _check_mask(ta, c)
    out, lse = gpu_forward(ta, dc, mask)
    torch.cuda.synchronize()
    check_attention(out, lse, *_oracle_attn(c), fp32=False, what=f"bf16 {lens}/{ns}")


def test_forward_many_sequences_full_check(ta):
    """16 ragged sequences x 8 KV heads: the 256-row, single-key-group
    workgroup shape with several key splits, checked on every node."""
    rng = np.random.default_rng(21)
    lens = [int(x) for x in rng.integers(0, 300, 16)]
    trees = [synthetic.random_tree(rng, 64, 1, 6, 4).tolist() for _ in range(16)]
    c = synthetic.make_case("many", prefix_lens=lens, trees=trees, Hq=32, Hkv=8, D=128, seed=21)
    dc, mask = _check_mask(ta, c)
    out, lse = gpu_forward(ta, dc, mask)
    check_attention(out, lse, *_oracle_attn(c), fp32=False, what="16 ragged sequences")


def test_forward_ragged_pieces_longest_first_full_check(ta):
    """Strongly ragged prefixes (17 to 2100 keys) over 16 sequences x 8 KV heads:
    long sequences are cut into several equal pieces that workgroups take
    longest first, short ones stay whole.  Every node, both forward entry
    points (mask given, mask built in the kernel), against the oracle.
    (Prefixes of only a few keys give outputs near 4 in size, whose bf16
    rounding alone takes 0.008 of the 0.01 max-abs bar; the L = 0 shapes
    above cover them.)"""
    rng = np.random.default_rng(33)
    lens = [2100, 40, 1500, 90, 900, 33, 1200, 64, 2000, 130, 700, 300, 1800, 17, 1100, 400]
    trees = [synthetic.random_tree(rng, 64, 1, 6, 4).tolist() for _ in range(16)]
    c = synthetic.make_case("pieces", prefix_lens=lens, trees=trees, Hq=32, Hkv=8, D=128, seed=33)
    dc, mask = _check_mask(ta, c)
    out, lse = gpu_forward(ta, dc, mask)
    check_attention(out, lse, *_oracle_attn(c), fp32=False, what="ragged pieces")
    fo, fl, fm, fd, fs = ta.mask_and_forward(dc.parents, dc.q, dc.k_tree, dc.v_tree, dc.k_prefix,
                                             dc.v_prefix, dc.prefix_offsets, dc.node_offsets,
                                             dc.max_nodes, dc.max_prefix, c.scale,
                                             return_lse=True)
    assert torch.equal(fo, out) and torch.equal(fl, lse)
    assert torch.equal(fm, mask) and int(fs.abs().sum()) == 0


def test_forward_ragged_pieces_bad_offsets_reported(ta):
    """Longest-first pieces with one sequence whose node count exceeds
    max_nodes: that sequence reports TA_ERR_INVALID_ARG from the kernel and
    every other sequence still meets the oracle."""
    rng = np.random.default_rng(41)
    lens = [1900, 60, 1300, 250, 700, 1600, 90, 1100, 40, 2000, 500, 150, 1200, 75, 800, 330]
    ns = [40] * 16
    ns[5] = 64                                   # over max_nodes below
    trees = [synthetic.random_tree(rng, n, 1, 6, 4).tolist() for n in ns]
    c = synthetic.make_case("badpieces", prefix_lens=lens, trees=trees, Hq=32, Hkv=8, D=128,
                            seed=41)
    dc = DevCase(c)
    max_nodes = 48
    out, lse, _, _, status = ta.mask_and_forward(
        dc.parents, dc.q, dc.k_tree, dc.v_tree, dc.k_prefix, dc.v_prefix, dc.prefix_offsets,
        dc.node_offsets, max_nodes, dc.max_prefix, c.scale, return_lse=True)
    st = status.cpu().numpy()
    assert st[5] == ta.TA_ERR_INVALID_ARG and (np.delete(st, 5) == 0).all(), st
    no = c.node_offsets
    rows = np.r_[np.arange(no[0], no[5]), np.arange(no[6], no[16])]
    ro, rl = _oracle_attn(c, nodes=rows)
    check_attention(out[torch.from_numpy(rows).cuda()], lse[torch.from_numpy(rows).cuda()],
                    ro, rl, fp32=False, what="pieces with a bad sequence")


def test_forward_ragged_pieces_with_empty_sequences(ta):
    """Longest-first pieces with two sequences that have no nodes: both
    report status 0 like the mask builder, and every node meets the oracle."""
    rng = np.random.default_rng(43)
    lens = [1800, 70, 1200, 300, 900, 1500, 60, 1000, 45, 2000, 450, 120, 1300, 80, 700, 350]
    ns = [48] * 16
    ns[3] = ns[11] = 0
    trees = [synthetic.random_tree(rng, n, 1, 6, 4).tolist() if n else [] for n in ns]
    c = synthetic.make_case("emptypieces", prefix_lens=lens, trees=trees, Hq=32, Hkv=8, D=128,
                            seed=43)
    dc = DevCase(c)
    out, lse, mask, _, status = ta.mask_and_forward(
        dc.parents, dc.q, dc.k_tree, dc.v_tree, dc.k_prefix, dc.v_prefix, dc.prefix_offsets,
        dc.node_offsets, dc.max_nodes, dc.max_prefix, c.scale, return_lse=True)
    assert int(status.abs().sum()) == 0, status.cpu().tolist()
    rm, _, _ = oracle.build_mask(c.parents, c.node_offsets, dc.max_nodes)
    np.testing.assert_array_equal(mask.cpu().numpy(), rm)
    check_attention(out, lse, *_oracle_attn(c), fp32=False, what="pieces with empty sequences")


def test_forward_ragged_many_sequences_piece_splits(ta):
    """80 ragged sequences (more than the longest-first order takes): pieces
    of about equal length with the standard item order, every node against
    the oracle, both forward entry points."""
    rng = np.random.default_rng(47)
    lens = [int(x) for x in rng.integers(20, 400, 80)]
    lens[7] = 1500
    trees = [synthetic.random_tree(rng, int(n), 1, 4, 3).tolist() for n in rng.integers(1, 9, 80)]
    c = synthetic.make_case("ragged80", prefix_lens=lens, trees=trees, Hq=4, Hkv=1, D=128, seed=47)
    dc, mask = _check_mask(ta, c)
    out, lse = gpu_forward(ta, dc, mask)
    check_attention(out, lse, *_oracle_attn(c), fp32=False, what="80 ragged sequences")
    fo, fl, _, _, fs = ta.mask_and_forward(dc.parents, dc.q, dc.k_tree, dc.v_tree, dc.k_prefix,
                                           dc.v_prefix, dc.prefix_offsets, dc.node_offsets,
                                           dc.max_nodes, dc.max_prefix, c.scale, return_lse=True)
    assert torch.equal(fo, out) and torch.equal(fl, lse) and int(fs.abs().sum()) == 0


def test_forward_llama3_8b_full_check(ta):
    """The benchmarked workload (one 8B-shaped layer, N=64, L=4096), every
    node and head, in the same launch configuration the benchmark times."""
    c = config_case("llama3_8b")
    dc, mask = _check_mask(ta, c)
    out, lse = gpu_forward(ta, dc, mask)
    check_attention(out, lse, *_oracle_attn(c), fp32=False, what="llama3_8b")


@pytest.mark.parametrize("name,per_seq", [("batched", 2), ("llama3_70b", 3), ("forest", 3)])
def test_forward_full_size_sampled(ta, name, per_seq):
    c = config_case(name)
    print(f"[fwd sampled] config={name}", flush=True)
    dc, mask = _check_mask(ta, c)
    out, lse = gpu_forward(ta, dc, mask)
    torch.cuda.synchronize()
    rng = np.random.default_rng(77)
    nodes = []
    seqs = range(c.B) if c.B <= 4 else sorted(rng.choice(c.B, 4, replace=False))
    for b in seqs:
        lo, hi = int(c.node_offsets[b]), int(c.node_offsets[b + 1])
        nodes += [lo, hi - 1] + sorted(rng.choice(np.arange(lo, hi), per_seq - 2 if per_seq > 2 else 0,
                                                  replace=False).tolist())
    nodes = sorted(set(nodes))
    ro, rl = _oracle_attn(c, nodes=nodes)
    check_attention(out[nodes], lse[nodes], ro, rl, fp32=False, what=f"{name} sampled {nodes}")


def test_forward_hidden_rows_do_not_change_output_bitwise(ta):
    rng = np.random.default_rng(8)
    parents = synthetic.random_tree(rng, 60, 2, 6, 4)
    c = synthetic.make_case("sib", prefix_lens=[200], trees=[parents.tolist()], Hq=8, Hkv=2,
                            D=128, seed=8)
    dc, mask = _check_mask(ta, c)
    out, lse = gpu_forward(ta, dc, mask)
    vis = oracle.ancestor_mask_dense(parents)
    i = 45
    hidden = torch.from_numpy(np.flatnonzero(~vis[i]))
    d2 = DevCase(c)
    d2.k_tree[hidden.cuda()] = (d2.k_tree[hidden.cuda()].float() * -3.0 + 1.0).to(torch.bfloat16)
    d2.v_tree[hidden.cuda()] = (d2.v_tree[hidden.cuda()].float() + 5.0).to(torch.bfloat16)
    out2, lse2 = gpu_forward(ta, d2, mask)
    assert torch.equal(out2[i], out[i]) and torch.equal(lse2[i], lse[i])


def test_forward_empty_prefix_root_is_its_value_row(ta):
    c = synthetic.make_case("root", prefix_lens=[0, 0], trees=[[-1, 0], [-1, -1, 1]], Hq=4,
                            Hkv=2, D=128, seed=9)
    dc, mask = _check_mask(ta, c)
    out, _ = gpu_forward(ta, dc, mask)
    for gi in (0, 2, 3):
        expect = c.v_tree[gi].repeat_interleave(2, dim=0)
        assert torch.equal(out[gi].cpu(), expect), gi


# ------------------------------------------------------------ verification

def _check_verify(ta, c, dc, mask):
    pred, alen, anodes, atok = ta.verify_greedy(dc.logits, dc.draft, mask, dc.node_offsets,
                                                dc.max_nodes)
    rp, rlen, rnodes, rtok = oracle.verify_greedy(c.logits, c.draft, c.parents, c.node_offsets,
                                                  dc.max_nodes)
    np.testing.assert_array_equal(pred.cpu().numpy(), rp)
    np.testing.assert_array_equal(alen.cpu().numpy(), rlen)
    np.testing.assert_array_equal(anodes.cpu().numpy(), rnodes)
    np.testing.assert_array_equal(atok.cpu().numpy(), rtok)
    return rlen


def test_verify_tiny_example(ta):
    c = synthetic.make_config_case("tiny")
    dc, mask = _check_mask(ta, c)
    rlen = _check_verify(ta, c, dc, mask)
    assert rlen.tolist() == [3]


@pytest.mark.parametrize("dtype,V", [(torch.bfloat16, 50000), (torch.float32, 1001),
                                     (torch.bfloat16, 77), (torch.float32, 4096),
                                     (torch.bfloat16, 600001), (torch.float32, 700000)])
def test_verify_random_trees(ta, dtype, V):
    rng = np.random.default_rng(V)
    trees = [synthetic.random_tree(rng, n, r, 8, 3).tolist() for n, r in
             ((1, 1), (30, 1), (200, 4), (64, 1), (5, 5))]
    c = synthetic.make_case("ver", prefix_lens=[0] * 5, trees=trees, Hq=1, Hkv=1, D=8,
                            dtype=dtype, seed=V, vocab=V, p_match=0.9)
    dc, mask = _check_mask(ta, c)
    _check_verify(ta, c, dc, mask)


def test_verify_forced_ties_across_chunks(ta):
    V = 128256
    trees = [[-1, 0, 1, 1, 2, 0]]
    c = synthetic.make_case("ties", prefix_lens=[0], trees=trees, Hq=1, Hkv=1, D=8, seed=4,
                            vocab=V, p_match=1.0)
    lg = c.logits
    lg[0, 100] = lg[0, 90000] = 20.0        # tie in different vocab chunks
    lg[1, :] = 0.0                          # all equal: index 0
    lg[2, :] = -1.0
    lg[2, 70000] = -0.0
    lg[2, 5] = 0.0                          # -0 == +0: index 5
    lg[3, V - 1] = 30.0                     # maximum in the last entry
    lg[4, :] = float("-inf")                # all -inf: index 0
    c.draft = torch.argmax(lg.float(), 1).numpy().astype(np.int32)
    c.draft[5] = (c.draft[5] + 1) % V
    dc, mask = _check_mask(ta, c)
    rlen = _check_verify(ta, c, dc, mask)
    assert rlen.tolist() == [4]


def test_verify_forest_full_size(ta):
    c = synthetic.make_config_case("forest", with_logits=True)
    print(f"[verify] forest logits {tuple(c.logits.shape)}", flush=True)
    dc, mask = _check_mask(ta, c)
    rlen = _check_verify(ta, c, dc, mask)
    print(f"[verify] accept_len={rlen.tolist()}", flush=True)
