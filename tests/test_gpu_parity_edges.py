"""GPU parity on the method's edge cases, against the fp64 oracle.

* Tree-only attention (empty verified prefix) of every node, roots and
  non-roots, at depths 1 to 8, in fp32 and in bf16.  A node then sees only
  itself and its ancestors ("Tree Attention", zhongzhoutan-coder.github.io,
  How It Works: every node sees the prefix, itself and its ancestors; an empty
  prefix leaves the last two).
* Prefixes of 1 to 16 keys in shapes whose tile ranges are cut into several
  key splits, so partial softmaxes over a handful of keys are merged.

Outputs here reach magnitude 2 to 4 (a node averages a few value rows drawn
from N(0, 1)), where bf16 rounding alone is 0.0078; the bf16 check allows the
rounding of the oracle's value to bf16 on top of the 1e-2 bar (see
helpers.check_attention).
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


def _chains_and_trees(seed):
    """Chains of depth 1..8 (2..9 nodes), a single root, and random trees and
    forests whose depth cap is 8."""
    rng = np.random.default_rng(seed)
    trees = [list(range(-1, d)) for d in range(1, 9)]
    trees.append([-1])
    trees.append(synthetic.random_tree(rng, 40, 1, 8, 3).tolist())
    trees.append(synthetic.random_tree(rng, 64, 3, 8, 2).tolist())
    trees.append(synthetic.random_tree(rng, 100, 2, 8, None).tolist())
    return trees


def _run(ta, c, entry):
    dc = DevCase(c)
    mask, depth, status = gpu_mask(ta, dc)
    rm, rd, rs = oracle.build_mask(c.parents, c.node_offsets, dc.max_nodes)
    np.testing.assert_array_equal(mask.cpu().numpy(), rm)
    np.testing.assert_array_equal(depth.cpu().numpy(), rd)
    if entry == "forward":
        out, lse = gpu_forward(ta, dc, mask)
    else:
        out, lse, fm, fd, fs = ta.mask_and_forward(
            dc.parents, dc.q, dc.k_tree, dc.v_tree, dc.k_prefix, dc.v_prefix, dc.prefix_offsets,
            dc.node_offsets, dc.max_nodes, dc.max_prefix, c.scale, return_lse=True)
        np.testing.assert_array_equal(fm.cpu().numpy(), rm)
        np.testing.assert_array_equal(fs.cpu().numpy(), rs)
    torch.cuda.synchronize()
    return out, lse


def _oracle(c):
    return oracle.tree_attention(c.q, c.k_tree, c.v_tree, c.k_prefix, c.v_prefix, c.parents,
                                 c.node_offsets, c.prefix_offsets, c.scale)


@pytest.mark.parametrize("Hq,Hkv,D", [(4, 2, 64), (6, 3, 128), (1, 1, 32)])
def test_empty_prefix_every_node_fp32(ta, Hq, Hkv, D):
    trees = _chains_and_trees(11 + D)
    c = synthetic.make_case("l0f32", prefix_lens=[0] * len(trees), trees=trees, Hq=Hq, Hkv=Hkv,
                            D=D, dtype=torch.float32, seed=100 + D)
    print(f"[L=0 fp32] Hq={Hq} Hkv={Hkv} D={D} nodes={c.total_nodes}", flush=True)
    out, lse = _run(ta, c, "forward")
    ro, rl = _oracle(c)
    check_attention(out, lse, ro, rl, fp32=True, what=f"L=0 fp32 Hq={Hq} Hkv={Hkv} D={D}")


@pytest.mark.parametrize("entry", ["forward", "mask_and_forward"])
@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (32, 8), (16, 2)])
def test_empty_prefix_every_node_bf16(ta, Hq, Hkv, entry):
    trees = _chains_and_trees(17 + Hq)
    c = synthetic.make_case("l0bf16", prefix_lens=[0] * len(trees), trees=trees, Hq=Hq,
                            Hkv=Hkv, D=128, seed=200 + Hq)
    print(f"[L=0 bf16] Hq={Hq} Hkv={Hkv} entry={entry} nodes={c.total_nodes}", flush=True)
    out, lse = _run(ta, c, entry)
    ro, rl = _oracle(c)
    check_attention(out, lse, ro, rl, fp32=False, what=f"L=0 bf16 Hq={Hq} Hkv={Hkv} {entry}")
    # Depth-0 nodes see only themselves: their output is their value row, bit for bit.
    roots = np.flatnonzero(np.asarray(c.parents) == -1)
    G = Hq // Hkv
    got = out[torch.from_numpy(roots).cuda()].cpu()
    want = c.v_tree[roots].repeat_interleave(G, dim=1)
    assert torch.equal(got, want)


@pytest.mark.parametrize("lens", [[8, 8, 8, 8], [1, 5, 16, 9], [3, 0, 12, 1]])
def test_few_key_prefixes_with_key_splits(ta, lens):
    """512-node forests over 1-16-key prefixes (Hq=4, Hkv=1): 16 row tiles per
    sequence, and the later row tiles cut their 17 tiles into 4 key splits, so
    partials of a few keys each are merged by log-sum-exp."""
    rng = np.random.default_rng(sum(lens) + 5)
    trees = [synthetic.random_tree(rng, 512, 8, 16, None).tolist() for _ in lens]
    c = synthetic.make_case("fewkeys", prefix_lens=lens, trees=trees, Hq=4, Hkv=1, D=128,
                            seed=300 + sum(lens))
    n = ta.forward_workspace_size(torch.bfloat16, c.B, c.total_nodes, c.max_nodes, c.Hq, c.Hkv,
                                  c.D, c.total_prefix, c.max_prefix)
    assert n > 0, "this shape is meant to split the key range"
    print(f"[few keys] lens={lens} workspace={n}", flush=True)
    out, lse = _run(ta, c, "forward")
    ro, rl = _oracle(c)
    check_attention(out, lse, ro, rl, fp32=False, what=f"few-key prefixes {lens}")


def test_few_key_prefixes_many_nodes_fused_mask(ta):
    """128-node trees (the largest the forward builds its own mask for) over
    1-16-key prefixes next to one long prefix, through both entry points."""
    rng = np.random.default_rng(61)
    lens = [2, 16, 7, 1, 4000, 11, 0, 5]
    trees = [synthetic.random_tree(rng, 128, 1, 8, 6).tolist() for _ in lens]
    c = synthetic.make_case("fewkeys128", prefix_lens=lens, trees=trees, Hq=8, Hkv=1, D=128,
                            seed=61)
    ro, rl = _oracle(c)
    for entry in ("forward", "mask_and_forward"):
        out, lse = _run(ta, c, entry)
        check_attention(out, lse, ro, rl, fp32=False, what=f"few keys, 128 nodes, {entry}")


@pytest.mark.parametrize("L", [0, 5, 30])
def test_few_keys_split_in_kernel_merge(ta, L):
    """One sequence, 8 KV heads of one query head each, 256 nodes: two row
    tiles per head, the second cut into 2 key splits merged inside the forward
    kernel (16 groups), over an empty or few-key prefix, so its splits hold a
    handful of keys and store wide partials.  The merge status stays 0."""
    rng = np.random.default_rng(71 + L)
    trees = [synthetic.random_tree(rng, 256, 2, 12, 3).tolist()]
    c = synthetic.make_case("fewkeys_ik", prefix_lens=[L], trees=trees, Hq=8, Hkv=8, D=128,
                            seed=71 + L)
    dc = DevCase(c)
    mask, _, _ = gpu_mask(ta, dc)
    n = ta.forward_workspace_size(torch.bfloat16, c.B, c.total_nodes, c.max_nodes, c.Hq, c.Hkv,
                                  c.D, c.total_prefix, c.max_prefix)
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    out, lse = gpu_forward(ta, dc, mask, workspace=ws)
    assert ta.merge_status(ws) == 0
    ro, rl = _oracle(c)
    check_attention(out, lse, ro, rl, fp32=False, what=f"few keys, in-kernel merge, L={L}")
