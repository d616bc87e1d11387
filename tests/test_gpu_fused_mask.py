"""tree_attn_mask_and_forward (mask built inside the forward kernel for trees
of at most 128 nodes, else the two calls) must give exactly what
tree_attn_build_mask followed by tree_attn_forward gives: masks, depths and
statuses bit for bit, attention bit for bit; and the attention must meet the
oracle on the benchmarked workload."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synthetic
from helpers import DevCase, check_attention, config_case, lib

pytestmark = pytest.mark.gpu


def _both(ta, c):
    dc = DevCase(c)
    mask, depth, status = ta.build_mask(dc.parents, dc.node_offsets, dc.max_nodes)
    out, lse = ta.forward(dc.q, dc.k_tree, dc.v_tree, dc.k_prefix, dc.v_prefix, dc.prefix_offsets,
                          dc.node_offsets, mask, dc.max_nodes, dc.max_prefix, c.scale,
                          return_lse=True)
    fo, fl, fm, fd, fs = ta.mask_and_forward(dc.parents, dc.q, dc.k_tree, dc.v_tree, dc.k_prefix,
                                             dc.v_prefix, dc.prefix_offsets, dc.node_offsets,
                                             dc.max_nodes, dc.max_prefix, c.scale,
                                             return_lse=True)
    torch.cuda.synchronize()
    return (out, lse, mask, depth, status), (fo, fl, fm, fd, fs)


def _same(sep, fused, what):
    names = ("out", "lse", "mask", "depth", "status")
    for n, a, b in zip(names, sep, fused):
        assert torch.equal(a, b), f"{what}: {n} differs"


@pytest.mark.parametrize("name", ["llama3_8b", "batched", "llama3_70b", "forest"])
def test_fused_equals_separate_on_the_workloads(name):
    ta = lib()
    c = config_case(name)
    print(f"[fused mask] config={name}", flush=True)
    sep, fused = _both(ta, c)
    _same(sep, fused, name)
    rm, rd, rs = oracle.build_mask(c.parents, c.node_offsets, max(c.max_nodes, 1))
    np.testing.assert_array_equal(fused[2].cpu().numpy(), rm)
    np.testing.assert_array_equal(fused[3].cpu().numpy(), rd)
    np.testing.assert_array_equal(fused[4].cpu().numpy(), rs)


def test_fused_meets_the_oracle_on_the_8b_layer():
    ta = lib()
    c = config_case("llama3_8b")
    _, fused = _both(ta, c)
    ro, rl = oracle.tree_attention(c.q, c.k_tree, c.v_tree, c.k_prefix, c.v_prefix, c.parents,
                                   c.node_offsets, c.prefix_offsets, c.scale)
    check_attention(fused[0], fused[1], ro, rl, fp32=False, what="fused llama3_8b")


CASES = [
    # (prefix lengths, trees as parent lists or (n, roots, depth, children), Hq, Hkv)
    ([0], [(1, 1, 6, 4)], 8, 2),                      # one root, empty prefix
    ([37, 0, 300], [(17, 1, 6, 4), (1, 1, 6, 4), (70, 1, 6, 4)], 8, 2),   # W = 2 for the batch
    ([1000], [(9, 2, 6, 4)], 16, 2),                  # forest, G = 8
    ([100, 200], [(128, 3, 10, 3), (128, 1, 127, 1)], 4, 1),   # 128 nodes: chain of 128
    ([129, 2049], [(130, 3, 6, 4), (33, 3, 6, 4)], 4, 1),      # 130 nodes: two-call path
    ([64, 64, 64], [[-1, 0, 1], [-1, 2, 0], [0, -1]], 8, 2),   # reranked tree; self-parent: status 2
    ([37, 50, 300], [(17, 1, 6, 4), [], (70, 1, 6, 4)], 8, 2),  # a sequence without nodes
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"L{c[0]}-H{c[2]}x{c[3]}")
def test_fused_equals_separate_small(case):
    ta = lib()
    lens, specs, Hq, Hkv = case
    rng = np.random.default_rng(sum(lens) + Hq)
    trees = [s if isinstance(s, list) else synthetic.random_tree(rng, *s).tolist() for s in specs]
    c = synthetic.make_case("fused", prefix_lens=lens, trees=trees, Hq=Hq, Hkv=Hkv, D=128,
                            seed=sum(lens) + 3)
    sep, fused = _both(ta, c)
    _same(sep, fused, f"lens={lens}")
    rm, rd, rs = oracle.build_mask(c.parents, c.node_offsets, max(c.max_nodes, 1))
    np.testing.assert_array_equal(fused[2].cpu().numpy(), rm)
    np.testing.assert_array_equal(fused[4].cpu().numpy(), rs)
