"""Full-size parity on every node of sequence 0 of the batched, 70B-shaped and
forest workloads, in the launch configuration the benchmark times
(tree_attn_mask_and_forward on the whole batch).

Sequence 0 holds every row tile of its (sequence, KV head) units and every key
split or longest-first piece of them, so each part of the work decomposition
is compared with the fp64 oracle on all of its rows.  The oracle's cost grows
with the prefix length, so the nodes are checked in chunks (one test each)
against one forward call per workload.
"""
import numpy as np
import pytest
import torch

import oracle
from helpers import DevCase, check_attention, config_case, lib

pytestmark = pytest.mark.gpu

# (workload, node chunks of sequence 0)
CHUNKS = [("batched", 1), ("llama3_70b", 4), ("forest", 4)]

_RESULTS = {}


def _gpu_result(name):
    """One tree_attn_mask_and_forward call on the whole workload, kept for the
    chunks of that workload."""
    if name not in _RESULTS:
        _RESULTS.clear()
        ta = lib()
        c = config_case(name)
        dc = DevCase(c)
        out, lse, mask, depth, status = ta.mask_and_forward(
            dc.parents, dc.q, dc.k_tree, dc.v_tree, dc.k_prefix, dc.v_prefix, dc.prefix_offsets,
            dc.node_offsets, dc.max_nodes, dc.max_prefix, c.scale, return_lse=True)
        torch.cuda.synchronize()
        rm, rd, rs = oracle.build_mask(c.parents, c.node_offsets, dc.max_nodes)
        np.testing.assert_array_equal(status.cpu().numpy(), rs)
        np.testing.assert_array_equal(mask.cpu().numpy(), rm)
        np.testing.assert_array_equal(depth.cpu().numpy(), rd)
        _RESULTS[name] = (c, out.cpu(), lse.cpu())
    return _RESULTS[name]


@pytest.mark.parametrize("name,chunk", [(n, k) for n, m in CHUNKS for k in range(m)],
                         ids=lambda v: str(v))
def test_full_size_sequence0_every_node(name, chunk):
    n_chunks = dict(CHUNKS)[name]
    c, out, lse = _gpu_result(name)
    lo, hi = int(c.node_offsets[0]), int(c.node_offsets[1])
    bounds = np.linspace(lo, hi, n_chunks + 1).round().astype(int)
    nodes = list(range(int(bounds[chunk]), int(bounds[chunk + 1])))
    print(f"[full size] {name} sequence 0 nodes {nodes[0]}..{nodes[-1]} "
          f"(L={c.prefix_lens[0]}, {hi - lo} nodes)", flush=True)
    ro, rl = oracle.tree_attention(c.q, c.k_tree, c.v_tree, c.k_prefix, c.v_prefix, c.parents,
                                   c.node_offsets, c.prefix_offsets, c.scale, nodes=nodes)
    check_attention(out[nodes], lse[nodes], ro, rl, fp32=False,
                    what=f"{name} sequence 0 chunk {chunk}")
