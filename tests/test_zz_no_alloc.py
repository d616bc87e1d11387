"""tree_attn_forward_noalloc (no workspace: the library's static scratch)
against tree_attn_forward on the same inputs, through the C ABI, on two calls
in a row, the second with a smaller input: the same kernels run, so the
outputs must agree bit for bit (which meets the parity bar), and the merge
status stays 0."""
import numpy as np
import pytest
import torch

import synthetic
from helpers import DevCase, lib

pytestmark = pytest.mark.gpu


def _both(ta, c):
    dc = DevCase(c)
    mask, _, _ = ta.build_mask(dc.parents, dc.node_offsets, dc.max_nodes)
    ref, ref_lse = ta.forward(dc.q, dc.k_tree, dc.v_tree, dc.k_prefix, dc.v_prefix,
                              dc.prefix_offsets, dc.node_offsets, mask, dc.max_nodes,
                              dc.max_prefix, c.scale, return_lse=True)
    out = torch.full_like(dc.q, float("nan"))
    lse = torch.full((c.total_nodes, c.Hq), float("nan"), device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    ta.forward_noalloc(dc.q, dc.k_tree, dc.v_tree, dc.k_prefix, dc.v_prefix, dc.prefix_offsets,
                       dc.node_offsets, mask, dc.max_nodes, dc.max_prefix, c.scale, out=out,
                       lse=lse, merge_status=status)
    torch.cuda.synchronize()
    return ref, ref_lse, out, lse, int(status.item())


def test_noalloc_matches_forward_on_two_calls():
    ta = lib()
    big = synthetic.make_config_case("llama3_8b", with_logits=False)
    n_big = ta.forward_workspace_size(torch.bfloat16, big.B, big.total_nodes, big.max_nodes,
                                      big.Hq, big.Hkv, big.D, big.total_prefix, big.max_prefix)
    assert 0 < n_big <= ta.TA_NOALLOC_MAX_WORKSPACE      # split partials in the scratch
    # The same head shape over a shorter prefix and a smaller tree: fewer key
    # splits, still merged inside the forward kernel, in less of the scratch.
    rng = np.random.default_rng(5)
    small = synthetic.make_case("small", prefix_lens=[1024],
                                trees=[synthetic.random_tree(rng, 32, 1, 6, 4).tolist()],
                                Hq=32, Hkv=8, D=128, seed=5)
    n_small = ta.forward_workspace_size(torch.bfloat16, small.B, small.total_nodes,
                                        small.max_nodes, small.Hq, small.Hkv, small.D,
                                        small.total_prefix, small.max_prefix)
    assert 0 < n_small < n_big
    for what, c in (("8B-shaped layer", big), ("smaller batch", small)):
        ref, ref_lse, out, lse, st = _both(ta, c)
        print(f"[noalloc] {what}: status {st}", flush=True)
        assert st == 0, what
        assert torch.equal(out, ref), what
        assert torch.equal(lse, ref_lse), what
