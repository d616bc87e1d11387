"""Prefix ranges that do not start at row 0 of the buffer, and a max_prefix
above every sequence's length, against the oracle: host sizes that look like
a uniform, packed batch (total = B * max) while the offsets say otherwise.
The forward must follow the offsets, never the host sizes; the plain uniform
batch is checked alongside."""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from helpers import DevCase, check_attention, gpu_mask, lib

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ta():
    return lib()


def _run(ta, c, prefix_offsets, max_prefix, entry):
    dc = DevCase(c)
    dc.prefix_offsets = torch.tensor(prefix_offsets, dtype=torch.int64, device="cuda")
    mask, _, _ = gpu_mask(ta, dc)
    if entry == "forward":
        out, lse = ta.forward(dc.q, dc.k_tree, dc.v_tree, dc.k_prefix, dc.v_prefix,
                              dc.prefix_offsets, dc.node_offsets, mask, dc.max_nodes, max_prefix,
                              c.scale, return_lse=True)
    else:
        out, lse, _, _, st = ta.mask_and_forward(
            dc.parents, dc.q, dc.k_tree, dc.v_tree, dc.k_prefix, dc.v_prefix, dc.prefix_offsets,
            dc.node_offsets, dc.max_nodes, max_prefix, c.scale, return_lse=True)
        assert int(st.abs().sum()) == 0
    ro, rl = oracle.tree_attention(c.q, c.k_tree, c.v_tree, c.k_prefix, c.v_prefix, c.parents,
                                   c.node_offsets, np.asarray(prefix_offsets), c.scale)
    return out, lse, ro, rl


@pytest.mark.parametrize("entry", ["forward", "mask_and_forward"])
def test_offset_prefix_in_kernel_merge_shape(ta, entry):
    """One sequence of the 8B-shaped layer (in-kernel merge) whose prefix is
    rows 8 .. 4103 of a 4104-row buffer, with max_prefix = 4104."""
    rng = np.random.default_rng(81)
    c = synthetic.make_case("offs1", prefix_lens=[4104],
                            trees=[synthetic.random_tree(rng, 64, 1, 6, 4).tolist()],
                            Hq=32, Hkv=8, D=128, seed=81)
    out, lse, ro, rl = _run(ta, c, [8, 4104], 4104, entry)
    check_attention(out, lse, ro, rl, fp32=False, what=f"prefix past row 0, in-kernel merge, {entry}")


def test_offset_prefix_separate_merge(ta):
    """Four sequences in a 4 x 300-row buffer whose first range is rows
    10 .. 299 (290 rows), the others 300 rows each."""
    rng = np.random.default_rng(82)
    c = synthetic.make_case("offs2", prefix_lens=[300] * 4,
                            trees=[synthetic.random_tree(rng, 40, 1, 6, 4).tolist()
                                   for _ in range(4)],
                            Hq=16, Hkv=2, D=128, seed=82)
    out, lse, ro, rl = _run(ta, c, [10, 300, 600, 900, 1200], 300, "forward")
    check_attention(out, lse, ro, rl, fp32=False, what="prefix past row 0, sequence 0")


def test_uniform_batch_packed_offsets(ta):
    """The plain uniform batch: every node against the oracle."""
    rng = np.random.default_rng(83)
    c = synthetic.make_case("offs3", prefix_lens=[700] * 3,
                            trees=[synthetic.random_tree(rng, 48, 1, 6, 4).tolist()
                                   for _ in range(3)], Hq=32, Hkv=8, D=128, seed=83)
    out, lse, ro, rl = _run(ta, c, [0, 700, 1400, 2100], 700, "mask_and_forward")
    check_attention(out, lse, ro, rl, fp32=False, what="uniform batch")
