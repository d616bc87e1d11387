"""The split merge that runs inside the forward kernel (few sequence x KV
head x row-tile groups, as in the 8B-shaped layer) keeps per-group counters at
the start of the caller's workspace and returns them to zero: one workspace
serves many calls, also of different shapes, and a workspace whose counters
were not zero gives NaN after a bounded wait, then is right again."""
from __future__ import annotations

import time

import numpy as np
import pytest
import torch

import oracle
import synthetic
from helpers import DevCase, check_attention, config_case, lib

pytestmark = pytest.mark.gpu


def _forward(ta, dc, mask, ws):
    c = dc.case
    return ta.forward(dc.q, dc.k_tree, dc.v_tree, dc.k_prefix, dc.v_prefix, dc.prefix_offsets,
                      dc.node_offsets, mask, dc.max_nodes, dc.max_prefix, c.scale,
                      return_lse=True, workspace=ws)


def _setup(ta, c):
    dc = DevCase(c)
    mask, _, _ = ta.build_mask(dc.parents, dc.node_offsets, dc.max_nodes)
    n = ta.forward_workspace_size(torch.bfloat16, c.B, c.total_nodes, dc.max_nodes, c.Hq, c.Hkv,
                                  c.D, c.total_prefix, dc.max_prefix)
    return dc, mask, n


def test_in_kernel_merge_reuses_one_workspace():
    ta = lib()
    ca = config_case("llama3_8b")
    cb = synthetic.make_config_case("llama3_8b", with_logits=False, seed=99)
    da, ma, n = _setup(ta, ca)
    db, mb, _ = _setup(ta, cb)
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    oa, la = _forward(ta, da, ma, ws)
    oa, la = oa.clone(), la.clone()
    ob, lb = _forward(ta, db, mb, ws)
    ob, lb = ob.clone(), lb.clone()
    for rep in range(3):
        o, l = _forward(ta, da, ma, ws)
        assert torch.equal(o, oa) and torch.equal(l, la), f"call {rep}: a differs"
        o, l = _forward(ta, db, mb, ws)
        assert torch.equal(o, ob) and torch.equal(l, lb), f"call {rep}: b differs"
    rng = np.random.default_rng(3)
    nodes = sorted(rng.choice(cb.total_nodes, 12, replace=False).tolist())
    ro, rl = oracle.tree_attention(cb.q, cb.k_tree, cb.v_tree, cb.k_prefix, cb.v_prefix,
                                   cb.parents, cb.node_offsets, cb.prefix_offsets, cb.scale,
                                   nodes=nodes)
    check_attention(ob[nodes], lb[nodes], ro, rl, fp32=False, what="second input, same workspace")


def test_in_kernel_merge_with_nonzero_workspace_fails_loudly_then_recovers():
    """Counters left non-zero (a workspace that was never zero-filled) must not
    hang the call: after the bounded wait the outputs that the in-kernel merge
    writes are NaN, never a plausible wrong value, the merge status word says
    so, and the counters are reset so the next call on that workspace is right
    again (status 0)."""
    ta = lib()
    c = config_case("llama3_8b")
    dc, mask, n = _setup(ta, c)
    clean = torch.zeros(n, dtype=torch.uint8, device="cuda")
    ref_o, ref_l = _forward(ta, dc, mask, clean)
    ref_o, ref_l = ref_o.clone(), ref_l.clone()
    assert ta.merge_status(clean) == 0
    dirty = torch.full((n,), 0x5A, dtype=torch.uint8, device="cuda")
    dirty[:4].zero_()                       # the status word alone starts clean
    o, l = _forward(ta, dc, mask, dirty)
    torch.cuda.synchronize()
    st = ta.merge_status(dirty, clear=True)
    print(f"merge status after the dirty call: {st}", flush=True)
    assert st & (ta.TA_MERGE_TIMEOUT | ta.TA_MERGE_STALE), st
    assert not st & ta.TA_MERGE_PLACEMENT, st
    bad = ~torch.isfinite(o.float()).all(dim=-1)
    assert bool(bad.any()), "a failed merge must not look like a result"
    assert torch.equal(o[~bad], ref_o[~bad]), "finite outputs must be the right ones"
    o, l = _forward(ta, dc, mask, dirty)
    assert torch.equal(o, ref_o) and torch.equal(l, ref_l)
    assert ta.merge_status(dirty) == 0


def test_in_kernel_merge_status_stays_zero_over_many_calls():
    """Clean calls, also alternating two inputs on one workspace, never set a
    status bit (the epoch tags of consecutive calls differ, and each call sees
    only its own arrivals)."""
    ta = lib()
    ca = config_case("llama3_8b")
    cb = synthetic.make_config_case("llama3_8b", with_logits=False, seed=7)
    da, ma, n = _setup(ta, ca)
    db, mb, _ = _setup(ta, cb)
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    oa, _ = _forward(ta, da, ma, ws)
    oa = oa.clone()
    ob, _ = _forward(ta, db, mb, ws)
    ob = ob.clone()
    for rep in range(20):
        o, _ = _forward(ta, da if rep % 2 else db, ma if rep % 2 else mb, ws)
        assert torch.equal(o, oa if rep % 2 else ob), rep
    assert ta.merge_status(ws) == 0


def test_workspace_shared_across_shapes():
    """A call of another shape (its splits merged by the separate kernel, its
    partials larger) on the same buffer leaves the counters at zero, so the
    in-kernel merge that follows needs no wait and gives the same bits."""
    ta = lib()
    ca = config_case("llama3_8b")
    da, ma, na = _setup(ta, ca)
    cb = config_case("batched")
    db, mb, nb = _setup(ta, cb)
    ws = torch.zeros(max(na, nb), dtype=torch.uint8, device="cuda")
    oa, la = _forward(ta, da, ma, ws)
    oa, la = oa.clone(), la.clone()
    ob, lb = _forward(ta, db, mb, ws)
    ob, lb = ob.clone(), lb.clone()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    o, l = _forward(ta, da, ma, ws)
    torch.cuda.synchronize()
    assert time.perf_counter() - t0 < 0.1, "the in-kernel merge waited out its bound"
    assert torch.equal(o, oa) and torch.equal(l, la)
    o, l = _forward(ta, db, mb, ws)
    assert torch.equal(o, ob) and torch.equal(l, lb)
    assert torch.isfinite(oa.float()).all() and torch.isfinite(ob.float()).all()
