"""Edge cases of the greedy verifier (tree_verify_greedy and
tree_verify_greedy_next) against the fp64 oracle, bit for bit: sequences
without nodes (at the start, between, at the end; more sequences than rows),
1800 sequences, node offsets out of order (each sequence still takes its own
range, a negative length accepts nothing), and one workspace reused over many
calls of four shapes."""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from helpers import DevCase, lib

pytestmark = pytest.mark.gpu

NAMES = ("target_argmax", "accept_len", "accept_nodes", "accept_tokens", "bonus_token")


@pytest.fixture(scope="module")
def ta():
    return lib()


def _case(trees, V, dtype, seed, p=0.85):
    return synthetic.make_case("vfused", prefix_lens=[0] * len(trees), trees=trees, Hq=1, Hkv=1,
                               D=8, dtype=dtype, seed=seed, vocab=V, p_match=p)


def _trees(rng, sizes):
    return [synthetic.random_tree(rng, n, 1, 8, 3).tolist() if n else [] for n in sizes]


def _same(got, ref, what):
    for n, a, r in zip(NAMES, got, ref):
        np.testing.assert_array_equal(a.cpu().numpy(), r, err_msg=f"{what}: {n}")


def _verify(ta, c, dc, mask, ws=None):
    got = ta.verify_greedy(dc.logits, dc.draft, mask, dc.node_offsets, dc.max_nodes, workspace=ws)
    ref = oracle.verify_greedy(c.logits, c.draft, c.parents, c.node_offsets, dc.max_nodes)
    return got, ref


def _root_logits(c, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn((c.B, c.vocab), generator=g).to(c.logits.dtype)


def _verify_next(ta, c, dc, mask, root, ws=None):
    got = ta.verify_greedy_next(dc.logits, root.cuda(), dc.draft, mask, dc.node_offsets,
                                dc.max_nodes, workspace=ws)
    ref = oracle.verify_greedy_next(c.logits, root, c.draft, c.parents, c.node_offsets,
                                    dc.max_nodes)
    return got, ref


@pytest.mark.parametrize("dtype,V", [(torch.bfloat16, 50000), (torch.float32, 4096),
                                     (torch.bfloat16, 128256)])
def test_sequences_without_nodes(ta, dtype, V):
    """Empty sequences at the start, between and at the end (7 sequences, 95
    rows: one launch); each accepts nothing, the others match the oracle."""
    rng = np.random.default_rng(V)
    c = _case(_trees(rng, [0, 30, 0, 0, 64, 1, 0]), V, dtype, seed=V)
    dc = DevCase(c)
    mask, _, _ = ta.build_mask(dc.parents, dc.node_offsets, dc.max_nodes)
    print(f"[verify, empty sequences] V={V} {dtype}", flush=True)
    got, ref = _verify(ta, c, dc, mask)
    _same(got, ref, "verify")
    assert [int(x) for x in got[1].cpu()[[0, 2, 3, 6]]] == [0, 0, 0, 0]
    root = _root_logits(c, V + 3)
    got, ref = _verify_next(ta, c, dc, mask, root)
    _same(got, ref, "verify_next")


def test_more_sequences_than_rows(ta):
    """Ten sequences over three rows, nine of them without nodes."""
    c = _case([[]] * 9 + [[-1, 0, 1]], 30000, torch.bfloat16, seed=5, p=1.0)
    dc = DevCase(c)
    mask, _, _ = ta.build_mask(dc.parents, dc.node_offsets, dc.max_nodes)
    got, ref = _verify(ta, c, dc, mask)
    _same(got, ref, "verify")
    assert int(got[1].cpu()[9]) == 3
    got, ref = _verify_next(ta, c, dc, mask, _root_logits(c, 6))
    _same(got, ref, "verify_next")


def test_many_sequences(ta):
    """1800 one- and two-node sequences."""
    rng = np.random.default_rng(41)
    sizes = [1 + int(x) for x in rng.integers(0, 2, size=1800)]
    c = _case(_trees(rng, sizes), 1000, torch.float32, seed=41, p=0.7)
    dc = DevCase(c)
    mask, _, _ = ta.build_mask(dc.parents, dc.node_offsets, dc.max_nodes)
    got, ref = _verify(ta, c, dc, mask)
    _same(got, ref, "verify, 1800 sequences")
    got, ref = _verify_next(ta, c, dc, mask, _root_logits(c, 42))
    _same(got, ref, "verify_next, 1800 sequences")


def test_offsets_out_of_order(ta):
    """Trees of 40, 30 and 50 nodes verified under offsets [70, 120, 0, 40]:
    sequence 0 is the third tree, sequence 1 has a negative length (nothing
    accepted), sequence 2 is the first tree; the middle tree's rows belong to
    no sequence, and their target argmax is not written."""
    rng = np.random.default_rng(9)
    V = 50000
    c = _case(_trees(rng, [40, 30, 50]), V, torch.bfloat16, seed=9)
    dc = DevCase(c)
    mask, _, _ = ta.build_mask(dc.parents, dc.node_offsets, dc.max_nodes)
    ref = oracle.verify_greedy(c.logits, c.draft, c.parents, c.node_offsets, dc.max_nodes)
    bad = torch.tensor([70, 120, 0, 40], dtype=torch.int32, device="cuda")
    for rep in range(3):
        pred, alen, anodes, atok = ta.verify_greedy(dc.logits, dc.draft, mask, bad, dc.max_nodes)
        pred, alen = pred.cpu().numpy(), alen.cpu().numpy()
        anodes, atok = anodes.cpu().numpy(), atok.cpu().numpy()
        np.testing.assert_array_equal(pred[:40], ref[0][:40])
        np.testing.assert_array_equal(pred[70:], ref[0][70:])
        for got_b, ref_b in ((0, 2), (2, 0)):
            assert alen[got_b] == ref[1][ref_b], (rep, got_b)
            np.testing.assert_array_equal(anodes[got_b], ref[2][ref_b])
            np.testing.assert_array_equal(atok[got_b], ref[3][ref_b])
        assert alen[1] == 0 and (anodes[1] == -1).all() and (atok[1] == -1).all()


def test_one_workspace_many_calls_and_shapes(ta):
    """One workspace for four shapes (one with 80 sequences), alternated six
    times: every call equals the first of its shape, and that the oracle."""
    rng = np.random.default_rng(21)
    ca = _case(_trees(rng, [30, 200, 64, 5]), 128256, torch.bfloat16, seed=21)
    cb = _case(_trees(rng, [0, 17, 100]), 50000, torch.bfloat16, seed=22)
    cc = _case([[]] * 6 + [[-1, 0]], 1000, torch.float32, seed=23, p=1.0)
    cd = _case(_trees(rng, [2] * 80), 4000, torch.bfloat16, seed=25, p=0.9)
    cases = []
    for c in (ca, cb, cc, cd):
        dc = DevCase(c)
        mask, _, _ = ta.build_mask(dc.parents, dc.node_offsets, dc.max_nodes)
        cases.append((c, dc, mask))
    root_b = _root_logits(cb, 24)
    need = max(ta.verify_workspace_size(ca.total_nodes, 200, 128256),
               ta.verify_workspace_size(cb.total_nodes + cb.B, 100, 50000),
               ta.verify_workspace_size(cc.total_nodes, 2, 1000),
               ta.verify_workspace_size(cd.total_nodes, 2, 4000))
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    first = {}
    for rep in range(6):
        for k, (c, dc, mask) in enumerate(cases):
            if k == 1:
                got, ref = _verify_next(ta, c, dc, mask, root_b, ws=ws)
            else:
                got, ref = _verify(ta, c, dc, mask, ws=ws)
            got = [g.clone() for g in got]
            torch.cuda.synchronize()
            if rep == 0:
                _same(got, ref, f"shape {k}")
                first[k] = got
            else:
                for n, a, b in zip(NAMES, got, first[k]):
                    assert torch.equal(a, b), f"call {rep}/{k}: {n} differs"
