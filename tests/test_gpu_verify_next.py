"""GPU parity of the greedy verifier on next-token rows
(tree_verify_greedy_next), through the C ABI, against the fp64 oracle: target
argmax, accepted paths and the bonus token bit for bit, over random trees and
forests (scalar and vector scans, up to 64 vocabulary chunks per row), forced
ties, and the identity with tree_verify_greedy on rows gathered from each
node's parent."""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from helpers import DevCase, lib

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ta():
    return lib()


def _draft_following(c, root_logits, rng, p):
    pred = np.argmax(c.logits.double().numpy(), axis=1)
    rpred = np.argmax(root_logits.double().numpy(), axis=1)
    draft = np.zeros(c.total_nodes, dtype=np.int32)
    for b in range(c.B):
        lo, hi = int(c.node_offsets[b]), int(c.node_offsets[b + 1])
        for i in range(hi - lo):
            par = int(c.parents[lo + i])
            want = rpred[b] if par < 0 else pred[lo + par]
            draft[lo + i] = want if rng.random() < p else int(rng.integers(c.vocab))
    return draft


def _run(ta, c, root_logits, draft):
    dc = DevCase(c)
    mask, _, _ = ta.build_mask(dc.parents, dc.node_offsets, dc.max_nodes)
    d = torch.device("cuda")
    got = ta.verify_greedy_next(dc.logits, root_logits.to(d), torch.from_numpy(draft).to(d), mask,
                                dc.node_offsets, dc.max_nodes)
    ref = oracle.verify_greedy_next(c.logits, root_logits, draft, c.parents, c.node_offsets,
                                    dc.max_nodes)
    names = ("target_argmax", "accept_len", "accept_nodes", "accept_tokens", "bonus_token")
    for n, a, r in zip(names, got, ref):
        np.testing.assert_array_equal(a.cpu().numpy(), r, err_msg=n)
    return dc, mask, ref


@pytest.mark.parametrize("dtype,V", [(torch.bfloat16, 50000), (torch.float32, 1001),
                                     (torch.bfloat16, 77), (torch.bfloat16, 128256),
                                     (torch.float32, 700000)])
def test_verify_next_random_trees(ta, dtype, V):
    rng = np.random.default_rng(V + 1)
    trees = [synthetic.random_tree(rng, n, r, 8, 3).tolist() for n, r in
             ((1, 1), (30, 1), (200, 4), (64, 1), (5, 5))]
    c = synthetic.make_case("vnext", prefix_lens=[0] * 5, trees=trees, Hq=1, Hkv=1, D=8,
                            dtype=dtype, seed=V + 1, vocab=V)
    g = torch.Generator().manual_seed(V + 2)
    root_logits = torch.randn((c.B, V), generator=g).to(dtype)
    draft = _draft_following(c, root_logits, rng, 0.9)
    print(f"[verify next] dtype={dtype} V={V}", flush=True)
    _, _, ref = _run(ta, c, root_logits, draft)
    print(f"[verify next] accept_len={ref[1].tolist()} bonus={ref[4].tolist()}", flush=True)


def test_verify_next_ties_and_empty_acceptance(ta):
    V = 128256
    trees = [[-1, 0, 1, 1], [-1, -1]]
    c = synthetic.make_case("nties", prefix_lens=[0, 0], trees=trees, Hq=1, Hkv=1, D=8, seed=6,
                            vocab=V)
    lg = c.logits
    lg[0, 100] = lg[0, 90000] = 20.0        # tie in different vocab chunks -> 100
    lg[1, :] = 0.0                          # all equal -> 0
    lg[3, V - 1] = 30.0                     # maximum in the last entry
    root = torch.randn((2, V), generator=torch.Generator().manual_seed(7)).to(torch.bfloat16)
    root[0, 3] = root[0, 70000] = 25.0      # -> 3
    draft = np.array([3, 100, 0, 100, 17, 18], dtype=np.int32)   # seq 1: both roots rejected
    _, _, ref = _run(ta, c, root, draft)
    assert ref[1].tolist() == [3, 0]
    assert ref[4][0] == int(torch.argmax(lg[2].float()))
    assert ref[4][1] == int(torch.argmax(root[1].float()))


def test_verify_next_equals_same_row_verifier_on_gathered_rows(ta):
    rng = np.random.default_rng(31)
    trees = [synthetic.random_tree(rng, 64, 2, 6, 4).tolist() for _ in range(3)]
    V = 4096
    c = synthetic.make_case("gather", prefix_lens=[0] * 3, trees=trees, Hq=1, Hkv=1, D=8, seed=31,
                            vocab=V)
    root_logits = torch.randn((3, V), generator=torch.Generator().manual_seed(32)).to(torch.bfloat16)
    draft = _draft_following(c, root_logits, rng, 0.85)
    dc, mask, ref = _run(ta, c, root_logits, draft)
    gathered = torch.empty_like(c.logits)
    for b in range(c.B):
        lo, hi = int(c.node_offsets[b]), int(c.node_offsets[b + 1])
        for i in range(hi - lo):
            par = int(c.parents[lo + i])
            gathered[lo + i] = root_logits[b] if par < 0 else c.logits[lo + par]
    d = torch.device("cuda")
    _, alen, anodes, atok = ta.verify_greedy(gathered.to(d), torch.from_numpy(draft).to(d), mask,
                                             dc.node_offsets, dc.max_nodes)
    np.testing.assert_array_equal(alen.cpu().numpy(), ref[1])
    np.testing.assert_array_equal(anodes.cpu().numpy(), ref[2])
    np.testing.assert_array_equal(atok.cpu().numpy(), ref[3])


def test_verify_next_at_the_node_limit(ta):
    """A 1024-node chain and a 1024-node forest (16 mask words per row): the
    parent search walks down through every word."""
    rng = np.random.default_rng(70)
    trees = [[-1] + list(range(1023)), synthetic.random_tree(rng, 1024, 5, 40, 3).tolist()]
    V = 300
    c = synthetic.make_case("nbig", prefix_lens=[0, 0], trees=trees, Hq=1, Hkv=1, D=8,
                            dtype=torch.float32, seed=70, vocab=V)
    root_logits = torch.randn((2, V), generator=torch.Generator().manual_seed(71))
    draft = _draft_following(c, root_logits, rng, 0.995)
    _, _, ref = _run(ta, c, root_logits, draft)
    print(f"[verify next] accept_len={ref[1].tolist()}", flush=True)
