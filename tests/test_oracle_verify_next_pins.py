"""Pins of the oracle's greedy verifier on next-token rows (with its bonus
token) against facts fixed outside that function: the same acceptance as the
same-row verifier once every node's row is gathered from its parent (the
indexing step the two readings differ by), the textbook speculative-decoding
loop on a chain written out position by position, numpy.argmax for the
predictions, and the degenerate cases."""
import numpy as np
import pytest
import torch

import oracle
import synthetic


def _case(seed, trees, V=50, p=0.8):
    rng = np.random.default_rng(seed)
    c = synthetic.make_case("next", prefix_lens=[0] * len(trees), trees=trees, Hq=1, Hkv=1, D=4,
                            dtype=torch.float32, seed=seed, vocab=V)
    B = len(trees)
    g = torch.Generator().manual_seed(seed + 1000)
    root_logits = torch.randn((B, V), generator=g)
    return c, root_logits, rng


def _draft_following(c, root_logits, rng, p):
    """Draft tokens that agree with the parent's (prefix's) prediction with
    probability p, else a random token."""
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


@pytest.mark.parametrize("seed", range(8))
def test_equals_same_row_verifier_on_rows_gathered_from_parents(seed):
    rng0 = np.random.default_rng(seed)
    trees = [synthetic.random_tree(rng0, int(n), int(r), 5, 3).tolist()
             for n, r in ((20, 1), (7, 2), (33, 3))]
    c, root_logits, rng = _case(seed, trees)
    draft = _draft_following(c, root_logits, rng, 0.85)
    got = oracle.verify_greedy_next(c.logits, root_logits, draft, c.parents, c.node_offsets, 40)
    gathered = torch.empty_like(c.logits)
    for b in range(c.B):
        lo, hi = int(c.node_offsets[b]), int(c.node_offsets[b + 1])
        for i in range(hi - lo):
            par = int(c.parents[lo + i])
            gathered[lo + i] = root_logits[b] if par < 0 else c.logits[lo + par]
    ref = oracle.verify_greedy(gathered, draft, c.parents, c.node_offsets, 40)
    for a, r in zip(got[1:4], ref[1:4]):
        np.testing.assert_array_equal(a, r)
    np.testing.assert_array_equal(got[0], np.argmax(c.logits.double().numpy(), axis=1))


@pytest.mark.parametrize("seed", range(6))
def test_chain_is_the_position_by_position_loop(seed):
    n = 9
    c, root_logits, rng = _case(seed, [[-1] + list(range(n - 1))], V=12)
    draft = _draft_following(c, root_logits, rng, 0.7)
    # Standard greedy speculative decoding on one sequence of drafted tokens:
    # the k-th drafted token is kept while it equals the target's prediction
    # at the previous position; the step then adds the target's own token.
    preds = [int(np.argmax(root_logits[0].double().numpy()))]
    preds += [int(np.argmax(c.logits[k].double().numpy())) for k in range(n)]
    k = 0
    while k < n and int(draft[k]) == preds[k]:
        k += 1
    pred, alen, anodes, atok, bonus = oracle.verify_greedy_next(c.logits, root_logits, draft,
                                                               c.parents, c.node_offsets, n)
    assert alen[0] == k
    assert anodes[0, :k].tolist() == list(range(k)) and (anodes[0, k:] == -1).all()
    assert atok[0, :k].tolist() == draft[:k].tolist()
    assert bonus[0] == preds[k]


def test_degenerate_cases():
    trees = [[-1, 0, 0, 1], [-1, -1, 0]]
    c, root_logits, rng = _case(3, trees)
    pred = np.argmax(c.logits.double().numpy(), axis=1)
    rpred = np.argmax(root_logits.double().numpy(), axis=1)
    # nothing matches: length 0, all -1, bonus = the prefix's prediction
    wrong = np.array([(int(rpred[0]) + 1) % c.vocab] * 4 + [(int(rpred[1]) + 1) % c.vocab] * 3,
                     dtype=np.int32)
    _, alen, anodes, atok, bonus = oracle.verify_greedy_next(c.logits, root_logits, wrong,
                                                            c.parents, c.node_offsets, 4)
    assert alen.tolist() == [0, 0] and (anodes == -1).all() and (atok == -1).all()
    assert bonus.tolist() == rpred.tolist()
    # everything matches: the deepest path, lowest index on ties; bonus from its leaf
    right = np.zeros(7, dtype=np.int32)
    for b, (lo, hi) in enumerate(((0, 4), (4, 7))):
        for i in range(hi - lo):
            par = int(c.parents[lo + i])
            right[lo + i] = rpred[b] if par < 0 else pred[lo + par]
    _, alen, anodes, _, bonus = oracle.verify_greedy_next(c.logits, root_logits, right,
                                                         c.parents, c.node_offsets, 4)
    assert alen.tolist() == [3, 2]
    assert anodes[0, :3].tolist() == [0, 1, 3] and anodes[1, :2].tolist() == [0, 2]
    assert bonus.tolist() == [int(pred[3]), int(pred[4 + 2])]
