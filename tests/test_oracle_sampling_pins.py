"""Pins of the stochastic verifier's oracle (oracle.speculative_sample) to
facts other than itself.

The defining property ([PL] Production Inference Runtimes: the speculative
step leaves the target's output distribution unchanged) is checked by Monte
Carlo on a tiny vocabulary: drafts drawn from the draft model, the step run
on them, and the first two emitted tokens compared with the target's own
two-token distribution (a chi-square bound); the same bound fails on an
oracle whose rejections skip the residual update (planted in a second test).
Exact special cases: a draft equal to the target accepts the
first child at every level; a token the target gives no mass is never
accepted; the bonus after a rejection is drawn from the target with the
rejected token removed; temperature scales logits; empty and invalid trees
sample the prefix row.
"""
import numpy as np
import pytest

import oracle

V = 4


def _dirichlet_world(seed):
    """Target and draft next-token distributions as functions of the token
    context (a tuple), so that equal contexts see equal rows."""
    rng = np.random.default_rng(seed)
    tgt, drf = {}, {}

    def get(table, ctx):
        if ctx not in table:
            table[ctx] = rng.dirichlet(np.full(V, 0.7))
        return table[ctx]

    return (lambda ctx: get(tgt, ctx)), (lambda ctx: get(drf, ctx))


def _run_step(target, draftd, rng, kids=(3, 2)):
    """One speculative step on a tree with kids[0] roots, each with kids[1]
    children; every node's token drawn from the draft at its context."""
    parents, tokens, ctxs = [], [], []
    for _ in range(kids[0]):
        parents.append(-1)
        t = int(rng.choice(V, p=draftd(())))
        tokens.append(t)
        ctxs.append((t,))
    for r in range(kids[0]):
        for _ in range(kids[1]):
            parents.append(r)
            t = int(rng.choice(V, p=draftd(ctxs[r])))
            tokens.append(t)
            ctxs.append(ctxs[r] + (t,))
    n = len(parents)
    logits = np.log(np.stack([target(c) for c in ctxs]))
    q = np.stack([draftd(c) for c in ctxs])
    root_logits = np.log(target(()))[None]
    root_q = draftd(())[None]
    u = rng.random(n)
    uf = rng.random(1)
    alen, anodes, atok, bonus, margin = oracle.speculative_sample(
        logits, root_logits, q, root_q, tokens, parents, [0, n], 1.0, u, uf, n)
    emitted = [int(t) for t in atok[0, :alen[0]]] + [int(bonus[0])]
    return emitted


def _chi2(counts, probs):
    exp = probs * counts.sum()
    return float(((counts - exp) ** 2 / exp).sum())


def test_first_two_tokens_follow_the_target():
    """Lossless in distribution: (t1, t2) ~ target(()) x target((t1,)), with
    t2 drawn from the target itself when the step emitted one token (what
    the next step would do)."""
    target, draftd = _dirichlet_world(1)
    rng = np.random.default_rng(2)
    trials = 12000
    counts = np.zeros((V, V))
    for _ in range(trials):
        em = _run_step(target, draftd, rng)
        t1 = em[0]
        t2 = em[1] if len(em) > 1 else int(rng.choice(V, p=target((t1,))))
        counts[t1, t2] += 1
    probs = np.array([[target(())[a] * target((a,))[b] for b in range(V)] for a in range(V)])
    stat = _chi2(counts.ravel(), probs.ravel())
    # 15 degrees of freedom: the 0.999 quantile is 37.7
    assert stat < 37.7, stat


def test_the_pin_rejects_a_step_without_the_residual(monkeypatch):
    """The same statistic on an oracle whose rejections keep P unchanged (a
    plausible slip, planted here) is far outside the bound: the pin has
    teeth."""
    import oracle.speculative_sampling as ss
    monkeypatch.setattr(ss, "residual", lambda P, Q: P)
    target, draftd = _dirichlet_world(1)
    rng = np.random.default_rng(2)
    counts = np.zeros(V)
    for _ in range(4000):
        counts[_run_step(target, draftd, rng)[0]] += 1
    stat = _chi2(counts, target(()))
    assert stat > 30.0, stat


def test_draft_equal_to_target_accepts_the_first_child_everywhere():
    rng = np.random.default_rng(5)
    parents = [-1, -1, 0, 0, 2, 1, 4]
    n = len(parents)
    Vb = 50
    logits = rng.normal(size=(n, Vb)) * 2
    root_logits = rng.normal(size=(1, Vb)) * 2
    T = 0.7
    q = np.stack([oracle.softmax_t(r, T) for r in logits])
    root_q = oracle.softmax_t(root_logits[0], T)[None]
    draft = rng.integers(Vb, size=n)
    u = np.full(n, 0.999)
    alen, anodes, atok, bonus, _ = oracle.speculative_sample(
        logits, root_logits, q, root_q, draft, parents, [0, n], T, u, [0.5], n)
    # first root 0, its first child 2, then 2's child 4, then 6
    assert alen[0] == 4 and anodes[0, :4].tolist() == [0, 2, 4, 6]
    assert atok[0, :4].tolist() == [int(draft[j]) for j in (0, 2, 4, 6)]
    cdf = np.cumsum(oracle.softmax_t(logits[6], T))
    assert bonus[0] == int(np.argmax(cdf > 0.5))


def test_token_without_target_mass_is_rejected_and_removed_from_the_bonus():
    """Root child token x with target logit -inf is rejected for any u; with
    the draft one-hot on x the residual is the target itself.  A second
    child x' with one-hot draft, rejected (u * 1 >= P(x')), removes x' from
    the bonus distribution."""
    Vb = 6
    p = np.array([0.1, 0.2, 0.0, 0.3, 0.15, 0.25])
    root_logits = np.log(np.where(p > 0, p, 1e-300))[None]
    root_logits[0, 2] = -np.inf
    parents = [-1, -1]
    draft = [2, 3]
    q_root = np.zeros((1, Vb))
    q_root[0, 2] = 1.0
    logits = np.zeros((2, Vb))
    q = np.full((2, Vb), 1.0 / Vb)
    # child 0 (token 2): P(2) = 0, rejected; residual max(0, p - e2) = p.
    # child 1 (token 3) is then tested against the same one-hot draft: u*Q(3)=0 < P(3): accepted
    alen, anodes, _, _, _ = oracle.speculative_sample(
        logits, root_logits, q, q_root, draft, parents, [0, 2], 1.0, [0.0, 0.9], [0.3], 2)
    assert alen[0] == 1 and anodes[0, 0] == 1
    # now draft one-hot on token 3 for the second test: reject it (0.9 * 1 >= 0.3)
    q_root2 = np.zeros((1, Vb))
    q_root2[0, 3] = 1.0
    for uf in (0.05, 0.2, 0.5, 0.75, 0.99):
        alen, _, _, bonus, _ = oracle.speculative_sample(
            logits, root_logits, q, q_root2, [3], [-1], [0, 1], 1.0, [0.9], [uf], 1)
        assert alen[0] == 0
        kept = p.copy()
        kept[3] = 0.0
        kept /= kept.sum()
        want = next(v for v in range(Vb) if kept[:v + 1].sum() > uf)
        assert bonus[0] == want


def test_temperature_divides_the_logits():
    rng = np.random.default_rng(9)
    parents = [-1, 0, 0, 1]
    n = 4
    Vb = 30
    p_rows = rng.dirichlet(np.ones(Vb), size=n)
    p_root = rng.dirichlet(np.ones(Vb), size=1)
    q = rng.dirichlet(np.ones(Vb), size=n)
    q_root = rng.dirichlet(np.ones(Vb), size=1)
    draft = rng.integers(Vb, size=n)
    u = rng.random(n)
    for uf in (0.1, 0.6):
        a = oracle.speculative_sample(np.log(p_rows), np.log(p_root), q, q_root, draft, parents,
                                      [0, n], 1.0, u, [uf], n)
        b = oracle.speculative_sample(2.5 * np.log(p_rows), 2.5 * np.log(p_root), q, q_root,
                                      draft, parents, [0, n], 2.5, u, [uf], n)
        for x, y in zip(a[:4], b[:4]):
            np.testing.assert_array_equal(x, y)


@pytest.mark.parametrize("parents", [[], [1, 0], [-1, 5]])
def test_empty_and_invalid_trees_sample_the_prefix_row(parents):
    rng = np.random.default_rng(3)
    Vb = 20
    n = len(parents)
    root_logits = rng.normal(size=(1, Vb))
    logits = rng.normal(size=(max(n, 1), Vb))[:n]
    q = np.full((n, Vb), 1.0 / Vb)
    q_root = np.full((1, Vb), 1.0 / Vb)
    draft = [0] * n
    for uf in (0.0, 0.37, 0.999):
        alen, anodes, _, bonus, margin = oracle.speculative_sample(
            logits, root_logits, q, q_root, draft, parents, [0, n], 1.0, np.zeros(n), [uf], 4)
        assert alen[0] == 0 and (anodes[0] == -1).all()
        p = np.exp(root_logits[0] - root_logits[0].max())
        p /= p.sum()
        assert bonus[0] == int(np.searchsorted(np.cumsum(p), uf, side="right"))
        assert margin[0] >= 0.0
