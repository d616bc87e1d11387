"""GPU parity of stochastic verification (tree_verify_sample) against the
fp64 oracle (oracle.speculative_sample), and its defining property on the GPU.

"Speculative Tree Attention" (news.premlal.in), Production Inference Runtimes:
the speculative step leaves the target's output distribution unchanged; the
rule is the published one (speculative sampling's accept test and residual
walked down the tree), see the oracle.

The decisions are integers decided by floating point: the kernel computes in
fp32, the oracle in fp64.  For each sequence the oracle reports the smallest
relative distance between the two sides of any of its accept tests (relative
to the operands P(x) came from); where it exceeds 1e-4 (fp32 keeps a softmax
over 128256 entries to ~1e-6 relative) the accepted path must match exactly:
length, nodes and tokens.  The bonus draw is then checked against the
oracle's final distribution: the GPU's token must be the inverse-CDF draw of
some u within 2e-5 of u_final (fp32 cumulative sums over the vocabulary
carry errors of order 1e-6), and must carry mass.  Sequences within the
accept margin are counted and must be a small minority.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from helpers import lib

pytestmark = pytest.mark.gpu

TOL = 1e-4


@pytest.fixture(scope="module")
def ta():
    return lib()


def _run(ta, c):
    d = torch.device("cuda")
    out = ta.verify_sample(
        c.logits.to(d), c.root_logits.to(d), torch.from_numpy(c.draft_probs).to(d),
        torch.from_numpy(c.root_draft_probs).to(d), torch.from_numpy(c.draft).to(d),
        torch.from_numpy(c.parents).to(d), torch.from_numpy(c.node_offsets).to(d), c.max_nodes,
        c.temperature, torch.from_numpy(c.u_accept).to(d), torch.from_numpy(c.u_final).to(d))
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in out]


def _oracle(c, final_p=None):
    return oracle.speculative_sample(c.logits, c.root_logits, c.draft_probs, c.root_draft_probs,
                                     c.draft, c.parents, c.node_offsets, c.temperature,
                                     c.u_accept, c.u_final, c.max_nodes, final_p=final_p)


EPS_CDF = 2e-5


def _valid_draw(p, u, v):
    """v is the lowest token whose cumulative probability exceeds some u'
    within EPS_CDF of u, and carries mass."""
    if not (0 <= v < len(p)) or p[v] <= 0:
        return False
    cdf = np.cumsum(p)
    lo = cdf[v - 1] if v > 0 else 0.0
    return lo - EPS_CDF <= u < cdf[v] + EPS_CDF


def _compare(got, c, what):
    alen, anodes, atok, bonus = got
    fp = []
    ralen, ranodes, ratok, rbonus, margin = _oracle(c, fp)
    checked = 0
    for b in range(len(ralen)):
        if margin[b] <= TOL:
            continue
        checked += 1
        msg = f"{what} sequence {b} (margin {margin[b]:.2e})"
        assert alen[b] == ralen[b], msg
        np.testing.assert_array_equal(anodes[b], ranodes[b], err_msg=msg)
        np.testing.assert_array_equal(atok[b], ratok[b], err_msg=msg)
        assert _valid_draw(fp[b], float(c.u_final[b]), int(bonus[b])), (
            f"{msg}: bonus {bonus[b]} (oracle {rbonus[b]})")
    print(f"[sample] {what}: {checked}/{len(ralen)} sequences checked, "
          f"accept_len={ralen.tolist()[:16]}, bonus equal to the oracle's: "
          f"{int((bonus == rbonus).sum())}/{len(rbonus)}", flush=True)
    return checked, ralen


@pytest.mark.parametrize("dtype,V", [(torch.bfloat16, 128256), (torch.bfloat16, 1000),
                                     (torch.float32, 777)])
def test_sample_matches_oracle_on_random_trees(ta, dtype, V):
    rng = np.random.default_rng(V)
    trees = [synthetic.random_tree(rng, n, r, d, k).tolist()
             for n, r, d, k in ((64, 1, 6, 4), (20, 2, None, None), (1, 1, None, None),
                                (100, 3, 8, 3), (40, 1, 10, 2))]
    trees.append([])               # empty sequence: the bonus from the prefix row
    trees.append([1, 2, 0])        # a cycle: walked as empty
    c = synthetic.make_sampling_case(trees, V, dtype=dtype, seed=V, temperature=0.8, noise=0.4)
    print(f"[sample] dtype={dtype} V={V} sizes={[len(t) for t in trees]}", flush=True)
    got = _run(ta, c)
    checked, ralen = _compare(got, c, f"{dtype} V={V}")
    assert checked >= len(trees) - 2
    assert ralen.max() >= 2, "the drafts should give accepted paths"
    assert ralen[-1] == 0 and ralen[-2] == 0


def test_sample_many_sequences_and_reranked_orders(ta):
    """32 sequences (one workgroup each) with reranked node orders."""
    rng = np.random.default_rng(31)
    trees = []
    for b in range(32):
        t = synthetic.random_tree(rng, int(rng.integers(1, 90)), 1 + b % 3, 7, 4)
        trees.append(synthetic.rerank_tree(t, rng.permutation(len(t))).tolist())
    c = synthetic.make_sampling_case(trees, 4096, seed=32, temperature=1.3, noise=0.3)
    got = _run(ta, c)
    checked, _ = _compare(got, c, "32 reranked")
    assert checked >= 28


@pytest.mark.parametrize("dtype,V,noise,scale", [(torch.bfloat16, 128256, 6.0, 4.0),
                                                 (torch.float32, 999, 3.0, 2.0)])
def test_sample_wide_fanout_many_rejections(ta, dtype, V, noise, scale):
    """Forty roots and forty children under root 0 (a forest plus a wide
    node), with a draft far from the target: long runs of rejections at one
    node, past the kernel's chain of eight kept residual steps (the ninth
    writes the residual out and the chain restarts from it)."""
    trees = [[-1] * 40 + [0] * 40, [-1] + [0] * 30 + list(range(1, 31))]
    c = synthetic.make_sampling_case(trees, V, dtype=dtype, seed=5, temperature=1.0,
                                     noise=noise, scale=scale)
    got = _run(ta, c)
    checked, ralen = _compare(got, c, f"wide fan-out {dtype} V={V}")
    assert checked == 2   # (41 rejections in both cases, margins above the bar)


def test_sample_draft_equal_to_target_accepts_first_children(ta):
    """With the draft given as the target's own distribution every tested
    child is accepted (u < 0.999 and the two sides differ only by rounding),
    so the path follows the first child at every level."""
    V = 3000
    parents = [-1, -1, 0, 0, 2, 1, 4, 4]
    c = synthetic.make_sampling_case([parents], V, dtype=torch.float32, seed=4)
    lg = np.concatenate([c.logits.numpy(), c.root_logits.numpy()]).astype(np.float64)
    T = c.temperature
    p = np.exp((lg - lg.max(axis=1, keepdims=True)) / T)
    p = (p / p.sum(axis=1, keepdims=True)).astype(np.float32)
    c.draft_probs, c.root_draft_probs = p[:len(parents)].copy(), p[len(parents):].copy()
    c.u_accept = np.minimum(c.u_accept, np.float32(0.999))
    got = _run(ta, c)
    assert got[0][0] == 4 and got[1][0, :4].tolist() == [0, 2, 4, 6]
    checked, ralen = _compare(got, c, "draft = target")
    assert checked == 1 and ralen[0] == 4


def test_sample_is_lossless_on_the_gpu(ta):
    """The defining property measured on the kernel itself: 20000 sequences of
    one small tree (three roots with two children each, V = 4), drafts drawn
    from the draft model, all in one call; the first two emitted tokens
    follow the target's two-token distribution (chi-square, 15 degrees of
    freedom, 0.999 quantile 37.7).  The context-dependent target and draft
    rows make equal contexts see equal distributions."""
    V = 4
    B = 20000
    rng = np.random.default_rng(77)
    tgt_ctx, drf_ctx = {}, {}

    def row(table, ctx):
        if ctx not in table:
            table[ctx] = rng.dirichlet(np.full(V, 0.7))
        return table[ctx]

    parents = [-1, -1, -1, 0, 0, 1, 1, 2, 2]
    n = len(parents)
    logits = np.zeros((B * n, V), np.float32)
    q = np.zeros((B * n, V), np.float32)
    root_logits = np.zeros((B, V), np.float32)
    root_q = np.zeros((B, V), np.float32)
    draft = np.zeros(B * n, np.int32)
    p0, q0 = row(tgt_ctx, ()), row(drf_ctx, ())
    for a in range(V):
        row(tgt_ctx, (a,)), row(drf_ctx, (a,))
        for b2 in range(V):
            row(tgt_ctx, (a, b2)), row(drf_ctx, (a, b2))
    for b in range(B):
        root_logits[b] = np.log(p0)
        root_q[b] = q0
        ctx = {}
        for i, pa in enumerate(parents):
            c0 = () if pa < 0 else ctx[pa]
            t = int(rng.choice(V, p=drf_ctx[c0]))
            draft[b * n + i] = t
            ctx[i] = c0 + (t,)
            logits[b * n + i] = np.log(tgt_ctx[ctx[i]] if len(ctx[i]) <= 2 else p0)
            q[b * n + i] = drf_ctx[ctx[i]] if len(ctx[i]) <= 2 else q0
    d = torch.device("cuda")
    offs = np.arange(0, B * n + 1, n, dtype=np.int32)
    out = ta.verify_sample(
        torch.from_numpy(logits).to(d), torch.from_numpy(root_logits).to(d),
        torch.from_numpy(q).to(d), torch.from_numpy(root_q).to(d), torch.from_numpy(draft).to(d),
        torch.from_numpy(np.tile(np.array(parents, np.int32), B)).to(d),
        torch.from_numpy(offs).to(d), n, 1.0,
        torch.from_numpy(rng.random(B * n).astype(np.float32)).to(d),
        torch.from_numpy(rng.random(B).astype(np.float32)).to(d))
    alen, _, atok, bonus = [t.cpu().numpy() for t in out]
    counts = np.zeros((V, V))
    for b in range(B):
        em = list(atok[b, :alen[b]]) + [int(bonus[b])]
        t1 = int(em[0])
        t2 = int(em[1]) if len(em) > 1 else int(rng.choice(V, p=tgt_ctx[(t1,)]))
        counts[t1, t2] += 1
    probs = np.array([[p0[a] * tgt_ctx[(a,)][b2] for b2 in range(V)] for a in range(V)])
    exp = probs.ravel() * B
    stat = float(((counts.ravel() - exp) ** 2 / exp).sum())
    print(f"[sample] lossless chi2={stat:.1f} mean accept_len={alen.mean():.2f}", flush=True)
    assert stat < 37.7
    assert alen.mean() > 0.5
