"""The whole step (mask -> forward -> verify) captured in a HIP graph and
replayed must reproduce the eager calls bit for bit, on every replay, with
eager work on other inputs (that overwrites the same output buffers) and
synchronisations in between."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synthetic
from helpers import lib

pytestmark = pytest.mark.gpu


# Two sequences (splits merged by a separate kernel) and one sequence (splits
# merged inside the forward kernel, through counters in the workspace).
SHAPES = {"two_sequences": ([700, 2001], [(64, 1, 6, 4), (37, 2, 5, None)]),
          "one_sequence": ([3000], [(64, 1, 6, 4)]),
          "one_sequence_fused_mask": ([3000], [(64, 1, 6, 4)])}


def _inputs(seed, shape):
    rng = np.random.default_rng(seed)
    lens, specs = SHAPES[shape]
    trees = [synthetic.random_tree(rng, *spec).tolist() for spec in specs]
    c = synthetic.make_case("graph", prefix_lens=lens, trees=trees, Hq=32, Hkv=8, D=128,
                            dtype=torch.bfloat16, seed=seed, vocab=5000, p_match=0.7)
    d = torch.device("cuda")
    t = {"parents": torch.from_numpy(c.parents).to(d),
         "noffs": torch.from_numpy(c.node_offsets).to(d),
         "poffs": torch.from_numpy(c.prefix_offsets).to(d),
         "q": c.q.to(d), "kt": c.k_tree.to(d), "vt": c.v_tree.to(d), "kp": c.k_prefix.to(d),
         "vp": c.v_prefix.to(d), "logits": c.logits.to(d),
         "draft": torch.from_numpy(c.draft).to(d)}
    return c, t


@pytest.mark.parametrize("shape", list(SHAPES))
def test_step_graph_replays_match_eager(shape):
    ta = lib()
    ca, a = _inputs(11, shape)
    cb, b = _inputs(12, shape)
    # Both cases must have the same node counts so they can share output buffers.
    assert ca.total_nodes == cb.total_nodes and ca.max_nodes == cb.max_nodes
    d = torch.device("cuda")
    n, max_nodes, B = ca.total_nodes, ca.max_nodes, ca.B
    W = ta.mask_words(max_nodes)
    bufs = {
        "mask": torch.empty((n, W), dtype=torch.uint64, device=d),
        "depth": torch.empty(n, dtype=torch.int32, device=d),
        "status": torch.empty(B, dtype=torch.int32, device=d),
        "out": torch.empty_like(a["q"]),
        "lse": torch.empty((n, 32), dtype=torch.float32, device=d),
        "pred": torch.empty(n, dtype=torch.int32, device=d),
        "alen": torch.empty(B, dtype=torch.int32, device=d),
        "anodes": torch.empty((B, max_nodes), dtype=torch.int32, device=d),
        "atok": torch.empty((B, max_nodes), dtype=torch.int32, device=d),
    }
    sum_l = int(ca.prefix_offsets[-1])
    fws = torch.zeros(max(ta.forward_workspace_size(torch.bfloat16, B, n, max_nodes, 32, 8, 128,
                                                    sum_l, ca.max_prefix), 16),
                      dtype=torch.uint8, device=d)
    vws = torch.empty(max(ta.verify_workspace_size(n, max_nodes, 5000), 16), dtype=torch.uint8,
                      device=d)

    fused = shape.endswith("fused_mask")

    def step(t, c):
        if fused:
            ta.mask_and_forward(t["parents"], t["q"], t["kt"], t["vt"], t["kp"], t["vp"],
                                t["poffs"], t["noffs"], max_nodes, c.max_prefix, c.scale,
                                out=bufs["out"], lse=bufs["lse"], mask=bufs["mask"],
                                depth=bufs["depth"], status=bufs["status"], workspace=fws)
        else:
            ta.build_mask(t["parents"], t["noffs"], max_nodes, mask=bufs["mask"],
                          depth=bufs["depth"], status=bufs["status"])
            ta.forward(t["q"], t["kt"], t["vt"], t["kp"], t["vp"], t["poffs"], t["noffs"],
                       bufs["mask"], max_nodes, c.max_prefix, c.scale, out=bufs["out"],
                       lse=bufs["lse"], workspace=fws)
        ta.verify_greedy(t["logits"], t["draft"], bufs["mask"], t["noffs"], max_nodes,
                         workspace=vws, target_argmax=bufs["pred"], accept_len=bufs["alen"],
                         accept_nodes=bufs["anodes"], accept_tokens=bufs["atok"])

    def snapshot():
        return {k: v.clone() for k, v in bufs.items()}

    step(a, ca)   # eager first: sets kernel attributes outside capture
    torch.cuda.synchronize()
    ref = snapshot()
    rp, rlen, rnodes, rtok = oracle.verify_greedy(ca.logits, ca.draft, ca.parents,
                                                  ca.node_offsets, max_nodes)
    np.testing.assert_array_equal(ref["alen"].cpu().numpy(), rlen)
    np.testing.assert_array_equal(ref["anodes"].cpu().numpy(), rnodes)

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(a, ca)
    for rep in range(4):
        step(b, cb)                      # eager work on the other inputs
        torch.cuda.synchronize()
        assert not torch.equal(bufs["out"], ref["out"])
        g.replay()
        torch.cuda.synchronize()
        got = snapshot()
        for k in bufs:
            assert torch.equal(got[k], ref[k]), f"replay {rep}: {k} differs from the eager step"


def test_large_verifier_and_sampler_graph_replays_match_eager():
    """The verifier's many-workgroup path (a 1500-node tree: four kernels with
    node-indexed scratch in the workspace) and the stochastic verifier,
    captured in one graph: every replay equals the eager calls bit for bit,
    with eager calls on other inputs into the same buffers in between."""
    ta = lib()
    d = torch.device("cuda")
    V = 3000

    def inputs(seed):
        rng = np.random.default_rng(seed)
        tree = synthetic.random_tree(rng, 1500, 3, 12, None).tolist()
        c = synthetic.make_case("graph_large", prefix_lens=[0], trees=[tree], Hq=1, Hkv=1, D=8,
                                dtype=torch.bfloat16, seed=seed, vocab=V, p_match=0.9)
        s = synthetic.make_sampling_case([tree[:200], tree[:50]], V, seed=seed)
        t = {"parents": torch.from_numpy(c.parents).to(d),
             "noffs": torch.from_numpy(c.node_offsets).to(d),
             "logits": c.logits.to(d), "draft": torch.from_numpy(c.draft).to(d),
             "s_lg": s.logits.to(d), "s_rl": s.root_logits.to(d),
             "s_q": torch.from_numpy(s.draft_probs).to(d),
             "s_rq": torch.from_numpy(s.root_draft_probs).to(d),
             "s_d": torch.from_numpy(s.draft).to(d), "s_p": torch.from_numpy(s.parents).to(d),
             "s_o": torch.from_numpy(s.node_offsets).to(d),
             "s_ua": torch.from_numpy(s.u_accept).to(d), "s_uf": torch.from_numpy(s.u_final).to(d)}
        return c, s, t

    ca, sa, a = inputs(21)
    cb, sb, b = inputs(22)
    n, mx = ca.total_nodes, ca.max_nodes
    bufs = {"mask": torch.empty((n, ta.mask_words(mx)), dtype=torch.uint64, device=d),
            "depth": torch.empty(n, dtype=torch.int32, device=d),
            "status": torch.empty(1, dtype=torch.int32, device=d),
            "pred": torch.empty(n, dtype=torch.int32, device=d),
            "alen": torch.empty(1, dtype=torch.int32, device=d),
            "anodes": torch.empty((1, mx), dtype=torch.int32, device=d),
            "atok": torch.empty((1, mx), dtype=torch.int32, device=d),
            "s_alen": torch.empty(2, dtype=torch.int32, device=d),
            "s_anodes": torch.empty((2, sa.max_nodes), dtype=torch.int32, device=d),
            "s_atok": torch.empty((2, sa.max_nodes), dtype=torch.int32, device=d),
            "s_bonus": torch.empty(2, dtype=torch.int32, device=d)}
    vws = torch.empty(ta.verify_workspace_size(n, mx, V), dtype=torch.uint8, device=d)
    sws = torch.empty(ta.verify_sample_workspace_size(2, 250, V), dtype=torch.uint8, device=d)

    def step(t, s):
        ta.build_mask(t["parents"], t["noffs"], mx, mask=bufs["mask"], depth=bufs["depth"],
                      status=bufs["status"])
        ta.verify_greedy(t["logits"], t["draft"], bufs["mask"], t["noffs"], mx, workspace=vws,
                         target_argmax=bufs["pred"], accept_len=bufs["alen"],
                         accept_nodes=bufs["anodes"], accept_tokens=bufs["atok"])
        ta.verify_sample(t["s_lg"], t["s_rl"], t["s_q"], t["s_rq"], t["s_d"], t["s_p"], t["s_o"],
                         s.max_nodes, s.temperature, t["s_ua"], t["s_uf"], workspace=sws,
                         accept_len=bufs["s_alen"], accept_nodes=bufs["s_anodes"],
                         accept_tokens=bufs["s_atok"], bonus_token=bufs["s_bonus"])

    step(a, sa)
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in bufs.items()}
    _, rlen, rnodes, _ = oracle.verify_greedy(ca.logits, ca.draft, ca.parents, ca.node_offsets, mx)
    np.testing.assert_array_equal(ref["alen"].cpu().numpy(), rlen)
    np.testing.assert_array_equal(ref["anodes"].cpu().numpy(), rnodes)
    assert int(rlen[0]) >= 2
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(a, sa)
    for rep in range(4):
        step(b, sb)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in bufs:
            assert torch.equal(bufs[k], ref[k]), f"replay {rep}: {k} differs from the eager call"
