"""The seeded generators follow their stated recipe (CPU only)."""
import numpy as np
import torch

import synthetic


def _depths(parents):
    d = np.zeros(len(parents), np.int64)
    for i, p in enumerate(parents):
        d[i] = 0 if p < 0 else d[p] + 1
    return d


def test_random_tree_respects_caps_and_order():
    for seed in range(20):
        rng = np.random.default_rng(seed)
        par = synthetic.random_tree(rng, 64, 1, 6, 4)
        assert par[0] == -1 and (par[1:] >= 0).all()
        assert all(par[i] < i for i in range(1, 64))
        assert _depths(par).max() <= 6
        assert np.bincount(par[par >= 0], minlength=64).max() <= 4
    par = synthetic.random_tree(np.random.default_rng(0), 512, 8, 16, None)
    assert (par[:8] == -1).all() and (par[8:] >= 0).all() and _depths(par).max() <= 16


def test_generators_are_deterministic():
    a = synthetic.make_config_case("llama3_8b", with_logits=False)
    b = synthetic.make_config_case("llama3_8b", with_logits=False)
    assert np.array_equal(a.parents, b.parents)
    assert torch.equal(a.q, b.q) and torch.equal(a.v_prefix, b.v_prefix)
    assert a.q.dtype == torch.bfloat16 and a.q.shape == (64, 32, 128)
    assert a.k_prefix.shape == (4096, 8, 128)


def test_batched_ragged_lengths_and_offsets():
    c = synthetic.make_config_case("batched", with_logits=False)
    lens = c.prefix_lens
    assert len(lens) == 32 and min(lens) >= 512 and max(lens) <= 8192
    assert c.prefix_offsets[-1] == sum(lens) and c.node_offsets[-1] == 32 * 64


def test_draft_rule_and_tiny_planting():
    c = synthetic.make_case("t", prefix_lens=[3], trees=[[-1, 0, 0, 1]], Hq=1, Hkv=1, D=4,
                            vocab=1000, seed=3, p_match=1.0)
    assert np.array_equal(c.draft, torch.argmax(c.logits, 1).numpy())
    t = synthetic.make_config_case("tiny")
    assert t.dtype == torch.float32 and t.k_prefix.shape == (16, 1, 64)
    assert t.parents.tolist() == synthetic.EXAMPLE_PARENTS
    assert t.draft.tolist() == synthetic.EXAMPLE_TOKENS
