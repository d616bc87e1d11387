"""Plain fp64 CPU oracle for tree attention and greedy tree verification.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package.  It shares no code with the HIP
library and never calls it.

Sources (the pages this follows):
  [IS]  "Tree Attention", inferensys.com glossary (Speculative Decoding):
        sections "What is Tree Attention?", "Key Mechanisms of Tree Attention"
        (Modified Causal Attention Mask; Multi-Token Acceptance & Rollback),
        and the "Tree Attention vs. Standard Attention" comparison table.
  [ZT]  "Tree Attention", zhongzhoutan-coder.github.io glossary term:
        sections "How It Works" and "Common Confusions".
  [PL]  "Speculative Tree Attention: How Multi-Candidate Draft Models and
        Parallel Verification Deliver 4x LLM Speedups", news.premlal.in:
        the code listing (build_tree_attention_mask, verify_candidate_tree and
        its __main__ demo); section "Production Inference Runtimes" (the
        claim that the speculative step leaves the target's output
        distribution unchanged), for the stochastic verifier, whose rule the
        pages do not give: speculative_sampling.py takes the published one.
"""
from .tree_attention import (  # noqa: F401
    STATUS_OK,
    STATUS_INVALID_ARG,
    STATUS_INVALID_TREE,
    tree_is_valid,
    root_path,
    ancestor_mask_dense,
    pack_mask_words,
    build_mask,
    path_causal_attention,
    tree_attention,
    target_argmax,
    verify_greedy,
    verify_greedy_next,
    kv_commit,
)
from .speculative_sampling import (  # noqa: F401
    softmax_t,
    sample_inverse_cdf,
    speculative_sample,
)
