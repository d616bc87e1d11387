"""Tree attention and tree verification (greedy, and by rejection sampling) on
AMD Instinct MI355X (gfx950).

The computation lives in ``libtreeattn.so`` (hand-written HIP kernels behind
the C ABI of ``include/tree_attn.h``); this package is its Python binding.
Importing the package loads the library and raises ImportError when it has not
been built (``python tree_masked_attention_forward_amd/build.py``).
"""
from ._binding import (  # noqa: F401
    LIBRARY_PATH,
    TA_BF16,
    TA_ERR_HIP,
    TA_ERR_INVALID_ARG,
    TA_ERR_INVALID_TREE,
    TA_ERR_UNSUPPORTED,
    TA_ERR_WORKSPACE,
    TA_F32,
    TA_MAX_NODES,
    TA_MERGE_PLACEMENT,
    TA_MERGE_STALE,
    TA_MERGE_TIMEOUT,
    TA_NOALLOC_MAX_WORKSPACE,
    TA_OK,
    TreeAttnError,
    build_mask,
    forward,
    forward_noalloc,
    forward_workspace_size,
    kv_commit,
    load_library,
    mask_and_forward,
    mask_words,
    merge_status,
    status_string,
    verify_greedy,
    verify_greedy_next,
    verify_sample,
    verify_sample_workspace_size,
    verify_workspace_size,
)

load_library()

# The C names, for readers who know the ABI.
tree_attn_build_mask = build_mask
tree_attn_forward = forward
tree_attn_forward_noalloc = forward_noalloc
tree_attn_mask_and_forward = mask_and_forward
tree_verify_greedy = verify_greedy
tree_kv_commit = kv_commit
tree_verify_greedy_next = verify_greedy_next
tree_verify_sample = verify_sample
