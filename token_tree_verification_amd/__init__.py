"""token_tree_verification_amd -- token-tree verification on AMD MI355X.

Python front end of libtv.so (include/tv.h): ancestor-masked tree attention
and the greedy / lossless speculative-sampling accept/reject walk, as
hand-written HIP kernels for gfx950.  Tensors are torch device tensors; torch
supplies memory and streams only.
"""
from ._binding import (  # noqa: F401
    ACCEPT_GREEDY,
    ACCEPT_SIBLINGS_WOR,
    LIB_PATH,
    TV_MAX_NODES,
    WAIT_DEFAULT,
    TVError,
    accept_plan,
    accept_workspace_bytes,
    attention_workspace_bytes,
    build_tree_mask,
    commit_kv,
    library,
    mask_words,
    philox_uniforms,
    set_wait_limit,
    spec_accept,
    tree_attention,
    tree_expand,
    tree_pool,
    tree_select,
)

__all__ = [
    "build_tree_mask",
    "tree_attention",
    "spec_accept",
    "commit_kv",
    "tree_pool",
    "tree_expand",
    "tree_select",
    "accept_plan",
    "set_wait_limit",
    "mask_words",
    "philox_uniforms",
    "attention_workspace_bytes",
    "accept_workspace_bytes",
    "library",
    "TVError",
    "LIB_PATH",
]
