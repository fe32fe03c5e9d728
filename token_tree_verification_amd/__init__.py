"""token_tree_verification_amd -- token-tree verification on AMD MI355X.

Python front end of libtv.so (include/tv.h): ancestor-masked tree attention
and the greedy / lossless speculative-sampling accept/reject walk, as
hand-written HIP kernels for gfx950.  Tensors are torch device tensors; torch
supplies memory and streams only.
"""
from ._binding import (  # noqa: F401
    LIB_PATH,
    TVError,
    accept_workspace_bytes,
    attention_workspace_bytes,
    build_tree_mask,
    library,
    philox_uniforms,
    spec_accept,
    tree_attention,
)

__all__ = [
    "build_tree_mask",
    "tree_attention",
    "spec_accept",
    "philox_uniforms",
    "attention_workspace_bytes",
    "accept_workspace_bytes",
    "library",
    "TVError",
    "LIB_PATH",
]
