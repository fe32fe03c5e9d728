"""CPU oracle for token-tree verification -- TEST INFRASTRUCTURE ONLY.

A plain, slow, fp64 reference of what the HIP library computes:

* ``tree_mask``      -- ancestor-or-self bitsets and depths of a draft tree;
* ``tree_attention`` -- ancestor-masked attention over committed KV + tree KV;
* ``spec_accept``    -- greedy and speculative-sampling accept/reject walk
  (plain C, ``oracle/csrc/accept_oracle.c``), with its own Philox-4x32-10;
  siblings drawn independently or without replacement; ragged batches;
* ``commit_kv``      -- the accepted path's keys and values appended to the cache;
* ``dynamic_tree``   -- draft-tree construction by cumulative draft probability
  (expansion steps and the final re-ranking).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with
``token_tree_verification_amd`` and never imports it; the product path must
not call into it.
"""
from .tree import tree_mask, ancestor_sets, children_lists  # noqa: F401
from .attention import tree_attention  # noqa: F401
from .commit import commit_kv  # noqa: F401
from . import dynamic_tree  # noqa: F401
from .accept import (  # noqa: F401
    spec_accept,
    philox4x32_10,
    uniform,
    uniforms,
    lossless_trials,
    build_liboracle,
)
