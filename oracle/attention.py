"""Ancestor-masked tree attention in fp64 (oracle; test infrastructure only).

EAGLE explainer (0h-n0.github.io, paper-2401-10774), section on parallel
verification with a static tree: one target forward pass with a tree
attention mask scores every root-to-leaf path.  In that pass draft node i
attends to the committed context (the KV cache) and to the tree positions on
its own root-to-node path -- its ancestors and itself -- and nothing else.
The speculative-decoding survey explainer (paper-2401-07851), formal
definition, verification phase, states the same for a chain: the target
distribution at draft position i is conditioned on the context and the drafts
before it.

Readings: scale 1/sqrt(D) unless given; query head h reads KV head h // G with
G = Hq / Hkv (grouped-query attention); no softcap, ALiBi or dropout; rotary
position encodings are applied by the caller beforehand.
"""
from __future__ import annotations

import numpy as np

from .tree import ancestor_sets


def tree_attention(Q, K_cache, V_cache, K_tree, V_tree, parent, scale=None, heads=None, seq_nodes=None,
                   seq_len=None):
    """All tensors float64 numpy arrays.

    Q [B,N,Hq,D]; K_cache, V_cache [B,Hkv,L,D]; K_tree, V_tree [B,N,Hkv,D];
    parent [B,N].  Returns out [B,N,Hq,D] float64.  ``heads`` optionally
    restricts the work to a list of (b, h) pairs (other entries stay NaN).
    Ragged batches: ``seq_nodes[b]`` nodes and ``seq_len[b]`` committed cache
    entries of sequence b are real (the rest is padding, never read; outputs
    of padding nodes stay NaN).
    """
    Q = np.asarray(Q, dtype=np.float64)
    B, N, Hq, D = Q.shape
    Hkv, L = K_cache.shape[1], K_cache.shape[2]
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out = np.full((B, N, Hq, D), np.nan)
    pairs = heads if heads is not None else [(b, h) for b in range(B) for h in range(Hq)]
    visible_cache = {}
    for b, h in pairs:
        g = h // G
        n = N if seq_nodes is None else int(seq_nodes[b])
        lb = L if seq_len is None else int(seq_len[b])
        if b not in visible_cache:
            anc = ancestor_sets(parent[b, :n])
            vis = np.zeros((n, lb + n), dtype=bool)
            vis[:, :lb] = True
            for i in range(n):
                for j in anc[i]:
                    vis[i, lb + j] = True
            visible_cache[b] = vis
        vis = visible_cache[b]
        keys = np.concatenate([np.asarray(K_cache[b, g, :lb], np.float64),
                               np.asarray(K_tree[b, :n, g], np.float64)], 0)
        vals = np.concatenate([np.asarray(V_cache[b, g, :lb], np.float64),
                               np.asarray(V_tree[b, :n, g], np.float64)], 0)
        s = scale * (Q[b, :n, h, :] @ keys.T)
        s = np.where(vis, s, -np.inf)
        s = s - s.max(axis=1, keepdims=True)
        e = np.exp(s)
        P = e / e.sum(axis=1, keepdims=True)
        out[b, :n, h, :] = P @ vals
    return out
