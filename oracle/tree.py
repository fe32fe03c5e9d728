"""Tree conventions and the tree attention mask (oracle; test infrastructure only).

EAGLE explainer (0h-n0.github.io, paper-2401-10774), section on parallel
verification with a static tree: the draft tokens form a tree, each
root-to-node path is one candidate continuation, and a tree attention mask
lets one target forward pass score every path.  A node therefore sees exactly
its own root-to-node path: its ancestors and itself.

Conventions (the pages fix none of them): node 0 is the root, i.e. the last
committed token, with parent -1; every other node's parent is an earlier
node; children of a node are taken in increasing index order.
"""
from __future__ import annotations

import numpy as np

BAD_TREE = -3


def tree_is_valid(parent_row) -> bool:
    p = [int(x) for x in parent_row]
    if len(p) < 1 or p[0] != -1:
        return False
    return all(0 <= p[i] < i for i in range(1, len(p)))


def ancestor_sets(parent_row):
    """List of Python sets: anc[i] = {i} plus every ancestor of i."""
    p = [int(x) for x in parent_row]
    out = []
    for i in range(len(p)):
        s, j = set(), i
        while j != -1:
            s.add(j)
            j = p[j]
        out.append(s)
    return out


def children_lists(parent_row):
    p = [int(x) for x in parent_row]
    ch = [[] for _ in p]
    for c in range(1, len(p)):
        ch[p[c]].append(c)
    return ch


def tree_mask(parent, seq_nodes=None):
    """parent: int array [B,N]; seq_nodes: optional int [B], the nodes of each
    sequence (the rest of its row is padding and is not read).

    Returns (anc, depth, status):
      anc    uint64 [B,N,W], W = ceil(N/64); bit j of word j//64 of anc[b,i]
             is set iff node j is i or an ancestor of i;
      depth  int32 [B,N], depth[root] = 0, depth[i] = depth[parent[i]] + 1;
      status int32 [B], 0 or BAD_TREE.  A sequence with an invalid parent
             array gets all-zero bitsets and depth -1 throughout, and so do
             the padding nodes of a ragged sequence.
    """
    parent = np.asarray(parent)
    B, N = parent.shape
    W = (N + 63) // 64
    anc = np.zeros((B, N, W), dtype=np.uint64)
    depth = np.full((B, N), -1, dtype=np.int32)
    status = np.zeros(B, dtype=np.int32)
    for b in range(B):
        n = N if seq_nodes is None else int(seq_nodes[b])
        if not 1 <= n <= N or not tree_is_valid(parent[b, :n]):
            status[b] = BAD_TREE
            continue
        for i, s in enumerate(ancestor_sets(parent[b, :n])):
            bits = 0
            for j in s:
                bits |= 1 << j
            for w in range(W):
                anc[b, i, w] = np.uint64((bits >> (64 * w)) & 0xFFFFFFFFFFFFFFFF)
            depth[b, i] = len(s) - 1
    return anc, depth, status
