"""KV commit after verification (oracle; test infrastructure only).

EAGLE explainer (0h-n0.github.io, paper-2401-10774), implementation notes:
verifying a tree needs KV-cache memory beyond the committed context, because
the target's forward pass writes keys and values for every tree node.
Speculative-decoding survey explainer (paper-2401-07851), formal definition,
accept/reject phase: the accepted drafts become part of the output.  Once the
walk has chosen its path, the keys and values of that path therefore move
from the tree's scratch rows into the cache, and the rest of the tree is
dropped.

Reading: the root (node 0) is the last committed token, whose keys and values
were computed by this verification pass and are not yet in the cache; the
extra token drawn by the walk gets its keys and values in the next pass.  So
sequence b with committed length L_b and accept_len a >= 0 appends a + 1
rows: the root, then its accepted nodes in path order, at cache positions
L_b .. L_b + a.  A sequence whose walk reported a failure (a < 0), or whose
new length would exceed the cache's capacity, commits nothing.
"""
from __future__ import annotations

import numpy as np

OK = 0
BAD_TREE = -3
NO_ROOM = -1


def commit_kv(K_cache, V_cache, K_tree, V_tree, accept_len, accepted_nodes, cache_len):
    """K_cache, V_cache [B,Hkv,Lcap,D]; K_tree, V_tree [B,N,Hkv,D];
    accept_len [B]; accepted_nodes [B,N]; cache_len [B].

    Returns (K_cache', V_cache', new_len [B], status [B]) with copies of the
    caches; inputs are not modified.
    """
    Kc = np.array(K_cache, copy=True)
    Vc = np.array(V_cache, copy=True)
    B, Hkv, Lcap, D = Kc.shape
    new_len = np.array(cache_len, dtype=np.int64).copy()
    status = np.zeros(B, dtype=np.int32)
    for b in range(B):
        a = int(accept_len[b])
        lb = int(cache_len[b])
        if a < 0:
            status[b] = BAD_TREE
            continue
        if lb < 0 or lb + a + 1 > Lcap:
            status[b] = NO_ROOM
            continue
        rows = [0] + [int(x) for x in accepted_nodes[b, :a]]
        for k, node in enumerate(rows):
            for g in range(Hkv):
                Kc[b, g, lb + k] = K_tree[b, node, g]
                Vc[b, g, lb + k] = V_tree[b, node, g]
        new_len[b] = lb + a + 1
    return Kc, Vc, new_len.astype(np.int32), status
