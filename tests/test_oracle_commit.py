"""Pins of the oracle's KV commit (CPU only).

After the walk, the root and the accepted path move from the tree's key/value
rows into the cache (EAGLE explainer, implementation notes: verifying a tree
needs KV memory beyond the committed context).  Pinned by a chain (the prefix
is copied), the empty path (only the root), failed walks and full caches (no
change), and by consistency with tree attention: each accepted node's tree
attention output equals plain attention over the committed cache up to its
own position (torch SDPA, fp64).
"""
import numpy as np
import torch

import oracle
from oracle.commit import BAD_TREE, NO_ROOM, commit_kv
from workloads import chain, random_tree


def _rand(rng, *shape):
    return rng.normal(size=shape)


def test_chain_copies_the_prefix():
    rng = np.random.default_rng(0)
    B, N, Hkv, Lcap, D = 3, 6, 2, 20, 8
    Kc, Vc = _rand(rng, B, Hkv, Lcap, D), _rand(rng, B, Hkv, Lcap, D)
    Kt, Vt = _rand(rng, B, N, Hkv, D), _rand(rng, B, N, Hkv, D)
    acc = np.array([5, 2, 0])
    nodes = np.tile(np.arange(1, N), (B, 1))
    nodes = np.concatenate([nodes, -np.ones((B, 1), int)], 1)
    for b in range(B):
        nodes[b, acc[b]:] = -1
    L = np.array([4, 0, 19])
    K2, V2, nl, st = commit_kv(Kc, Vc, Kt, Vt, acc, nodes, L)
    assert nl.tolist() == [10, 3, 20] and st.tolist() == [0, 0, 0]
    for b in range(B):
        a = acc[b]
        assert np.array_equal(K2[b, :, L[b]:L[b] + a + 1], Kt[b, :a + 1].transpose(1, 0, 2))
        assert np.array_equal(V2[b, :, L[b]:L[b] + a + 1], Vt[b, :a + 1].transpose(1, 0, 2))
        assert np.array_equal(K2[b, :, :L[b]], Kc[b, :, :L[b]])                 # earlier rows kept
        assert np.array_equal(K2[b, :, L[b] + a + 1:], Kc[b, :, L[b] + a + 1:])  # later rows untouched


def test_failed_walk_and_full_cache_commit_nothing():
    rng = np.random.default_rng(1)
    B, N, Hkv, Lcap, D = 2, 4, 1, 8, 4
    Kc, Vc = _rand(rng, B, Hkv, Lcap, D), _rand(rng, B, Hkv, Lcap, D)
    Kt, Vt = _rand(rng, B, N, Hkv, D), _rand(rng, B, N, Hkv, D)
    acc = np.array([-1, 3])
    nodes = np.array([[-1, -1, -1, -1], [1, 2, 3, -1]])
    K2, V2, nl, st = commit_kv(Kc, Vc, Kt, Vt, acc, nodes, np.array([2, 5]))
    assert st.tolist() == [BAD_TREE, NO_ROOM] and nl.tolist() == [2, 5]
    assert np.array_equal(K2, Kc) and np.array_equal(V2, Vc)


def test_commit_matches_tree_attention_of_the_accepted_path():
    rng = np.random.default_rng(2)
    B, N, Hq, Hkv, L, D = 2, 15, 4, 2, 9, 16
    Lcap = L + N
    Q = _rand(rng, B, N, Hq, D)
    Kc, Vc = np.zeros((B, Hkv, Lcap, D)), np.zeros((B, Hkv, Lcap, D))
    Kc[:, :, :L], Vc[:, :, :L] = _rand(rng, B, Hkv, L, D), _rand(rng, B, Hkv, L, D)
    Kt, Vt = _rand(rng, B, N, Hkv, D), _rand(rng, B, N, Hkv, D)
    par = np.stack([random_tree(N, 5, 70 + b) for b in range(B)])
    out = oracle.tree_attention(Q, Kc[:, :, :L], Vc[:, :, :L], Kt, Vt, par)
    # take a deepest node's path as the accepted one
    acc, nodes = [], np.full((B, N), -1)
    for b in range(B):
        _, depth, _ = oracle.tree_mask(par[b:b + 1])
        e = int(np.argmax(depth[0]))
        path, j = [], e
        while j != 0:
            path.append(j)
            j = par[b, j]
        path = path[::-1]
        acc.append(len(path))
        nodes[b, :len(path)] = path
    K2, V2, nl, st = commit_kv(Kc, Vc, Kt, Vt, np.array(acc), nodes, np.full(B, L))
    G = Hq // Hkv
    for b in range(B):
        for k, node in enumerate([0] + [int(x) for x in nodes[b, :acc[b]]]):
            n = L + k + 1  # cache rows visible to the node at position L + k
            for h in range(Hq):
                g = h // G
                t = lambda a: torch.from_numpy(np.ascontiguousarray(a))[None, None]
                ref = torch.nn.functional.scaled_dot_product_attention(
                    t(Q[b, node:node + 1, h]), t(K2[b, g, :n]), t(V2[b, g, :n]))[0, 0, 0].numpy()
                np.testing.assert_allclose(out[b, node, h], ref, rtol=0, atol=1e-12)
