"""Pins of the oracle's tree attention against an independent library routine
(torch's CPU scaled_dot_product_attention in fp64) and closed forms."""
import itertools

import numpy as np
import pytest
import torch

import oracle
from workloads import chain, random_tree


def _inputs(rng, B, N, Hq, Hkv, L, D):
    Q = rng.normal(size=(B, N, Hq, D))
    Kc = rng.normal(size=(B, Hkv, L, D))
    Vc = rng.normal(size=(B, Hkv, L, D))
    Kt = rng.normal(size=(B, N, Hkv, D))
    Vt = rng.normal(size=(B, N, Hkv, D))
    return Q, Kc, Vc, Kt, Vt


def _sdpa(q, k, v, mask):
    """q [n,D], k/v [m,D], mask bool [n,m] -> [n,D] via torch SDPA (fp64)."""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))[None, None]
    o = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=torch.from_numpy(mask))
    return o[0, 0].numpy()


@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (4, 2), (6, 1)])
def test_chain_equals_causal_attention(Hq, Hkv):
    rng = np.random.default_rng(Hq * 10 + Hkv)
    B, N, L, D = 2, 6, 9, 16
    Q, Kc, Vc, Kt, Vt = _inputs(rng, B, N, Hq, Hkv, L, D)
    par = np.tile(chain(N), (B, 1))
    out = oracle.tree_attention(Q, Kc, Vc, Kt, Vt, par)
    G = Hq // Hkv
    # causal over [cache ; drafts]: query i sits at position L + i
    mask = np.zeros((N, L + N), dtype=bool)
    for i in range(N):
        mask[i, : L + i + 1] = True
    for b in range(B):
        for h in range(Hq):
            k = np.concatenate([Kc[b, h // G], Kt[b, :, h // G]])
            v = np.concatenate([Vc[b, h // G], Vt[b, :, h // G]])
            ref = _sdpa(Q[b, :, h], k, v, mask)
            np.testing.assert_allclose(out[b, :, h], ref, rtol=0, atol=1e-12)


def _all_recursive_trees(n):
    for choice in itertools.product(*[range(i) for i in range(1, n)]):
        yield np.array([-1, *choice])


def _check_per_path(par, rng, L=5, D=8, Hq=2, Hkv=1):
    N = len(par)
    Q, Kc, Vc, Kt, Vt = _inputs(rng, 1, N, Hq, Hkv, L, D)
    out = oracle.tree_attention(Q, Kc, Vc, Kt, Vt, par[None])
    children = oracle.children_lists(par)
    leaves = [i for i in range(N) if not children[i]]
    G = Hq // Hkv
    for leaf in leaves:
        path, j = [], leaf
        while j != -1:
            path.append(j)
            j = par[j]
        path = path[::-1]
        P = len(path)
        mask = np.zeros((P, L + P), dtype=bool)
        for a in range(P):
            mask[a, : L + a + 1] = True
        for h in range(Hq):
            k = np.concatenate([Kc[0, h // G], Kt[0, path, h // G]])
            v = np.concatenate([Vc[0, h // G], Vt[0, path, h // G]])
            ref = _sdpa(Q[0, path, h], k, v, mask)
            np.testing.assert_allclose(out[0, path, h], ref, rtol=0, atol=1e-12)


def test_tree_equals_per_path_causal_exhaustive():
    rng = np.random.default_rng(5)
    count = 0
    for n in range(1, 7):
        for par in _all_recursive_trees(n):
            _check_per_path(par, rng)
            count += 1
    assert count == 1 + 1 + 2 + 6 + 24 + 120


def test_tree_equals_per_path_causal_random():
    rng = np.random.default_rng(6)
    for s in range(25):
        n = int(rng.integers(7, 17))
        _check_per_path(random_tree(n, 1 + s % 6, 100 + s), rng, L=int(rng.integers(0, 33)), Hq=4, Hkv=2)


def test_empty_cache_single_node_returns_root_value():
    rng = np.random.default_rng(1)
    Q, Kc, Vc, Kt, Vt = _inputs(rng, 3, 1, 4, 2, 0, 16)
    out = oracle.tree_attention(Q, Kc, Vc, Kt, Vt, np.full((3, 1), -1))
    for h in range(4):
        assert np.array_equal(out[:, 0, h], Vt[:, 0, h // 2])


def test_zero_query_gives_mean_of_visible_values():
    rng = np.random.default_rng(2)
    B, N, Hq, Hkv, L, D = 2, 12, 4, 2, 7, 8
    Q, Kc, Vc, Kt, Vt = _inputs(rng, B, N, Hq, Hkv, L, D)
    Q[:] = 0
    par = np.stack([random_tree(N, 4, 7), random_tree(N, 4, 8)])
    out = oracle.tree_attention(Q, Kc, Vc, Kt, Vt, par)
    for b in range(B):
        anc = oracle.ancestor_sets(par[b])
        for i in range(N):
            for h in range(Hq):
                g = h // 2
                rows = np.concatenate([Vc[b, g], Vt[b, sorted(anc[i]), g]])
                np.testing.assert_allclose(out[b, i, h], rows.mean(0), rtol=0, atol=1e-13)


def test_heads_subset_matches_full():
    rng = np.random.default_rng(3)
    Q, Kc, Vc, Kt, Vt = _inputs(rng, 2, 9, 4, 2, 11, 8)
    par = np.stack([random_tree(9, 3, 1), chain(9)])
    full = oracle.tree_attention(Q, Kc, Vc, Kt, Vt, par)
    part = oracle.tree_attention(Q, Kc, Vc, Kt, Vt, par, heads=[(1, 3), (0, 0)])
    assert np.array_equal(part[1, :, 3], full[1, :, 3]) and np.array_equal(part[0, :, 0], full[0, :, 0])
    assert np.isnan(part[0, :, 1]).all()


@pytest.mark.parametrize("n", [65, 100, 128])
def test_large_tree_equals_per_path_causal(n):
    """Trees past one 64-bit ancestor word: every root-to-leaf path against
    causal attention over [cache ; path]."""
    rng = np.random.default_rng(n)
    _check_per_path(random_tree(n, 9, 300 + n), rng, L=int(rng.integers(0, 20)), Hq=2, Hkv=1)


def test_ragged_batch_equals_per_path_causal():
    """Per-sequence node counts and cache lengths: each sequence's nodes see
    only its own cache prefix and path (per-path causal attention via torch
    SDPA); padding is never read."""
    rng = np.random.default_rng(12)
    B, N, Hq, Hkv, L, D = 4, 24, 4, 2, 30, 8
    Q, Kc, Vc, Kt, Vt = _inputs(rng, B, N, Hq, Hkv, L, D)
    nodes = np.array([24, 1, 9, 17])
    lens = np.array([30, 0, 13, 1])
    par = np.stack([random_tree(N, 6, 60 + b) for b in range(B)])
    for b in range(B):  # poison the padding
        par[b, nodes[b]:] = 1000
        Kc[b, :, lens[b]:] = np.nan
        Vc[b, :, lens[b]:] = np.nan
        Kt[b, nodes[b]:] = np.nan
        Vt[b, nodes[b]:] = np.nan
        Q[b, nodes[b]:] = np.nan
    out = oracle.tree_attention(Q, Kc, Vc, Kt, Vt, par, seq_nodes=nodes, seq_len=lens)
    G = Hq // Hkv
    for b in range(B):
        n, lb = nodes[b], lens[b]
        assert np.isnan(out[b, n:]).all() and np.isfinite(out[b, :n]).all()
        ch = oracle.children_lists(par[b, :n])
        for leaf in [i for i in range(n) if not ch[i]]:
            path, j = [], leaf
            while j != -1:
                path.append(j)
                j = par[b, j]
            path = path[::-1]
            P = len(path)
            mask = np.zeros((P, lb + P), dtype=bool)
            for a in range(P):
                mask[a, : lb + a + 1] = True
            for h in range(Hq):
                k = np.concatenate([Kc[b, h // G, :lb], Kt[b, path, h // G]])
                v = np.concatenate([Vc[b, h // G, :lb], Vt[b, path, h // G]])
                ref = _sdpa(Q[b, path, h], k, v, mask)
                np.testing.assert_allclose(out[b, path, h], ref, rtol=0, atol=1e-12)
