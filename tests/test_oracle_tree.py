"""Pins of the oracle's tree mask (CPU only)."""
import os

import numpy as np
import pytest

import oracle
from workloads import chain, random_tree, static_tree_60

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bits(word):
    return {j for j in range(64) if (int(word) >> j) & 1}


def test_hand_worked_tree():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "tree_small.txt")) if l.strip() and not l.startswith("#")]
    parent = np.array([[int(r[1]) for r in rows]])
    anc, depth, status = oracle.tree_mask(parent)
    assert status[0] == 0
    for r in rows:
        i = int(r[0])
        assert depth[0, i] == int(r[2])
        assert _bits(anc[0, i, 0]) == {int(x) for x in r[3].split(",")}


def test_transitive_closure_matches():
    # anc(i) is the reflexive-transitive closure of the child->parent relation,
    # computed here by repeated boolean matrix products.
    for seed in range(20):
        n = 1 + seed * 3
        par = random_tree(n, 8, seed)
        A = np.zeros((n, n), dtype=np.int64)
        for i in range(1, n):
            A[i, par[i]] = 1
        R = np.eye(n, dtype=np.int64)
        for _ in range(n):
            R = np.minimum(1, R + R @ A)
        anc, depth, status = oracle.tree_mask(par[None])
        for i in range(n):
            want = set(np.nonzero(R[i])[0].tolist())
            got = set()
            for w in range(anc.shape[2]):
                got |= {64 * w + j for j in _bits(anc[0, i, w])}
            assert got == want
            assert depth[0, i] == len(want) - 1


def test_popcount_is_depth_plus_one_and_contains_root():
    par = np.stack([random_tree(64, 8, s) for s in range(8)])
    anc, depth, status = oracle.tree_mask(par)
    assert (status == 0).all()
    for b in range(8):
        for i in range(64):
            s = _bits(anc[b, i, 0])
            assert len(s) == depth[b, i] + 1 and 0 in s and i in s and max(s) == i


def test_chain_is_lower_triangular_and_star():
    anc, depth, _ = oracle.tree_mask(chain(10)[None])
    for i in range(10):
        assert _bits(anc[0, i, 0]) == set(range(i + 1))
    star = np.array([[-1] + [0] * 9])
    anc, depth, _ = oracle.tree_mask(star)
    for i in range(1, 10):
        assert _bits(anc[0, i, 0]) == {0, i} and depth[0, i] == 1


def test_multiword_for_large_trees():
    par = chain(130)[None]
    anc, depth, _ = oracle.tree_mask(par)
    assert anc.shape == (1, 130, 3)
    assert depth[0, 129] == 129
    assert int(anc[0, 129, 2]) == (1 << 2) - 1 and int(anc[0, 129, 0]) == 2 ** 64 - 1


@pytest.mark.parametrize("bad", [
    [0, 0, 1],        # root must have parent -1
    [-1, 1, 1],       # parent must be an earlier node
    [-1, 0, -1],      # only the root is parentless
    [-1, 0, -2],
    [-1, 0, 5],
])
def test_invalid_trees_rejected(bad):
    par = np.array([bad, [-1, 0, 0]])
    anc, depth, status = oracle.tree_mask(par)
    assert status[0] == oracle.tree.BAD_TREE and status[1] == 0
    assert (anc[0] == 0).all() and (depth[0] == -1).all()


def test_static_tree_matches_page():
    vals = dict(l.split() for l in open(os.path.join(GOLDEN, "eagle_static_tree.txt")) if l.strip() and not l.startswith("#"))
    par = static_tree_60()
    _, depth, status = oracle.tree_mask(par[None])
    assert status[0] == 0
    assert len(par) == int(vals["size"])
    assert depth.max() == int(vals["depth"])
    widths = np.bincount(depth[0])
    assert widths.max() == int(vals["max_level_width"])


def test_ragged_sequences_ignore_their_padding():
    """Per-sequence node counts: the first n_b nodes get the mask of the
    truncated tree (by pointer chasing here), the padding gets 0 / -1, and an
    invalid parent inside the padding does not invalidate the sequence."""
    N = 70
    par = np.stack([random_tree(N, 8, 5), chain(N), random_tree(N, 3, 6)])
    nodes = np.array([70, 1, 66])
    par[1, 1:] = 55  # all padding, invalid if it were read
    anc, depth, status = oracle.tree_mask(par, seq_nodes=nodes)
    assert status.tolist() == [0, 0, 0]
    for b in range(3):
        n = nodes[b]
        for i in range(N):
            got = set()
            for w in range(anc.shape[2]):
                got |= {64 * w + j for j in _bits(anc[b, i, w])}
            if i >= n:
                assert not got and depth[b, i] == -1
                continue
            want, j = set(), i
            while j != -1:
                want.add(j)
                j = int(par[b, j])
            assert got == want and depth[b, i] == len(want) - 1
    _, _, st = oracle.tree_mask(par, seq_nodes=np.array([70, 2, 66]))
    assert st.tolist() == [0, oracle.tree.BAD_TREE, 0]
