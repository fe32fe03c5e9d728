"""Pins of the oracle's dynamic tree construction (CPU only).

EAGLE-3 explainer, integration with EAGLE-2: the draft tree is generated at
inference time.  The oracle grows it by cumulative draft probability (expand
the most probable frontier nodes with their top-k tokens) and keeps the most
probable nodes at the end.  Pinned by: brute-force enumeration of every path
when the expansion covers the whole vocabulary; the greedy chain for k = 1;
and, on random inputs, the structural facts the construction must keep (a
valid, ancestor-closed tree whose kept values dominate the dropped ones and
whose tokens are the top-k of their parent's row).
"""
import itertools

import numpy as np
import pytest

from oracle import dynamic_tree as dt


def _softmax(x, T):
    z = np.asarray(x, np.float64) / T
    e = np.exp(z - z.max())
    return e / e.sum()


def _table_draft(seed, V, scale=1.5):
    """A synthetic draft model: a fixed random logit row per path prefix."""
    cache = {}

    def fn(b, path):
        key = (b, tuple(path))
        if key not in cache:
            h = abs(hash((seed,) + key)) % (2 ** 32)
            cache[key] = np.random.default_rng(h).normal(scale=scale, size=V).astype(np.float32)
        return cache[key]
    return fn


@pytest.mark.parametrize("T", [1.0, 0.6])
def test_full_expansion_keeps_most_probable_paths(T):
    """topk = V and depth 2: every path of length 1 and 2 enters the pool, so
    the kept nodes must be the m - 1 most probable paths (products of softmax
    probabilities, enumerated here)."""
    V, m = 4, 9
    fn = _table_draft(3, V)
    (score, par, tok), (parent, tokens, index, nodes) = dt.build_tree(fn, 2, V, 2, V, m, T)
    for b in range(2):
        probs = {}
        for d in (1, 2):
            for path in itertools.product(range(V), repeat=d):
                pr = 1.0
                for i in range(d):
                    pr *= _softmax(fn(b, list(path[:i])), T)[path[i]]
                probs[path] = pr
        ranked = sorted(probs, key=lambda p: -probs[p])
        want = set(ranked[: m - 1])
        assert probs[ranked[m - 2]] > probs[ranked[m - 1]] * (1 + 1e-6)  # no near tie at the cut
        got = set()
        for i in range(1, nodes[b]):
            path, j = [], i
            while j > 0:
                path.append(int(tokens[b, j]))
                j = int(parent[b, j])
            got.add(tuple(path[::-1]))
        assert got == want


def test_topk_one_is_the_greedy_chain():
    V, depth = 50, 5
    fn = _table_draft(5, V)
    _, (parent, tokens, index, nodes) = dt.build_tree(fn, 3, V, depth, 1, depth + 1, 1.0)
    for b in range(3):
        assert nodes[b] == depth + 1
        assert parent[b].tolist() == [-1] + list(range(depth))
        path = []
        for i in range(1, depth + 1):
            path.append(int(np.argmax(fn(b, path))))
            assert tokens[b, i] == path[-1]


@pytest.mark.parametrize("topk,depth,m", [(3, 4, 12), (6, 5, 40), (10, 6, 60)])
def test_structure_on_random_drafts(topk, depth, m):
    V = 200
    fn = _table_draft(topk * 100 + depth, V, scale=2.0)
    B = 3
    (score, par, tok), (parent, tokens, index, nodes) = dt.build_tree(fn, B, V, depth, topk, m, 0.8)
    P = score.shape[1]
    for b in range(B):
        n = nodes[b]
        assert n == m
        assert parent[b, 0] == -1 and all(0 <= parent[b, i] < i for i in range(1, n))
        kept = set(index[b, :n].tolist())
        assert 0 in kept
        for s in kept - {0}:
            assert int(par[b, s]) in kept                       # ancestor-closed
            assert score[b, s] <= score[b, int(par[b, s])]       # values never increase
        dropped = [s for s in range(1, P) if s not in kept and par[b, s] >= 0]
        lo = min(score[b, s] for s in kept - {0})
        assert all(score[b, s] <= lo for s in dropped)
        # every pool child holds one of the top-k tokens of its parent's row
        for s in range(1, P):
            if par[b, s] < 0:
                continue
            row = fn(b, dt.path_tokens(par[b], tok[b], int(par[b, s])))
            kth = np.sort(row)[-topk]
            assert row[tok[b, s]] >= kth
