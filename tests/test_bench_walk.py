"""The benchmark's counts of the rows the sampling call reads -- the families
of the nodes its walk reaches, and the walk's row passes -- against a direct
re-walk on small random trees and against hand-worked cases."""
import numpy as np

import bench
import oracle
from workloads import Workload


def _small(B, N, V):
    return Workload("t", B=B, N=N, Hq=1, Hkv=1, D=128, L=0, V=V, sigma_q=2.0, sigma_n=1.0, temperatures=(1.0,),
                    tree="random")


def test_walk_bytes_hand_cases():
    w = _small(1, 4, 10)
    chain = np.array([[-1, 0, 1, 2]])
    # one accepted node, its only child rejected: one p pass plus node 1's q row
    assert bench.walk_bytes(w, chain, np.array([1]), np.array([[1, -1, -1, -1]]), 2) == 2 * 10 * 4
    # every node accepted: no pass; the bonus comes from leaf 3's q row in one member's slice
    assert bench.walk_bytes(w, chain, np.array([3]), np.array([[1, 2, 3, -1]]), 2) == 5 * 4
    star = np.array([[-1, 0, 0, 0]])
    # the third child accepted after two rejections at the root, then a leaf
    assert bench.walk_bytes(w, star, np.array([1]), np.array([[3, -1, -1, -1]]), 4) == 3 * 10 * 4 + 3 * 4
    # all three rejected: three p passes and the root's q row, the draw from the residual reads nothing
    assert bench.walk_bytes(w, star, np.array([0]), np.array([[-1, -1, -1, -1]]), 4) == 4 * 10 * 4


def test_family_bytes_hand_cases():
    w = _small(1, 4, 10)
    chain = np.array([[-1, 0, 1, 2]])
    # root family (q0, p1), node 1's (q1, p2): two nodes reached
    assert bench.family_bytes(w, chain, np.array([1]), np.array([[1, -1, -1, -1]])) == 4 * 10 * 4
    # every node reached: three families of two rows and the leaf's target row
    assert bench.family_bytes(w, chain, np.array([3]), np.array([[1, 2, 3, -1]])) == 7 * 10 * 4
    star = np.array([[-1, 0, 0, 0]])
    # the root's family has its three children's draft rows; leaf 3 adds its target row
    assert bench.family_bytes(w, star, np.array([1]), np.array([[3, -1, -1, -1]])) == 5 * 10 * 4
    # without replacement the children share the root's draft row
    assert bench.family_bytes(w, star, np.array([0]), np.array([[-1, -1, -1, -1]]), wor=True) == 2 * 10 * 4


def _rewalk(q, p, d, par, seed, T):
    """Rejections and q-row reads of the walk, taken step by step in fp64."""
    N, V = q.shape
    def sm(x):
        y = x.astype(np.float64) / T
        e = np.exp(y - y.max())
        return e / e.sum()
    u, rows, leaf, fam = 0, 0, False, 0
    R = sm(q[0])
    while True:
        kids = [c for c in range(u + 1, N) if par[c] == u]
        fam += 1 + len(kids)  # u reached: its target row and its children's draft rows
        if not kids:
            leaf = True
            break
        moved, rej = False, 0
        for c in kids:
            P = sm(p[c])
            x = d[c]
            a = 1.0 if P[x] == 0 else min(1.0, R[x] / P[x])
            if oracle.uniform(seed, c, 0, 0) < a:
                u, R, moved = c, sm(q[c]), True
                break
            rej += 1
            Wr = np.maximum(0.0, R - P)
            R = Wr / Wr.sum() if Wr.sum() > 0 else R
        rows += rej + (1 if rej else 0)
        if not moved:
            break
    return rows, leaf, fam


def test_walk_bytes_match_a_rewalk():
    rng = np.random.default_rng(11)
    V, N, team = 24, 12, 3
    w = _small(1, N, V)
    checked = 0
    for trial in range(60):
        par = np.array([-1] + [int(rng.integers(0, i)) for i in range(1, N)])
        q = rng.normal(0, 2.0, (N, V)).astype(np.float32)
        p = (q[np.maximum(par, 0)] + rng.normal(0, 1.0, (N, V))).astype(np.float32)
        p[0] = 0
        d = p.argmax(axis=1).astype(np.int32)
        d[0] = 0
        res = oracle.spec_accept(q[None], p[None], d[None], par[None].astype(np.int32), seed=trial, temperature=1.0)
        if res["flags"][0]:
            continue
        rows, leaf, fam = _rewalk(q, p, d, par, trial, 1.0)
        want = rows * V * 4 + ((V + team - 1) // team * 4 if leaf else 0)
        got = bench.walk_bytes(w, par[None], res["accept_len"], res["accepted_nodes"], team)
        assert got == want, (trial, got, want)
        assert bench.family_bytes(w, par[None], res["accept_len"], res["accepted_nodes"]) == fam * V * 4, trial
        checked += 1
    assert checked >= 50


def test_greedy_bytes_hand_cases():
    w = _small(1, 4, 10)
    star = np.array([[-1, 0, 0, 0]])
    # the root's argmax is token 5: only child 2 matches, so two target rows
    assert bench.greedy_bytes(w, star, np.array([[0, 1, 5, 7]]), np.array([[5, 0, 0, 0]])) == 2 * 10 * 4
    chain = np.array([[-1, 0, 1, 2]])
    # node 2 does not match, so node 3 below it is never reached although its token matches
    assert bench.greedy_bytes(w, chain, np.array([[0, 3, 9, 2]]), np.array([[3, 4, 2, 0]])) == 2 * 10 * 4
    # nothing matches: the root's row alone
    assert bench.greedy_bytes(w, chain, np.array([[0, 1, 1, 1]]), np.array([[0, 0, 0, 0]])) == 10 * 4


def test_greedy_bytes_reach_the_greedy_end():
    """The deepest node the count includes is as deep as the greedy path."""
    rng = np.random.default_rng(5)
    V, N = 6, 14
    w = _small(1, N, V)
    for trial in range(40):
        par = np.array([-1] + [int(rng.integers(0, i)) for i in range(1, N)])
        q = rng.normal(0, 1.0, (N, V)).astype(np.float32)
        am = q.argmax(axis=1)
        d = np.where(rng.random(N) < 0.6, am[np.maximum(par, 0)], rng.integers(0, V, N)).astype(np.int32)
        d[0] = 0
        res = oracle.spec_accept(q[None], None, d[None], par[None].astype(np.int32), greedy=True)
        depth = np.zeros(N, dtype=np.int64)
        match = np.zeros(N, dtype=bool)
        match[0] = True
        for i in range(1, N):
            depth[i] = depth[par[i]] + 1
            match[i] = match[par[i]] and d[i] == am[par[i]]
        assert int(res["accept_len"][0]) == int(depth[match].max()), trial
        assert bench.greedy_bytes(w, par[None], d[None], am[None]) == int(match.sum()) * V * 4
