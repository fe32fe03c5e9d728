"""Pins of the oracle's accept/reject walk (CPU only).

Greedy mode is checked by brute-force path enumeration; sampling mode by the
lossless property of the speculative-decoding survey explainer (formal
definition, accept/reject phase: the emitted tokens follow the target
distribution exactly), by closed-form acceptance rates and by the residual
distribution.  Negative controls plant mistakes in the oracle (variant 1) or
break the guarantee's precondition (argmax drafts) and must fail.
"""
import os

import numpy as np
import pytest

import oracle
from workloads import chain, random_tree

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
CHI2_7DOF_P01 = 18.475   # chi-square, 7 dof, p = 0.01
CHI2_7DOF_P001 = 24.322  # chi-square, 7 dof, p = 0.001
TREE8 = np.array([-1, 0, 0, 0, 1, 1, 2, 4])


def _softmax(x, T=1.0):
    z = np.asarray(x, np.float64) / T
    e = np.exp(z - z.max())
    return e / e.sum()


def _chi2(counts, probs):
    n = counts.sum()
    e = n * np.asarray(probs)
    keep = e > 0
    assert counts[~keep].sum() == 0
    return float((((counts - e) ** 2)[keep] / e[keep]).sum())


def _logits(seed, N, V):
    rng = np.random.default_rng(seed)
    return rng.normal(size=(N, V)).astype(np.float32), rng.normal(size=(N, V)).astype(np.float32)


# ---------------------------------------------------------------- greedy ---
def _brute_greedy(q, draft, par):
    N = len(par)
    a = [int(np.argmax(q[u])) for u in range(N)]  # numpy argmax: first maximum
    best = None
    for e in range(N):
        path, j = [], e
        while j != 0:
            path.append(j)
            j = par[j]
        path = path[::-1]
        if all(draft[c] == a[par[c]] for c in path):
            if best is None or len(path) > len(best):
                best = path
    e = best[-1] if best else 0
    return best, [int(draft[c]) for c in best] + [a[e]]


def test_greedy_matches_path_enumeration():
    rng = np.random.default_rng(0)
    for trial in range(300):
        N = int(rng.integers(1, 20))
        V = int(rng.integers(2, 5))
        par = random_tree(N, int(rng.integers(1, 7)), trial)
        q = rng.integers(0, 3, size=(N, V)).astype(np.float32)  # many ties
        draft = rng.integers(0, V, size=N).astype(np.int32)
        r = oracle.spec_accept(q[None], None, draft[None], par[None], greedy=True)
        path, toks = _brute_greedy(q, draft, par)
        n = len(path)
        assert r["accept_len"][0] == n
        assert list(r["accepted_nodes"][0, :n]) == path and (r["accepted_nodes"][0, n:] == -1).all()
        assert list(r["out_tokens"][0, : n + 1]) == toks and (r["out_tokens"][0, n + 1:] == -1).all()


def test_greedy_chain_counts_leading_matches():
    rng = np.random.default_rng(1)
    V = 3
    for _ in range(200):
        N = int(rng.integers(2, 9))
        q = rng.normal(size=(N, V)).astype(np.float32)
        a = q.argmax(1)
        draft = rng.integers(0, V, size=N).astype(np.int32)
        k = 0
        while k + 1 < N and draft[k + 1] == a[k]:
            k += 1
        r = oracle.spec_accept(q[None], None, draft[None], chain(N)[None], greedy=True)
        assert r["accept_len"][0] == k
        assert r["out_tokens"][0, k] == a[k]


def test_greedy_no_match_emits_root_argmax():
    q = np.array([[0.0, 3.0, 1.0], [5.0, 0.0, 0.0], [0.0, 0.0, 9.0]], np.float32)
    draft = np.array([0, 0, 2], np.int32)  # root argmax is 1; neither child drafted 1
    r = oracle.spec_accept(q[None], None, draft[None], np.array([[-1, 0, 0]]), greedy=True)
    assert r["accept_len"][0] == 0 and r["out_tokens"][0, 0] == 1 and (r["accepted_nodes"][0] == -1).all()


def test_greedy_argmax_ties_take_smallest_token():
    q = np.array([[2.0, 7.0, 7.0, 1.0]], np.float32)
    r = oracle.spec_accept(q[None], None, np.zeros((1, 1), np.int32), np.array([[-1]]), greedy=True)
    assert r["out_tokens"][0, 0] == 1


# -------------------------------------------------------------- sampling ---
@pytest.mark.parametrize("T", [1.0, 0.7])
def test_lossless_first_token_chi_square(T):
    q, p = _logits(7, 8, 8)
    r = oracle.lossless_trials(q, p, TREE8, T, seed0=0, ntrials=1_000_000)
    counts = np.bincount(r["tokens"][:, 0], minlength=8)
    assert _chi2(counts, _softmax(q[0], T)) < CHI2_7DOF_P01


@pytest.mark.parametrize("T", [1.0, 0.7])
def test_lossless_next_token_after_accepting_a_child(T):
    """Given that depth-1 node c was accepted, the next emitted token must follow
    the target row of c (the walk restarts at c)."""
    q, p = _logits(7, 8, 8)
    r = oracle.lossless_trials(q, p, TREE8, T, seed0=0, ntrials=1_000_000)
    for c in (1, 2, 3):
        sel = r["accepted"][:, 0] == c
        assert sel.sum() > 20000
        counts = np.bincount(r["tokens"][sel, 1], minlength=8)
        assert _chi2(counts, _softmax(q[c], T)) < CHI2_7DOF_P001


@pytest.mark.parametrize("par", [chain(5), np.array([-1, 0, 0, 0, 0, 0])], ids=["chain", "star"])
def test_lossless_chain_and_star(par):
    q, p = _logits(9, len(par), 8)
    r = oracle.lossless_trials(q, p, par, 1.0, seed0=5_000_000, ntrials=400_000)
    counts = np.bincount(r["tokens"][:, 0], minlength=8)
    assert _chi2(counts, _softmax(q[0])) < CHI2_7DOF_P01


def test_negative_control_unupdated_sibling_target_fails():
    q, p = _logits(7, 8, 8)
    r = oracle.lossless_trials(q, p, TREE8, 1.0, seed0=0, ntrials=1_000_000, variant=1)
    counts = np.bincount(r["tokens"][:, 0], minlength=8)
    assert _chi2(counts, _softmax(q[0])) > 1000.0


def test_negative_control_argmax_drafts_fail():
    q, p = _logits(7, 8, 8)
    r = oracle.lossless_trials(q, p, TREE8, 1.0, seed0=0, ntrials=1_000_000, draft_mode=1)
    counts = np.bincount(r["tokens"][:, 0], minlength=8)
    assert _chi2(counts, _softmax(q[0])) > 1000.0


def test_acceptance_rate_closed_forms():
    q, p = _logits(3, 2, 6)
    n = 400_000
    # drafts sampled from p: P(accept) = sum_v min(p(v), q(v))
    r = oracle.lossless_trials(q, p, chain(2), 1.0, seed0=0, ntrials=n)
    pa = np.minimum(_softmax(p[1]), _softmax(q[0])).sum()
    assert abs(r["accept_len"].mean() - pa) < 5 * np.sqrt(pa * (1 - pa) / n)
    # argmax draft x: P(accept) = min(1, q(x)/p(x))
    r = oracle.lossless_trials(q, p, chain(2), 1.0, seed0=0, ntrials=n, draft_mode=1)
    x = int(np.argmax(p[1]))
    pa = min(1.0, _softmax(q[0])[x] / _softmax(p[1])[x])
    assert abs(r["accept_len"].mean() - pa) < 5 * np.sqrt(pa * (1 - pa) / n) + 1e-12


def test_residual_distribution_after_rejection():
    q, p = _logits(4, 2, 8)
    r = oracle.lossless_trials(q, p, chain(2), 1.0, seed0=0, ntrials=600_000)
    rej = r["accept_len"] == 0
    res = np.maximum(0.0, _softmax(q[0]) - _softmax(p[1]))
    res /= res.sum()
    counts = np.bincount(r["tokens"][rej, 0], minlength=8)
    support = res > 0
    assert counts[~support].sum() == 0
    assert _chi2(counts, res) < 24.322  # at most 7 dof


def test_two_token_worked_case():
    vals = {l.split()[0]: [float(x) for x in l.split()[1:]] for l in open(os.path.join(GOLDEN, "rule_two_token.txt"))
            if l.strip() and not l.startswith("#")}
    p = np.log(np.array([[1.0, 1.0], vals["p"]], np.float32))
    q = np.log(np.array([vals["q"], [1.0, 1.0]], np.float32))
    n = 400_000
    for mode, key in ((0, "emit0_sampled_draft"), (1, "emit0_argmax_draft")):
        r = oracle.lossless_trials(q, p, chain(2), 1.0, seed0=0, ntrials=n, draft_mode=mode)
        f = (r["tokens"][:, 0] == 0).mean()
        e = vals[key][0]
        assert abs(f - e) < 5 * np.sqrt(e * (1 - e) / n)


def test_bonus_token_comes_from_leaf_row():
    # q rows make every draft certain to be accepted: the emitted extra token
    # must then follow the leaf's own row.
    V, N = 4, 3
    big = 30.0
    q = np.zeros((N, V), np.float32)
    p = np.zeros((N, V), np.float32)
    q[0, 2] = big; p[1, 2] = big       # node 1 drafts token 2 with q/p ~ 1
    q[1, 1] = big; p[2, 1] = big       # node 2 drafts token 1
    q[2] = [0.0, 1.0, 2.0, 3.0]        # leaf row
    draft = np.array([[0, 2, 1]] * 2000, np.int32)
    par = np.tile(chain(N), (2000, 1))
    qs = np.tile(q, (2000, 1, 1)); ps = np.tile(p, (2000, 1, 1))
    r = oracle.spec_accept(qs, ps, draft, par, seed=11, temperature=1.0)
    assert (r["accept_len"] == 2).all()
    counts = np.bincount(r["out_tokens"][:, 2], minlength=V)
    assert _chi2(counts, _softmax(q[2])) < 16.27  # 3 dof, p = 0.001


def test_determinism_and_flags():
    rng = np.random.default_rng(5)
    B, N, V = 6, 12, 50
    q = rng.normal(scale=3, size=(B, N, V)).astype(np.float32)
    p = q + rng.normal(size=(B, N, V)).astype(np.float32)
    draft = p.argmax(-1).astype(np.int32)
    par = np.stack([random_tree(N, 4, s) for s in range(B)])
    r1 = oracle.spec_accept(q, p, draft, par, seed=3, temperature=0.7)
    r2 = oracle.spec_accept(q, p, draft, par, seed=3, temperature=0.7)
    for k in ("accept_len", "accepted_nodes", "out_tokens", "flags"):
        assert np.array_equal(r1[k], r2[k])
    assert (r1["margin"] > 0).all()
    r3 = oracle.spec_accept(q, p, draft, par, seed=4, temperature=0.7)
    assert not np.array_equal(r1["out_tokens"], r3["out_tokens"])


def test_rejects_bad_inputs():
    q = np.zeros((1, 3, 4), np.float32)
    with pytest.raises(ValueError):
        oracle.spec_accept(q, q, np.zeros((1, 3), np.int32), np.array([[-1, 0, 2]]))
    with pytest.raises(ValueError):
        oracle.spec_accept(q, q, np.array([[0, 9, 0]], np.int32), np.array([[-1, 0, 0]]))
    with pytest.raises(ValueError):
        oracle.spec_accept(q, q, np.zeros((1, 3), np.int32), np.array([[-1, 0, 0]]), temperature=0.0)
