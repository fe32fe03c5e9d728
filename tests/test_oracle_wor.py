"""Pins of the oracle's walk for siblings drawn without replacement, and of
ragged batches (CPU only).

EAGLE explainer, static-tree verification: the children of a node are several
candidate tokens for the same next position, taken from the draft's
distribution at that node.  Drawn without replacement, child k follows the
node's draft row with the tokens of children 1..k-1 removed and the rest
renormalised; the walk tests it against exactly that distribution, and the
survey explainer's accept/reject rule (formal definition) then keeps the
emitted tokens distributed as the target.  Pinned by the lossless chi-square
over 10^6 Philox seeds, a hand-worked two-token case, two planted mistakes
that must fail, and the reduction of a chain to the plain rule.
"""
import os

import numpy as np
import pytest

import oracle
from workloads import chain, random_tree

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
CHI2_7DOF_P01 = 18.475
TREE8 = np.array([-1, 0, 0, 0, 1, 1, 2, 4])


def _softmax(x, T=1.0):
    z = np.asarray(x, np.float64) / T
    e = np.exp(z - z.max())
    return e / e.sum()


def _chi2(counts, probs):
    e = counts.sum() * np.asarray(probs)
    return float(((counts - e) ** 2 / e).sum())


def _logits(seed, N, V):
    rng = np.random.default_rng(seed)
    return rng.normal(size=(N, V)).astype(np.float32), rng.normal(size=(N, V)).astype(np.float32)


@pytest.mark.parametrize("T", [1.0, 0.7])
def test_wor_lossless_first_token_chi_square(T):
    q, p = _logits(7, 8, 8)
    r = oracle.lossless_trials(q, p, TREE8, T, seed0=0, ntrials=1_000_000, draft_mode=2)
    # the drafts really are distinct among siblings
    d = r["drafts"]
    assert (d[:, 1] != d[:, 2]).all() and (d[:, 1] != d[:, 3]).all() and (d[:, 2] != d[:, 3]).all()
    assert (d[:, 4] != d[:, 5]).all()
    counts = np.bincount(r["tokens"][:, 0], minlength=8)
    assert _chi2(counts, _softmax(q[0], T)) < CHI2_7DOF_P01


def test_wor_negative_control_shared_row_without_renormalising_fails():
    q, p = _logits(7, 8, 8)
    r = oracle.lossless_trials(q, p, TREE8, 1.0, seed0=0, ntrials=1_000_000, variant=2, draft_mode=2)
    counts = np.bincount(r["tokens"][:, 0], minlength=8)
    assert _chi2(counts, _softmax(q[0])) > 1000.0


def test_wor_negative_control_drafts_with_replacement_fail():
    q, p = _logits(7, 8, 8)
    r = oracle.lossless_trials(q, p, TREE8, 1.0, seed0=0, ntrials=1_000_000, draft_mode=3)
    counts = np.bincount(r["tokens"][:, 0], minlength=8)
    assert _chi2(counts, _softmax(q[0])) > 1000.0


def test_wor_two_token_worked_case():
    vals = {l.split()[0]: [float(x) for x in l.split()[1:]] for l in open(os.path.join(GOLDEN, "wor_two_siblings.txt"))
            if l.strip() and not l.startswith("#")}
    par = np.array([-1, 0, 0])
    q = np.log(np.array([vals["q"], [1.0, 1.0], [1.0, 1.0]], np.float32))
    p = np.log(np.array([vals["p"], [1.0, 1.0], [1.0, 1.0]], np.float32))
    n = 400_000
    r = oracle.lossless_trials(q, p, par, 1.0, seed0=0, ntrials=n, draft_mode=2)
    for key, got in (("emit0", (r["tokens"][:, 0] == 0).mean()),
                     ("first_child_kept", (r["accepted"][:, 0] == 1).mean()),
                     ("second_child_kept", (r["accepted"][:, 0] == 2).mean())):
        e = vals[key][0]
        assert abs(got - e) < 5 * np.sqrt(e * (1 - e) / n), key


@pytest.mark.parametrize("T", [1.0, 0.8])
def test_wor_chain_reduces_to_the_plain_rule(T):
    """With one child per node there is nothing to remove: the walk with the
    draft row at the parent equals the plain walk with that row at the child."""
    rng = np.random.default_rng(3)
    B, N, V = 8, 7, 40
    q = rng.normal(scale=2, size=(B, N, V)).astype(np.float32)
    p_child = (q[:, np.r_[0, 0:N - 1]] + rng.normal(size=(B, N, V))).astype(np.float32)
    p_child[:, 0] = 0.0
    p_parent = np.zeros_like(p_child)
    p_parent[:, :N - 1] = p_child[:, 1:]
    draft = p_child.argmax(-1).astype(np.int32)
    par = np.tile(chain(N), (B, 1))
    for seed in range(20):
        a = oracle.spec_accept(q, p_child, draft, par, seed=seed, temperature=T)
        b = oracle.spec_accept(q, p_parent, draft, par, seed=seed, temperature=T, wor=True)
        for k in ("accept_len", "accepted_nodes", "out_tokens"):
            assert np.array_equal(a[k], b[k])


def test_ragged_batch_equals_each_sequence_alone():
    """A ragged batch (per-sequence node counts, stride N) gives every sequence
    what it gets alone with its own node count and Philox sequence number."""
    rng = np.random.default_rng(9)
    B, N, V = 6, 20, 64
    nodes = np.array([20, 1, 7, 13, 2, 20], np.int32)
    q = rng.normal(scale=2, size=(B, N, V)).astype(np.float32)
    p = (q + rng.normal(size=(B, N, V))).astype(np.float32)
    draft = p.argmax(-1).astype(np.int32)
    par = np.stack([random_tree(N, 5, 40 + b) for b in range(B)])
    # padding past each sequence's nodes is garbage that must not be read
    for b in range(B):
        par[b, nodes[b]:] = 99
        draft[b, nodes[b]:] = -5
    for wor in (False, True):
        for greedy in (False, True):
            r = oracle.spec_accept(q, p, draft, par, seed=4, temperature=0.9, greedy=greedy, seq_nodes=nodes, wor=wor)
            for b in range(B):
                n = nodes[b]
                one = oracle.spec_accept(q[b:b + 1, :n], p[b:b + 1, :n], draft[b:b + 1, :n], par[b:b + 1, :n], seed=4,
                                         temperature=0.9, greedy=greedy, wor=wor, seq_offset=b)
                assert r["accept_len"][b] == one["accept_len"][0]
                assert np.array_equal(r["accepted_nodes"][b, :n], one["accepted_nodes"][0])
                assert np.array_equal(r["out_tokens"][b, :n], one["out_tokens"][0])
                assert (r["out_tokens"][b, n:] == -1).all() and (r["accepted_nodes"][b, n:] == -1).all()
                assert r["flags"][b] == one["flags"][0]
