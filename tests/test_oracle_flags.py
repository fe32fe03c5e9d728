"""Pins of the oracle's near-boundary bookkeeping (CPU only).

The GPU walk computes in fp32/fp64 and the oracle in fp64, so a decision may
differ only where the oracle's uniform lies within 1e-5 of the boundary it is
compared with: the accept test r < min(1, R(x)/P(x)) of the survey explainer's
accept/reject phase (formal definition), and the inverse-CDF draw of the extra
token.  The parity tests excuse a mismatch only on sequences whose oracle walk
flagged such a decision, so the flags themselves are pinned here: each case
builds logits whose decision sits a chosen distance from its boundary,
computes that distance independently from the closed form of a two-outcome
softmax, and checks that the oracle flags it exactly when the distance is
below 1e-5 and reports it as the margin.
"""
import numpy as np
import pytest

import oracle

EPS = 1e-5
NEG = -1.0e4  # exp(NEG - max) underflows to exactly 0 in fp64


def _two_point(l0, l1):
    """P(outcome 0) of softmax([l0, l1]) in fp64, closed form."""
    return 1.0 / (1.0 + np.exp(np.float64(l1) - np.float64(l0)))


def _seed_where(pred, start=0):
    for s in range(start, start + 100000):
        if pred(s):
            return s
    raise AssertionError("no seed found")


def _logit_for(prob):
    """fp32 logit l1 with softmax([0, l1])[0] close to prob."""
    return np.float32(np.log(1.0 / prob - 1.0))


@pytest.mark.parametrize("delta", [5e-6, -5e-6, 2e-5, -2e-5, 0.3])
def test_accept_test_flag(delta):
    """Chain root -> node 1, V = 2, draft token 0; the ratio q0(0)/p1(0) is set
    to r + delta for the node's accept uniform r."""
    seq, node = 0, 1
    # r well inside (0.2, 0.6); the extra token's uniform far from every CDF
    # boundary of the rows it may be drawn from
    seed = _seed_where(lambda s: 0.2 < oracle.uniform(s, node, seq, 0) < 0.6
                       and 0.05 < oracle.uniform(s, node, seq, 1) < 0.45)
    r = oracle.uniform(seed, node, seq, 0)
    p1 = np.float32(0.8)
    lp = np.array([0.0, _logit_for(p1)], np.float32)
    p1_true = _two_point(lp[0], lp[1])
    target = (r + delta) * p1_true
    lq = np.array([0.0, _logit_for(target)], np.float32)
    a_true = min(1.0, _two_point(lq[0], lq[1]) / p1_true)
    d_true = abs(r - a_true)
    assert abs(d_true - abs(delta)) < 1e-7, "construction missed its window"
    q = np.stack([lq, np.zeros(2, np.float32)])          # leaf row 1 uniform: boundary at 0.5
    p = np.stack([np.zeros(2, np.float32), lp])
    out = oracle.spec_accept(q[None], p[None], np.array([[0, 0]], np.int32), np.array([[-1, 0]], np.int32),
                             seed=seed, temperature=1.0)
    accepted = r < a_true
    assert out["accept_len"][0] == int(accepted)
    assert out["flags"][0] == int(d_true < EPS)
    if abs(delta) < 0.01:  # the extra token's uniform lies >= 0.05 from its boundaries
        assert abs(out["margin"][0] - d_true) < 1e-9
    else:
        assert EPS < out["margin"][0] <= d_true


@pytest.mark.parametrize("delta", [5e-6, -5e-6, 2e-5, -2e-5])
def test_final_draw_flag_target_row(delta):
    """Root only (N = 1): the extra token is drawn from softmax(q0) with
    P(token 0) = u + delta for the draw's uniform u; the boundary between
    tokens 0 and 1 then lies |delta| from u."""
    seed = _seed_where(lambda s: 0.1 < oracle.uniform(s, 0, 0, 1) < 0.9)
    u = oracle.uniform(seed, 0, 0, 1)
    lq = np.array([0.0, _logit_for(u + delta)], np.float32)
    p0 = _two_point(lq[0], lq[1])
    d_true = abs(p0 - u)
    assert abs(d_true - abs(delta)) < 1e-7
    q = lq[None, None, :]
    out = oracle.spec_accept(q, q, np.zeros((1, 1), np.int32), np.array([[-1]], np.int32), seed=seed,
                             temperature=1.0)
    assert out["accept_len"][0] == 0
    assert out["out_tokens"][0, 0] == (0 if p0 > u else 1)
    assert out["flags"][0] == int(d_true < EPS)
    assert abs(out["margin"][0] - d_true) < 1e-9


@pytest.mark.parametrize("delta", [5e-6, -5e-6, 2e-5, -2e-5])
def test_final_draw_flag_residual(delta):
    """Chain root -> node 1, V = 3, draft token 1 with P1 = (0, 1, 0) and
    q0(1) = 0, so the node is always rejected and the extra token comes from
    the residual norm(max(0, q0 - P1)) = (q0(0), 0, q0(2)).  q0(0) is set to
    u + delta."""
    seed = _seed_where(lambda s: 0.1 < oracle.uniform(s, 0, 0, 1) < 0.9 and oracle.uniform(s, 1, 0, 0) > 1e-3)
    u = oracle.uniform(seed, 0, 0, 1)
    lq = np.array([0.0, NEG, _logit_for(u + delta)], np.float32)
    lp = np.array([NEG, 0.0, NEG], np.float32)
    r0 = _two_point(lq[0], lq[2])  # residual mass of token 0 (token 1 carries none)
    d_true = abs(r0 - u)
    assert abs(d_true - abs(delta)) < 1e-7
    q = np.stack([lq, np.zeros(3, np.float32)])
    p = np.stack([np.zeros(3, np.float32), lp])
    out = oracle.spec_accept(q[None], p[None], np.array([[0, 1]], np.int32), np.array([[-1, 0]], np.int32),
                             seed=seed, temperature=1.0)
    assert out["accept_len"][0] == 0
    assert out["out_tokens"][0, 0] == (0 if r0 > u else 2)
    assert out["flags"][0] == int(d_true < EPS)
    assert abs(out["margin"][0] - d_true) < 1e-9


def test_flags_count_every_near_decision():
    """A sequence with a near accept test and a near final draw counts two
    flags; a second sequence in the same batch with neither counts none."""
    seed = _seed_where(lambda s: 0.2 < oracle.uniform(s, 1, 0, 0) < 0.6 and 0.2 < oracle.uniform(s, 1, 0, 1) < 0.8
                       and 0.2 < oracle.uniform(s, 1, 1, 0) < 0.6 and 0.2 < oracle.uniform(s, 1, 1, 1) < 0.45)
    rows_q, rows_p = [], []
    for seq, near in ((0, True), (1, False)):
        r = oracle.uniform(seed, 1, seq, 0)
        u = oracle.uniform(seed, 1, seq, 1)
        lp = np.array([0.0, _logit_for(0.8)], np.float32)
        d = 4e-6 if near else 0.1
        lq0 = np.array([0.0, _logit_for((r + d) * _two_point(lp[0], lp[1]))], np.float32)  # accepted: r < a
        lq1 = np.array([0.0, _logit_for(u + (3e-6 if near else 0.05))], np.float32)      # leaf row
        rows_q.append(np.stack([lq0, lq1]))
        rows_p.append(np.stack([np.zeros(2, np.float32), lp]))
    q, p = np.stack(rows_q), np.stack(rows_p)
    par = np.array([[-1, 0], [-1, 0]], np.int32)
    out = oracle.spec_accept(q, p, np.zeros((2, 2), np.int32), par, seed=seed, temperature=1.0)
    assert out["accept_len"].tolist() == [1, 1]
    assert out["flags"].tolist() == [2, 0]
