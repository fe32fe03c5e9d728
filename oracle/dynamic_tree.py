"""Dynamic draft-tree construction (oracle; test infrastructure only).

EAGLE-3 explainer (0h-n0.github.io, paper-2501-05370), section on the
integration with EAGLE-2, and the EAGLE explainer's conclusion
(paper-2401-10774): EAGLE-2 replaces the fixed tree by a dynamic one whose
shape is generated at inference time from the draft.  The pages name the
method but give no steps, so this follows the plainest reading that the rest
supports (each step is listed in the design notes):

* a node's value is the draft's probability of its whole path from the root,
  kept as a cumulative log-probability: value(child) = value(parent) +
  log softmax(draft logits at the parent / T)[token];
* expansion: the tree grows one depth at a time; the nodes of the current
  frontier each take their top-k tokens (largest draft logits; ties to the
  smaller token id) as children, and the k children with the largest values
  among all new candidates form the next frontier;
* re-ranking: when the last depth is expanded, the root and the m - 1 nodes
  with the largest values are kept (ties to the earlier pool slot).  A
  child's value never exceeds its parent's, so the kept set is closed under
  ancestors; it is renumbered in pool order, which keeps parents before
  children.

Values are stored as binary32, as the kernels store them: each addition is
done in fp64 from the stored parent value and rounded once, so both sides
compare the same numbers (the fp64 log-softmax here is exact to ~1e-16).
"""
from __future__ import annotations

import numpy as np


def log_softmax_row(x, T):
    z = np.asarray(x, np.float64) / float(np.float32(T))
    m = z.max()
    return z - m - np.log(np.exp(z - m).sum())


def top_tokens(x, k):
    """The k largest entries of x (ties to the smaller index), largest first."""
    x = np.asarray(x)
    order = sorted(range(len(x)), key=lambda v: (-float(x[v]), v))
    return order[:k]


def expand(draft_logits, frontier, pool_score, pool_parent, pool_token, pool_base, topk, n_next, temperature,
           root_token=None):
    """One expansion step, in place on the pool arrays.

    draft_logits float32 [B,F,V] (row f: the draft's logits at frontier node
    f); frontier int [B,F] pool slots (-1: empty), or None to expand the
    root (slot 0, which this call then initialises with value 0, parent -1
    and ``root_token[b]``).  Candidates of frontier row f go to pool slots
    pool_base + f*topk + j.  Returns the next frontier int32 [B,n_next]
    (-1 where fewer valid candidates exist).
    """
    B, F, V = draft_logits.shape
    nxt = np.full((B, n_next), -1, np.int32)
    for b in range(B):
        if frontier is None:
            pool_score[b, 0] = np.float32(0.0)
            pool_parent[b, 0] = -1
            pool_token[b, 0] = -1 if root_token is None else int(root_token[b])
            rows = [(0, 0)]
        else:
            rows = [(f, int(frontier[b, f])) for f in range(F)]
        cands = []
        for f, slot in rows:
            base = pool_base + f * topk
            if slot < 0:
                for j in range(topk):
                    pool_score[b, base + j] = -np.inf
                    pool_parent[b, base + j] = -1
                    pool_token[b, base + j] = -1
                continue
            lp = log_softmax_row(draft_logits[b, f], temperature)
            for j, v in enumerate(top_tokens(draft_logits[b, f], topk)):
                val = np.float32(np.float64(pool_score[b, slot]) + lp[v])
                pool_score[b, base + j] = val
                pool_parent[b, base + j] = slot
                pool_token[b, base + j] = v
                cands.append((-float(val), base + j))
        cands.sort()
        for i, (_, s) in enumerate(cands[:n_next]):
            nxt[b, i] = s
    return nxt


def select(pool_score, pool_parent, pool_token, pool_count, m):
    """Re-rank: keep the root and the m - 1 valid pool nodes of largest value
    (ties to the earlier slot), renumbered in pool order.  Returns
    (parent int32 [B,m], tokens int32 [B,m], pool_index int32 [B,m],
    seq_nodes int32 [B]); padding past a sequence's node count is -1 (and
    parent -1)."""
    B = pool_score.shape[0]
    parent = np.full((B, m), -1, np.int32)
    tokens = np.full((B, m), -1, np.int32)
    index = np.full((B, m), -1, np.int32)
    nodes = np.zeros(B, np.int32)
    for b in range(B):
        valid = [s for s in range(1, pool_count) if pool_parent[b, s] >= 0 and np.isfinite(pool_score[b, s])]
        ranked = sorted(valid, key=lambda s: (-float(pool_score[b, s]), s))
        keep = sorted([0] + ranked[: m - 1])
        new = {s: i for i, s in enumerate(keep)}
        for i, s in enumerate(keep):
            index[b, i] = s
            tokens[b, i] = pool_token[b, s]
            parent[b, i] = -1 if s == 0 else new[int(pool_parent[b, s])]
        nodes[b] = len(keep)
    return parent, tokens, index, nodes


def build_tree(draft_fn, B, V, depth, topk, m, temperature, root_token=None):
    """The whole construction: ``draft_fn(b, path_tokens) -> float32 [V]``
    stands in for the draft model at the node reached by that path.  Returns
    the pool and the selected tree (as ``select``)."""
    P = 1 + topk + (depth - 1) * topk * topk
    score = np.full((B, P), -np.inf, np.float32)
    par = np.full((B, P), -1, np.int32)
    tok = np.full((B, P), -1, np.int32)
    frontier, base = None, 1
    for d in range(depth):
        F = 1 if frontier is None else frontier.shape[1]
        logits = np.zeros((B, F, V), np.float32)
        for b in range(B):
            for f in range(F):
                slot = 0 if frontier is None else int(frontier[b, f])
                if slot >= 0:
                    logits[b, f] = draft_fn(b, path_tokens(par[b], tok[b], slot))
        frontier = expand(logits, frontier, score, par, tok, base, topk, topk, temperature, root_token)
        base += F * topk
    return (score, par, tok), select(score, par, tok, base, m)


def path_tokens(par_row, tok_row, slot):
    """Tokens on the path root -> slot, root excluded."""
    out = []
    while slot > 0:
        out.append(int(tok_row[slot]))
        slot = int(par_row[slot])
    return out[::-1]
