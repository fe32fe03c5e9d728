/*
 * Plain fp64 CPU reference of the accept/reject walk of token-tree
 * verification, and of the Philox-4x32-10 counter-based generator that the
 * walk draws its uniforms from.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the oracle: it is built by gcc into
 * oracle/liboracle.so and is loaded only by the test suite, the smoke check
 * and the CPU-baseline leg of the benchmark.  It shares no code, header,
 * table or constant with the HIP library.
 *
 * What it follows:
 *  - Speculative-decoding survey explainer (0h-n0.github.io, paper-2401-07851),
 *    section "Formal Definition", accept/reject phase: a draft token x drawn
 *    from the draft distribution p is accepted when r < min(1, q(x)/p(x)) with
 *    r ~ U[0,1]; at the first rejection the token is drawn from
 *    norm(max(0, q - p)); the verification phase computes K+1 target
 *    distributions so that a token can always be emitted.
 *  - Same page, section "Classification by verification method" (table):
 *    greedy verification accepts a draft while it equals the target's greedy
 *    choice; token-tree verification checks several candidate paths at once
 *    and is lossless.
 *  - EAGLE explainer (paper-2401-10774), section on static-tree parallel
 *    verification: each node of the draft tree is a candidate token and every
 *    root-to-node path is a candidate continuation.
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *  - q row u is the target distribution AT tree position u (it predicts u's
 *    children, and is u's bonus distribution); p row c is the draft
 *    distribution that produced node c.  Node 0 is the root.
 *  - Several children of one node are tried in increasing index order; after
 *    rejecting child c the target at the node becomes norm(max(0, R - P_c))
 *    (recursive residual rule).  With one child this is exactly the pages'
 *    rule.  If the residual mass is 0 the target is kept unchanged.
 *  - If every child of the current node is rejected the extra token is drawn
 *    from the current residual; if the walk reaches a leaf it is drawn from
 *    that leaf's own target row (the (K+1)-th distribution).
 *  - Temperature T divides both target and draft logits before softmax.
 *  - Inverse CDF over ascending token ids with a strict '>' comparison;
 *    fallback to the largest token with positive mass.
 *  - Greedy: argmax ties go to the smallest token id; among equally deep
 *    fully-matching paths the one ending at the smallest node index wins.
 *  - Uniforms: Philox-4x32-10 with key (seed lo, seed hi) and counter
 *    (node, sequence, purpose, 0); U = (first output word >> 8) * 2^-24.
 *    Purpose 0 = accept test, 1 = final sample, 2 = draft sampling in the
 *    lossless harness.
 *  - Siblings drawn without replacement (EAGLE explainer, static-tree
 *    verification: the children of a node are several candidates for the
 *    same next position, taken from the draft's distribution at that node;
 *    survey explainer, classification table: token-tree verification stays
 *    lossless).  In this mode p row u is the draft distribution AT node u,
 *    shared by all of u's children, and child k of u was drawn from it with
 *    the tokens of children 1..k-1 removed and the rest renormalised.  The
 *    walk tests child k against exactly that distribution, P^(k), and on
 *    rejection updates R <- norm(max(0, R - P^(k))).
 *  - Ragged batches: sequence b uses only its first seq_nodes[b] nodes; the
 *    arrays keep the batch-wide stride N and the outputs are -1 padded.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_ERR_ARG (-1)
#define ORC_ERR_TREE (-3)
#define ORC_ERR_NOMEM (-6)

/* Distance from a decision boundary below which a decision is flagged as
 * "near boundary": fp32 and fp64 may legitimately disagree there. */
#define ORC_FLAG_EPS 1e-5

/* ------------------------------------------------------------------------ */
/* Philox-4x32-10, from Salmon, Moraes, Dror and Shaw, "Parallel Random      */
/* Numbers: As Easy as 1, 2, 3" (SC'11).  Each round multiplies words 0 and  */
/* 2 by the two round multipliers, and the new state is                     */
/* (hi(M1*c2) ^ c1 ^ k0, lo(M1*c2), hi(M0*c0) ^ c3 ^ k1, lo(M0*c0)); the key */
/* is advanced by the two Weyl constants between rounds.                     */
/* ------------------------------------------------------------------------ */
static const uint32_t ORC_PHILOX_M0 = 0xD2511F53u;
static const uint32_t ORC_PHILOX_M1 = 0xCD9E8D57u;
static const uint32_t ORC_WEYL_0 = 0x9E3779B9u; /* golden ratio */
static const uint32_t ORC_WEYL_1 = 0xBB67AE85u; /* sqrt(3) - 1 */

void orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
    uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += ORC_WEYL_0;
            k1 += ORC_WEYL_1;
        }
        uint64_t prod0 = (uint64_t)ORC_PHILOX_M0 * (uint64_t)c0;
        uint64_t prod1 = (uint64_t)ORC_PHILOX_M1 * (uint64_t)c2;
        uint32_t hi0 = (uint32_t)(prod0 >> 32), lo0 = (uint32_t)prod0;
        uint32_t hi1 = (uint32_t)(prod1 >> 32), lo1 = (uint32_t)prod1;
        uint32_t n0 = hi1 ^ c1 ^ k0;
        uint32_t n1 = lo1;
        uint32_t n2 = hi0 ^ c3 ^ k1;
        uint32_t n3 = lo0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

double orc_uniform(uint64_t seed, uint32_t node, uint32_t seq, uint32_t purpose) {
    uint32_t key[2] = {(uint32_t)(seed & 0xffffffffu), (uint32_t)(seed >> 32)};
    uint32_t ctr[4] = {node, seq, purpose, 0u};
    uint32_t out[4];
    orc_philox4x32_10(ctr, key, out);
    return (double)(out[0] >> 8) * (1.0 / 16777216.0);
}

/* Batch forms used by the tests: raw blocks for explicit (counter, key) pairs,
 * and uniforms for (node, seq, purpose) triples under one seed. */
void orc_philox_batch(const uint32_t* ctr, const uint32_t* key, int64_t n, uint32_t* out) {
    for (int64_t i = 0; i < n; ++i) orc_philox4x32_10(ctr + 4 * i, key + 2 * i, out + 4 * i);
}

void orc_uniform_batch(uint64_t seed, const uint32_t* triples, int64_t n, double* out) {
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_uniform(seed, triples[3 * i], triples[3 * i + 1], triples[3 * i + 2]);
}

/* ------------------------------------------------------------------------ */
/* Tree validity: node 0 is the root (parent -1); every other node's parent  */
/* is an earlier node.                                                       */
/* ------------------------------------------------------------------------ */
static int tree_is_valid(const int32_t* parent, int N) {
    if (N < 1 || parent[0] != -1) return 0;
    for (int i = 1; i < N; ++i)
        if (parent[i] < 0 || parent[i] >= i) return 0;
    return 1;
}

/* softmax(logits / T) in fp64. */
static void softmax_T(const float* logits, int V, double T, double* out) {
    double m = -INFINITY;
    for (int v = 0; v < V; ++v) {
        double z = (double)logits[v] / T;
        if (z > m) m = z;
    }
    double s = 0.0;
    for (int v = 0; v < V; ++v) {
        out[v] = exp((double)logits[v] / T - m);
        s += out[v];
    }
    for (int v = 0; v < V; ++v) out[v] /= s;
}

static int argmax_row(const float* row, int V) {
    int best = 0;
    for (int v = 1; v < V; ++v)
        if (row[v] > row[best]) best = v; /* strict: ties keep the smaller id */
    return best;
}

/* Inverse CDF: smallest k with cumsum(R)[k] > u; if none, the largest k with
 * R[k] > 0.  Flags a boundary closer than ORC_FLAG_EPS. */
static int sample_inverse_cdf(const double* R, int V, double u, int* flags, double* margin) {
    double cum = 0.0;
    for (int k = 0; k < V; ++k) {
        double before = cum;
        cum += R[k];
        if (cum > u) {
            double d = fmin(fabs(cum - u), fabs(before - u));
            if (d < *margin) *margin = d;
            if (d < ORC_FLAG_EPS) ++*flags;
            return k;
        }
    }
    double d = fabs(cum - u);
    if (d < *margin) *margin = d;
    if (d < ORC_FLAG_EPS) ++*flags;
    for (int k = V - 1; k >= 0; --k)
        if (R[k] > 0.0) return k;
    return V - 1;
}

/* variant: 0 = the rule; 1 = planted mistake for negative controls (siblings
 * are tested against the un-updated target of their parent); 2 = planted
 * mistake for siblings drawn without replacement (each is tested against the
 * shared row P_p(u) itself instead of P^(k)). */
typedef struct {
    double* R;   /* current target at the node being expanded */
    double* R0;  /* un-updated target (variant 1 only) */
    double* Pc;  /* draft distribution of the child being tested */
    double* Pu;  /* without replacement: the shared draft row of the node */
    int32_t* drawn; /* without replacement: tokens of the node's rejected children */
} orc_scratch;

/* P^(k): Pu with the tokens drawn[0..nd-1] removed, renormalised.  If no mass
 * remains the result is all zero. */
static void without_replacement(const double* Pu, const int32_t* drawn, int nd, int V, double* out) {
    memcpy(out, Pu, sizeof(double) * (size_t)V);
    for (int j = 0; j < nd; ++j) out[drawn[j]] = 0.0;
    double s = 0.0;
    for (int v = 0; v < V; ++v) s += out[v];
    for (int v = 0; v < V; ++v) out[v] = (s > 0.0) ? out[v] / s : 0.0;
}

static int walk_sampling(const float* q, const float* p, const int32_t* draft, const int32_t* parent,
                         int N, int V, uint64_t seed, uint32_t seq, double T, int variant, int wor,
                         orc_scratch* w, int32_t* acc_nodes, int32_t* tokens, int* flags,
                         double* margin) {
    int u = 0, len = 0;
    int32_t* drawn = w->drawn;
    for (;;) {
        softmax_T(q + (size_t)u * V, V, T, w->R); /* R = P_q(u) */
        if (variant == 1) memcpy(w->R0, w->R, sizeof(double) * (size_t)V);
        if (wor) softmax_T(p + (size_t)u * V, V, T, w->Pu); /* the node's draft row */
        int has_child = 0, accepted = -1, nd = 0;
        for (int c = u + 1; c < N; ++c) {
            if (parent[c] != u) continue;
            has_child = 1;
            int x = draft[c];
            if (!wor)
                softmax_T(p + (size_t)c * V, V, T, w->Pc);
            else if (variant == 2)
                memcpy(w->Pc, w->Pu, sizeof(double) * (size_t)V);
            else
                without_replacement(w->Pu, drawn, nd, V, w->Pc);
            double px = w->Pc[x];
            double rx = (variant == 1) ? w->R0[x] : w->R[x];
            double a = (px == 0.0) ? 1.0 : fmin(1.0, rx / px);
            double r = orc_uniform(seed, (uint32_t)c, seq, 0u);
            double d = fabs(r - a);
            if (d < *margin) *margin = d;
            if (d < ORC_FLAG_EPS) ++*flags;
            if (r < a) {
                accepted = c;
                break;
            }
            /* rejected: R <- norm(max(0, R - P_c)) */
            double Z = 0.0;
            for (int v = 0; v < V; ++v) {
                double t = w->R[v] - w->Pc[v];
                Z += (t > 0.0) ? t : 0.0;
            }
            if (Z > 0.0) {
                for (int v = 0; v < V; ++v) {
                    double t = w->R[v] - w->Pc[v];
                    w->R[v] = (t > 0.0) ? t / Z : 0.0;
                }
            }
            drawn[nd++] = x; /* at most N - 1 children */
        }
        if (!has_child || accepted < 0) break; /* leaf: bonus from P_q(u); else residual */
        acc_nodes[len] = accepted;
        tokens[len] = draft[accepted];
        ++len;
        u = accepted;
    }
    double ut = orc_uniform(seed, (uint32_t)u, seq, 1u);
    tokens[len] = sample_inverse_cdf(w->R, V, ut, flags, margin);
    return len;
}

static int walk_greedy(const float* q, const int32_t* draft, const int32_t* parent, int N, int V,
                       int32_t* acc_nodes, int32_t* tokens) {
    int* amax = (int*)malloc(sizeof(int) * (size_t)N * 3);
    if (!amax) return -1;
    int* valid = amax + N;
    int* depth = amax + 2 * N;
    for (int u = 0; u < N; ++u) amax[u] = argmax_row(q + (size_t)u * V, V);
    valid[0] = 1;
    depth[0] = 0;
    for (int i = 1; i < N; ++i) {
        valid[i] = valid[parent[i]] && (draft[i] == amax[parent[i]]);
        depth[i] = depth[parent[i]] + 1;
    }
    int e = 0;
    for (int i = 1; i < N; ++i)
        if (valid[i] && depth[i] > depth[e]) e = i;
    int len = depth[e];
    for (int i = e, k = len - 1; i != 0; i = parent[i], --k) {
        acc_nodes[k] = i;
        tokens[k] = draft[i];
    }
    tokens[len] = amax[e];
    free(amax);
    return len;
}

/*
 * q_logits, p_logits: [B,N,V] fp32 (p may be NULL when greedy).  draft, parent:
 * [B,N].  seq_nodes: [B] nodes of each sequence (NULL: all N).  wor: siblings
 * drawn without replacement (p row u is shared by u's children).  seq_offset:
 * the Philox sequence counter of batch entry b is seq_offset + b.  Outputs:
 * accept_len [B]; accepted_nodes, out_tokens [B,N], -1 padded; nflags [B]
 * near-boundary decision counts; min_margin [B] smallest distance to a
 * decision boundary (both may be NULL).
 */
int orc_spec_accept_ex(const float* q, const float* p, const int32_t* draft, const int32_t* parent,
                       const int32_t* seq_nodes, int B, int N, int V, uint64_t seed, double T, int greedy,
                       int variant, int wor, uint32_t seq_offset, int32_t* accept_len, int32_t* accepted_nodes,
                       int32_t* out_tokens, int32_t* nflags, double* min_margin) {
    if (B < 0 || N < 1 || V < 1 || !q || !draft || !parent || !accept_len || !accepted_nodes ||
        !out_tokens)
        return ORC_ERR_ARG;
    if (!greedy && (!p || !(T > 0.0) || !isfinite(T))) return ORC_ERR_ARG;
    for (int b = 0; b < B; ++b) {
        int nb = seq_nodes ? seq_nodes[b] : N;
        if (nb < 1 || nb > N) return ORC_ERR_ARG;
        if (!tree_is_valid(parent + (size_t)b * N, nb)) return ORC_ERR_TREE;
        for (int c = 1; c < nb; ++c)
            if (draft[(size_t)b * N + c] < 0 || draft[(size_t)b * N + c] >= V) return ORC_ERR_ARG;
    }
    orc_scratch w;
    w.R = (double*)malloc(sizeof(double) * (size_t)V * 4);
    w.drawn = (int32_t*)malloc(sizeof(int32_t) * (size_t)N);
    if (!w.R || !w.drawn) {
        free(w.R);
        free(w.drawn);
        return ORC_ERR_NOMEM;
    }
    w.R0 = w.R + V;
    w.Pc = w.R + 2 * (size_t)V;
    w.Pu = w.R + 3 * (size_t)V;
    for (int b = 0; b < B; ++b) {
        int nb = seq_nodes ? seq_nodes[b] : N;
        int32_t* an = accepted_nodes + (size_t)b * N;
        int32_t* tk = out_tokens + (size_t)b * N;
        for (int i = 0; i < N; ++i) an[i] = tk[i] = -1;
        int flags = 0;
        double margin = INFINITY;
        int len;
        if (greedy)
            len = walk_greedy(q + (size_t)b * N * V, draft + (size_t)b * N, parent + (size_t)b * N, nb, V,
                              an, tk);
        else
            len = walk_sampling(q + (size_t)b * N * V, p + (size_t)b * N * V, draft + (size_t)b * N,
                                parent + (size_t)b * N, nb, V, seed, seq_offset + (uint32_t)b, T, variant, wor,
                                &w, an, tk, &flags, &margin);
        if (len < 0) {
            free(w.R);
            free(w.drawn);
            return ORC_ERR_NOMEM;
        }
        accept_len[b] = len;
        if (nflags) nflags[b] = flags;
        if (min_margin) min_margin[b] = margin;
    }
    free(w.R);
    free(w.drawn);
    return ORC_OK;
}

int orc_spec_accept(const float* q, const float* p, const int32_t* draft, const int32_t* parent,
                    int B, int N, int V, uint64_t seed, double T, int greedy, int variant,
                    int32_t* accept_len, int32_t* accepted_nodes, int32_t* out_tokens,
                    int32_t* nflags, double* min_margin) {
    return orc_spec_accept_ex(q, p, draft, parent, NULL, B, N, V, seed, T, greedy, variant, 0, 0u, accept_len,
                              accepted_nodes, out_tokens, nflags, min_margin);
}

/*
 * Lossless harness (tests only): one sequence, fixed logits, ntrials Philox
 * seeds seed0 .. seed0+ntrials-1.  Per trial the draft token of every node c
 * is drawn by inverse CDF with U(seed, c, 0, 2):
 *   draft_mode 0: from P_p(c) (independent siblings; walk with p row c);
 *   draft_mode 1: taken as argmax p_c (negative control);
 *   draft_mode 2: from P_p(parent(c)) without the tokens of c's earlier
 *                 siblings, renormalised (walk in the without-replacement mode);
 *   draft_mode 3: like 2 but with replacement (independent draws from the
 *                 shared row), walked in the without-replacement mode.
 * then the walk runs with the same seed.  Outputs per trial: drafts
 * [ntrials,N], accept_len [ntrials], accepted [ntrials,N], tokens [ntrials,N].
 */
int orc_lossless_trials(const float* q, const float* p, const int32_t* parent, int N, int V, double T,
                        uint64_t seed0, int64_t ntrials, int variant, int draft_mode, int32_t* drafts,
                        int32_t* accept_len, int32_t* accepted, int32_t* tokens) {
    if (N < 1 || V < 1 || !q || !p || !parent || !(T > 0.0)) return ORC_ERR_ARG;
    if (!tree_is_valid(parent, N)) return ORC_ERR_TREE;
    const int wor = draft_mode >= 2;
    orc_scratch w;
    w.R = (double*)malloc(sizeof(double) * (size_t)V * 4);
    double* Pd = (double*)malloc(sizeof(double) * (size_t)V * 2);
    int32_t* sib = (int32_t*)malloc(sizeof(int32_t) * (size_t)N);
    w.drawn = (int32_t*)malloc(sizeof(int32_t) * (size_t)N);
    if (!w.R || !Pd || !sib || !w.drawn) {
        free(w.R);
        free(Pd);
        free(sib);
        free(w.drawn);
        return ORC_ERR_NOMEM;
    }
    w.R0 = w.R + V;
    w.Pc = w.R + 2 * (size_t)V;
    w.Pu = w.R + 3 * (size_t)V;
    for (int64_t t = 0; t < ntrials; ++t) {
        uint64_t seed = seed0 + (uint64_t)t;
        int32_t* dr = drafts + t * N;
        int32_t* an = accepted + t * N;
        int32_t* tk = tokens + t * N;
        dr[0] = 0;
        for (int c = 1; c < N; ++c) {
            int dflags = 0;
            double dmargin = INFINITY;
            double ud = orc_uniform(seed, (uint32_t)c, 0u, 2u);
            if (draft_mode == 1) {
                dr[c] = argmax_row(p + (size_t)c * V, V);
            } else if (draft_mode == 0) {
                softmax_T(p + (size_t)c * V, V, T, Pd);
                dr[c] = sample_inverse_cdf(Pd, V, ud, &dflags, &dmargin);
            } else {
                /* the earlier siblings of c, in index order */
                int ns = 0;
                for (int j = 1; j < c; ++j)
                    if (parent[j] == parent[c]) sib[ns++] = dr[j];
                softmax_T(p + (size_t)parent[c] * V, V, T, Pd);
                if (draft_mode == 2) {
                    without_replacement(Pd, sib, ns, V, Pd + V);
                    dr[c] = sample_inverse_cdf(Pd + V, V, ud, &dflags, &dmargin);
                } else {
                    dr[c] = sample_inverse_cdf(Pd, V, ud, &dflags, &dmargin);
                }
            }
        }
        for (int i = 0; i < N; ++i) an[i] = tk[i] = -1;
        int flags = 0;
        double margin = INFINITY;
        accept_len[t] = walk_sampling(q, p, dr, parent, N, V, seed, 0u, T, variant, wor, &w, an, tk, &flags,
                                      &margin);
    }
    free(w.R);
    free(Pd);
    free(sib);
    free(w.drawn);
    return ORC_OK;
}
