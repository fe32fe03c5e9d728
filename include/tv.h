/*
 * libtv -- token-tree verification on AMD MI355X (gfx950).  C ABI.
 *
 * The verification step of draft-then-verify speculative decoding: the
 * target model scores a whole draft tree in one forward pass under a tree
 * attention mask, then an accept/reject walk decides which draft tokens are
 * kept and draws one extra token.
 *
 * Conventions shared by every call
 *  - All array pointers are DEVICE pointers unless stated otherwise.  The
 *    caller owns every buffer; the library never allocates, frees or
 *    synchronises.  Scratch space comes from the caller's `workspace`.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Every call only enqueues work on it and returns.
 *  - bf16 tensors are passed as uint16_t bit patterns (IEEE binary32 with the
 *    low 16 mantissa bits dropped).
 *  - Scalar and shape arguments are checked on the host before anything is
 *    enqueued; a failed check returns a negative tv_status and enqueues
 *    nothing.  A failed launch returns TV_ERR_HIP.
 *  - Tree conventions: nodes 0..N-1 of each sequence; node 0 is the root (the
 *    last committed token) with parent -1; parent[i] < i for i >= 1;
 *    children of a node are taken in increasing index order.
 *  - Calls are stateless and deterministic for fixed inputs and seed.  Calls
 *    on different streams must not share a workspace.
 *
 *  - Ragged batches: the _ex calls take seq_nodes [B] (nodes of each
 *    sequence, 1..N; arrays keep the batch-wide stride N and the rest of a
 *    sequence's rows is padding that is never read) and, for attention,
 *    seq_len [B] (committed cache entries of each sequence, 0..L).  A NULL
 *    array means every sequence uses all N nodes (all L entries).
 *
 * Sources: the pages this library follows are cited per call by page and
 * section: the EAGLE explainer (0h-n0.github.io/posts/paper-2401-10774), the
 * EAGLE-3 explainer (0h-n0.github.io/posts/paper-2501-05370) and the
 * speculative-decoding survey explainer
 * (0h-n0.github.io/posts/paper-2401-07851).
 */
#ifndef TV_H_
#define TV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    TV_OK = 0,
    TV_ERR_INVALID_ARG = -1, /* null pointer, non-positive size, bad temperature, ... */
    TV_ERR_UNSUPPORTED = -2, /* valid but not implemented here: N > TV_MAX_NODES, D != 128 */
    TV_ERR_BAD_TREE = -3,    /* parent[] violates the tree conventions (per-sequence status) */
    TV_ERR_WORKSPACE = -4,   /* workspace missing or smaller than the query says */
    TV_ERR_HIP = -5,         /* a HIP launch or runtime call failed */
    TV_ERR_SCRATCH = -6      /* the shape needs more than TV_NOALLOC_SCRATCH_BYTES (allocation-free call) */
} tv_status;

/* Largest tree (nodes including the root) handled. */
#define TV_MAX_NODES 256
/* 64-bit ancestor words per node of an N-node tree: bit j % 64 of word j / 64. */
#define TV_MASK_WORDS(N) (((N) + 63) / 64)
/* Head dimension handled by the attention kernels. */
#define TV_HEAD_DIM 128

/* Human-readable text for a tv_status value (static storage, never NULL). */
const char* tv_status_string(int status);

/* Library version as 10000*major + 100*minor + patch. */
int tv_version(void);

/*
 * tv_build_tree_mask -- ancestor bitsets of a draft tree.
 *
 * EAGLE explainer, section on parallel verification with a static tree: one
 * target pass with a tree attention mask verifies every root-to-node path, so
 * node i may see exactly its ancestors and itself.
 *
 *   parent     int32 [B,N]     parent index of each node (root: -1).
 *   anc_mask   uint64 [B,N,W]  out, W = TV_MASK_WORDS(N): bit j % 64 of word
 *                              j / 64 set iff node j is i or an ancestor of i.
 *   depth      int32 [B,N]     out: depth of each node (root 0); callers derive
 *                              rotary positions as L + depth.
 *   seq_status int32 [B]       out, may be NULL: 0, or TV_ERR_BAD_TREE when the
 *                              sequence's parent[] is invalid (or, ragged, its
 *                              node count is outside 1..N); such a sequence
 *                              gets anc_mask 0 and depth -1 throughout.
 * Sizes: B >= 0 (B == 0 is a no-op), 1 <= N <= TV_MAX_NODES.
 * tv_build_tree_mask_ex: ragged batches (seq_nodes may be NULL); padding nodes
 * get anc_mask 0 and depth -1.
 */
int tv_build_tree_mask(const int32_t* parent, int B, int N, uint64_t* anc_mask, int32_t* depth,
                       int32_t* seq_status, void* stream);
int tv_build_tree_mask_ex(const int32_t* parent, const int32_t* seq_nodes, int B, int N, uint64_t* anc_mask,
                          int32_t* depth, int32_t* seq_status, void* stream);

/*
 * tv_tree_attention -- ancestor-masked attention of every tree node over the
 * committed KV cache plus its own root-to-node path.
 *
 * EAGLE explainer, section on parallel verification with a static tree (tree
 * attention mask); survey explainer, formal definition, verification phase
 * (the target distribution at draft position i conditions on the context and
 * the drafts before it).
 *
 * For sequence b, query head h (KV head g = h / (Hq/Hkv)) and node i:
 *   out[b,i,h] = sum_j softmax_j(scale * Q[b,i,h] . k_j) v_j over
 *   j in { K_cache[b,g,0..L-1] } and { K_tree[b,j,g] : j ancestor-or-self of i }.
 *
 *   Q        bf16 [B,N,Hq,D]      queries (rotary encoding already applied).
 *   K_cache  bf16 [B,Hkv,L,D]     committed keys, head-major (may be NULL if L == 0).
 *   V_cache  bf16 [B,Hkv,L,D]     committed values (may be NULL if L == 0).
 *   K_tree   bf16 [B,N,Hkv,D]     keys of the tree nodes.
 *   V_tree   bf16 [B,N,Hkv,D]     values of the tree nodes.
 *   anc_mask uint64 [B,N,W]       from tv_build_tree_mask (W = TV_MASK_WORDS(N));
 *                                 must describe a valid tree.
 *   out      fp32 [B,N,Hq,D]      out (rows of padding nodes are not written).
 *   scale    softmax scale, conventionally 1/sqrt(D); finite and > 0.
 * Sizes: B >= 0, 1 <= N <= TV_MAX_NODES, Hq >= Hkv >= 1 with Hq % Hkv == 0,
 * D == TV_HEAD_DIM, L >= 0 (the cache's row stride; ragged calls read only the
 * first seq_len[b] rows of sequence b).
 * Numerics: QK^T in bf16 with fp32 accumulation, softmax in fp32, P.V with
 * P and V in fp16 and fp32 accumulation.  V values beyond the fp16 range
 * (|v| > 65504) saturate to +-65504 in the P.V product.
 * Workspace: at least tv_tree_attention_workspace(...) bytes, 256-byte aligned
 * (may be NULL when that size is 0), zero-filled before its first use: when the
 * cache is split across workgroups it holds their partial results and one
 * arrival counter per row tile, which the last workgroup resets to zero.
 * Calls that share a workspace must not overlap.
 */
size_t tv_tree_attention_workspace(int B, int N, int Hq, int Hkv, int D, int L);
int tv_tree_attention(const uint16_t* Q, const uint16_t* K_cache, const uint16_t* V_cache,
                      const uint16_t* K_tree, const uint16_t* V_tree, const uint64_t* anc_mask,
                      float* out, int B, int N, int Hq, int Hkv, int D, int L, float scale,
                      void* workspace, size_t workspace_bytes, void* stream);
/* Ragged batches (survey explainer, open problems, batch inference: the
 * sequences of a batch accept different numbers of drafts, so their caches
 * and trees differ in length).  seq_nodes [B] and seq_len [B] may be NULL;
 * values are taken as given (precondition 1 <= seq_nodes[b] <= N and
 * 0 <= seq_len[b] <= L; others are clamped into those ranges). */
int tv_tree_attention_ex(const uint16_t* Q, const uint16_t* K_cache, const uint16_t* V_cache,
                         const uint16_t* K_tree, const uint16_t* V_tree, const uint64_t* anc_mask,
                         float* out, const int32_t* seq_nodes, const int32_t* seq_len, int B, int N, int Hq,
                         int Hkv, int D, int L, float scale, void* workspace, size_t workspace_bytes,
                         void* stream);

/*
 * tv_spec_accept -- accept/reject walk over the tree (greedy or lossless
 * speculative sampling).
 *
 * Survey explainer, formal definition, accept/reject phase: a draft x drawn
 * from the draft distribution p is accepted if r < min(1, q(x)/p(x)),
 * r ~ U[0,1]; at the first rejection a token is drawn from
 * norm(max(0, q - p)); the verification phase provides K+1 target
 * distributions so that one extra token is always emitted.  Same page,
 * classification of verification methods: greedy verification keeps drafts
 * that equal the target's greedy choice; token-tree verification checks
 * all candidate paths at once and stays lossless.
 *
 *   q_logits     fp32 [B,N,V]  row u = target logits at tree position u (they
 *                              predict u's children; row u is u's bonus row).
 *   p_logits     fp32 [B,N,V]  row c = draft logits that produced node c (row 0
 *                              unused).  May be NULL when greedy.
 *   draft_tokens int32 [B,N]   token of node c (entry 0 ignored); each in [0,V).
 *   parent       int32 [B,N]   the tree (conventions above).  It is checked on
 *                              the device: a sequence whose parent[] breaks them
 *                              gets accept_len -1 and -1 in both outputs.
 *   philox_seed  key of the Philox-4x32-10 uniforms: the accept test of node c
 *                in sequence b uses counter (c, b, 0, 0), the final draw after
 *                stopping at node u uses (u, b, 1, 0); U = (word0 >> 8) * 2^-24.
 *   temperature  > 0 and finite in sampling mode (logits are divided by it);
 *                ignored when greedy.
 *   greedy       nonzero: keep the deepest path whose every draft equals the
 *                argmax of its parent's target row (ties: smallest token, then
 *                smallest end node); extra token = argmax of the end node's row.
 *                zero: children of the current node are tested in index order;
 *                each rejection replaces the target by norm(max(0, R - P_c));
 *                if all children are rejected the extra token is drawn from the
 *                residual, at a leaf from the leaf's own target row.
 *   accept_len     int32 [B]   out: accepted draft nodes.
 *   accepted_nodes int32 [B,N] out: their node indices root-to-leaf, -1 padded.
 *   out_tokens     int32 [B,N] out: accepted tokens then the extra token, -1 padded.
 * Sizes: B >= 0, 1 <= N <= TV_MAX_NODES, V >= 1.  Logits must be finite.
 * Workspace: at least tv_spec_accept_workspace(B,N,V,greedy) bytes, 256-byte
 * aligned, zero-filled before its first use.  The call keeps its team barrier
 * words there (generation-tagged, so they never need clearing again): the
 * same workspace can be reused by later calls of any shape without clearing.
 * The size depends on the current device (it is planned for the device's
 * resident workgroup capacity).
 * Execution: one launch sized to the device's resident workgroup capacity;
 * every sequence is walked by a team of workgroups that synchronise through
 * the workspace, so calls that share a workspace must not overlap, and calls
 * on other streams (or other processes) that hold compute units for long can
 * starve a team.  Each wait is bounded (about a second); when one runs out the
 * call still finishes, and every sequence of that team reports accept_len -2
 * (its other outputs undefined); the workspace stays reusable.
 */
size_t tv_spec_accept_workspace(int B, int N, int V, int greedy);
int tv_spec_accept(const float* q_logits, const float* p_logits, const int32_t* draft_tokens,
                   const int32_t* parent, int B, int N, int V, uint64_t philox_seed, float temperature,
                   int greedy, int32_t* accept_len, int32_t* accepted_nodes, int32_t* out_tokens,
                   void* workspace, size_t workspace_bytes, void* stream);

/* Flags of tv_spec_accept_ex. */
#define TV_ACCEPT_GREEDY 1
/* Siblings drawn without replacement (EAGLE explainer, static-tree
 * verification: the children of a node are alternative candidates for the
 * same position, taken from the draft's distribution at that node).  p row u
 * is then the draft distribution AT node u, shared by u's children (rows of
 * leaves are not read), and the children of u carry distinct tokens, child k
 * drawn from that row with the tokens of children 1..k-1 removed.  Child k is
 * tested against exactly that distribution; a rejection leaves
 * norm(max(0, R - P^(k))).  Same lossless guarantee (survey explainer,
 * classification of verification methods). */
#define TV_ACCEPT_SIBLINGS_WOR 2

/*
 * tv_spec_accept_ex -- tv_spec_accept for ragged batches and without-
 * replacement siblings.  seq_nodes [B] may be NULL; a sequence whose count is
 * outside 1..N is reported like an invalid tree (accept_len -1).  flags:
 * TV_ACCEPT_GREEDY and/or TV_ACCEPT_SIBLINGS_WOR (ignored when greedy).  The
 * workspace is sized as for tv_spec_accept.
 */
int tv_spec_accept_ex(const float* q_logits, const float* p_logits, const int32_t* draft_tokens,
                      const int32_t* parent, const int32_t* seq_nodes, int B, int N, int V, uint64_t philox_seed,
                      float temperature, int flags, int32_t* accept_len, int32_t* accepted_nodes,
                      int32_t* out_tokens, void* workspace, size_t workspace_bytes, void* stream);

/* The plan tv_spec_accept would use on the current device: workgroups per
 * team (each owns one vocabulary slice of every row), teams, and the slice
 * length.  Any output pointer may be NULL.  Host only. */
int tv_spec_accept_plan(int B, int N, int V, int greedy, int* team_size, int* teams, int* slice);

/*
 * tv_spec_accept_noalloc -- tv_spec_accept_ex without a workspace argument and
 * without any allocation, for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Its scratch is a static device array of
 * TV_NOALLOC_SCRATCH_BYTES (4 MiB) per GPU, held until the process ends; it
 * covers every plan of trees up to 64 nodes, and of larger trees with few
 * enough sequences (256-node trees in sampling mode with 256 sequences need
 * 8.1 MiB and are refused); the first
 * call on a device puts the array's control words in order with a small
 * kernel on `stream` (every team line set to the largest generation found,
 * wait marks and the arrival word cleared): if that first call is captured
 * into a HIP graph, the kernel runs on every replay and each replay still
 * gets a new generation.
 * Shapes whose plan (tv_spec_accept_workspace) needs more return
 * TV_ERR_SCRATCH before anything is enqueued.  Every call on one GPU shares
 * that GPU's array: calls that overlap on one GPU (other streams, other
 * threads) race and must be serialised by the caller.
 */
#define TV_NOALLOC_SCRATCH_BYTES ((size_t)4 << 20)
int tv_spec_accept_noalloc(const float* q_logits, const float* p_logits, const int32_t* draft_tokens,
                           const int32_t* parent, const int32_t* seq_nodes, int B, int N, int V,
                           uint64_t philox_seed, float temperature, int flags, int32_t* accept_len,
                           int32_t* accepted_nodes, int32_t* out_tokens, void* stream);

/* For tests and diagnostics: the number of polls each team wait of later
 * accept calls makes before it gives up (process-wide).  0 makes every wait
 * give up at once, so every sequence that needs its team reports -2;
 * TV_WAIT_DEFAULT restores the default (about a second).  Returns the
 * previous setting.  Host only. */
#define TV_WAIT_DEFAULT 0xFFFFFFFFu
uint32_t tv_set_wait_limit(uint32_t polls);

/*
 * tv_commit_kv -- append the accepted path's keys and values to the cache.
 *
 * EAGLE explainer, implementation notes: verifying a tree needs KV memory
 * beyond the committed context (the pass computes keys and values for every
 * tree node); survey explainer, formal definition, accept/reject phase: the
 * accepted drafts become output.  Sequence b with committed length
 * cache_len[b] and accept_len[b] = a >= 0 appends a + 1 rows: the root (node 0,
 * the last committed token, whose keys and values this pass computed) and
 * accepted_nodes[b, 0..a-1] in path order, at positions cache_len[b] ..
 * cache_len[b] + a, for every KV head.  The extra token drawn by the walk gets
 * its keys and values in the next pass.
 *
 *   K_tree, V_tree   bf16 [B,N,Hkv,D]  keys and values of the tree nodes.
 *   accept_len       int32 [B]         from tv_spec_accept (negative: failed walk).
 *   accepted_nodes   int32 [B,N]       from tv_spec_accept.
 *   cache_len        int32 [B]         committed lengths before the call.
 *   K_cache, V_cache bf16 [B,Hkv,L,D]  updated in place (L = capacity per head).
 *   new_cache_len    int32 [B]         out: cache_len + a + 1, or cache_len
 *                                      when nothing is committed.  Must not
 *                                      alias cache_len.
 *   seq_status       int32 [B]         out, may be NULL: 0; TV_ERR_BAD_TREE when
 *                                      a < 0 or the path names a node outside
 *                                      1..N-1; TV_ERR_INVALID_ARG when the rows
 *                                      do not fit (cache_len + a + 1 > L, or
 *                                      a > N - 1).  Those sequences commit
 *                                      nothing.
 * The tree and cache buffers must not overlap.  Sizes: B >= 0,
 * 1 <= N <= TV_MAX_NODES, Hkv >= 1, D == TV_HEAD_DIM, L >= 0.
 */
int tv_commit_kv(const uint16_t* K_tree, const uint16_t* V_tree, const int32_t* accept_len,
                 const int32_t* accepted_nodes, const int32_t* cache_len, uint16_t* K_cache, uint16_t* V_cache,
                 int32_t* new_cache_len, int32_t* seq_status, int B, int N, int Hkv, int D, int L,
                 void* stream);

/*
 * tv_tree_expand / tv_tree_select -- dynamic draft-tree construction.
 *
 * EAGLE-3 explainer, integration with EAGLE-2 (the draft head plugs into
 * EAGLE-2's dynamic tree generation at inference time), and the EAGLE
 * explainer's conclusion (EAGLE-2 turns the static tree into a dynamic one).
 * The pages give no steps; the construction taken is: a node's value is the
 * draft's probability of its path from the root, kept as a cumulative log
 * probability; each expansion gives every frontier node its top-k tokens as
 * children and keeps the Fn most valuable new nodes as the next frontier; the
 * final tree is the root plus the m - 1 most valuable nodes of the pool.
 *
 * A pool of P slots per sequence holds every node created: value (fp32),
 * parent slot (-1: root or empty slot) and token.  Slot 0 is the root.
 *
 * tv_tree_expand: one expansion step.
 *   draft_logits fp32 [B,F,V]  row f: the draft's logits at frontier node f.
 *   frontier     int32 [B,F]   pool slots of the frontier (-1: empty), or NULL
 *                              for the first step, which expands the root
 *                              (F must be 1) and initialises slot 0 (value 0,
 *                              parent -1, token root_token[b], or -1 when
 *                              root_token is NULL).
 *   topk         children per frontier node, 1..16: its topk largest logits
 *                (ties to the smaller token id).  Child j of row f goes to
 *                slot pool_base + f*topk + j, with value
 *                fp32(value(parent) + log softmax(logits/T)[token]), the
 *                log-softmax computed in fp64.  Rows of empty slots (and
 *                children past V tokens) give empty slots (value -inf,
 *                parent -1, token -1).
 *   temperature  > 0 and finite.
 *   next_frontier int32 [B,Fn]  out: the Fn best new slots by (value desc,
 *                slot asc), -1 where fewer exist; may be NULL when Fn == 0.
 *   Requires pool_base >= 1 and pool_base + F*topk <= P.
 * tv_tree_select: the tree.  Keeps the root and the M - 1 best valid slots
 * among 1..pool_count-1 (ties to the earlier slot; a child never outranks its
 * parent, so the kept set is a tree), renumbered in slot order:
 *   parent int32 [B,M]   out: parent node index (-1 for the root and padding).
 *   tokens int32 [B,M]   out: tokens (slot 0's token for the root).
 *   pool_index int32 [B,M] out: the pool slot of each node (-1 padding).
 *   seq_nodes int32 [B]  out: nodes of each tree (a ragged batch when pools
 *                        hold fewer than M - 1 valid slots).
 *   Sizes: pool_count <= 4096, M <= TV_MAX_NODES.
 */
int tv_tree_expand(const float* draft_logits, const int32_t* frontier, const int32_t* root_token, int B, int F,
                   int V, int topk, float temperature, float* pool_score, int32_t* pool_parent,
                   int32_t* pool_token, int P, int pool_base, int32_t* next_frontier, int Fn, void* stream);
int tv_tree_select(const float* pool_score, const int32_t* pool_parent, const int32_t* pool_token, int B, int P,
                   int pool_count, int M, int32_t* parent, int32_t* tokens, int32_t* pool_index,
                   int32_t* seq_nodes, void* stream);

/*
 * tv_philox_uniforms -- the uniforms tv_spec_accept draws, for auditing.
 *
 *   triples  uint32 [n,3]  (node, sequence, purpose) counters, device memory.
 *   out_u    fp32 [n]      out: U(seed, node, sequence, purpose), may be NULL.
 *   out_raw  uint32 [n,4]  out: the raw Philox-4x32-10 block, may be NULL.
 */
int tv_philox_uniforms(uint64_t seed, const uint32_t* triples, int n, float* out_u, uint32_t* out_raw,
                       void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TV_H_ */
