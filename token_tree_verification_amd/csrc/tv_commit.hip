// tv_commit_kv: the accepted path's keys and values move from the tree rows
// into the KV cache.
//
// EAGLE explainer (paper-2401-10774), implementation notes: verifying a tree
// needs KV-cache memory beyond the committed context, because the target's
// pass computes keys and values for every tree node.  Survey explainer
// (paper-2401-07851), formal definition, accept/reject phase: the accepted
// drafts become output.  Sequence b appends the root (the last committed
// token, whose keys and values this pass computed) and its accepted nodes in
// path order at cache positions cache_len[b] .. cache_len[b] + accept_len[b].
//
// A plain HBM gather-scatter: each lane moves one 16-byte piece of one
// (row, KV head) of K or V (256 bytes = 16 lanes).  Every workgroup of a
// sequence first checks the path (lengths and node ids) itself, so all of
// them reach the same verdict without communicating.
#include "tv_device.h"
#include "tv_internal.h"

namespace tv {
namespace {

constexpr int kCommitThreads = 256;
constexpr int kPieces = TV_HEAD_DIM * 2 / 16;  // 16-byte pieces of one key (or value) row

__global__ __launch_bounds__(kCommitThreads) void commit_kv_kernel(
    const uint16_t* __restrict__ K_tree, const uint16_t* __restrict__ V_tree, const int32_t* __restrict__ accept_len,
    const int32_t* __restrict__ accepted_nodes, const int32_t* __restrict__ cache_len, uint16_t* __restrict__ K_cache,
    uint16_t* __restrict__ V_cache, int32_t* __restrict__ new_len, int32_t* __restrict__ seq_status, int N, int Hkv,
    int L) {
    const int b = blockIdx.y;
    const int a = accept_len[b];
    const int lb = cache_len[b];
    // the verdict: a walk that failed (or an invalid tree) commits nothing; so
    // does a path that would not fit the cache or names a node outside 1..N-1
    int st = a < 0 ? TV_ERR_BAD_TREE : ((lb < 0 || a > N - 1 || (long)lb + a + 1 > (long)L) ? TV_ERR_INVALID_ARG : TV_OK);
    int bad = 0;
    if (st == TV_OK) {
        for (int k = threadIdx.x; k < a; k += kCommitThreads) {
            const int node = accepted_nodes[(size_t)b * N + k];
            bad |= node < 1 || node >= N;
        }
    }
    if (__syncthreads_or(bad)) st = TV_ERR_BAD_TREE;
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        new_len[b] = st == TV_OK ? lb + a + 1 : lb;
        if (seq_status) seq_status[b] = st;
    }
    if (st != TV_OK) return;
    // item = ((row k, head g), K or V, piece)
    const int item = blockIdx.x * kCommitThreads + threadIdx.x;
    const int piece = item % kPieces;
    const int kv = (item / kPieces) & 1;
    const int pair = item / (2 * kPieces);
    const int k = pair / Hkv, g = pair % Hkv;
    if (k > a) return;
    const int node = k == 0 ? 0 : accepted_nodes[(size_t)b * N + k - 1];
    const uint16_t* src = (kv ? V_tree : K_tree) + (((size_t)b * N + node) * Hkv + g) * TV_HEAD_DIM;
    uint16_t* dst = (kv ? V_cache : K_cache) + (((size_t)b * Hkv + g) * L + lb + k) * TV_HEAD_DIM;
    reinterpret_cast<u32x4*>(dst)[piece] = reinterpret_cast<const u32x4*>(src)[piece];
}

}  // namespace
}  // namespace tv

extern "C" int tv_commit_kv(const uint16_t* K_tree, const uint16_t* V_tree, const int32_t* accept_len,
                            const int32_t* accepted_nodes, const int32_t* cache_len, uint16_t* K_cache,
                            uint16_t* V_cache, int32_t* new_cache_len, int32_t* seq_status, int B, int N, int Hkv,
                            int D, int L, void* stream) {
    using namespace tv;
    if (B < 0 || N < 1 || Hkv < 1 || L < 0) return TV_ERR_INVALID_ARG;
    if (N > TV_MAX_NODES || D != TV_HEAD_DIM) return TV_ERR_UNSUPPORTED;
    if (B == 0) return TV_OK;
    if (!K_tree || !V_tree || !accept_len || !accepted_nodes || !cache_len || !new_cache_len) return TV_ERR_INVALID_ARG;
    if (L > 0 && (!K_cache || !V_cache)) return TV_ERR_INVALID_ARG;
    if (!aligned(K_tree, 16) || !aligned(V_tree, 16) || (L > 0 && (!aligned(K_cache, 16) || !aligned(V_cache, 16))))
        return TV_ERR_INVALID_ARG;
    if (B > 65535) return TV_ERR_UNSUPPORTED;  // one grid row per sequence
    const long items = (long)N * Hkv * 2 * kPieces;
    const int blocks = (int)((items + kCommitThreads - 1) / kCommitThreads);
    hipLaunchKernelGGL(commit_kv_kernel, dim3(blocks, B), dim3(kCommitThreads), 0, (hipStream_t)stream, K_tree, V_tree,
                       accept_len, accepted_nodes, cache_len, K_cache, V_cache, new_cache_len, seq_status, N, Hkv, L);
    return launch_status();
}
