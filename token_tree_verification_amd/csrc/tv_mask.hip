// tv_build_tree_mask: ancestor-or-self bitsets and depths of draft trees.
//
// EAGLE explainer (paper-2401-10774), section on parallel verification with a
// static tree: one forward pass with a tree attention mask verifies every
// root-to-node path, so node i sees exactly its ancestors and itself.
#include "tv_device.h"
#include "tv_internal.h"

namespace tv {
namespace {

constexpr int kMaskWords = TV_MASK_WORDS(TV_MAX_NODES);

// One workgroup per sequence, one lane per node (up to TV_MAX_NODES lanes).
// Node i chases parent pointers (held in LDS) up to the root, setting one bit
// per node on the way; parent[j] < j makes every chase end within i steps.
__global__ __launch_bounds__(TV_MAX_NODES) void tree_mask_kernel(const int32_t* __restrict__ parent,
                                                                  const int32_t* __restrict__ seq_nodes, int N,
                                                                  uint64_t* __restrict__ anc, int32_t* __restrict__ depth,
                                                                  int32_t* __restrict__ seq_status) {
    const int b = blockIdx.x;
    const int i = threadIdx.x;
    const int W = TV_MASK_WORDS(N);
    const int32_t* par = parent + (size_t)b * N;
    const int nb = seq_nodes ? seq_nodes[b] : N;
    __shared__ int32_t sp[TV_MAX_NODES];
    int ok = nb >= 1 && nb <= N;
    if (ok && i < nb) {
        const int p = par[i];
        sp[i] = p;
        ok = (i == 0) ? (p == -1) : (p >= 0 && p < i);
    }
    // any invalid node invalidates the sequence (the barrier also publishes sp)
    const bool all_ok = __syncthreads_and(ok) != 0;
    if (i < N) {
        uint64_t bits[kMaskWords] = {};
        int d = -1;
        if (all_ok && i < nb) {
            for (int j = i; j != -1; j = sp[j]) {
#pragma unroll
                for (int w = 0; w < kMaskWords; ++w)
                    if (w == (j >> 6)) bits[w] |= 1ull << (j & 63);
                ++d;
            }
        }
        for (int w = 0; w < W; ++w) {
            uint64_t v = 0;
#pragma unroll
            for (int k = 0; k < kMaskWords; ++k)
                if (k == w) v = bits[k];
            anc[((size_t)b * N + i) * W + w] = v;
        }
        depth[(size_t)b * N + i] = d;
    }
    if (i == 0 && seq_status) seq_status[b] = all_ok ? TV_OK : TV_ERR_BAD_TREE;
}

}  // namespace
}  // namespace tv

extern "C" int tv_build_tree_mask_ex(const int32_t* parent, const int32_t* seq_nodes, int B, int N,
                                     uint64_t* anc_mask, int32_t* depth, int32_t* seq_status, void* stream) {
    if (B < 0 || N < 1) return TV_ERR_INVALID_ARG;
    if (N > TV_MAX_NODES) return TV_ERR_UNSUPPORTED;
    if (B == 0) return TV_OK;
    if (!parent || !anc_mask || !depth) return TV_ERR_INVALID_ARG;
    if (!tv::aligned(anc_mask, 8) || !tv::aligned(parent, 4) || !tv::aligned(depth, 4) ||
        (seq_nodes && !tv::aligned(seq_nodes, 4)))
        return TV_ERR_INVALID_ARG;
    const int threads = (N + 63) / 64 * 64;
    hipLaunchKernelGGL(tv::tree_mask_kernel, dim3(B), dim3(threads), 0, (hipStream_t)stream, parent, seq_nodes, N,
                       anc_mask, depth, seq_status);
    return tv::launch_status();
}

extern "C" int tv_build_tree_mask(const int32_t* parent, int B, int N, uint64_t* anc_mask, int32_t* depth,
                                  int32_t* seq_status, void* stream) {
    return tv_build_tree_mask_ex(parent, nullptr, B, N, anc_mask, depth, seq_status, stream);
}
