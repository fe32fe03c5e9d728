// tv_build_tree_mask: ancestor-or-self bitsets and depths of draft trees.
//
// EAGLE explainer (paper-2401-10774), section on parallel verification with a
// static tree: one forward pass with a tree attention mask verifies every
// root-to-node path, so node i sees exactly its ancestors and itself.
#include "tv_device.h"
#include "tv_internal.h"

namespace tv {
namespace {

// One workgroup of 64 lanes per sequence, one lane per node (N <= 64).
__global__ __launch_bounds__(64) void tree_mask_kernel(const int32_t* __restrict__ parent, int N,
                                                        uint64_t* __restrict__ anc, int32_t* __restrict__ depth,
                                                        int32_t* __restrict__ seq_status) {
    const int b = blockIdx.x;
    const int i = threadIdx.x;
    const int32_t* par = parent + (size_t)b * N;
    __shared__ int32_t sp[TV_MAX_NODES];
    int ok = 1;
    if (i < N) {
        const int p = par[i];
        sp[i] = p;
        ok = (i == 0) ? (p == -1) : (p >= 0 && p < i);
    }
    // every lane of the single wave votes; any invalid node invalidates the sequence
    const bool all_ok = __all(ok);
    __syncthreads();
    if (i < N) {
        uint64_t bits = 0;
        int d = -1;
        if (all_ok) {
            // parent[j] < j guarantees the chase ends at the root within i steps
            for (int j = i; j != -1; j = sp[j]) {
                bits |= 1ull << j;
                ++d;
            }
        }
        anc[(size_t)b * N + i] = all_ok ? bits : 0ull;
        depth[(size_t)b * N + i] = all_ok ? d : -1;
    }
    if (i == 0 && seq_status) seq_status[b] = all_ok ? TV_OK : TV_ERR_BAD_TREE;
}

}  // namespace
}  // namespace tv

extern "C" int tv_build_tree_mask(const int32_t* parent, int B, int N, uint64_t* anc_mask, int32_t* depth,
                                  int32_t* seq_status, void* stream) {
    if (B < 0 || N < 1) return TV_ERR_INVALID_ARG;
    if (N > TV_MAX_NODES) return TV_ERR_UNSUPPORTED;
    if (B == 0) return TV_OK;
    if (!parent || !anc_mask || !depth) return TV_ERR_INVALID_ARG;
    if (!tv::aligned(anc_mask, 8) || !tv::aligned(parent, 4) || !tv::aligned(depth, 4)) return TV_ERR_INVALID_ARG;
    hipLaunchKernelGGL(tv::tree_mask_kernel, dim3(B), dim3(64), 0, (hipStream_t)stream, parent, N, anc_mask, depth,
                       seq_status);
    return tv::launch_status();
}
