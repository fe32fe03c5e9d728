// tv_tree_expand / tv_tree_select: dynamic draft-tree construction.
//
// EAGLE-3 explainer (paper-2501-05370), integration with EAGLE-2, and the
// EAGLE explainer's conclusion (paper-2401-10774): EAGLE-2 builds the draft
// tree at inference time instead of using a fixed shape.  A node's value is
// the draft's probability of its whole path, kept as a cumulative log
// probability; a step expands the frontier nodes with their top-k tokens and
// keeps the k most valuable new nodes as the next frontier; at the end the
// root and the m - 1 most valuable nodes of the pool form the tree.
//
// Values are binary32: value(child) = fp32(value(parent) + log softmax(x/T)
// [token]) with the log-softmax in fp64 (fp64 exponentials, fp64 sum), so two
// implementations round the same sums the same way.  Every ordering is by
// (value descending, index ascending): top-k tokens by raw logit (ties to the
// smaller token id), candidates and pool nodes by value (ties to the earlier
// pool slot).
#include <float.h>

#include "tv_device.h"
#include "tv_internal.h"

namespace tv {
namespace {

constexpr int kExpandThreads = 512;
constexpr int kExpandWaves = kExpandThreads / kWave;
constexpr int kMaxTopK = 16;
constexpr int kSelectThreads = 1024;
constexpr int kMaxPool = 4096;

// Larger value wins; equal values go to the smaller index.
__device__ __forceinline__ bool better(float v, int i, float v2, int i2) { return v > v2 || (v == v2 && i < i2); }

// A thread's top K of the elements it saw, sorted best first (registers; the
// insertion is unrolled so no array is indexed dynamically).
template <int K>
struct TopK {
    float v[K];
    int i[K];
    __device__ __forceinline__ void init() {
#pragma unroll
        for (int k = 0; k < K; ++k) {
            v[k] = -INFINITY;
            i[k] = 0x7fffffff;
        }
    }
    __device__ __forceinline__ void offer(float x, int idx) {
        if (!better(x, idx, v[K - 1], i[K - 1])) return;
        // from the end: shift worse entries down one place, drop x in the gap
        bool placed = false;
#pragma unroll
        for (int k = K - 1; k >= 0; --k) {
            if (placed) continue;
            if (k > 0 && better(x, idx, v[k - 1], i[k - 1])) {
                v[k] = v[k - 1];
                i[k] = i[k - 1];
            } else {
                v[k] = x;
                i[k] = idx;
                placed = true;
            }
        }
    }
    __device__ __forceinline__ void pop() {
#pragma unroll
        for (int k = 0; k < K - 1; ++k) {
            v[k] = v[k + 1];
            i[k] = i[k + 1];
        }
        v[K - 1] = -INFINITY;
        i[K - 1] = 0x7fffffff;
    }
};

struct ExpandArgs {
    const float* logits;      // [B][F][V]
    const int32_t* frontier;  // [B][F] pool slots, or null: the root
    const int32_t* root_token;
    float* score;             // [B][P]
    int32_t* parent;
    int32_t* token;
    int F, V, P, topk, base;
    double inv_t;             // 1 / T
};

// One workgroup per (sequence, frontier row): a streamed pass (16-byte loads,
// the next chunk in flight while one is processed) keeps each thread's
// running maximum, its fp64 sum of exp((x - max) / T) (rescaled when the
// maximum rises; the exponentials in fp64, four independent ones per chunk)
// and its top K logits; the block then merges the threads' lists in topk
// rounds and writes the candidates.
template <int K, bool VEC4>
__global__ __launch_bounds__(kExpandThreads) void expand_rows_kernel(const ExpandArgs a) {
    const int b = blockIdx.y, f = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int slot = a.frontier ? a.frontier[(size_t)b * a.F + f] : 0;
    const size_t out0 = (size_t)b * a.P + a.base + (size_t)f * a.topk;
    if (!a.frontier && tid == 0) {  // expanding the root: initialise its pool slot
        a.score[(size_t)b * a.P] = 0.f;
        a.parent[(size_t)b * a.P] = -1;
        a.token[(size_t)b * a.P] = a.root_token ? a.root_token[b] : -1;
    }
    if (slot < 0) {  // an empty frontier slot: empty candidates
        for (int j = tid; j < a.topk; j += kExpandThreads) {
            a.score[out0 + j] = -INFINITY;
            a.parent[out0 + j] = -1;
            a.token[out0 + j] = -1;
        }
        return;
    }
    __shared__ double s_tab[32];
    __shared__ float s_wv[kExpandWaves];
    __shared__ int s_wi[kExpandWaves];
    __shared__ double s_ws[kExpandWaves];
    __shared__ float s_wm[kExpandWaves];
    __shared__ int s_pick;
    if (tid < 32) exp2_table(s_tab, tid);
    __syncthreads();

    const float* row = a.logits + ((size_t)b * a.F + f) * a.V;
    const double inv_t = a.inv_t;
    const int V = a.V;
    TopK<K> top;
    top.init();
    float m = -INFINITY;
    double s = 0.0;
    // chunk c covers elements 4c .. 4c+3; thread tid takes chunks tid, tid + T, ...
    const int nchunk = (V + 3) / 4;
    auto load = [&](int ch) {
        f32x4 x;
        const int e = 4 * min(ch, nchunk - 1);
        if constexpr (VEC4) {
            x = *reinterpret_cast<const f32x4*>(row + e);
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) x[k] = row[min(e + k, V - 1)];
        }
        return x;
    };
    auto process = [&](const f32x4& x, int ch) {
        const int e = 4 * ch;
        f32x4 y = x;
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (e + k >= V) y[k] = -INFINITY;
        const float m4 = fmaxf(fmaxf(y[0], y[1]), fmaxf(y[2], y[3]));
        if (m4 > m) {
            if (m != -INFINITY) s *= exp_nonpos(((double)m - (double)m4) * inv_t, s_tab);
            m = m4;
        }
        double e01 = exp_nonpos(((double)y[0] - (double)m) * inv_t, s_tab) +
                     exp_nonpos(((double)y[1] - (double)m) * inv_t, s_tab);
        double e23 = exp_nonpos(((double)y[2] - (double)m) * inv_t, s_tab) +
                     exp_nonpos(((double)y[3] - (double)m) * inv_t, s_tab);
        s += e01 + e23;
#pragma unroll
        for (int k = 0; k < 4; ++k) top.offer(y[k], e + k);
    };
    int ch = tid;
    f32x4 cur = load(ch);
    while (ch < nchunk) {
        const int nx = ch + kExpandThreads;
        const f32x4 nxt = load(nx);
        process(cur, ch);
        cur = nxt;
        ch = nx;
    }
    // row maximum and sum over the block (fixed association: waves in order)
    const float wm = group_max_dpp(m, kWave);
    const double ws = group_sum_dpp(m == -INFINITY ? 0.0 : s * exp_nonpos(((double)m - (double)wm) * inv_t, s_tab),
                                    kWave);
    if (lane == 0) {
        s_wm[wave] = wm;
        s_ws[wave] = ws;
    }
    __syncthreads();
    float M = s_wm[0];
    for (int k = 1; k < kExpandWaves; ++k) M = fmaxf(M, s_wm[k]);
    double S = 0.0;
    for (int k = 0; k < kExpandWaves; ++k)
        if (s_wm[k] != -INFINITY) S += s_ws[k] * exp_nonpos(((double)s_wm[k] - (double)M) * inv_t, s_tab);
    const double lse = log(S);
    const float parent_score = a.frontier ? a.score[(size_t)b * a.P + slot] : 0.f;

    // topk rounds: the block's best head wins and its thread pops it
    for (int j = 0; j < a.topk; ++j) {
        float bv = top.v[0];
        int bi = top.i[0];
        group_argmax_dpp(bv, bi, kWave);
        if (lane == 0) {
            s_wv[wave] = bv;
            s_wi[wave] = bi;
        }
        __syncthreads();
        if (tid == 0) {
            float v0 = s_wv[0];
            int i0 = s_wi[0];
            for (int k = 1; k < kExpandWaves; ++k)
                if (better(s_wv[k], s_wi[k], v0, i0)) {
                    v0 = s_wv[k];
                    i0 = s_wi[k];
                }
            s_pick = i0;
            const bool valid = i0 < V;  // fewer tokens than topk: the rest stay empty
            const double lp = ((double)v0 - (double)M) * inv_t - lse;
            a.score[out0 + j] = valid ? (float)((double)parent_score + lp) : -INFINITY;
            a.parent[out0 + j] = valid ? slot : -1;
            a.token[out0 + j] = valid ? i0 : -1;
        }
        __syncthreads();
        if (top.i[0] == s_pick) top.pop();
        __syncthreads();
    }
}

// Next frontier: the Fn best of this step's candidates (slots base ..
// base + C - 1) by (value, slot); empty candidates never qualify.
__global__ __launch_bounds__(kSelectThreads) void pick_frontier_kernel(const float* __restrict__ score,
                                                                       const int32_t* __restrict__ parent, int P,
                                                                       int base, int C, int32_t* __restrict__ next,
                                                                       int Fn) {
    const int b = blockIdx.x;
    for (int k = threadIdx.x; k < Fn; k += kSelectThreads) next[(size_t)b * Fn + k] = -1;
    __syncthreads();
    const float* sc = score + (size_t)b * P + base;
    const int32_t* pa = parent + (size_t)b * P + base;
    for (int i = threadIdx.x; i < C; i += kSelectThreads) {
        if (pa[i] < 0) continue;
        const float si = sc[i];
        int rank = 0;
        for (int j = 0; j < C; ++j)
            if (pa[j] >= 0 && better(sc[j], j, si, i)) ++rank;
        if (rank < Fn) next[(size_t)b * Fn + rank] = base + i;
    }
}

// Re-ranking: the root plus the m - 1 best valid pool nodes, renumbered in
// pool order (parents precede children, and a kept node's parent is kept: a
// child's value never exceeds its parent's and ties go to the earlier slot).
__global__ __launch_bounds__(kSelectThreads) void select_tree_kernel(const float* __restrict__ score,
                                                                     const int32_t* __restrict__ parent,
                                                                     const int32_t* __restrict__ token, int P,
                                                                     int count, int M, int32_t* __restrict__ out_parent,
                                                                     int32_t* __restrict__ out_token,
                                                                     int32_t* __restrict__ out_index,
                                                                     int32_t* __restrict__ out_nodes) {
    const int b = blockIdx.x;
    __shared__ float s_sc[kMaxPool];
    __shared__ int s_pa[kMaxPool];
    __shared__ int s_new[kMaxPool];  // keep flag, then the new index
    __shared__ int s_wsum[kSelectThreads / kWave];
    const float* sc = score + (size_t)b * P;
    const int32_t* pa = parent + (size_t)b * P;
    for (int i = threadIdx.x; i < count; i += kSelectThreads) {
        s_sc[i] = sc[i];
        s_pa[i] = pa[i];
    }
    __syncthreads();
    for (int i = threadIdx.x; i < count; i += kSelectThreads) {
        int keep = i == 0;
        if (i > 0 && s_pa[i] >= 0) {
            const float si = s_sc[i];
            int rank = 0;
            for (int j = 1; j < count; ++j)
                if (s_pa[j] >= 0 && better(s_sc[j], j, si, i)) ++rank;
            keep = rank < M - 1;
        }
        s_new[i] = keep;
    }
    __syncthreads();
    // new index = kept slots before i (exclusive scan in chunks of the block)
    int carry = 0;
    for (int c0 = 0; c0 < count; c0 += kSelectThreads) {
        const int i = c0 + threadIdx.x;
        const int k = i < count ? s_new[i] : 0;
        const uint64_t bal = __ballot(k);
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        const int before = __popcll(bal & ((1ull << lane) - 1ull));
        if (lane == 0) s_wsum[wave] = __popcll(bal);
        __syncthreads();
        int off = carry, tot = 0;
        for (int w = 0; w < kSelectThreads / kWave; ++w) {
            if (w < wave) off += s_wsum[w];
            tot += s_wsum[w];
        }
        __syncthreads();
        if (i < count) s_new[i] = k ? off + before : -1;
        carry += tot;
    }
    __syncthreads();
    const int n = carry;
    for (int i = threadIdx.x; i < M; i += kSelectThreads) {
        out_parent[(size_t)b * M + i] = -1;
        out_token[(size_t)b * M + i] = -1;
        out_index[(size_t)b * M + i] = -1;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < count; i += kSelectThreads) {
        const int ni = s_new[i];
        if (ni < 0) continue;
        out_parent[(size_t)b * M + ni] = i == 0 ? -1 : s_new[s_pa[i]];
        out_token[(size_t)b * M + ni] = token[(size_t)b * P + i];
        out_index[(size_t)b * M + ni] = i;
    }
    if (threadIdx.x == 0) out_nodes[b] = n;
}

template <int K>
int launch_expand(const ExpandArgs& a, int B, int Frows, bool vec4, hipStream_t st) {
    if (vec4)
        hipLaunchKernelGGL((expand_rows_kernel<K, true>), dim3(Frows, B), dim3(kExpandThreads), 0, st, a);
    else
        hipLaunchKernelGGL((expand_rows_kernel<K, false>), dim3(Frows, B), dim3(kExpandThreads), 0, st, a);
    return launch_status();
}

}  // namespace
}  // namespace tv

extern "C" int tv_tree_expand(const float* draft_logits, const int32_t* frontier, const int32_t* root_token, int B,
                              int F, int V, int topk, float temperature, float* pool_score, int32_t* pool_parent,
                              int32_t* pool_token, int P, int pool_base, int32_t* next_frontier, int Fn,
                              void* stream) {
    using namespace tv;
    if (B < 0 || F < 1 || V < 1 || topk < 1 || Fn < 0 || P < 1 || pool_base < 1) return TV_ERR_INVALID_ARG;
    if (!frontier && F != 1) return TV_ERR_INVALID_ARG;  // the root step has one row
    if (topk > kMaxTopK) return TV_ERR_UNSUPPORTED;
    if (!(temperature > 0.f && temperature <= FLT_MAX)) return TV_ERR_INVALID_ARG;
    if ((long)pool_base + (long)F * topk > P) return TV_ERR_INVALID_ARG;
    if (B == 0) return TV_OK;
    if (B > 65535 || F > 0x7fffffff / topk) return TV_ERR_UNSUPPORTED;
    if (!draft_logits || !pool_score || !pool_parent || !pool_token || (Fn > 0 && !next_frontier))
        return TV_ERR_INVALID_ARG;
    ExpandArgs a;
    a.logits = draft_logits;
    a.frontier = frontier;
    a.root_token = root_token;
    a.score = pool_score;
    a.parent = pool_parent;
    a.token = pool_token;
    a.F = F;
    a.V = V;
    a.P = P;
    a.topk = topk;
    a.base = pool_base;
    a.inv_t = 1.0 / (double)temperature;
    hipStream_t st = (hipStream_t)stream;
    const bool vec4 = V % 4 == 0 && aligned(draft_logits, 16);
    int rc;
    if (topk <= 1)
        rc = launch_expand<1>(a, B, F, vec4, st);
    else if (topk <= 2)
        rc = launch_expand<2>(a, B, F, vec4, st);
    else if (topk <= 4)
        rc = launch_expand<4>(a, B, F, vec4, st);
    else if (topk <= 8)
        rc = launch_expand<8>(a, B, F, vec4, st);
    else
        rc = launch_expand<16>(a, B, F, vec4, st);
    if (rc != TV_OK || Fn == 0) return rc;
    hipLaunchKernelGGL(pick_frontier_kernel, dim3(B), dim3(kSelectThreads), 0, st, pool_score, pool_parent, P,
                       pool_base, F * topk, next_frontier, Fn);
    return launch_status();
}

extern "C" int tv_tree_select(const float* pool_score, const int32_t* pool_parent, const int32_t* pool_token, int B,
                              int P, int pool_count, int M, int32_t* parent, int32_t* tokens, int32_t* pool_index,
                              int32_t* seq_nodes, void* stream) {
    using namespace tv;
    if (B < 0 || P < 1 || pool_count < 1 || pool_count > P || M < 1) return TV_ERR_INVALID_ARG;
    if (pool_count > kMaxPool || M > TV_MAX_NODES) return TV_ERR_UNSUPPORTED;
    if (B == 0) return TV_OK;
    if (!pool_score || !pool_parent || !pool_token || !parent || !tokens || !pool_index || !seq_nodes)
        return TV_ERR_INVALID_ARG;
    hipLaunchKernelGGL(select_tree_kernel, dim3(B), dim3(kSelectThreads), 0, (hipStream_t)stream, pool_score,
                       pool_parent, pool_token, P, pool_count, M, parent, tokens, pool_index, seq_nodes);
    return launch_status();
}
