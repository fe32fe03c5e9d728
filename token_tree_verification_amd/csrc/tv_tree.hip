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

// Wave-level top-k: each wave keeps, in LDS, its best k elements so far
// (sorted best first) followed by the new elements that beat the k-th of them;
// a ballot compacts those into the buffer, and when the buffer could overflow
// the wave re-selects its best k from it (k rounds of a wave argmax).  After
// the first few batches almost nothing beats the k-th best, so an element
// costs one comparison.  (A per-thread sorted list instead made nearly every
// element run the insertion in some lane of the wave.)
constexpr int kCandCap = 4 * kWave * 2 + kMaxTopK;  // two batches of candidates plus the kept k

struct WaveTop {
    float* v;  // [kCandCap] this wave's buffer in LDS
    int* i;
};

// Re-select the best k of the first n buffer entries into entries 0..k-1
// (sorted best first); returns the new count (min(n, k)).  Wave-uniform.
__device__ int wave_select(WaveTop t, int n, int k) {
    const int lane = threadIdx.x & 63;
    // the selected entries go to a scratch tail and are copied back at the end
    float* ov = t.v + kCandCap - kMaxTopK;
    int* oi = t.i + kCandCap - kMaxTopK;
    const int m = min(n, k);
    for (int j = 0; j < m; ++j) {
        float bv = -INFINITY;
        int bi = 0x7fffffff, bp = -1;
        for (int p = lane; p < n; p += kWave) {
            const float v = t.v[p];
            const int i = t.i[p];
            if (bp < 0 || better(v, i, bv, bi)) {
                bv = v;
                bi = i;
                bp = p;
            }
        }
        int key = bi;
        float kv = bv;
        group_argmax_dpp(kv, key, kWave);  // ties to the smaller index
        // the lane holding the winner removes it
        if (bp >= 0 && bi == key && bv == kv) t.i[bp] = 0x7fffffff, t.v[bp] = -INFINITY;
        if (lane == 0) {
            ov[j] = kv;
            oi[j] = key;
        }
        __builtin_amdgcn_wave_barrier();
    }
    for (int j = lane; j < m; j += kWave) {
        t.v[j] = ov[j];
        t.i[j] = oi[j];
    }
    __builtin_amdgcn_wave_barrier();
    return m;
}

// One workgroup per (sequence, frontier row).  Wave w streams batches of 256
// logits w, w + 8, ... (16-byte loads, the next batch in flight); each lane
// keeps its running maximum and an fp64 sum of exp((x - max) / T) (our fp64
// exponential, four independent ones per batch, rescaled when the maximum
// rises); the wave keeps its top k as above.  The block then combines the
// waves' maxima and sums (waves in order) and wave 0 selects the row's top k
// from the eight wave lists.
template <bool VEC4>
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
    __shared__ float s_cv[kExpandWaves][kCandCap];
    __shared__ int s_ci[kExpandWaves][kCandCap];
    __shared__ double s_ws[kExpandWaves];
    __shared__ float s_wm[kExpandWaves];
    __shared__ int s_wn[kExpandWaves];
    if (tid < 32) exp2_table(s_tab, tid);
    __syncthreads();

    const float* row = a.logits + ((size_t)b * a.F + f) * a.V;
    const double inv_t = a.inv_t;
    const int V = a.V, k = a.topk;
    WaveTop top{s_cv[wave], s_ci[wave]};
    int n = 0;                       // buffer entries (wave-uniform)
    float tv = -INFINITY;            // the k-th best so far (wave-uniform), or none yet
    int ti = 0x7fffffff;
    bool full = false;
    float m = -INFINITY;
    double s = 0.0;
    const int nbatch = (V + 4 * kWave - 1) / (4 * kWave);
    auto load = [&](int bt) {
        f32x4 x;
        const int e = 4 * (min(bt, nbatch - 1) * kWave + lane);
        if constexpr (VEC4) {
            x = *reinterpret_cast<const f32x4*>(row + min(e, V - 4));
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) x[q] = row[min(e + q, V - 1)];
        }
        return x;
    };
    int bt = wave;
    f32x4 cur = load(bt);
    while (bt < nbatch) {
        const int nx = bt + kExpandWaves;
        const f32x4 nxt = load(nx);
        const int e = 4 * (bt * kWave + lane);
        f32x4 y = cur;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (e + q >= V) y[q] = -INFINITY;
        // softmax statistics
        const float m4 = fmaxf(fmaxf(y[0], y[1]), fmaxf(y[2], y[3]));
        if (m4 > m) {
            if (m != -INFINITY) s *= exp_nonpos(((double)m - (double)m4) * inv_t, s_tab);
            m = m4;
        }
        if (m != -INFINITY) {
            const double e01 = exp_nonpos(((double)y[0] - (double)m) * inv_t, s_tab) +
                               exp_nonpos(((double)y[1] - (double)m) * inv_t, s_tab);
            const double e23 = exp_nonpos(((double)y[2] - (double)m) * inv_t, s_tab) +
                               exp_nonpos(((double)y[3] - (double)m) * inv_t, s_tab);
            s += e01 + e23;
        }
        // candidates: valid elements that beat the k-th best so far
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const bool pass = e + q < V && (!full || better(y[q], e + q, tv, ti));
            const uint64_t bal = __ballot(pass);
            if (pass) {
                const int pos = n + __popcll(bal & ((1ull << lane) - 1ull));
                top.v[pos] = y[q];
                top.i[pos] = e + q;
            }
            n += __popcll(bal);
        }
        __builtin_amdgcn_wave_barrier();
        if (n > kCandCap - kMaxTopK - 4 * kWave) {  // the next batch could overflow: re-select
            n = wave_select(top, n, k);
            full = n >= k;
            if (full) {
                tv = top.v[k - 1];
                ti = top.i[k - 1];
            }
        }
        cur = nxt;
        bt = nx;
    }
    n = wave_select(top, n, k);
    // row maximum and sum over the block (fixed association: waves in order)
    const float wm = group_max_dpp(m, kWave);
    const double ws = group_sum_dpp(m == -INFINITY ? 0.0 : s * exp_nonpos(((double)m - (double)wm) * inv_t, s_tab),
                                    kWave);
    if (lane == 0) {
        s_wm[wave] = wm;
        s_ws[wave] = ws;
        s_wn[wave] = n;
    }
    __syncthreads();
    if (wave != 0) return;
    float M = s_wm[0];
    for (int q = 1; q < kExpandWaves; ++q) M = fmaxf(M, s_wm[q]);
    double S = 0.0;
    for (int q = 0; q < kExpandWaves; ++q)
        if (s_wm[q] != -INFINITY) S += s_ws[q] * exp_nonpos(((double)s_wm[q] - (double)M) * inv_t, s_tab);
    const double lse = log(S);
    const float parent_score = a.frontier ? a.score[(size_t)b * a.P + slot] : 0.f;
    // gather the waves' lists into wave 0's buffer (after its own k entries)
    int cnt = s_wn[0];
    for (int w = 1; w < kExpandWaves; ++w) {
        const int nw = s_wn[w];
        for (int j = lane; j < nw; j += kWave) {
            top.v[cnt + j] = s_cv[w][j];
            top.i[cnt + j] = s_ci[w][j];
        }
        cnt += nw;
    }
    __builtin_amdgcn_wave_barrier();
    const int got = wave_select(top, cnt, k);
    for (int j = lane; j < k; j += kWave) {
        const bool valid = j < got && top.i[j] < V;  // fewer tokens than topk: the rest stay empty
        const double lp = ((double)top.v[j] - (double)M) * inv_t - lse;
        a.score[out0 + j] = valid ? (float)((double)parent_score + lp) : -INFINITY;
        a.parent[out0 + j] = valid ? slot : -1;
        a.token[out0 + j] = valid ? top.i[j] : -1;
    }
}

// Next frontier: the Fn best of this step's candidates (slots base ..
// base + C - 1) by (value, slot); empty candidates never qualify.  One thread
// per candidate counts the candidates that beat it (staged in LDS when they
// fit).
__global__ __launch_bounds__(kSelectThreads) void pick_frontier_kernel(const float* __restrict__ score,
                                                                       const int32_t* __restrict__ parent, int P,
                                                                       int base, int C, int32_t* __restrict__ next,
                                                                       int Fn) {
    const int b = blockIdx.x;
    __shared__ float s_sc[kMaxPool];
    for (int k = threadIdx.x; k < Fn; k += kSelectThreads) next[(size_t)b * Fn + k] = -1;
    const float* sc = score + (size_t)b * P + base;
    const int32_t* pa = parent + (size_t)b * P + base;
    const bool staged = C <= kMaxPool;
    if (staged)  // empty candidates enter as NaN, which never beats or ties anything
        for (int i = threadIdx.x; i < C; i += kSelectThreads) s_sc[i] = pa[i] >= 0 ? sc[i] : __builtin_nanf("");
    __syncthreads();
    for (int i = threadIdx.x; i < C; i += kSelectThreads) {
        if (pa[i] < 0) continue;
        const float si = sc[i];
        int rank = 0;
        if (staged) {
            for (int j = 0; j < C; ++j) rank += better(s_sc[j], j, si, i);
        } else {
            for (int j = 0; j < C; ++j)
                if (pa[j] >= 0 && better(sc[j], j, si, i)) ++rank;
        }
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

int launch_expand(const ExpandArgs& a, int B, int Frows, bool vec4, hipStream_t st) {
    if (vec4)
        hipLaunchKernelGGL((expand_rows_kernel<true>), dim3(Frows, B), dim3(kExpandThreads), 0, st, a);
    else
        hipLaunchKernelGGL((expand_rows_kernel<false>), dim3(Frows, B), dim3(kExpandThreads), 0, st, a);
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
    const int rc = launch_expand(a, B, F, vec4, st);
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
