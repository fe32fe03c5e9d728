// tv_spec_accept: greedy and lossless speculative-sampling accept/reject walk
// over a draft tree.
//
// Survey explainer (paper-2401-07851), formal definition, accept/reject phase:
// accept draft x when r < min(1, q(x)/p(x)), r ~ U[0,1]; at the first
// rejection draw from norm(max(0, q - p)); K+1 target rows let the walk always
// emit one extra token.  Same page, classification of verification methods:
// greedy verification keeps drafts equal to the target's greedy choice;
// token-tree verification checks every candidate path and stays lossless.
//
// Pass 1 (accept_stats_kernel) streams every logit row once with coalesced
// 16-byte loads, split over vocabulary chunks so even a single sequence fills
// the GPU: per (row, chunk) it keeps the running max and the sum of
// exp(z - max) of z = logits / T (sampling), or the max and its first index
// (greedy).  Pass 2 (accept_walk_kernel) runs one 1024-lane workgroup per
// sequence: it merges the chunk partials, walks the tree (children in index
// order, Philox-4x32-10 uniforms keyed by (node, sequence, purpose)), runs a
// vocabulary pass for every rejection to build the residual
// max(0, R - P_c), and draws the extra token by inverse CDF.
#include "tv_device.h"
#include "tv_internal.h"

namespace tv {
namespace {

constexpr int kStatsThreads = 256;
constexpr int kStatsPerThread = 16;
constexpr int kChunk = kStatsThreads * kStatsPerThread;  // logits per stats workgroup
constexpr int kWalkThreads = 1024;
constexpr int kWalkWaves = kWalkThreads / kWave;

struct AcceptLayout {
    int nchunk;
    size_t stats_bytes, resid_offset, total;
};

AcceptLayout accept_layout(int B, int N, int V, int greedy) {
    AcceptLayout l;
    l.nchunk = (V + kChunk - 1) / kChunk;
    l.stats_bytes = round_up((size_t)B * 2 * N * l.nchunk * sizeof(float2), 256);
    l.resid_offset = l.stats_bytes;
    l.total = l.stats_bytes + (greedy ? 0 : round_up((size_t)B * 2 * V * sizeof(float), 256));
    return l;
}

// (max, sum exp(z - max)) merge
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
    const float M = fmaxf(m, m2);
    if (M == -INFINITY) return;
    s = s * exp2f((m - M) * 1.4426950408889634f) + s2 * exp2f((m2 - M) * 1.4426950408889634f);
    m = M;
}

// Larger value wins; on equal values the smaller index wins.
__device__ __forceinline__ void argmax_merge(float& v, int& i, float v2, int i2) {
    if (v2 > v || (v2 == v && i2 < i)) {
        v = v2;
        i = i2;
    }
}

// grid: (B * rows_per_seq, nchunk).  Sampling rows: q rows 0..N-1 then p rows
// 1..N-1; greedy rows: q rows 0..N-1.  Output: stats[(b*2N + row)*nchunk + chunk],
// row = u for q row u and N + c for p row c.
template <bool GREEDY, bool VEC4>
__global__ __launch_bounds__(kStatsThreads) void accept_stats_kernel(const float* __restrict__ q,
                                                                     const float* __restrict__ p, int N, int V,
                                                                     float inv_t, int rows_per_seq, int nchunk,
                                                                     float2* __restrict__ stats) {
    const int chunk = blockIdx.y;
    const int b = blockIdx.x / rows_per_seq;
    const int ri = blockIdx.x % rows_per_seq;
    const bool is_q = ri < N;
    const int row = is_q ? ri : ri + 1;  // p rows are stored at N + c, c >= 1
    const float* src = is_q ? q + ((size_t)b * N + ri) * V : p + ((size_t)b * N + (ri - N + 1)) * V;
    const int tid = threadIdx.x;
    const int c0 = chunk * kChunk;

    float vals[kStatsPerThread];
#pragma unroll
    for (int i = 0; i < kStatsPerThread / 4; ++i) {
        const int v0 = c0 + 4 * (tid + kStatsThreads * i);
        if (VEC4 && v0 + 3 < V) {
            const f32x4 x = *reinterpret_cast<const f32x4*>(src + v0);
            vals[4 * i] = x[0];
            vals[4 * i + 1] = x[1];
            vals[4 * i + 2] = x[2];
            vals[4 * i + 3] = x[3];
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) vals[4 * i + j] = (v0 + j < V) ? src[v0 + j] : -INFINITY;
        }
    }

    __shared__ float red_a[kStatsThreads / kWave];
    __shared__ float red_b[kStatsThreads / kWave];
    const int lane = tid & 63, wave = tid >> 6;
    if (GREEDY) {
        float bv = -INFINITY;
        int bi = 0x7fffffff;
#pragma unroll
        for (int i = 0; i < kStatsPerThread; ++i) {
            const int v = c0 + 4 * (tid + kStatsThreads * (i >> 2)) + (i & 3);
            if (v < V && vals[i] > bv) {
                bv = vals[i];
                bi = v;
            }
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) argmax_merge(bv, bi, __shfl_xor(bv, o), __shfl_xor(bi, o));
        if (lane == 0) {
            red_a[wave] = bv;
            red_b[wave] = __int_as_float(bi);
        }
        __syncthreads();
        if (tid == 0) {
            for (int w = 1; w < kStatsThreads / kWave; ++w) argmax_merge(bv, bi, red_a[w], __float_as_int(red_b[w]));
            stats[((size_t)b * 2 * N + row) * nchunk + chunk] = float2{bv, __int_as_float(bi)};
        }
    } else {
        float m = -INFINITY;
#pragma unroll
        for (int i = 0; i < kStatsPerThread; ++i) {
            vals[i] *= inv_t;
            m = fmaxf(m, vals[i]);
        }
        m = wave_max(m);
        if (lane == 0) red_a[wave] = m;
        __syncthreads();
        float M = red_a[0];
#pragma unroll
        for (int w = 1; w < kStatsThreads / kWave; ++w) M = fmaxf(M, red_a[w]);
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < kStatsPerThread; ++i) s += __expf(vals[i] - M);
        s = wave_sum(s);
        if (lane == 0) red_b[wave] = s;
        __syncthreads();
        if (tid == 0) {
            float S = 0.f;
            for (int w = 0; w < kStatsThreads / kWave; ++w) S += red_b[w];
            stats[((size_t)b * 2 * N + row) * nchunk + chunk] = float2{M, S};
        }
    }
}

struct WalkArgs {
    const float* q;
    const float* p;
    const int32_t* draft;
    const int32_t* parent;
    const float2* stats;
    float* resid;  // [B][2][V]
    int32_t* accept_len;
    int32_t* accepted;
    int32_t* tokens;
    int N, V, nchunk;
    float inv_t;
    uint64_t seed;
};

__device__ __forceinline__ float block_sum(float v, float* red, int tid) {
    v = wave_sum(v);
    __syncthreads();
    if ((tid & 63) == 0) red[tid >> 6] = v;
    __syncthreads();
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < kWalkWaves; ++w) s += red[w];
    return s;
}

template <bool GREEDY>
__global__ __launch_bounds__(kWalkThreads) void accept_walk_kernel(const WalkArgs a) {
    const int b = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int N = a.N, V = a.V;
    __shared__ int s_par[TV_MAX_NODES], s_draft[TV_MAX_NODES];
    __shared__ float s_m[2 * TV_MAX_NODES], s_s[2 * TV_MAX_NODES];
    __shared__ int s_amax[TV_MAX_NODES];
    __shared__ float red[kWalkWaves];
    __shared__ float s_wsum[kWalkWaves];
    __shared__ int s_ok, s_dec, s_tok;

    if (tid < kWave) {
        int ok = 1;
        if (tid < N) {
            const int pr = a.parent[(size_t)b * N + tid];
            int d = a.draft[(size_t)b * N + tid];
            d = d < 0 ? 0 : (d >= V ? V - 1 : d);  // out-of-range drafts are a precondition violation
            s_par[tid] = pr;
            s_draft[tid] = d;
            ok = tid == 0 ? pr == -1 : (pr >= 0 && pr < tid);
        }
        const bool all_ok = __all(ok);
        if (tid == 0) s_ok = all_ok;
    }
    // merge the per-chunk statistics of every row (one wave per row)
    const int nrows = GREEDY ? N : 2 * N;
    for (int row = wave; row < nrows; row += kWalkWaves) {
        if (!GREEDY && row == N) continue;  // p row 0 is unused
        const float2* st = a.stats + ((size_t)b * 2 * N + row) * a.nchunk;
        if (GREEDY) {
            float bv = -INFINITY;
            int bi = 0x7fffffff;
            for (int j = lane; j < a.nchunk; j += kWave) argmax_merge(bv, bi, st[j].x, __float_as_int(st[j].y));
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) argmax_merge(bv, bi, __shfl_xor(bv, o), __shfl_xor(bi, o));
            if (lane == 0) s_amax[row] = bi;
        } else {
            float m = -INFINITY, s = 0.f;
            for (int j = lane; j < a.nchunk; j += kWave) lse_merge(m, s, st[j].x, st[j].y);
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) {
                const float m2 = __shfl_xor(m, o), s2 = __shfl_xor(s, o);
                lse_merge(m, s, m2, s2);
            }
            if (lane == 0) {
                s_m[row] = m;
                s_s[row] = s;
            }
        }
    }
    __syncthreads();

    int32_t* out_nodes = a.accepted + (size_t)b * N;
    int32_t* out_toks = a.tokens + (size_t)b * N;
    for (int i = tid; i < N; i += kWalkThreads) {
        out_nodes[i] = -1;
        out_toks[i] = -1;
    }
    __syncthreads();  // the -1 fill must land before thread 0 writes the path
    if (!s_ok) {
        if (tid == 0) a.accept_len[b] = -1;
        return;
    }

    if (GREEDY) {
        if (tid == 0) {
            // valid(i): every draft on the root-to-i path equals its parent's argmax
            uint64_t valid = 1ull;
            int depth[TV_MAX_NODES];
            depth[0] = 0;
            int e = 0;
            for (int i = 1; i < N; ++i) {
                const int pr = s_par[i];
                depth[i] = depth[pr] + 1;
                if (((valid >> pr) & 1ull) && s_draft[i] == s_amax[pr]) {
                    valid |= 1ull << i;
                    if (depth[i] > depth[e]) e = i;
                }
            }
            const int len = depth[e];
            for (int i = e, k = len - 1; i != 0; i = s_par[i], --k) {
                out_nodes[k] = i;
                out_toks[k] = s_draft[i];
            }
            out_toks[len] = s_amax[e];
            a.accept_len[b] = len;
        }
        return;
    }

    // ---------------------------- sampling walk ----------------------------
    const float* qb = a.q + (size_t)b * N * V;
    const float* pb = a.p + (size_t)b * N * V;
    float* rbuf[2] = {a.resid + (size_t)b * 2 * V, a.resid + (size_t)b * 2 * V + V};
    const float inv_t = a.inv_t;
    int u = 0, len = 0, cur = 0;
    bool res_active = false;  // target at u: residual rbuf[cur]/Z, else softmax(q_u / T)
    float Z = 1.f;
    int c = 1;  // next child candidate index to scan from
    for (;;) {
        // next child of u at index >= c (children are later nodes)
        while (c < N && s_par[c] != u) ++c;
        if (c >= N) break;  // no (more) children: stop at u
        if (tid == 0) {
            const int x = s_draft[c];
            const float qm = s_m[u], qs = s_s[u];
            const float pm = s_m[N + c], ps = s_s[N + c];
            const float rx = res_active ? rbuf[cur][x] / Z : __expf(qb[(size_t)u * V + x] * inv_t - qm) / qs;
            const float px = __expf(pb[(size_t)c * V + x] * inv_t - pm) / ps;
            const float acc = px == 0.f ? 1.f : fminf(1.f, rx / px);
            const float r = philox_uniform(a.seed, (uint32_t)c, (uint32_t)b, 0u);
            s_dec = r < acc;
        }
        __syncthreads();
        const bool accepted = s_dec;
        __syncthreads();
        if (accepted) {
            if (tid == 0) {
                out_nodes[len] = c;
                out_toks[len] = s_draft[c];
            }
            ++len;
            u = c;
            c = u + 1;
            res_active = false;
            Z = 1.f;
            continue;
        }
        // rejected: R <- max(0, R - P_c) (kept unnormalised with its sum Z)
        {
            const float qm = s_m[u], qs = s_s[u];
            const float pm = s_m[N + c], ps = s_s[N + c];
            const float* qrow = qb + (size_t)u * V;
            const float* prow = pb + (size_t)c * V;
            const float* src = rbuf[cur];
            float* dst = rbuf[cur ^ 1];
            const float invZ = 1.f / Z, invqs = 1.f / qs, invps = 1.f / ps;
            float part = 0.f;
            for (int v = tid; v < V; v += kWalkThreads) {
                const float rv = res_active ? src[v] * invZ : __expf(qrow[v] * inv_t - qm) * invqs;
                const float pv = __expf(prow[v] * inv_t - pm) * invps;
                const float w = fmaxf(0.f, rv - pv);
                dst[v] = w;
                part += w;
            }
            const float Znew = block_sum(part, red, tid);
            if (Znew > 0.f) {
                cur ^= 1;
                Z = Znew;
                res_active = true;
            }
        }
        ++c;
    }

    // final draw: smallest k with prefix(w)[k] > U * sum(w), w = residual or
    // exp(q_u/T - max); each wave owns a contiguous segment of the vocabulary
    const float ut = philox_uniform(a.seed, (uint32_t)u, (uint32_t)b, 1u);
    const float qm = s_m[u];
    const float* qrow = qb + (size_t)u * V;
    const float* src = rbuf[cur];
    const int seg = (V + kWalkWaves - 1) / kWalkWaves;
    const int s0 = wave * seg;
    const int s1 = s0 + seg < V ? s0 + seg : V;
    float part = 0.f;
    for (int v = s0 + lane; v < s1; v += kWave)
        part += res_active ? src[v] : __expf(qrow[v] * inv_t - qm);
    part = wave_sum(part);
    if (lane == 0) s_wsum[wave] = part;
    if (tid == 0) s_tok = -1;
    __syncthreads();
    float total = 0.f;
    for (int w = 0; w < kWalkWaves; ++w) total += s_wsum[w];
    const float target = ut * total;
    float before = 0.f;
    int w_sel = -1;
    for (int w = 0; w < kWalkWaves; ++w) {
        if (before + s_wsum[w] > target) {
            w_sel = w;
            break;
        }
        before += s_wsum[w];
    }
    if (wave == w_sel) {
        float run = before;
        int found = -1, last_pos = -1;
        for (int v0 = s0; v0 < s1 && found < 0; v0 += kWave) {
            const int v = v0 + lane;
            const float w = v < s1 ? (res_active ? src[v] : __expf(qrow[v] * inv_t - qm)) : 0.f;
            float incl = w;
#pragma unroll
            for (int o = 1; o < kWave; o <<= 1) {
                const float t = __shfl_up(incl, o);
                if (lane >= o) incl += t;
            }
            const uint64_t hit = __ballot(run + incl > target && w > 0.f);
            const uint64_t pos = __ballot(w > 0.f);
            if (hit) found = v0 + __ffsll((unsigned long long)hit) - 1;
            if (pos) last_pos = v0 + 63 - __clzll((unsigned long long)pos);
            run += __shfl(incl, 63);
        }
        if (lane == 0) s_tok = found >= 0 ? found : last_pos;
    }
    __syncthreads();
    if (tid == 0) {
        int tok = s_tok;
        if (tok < 0) {
            // rounding left the target beyond the total: last token with mass
            for (int v = V - 1; v >= 0; --v) {
                const float w = res_active ? src[v] : __expf(qrow[v] * inv_t - qm);
                if (w > 0.f) {
                    tok = v;
                    break;
                }
            }
            if (tok < 0) tok = V - 1;
        }
        out_toks[len] = tok;
        a.accept_len[b] = len;
    }
}

__global__ void philox_audit_kernel(uint64_t seed, const uint32_t* __restrict__ triples, int n,
                                    float* __restrict__ out_u, uint32_t* __restrict__ out_raw) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const u32x4 r = philox4x32_10(u32x4{triples[3 * i], triples[3 * i + 1], triples[3 * i + 2], 0u}, (uint32_t)seed,
                                  (uint32_t)(seed >> 32));
    if (out_u) out_u[i] = (float)(r.x >> 8) * (1.0f / 16777216.0f);
    if (out_raw) {
        out_raw[4 * i] = r.x;
        out_raw[4 * i + 1] = r.y;
        out_raw[4 * i + 2] = r.z;
        out_raw[4 * i + 3] = r.w;
    }
}

}  // namespace
}  // namespace tv

extern "C" size_t tv_spec_accept_workspace(int B, int N, int V, int greedy) {
    if (B <= 0 || N < 1 || N > TV_MAX_NODES || V < 1) return 0;
    return tv::accept_layout(B, N, V, greedy).total;
}

extern "C" int tv_spec_accept(const float* q_logits, const float* p_logits, const int32_t* draft_tokens,
                              const int32_t* parent, int B, int N, int V, uint64_t philox_seed, float temperature,
                              int greedy, int32_t* accept_len, int32_t* accepted_nodes, int32_t* out_tokens,
                              void* workspace, size_t workspace_bytes, void* stream) {
    using namespace tv;
    if (B < 0 || N < 1 || V < 1) return TV_ERR_INVALID_ARG;
    if (N > TV_MAX_NODES) return TV_ERR_UNSUPPORTED;
    if (!greedy && !(temperature > 0.f && temperature <= 3.4e38f)) return TV_ERR_INVALID_ARG;
    if (B == 0) return TV_OK;
    if (!q_logits || (!greedy && !p_logits) || !draft_tokens || !parent || !accept_len || !accepted_nodes ||
        !out_tokens)
        return TV_ERR_INVALID_ARG;
    if (!aligned(q_logits, 4) || (!greedy && !aligned(p_logits, 4))) return TV_ERR_INVALID_ARG;
    const AcceptLayout lay = accept_layout(B, N, V, greedy);
    if (!workspace || workspace_bytes < lay.total || !aligned(workspace, 256)) return TV_ERR_WORKSPACE;
    const int rows_per_seq = greedy ? N : 2 * N - 1;
    if ((long)B * rows_per_seq > 0x7fffffffL || lay.nchunk > 65535) return TV_ERR_UNSUPPORTED;

    hipStream_t st = (hipStream_t)stream;
    float2* stats = static_cast<float2*>(workspace);
    const float inv_t = greedy ? 1.f : (float)(1.0 / (double)temperature);
    const bool vec4 = (V % 4 == 0) && aligned(q_logits, 16) && (greedy || aligned(p_logits, 16));
    const dim3 grid(B * rows_per_seq, lay.nchunk);
    if (greedy) {
        if (vec4)
            hipLaunchKernelGGL((accept_stats_kernel<true, true>), grid, dim3(kStatsThreads), 0, st, q_logits, p_logits,
                               N, V, inv_t, rows_per_seq, lay.nchunk, stats);
        else
            hipLaunchKernelGGL((accept_stats_kernel<true, false>), grid, dim3(kStatsThreads), 0, st, q_logits,
                               p_logits, N, V, inv_t, rows_per_seq, lay.nchunk, stats);
    } else {
        if (vec4)
            hipLaunchKernelGGL((accept_stats_kernel<false, true>), grid, dim3(kStatsThreads), 0, st, q_logits,
                               p_logits, N, V, inv_t, rows_per_seq, lay.nchunk, stats);
        else
            hipLaunchKernelGGL((accept_stats_kernel<false, false>), grid, dim3(kStatsThreads), 0, st, q_logits,
                               p_logits, N, V, inv_t, rows_per_seq, lay.nchunk, stats);
    }
    if (hipGetLastError() != hipSuccess) return TV_ERR_HIP;

    WalkArgs w;
    w.q = q_logits;
    w.p = p_logits;
    w.draft = draft_tokens;
    w.parent = parent;
    w.stats = stats;
    w.resid = greedy ? nullptr : reinterpret_cast<float*>(static_cast<char*>(workspace) + lay.resid_offset);
    w.accept_len = accept_len;
    w.accepted = accepted_nodes;
    w.tokens = out_tokens;
    w.N = N;
    w.V = V;
    w.nchunk = lay.nchunk;
    w.inv_t = inv_t;
    w.seed = philox_seed;
    if (greedy)
        hipLaunchKernelGGL(accept_walk_kernel<true>, dim3(B), dim3(kWalkThreads), 0, st, w);
    else
        hipLaunchKernelGGL(accept_walk_kernel<false>, dim3(B), dim3(kWalkThreads), 0, st, w);
    return launch_status();
}

extern "C" int tv_philox_uniforms(uint64_t seed, const uint32_t* triples, int n, float* out_u, uint32_t* out_raw,
                                  void* stream) {
    if (n < 0) return TV_ERR_INVALID_ARG;
    if (n == 0) return TV_OK;
    if (!triples || (!out_u && !out_raw)) return TV_ERR_INVALID_ARG;
    hipLaunchKernelGGL(tv::philox_audit_kernel, dim3((n + 255) / 256), dim3(256), 0, (hipStream_t)stream, seed,
                       triples, n, out_u, out_raw);
    return tv::launch_status();
}
