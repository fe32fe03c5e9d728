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
// One launch.  A team of W workgroups owns one sequence at a time; member w
// owns vocabulary slice w of every logit row.
//  1. Statistics: each member streams its slice of every row once (coalesced
//     16-byte loads, several rows in flight per wave) and publishes the slice
//     max and sum of exp((x - max)/T) -- or the max and its first index in
//     greedy mode.  Rows whose exact normaliser is likely needed (all rows of
//     small problems, otherwise the root's target row and the draft rows of
//     its children) also get an fp64 slice sum.
//  2. Team barrier.  Every member then runs the same walk redundantly: the
//     decisions only need merged row statistics and a few gathered logits,
//     so all members agree bit for bit without communicating.
//  3. A rejection needs vocabulary passes: missing fp64 normalisers of the
//     parent target and the rejected child's draft row, then the residual
//     max(0, R - P_c) over the slices in fp64 (kept per team), each followed by
//     a team barrier.  The residual pass also forms the next sibling's fp64
//     normaliser in case it is rejected too.
//  4. The extra token: every member publishes the fp64 mass of its slice, and
//     the member whose slice holds U * total scans it to find the token.
// fp64 in steps 3-4 keeps inverse-CDF boundaries within ~1e-15 of the exact
// values: with 1e5-token vocabularies fp32 masses move a boundary by ~1e-7,
// which changes the drawn token far more often.
//
// Team barrier: members store a generation-tagged arrival word, member 0
// gathers them and stores one release word.  Data crossing members goes
// through device-scope loads and stores (coherent across XCDs without L2
// write-back or invalidation); a member waits for its own stores to land
// before it arrives.  Tags grow monotonically per team across calls (member 0
// advances the team's generation word at the first barrier of a call), so the
// control words never need clearing after the workspace was zero-filled once.
// The grid never exceeds the device's resident capacity, so all members of a
// team run together; spins are bounded.
#include <float.h>

#include <mutex>

#include "tv_device.h"
#include "tv_internal.h"

namespace tv {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kMaxTeamSize = 256;
constexpr int kMaxTeams = 1024;
constexpr int kMinSlice = 512;       // logits per member and row, at least
constexpr int kCtrlLine = 16;        // u64 words per team: [0] generation, [1] release, [2] error
constexpr int kP64Slots = 4;         // fp64 values a member publishes per phase
constexpr int kTagShift = 24;        // barrier tag = (generation << 24) + barrier index
constexpr uint32_t kSpinLimit = 1u << 20;
constexpr long kSmallWork = 1L << 24;  // logits below which every row gets an fp64 sum in step 1
constexpr int kRowsInFlight = 2;     // rows a wave streams together in step 1
constexpr int kVecPerRow = 4;        // float4 loads per lane and row per step-1 chunk

struct AcceptPlan {
    int W, nteams, slice;
    size_t ctrl_off, arrive_off, stats_off, stats64_off, p64_off, rbuf_off, total;
};

struct AccArgs {
    const float* q;
    const float* p;
    const int32_t* draft;
    const int32_t* parent;
    int32_t* accept_len;
    int32_t* accepted;
    int32_t* tokens;
    uint64_t* ctrl;     // [kMaxTeams][kCtrlLine]
    uint64_t* arrive;   // [kMaxTeams][kMaxTeamSize]
    uint64_t* stats;    // [nteams][2][2N][W] packed (max, sum) or (max, argmax)
    double* stats64;    // [nteams][2][2N][W] fp64 slice sums of exp((x - slice max)/T)
    double* p64;        // [nteams][2][kP64Slots][W]
    double* rbuf;       // [nteams][2][V]
    int B, N, V, W, slice, nteams, all64;
    float inv_t;
    double inv_t64;
    uint64_t seed;
};

// ---------------------------------------------- device-scope data exchange --
__device__ __forceinline__ void st_dev(uint64_t* p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_dev(const uint64_t* p) {
    return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev_d(double* p, double v) {
    st_dev(reinterpret_cast<uint64_t*>(p), (uint64_t)__double_as_longlong(v));
}
__device__ __forceinline__ double ld_dev_d(const double* p) {
    return __longlong_as_double((long long)ld_dev(reinterpret_cast<const uint64_t*>(p)));
}
__device__ __forceinline__ uint64_t pack2(float a, float b) {
    return (uint64_t)__float_as_uint(a) | ((uint64_t)__float_as_uint(b) << 32);
}
__device__ __forceinline__ float lo_f(uint64_t v) { return __uint_as_float((uint32_t)v); }
__device__ __forceinline__ float hi_f(uint64_t v) { return __uint_as_float((uint32_t)(v >> 32)); }

struct TeamSync {
    uint64_t* line;    // this team's control line
    uint64_t* arrive;  // this team's arrival words
    uint64_t base;     // (generation of this call) << kTagShift
    uint32_t k;        // barriers passed so far in this call
};

__device__ void team_sync(TeamSync& s, int w, int W) {
    ++s.k;
    const uint64_t tag = s.base + s.k;
    __builtin_amdgcn_s_waitcnt(0);  // this wave's device-scope stores have landed
    __syncthreads();
    if (w == 0) {
        const int t = threadIdx.x;
        if (t > 0 && t < W) {
            uint32_t spins = 0;
            while (ld_dev(&s.arrive[t]) < tag) {
                __builtin_amdgcn_s_sleep(1);
                if (++spins > kSpinLimit) {
                    st_dev(&s.line[2], 1ull);
                    break;
                }
            }
        }
        __syncthreads();
        if (t == 0) {
            if (s.k == 1) st_dev(&s.line[0], s.base >> kTagShift);  // the next call starts after this generation
            st_dev(&s.line[1], tag);
        }
    } else if (threadIdx.x == 0) {
        st_dev(&s.arrive[w], tag);
        uint32_t spins = 0;
        while (ld_dev(&s.line[1]) < tag) {
            __builtin_amdgcn_s_sleep(1);
            if (++spins > kSpinLimit) {
                st_dev(&s.line[2], 1ull);
                break;
            }
        }
    }
    __syncthreads();
}

// ------------------------------------------------------------------ helpers --
__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// Block scan in fp64 with a fixed association (identical on every member):
// shuffle scan per wave, then the wave totals in order.  Returns the inclusive
// value; `excl` receives the exclusive one, bitwise equal to the previous
// thread's inclusive value, and `tot` the block total.  `wt` is LDS for the
// kWaves wave totals.
__device__ __forceinline__ double block_scan_d(double v, double* wt, double& excl, double& tot) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const double y = __shfl_up(v, o);
        if (lane >= o) v += y;
    }
    const double prev = __shfl_up(v, 1);
    __syncthreads();
    if (lane == kWave - 1) wt[wave] = v;
    __syncthreads();
    double pre = 0.0, t = 0.0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
        if (i < wave) pre += wt[i];
        t += wt[i];
    }
    tot = t;
    excl = lane == 0 ? pre : pre + prev;
    return pre + v;
}

__device__ __forceinline__ double block_sum_d(double v, double* wt) {
    double excl, tot;
    block_scan_d(v, wt, excl, tot);
    return tot;
}

// Larger value wins; equal values go to the smaller index.
__device__ __forceinline__ void argmax_merge(float& v, int& i, float v2, int i2) {
    if (v2 > v || (v2 == v && i2 < i)) {
        v = v2;
        i = i2;
    }
}

// Sum of the W values published in one slot, identical on every member.
__device__ double gather_sum(const double* slot, int W, double* wt) {
    const double v = (int)threadIdx.x < W ? ld_dev_d(&slot[threadIdx.x]) : 0.0;
    return block_sum_d(v, wt);
}

// exp((x - m) / T) in fp64 for x <= m.
__device__ __forceinline__ double exp_scaled(float x, float m, double inv_t64, const double* tab) {
    return exp_nonpos(((double)x - (double)m) * inv_t64, tab);
}

// ------------------------------------------------------------ step 1 pieces --
struct RowAcc {
    float m, s, bv;
    int bi;
    double s64;
};

// Streams up to kRowsInFlight rows of this member's slice with one wave and
// leaves the wave-merged result in every lane (sampling: max, sum, optional
// fp64 sum; greedy: max and first argmax).
template <bool GREEDY, bool VEC4>
__device__ void stream_rows(const float* const* rows, const bool* want64, int nr, int s0, int s1, int lane,
                            float inv_t, double inv_t64, const double* tab, RowAcc* acc) {
#pragma unroll
    for (int r = 0; r < kRowsInFlight; ++r) {
        acc[r].m = -INFINITY;
        acc[r].s = 0.f;
        acc[r].bv = -INFINITY;
        acc[r].bi = 0x7fffffff;
        acc[r].s64 = 0.0;
    }
    constexpr int kStep = VEC4 ? 4 * kWave * kVecPerRow : kWave * kVecPerRow;
    for (int c0 = s0; c0 < s1; c0 += kStep) {
        float x[kRowsInFlight][4 * kVecPerRow];
        // issue every load of the chunk first
#pragma unroll
        for (int r = 0; r < kRowsInFlight; ++r) {
#pragma unroll
            for (int j = 0; j < kVecPerRow; ++j) {
                if constexpr (VEC4) {
                    const int v = c0 + 4 * (lane + kWave * j);
                    f32x4 t = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
                    if (r < nr && v < s1) t = *reinterpret_cast<const f32x4*>(rows[r] + v);
#pragma unroll
                    for (int e = 0; e < 4; ++e) x[r][4 * j + e] = t[e];
                } else {
                    const int v = c0 + lane + kWave * j;
                    x[r][4 * j] = (r < nr && v < s1) ? rows[r][v] : -INFINITY;
#pragma unroll
                    for (int e = 1; e < 4; ++e) x[r][4 * j + e] = -INFINITY;
                }
            }
        }
#pragma unroll
        for (int r = 0; r < kRowsInFlight; ++r) {
            if (r >= nr) continue;
            RowAcc& A = acc[r];
            if constexpr (GREEDY) {
#pragma unroll
                for (int j = 0; j < kVecPerRow; ++j)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int v = VEC4 ? c0 + 4 * (lane + kWave * j) + e : c0 + lane + kWave * j;
                        if (x[r][4 * j + e] > A.bv) {  // indices increase along a lane: first maximum kept
                            A.bv = x[r][4 * j + e];
                            A.bi = v;
                        }
                    }
            } else {
                float mx = -INFINITY;
#pragma unroll
                for (int i = 0; i < 4 * kVecPerRow; ++i) mx = fmaxf(mx, x[r][i]);
                if (mx > A.m) {
                    if (A.m != -INFINITY) {
                        A.s *= __expf((A.m - mx) * inv_t);
                        if (want64[r]) A.s64 *= exp_scaled(A.m, mx, inv_t64, tab);
                    }
                    A.m = mx;
                }
                if (A.m != -INFINITY) {
#pragma unroll
                    for (int i = 0; i < 4 * kVecPerRow; ++i) A.s += __expf((x[r][i] - A.m) * inv_t);
                    if (want64[r]) {
#pragma unroll
                        for (int i = 0; i < 4 * kVecPerRow; ++i) A.s64 += exp_scaled(x[r][i], A.m, inv_t64, tab);
                    }
                }
            }
        }
    }
    // wave merge
#pragma unroll
    for (int r = 0; r < kRowsInFlight; ++r) {
        if (r >= nr) continue;
        RowAcc& A = acc[r];
        if constexpr (GREEDY) {
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) argmax_merge(A.bv, A.bi, __shfl_xor(A.bv, o), __shfl_xor(A.bi, o));
        } else {
            const float M = wave_max(A.m);
            const double f64 = (A.m == -INFINITY) ? 0.0 : exp_scaled(A.m, M, inv_t64, tab);
            const float f32 = (A.m == -INFINITY) ? 0.f : __expf((A.m - M) * inv_t);
            A.s = wave_sum(A.s * f32);
            if (want64[r]) A.s64 = wave_sum_d(A.s64 * f64);
            A.m = M;
        }
    }
}

// Row r (storage index: q row u at u, p row c at N + c) carries an fp64 slice
// sum from step 1.
__device__ __forceinline__ bool row_has64(int r, int N, int all64, const int* par) {
    return all64 || (r < N ? r == 0 : par[r - N] == 0);
}

// Merges the statistics of up to 2 rows per wave over the team: raw max, the
// normaliser from the fp32 slice sums (assembled in fp64) and, where step 1
// formed them, the exact fp64 normaliser.  Rows come from the LDS list mrow.
__device__ void merge_rows(const int* mrow, int nm, const uint64_t* stats, const double* stats64, int W, int N,
                           int all64, const int* par, double inv_t64, const double* tab, float* sM, double* sS,
                           double* sS64) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int i0 = 2 * wave; i0 < nm; i0 += 2 * kWaves) {
        uint64_t e[2][4];
        double e64[2][4];
        int rr[2];
        bool h64[2];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            rr[k] = mrow[min(i0 + k, nm - 1)];
            h64[k] = (i0 + k < nm) && row_has64(rr[k], N, all64, par);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int j = lane + kWave * q;
                const bool ok = (i0 + k < nm) && j < W;
                e[k][q] = ok ? ld_dev(&stats[(size_t)rr[k] * W + j]) : pack2(-INFINITY, 0.f);
                e64[k][q] = (ok && h64[k]) ? ld_dev_d(&stats64[(size_t)rr[k] * W + j]) : 0.0;
            }
        }
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            if (i0 + k >= nm) continue;
            float m = -INFINITY;
#pragma unroll
            for (int q = 0; q < 4; ++q) m = fmaxf(m, lo_f(e[k][q]));
            m = wave_max(m);
            double s = 0.0, s64 = 0.0;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float mj = lo_f(e[k][q]);
                if (mj == -INFINITY) continue;
                const double f = exp_scaled(mj, m, inv_t64, tab);
                s += (double)hi_f(e[k][q]) * f;
                s64 += e64[k][q] * f;
            }
            s = wave_sum_d(s);
            s64 = wave_sum_d(s64);
            if (lane == 0) {
                sM[rr[k]] = m;
                sS[rr[k]] = h64[k] ? s64 : s;
                sS64[rr[k]] = h64[k] ? s64 : -1.0;
            }
        }
    }
}

// ---------------------------------------------------------------- the kernel --
template <bool GREEDY, bool VEC4>
__global__ __launch_bounds__(kThreads) void spec_accept_kernel(const AccArgs a) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int team = blockIdx.x / a.W;
    const int w = blockIdx.x % a.W;
    const int N = a.N, V = a.V, W = a.W;
    const int s0 = w * a.slice;
    const int s1 = min(V, s0 + a.slice);
    // each thread owns a contiguous run of the slice in the vocabulary passes
    const int run = (s1 - s0 + kThreads - 1) / kThreads;
    const int r0 = min(s1, s0 + tid * run);
    const int r1 = min(s1, r0 + run);
    const size_t rowsW = (size_t)2 * N * W;
    uint64_t* stats_team = a.stats + (size_t)team * 2 * rowsW;
    double* stats64_team = GREEDY ? nullptr : a.stats64 + (size_t)team * 2 * rowsW;
    double* p64 = a.p64 + (size_t)team * 2 * kP64Slots * W;
    double* rb = GREEDY ? nullptr : a.rbuf + (size_t)team * 2 * V;

    __shared__ int s_par[TV_MAX_NODES], s_draft[TV_MAX_NODES], s_amax[TV_MAX_NODES], s_depth[TV_MAX_NODES];
    __shared__ int s_path[TV_MAX_NODES], s_mrow[TV_MAX_NODES + 1];
    __shared__ float s_M[2 * TV_MAX_NODES];
    __shared__ double s_S[2 * TV_MAX_NODES], s_S64[2 * TV_MAX_NODES];
    __shared__ double s_wt[kWaves];
    __shared__ double s_excl[kThreads];
    __shared__ double s_tab[32];
    __shared__ int s_ok, s_nm, s_hit[kWaves], s_last[kWaves], s_tok;
    __shared__ uint64_t s_base;

    if (tid < 32) exp2_table(s_tab, tid);
    TeamSync sync;
    sync.line = a.ctrl + (size_t)team * kCtrlLine;
    sync.arrive = a.arrive + (size_t)team * kMaxTeamSize;
    sync.k = 0;
    if (tid == 0) s_base = (ld_dev(&sync.line[0]) + 1) << kTagShift;
    __syncthreads();
    sync.base = s_base;
    int phase = 0;  // parity of the fp64 publication slots

    int iter = 0;
    for (int b = team; b < a.B; b += a.nteams, ++iter) {
        // member 0 may still read the previous sequence's statistics while the
        // others stream this one: alternate between two buffers
        uint64_t* stats = stats_team + (size_t)(iter & 1) * rowsW;
        double* stats64 = GREEDY ? nullptr : stats64_team + (size_t)(iter & 1) * rowsW;

        // ---- tree and drafts of this sequence ----
        if (tid < kWave) {
            int ok = 1;
            if (tid < N) {
                const int pr = a.parent[(size_t)b * N + tid];
                int d = a.draft[(size_t)b * N + tid];
                d = d < 0 ? 0 : (d >= V ? V - 1 : d);  // out-of-range drafts violate the precondition
                s_par[tid] = pr;
                s_draft[tid] = d;
                ok = tid == 0 ? pr == -1 : (pr >= 0 && pr < tid);
            }
            const bool all_ok = __all(ok);
            if (tid == 0) s_ok = all_ok;
        }
        __syncthreads();
        const bool valid = s_ok;

        // ---- 1. slice statistics of every row ----
        const float* qb = a.q + (size_t)b * N * V;
        const float* pb = GREEDY ? nullptr : a.p + (size_t)b * N * V;
        const int nrows = valid ? (GREEDY ? N : 2 * N - 1) : 0;
        for (int rs = wave * kRowsInFlight; rs < nrows; rs += kWaves * kRowsInFlight) {
            const float* rows[kRowsInFlight];
            bool want64[kRowsInFlight];
            int srow[kRowsInFlight];
            const int nr = min(kRowsInFlight, nrows - rs);
#pragma unroll
            for (int i = 0; i < kRowsInFlight; ++i) {
                const int r = min(rs + i, nrows - 1);
                const bool is_q = r < N;
                srow[i] = is_q ? r : r + 1;  // p row c is stored at N + c
                if constexpr (GREEDY) {
                    rows[i] = qb + (size_t)r * V;  // greedy streams target rows only
                    want64[i] = false;
                } else {
                    rows[i] = is_q ? qb + (size_t)r * V : pb + (size_t)(r - N + 1) * V;
                    want64[i] = row_has64(srow[i], N, a.all64, s_par);
                }
            }
            RowAcc acc[kRowsInFlight];
            stream_rows<GREEDY, VEC4>(rows, want64, nr, s0, s1, lane, a.inv_t, a.inv_t64, s_tab, acc);
            if (lane == 0) {
#pragma unroll
                for (int i = 0; i < kRowsInFlight; ++i) {
                    if (i >= nr) continue;  // fully unrolled: the arrays stay in registers
                    if constexpr (GREEDY) {
                        st_dev(&stats[(size_t)srow[i] * W + w], pack2(acc[i].bv, __int_as_float(acc[i].bi)));
                    } else {
                        st_dev(&stats[(size_t)srow[i] * W + w], pack2(acc[i].m, acc[i].s));
                        if (want64[i]) st_dev_d(&stats64[(size_t)srow[i] * W + w], acc[i].s64);
                    }
                }
            }
        }
        team_sync(sync, w, W);

        int32_t* out_nodes = a.accepted + (size_t)b * N;
        int32_t* out_toks = a.tokens + (size_t)b * N;
        if (!valid) {
            if (w == 0) {
                if (tid == 0) a.accept_len[b] = -1;
                for (int i = tid; i < N; i += kThreads) {
                    out_nodes[i] = -1;
                    out_toks[i] = -1;
                }
            }
            __syncthreads();
            continue;
        }

        if constexpr (GREEDY) {
            if (w == 0) {
                // member 0 merges the argmax of every target row (4 rows in
                // flight per wave) and writes the path
                for (int rq = wave; rq < N; rq += 4 * kWaves) {
                    uint64_t e[4][4];
#pragma unroll
                    for (int k = 0; k < 4; ++k)
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const int r = rq + kWaves * k, j = lane + kWave * q;
                            e[k][q] = (r < N && j < W) ? ld_dev(&stats[(size_t)r * W + j])
                                                       : pack2(-INFINITY, __int_as_float(0x7fffffff));
                        }
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const int r = rq + kWaves * k;
                        if (r >= N) continue;
                        float bv = -INFINITY;
                        int bi = 0x7fffffff;
#pragma unroll
                        for (int q = 0; q < 4; ++q) argmax_merge(bv, bi, lo_f(e[k][q]), __float_as_int(hi_f(e[k][q])));
#pragma unroll
                        for (int o = 32; o > 0; o >>= 1) argmax_merge(bv, bi, __shfl_xor(bv, o), __shfl_xor(bi, o));
                        if (lane == 0) s_amax[r] = bi;
                    }
                }
                for (int i = tid; i < N; i += kThreads) {
                    out_nodes[i] = -1;
                    out_toks[i] = -1;
                }
                __syncthreads();
                if (tid == 0) {
                    // valid(i): every draft on the root-to-i path equals its parent's argmax
                    uint64_t ok = 1ull;
                    s_depth[0] = 0;
                    int e = 0;
                    for (int i = 1; i < N; ++i) {
                        const int pr = s_par[i];
                        s_depth[i] = s_depth[pr] + 1;
                        if (((ok >> pr) & 1ull) && s_draft[i] == s_amax[pr]) {
                            ok |= 1ull << i;
                            if (s_depth[i] > s_depth[e]) e = i;
                        }
                    }
                    const int len = s_depth[e];
                    for (int i = e, k = len - 1; i != 0; i = s_par[i], --k) {
                        out_nodes[k] = i;
                        out_toks[k] = s_draft[i];
                    }
                    out_toks[len] = s_amax[e];
                    a.accept_len[b] = len;
                }
            }
            __syncthreads();
        } else {
            const double inv_t64 = a.inv_t64;
            // merged statistics of node u's target row and its children's draft rows
            auto visit = [&](int u) {
                if (tid == 0) {
                    int nm = 0;
                    s_mrow[nm++] = u;
                    for (int c = u + 1; c < N; ++c)
                        if (s_par[c] == u) s_mrow[nm++] = N + c;
                    s_nm = nm;
                }
                __syncthreads();
                merge_rows(s_mrow, s_nm, stats, stats64, W, N, a.all64, s_par, inv_t64, s_tab, s_M, s_S, s_S64);
                __syncthreads();
            };

            // ---- 2./3. the walk (identical on every member) ----
            int u = 0, len = 0, cur = 0;
            bool res_active = false;  // target at u: residual rb[cur]/Z, else softmax(q_u / T)
            bool masses_ready = false;  // the last residual pass left the draw's slice masses
            double Z = 1.0, my_excl = 0.0, my_incl = 0.0, tsum = 0.0;
            const double* mass_slot = nullptr;
            for (int i = tid; i < 2 * N; i += kThreads) s_S64[i] = -1.0;  // no exact normaliser yet
            visit(0);
            int c = 1;
            for (;;) {
                while (c < N && s_par[c] != u) ++c;
                if (c >= N) break;  // every child of u tried, or u is a leaf
                {
                    // accept test in fp64, the same on every member and thread
                    const int x = s_draft[c];
                    const double rx = res_active ? ld_dev_d(&rb[(size_t)cur * V + x]) / Z
                                                 : exp_scaled(qb[(size_t)u * V + x], s_M[u], inv_t64, s_tab) / s_S[u];
                    const double px = exp_scaled(pb[(size_t)c * V + x], s_M[N + c], inv_t64, s_tab) / s_S[N + c];
                    const double acc = px == 0.0 ? 1.0 : fmin(1.0, rx / px);
                    const double r = (double)philox_uniform(a.seed, (uint32_t)c, (uint32_t)b, 0u);
                    if (r < acc) {
                        if (tid == 0) s_path[len] = c;
                        ++len;
                        u = c;
                        c = u + 1;
                        res_active = false;
                        masses_ready = false;
                        Z = 1.0;
                        visit(u);
                        continue;
                    }
                }
                // rejected: make sure the exact normalisers of q_u and p_c exist
                const bool need_q = !res_active && s_S64[u] < 0.0;
                const bool need_p = s_S64[N + c] < 0.0;
                if (need_q || need_p) {
                    double sq = 0.0, sp = 0.0;
                    const float Mq = s_M[u], Mp = s_M[N + c];
                    for (int v = s0 + tid; v < s1; v += kThreads) {
                        if (need_q) sq += exp_scaled(qb[(size_t)u * V + v], Mq, inv_t64, s_tab);
                        if (need_p) sp += exp_scaled(pb[(size_t)c * V + v], Mp, inv_t64, s_tab);
                    }
                    sq = block_sum_d(sq, s_wt);
                    sp = block_sum_d(sp, s_wt);
                    double* slot = p64 + (size_t)(phase & 1) * kP64Slots * W;
                    if (tid == 0) {
                        st_dev_d(&slot[w], sq);
                        st_dev_d(&slot[W + w], sp);
                    }
                    team_sync(sync, w, W);
                    sq = gather_sum(slot, W, s_wt);
                    sp = gather_sum(slot + W, W, s_wt);
                    ++phase;
                    if (tid == 0) {
                        if (need_q) s_S64[u] = sq;
                        if (need_p) s_S64[N + c] = sp;
                    }
                    __syncthreads();
                }
                // next sibling, whose exact normaliser this pass forms as well
                int nxt = c + 1;
                while (nxt < N && s_par[nxt] != u) ++nxt;
                const bool spec = nxt < N && s_S64[N + nxt] < 0.0;
                {
                    const float Mq = s_M[u], Mp = s_M[N + c];
                    const float Mn = spec ? s_M[N + nxt] : 0.f;
                    const double invSq = res_active ? 0.0 : 1.0 / s_S64[u];
                    const double invSp = 1.0 / s_S64[N + c];
                    const double invZ = 1.0 / Z;
                    const double* src = rb + (size_t)cur * V;
                    double* dst = rb + (size_t)(cur ^ 1) * V;
                    double part = 0.0, pn = 0.0;
                    for (int v = r0; v < r1; ++v) {
                        const double rv = res_active ? ld_dev_d(&src[v]) * invZ
                                                     : exp_scaled(qb[(size_t)u * V + v], Mq, inv_t64, s_tab) * invSq;
                        const double pv = exp_scaled(pb[(size_t)c * V + v], Mp, inv_t64, s_tab) * invSp;
                        const double wv = rv > pv ? rv - pv : 0.0;
                        st_dev_d(&dst[v], wv);
                        part += wv;
                        if (spec) pn += exp_scaled(pb[(size_t)nxt * V + v], Mn, inv_t64, s_tab);
                    }
                    double slice_mass, excl;
                    const double incl = block_scan_d(part, s_wt, excl, slice_mass);
                    pn = block_sum_d(pn, s_wt);
                    double* slot = p64 + (size_t)(phase & 1) * kP64Slots * W;
                    if (tid == 0) {
                        st_dev_d(&slot[w], slice_mass);
                        st_dev_d(&slot[W + w], pn);
                    }
                    team_sync(sync, w, W);
                    const double Znew = gather_sum(slot, W, s_wt);
                    const double Sn = gather_sum(slot + W, W, s_wt);
                    ++phase;
                    if (spec && tid == 0) s_S64[N + nxt] = Sn;
                    __syncthreads();
                    if (Znew > 0.0) {  // zero mass cannot follow a rejection in exact arithmetic: keep R then
                        cur ^= 1;
                        Z = Znew;
                        res_active = true;
                        // these slice masses and run sums serve the draw if no sibling follows
                        masses_ready = true;
                        mass_slot = slot;
                        tsum = part;
                        my_incl = incl;
                        my_excl = excl;
                    }
                }
                ++c;
            }

            // ---- 4. the extra token: inverse CDF over the team's slices ----
            const double ut = (double)philox_uniform(a.seed, (uint32_t)u, (uint32_t)b, 1u);
            const float Mu = s_M[u];
            const double* src = rb + (size_t)cur * V;
            const float* qrow = qb + (size_t)u * V;
            if (!masses_ready) {
                // draw from softmax(q_u / T) (leaf bonus or residual kept unchanged):
                // unnormalised weights exp((q - max)/T), masses per run and slice
                tsum = 0.0;
                for (int v = r0; v < r1; ++v)
                    tsum += res_active ? ld_dev_d(&src[v]) : exp_scaled(qrow[v], Mu, inv_t64, s_tab);
                double slice_mass;
                my_incl = block_scan_d(tsum, s_wt, my_excl, slice_mass);
                double* slot = p64 + (size_t)(phase & 1) * kP64Slots * W;
                if (tid == 0) st_dev_d(&slot[w], slice_mass);
                team_sync(sync, w, W);
                ++phase;
                mass_slot = slot;
            }
            // every member finds the owner slice the same way: the first slice
            // whose running mass exceeds U * total (the last slice with mass if
            // rounding left the target at the total)
            const double my_t = tid < W ? ld_dev_d(&mass_slot[tid]) : 0.0;
            double total, slot_excl;
            const double prefix = block_scan_d(my_t, s_wt, slot_excl, total);
            s_excl[tid] = slot_excl;
            const double target = ut * total;
            const bool has = tid < W && my_t > 0.0;
            const uint64_t hit = __ballot(has && prefix > target);
            const uint64_t pos = __ballot(has);
            if (lane == 0) {
                s_hit[wave] = hit ? wave * kWave + __ffsll((unsigned long long)hit) - 1 : -1;
                s_last[wave] = pos ? wave * kWave + 63 - __clzll((unsigned long long)pos) : -1;
            }
            __syncthreads();
            int owner = -1, last_pos = -1;
            for (int i = 0; i < kWaves; ++i) {
                if (owner < 0) owner = s_hit[i];
                last_pos = max(last_pos, s_last[i]);
            }
            const bool fallback = owner < 0;
            if (fallback) owner = last_pos;
            const double before = owner >= 0 ? s_excl[owner] : 0.0;
            if (w == owner) {
                if (tid == 0) s_tok = -1;
                __syncthreads();
                const double tgt = target - before;
                if (!fallback && my_excl <= tgt && my_incl > tgt && tsum > 0.0) {
                    double cum = my_excl;
                    int tok = -1, lastp = -1;
                    for (int v = r0; v < r1; ++v) {
                        const double wv = res_active ? ld_dev_d(&src[v]) : exp_scaled(qrow[v], Mu, inv_t64, s_tab);
                        if (wv > 0.0) lastp = v;
                        cum += wv;
                        if (wv > 0.0 && cum > tgt) {
                            tok = v;
                            break;
                        }
                    }
                    s_tok = tok >= 0 ? tok : lastp;
                }
                __syncthreads();
                if (s_tok < 0 && tid == 0) {
                    // target at or beyond the slice total (rounding), or fallback: last token with mass
                    int tok = -1;
                    for (int v = s1 - 1; v >= s0; --v) {
                        const double wv = res_active ? ld_dev_d(&src[v]) : exp_scaled(qrow[v], Mu, inv_t64, s_tab);
                        if (wv > 0.0) {
                            tok = v;
                            break;
                        }
                    }
                    s_tok = tok >= 0 ? tok : s1 - 1;
                }
                __syncthreads();
                for (int i = tid; i < N; i += kThreads) {
                    out_nodes[i] = i < len ? s_path[i] : -1;
                    out_toks[i] = i < len ? s_draft[s_path[i]] : (i == len ? s_tok : -1);
                }
                if (tid == 0) a.accept_len[b] = len;
            }
            __syncthreads();
        }  // sampling
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

// ---------------------------------------------------------------- planning --
typedef void (*KernelFn)(AccArgs);

KernelFn pick(bool greedy, bool vec4) {
    if (greedy) return vec4 ? spec_accept_kernel<true, true> : spec_accept_kernel<true, false>;
    return vec4 ? spec_accept_kernel<false, true> : spec_accept_kernel<false, false>;
}

// Workgroups of the accept kernel resident at once on the current device
// (occupancy query, cached per device, at most 4 per CU).
int resident_capacity() {
    static std::mutex mu;
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    std::lock_guard<std::mutex> lock(mu);
    if (cache[dev] == 0) {
        int ncu = 0, per = 0, per_min = 1 << 30;
        if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu <= 0)
            return 0;
        const bool modes[2] = {false, true};
        for (bool g : modes)
            for (bool v4 : modes) {
                if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, reinterpret_cast<const void*>(pick(g, v4)),
                                                                 kThreads, 0) != hipSuccess)
                    return 0;
                per_min = per < per_min ? per : per_min;
            }
        if (per_min > 4) per_min = 4;  // a few members per CU cover HBM latency
        if (per_min < 1) return 0;
        cache[dev] = ncu * per_min;
    }
    return cache[dev];
}

bool make_plan(int B, int N, int V, int greedy, AcceptPlan& pl) {
    const int cap = resident_capacity();
    if (cap <= 0) return false;
    int wmax = (V + kMinSlice - 1) / kMinSlice;
    if (wmax > kMaxTeamSize) wmax = kMaxTeamSize;
    int W = cap / (B > 0 ? B : 1);
    if (W > wmax) W = wmax;
    if (W < 1) W = 1;
    int slice = (V + W - 1) / W;
    slice = (slice + 3) / 4 * 4;
    W = (V + slice - 1) / slice;
    int nteams = cap / W;
    if (nteams > B) nteams = B;
    if (nteams > kMaxTeams) nteams = kMaxTeams;
    if (nteams < 1) nteams = 1;
    pl.W = W;
    pl.nteams = nteams;
    pl.slice = slice;
    size_t off = 0;
    pl.ctrl_off = off;
    off += round_up((size_t)kMaxTeams * kCtrlLine * sizeof(uint64_t), 256);
    pl.arrive_off = off;
    off += round_up((size_t)kMaxTeams * kMaxTeamSize * sizeof(uint64_t), 256);
    pl.stats_off = off;
    off += round_up((size_t)nteams * 2 * 2 * N * W * sizeof(uint64_t), 256);
    pl.stats64_off = off;
    if (!greedy) off += round_up((size_t)nteams * 2 * 2 * N * W * sizeof(double), 256);
    pl.p64_off = off;
    off += round_up((size_t)nteams * 2 * kP64Slots * W * sizeof(double), 256);
    pl.rbuf_off = off;
    if (!greedy) off += round_up((size_t)nteams * 2 * V * sizeof(double), 256);
    pl.total = off;
    return true;
}

}  // namespace
}  // namespace tv

extern "C" size_t tv_spec_accept_workspace(int B, int N, int V, int greedy) {
    if (B <= 0 || N < 1 || N > TV_MAX_NODES || V < 1) return 0;
    tv::AcceptPlan pl;
    if (!tv::make_plan(B, N, V, greedy, pl)) return 0;
    return pl.total;
}

extern "C" int tv_spec_accept(const float* q_logits, const float* p_logits, const int32_t* draft_tokens,
                              const int32_t* parent, int B, int N, int V, uint64_t philox_seed, float temperature,
                              int greedy, int32_t* accept_len, int32_t* accepted_nodes, int32_t* out_tokens,
                              void* workspace, size_t workspace_bytes, void* stream) {
    using namespace tv;
    if (B < 0 || N < 1 || V < 1) return TV_ERR_INVALID_ARG;
    if (N > TV_MAX_NODES) return TV_ERR_UNSUPPORTED;
    if (!greedy && !(temperature > 0.f && temperature <= FLT_MAX)) return TV_ERR_INVALID_ARG;
    if (B == 0) return TV_OK;
    if (!q_logits || (!greedy && !p_logits) || !draft_tokens || !parent || !accept_len || !accepted_nodes ||
        !out_tokens)
        return TV_ERR_INVALID_ARG;
    if (!aligned(q_logits, 4) || (!greedy && !aligned(p_logits, 4))) return TV_ERR_INVALID_ARG;
    if (!workspace || !aligned(workspace, 256)) return TV_ERR_WORKSPACE;
    AcceptPlan pl;
    if (!make_plan(B, N, V, greedy, pl)) return TV_ERR_HIP;
    if (workspace_bytes < pl.total) return TV_ERR_WORKSPACE;

    char* ws = static_cast<char*>(workspace);
    AccArgs a;
    a.q = q_logits;
    a.p = p_logits;
    a.draft = draft_tokens;
    a.parent = parent;
    a.accept_len = accept_len;
    a.accepted = accepted_nodes;
    a.tokens = out_tokens;
    a.ctrl = reinterpret_cast<uint64_t*>(ws + pl.ctrl_off);
    a.arrive = reinterpret_cast<uint64_t*>(ws + pl.arrive_off);
    a.stats = reinterpret_cast<uint64_t*>(ws + pl.stats_off);
    a.stats64 = greedy ? nullptr : reinterpret_cast<double*>(ws + pl.stats64_off);
    a.p64 = reinterpret_cast<double*>(ws + pl.p64_off);
    a.rbuf = greedy ? nullptr : reinterpret_cast<double*>(ws + pl.rbuf_off);
    a.B = B;
    a.N = N;
    a.V = V;
    a.W = pl.W;
    a.slice = pl.slice;
    a.nteams = pl.nteams;
    a.all64 = !greedy && (long)B * (2 * N - 1) * V <= kSmallWork;
    a.inv_t = greedy ? 1.f : (float)(1.0 / (double)temperature);
    a.inv_t64 = greedy ? 1.0 : 1.0 / (double)temperature;
    a.seed = philox_seed;
    const bool vec4 = (V % 4 == 0) && aligned(q_logits, 16) && (greedy || aligned(p_logits, 16));
    // The grid never exceeds the resident capacity from the occupancy query, so
    // once earlier work on the stream drains every member is resident and the
    // team barriers make progress (their spins are bounded regardless).
    hipLaunchKernelGGL(pick(greedy, vec4), dim3(pl.nteams * pl.W), dim3(kThreads), 0, (hipStream_t)stream, a);
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
