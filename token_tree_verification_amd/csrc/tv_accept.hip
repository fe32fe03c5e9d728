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
// One launch of one 1024-thread workgroup per CU (no co-resident workgroups
// competing for a CU's bandwidth).  A team of W workgroups owns one sequence
// at a time; member w owns vocabulary slice w of every logit row.
//  1. Statistics: each member streams its slice of a list of rows once
//     (coalesced 16-byte loads, non-temporal in greedy mode when the call's
//     logits exceed twice the Infinity Cache, prefetched a group ahead; its sixteen waves
//     take rows from an LDS counter) and publishes per row the slice max and
//     sum of exp((x - max)/T) -- or the max and its first index in greedy mode.
//  2. Greedy: every member merges the argmax of target rows from the other
//     members' entries; member 0 writes the path.  When a member's share of
//     every target row is small (768 KB at most) all rows are streamed up
//     front and the deepest matching node is found with one ancestor chase
//     per node; otherwise the tree is searched one level at a time, streaming
//     only the rows of the nodes whose path has matched so far.
//  3. Sampling: the walk reads few of the rows (on random trees ~6% of the
//     logits), so statistics are computed per node as the walk reaches it:
//     its family, the node's target row and the draft rows its children were
//     drawn from, is streamed and merged before its children are tested.
//     Every member runs the same walk redundantly: decisions need only the
//     merged statistics and the gathered logits q_parent(c)(x_c) and p_c(x_c),
//     so all members agree bit for bit without communicating.
//  4. A rejection costs one pass over the slices: the residual
//     max(0, R - P_c) replaces the member's slice of R in LDS, and its slice
//     mass and the residual at the next sibling's token are exchanged.
//  5. The extra token: every member knows every slice's mass (from the last
//     residual pass, or from the statistics when drawing from a target row),
//     so the member whose slice holds U * total scans its slice alone.
// Precision: per-element exponentials are fp32 (v_exp_f32 of (x - max) * c,
// with the subtraction first so the heavy terms carry ~1e-7 relative error);
// sums and masses accumulate in fp64; the accept ratio is formed in fp64 from
// the gathered logits.  Decisions can differ from exact arithmetic only within
// ~1e-6 of a boundary.
//
// Cross-member data (statistics entries, walk-step records) are 64-bit words
// carrying a tag (call generation, sequence or step) in their upper half,
// written with device-scope stores (coherent across XCDs without L2
// write-back or invalidation); a reader polls the words it needs until they
// carry the expected tag, so no barrier separates writer and reader.  The
// generation is one per call: every team's control line holds the same
// generation word; every workgroup reads its team's when it starts, and once
// its first merge has seen every member's entries (every member read the word
// before streaming), member 0 of team t advances line t and the lines of the
// teams this call does not have (t + k nteams), so every line advances once a
// call and the next call's tags differ from every tag of this one, whatever
// its shape.  Nothing in the workspace needs clearing after it was
// zero-filled once.  The grid never exceeds the device's resident capacity, so all members
// of a team run together; spins are bounded.  A wait that runs out is counted
// in the workspace's arrival word; the last workgroup to finish then reports
// every sequence of the teams concerned as failed (accept_len -2), and the
// workspace stays usable.
//
// Without-replacement siblings (EAGLE explainer, static-tree verification:
// the children of a node are alternative candidates for the next position,
// drawn from the draft's distribution at that node): p row u is then the
// draft distribution at node u, shared by its children, and child k is tested
// against it with the earlier (rejected) siblings' tokens removed and the rest
// renormalised -- P^(k)(x) = P_u(x) / (1 - sum_j<k P_u(x_j)) -- and a rejection
// leaves norm(max(0, R - P^(k))).  The residual already holds no mass at the
// removed tokens (each was rejected with R < P there), so a pass needs only
// the scale.
#include <float.h>

#include <atomic>
#include <mutex>

#include "tv_device.h"
#include "tv_internal.h"

namespace tv {
namespace {

constexpr int kThreads = 1024;       // one workgroup per CU: no co-resident workgroups competing for its bandwidth
constexpr int kWaves = kThreads / kWave;
constexpr int kMaxTeamSize = 256;
constexpr int kMaxTeams = 1024;
constexpr long kMinMemberBytes = 88 * 1024;  // sampling: logit bytes streamed per member and sequence, at least
constexpr int kMinSlice = 1024;      // logits per member and row, at least
constexpr int kMaxSlice = 32768;     // sampling: a member's residual slice lives in LDS (128 KB)
constexpr int kMaxSpans = 4095;      // greedy: spans of 256 logits per slice, at most
constexpr int kSpan = 4 * kWave;     // logits one wave covers with one 16-byte load per lane
constexpr int kGroup = 4;            // spans per prefetch group (two groups in flight per wave)
constexpr int kMinChunkSpans = 8;    // a row split over waves: spans per chunk, at least (8 KB)
constexpr double kGreedyRowsUpFront = 768.0 * 1024;  // greedy: member bytes of every target row, at most, to stream them up front
constexpr int kCtrlLine = 16;        // u64 words per team: [0] generation, [2] a wait ran out in this call
constexpr int kTagShift = 24;        // TeamSync::base = generation << kTagShift
constexpr uint32_t kSpinLimit = 1u << 20;  // polls of one wait (about a second)
constexpr int kMaxNodes = TV_MAX_NODES;
constexpr int kMassRec = 4;          // tagged u64 words per (pass, member): mass (two halves), new and old
constexpr double kNonTemporalBytes = 512.0 * 1024 * 1024;  // twice the Infinity Cache: larger streams skip caching
                                     // residual at the next token

struct AcceptPlan {
    int W, nteams, slice;
    size_t ctrl_off, done_off, stats_off, mass_off, total;
};

struct AccArgs {
    const float* q;
    const float* p;
    const int32_t* draft;
    const int32_t* parent;
    const int32_t* seq_nodes;  // [B] nodes of each sequence, or null (all N)
    int32_t* accept_len;
    int32_t* accepted;
    int32_t* tokens;
    uint64_t* ctrl;      // [kMaxTeams][kCtrlLine]
    uint64_t* done;      // arrivals of this call (low half), waits that ran out (high half)
    uint64_t* stats;     // [nteams][2][2N][W][2] tagged (max), (sum); greedy [nteams][2][N][W][2] (max), (index)
    double* mass;        // sampling: [nteams][2][N][W][kMassRec] (per team, two sequence buffers)
    int B, N, V, W, slice, nteams;
    int lines;           // control lines in use: teams never exceed the device's resident workgroups
    int wor;             // siblings drawn without replacement: p row u serves u's children
    int greedy_rows;     // greedy: every target row's statistics up front (else one tree level at a time)
    uint32_t spin_limit; // polls a wait makes before it gives up
    float c;             // log2(e) / T
    double inv_t64;      // 1 / T
    uint64_t seed;
};

// ---------------------------------------------- device-scope data exchange --
__device__ __forceinline__ void st_dev(uint64_t* p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_dev(const uint64_t* p) {
    return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float lo_f(uint64_t v) { return __uint_as_float((uint32_t)v); }

struct TeamSync {
    uint64_t* line;    // this team's control line
    uint64_t* ctrl;    // every team's control line ([kMaxTeams][kCtrlLine])
    int team, nteams, lines;
    uint64_t* done;    // the call's arrival word
    uint64_t base;     // (generation of this call) << kTagShift: one per call, for every team
    uint32_t limit;    // polls per wait
};

// A wait ran out: mark the team and count it in the arrival word (released,
// so that the last workgroup, which acquires that word, sees the mark).  The
// count's old value is consumed, so the wave does not go on before the
// atomic has been performed.
__device__ __forceinline__ void wait_failed(uint64_t* line, uint64_t* done) {
    st_dev(&line[2], 1ull);
    const uint64_t old = __hip_atomic_fetch_add(done, 1ull << 32, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    asm volatile("" : : "v"(old));
}

// Walk steps exchange tagged words: the tag is (1 << 31 | generation mod 2^19
// << 12 | sequence iteration mod 16 << 8 | rejection pass) in the upper 32
// bits of every 64-bit word; statistics entries carry (1 << 31 | generation
// << 12 | sequence iteration mod 4096).  The generation is the call's, the
// same for every team (a workspace reused with another shape puts other
// teams' words at the same addresses: a generation per team could repeat
// there), and the top bit keeps every tag apart from never-written (zero)
// memory.  Tags alone cannot keep old words out: a slot that no sequence
// writes for a while keeps its word, and sixteen sequences (or 2^19 calls)
// later the same tag comes round again.  So both kinds of words sit in two
// buffers per team, one per parity of the team's sequence iteration, and a
// member clears its own words of a buffer when it starts the sequence that
// uses it.  Nobody still reads them then: this member finished the previous
// sequence, which needed every member's statistics of that sequence, which
// each member published only after finishing the sequence before, the
// buffer's last user.  A member reads another's walk records of sequence i
// only after merging that member's statistics of i, published after its
// clear, so a record it polls is cleared or of sequence i; a statistics entry
// polled before its owner cleared it is of sequence i - 2 or of an earlier
// call, which the tag tells apart.
__device__ __forceinline__ uint32_t gen_tag(const TeamSync& s) {
    return 0x80000000u | (((uint32_t)(s.base >> kTagShift) & 0x7ffffu) << 12);
}
__device__ __forceinline__ uint32_t exchange_tag(const TeamSync& s, int iter, int pass) {
    static_assert(kMaxNodes <= 257, "rejection passes of one walk fit eight bits");
    return gen_tag(s) | ((uint32_t)(iter & 15) << 8) | (uint32_t)(pass & 255);
}
// Poll one member's first nw words until all carry tag `tg` (upper half); at
// most s.limit polls (none when the limit is 0).
__device__ __forceinline__ void gather_tagged(const TeamSync& s, const uint64_t* src, uint64_t tg, int nw, uint64_t* e) {
    for (uint32_t polls = 0;; ++polls) {
        if (polls >= s.limit) {
            wait_failed(s.line, s.done);
            return;
        }
        bool ok = true;
#pragma unroll
        for (int i = 0; i < kMassRec; ++i) {
            if (i >= nw) continue;
            e[i] = ld_dev(&src[i]);
            ok = ok && (e[i] & 0xffffffff00000000ull) == tg;
        }
        if (ok) return;
        __builtin_amdgcn_s_sleep(1);
    }
}

// After the first merge of a call every member of the team has read the
// team's generation word (before it streamed): member 0 advances it for the
// next call, and with it the lines of the teams this call does not have (one
// store per thread; lines up to the device's resident workgroups, which no
// team index reaches), so that every line holds the same generation.  Called
// by every thread of the workgroup.
__device__ __forceinline__ void advance_generation(const TeamSync& s, int w, bool& done) {
    if (!done && w == 0) {
        const int L = s.team + (int)threadIdx.x * s.nteams;
        if (L < s.lines) st_dev(&s.ctrl[(size_t)L * kCtrlLine], s.base >> kTagShift);
    }
    done = true;
}

// ------------------------------------------------------------------ helpers --
// Block scan in fp64 with a fixed association (identical on every member):
// shuffle scan per wave, then the wave totals in order.  Returns the inclusive
// value; `excl` receives the exclusive one and `tot` the block total.  `wt` is
// LDS for the kWaves wave totals.
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

// Block sum in fp64 with one barrier: a DPP reduction per wave, then the wave
// totals in order (a fixed association, identical on every member).  The
// caller guarantees that a workgroup barrier separates every earlier read of
// `wt` from this call (the walk alternates two such arrays between its two
// sums per step).
__device__ __forceinline__ double block_sum_1b(double v, double* wt) {
    v = group_sum_dpp(v, kWave);
    if ((threadIdx.x & (kWave - 1)) == 0) wt[threadIdx.x >> 6] = v;
    __syncthreads();
    double t = 0.0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) t += wt[i];
    return t;
}

// Larger value wins; equal values go to the smaller index.
__device__ __forceinline__ void argmax_merge(float& v, int& i, float v2, int i2) {
    if (v2 > v || (v2 == v && i2 < i)) {
        v = v2;
        i = i2;
    }
}

// exp((x - m) / T) in fp64 for x <= m.
__device__ __forceinline__ double exp_scaled(float x, float m, double inv_t64, const double* tab) {
    return exp_nonpos(((double)x - (double)m) * inv_t64, tab);
}

// Streamed rows are claimed in order i = 0, 1, ...; srow[i] (in LDS) is the
// storage index of claim i: target row u at u, draft row k at N + k (N the
// batch-wide node stride).  Target rows come first, then the draft rows the
// walk may read: rows 1..n-1 (one per child), or, without replacement, the
// rows of the nodes that have children.

// Row pointer of a storage index.
__device__ __forceinline__ const float* row_ptr(const float* qb, const float* pb, int r, int N, int V) {
    return r < N ? qb + (size_t)r * V : pb + (size_t)(r - N) * V;
}

// ------------------------------------------------------- 1. statistics pass --
// The workgroup streams its slice of every row (storage order: target rows,
// then draft rows); its sixteen waves take rows one at a time from an LDS
// counter, so a wave that gets less of the CU's issue bandwidth takes fewer
// rows.  A row is streamed with one 16-byte load per lane per span of 256
// logits, a prefetch group ahead of the arithmetic (across row boundaries);
// every loaded span carries a tag (row << 12 | span, bit 31 on the row's last
// span) and the row's slice statistics are published when its last span is
// processed: sampling (max, sum of exp((x - max) c), accumulated in fp64,
// stored as fp32), greedy (max, first index).
template <bool GREEDY, bool VEC4, bool NT, bool CHUNKS>
__device__ __forceinline__ void stream_slices(const float* qb, const float* pb, int nrows, int N, int V, int s0,
                                              int nsl, float c, uint64_t* stats, int W, int w, int* rowctr,
                                              uint64_t tg, const int* srow) {
    const int lane = threadIdx.x & 63;
    const int nspan = (nsl + kSpan - 1) / kSpan;
    auto take = [&]() -> int {
        int v = 0;
        if (lane == 0) v = __hip_atomic_fetch_add(rowctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        return __builtin_amdgcn_readfirstlane(v);
    };
    static_assert(2 * kMaxNodes <= 1024 && kMaxSpans < 4096, "tag fields");
    // Fewer rows than waves: each row is cut into ch chunks of spc spans (at
    // least kMinChunkSpans), so that every wave has work; a chunk's statistics
    // go to LDS and are combined per row, in chunk order, after the stream.
    // Waves claim units (row li = unit / ch, chunk unit % ch).
    int ch = 1, spc = nspan;
    if constexpr (CHUNKS) {
        ch = nrows >= kWaves ? 1 : kWaves / nrows;
        if (ch > nspan / kMinChunkSpans) ch = max(1, nspan / kMinChunkSpans);
        spc = (nspan + ch - 1) / ch;
        ch = (nspan + spc - 1) / spc;  // no empty chunk
    }
    const int nunits = nrows * ch;
    __shared__ float s_cm[kWaves];   // per chunk: max (or best value, greedy)
    __shared__ double s_cs[kWaves];  // sum of exp((x - max)/T)
    __shared__ int s_ci[kWaves];     // greedy: first index of the best value
    // load cursor: unit lu, its row li and span lj of [lbeg, lend); past the
    // last unit the cursor stays on its last span and marks the loads as fillers
    int lu = take();
    int li = 0, lj = 0, lbeg = 0, lend = 0;
    auto start = [&](int u) {
        if (!CHUNKS || ch == 1) {  // uniform: whole rows
            li = u;
            lbeg = lj = 0;
            lend = nspan;
        } else {
            li = u / ch;
            lbeg = lj = (u % ch) * spc;
            lend = min(nspan, lbeg + spc);
        }
    };
    bool lvalid = lu < nunits;
    start(lvalid ? lu : 0);
    const float* lrow = row_ptr(qb, pb, srow[li], N, V) + s0;
    auto load = [&](f32x4& x, int& xt) {
        const int e = lj * kSpan;
        if constexpr (VEC4) {
            const int v = e + 4 * lane;
            const f32x4* src = reinterpret_cast<const f32x4*>(lrow + min(v, nsl - 4));
            f32x4 t;
            if constexpr (NT)
                t = __builtin_nontemporal_load(src);
            else
                t = *src;
#pragma unroll
            for (int k = 0; k < 4; ++k) x[k] = v < nsl ? t[k] : -INFINITY;
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int v = e + lane + kWave * k;
                const float* src = lrow + min(v, nsl - 1);
                float t;
                if constexpr (NT)
                    t = __builtin_nontemporal_load(src);
                else
                    t = *src;
                x[k] = v < nsl ? t : -INFINITY;
            }
        }
        // tag: unit, span, first (bit 30) and last (bit 31) span of the unit
        xt = lvalid ? (lu << 12 | lj | (lj == lbeg ? 0x40000000 : 0) | (lj == lend - 1 ? (int)0x80000000 : 0)) : -1;
        if (!lvalid) return;
        if (++lj == lend) {
            const int nxt = take();
            if (nxt < nunits) {
                lu = nxt;
                start(lu);
                lrow = row_ptr(qb, pb, srow[li], N, V) + s0;
            } else {
                lvalid = false;
                lj = lend - 1;
            }
        }
    };

    float m = -INFINITY, bv = -INFINITY;
    double s = 0.0;
    int bi = 0x7fffffff;
    bool done = false;
    auto process = [&](const f32x4& x, int tag) {
        if (tag == -1) {
            done = true;
            return;
        }
        const int j = tag & 4095;
        if (tag & 0x40000000) {
            m = -INFINITY;
            s = 0.0;
            bv = -INFINITY;
            bi = 0x7fffffff;
        }
        const int e = j * kSpan;
        if constexpr (GREEDY) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int v = VEC4 ? e + 4 * lane + k : e + lane + kWave * k;  // increasing along the lane
                if (x[k] > bv) {
                    bv = x[k];
                    bi = s0 + v;
                }
            }
        } else {
            const float cm = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
            if (cm > m) {
                if (m != -INFINITY) s *= (double)__builtin_amdgcn_exp2f((m - cm) * c);
                m = cm;
            }
            if (m != -INFINITY) {
                const float e0 = __builtin_amdgcn_exp2f((x[0] - m) * c) + __builtin_amdgcn_exp2f((x[1] - m) * c);
                const float e1 = __builtin_amdgcn_exp2f((x[2] - m) * c) + __builtin_amdgcn_exp2f((x[3] - m) * c);
                s += (double)(e0 + e1);
            }
        }
        if (tag < 0) {  // the unit's last span: reduce over the wave, publish or keep
            const int u = (tag >> 12) & 0x3ffff;
            if constexpr (GREEDY) {
                group_argmax_dpp(bv, bi, kWave);
                if (lane == 0) {
                    if (!CHUNKS || ch == 1) {
                        const int r = srow[u];
                        st_dev(&stats[2 * ((size_t)r * W + w)], tg | __float_as_uint(bv));
                        st_dev(&stats[2 * ((size_t)r * W + w) + 1], tg | (uint32_t)bi);
                    } else {
                        s_cm[u] = bv;
                        s_ci[u] = bi;
                    }
                }
            } else {
                const float M = group_max_dpp(m, kWave);
                const double f = (m == -INFINITY) ? 0.0 : (double)__builtin_amdgcn_exp2f((m - M) * c);
                const double S = group_sum_dpp(s * f, kWave);
                if (lane == 0) {
                    if (!CHUNKS || ch == 1) {
                        const int r = srow[u];
                        st_dev(&stats[2 * ((size_t)r * W + w)], tg | __float_as_uint(M));
                        st_dev(&stats[2 * ((size_t)r * W + w) + 1], tg | __float_as_uint((float)S));
                    } else {
                        s_cm[u] = M;
                        s_cs[u] = S;
                    }
                }
            }
        }
    };

    // the scalar-load path holds half the groups (it stays within 128 VGPRs)
    constexpr int NG = VEC4 ? kGroup : kGroup / 2;
    f32x4 xa[NG], xb[NG];
    int ta[NG], tb[NG];
#pragma unroll
    for (int i = 0; i < NG; ++i) load(xa[i], ta[i]);
    while (!done) {
#pragma unroll
        for (int i = 0; i < NG; ++i) load(xb[i], tb[i]);
#pragma unroll
        for (int i = 0; i < NG; ++i)
            if (!done) process(xa[i], ta[i]);
#pragma unroll
        for (int i = 0; i < NG; ++i) load(xa[i], ta[i]);
#pragma unroll
        for (int i = 0; i < NG; ++i)
            if (!done) process(xb[i], tb[i]);
    }
    if (CHUNKS && ch > 1) {  // uniform: a row's chunks, combined in order, then published
        __syncthreads();
        const int t = threadIdx.x;
        if (t < nrows) {
            const int r = srow[t];
            if constexpr (GREEDY) {
                float v = -INFINITY;
                int i = 0x7fffffff;
                for (int k = 0; k < ch; ++k) argmax_merge(v, i, s_cm[t * ch + k], s_ci[t * ch + k]);
                st_dev(&stats[2 * ((size_t)r * W + w)], tg | __float_as_uint(v));
                st_dev(&stats[2 * ((size_t)r * W + w) + 1], tg | (uint32_t)i);
            } else {
                float M = -INFINITY;
                for (int k = 0; k < ch; ++k) M = fmaxf(M, s_cm[t * ch + k]);
                double S = 0.0;
                for (int k = 0; k < ch; ++k) {
                    const float mk = s_cm[t * ch + k];
                    if (mk != -INFINITY) S += s_cs[t * ch + k] * (double)__builtin_amdgcn_exp2f((mk - M) * c);
                }
                st_dev(&stats[2 * ((size_t)r * W + w)], tg | __float_as_uint(M));
                st_dev(&stats[2 * ((size_t)r * W + w) + 1], tg | __float_as_uint((float)S));
            }
        }
    }
}

// ------------------------------------------------------- merge of statistics --
// Lanes are grouped LPR to a row (LPR = W rounded up to a power of two, at most
// 64); each lane takes members lane % LPR + LPR * i.  Group-local shuffles
// reduce; rows are taken 64 / LPR per wave and several batches are in flight.
__device__ __forceinline__ int lanes_per_row(int W) {
    int l = 1;
    while (l < W && l < kWave) l <<= 1;
    return l;
}


// Statistics entries are two tagged words, (tag, first value) and (tag, second
// value); a merge polls them until every word carries the sequence's tag, so
// no team barrier separates the stream from the merge.  Lanes whose entries
// are not yet published load them again.  A lane covers PER members of a row
// (lanes_per_row(W) lanes per row) and issues the loads of KB row groups
// before it waits.  Teams of up to 64 members take one member per lane and
// four groups, so one round trip covers 4096 / lanes_per_row(W) rows (every
// row of a 64-node tree for teams of up to 32); larger teams take four
// members per lane and one group (16 rows per round trip).
template <int KB, int PER>
__device__ __forceinline__ void poll_entries(const uint64_t* stats, const uint32_t (&idx)[KB][PER], int nk, uint64_t tg,
                                             uint64_t (&e)[KB][PER][2], const TeamSync& sync) {
    auto fetch = [&]() {
        bool ok = true;
#pragma unroll
        for (int k = 0; k < KB; ++k) {
            if (k >= nk) break;  // wave-uniform
#pragma unroll
            for (int i = 0; i < PER; ++i) {
                e[k][i][0] = ld_dev(&stats[2 * (size_t)idx[k][i]]);
                e[k][i][1] = ld_dev(&stats[2 * (size_t)idx[k][i] + 1]);
                ok = ok && (e[k][i][0] & 0xffffffff00000000ull) == tg && (e[k][i][1] & 0xffffffff00000000ull) == tg;
            }
        }
        return ok;
    };
    bool ok = false;
    uint32_t polls = 0;
    if (sync.limit > 0) {
        ok = fetch();
        polls = 1;
    } else {
#pragma unroll
        for (int k = 0; k < KB; ++k)
#pragma unroll
            for (int i = 0; i < PER; ++i) e[k][i][0] = e[k][i][1] = 0;
    }
    while (__ballot(!ok)) {
        if (polls >= sync.limit) {
            if (!ok) wait_failed(sync.line, sync.done);
            break;
        }
        __builtin_amdgcn_s_sleep(1);
        if (!ok) ok = fetch();
        ++polls;
    }
}

// Row groups of a merge pass: group k of wave w starts at row
// base + (k kWaves + w) rpw, so every wave takes a group before any takes a
// second; a wave's groups past the last row are skipped (nk counts the
// others).  Entry indices are r W + member with r the storage index of the
// claimed row (srow, or the claim itself when null), with rows past the last
// and members past W clamped so that the loads stay unconditional.
template <int KB, int PER>
__device__ __forceinline__ int entry_indices(int base, int wave, int rpw, int g, int li, int lpr, int nrows,
                                             int W, const int* srow, uint32_t (&idx)[KB][PER]) {
    int nk = 0;
#pragma unroll
    for (int k = 0; k < KB; ++k) {
        const int r0 = base + (k * kWaves + wave) * rpw;
        if (r0 < nrows) nk = k + 1;
        const int ri = min(r0 + g, nrows - 1);
        const int r = srow ? srow[ri] : ri;
#pragma unroll
        for (int i = 0; i < PER; ++i) idx[k][i] = (uint32_t)(r * W + min(li + lpr * i, W - 1));
    }
    return nk;
}

// Sampling: merged max sM[r] and normaliser sS[r] = sum_w s_w exp((m_w - M)/T)
// of every streamed row, from the entries [r][W].  The factors are fp32
// (relative error ~1e-7), the sums fp64.
template <int KB, int PER>
__device__ __forceinline__ void merge_sampling_t(const uint64_t* stats, int nrows, const int* srow, int W, float c,
                                                 float* sM, double* sS, uint64_t tg, const TeamSync& sync) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lpr = lanes_per_row(W);
    const int rpw = kWave / lpr;  // rows per wave per group
    const int g = lane / lpr, li = lane % lpr;
    for (int base = 0; base < nrows; base += KB * kWaves * rpw) {
        uint32_t idx[KB][PER];
        const int nk = entry_indices<KB, PER>(base, wave, rpw, g, li, lpr, nrows, W, srow, idx);
        if (nk == 0) break;
        uint64_t e[KB][PER][2];
        poll_entries<KB, PER>(stats, idx, nk, tg, e, sync);
#pragma unroll
        for (int k = 0; k < KB; ++k) {
            if (k >= nk) break;
            const int ri = base + (k * kWaves + wave) * rpw + g;
            float mk[PER];
#pragma unroll
            for (int i = 0; i < PER; ++i) mk[i] = li + lpr * i < W ? lo_f(e[k][i][0]) : -INFINITY;
            float M = mk[0];
#pragma unroll
            for (int i = 1; i < PER; ++i) M = fmaxf(M, mk[i]);
            M = group_max_dpp(M, lpr);
            double S = 0.0;
#pragma unroll
            for (int i = 0; i < PER; ++i)
                if (mk[i] != -INFINITY) S += (double)lo_f(e[k][i][1]) * (double)__builtin_amdgcn_exp2f((mk[i] - M) * c);
            S = group_sum_dpp(S, lpr);
            if (ri < nrows && li == 0) {
                const int r = srow[ri];
                sM[r] = M;
                sS[r] = S;
            }
        }
    }
}

__device__ __forceinline__ void merge_sampling(const uint64_t* stats, int nrows, const int* srow, int W, float c,
                                               float* sM, double* sS, uint64_t tg, const TeamSync& sync) {
    if (W <= kWave)
        merge_sampling_t<4, 1>(stats, nrows, srow, W, c, sM, sS, tg, sync);
    else
        merge_sampling_t<1, kMaxTeamSize / kWave>(stats, nrows, srow, W, c, sM, sS, tg, sync);
}

// Greedy: argmax amax[r] of the listed target rows r = srow[0..nrows) from
// the entries [r][W].
template <int KB, int PER>
__device__ __forceinline__ void merge_greedy_t(const uint64_t* stats, int nrows, const int* srow, int W, int* amax,
                                               uint64_t tg, const TeamSync& sync) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lpr = lanes_per_row(W);
    const int rpw = kWave / lpr;
    const int g = lane / lpr, li = lane % lpr;
    for (int base = 0; base < nrows; base += KB * kWaves * rpw) {
        uint32_t idx[KB][PER];
        const int nk = entry_indices<KB, PER>(base, wave, rpw, g, li, lpr, nrows, W, srow, idx);
        if (nk == 0) break;
        uint64_t e[KB][PER][2];
        poll_entries<KB, PER>(stats, idx, nk, tg, e, sync);
#pragma unroll
        for (int k = 0; k < KB; ++k) {
            if (k >= nk) break;
            const int ri = base + (k * kWaves + wave) * rpw + g;
            float bv = -INFINITY;
            int bi = 0x7fffffff;
#pragma unroll
            for (int i = 0; i < PER; ++i)
                if (li + lpr * i < W) argmax_merge(bv, bi, lo_f(e[k][i][0]), (int)(uint32_t)e[k][i][1]);
            group_argmax_dpp(bv, bi, lpr);
            if (ri < nrows && li == 0) amax[srow[ri]] = bi;
        }
    }
}

__device__ __forceinline__ void merge_greedy(const uint64_t* stats, int nrows, const int* srow, int W, int* amax,
                                             uint64_t tg, const TeamSync& sync) {
    if (W <= kWave)
        merge_greedy_t<4, 1>(stats, nrows, srow, W, amax, tg, sync);
    else
        merge_greedy_t<1, kMaxTeamSize / kWave>(stats, nrows, srow, W, amax, tg, sync);
}

// --------------------------------------------------------- residual passes --
// Slice passes walk the slice in blocks of pass_vec<VEC4>() 4-element vectors
// per thread; a block's loads are issued together (addresses clamped into the
// slice), then its arithmetic runs under the per-element bounds.
template <bool VEC4>
__device__ constexpr int pass_vec() { return VEC4 ? 4 : 1; }

template <bool VEC4>
__device__ __forceinline__ f32x4 load_slice4(const float* row, int e, int nsl) {
    f32x4 x;
    if constexpr (VEC4) {
        x = *reinterpret_cast<const f32x4*>(row + min(e, nsl - 4));
    } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) x[k] = row[min(e + k, nsl - 1)];
    }
    return x;
}

// One member's slice of w = max(0, R - P_c) into res[] (in place), with R the
// target at u: softmax(q_u / T) (q row pointer given) or the stored residual
// scaled by invZ.  Returns this thread's fp64 share of the slice mass; at `x2`
// (slice-local, or -1) it reports the stored residual before the update (0 when
// R was the target row) and the new one.
template <bool VEC4>
__device__ __forceinline__ double residual_pass(const float* qrow, const float* prow, float Mq, float invSq, float Mp,
                                                float invSp, float invZ, float c, int nsl, float* res, int x2,
                                                float* w_old, float* w_new) {
    double part = 0.0;
    const int n4 = (nsl + 3) / 4;
    constexpr int kPassVec = pass_vec<VEC4>();
    for (int base = 0; base < n4; base += kPassVec * kThreads) {
        f32x4 xq[kPassVec], xp[kPassVec];
#pragma unroll
        for (int i = 0; i < kPassVec; ++i) {
            const int e = 4 * (base + threadIdx.x + kThreads * i);
            xp[i] = load_slice4<VEC4>(prow, e, nsl);
            if (qrow) xq[i] = load_slice4<VEC4>(qrow, e, nsl);
        }
#pragma unroll
        for (int i = 0; i < kPassVec; ++i) {
            const int e4 = base + threadIdx.x + kThreads * i;
            if (e4 >= n4) continue;
            const int e = 4 * e4;
            const f32x4 r = *reinterpret_cast<const f32x4*>(res + e);
            f32x4 wv;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float rv = qrow ? __builtin_amdgcn_exp2f((xq[i][k] - Mq) * c) * invSq : r[k] * invZ;
                const float pv = __builtin_amdgcn_exp2f((xp[i][k] - Mp) * c) * invSp;
                const float w = (e + k < nsl && rv > pv) ? rv - pv : 0.f;
                if (e + k == x2) {
                    *w_old = qrow ? 0.f : r[k];
                    *w_new = w;
                }
                wv[k] = w;
                part += (double)w;
            }
            *reinterpret_cast<f32x4*>(res + e) = wv;
        }
    }
    return part;
}

// softmax(q_u / T) of one slice, unnormalised: res[e] = exp((q - Mq) / T).
template <bool VEC4>
__device__ __forceinline__ void target_slice(const float* qrow, float Mq, float c, int nsl, float* res) {
    const int n4 = (nsl + 3) / 4;
    constexpr int kPassVec = pass_vec<VEC4>();
    for (int base = 0; base < n4; base += kPassVec * kThreads) {
        f32x4 xq[kPassVec];
#pragma unroll
        for (int i = 0; i < kPassVec; ++i) xq[i] = load_slice4<VEC4>(qrow, 4 * (base + threadIdx.x + kThreads * i), nsl);
#pragma unroll
        for (int i = 0; i < kPassVec; ++i) {
            const int e4 = base + threadIdx.x + kThreads * i;
            if (e4 >= n4) continue;
            const int e = 4 * e4;
            f32x4 wv;
#pragma unroll
            for (int k = 0; k < 4; ++k) wv[k] = e + k < nsl ? __builtin_amdgcn_exp2f((xq[i][k] - Mq) * c) : 0.f;
            *reinterpret_cast<f32x4*>(res + e) = wv;
        }
    }
}

// Inverse CDF within one member's slice: the first element e (ascending) whose
// running fp64 sum exceeds tau with res[e] > 0; if none does (tau at or beyond
// the slice total through rounding, or tau < 0 meaning "fallback"), the last
// element with res[e] > 0.  Returns the slice-local index (or -1 if no mass).
__device__ __forceinline__ int slice_draw(const float* res, int nsl, double tau, double* wt, int* s_tok) {
    // an opaque copy of the thread index: what is derived from it stays here
    // instead of occupying registers across the kernel's sequence loop
    int t = threadIdx.x;
    asm volatile("" : "+v"(t));
    const int run = (nsl + kThreads - 1) / kThreads;
    const int a0 = min(nsl, t * run), a1 = min(nsl, a0 + run);
    // the run's total, read from a rotated start (thread t begins t steps in):
    // the lanes of a wave then touch different LDS banks at every step instead
    // of runs `run` words apart (a 32-way conflict for 32-element runs)
    double sum = 0.0;
    int lastp = -1;
    const int len = a1 - a0;
    for (int i = 0, k = len > 0 ? t % len : 0; i < len; ++i) {
        const float v = res[a0 + k];
        sum += (double)v;
        if (v > 0.f) lastp = max(lastp, a0 + k);
        if (++k == len) k = 0;
    }
    double excl, tot;
    const double incl = block_scan_d(sum, wt, excl, tot);
    if (t == 0) *s_tok = -1;
    __syncthreads();
    if (tau >= 0.0 && sum > 0.0 && excl <= tau && incl > tau) {
        double cum = excl;
        int tok = lastp;  // the run's total rounds above tau: its last element with mass
        for (int e = a0; e < a1; ++e) {
            const float v = res[e];
            cum += (double)v;
            if (v > 0.f && cum > tau) {
                tok = e;
                break;
            }
        }
        *s_tok = tok;
    }
    __syncthreads();
    int tok = *s_tok;
    if (tok < 0) {
        // fallback: the last element with mass
        __syncthreads();
        atomicMax(s_tok, lastp);
        __syncthreads();
        tok = *s_tok;
    }
    return tok;
}

// The first set bit at or above `from` of a kMaxNodes-bit mask (kMaxNodes /
// 64 words), or `none`.
__device__ __forceinline__ int first_bit_from(const uint64_t* m, int from, int none) {
    for (int k = from >> 6; k < kMaxNodes / kWave; ++k) {
        uint64_t x = m[k];
        if (k == (from >> 6)) x &= ~0ull << (from & 63);
        if (x) return k * kWave + __ffsll((unsigned long long)x) - 1;
    }
    return none;
}

// A walk candidate prepared ahead: child c of u, with what its test needs
// before the exchange's total is known (pfull: its probability in the draft
// row it was drawn from; px: the probability it is tested against; r: its
// uniform; rx0: its probability under softmax(q_u / T)) and what a rejection
// of it needs (invSp: the scale of the residual pass against its row).  The walk tries each node at most once and always in the
// same state (the same parent and undrawn mass), so a value prepared for node
// c is the value the walk would compute on reaching c.
struct WalkCand {
    double pfull, px, r, rx0;
    float invSp;
    int c;
};

// ---------------------------------------------------------------- the kernel --
template <bool GREEDY, bool VEC4, bool NT>
__global__ __launch_bounds__(kThreads) void spec_accept_kernel(const AccArgs a) {
    const int tid = threadIdx.x;
    const int team = blockIdx.x / a.W;
    const int w = blockIdx.x % a.W;
    const int N = a.N, V = a.V, W = a.W;
    const int s0 = w * a.slice;
    const int nsl = min(V, s0 + a.slice) - s0;
    const float c = a.c;

    __shared__ int s_par[kMaxNodes], s_draft[kMaxNodes], s_path[kMaxNodes], s_depth[kMaxNodes];
    __shared__ int s_srow[2 * kMaxNodes];  // storage index of each claimed row
    __shared__ float s_gq[kMaxNodes], s_gp[kMaxNodes];
    __shared__ float s_M[2 * kMaxNodes];
    __shared__ double s_S[2 * kMaxNodes];
    // sampling: the member's slice of the current residual
    __shared__ __attribute__((aligned(16))) float s_res[GREEDY ? 4 : kMaxSlice];
    __shared__ double s_wt[kWaves];
    __shared__ double s_wtw[2][GREEDY ? 1 : kWaves];  // the walk's two sums per step
    __shared__ double s_mass[GREEDY ? 1 : kMaxTeamSize];
    __shared__ double s_tab[32];
    __shared__ double s_rejZ[GREEDY ? 1 : kMaxNodes];
    __shared__ float s_rejP[GREEDY ? 1 : kMaxNodes];
    __shared__ int s_rej[GREEDY ? 1 : kMaxNodes];
    __shared__ uint64_t s_bal[kMaxNodes / kWave];
    __shared__ float s_wx[2], s_nwx[2];
    __shared__ WalkCand s_prep;     // the walk candidate prepared during an exchange
    __shared__ int s_fc[GREEDY ? 1 : kMaxNodes];  // first child of each node (nb: none)
    __shared__ int s_ns[GREEDY ? 1 : kMaxNodes];  // next sibling of each node (nb: none)
    __shared__ double s_oexcl, s_target;
    __shared__ int s_tok, s_owner, s_fallback, s_rowctr, s_last, s_hitw[kWaves], s_lastw[kWaves];
    __shared__ uint64_t s_base;

    if (tid < 32) exp2_table(s_tab, tid);
    TeamSync sync;
    sync.line = a.ctrl + (size_t)team * kCtrlLine;
    sync.ctrl = a.ctrl;
    sync.team = team;
    sync.nteams = a.nteams;
    sync.lines = a.lines;
    sync.done = a.done;
    sync.limit = a.spin_limit;
    sync.base = 0;
    // this call's tags carry the generation after the workspace's last one
    // (read from the team's own line; the load overlaps the first tree load).
    // Member 0 of each team advances the team's lines once every member has
    // read them (after its first merge, or at the end when the team verified
    // only invalid trees); when a wait ran out, the last workgroup to arrive
    // moves every line past this call
    if (tid == 0) s_base = (ld_dev(&sync.line[0]) + 1) << kTagShift;
    bool have_base = false, gen_done = false;

    int iter = 0;
    for (int b = team; b < a.B; b += a.nteams, ++iter) {
        // ---- tree and drafts of this sequence (its first nb nodes) ----
        const int nb = a.seq_nodes ? a.seq_nodes[b] : N;
        int ok = nb >= 1 && nb <= N;
        if (ok && tid < nb) {
            const int pr = a.parent[(size_t)b * N + tid];
            int d = a.draft[(size_t)b * N + tid];
            d = d < 0 ? 0 : (d >= V ? V - 1 : d);  // out-of-range drafts violate the precondition
            s_par[tid] = pr;
            s_draft[tid] = d;
            ok = tid == 0 ? pr == -1 : (pr >= 0 && pr < tid);
        }
        if (tid == 0) s_rowctr = 0;  // every wave finished the previous stream (workgroup barriers followed it)
        // sampling: children masks of the nodes, built in the residual slice's
        // space (the walk and the final draw of the previous sequence, its only
        // users, ended behind workgroup barriers); one word per thread
        uint64_t* const s_kids = reinterpret_cast<uint64_t*>(s_res);
        if (!GREEDY) {
            static_assert(kMaxNodes * (kMaxNodes / 64) <= kThreads, "one mask word per thread");
            static_assert(GREEDY || kMaxNodes * (kMaxNodes / 64) * 2 <= kMaxSlice, "masks fit the slice space");
            int t = tid;
            asm volatile("" : "+v"(t));  // formed here, not held across the sequence loop
            if (t < kMaxNodes * (kMaxNodes / kWave)) s_kids[t] = 0;
        }
        const bool all_ok = __syncthreads_and(ok) != 0;
        int32_t* out_nodes = a.accepted + (size_t)b * N;
        int32_t* out_toks = a.tokens + (size_t)b * N;
        if (!all_ok) {
            // every member sees the same tree: nobody streams or synchronises.
            // The sequence takes no statistics buffer (iter does not advance):
            // the next one reuses the buffer this one would have taken, so a
            // member never overwrites entries of the sequence before the last
            // one it merged, which another member may still be merging.
            if (w == 0) {
                if (tid == 0) __hip_atomic_store(&a.accept_len[b], -1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                for (int i = tid; i < N; i += kThreads) {
                    out_nodes[i] = -1;
                    out_toks[i] = -1;
                }
            }
            __syncthreads();
            --iter;
            continue;
        }

        const float* qb = a.q + (size_t)b * N * V;
        const float* pb = GREEDY ? nullptr : a.p + (size_t)b * N * V;
        // ---- the rows to stream: target rows 0..nb-1, then (sampling) the
        // draft rows: 1..nb-1, or without replacement the rows of the nodes
        // that have children ----
        if (!GREEDY) {
            int t = tid;
            asm volatile("" : "+v"(t));  // formed here, not held across the sequence loop
            if (t >= 1 && t < nb)
                atomicOr(reinterpret_cast<unsigned long long*>(&s_kids[s_par[t] * (kMaxNodes / kWave) + (t >> 6)]),
                         1ull << (t & 63));
        }
        if (GREEDY && tid < nb) {
            // the first rows: every target row, or the root's (s_depth: see below)
            if (a.greedy_rows) s_srow[tid] = tid;
            else if (tid == 0) s_srow[0] = 0;
            s_depth[tid] = tid == 0 ? 1 : 0;
        }
        {
            // this member's words of the buffer this sequence uses (its
            // statistics entries, then its walk records) are cleared before it
            // writes any of them: the stores complete before the barrier below
            const int R = GREEDY ? N : 2 * N;
            const int nclr = 2 * R + (GREEDY ? 0 : N * kMassRec);
            uint64_t* const sb = a.stats + ((size_t)team * 2 + (iter & 1)) * (size_t)2 * R * W;
            uint64_t* const mb =
                GREEDY ? nullptr
                       : reinterpret_cast<uint64_t*>(a.mass + ((size_t)team * 2 + (iter & 1)) * N * W * kMassRec);
            for (int i = tid; i < nclr; i += kThreads) {
                if (i < 2 * R) st_dev(&sb[2 * ((size_t)(i >> 1) * W + w) + (i & 1)], 0ull);
                else st_dev(&mb[((size_t)((i - 2 * R) / kMassRec) * W + w) * kMassRec + (i - 2 * R) % kMassRec], 0ull);
            }
            __builtin_amdgcn_s_waitcnt(0);
        }
        __syncthreads();  // the row table and the children masks are complete; the clears are done
        if (!GREEDY) {
            // the walk's links, published by the merge's barriers
            int t = tid;
            asm volatile("" : "+v"(t));  // formed here, not held across the sequence loop
            if (t < nb) {
                s_fc[t] = first_bit_from(&s_kids[t * (kMaxNodes / kWave)], t + 1, nb);
                s_ns[t] = t == 0 ? nb : first_bit_from(&s_kids[s_par[t] * (kMaxNodes / kWave)], t + 1, nb);
            }
        }
        // gathered logits of the accept tests, in flight during the stream
        float gq = 0.f, gp = 0.f;
        const int gc = tid + 1;
        if (!GREEDY && gc < nb) {
            const int x = s_draft[gc];
            gq = qb[(size_t)s_par[gc] * V + x];
            gp = pb[(size_t)(a.wor ? s_par[gc] : gc) * V + x];
        }

        // ---- 1. slice statistics of every row, published as entries tagged
        // with (call generation, sequence of this team).  Double-buffered per
        // team: a member starts streaming sequence i + 1 only after it merged
        // sequence i, which needs every member's entries of i, so no member can
        // overwrite a buffer that another still merges ----
        if (!have_base) {
            // written before the tree barrier; uniform (kept in scalar registers)
            sync.base = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(s_base >> 32)) << 32) |
                        (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)s_base);
            have_base = true;
        }
        const uint64_t stag = (uint64_t)(gen_tag(sync) | ((uint32_t)iter & 0xfffu)) << 32;
        uint64_t* stats = a.stats + ((size_t)team * 2 + (iter & 1)) * (size_t)2 * (GREEDY ? N : 2 * N) * W;
        if constexpr (GREEDY) {
            // ---- 2. the end node: the deepest node whose path matches (every
            // node's draft equals its parent's argmax), ties to the smallest
            // index.  Small rows: every target row's argmax up front, then each
            // node checks its own path (s_depth[t]: node t matches).  Large
            // rows: breadth-first, each level's target rows streamed and merged
            // as it is reached (level 0 is the root, level k + 1 the matching
            // children of level-k nodes; s_depth[t]: level of t + 1 on a
            // matching path, else 0; s_srow: the level's nodes in index order),
            // and the end node is the first node of the last level ----
            int* s_amax = s_path;  // reuse: argmax per target row
            const bool all_rows = a.greedy_rows != 0;
            int lvl = 0, nl = 1, e = 0;
            for (;;) {
                if (lvl == 0 || !all_rows) {  // uniform: one stream and merge site for both forms
                    const int nr = all_rows ? nb : nl;
                    stream_slices<GREEDY, VEC4, NT, true>(qb, pb, nr, N, V, s0, nsl, c, stats, W, w, &s_rowctr, stag,
                                                          s_srow);
                    merge_greedy(stats, nr, s_srow, W, s_amax, stag, sync);
                    __syncthreads();
                    advance_generation(sync, w, gen_done);
                }
                if (all_rows) {
                    // every node checks its own path (s_depth[t]: node t matches);
                    // member 0 alone, which writes the path
                    if (w != 0) break;
                    if (tid < nb) s_depth[tid] = tid == 0 ? 1 : (s_draft[tid] == s_amax[s_par[tid]]);
                    __syncthreads();
                    float key = -1.f;
                    int kidx = tid;
                    if (tid < nb) {
                        int d = 0;
                        bool v = true;
                        for (int j = tid; j != 0; j = s_par[j]) {
                            v = v && s_depth[j] != 0;
                            ++d;
                        }
                        key = v ? (float)d : -1.f;
                    }
                    group_argmax_dpp(key, kidx, kWave);
                    if ((tid & (kWave - 1)) == 0) {
                        s_hitw[tid >> 6] = kidx;
                        s_wt[tid >> 6] = key;
                    }
                    __syncthreads();
                    float bk = s_wt[0];
                    e = s_hitw[0];
                    for (int k = 1; k < kWaves; ++k) argmax_merge(bk, e, (float)s_wt[k], s_hitw[k]);
                    lvl = (int)bk;
                    break;
                }
                // the next level: the matching children of this level's nodes
                e = s_srow[0];
                int t = tid;
                asm volatile("" : "+v"(t));  // formed here, not held across the sequence loop
                const bool next = t >= 1 && t < nb && s_depth[s_par[t]] == lvl + 1 && s_draft[t] == s_amax[s_par[t]];
                if (t < kMaxNodes) {
                    const uint64_t bal = __ballot(next);
                    if ((t & (kWave - 1)) == 0) s_bal[t >> 6] = bal;
                }
                if (tid == 0) s_rowctr = 0;  // every wave finished the stream (the merge's barrier)
                __syncthreads();  // every read of s_srow, s_depth and s_bal's old words is done
                int before = 0, total = 0;
#pragma unroll
                for (int k = 0; k < kMaxNodes / kWave; ++k) {
                    const int pc = __popcll(s_bal[k]);
                    total += pc;
                    if (k < (t >> 6)) before += pc;
                }
                if (total == 0) break;  // uniform
                if (next) {
                    s_depth[t] = lvl + 2;
                    s_srow[before + __popcll(s_bal[t >> 6] & ((1ull << (t & 63)) - 1ull))] = t;
                }
                ++lvl;
                nl = total;
                __syncthreads();  // the next level's list
            }
            if (w != 0) continue;  // member 0 writes the path
            // member 0 writes the path to e and the extra token, e's argmax
            if (w == 0) {
                for (int i = tid; i < N; i += kThreads) {
                    if (i >= lvl) out_nodes[i] = -1;
                    if (i > lvl) out_toks[i] = -1;
                }
                if (tid == 0) {
                    for (int i = e, k = lvl - 1; i != 0; i = s_par[i], --k) {
                        out_nodes[k] = i;
                        out_toks[k] = s_draft[i];
                    }
                    out_toks[lvl] = s_amax[e];
                    __hip_atomic_store(&a.accept_len[b], lvl, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
            }
            __syncthreads();
        } else {
            // ---- 3. every member merges every row ----
            if (gc < nb) {
                s_gq[gc] = gq;
                s_gp[gc] = gp;
            }
            if (tid == 0) s_prep.c = -1;  // published by the family's barriers
            const bool wor = a.wor != 0;
            // The rows of node un's family: its target row and the draft rows
            // its children were drawn from (their own rows, or without
            // replacement un's row), listed in s_srow; returns their number.
            // Every member lists the same rows in the same order.
            const auto family = [&](int un) -> int {
                int t = tid;
                asm volatile("" : "+v"(t));  // formed here, not held across the sequence loop
                const bool kid = t >= 1 && t < nb && s_par[t] == un;
                if (t < kMaxNodes) {
                    const uint64_t bal = __ballot(kid);
                    if ((t & (kWave - 1)) == 0) s_bal[t >> 6] = bal;
                }
                if (tid == 0) s_rowctr = 0;  // every wave finished the previous stream
                __syncthreads();
                int before = 0, total = 0;
#pragma unroll
                for (int k = 0; k < kMaxNodes / kWave; ++k) {
                    const int pc = __popcll(s_bal[k]);
                    total += pc;
                    if (k < (t >> 6)) before += pc;
                }
                if (kid) before += __popcll(s_bal[t >> 6] & ((1ull << (t & 63)) - 1ull));
                int nn = N;
                asm volatile("" : "+s"(nn));  // formed here, not held across the sequence loop
                if (tid == 0) {
                    s_srow[0] = un;
                    if (wor && total > 0) s_srow[1] = nn + un;
                }
                if (!wor && kid) s_srow[1 + before] = nn + t;
                __syncthreads();
                return 1 + (wor ? (total > 0 ? 1 : 0) : total);
            };
            // statistics of node un's family, streamed and merged
            const auto family_stats = [&](int un) {
                const int nf = family(un);
                stream_slices<GREEDY, VEC4, NT, true>(qb, pb, nf, N, V, s0, nsl, c, stats, W, w, &s_rowctr, stag,
                                                      s_srow);
                merge_sampling(stats, nf, s_srow, W, c, s_M, s_S, stag, sync);
                __syncthreads();
            };

            // ---- the walk (identical on every member) ----
            const double inv_t64 = a.inv_t64;
            double* massb = a.mass + ((size_t)team * 2 + (iter & 1)) * N * W * kMassRec;
            int u = 0, len = 0, pass = 0, nrej = 0;
            bool res_active = false;  // target at u: residual s_res / Z, else softmax(q_u / T)
            double Z = 1.0, wx_cur = 0.0;
            double zrem = 1.0;        // without replacement: draft mass at u not yet drawn
            // a candidate's values, one expression each (the same code computes
            // them here and when they are prepared ahead)
            const auto cand_pfull = [&](int cn, int pr) {
                return exp_scaled(s_gp[cn], s_M[N + pr], inv_t64, s_tab) / s_S[N + pr];
            };
            const auto cand_px = [&](double pf, int cn, int un, double zr) {
                if (!wor) return pf;
                // a token already drawn by an earlier sibling has no mass left
                bool dup = false;
                for (int j = un + 1; j < cn; ++j) dup = dup || (s_par[j] == un && s_draft[j] == s_draft[cn]);
                return (dup || !(zr > 0.0)) ? 0.0 : pf / zr;
            };
            const auto cand_r = [&](int cn) {
                uint64_t sd = a.seed;
                asm volatile("" : "+s"(sd));  // the key schedule is formed here, not held across the kernel
                return (double)philox_uniform(sd, (uint32_t)cn, (uint32_t)b, 0u);
            };
            const auto cand_rx0 = [&](int cn, int un) { return exp_scaled(s_gq[cn], s_M[un], inv_t64, s_tab) / s_S[un]; };
            const auto cand_invSp = [&](int pr, double zr) { return (float)(1.0 / (s_S[N + pr] * zr)); };
            int c_cur = nb;  // the next child of u to try (nb: none left)
            int invSq_u = -1;  // the node invSq belongs to
            float invSq = 0.f;
            bool arrived = true;  // at u, whose family's statistics are still to come
            for (;;) {
                if (arrived) {
                    // the rows of u's tests (one call site: the stream is inlined
                    // once); its barriers also publish the tree's links
                    family_stats(u);
                    advance_generation(sync, w, gen_done);
                    c_cur = s_fc[u];
                    arrived = false;
                }
                if (c_cur >= nb) break;  // every child of u tried, or u is a leaf
                const int cc = c_cur;
                const int pr_c = wor ? u : cc;  // the draft row cc was drawn from
                const bool pk = s_prep.c == cc;
                const double pfull = pk ? s_prep.pfull : cand_pfull(cc, pr_c);
                {
                    const double rx = res_active ? wx_cur / Z : (pk ? s_prep.rx0 : cand_rx0(cc, u));
                    const double px = pk ? s_prep.px : cand_px(pfull, cc, u, zrem);
                    const double acc = px == 0.0 ? 1.0 : fmin(1.0, rx / px);
                    const double r = pk ? s_prep.r : cand_r(cc);
                    if (r < acc) {
                        if (tid == 0) s_path[len] = cc;
                        ++len;
                        u = cc;
                        res_active = false;
                        Z = 1.0;
                        zrem = 1.0;
                        nrej = 0;
                        arrived = true;
                        continue;
                    }
                }
                // ---- 4. rejected: residual pass over the slices.  Only the member
                // that owns the next sibling's token publishes words 2 and 3 that
                // anyone reads, and its pass always writes them (x2l is in its
                // slice), so s_wx needs no reset.  Barriers: the two sums (each on
                // its own array, so no leading barrier) ----
                const int nxt = s_ns[cc];
                const int x2 = nxt < nb ? s_draft[nxt] - s0 : -1;
                const int x2l = (x2 >= 0 && x2 < nsl) ? x2 : -1;
                const float Mq = s_M[u];
                if (invSq_u != u) {
                    invSq = (float)(1.0 / s_S[u]);
                    invSq_u = u;
                }
                const float invZ = (float)(1.0 / Z);
                const float invSp = pk ? s_prep.invSp : cand_invSp(pr_c, zrem);
                const float* q_u = qb + (size_t)u * V + s0;
                const float* p_c = pb + (size_t)pr_c * V + s0;
                const double part = residual_pass<VEC4>(res_active ? nullptr : q_u, p_c, Mq, invSq, s_M[N + pr_c],
                                                        invSp, invZ, c, nsl, s_res, x2l, &s_wx[1], &s_wx[0]);
                if (wor) zrem -= pfull;
                const double smass = block_sum_1b(part, s_wtw[0]);  // its barrier publishes s_wx
                // publish and gather in one step: every word carries the step's tag,
                // so a member polls the other members' words directly
                uint64_t* slot = reinterpret_cast<uint64_t*>(massb + (size_t)pass * W * kMassRec);
                const uint64_t tg = (uint64_t)exchange_tag(sync, iter, pass) << 32;
                if (tid == 0) {
                    const uint64_t mb = (uint64_t)__double_as_longlong(smass);
                    st_dev(&slot[w * kMassRec + 0], tg | (uint32_t)mb);
                    st_dev(&slot[w * kMassRec + 1], tg | (uint32_t)(mb >> 32));
                    st_dev(&slot[w * kMassRec + 2], tg | __float_as_uint(s_wx[0]));  // new residual at the next token
                    st_dev(&slot[w * kMassRec + 3], tg | __float_as_uint(s_wx[1]));  // stored residual before the pass
                }
                const int xo = nxt < nb ? s_draft[nxt] / a.slice : -1;
                double mt = 0.0;
                if (tid < W) {
                    // the residuals at the next token only from the member that owns it
                    uint64_t e[kMassRec] = {0, 0, 0, 0};
                    gather_tagged(sync, &slot[tid * kMassRec], tg, tid == xo ? kMassRec : 2, e);
                    mt = __longlong_as_double((long long)((e[1] << 32) | (uint32_t)e[0]));
                    if (tid == xo) {
                        s_nwx[0] = __uint_as_float((uint32_t)e[2]);
                        s_nwx[1] = __uint_as_float((uint32_t)e[3]);
                    }
                }
                // The last wave takes no part in the polls: while they run its
                // first lane prepares the next candidate (the next sibling, with
                // the mass left after this pass; its row is in u's family).  The
                // barrier of the sum below publishes it.
                if (tid == kThreads - kWave) {
                    if (nxt < nb) {
                        const int pr = wor ? u : nxt;
                        WalkCand wc;
                        wc.c = nxt;
                        wc.pfull = cand_pfull(nxt, pr);
                        wc.px = cand_px(wc.pfull, nxt, u, zrem);
                        wc.r = cand_r(nxt);
                        wc.rx0 = cand_rx0(nxt, u);
                        wc.invSp = cand_invSp(pr, zrem);
                        s_prep = wc;
                    } else {
                        s_prep.c = -1;
                    }
                }
                const double Znew = block_sum_1b(mt, s_wtw[1]);  // its barrier publishes s_nwx and s_prep
                ++pass;
                if (Znew > 0.0) {
                    if (tid < W) s_mass[tid] = mt;
                    if (tid == 0) {
                        s_rej[nrej] = cc;
                        s_rejZ[nrej] = Znew;
                        s_rejP[nrej] = invSp;
                    }
                    ++nrej;
                    res_active = true;
                    Z = Znew;
                    wx_cur = (double)s_nwx[0];
                } else {
                    // zero mass cannot follow a rejection in exact arithmetic: keep R.  The
                    // slice was overwritten, so rebuild it from q_u and the earlier rejections.
                    if (res_active) wx_cur = (double)s_nwx[1];
                    __syncthreads();
                    for (int k = 0; k < nrej; ++k) {
                        const int ck = s_rej[k];
                        const int pk = wor ? u : ck;
                        const float iz = (float)(1.0 / (k == 0 ? 1.0 : s_rejZ[k - 1]));
                        residual_pass<VEC4>(k == 0 ? q_u : nullptr, pb + (size_t)pk * V + s0, Mq, invSq, s_M[N + pk],
                                            s_rejP[k], iz, c, nsl, s_res, -1, &s_wx[1], &s_wx[1]);
                    }
                }
                c_cur = nxt;
            }

            // ---- 5. the extra token: inverse CDF over the slices ----
            uint64_t sd = a.seed;
            asm volatile("" : "+s"(sd));  // the key schedule is formed here, not held across the kernel
            const double ut = (double)philox_uniform(sd, (uint32_t)u, (uint32_t)b, 1u);
            // slice masses: of the last residual pass, or from the statistics when
            // drawing from softmax(q_u / T)
            double mt = 0.0;
            if (tid < W) {
                if (res_active) {
                    mt = s_mass[tid];
                } else {
                    const float em = lo_f(ld_dev(&stats[2 * ((size_t)u * W + tid)]));
                    const float es = lo_f(ld_dev(&stats[2 * ((size_t)u * W + tid) + 1]));
                    mt = em == -INFINITY ? 0.0 : (double)es * (double)__builtin_amdgcn_exp2f((em - s_M[u]) * c);
                }
            }
            // owner: the first slice whose running mass exceeds the target; else the last with mass
            double target;
            if (W <= kWave) {
                // every mass sits in wave 0, whose own scan is the block scan's result
                // (the other waves add exact zeros): one barrier publishes the owner
                if (tid < kWave) {
                    int lane = tid;
                    asm volatile("" : "+v"(lane));  // formed here, not held across the sequence loop
                    double v = mt;
#pragma unroll
                    for (int o = 1; o < kWave; o <<= 1) {
                        const double y = __shfl_up(v, o);
                        if (lane >= o) v += y;
                    }
                    const double prev = __shfl_up(v, 1);
                    const double tot = __shfl(v, kWave - 1);
                    const double tg = ut * tot;
                    const bool has = tid < W && mt > 0.0;
                    const uint64_t hit = __ballot(has && v > tg);
                    const uint64_t pos = __ballot(has);
                    const int own = hit ? __ffsll((unsigned long long)hit) - 1
                                        : (pos ? 63 - __clzll((unsigned long long)pos) : -1);
                    if (tid == 0) {
                        s_owner = own;
                        s_fallback = hit == 0;
                        s_target = tg;
                    }
                    if (tid == own) s_oexcl = lane == 0 ? 0.0 : prev;
                }
                __syncthreads();
                target = s_target;
            } else {
                double mexcl, total;
                const double mincl = block_scan_d(mt, s_wt, mexcl, total);
                target = ut * total;
                const bool has = tid < W && mt > 0.0;
                const uint64_t hit = __ballot(has && mincl > target);
                const uint64_t pos = __ballot(has);
                int t = tid;
                asm volatile("" : "+v"(t));  // formed here, not held across the sequence loop
                const int lane = t & 63, wv = t >> 6;
                if (lane == 0) {
                    s_hitw[wv] = hit ? wv * kWave + __ffsll((unsigned long long)hit) - 1 : -1;
                    s_lastw[wv] = pos ? wv * kWave + 63 - __clzll((unsigned long long)pos) : -1;
                }
                __syncthreads();
                if (tid == 0) {
                    int owner = -1, lastm = -1;
                    for (int k = 0; k < kWaves; ++k) {
                        if (owner < 0) owner = s_hitw[k];
                        lastm = max(lastm, s_lastw[k]);
                    }
                    s_fallback = owner < 0;
                    s_owner = owner < 0 ? lastm : owner;
                }
                __syncthreads();
                if (tid == s_owner) s_oexcl = mexcl;
                __syncthreads();
            }
            const int owner = s_owner;
            if (w == owner) {
                if (!res_active) target_slice<VEC4>(qb + (size_t)u * V + s0, s_M[u], c, nsl, s_res);
                __syncthreads();
                const double tau = s_fallback ? -1.0 : target - s_oexcl;
                int tok = slice_draw(s_res, nsl, tau, s_wt, &s_tok);
                tok = tok < 0 ? nsl - 1 : tok;
                for (int i = tid; i < N; i += kThreads) {
                    out_nodes[i] = i < len ? s_path[i] : -1;
                    out_toks[i] = i < len ? s_draft[s_path[i]] : (i == len ? s0 + tok : -1);
                }
                if (tid == 0) __hip_atomic_store(&a.accept_len[b], len, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            } else if (owner < 0 && w == 0) {
                // no mass anywhere (only possible with non-finite logits): last token
                for (int i = tid; i < N; i += kThreads) {
                    out_nodes[i] = i < len ? s_path[i] : -1;
                    out_toks[i] = i < len ? s_draft[s_path[i]] : (i == len ? V - 1 : -1);
                }
                if (tid == 0) __hip_atomic_store(&a.accept_len[b], len, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            __syncthreads();
        }  // sampling
    }
    // A team whose every tree was invalid merged nothing and so never advanced
    // its lines: it does now.  None of its members tags a word in this call,
    // so it does not matter when the others read the line.
    if (!gen_done) {
        if (!have_base)
            sync.base = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(s_base >> 32)) << 32) |
                        (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)s_base);
        advance_generation(sync, w, gen_done);
    }

    // ---- arrival: the last workgroup reports the teams whose waits ran out.
    // Each workgroup's accept_len stores are made by its thread 0 before this
    // release; a wait that ran out released its team mark with its count ----
    __syncthreads();
    if (tid == 0) {
        const uint64_t old = __hip_atomic_fetch_add(a.done, 1ull, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        const bool last = (uint32_t)old == gridDim.x - 1;
        s_last = last ? ((old >> 32) != 0 ? 2 : 1) : 0;
        if (last) st_dev(a.done, 0ull);  // every workgroup has arrived: ready for the next call
    }
    __syncthreads();
    if (s_last == 2) {
        for (int t = tid; t < a.nteams; t += kThreads) {
            uint64_t* line = a.ctrl + (size_t)t * kCtrlLine;
            if (ld_dev(&line[2]) == 0) continue;
            for (int bb = t; bb < a.B; bb += a.nteams)
                __hip_atomic_store(&a.accept_len[bb], -2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            st_dev(&line[2], 0ull);
        }
        // members may have tagged words with this call's generation or the
        // next one (a member that read its line after member 0 advanced it):
        // every line moves past both
        const uint64_t gen = s_base >> kTagShift;
        for (int t = tid; t < a.lines; t += kThreads) st_dev(&a.ctrl[(size_t)t * kCtrlLine], gen + 1);
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

KernelFn pick(bool greedy, bool vec4, bool nt) {
    if (nt) {
        if (greedy) return vec4 ? spec_accept_kernel<true, true, true> : spec_accept_kernel<true, false, true>;
        return vec4 ? spec_accept_kernel<false, true, true> : spec_accept_kernel<false, false, true>;
    }
    if (greedy) return vec4 ? spec_accept_kernel<true, true, false> : spec_accept_kernel<true, false, false>;
    return vec4 ? spec_accept_kernel<false, true, false> : spec_accept_kernel<false, false, false>;
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
            for (bool v4 : modes)
                for (bool nt : modes) {
                    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
                            &per, reinterpret_cast<const void*>(pick(g, v4, nt)), kThreads, 0) != hipSuccess)
                        return 0;
                    per_min = per < per_min ? per : per_min;
                }
        if (per_min < 1) return 0;
        cache[dev] = ncu * per_min;
    }
    return cache[dev];
}

// 0 ok, else a tv_status.
int make_plan(int B, int N, int V, int greedy, AcceptPlan& pl) {
    const int cap = resident_capacity();
    if (cap <= 0) return TV_ERR_HIP;
    int wmax = (V + kMinSlice - 1) / kMinSlice;
    if (wmax > kMaxTeamSize) wmax = kMaxTeamSize;
    // sampling: a small stream (few rows) spread over many members costs more
    // in merge and exchange round trips than their shares save (a 6-node chain
    // over 128256 tokens: 62 members took 6% less time than 126, which also
    // leaves the team on the merge for at most 64 members).  Greedy merges
    // only (max, argmax) and was slower with the same floor.
    if (!greedy) {
        const long wbytes = (2L * N - 1) * (long)V * 4 / kMinMemberBytes;
        if (wbytes < wmax) wmax = wbytes < 1 ? 1 : (int)wbytes;
    }
    // sampling keeps a member's residual slice in LDS
    const int wmin = greedy ? (V + kMaxSpans * kSpan - 1) / (kMaxSpans * kSpan) : (V + kMaxSlice - 1) / kMaxSlice;
    if (wmin > kMaxTeamSize) return TV_ERR_UNSUPPORTED;
    if (wmax < wmin) wmax = wmin;
    int W = cap / (B > 0 ? B : 1);
    if (W > wmax) W = wmax;
    if (W < wmin) W = wmin;
    if (W < 1) W = 1;
    if (W > cap) return TV_ERR_UNSUPPORTED;  // a team must be resident at once
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
    // The team lines sit at the same offsets for every shape and mode and
    // every other word is tagged with its call's generation, so a workspace
    // serves later calls of any shape without clearing.
    size_t off = 0;
    pl.ctrl_off = off;
    off += round_up((size_t)kMaxTeams * kCtrlLine * sizeof(uint64_t), 256);
    pl.done_off = off;
    off += 256;
    pl.stats_off = off;
    off += round_up((size_t)nteams * 2 * 2 * (greedy ? N : 2 * N) * W * sizeof(uint64_t), 256);
    pl.mass_off = off;
    if (!greedy) off += round_up((size_t)nteams * 2 * N * W * kMassRec * sizeof(double), 256);
    pl.total = off;
    return TV_OK;
}

std::atomic<uint32_t> g_wait_limit{kSpinLimit};

// Host checks and the launch; `ws` holds at least pl.total bytes.
int launch_accept(const float* q_logits, const float* p_logits, const int32_t* draft_tokens, const int32_t* parent,
                  const int32_t* seq_nodes, int B, int N, int V, uint64_t philox_seed, float temperature, int flags,
                  int32_t* accept_len, int32_t* accepted_nodes, int32_t* out_tokens, char* ws, const AcceptPlan& pl,
                  hipStream_t stream) {
    const bool greedy = (flags & TV_ACCEPT_GREEDY) != 0;
    AccArgs a;
    a.q = q_logits;
    a.p = p_logits;
    a.draft = draft_tokens;
    a.parent = parent;
    a.seq_nodes = seq_nodes;
    a.accept_len = accept_len;
    a.accepted = accepted_nodes;
    a.tokens = out_tokens;
    a.ctrl = reinterpret_cast<uint64_t*>(ws + pl.ctrl_off);
    a.done = reinterpret_cast<uint64_t*>(ws + pl.done_off);
    a.stats = reinterpret_cast<uint64_t*>(ws + pl.stats_off);
    a.mass = greedy ? nullptr : reinterpret_cast<double*>(ws + pl.mass_off);
    a.B = B;
    a.N = N;
    a.V = V;
    a.W = pl.W;
    a.slice = pl.slice;
    a.nteams = pl.nteams;
    a.lines = min(resident_capacity(), kMaxTeams);  // every plan's teams fit (nteams <= capacity / W)
    a.wor = (!greedy && (flags & TV_ACCEPT_SIBLINGS_WOR)) ? 1 : 0;
    // greedy: a member's share of every target row up front when it is small
    // (its stream costs less than the round trips of a walk level by level)
    a.greedy_rows = (double)N * pl.slice * 4.0 <= kGreedyRowsUpFront ? 1 : 0;
    a.spin_limit = g_wait_limit.load(std::memory_order_relaxed);
    a.c = greedy ? 1.f : (float)(1.4426950408889634 / (double)temperature);
    a.inv_t64 = greedy ? 1.0 : 1.0 / (double)temperature;
    a.seed = philox_seed;
    const bool vec4 = (V % 4 == 0) && aligned(q_logits, 16) && (greedy || aligned(p_logits, 16));
    // Logits that cannot stay in the device's 256 MB Infinity Cache between
    // their producer and this pass are streamed with non-temporal loads
    // (a plain read of 4 GiB: ~6.8-7.0 TB/s against ~6.1-6.3 with ordinary
    // loads); below twice its size, cached reuse is worth more.
    const double stream_bytes = (double)B * (greedy ? N : 2 * N - 1) * (double)V * 4.0;
    // (sampling streams only the rows of the nodes the walk reaches, and its
    // residual passes read them again: its loads keep the lines cached)
    const bool nt = greedy && stream_bytes > kNonTemporalBytes;
    // The grid never exceeds the resident capacity from the occupancy query, so
    // once earlier work on the stream drains every member is resident and the
    // polls for other members' words make progress (their waits are bounded
    // regardless, and one that runs out is reported as accept_len -2).
    hipLaunchKernelGGL(pick(greedy, vec4, nt), dim3(pl.nteams * pl.W), dim3(kThreads), 0, stream, a);
    return launch_status();
}

// Argument checks shared by the entry points: TV_OK or a tv_status.
int check_accept_args(const float* q_logits, const float* p_logits, const int32_t* draft_tokens,
                      const int32_t* parent, int B, int N, int V, float temperature, int flags, int32_t* accept_len,
                      int32_t* accepted_nodes, int32_t* out_tokens) {
    const bool greedy = (flags & TV_ACCEPT_GREEDY) != 0;
    if (B < 0 || N < 1 || V < 1) return TV_ERR_INVALID_ARG;
    if ((flags & ~(TV_ACCEPT_GREEDY | TV_ACCEPT_SIBLINGS_WOR)) != 0) return TV_ERR_INVALID_ARG;
    if (N > TV_MAX_NODES) return TV_ERR_UNSUPPORTED;
    if (!greedy && !(temperature > 0.f && temperature <= FLT_MAX)) return TV_ERR_INVALID_ARG;
    if (B == 0) return TV_OK;
    if (!q_logits || (!greedy && !p_logits) || !draft_tokens || !parent || !accept_len || !accepted_nodes ||
        !out_tokens)
        return TV_ERR_INVALID_ARG;
    if (!aligned(q_logits, 4) || (!greedy && !aligned(p_logits, 4))) return TV_ERR_INVALID_ARG;
    return TV_OK;
}

}  // namespace
}  // namespace tv

extern "C" size_t tv_spec_accept_workspace(int B, int N, int V, int greedy) {
    if (B <= 0 || N < 1 || N > TV_MAX_NODES || V < 1) return 0;
    tv::AcceptPlan pl;
    if (tv::make_plan(B, N, V, greedy, pl) != TV_OK) return 0;
    return pl.total;
}

extern "C" int tv_spec_accept_plan(int B, int N, int V, int greedy, int* team_size, int* teams, int* slice) {
    if (B <= 0 || N < 1 || N > TV_MAX_NODES || V < 1) return TV_ERR_INVALID_ARG;
    tv::AcceptPlan pl;
    const int st = tv::make_plan(B, N, V, greedy, pl);
    if (st != TV_OK) return st;
    if (team_size) *team_size = pl.W;
    if (teams) *teams = pl.nteams;
    if (slice) *slice = pl.slice;
    return TV_OK;
}

extern "C" uint32_t tv_set_wait_limit(uint32_t polls) {
    return tv::g_wait_limit.exchange(polls == TV_WAIT_DEFAULT ? tv::kSpinLimit : polls);
}

extern "C" int tv_spec_accept_ex(const float* q_logits, const float* p_logits, const int32_t* draft_tokens,
                                 const int32_t* parent, const int32_t* seq_nodes, int B, int N, int V,
                                 uint64_t philox_seed, float temperature, int flags, int32_t* accept_len,
                                 int32_t* accepted_nodes, int32_t* out_tokens, void* workspace, size_t workspace_bytes,
                                 void* stream) {
    using namespace tv;
    int st = check_accept_args(q_logits, p_logits, draft_tokens, parent, B, N, V, temperature, flags, accept_len,
                               accepted_nodes, out_tokens);
    if (st != TV_OK || B == 0) return st;
    if (!workspace || !aligned(workspace, 256)) return TV_ERR_WORKSPACE;
    AcceptPlan pl;
    st = make_plan(B, N, V, flags & TV_ACCEPT_GREEDY, pl);
    if (st != TV_OK) return st;
    if (workspace_bytes < pl.total) return TV_ERR_WORKSPACE;
    return launch_accept(q_logits, p_logits, draft_tokens, parent, seq_nodes, B, N, V, philox_seed, temperature, flags,
                         accept_len, accepted_nodes, out_tokens, static_cast<char*>(workspace), pl,
                         (hipStream_t)stream);
}

namespace tv {
namespace {

// ---------------------------------------------- the allocation-free variant --
// Scratch of tv_spec_accept_noalloc: file-scope device memory, one copy per
// GPU (held until the process ends).  Host code never passes `scratch` itself
// to a kernel (in host code it is only a stand-in for the symbol): it uses the
// device address that hipGetSymbolAddress returns, looked up once per device.
constexpr size_t kScratchBytes = TV_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Puts the scratch's control words in the state a call leaves them in: every
// team line holds the same generation (the largest one found, so that running
// this again never moves a generation back), no wait marks, arrival word 0.
// Safe to run between any two calls: when the first call on a device is
// captured into a HIP graph, this runs before the accept kernel on every
// replay, and the replays still see a new generation each (zeroing the lines
// instead would give every replay the same one, and a replay could take the
// previous replay's statistics entries for its own).  One workgroup of
// kMaxTeams threads.
__global__ __launch_bounds__(kMaxTeams) void scratch_init_kernel(uint64_t* __restrict__ ctrl, uint64_t* __restrict__ done) {
    __shared__ uint64_t s_g[kMaxTeams / kWave];
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    uint64_t g = ctrl[(size_t)t * kCtrlLine];
    for (int off = 32; off > 0; off >>= 1) {
        const uint64_t o = __shfl_xor(g, off);
        g = o > g ? o : g;
    }
    if (lane == 0) s_g[wv] = g;
    __syncthreads();
    g = s_g[0];
    for (int i = 1; i < kMaxTeams / kWave; ++i) g = s_g[i] > g ? s_g[i] : g;
    ctrl[(size_t)t * kCtrlLine] = g;
    ctrl[(size_t)t * kCtrlLine + 2] = 0ull;
    if (t == 0) *done = 0ull;
}

// The scratch's device address on the current device, with its control words
// (team generations, wait marks, arrival word) put in order once, on
// `stream`, before first use.  Every other word the kernel reads carries a
// nonzero tag and is cleared by its owner before use, so never-written
// scratch is never taken for data.  nullptr on failure.
char* device_scratch(hipStream_t stream) {
    static std::mutex mu;
    static char* ptr[64] = {nullptr};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    std::lock_guard<std::mutex> lock(mu);
    if (ptr[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
        // the plan's layout: control lines at offset 0, the arrival word after them
        char* base = static_cast<char*>(p);
        const size_t done_off = round_up((size_t)kMaxTeams * kCtrlLine * sizeof(uint64_t), 256);
        hipLaunchKernelGGL(scratch_init_kernel, dim3(1), dim3(kMaxTeams), 0, stream, reinterpret_cast<uint64_t*>(base),
                           reinterpret_cast<uint64_t*>(base + done_off));
        if (hipGetLastError() != hipSuccess) return nullptr;
        ptr[dev] = static_cast<char*>(p);
    }
    return ptr[dev];
}

}  // namespace
}  // namespace tv

extern "C" int tv_spec_accept_noalloc(const float* q_logits, const float* p_logits, const int32_t* draft_tokens,
                                      const int32_t* parent, const int32_t* seq_nodes, int B, int N, int V,
                                      uint64_t philox_seed, float temperature, int flags, int32_t* accept_len,
                                      int32_t* accepted_nodes, int32_t* out_tokens, void* stream) {
    using namespace tv;
    int st = check_accept_args(q_logits, p_logits, draft_tokens, parent, B, N, V, temperature, flags, accept_len,
                               accepted_nodes, out_tokens);
    if (st != TV_OK || B == 0) return st;
    AcceptPlan pl;
    st = make_plan(B, N, V, flags & TV_ACCEPT_GREEDY, pl);
    if (st != TV_OK) return st;
    if (pl.total > kScratchBytes) return TV_ERR_SCRATCH;
    char* ws = device_scratch((hipStream_t)stream);
    if (!ws) return TV_ERR_HIP;
    return launch_accept(q_logits, p_logits, draft_tokens, parent, seq_nodes, B, N, V, philox_seed, temperature, flags,
                         accept_len, accepted_nodes, out_tokens, ws, pl, (hipStream_t)stream);
}

extern "C" int tv_spec_accept(const float* q_logits, const float* p_logits, const int32_t* draft_tokens,
                              const int32_t* parent, int B, int N, int V, uint64_t philox_seed, float temperature,
                              int greedy, int32_t* accept_len, int32_t* accepted_nodes, int32_t* out_tokens,
                              void* workspace, size_t workspace_bytes, void* stream) {
    return tv_spec_accept_ex(q_logits, p_logits, draft_tokens, parent, nullptr, B, N, V, philox_seed, temperature,
                             greedy ? TV_ACCEPT_GREEDY : 0, accept_len, accepted_nodes, out_tokens, workspace,
                             workspace_bytes, stream);
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
