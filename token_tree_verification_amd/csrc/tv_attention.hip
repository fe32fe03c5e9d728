// tv_tree_attention: ancestor-masked attention of draft-tree nodes over the
// committed KV cache plus their own root-to-node path.
//
// EAGLE explainer (paper-2401-10774), section on parallel verification with a
// static tree: the target scores every root-to-node path in one forward pass
// under a tree attention mask.  Survey explainer (paper-2401-07851), formal
// definition, verification phase: the target distribution at a draft position
// conditions on the context and the drafts before it.
//
// Design (gfx950):
//  * The G = Hq/Hkv query heads sharing a KV head and the N tree nodes are
//    packed into R = G*N query rows per (sequence, KV head).  A wave owns 32
//    or 64 rows (one or two 32-row MFMA blocks); a workgroup's four waves form
//    KG key groups of 4/KG row-waves (up to 64 rows on grids larger than the
//    device: two key groups of two 32-row waves, small enough in LDS for two
//    workgroups per CU), and the large-row kernel's eight waves own 256 rows,
//    so one K/V byte read from HBM serves up to 256 rows (grouped-query heads
//    share it).
//  * K and V tiles go from HBM straight to LDS (global_load_lds, 16 bytes per
//    lane) into an S-stage ring per key group, S - 1 tiles ahead of the
//    arithmetic.  Rows of 256 bytes are stored with their 16-byte chunks
//    XOR-swizzled by the low key bits (K: chunk ^ (key & 15); V: chunk ^
//    4 (key & 3)), so that the K fragment reads (16 lanes per cycle) and the
//    transposed V reads (32 lanes per cycle) each cover all 64 LDS banks.
//  * Scores are computed transposed, S^T = K . Q^T, with
//    v_mfma_f32_32x32x16_bf16 (keys on the M side): a lane holds the scores of
//    a single query row, so max, sum and the output rescale are lane-local
//    (plus one cross-half exchange).  The K fragment read from LDS feeds both
//    row blocks.
//  * P.V runs as O^T = V^T . P^T with v_mfma_f32_32x32x16_f16: P is rounded to
//    fp16 (bf16 P would cost ~1.5e-3 relative error).  V^T fragments come from
//    the bf16 V tile with ds_read_b64_tr_b16 (each lane receives four keys at
//    one head-dim position) and are converted to fp16 in registers; the
//    score accumulator already holds P^T in B-operand order once the keys of
//    each 16-key step are permuted, and the transposed reads use the same
//    permutation.
//  * Softmax in the exp2 domain with the scale folded into one FMA per score;
//    the running max is raised lazily (only when a score exceeds it by more
//    than 2^8), so most tiles skip the accumulator rescale; masks are applied
//    only on tree tiles and the ragged last tile.  The exponentials of one row
//    block are scheduled between the MFMAs of the other.
//  * Tree keys are extra tiles processed by the last KV split; the mask bit for
//    (row, key j) is bit j % 64 of the row's ancestor word j / 64 (the first
//    word is held in a register, later ones are loaded by the tree tiles that
//    need them).
//  * Ragged batches: a sequence's own node count bounds its query rows, its own
//    cache length bounds its key tiles; splits past a short cache publish an
//    empty partial.
//  * Long caches are split across workgroups; each writes its partial
//    (max, sum, unnormalised O) with device-scope stores, and the last one to
//    finish (device-scope counter) merges them and writes the output.
//  * Workgroup ids are remapped so that workgroups sharing a KV range run on
//    the same XCD (same L2).
#include <float.h>

#include "tv_device.h"
#include "tv_internal.h"

namespace tv {
namespace {

constexpr int HD = TV_HEAD_DIM;
constexpr int kRowBytes = HD * 2;            // one key row of K or V (bf16)
constexpr int kTargetWorkgroups = 256;   // one per CU (a workgroup fills a CU)
constexpr int kBalance = 1;              // splits beyond kBalance * sqrt(L / R) are not worth their merge
constexpr double kNonTemporalKvBytes = 512.0 * 1024 * 1024;  // twice the Infinity Cache
constexpr float kLazyThresh = 8.f;           // log2 units the running max may lag the true max

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

struct AttnArgs {
    const uint16_t* Q;
    const uint16_t* Kc;
    const uint16_t* Vc;
    const uint16_t* Kt;
    const uint16_t* Vt;
    const uint64_t* anc;        // [B][N][W]
    const int32_t* seq_nodes;   // [B] or null
    const int32_t* seq_len;     // [B] or null
    float* out;
    float* part_o;     // [groups][nsplit][rows per tile][HD]
    float* part_ml;    // [groups][nsplit][rows per tile][2]
    uint32_t* counter; // [groups], zero between calls
    int N, Hq, Hkv, G, L, R, W;
    int row_tiles, nsplit, tiles_per_split, cache_tiles, tree_tiles, nblocks;
    float scale_log2;
};

struct Plan {
    int variant;  // key groups x tile keys x stages x row blocks per wave x waves:
                  // 4x32x2x1x4, 4x32x2x2x4, 2x64x2x2x4, 1x64x4x1x8, 2x32x2x1x4
    int kg, kt, nw, rows, R, row_tiles, nsplit, tiles_per_split, cache_tiles, tree_tiles;
};

// Row tiles, tiles and splits of a plan whose kernel shape (kg, kt, nw, rows)
// is set.
void plan_splits(Plan& p, int B, int N, int Hkv, int L) {
    p.row_tiles = (p.R + p.rows - 1) / p.rows;
    p.cache_tiles = (L + p.kt - 1) / p.kt;
    p.tree_tiles = (N + p.kt - 1) / p.kt;
    const long base = (long)B * Hkv * p.row_tiles;
    int nsplit = 1;
    p.tiles_per_split = 0;
    if (p.cache_tiles > 0) {
        // enough workgroups for one per CU, but the last workgroup of a group
        // merges nsplit partials of R rows while each split streams L / nsplit
        // keys: beyond about sqrt(L / R) splits the merge costs more than it saves
        const long want = (kTargetWorkgroups + base - 1) / base;
        int balance = 1;
        while ((long)(balance + 1) * (balance + 1) * p.R <= (long)kBalance * kBalance * L) ++balance;
        const int max_split = (p.cache_tiles + p.kg - 1) / p.kg;  // at least one tile per key group
        nsplit = (int)(want < max_split ? want : max_split);
        if (nsplit > balance) nsplit = balance;
        if (nsplit < 1) nsplit = 1;
        if (nsplit > 64) nsplit = 64;  // the merging workgroup keeps one weight per (row, split) in LDS
        int tps = (p.cache_tiles + nsplit - 1) / nsplit;
        tps = (tps + p.kg - 1) / p.kg * p.kg;
        p.tiles_per_split = tps;
        nsplit = (p.cache_tiles + tps - 1) / tps;
    }
    p.nsplit = nsplit;
}

Plan make_plan(int B, int N, int Hq, int Hkv, int L) {
    Plan p;
    const int G = Hq / Hkv;
    p.R = G * N;
    int rbw = 2;
    p.nw = 4;
    if (p.R <= 32) {
        p.variant = 0; p.kg = 4; p.kt = 32; rbw = 1;
    } else if (p.R <= 64) {
        p.variant = 1; p.kg = 4; p.kt = 32;
    } else if (p.R <= 128) {
        p.variant = 2; p.kg = 2; p.kt = 64;
    } else {
        p.variant = 3; p.kg = 1; p.kt = 64; rbw = 1; p.nw = 8;
    }
    p.rows = (p.nw / p.kg) * 32 * rbw;
    plan_splits(p, B, N, Hkv, L);
    // Up to 64 rows and more workgroups than CUs: two key groups of two
    // 32-row waves (67 KB of LDS instead of 128) let two workgroups share a CU,
    // so the grid runs in about half as many rounds and each CU keeps twice
    // the copies in flight (B = 16, 40 heads, 60 nodes, L = 2048: 640
    // workgroups, 141-142 us against 154-155 us).
    if (p.variant == 1 && (long)B * Hkv * p.row_tiles * p.nsplit > kTargetWorkgroups) {
        p.variant = 4; p.kg = 2; p.kt = 32;
        p.rows = (p.nw / p.kg) * 32;
        plan_splits(p, B, N, Hkv, L);
    }
    return p;
}

struct WsLayout {
    size_t counter_off, part_o_off, part_ml_off, total;
};

WsLayout workspace_layout(int B, int Hkv, const Plan& p) {
    WsLayout w{0, 0, 0, 0};
    if (p.nsplit <= 1) return w;
    const size_t groups = (size_t)B * Hkv * p.row_tiles;
    const size_t rows = groups * p.nsplit * p.rows;
    w.counter_off = 0;
    w.part_o_off = round_up(groups * sizeof(uint32_t), 256);
    w.part_ml_off = w.part_o_off + round_up(rows * HD * sizeof(float), 256);
    w.total = w.part_ml_off + round_up(rows * 2 * sizeof(float), 256);
    return w;
}

// Nodes and committed cache length of sequence b (ragged batches), clamped
// into 0..N and 0..L.
__device__ __forceinline__ int seq_nodes_of(const AttnArgs& a, int b) {
    return a.seq_nodes ? min(max(a.seq_nodes[b], 0), a.N) : a.N;
}
__device__ __forceinline__ int seq_len_of(const AttnArgs& a, int b) {
    return a.seq_len ? min(max(a.seq_len[b], 0), a.L) : a.L;
}
// Ancestor word w of node `node` of sequence b.
__device__ __forceinline__ uint64_t anc_word(const AttnArgs& a, int b, int node, int w) {
    return a.anc[((size_t)b * a.N + node) * a.W + w];
}

__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
    // Dispatch places consecutive workgroup ids on consecutive XCDs (8 of
    // them); give each XCD a contiguous range of logical ids instead.
    const int xcd = bid & 7, idx = bid >> 3;
    const int per = nblocks >> 3, rem = nblocks & 7;
    return xcd < rem ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
}

// Split partials cross workgroups (and XCDs, whose L2s are not coherent with
// each other) through 16-byte buffer accesses with the cache policy of an
// agent-scope atomic access (sc1): one instruction per float4 where two 8-byte
// atomics would be needed.  A resource covers one range of under 4 GiB.
constexpr int kDevCoherent = 1 << 4;  // cache-policy operand: sc1
__device__ __forceinline__ __amdgpu_buffer_rsrc_t dev_rsrc(const float* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ void st_dev_b128(__amdgpu_buffer_rsrc_t r, uint32_t off, f32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, kDevCoherent);
}
__device__ __forceinline__ f32x4 ld_dev_b128(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kDevCoherent));
}
__device__ __forceinline__ void st_dev_f(float* p, float v) {
    __hip_atomic_store(reinterpret_cast<uint32_t*>(p), __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev_f(const float* p) {
    return __uint_as_float(__hip_atomic_load(reinterpret_cast<uint32_t*>(const_cast<float*>(p)), __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT));
}

// s_waitcnt vmcnt(n) (gfx9 encoding: vmcnt split over bits 3:0 and 15:14;
// expcnt and lgkmcnt left at their maxima, i.e. not waited for).
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(n >= 0 && n < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// 16-byte HBM -> LDS copy per lane (global_load_lds_dwordx4): lane i writes
// lds_addr + 16 i.  Issued as inline assembly so that the compiler does not
// treat every later LDS read as dependent on it (it would wait for the whole
// ring); completion is tracked explicitly with wait_vmcnt.  With NT the load
// is marked non-temporal: KV caches that cannot stay in the Infinity Cache
// stream faster that way.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // m0 is reserved but only this copy writes it
template <bool NT>
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds_addr) {
    const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_addr);
    if constexpr (NT)
        asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off nt" : : "s"(m0v), "v"(gptr) : "memory", "m0");
    else
        asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" : : "s"(m0v), "v"(gptr) : "memory", "m0");
}
// Same copy with a uniform 64-bit base and a 32-bit per-lane byte offset.
template <bool NT>
__device__ __forceinline__ void dma16s(const void* sbase, uint32_t voff, uint32_t lds_addr) {
    const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_addr);
    if constexpr (NT)
        asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 nt"
                     :
                     : "s"(m0v), "v"(voff), "s"(sbase)
                     : "memory", "m0");
    else
        asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
                     :
                     : "s"(m0v), "v"(voff), "s"(sbase)
                     : "memory", "m0");
}
#pragma clang diagnostic pop

// LDS accesses by byte address (32-bit, address space 3).
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
__device__ __forceinline__ u32x4 lds_ld128(uint32_t addr) { return *(const lds_u32x4*)(uintptr_t)addr; }
__device__ __forceinline__ u32x2 lds_tr16(uint32_t addr) {
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(uintptr_t)addr));
}


// Two floats to fp16 rounded toward zero (v_cvt_pkrtz_f16_f32).  V values
// come from bf16, whose 8-bit significands fp16 holds exactly over its normal
// range, so the rounding mode matters only there: beyond +-65504 rounding
// toward zero gives +-65504 (a saturating conversion, where rounding to
// nearest would give infinities that turn whole output rows into NaN), and
// below the normal range it truncates instead of rounding (< 6e-8).
__device__ __forceinline__ uint32_t f32x2_to_f16x2_sat(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(a, b));
}

// bf16 bits -> fp16, two values per dword, saturated.
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w) {
    return f32x2_to_f16x2_sat(__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u));
}

// Max over the two halves of the wave (lanes l and l ^ 32 hold one query row).
__device__ __forceinline__ float halves_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// The merge itself.  Per row, w_s = 2^(m_s - M) / sum_s 2^(m_s - M) l_s and
// out = sum_s w_s O_s.  Each thread owns U output float4s at a time (stride
// NT) and loads SC splits of each per round, U * SC loads in flight.  With
// HOIST the first round's loads are issued before the (m, l) loads, so that
// both arrive in one round trip.  `lds` holds at least 2 * nrows * nsplit
// floats.
template <int NT, int ROWS, int U, int SC, bool HOIST>
__device__ void merge_partials(const AttnArgs& a, char* lds, int grp, int row0, int nrows, int b, int g) {
    const int ns = a.nsplit;
    float* wts = reinterpret_cast<float*>(lds);  // [nrows][ns] (m_s, then the weight)
    float* lsv = wts + nrows * ns;               // [nrows][ns] l_s
    const size_t pbase = (size_t)grp * ns * ROWS;
    const int nout = nrows * (HD / 4);
    f32x4 v[U][SC];
    const __amdgpu_buffer_rsrc_t po = dev_rsrc(a.part_o + pbase * HD, (uint32_t)(ns * ROWS * HD * 4));
    auto load = [&](int e0, int s0) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int e = min(e0 + u * NT, nout - 1);
            const uint32_t off = (uint32_t)(((e / (HD / 4)) * HD + 4 * (e % (HD / 4))) * 4);
#pragma unroll
            for (int k = 0; k < SC; ++k) v[u][k] = ld_dev_b128(po, off + (uint32_t)(min(s0 + k, ns - 1) * ROWS * HD * 4));
        }
    };
    int e0 = threadIdx.x, s0 = 0;
    if (HOIST) load(e0, s0);

    for (int f0 = 0; f0 < nrows * ns; f0 += 8 * NT) {
        float mv[8], lv[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int e = min(f0 + k * NT + (int)threadIdx.x, nrows * ns - 1);
            const float* ml = a.part_ml + (pbase + (size_t)(e % ns) * ROWS + e / ns) * 2;
            mv[k] = ld_dev_f(ml);
            lv[k] = ld_dev_f(ml + 1);
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int e = f0 + k * NT + (int)threadIdx.x;
            if (e < nrows * ns) {
                wts[e] = mv[k];
                lsv[e] = lv[k];
            }
        }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < nrows; i += NT) {
        float M = -INFINITY;
        for (int s = 0; s < ns; ++s) M = fmaxf(M, wts[i * ns + s]);
        float Lsum = 0.f;
        for (int s = 0; s < ns; ++s) {
            const float wv = (M == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(wts[i * ns + s] - M);
            wts[i * ns + s] = wv;
            Lsum += wv * lsv[i * ns + s];
        }
        const float inv = 1.f / Lsum;
        for (int s = 0; s < ns; ++s) wts[i * ns + s] *= inv;
    }
    __syncthreads();

    f32x4 acc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (!HOIST && e0 < nout) load(e0, s0);
    while (e0 < nout) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = min(e0 + u * NT, nout - 1) / (HD / 4);
#pragma unroll
            for (int k = 0; k < SC; ++k)
                if (s0 + k < ns) acc[u] += wts[i * ns + s0 + k] * v[u][k];
        }
        s0 += SC;
        if (s0 >= ns) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int e = e0 + u * NT;
                if (e < nout) {
                    const int i = e / (HD / 4), d4 = e % (HD / 4);
                    const int rr = row0 + i;
                    const int nd = rr / a.G, hd = g * a.G + rr % a.G;
                    *reinterpret_cast<f32x4*>(a.out + ((size_t)(b * a.N + nd) * a.Hq + hd) * HD + 4 * d4) = acc[u];
                }
                acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
            s0 = 0;
            e0 += U * NT;
        }
        if (e0 < nout) load(e0, s0);
    }
}

// Split-KV merge: every workgroup of a row group has published its partial
// (max, sum, unnormalised O); the last one to arrive (device-scope counter)
// combines them, w_s = 2^(m_s - M) / sum_s 2^(m_s - M) l_s, writes the output
// and resets the counter for the next call.  `lds` holds at least
// 2 * nrows * nsplit floats; `s_flag` is a workgroup-shared int outside them.
template <int NT, int ROWS>
__device__ void merge_splits(const AttnArgs& a, char* lds, int* s_flag, int grp, int row0, int nrows, int b,
                             int g) {
    // Every wave waits until its partial stores have completed, the barrier
    // orders them before thread 0's arrival, and that arrival is a release at
    // agent scope (it writes back what this XCD's L2 holds for other XCDs); the
    // last workgroup's arrival is also an acquire, and its barrier orders every
    // wave's loads after it (the loads are device-coherent besides).  One fence
    // per workgroup: a release fence in every wave cost 2-3 us per call on the
    // single-sequence workloads.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t prev =
            __hip_atomic_fetch_add(&a.counter[grp], 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        *s_flag = prev == (uint32_t)a.nsplit - 1;
    }
    __syncthreads();
    if (!*s_flag) return;
    if (nrows <= 0) {  // a row tile of padding nodes only (ragged batch): nothing to merge
        if (threadIdx.x == 0) __hip_atomic_store(&a.counter[grp], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
    }

    // last workgroup of the group.  Up to four splits: 32 loads in flight per
    // thread (16 in the 512-thread kernel, whose register budget is half as
    // large), the first round issued early.  More splits: chunks of twelve
    // splits for four (two) outputs, 48 (24) loads issued once the weights are
    // known (eleven splits of 24 rows: one round, no issue-early gain).
    constexpr int F = NT >= 512 ? 16 : 32;
    if (a.nsplit <= 4)
        merge_partials<NT, ROWS, F / 4, 4, true>(a, lds, grp, row0, nrows, b, g);
    else
        merge_partials<NT, ROWS, F / 8, 12, false>(a, lds, grp, row0, nrows, b, g);
    if (threadIdx.x == 0)
        __hip_atomic_store(&a.counter[grp], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // ready for the next call
}

template <int KG, int KT, int S, int RBW, int NW, bool NT>
__global__ __launch_bounds__(64 * NW) void tree_attention_kernel(const AttnArgs a) {
    constexpr int kThreads = 64 * NW;              // NW waves: one or two per SIMD
    constexpr int RW = NW / KG;                    // row-waves per key group
    constexpr int WROWS = RBW * 32;                // rows per wave
    constexpr int ROWS = RW * WROWS;               // rows per workgroup
    constexpr bool CONV_LDS = RW > 1;              // V converted to fp16 once per tile in LDS
    constexpr int KB = KT / 32;                    // 32-key MFMA blocks per tile
    constexpr int TILE = KT * kRowBytes;           // bytes of a K (or V) tile
    constexpr int STAGE = 2 * TILE;                // K then V
    constexpr int RING = S * STAGE;                // one key group's ring
    constexpr int DMA = KT * kRowBytes / (16 * kWave) / RW;  // 16-byte DMA instructions per wave per operand
    constexpr int O_STRIDE = HD + 4;               // floats per row of a key-group merge slot (conflict-free)
    constexpr int DPW = HD / KG;                   // head dims each key group merges
    static_assert(DMA >= 1, "tile too small for the key group");
    constexpr int MERGE = KG > 1 ? KG * ROWS * (O_STRIDE + 2) * 4 : 0;  // key-group merge slots
    constexpr int LDS_BYTES = KG * RING > MERGE ? KG * RING : MERGE;
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
    __shared__ __attribute__((aligned(1024))) char lds[LDS_BYTES];  // rows 256-byte aligned
    __shared__ int s_last;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int kg = wave / RW;
    const int rw = wave % RW;
    const int n = lane & 31;   // MFMA column: query row within a block / key within a 32-key block
    const int hf = lane >> 5;  // which half of the k-slots this lane carries

    const int logical = xcd_remap(blockIdx.x, a.nblocks);
    const int rt = logical % a.row_tiles;
    const int tmp = logical / a.row_tiles;
    const int split = tmp % a.nsplit;
    const int bg = tmp / a.nsplit;
    const int b = bg / a.Hkv;
    const int g = bg % a.Hkv;
    const float c = a.scale_log2;
    const int Rb = a.G * seq_nodes_of(a, b);  // this sequence's query rows
    const int lb = seq_len_of(a, b);          // and its committed cache entries

    // ---- the query rows this lane carries as B-operand columns ----
    int row[RBW];
    bool row_ok[RBW];
    bf16x8 qf[RBW][8];
    uint64_t anc_row[RBW];  // ancestor word 0
#pragma unroll
    for (int j = 0; j < RBW; ++j) {
        row[j] = rt * ROWS + rw * WROWS + 32 * j + n;
        row_ok[j] = row[j] < Rb;
        const int node = row_ok[j] ? row[j] / a.G : 0;
        const int head = g * a.G + (row_ok[j] ? row[j] % a.G : 0);
        const uint16_t* qrow = a.Q + ((size_t)(b * a.N + node) * a.Hq + head) * HD;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const u32x4 v = *reinterpret_cast<const u32x4*>(qrow + 16 * s + 8 * hf);
            qf[j][s] = __builtin_bit_cast(bf16x8, row_ok[j] ? v : u32x4{0, 0, 0, 0});
        }
        anc_row[j] = row_ok[j] ? anc_word(a, b, node, 0) : 0ull;
    }

    // ---- tiles of this workgroup: cache tiles of the split, then tree tiles ----
    const int t_begin = split * a.tiles_per_split;
    int n_cache = (lb + KT - 1) / KT - t_begin;
    if (n_cache > a.tiles_per_split) n_cache = a.tiles_per_split;
    if (n_cache < 0) n_cache = 0;
    const int n_tree = (split == a.nsplit - 1) ? a.tree_tiles : 0;
    const int n_tiles = n_cache + n_tree;
    const int iters = (n_tiles + KG - 1) / KG;
    char* ring = lds + kg * RING;
    const uint32_t ring_addr = (uint32_t)(uintptr_t)(lds_void*)ring;

    // Issue this wave's share of the DMA of tile t (this key group's t-th
    // tile, index k_idx = t * KG + kg) into stage st.
    auto issue_tile = [&](int t, int st) {
        const int k_idx = t * KG + kg;
        if (k_idx >= n_tiles) return;  // uniform: nothing to load
        const bool is_tree = k_idx >= n_cache;
        int key0, nk;
        const uint16_t *ks, *vs;
        size_t stride;
        if (!is_tree) {
            key0 = (t_begin + k_idx) * KT;
            nk = min(KT, lb - key0);
            const size_t base = ((size_t)bg * a.L + key0) * HD;
            ks = a.Kc + base;
            vs = a.Vc + base;
            stride = HD;
        } else {
            key0 = (k_idx - n_cache) * KT;
            nk = min(KT, a.N - key0);
            const size_t base = ((size_t)(b * a.N + key0) * a.Hkv + g) * HD;
            ks = a.Kt + base;
            vs = a.Vt + base;
            stride = (size_t)a.Hkv * HD;
        }
        const uint32_t kdst_addr = ring_addr + st * STAGE;
#pragma unroll
        for (int i = 0; i < DMA; ++i) {
            const int inst = rw * DMA + i;          // 1 KB block of the tile
            const int p = inst * kWave + lane;      // 16-byte chunk written by this lane
            const int key = p >> 4, pc = p & 15;
            const size_t row_off = (size_t)min(key, nk - 1) * stride;  // ragged keys repeat a valid row
            // logical chunks stored at physical chunk pc of K and of V
            dma16<NT>(ks + row_off + (pc ^ (key & 15)) * 8, kdst_addr + inst * 1024);
            dma16<NT>(vs + row_off + (pc ^ (4 * (key & 3))) * 8, kdst_addr + TILE + inst * 1024);
        }
    };

    f32x16 o_acc[RBW][4];
#pragma unroll
    for (int j = 0; j < RBW; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) o_acc[j][i] = f32x16{};
    float m_used[RBW], l_run[RBW];  // m_used in raw score units
#pragma unroll
    for (int j = 0; j < RBW; ++j) {
        m_used[j] = -INFINITY;
        l_run[j] = 0.f;
    }

    // prologue: the first S - 1 tiles of every key group
#pragma unroll
    for (int t = 0; t < S - 1; ++t) issue_tile(t, t);

    // tiles of this key group
    const int ntk = kg < n_tiles ? (n_tiles - kg + KG - 1) / KG : 0;
    for (int it = 0; it < iters; ++it) {
        // tile `it` of this key group has landed: wait until at most the DMA of
        // the later tiles already issued (up to S - 2 of them) is outstanding
        const int later = min(S - 2, ntk - 1 - it);
        if (later <= 0) {
            wait_vmcnt<0>();
        } else if constexpr (S > 2) {
            if (later == 1) wait_vmcnt<2 * DMA>();
            else wait_vmcnt<(S - 2) * 2 * DMA>();
            static_assert(S <= 4, "wait counts cover rings of up to four stages");
        }
        __syncthreads();  // every wave's part is in LDS; the stage refilled below is free
        issue_tile(it + S - 1, (it + S - 1) % S);
        const int k_idx = it * KG + kg;
        const char* kt = ring + (it % S) * STAGE;
        const char* vt = kt + TILE;
        // V of this tile to fp16 in place, shared by the key group's row-waves
        // (a single row-wave converts its fragments in registers instead)
        if (CONV_LDS && k_idx < n_tiles) {
            constexpr int CH = TILE / 16 / (RW * kWave);  // 16-byte chunks per lane
#pragma unroll
            for (int i = 0; i < CH; ++i) {
                u32x4* ch = reinterpret_cast<u32x4*>(const_cast<char*>(vt)) + (rw * CH + i) * kWave + lane;
                const u32x4 x = *ch;
                *ch = u32x4{bf16x2_to_f16x2(x[0]), bf16x2_to_f16x2(x[1]), bf16x2_to_f16x2(x[2]),
                            bf16x2_to_f16x2(x[3])};
            }
        }
        if constexpr (CONV_LDS) __syncthreads();  // the converted V is visible to every row-wave
        if (k_idx >= n_tiles) continue;  // uniform per wave
        const bool is_tree = k_idx >= n_cache;
        const int key0 = is_tree ? (k_idx - n_cache) * KT : (t_begin + k_idx) * KT;
        const int nk = is_tree ? min(KT, a.N - key0) : min(KT, lb - key0);
        const bool masked = is_tree || nk < KT;

        // LDS byte addresses.  Rows are 256-byte aligned, so a chunk index can
        // be XORed into bits 4..7 of a row address.
        //  K fragment (kb, s): key 32 kb + n, logical chunk 2s + hf, stored at
        //  (2s + hf) ^ (n & 15): address = (k_base ^ (s << 5)) + 8192 kb.
        const uint32_t kt_addr = (uint32_t)(uintptr_t)(lds_void*)kt;
        const uint32_t k_base = (kt_addr + n * kRowBytes + hf * 16) ^ ((n & 15) << 4);
        //  V^T fragment of 16-key step t, head-dim block blk: lane (n, hf) gets
        //  V[keys 16t + 4hf + 0..3 and 16t + 8 + 4hf + 0..3][32 blk + n].  For a
        //  transposed read, the 16 lanes of group gq supply rows r = 0..3 (lanes
        //  4r..4r+3, four head-dim values each) and receive one column each:
        //  lane supplies key 16t + kr (+8), head dims d0 .. d0+3 with
        //  kr = 4 (gq >> 1) + (w16 >> 2), d0 = 32 blk + 16 (gq & 1) + 4 (w16 & 3).
        //  Its chunk d0 / 8 = 4 blk + c0 is stored at 4 (blk ^ (kr & 3)) + c0
        //  (the same for key + 8), so with v_base = row kr | (c0 << 4) |
        //  ((kr & 3) << 6) | byte (d0 & 7) * 2: lo address = (v_base ^ (blk << 6))
        //  + 4096 t, hi = lo + 2048 (eight rows further).
        const int gq = lane >> 4, w16 = lane & 15;
        const int kr = 4 * (gq >> 1) + (w16 >> 2);
        const int c0 = 2 * (gq & 1) + ((w16 & 3) >> 1);
        const uint32_t v_base =
            ((kt_addr + TILE + kr * kRowBytes) | (c0 << 4) | ((kr & 3) << 6)) + 8 * (w16 & 1);
        uint32_t v_blk[4];
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) v_blk[blk] = v_base ^ (blk << 6);

        // the tile is processed in blocks of 32 keys (online softmax per block)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            // ---- S^T[key][row] for this block and the wave's row blocks ----
            f32x16 s_acc[RBW];
#pragma unroll
            for (int j = 0; j < RBW; ++j) s_acc[j] = f32x16{};
            bf16x8 kf[8];  // the block's K fragments, all reads in flight before the MFMAs
#pragma unroll
            for (int s = 0; s < 8; ++s) kf[s] = __builtin_bit_cast(bf16x8, lds_ld128((k_base ^ (s << 5)) + 8192 * kb));
#pragma unroll
            for (int s = 0; s < 8; ++s)
#pragma unroll
                for (int j = 0; j < RBW; ++j)
                    s_acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s], qf[j][s], s_acc[j], 0, 0, 0);
            // element e is key 32 kb + 8 (e/4) + 4 hf + (e%4) of the tile
            if (masked) {
                const int kbase = 32 * kb;
                const uint32_t ragged = nk - kbase >= 32 ? 0xffffffffu
                                                         : (nk - kbase <= 0 ? 0u : (1u << (nk - kbase)) - 1u);
#pragma unroll
                for (int j = 0; j < RBW; ++j) {
                    uint32_t vis = ragged;
                    if (is_tree) {
                        const int word = (key0 + kbase) >> 6;  // uniform
                        const uint64_t aw = word == 0 ? anc_row[j]
                                                      : (row_ok[j] ? anc_word(a, b, row[j] / a.G, word) : 0ull);
                        vis &= (uint32_t)(aw >> ((key0 + kbase) & 63));
                    }
                    vis >>= 4 * hf;
#pragma unroll
                    for (int e = 0; e < 16; ++e)
                        if (!((vis >> (8 * (e >> 2) + (e & 3))) & 1u)) s_acc[j][e] = -INFINITY;
                }
            }
            // ---- running max: raised only when a score runs more than 2^8 above it ----
            float mc[RBW];
#pragma unroll
            for (int j = 0; j < RBW; ++j) {
                float tmax = -INFINITY;
#pragma unroll
                for (int e = 0; e < 16; ++e) tmax = fmaxf(tmax, s_acc[j][e]);
                tmax = halves_max(tmax);
                const bool raise = tmax > m_used[j] + kLazyThresh / c || m_used[j] == -INFINITY;
                if (__ballot(raise)) {
                    const float m_new = raise ? fmaxf(m_used[j], tmax) : m_used[j];
                    const float alpha =
                        (m_used[j] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((m_used[j] - m_new) * c);
                    if (raise) {
                        l_run[j] *= alpha;
#pragma unroll
                        for (int i = 0; i < 4; ++i) o_acc[j][i] *= alpha;
                    }
                    m_used[j] = m_new;
                }
                mc[j] = (m_used[j] == -INFINITY) ? 0.f : m_used[j] * c;
            }
            // ---- per 16-key step: P = exp2(s c - m c) as fp16 B operands, V^T
            // fragments, O^T += V^T P^T.  Step h holds accumulator elements
            // 8h .. 8h + 7 (keys in the permuted order above).
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                u32x4 pf[RBW];
#pragma unroll
                for (int j = 0; j < RBW; ++j) {
                    uint32_t w[4];
                    float ls = 0.f;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const float p0 = __builtin_amdgcn_exp2f(fmaf(s_acc[j][8 * h + 2 * q], c, -mc[j]));
                        const float p1 = __builtin_amdgcn_exp2f(fmaf(s_acc[j][8 * h + 2 * q + 1], c, -mc[j]));
                        ls += p0 + p1;
                        w[q] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)p0) |
                               ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)p1) << 16);
                    }
                    l_run[j] += ls;
                    pf[j] = u32x4{w[0], w[1], w[2], w[3]};
                }
                const int t = 2 * kb + h;
                u32x2 vl[4], vh[4];  // the step's V^T fragments, all reads in flight before the MFMAs
#pragma unroll
                for (int blk = 0; blk < 4; ++blk) {
                    vl[blk] = lds_tr16(v_blk[blk] + 4096 * t);
                    vh[blk] = lds_tr16(v_blk[blk] + 4096 * t + 2048);
                }
#pragma unroll
                for (int blk = 0; blk < 4; ++blk) {
                    const u32x2 l2 = vl[blk], h2 = vh[blk];
                    f16x8 vf;
                    if constexpr (CONV_LDS) {
                        vf = __builtin_bit_cast(f16x8, u32x4{l2.x, l2.y, h2.x, h2.y});
                    } else {
                        vf = __builtin_bit_cast(f16x8, u32x4{bf16x2_to_f16x2(l2.x), bf16x2_to_f16x2(l2.y),
                                                             bf16x2_to_f16x2(h2.x), bf16x2_to_f16x2(h2.y)});
                    }
#pragma unroll
                    for (int j = 0; j < RBW; ++j)
                        o_acc[j][blk] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, __builtin_bit_cast(f16x8, pf[j]),
                                                                               o_acc[j][blk], 0, 0, 0);
                }
            }
        }
    }

    float l_tot[RBW], m_log[RBW];
#pragma unroll
    for (int j = 0; j < RBW; ++j) {
        l_tot[j] = halves_sum(l_run[j]);
        m_log[j] = (m_used[j] == -INFINITY) ? -INFINITY : m_used[j] * c;  // log2 units from here on
    }

    // ---- results per row: a lane holds head dims [d_lo, d_lo + DOUT) of row
    // r_out (workgroup-relative), unnormalised, with its (m, l) ----
    //  KG == 1: the MFMA layout itself (DOUT = 4-float pieces scattered); the
    //  merged path below gathers rows instead.
    const int grp = bg * a.row_tiles + rt;
    const int row0 = rt * ROWS;
    const int nrows = min(ROWS, Rb - row0);

    if constexpr (KG == 1) {
        if (a.nsplit == 1) {
#pragma unroll
            for (int j = 0; j < RBW; ++j) {
                if (!row_ok[j]) continue;
                const int node = row[j] / a.G, head = g * a.G + row[j] % a.G;
                const float inv = 1.f / l_tot[j];
                float* dst = a.out + ((size_t)(b * a.N + node) * a.Hq + head) * HD;
#pragma unroll
                for (int blk = 0; blk < 4; ++blk)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        *reinterpret_cast<f32x4*>(dst + 32 * blk + 8 * q + 4 * hf) =
                            f32x4{o_acc[j][blk][4 * q] * inv, o_acc[j][blk][4 * q + 1] * inv,
                                  o_acc[j][blk][4 * q + 2] * inv, o_acc[j][blk][4 * q + 3] * inv};
            }
            return;
        }
        const __amdgpu_buffer_rsrc_t pw =
            dev_rsrc(a.part_o + ((size_t)grp * a.nsplit + split) * ROWS * HD, (uint32_t)(ROWS * HD * 4));
#pragma unroll
        for (int j = 0; j < RBW; ++j) {
            if (!row_ok[j]) continue;
            const size_t prow = ((size_t)grp * a.nsplit + split) * ROWS + (row[j] - row0);
            const uint32_t ob = (uint32_t)((row[j] - row0) * HD * 4);
#pragma unroll
            for (int blk = 0; blk < 4; ++blk)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    st_dev_b128(pw, ob + (uint32_t)((32 * blk + 8 * q + 4 * hf) * 4),
                                f32x4{o_acc[j][blk][4 * q], o_acc[j][blk][4 * q + 1], o_acc[j][blk][4 * q + 2],
                                      o_acc[j][blk][4 * q + 3]});
            if (hf == 0) {
                st_dev_f(a.part_ml + prow * 2, m_log[j]);
                st_dev_f(a.part_ml + prow * 2 + 1, l_tot[j]);
            }
        }
    } else {
        // ---- merge the key groups through LDS, every wave taking DPW head dims ----
        wait_vmcnt<0>();
        __syncthreads();  // the ring is free
        float* slots = reinterpret_cast<float*>(lds);                      // [KG][ROWS][O_STRIDE]
        float* mls = slots + (size_t)KG * ROWS * O_STRIDE;                  // [KG][ROWS][2]
#pragma unroll
        for (int j = 0; j < RBW; ++j) {
            const int rr = rw * WROWS + 32 * j + n;  // workgroup-relative row
            float* so = slots + ((size_t)kg * ROWS + rr) * O_STRIDE;
#pragma unroll
            for (int blk = 0; blk < 4; ++blk)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    *reinterpret_cast<f32x4*>(so + 32 * blk + 8 * q + 4 * hf) =
                        f32x4{o_acc[j][blk][4 * q], o_acc[j][blk][4 * q + 1], o_acc[j][blk][4 * q + 2],
                              o_acc[j][blk][4 * q + 3]};
            if (hf == 0) {
                mls[((size_t)kg * ROWS + rr) * 2] = m_log[j];
                mls[((size_t)kg * ROWS + rr) * 2 + 1] = l_tot[j];
            }
        }
        __syncthreads();
        // wave w merges head dims [DPW * (w % KG), + DPW) of rows (w / KG) + 4/KG * i:
        // lanes hold rows, each lane DPW contiguous head dims
        const int d_lo = DPW * (wave % KG);
        for (int rr = wave / KG * kWave + lane; rr < ROWS; rr += RW * kWave) {
            if (rr >= nrows) break;
            float M = -INFINITY;
#pragma unroll
            for (int k = 0; k < KG; ++k) M = fmaxf(M, mls[((size_t)k * ROWS + rr) * 2]);
            float wk[KG], Lsum = 0.f;
#pragma unroll
            for (int k = 0; k < KG; ++k) {
                const float mk = mls[((size_t)k * ROWS + rr) * 2];
                wk[k] = (M == -INFINITY || mk == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mk - M);
                Lsum += wk[k] * mls[((size_t)k * ROWS + rr) * 2 + 1];
            }
            const int grow = row0 + rr;
            const int node = grow / a.G, head = g * a.G + grow % a.G;
            const float inv = 1.f / Lsum;
            const size_t prow = ((size_t)grp * a.nsplit + split) * ROWS + rr;
#pragma unroll
            for (int d4 = 0; d4 < DPW / 4; ++d4) {
                f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int k = 0; k < KG; ++k)
                    acc += wk[k] * *reinterpret_cast<const f32x4*>(slots + ((size_t)k * ROWS + rr) * O_STRIDE + d_lo +
                                                                   4 * d4);
                if (a.nsplit == 1)
                    *reinterpret_cast<f32x4*>(a.out + ((size_t)(b * a.N + node) * a.Hq + head) * HD + d_lo + 4 * d4) =
                        acc * inv;
                else
                    st_dev_b128(dev_rsrc(a.part_o + ((size_t)grp * a.nsplit + split) * ROWS * HD,
                                         (uint32_t)(ROWS * HD * 4)),
                                (uint32_t)((rr * HD + d_lo + 4 * d4) * 4), acc);
            }
            if (a.nsplit > 1 && wave % KG == 0) {
                st_dev_f(a.part_ml + prow * 2, M);
                st_dev_f(a.part_ml + prow * 2 + 1, Lsum);
            }
        }
        if (a.nsplit == 1) return;
    }

    // ---- split-KV: the partials are published; the last workgroup merges ----
    merge_splits<kThreads, ROWS>(a, lds, &s_last, grp, row0, nrows, b, g);
}

// fp16 packing for the large-row kernel below
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_f16(float x, float y) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x, y}, f16x2));
}

// Large row groups (R > 128).  Eight waves (two per SIMD) own 256 query
// rows, 32 each, and stream 64-key tiles of K and V through a five-stage LDS
// ring.  Per 32-key block j every wave issues one stream in a fixed order:
//   O^T  += V(j-1)^T P(j-1)^T    8 fp16 MFMAs, with the softmax of S(j)
//                                threaded through them and each V fragment
//                                register refilled with V(j)^T after its MFMA
//   S(j+1) = K(j+1) Q^T          8 bf16 MFMAs, each K fragment register
//                                refilled with K(j+2)
// so that a wave's exponentials run under its own matrix products.  The
// running max is tested before the stream (one compare and a uniform branch;
// a rise is rare after the first block); a raise rescales O after it, once
// P(j-1) V(j-1) is in.
//
// Ring.  Tiles go from HBM to LDS by direct DMA, three tiles ahead, in eight
// key groups: group k holds the 8 keys that form one MFMA k-group of V,
// 16-key step k/2, key half k%2, i.e. keys 16 (k/2) + 4 (k%2) + {0..3} and
// the same + 8.  Waves 0-3 copy groups w and w+4 (32 keys further on); waves
// 4-7 copy nothing.  The older wave of each SIMD is favoured by the issue
// arbiter and would otherwise wait at the tile's barrier for the younger one.
// After a wave's own copies land it converts them alone: transposing reads of
// a group's 8 bf16 rows give each lane the 8 keys at one head dim, rounded to
// fp16 and written back over the same 2 KB (dims 0-63 over the first four
// rows, 64-127 over the second), so a V^T fragment is one 16-byte read.  K stays as copied
// (16-byte chunks of key k at chunk ^ (k & 15)); V rows are copied with chunk
// ^ 4 (k & 3) so that the transposing reads are conflict-free.  One workgroup
// barrier per tile: tile t starts by issuing the DMA of tile t+3 (into the
// stage of tile t-2, last read in block 2t-3 and consumed before the previous
// barrier) and ends by waiting for the DMA of tile t+2 and converting it;
// the barrier then publishes tile t+2, first read in block 2t+2.  Full cache
// tiles are copied from source pointers that advance by one tile per
// iteration, and the stage addresses of tiles t .. t+4 rotate through scalar
// registers, so the loop recomputes neither (fewer scalar instructions per
// tile: c4 ~2-3% faster, outputs bit-identical).
template <int S, bool NT>
__global__ __launch_bounds__(512) void tree_attention_wide_kernel(const AttnArgs a) {
    constexpr int NW = 8;
    constexpr int KT = 64;                 // keys per tile (two 32-key MFMA blocks)
    constexpr int TILE = KT * kRowBytes;   // bytes of a K (or V) tile
    constexpr int STAGE = 2 * TILE;        // K then V
    constexpr int RING = S * STAGE;
    constexpr int ROWS = NW * 32;          // one 32-row MFMA block per wave
    static_assert(S == 5, "five stages: tiles t-1 .. t+3 are live during tile t");
    static_assert(RING <= 160 * 1024, "LDS budget");
    static_assert(2 * ROWS * 64 * 4 + 64 <= RING, "split-merge scratch and its flag fit in the ring");
    __shared__ __attribute__((aligned(1024))) char lds[RING];
    int* const s_flag = reinterpret_cast<int*>(lds + RING - 64);  // used only by the split merge

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 31;   // MFMA column: query row within the block / key within a 32-key block
    const int hf = lane >> 5;  // which half of the k-slots this lane carries

    const int logical = xcd_remap(blockIdx.x, a.nblocks);
    const int rt = logical % a.row_tiles;
    const int tmp = logical / a.row_tiles;
    const int split = tmp % a.nsplit;
    const int bg = tmp / a.nsplit;
    const int b = bg / a.Hkv;
    const int g = bg % a.Hkv;
    const float c = a.scale_log2;

    const int Rb = a.G * seq_nodes_of(a, b);  // this sequence's query rows
    const int lb = seq_len_of(a, b);          // and its committed cache entries

    // ---- the query row this lane carries as a B-operand column ----
    const int row = rt * ROWS + wave * 32 + n;
    const bool row_ok = row < Rb;
    bf16x8 qf[8];
    uint64_t anc_row;  // ancestor word 0
    {
        const int node = row_ok ? row / a.G : 0;
        const int head = g * a.G + (row_ok ? row % a.G : 0);
        const uint16_t* qrow = a.Q + ((size_t)(b * a.N + node) * a.Hq + head) * HD;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const u32x4 v = *reinterpret_cast<const u32x4*>(qrow + 16 * s + 8 * hf);
            qf[s] = __builtin_bit_cast(bf16x8, row_ok ? v : u32x4{0, 0, 0, 0});
        }
        anc_row = row_ok ? anc_word(a, b, node, 0) : 0ull;
    }

    // ---- tiles of this workgroup: cache tiles of the split, then tree tiles ----
    const int t_begin = split * a.tiles_per_split;
    int n_cache = (lb + KT - 1) / KT - t_begin;
    if (n_cache > a.tiles_per_split) n_cache = a.tiles_per_split;
    if (n_cache < 0) n_cache = 0;
    const int nt = n_cache + ((split == a.nsplit - 1) ? a.tree_tiles : 0);
    const uint32_t ring_addr = (uint32_t)(uintptr_t)(lds_void*)lds;
    auto stage = [&](int t) { return ring_addr + (uint32_t)(t % S) * STAGE; };

    // ---- key group of this wave (waves 0-3 also copy group wave+4, rows
    // +32): rows r0 .. r0+3 and r0+8 .. r0+11 ----
    const int r0 = 16 * (wave >> 1) + 4 * (wave & 1);
    // DMA of a key group (rows r0 + roff ..) of tile u into stage u % S (1 KB
    // = four rows per copy).  Past the last tile the last tile is loaded again into the
    // (free) stage, so that every tile issues the same copies and the wait
    // counts stay static.  Per-lane byte offsets of a full cache tile's
    // copies are kept; other tiles recompute them.
    uint32_t dk[2], dv[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int key = r0 + 8 * i + (lane >> 4), pc = lane & 15;
        dk[i] = (uint32_t)(key * kRowBytes + ((pc ^ (key & 15)) << 4));
        dv[i] = (uint32_t)(key * kRowBytes + ((pc ^ (4 * (key & 3))) << 4));
    }
    // The four base pointers stay in SGPRs across the loop (selected from the
    // argument block, they would be reloaded, with a wait, every tile).
    const uint16_t* kc_p = a.Kc;
    const uint16_t* kt_p = a.Kt;
    const uint16_t* vc_p = a.Vc;
    const uint16_t* vt_p = a.Vt;
    asm volatile("" : "+s"(kc_p), "+s"(kt_p), "+s"(vc_p), "+s"(vt_p));
    auto issue_dma = [&](int u, int roff) {
        // (uniform selects rather than branches for the source)
        const int tt = min(u, nt - 1);
        const bool tree = tt >= n_cache;
        const int key0 = tree ? (tt - n_cache) * KT : (t_begin + tt) * KT;
        const size_t base = tree ? ((size_t)(b * a.N + key0) * a.Hkv + g) * HD : ((size_t)bg * a.L + key0) * HD;
        const char* ks = reinterpret_cast<const char*>((tree ? kt_p : kc_p) + base);
        const char* vs = reinterpret_cast<const char*>((tree ? vt_p : vc_p) + base);
        const uint32_t stride = tree ? (uint32_t)a.Hkv * kRowBytes : (uint32_t)kRowBytes;
        const int nk = min(KT, (tree ? a.N : lb) - key0);
        const uint32_t dst = stage(u) + (r0 + roff) * kRowBytes;
        if (!tree && nk == KT) {  // uniform: a full cache tile
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                dma16s<NT>(ks + roff * kRowBytes, dk[i], dst + 8 * i * kRowBytes);
                dma16s<NT>(vs + roff * kRowBytes, dv[i], dst + TILE + 8 * i * kRowBytes);
            }
            return;
        }
        int l = lane;
        asm volatile("" : "+v"(l));  // recomputed per call rather than held in registers
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int key = r0 + roff + 8 * i + (l >> 4), pc = l & 15;
            const uint32_t off = (uint32_t)min(key, nk - 1) * stride;  // ragged keys repeat a valid row
            dma16s<NT>(ks, off + ((pc ^ (key & 15)) << 4), dst + 8 * i * kRowBytes);
            dma16s<NT>(vs, off + ((pc ^ (4 * (key & 3))) << 4), dst + TILE + 8 * i * kRowBytes);
        }
    };
    // In-place conversion of a key group's V rows of tile u (rows r0 + roff
    // ..; roff = 32 keeps every bank pattern below).  Transposing read
    // (dims half hh, rows part p): in each 16-lane group, source lane j reads
    // row r0 + 8p + j/4 at head dims 64 hh + 16 (lane/16) + 4 (j%4) + {0..3},
    // so result lane i of the group holds rows r0 + 8p + {0..3} at dim
    // 64 hh + 16 (lane/16) + i.  The two parts make the lane's 8-key chunk
    // for that dim, written at row r0 + 8 hh, chunk lane (1 KB per copy).
    // All reads are issued before the writes over the same bytes.
    const uint32_t conv_src = (uint32_t)(TILE + (r0 + ((lane & 15) >> 2)) * kRowBytes +
                                         (((2 * (lane >> 4) + ((lane & 3) >> 1)) ^ (4 * ((lane & 15) >> 2))) << 4) +
                                         8 * (lane & 1));
    auto convert_at = [&](uint32_t st, int roff) {
        uint32_t sb = st + roff * kRowBytes;
        asm volatile("" : "+v"(sb));
        u32x2 part[2][2];  // [dims half][rows part]
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int pp = 0; pp < 2; ++pp)
                // dims half hh is logical chunk ^ 8 hh, so its physical chunk
                // is the half-0 one ^ 8: address bit 7 (rows and stages are
                // 256-byte aligned)
                part[hh][pp] = lds_tr16((sb + conv_src + 8 * pp * kRowBytes) ^ (128 * hh));
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            u32x4 w;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t x = e < 2 ? part[hh][0][e] : part[hh][1][e - 2];
                w[e] = f32x2_to_f16x2_sat(__uint_as_float(x << 16), __uint_as_float(x & 0xffff0000u));
            }
            *(lds_u32x4*)(uintptr_t)(sb + TILE + (r0 + 8 * hh) * kRowBytes + lane * 16) = w;
        }
    };
    auto convert = [&](int u, int roff) { convert_at(stage(u), roff); };
    // DMA of a full cache tile from running source pointers into stage st
    auto dma_full = [&](const char* kp, const char* vp, uint32_t st, int roff) {
        const uint32_t dst = st + (r0 + roff) * kRowBytes;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            dma16s<NT>(kp + roff * kRowBytes, dk[i], dst + 8 * i * kRowBytes);
            dma16s<NT>(vp + roff * kRowBytes, dv[i], dst + TILE + 8 * i * kRowBytes);
        }
    };

    // fragment reads: K of 32-key block kb of a stage (one 16-byte chunk per
    // 16 head dims; stage bases are 1 KB aligned, so the xor of bits 5-7
    // commutes with the add).  V^T of 16-key step h', dims block blk: chunk
    // of dim 32 blk + n for key half hf, at row 16 h' + 4 hf + 8 (blk/2),
    // chunk (32 blk + n) % 64.
    const uint32_t k_off = (uint32_t)((n * kRowBytes + hf * 16) ^ ((n & 15) << 4));
    const uint32_t vt_lane = (uint32_t)(TILE + hf * 4 * kRowBytes + n * 16);
    bf16x8 kf[8];
    u32x4 vf[2][4];
    auto read_k = [&](uint32_t sb, int kb) {
        const uint32_t ka = sb + 8192 * kb + k_off;
#pragma unroll
        for (int s = 0; s < 8; ++s) kf[s] = __builtin_bit_cast(bf16x8, lds_ld128(ka ^ (s << 5)));
    };

    f32x16 o_acc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) o_acc[i] = f32x16{};
    f32x16 s_cur;    // S(j)
    u32x4 pf[2];     // P(j-1)
    float m_used = -INFINITY;  // raw score units
    float l_run = 0.f;
    // derived from m_used, updated only when it rises: the raise threshold,
    // -m_used * c (0 while m_used is -inf) and the lanes whose m_used is -inf
    float m_thr = -INFINITY;
    float neg_mc = 0.f;
    uint64_t m_ninf = ~0ull;

    // block j = 2t + kb of tile t.  V(j)^T is block kb of tile t; K(j+2) is
    // block kb of tile t+1.
    auto block = [&](bool masked, int t, int kb, uint32_t st0, uint32_t st1) {
        // (opaque to the compiler, so that the constant parts of the
        // addresses fold into the instructions' offsets instead of being
        // precomputed into registers outside the loop)
        uint32_t sv = st0 + 8192 * kb + vt_lane;
        uint32_t ka = st1 + 8192 * kb + k_off;
        asm volatile("" : "+v"(sv), "+v"(ka));
        auto pv = [&](int s) {
            const int h = s >> 2, q = s & 3;
            o_acc[q] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, vf[h][q]),
                                                              __builtin_bit_cast(f16x8, pf[h]), o_acc[q], 0, 0, 0);
            vf[h][q] = lds_ld128(sv + 4096 * h + 2048 * (q >> 1) + 512 * (q & 1));
        };
        // two P.V MFMAs depend on nothing computed here: they run under the max
        pv(0);
        pv(1);
        // mask (tree / ragged tiles); element e of the block is key
        // 8 (e/4) + 4 hf + (e%4).  The tree is one tile (at most 64 nodes),
        // so block kb of it is word kb of the row's ancestor bits.
        if (masked) {  // uniform
            const bool is_tree = t >= n_cache;
            const int tt = t - n_cache;  // tree tile: keys 64 tt .., ancestor word tt
            const int nk = is_tree ? min(KT, a.N - KT * tt) : min(KT, lb - (t_begin + t) * KT);
            const int kbase = 32 * kb;
            uint32_t vis = nk - kbase >= 32 ? 0xffffffffu : (nk - kbase <= 0 ? 0u : (1u << (nk - kbase)) - 1u);
            if (is_tree) {
                const uint64_t aw = tt == 0 ? anc_row : (row_ok ? anc_word(a, b, row / a.G, tt) : 0ull);
                vis &= (uint32_t)(aw >> kbase);
            }
            vis >>= 4 * hf;
#pragma unroll
            for (int e = 0; e < 16; ++e)
                if (!((vis >> (8 * (e >> 2) + (e & 3))) & 1u)) s_cur[e] = -INFINITY;
        }
        // lazy running max: raised only when a score exceeds it by 2^kLazyThresh
        // (one v_max3 per pair of scores)
        float tmax = fmaxf(s_cur[0], s_cur[1]);
#pragma unroll
        for (int e = 2; e < 16; e += 2) tmax = fmaxf(fmaxf(tmax, s_cur[e]), s_cur[e + 1]);
        tmax = halves_max(tmax);
        const uint64_t rmask = __ballot(tmax > m_thr) | m_ninf;
        const bool any_raise = rmask != 0;
        float alpha = 1.f;
        if (any_raise) {  // uniform, rare after the first block
            if ((rmask >> lane) & 1ull) {
                const float m_new = fmaxf(m_used, tmax);
                alpha = (m_used == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((m_used - m_new) * c);
                m_used = m_new;
                l_run *= alpha;
            }
            m_thr = m_used + kLazyThresh / c;
            neg_mc = (m_used == -INFINITY) ? 0.f : -(m_used * c);
            m_ninf = __ballot(m_used == -INFINITY);
        }

        // P(j), software-pipelined over score pairs (pair k = elements
        // 8 (k/4) + 2 (k%4) + {0, 1}): step k issues P.V MFMA k+2, the
        // exponentials of pair k, the scaling of pair k+1 and the packing and
        // sum of pair k-1.  The packed pair goes over P(j-1) in place: the
        // MFMAs reading that half of P(j-1) are issued by then.  The sum uses
        // the fp16 values handed to the MFMA.
        const f16x2 ones = f16x2{(_Float16)1.f, (_Float16)1.f};
        float x0 = fmaf(s_cur[0], c, neg_mc), x1 = fmaf(s_cur[1], c, neg_mc);
        float e0 = 0.f, e1 = 0.f;
#pragma unroll
        for (int k = 0; k <= 8; ++k) {
            if (k + 2 < 8) pv(k + 2);
            float n0 = 0.f, n1 = 0.f;
            if (k < 8) {
                n0 = __builtin_amdgcn_exp2f(x0);
                n1 = __builtin_amdgcn_exp2f(x1);
            }
            if (k + 1 < 8) {
                const int e = 8 * ((k + 1) >> 2) + 2 * ((k + 1) & 3);
                x0 = fmaf(s_cur[e], c, neg_mc);
                x1 = fmaf(s_cur[e + 1], c, neg_mc);
            }
            if (k >= 1) {
                uint32_t w = pack_f16(e0, e1);
                asm volatile("" : "+v"(w));  // packed here, not sunk to its use in the next block
                l_run = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w), ones, l_run, false);
                pf[(k - 1) >> 2][(k - 1) & 3] = w;
            }
            e0 = n0;
            e1 = n1;
            __builtin_amdgcn_sched_barrier(0);
        }
        // S(j) is dead: S(j+1) takes its registers
        f32x16 s_next = f32x16{};
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            s_next = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s], qf[s], s_next, 0, 0, 0);
            kf[s] = __builtin_bit_cast(bf16x8, lds_ld128(ka ^ (s << 5)));
        }
        // a raise rescales everything accumulated so far, P(j-1) V(j-1) included
        if (any_raise) {
#pragma unroll
            for (int i = 0; i < 4; ++i) o_acc[i] *= alpha;
        }
        s_cur = s_next;
    };

    // a split past a short cache (ragged batch) has no tiles: it publishes an
    // empty partial (m = -inf, l = 0, O = 0) and joins the merge
    if (nt > 0) {
        // ---- prologue: DMA of tiles 0-2; tiles 0 and 1 converted; S(0); K(1)
        // in registers; P(-1) = 0 with finite V(-1) ----
        if (wave < 4)
#pragma unroll
            for (int u = 0; u < 3; ++u) {
                issue_dma(u, 0);
                issue_dma(u, 32);
            }
        wait_vmcnt<8>();  // tiles 0 and 1 have landed
        if (wave < 4) {
            convert(0, 0);
            convert(0, 32);
            convert(1, 0);
            convert(1, 32);
        }
        __syncthreads();  // tiles 0 and 1 are visible
        read_k(ring_addr, 0);
        {
            f32x16 acc = f32x16{};
#pragma unroll
            for (int s = 0; s < 8; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s], qf[s], acc, 0, 0, 0);
            s_cur = acc;
        }
        read_k(ring_addr, 1);
        pf[0] = pf[1] = u32x4{0, 0, 0, 0};
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int blk = 0; blk < 4; ++blk) vf[h][blk] = u32x4{0, 0, 0, 0};

        const int n_full = (t_begin + n_cache) * KT <= lb ? n_cache : n_cache - 1;
        // full cache tiles (the DMA's fast path): u < n_dfull
        const int n_dfull = max(0, min(n_cache, lb / KT - t_begin));
        // stage addresses of tiles t .. t+4 (t+4 is tile t-1's), rotated per tile
        uint32_t sr0 = ring_addr, sr1 = ring_addr + STAGE, sr2 = ring_addr + 2 * STAGE, sr3 = ring_addr + 3 * STAGE,
                 sr4 = ring_addr + 4 * STAGE;
        // sources of tile t+3 when it is a full cache tile
        const char* kp = reinterpret_cast<const char*>(kc_p + ((size_t)bg * a.L + (size_t)(t_begin + 3) * KT) * HD);
        const char* vp = reinterpret_cast<const char*>(vc_p + ((size_t)bg * a.L + (size_t)(t_begin + 3) * KT) * HD);
        for (int t = 0; t < nt; ++t) {
            const bool masked = t >= n_full;  // tree tiles and a ragged last cache tile
            asm volatile("" : "+s"(kp), "+s"(vp), "+s"(sr0), "+s"(sr1), "+s"(sr2), "+s"(sr3), "+s"(sr4));
            if (wave < 4) {
                if (t + 3 < n_dfull) {
                    dma_full(kp, vp, sr3, 0);
                    dma_full(kp, vp, sr3, 32);
                } else {
                    issue_dma(t + 3, 0);
                    issue_dma(t + 3, 32);
                }
            }
            kp += TILE;
            vp += TILE;
            block(masked, t, 0, sr0, sr1);
            block(masked, t, 1, sr0, sr1);
            wait_vmcnt<8>();  // tile t+2 has landed (tile t+3 still in flight)
            if (wave < 4) {
                convert_at(sr2, 0);
                convert_at(sr2, 32);
            }
            __syncthreads();  // tile t+2 is visible; tile t-1's last reads are consumed
            const uint32_t sfree = sr0;
            sr0 = sr1;
            sr1 = sr2;
            sr2 = sr3;
            sr3 = sr4;
            sr4 = sfree;
        }
        // the last block's P.V
#pragma unroll
        for (int s = 0; s < 8; ++s)
            o_acc[s & 3] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, vf[s >> 2][s & 3]),
                                                                  __builtin_bit_cast(f16x8, pf[s >> 2]), o_acc[s & 3], 0,
                                                                  0, 0);
        wait_vmcnt<0>();  // no copy into this workgroup's LDS outlives it
    }

    const float l_tot = halves_sum(l_run);
    const float m_log = (m_used == -INFINITY) ? -INFINITY : m_used * c;  // log2 units from here on
    const int grp = bg * a.row_tiles + rt;
    const int row0 = rt * ROWS;
    const int nrows = min(ROWS, Rb - row0);

    if (a.nsplit == 1) {
        if (row_ok) {
            const int node = row / a.G, head = g * a.G + row % a.G;
            const float inv = 1.f / l_tot;
            float* dst = a.out + ((size_t)(b * a.N + node) * a.Hq + head) * HD;
#pragma unroll
            for (int blk = 0; blk < 4; ++blk)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    *reinterpret_cast<f32x4*>(dst + 32 * blk + 8 * q + 4 * hf) =
                        f32x4{o_acc[blk][4 * q] * inv, o_acc[blk][4 * q + 1] * inv, o_acc[blk][4 * q + 2] * inv,
                              o_acc[blk][4 * q + 3] * inv};
        }
        return;
    }
    if (row_ok) {
        const size_t prow = ((size_t)grp * a.nsplit + split) * ROWS + (row - row0);
        const __amdgpu_buffer_rsrc_t pw =
            dev_rsrc(a.part_o + ((size_t)grp * a.nsplit + split) * ROWS * HD, (uint32_t)(ROWS * HD * 4));
        const uint32_t ob = (uint32_t)((row - row0) * HD * 4);
#pragma unroll
        for (int blk = 0; blk < 4; ++blk)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                st_dev_b128(pw, ob + (uint32_t)((32 * blk + 8 * q + 4 * hf) * 4),
                            f32x4{o_acc[blk][4 * q], o_acc[blk][4 * q + 1], o_acc[blk][4 * q + 2], o_acc[blk][4 * q + 3]});
        if (hf == 0) {
            st_dev_f(a.part_ml + prow * 2, m_log);
            st_dev_f(a.part_ml + prow * 2 + 1, l_tot);
        }
    }
    merge_splits<64 * NW, ROWS>(a, lds, s_flag, grp, row0, nrows, b, g);
}

}  // namespace
}  // namespace tv

extern "C" size_t tv_tree_attention_workspace(int B, int N, int Hq, int Hkv, int D, int L) {
    if (B <= 0 || N < 1 || N > TV_MAX_NODES || Hkv < 1 || Hq < Hkv || Hq % Hkv != 0 || D != TV_HEAD_DIM || L < 0)
        return 0;
    const tv::Plan p = tv::make_plan(B, N, Hq, Hkv, L);
    return tv::workspace_layout(B, Hkv, p).total;
}

extern "C" int tv_tree_attention_ex(const uint16_t* Q, const uint16_t* K_cache, const uint16_t* V_cache,
                                    const uint16_t* K_tree, const uint16_t* V_tree, const uint64_t* anc_mask,
                                    float* out, const int32_t* seq_nodes, const int32_t* seq_len, int B, int N,
                                    int Hq, int Hkv, int D, int L, float scale, void* workspace,
                                    size_t workspace_bytes, void* stream) {
    using namespace tv;
    if (B < 0 || N < 1 || Hkv < 1 || Hq < Hkv || Hq % Hkv != 0 || L < 0) return TV_ERR_INVALID_ARG;
    if (N > TV_MAX_NODES || D != TV_HEAD_DIM) return TV_ERR_UNSUPPORTED;
    if (!(scale > 0.f) || scale == INFINITY) return TV_ERR_INVALID_ARG;
    if (B == 0) return TV_OK;
    if (!Q || !K_tree || !V_tree || !anc_mask || !out) return TV_ERR_INVALID_ARG;
    if (L > 0 && (!K_cache || !V_cache)) return TV_ERR_INVALID_ARG;
    if (!aligned(Q, 16) || !aligned(K_tree, 16) || !aligned(V_tree, 16) || !aligned(out, 16) ||
        !aligned(anc_mask, 8) || (L > 0 && (!aligned(K_cache, 16) || !aligned(V_cache, 16))) ||
        (seq_nodes && !aligned(seq_nodes, 4)) || (seq_len && !aligned(seq_len, 4)))
        return TV_ERR_INVALID_ARG;
    const long rows = (long)B * Hkv * (Hq / Hkv) * N;
    if ((long)B * N * Hq > (1L << 30) || rows > (1L << 30)) return TV_ERR_UNSUPPORTED;

    const Plan p = make_plan(B, N, Hq, Hkv, L);
    const WsLayout wl = workspace_layout(B, Hkv, p);
    if (wl.total > 0 && (!workspace || workspace_bytes < wl.total || !aligned(workspace, 256))) return TV_ERR_WORKSPACE;

    AttnArgs a;
    a.Q = Q;
    a.Kc = K_cache;
    a.Vc = V_cache;
    a.Kt = K_tree;
    a.Vt = V_tree;
    a.anc = anc_mask;
    a.seq_nodes = seq_nodes;
    a.seq_len = seq_len;
    a.out = out;
    char* ws = static_cast<char*>(workspace);
    a.counter = wl.total ? reinterpret_cast<uint32_t*>(ws + wl.counter_off) : nullptr;
    a.part_o = wl.total ? reinterpret_cast<float*>(ws + wl.part_o_off) : nullptr;
    a.part_ml = wl.total ? reinterpret_cast<float*>(ws + wl.part_ml_off) : nullptr;
    a.N = N;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.G = Hq / Hkv;
    a.L = L;
    a.R = p.R;
    a.W = TV_MASK_WORDS(N);
    a.row_tiles = p.row_tiles;
    a.nsplit = p.nsplit;
    a.tiles_per_split = p.tiles_per_split;
    a.cache_tiles = p.cache_tiles;
    a.tree_tiles = p.tree_tiles;
    a.scale_log2 = (float)((double)scale * 1.4426950408889634);
    // A KV cache larger than twice the device's 256 MB Infinity Cache cannot
    // stay cached from one step to the next: its copies are marked
    // non-temporal (c3-c5 sized caches streamed 1.5-6% faster that way; small
    // ones that stay cached lost 2-5%).
    const bool nt = 2.0 * B * Hkv * (double)L * D * 2.0 > kNonTemporalKvBytes;
    const long nblocks = (long)B * Hkv * p.nsplit * p.row_tiles;
    if (nblocks > 0x7fffffffL) return TV_ERR_UNSUPPORTED;
    a.nblocks = (int)nblocks;

    hipStream_t st = (hipStream_t)stream;
    switch (p.variant) {
        case 0:
            if (nt)
                hipLaunchKernelGGL((tree_attention_kernel<4, 32, 2, 1, 4, true>), dim3(a.nblocks), dim3(256), 0, st, a);
            else
                hipLaunchKernelGGL((tree_attention_kernel<4, 32, 2, 1, 4, false>), dim3(a.nblocks), dim3(256), 0, st,
                                   a);
            break;
        case 1:
            if (nt)
                hipLaunchKernelGGL((tree_attention_kernel<4, 32, 2, 2, 4, true>), dim3(a.nblocks), dim3(256), 0, st, a);
            else
                hipLaunchKernelGGL((tree_attention_kernel<4, 32, 2, 2, 4, false>), dim3(a.nblocks), dim3(256), 0, st,
                                   a);
            break;
        case 2:
            if (nt)
                hipLaunchKernelGGL((tree_attention_kernel<2, 64, 2, 2, 4, true>), dim3(a.nblocks), dim3(256), 0, st, a);
            else
                hipLaunchKernelGGL((tree_attention_kernel<2, 64, 2, 2, 4, false>), dim3(a.nblocks), dim3(256), 0, st,
                                   a);
            break;
        case 4:
            if (nt)
                hipLaunchKernelGGL((tree_attention_kernel<2, 32, 2, 1, 4, true>), dim3(a.nblocks), dim3(256), 0, st, a);
            else
                hipLaunchKernelGGL((tree_attention_kernel<2, 32, 2, 1, 4, false>), dim3(a.nblocks), dim3(256), 0, st,
                                   a);
            break;
        default:
            if (nt)
                hipLaunchKernelGGL((tree_attention_wide_kernel<5, true>), dim3(a.nblocks), dim3(512), 0, st, a);
            else
                hipLaunchKernelGGL((tree_attention_wide_kernel<5, false>), dim3(a.nblocks), dim3(512), 0, st, a);
            break;
    }
    return launch_status();
}

extern "C" int tv_tree_attention(const uint16_t* Q, const uint16_t* K_cache, const uint16_t* V_cache,
                                 const uint16_t* K_tree, const uint16_t* V_tree, const uint64_t* anc_mask,
                                 float* out, int B, int N, int Hq, int Hkv, int D, int L, float scale,
                                 void* workspace, size_t workspace_bytes, void* stream) {
    return tv_tree_attention_ex(Q, K_cache, V_cache, K_tree, V_tree, anc_mask, out, nullptr, nullptr, B, N, Hq, Hkv,
                                D, L, scale, workspace, workspace_bytes, stream);
}
