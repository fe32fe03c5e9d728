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
//    packed into R = G*N query rows per (sequence, KV head).  A wave owns 64
//    rows as two 32-row MFMA blocks; a workgroup's four waves form KG key
//    groups of 4/KG row-waves, so one K/V byte read from HBM serves up to 256
//    rows (grouped-query heads share it).
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
//  * Tree keys are one or two extra tiles processed by the last KV split; the
//    mask bit for (row, key j) is bit j of the row's 64-bit ancestor word,
//    held in a register.
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
constexpr float kLazyThresh = 8.f;           // log2 units the running max may lag the true max

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

struct AttnArgs {
    const uint16_t* Q;
    const uint16_t* Kc;
    const uint16_t* Vc;
    const uint16_t* Kt;
    const uint16_t* Vt;
    const uint64_t* anc;
    float* out;
    float* part_o;     // [groups][nsplit][rows per tile][HD]
    float* part_ml;    // [groups][nsplit][rows per tile][2]
    uint32_t* counter; // [groups], zero between calls
    int N, Hq, Hkv, G, L, R;
    int row_tiles, nsplit, tiles_per_split, cache_tiles, tree_tiles, nblocks;
    float scale_log2;
};

struct Plan {
    int variant;  // key groups x tile keys x stages x row blocks per wave x waves:
                  // 4x32x2x1x4, 4x32x2x2x4, 2x64x2x2x4, 1x64x4x1x8
    int kg, kt, nw, rows, R, row_tiles, nsplit, tiles_per_split, cache_tiles, tree_tiles;
};

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

__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
    // Dispatch places consecutive workgroup ids on consecutive XCDs (8 of
    // them); give each XCD a contiguous range of logical ids instead.
    const int xcd = bid & 7, idx = bid >> 3;
    const int per = nblocks >> 3, rem = nblocks & 7;
    return xcd < rem ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
}

__device__ __forceinline__ void st_dev_f4(float* p, f32x4 v) {
    uint64_t* q = reinterpret_cast<uint64_t*>(p);
    __hip_atomic_store(q, (uint64_t)__float_as_uint(v[0]) | ((uint64_t)__float_as_uint(v[1]) << 32), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(q + 1, (uint64_t)__float_as_uint(v[2]) | ((uint64_t)__float_as_uint(v[3]) << 32),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ f32x4 ld_dev_f4(const float* p) {
    uint64_t* q = reinterpret_cast<uint64_t*>(const_cast<float*>(p));
    const uint64_t a = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t b = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return f32x4{__uint_as_float((uint32_t)a), __uint_as_float((uint32_t)(a >> 32)), __uint_as_float((uint32_t)b),
                 __uint_as_float((uint32_t)(b >> 32))};
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
// ring); completion is tracked explicitly with wait_vmcnt.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // m0 is reserved but only this copy writes it
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
                 :
                 : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(gptr)
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


// bf16 bits -> fp16, two values per dword (exact for normal fp16 magnitudes).
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w) {
    const float a = __uint_as_float(w << 16), b = __uint_as_float(w & 0xffff0000u);
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)a) |
           ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)b) << 16);
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

// Split-KV merge: every workgroup of a row group has published its partial
// (max, sum, unnormalised O); the last one to arrive (device-scope counter)
// combines them, w_s = 2^(m_s - M) / sum_s 2^(m_s - M) l_s, writes the output
// and resets the counter for the next call.  `lds` holds at least
// 2 * nrows * nsplit floats; `s_flag` is a workgroup-shared int outside them.
template <int NT, int ROWS>
__device__ void merge_splits(const AttnArgs& a, char* lds, int* s_flag, int grp, int row0, int nrows, int b,
                             int g) {
    __builtin_amdgcn_s_waitcnt(0);  // this wave's partial stores have landed
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t prev =
            __hip_atomic_fetch_add(&a.counter[grp], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *s_flag = prev == (uint32_t)a.nsplit - 1;
    }
    __syncthreads();
    if (!*s_flag) return;

    // last workgroup of the group: per row, w_s = 2^(m_s - M) / sum_s 2^(m_s - M) l_s
    const int ns = a.nsplit;
    float* wts = reinterpret_cast<float*>(lds);  // [nrows][ns] (m_s, then the weight)
    float* lsv = wts + nrows * ns;               // [nrows][ns] l_s
    const size_t pbase = (size_t)grp * ns * ROWS;
    for (int e0 = 0; e0 < nrows * ns; e0 += 8 * NT) {
        float mv[8], lv[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int e = min(e0 + k * NT + (int)threadIdx.x, nrows * ns - 1);
            const float* ml = a.part_ml + (pbase + (size_t)(e % ns) * ROWS + e / ns) * 2;
            mv[k] = ld_dev_f(ml);
            lv[k] = ld_dev_f(ml + 1);
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int e = e0 + k * NT + (int)threadIdx.x;
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
    // each thread owns output float4s, two at a time, with 16 split loads in flight
    const int nout = nrows * (HD / 4);
    for (int e0 = threadIdx.x; e0 < nout; e0 += 2 * NT) {
        int ei[2];
        f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
        for (int s0 = 0; s0 < ns; s0 += 8) {
            f32x4 v[2][8];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                ei[u] = min(e0 + u * NT, nout - 1);
                const float* src = a.part_o + (pbase + ei[u] / (HD / 4)) * HD + 4 * (ei[u] % (HD / 4));
#pragma unroll
                for (int k = 0; k < 8; ++k) v[u][k] = ld_dev_f4(src + (size_t)min(s0 + k, ns - 1) * ROWS * HD);
            }
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int k = 0; k < 8; ++k)
                    if (s0 + k < ns) acc[u] += wts[(ei[u] / (HD / 4)) * ns + s0 + k] * v[u][k];
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int e = e0 + u * NT;
            if (e >= nout) continue;
            const int i = e / (HD / 4), d4 = e % (HD / 4);
            const int rr = row0 + i;
            const int nd = rr / a.G, hd = g * a.G + rr % a.G;
            *reinterpret_cast<f32x4*>(a.out + ((size_t)(b * a.N + nd) * a.Hq + hd) * HD + 4 * d4) = acc[u];
        }
    }
    if (threadIdx.x == 0)
        __hip_atomic_store(&a.counter[grp], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // ready for the next call
}

template <int KG, int KT, int S, int RBW, int NW>
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

    // ---- the query rows this lane carries as B-operand columns ----
    int row[RBW];
    bool row_ok[RBW];
    bf16x8 qf[RBW][8];
    uint64_t anc_row[RBW];
#pragma unroll
    for (int j = 0; j < RBW; ++j) {
        row[j] = rt * ROWS + rw * WROWS + 32 * j + n;
        row_ok[j] = row[j] < a.R;
        const int node = row_ok[j] ? row[j] / a.G : 0;
        const int head = g * a.G + (row_ok[j] ? row[j] % a.G : 0);
        const uint16_t* qrow = a.Q + ((size_t)(b * a.N + node) * a.Hq + head) * HD;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const u32x4 v = *reinterpret_cast<const u32x4*>(qrow + 16 * s + 8 * hf);
            qf[j][s] = __builtin_bit_cast(bf16x8, row_ok[j] ? v : u32x4{0, 0, 0, 0});
        }
        anc_row[j] = row_ok[j] ? a.anc[(size_t)b * a.N + node] : 0ull;
    }

    // ---- tiles of this workgroup: cache tiles of the split, then tree tiles ----
    const int t_begin = split * a.tiles_per_split;
    int n_cache = a.cache_tiles - t_begin;
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
            nk = min(KT, a.L - key0);
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
            dma16(ks + row_off + (pc ^ (key & 15)) * 8, kdst_addr + inst * 1024);
            dma16(vs + row_off + (pc ^ (4 * (key & 3))) * 8, kdst_addr + TILE + inst * 1024);
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
        const int nk = is_tree ? min(KT, a.N - key0) : min(KT, a.L - key0);
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
                    if (is_tree) vis &= (uint32_t)(anc_row[j] >> ((key0 + kbase) & 63));
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
    const int nrows = min(ROWS, a.R - row0);

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
#pragma unroll
        for (int j = 0; j < RBW; ++j) {
            if (!row_ok[j]) continue;
            const size_t prow = ((size_t)grp * a.nsplit + split) * ROWS + (row[j] - row0);
            float* dst = a.part_o + prow * HD;
#pragma unroll
            for (int blk = 0; blk < 4; ++blk)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    st_dev_f4(dst + 32 * blk + 8 * q + 4 * hf,
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
                    st_dev_f4(a.part_o + prow * HD + d_lo + 4 * d4, acc);
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

// Large row groups (R > 128): eight waves (two per SIMD) own 256 query rows
// and step through 64-key tiles.  K/V tiles are staged through registers:
// each wave loads its 4 KB share of a tile with coalesced 16-byte loads one
// iteration ahead, converts the V half to fp16 in registers and writes both
// halves into a four-stage LDS ring with swizzled chunks.  The loop is
// software-pipelined so that the score MFMAs of the next 32-key block are in
// flight while the vector ALUs run the softmax of the current block, with one
// barrier per tile:
//   step 1  S(t,1) = K(t,1) Q^T       ||  softmax of S(t,0) -> P(t,0);
//           loads of tile t+3 issued
//   step 2  O^T += V(t,0)^T P(t,0)^T  ||  tile t+2 (loaded in step 1 of the
//           previous tile) converted and written to its stage
//   step 3  barrier: tile t+2 visible to every wave
//   step 4  S(t+1,0) = K(t+1,0) Q^T   ||  softmax of S(t,1) -> P(t,1)
//   step 5  O^T += V(t,1)^T P(t,1)^T
// Tile t+2 is written into the stage of tile t-2, whose last reads ended
// before the previous barrier.  The softmax sums the fp16-rounded P it hands
// to the MFMA (v_dot2 with fp32 accumulation), so the normaliser matches the
// weights used.
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
template <bool B>
struct Flag {
    static constexpr bool value = B;
};

__device__ __forceinline__ uint32_t pack_f16(float x, float y) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x, y}, f16x2));
}

template <int S>
__global__ __launch_bounds__(512) void tree_attention_wide_kernel(const AttnArgs a) {
    constexpr int NW = 8;
    constexpr int KT = 64;                          // keys per tile (two 32-key MFMA blocks)
    constexpr int TILE = KT * kRowBytes;            // bytes of a K (or V) tile
    constexpr int STAGE = 2 * TILE;                 // K then V
    constexpr int RING = S * STAGE;
    constexpr int ROWS = NW * 32;                   // one 32-row MFMA block per wave
    constexpr int LD = TILE / (16 * kWave) / NW;    // 16-byte loads per lane per operand
    static_assert(S == 4, "stage indices below use t & 3");
    static_assert(RING <= 160 * 1024, "LDS budget");
    static_assert(2 * ROWS * 64 * 4 <= RING, "split-merge scratch fits in the ring");
    __shared__ __attribute__((aligned(1024))) char lds[RING];
    __shared__ int s_flag;

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

    // ---- the query row this lane carries as a B-operand column ----
    const int row = rt * ROWS + wave * 32 + n;
    const bool row_ok = row < a.R;
    bf16x8 qf[8];
    uint64_t anc_row;
    {
        const int node = row_ok ? row / a.G : 0;
        const int head = g * a.G + (row_ok ? row % a.G : 0);
        const uint16_t* qrow = a.Q + ((size_t)(b * a.N + node) * a.Hq + head) * HD;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const u32x4 v = *reinterpret_cast<const u32x4*>(qrow + 16 * s + 8 * hf);
            qf[s] = __builtin_bit_cast(bf16x8, row_ok ? v : u32x4{0, 0, 0, 0});
        }
        anc_row = row_ok ? a.anc[(size_t)b * a.N + node] : 0ull;
    }

    // ---- tiles of this workgroup: cache tiles of the split, then tree tiles ----
    const int t_begin = split * a.tiles_per_split;
    int n_cache = a.cache_tiles - t_begin;
    if (n_cache > a.tiles_per_split) n_cache = a.tiles_per_split;
    if (n_cache < 0) n_cache = 0;
    const int nt = n_cache + ((split == a.nsplit - 1) ? a.tree_tiles : 0);
    const uint32_t ring_addr = (uint32_t)(uintptr_t)(lds_void*)lds;

    // This lane moves 16-byte chunks p = (wave LD + i) 64 + lane of a tile:
    // key p / 16, logical chunk p % 16, stored at chunk ^ (key & 15) for K
    // and chunk ^ 4 (key & 3) for V.
    struct Slot {
        u32x4 k[LD], v[LD];
    };
    uint32_t lds_k[LD], lds_v[LD];
#pragma unroll
    for (int i = 0; i < LD; ++i) {
        const int p = (wave * LD + i) * kWave + lane;
        const int key = p >> 4, lc = p & 15;
        lds_k[i] = (uint32_t)(key * kRowBytes + ((lc ^ (key & 15)) << 4));
        lds_v[i] = (uint32_t)(TILE + key * kRowBytes + ((lc ^ (4 * (key & 3))) << 4));
    }
    // Loads are issued for every iteration so that the number in flight is
    // the same on every path (the wait before a slot's store then covers
    // only that slot); past the last tile the last tile is loaded again
    // (recently read, so served from cache) and never stored.
    auto load_tile = [&](int t, Slot& sl) {
        t = min(t, nt - 1);
        const char *ks, *vs;
        uint32_t stride, nk;
        if (t < n_cache) {
            const int key0 = (t_begin + t) * KT;
            const size_t base = ((size_t)bg * a.L + key0) * HD;
            ks = reinterpret_cast<const char*>(a.Kc + base);
            vs = reinterpret_cast<const char*>(a.Vc + base);
            stride = kRowBytes;
            nk = (uint32_t)min(KT, a.L - key0);
        } else {
            const int key0 = (t - n_cache) * KT;
            const size_t base = ((size_t)(b * a.N + key0) * a.Hkv + g) * HD;
            ks = reinterpret_cast<const char*>(a.Kt + base);
            vs = reinterpret_cast<const char*>(a.Vt + base);
            stride = (uint32_t)a.Hkv * kRowBytes;
            nk = (uint32_t)min(KT, a.N - key0);
        }
#pragma unroll
        for (int i = 0; i < LD; ++i) {
            const uint32_t p = (uint32_t)((wave * LD + i) * kWave + lane);
            const uint32_t key = p >> 4;
            // ragged tiles repeat their last valid row (masked, finite)
            const uint32_t off = (key < nk ? key : nk - 1) * stride + ((p & 15) << 4);
            sl.k[i] = *reinterpret_cast<const u32x4*>(ks + off);
            sl.v[i] = *reinterpret_cast<const u32x4*>(vs + off);
        }
    };
    // V to fp16 (exact bf16 -> fp32, then round to nearest), both halves to LDS
    auto store_tile = [&](int t, const Slot& sl) {
        if (t >= nt) return;  // uniform
        char* st = lds + (t & 3) * STAGE;
#pragma unroll
        for (int i = 0; i < LD; ++i) {
            u32x4 y;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                y[e] = pack_f16(__uint_as_float(sl.v[i][e] << 16), __uint_as_float(sl.v[i][e] & 0xffff0000u));
            *reinterpret_cast<u32x4*>(st + lds_k[i]) = sl.k[i];
            *reinterpret_cast<u32x4*>(st + lds_v[i]) = y;
        }
    };

    // LDS offsets within a stage (the generic kernel derives them):
    //  K fragment (kb, s): (k_off ^ (s << 5)) + 8192 kb
    //  V^T fragment (step tt, block blk): (v_off ^ (blk << 6)) + 4096 tt (+ 2048 for keys + 8)
    const uint32_t k_off = (uint32_t)((n * kRowBytes + hf * 16) ^ ((n & 15) << 4));
    const int gq = lane >> 4, w16 = lane & 15;
    const int kr = 4 * (gq >> 1) + (w16 >> 2);
    const int c0 = 2 * (gq & 1) + ((w16 & 3) >> 1);
    const uint32_t v_off = (uint32_t)(TILE + ((kr * kRowBytes) | (c0 << 4) | ((kr & 3) << 6)) + 8 * (w16 & 1));
    uint32_t k_s[8], v_b[4];
#pragma unroll
    for (int s = 0; s < 8; ++s) k_s[s] = k_off ^ (s << 5);
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) v_b[blk] = v_off ^ (blk << 6);

    // per-lane K fragment addresses of a stage (uniform stage base + lane offset)
    auto k_addrs = [&](uint32_t sb, uint32_t (&ka)[8]) {
#pragma unroll
        for (int s = 0; s < 8; ++s) ka[s] = sb + k_s[s];
    };
    auto read_k = [&](const uint32_t (&ka)[8], int kb, bf16x8 (&kf)[8]) {
#pragma unroll
        for (int s = 0; s < 8; ++s) kf[s] = __builtin_bit_cast(bf16x8, lds_ld128(ka[s] + 8192 * kb));
    };
    auto qk = [&](const bf16x8 (&kf)[8]) {
        f32x16 acc = f32x16{};
#pragma unroll
        for (int s = 0; s < 8; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s], qf[s], acc, 0, 0, 0);
        return acc;
    };

    f32x16 o_acc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) o_acc[i] = f32x16{};
    float m_used = -INFINITY;  // raw score units
    float l_run = 0.f;

    // mask (tree / ragged tiles) and lazy running max of one 32-key block;
    // returns m c for the exponentials.  Element e of the block is key
    // 8 (e/4) + 4 hf + (e%4).
    auto softmax_max = [&](auto masked_tag, f32x16& sv, bool is_tree, int key0, int nk, int kb) {
        if constexpr (decltype(masked_tag)::value) {
            const int kbase = 32 * kb;
            uint32_t vis = nk - kbase >= 32 ? 0xffffffffu : (nk - kbase <= 0 ? 0u : (1u << (nk - kbase)) - 1u);
            if (is_tree) vis &= (uint32_t)(anc_row >> ((key0 + kbase) & 63));
            vis >>= 4 * hf;
#pragma unroll
            for (int e = 0; e < 16; ++e)
                if (!((vis >> (8 * (e >> 2) + (e & 3))) & 1u)) sv[e] = -INFINITY;
        }
        float tmax = fmaxf(sv[0], sv[1]);
#pragma unroll
        for (int e = 2; e < 16; e += 2) tmax = fmaxf(tmax, fmaxf(sv[e], sv[e + 1]));
        tmax = halves_max(tmax);
        const bool raise = tmax > m_used + kLazyThresh / c || m_used == -INFINITY;
        if (__ballot(raise)) {
            const float m_new = raise ? fmaxf(m_used, tmax) : m_used;
            const float alpha = (m_used == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((m_used - m_new) * c);
            if (raise) {
                l_run *= alpha;
#pragma unroll
                for (int i = 0; i < 4; ++i) o_acc[i] *= alpha;
            }
            m_used = m_new;
        }
        return (m_used == -INFINITY) ? 0.f : m_used * c;
    };
    // P = exp2(s c - m c) as fp16 B operands of the block's two 16-key steps
    auto softmax_exp = [&](const f32x16& sv, float mc, u32x4 (&pf)[2]) {
        const f16x2 ones = f16x2{(_Float16)1.f, (_Float16)1.f};
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t w = pack_f16(__builtin_amdgcn_exp2f(fmaf(sv[8 * h + 2 * q], c, -mc)),
                                            __builtin_amdgcn_exp2f(fmaf(sv[8 * h + 2 * q + 1], c, -mc)));
                l_run = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w), ones, l_run, false);
                pf[h][q] = w;
            }
    };
    // V^T fragments of 16-key step h of block kb
    auto read_v = [&](const uint32_t (&va)[4], int kb, int h, u32x2 (&vl)[4], u32x2 (&vh)[4]) {
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) {
            vl[blk] = lds_tr16(va[blk] + 4096 * (2 * kb + h));
            vh[blk] = lds_tr16(va[blk] + 4096 * (2 * kb + h) + 2048);
        }
    };
    auto pv = [&](const u32x2 (&vl)[4], const u32x2 (&vh)[4], const u32x4& p) {
#pragma unroll
        for (int blk = 0; blk < 4; ++blk)
            o_acc[blk] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                __builtin_bit_cast(f16x8, u32x4{vl[blk].x, vl[blk].y, vh[blk].x, vh[blk].y}),
                __builtin_bit_cast(f16x8, p), o_acc[blk], 0, 0, 0);
    };
    // scheduling: the eight score MFMAs of the next block each followed by
    // six vector-ALU instructions of the current block's exponentials
    auto interleave_qk_exp = [&]() {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
        }
    };

    uint32_t sb = ring_addr;  // stage base of tile t (uniform)
    uint32_t ka[8];           // K fragment addresses of tile t
    f32x16 s_a;               // scores of block 0 of tile t

    // one tile; `ld` receives tile t+3, `st` holds tile t+2.  Tiles that need
    // the mask (tree tiles, a ragged last tile) run a separate instance.
    auto iteration = [&](auto masked_tag, int t, Slot& ld, Slot& st) {
        const bool is_tree = t >= n_cache;
        const int key0 = is_tree ? (t - n_cache) * KT : (t_begin + t) * KT;
        const int nk = is_tree ? min(KT, a.N - key0) : min(KT, a.L - key0);
        u32x4 pf[2];
        u32x2 vl[2][4], vh[2][4];
        bf16x8 kf[8];
        uint32_t va[4];
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) va[blk] = sb + v_b[blk];
        const uint32_t sb_next = sb + STAGE == ring_addr + RING ? ring_addr : sb + STAGE;
        // step 1
        read_k(ka, 1, kf);
        float mc = softmax_max(masked_tag, s_a, is_tree, key0, nk, 0);
        f32x16 s_b = qk(kf);
        softmax_exp(s_a, mc, pf);
        interleave_qk_exp();
        load_tile(t + 3, ld);
        // step 2
        // (the P.V steps run at raised wave priority: the SIMD's other wave is
        // then in its exponentials, which fill the MFMA gaps)
        __builtin_amdgcn_s_setprio(1);
        read_v(va, 0, 0, vl[0], vh[0]);
        read_v(va, 0, 1, vl[1], vh[1]);
        store_tile(t + 2, st);
        pv(vl[0], vh[0], pf[0]);
        pv(vl[1], vh[1], pf[1]);
        __builtin_amdgcn_s_setprio(0);
        // step 3
        __syncthreads();
        // step 4 (past the last tile the scores come from a stage no tile
        // uses and are dropped)
        k_addrs(sb_next, ka);
        read_k(ka, 0, kf);
        mc = softmax_max(masked_tag, s_b, is_tree, key0, nk, 1);
        s_a = qk(kf);
        softmax_exp(s_b, mc, pf);
        interleave_qk_exp();
        // step 5
        __builtin_amdgcn_s_setprio(1);
        read_v(va, 1, 0, vl[0], vh[0]);
        read_v(va, 1, 1, vl[1], vh[1]);
        pv(vl[0], vh[0], pf[0]);
        pv(vl[1], vh[1], pf[1]);
        __builtin_amdgcn_s_setprio(0);
        sb = sb_next;
    };

    // ---- prologue: tiles 0 and 1 in LDS, tile 2 in flight ----
    Slot s0, s1;
    load_tile(0, s0);
    load_tile(1, s1);
    store_tile(0, s0);
    store_tile(1, s1);
    load_tile(2, s0);
    __syncthreads();
    k_addrs(sb, ka);
    {
        bf16x8 kf[8];
        read_k(ka, 0, kf);
        s_a = qk(kf);
    }
    // full cache tiles (no mask) in pairs, so that the slots alternate
    // statically; then the rest (a ragged last cache tile, the tree tiles and
    // an odd leftover) with the mask
    const int n_full = (t_begin + n_cache) * KT <= a.L ? n_cache : n_cache - 1;
    int t = 0;
    for (; t + 1 < n_full; t += 2) {
        iteration(Flag<false>{}, t, s1, s0);
        iteration(Flag<false>{}, t + 1, s0, s1);
    }
    for (; t < nt; ++t) {
        iteration(Flag<true>{}, t, s1, s0);
        const Slot tmp_slot = s0;  // the slot roles alternate
        s0 = s1;
        s1 = tmp_slot;
    }

    const float l_tot = halves_sum(l_run);
    const float m_log = (m_used == -INFINITY) ? -INFINITY : m_used * c;  // log2 units from here on
    const int grp = bg * a.row_tiles + rt;
    const int row0 = rt * ROWS;
    const int nrows = min(ROWS, a.R - row0);

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
        float* dst = a.part_o + prow * HD;
#pragma unroll
        for (int blk = 0; blk < 4; ++blk)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                st_dev_f4(dst + 32 * blk + 8 * q + 4 * hf,
                          f32x4{o_acc[blk][4 * q], o_acc[blk][4 * q + 1], o_acc[blk][4 * q + 2], o_acc[blk][4 * q + 3]});
        if (hf == 0) {
            st_dev_f(a.part_ml + prow * 2, m_log);
            st_dev_f(a.part_ml + prow * 2 + 1, l_tot);
        }
    }
    merge_splits<64 * NW, ROWS>(a, lds, &s_flag, grp, row0, nrows, b, g);
}

}  // namespace
}  // namespace tv

extern "C" size_t tv_tree_attention_workspace(int B, int N, int Hq, int Hkv, int D, int L) {
    if (B <= 0 || N < 1 || N > TV_MAX_NODES || Hkv < 1 || Hq < Hkv || Hq % Hkv != 0 || D != TV_HEAD_DIM || L < 0)
        return 0;
    const tv::Plan p = tv::make_plan(B, N, Hq, Hkv, L);
    return tv::workspace_layout(B, Hkv, p).total;
}

extern "C" int tv_tree_attention(const uint16_t* Q, const uint16_t* K_cache, const uint16_t* V_cache,
                                 const uint16_t* K_tree, const uint16_t* V_tree, const uint64_t* anc_mask,
                                 float* out, int B, int N, int Hq, int Hkv, int D, int L, float scale,
                                 void* workspace, size_t workspace_bytes, void* stream) {
    using namespace tv;
    if (B < 0 || N < 1 || Hkv < 1 || Hq < Hkv || Hq % Hkv != 0 || L < 0) return TV_ERR_INVALID_ARG;
    if (N > TV_MAX_NODES || D != TV_HEAD_DIM) return TV_ERR_UNSUPPORTED;
    if (!(scale > 0.f) || scale == INFINITY) return TV_ERR_INVALID_ARG;
    if (B == 0) return TV_OK;
    if (!Q || !K_tree || !V_tree || !anc_mask || !out) return TV_ERR_INVALID_ARG;
    if (L > 0 && (!K_cache || !V_cache)) return TV_ERR_INVALID_ARG;
    if (!aligned(Q, 16) || !aligned(K_tree, 16) || !aligned(V_tree, 16) || !aligned(out, 16) ||
        !aligned(anc_mask, 8) || (L > 0 && (!aligned(K_cache, 16) || !aligned(V_cache, 16))))
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
    a.row_tiles = p.row_tiles;
    a.nsplit = p.nsplit;
    a.tiles_per_split = p.tiles_per_split;
    a.cache_tiles = p.cache_tiles;
    a.tree_tiles = p.tree_tiles;
    a.scale_log2 = (float)((double)scale * 1.4426950408889634);
    const long nblocks = (long)B * Hkv * p.nsplit * p.row_tiles;
    if (nblocks > 0x7fffffffL) return TV_ERR_UNSUPPORTED;
    a.nblocks = (int)nblocks;

    hipStream_t st = (hipStream_t)stream;
    switch (p.variant) {
        case 0:
            hipLaunchKernelGGL((tree_attention_kernel<4, 32, 2, 1, 4>), dim3(a.nblocks), dim3(256), 0, st, a);
            break;
        case 1:
            hipLaunchKernelGGL((tree_attention_kernel<4, 32, 2, 2, 4>), dim3(a.nblocks), dim3(256), 0, st, a);
            break;
        case 2:
            hipLaunchKernelGGL((tree_attention_kernel<2, 64, 2, 2, 4>), dim3(a.nblocks), dim3(256), 0, st, a);
            break;
        default:
            hipLaunchKernelGGL((tree_attention_wide_kernel<4>), dim3(a.nblocks), dim3(512), 0, st, a);
            break;
    }
    return launch_status();
}
