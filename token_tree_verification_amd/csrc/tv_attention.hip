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
//    packed into R = G*N query rows per (sequence, KV head); a workgroup covers
//    up to 8 blocks of 32 rows, so for grouped-query heads each K/V byte read
//    from HBM serves every row of the group.
//  * One wave owns 32 query rows.  Scores are computed transposed,
//    S^T = K_tile . Q^T, with v_mfma_f32_32x32x16_bf16 (keys on the M side),
//    so a lane holds scores of a single query row: max, sum and the rescale of
//    the output accumulator are lane-local (one cross-half shuffle).
//  * P.V runs as O^T = V^T . P^T with v_mfma_f32_32x32x16_f16: P is rounded to
//    fp16 (bf16 P would cost ~1.5e-3 relative error), V is converted to fp16
//    while it is staged, transposed, into LDS.  The score accumulator already
//    holds P^T in B-operand order once the keys of each 16-key step are
//    permuted; V^T is read with the same permutation.
//  * Softmax in the exp2 domain with the scale folded into one FMA per score;
//    the running max is raised lazily (only when a score exceeds it by more
//    than 2^8), so most tiles skip the accumulator rescale; masks are applied
//    only on tree tiles and the ragged last tile.
//  * The next tile's global loads are issued before the current tile is
//    computed (register prefetch), so HBM latency overlaps the MFMA work.
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
constexpr int kTargetWorkgroups = 1024;
constexpr float kLazyThresh = 8.f;  // log2 units the running max may lag the true max

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
    int variant;  // 0: 1 row block x 4 key groups, 32-key tiles; 1: 2 x 2, 32; 2: 4 x 1, 64; 3: 8 x 1, 64
    int R, rb, kg, kt, row_tiles, nsplit, tiles_per_split, cache_tiles, tree_tiles;
};

Plan make_plan(int B, int N, int Hq, int Hkv, int L) {
    Plan p;
    const int G = Hq / Hkv;
    p.R = G * N;
    const int r32 = (p.R + 31) / 32;
    if (r32 <= 1) {
        p.variant = 0; p.rb = 1; p.kg = 4; p.kt = 32;
    } else if (r32 <= 2) {
        p.variant = 1; p.rb = 2; p.kg = 2; p.kt = 32;
    } else if (r32 <= 4) {
        p.variant = 2; p.rb = 4; p.kg = 1; p.kt = 64;
    } else {
        p.variant = 3; p.rb = 8; p.kg = 1; p.kt = 64;
    }
    p.row_tiles = (r32 + p.rb - 1) / p.rb;
    p.cache_tiles = (L + p.kt - 1) / p.kt;
    p.tree_tiles = (N + p.kt - 1) / p.kt;
    const long base = (long)B * Hkv * p.row_tiles;
    int nsplit = 1;
    p.tiles_per_split = 0;
    if (p.cache_tiles > 0) {
        const long want = (kTargetWorkgroups + base - 1) / base;
        const int max_split = (p.cache_tiles + 2 * p.kg - 1) / (2 * p.kg);  // at least two tiles per key group
        nsplit = (int)(want < max_split ? want : max_split);
        if (nsplit < 1) nsplit = 1;
        // the merging workgroup keeps one weight per (row, split) in the tile LDS
        const int tile_lds = p.kg * (p.kt * (2 * TV_HEAD_DIM + 16) + TV_HEAD_DIM * (2 * p.kt + 8));
        const int cap = tile_lds / (p.rb * 32 * 8);
        if (nsplit > cap) nsplit = cap;
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
    const size_t rows = groups * p.nsplit * p.rb * 32;
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

template <int RB, int KG, int KT>
__global__ __launch_bounds__(64 * RB * KG) void tree_attention_kernel(const AttnArgs a) {
    constexpr int NT = 64 * RB * KG;        // threads
    constexpr int TPK = 64 * RB;            // threads per key group
    constexpr int KB = KT / 32;             // 32-key MFMA blocks per tile
    constexpr int K_STRIDE = HD * 2 + 16;   // LDS bytes per key row of the bf16 K tile
    constexpr int V_STRIDE = KT * 2 + 8;    // LDS bytes per d row of the fp16 V^T tile (8-byte rows)
    constexpr int K_BYTES = KT * K_STRIDE;
    constexpr int V_BYTES = HD * V_STRIDE;
    constexpr int BUF = (K_BYTES + V_BYTES + 15) / 16 * 16;
    constexpr int KCH = KT * 16 / TPK;      // 16-byte K chunks per thread per tile
    constexpr int VUN = KT * 8 / TPK;       // V units (2 keys x 8 d) per thread per tile
    constexpr int O_STRIDE = HD + 4;        // floats per row of a key-group merge slot
    constexpr int SLOT = 32 * O_STRIDE * 4 + 64 * 4;
    static_assert(KCH >= 1 && VUN >= 1, "tile too small for the key group");
    static_assert(KG == 1 || (KG - 1) * RB * SLOT <= KG * BUF, "merge slots must fit in the tile LDS");
    __shared__ __attribute__((aligned(16))) char lds[KG * BUF];
    __shared__ int s_last;

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int rb = wave % RB;
    const int kg = wave / RB;
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
    const int r = (rt * RB + rb) * 32 + n;
    const bool row_ok = r < a.R;
    const int node = row_ok ? r / a.G : 0;
    const int head = g * a.G + (row_ok ? r % a.G : 0);
    bf16x8 qf[8];
    {
        const uint16_t* qrow = a.Q + ((size_t)(b * a.N + node) * a.Hq + head) * HD;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const u32x4 v = row_ok ? *reinterpret_cast<const u32x4*>(qrow + 16 * s + 8 * hf) : u32x4{0, 0, 0, 0};
            qf[s] = __builtin_bit_cast(bf16x8, v);
        }
    }
    const uint64_t anc_row = row_ok ? a.anc[(size_t)b * a.N + node] : 0ull;

    // ---- tiles of this workgroup: cache tiles of the split, then tree tiles ----
    const int t_begin = split * a.tiles_per_split;
    int n_cache = a.cache_tiles - t_begin;
    if (n_cache > a.tiles_per_split) n_cache = a.tiles_per_split;
    if (n_cache < 0) n_cache = 0;
    const int n_tree = (split == a.nsplit - 1) ? a.tree_tiles : 0;
    const int n_tiles = n_cache + n_tree;
    const int iters = (n_tiles + KG - 1) / KG;

    char* k_lds = lds + kg * BUF;
    char* v_lds = k_lds + K_BYTES;
    const int tk = rb * 64 + lane;  // thread index within the key group

    // global source of tile k_idx (cache or tree) and its valid key count
    auto tile_src = [&](int k_idx, const uint16_t*& ks, const uint16_t*& vs, size_t& stride, int& key0, int& nk,
                        bool& is_tree) {
        is_tree = k_idx >= n_cache;
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
    };

    // register stage of one tile: KCH K chunks, VUN V units (2 keys each)
    u32x4 kreg[KCH], vreg[VUN][2];
    auto load_tile = [&](int k_idx) {
        const uint16_t *ks, *vs;
        size_t stride;
        int key0, nk;
        bool is_tree;
        tile_src(k_idx, ks, vs, stride, key0, nk, is_tree);
#pragma unroll
        for (int i = 0; i < KCH; ++i) {
            const int ch = tk + TPK * i, key = ch >> 4, dc = ch & 15;
            kreg[i] = key < nk ? *reinterpret_cast<const u32x4*>(ks + key * stride + dc * 8) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int i = 0; i < VUN; ++i) {
            const int un = tk + TPK * i, kp = un >> 4, dc = un & 15;
            const int k0 = 2 * kp;
            vreg[i][0] = k0 < nk ? *reinterpret_cast<const u32x4*>(vs + k0 * stride + dc * 8) : u32x4{0, 0, 0, 0};
            vreg[i][1] = k0 + 1 < nk ? *reinterpret_cast<const u32x4*>(vs + (k0 + 1) * stride + dc * 8)
                                     : u32x4{0, 0, 0, 0};
        }
    };
    auto store_tile = [&]() {
#pragma unroll
        for (int i = 0; i < KCH; ++i) {
            const int ch = tk + TPK * i, key = ch >> 4, dc = ch & 15;
            *reinterpret_cast<u32x4*>(k_lds + key * K_STRIDE + dc * 16) = kreg[i];
        }
#pragma unroll
        for (int i = 0; i < VUN; ++i) {
            const int un = tk + TPK * i, kp = un >> 4, dc = un & 15;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                // V^T[d][2kp], V^T[d][2kp+1] as one fp16 pair, d = 8 dc + j
                const uint32_t w0 = vreg[i][0][j >> 1], w1 = vreg[i][1][j >> 1];
                const uint32_t h0 = (j & 1) ? (w0 >> 16) : (w0 & 0xffffu);
                const uint32_t h1 = (j & 1) ? (w1 >> 16) : (w1 & 0xffffu);
                const _Float16 f0 = (_Float16)bf16_bits_to_float(h0);
                const _Float16 f1 = (_Float16)bf16_bits_to_float(h1);
                const uint32_t pk = (uint32_t)__builtin_bit_cast(uint16_t, f0) |
                                    ((uint32_t)__builtin_bit_cast(uint16_t, f1) << 16);
                *reinterpret_cast<uint32_t*>(v_lds + (dc * 8 + j) * V_STRIDE + kp * 4) = pk;
            }
        }
    };

    f32x16 o_acc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) o_acc[i] = f32x16{};
    float m_used = -INFINITY, l_run = 0.f;  // m_used in raw score units

    if (kg < n_tiles) load_tile(kg);
    for (int it = 0; it < iters; ++it) {
        const int k_idx = it * KG + kg;
        const bool active = k_idx < n_tiles;
        if (it > 0) __syncthreads();  // the previous tile is consumed by every wave
        if (active) store_tile();
        __syncthreads();
        if (active && k_idx + KG < n_tiles) load_tile(k_idx + KG);  // in flight during the compute below
        if (active) {
            const uint16_t *ks_, *vs_;
            size_t st_;
            int key0, nk;
            bool is_tree;
            tile_src(k_idx, ks_, vs_, st_, key0, nk, is_tree);
            const bool masked = is_tree || nk < KT;
            // S^T[key][row] for KB blocks of 32 keys
            f32x16 s_acc[KB];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                s_acc[kb] = f32x16{};
#pragma unroll
                for (int s = 0; s < 8; ++s) {
                    const bf16x8 kf = __builtin_bit_cast(
                        bf16x8,
                        *reinterpret_cast<const u32x4*>(k_lds + (32 * kb + n) * K_STRIDE + (16 * s + 8 * hf) * 2));
                    s_acc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], s_acc[kb], 0, 0, 0);
                }
            }
            // element e of block kb is key 32 kb + 8 (e/4) + 4 hf + (e%4) of the tile
            if (masked) {
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int key = 32 * kb + 8 * (e >> 2) + 4 * hf + (e & 3);
                        bool vis = key < nk;
                        if (is_tree) vis = vis && ((anc_row >> ((key0 + key) & 63)) & 1ull);
                        if (!vis) s_acc[kb][e] = -INFINITY;
                    }
            }
            float tmax = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int e = 0; e < 16; ++e) tmax = fmaxf(tmax, s_acc[kb][e]);
            tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
            // raise the running max only when a score runs more than 2^8 above it
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
            const float mc = (m_used == -INFINITY) ? 0.f : m_used * c;
            f16x8 pf[2 * KB];
            float lsum = 0.f;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const float p = __builtin_amdgcn_exp2f(fmaf(s_acc[kb][e], c, -mc));
                    lsum += p;
                    pf[2 * kb + (e >> 3)][e & 7] = (_Float16)p;
                }
            l_run += lsum;
            // O^T[d][row] += V^T[d][key] P^T[key][row]
#pragma unroll
            for (int t = 0; t < 2 * KB; ++t) {
#pragma unroll
                for (int blk = 0; blk < 4; ++blk) {
                    const char* vrow = v_lds + (32 * blk + n) * V_STRIDE + (16 * t + 4 * hf) * 2;
                    const u32x2 lo = *reinterpret_cast<const u32x2*>(vrow);
                    const u32x2 hi = *reinterpret_cast<const u32x2*>(vrow + 16);
                    const f16x8 vf = __builtin_bit_cast(f16x8, u32x4{lo.x, lo.y, hi.x, hi.y});
                    o_acc[blk] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, pf[t], o_acc[blk], 0, 0, 0);
                }
            }
        }
    }

    float l_tot = l_run + __shfl_xor(l_run, 32);
    float m_log = (m_used == -INFINITY) ? -INFINITY : m_used * c;  // log2 units from here on

    // ---- merge the key groups of each row block through LDS ----
    if constexpr (KG > 1) {
        __syncthreads();
        if (kg > 0) {
            float* so = reinterpret_cast<float*>(lds + ((kg - 1) * RB + rb) * SLOT);
            float* sml = so + 32 * O_STRIDE;
#pragma unroll
            for (int blk = 0; blk < 4; ++blk)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    *reinterpret_cast<f32x4*>(so + n * O_STRIDE + 32 * blk + 8 * j + 4 * hf) =
                        f32x4{o_acc[blk][4 * j], o_acc[blk][4 * j + 1], o_acc[blk][4 * j + 2], o_acc[blk][4 * j + 3]};
            if (hf == 0) {
                sml[n] = m_log;
                sml[32 + n] = l_tot;
            }
        }
        __syncthreads();
        if (kg == 0) {
#pragma unroll
            for (int k = 1; k < KG; ++k) {
                const float* so = reinterpret_cast<const float*>(lds + ((k - 1) * RB + rb) * SLOT);
                const float* sml = so + 32 * O_STRIDE;
                const float mk = sml[n], lk = sml[32 + n];
                const float M = fmaxf(m_log, mk);
                const float a0 = (M == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_log - M);
                const float ak = (M == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mk - M);
#pragma unroll
                for (int blk = 0; blk < 4; ++blk)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const f32x4 ov = *reinterpret_cast<const f32x4*>(so + n * O_STRIDE + 32 * blk + 8 * j + 4 * hf);
#pragma unroll
                        for (int q = 0; q < 4; ++q) o_acc[blk][4 * j + q] = o_acc[blk][4 * j + q] * a0 + ov[q] * ak;
                    }
                l_tot = l_tot * a0 + lk * ak;
                m_log = M;
            }
        }
    }

    if (a.nsplit == 1) {
        if (kg != 0 || !row_ok) return;
        const float inv = 1.f / l_tot;
        float* dst = a.out + ((size_t)(b * a.N + node) * a.Hq + head) * HD;
#pragma unroll
        for (int blk = 0; blk < 4; ++blk)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                *reinterpret_cast<f32x4*>(dst + 32 * blk + 8 * j + 4 * hf) =
                    f32x4{o_acc[blk][4 * j] * inv, o_acc[blk][4 * j + 1] * inv, o_acc[blk][4 * j + 2] * inv,
                          o_acc[blk][4 * j + 3] * inv};
        return;
    }

    // ---- split-KV: publish this split's partial; the last workgroup merges ----
    constexpr int RBR = RB * 32;                   // rows per row tile
    const int grp = bg * a.row_tiles + rt;
    const int row0 = rt * RBR;
    const int nrows = min(RBR, a.R - row0);
    if (kg == 0 && row_ok) {
        const size_t prow = ((size_t)grp * a.nsplit + split) * RBR + (r - row0);
        float* dst = a.part_o + prow * HD;
#pragma unroll
        for (int blk = 0; blk < 4; ++blk)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                st_dev_f4(dst + 32 * blk + 8 * j + 4 * hf,
                          f32x4{o_acc[blk][4 * j], o_acc[blk][4 * j + 1], o_acc[blk][4 * j + 2], o_acc[blk][4 * j + 3]});
        if (hf == 0) {
            st_dev_f(a.part_ml + prow * 2, m_log);
            st_dev_f(a.part_ml + prow * 2 + 1, l_tot);
        }
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wave's partial stores have landed
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t prev =
            __hip_atomic_fetch_add(&a.counter[grp], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = prev == (uint32_t)a.nsplit - 1;
    }
    __syncthreads();
    if (!s_last) return;

    // last workgroup of the group: per row, w_s = 2^(m_s - M) / sum_s 2^(m_s - M) l_s
    float* wts = reinterpret_cast<float*>(lds);  // [nrows][nsplit] (m_s, then the weight)
    float* lsv = wts + nrows * a.nsplit;          // [nrows][nsplit] l_s
    const size_t pbase = (size_t)grp * a.nsplit * RBR;
    for (int e = threadIdx.x; e < nrows * a.nsplit; e += NT) {
        const int i = e / a.nsplit, s = e % a.nsplit;
        const float* ml = a.part_ml + (pbase + (size_t)s * RBR + i) * 2;
        wts[e] = ld_dev_f(ml);
        lsv[e] = ld_dev_f(ml + 1);
    }
    __syncthreads();
    for (int i = threadIdx.x; i < nrows; i += NT) {
        float M = -INFINITY;
        for (int s = 0; s < a.nsplit; ++s) M = fmaxf(M, wts[i * a.nsplit + s]);
        float Lsum = 0.f;
        for (int s = 0; s < a.nsplit; ++s) {
            const float wv = (M == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(wts[i * a.nsplit + s] - M);
            wts[i * a.nsplit + s] = wv;
            Lsum += wv * lsv[i * a.nsplit + s];
        }
        const float inv = 1.f / Lsum;
        for (int s = 0; s < a.nsplit; ++s) wts[i * a.nsplit + s] *= inv;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < nrows * (HD / 4); e += NT) {
        const int i = e / (HD / 4), d4 = e % (HD / 4);
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
        for (int s = 0; s < a.nsplit; ++s)
            acc += wts[i * a.nsplit + s] * ld_dev_f4(a.part_o + (pbase + (size_t)s * RBR + i) * HD + 4 * d4);
        const int rr = row0 + i;
        const int nd = rr / a.G, hd = g * a.G + rr % a.G;
        *reinterpret_cast<f32x4*>(a.out + ((size_t)(b * a.N + nd) * a.Hq + hd) * HD + 4 * d4) = acc;
    }
    if (threadIdx.x == 0)
        __hip_atomic_store(&a.counter[grp], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // ready for the next call
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
            hipLaunchKernelGGL((tree_attention_kernel<1, 4, 32>), dim3(a.nblocks), dim3(256), 0, st, a);
            break;
        case 1:
            hipLaunchKernelGGL((tree_attention_kernel<2, 2, 32>), dim3(a.nblocks), dim3(256), 0, st, a);
            break;
        case 2:
            hipLaunchKernelGGL((tree_attention_kernel<4, 1, 64>), dim3(a.nblocks), dim3(256), 0, st, a);
            break;
        default:
            hipLaunchKernelGGL((tree_attention_kernel<8, 1, 64>), dim3(a.nblocks), dim3(512), 0, st, a);
            break;
    }
    return launch_status();
}
