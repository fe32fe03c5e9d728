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
//    packed into R = G*N query rows per (sequence, KV head), so each K/V byte
//    streamed from HBM serves all R rows (grouped-query sharing).
//  * One wave owns 32 query rows.  Scores are computed transposed,
//    S^T = K_tile . Q^T, with v_mfma_f32_32x32x16_bf16 (keys on the M side),
//    so a lane holds 16 scores of a single query row: the online-softmax
//    rescale of the output accumulator is lane-local.
//  * P.V runs as O^T = V^T . P^T with v_mfma_f32_32x32x16_f16: P is rounded to
//    fp16 (bf16 P would cost ~1.5e-3 relative error), V is converted to fp16
//    while it is staged, transposed, into LDS.  The score accumulator lanes
//    already hold P^T in the B-operand order once the keys of each 16-key
//    MFMA step are permuted; V^T is read with the same permutation.
//  * A workgroup has 4 waves = RB row blocks x KG key groups.  Waves of one
//    key group share a 32-key K/V tile in LDS; key groups take interleaved
//    tiles and are merged through LDS at the end.
//  * Tree keys form at most two extra 32-key tiles, processed by the last KV
//    split; the mask bit for (row, key j) is bit j of the row's 64-bit
//    ancestor word, held in a register.
//  * Long caches are split across workgroups (split-KV); partial
//    (max, sum, unnormalised O) are merged by a log-sum-exp combine kernel.
//  * Workgroup ids are remapped so that the row tiles sharing a KV chunk run
//    on the same XCD (same L2).
#include <float.h>

#include "tv_device.h"
#include "tv_internal.h"

namespace tv {
namespace {

constexpr int HD = TV_HEAD_DIM;            // head dim
constexpr int KT = 32;                     // keys per tile
constexpr int K_STRIDE = HD * 2 + 16;      // LDS bytes per key row of the bf16 K tile
constexpr int V_STRIDE = KT * 2 + 8;       // LDS bytes per d row of the fp16 V^T tile
constexpr int K_TILE_BYTES = KT * K_STRIDE;
constexpr int V_TILE_BYTES = HD * V_STRIDE;
constexpr int KG_BYTES = K_TILE_BYTES + V_TILE_BYTES;
constexpr int O_STRIDE = HD + 4;           // floats per row of a merge slot
constexpr int SLOT_BYTES = 32 * O_STRIDE * 4 + 64 * 4;
constexpr int kTargetWorkgroups = 2048;

struct AttnArgs {
    const uint16_t* Q;
    const uint16_t* Kc;
    const uint16_t* Vc;
    const uint16_t* Kt;
    const uint16_t* Vt;
    const uint64_t* anc;
    float* out;
    float* part_o;   // [B*Hkv][nsplit][R][HD]
    float* part_ml;  // [B*Hkv][nsplit][R][2]
    int N, Hq, Hkv, G, L, R;
    int row_tiles, nsplit, tiles_per_split, cache_tiles, tree_tiles, nblocks;
    float scale_log2;
};

struct Plan {
    int R, rb, kg, row_tiles, nsplit, tiles_per_split, cache_tiles, tree_tiles;
};

Plan make_plan(int B, int N, int Hq, int Hkv, int L) {
    Plan p;
    const int G = Hq / Hkv;
    p.R = G * N;
    const int r32 = (p.R + 31) / 32;
    p.rb = r32 >= 3 ? 4 : r32;
    p.kg = 4 / p.rb;
    p.row_tiles = (r32 + p.rb - 1) / p.rb;
    p.cache_tiles = (L + KT - 1) / KT;
    p.tree_tiles = (N + KT - 1) / KT;
    const long base = (long)B * Hkv * p.row_tiles;
    int nsplit = 1;
    if (p.cache_tiles > 0) {
        const long want = (kTargetWorkgroups + base - 1) / base;
        const int max_split = (p.cache_tiles + p.kg - 1) / p.kg;  // at least one tile per key group
        nsplit = (int)(want < max_split ? want : max_split);
        if (nsplit < 1) nsplit = 1;
        int tps = (p.cache_tiles + nsplit - 1) / nsplit;
        tps = (tps + p.kg - 1) / p.kg * p.kg;
        p.tiles_per_split = tps;
        nsplit = (p.cache_tiles + tps - 1) / tps;
    } else {
        p.tiles_per_split = 0;
    }
    p.nsplit = nsplit;
    return p;
}

size_t workspace_bytes(int B, int Hkv, const Plan& p) {
    if (p.nsplit <= 1) return 0;
    const size_t rows = (size_t)B * Hkv * p.nsplit * p.R;
    return round_up(rows * HD * sizeof(float), 256) + round_up(rows * 2 * sizeof(float), 256);
}

__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
    // Dispatch places consecutive workgroup ids on consecutive XCDs (8 of
    // them); give each XCD a contiguous range of logical ids instead.
    const int xcd = bid & 7, idx = bid >> 3;
    const int per = nblocks >> 3, rem = nblocks & 7;
    return xcd < rem ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
}

template <int RB, int KG>
__global__ __launch_bounds__(256) void tree_attention_kernel(const AttnArgs a) {
    __shared__ __attribute__((aligned(16))) char lds[KG * KG_BYTES];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int rb = wave % RB;
    const int kg = wave / RB;
    const int n = lane & 31;  // MFMA column: query row within the block / key within a tile
    const int hf = lane >> 5; // which half of the k-slots this lane carries

    const int logical = xcd_remap(blockIdx.x, a.nblocks);
    const int rt = logical % a.row_tiles;
    const int tmp = logical / a.row_tiles;
    const int split = tmp % a.nsplit;
    const int bg = tmp / a.nsplit;
    const int b = bg / a.Hkv;
    const int g = bg % a.Hkv;

    // ---- query row owned by this lane (as the B-operand column) ----
    const int r = (rt * RB + rb) * 32 + n;
    const bool row_ok = r < a.R;
    const int node = row_ok ? r / a.G : 0;
    const int head = g * a.G + (row_ok ? r % a.G : 0);
    bf16x8 qf[8];
    {
        const uint16_t* qrow = a.Q + ((size_t)(b * a.N + node) * a.Hq + head) * HD;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            u32x4 v = row_ok ? *reinterpret_cast<const u32x4*>(qrow + 16 * s + 8 * hf) : u32x4{0, 0, 0, 0};
            qf[s] = __builtin_bit_cast(bf16x8, v);
        }
    }
    const uint64_t anc_row = row_ok ? a.anc[(size_t)b * a.N + node] : 0ull;

    // ---- the tiles this workgroup covers: cache tiles, then tree tiles ----
    const int t_begin = split * a.tiles_per_split;
    int n_cache = a.cache_tiles - t_begin;
    if (n_cache > a.tiles_per_split) n_cache = a.tiles_per_split;
    if (n_cache < 0) n_cache = 0;
    const int n_tree = (split == a.nsplit - 1) ? a.tree_tiles : 0;
    const int n_tiles = n_cache + n_tree;
    const int iters = (n_tiles + KG - 1) / KG;

    char* k_lds = lds + kg * KG_BYTES;
    char* v_lds = k_lds + K_TILE_BYTES;
    const int tk = rb * 64 + lane;  // thread index within the key group

    f32x16 o_acc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) o_acc[i] = f32x16{};
    float m_run = -INFINITY, l_run = 0.f;

    for (int it = 0; it < iters; ++it) {
        const int k_idx = it * KG + kg;
        const bool active = k_idx < n_tiles;
        const bool is_tree = k_idx >= n_cache;
        int key0 = 0, nkeys = 0;
        const uint16_t* ksrc = nullptr;
        const uint16_t* vsrc = nullptr;
        size_t row_stride = HD;
        if (active) {
            if (!is_tree) {
                key0 = (t_begin + k_idx) * KT;
                nkeys = a.L - key0 < KT ? a.L - key0 : KT;
                const size_t base = ((size_t)bg * a.L + key0) * HD;
                ksrc = a.Kc + base;
                vsrc = a.Vc + base;
            } else {
                key0 = (k_idx - n_cache) * KT;
                nkeys = a.N - key0 < KT ? a.N - key0 : KT;
                const size_t base = ((size_t)(b * a.N + key0) * a.Hkv + g) * HD;
                ksrc = a.Kt + base;
                vsrc = a.Vt + base;
                row_stride = (size_t)a.Hkv * HD;
            }
            // stage K (bf16, row-major) and V^T (fp16, transposed) for 32 keys
#pragma unroll
            for (int c = tk; c < KT * 16; c += RB * 64) {
                const int key = c >> 4, dc = c & 15;
                u32x4 kv = u32x4{0, 0, 0, 0}, vv = u32x4{0, 0, 0, 0};
                if (key < nkeys) {
                    kv = *reinterpret_cast<const u32x4*>(ksrc + key * row_stride + dc * 8);
                    vv = *reinterpret_cast<const u32x4*>(vsrc + key * row_stride + dc * 8);
                }
                *reinterpret_cast<u32x4*>(k_lds + key * K_STRIDE + dc * 16) = kv;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const _Float16 lo = (_Float16)bf16_bits_to_float(vv[j] & 0xffffu);
                    const _Float16 hi = (_Float16)bf16_bits_to_float(vv[j] >> 16);
                    *reinterpret_cast<_Float16*>(v_lds + (dc * 8 + 2 * j) * V_STRIDE + key * 2) = lo;
                    *reinterpret_cast<_Float16*>(v_lds + (dc * 8 + 2 * j + 1) * V_STRIDE + key * 2) = hi;
                }
            }
        }
        __syncthreads();
        if (active) {
            // S^T[key][row] = sum_d K[key][d] Q[row][d]
            f32x16 s_acc = f32x16{};
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                const bf16x8 kf = __builtin_bit_cast(
                    bf16x8, *reinterpret_cast<const u32x4*>(k_lds + n * K_STRIDE + (16 * s + 8 * hf) * 2));
                s_acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], s_acc, 0, 0, 0);
            }
            // element e of this lane is key 8*(e/4) + 4*hf + (e%4) of the tile
            float sc[16];
            float tmax = -INFINITY;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int key = 8 * (e >> 2) + 4 * hf + (e & 3);
                bool vis = key < nkeys;
                if (is_tree) vis = vis && ((anc_row >> (key0 + key)) & 1ull);
                sc[e] = vis ? s_acc[e] * a.scale_log2 : -INFINITY;
                tmax = fmaxf(tmax, sc[e]);
            }
            tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
            const float m_new = fmaxf(m_run, tmax);
            const bool any = m_new != -INFINITY;
            const float alpha = any ? exp2f(m_run - m_new) : 1.f;
            f16x8 pf[2];
            float lsum = 0.f;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const float p = any ? exp2f(sc[e] - m_new) : 0.f;
                const _Float16 ph = (_Float16)p;
                lsum += (float)ph;
                pf[e >> 3][e & 7] = ph;
            }
            l_run = l_run * alpha + lsum;
            m_run = m_new;
#pragma unroll
            for (int i = 0; i < 4; ++i) o_acc[i] *= alpha;
            // O^T[d][row] += sum_key V^T[d][key] P^T[key][row]
#pragma unroll
            for (int t = 0; t < 2; ++t) {
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
        __syncthreads();
    }

    float l_tot = l_run + __shfl_xor(l_run, 32);

    // ---- merge the key groups of each row block through LDS ----
    if constexpr (KG > 1) {
        if (kg > 0) {
            char* slot = lds + ((kg - 1) * RB + rb) * SLOT_BYTES;
            float* so = reinterpret_cast<float*>(slot);
            float* sml = so + 32 * O_STRIDE;
#pragma unroll
            for (int blk = 0; blk < 4; ++blk)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    *reinterpret_cast<f32x4*>(so + n * O_STRIDE + 32 * blk + 8 * j + 4 * hf) =
                        f32x4{o_acc[blk][4 * j], o_acc[blk][4 * j + 1], o_acc[blk][4 * j + 2], o_acc[blk][4 * j + 3]};
            if (hf == 0) {
                sml[n] = m_run;
                sml[32 + n] = l_tot;
            }
        }
        __syncthreads();
        if (kg == 0) {
#pragma unroll
            for (int k = 1; k < KG; ++k) {
                const float* so = reinterpret_cast<const float*>(lds + ((k - 1) * RB + rb) * SLOT_BYTES);
                const float* sml = so + 32 * O_STRIDE;
                const float mk = sml[n], lk = sml[32 + n];
                const float M = fmaxf(m_run, mk);
                const float a0 = (M == -INFINITY) ? 0.f : exp2f(m_run - M);
                const float ak = (M == -INFINITY) ? 0.f : exp2f(mk - M);
#pragma unroll
                for (int blk = 0; blk < 4; ++blk)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const f32x4 ov = *reinterpret_cast<const f32x4*>(so + n * O_STRIDE + 32 * blk + 8 * j + 4 * hf);
#pragma unroll
                        for (int q = 0; q < 4; ++q) o_acc[blk][4 * j + q] = o_acc[blk][4 * j + q] * a0 + ov[q] * ak;
                    }
                l_tot = l_tot * a0 + lk * ak;
                m_run = M;
            }
        }
    }
    if (kg != 0 || !row_ok) return;

    if (a.nsplit == 1) {
        const float inv = 1.f / l_tot;
        float* dst = a.out + ((size_t)(b * a.N + node) * a.Hq + head) * HD;
#pragma unroll
        for (int blk = 0; blk < 4; ++blk)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                *reinterpret_cast<f32x4*>(dst + 32 * blk + 8 * j + 4 * hf) =
                    f32x4{o_acc[blk][4 * j] * inv, o_acc[blk][4 * j + 1] * inv, o_acc[blk][4 * j + 2] * inv,
                          o_acc[blk][4 * j + 3] * inv};
    } else {
        const size_t prow = ((size_t)bg * a.nsplit + split) * a.R + r;
        float* dst = a.part_o + prow * HD;
#pragma unroll
        for (int blk = 0; blk < 4; ++blk)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                *reinterpret_cast<f32x4*>(dst + 32 * blk + 8 * j + 4 * hf) =
                    f32x4{o_acc[blk][4 * j], o_acc[blk][4 * j + 1], o_acc[blk][4 * j + 2], o_acc[blk][4 * j + 3]};
        if (hf == 0) {
            a.part_ml[prow * 2] = m_run;
            a.part_ml[prow * 2 + 1] = l_tot;
        }
    }
}

// Log-sum-exp merge of the split-KV partials: 8 rows per workgroup, 32 lanes
// per row, 4 head-dim elements per lane.
__global__ __launch_bounds__(256) void attention_combine_kernel(const float* __restrict__ part_o,
                                                                const float* __restrict__ part_ml,
                                                                float* __restrict__ out, int N, int Hq, int Hkv,
                                                                int G, int R, int nsplit, int rows_total) {
    const int gr = blockIdx.x * 8 + (threadIdx.x >> 5);
    if (gr >= rows_total) return;
    const int d4 = threadIdx.x & 31;
    const int bg = gr / R, r = gr % R;
    const size_t base = (size_t)bg * nsplit * R + r;
    float M = -INFINITY;
    for (int s = 0; s < nsplit; ++s) M = fmaxf(M, part_ml[(base + (size_t)s * R) * 2]);
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    float lsum = 0.f;
    for (int s = 0; s < nsplit; ++s) {
        const size_t row = base + (size_t)s * R;
        const float w = exp2f(part_ml[row * 2] - M);
        lsum += w * part_ml[row * 2 + 1];
        acc += w * *reinterpret_cast<const f32x4*>(part_o + row * HD + 4 * d4);
    }
    const int b = bg / Hkv, g = bg % Hkv;
    const int node = r / G, head = g * G + r % G;
    *reinterpret_cast<f32x4*>(out + ((size_t)(b * N + node) * Hq + head) * HD + 4 * d4) = acc * (1.f / lsum);
}

}  // namespace
}  // namespace tv

extern "C" size_t tv_tree_attention_workspace(int B, int N, int Hq, int Hkv, int D, int L) {
    if (B <= 0 || N < 1 || N > TV_MAX_NODES || Hkv < 1 || Hq < Hkv || Hq % Hkv != 0 || D != TV_HEAD_DIM || L < 0)
        return 0;
    return tv::workspace_bytes(B, Hkv, tv::make_plan(B, N, Hq, Hkv, L));
}

extern "C" int tv_tree_attention(const uint16_t* Q, const uint16_t* K_cache, const uint16_t* V_cache,
                                 const uint16_t* K_tree, const uint16_t* V_tree, const uint64_t* anc_mask,
                                 float* out, int B, int N, int Hq, int Hkv, int D, int L, float scale,
                                 void* workspace, size_t workspace_bytes, void* stream) {
    using namespace tv;
    if (B < 0 || N < 1 || Hkv < 1 || Hq < Hkv || Hq % Hkv != 0 || L < 0) return TV_ERR_INVALID_ARG;
    if (N > TV_MAX_NODES || D != TV_HEAD_DIM) return TV_ERR_UNSUPPORTED;
    if (!(scale == scale) || scale == INFINITY || scale == -INFINITY) return TV_ERR_INVALID_ARG;
    if (B == 0) return TV_OK;
    if (!Q || !K_tree || !V_tree || !anc_mask || !out) return TV_ERR_INVALID_ARG;
    if (L > 0 && (!K_cache || !V_cache)) return TV_ERR_INVALID_ARG;
    if (!aligned(Q, 16) || !aligned(K_tree, 16) || !aligned(V_tree, 16) || !aligned(out, 16) ||
        !aligned(anc_mask, 8) || (L > 0 && (!aligned(K_cache, 16) || !aligned(V_cache, 16))))
        return TV_ERR_INVALID_ARG;
    const long rows = (long)B * Hkv * (Hq / Hkv) * N;
    if ((long)B * N * Hq > (1L << 30) || rows > (1L << 30)) return TV_ERR_UNSUPPORTED;

    const Plan p = make_plan(B, N, Hq, Hkv, L);
    const size_t need = tv::workspace_bytes(B, Hkv, p);
    if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 256))) return TV_ERR_WORKSPACE;

    AttnArgs a;
    a.Q = Q;
    a.Kc = K_cache;
    a.Vc = V_cache;
    a.Kt = K_tree;
    a.Vt = V_tree;
    a.anc = anc_mask;
    a.out = out;
    const size_t rows_part = (size_t)B * Hkv * p.nsplit * p.R;
    a.part_o = need ? static_cast<float*>(workspace) : nullptr;
    a.part_ml = need ? reinterpret_cast<float*>(static_cast<char*>(workspace) + round_up(rows_part * HD * 4, 256))
                     : nullptr;
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
    if (p.rb == 1)
        hipLaunchKernelGGL((tree_attention_kernel<1, 4>), dim3(a.nblocks), dim3(256), 0, st, a);
    else if (p.rb == 2)
        hipLaunchKernelGGL((tree_attention_kernel<2, 2>), dim3(a.nblocks), dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL((tree_attention_kernel<4, 1>), dim3(a.nblocks), dim3(256), 0, st, a);
    if (hipGetLastError() != hipSuccess) return TV_ERR_HIP;
    if (p.nsplit > 1) {
        const int rows_total = B * Hkv * p.R;
        hipLaunchKernelGGL(attention_combine_kernel, dim3((rows_total + 7) / 8), dim3(256), 0, st, a.part_o,
                           a.part_ml, out, N, Hq, Hkv, a.G, p.R, p.nsplit, rows_total);
        if (hipGetLastError() != hipSuccess) return TV_ERR_HIP;
    }
    return TV_OK;
}
