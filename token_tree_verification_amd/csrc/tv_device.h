// Device-side helpers shared by the libtv HIP kernels (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// Philox-4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As
// Easy as 1, 2, 3", SC'11): ten rounds of two 32x32->64-bit multiplies by the
// round multipliers, state (hi(M1*c2)^c1^k0, lo(M1*c2), hi(M0*c0)^c3^k1,
// lo(M0*c0)), with the key bumped by the Weyl constants between rounds.
__device__ __forceinline__ u32x4 philox4x32_10(u32x4 c, uint32_t k0, uint32_t k1) {
    constexpr uint32_t kMul0 = 0xD2511F53u, kMul1 = 0xCD9E8D57u;
    constexpr uint32_t kBump0 = 0x9E3779B9u, kBump1 = 0xBB67AE85u;
#pragma unroll
    for (int round = 0; round < 10; ++round) {
        const uint32_t lo0 = kMul0 * c.x, hi0 = __umulhi(kMul0, c.x);
        const uint32_t lo1 = kMul1 * c.z, hi1 = __umulhi(kMul1, c.z);
        c = u32x4{hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0};
        k0 += kBump0;
        k1 += kBump1;
    }
    return c;
}

// Uniform in [0,1) on the 2^-24 grid from counter (node, seq, purpose, 0).
__device__ __forceinline__ float philox_uniform(uint64_t seed, uint32_t node, uint32_t seq, uint32_t purpose) {
    const u32x4 r = philox4x32_10(u32x4{node, seq, purpose, 0u}, (uint32_t)seed, (uint32_t)(seed >> 32));
    return (float)(r.x >> 8) * (1.0f / 16777216.0f);
}

// exp(y) for y <= 0 to ~1e-15 relative, in fp64: y = (k/32) ln 2 + r with
// k = rint(32 y / ln 2) (Cody-Waite reduction, ln 2 / 32 split into a double
// and its remainder), exp(r) by its degree-5 Taylor polynomial (|r| <= ln2/64,
// truncation < 3e-15), and 2^(k/32) = 2^(k >> 5) * tab[k & 31] where
// tab[j] = 2^(j/32) comes from exp2_table().  Returns 0 below -745.
__host__ __device__ __forceinline__ double exp_nonpos(double y, const double* tab) {
    if (!(y > -745.0)) return 0.0;
    const double kInv = 0x1.71547652b82fep+5;   // 32 / ln 2
    const double kLhi = 0x1.62e42fefa39efp-6;   // ln 2 / 32, rounded to double
    const double kLlo = 0x1.abc9e3b39803fp-61;  // ln 2 / 32 - kLhi
    const double kd = rint(y * kInv);
    const int k = (int)kd;
    double r = fma(-kd, kLhi, y);
    r = fma(-kd, kLlo, r);
    double p = fma(r, 1.0 / 120.0, 1.0 / 24.0);
    p = fma(r, p, 1.0 / 6.0);
    p = fma(r, p, 0.5);
    p = fma(r, p, 1.0);
    p = fma(r, p, 1.0);
    return ldexp(tab[k & 31] * p, k >> 5);
}

// tab[j] = 2^(j/32), j = 0..31 (from the library's exp2).
__host__ __device__ __forceinline__ void exp2_table(double* tab, int j) { tab[j] = exp2((double)j / 32.0); }

// ---- wave reductions on DPP lane moves (no LDS round trips) ----
// quad_perm [1,0,3,2] and [2,3,0,1] combine the lanes of a quad, row_half_mirror
// the two quads of each 8-lane half-row, row_mirror the two halves of each
// 16-lane row; readlane then combines the four rows.  Every step pairs lanes
// whose values are already uniform over the smaller group, so mirrors act as
// xor exchanges.  All 64 lanes must be active.
constexpr int kDppQuadXor1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, true);
}
template <int CTRL>
__device__ __forceinline__ double dpp_d(double v) {
    const uint64_t b = (uint64_t)__double_as_longlong(v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, CTRL, 0xF, 0xF, true);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(b >> 32), CTRL, 0xF, 0xF, true);
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
__device__ __forceinline__ float readlane_f(float v, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
__device__ __forceinline__ double readlane_d(double v, int l) {
    const uint64_t b = (uint64_t)__double_as_longlong(v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), l);
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Reductions over aligned groups of `g` lanes (g a power of two, 1..64,
// wave-uniform); every lane of a group receives the group's result.
__device__ __forceinline__ float group_max_dpp(float v, int g) {
    if (g >= 2) v = fmaxf(v, dpp_f<kDppQuadXor1>(v));
    if (g >= 4) v = fmaxf(v, dpp_f<kDppQuadXor2>(v));
    if (g >= 8) v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
    if (g >= 16) v = fmaxf(v, dpp_f<kDppRowMirror>(v));
    if (g >= 32) {
        const float r0 = readlane_f(v, 0), r1 = readlane_f(v, 16), r2 = readlane_f(v, 32), r3 = readlane_f(v, 48);
        const int lane = threadIdx.x & 63;
        v = g == 64 ? fmaxf(fmaxf(r0, r1), fmaxf(r2, r3)) : (lane < 32 ? fmaxf(r0, r1) : fmaxf(r2, r3));
    }
    return v;
}
__device__ __forceinline__ double group_sum_dpp(double v, int g) {
    if (g >= 2) v += dpp_d<kDppQuadXor1>(v);
    if (g >= 4) v += dpp_d<kDppQuadXor2>(v);
    if (g >= 8) v += dpp_d<kDppHalfMirror>(v);
    if (g >= 16) v += dpp_d<kDppRowMirror>(v);
    if (g >= 32) {
        const double r0 = readlane_d(v, 0), r1 = readlane_d(v, 16), r2 = readlane_d(v, 32), r3 = readlane_d(v, 48);
        const int lane = threadIdx.x & 63;
        v = g == 64 ? (r0 + r1) + (r2 + r3) : (lane < 32 ? r0 + r1 : r2 + r3);
    }
    return v;
}
// (value, index) maximum: larger value wins, equal values go to the smaller index.
__device__ __forceinline__ void argmax_step(float& v, int& i, float v2, int i2) {
    if (v2 > v || (v2 == v && i2 < i)) {
        v = v2;
        i = i2;
    }
}
__device__ __forceinline__ void group_argmax_dpp(float& v, int& i, int g) {
    if (g >= 2) argmax_step(v, i, dpp_f<kDppQuadXor1>(v), dpp_i<kDppQuadXor1>(i));
    if (g >= 4) argmax_step(v, i, dpp_f<kDppQuadXor2>(v), dpp_i<kDppQuadXor2>(i));
    if (g >= 8) argmax_step(v, i, dpp_f<kDppHalfMirror>(v), dpp_i<kDppHalfMirror>(i));
    if (g >= 16) argmax_step(v, i, dpp_f<kDppRowMirror>(v), dpp_i<kDppRowMirror>(i));
    if (g >= 32) {
        float rv[4];
        int ri[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            rv[k] = readlane_f(v, 16 * k);
            ri[k] = __builtin_amdgcn_readlane(i, 16 * k);
        }
        const int lane = threadIdx.x & 63;
        float a = rv[0], b = rv[2];
        int ai = ri[0], bi = ri[2];
        argmax_step(a, ai, rv[1], ri[1]);
        argmax_step(b, bi, rv[3], ri[3]);
        if (g == 64) {
            argmax_step(a, ai, b, bi);
            v = a;
            i = ai;
        } else {
            v = lane < 32 ? a : b;
            i = lane < 32 ? ai : bi;
        }
    }
}

}  // namespace tv
