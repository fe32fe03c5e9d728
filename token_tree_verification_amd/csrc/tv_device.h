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

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

}  // namespace tv
