// libtv_probe: the rates this device reaches on plain kernels, for the
// benchmark's roofline context (declared in include/tv_probe.h).  Not part of
// the verification path.
//  * stream_read: every workgroup reads a contiguous share of a buffer with
//    16-byte loads, eight in flight per thread, and keeps one sum per thread
//    (so the loads are live).  Its bytes per second is a streaming-read rate,
//    with ordinary loads or with loads marked non-temporal (which skip the
//    caches' retention and stream faster once the data cannot stay cached).
//  * mfma_loop: every wave runs four independent chains of
//    v_mfma_f32_32x32x16_bf16 (32 x 32 x 16 multiply-adds each) on register
//    operands; nothing else in the loop.  Its FLOP/s is the dense bf16 MFMA
//    rate the chip sustains at the clock it holds under that load.  With
//    constant operands few bits toggle and the clock stays near its maximum;
//    with random operands (a different pair for each chain, drawn from a
//    hash of the thread and workgroup) the power drawn is that of real data
//    and the clock the chip holds is lower.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tv_probe.h"

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kProbeThreads = 256;
constexpr int kChains = 4;

template <bool NT>
__device__ __forceinline__ f32x4 load16(const f32x4* p) {
    if constexpr (NT)
        return __builtin_nontemporal_load(p);
    else
        return *p;
}

template <bool NT>
__global__ __launch_bounds__(kProbeThreads) void stream_read_kernel(const f32x4* __restrict__ src, size_t n16,
                                                                    float* __restrict__ out) {
    // workgroup b reads the contiguous range [b * per, (b + 1) * per) of
    // 16-byte vectors, 8 * 256 of them (32 KB) per round, eight loads in
    // flight per thread (marked non-temporal with NT)
    constexpr int kRound = 8 * kProbeThreads;
    const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
    const size_t lo = min(n16, (size_t)blockIdx.x * per), hi = min(n16, lo + per);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    size_t i = lo + threadIdx.x;
    for (; i + 7 * kProbeThreads < hi; i += kRound) {
        f32x4 x[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) x[k] = load16<NT>(src + i + k * kProbeThreads);
#pragma unroll
        for (int k = 0; k < 8; ++k) acc += x[k];
    }
    for (; i < hi; i += kProbeThreads) acc += load16<NT>(src + i);
    out[(size_t)blockIdx.x * kProbeThreads + threadIdx.x] = acc[0] + acc[1] + acc[2] + acc[3];
}

__device__ __forceinline__ uint32_t mix32(uint32_t x) {
    // an integer hash (xor-shift-multiply rounds) for operand values
    x ^= x >> 16;
    x *= 0x7feb352du;
    x ^= x >> 15;
    x *= 0x846ca68bu;
    x ^= x >> 16;
    return x;
}

template <bool RANDOM>
__global__ __launch_bounds__(kProbeThreads) void mfma_loop_kernel(int iters, float* __restrict__ out) {
    const int t = threadIdx.x;
    bf16x8 a[kChains], b[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c)
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            if (RANDOM) {
                // values in [-2, 2): every mantissa bit of the bf16 varies
                const uint32_t h = mix32((uint32_t)(t * 131 + blockIdx.x * 7919 + c * 17 + k));
                a[c][k] = (__bf16)((float)((int)(h & 0xffff) - 32768) * (1.f / 16384.f));
                b[c][k] = (__bf16)((float)((int)(h >> 16) - 32768) * (1.f / 16384.f));
            } else {
                a[c][k] = (__bf16)(0.001f * (float)((t + k) & 15));
                b[c][k] = (__bf16)(0.002f * (float)((t * 3 + k) & 15));
            }
        }
    f32x16 acc[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c)
#pragma unroll
        for (int k = 0; k < 16; ++k) acc[c][k] = 0.f;
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int c = 0; c < kChains; ++c)
            acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[c], b[(c + 1) % kChains], acc[c], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < kChains; ++c)
#pragma unroll
        for (int k = 0; k < 16; ++k) s += acc[c][k];
    out[(size_t)blockIdx.x * kProbeThreads + t] = s;
}

}  // namespace

extern "C" int tv_probe_stream_read(const void* src, size_t bytes, int nontemporal, float* out, int nblocks,
                                    void* stream) {
    if (!src || !out || nblocks < 1 || bytes < 16 || (uintptr_t)src % 16 != 0) return -1;
    if (nontemporal)
        hipLaunchKernelGGL(stream_read_kernel<true>, dim3(nblocks), dim3(kProbeThreads), 0, (hipStream_t)stream,
                           static_cast<const f32x4*>(src), bytes / 16, out);
    else
        hipLaunchKernelGGL(stream_read_kernel<false>, dim3(nblocks), dim3(kProbeThreads), 0, (hipStream_t)stream,
                           static_cast<const f32x4*>(src), bytes / 16, out);
    return hipGetLastError() == hipSuccess ? 0 : -5;
}

extern "C" int tv_probe_mfma_loop(int nblocks, int iters, int random_operands, float* out, void* stream) {
    if (!out || nblocks < 1 || iters < 1) return -1;
    if (random_operands)
        hipLaunchKernelGGL(mfma_loop_kernel<true>, dim3(nblocks), dim3(kProbeThreads), 0, (hipStream_t)stream, iters,
                           out);
    else
        hipLaunchKernelGGL(mfma_loop_kernel<false>, dim3(nblocks), dim3(kProbeThreads), 0, (hipStream_t)stream, iters,
                           out);
    return hipGetLastError() == hipSuccess ? 0 : -5;
}

extern "C" double tv_probe_mfma_loop_flops(int nblocks, int iters) {
    // 2 * 32 * 32 * 16 per MFMA, kChains per iteration, kProbeThreads / 64 waves per workgroup
    return 2.0 * 32 * 32 * 16 * kChains * (double)iters * (kProbeThreads / 64) * (double)nblocks;
}
