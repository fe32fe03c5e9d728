/*
 * libtv_probe -- rates the device reaches on plain kernels (gfx950).  C ABI.
 *
 * Measurement aids for the benchmark's roofline context; not part of the
 * verification path (libtv).  Pointers are DEVICE pointers; `stream` is a
 * hipStream_t passed as void*.  Calls only enqueue work.  Return 0 on
 * success, -1 for an invalid argument (nothing enqueued), -5 if the launch
 * failed.
 */
#ifndef TV_PROBE_H
#define TV_PROBE_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Streaming read of `bytes` (a multiple of 16 is read; `src` 16-byte aligned)
 * by `nblocks` workgroups of 256 threads with 16-byte loads, ordinary ones or
 * (nontemporal != 0) ones marked non-temporal.  Writes one float per thread to
 * out[nblocks * 256] so that the loads are live.  Bytes read per launch: bytes
 * rounded down to 16. */
int tv_probe_stream_read(const void* src, size_t bytes, int nontemporal, float* out, int nblocks, void* stream);

/* `nblocks` workgroups of four waves; each wave issues `iters` rounds of four
 * independent v_mfma_f32_32x32x16_bf16 on register operands: constant ones
 * (random_operands == 0: few bits toggle, the clock stays near its maximum)
 * or random ones, a different pair per chain (the power drawn by real data,
 * at the lower clock the chip then holds).  Writes one float per thread to
 * out[nblocks * 256].  FLOPs per launch: tv_probe_mfma_loop_flops(nblocks,
 * iters). */
int tv_probe_mfma_loop(int nblocks, int iters, int random_operands, float* out, void* stream);

/* 2 * 32 * 32 * 16 * 4 * iters * 4 * nblocks. */
double tv_probe_mfma_loop_flops(int nblocks, int iters);

#ifdef __cplusplus
}
#endif

#endif /* TV_PROBE_H */
