/*
 * librkv_peaks: microbenchmarks of the peaks that the eviction kernels'
 * rooflines are quoted against (bf16 MFMA issue rate, HBM read and copy
 * bandwidth), for measurement only. Every pointer is a device pointer the
 * caller owns; each call launches one kernel on `stream` and returns the
 * hipError_t of the launch (0 = success, hipErrorInvalidValue for a rejected
 * argument, in which case nothing is launched).
 */
#ifndef RKV_PEAKS_H
#define RKV_PEAKS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* `blocks` work-groups of rkv_peak_threads_per_block() threads; every wave
 * runs `iters` rounds of four independent 32x32x16 bf16 MFMAs (32768 flop
 * each). out: float [blocks * rkv_peak_threads_per_block()], written. */
int rkv_peak_mfma_bf16(int32_t blocks, int32_t iters, float* out, void* stream);

/* The same with operands of random sign, exponent and mantissa (as keys drawn
 * from N(0, 1) have): the matrix units then draw more power and the chip
 * clocks lower, so this is the rate reachable on real keys. */
int rkv_peak_mfma_bf16_random(int32_t blocks, int32_t iters, float* out, void* stream);

/* Reads `bytes` (a multiple of 16, 16-byte aligned) of src with `blocks`
 * work-groups; out: uint32 [blocks], a fold of what was read. */
int rkv_peak_hbm_read(const void* src, size_t bytes, int32_t blocks, uint32_t* out, void* stream);

/* Copies `bytes` (a multiple of 16; both pointers 16-byte aligned, the
 * ranges disjoint) from src to dst with `blocks` work-groups. */
int rkv_peak_hbm_copy(const void* src, void* dst, size_t bytes, int32_t blocks, void* stream);

/* Threads per work-group of the kernels above. */
int rkv_peak_threads_per_block(void);

#ifdef __cplusplus
}
#endif
#endif /* RKV_PEAKS_H */
