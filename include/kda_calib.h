/*
 * kda_calib.h — measured ceilings of the device, for the roofline figures.
 *
 * libkda_calib.so is measurement infrastructure beside libkda.so: the
 * benchmark times these kernels to set the measured ceilings it reports next
 * to the published peaks. Nothing on the gated delta rule path calls them.
 */
#ifndef KDA_CALIB_H
#define KDA_CALIB_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Enqueues an fp16 MFMA loop (v_mfma_f32_16x16x32_f16, fp32 accumulation) on
 * `hip_stream`: `blocks` workgroups of 256 threads, each wavefront running
 * `iters` iterations of 8 independent 16x16x32 products, then writing its
 * accumulators to `out` (device, 16-byte aligned, at least
 * blocks * 256 * 4 floats; caller-owned). Flops enqueued:
 * blocks * 4 * iters * 8 * 16384.
 * Returns 0, -1 for bad arguments, -5 for a HIP launch error. */
int kda_calib_mfma_f16(int32_t blocks, int32_t iters, float* out, void* hip_stream);

/* Enqueues a streaming copy of `n_vec` 16-byte vectors from `src` to `dst`
 * (device, 16-byte aligned, caller-owned, not overlapping): nontemporal
 * vector loads and stores, four per thread per step, grid-stride over
 * `blocks` workgroups of 256 threads. Bytes moved:
 * 16 * n_vec read plus 16 * n_vec written.
 * Returns 0, -1 for bad arguments, -5 for a HIP launch error. */
int kda_calib_copy(const void* src, void* dst, int64_t n_vec, int32_t blocks, void* hip_stream);

#ifdef __cplusplus
}
#endif
#endif /* KDA_CALIB_H */
