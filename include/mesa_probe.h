/*
 * mesa_probe.h -- measurement kernels of libmesa (not part of the method).
 *
 * Kernels whose work is known exactly, used to measure the attainable peaks
 * of the GPU the library runs on, so that achieved rates can be stated both
 * against the datasheet peaks and against these measured ones.  Same
 * conventions as mesa.h: device pointers, asynchronous on `stream`, host-side
 * validation, a mesa_status result.
 */
#ifndef MESA_PROBE_H
#define MESA_PROBE_H

#include <stddef.h>
#include <stdint.h>

#include "mesa.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Register-resident MFMA loop: n_workgroups workgroups of 4 waves; every wave
 * issues iters x 8 independent v_mfma_f32_16x16x4_f32 (2048 flops each).
 * Total flops = n_workgroups * 4 * iters * 8 * 2048.  sink: n_workgroups * 256
 * floats, written (keeps the work observable).
 */
mesa_status mesa_probe_mfma_f32(int n_workgroups, int iters, float *sink, void *stream);

/*
 * Same with v_mfma_f32_16x16x32_bf16 (16384 flops each).
 * Total flops = n_workgroups * 4 * iters * 8 * 16384.
 */
mesa_status mesa_probe_mfma_bf16(int n_workgroups, int iters, float *sink, void *stream);

/*
 * Streaming copy of `bytes` (a multiple of 16) from src to dst, 16-byte
 * aligned, non-overlapping: reads `bytes` and writes `bytes` of HBM.
 */
mesa_status mesa_probe_copy(const void *src, void *dst, size_t bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MESA_PROBE_H */
