/*
 * moelora_probe.h — measurement probes of libmoelora: the on-box ceilings that the layer's
 * throughput is compared with, next to the MI355X's published peaks (8 TB/s of HBM3E, 2.5
 * PFLOP/s of dense bf16 MFMA). They are not steps of the layer and no page defines them: the
 * layer is HBM-bound at decode sizes and MFMA-bound at prefill sizes, and a fraction of a peak
 * the part cannot sustain says less than one of what it does sustain on this machine.
 *
 * Both probes enqueue one kernel on `stream` (a hipStream_t) and return MOELORA_OK, or a
 * negative MOELORA_E* code before any device work (moelora.h). The caller times the launch
 * (events on the same stream) and owns every buffer.
 */
#ifndef MOELORA_PROBE_H
#define MOELORA_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Streaming read of `bytes` bytes at src (device memory, 16-byte aligned, bytes a positive
 * multiple of 16): 2048 workgroups of 256 threads read it once in 16-byte loads, eight in
 * flight per thread, and each thread writes one 32-bit word derived from what it read to
 * sink[2048 * 256] (so the loads cannot be dropped). Bytes moved: `bytes` read + 2 MiB
 * written. */
int moe_lora_probe_read(const void *src, size_t bytes, uint32_t *sink, void *stream);

/* MFMA loop: n_workgroups workgroups of four wavefronts, each wavefront issuing iters x 8
 * independent 32x32x16 bf16 MFMAs (fp32 accumulate) on register operands of random sign and
 * mantissa (magnitudes in [0.5, 2)), then writing one float per lane to sink[n_workgroups *
 * 256]. Work: n_workgroups * 4 * iters * 8 * 32768 flops. iters >= 1, n_workgroups >= 1. */
int moe_lora_probe_mfma(int32_t iters, int32_t n_workgroups, float *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MOELORA_PROBE_H */
