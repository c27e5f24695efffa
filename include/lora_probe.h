/*
 * lora_probe.h — measurement probes for AMD MI355X (gfx950).  Not part of the
 * projection: they measure what this chip sustains, so that a kernel's
 * throughput can be stated as a fraction of a measured peak beside the
 * published one.
 *
 *   lora_probe_mfma_bf16  dense bf16 MFMA with no memory traffic: every wave
 *                         runs `iters` rounds of four independent chains of
 *                         v_mfma_f32_32x32x16_bf16 (32 x 32 x 16 products).
 *                         *flop receives the floating-point operations it
 *                         performs (2 per multiply-add).  sink: device, at
 *                         least 1024 floats, written only in a case that does
 *                         not occur (it keeps the work from being removed).
 *   lora_probe_read       a plain streaming read of `bytes` bytes of device
 *                         memory at `src` (16-byte nontemporal loads,
 *                         coalesced, four in flight per thread, 8192
 *                         workgroups); sink as above.
 *
 * Both launch one kernel on `stream` and return without waiting; time them
 * with events on that stream.  Errors: iters outside 1..2^24, bytes not a
 * positive multiple of 16 below 2^40, a null or unaligned pointer give
 * LORA_EINVAL; a launch failure gives LORA_EHIP.
 */
#ifndef LORA_PROBE_H
#define LORA_PROBE_H

#include "lora_proj.h"

#ifdef __cplusplus
extern "C" {
#endif

lora_status lora_probe_mfma_bf16(int32_t iters, float* sink, double* flop, hipStream_t stream);
lora_status lora_probe_read(const void* src, size_t bytes, float* sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LORA_PROBE_H */
