/*
 * sdpa_probe — streaming kernels used to calibrate the measurements of the
 * sdpa_math library on one MI355X (not part of the attention path).
 *
 * The benchmark reports an HBM roofline fraction against the chip's
 * published 8 TB/s, and the hardware write/fetch counters are scaled by what
 * they read for a transfer of known size. These two kernels provide those
 * references: a plain fill (write-only stream) and a plain copy (one read
 * and one write stream), both with 16-byte accesses per lane, fully
 * coalesced, grid-stride over the buffer. The cudnn-frontend pull request
 * "[SDPA] SM80 fwd: TemplateParams kernels, plan-time compile, sym_int THD
 * extents" describes reporting generation kernels as GB/s against memory
 * speed-of-light (merge-log notes on measurement); these kernels measure
 * that ceiling here.
 *
 * Pointers are device pointers, `bytes` a multiple of 16, `dst`/`src`
 * 16-byte aligned. Work is enqueued on `hip_stream` (a hipStream_t, NULL =
 * null stream) without synchronising. Returns 0, or a hipError_t value on a
 * launch error or bad argument (hipErrorInvalidValue).
 */
#ifndef SDPA_PROBE_H
#define SDPA_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int sdpa_probe_fill(void* dst, size_t bytes, uint32_t value, void* hip_stream);
int sdpa_probe_copy(void* dst, const void* src, size_t bytes, void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* SDPA_PROBE_H */
