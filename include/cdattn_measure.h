/*
 * cdattn_measure.h -- measurement helper exported by libcdattn.so.  Not part
 * of the method: it gives the streaming-read ceiling that the decode's
 * bandwidth on compressed bytes is reported against, beside the HBM peak.
 */
#ifndef CDATTN_MEASURE_H
#define CDATTN_MEASURE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * codec_measure_read -- read `bytes` of device memory at `src` once, with
 * 16-byte loads spread over `workgroups` workgroups of 256 threads (a
 * grid-stride pattern, sixteen loads requested together per thread), and
 * write one XOR of the data per workgroup to sink[0 .. workgroups-1] so that
 * no load is dropped.  Enqueued on `stream`; allocates nothing.
 *   src         device, 16-byte aligned; bytes a positive multiple of 16, at
 *               most 2^31.
 *   sink        device, at least `workgroups` uint32 words.
 *   workgroups  1 .. 65536.
 * Returns 0 (CODEC_OK), 1 (CODEC_ERR_NULL), 2 (CODEC_ERR_SHAPE: alignment,
 * size or workgroup count) or 8 (CODEC_ERR_HIP: launch failure); every check
 * runs before the launch.
 */
int codec_measure_read(const void *src, size_t bytes, uint32_t *sink, int32_t workgroups, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* CDATTN_MEASURE_H */
