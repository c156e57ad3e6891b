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

/*
 * codec_timeline_set -- exported only by the measurement build (compiled with
 * CDATTN_TIMELINE: python -m compressed_domain_attention_amd.build --timeline,
 * into compressed_domain_attention_amd/timeline/).  Every later decode launch
 * writes, for each wave, eight uint64 stamps of the 100 MHz clock
 * (s_memrealtime) to buf[((workgroup * 8 + wave) * 8 + phase)], workgroup =
 * the linear workgroup index, phase 0 start, 1 query converted, 2 raw tail
 * done, 3 tile loop done, 4 waves merged, 5 partial published, 6 arrival
 * counted, 7 output written (0: phase not reached).  Waves past `bytes` write
 * nothing.  buf is a device pointer owned by the caller; NULL stops the
 * stamps.  Returns 0.
 */
int codec_timeline_set(void *buf, size_t bytes);

#ifdef __cplusplus
}
#endif
#endif /* CDATTN_MEASURE_H */
