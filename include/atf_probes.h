/*
 * atf_probes.h -- C ABI of librfw_probes.so: two microbenchmarks that measure
 * what one MI355X (gfx950) actually sustains, so that the attention kernels'
 * roofline fractions can be read against attainable peaks as well as the
 * published ones (dense bf16 MFMA 2.5 PFLOP/s, HBM3E 8 TB/s).  They are
 * measurement tools, not part of the attention path.
 *
 * Both calls only queue work on `stream` (hipStream_t; NULL = default); the
 * caller times them (e.g. with events) and owns every buffer.  Return value:
 * 0 on success, 1 for a bad argument (checked on the host, nothing queued),
 * 4 if the launch failed.
 */
#ifndef ATF_PROBES_H
#define ATF_PROBES_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t *atf_probe_stream_t; /* same object as hipStream_t */

/*
 * Dense bf16 MFMA throughput: n_wg workgroups of 256 threads (4 waves); each
 * wave issues `iters` rounds of 8 independent v_mfma_f32_32x32x16_bf16 (32768
 * flops each).  Total flops = n_wg * 4 * 8 * iters * 32768.
 *   operands: DEVICE pointer to >= 64 bytes (the A and B fragments, any bits)
 *   sink:     DEVICE pointer to n_wg * 256 floats (results, keeps the work live)
 * n_wg >= 1, iters >= 1.
 */
int atf_probe_mfma_bf16(const void *operands, float *sink, int32_t n_wg, int32_t iters,
                        atf_probe_stream_t stream);

/*
 * HBM read bandwidth: n_wg workgroups of 256 threads stream `bytes` bytes of
 * `buf` once with 16-byte loads (grid-stride, 4 loads in flight per thread)
 * and fold them into sink[n_wg * 256] (XOR, keeps the loads live).
 *   buf:  DEVICE pointer, 16-byte aligned; bytes a positive multiple of 64 * 256 * 16
 *   sink: DEVICE pointer to n_wg * 256 uint32
 */
int atf_probe_hbm_read(const void *buf, size_t bytes, uint32_t *sink, int32_t n_wg,
                       atf_probe_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* ATF_PROBES_H */
