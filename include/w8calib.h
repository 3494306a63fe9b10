/* w8calib.h -- measurement helpers for the W8A16 decode library (libw8calib.so).
 *
 * Not part of the decode path: two calibration kernels whose rates frame the
 * roofline figures that bench.py reports beside the projection.
 *   - w8c_stream_read: the practical HBM read ceiling of one launch -- a bare
 *     streaming read (16-byte nontemporal loads, 8 in flight per thread,
 *     512 threads per workgroup, each workgroup one contiguous chunk).
 *   - w8c_mfma_bf16: the dense bf16 matrix-core rate -- every wave issues
 *     independent v_mfma_f32_32x32x16_bf16 chains with no memory traffic.
 *
 * Conventions are those of w8inv.h: device pointers owned by the caller, work
 * enqueued on `stream` (a hipStream_t, NULL = the default stream), nothing
 * allocated, freed or synchronised; the return value is a w8i_status code of
 * the host-side validation and launch.
 */
#ifndef W8CALIB_H
#define W8CALIB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Read `bytes` bytes of `buf` once (bytes a positive multiple of 16, buf
 * 16-byte aligned) with `workgroups` workgroups (1..65536), each taking one
 * contiguous chunk.  `sink` (device, at least workgroups * 2048 bytes) keeps
 * the loads alive: it is written only if a lane's XOR of everything it read
 * equals a fixed constant, so its contents are unspecified.
 * W8I_ENULL, W8I_ESHAPE, W8I_EALIGN, W8I_EWORKSPACE (sink too small), W8I_EHIP. */
int w8c_stream_read(const void *buf, int64_t bytes, int32_t workgroups, void *sink, size_t sink_bytes,
                    void *stream);

/* Issue `workgroups` (1..65536) workgroups of 4 waves; each wave runs 4
 * independent chains of `iters` (1..2^20) v_mfma_f32_32x32x16_bf16, so one
 * call executes workgroups * 4 * 4 * iters * 32768 flops.  `sink` (device,
 * at least workgroups * 1024 bytes) is written only if a lane's accumulators
 * sum to a fixed constant.  Errors as above. */
int w8c_mfma_bf16(int32_t workgroups, int32_t iters, void *sink, size_t sink_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* W8CALIB_H */
