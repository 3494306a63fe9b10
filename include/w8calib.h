/* w8calib.h -- measurement helpers for the W8A16 decode library (libw8calib.so).
 *
 * Not part of the decode path: two calibration kernels whose rates frame the
 * roofline figures that bench.py reports beside the projection.
 *   - w8c_stream_read: the practical HBM read ceiling of one launch -- a bare
 *     streaming read (16-byte nontemporal loads, 8 in flight per thread,
 *     512 threads per workgroup, each workgroup one contiguous chunk).
 *   - w8c_strip_read: the read ceiling in the persistent projection's own
 *     decomposition over the packed layout (tiles of 8 strips, one wave per
 *     strip, 2 KB code blocks and 128-byte scale lines in order, 8 blocks in
 *     flight per wave).
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

/* Read `strips` x `pairs` blocks of 2048 bytes of `codes` (16-byte aligned) and 128 bytes of
 * `scales` (4-byte aligned) -- the packed layout's codes and scales of a projection of 32
 * strips rows and 64 pairs columns, strips * pairs * 2048 < 2^32 -- once, with `workgroups`
 * (1..65536) workgroups of 8 waves: workgroup b takes tiles b, b + workgroups, ... of 8 strips,
 * wave w strip w of its tile, each wave its strip's blocks in order.  `sink` as above.
 * W8I_ENULL, W8I_ESHAPE, W8I_EALIGN, W8I_EWORKSPACE, W8I_EHIP. */
int w8c_strip_read(const void *codes, const void *scales, int32_t strips, int32_t pairs, int32_t workgroups,
                   void *sink, size_t sink_bytes, void *stream);

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
