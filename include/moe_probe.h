/* moe_probe.h -- measurement helper, not part of the MoE layer's ABI.
 *
 * libmoe_probe.so reads a device buffer once with a plain streaming kernel:
 * the read bandwidth it reaches is the ceiling the benchmark compares the
 * layer's weight-streaming kernels with (their roofline peak stays the HBM
 * specification, 8 TB/s on MI355X).
 */
#ifndef MOE_PROBE_H
#define MOE_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Enqueue one read of bytes bytes at buf (device memory, 16-byte aligned) on
 * hip_stream (a hipStream_t; NULL = the null stream) with grid workgroups of
 * 256 threads, each reading its own contiguous share.  bytes must be a
 * multiple of grid * 65536.  sink is a device buffer of 256 uint32 that the
 * kernel may write (its contents are meaningless).  Returns 0 once the
 * kernel is queued, -1 for a bad argument (nothing queued), -3 if the launch
 * failed.  The caller owns both buffers. */
int32_t moe_probe_stream_read(const void* buf, int64_t bytes, int32_t grid, void* hip_stream,
                              uint32_t* sink);

#ifdef __cplusplus
}
#endif

#endif /* MOE_PROBE_H */
