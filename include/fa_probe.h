/*
 * fa_probe.h — measurement aid, not part of the attention path.
 *
 * The decode kernels are bound by HBM bandwidth, and the bandwidth a read of
 * a given size can reach on the device (launch, ramp and tail included) is
 * well below the data-sheet peak for small reads.  This entry point runs a
 * plain streaming-read kernel over a device buffer so that the decode rates
 * can be set beside the empirical ceiling for the same number of bytes.
 */
#ifndef FA_PROBE_H
#define FA_PROBE_H

#include <stddef.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Reads `bytes` bytes at `src` (device, 16-byte aligned, bytes a positive
 * multiple of 16) with non-temporal 16-byte loads, 256 KB per 256-thread workgroup, eight
 * loads in flight per lane, and keeps nothing: `sink` (device, >= 4 bytes,
 * owned by the caller) is written only if the XOR of the data equals a fixed
 * constant, so the loads cannot be dropped.  Enqueued on `stream`; returns
 * FA_OK (0), FA_ERR_INVALID_ARG (-1) for a null or misaligned pointer or a
 * bad size, or FA_ERR_HIP (-4) if the launch fails.
 */
int fa_probe_read(const void* src, size_t bytes, unsigned* sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_PROBE_H */
