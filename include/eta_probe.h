/*
 * eta_probe.h -- a measurement aid beside the ETA library, not part of the
 * method: a plain streaming read of a device buffer with the same 16-byte
 * loads the ETA kernels use, so a benchmark can state, in its own process and
 * machine state, the read bandwidth the HBM actually sustains next to the
 * kernels' achieved figures (libeta_probe.so, built with libeta.so).
 *
 * eta_probe_stream_read: every workgroup of 256 threads reads one contiguous
 * 32 KiB chunk of `buf` (each thread eight 16-byte loads, consecutive threads
 * on consecutive 16 bytes), with the non-temporal hint when `nontemporal` is
 * non-zero, and folds the words into a register. `sink` (device, at least 256
 * uint32) is written only if that fold hits one fixed 32-bit value, so the
 * loads cannot be dropped and, in practice, nothing is written.
 * buf: device pointer, 16-byte aligned; bytes: a non-zero multiple of 32768
 * (at most 2^31 - 1 chunks). Enqueues one launch on `stream` and returns 0;
 * -1 for invalid arguments (nothing enqueued), -4 if the launch fails.
 *
 * eta_probe_pair_read: the decode attention's access pattern stripped of its
 * arithmetic: workgroup c of 256 threads reads 16 KiB chunk c of `a` and chunk c
 * of `b` together (non-temporal 16-byte loads), as the attention reads the K and
 * V rows of one block, and folds them like eta_probe_stream_read. Run on the
 * attention's own K and V buffers it gives the rate their physical placement
 * allows: two buffers read together can stream several percent slower or
 * faster depending on where the driver placed them, which one buffer read alone
 * does not show. a, b: device pointers, 16-byte aligned, each at least `bytes`
 * long; bytes: a non-zero multiple of 16384 (at most 2^31 - 1 chunks); sink as
 * above. Enqueues one launch on `stream` and returns 0; -1 for invalid
 * arguments (nothing enqueued), -4 if the launch fails.
 */
#ifndef ETA_PROBE_H
#define ETA_PROBE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

int eta_probe_stream_read(const void *buf, size_t bytes, int nontemporal, uint32_t *sink,
                          hipStream_t stream);
int eta_probe_pair_read(const void *a, const void *b, size_t bytes, uint32_t *sink,
                        hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* ETA_PROBE_H */
