/*
 * mla_probe.h -- C ABI of libmla_probe: a streaming-read kernel that measures
 * the HBM read rate plain, well-formed loads reach on this GPU.  It is a
 * yardstick for the decode kernels' rates (the decode is bound by reading
 * the latent cache), not part of the attention path, and lives in a library
 * of its own.
 */
#ifndef MLA_PROBE_H
#define MLA_PROBE_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Bytes of device memory the probe's `sink` must hold. */
#define MLA_PROBE_SINK_BYTES 8192

/*
 * Reads every byte of buf[0 .. bytes) once: 512 workgroups of 256 threads,
 * each streaming one contiguous range with 16-byte loads, 16 in flight per
 * thread.  Folds what it read into one 32-bit word per wave, written to
 * sink (device memory of MLA_PROBE_SINK_BYTES, caller-owned; contents
 * meaningless).  Enqueued on `stream` (a hipStream_t, NULL = default);
 * time it with events on that stream.
 *
 * Returns 0 on success (bytes == 0 enqueues nothing), 1 if buf or sink is
 * NULL, 2 if bytes is not a multiple of 16, 4 if buf is not 16-byte
 * aligned, 6 if the launch failed.
 */
int mla_probe_read(const void* buf, size_t bytes, void* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_PROBE_H */
