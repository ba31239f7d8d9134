/*
 * dwprobe.h -- C ABI of the HBM streaming probe (measurement only).
 *
 * The roofline framing of the reson8 wiki ("GPU inference for speech",
 * "Where the time goes") bounds a memory-bound kernel by the bytes it must
 * move.  What a plain kernel actually reaches on a given part, for a given
 * number of bytes, is below the 8 TB/s peak and depends on the size of the
 * transfer.  This probe moves an exact number of bytes with the simplest
 * possible streaming kernel, so that a convolution kernel can be compared
 * with a copy of its own read and write bytes, timed the same way.
 *
 * It is not part of the convolution path and computes nothing the pages
 * define.
 */
#ifndef DWPROBE_H
#define DWPROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * dw_probe_stream -- read read_bytes from src and write write_bytes to dst.
 *
 * One 16-byte access per thread, 256 threads (4 KiB) per workgroup, one
 * workgroup per 4 KiB of the larger of the two sizes; a thread that has both
 * a read and a write stores what it read, so the work cannot be skipped.
 * policy selects the cache-policy bits of the loads / stores:
 *   0  default / default
 *   1  non-temporal / non-temporal
 *   2  non-temporal / non-temporal with the sc1 bit (the fastest copy measured)
 * src and dst are device pointers, 16-byte aligned, owned by the caller, and
 * must not overlap; sizes are rounded down to a multiple of 16 bytes.  The
 * work is enqueued on `stream` (a hipStream_t; NULL = default stream).
 * Returns 0, -1 for an invalid argument (NULL with a non-zero size, a
 * misaligned pointer, a negative size, an unknown policy, more than 2^42
 * bytes), or -4 if the launch was rejected.
 */
int dw_probe_stream(const void *src, void *dst, int64_t read_bytes, int64_t write_bytes, int policy,
                    void *stream);

#ifdef __cplusplus
}
#endif

#endif /* DWPROBE_H */
