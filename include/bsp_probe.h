/*
 * bsp_probe.h -- C ABI of the streaming-read probe (libbsp_probe.so), a
 * measurement aid kept apart from the SpMM library: it reports how fast one
 * kernel launch can read a given byte count from HBM on this GPU, the
 * achievable ceiling the SpMM's bandwidth is set against (the bandwidth
 * roofline of SPDP, Sec. 3.1, Eq. 1-2, taken with the measured rather than
 * the vendor peak).
 */
#ifndef BSP_PROBE_H
#define BSP_PROBE_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * bsp_probe_read -- one launch that reads `bytes` bytes at `buf` (DEVICE) in
 * 16-byte granules and writes one XOR fold per wavefront to `sink` (DEVICE,
 * bsp_probe_sink_words(grid, block) uint32 words). Asynchronous on `stream`.
 *   bytes  a positive multiple of 16, below 2^32.
 *   mode   0: loads into registers; 1: the same, non-temporal;
 *          2: direct-to-LDS loads (16 B per lane, non-temporal).
 *   grid, block  launch shape (block a multiple of 64, at most 1024).
 * Returns 0, 1 for an invalid argument (nothing launched), 5 for a launch error.
 */
int bsp_probe_read(const void *buf, int64_t bytes, uint32_t *sink, int mode, int grid, int block,
                   hipStream_t stream);

/* Number of uint32 words bsp_probe_read writes to sink for a launch shape. */
int64_t bsp_probe_sink_words(int grid, int block);

#ifdef __cplusplus
}
#endif

#endif /* BSP_PROBE_H */
