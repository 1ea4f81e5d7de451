/* Measurement helper beside the decode library (librs_probe.so), not part of
 * the decode ABI: a read-only stream with the decode kernels' access pattern,
 * the reference for how much of the chip's read bandwidth a kernel that
 * streams such tiles can reach, and the same stream with a small write per
 * tile, which prices the output and append writes a decode step mixes into
 * its read stream. */
#ifndef RS_PROBE_H
#define RS_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Read `bytes` of device memory at `src` (16-byte aligned) as tiles of
 * threads x per_thread 16-byte non-temporal loads, one tile per workgroup of
 * `threads` threads; each workgroup writes the sum of its tile to
 * out[tile] (device float[bytes / tile bytes], caller-owned). Shapes offered:
 * 256 x 8 (32 KiB tiles, the decode kernels' state tile), 256 x 4 (16 KiB),
 * 128 x 16 (32 KiB). Returns 0 when launched on `stream` (a hipStream_t, may
 * be NULL); -1 bad pointer, -2 bytes not a positive multiple of the tile (or
 * too many tiles), -3 launch error, -4 shape not offered. Asynchronous. */
int32_t rs_probe_read(const void* src, float* out, uint64_t bytes, int32_t threads, int32_t per_thread,
                      void* stream);

/* The same tiled read of `bytes` at `src`; after its tile is summed, each
 * workgroup writes `write_bytes` bytes (a positive multiple of 16, at most
 * threads x 16) to dst + tile * write_bytes as 16-byte non-temporal stores
 * (device memory of bytes / tile bytes x write_bytes bytes, caller-owned,
 * 16-byte aligned; the values are sums, only the traffic matters). Same
 * shapes and return codes as rs_probe_read, plus -5 for a write size out of
 * range. Asynchronous. */
int32_t rs_probe_read_write(const void* src, void* dst, uint64_t bytes, int32_t threads, int32_t per_thread,
                            int32_t write_bytes, void* stream);

/* Variants of the read stream, for how far a tile stream can go on this chip
 * beyond the decode kernels' own scheme. Each reads `bytes` (a positive
 * multiple of its tile) at `src` (16-byte aligned) and writes one float per
 * tile to out[tile] (device float[bytes / tile bytes], caller-owned):
 *   RS_PROBE_REG_256X8        32 KiB tiles into registers, non-temporal loads
 *                             (the same stream as rs_probe_read at 256 x 8);
 *   RS_PROBE_PLAIN_256X8      the same with ordinary (cached) loads;
 *   RS_PROBE_REG_256X16       64 KiB tiles into registers;
 *   RS_PROBE_LDS_256X8        32 KiB tiles by 16-byte global-to-LDS loads;
 *   RS_PROBE_LDS_256X16       64 KiB tiles by 16-byte global-to-LDS loads;
 *   RS_PROBE_PERSISTENT_256X8 persistent workgroups, as many as fit on the
 *                             device at once, each looping over pairs of
 *                             32 KiB tiles with both tiles of a pair in flight
 *                             (bytes must be a multiple of 64 KiB).
 * Returns as rs_probe_read (-4: unknown variant). Asynchronous. */
#define RS_PROBE_REG_256X8 0
#define RS_PROBE_PLAIN_256X8 1
#define RS_PROBE_REG_256X16 2
#define RS_PROBE_LDS_256X8 3
#define RS_PROBE_LDS_256X16 4
#define RS_PROBE_PERSISTENT_256X8 5
int32_t rs_probe_read_variant(const void* src, float* out, uint64_t bytes, int32_t variant, void* stream);

#ifdef __cplusplus
}
#endif

#endif
