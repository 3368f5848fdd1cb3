/* Measurement library libtafloor.so: not part of the tree-attention path.
 *
 * ta_floor_read streams `bytes` from device memory at `src` and does nothing
 * else, so its time per launch is the floor for any kernel that has to read
 * the same bytes once (the benchmark's floor mode times it beside the
 * attention kernel over the same algorithmic bytes); ta_floor_gather (below)
 * does the same for a list of tiles, the paged layout of a KV cache.
 *
 *   src      device pointer, 16-byte aligned; read only.
 *   bytes    a positive multiple of 16.
 *   grid     workgroups, 1 .. 65536; workgroup i reads the i-th contiguous
 *            share of ceil(bytes / 16 / grid) 16-byte words (the last shares
 *            may be short or empty).
 *   threads  threads per workgroup, a multiple of 64 in 64 .. 512.
 *   loads    16-byte loads in flight per thread: 2, 4 or 8.
 *   sink     device pointer to `grid` 32-bit words, owned by the caller;
 *            word i receives the XOR of every 32-bit word of share i (0 for an
 *            empty share).
 *   stream   HIP stream the kernel is queued on; the call does not wait.
 *
 * Returns 0, TA_FLOOR_BAD_ARGS before anything is queued, or
 * TA_FLOOR_LAUNCH_FAILED if the launch itself failed.
 */
#ifndef TA_FLOOR_H
#define TA_FLOOR_H

#include <hip/hip_runtime.h>
#include <stddef.h>

#define TA_FLOOR_BAD_ARGS 1
#define TA_FLOOR_LAUNCH_FAILED 2

#ifdef __cplusplus
extern "C" {
#endif

int ta_floor_read(const void* src, size_t bytes, int grid, int threads, int loads, unsigned* sink,
                  hipStream_t stream);

/* ta_floor_gather reads `ntiles` tiles of `tile_bytes` each (a positive
 * multiple of 16, at most 16 MiB), tile k at byte offset tile_offsets[k] from
 * `base` (device pointers; base and every offset 16-byte aligned, every tile
 * inside the caller's allocation), the way the attention kernel reads paged
 * K/V tiles.  Workgroup i takes tiles [i * per, (i + 1) * per), per =
 * ceil(ntiles / grid) <= 4096, in list order; sink word i receives the XOR of
 * every 32-bit word of its tiles.  grid, threads, loads and the return codes
 * as ta_floor_read. */
int ta_floor_gather(const void* base, const long long* tile_offsets, int ntiles, size_t tile_bytes,
                    int grid, int threads, int loads, unsigned* sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* TA_FLOOR_H */
