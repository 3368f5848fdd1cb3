// Measurement kernels, not part of the attention path: they stream device
// memory from HBM and nothing else, so that their time per launch is the floor
// for any launch that has to read the same bytes once.  ta_floor_read reads a
// buffer (each workgroup one contiguous share); ta_floor_gather reads a list
// of equal tiles at arbitrary offsets, as the attention kernel reads the
// paged KV tiles.  16-byte loads, `loads` of them in flight per thread, the
// words folded with XOR (so the loads cannot be dropped), one word written per
// workgroup.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "ta_floor.h"

namespace {

template <int U>
__global__ void __launch_bounds__(512) stream_read_kernel(const uint4* __restrict__ src, long n16,
                                                         long per_wg, unsigned* __restrict__ sink) {
  __shared__ unsigned wave_fold[8];
  const long begin = long(blockIdx.x) * per_wg;
  const long end = begin + per_wg < n16 ? begin + per_wg : n16;
  const long step = long(blockDim.x) * U;
  unsigned acc = 0;
  for (long i = begin + threadIdx.x; i < end; i += step) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const long j = i + long(u) * blockDim.x;
      v[u] = j < end ? src[j] : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o);
  if ((threadIdx.x & 63) == 0) wave_fold[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned a = 0;
    for (unsigned w = 0; w < blockDim.x / 64; ++w) a ^= wave_fold[w];
    sink[blockIdx.x] = a;
  }
}

// Gather form: workgroup i reads tiles [i * per, (i + 1) * per) of a list of
// equal tiles at byte offsets from `base` (the list staged in LDS first), in
// list order, 16-byte loads, U in flight per thread.
constexpr int kMaxTilesPerWg = 4096;

template <int U>
__global__ void __launch_bounds__(512) gather_read_kernel(const unsigned char* __restrict__ base,
                                                         const long long* __restrict__ tile_off,
                                                         int ntiles, int per_wg, int wshift,
                                                         unsigned* __restrict__ sink) {
  __shared__ long long offs[kMaxTilesPerWg];
  __shared__ unsigned wave_fold[8];
  const int t0 = int(blockIdx.x) * per_wg;
  const int nt = max(0, min(per_wg, ntiles - t0));
  for (int i = threadIdx.x; i < nt; i += blockDim.x) offs[i] = tile_off[t0 + i];
  __syncthreads();
  const long nw = long(nt) << wshift;
  const long wmask = (1L << wshift) - 1;
  const long step = long(blockDim.x) * U;
  unsigned acc = 0;
  for (long i = threadIdx.x; i < nw; i += step) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const long j = i + long(u) * blockDim.x;
      v[u] = j < nw ? *reinterpret_cast<const uint4*>(base + offs[j >> wshift] + 16 * (j & wmask))
                    : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o);
  if ((threadIdx.x & 63) == 0) wave_fold[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned a = 0;
    for (unsigned w = 0; w < blockDim.x / 64; ++w) a ^= wave_fold[w];
    sink[blockIdx.x] = a;
  }
}

}  // namespace

extern "C" int ta_floor_gather(const void* base, const long long* tile_offsets, int ntiles,
                               size_t tile_bytes, int grid, int threads, int loads, unsigned* sink,
                               hipStream_t stream) {
  if (base == nullptr || tile_offsets == nullptr || sink == nullptr || ntiles < 1)
    return TA_FLOOR_BAD_ARGS;
  if (reinterpret_cast<uintptr_t>(base) % 16 != 0 || tile_bytes < 16 || tile_bytes % 16 != 0 ||
      tile_bytes / 16 > size_t(1) << 20 || ((tile_bytes / 16) & (tile_bytes / 16 - 1)) != 0)
    return TA_FLOOR_BAD_ARGS;
  if (grid < 1 || grid > 65536 || threads < 64 || threads > 512 || threads % 64 != 0)
    return TA_FLOOR_BAD_ARGS;
  const int per_wg = (ntiles + grid - 1) / grid;
  if (per_wg > kMaxTilesPerWg) return TA_FLOOR_BAD_ARGS;
  const auto* b = static_cast<const unsigned char*>(base);
  int wshift = 0;
  while ((size_t(1) << wshift) < tile_bytes / 16) ++wshift;
  switch (loads) {
    case 2: gather_read_kernel<2><<<grid, threads, 0, stream>>>(b, tile_offsets, ntiles, per_wg, wshift, sink); break;
    case 4: gather_read_kernel<4><<<grid, threads, 0, stream>>>(b, tile_offsets, ntiles, per_wg, wshift, sink); break;
    case 8: gather_read_kernel<8><<<grid, threads, 0, stream>>>(b, tile_offsets, ntiles, per_wg, wshift, sink); break;
    default: return TA_FLOOR_BAD_ARGS;
  }
  return hipGetLastError() == hipSuccess ? 0 : TA_FLOOR_LAUNCH_FAILED;
}

extern "C" int ta_floor_read(const void* src, size_t bytes, int grid, int threads, int loads,
                             unsigned* sink, hipStream_t stream) {
  if (src == nullptr || sink == nullptr || bytes == 0 || bytes % 16 != 0) return TA_FLOOR_BAD_ARGS;
  if (reinterpret_cast<uintptr_t>(src) % 16 != 0) return TA_FLOOR_BAD_ARGS;
  if (grid < 1 || grid > 65536 || threads < 64 || threads > 512 || threads % 64 != 0)
    return TA_FLOOR_BAD_ARGS;
  const long n16 = long(bytes / 16);
  const long per_wg = (n16 + grid - 1) / grid;
  const uint4* p = static_cast<const uint4*>(src);
  switch (loads) {
    case 2: stream_read_kernel<2><<<grid, threads, 0, stream>>>(p, n16, per_wg, sink); break;
    case 4: stream_read_kernel<4><<<grid, threads, 0, stream>>>(p, n16, per_wg, sink); break;
    case 8: stream_read_kernel<8><<<grid, threads, 0, stream>>>(p, n16, per_wg, sink); break;
    default: return TA_FLOOR_BAD_ARGS;
  }
  return hipGetLastError() == hipSuccess ? 0 : TA_FLOOR_LAUNCH_FAILED;
}
