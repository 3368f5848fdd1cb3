// A measurement kernel, not part of the attention path: it streams a device
// buffer from HBM and nothing else, so that its time per launch is the floor
// for any launch that has to read the same bytes once.  Each workgroup reads
// one contiguous share with 16-byte loads, `loads` of them in flight per
// thread, folds the words with XOR (so the loads cannot be dropped) and
// writes one word per workgroup.
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

}  // namespace

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
