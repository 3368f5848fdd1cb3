// tree_attn_verify_noalloc: the fused verify for callers that cannot allocate
// device memory (code under HIP-graph capture, tight serving loops, harnesses
// that forbid hipMalloc).  Its workspace is a static device array of this
// file, one per GPU, held until the process ends; the call allocates nothing.
//
// Included at the end of ta_api.hip (one translation unit), after the helpers
// it shares with tree_attn_verify.

namespace ta {
namespace {

// Size of the static workspace: the header and the two counter regions
// (about 1.3 MB), the rest for chunk partials.  Enough for one-sequence
// verifies up to 64K prefix tokens and for batches whose items fit one round
// of workgroups; larger shapes are refused with TA_ERR_SCRATCH.
constexpr size_t kScratchBytes = size_t(32) << 20;
constexpr int kMaxDevices = 64;

}  // namespace
}  // namespace ta

// The workspace of tree_attn_verify_noalloc.  In host code this name is only
// a stand-in for the device symbol: kernels get its device address, taken
// once per device with hipGetSymbolAddress, never the name itself.
static __device__ __align__(256) unsigned char scratch[ta::kScratchBytes];

namespace ta {
namespace {

// After the verify kernel, on the same stream: report the call's device error
// into *status (when given) and clear it.  A call that raised an error may
// have left arrival counters or the ticket counter set; they are cleared
// then, so that the next call finds them at zero, as a call that completes
// without an error leaves them.  One workgroup.
__global__ void __launch_bounds__(256) scratch_epilogue_kernel(WsHeader* hdr, uint4* counters,
                                                               size_t n16, int32_t* status) {
  __shared__ int err_sh;
  if (threadIdx.x == 0) err_sh = __hip_atomic_load(&hdr->error, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const int err = err_sh;
  if (err != 0) {
    for (size_t i = threadIdx.x; i < n16; i += blockDim.x) counters[i] = make_uint4(0, 0, 0, 0);
    if (threadIdx.x == 0) {
      hdr->done = 0;
      hdr->ticket = 0;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    if (status) *status = err;
    hdr->error = 0;
  }
}

std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of the current device's copy of `scratch`, taken with
// hipGetSymbolAddress on the first call on that device and kept.
int scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return kErrHip;
  if (dev < 0 || dev >= kMaxDevices) return kErrUnsupported;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return kErrHip;
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return kOk;
}

}  // namespace
}  // namespace ta

extern "C" ta_status tree_attn_verify_noalloc(const ta_shape* shape, const void* q,
                                              const void* k_cache, const void* v_cache,
                                              const int32_t* block_table,
                                              const int32_t* prefix_lens, const void* k_tree,
                                              const void* v_tree, const int32_t* parents,
                                              const int32_t* tree_offsets, void* out,
                                              float* lse_out, int32_t* device_status,
                                              hipStream_t stream) {
  using namespace ta;
  int st = check_shape(shape);
  if (st != kOk) return static_cast<ta_status>(st);
  const WsLayout L = layout_for(shape, choose_chunk(shape, true), auto_cap(shape, true));
  if (L.total > kScratchBytes) return TA_ERR_SCRATCH;
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != kOk) return static_cast<ta_status>(st);
  st = fused_verify(shape, q, k_cache, v_cache, block_table, prefix_lens, k_tree, v_tree, parents,
                    tree_offsets, out, lse_out, ws, kScratchBytes, stream);
  if (st != kOk) return static_cast<ta_status>(st);
  char* w = static_cast<char*>(ws);
  const size_t counter_bytes = L.partial_off - L.arrive_off;
  hipLaunchKernelGGL(scratch_epilogue_kernel, dim3(1), dim3(256), 0, stream,
                     reinterpret_cast<WsHeader*>(w), reinterpret_cast<uint4*>(w + L.arrive_off),
                     counter_bytes / 16, device_status);
  return static_cast<ta_status>(launch_status());
}
