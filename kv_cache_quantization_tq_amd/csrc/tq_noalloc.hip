/*
 * Library-held decode workspace for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops): one file-scope
 * device array per GPU, found once per device through its symbol address.
 *
 * The array holds what tq_decode_attn keeps in its caller's workspace: the
 * per-unit arrival counters (which must be zero when a call starts) and the
 * split records.  It is zero when the code object loads; the set-up call
 * clears it once more with a fill kernel (no memset node, so a captured
 * first call replays correctly), and every decode call leaves the counters
 * at zero again (the last split of a unit resets its counter).  Calls that
 * overlap on one GPU share the array and race.
 */
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "tq_internal.h"

namespace {

static __device__ __align__(256) uint8_t scratch[TQ_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_ptr[kMaxDevices];
std::mutex g_mu;

__global__ void __launch_bounds__(256) zero_fill(uint4* p, int64_t n16) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

}  // namespace

tq_status tq_noalloc_scratch(void** out, hipStream_t stream) {
  *out = nullptr;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return TQ_ERR_DEVICE;
  void* p = g_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_mu);
    p = g_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      /* this device's copy of the array (the host name is only a stand-in) */
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
        (void)hipGetLastError();
        return TQ_ERR_DEVICE;
      }
      hipLaunchKernelGGL(zero_fill, dim3(256), dim3(256), 0, stream, (uint4*)p,
                         (int64_t)(TQ_NOALLOC_SCRATCH_BYTES / 16));
      if (hipGetLastError() != hipSuccess) return TQ_ERR_DEVICE;
      g_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return TQ_OK;
}
