// Scratch of the entry point that allocates nothing (w4a16_gemm_noalloc):
// a fixed device array of kStaticScratchBytes, one copy per GPU, held until
// the process ends. Its first kCounterBytes are the arrival counters of the
// split-K hand-off, the rest the fp32 partials, as in every workspace.
//
// In host code `scratch` names a host-side stand-in, not device memory: its
// device address on the current GPU comes from hipGetSymbolAddress, taken
// once per device and kept; only that address is ever passed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>
#include <vector>

#include "w4a16_internal.h"

namespace w4a16 {
namespace {

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

// Clears `n` words (the counter region) with plain vector stores.
__global__ __launch_bounds__(256) void clear_words(uint32_t* p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0u;
}

struct DeviceScratch {
  void* ptr = nullptr;  // device address of this GPU's copy of `scratch`
  bool cleared = false; // counter region cleared by an uncaptured launch
};
std::mutex g_mu;
std::vector<DeviceScratch> g_dev;

}  // namespace

hipError_t static_scratch(hipStream_t stream, void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(g_mu);
  if ((int)g_dev.size() <= dev) g_dev.resize(dev + 1);
  DeviceScratch& d = g_dev[dev];
  if (d.ptr == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    d.ptr = p;
  }
  if (!d.cleared) {
    // The loader zero-fills the array, but the counter region is cleared
    // once more before its first use on this device, on the caller's
    // stream (a kernel, not a memset: the call may be under capture). A
    // clear recorded into a graph runs at each replay and is not counted.
    const int words = (int)(kCounterBytes / 4);
    hipLaunchKernelGGL(clear_words, dim3((words + 255) / 256), dim3(256), 0, stream,
                       (uint32_t*)d.ptr, words);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cs) != hipSuccess) {
      (void)hipGetLastError();
      cs = hipStreamCaptureStatusActive;
    }
    if (cs == hipStreamCaptureStatusNone) d.cleared = true;
  }
  *ptr = d.ptr;
  return hipSuccess;
}

}  // namespace w4a16
