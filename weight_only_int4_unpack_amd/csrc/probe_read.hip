// Measurement probe (not part of the GEMM): a plain streaming read of a
// device buffer, to measure what one launch of a given size can pull from
// HBM on this GPU, so the GEMM's bandwidth can be read against an
// achievable figure next to the 8 TB/s specification.
//
// Every thread reads 16-byte pieces, four in flight per loop trip, strided
// over the whole grid (fully coalesced: a wavefront reads 1 KiB contiguous
// per load), and folds them into one word with XOR. The word is written only
// when it equals a value the host passes and never expects, so the loads
// cannot be removed and nothing but the reads reaches memory.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void probe_read_kernel(const u32x4* __restrict__ src,
                                                         int64_t n16, uint32_t never,
                                                         uint32_t* out) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    acc ^= a ^ b ^ c ^ d;
  }
  for (; i < n16; i += stride) acc ^= src[i];
  const uint32_t v = acc.x ^ acc.y ^ acc.z ^ acc.w;
  if (v == never) out[blockIdx.x] = v;
}

extern "C" {

// Reads `bytes` (a multiple of 16) at `src` (16-byte aligned) on `stream`
// with `blocks` workgroups of 256 threads; `out` must hold `blocks` words
// (written only if the XOR of the data equals `never`). Returns a hipError_t.
int w4a16_probe_read(const void* src, int64_t bytes, int32_t blocks, uint32_t never, void* out,
                     void* stream) {
  if (src == nullptr || out == nullptr || bytes <= 0 || bytes % 16 != 0 || blocks <= 0 ||
      (reinterpret_cast<uintptr_t>(src) & 15u) != 0)
    return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(probe_read_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                     (const u32x4*)src, bytes / 16, never, (uint32_t*)out);
  return (int)hipGetLastError();
}

}  // extern "C"
