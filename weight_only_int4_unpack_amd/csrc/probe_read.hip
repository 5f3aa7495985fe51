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

// ---------------------------------------------------------------------------
// Measurement probe: instruction issue of one wavefront. Eight independent
// MFMA 16x16x32 bf16 chains, each MFMA followed by NV independent fp32 FMAs
// (NV = 0, 8, 16 or 32), or (NV < 0) 64 FMAs and no MFMA per loop trip.
// Workgroup 0's first lane records the shader-clock cycles of the loop; the
// host divides by the trip count. Results are written only when they equal
// a value never produced, so nothing is stored.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <int NV>
__global__ __launch_bounds__(256) void probe_issue_kernel(float* out, int iters, float x, float y,
                                                          long long* clk) {
  f32x4_t a0 = {1.f, 0.f, 0.f, (float)threadIdx.x}, a1 = a0, a2 = a0, a3 = a0, a4 = a0, a5 = a0,
          a6 = a0, a7 = a0;
  const u32x4 a = {threadIdx.x, 2u, 3u, 4u};
  const u32x4 b0 = {0x3f803f80u, 1u, 7u, 8u}, b1 = b0 + 1u, b2 = b0 + 2u, b3 = b0 + 3u,
              b4 = b0 + 4u, b5 = b0 + 5u, b6 = b0 + 6u, b7 = b0 + 7u;
  float v0 = threadIdx.x * 1e-3f, v1 = v0 + 1, v2 = v0 + 2, v3 = v0 + 3, v4 = v0 + 4, v5 = v0 + 5,
        v6 = v0 + 6, v7 = v0 + 7;
  const long long c0 = clock64();
#pragma nounroll
  for (int it = 0; it < iters; ++it) {
#define PROBE_V8                                                                             \
  v0 = __builtin_fmaf(v0, x, y); v1 = __builtin_fmaf(v1, x, y); v2 = __builtin_fmaf(v2, x, y); \
  v3 = __builtin_fmaf(v3, x, y); v4 = __builtin_fmaf(v4, x, y); v5 = __builtin_fmaf(v5, x, y); \
  v6 = __builtin_fmaf(v6, x, y); v7 = __builtin_fmaf(v7, x, y);
#define PROBE_M(A, B)                                                                         \
  A = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),                \
                                              __builtin_bit_cast(bf16x8_t, B), A, 0, 0, 0);   \
  if (NV >= 8) { PROBE_V8 }                                                                   \
  if (NV >= 16) { PROBE_V8 }                                                                  \
  if (NV >= 24) { PROBE_V8 }                                                                  \
  if (NV >= 32) { PROBE_V8 }
    if constexpr (NV >= 0) {
      PROBE_M(a0, b0) PROBE_M(a1, b1) PROBE_M(a2, b2) PROBE_M(a3, b3)
      PROBE_M(a4, b4) PROBE_M(a5, b5) PROBE_M(a6, b6) PROBE_M(a7, b7)
    } else {
      PROBE_V8 PROBE_V8 PROBE_V8 PROBE_V8 PROBE_V8 PROBE_V8 PROBE_V8 PROBE_V8
    }
#undef PROBE_M
#undef PROBE_V8
  }
  const long long c1 = clock64();
  if (blockIdx.x == 0 && threadIdx.x == 0) clk[0] = c1 - c0;
  const float s = a0[0] + a1[1] + a2[2] + a3[3] + a4[0] + a5[1] + a6[2] + a7[3] + v0 + v1 + v2 +
                  v3 + v4 + v5 + v6 + v7;
  if (s == 12345.678f) out[blockIdx.x * 256 + threadIdx.x] = s;
}

extern "C" {

// Launches probe_issue_kernel<nv> (nv in {-1, 0, 8, 16, 32}) with `blocks`
// workgroups of 256 threads and `lds` bytes of dynamic LDS (which sets how
// many workgroups share a CU); `out` holds blocks * 256 floats, `clk` one
// 64-bit word (loop cycles of workgroup 0). Returns a hipError_t.
int w4a16_probe_issue(int32_t nv, int32_t blocks, int32_t lds, int32_t iters, void* out,
                      void* clk, void* stream) {
  if (out == nullptr || clk == nullptr || blocks <= 0 || iters <= 0 || lds < 0 ||
      lds > 160 * 1024)
    return (int)hipErrorInvalidValue;
  hipStream_t st = (hipStream_t)stream;
  float* o = (float*)out;
  long long* c = (long long*)clk;
  switch (nv) {
    case -1: hipLaunchKernelGGL(probe_issue_kernel<-1>, dim3(blocks), dim3(256), lds, st, o, iters, 1.0001f, 0.5f, c); break;
    case 0: hipLaunchKernelGGL(probe_issue_kernel<0>, dim3(blocks), dim3(256), lds, st, o, iters, 1.0001f, 0.5f, c); break;
    case 8: hipLaunchKernelGGL(probe_issue_kernel<8>, dim3(blocks), dim3(256), lds, st, o, iters, 1.0001f, 0.5f, c); break;
    case 16: hipLaunchKernelGGL(probe_issue_kernel<16>, dim3(blocks), dim3(256), lds, st, o, iters, 1.0001f, 0.5f, c); break;
    case 32: hipLaunchKernelGGL(probe_issue_kernel<32>, dim3(blocks), dim3(256), lds, st, o, iters, 1.0001f, 0.5f, c); break;
    default: return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

}  // extern "C"
