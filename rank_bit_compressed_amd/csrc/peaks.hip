// peaks.hip -- measurement kernels: the HBM read rate a plain 16-byte-per-lane stream reaches, the rate of the
// fp16 matrix instruction the decode kernels use, and the shader clock.  They give measured peaks to set beside
// the published ones; nothing on the decode path calls them.
#include <hip/hip_runtime.h>

#include "kvc_common.hpp"

namespace kvc {
namespace {

// Every lane reads 16-byte words, eight in flight per iteration, striding the whole grid; the xor of what it read
// goes to one word per workgroup so that no load can be dropped.  (A sweep on this chip: nontemporal loads, 8 or 16
// in flight and some 32768 workgroups over 4 GiB read fastest, about 7.0-7.1 TB/s; plain loads about 6.2.)
__global__ __launch_bounds__(256) void stream_read_kernel(const u4* __restrict__ src, size_t n16, uint32_t* sink) {
  constexpr int U = 8;
  const size_t stride = (size_t)gridDim.x * 256;
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  u4 x = {0u, 0u, 0u, 0u};
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    u4 v[U];
#pragma unroll
    for (int k = 0; k < U; ++k) v[k] = __builtin_nontemporal_load(src + i + k * stride);
#pragma unroll
    for (int k = 0; k < U; ++k) x ^= v[k];
  }
  for (; i < n16; i += stride) x ^= __builtin_nontemporal_load(src + i);
  const uint32_t r = x[0] ^ x[1] ^ x[2] ^ x[3];
  __shared__ uint32_t red[256];
  red[threadIdx.x] = r;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t y = 0;
    for (int k = 0; k < 256; ++k) y ^= red[k];
    sink[blockIdx.x] = y;
  }
}

// Eight independent accumulator chains of v_mfma_f32_32x32x16_f16 per wave, operands in registers.
__global__ __launch_bounds__(256) void mfma_f16_kernel(int iters, float* sink) {
  typedef float f16v __attribute__((ext_vector_type(16)));
  const int lane = threadIdx.x & 63;
  h8 a, b;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = (_Float16)(0.001f * (lane + j));
    b[j] = (_Float16)(0.002f * (lane - j));
  }
  f16v c[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) c[k] = f16v{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 8; ++k) c[k] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c[k], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int k = 0; k < 8; ++k)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += c[k][e];
  if (s == 1234.5f) sink[blockIdx.x] = s;  // practically never: keeps the products alive without a store per wave
}

// Shader clock cycles (s_memtime) and 100 MHz reference ticks (s_memrealtime) over a spin of `spins` iterations.
__global__ void clock_kernel(int spins, uint64_t* out) {
  const uint64_t c0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  uint32_t x = threadIdx.x;
  for (int i = 0; i < spins; ++i) x = x * 1664525u + 1013904223u;
  const uint64_t c1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0) {
    out[0] = c1 - c0;
    out[1] = r1 - r0;
    out[2] = x;
  }
}

}  // namespace
}  // namespace kvc

using namespace kvc;

extern "C" kvc_status kvc_probe_stream_read(const void* src, size_t bytes, uint32_t* sink, int32_t grid, void* stream) {
  if (!src || !sink || bytes < 16 || (bytes & 15) || grid <= 0 || ((uintptr_t)src & 15)) return KVC_ERR_INVALID_ARG;
  hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, (const u4*)src, bytes / 16,
                     sink);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? KVC_OK : hip_fail(e);
}

extern "C" kvc_status kvc_probe_mfma_f16(int32_t iters, int32_t grid, float* sink, void* stream) {
  if (iters <= 0 || grid <= 0 || !sink) return KVC_ERR_INVALID_ARG;
  hipLaunchKernelGGL(mfma_f16_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, iters, sink);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? KVC_OK : hip_fail(e);
}

extern "C" kvc_status kvc_probe_clock(int32_t spins, uint64_t* out, void* stream) {
  if (spins <= 0 || !out) return KVC_ERR_INVALID_ARG;
  hipLaunchKernelGGL(clock_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream, spins, out);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? KVC_OK : hip_fail(e);
}
