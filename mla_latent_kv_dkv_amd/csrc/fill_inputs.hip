// Device twin of the host input generator (see include/mla_inputs.h).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mla_inputs.h"

namespace {

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__device__ __forceinline__ float value(uint64_t key, uint64_t idx, float scale) {
  const uint64_t w = mix64(key + (idx + 1) * kGamma);
  const int s = static_cast<int>(w & 0xFFFF) + static_cast<int>((w >> 16) & 0xFFFF) +
                static_cast<int>((w >> 32) & 0xFFFF) + static_cast<int>(w >> 48) - 131070;
  return __fmul_rn(static_cast<float>(s), scale);
}

__global__ void k_fill_f32(float* dst, int64_t n, uint64_t key, uint64_t start, float scale) {
  for (int64_t i = blockIdx.x * int64_t{256} + threadIdx.x; i < n; i += int64_t{256} * gridDim.x)
    dst[i] = value(key, start + i, scale);
}

__global__ void k_fill_bf16(uint16_t* dst, int64_t n, uint64_t key, uint64_t start, float scale) {
  for (int64_t i = blockIdx.x * int64_t{256} + threadIdx.x; i < n; i += int64_t{256} * gridDim.x) {
    uint32_t u = __float_as_uint(value(key, start + i, scale));
    u += 0x7FFFu + ((u >> 16) & 1u);
    dst[i] = static_cast<uint16_t>(u >> 16);
  }
}

}  // namespace

extern "C" int32_t mla_fill_normal(void* dst, int64_t n, int32_t dtype, uint64_t key,
                                   uint64_t start, float scale, hipStream_t stream) {
  if (n < 0) return -1;
  if (n == 0) return 0;
  if (!dst) return -1;
  if (dtype != 0 && dtype != 1) return -3;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (dtype == 0)
    hipLaunchKernelGGL(k_fill_f32, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream,
                       static_cast<float*>(dst), n, key, start, scale);
  else
    hipLaunchKernelGGL(k_fill_bf16, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream,
                       static_cast<uint16_t*>(dst), n, key, start, scale);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}
