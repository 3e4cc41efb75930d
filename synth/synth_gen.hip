// Device side of the seeded input generator: the same counter-based definition as synth/__init__.py
// (SplitMix64 outputs -> Irwin-Hall sum of twelve 16-bit uniforms -> one fp32 product), so the GPU can
// draw multi-gigabyte weight sets in place, bit-identical to the host draws.  No method arithmetic here.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;

__device__ __forceinline__ uint64_t mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__device__ __forceinline__ int32_t field_sum(uint64_t r) {
  return (int32_t)(r & 0xffff) + (int32_t)((r >> 16) & 0xffff) + (int32_t)((r >> 32) & 0xffff) + (int32_t)(r >> 48);
}

__global__ void normals_kernel(uint64_t seed, uint64_t start, uint64_t count, float scale, float* __restrict__ out) {
  const uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= count) return;
  const uint64_t n = start + i;
  const uint64_t base = seed + (3 * n + 1) * kGamma;
  const int32_t s = field_sum(mix(base)) + field_sum(mix(base + kGamma)) + field_sum(mix(base + 2 * kGamma));
  out[i] = (float)(s - 393210) * scale;
}

}  // namespace

// Returns 0 or the hipError_t of the failure.
extern "C" int synth_normals_f32(uint64_t seed, uint64_t start, uint64_t count, float sigma, float* out_dev, void* stream) {
  if (!out_dev) return (int)hipErrorInvalidValue;
  if (count == 0) return 0;
  const float scale = sigma * 0x1p-16f;   // the fp32 product of the spec: float32(sigma) * 2^-16 (exact)
  const uint64_t blocks = (count + 255) / 256;
  if (blocks > 0x7fffffffull) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(normals_kernel, dim3((unsigned)blocks), dim3(256), 0, reinterpret_cast<hipStream_t>(stream), seed, start,
                     count, scale, out_dev);
  return (int)hipGetLastError();
}
