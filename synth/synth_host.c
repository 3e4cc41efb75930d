/* Host side of the seeded input generator in plain C: the same counter-based definition as
 * synth/__init__.py and synth_gen.hip (SplitMix64 outputs -> Irwin-Hall sum of twelve 16-bit uniforms ->
 * one fp32 product), threaded with OpenMP over the elements.  It only draws inputs: no method arithmetic.
 * Built with gcc by the package's build step into synth/libsynth_host.so. */
#include <stdint.h>

#define GAMMA 0x9E3779B97F4A7C15ull

static inline uint64_t mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static inline int32_t field_sum(uint64_t r) {
  return (int32_t)(r & 0xffff) + (int32_t)((r >> 16) & 0xffff) + (int32_t)((r >> 32) & 0xffff) + (int32_t)(r >> 48);
}

/* out[i] = normal number start + i of the stream `seed`, i < count, as float32(z) * float32(sigma * 2^-16).
 * threads <= 0: OpenMP's default. */
void synth_host_normals_f32(uint64_t seed, uint64_t start, uint64_t count, float sigma, float* out, int threads) {
  const float scale = sigma * 0x1p-16f;   /* exact: a power-of-two scaling of float32(sigma) */
  const int64_t n = (int64_t)count;
  if (threads <= 0) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
      const uint64_t base = seed + (3 * (start + (uint64_t)i) + 1) * GAMMA;
      const int32_t s = field_sum(mix(base)) + field_sum(mix(base + GAMMA)) + field_sum(mix(base + 2 * GAMMA));
      out[i] = (float)(s - 393210) * scale;
    }
  } else {
#pragma omp parallel for schedule(static) num_threads(threads)
    for (int64_t i = 0; i < n; ++i) {
      const uint64_t base = seed + (3 * (start + (uint64_t)i) + 1) * GAMMA;
      const int32_t s = field_sum(mix(base)) + field_sum(mix(base + GAMMA)) + field_sum(mix(base + 2 * GAMMA));
      out[i] = (float)(s - 393210) * scale;
    }
  }
}
