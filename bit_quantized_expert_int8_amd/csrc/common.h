// Internal helpers shared by the library's translation units (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "moeq4.h"

namespace moeq4 {

// Record the thread-local message behind a non-OK status and return the status.
moe_status fail(moe_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

// MOE_OK, or MOE_ERR_HIP with the launch error text.
moe_status check_launch(const char* what);

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

struct RecordOffsets {
  size_t gate_up_q, gate_up_sb, down_q, down_sb, total;
};

// Host-side layout of one expert record (sections 256-byte aligned).
bool record_offsets(int32_t d, int32_t F, moe_dtype sb, RecordOffsets* out);

inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// ------------------------------------------------------------------------------------------------
// device helpers
// ------------------------------------------------------------------------------------------------

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> bf16 bits, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ float wave_min(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fminf(v, __shfl_xor(v, o, 64));
  return v;
}

// Maximum of an unsigned value over the 64 lanes of a wavefront, returned to every lane: row shifts
// within each row of 16 lanes, then row broadcasts across rows, all in DPP (no LDS traffic).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  auto mx = [](uint32_t a, uint32_t b) { return a > b ? a : b; };
  v = mx(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, true));   // row_shr:1
  v = mx(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, true));   // row_shr:2
  v = mx(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, true));   // row_shr:4
  v = mx(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, true));   // row_shr:8
  v = mx(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false));  // row_bcast:15
  v = mx(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false));  // row_bcast:31
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Top-k of lg[0..E) by wavefront 0 of the calling block (threads 0..63; E <= 64 * PER): k rounds of an
// argmax over order-preserving keys.  Larger logits first; equal logits (+0 and -0 are equal) -> the lower
// id first.  Writes sel_i[0..k) and sel_v[0..k) (the logits); -1 / NaN when fewer than k candidates.
template <int PER>
__device__ __forceinline__ void topk_wave(const float* lg, int E, int k, int* sel_i, float* sel_v) {
  const int lane = threadIdx.x;
  uint32_t key[PER];
#pragma unroll
  for (int m = 0; m < PER; ++m) {
    const int idx = lane + 64 * m;
    uint32_t u = idx < E ? __float_as_uint(lg[idx] + 0.0f) : 0u;
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    key[m] = idx < E ? (u ? u : 1u) : 0u;          // 0 marks "absent / taken"
  }
  const int nm = (E + 63) / 64;                    // key groups holding candidates (uniform)
  for (int rr = 0; rr < k; ++rr) {
    uint32_t mx = key[0];
#pragma unroll
    for (int m = 1; m < PER; ++m)
      if (m < nm) mx = key[m] > mx ? key[m] : mx;
    mx = wave_max_u32(mx);
    int sel = -1;
#pragma unroll
    for (int m = 0; m < PER; ++m) {
      if (m >= nm || sel >= 0) continue;
      const unsigned long long hit = __ballot(key[m] == mx && mx != 0u);
      if (hit) sel = 64 * m + (__ffsll((long long)hit) - 1);
    }
#pragma unroll
    for (int m = 0; m < PER; ++m)
      if (m < nm && lane + 64 * m == sel) key[m] = 0u;
    if (lane == 0) {
      sel_i[rr] = sel;
      sel_v[rr] = sel >= 0 ? lg[sel] : __builtin_nanf("");
    }
  }
}

}  // namespace moeq4
