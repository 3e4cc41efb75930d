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

// Cross-lane reads by DPP (VALU only: no trip through the LDS unit, which co-resident blocks keep busy).
// dpp_f<CTRL>(v) in lane i is v of the lane CTRL names; lanes whose source falls outside the row read 0.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
constexpr int kDppXor1 = 0xB1;    // quad_perm [1,0,3,2]: lane i ^ 1
constexpr int kDppXor2 = 0x4E;    // quad_perm [2,3,0,1]: lane i ^ 2
constexpr int kDppShl4 = 0x104;   // row_shl:4: lane i + 4 of the row of 16
constexpr int kDppShr4 = 0x114;   // row_shr:4: lane i - 4
constexpr int kDppRor8 = 0x128;   // row_ror:8: lane i ^ 8 within the row

// v of lane i ^ 4
__device__ __forceinline__ float xor4_f(float v) {
  const float up = dpp_f<kDppShl4>(v), dn = dpp_f<kDppShr4>(v);
  return (threadIdx.x & 4) ? dn : up;
}

// Sum over the wavefront, the same value in every lane: pairwise sums over lanes i ^ 1, i ^ 2, i ^ 4, i ^ 8
// (both lanes of a pair compute the same sum, addition being commutative), then the four row sums as
// (r0 + r1) + (r2 + r3).
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<kDppXor1>(v);
  v += dpp_f<kDppXor2>(v);
  v += xor4_f(v);
  v += dpp_f<kDppRor8>(v);
  auto row = [](float x, int l) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l)); };
  return (row(v, 0) + row(v, 16)) + (row(v, 32) + row(v, 48));
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

// Top-k of E values held by one wavefront (value lane + 64 m in v[m], E <= 64 * PER): k rounds of an argmax
// over order-preserving keys, the maximum of a round being a DPP reduction (no LDS traffic).  Larger
// values first; equal values (+0 and -0 are equal) -> the lower index first.  Lane r < k receives the r-th
// selection in (id, val); the other lanes, and lanes past the last candidate, get -1 / NaN.
// Order-preserving key of a float for unsigned comparison: larger float -> larger key, +0 and -0 equal;
// never 0 (0 marks an absent candidate).
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f + 0.0f);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return u ? u : 1u;
}

template <int PER>
__device__ __forceinline__ void topk_wave(const float (&v)[PER], int E, int k, int& id, float& val) {
  const int lane = threadIdx.x & 63;
  uint32_t key[PER];
#pragma unroll
  for (int m = 0; m < PER; ++m) {
    const int idx = lane + 64 * m;
    key[m] = idx < E ? order_key(v[m]) : 0u;       // 0 marks "absent / taken"
  }
  id = -1;
  val = __builtin_nanf("");
  for (int rr = 0; rr < k; ++rr) {
    uint32_t mx = key[0];
#pragma unroll
    for (int m = 1; m < PER; ++m) mx = key[m] > mx ? key[m] : mx;
    mx = wave_max_u32(mx);
    if (mx == 0u) break;                           // uniform: no candidate left
    int sel = -1;
    float sv = 0.f;
#pragma unroll
    for (int m = 0; m < PER; ++m) {
      if (sel >= 0) continue;
      const unsigned long long hit = __ballot(key[m] == mx);
      if (hit) {
        const int ln = __ffsll((long long)hit) - 1;
        sel = 64 * m + ln;
        sv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v[m]), ln));
      }
    }
#pragma unroll
    for (int m = 0; m < PER; ++m)
      if (lane + 64 * m == sel) key[m] = 0u;
    if (lane == rr) {
      id = sel;
      val = sv;
    }
  }
}

}  // namespace moeq4
