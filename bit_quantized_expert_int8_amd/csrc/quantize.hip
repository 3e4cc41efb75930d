// q4_quantize / q4_pack_expert: fp32 weights -> 4-bit affine codes + (scale, bias) per group of 64.
//
// One wavefront encodes one group: lane l holds column 64g+l, min/max are wave reductions, each lane
// takes its code, and eight-lane OR reductions assemble the packed uint32 words.  The integer decisions
// are taken in IEEE fp32 (correctly rounded subtract and divide, rint = round-half-even) so that any
// other fp32 encoder following the same definition produces identical bytes.
#include "common.h"

#pragma clang fp contract(off)

namespace moeq4 {
namespace {

template <bool SB_BF16>
__global__ __launch_bounds__(256) void quantize_kernel(const float* __restrict__ w, int64_t n_groups, int K,
                                                       uint32_t* __restrict__ codes, void* __restrict__ sb) {
  const int lane = threadIdx.x & 63;
  const int64_t grp = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (grp >= n_groups) return;
  const int gpr = K / 64;                       // groups per row
  const int64_t row = grp / gpr;
  const int g = (int)(grp % gpr);
  const float v = w[row * K + (int64_t)g * 64 + lane];

  const float mn = wave_min(v);
  const float mx = wave_max(v);
  float scale = __fdiv_rn(mx - mn, 15.0f);
  float bias = mn;
  if (SB_BF16) {
    scale = bf16_bits_to_f32(f32_to_bf16_bits(scale));
    bias = bf16_bits_to_f32(f32_to_bf16_bits(bias));
  }
  uint32_t code = 0;
  if (scale != 0.0f) {
    float t = __builtin_rintf(__fdiv_rn(v - bias, scale));
    t = fminf(fmaxf(t, 0.0f), 15.0f);
    code = (uint32_t)t;
  }
  uint32_t word = code << (4 * (lane & 7));
  word |= __shfl_xor(word, 1, 64);
  word |= __shfl_xor(word, 2, 64);
  word |= __shfl_xor(word, 4, 64);
  if ((lane & 7) == 0) codes[row * (K / 8) + (int64_t)g * 8 + (lane >> 3)] = word;
  if (lane == 0) {
    if (SB_BF16) {
      uint32_t pair = f32_to_bf16_bits(scale) | (f32_to_bf16_bits(bias) << 16);
      reinterpret_cast<uint32_t*>(sb)[grp] = pair;
    } else {
      reinterpret_cast<float2*>(sb)[grp] = make_float2(scale, bias);
    }
  }
}

moe_status launch_quantize(const float* w, int32_t N, int32_t K, moe_dtype sb, uint32_t* codes, void* sbp,
                           hipStream_t s) {
  const int64_t groups = (int64_t)N * (K / 64);
  const int64_t blocks = (groups + 3) / 4;
  if (blocks > 0x7fffffff) return fail(MOE_ERR_UNSUPPORTED, "q4_quantize: %lld groups is too many", (long long)groups);
  if (sb == MOE_BF16)
    hipLaunchKernelGGL(quantize_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, s, w, groups, K, codes, sbp);
  else
    hipLaunchKernelGGL(quantize_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, s, w, groups, K, codes, sbp);
  return check_launch("q4_quantize");
}

}  // namespace
}  // namespace moeq4

using namespace moeq4;

extern "C" moe_status q4_quantize(const float* w_dev, int32_t N, int32_t K, moe_dtype sb_dtype, uint32_t* codes_dev,
                                  void* sb_dev, void* stream) {
  if (!w_dev || !codes_dev || !sb_dev) return fail(MOE_ERR_INVALID_ARG, "q4_quantize: NULL pointer");
  if (N < 1 || K < 64 || K % 64) return fail(MOE_ERR_INVALID_ARG, "q4_quantize: N=%d K=%d (K must be a multiple of 64)", N, K);
  if (sb_dtype != MOE_F32 && sb_dtype != MOE_BF16) return fail(MOE_ERR_INVALID_ARG, "q4_quantize: bad sb_dtype %d", (int)sb_dtype);
  if (!aligned(w_dev, 4) || !aligned(codes_dev, 4) || !aligned(sb_dev, sb_dtype == MOE_BF16 ? 4 : 8))
    return fail(MOE_ERR_INVALID_ARG, "q4_quantize: misaligned pointer");
  return launch_quantize(w_dev, N, K, sb_dtype, codes_dev, sb_dev, as_stream(stream));
}

extern "C" moe_status q4_pack_expert(const float* w_gate_up_dev, const float* w_down_dev, int32_t d, int32_t F,
                                     moe_dtype sb_dtype, void* record_dev, void* stream) {
  RecordOffsets o;
  if (!w_gate_up_dev || !w_down_dev || !record_dev) return fail(MOE_ERR_INVALID_ARG, "q4_pack_expert: NULL pointer");
  if (!record_offsets(d, F, sb_dtype, &o))
    return fail(MOE_ERR_INVALID_ARG, "q4_pack_expert: d=%d F=%d must be positive multiples of 64", d, F);
  if (!aligned(record_dev, 256)) return fail(MOE_ERR_INVALID_ARG, "q4_pack_expert: record not 256-byte aligned");
  char* rec = static_cast<char*>(record_dev);
  moe_status st = launch_quantize(w_gate_up_dev, 2 * F, d, sb_dtype, reinterpret_cast<uint32_t*>(rec + o.gate_up_q),
                                  rec + o.gate_up_sb, as_stream(stream));
  if (st != MOE_OK) return st;
  return launch_quantize(w_down_dev, d, F, sb_dtype, reinterpret_cast<uint32_t*>(rec + o.down_q), rec + o.down_sb,
                         as_stream(stream));
}
