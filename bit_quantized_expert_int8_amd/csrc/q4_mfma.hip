// Grouped expert products for T > 1 tokens on the matrix cores ([G26] "Le pipeline de traitement": a
// prompt's tokens processed together share each expert's weights; [REMIO] "L'affirmation des 2 Go fait de
// la bande passante SSD la nouvelle contrainte": 4-bit affine MLX weights).
//
// With several tokens per expert the one-token kernels' dot2 chains become the bottleneck (every token
// repeats the dequantization and 36 VALU operations per 32 codes).  Here a block holds 16 weight rows in
// registers and multiplies them with up to 16 tokens at a time by v_mfma_f32_16x16x32_f16:
//
//   A (16 tokens x 32 k, fp16)   lane l: token l % 16, k block l / 16 (8 values)
//   B (32 k x 16 rows)           lane l: row l % 16, the same 8 k = one 32-bit word of 8 codes
//   D (16 x 16, fp32)            lane l: tokens 4 (l / 16) + i, i < 4, row l % 16
//
// The code word becomes B with the one-token kernels' trick: (w & 0x000F000F) | 0x64006400 and its three
// siblings are the fp16 pairs (1024 + n0, 1024 + n4), (1024 + 16 n1, 1024 + 16 n5), (1024 + n2, 1024 + n6),
// (1024 + 16 n3, 1024 + 16 n7).  The contraction is a sum over k, so A is staged in that order, with the
// positions of the 16 n codes divided by 16: per 8 values [x0, x4, x1/16, x5/16, x2, x6, x3/16, x7/16],
// all times 2^-e, one power of two per row (stage_rows_kernel).  The MFMA sum over a group of 64 k is then
// 1024 O + sum_c q_c x_c 2^-e with O the sum of the group's staged values, and per group
//   y += scale * (acc - 1024 O) + bias * Sx,        Sx = sum_c x_c 2^-e (from the staged values),
// and finally y *= 2^e.  Products of an 11-bit and an 11-bit significand are exact in fp32.
//
// Each pair of MFMA steps covers one group: lane (row, k block kb) takes the two code words 8 g + 2 kb
// and 8 g + 2 kb + 1 of its row (one 8-byte load), and the A lanes read the matching 32 staged bytes of
// their token (k order within a group is a permutation shared by A and B).  The block's 4 waves split the
// row's groups; their 16 x 16 partial results are added in LDS in wave order.  Results match the
// one-token kernels within rounding (the activation is scaled per token, not per half-group).
#include "q4_device.h"

namespace moeq4 {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreadsM = 256;
constexpr int kStageIt = kMaxK / 8 / kThreadsM;   // 8-value blocks per thread of a staged row (K <= 8192)

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<kDppXor1>(v));
  v = fmaxf(v, dpp_f<kDppXor2>(v));
  v = fmaxf(v, xor4_f(v));
  v = fmaxf(v, dpp_f<kDppRor8>(v));
  auto row = [](float x, int l) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l)); };
  return fmaxf(fmaxf(row(v, 0), row(v, 16)), fmaxf(row(v, 32), row(v, 48)));
}

// One block per row: xq[row] (fp16, the MFMA order above), os[row][g] = (1024 O_g, Sx_g), ef[row] = 2^e.
// Fixed summation order: per 8 values ((a0 + a4) + (a2 + a6)) and ((b1 + b5) + (b3 + b7)), then the 8
// blocks of a group by an xor butterfly.
template <typename XT>
__global__ __launch_bounds__(kThreadsM) void stage_rows_kernel(const XT* __restrict__ x, int K, StagedRows out) {
  __shared__ float wmax[kThreadsM / 64];
  const int row = blockIdx.x, t = threadIdx.x;
  const int nb = K / 8;
  const XT* xr = x + (int64_t)row * K;
  float v[kStageIt][8];
  float amax = 0.f;
#pragma unroll
  for (int it = 0; it < kStageIt; ++it) {
    const int b = t + it * kThreadsM;
    if (b < nb) {
      XWord<XT> w;
      load_word<XT>(xr, b >> 2, b & 3, w);
      word_to_f32<XT>(w, v[it]);
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[it][i]));
    }
  }
  amax = wave_max(amax);
  if ((t & 63) == 0) wmax[t >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  int e = 0;
  if (amax > 0.f && amax <= 3.0e38f) e = max(-100, min(100, ilogbf(amax) - 13));   // amax * 2^-e in [2^13, 2^14)
  const float inv = ldexpf(1.0f, -e), inv16 = inv * 0.0625f;
#pragma unroll
  for (int it = 0; it < kStageIt; ++it) {
    const int b = t + it * kThreadsM;
    if (it * kThreadsM >= nb) break;   // uniform: the group butterfly needs every lane of the block
    const bool live = b < nb;
    const _Float16 a0 = (_Float16)(v[it][0] * inv), a4 = (_Float16)(v[it][4] * inv);
    const _Float16 b1 = (_Float16)(v[it][1] * inv16), b5 = (_Float16)(v[it][5] * inv16);
    const _Float16 a2 = (_Float16)(v[it][2] * inv), a6 = (_Float16)(v[it][6] * inv);
    const _Float16 b3 = (_Float16)(v[it][3] * inv16), b7 = (_Float16)(v[it][7] * inv16);
    const float sa = ((float)a0 + (float)a4) + ((float)a2 + (float)a6);
    const float sb = ((float)b1 + (float)b5) + ((float)b3 + (float)b7);
    float osum = live ? sa + sb : 0.f, ssum = live ? sa + 16.0f * sb : 0.f;
    osum += dpp_f<kDppXor1>(osum);
    ssum += dpp_f<kDppXor1>(ssum);
    osum += dpp_f<kDppXor2>(osum);
    ssum += dpp_f<kDppXor2>(ssum);
    osum += xor4_f(osum);
    ssum += xor4_f(ssum);
    if (live) {
      u32x4 q;
      q.x = pack_h2(a0, a4);
      q.y = pack_h2(b1, b5);
      q.z = pack_h2(a2, a6);
      q.w = pack_h2(b3, b7);
      *reinterpret_cast<u32x4*>(out.xq + (int64_t)row * K + b * 8) = q;
      if ((b & 7) == 0) out.os[(int64_t)row * (K / 64) + (b >> 3)] = make_float2(1024.0f * osum, ssum);
    }
  }
  if (t == 0) out.ef[row] = ldexpf(1.0f, e);
}

// Dynamic LDS of a block: red [4][16][16] fp32, os [G][16] float2, ef [16], rows [16] (stage and output rows)
inline size_t mfma_lds_bytes(int K) { return (size_t)4 * 256 * 4 + (size_t)(K / 64) * 16 * 8 + 16 * 4 + 16 * 4 * 2; }

constexpr int kAhead = 3;   // groups of A in flight per wave

template <bool SB_BF16>
__device__ __forceinline__ void opaque_sb(SbWord<SB_BF16>& w);
template <>
__device__ __forceinline__ void opaque_sb<true>(SbWord<true>& w) {
  asm volatile("" : "+v"(w.s));
}
template <>
__device__ __forceinline__ void opaque_sb<false>(SbWord<false>&) {}

// A block's 4 waves take 4 / wk tiles of 16 weight rows; the wk waves of a tile split its groups.  Blocks
// [0, n_shared_blocks) hold the shared matrix's tiles with all T tokens; the rest, n_routed_blocks per
// group, the tiles of a routed group with that group's pairs.  Tokens go through in chunks of 16.
template <int NG, bool SB_BF16>
__global__ __launch_bounds__(kThreadsM) void grouped_mfma_kernel(MfmaArgs a) {
  extern __shared__ __align__(16) uint32_t lds[];
  float* red = reinterpret_cast<float*>(lds);                       // [4 waves][16 tokens][16 rows]

  int u = blockIdx.x;
  const bool shared = u < a.n_shared_blocks;
  int e = 0, start = 0, count = a.T;
  bool valid = true;
  if (!shared) {
    u -= a.n_shared_blocks;
    const int j = u / a.n_routed_blocks;
    u -= j * a.n_routed_blocks;
    if (j >= *a.n_groups) return;
    const int4 g = a.groups[j];
    valid = (unsigned)g.x < (unsigned)a.routed.n_records;
    e = valid ? g.x : 0;
    start = g.y;
    count = g.z;
  }
  const Pool P = shared ? a.shared : a.routed;                 // copies: held in SGPRs, not re-read
  const StagedRows xs = shared ? a.xs_shared : a.xs_routed;
  const int K = shared ? a.K_shared : a.K_routed, wk = shared ? a.wk_shared : a.wk_routed;
  const int G = K / 64;
  float2* os_l = reinterpret_cast<float2*>(lds + 4 * 256);            // [G][16]
  float* ef_l = reinterpret_cast<float*>(lds + 4 * 256 + G * 32);      // [16]
  int* srow_l = reinterpret_cast<int*>(ef_l + 16);                     // [16] staged row of token m
  int* orow_l = srow_l + 16;                                           // [16] output row of token m

  // the wave index through readfirstlane, so that the compiler sees the group range as wave-uniform
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63, n = lane & 15,
            kb = lane >> 4;
  const int tpb = 4 / wk, part = wave % wk;
  const int tile = u * tpb + wave / wk;
  // this lane's weight row
  const int row = a.gate_up ? (n < 8 ? tile * 8 + n : P.F + tile * 8 + (n - 8)) : tile * 16 + n;
  const char* rec = P.base + (int64_t)e * P.record_bytes;
  const uint32_t* qrow = reinterpret_cast<const uint32_t*>(rec + P.off_q + (int64_t)row * (K / 2));
  const char* sbrow = rec + P.off_sb + (int64_t)row * (G * (SB_BF16 ? 4 : 8));
  // this wave's groups [g0, g0 + nw)
  const int g0 = (part * G) / wk, nw = ((part + 1) * G) / wk - g0;
  // all NG loads issued unconditionally (no branch, so no wait between them): slots past the wave's range
  // read the row's last group again, an invalid expert reads record 0; neither value is used
  u32x2 q[NG];
  SbWord<SB_BF16> sbw[NG];
#pragma unroll
  for (int i = 0; i < NG; ++i) sbw[i] = load_sb<SB_BF16>(sbrow, min(g0 + i, G - 1));
#pragma unroll
  for (int i = 0; i < NG; ++i)
    q[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(qrow + min(g0 + i, G - 1) * 8 + 2 * kb));

  for (int c0 = 0; c0 < count; c0 += 16) {
    const Dequant dq = opaque_dequant();   // the dequantized words stay inside the chunk loop
    uint32_t sh8 = 8;                      // and so do the shifted code words
    asm volatile("" : "+v"(sh8));
    const int nlive = min(16, count - c0);
    // the chunk's tokens: staged row, output row, 2^e, and the groups' (1024 O, Sx).  Slots past the last
    // token repeat the first token's staged row, so their A loads fall on lines the wave reads anyway.
    if ((int)threadIdx.x < 16) {
      const int m = threadIdx.x;
      const int mm = m < nlive ? m : 0;
      const int pr = shared ? c0 + mm : a.perm[start + c0 + mm];
      const int sr = (shared || !a.gate_up) ? pr : pr / a.k;
      srow_l[m] = sr;
      orow_l[m] = pr;
      ef_l[m] = m < nlive ? xs.ef[sr] : 0.f;
    }
    __syncthreads();
    {
      // thread i stages (group i / 16 + 16 r, token i % 16) for every r: one token row per thread, the loads
      // issued together with the group clamped into the row (slots past the last token read the first
      // token's row; those values are never used)
      constexpr int kRep = (NG + 3) / 4;   // G <= 4 NG (a wave has at most NG groups, wk <= 4), so G * 16 <= kRep * 256
      const int nrep = (G * 16 + kThreadsM - 1) / kThreadsM;
      const float2* orow = xs.os + (int64_t)srow_l[threadIdx.x & 15] * G;
      const int gq = threadIdx.x >> 4;
      float2 ov[kRep];
#pragma unroll
      for (int r = 0; r < kRep; ++r)
        if (r < nrep) ov[r] = orow[min(gq + 16 * r, G - 1)];
#pragma unroll
      for (int r = 0; r < kRep; ++r)
        if (r < nrep && gq + 16 * r < G) os_l[threadIdx.x + r * kThreadsM] = ov[r];
    }
    const _Float16* arow = xs.xq + (int64_t)srow_l[n] * K + 16 * kb;   // token n's 32 bytes per group
    __syncthreads();
    f32x4 y = {0.f, 0.f, 0.f, 0.f};
    if (valid) {
      // A for the next kAhead groups in flight; group indexes past the wave's range are clamped to the
      // row's last group (loads that stay in the row; their values are not used)
      half8 ar[kAhead][2];
#pragma unroll
      for (int p = 0; p < kAhead; ++p) {
        const u32x4* ap = reinterpret_cast<const u32x4*>(arow + min(g0 + p, G - 1) * 64);
        ar[p][0] = __builtin_bit_cast(half8, ap[0]);
        ar[p][1] = __builtin_bit_cast(half8, ap[1]);
      }
#pragma unroll
      for (int i = 0; i < NG; ++i) {
        const half8 a0 = ar[i % kAhead][0], a1 = ar[i % kAhead][1];
        if (i + kAhead < NG) {
          const u32x4* ap = reinterpret_cast<const u32x4*>(arow + min(g0 + i + kAhead, G - 1) * 64);
          ar[i % kAhead][0] = __builtin_bit_cast(half8, ap[0]);
          ar[i % kAhead][1] = __builtin_bit_cast(half8, ap[1]);
        }
        if (i >= nw) continue;   // wave-uniform; a break would keep the loop from unrolling
        const int g = g0 + i;
        const uint32_t w0 = q[i].x, w1 = q[i].y, t0 = w0 >> sh8, t1 = w1 >> sh8;
        u32x4 b0, b1;
        b0.x = (w0 & dq.lo) | dq.magic;
        b0.y = (w0 & dq.hi) | dq.magic;
        b0.z = (t0 & dq.lo) | dq.magic;
        b0.w = (t0 & dq.hi) | dq.magic;
        b1.x = (w1 & dq.lo) | dq.magic;
        b1.y = (w1 & dq.hi) | dq.magic;
        b1.z = (t1 & dq.lo) | dq.magic;
        b1.w = (t1 & dq.hi) | dq.magic;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, __builtin_bit_cast(half8, b0), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, __builtin_bit_cast(half8, b1), acc, 0, 0, 0);
        SbWord<SB_BF16> sw = sbw[i];
        opaque_sb(sw);   // decoded here, not once above the chunk loop (two registers a group instead of one)
        float s, b;
        sb_values<SB_BF16>(sw, s, b);
        const float4* osp = reinterpret_cast<const float4*>(os_l + g * 16 + 4 * kb);
        const float4 o01 = osp[0], o23 = osp[1];   // (1024 O, Sx) of tokens 4 kb .. 4 kb + 3
        y[0] = fmaf(s, acc[0] - o01.x, fmaf(b, o01.y, y[0]));
        y[1] = fmaf(s, acc[1] - o01.z, fmaf(b, o01.w, y[1]));
        y[2] = fmaf(s, acc[2] - o23.x, fmaf(b, o23.y, y[2]));
        y[3] = fmaf(s, acc[3] - o23.z, fmaf(b, o23.w, y[3]));
        __builtin_amdgcn_sched_barrier(0);   // one group at a time: the next group's B is made after this one
      }
    }
    // the waves' partial sums, added in wave order; thread (m, nn) finishes token m, row nn of each tile
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave * 256 + (4 * kb + i) * 16 + n] = y[i];
    __syncthreads();
    {
      const int m = threadIdx.x >> 4, nn = threadIdx.x & 15;
      float* out = shared ? a.out_shared : a.out_routed;
      const int out_len = shared ? a.out_len_shared : a.out_len_routed;
      if (m < nlive) {
        const float sc = ef_l[m];
        for (int tt = 0; tt < tpb; ++tt) {
          auto total = [&](int col) {
            float acc = red[(tt * wk) * 256 + m * 16 + col];
            for (int w = 1; w < wk; ++w) acc += red[(tt * wk + w) * 256 + m * 16 + col];
            return acc;
          };
          const int t_out = u * tpb + tt;
          if (a.gate_up) {
            if (nn < 8)
              out[(int64_t)orow_l[m] * out_len + t_out * 8 + nn] =
                  valid ? activation(sc * total(nn), a.act) * (sc * total(nn + 8)) : __builtin_nanf("");
          } else {
            out[(int64_t)orow_l[m] * out_len + t_out * 16 + nn] = valid ? sc * total(nn) : __builtin_nanf("");
          }
        }
      }
    }
    __syncthreads();   // red, os and the token rows are rewritten by the next chunk
  }
}

}  // namespace

moe_status launch_stage_rows(const void* x, bool x_bf16, int rows, int K, const StagedRows& out, hipStream_t s) {
  if (rows <= 0) return MOE_OK;
  if (x_bf16) hipLaunchKernelGGL((stage_rows_kernel<uint16_t>), dim3(rows), dim3(kThreadsM), 0, s,
                                 static_cast<const uint16_t*>(x), K, out);
  else hipLaunchKernelGGL((stage_rows_kernel<float>), dim3(rows), dim3(kThreadsM), 0, s, static_cast<const float*>(x), K,
                          out);
  return check_launch("stage_rows_kernel");
}

int mfma_waves_per_tile(int K) {
  const int G = K / 64;
  return G <= 12 ? 1 : G <= 24 ? 2 : 4;
}

moe_status launch_grouped_mfma(const MfmaArgs& a, int gmax, bool sb_bf16, hipStream_t s) {
  const int n_routed = a.n_routed_blocks > 0 ? gmax * a.n_routed_blocks : 0;
  const dim3 grid(a.n_shared_blocks + n_routed);
  if (grid.x == 0) return MOE_OK;
  int per_wave = 0, kmax = 0;
  if (a.n_shared_blocks > 0) {
    per_wave = (a.K_shared / 64 + a.wk_shared - 1) / a.wk_shared;
    kmax = a.K_shared;
  }
  if (n_routed > 0) {
    per_wave = max(per_wave, (a.K_routed / 64 + a.wk_routed - 1) / a.wk_routed);
    kmax = max(kmax, a.K_routed);
  }
  const size_t lds = mfma_lds_bytes(kmax);
  auto go = [&](auto ng) {
    constexpr int NG = decltype(ng)::value;
    if (sb_bf16) hipLaunchKernelGGL((grouped_mfma_kernel<NG, true>), grid, dim3(kThreadsM), lds, s, a);
    else hipLaunchKernelGGL((grouped_mfma_kernel<NG, false>), grid, dim3(kThreadsM), lds, s, a);
    return check_launch("grouped_mfma_kernel");
  };
  if (per_wave <= 4) return go(std::integral_constant<int, 4>());
  if (per_wave <= 8) return go(std::integral_constant<int, 8>());
  if (per_wave <= 12) return go(std::integral_constant<int, 12>());
  if (per_wave <= 16) return go(std::integral_constant<int, 16>());
  if (per_wave <= 24) return go(std::integral_constant<int, 24>());
  return go(std::integral_constant<int, 32>());
}

}  // namespace moeq4
