// Grouped expert products for T > 1 tokens on the matrix cores ([G26] "Le pipeline de traitement": a
// prompt's tokens processed together share each expert's weights; [REMIO] "L'affirmation des 2 Go fait de
// la bande passante SSD la nouvelle contrainte": 4-bit affine MLX weights).
//
// With several tokens per expert the one-token kernels' dot2 chains become the bottleneck (every token
// repeats the dequantization and 36 VALU operations per 32 codes).  Here 16 weight rows are multiplied with
// up to 16 tokens at a time by v_mfma_f32_16x16x32_f16:
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
// and 8 g + 2 kb + 1 of its row, and the A lanes hold the matching 32 staged bytes of their token (k order
// within a group is a permutation shared by A and B).  The waves of a tile split the row's groups; their
// 16 x 16 partial results are added in LDS in wave order.  Results match the one-token kernels within
// rounding (the activation is scaled per token row, not per 32 values).
#include <map>
#include <mutex>
#include <tuple>

#include "q4_grouping.h"

namespace moeq4 {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreadsM = 256;                     // staging block
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
// Blocks [0, rows0) stage the rows of j0, the rest those of j1 (the down launch stages the routed and the
// shared hidden vectors together).
template <typename XT>
struct StageJob {
  const XT* x;
  int K;
  StagedRows out;
};

template <typename XT>
__device__ __forceinline__ void stage_row(const StageJob<XT>& j, int row) {
  __shared__ float wmax[kThreadsM / 64];
  const XT* __restrict__ x = j.x;
  const int K = j.K;
  const StagedRows out = j.out;
  const int t = threadIdx.x;
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

template <typename XT>
__global__ __launch_bounds__(kThreadsM) void stage_rows_kernel(StageJob<XT> j0, StageJob<XT> j1, int rows0) {
  const bool second = (int)blockIdx.x >= rows0;
  stage_row<XT>(second ? j1 : j0, second ? (int)blockIdx.x - rows0 : (int)blockIdx.x);
}

// The grouping of the pairs (block 0) and the staging of the tokens (blocks 1 .. rows) in one launch: the
// two are independent and each alone is a launch of a few microseconds.
constexpr int kPlanBlocks = 8;   // blocks of the grouping launch that write the products' descriptors (half each)
struct GroupJob {
  const int32_t* ids;
  int P, n_valid;
  int32_t *n_groups, *perm, *n_chunks;
  int4 *groups, *chunks;
  int4 *plan0, *plan1;    // work descriptors of the two product launches that follow, or NULL
  SplitShape shape0, shape1;
};

template <typename XT>
__global__ __launch_bounds__(kThreadsM) void group_and_stage_kernel(GroupJob g, StageJob<XT> j) {
  static_assert(kThreadsM == kGroupThreads, "one block shape for both");
  // blocks: 0 groups, 1 .. rows stage, the last kPlanBlocks (with descriptors) write the descriptors
  const int rows = (int)gridDim.x - 1 - ((g.plan0 || g.plan1) ? kPlanBlocks : 0);
  if (blockIdx.x == 0) {
    group_pairs_block(g.ids, g.P, g.n_valid, g.n_groups, g.groups, g.perm, g.n_chunks, g.chunks);
  } else if ((int)blockIdx.x <= rows) {
    stage_row<XT>(j, (int)blockIdx.x - 1);
  } else {
    // the first half of these blocks write the first launch's descriptors, the second half the second's
    const int q = (int)blockIdx.x - 1 - rows, half = kPlanBlocks / 2, i = q / half;
    PlanOut po{{nullptr, nullptr}, {g.shape0, g.shape1}};
    po.plan[i] = i == 0 ? g.plan0 : g.plan1;
    plan_share(po, g.ids, g.P, g.n_valid, q % half, half);
  }
}

constexpr int kWavesG = 4;                 // wavefronts of a grouped-product block
constexpr int kThreadsG = 64 * kWavesG;

// A wave's code words of one step, staged in LDS: 16 rows of NG groups (32 bytes each), rows padded by 16
// bytes so that the 16 rows of an MFMA operand read fall on different banks.
constexpr int slice_stride(int ng) { return ng * 32 + 16; }

// Dynamic LDS of a block: red [4][16][16] fp32, the waves' code-word slices [4][16][stride], os [G][16]
// float2, ef [16], rows [16] (stage and output rows)
inline size_t mfma_lds_bytes(int K, int ng) {
  return (size_t)kWavesG * 256 * 4 + (size_t)kWavesG * 16 * slice_stride(ng) + (size_t)(K / 64) * 16 * 8 + 16 * 4 +
         16 * 4 * 2;
}

template <bool SB_BF16>
__device__ __forceinline__ void opaque_sb(SbWord<SB_BF16>& w);
template <>
__device__ __forceinline__ void opaque_sb<true>(SbWord<true>& w) {
  asm volatile("" : "+v"(w.s));
}
template <>
__device__ __forceinline__ void opaque_sb<false>(SbWord<false>&) {}

// Buffer loads: a uniform base (the resource, in SGPRs) + a per-lane 32-bit offset + a uniform offset, so
// that per-group loads need no 64-bit address registers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, 0x00020000);
}
// Scale/bias of 16 bytes per load: 4 groups (bf16 pairs) or 2 (fp32 pairs) of a row; word i of a load.
template <bool SB_BF16>
__device__ __forceinline__ SbWord<SB_BF16> sb_word(const u32x4& v, int i) {
  SbWord<SB_BF16> w;
  if constexpr (SB_BF16) {
    w.s = v[i];
    w.b = 0;
  } else {
    w.s = v[2 * i];
    w.b = v[2 * i + 1];
  }
  return w;
}

// One block's work: steps [s0, s1) of one matrix (a step = 4 / wk tiles of 16 rows, one per group of wk
// waves) for a list of tokens, 16 at a time.  Per chunk of tokens each wave loads its A operands (its
// groups' staged activations) once; per step it stages the step's code words in its LDS slice and at once
// requests the next step's (and the scale/bias words as soon as they are unpacked), so a step's weights are
// in flight while the previous step is multiplied, reduced and stored.
template <int NG, bool SB_BF16>
__device__ __forceinline__ void mfma_item(const MfmaArgs& a, bool shared, int e, bool valid, int start, int count,
                                          int s0, int s1, uint32_t* lds) {
  float* red = reinterpret_cast<float*>(lds);                      // [4 waves][16 tokens][16 rows]
  const Pool P = shared ? a.shared : a.routed;                      // copies: held in SGPRs, not re-read
  const StagedRows xs = shared ? a.xs_shared : a.xs_routed;
  const int K = shared ? a.K_shared : a.K_routed, wk = shared ? a.wk_shared : a.wk_routed;
  const int n_tiles = shared ? a.tiles_shared : a.tiles_routed;
  float* const out = shared ? a.out_shared : a.out_routed;
  const int out_len = shared ? a.out_len_shared : a.out_len_routed;
  const int G = K / 64, tps = kWavesG / wk;
  constexpr int kStride = slice_stride(NG);                         // bytes
  char* slice = reinterpret_cast<char*>(lds) + kWavesG * 256 * 4;   // [4 waves][16 rows][kStride]
  float2* os_l = reinterpret_cast<float2*>(slice + kWavesG * 16 * kStride);   // [G][16]
  float* ef_l = reinterpret_cast<float*>(os_l + G * 16);
  int* srow_l = reinterpret_cast<int*>(ef_l + 16);
  int* orow_l = srow_l + 16;

  // the wave index through readfirstlane, so that the compiler sees the group range as wave-uniform
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63, n = lane & 15,
            kb = lane >> 4;
  const int part = wave % wk, wt = wave / wk;
  const int g0 = (part * G) / wk, nw = ((part + 1) * G) / wk - g0;
  const char* rec = P.base + (int64_t)e * P.record_bytes;
  const int sb_row = G * (SB_BF16 ? 4 : 8);
  const int mat_rows = a.gate_up ? 2 * P.F : n_tiles * 16;
  const __amdgpu_buffer_rsrc_t qr = buf_rsrc(rec + P.off_q, (uint32_t)mat_rows * (K / 2));
  const __amdgpu_buffer_rsrc_t sr = buf_rsrc(rec + P.off_sb, (uint32_t)mat_rows * sb_row);
  const __amdgpu_buffer_rsrc_t ar = buf_rsrc(xs.xq, (uint32_t)xs.rows * K * 2);
  // this lane's row in tile t (tiles past the matrix read its last tile; their results are not stored)
  auto row_of = [&](int t) {
    t = min(t, n_tiles - 1);
    return a.gate_up ? (n < 8 ? t * 8 + n : P.F + t * 8 + (n - 8)) : t * 16 + n;
  };

  for (int c0 = 0; c0 < count; c0 += 16) {
    const int nlive = min(16, count - c0);
    // the chunk's tokens: staged row, output row, 2^e.  Slots past the last token repeat the first token's
    // staged row, so their A loads fall on lines the wave reads anyway; their results are not stored.
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
      // (1024 O, Sx) of every (group, token): thread i stages group i / 16 + 16 r of token i % 16
      constexpr int kRep = (NG * kWavesG + 15) / 16;   // G <= 4 NG, so G * 16 <= kRep * 256
      const int nrep = (G * 16 + kThreadsG - 1) / kThreadsG;
      const float2* orow = xs.os + (int64_t)srow_l[threadIdx.x & 15] * G;
      const int gq = threadIdx.x >> 4;
      float2 ov[kRep];
#pragma unroll
      for (int r = 0; r < kRep; ++r)
        if (r < nrep) ov[r] = orow[min(gq + 16 * r, G - 1)];
#pragma unroll
      for (int r = 0; r < kRep; ++r)
        if (r < nrep && gq + 16 * r < G) os_l[threadIdx.x + r * kThreadsG] = ov[r];
    }
    // A of this wave's groups for the whole chunk: token n's 32 bytes of each group (index clamped into
    // the row for slots past the wave's range)
    const int a_off = (srow_l[n] * K + 16 * kb) * 2;
    half8 A0[NG], A1[NG];
#pragma unroll
    for (int i = 0; i < NG; ++i) {
      const int gi = min(g0 + i, G - 1);
      A0[i] = __builtin_bit_cast(half8, __builtin_amdgcn_raw_buffer_load_b128(ar, a_off, gi * 128, 0));
      A1[i] = __builtin_bit_cast(half8, __builtin_amdgcn_raw_buffer_load_b128(ar, a_off + 16, gi * 128, 0));
    }
    // the first step's code words and scale/bias (record 0 for an invalid expert: never used).  Plain
    // loads, not streaming ones: a lane reads 8 bytes of a 128-byte line whose other bytes the row's next
    // groups read soon after, so the line should stay in L2 (streaming loads measured 17% slower).
    // scale/bias: the 4 lanes of a row read the same 16 bytes (one request), a load per SPL groups; bytes
    // past the row's groups belong to slots that carry weight zero (or lie outside the buffer: zeros)
    constexpr int SPL = SB_BF16 ? 4 : 2, NS = (NG + SPL - 1) / SPL, SB_BYTES = SB_BF16 ? 4 : 8;
    // code words: each wave streams its 16 rows x NG groups as whole 16-byte pieces of the rows (22 lanes
    // cover a row's 352 bytes at 11 groups, so a load instruction reads whole 128-byte lines), writes them
    // to its LDS slice and reads them back in the MFMA operand layout
    constexpr int CPR = 2 * NG, NCH = (16 * CPR + 63) / 64;   // 16-byte pieces per row; loads per lane
    char* my_slice = slice + wave * 16 * kStride;
    // piece j of a lane: row (lane + 64 j) / CPR of the tile, column (lane + 64 j) % CPR (lanes past the
    // last piece repeat it and do not store it); recomputed where used rather than held in registers
    auto piece_c = [&](int j) { return min(lane + 64 * j, 16 * CPR - 1); };
    auto piece_off = [&](int t, int j) {   // byte offset of piece j of tile t in the matrix (group g0 first)
      t = min(t, n_tiles - 1);
      const int c = piece_c(j), rt = c / CPR;
      const int row = a.gate_up ? (rt < 8 ? t * 8 + rt : P.F + t * 8 + (rt - 8)) : t * 16 + rt;
      return row * (K / 2) + (c % CPR) * 16;
    };
    u32x4 wq[NCH];
    u32x4 sbv[NS];
    {
      const int r = row_of(s0 * tps + wt);
      const int s_off = r * sb_row;
#pragma unroll
      for (int j = 0; j < NS; ++j) sbv[j] = __builtin_amdgcn_raw_buffer_load_b128(sr, s_off, (g0 + j * SPL) * SB_BYTES, 0);
#pragma unroll
      for (int j = 0; j < NCH; ++j) wq[j] = __builtin_amdgcn_raw_buffer_load_b128(qr, piece_off(s0 * tps + wt, j), g0 * 32, 0);
    }
    __syncthreads();   // os, ef and the token rows are in LDS

    for (int s = s0; s < s1; ++s) {
      const Dequant dq = opaque_dequant();   // the dequantized words stay inside the step loop
      uint32_t sh8 = 8;
      asm volatile("" : "+v"(sh8));
      // the groups' (1024 O, Sx) are read from LDS in every step, not held in registers across steps
      int os_off = 4 * kb;
      asm volatile("" : "+v"(os_off));
      // the next step's rows (the last step reads its own again: cache hits, no branch)
      const int tn = min(s + 1, s1 - 1) * tps + wt;
      const int rn = row_of(tn), sn_off = rn * sb_row;
      // this step's pieces into the slice, then the next step's requested into the same registers (the
      // pieces past a row's groups, or past the matrix, read zeros or other rows: never multiplied)
#pragma unroll
      for (int j = 0; j < NCH; ++j)
        if (lane + 64 * j < 16 * CPR) {
          const int c = lane + 64 * j;
          *reinterpret_cast<u32x4*>(my_slice + (c / CPR) * kStride + (c % CPR) * 16) = wq[j];
        }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < NCH; ++j) wq[j] = __builtin_amdgcn_raw_buffer_load_b128(qr, piece_off(tn, j), g0 * 32, 0);
      // the MFMA operand words: row n, group i, words 2 kb and 2 kb + 1, read two groups ahead
      const char* opnd = my_slice + n * kStride + kb * 8;
      u32x2 qr3[3];
      qr3[0] = *reinterpret_cast<const u32x2*>(opnd);
      if (NG > 1) qr3[1] = *reinterpret_cast<const u32x2*>(opnd + 32);
      f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < NG; ++i) {
        if (i + 2 < NG) qr3[(i + 2) % 3] = *reinterpret_cast<const u32x2*>(opnd + (i + 2) * 32);
        const u32x2 qi = qr3[i % 3];
        const uint32_t w0 = qi.x, w1 = qi.y, t0 = w0 >> sh8, t1 = w1 >> sh8;
        u32x4 b0, b1;
        b0.x = (w0 & dq.lo) | dq.magic;
        b0.y = (w0 & dq.hi) | dq.magic;
        b0.z = (t0 & dq.lo) | dq.magic;
        b0.w = (t0 & dq.hi) | dq.magic;
        b1.x = (w1 & dq.lo) | dq.magic;
        b1.y = (w1 & dq.hi) | dq.magic;
        b1.z = (t1 & dq.lo) | dq.magic;
        b1.w = (t1 & dq.hi) | dq.magic;
        SbWord<SB_BF16> sw = sb_word<SB_BF16>(sbv[i / SPL], i % SPL);
        opaque_sb(sw);
        float sc, bi;
        sb_values<SB_BF16>(sw, sc, bi);
        // slots past the wave's groups multiply the row's last group again, with weight zero: no branch, so
        // the unpacking above cannot sink below the reload
        if (i >= nw) sc = bi = 0.f;
        // the barrier keeps the unpacking above the reload, so the new scale/bias words reuse the old ones'
        // registers instead of being copied back
        __builtin_amdgcn_sched_barrier(0);
        const int gi = min(g0 + i, G - 1);
        if (i % SPL == SPL - 1 || i == NG - 1)
          sbv[i / SPL] = __builtin_amdgcn_raw_buffer_load_b128(sr, sn_off, (g0 + (i / SPL) * SPL) * SB_BYTES, 0);
        {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A0[i], __builtin_bit_cast(half8, b0), acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A1[i], __builtin_bit_cast(half8, b1), acc, 0, 0, 0);
          const float4* osp = reinterpret_cast<const float4*>(os_l + gi * 16 + os_off);
          const float4 o01 = osp[0], o23 = osp[1];   // (1024 O, Sx) of tokens 4 kb .. 4 kb + 3
          y[0] = fmaf(sc, acc[0] - o01.x, fmaf(bi, o01.y, y[0]));
          y[1] = fmaf(sc, acc[1] - o01.z, fmaf(bi, o01.w, y[1]));
          y[2] = fmaf(sc, acc[2] - o23.x, fmaf(bi, o23.y, y[2]));
          y[3] = fmaf(sc, acc[3] - o23.z, fmaf(bi, o23.w, y[3]));
        }
        __builtin_amdgcn_sched_barrier(0);   // one group at a time
      }
      // the waves' partial tiles, added in wave order
#pragma unroll
      for (int i = 0; i < 4; ++i) red[wave * 256 + (4 * kb + i) * 16 + n] = y[i];
      __syncthreads();
      for (int idx = threadIdx.x; idx < tps * 256; idx += kThreadsG) {
        const int tt = idx >> 8, m = (idx >> 4) & 15, nn = idx & 15;
        const int tile = s * tps + tt;
        if (m >= nlive || tile >= n_tiles || (a.gate_up && nn >= 8)) continue;
        auto total = [&](int col) {
          float v = red[(tt * wk) * 256 + m * 16 + col];
          for (int w = 1; w < wk; ++w) v += red[(tt * wk + w) * 256 + m * 16 + col];
          return v;
        };
        const float sc = ef_l[m];
        float v;
        if (!valid) v = __builtin_nanf("");
        else if (a.gate_up) v = activation(sc * total(nn), a.act) * (sc * total(nn + 8));
        else v = sc * total(nn);
        out[(int64_t)orow_l[m] * out_len + tile * (a.gate_up ? 8 : 16) + nn] = v;
      }
      __syncthreads();   // red is rewritten by the next step
    }
  }
}

// ---------------------------------------------------------------------------------------------------------
// The ring variant (at most 11 groups per wave, every row length up to 44 groups with 4 waves a tile).
//
// Streaming was the limit of the register-staged item above: with the activations of a chunk held in
// registers a wave has room for one step of code words in flight, and at two waves per SIMD that is about
// 48 KiB per compute unit, too little to cover the memory latency under full load.  Here the code words and
// the scale/bias words go from memory straight into LDS (buffer loads with the LDS bit), two slots per wave:
// while step s is multiplied, steps s + 1 and s + 2 are in flight, about 100 KiB per compute unit, and no
// register holds them.  At the start of a step the wave waits for its slot's loads (a vmcnt that leaves the
// next step's loads in flight), reads the slot into registers and refills it with step s + 2.
//
// The wait is written by hand: the compiler's own wait before an LDS read that a load may have written is
// vmcnt(0) whenever a store is also outstanding, which would drain the ring at every step.  The slot reads
// are therefore inline assembly (ending in their own lgkmcnt(0)), invisible to the compiler as LDS reads,
// after an explicit vmcnt(N), N the loads issued after the slot's (the next step's).  Loads return in order,
// so the wait holds whatever the stores do; the outputs of step s are stored at the start of step s + 1,
// before its loads are issued, so that they are old by the time a wait could cover them.
//
// The products also drop the 1024 offset of the code-to-fp16 step: a code word masked with 0x000F000F (and
// its siblings) is, as fp16 bits, the subnormal pair (n0 2^-24, n4 2^-24), which the matrix cores multiply
// exactly.  A group's MFMA sum is then sum_c q_c x_c 2^-(e+24) with no cancellation, and
//   y = 2^(e+24) (sum_g scale_g acc_g + sum_g bias_g Sx_g 2^-24),
// the bias sum as fp32 MFMAs (16 tokens x 4 groups x 16 rows) on the chunk's Sx values.
template <int NG, bool SB_BF16>
struct Ring {
  static constexpr int kSbWords = SB_BF16 ? 1 : 2;          // 32-bit scale/bias words per (row, group)
  static constexpr int kCodeLoads = (NG + 1) / 2;           // 1 KiB loads (two groups of 16 rows each)
  static constexpr int kCode = kCodeLoads * 1024;           // bytes of a wave's slot (the odd group's pad)
  static constexpr int kSbUsed = 16 * NG * kSbWords;        // scale/bias words of a wave's step
  static constexpr int kSbLoads = (kSbUsed + 63) / 64;      // 256-byte loads (one word a lane)
  static constexpr int kSb = kSbLoads * 64;                 // words of a wave's slot
  static constexpr int kBias = (NG + 3) / 4;                // bias MFMAs (4 groups each)
  static constexpr int kLoads = kCodeLoads + kSbLoads;      // loads of one step
  static_assert(kLoads <= 31, "two steps of loads must fit the 6-bit vmcnt");
  static_assert(NG <= 11, "the slot reads are two asm blocks of at most 11 pairs");
};

typedef __attribute__((address_space(3))) void* lds_ptr_t;
constexpr int kNt = 2;   // cache-policy operand of a buffer load: nontemporal

// s_waitcnt vmcnt(N) (the other counters not waited for), as a builtin so that the compiler counts it.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "6-bit vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// The block's LDS writes done, then the barrier.  __syncthreads would also wait for every load in flight
// (the slot loads write LDS), which would drain the ring at each step.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Reads of a slot in inline assembly (the compiler does not see them as LDS reads, so it places no wait of
// its own for the slot's loads): pairs of 32-bit words at byte offsets i * GS and words at i * 4 * W from
// two base addresses, after an explicit vmcnt(N); each block ends with its reads complete.
#define MOE_RD64(i) "ds_read_b64 %" #i ", %[pa] offset:" #i "*%[gs]\n\t"
template <int N, int NG, int W, int GS>
__device__ __forceinline__ void read_slot(const char* pa, const uint32_t* pb, const uint32_t* pc, u32x2 (&q)[NG],
                                          uint32_t (&sw)[NG], uint32_t (&bw)[(NG + 3) / 4]) {
  static_assert(NG == 4 || NG == 8 || NG == 11, "slot shapes");
  const uint32_t ua = (uint32_t)(uintptr_t)pa, ub = (uint32_t)(uintptr_t)pb, uc = (uint32_t)(uintptr_t)pc;
  if constexpr (NG == 4) {
    asm volatile("s_waitcnt vmcnt(%[n])\n\t" MOE_RD64(0) MOE_RD64(1) MOE_RD64(2) MOE_RD64(3) "s_waitcnt lgkmcnt(0)"
                 : "=&v"(q[0]), "=&v"(q[1]), "=&v"(q[2]), "=&v"(q[3])
                 : [pa] "v"(ua), [n] "n"(N), [gs] "n"(GS)
                 : "memory");
  } else if constexpr (NG == 8) {
    asm volatile("s_waitcnt vmcnt(%[n])\n\t" MOE_RD64(0) MOE_RD64(1) MOE_RD64(2) MOE_RD64(3) MOE_RD64(4) MOE_RD64(5)
                     MOE_RD64(6) MOE_RD64(7) "s_waitcnt lgkmcnt(0)"
                 : "=&v"(q[0]), "=&v"(q[1]), "=&v"(q[2]), "=&v"(q[3]), "=&v"(q[4]), "=&v"(q[5]), "=&v"(q[6]),
                   "=&v"(q[7])
                 : [pa] "v"(ua), [n] "n"(N), [gs] "n"(GS)
                 : "memory");
  } else {
    asm volatile("s_waitcnt vmcnt(%[n])\n\t" MOE_RD64(0) MOE_RD64(1) MOE_RD64(2) MOE_RD64(3) MOE_RD64(4) MOE_RD64(5)
                     MOE_RD64(6) MOE_RD64(7) MOE_RD64(8) MOE_RD64(9) MOE_RD64(10) "s_waitcnt lgkmcnt(0)"
                 : "=&v"(q[0]), "=&v"(q[1]), "=&v"(q[2]), "=&v"(q[3]), "=&v"(q[4]), "=&v"(q[5]), "=&v"(q[6]),
                   "=&v"(q[7]), "=&v"(q[8]), "=&v"(q[9]), "=&v"(q[10])
                 : [pa] "v"(ua), [n] "n"(N), [gs] "n"(GS)
                 : "memory");
  }
  // scale words (group i at i * 4 W) and bias words (group 4 j + kb at pc + 16 j W); the slot's loads are
  // already complete
  constexpr int B = (NG + 3) / 4;
  uint32_t t[11 + 3];
#define MOE_S(i) "ds_read_b32 %" #i ", %[pb] offset:" #i "*%[w4]\n\t"
  if constexpr (NG == 4) {
    asm volatile(MOE_S(0) MOE_S(1) MOE_S(2) MOE_S(3) "ds_read_b32 %4, %[pc]\n\ts_waitcnt lgkmcnt(0)"
                 : "=&v"(t[0]), "=&v"(t[1]), "=&v"(t[2]), "=&v"(t[3]), "=&v"(t[4])
                 : [pb] "v"(ub), [pc] "v"(uc), [w4] "n"(4 * W)
                 : "memory");
  } else if constexpr (NG == 8) {
    asm volatile(MOE_S(0) MOE_S(1) MOE_S(2) MOE_S(3) MOE_S(4) MOE_S(5) MOE_S(6) MOE_S(7)
                 "ds_read_b32 %8, %[pc]\n\tds_read_b32 %9, %[pc] offset:%[o1]\n\ts_waitcnt lgkmcnt(0)"
                 : "=&v"(t[0]), "=&v"(t[1]), "=&v"(t[2]), "=&v"(t[3]), "=&v"(t[4]), "=&v"(t[5]), "=&v"(t[6]),
                   "=&v"(t[7]), "=&v"(t[8]), "=&v"(t[9])
                 : [pb] "v"(ub), [pc] "v"(uc), [o1] "n"(16 * W), [w4] "n"(4 * W)
                 : "memory");
  } else {
    asm volatile(MOE_S(0) MOE_S(1) MOE_S(2) MOE_S(3) MOE_S(4) MOE_S(5) MOE_S(6) MOE_S(7) MOE_S(8) MOE_S(9) MOE_S(10)
                 "ds_read_b32 %11, %[pc]\n\tds_read_b32 %12, %[pc] offset:%[o1]\n\t"
                 "ds_read_b32 %13, %[pc] offset:%[o2]\n\ts_waitcnt lgkmcnt(0)"
                 : "=&v"(t[0]), "=&v"(t[1]), "=&v"(t[2]), "=&v"(t[3]), "=&v"(t[4]), "=&v"(t[5]), "=&v"(t[6]),
                   "=&v"(t[7]), "=&v"(t[8]), "=&v"(t[9]), "=&v"(t[10]), "=&v"(t[11]), "=&v"(t[12]), "=&v"(t[13])
                 : [pb] "v"(ub), [pc] "v"(uc), [o1] "n"(16 * W), [o2] "n"(32 * W), [w4] "n"(4 * W)
                 : "memory");
  }
#undef MOE_S
#pragma unroll
  for (int i = 0; i < NG; ++i) sw[i] = t[i];
#pragma unroll
  for (int j = 0; j < B; ++j) bw[j] = t[NG + j];
}
#undef MOE_RD64

// The LDS of a block of the ring kernel: each wave's two slots of code and scale/bias words, the partial
// tiles by step parity ([wave][16 tokens][16 rows]), and the chunk's token scales and rows.
template <int NG, bool SB_BF16>
struct RingLds {
  using R = Ring<NG, SB_BF16>;
  __align__(16) char code0[kWavesG * R::kCode];
  __align__(16) char code1[kWavesG * R::kCode];
  __align__(16) uint32_t sbl0[kWavesG * R::kSb];
  __align__(16) uint32_t sbl1[kWavesG * R::kSb];
  float red0[kWavesG * 256], red1[kWavesG * 256];
  float ef_l[16];
  int srow_l[16], orow_l[16];
};

// CONTIG: the item's tiles are contiguous runs of whole rows (below); the two forms are separate
// instantiations, each with the registers of one.
template <int NG, bool SB_BF16, bool CONTIG>
__device__ __forceinline__ void ring_item(const MfmaArgs& a, bool shared, int e, bool valid, int start, int count,
                                          int s0, int s1, RingLds<NG, SB_BF16>& lds) {
  using R = Ring<NG, SB_BF16>;
  constexpr int W = R::kSbWords;
  char* const code0 = lds.code0;
  char* const code1 = lds.code1;
  uint32_t* const sbl0 = lds.sbl0;
  uint32_t* const sbl1 = lds.sbl1;
  float* const red0 = lds.red0;
  float* const red1 = lds.red1;
  float* const ef_l = lds.ef_l;
  int* const srow_l = lds.srow_l;
  int* const orow_l = lds.orow_l;

  const Pool P = shared ? a.shared : a.routed;
  const StagedRows xs = shared ? a.xs_shared : a.xs_routed;
  const int K = shared ? a.K_shared : a.K_routed, wk = shared ? a.wk_shared : a.wk_routed;
  const int n_tiles = shared ? a.tiles_shared : a.tiles_routed;
  float* const out = shared ? a.out_shared : a.out_routed;
  const int out_len = shared ? a.out_len_shared : a.out_len_routed;
  const int G = K / 64, tps = kWavesG / wk;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63, n = lane & 15,
            kb = lane >> 4;
  const int part = wave % wk, wt = wave / wk;
  const int g0 = (part * G) / wk, nw = ((part + 1) * G) / wk - g0;
  const char* rec = P.base + (int64_t)e * P.record_bytes;
  const int sb_row = G * 4 * W;
  const int mat_rows = a.gate_up ? 2 * P.F : n_tiles * 16;
  const __amdgpu_buffer_rsrc_t qr = buf_rsrc(rec + P.off_q, (uint32_t)mat_rows * (K / 2));
  const __amdgpu_buffer_rsrc_t sr = buf_rsrc(rec + P.off_sb, (uint32_t)mat_rows * sb_row);
  const __amdgpu_buffer_rsrc_t ar = buf_rsrc(xs.xq, (uint32_t)xs.rows * K * 2);
  // row r of a tile: tile t's rows start t * rpt rows further (gate/up: 8 gate rows, then the 8 matching up
  // rows F further)
  const int rpt = a.gate_up ? 8 : 16;
  auto row0 = [&](int r) { return a.gate_up ? (r < 8 ? r : P.F + r - 8) : r; };
  // lane offsets of the loads into the slots.  Code load j, lane l: group 2 j + l / 32 of the wave, half
  // (l / 16) % 2 of it, row l % 16 (so group i of the slot is 512 bytes at i * 512, half h at + 256 h, row r
  // at + 16 r: an operand read of one group is 512 contiguous bytes).  Scale/bias load j, lane l: word
  // 64 j + l of the wave's [16 rows][NG groups][W] words.  Lanes past the wave's groups read other bytes of
  // the matrix, or zeros past its end, into the slot's padding or into groups that carry weight 0.
  //
  // A wave that multiplies whole rows of the plain 16-row layout (down, wk == 1) owns a tile that is one
  // contiguous run of 16 K / 2 bytes, starting on a 128-byte line (K is a multiple of 64 and records are
  // 256-byte aligned).  It is loaded as is, 1 KiB per load, so that every load covers whole lines and can be
  // marked nontemporal (a streaming probe moved 7.0 TB/s so against 6.2 with the default policy; half-line
  // pieces do not gain); the slot then holds the tile row-major (row r at r K / 2, group i at + 32 i), and
  // the last load's lanes past the tile's end read nothing.
  constexpr bool contig = CONTIG;
  const uint32_t tile_bytes = 16u * (uint32_t)(K / 2);
  const uint32_t code_lane = contig ? 16u * (uint32_t)lane
                                    : (uint32_t)(row0(n) * (K / 2) + (lane >> 5) * 32 + ((lane >> 4) & 1) * 16 + g0 * 32);
  uint32_t sb_lane[R::kSbLoads];
#pragma unroll
  for (int j = 0; j < R::kSbLoads; ++j) {
    const int w = min(64 * j + lane, R::kSbUsed - 1);
    const int r = w / (NG * W), c = w % (NG * W);
    sb_lane[j] = (uint32_t)(row0(r) * sb_row + g0 * 4 * W + 4 * c);
  }
  // step s's words into slot SL; past the last step the offsets lie outside the buffers (zeros, no traffic),
  // so that every step issues the same loads and the waits stay exact
  auto issue = [&](auto slot_c, int s) __attribute__((always_inline)) {
    constexpr int SL = decltype(slot_c)::value;
    char* cb = (SL ? code1 : code0) + wave * R::kCode;
    uint32_t* sbb = (SL ? sbl1 : sbl0) + wave * R::kSb;
    const int t = min(s * tps + wt, n_tiles - 1);
    const uint32_t cbase = s < s1 ? (uint32_t)(t * rpt) * (uint32_t)(K / 2) : 0x80000000u;
    const uint32_t sbase = s < s1 ? (uint32_t)(t * rpt) * (uint32_t)sb_row : 0x80000000u;
    if constexpr (contig) {
      constexpr int L = R::kCodeLoads;
      const uint32_t vo = cbase + code_lane;
      const uint32_t vl = code_lane + 1024u * (L - 1) < tile_bytes ? vo + 1024u * (L - 1) : 0x80000000u;
#pragma unroll
      for (int j = 0; j < L - 1; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(qr, (lds_ptr_t)(cb + 1024 * j), 16, vo, 1024 * j, 0, kNt);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(qr, (lds_ptr_t)(cb + 1024 * (L - 1)), 16, vl, 0, 0, kNt);
    } else {
#pragma unroll
      for (int j = 0; j < R::kCodeLoads; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(qr, (lds_ptr_t)(cb + 1024 * j), 16, cbase + code_lane + 64 * j, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < R::kSbLoads; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(sr, (lds_ptr_t)(sbb + 64 * j), 4, sbase + sb_lane[j], 0, 0, 0);
  };

  for (int c0 = 0; c0 < count; c0 += 16) {
    const int nlive = min(16, count - c0);
    // the chunk's tokens (staged row and output row; slots past the last token repeat the first token's
    // staged row, their results are not stored), loaded before the first step's loads so that they do not
    // wait behind them; the step's loads depend on the expert only
    int pr = 0;
    if ((int)threadIdx.x < 16) {
      const int m = threadIdx.x;
      const int mm = m < nlive ? m : 0;
      pr = shared ? start + c0 + mm : a.perm[start + c0 + mm];
    }
    __builtin_amdgcn_sched_barrier(0);
    issue(std::integral_constant<int, 0>(), s0);
    if ((int)threadIdx.x < 16) {
      srow_l[threadIdx.x] = (shared || !a.gate_up) ? pr : pr / a.k;
      orow_l[threadIdx.x] = pr;
    }
    lds_barrier();
    // A of this wave's groups for the whole chunk (indices clamped into the row past the wave's range), the
    // bias MFMAs' A (Sx of token n, group 4 j + kb) and the tokens' 2^e; then the second step's loads, and a
    // wait that leaves exactly those in flight (a wait the compiler sees, so it adds none of its own)
    const int srow = srow_l[n];
    const int a_off = (srow * K + 16 * kb) * 2;
    half8 A0[NG], A1[NG];
#pragma unroll
    for (int i = 0; i < NG; ++i) {
      const int gi = min(g0 + i, G - 1);
      A0[i] = __builtin_bit_cast(half8, __builtin_amdgcn_raw_buffer_load_b128(ar, a_off, gi * 128, 0));
      A1[i] = __builtin_bit_cast(half8, __builtin_amdgcn_raw_buffer_load_b128(ar, a_off + 16, gi * 128, 0));
    }
    float sx[R::kBias];
#pragma unroll
    for (int j = 0; j < R::kBias; ++j) sx[j] = xs.os[(int64_t)srow * G + min(g0 + 4 * j + kb, G - 1)].y;
    const float ef = xs.ef[srow_l[threadIdx.x & 15]];
    __builtin_amdgcn_sched_barrier(0);   // the operand loads before the second step's
    issue(std::integral_constant<int, 1>(), s0 + 1);
    wait_vm<R::kLoads>();
    // 2^(e + 24) per token (the products carry 2^-24), read in the steps' reductions after a barrier
    if ((int)threadIdx.x < 16) ef_l[threadIdx.x] = (int)threadIdx.x < nlive ? ef * 16777216.0f : 0.f;
#pragma unroll
    for (int j = 0; j < R::kBias; ++j) sx[j] *= 0x1p-24f;

    // a step's outputs (stored at the start of the next step): the reduction leaves output (m, nn) of tile
    // tt in place of wave tt * wk's partial sum of it in red, which only this thread reads
    auto out_slot = [&](int it, int s, int& m, int& nn, int& tile) __attribute__((always_inline)) {
      const int idx = threadIdx.x + it * kThreadsG, tt = idx >> 8;
      m = (idx >> 4) & 15;
      nn = idx & 15;
      tile = s * tps + tt;
      return it < tps && m < nlive && tile < n_tiles && !(a.gate_up && nn >= 8);
    };
    auto flush = [&](const float* red, int s) __attribute__((always_inline)) {
#pragma unroll
      for (int it = 0; it < kWavesG; ++it) {
        int m, nn, tile;
        if (out_slot(it, s, m, nn, tile))
          out[(int64_t)orow_l[m] * out_len + tile * (a.gate_up ? 8 : 16) + nn] =
              red[((tile - s * tps) * wk) * 256 + m * 16 + nn];
      }
    };

    auto step = [&](auto slot_c, int s) __attribute__((always_inline)) {
      constexpr int SL = decltype(slot_c)::value;
      const char* cb = (SL ? code1 : code0) + wave * R::kCode;
      const uint32_t* sbb = (SL ? sbl1 : sbl0) + wave * R::kSb;
      float* red = SL ? red1 : red0;
      // the slot into registers (row n's words 2 kb, 2 kb + 1 of each group, its scale words, and the bias
      // words of groups 4 j + kb), once the step's loads have arrived: at most the next step's are in flight
      u32x2 qw[NG];
      uint32_t sw[NG], bw[R::kBias];
      const uint32_t* sp = sbb + n * NG * W;
      if constexpr (contig)
        read_slot<R::kLoads, NG, W, 32>(cb + n * (K / 2) + kb * 8, sp, sp + kb * W + (W - 1), qw, sw, bw);
      else
        read_slot<R::kLoads, NG, W, 512>(cb + (kb >> 1) * 256 + n * 16 + (kb & 1) * 8, sp, sp + kb * W + (W - 1), qw, sw,
                                         bw);
      // the previous step's outputs, then step s + 2's loads into the slot just read
      if (s > s0) flush(SL ? red0 : red1, s - 1);
      __builtin_amdgcn_sched_barrier(0);
      issue(slot_c, s + 2);
      const Dequant dq = opaque_dequant();
      uint32_t sh8 = 8;
      asm volatile("" : "+v"(sh8));
      f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < NG; ++i) {
        const uint32_t w0 = qw[i].x, w1 = qw[i].y, t0 = w0 >> sh8, t1 = w1 >> sh8;
        u32x4 b0, b1;
        b0.x = w0 & dq.lo;
        b0.y = w0 & dq.hi;
        b0.z = t0 & dq.lo;
        b0.w = t0 & dq.hi;
        b1.x = w1 & dq.lo;
        b1.y = w1 & dq.hi;
        b1.z = t1 & dq.lo;
        b1.w = t1 & dq.hi;
        float sc = SB_BF16 ? __uint_as_float(sw[i] << 16) : __uint_as_float(sw[i]);
        if (i >= nw) sc = 0.f;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A0[i], __builtin_bit_cast(half8, b0), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A1[i], __builtin_bit_cast(half8, b1), acc, 0, 0, 0);
        y[0] = fmaf(sc, acc[0], y[0]);
        y[1] = fmaf(sc, acc[1], y[1]);
        y[2] = fmaf(sc, acc[2], y[2]);
        y[3] = fmaf(sc, acc[3], y[3]);
      }
#pragma unroll
      for (int j = 0; j < R::kBias; ++j) {
        const float b = SB_BF16 ? __uint_as_float(bw[j] & 0xffff0000u) : __uint_as_float(bw[j]);
        y = __builtin_amdgcn_mfma_f32_16x16x4f32(sx[j], 4 * j + kb < nw ? b : 0.f, y, 0, 0, 0);
      }
      // the waves' partial tiles, added in wave order (red alternates with the step, so one barrier a step)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[wave * 256 + (4 * kb + i) * 16 + n] = y[i];
      lds_barrier();
#pragma unroll
      for (int it = 0; it < kWavesG; ++it) {
        int m, nn, tile;
        if (!out_slot(it, s, m, nn, tile)) continue;
        const int tt = tile - s * tps;
        auto total = [&](int col) {
          float v = red[(tt * wk) * 256 + m * 16 + col];
          for (int w = 1; w < wk; ++w) v += red[(tt * wk + w) * 256 + m * 16 + col];
          return v;
        };
        const float sc = ef_l[m];
        float v;
        if (!valid) v = __builtin_nanf("");
        else if (a.gate_up) v = activation(sc * total(nn), a.act) * (sc * total(nn + 8));
        else v = sc * total(nn);
        red[(tt * wk) * 256 + m * 16 + nn] = v;
      }
    };
    int s = s0;
    for (; s + 1 < s1; s += 2) {
      step(std::integral_constant<int, 0>(), s);
      step(std::integral_constant<int, 1>(), s + 1);
    }
    if (s < s1) step(std::integral_constant<int, 0>(), s);
    flush(((s1 - s0) & 1) ? red0 : red1, s1 - 1);
    // the loads past the last step (zeros) land, and every wave is done with red and the token rows, before
    // they are written again or the block ends
    wait_vm<0>();
    lds_barrier();
  }
}

// The work of a block.  The grid is one wave of resident blocks.  Routed work comes as chunks (runs of at
// most 16 pairs of one expert, so a chunk is one pass of the token loop).  Each block reads the chunk count
// c and splits the work the same way: the shared matrix gets blocks in proportion to its steps (times its
// token chunks) against the routed steps of the c chunks, and splits its steps evenly over them; with R
// blocks left, block b takes part b / c of chunk b % c when c < R (each chunk's steps split as evenly as the
// blocks allow), else chunks b, b + R, ... whole.
template <typename Item>
__device__ __forceinline__ void block_work(const MfmaArgs& a, Item&& item) {
  const int b = blockIdx.x, nb = gridDim.x;
  const int ng = a.steps_routed > 0 ? *a.n_chunks : 0;
  int nsb = 0;
  if (a.steps_shared > 0) {
    if (ng <= 0) {
      nsb = nb;
    } else {
      const int64_t us = (int64_t)a.steps_shared * ((a.T + 15) / 16), ur = (int64_t)a.steps_routed * ng;
      nsb = (int)((nb * us + (us + ur) / 2) / (us + ur));
      nsb = max(1, min(nsb, min(a.steps_shared, nb - 1)));
    }
  }
  if (b < nsb) {
    const int spb = (a.steps_shared + nsb - 1) / nsb;
    const int s0 = b * spb, s1 = min(s0 + spb, a.steps_shared);
    if (s0 < s1) item(true, 0, true, 0, a.T, s0, s1);
    return;
  }
  if (ng <= 0) return;
  const int rb = b - nsb, R = nb - nsb;
  const int steps = a.steps_routed;
  for (int j = rb % ng, part = rb / ng; j < ng; j += R) {
    int s0 = 0, s1 = steps;
    if (ng < R) {
      const int parts = (R - 1 - j) / ng + 1;   // blocks given to chunk j
      s0 = (int)((int64_t)part * steps / parts);
      s1 = (int)((int64_t)(part + 1) * steps / parts);
    }
    const int4 g = a.chunks[j];
    const bool valid = (unsigned)g.x < (unsigned)a.routed.n_records;
    if (s0 < s1) item(false, valid ? g.x : 0, valid, g.y, g.z, s0, s1);
    if (ng < R) break;
  }
}

template <int NG, bool SB_BF16>
__global__ __launch_bounds__(kThreadsG) void grouped_mfma_kernel(MfmaArgs a) {
  extern __shared__ __align__(16) uint32_t lds[];
  block_work(a, [&](bool shared, int e, bool valid, int start, int count, int s0, int s1) __attribute__((always_inline)) {
    mfma_item<NG, SB_BF16>(a, shared, e, valid, start, count, s0, s1, lds);
  });
}

// Item `it` of this block (false: no more): the split of q4_grouping.h on the chunk count the grouping wrote.
struct WorkItem {
  bool shared, valid;
  int e, start, count, s0, s1;
};
__device__ __forceinline__ bool next_item(const MfmaArgs& a, int it, WorkItem& x) {
  const int ng = a.steps_routed > 0 ? *a.n_chunks : 0;
  SplitItem si;
  if (!split_item(SplitShape{(int)gridDim.x, a.T, a.steps_shared, a.steps_routed}, ng, (int)blockIdx.x, it, si))
    return false;
  if (si.shared) {
    x = WorkItem{true, true, 0, 16 * si.j, min(16, a.T - 16 * si.j), si.s0, si.s1};
  } else {
    const int4 g = a.chunks[si.j];
    const bool valid = (unsigned)g.x < (unsigned)a.routed.n_records;
    x = WorkItem{false, valid, valid ? g.x : 0, g.y, g.z, si.s0, si.s1};
  }
  return true;
}

// PLAN: each block's one item from the descriptor the grouping launch wrote (a.plan); else the blocks split
// the work themselves (any number of items per block).
template <int NG, bool SB_BF16, bool PLAN>
__global__ __launch_bounds__(kThreadsG, 2) void grouped_ring_kernel(MfmaArgs a) {
  __shared__ RingLds<NG, SB_BF16> lds;
  auto run = [&](const WorkItem& x) __attribute__((always_inline)) {
    if (!a.gate_up && (x.shared ? a.wk_shared : a.wk_routed) == 1)
      ring_item<NG, SB_BF16, true>(a, x.shared, x.e, x.valid, x.start, x.count, x.s0, x.s1, lds);
    else
      ring_item<NG, SB_BF16, false>(a, x.shared, x.e, x.valid, x.start, x.count, x.s0, x.s1, lds);
  };
  if constexpr (PLAN) {
    const int4 p = a.plan[blockIdx.x];
    const uint32_t w = (uint32_t)p.w;
    const int s0 = (int)(w & 0x7fffu), s1 = (int)((w >> 15) & 0x7fffu);
    if (s0 < s1) run(WorkItem{(w >> 30 & 1u) != 0, (w >> 31) != 0, p.x, p.y, p.z, s0, s1});
  } else {
    WorkItem x;
    for (int it = 0; next_item(a, it, x); ++it)
      if (x.s0 < x.s1) run(x);
  }
}

}  // namespace

moe_status launch_stage_rows(const void* x, bool x_bf16, int rows, int K, const StagedRows& out, hipStream_t s) {
  if (rows <= 0) return MOE_OK;
  if (x_bf16) {
    const StageJob<uint16_t> j{static_cast<const uint16_t*>(x), K, out};
    hipLaunchKernelGGL((stage_rows_kernel<uint16_t>), dim3(rows), dim3(kThreadsM), 0, s, j, j, rows);
  } else {
    const StageJob<float> j{static_cast<const float*>(x), K, out};
    hipLaunchKernelGGL((stage_rows_kernel<float>), dim3(rows), dim3(kThreadsM), 0, s, j, j, rows);
  }
  return check_launch("stage_rows_kernel");
}

moe_status launch_group_and_stage(const int32_t* ids, int P, int n_valid, int32_t* n_groups, int4* groups,
                                  int32_t* perm, int32_t* n_chunks, int4* chunks, const void* x, bool x_bf16, int rows,
                                  int K, const StagedRows& out, hipStream_t s, int4* plan0, const SplitShape* shape0,
                                  int4* plan1, const SplitShape* shape1) {
  const GroupJob g{ids, P, n_valid, n_groups, perm, n_chunks, groups, chunks, plan0, plan1,
                   plan0 ? *shape0 : SplitShape{}, plan1 ? *shape1 : SplitShape{}};
  const int np = (plan0 || plan1) ? kPlanBlocks : 0;
  if (x_bf16) {
    const StageJob<uint16_t> j{static_cast<const uint16_t*>(x), K, out};
    hipLaunchKernelGGL((group_and_stage_kernel<uint16_t>), dim3(rows + 1 + np), dim3(kThreadsM), 0, s, g, j);
  } else {
    const StageJob<float> j{static_cast<const float*>(x), K, out};
    hipLaunchKernelGGL((group_and_stage_kernel<float>), dim3(rows + 1 + np), dim3(kThreadsM), 0, s, g, j);
  }
  return check_launch("group_and_stage_kernel");
}

moe_status launch_stage_rows2(const float* x0, int rows0, int K0, const StagedRows& out0, const float* x1, int rows1,
                              int K1, const StagedRows& out1, hipStream_t s) {
  if (rows0 + rows1 <= 0) return MOE_OK;
  const StageJob<float> j0{x0, K0, out0}, j1{x1, K1, out1};
  hipLaunchKernelGGL((stage_rows_kernel<float>), dim3(rows0 + rows1), dim3(kThreadsM), 0, s, j0, j1, rows0);
  return check_launch("stage_rows_kernel");
}

int mfma_waves_per_tile(int K) {
  // a wave holds its groups' A operands and code words in registers: at most 11 groups where possible
  const int G = K / 64;
  int wk = 1;
  while (wk < kWavesG && (G + wk - 1) / wk > 11) wk *= 2;
  return wk;
}

int mfma_device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    cus[dev] = (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0) ? n : 256;
  }
  return cus[dev];
}

namespace {
// The kernel, dynamic LDS, grid and step counts of a grouped launch.
struct LaunchShape {
  void (*kern)(MfmaArgs);
  size_t lds;
  int nb, steps_shared, steps_routed;
  bool ring;
};

// Resident blocks per compute unit for one kernel and dynamic LDS size, per device (queried once).
int resident_blocks(const void* kern, size_t lds) {
  static std::mutex mu;
  static std::map<std::tuple<int, const void*, size_t>, int> cache;
  int dev = 0;
  (void)hipGetDevice(&dev);
  std::lock_guard<std::mutex> lock(mu);
  const auto key = std::make_tuple(dev, kern, lds);
  auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kThreadsG, lds) != hipSuccess || per_cu < 1) per_cu = 1;
  cache.emplace(key, per_cu);
  return per_cu;
}

LaunchShape launch_shape(const MfmaArgs& a, bool has_shared, bool has_routed, bool sb_bf16) {
  // steps per matrix (a step: one tile per group of wk waves)
  auto steps_of = [](int tiles, int wk) { const int tps = kWavesG / wk; return (tiles + tps - 1) / tps; };
  LaunchShape sh{};
  sh.steps_shared = has_shared ? steps_of(a.tiles_shared, a.wk_shared) : 0;
  sh.steps_routed = has_routed ? steps_of(a.tiles_routed, a.wk_routed) : 0;
  int per_wave = 0, kmax = 0;
  if (has_shared) {
    per_wave = (a.K_shared / 64 + a.wk_shared - 1) / a.wk_shared;
    kmax = a.K_shared;
  }
  if (has_routed) {
    per_wave = max(per_wave, (a.K_routed / 64 + a.wk_routed - 1) / a.wk_routed);
    kmax = max(kmax, a.K_routed);
  }
  auto pick = [&](auto ng) {
    constexpr int NG = decltype(ng)::value;
    if constexpr (NG <= 11) {
      // static LDS only
      if (a.plan) sh.kern = sb_bf16 ? grouped_ring_kernel<NG, true, true> : grouped_ring_kernel<NG, false, true>;
      else sh.kern = sb_bf16 ? grouped_ring_kernel<NG, true, false> : grouped_ring_kernel<NG, false, false>;
      sh.lds = 0;
      sh.ring = true;
    } else {
      sh.kern = sb_bf16 ? grouped_mfma_kernel<NG, true> : grouped_mfma_kernel<NG, false>;
      sh.lds = mfma_lds_bytes(kmax, NG);
      sh.ring = false;
    }
  };
  if (per_wave <= 4) pick(std::integral_constant<int, 4>());
  else if (per_wave <= 8) pick(std::integral_constant<int, 8>());
  else if (per_wave <= 11) pick(std::integral_constant<int, 11>());
  else if (per_wave <= 16) pick(std::integral_constant<int, 16>());
  else pick(std::integral_constant<int, 32>());
  // one wave of resident blocks (at least one per role)
  const int per_cu = resident_blocks(reinterpret_cast<const void*>(sh.kern), sh.lds);
  sh.nb = max(2, per_cu * mfma_device_cus());
  return sh;
}
}  // namespace

bool mfma_plan_shape(MfmaArgs a, bool has_shared, bool has_routed, bool sb_bf16, SplitShape* out) {
  a.plan = reinterpret_cast<const int4*>(alignof(int4));   // any non-NULL pointer selects the instantiation
  const LaunchShape sh = launch_shape(a, has_shared, has_routed, sb_bf16);
  if (!sh.ring || sh.nb > kPlanMaxBlocks || sh.steps_shared >= kPlanMaxSteps || sh.steps_routed >= kPlanMaxSteps)
    return false;
  *out = SplitShape{sh.nb, a.T, sh.steps_shared, sh.steps_routed};
  return true;
}

moe_status launch_grouped_mfma(MfmaArgs a, bool has_shared, bool has_routed, bool sb_bf16, hipStream_t s) {
  const LaunchShape sh = launch_shape(a, has_shared, has_routed, sb_bf16);
  a.steps_shared = sh.steps_shared;
  a.steps_routed = sh.steps_routed;
  hipLaunchKernelGGL(sh.kern, dim3(sh.nb), dim3(kThreadsG), sh.lds, s, a);
  return check_launch(sh.ring ? "grouped_ring_kernel" : "grouped_mfma_kernel");
}

}  // namespace moeq4
