// Device-side building blocks of the 4-bit expert GEMV kernels (single-token and grouped), shared by
// the translation units that launch them.  Not part of the C ABI.
//
// q4_expert_gemv: fused dequantize + matrix-vector products over 4-bit affine expert records.
//
// Two launches per call, each covering the routed experts and the shared expert together:
//   gate_up:  h[f] = act(W_gate[f] . x) * (W_up[f] . x)   for every feature f of every selected expert
//   down:     y[r] = W_down[r] . h                         for every output row r
//
// Work mapping.  A block owns 16 matrix rows: the gate and up rows of 8 features (gate_up) or 16
// consecutive output rows (down).  Within a wavefront, 8 lanes share a row pair and split the row in
// 16-byte chunks (32 codes = half a quantization group): lane j takes chunks 8i + j, so a row's eight
// lanes read 128 contiguous bytes per load.  The W wavefronts of the block split the chunk iterations i
// between them (wave w takes i = w, w + W, ...), so one row's bytes are streamed by 8W lanes and the SIMDs
// hold several short wavefronts instead of one long one: a single wavefront issues a VALU instruction
// only every ~5-8 cycles, and this kernel needs ~2 cycles per instruction to keep up with HBM.  The row
// sums of the W waves are added in LDS in a fixed order (deterministic).
//
// Per wave, loads are issued in the order they are consumed: the activation half-groups this wave
// uses, the scale/bias words of its chunks, then its weight chunks.  The wave converts its activation
// half-groups into LDS (4 lanes per half-group) while the weights are still in flight.
//
// Dequantization without per-code conversions: the activation is staged in LDS as fp16 pairs, scaled
// per half-group by a power of two (exact), and a packed code word w (codes n0..n7) is turned into four
// fp16 pairs with one shift and four and-or operations:
//   (w & 0x000F000F) | 0x64006400  = (1024 + n0, 1024 + n4)
//   (w & 0x00F000F0) | 0x64006400  = (1024 + 16 n1, 1024 + 16 n5)      (paired with x/16)
//   and the same on w >> 8 for (n2, n6), (n3, n7).
// v_dot2_f32_f16 multiplies each pair with its activation pair into an fp32 accumulator (products of
// an 11-bit and an 8..11-bit significand are exact in fp32).  The constant 1024 parts sum to a
// per-half-group offset O known from the activation alone, so for one half-group of one row
//   sum_c w_hat[c] x[c] = 2^e * ( scale * (acc - O) + bias * Sx )   (acc starts at -O),
// with Sx the sum of the (scaled) activations.
#pragma once

#include <type_traits>

#include "common.h"

namespace moeq4 {

typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kMaxWaves = 4;           // wavefronts per block (split of the chunk iterations)
constexpr int kLanesPerRow = 8;
constexpr int kHgStride = 20;          // dwords per staged half-group (16 used; padding spreads LDS banks)
constexpr uint32_t kMagic = 0x64006400u;
constexpr int kMaxK = 8192;

struct Stage {
  uint32_t* xw;     // [nhg][kHgStride] permuted fp16 pairs
  float4* hg;       // [nhg] (2^e, O, Sx, 0)
};

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2v, a), __builtin_bit_cast(half2v, b), c, false);
}

__device__ __forceinline__ uint32_t pack_h2(_Float16 lo, _Float16 hi) {
  half2v h;
  h.x = lo;
  h.y = hi;
  return __builtin_bit_cast(uint32_t, h);
}

// The three constants of the code-to-fp16 step, held in VGPRs.  With 32-bit literals the compiler must
// split (a & mask) | magic into v_and + v_or (a gfx9 VOP3 instruction takes no literal); with register
// operands it selects the single v_and_or_b32.
struct Dequant {
  uint32_t lo, hi, magic;   // 0x000F000F, 0x00F000F0, 0x64006400
};

__device__ __forceinline__ Dequant make_dequant() {
  Dequant k{0x000F000Fu, 0x00F000F0u, kMagic};
  asm("" : "+v"(k.lo), "+v"(k.hi), "+v"(k.magic));
  return k;
}

// make_dequant as values the compiler cannot see through from one call to the next: called inside a loop
// over tokens whose codes stay the same, it keeps the dequantized words from being hoisted out of the
// loop (which would hold 16 more registers per code chunk live for the whole loop).
__device__ __forceinline__ Dequant opaque_dequant() {
  Dequant k{0x000F000Fu, 0x00F000F0u, kMagic};
  asm volatile("" : "+v"(k.lo), "+v"(k.hi), "+v"(k.magic));
  return k;
}

// Dot product of one 16-byte chunk (4 words, 32 codes) with its staged activation (16 dwords),
// accumulated onto `acc` (the caller passes -O, so the result is sum_c code[c] * x_scaled[c]).
__device__ __forceinline__ float chunk_dot(u32x4 q, const u32x4 x0, const u32x4 x1, const u32x4 x2, const u32x4 x3,
                                           const Dequant& k, float acc) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
  const u32x4 xs[4] = {x0, x1, x2, x3};
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const uint32_t v = w[m], t = v >> 8;
    acc = dot2((v & k.lo) | k.magic, xs[m].x, acc);
    acc = dot2((v & k.hi) | k.magic, xs[m].y, acc);
    acc = dot2((t & k.lo) | k.magic, xs[m].z, acc);
    acc = dot2((t & k.hi) | k.magic, xs[m].w, acc);
  }
  return acc;
}

__device__ __forceinline__ u32x4 load_nt(const char* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// ------------------------------------------------------------------------------------------------
// activation staging, per wave: the half-groups of the wave's chunk iterations, one 8-element word
// per lane (4 lanes per half-group).  Slot s = lane + 64 p maps to (iteration slot m = s / 32,
// half-group in the iteration jj = (s / 4) % 8, word q = s % 4).
// ------------------------------------------------------------------------------------------------
template <typename XT>
struct XWord {
  static constexpr int kVec = sizeof(XT) == 2 ? 1 : 2;   // 16-byte loads per 8 elements
  u32x4 v[kVec];
};

template <typename XT>
__device__ __forceinline__ void load_word(const XT* x, int hg, int q, XWord<XT>& w) {
  const u32x4* p = reinterpret_cast<const u32x4*>(x + hg * 32 + q * 8);
#pragma unroll
  for (int i = 0; i < XWord<XT>::kVec; ++i) w.v[i] = p[i];
}

template <typename XT>
__device__ __forceinline__ void word_to_f32(const XWord<XT>& w, float v[8]);

template <>
__device__ __forceinline__ void word_to_f32<uint16_t>(const XWord<uint16_t>& w, float v[8]) {
  const uint32_t u[4] = {w.v[0].x, w.v[0].y, w.v[0].z, w.v[0].w};
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    v[2 * m] = __uint_as_float(u[m] << 16);
    v[2 * m + 1] = __uint_as_float(u[m] & 0xffff0000u);
  }
}

template <>
__device__ __forceinline__ void word_to_f32<float>(const XWord<float>& w, float v[8]) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    v[4 * i] = __uint_as_float(w.v[i].x);
    v[4 * i + 1] = __uint_as_float(w.v[i].y);
    v[4 * i + 2] = __uint_as_float(w.v[i].z);
    v[4 * i + 3] = __uint_as_float(w.v[i].w);
  }
}

// Convert one word of a half-group; the 4 lanes of the half-group cooperate (xor 1, xor 2).
__device__ __forceinline__ void stage_word(const float v[8], bool live, int hg, int q, Stage st) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  amax = fmaxf(amax, dpp_f<kDppXor1>(amax));
  amax = fmaxf(amax, dpp_f<kDppXor2>(amax));
  int e = 0;
  if (amax > 0.f && amax <= 3.0e38f) e = max(-100, min(100, ilogbf(amax) - 13));   // amax * 2^-e in [2^13, 2^14)
  const float inv = ldexpf(1.0f, -e);
  const float inv16 = inv * 0.0625f;
  const _Float16 a0 = (_Float16)(v[0] * inv), a4 = (_Float16)(v[4] * inv);
  const _Float16 b1 = (_Float16)(v[1] * inv16), b5 = (_Float16)(v[5] * inv16);
  const _Float16 a2 = (_Float16)(v[2] * inv), a6 = (_Float16)(v[6] * inv);
  const _Float16 b3 = (_Float16)(v[3] * inv16), b7 = (_Float16)(v[7] * inv16);
  const float sa = ((float)a0 + (float)a4) + ((float)a2 + (float)a6);
  const float sb = ((float)b1 + (float)b5) + ((float)b3 + (float)b7);
  float osum = sa + sb, ssum = sa + 16.0f * sb;
  osum += dpp_f<kDppXor1>(osum);
  ssum += dpp_f<kDppXor1>(ssum);
  osum += dpp_f<kDppXor2>(osum);
  ssum += dpp_f<kDppXor2>(ssum);
  if (live) {
    u32x4 qv;
    qv.x = pack_h2(a0, a4);
    qv.y = pack_h2(b1, b5);
    qv.z = pack_h2(a2, a6);
    qv.w = pack_h2(b3, b7);
    *reinterpret_cast<u32x4*>(st.xw + hg * kHgStride + 4 * q) = qv;
    if (q == 0) st.hg[hg] = make_float4(ldexpf(1.0f, e), 1024.0f * osum, ssum, 0.f);
  }
}

template <bool SB_BF16>
struct SbWord {
  uint32_t s, b;   // bf16: the (scale, bias) pair in `s`; fp32: scale in s, bias in b
};

template <bool SB_BF16>
__device__ __forceinline__ SbWord<SB_BF16> load_sb(const char* row_sb, int grp) {
  SbWord<SB_BF16> w;
  if (SB_BF16) {
    w.s = reinterpret_cast<const uint32_t*>(row_sb)[grp];
    w.b = 0;
  } else {
    const uint2 p = reinterpret_cast<const uint2*>(row_sb)[grp];
    w.s = p.x;
    w.b = p.y;
  }
  return w;
}

template <bool SB_BF16>
__device__ __forceinline__ void sb_values(const SbWord<SB_BF16>& w, float& s, float& b) {
  if (SB_BF16) {
    s = __uint_as_float(w.s << 16);
    b = __uint_as_float(w.s & 0xffff0000u);
  } else {
    s = __uint_as_float(w.s);
    b = __uint_as_float(w.b);
  }
}

// One wave's share of the dot products of its lane group's two rows (A, B) with the staged vector.
// NBW = iteration slots per wave.  Returns this lane's partial sums (before the 8-lane reduction).
template <int NBW, typename XT, bool SB_BF16>
__device__ __forceinline__ void rowpair_partial(const char* rowA, const char* rowB, const char* sbA, const char* sbB,
                                                const XT* x, int K, Stage st, bool valid, float& yA, float& yB) {
  const int W = blockDim.x >> 6, wave = threadIdx.x >> 6, lane = threadIdx.x & 63, j = lane & 7;
  const int C = K / 32, nit = (C + kLanesPerRow - 1) / kLanesPerRow;
  constexpr int kPasses = (NBW * 32 + 63) / 64;
  // 1. activation words of this wave's half-groups
  XWord<XT> xw[kPasses];
  int hgp[kPasses];
  bool livep[kPasses];
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    const int s = lane + 64 * p, m = s >> 5, jj = (s >> 2) & 7, q = s & 3;
    const int it = wave + W * m;
    hgp[p] = it * kLanesPerRow + jj;
    livep[p] = m < NBW && it < nit && hgp[p] < C;
    if (livep[p]) load_word<XT>(x, hgp[p], q, xw[p]);
  }
  // 2. scale/bias of this lane's chunks, 3. weight chunks
  SbWord<SB_BF16> sa[NBW], sbw[NBW];
  u32x4 qa[NBW], qb[NBW];
  if (valid) {
#pragma unroll
    for (int m = 0; m < NBW; ++m) {
      const int c = (wave + W * m) * kLanesPerRow + j;
      if (c < C) {
        sa[m] = load_sb<SB_BF16>(sbA, c >> 1);
        sbw[m] = load_sb<SB_BF16>(sbB, c >> 1);
      }
    }
#pragma unroll
    for (int m = 0; m < NBW; ++m) {
      const int c = (wave + W * m) * kLanesPerRow + j;
      if (c < C) {
        qa[m] = load_nt(rowA + c * 16);
        qb[m] = load_nt(rowB + c * 16);
      }
    }
  }
  // 4. stage the activation while the weights are in flight (wave-local: no block barrier)
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    float v[8];
    if (livep[p]) word_to_f32<XT>(xw[p], v);
    else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = 0.f;
    }
    stage_word(v, livep[p], hgp[p], (lane + 64 * p) & 3, st);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // 5. consume the chunks in arrival order
  yA = 0.f;
  yB = 0.f;
  if (!valid) return;
  const Dequant dq = make_dequant();
#pragma unroll
  for (int m = 0; m < NBW; ++m) {
    const int c = (wave + W * m) * kLanesPerRow + j;
    if (c < C) {
      const u32x4* xv = reinterpret_cast<const u32x4*>(st.xw + c * kHgStride);
      const u32x4 x0 = xv[0], x1 = xv[1], x2 = xv[2], x3 = xv[3];
      const float4 h = st.hg[c];
      const float accA = chunk_dot(qa[m], x0, x1, x2, x3, dq, -h.y);
      const float accB = chunk_dot(qb[m], x0, x1, x2, x3, dq, -h.y);
      float s0, b0, s1, b1;
      sb_values<SB_BF16>(sa[m], s0, b0);
      sb_values<SB_BF16>(sbw[m], s1, b1);
      yA = fmaf(h.x, fmaf(s0, accA, b0 * h.z), yA);
      yB = fmaf(h.x, fmaf(s1, accB, b1 * h.z), yB);
    }
  }
}

__device__ __forceinline__ float reduce8(float v) {
  v += dpp_f<kDppXor1>(v);
  v += dpp_f<kDppXor2>(v);
  v += xor4_f(v);
  return v;
}

// Sum the row pair over the block's waves (fixed order); true on the lanes that hold the totals.
__device__ __forceinline__ bool block_sum(float& yA, float& yB) {
  __shared__ float red[kMaxWaves][16];
  const int W = blockDim.x >> 6, wave = threadIdx.x >> 6, lane = threadIdx.x & 63, ra = lane >> 3, j = lane & 7;
  yA = reduce8(yA);
  yB = reduce8(yB);
  if (W == 1) return j == 0;
  if (j == 0) {
    red[wave][ra] = yA;
    red[wave][8 + ra] = yB;
  }
  __syncthreads();
  if (wave != 0 || j != 0) return false;
  yA = red[0][ra];
  yB = red[0][8 + ra];
  for (int w = 1; w < W; ++w) {
    yA += red[w][ra];
    yB += red[w][8 + ra];
  }
  return true;
}

__device__ __forceinline__ float activation(float z, int act) {
  if (act == MOE_ACT_SILU) return z / (1.0f + expf(-z));
  const float c = 0.7978845608028654f;   // sqrt(2/pi)
  return 0.5f * z * (1.0f + tanhf(c * (z + 0.044715f * z * z * z)));
}

struct Pool {
  const char* base;
  int64_t record_bytes;
  int32_t n_records;
  int32_t F;
  int64_t off_q;     // codes section of the matrix this launch reads
  int64_t off_sb;    // scale/bias section of that matrix
};

struct GemvArgs {
  Pool routed, shared;
  const int32_t* ids;
  int32_t k;
  int32_t d;
  const void* in;          // gate_up: x [T][d]; down: unused (h comes from the workspace)
  float* h_routed;         // [T][k][F]
  float* h_shared;         // [T][S]
  float* y_routed;         // [T][k][d]
  float* y_shared;         // [T][d]
  int32_t nb_shared;       // blocks of the shared expert per token
  int32_t nb_routed;       // blocks per routed expert
  int32_t act;
  // fused combine (down launch only): out[t] = round(sum_i w[t][i] y_routed[t][i] + y_shared[t] + residual[t])
  const float* weights;    // [T][k]
  const void* residual;    // [T][d] or NULL
  int32_t res_bf16, out_bf16;
  void* out;               // [T][d]
  uint32_t* tile_counters; // [T][d/16], zero between calls
  // grouped launches (T > 1): the (token, slot) pairs t*k + i sorted by expert
  int32_t T;
  int32_t* n_groups;       // [1] non-empty groups (written by the grouping kernel)
  int4* groups;            // [groups_max] (expert or n_records for invalid ids, first index into perm, count, 0)
  int32_t* perm;           // [T*k] pair indices, grouped by expert, ascending within a group
  int32_t* n_chunks;       // [1] the groups' runs of at most 16 pairs (written by the grouping kernel)
  int4* chunks;            // [chunks_max] (expert or n_records, first index into perm, count <= 16, 0)
  char* stage;             // activations staged for the matrix cores (StagedRows), T > 1
  int4* plan_gu;           // [kPlanMaxBlocks] work descriptors of the grouped gate/up and down launches, T > 1
  int4* plan_dn;
};

// The combine of one 16-row tile of token t, summed in the order i = 0..k-1, shared, residual (the
// order of moe_combine), by threads 0..15 of the block that completed the tile.  y_routed / y_shared
// were published by other blocks with device-coherent stores, so they are read the same way.
__device__ __forceinline__ void combine_tile(const GemvArgs& a, int t, int tile) {
  const int d = a.d, row = tile * 16 + (int)threadIdx.x;
  float acc = 0.f;
  for (int i = 0; i < a.k; ++i)
    acc = __builtin_fmaf(a.weights[(int64_t)t * a.k + i],
                         __hip_atomic_load(a.y_routed + ((int64_t)t * a.k + i) * d + row, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT),
                         acc);
  if (a.nb_shared) acc += __hip_atomic_load(a.y_shared + (int64_t)t * d + row, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (a.residual)
    acc += a.res_bf16 ? bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(a.residual)[(int64_t)t * d + row])
                      : reinterpret_cast<const float*>(a.residual)[(int64_t)t * d + row];
  if (a.out_bf16)
    reinterpret_cast<uint16_t*>(a.out)[(int64_t)t * d + row] = (uint16_t)f32_to_bf16_bits(acc);
  else
    reinterpret_cast<float*>(a.out)[(int64_t)t * d + row] = acc;
}

// The grouping of a batch's T*k (token, slot) pairs by expert (q4_grouped.hip): a.ids sorted into
// a.groups / a.perm / a.n_groups, so that the grouped products (q4_mfma.hip) stream each selected expert's
// rows once for all of its tokens.
constexpr int kMaxGroupedRecords = 4096;   // routed pool records supported with T > 1
constexpr int kChunkPairs = 16;            // pairs per chunk (the tokens of one matrix-core pass)
// n_chunks / chunks (optional): each group split into runs of at most kChunkPairs pairs, in group order,
// (expert, first index into perm, count, 0); at most groups + P / kChunkPairs entries
moe_status launch_group_pairs(const int32_t* ids, int P, int n_valid, int32_t* n_groups, int4* groups, int32_t* perm,
                              hipStream_t s, int32_t* n_chunks = nullptr, int4* chunks = nullptr);

inline size_t lds_bytes(int K) { return (size_t)(K / 32) * (kHgStride * 4 + 16); }

// Matrix-core path for T > 1 (q4_mfma.hip).  Activation rows are staged once per call in the fp16 form the
// MFMA kernel multiplies (one power-of-two scale per row, per-64-group sums); then one block per 16 weight
// rows and (group or shared matrix) multiplies them with up to 16 tokens at a time.
struct StagedRows {
  int32_t rows;
  _Float16* xq;   // [rows][K]
  float2* os;     // [rows][K/64]: (1024 * sum of the group's staged values, sum of its values / 2^e)
  float* ef;      // [rows] 2^e
};
inline size_t staged_rows_bytes(int64_t rows, int K) {
  auto a256 = [](size_t x) { return (x + 255) / 256 * 256; };
  return a256((size_t)rows * K * 2) + a256((size_t)rows * (K / 64) * 8) + a256((size_t)rows * 4);
}
inline StagedRows staged_rows_at(char* base, int64_t rows, int K) {
  auto a256 = [](size_t x) { return (x + 255) / 256 * 256; };
  StagedRows r;
  r.rows = (int32_t)rows;
  r.xq = reinterpret_cast<_Float16*>(base);
  r.os = reinterpret_cast<float2*>(base + a256((size_t)rows * K * 2));
  r.ef = reinterpret_cast<float*>(base + a256((size_t)rows * K * 2) + a256((size_t)rows * (K / 64) * 8));
  return r;
}
moe_status launch_stage_rows(const void* x, bool x_bf16, int rows, int K, const StagedRows& out, hipStream_t s);
// two fp32 row sets staged in one launch (rows0 of x0, then rows1 of x1)
moe_status launch_stage_rows2(const float* x0, int rows0, int K0, const StagedRows& out0, const float* x1, int rows1,
                              int K1, const StagedRows& out1, hipStream_t s);
// The grouped products of T > 1 tokens on the matrix cores (q4_mfma.hip).  A tile is 16 weight rows
// (gate_up: 8 gate rows and the matching 8 up rows); wk waves of a block split a tile's K, so a block
// of 8 waves works on 8 / wk tiles at a time (one step).  Fill the per-matrix fields; the launcher sets
// the step counts and the block split.
struct MfmaArgs {
  Pool routed, shared;          // off_q / off_sb select the matrix
  int32_t K_routed, K_shared;   // row lengths
  int32_t wk_routed, wk_shared; // waves per tile: 1, 2, 4 or 8 (mfma_waves_per_tile)
  int32_t tiles_routed, tiles_shared;
  int32_t gate_up;              // 1: out = act(gate) * up per feature; 0: out = the 16 rows' products
  int32_t act;
  int32_t T, k;
  const int32_t* n_chunks;      // routed work: runs of at most 16 pairs of one expert (device count)
  const int4* chunks;           // (expert or n_records, first index into perm, count, 0)
  const int32_t* perm;
  StagedRows xs_routed, xs_shared;   // routed rows are tokens (gate_up) or pairs (down); shared rows are tokens
  float* out_routed;            // gate_up: h [pairs][F]; down: y [pairs][d]
  float* out_shared;            // gate_up: h [T][S];     down: y [T][d]
  int32_t out_len_routed, out_len_shared;
  // one work descriptor per block of the launch, written by the grouping launch (see q4_grouping.h), or NULL
  // (the blocks split the work themselves)
  const int4* plan;
  // set by launch_grouped_mfma
  int32_t steps_routed, steps_shared;   // steps of a matrix (0: no such matrix)
};
int mfma_waves_per_tile(int K);
moe_status launch_grouped_mfma(MfmaArgs a, bool has_shared, bool has_routed, bool sb_bf16, hipStream_t s);

struct Slot {
  bool shared, valid;
  int slot, tile, e;
};

__device__ __forceinline__ Slot block_slot(const GemvArgs& a, int t) {
  Slot s;
  int u = blockIdx.x;
  s.shared = u < a.nb_shared;
  s.slot = 0;
  s.tile = u;
  s.e = 0;
  s.valid = true;
  if (!s.shared) {
    u -= a.nb_shared;
    s.slot = u / a.nb_routed;
    s.tile = u % a.nb_routed;
    s.e = a.ids[t * a.k + s.slot];
    s.valid = (unsigned)s.e < (unsigned)a.routed.n_records;
  }
  return s;
}

template <typename Fn>
moe_status dispatch_nbw(int nbw, Fn&& fn) {
  switch (nbw) {
    case 1: return fn(std::integral_constant<int, 1>());
    case 2: return fn(std::integral_constant<int, 2>());
    case 3: return fn(std::integral_constant<int, 3>());
    case 4: return fn(std::integral_constant<int, 4>());
    case 5:
    case 6: return fn(std::integral_constant<int, 6>());
    default: return fn(std::integral_constant<int, 8>());
  }
}

inline int iterations(int K) { return (K / 32 + kLanesPerRow - 1) / kLanesPerRow; }

}  // namespace moeq4
