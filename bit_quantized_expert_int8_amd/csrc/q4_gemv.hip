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
#include <type_traits>

#include "common.h"

namespace moeq4 {
namespace {

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
  amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
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
  osum += __shfl_xor(osum, 1, 64);
  ssum += __shfl_xor(ssum, 1, 64);
  osum += __shfl_xor(osum, 2, 64);
  ssum += __shfl_xor(ssum, 2, 64);
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
  v += __shfl_xor(v, 1, 64);
  v += __shfl_xor(v, 2, 64);
  v += __shfl_xor(v, 4, 64);
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
};

inline size_t lds_bytes(int K) { return (size_t)(K / 32) * (kHgStride * 4 + 16); }

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

// ------------------------------------------------------------------------------------------------
// gate_up + activation: block = 8 features of one expert (gate rows f0.., up rows F + f0..)
// ------------------------------------------------------------------------------------------------
template <int NBW, typename XT, bool SB_BF16>
__global__ __launch_bounds__(64 * kMaxWaves) void gate_up_kernel(GemvArgs a) {
  extern __shared__ __align__(16) uint32_t lds[];
  const int K = a.d, nhg = K / 32;
  const int t = blockIdx.y;
  const Slot sl = block_slot(a, t);
  const Pool& P = sl.shared ? a.shared : a.routed;
  const int lane = threadIdx.x & 63, ra = lane >> 3;
  const int F = P.F, f = sl.tile * 8 + ra;
  const char* rec = P.base + (int64_t)(sl.valid ? sl.e : 0) * P.record_bytes;
  const int64_t rowb = K / 2, sbrow = (int64_t)(K / 64) * (SB_BF16 ? 4 : 8);
  Stage st{lds, reinterpret_cast<float4*>(lds + nhg * kHgStride)};
  float yA, yB;
  rowpair_partial<NBW, XT, SB_BF16>(rec + P.off_q + f * rowb, rec + P.off_q + (F + f) * rowb, rec + P.off_sb + f * sbrow,
                                     rec + P.off_sb + (F + f) * sbrow, reinterpret_cast<const XT*>(a.in) + (int64_t)t * K,
                                     K, st, sl.valid, yA, yB);
  if (!block_sum(yA, yB)) return;
  const float h = sl.valid ? activation(yA, a.act) * yB : __builtin_nanf("");
  if (sl.shared)
    a.h_shared[(int64_t)t * F + f] = h;
  else
    a.h_routed[((int64_t)t * a.k + sl.slot) * F + f] = h;
}

// ------------------------------------------------------------------------------------------------
// down: block = 16 consecutive output rows of one expert; input = that expert's h from gate_up
// ------------------------------------------------------------------------------------------------
template <int NBW, bool SB_BF16, bool COMBINE>
__global__ __launch_bounds__(64 * kMaxWaves) void down_kernel(GemvArgs a) {
  extern __shared__ __align__(16) uint32_t lds[];
  const int d = a.d;
  const int t = blockIdx.y;
  const Slot sl = block_slot(a, t);
  const Pool& P = sl.shared ? a.shared : a.routed;
  const int K = P.F, nhg = K / 32;
  const int lane = threadIdx.x & 63, ra = lane >> 3;
  const int r = sl.tile * 16 + ra;
  const char* rec = P.base + (int64_t)(sl.valid ? sl.e : 0) * P.record_bytes;
  const int64_t rowb = K / 2, sbrow = (int64_t)(K / 64) * (SB_BF16 ? 4 : 8);
  const float* h = sl.shared ? a.h_shared + (int64_t)t * K : a.h_routed + ((int64_t)t * a.k + sl.slot) * K;
  Stage st{lds, reinterpret_cast<float4*>(lds + nhg * kHgStride)};
  float yA, yB;
  rowpair_partial<NBW, float, SB_BF16>(rec + P.off_q + r * rowb, rec + P.off_q + (r + 8) * rowb, rec + P.off_sb + r * sbrow,
                                        rec + P.off_sb + (r + 8) * sbrow, h, K, st, sl.valid, yA, yB);
  const bool total = block_sum(yA, yB);
  if (!sl.valid) yA = yB = __builtin_nanf("");
  float* y = sl.shared ? a.y_shared + (int64_t)t * d : a.y_routed + ((int64_t)t * a.k + sl.slot) * d;
  if (!COMBINE) {
    if (total) {
      y[r] = yA;
      y[r + 8] = yB;
    }
    return;
  }
  // Fused combine: the k routed blocks and the shared block of a 16-row tile publish their rows with
  // device-coherent stores and take a ticket; the last of them sums the tile in the fixed order
  // i = 0..k-1, shared, residual (the order of moe_combine) and writes the rounded output.
  __shared__ uint32_t last;
  if (total) {
    __hip_atomic_store(y + r, yA, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(y + r + 8, yB, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  const int ntiles = d / 16;
  uint32_t* ctr = a.tile_counters + (int64_t)t * ntiles + sl.tile;
  const uint32_t units = (uint32_t)a.k + (a.nb_shared ? 1u : 0u);
  if (threadIdx.x == 0) last = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == units - 1;
  __syncthreads();
  if (!last || threadIdx.x >= 16) return;
  const int row = sl.tile * 16 + threadIdx.x;
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
  if (threadIdx.x == 0) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------------------------------------------
// host side
// ------------------------------------------------------------------------------------------------
template <int NBW>
moe_status launch_gate_up(const GemvArgs& a, moe_dtype xdt, bool sb_bf16, dim3 grid, int waves, size_t lds, hipStream_t s) {
  const dim3 block(64 * waves);
  if (xdt == MOE_BF16) {
    if (sb_bf16) hipLaunchKernelGGL((gate_up_kernel<NBW, uint16_t, true>), grid, block, lds, s, a);
    else hipLaunchKernelGGL((gate_up_kernel<NBW, uint16_t, false>), grid, block, lds, s, a);
  } else {
    if (sb_bf16) hipLaunchKernelGGL((gate_up_kernel<NBW, float, true>), grid, block, lds, s, a);
    else hipLaunchKernelGGL((gate_up_kernel<NBW, float, false>), grid, block, lds, s, a);
  }
  return check_launch("q4_expert_gemv(gate_up)");
}

template <int NBW>
moe_status launch_down(const GemvArgs& a, bool sb_bf16, bool combine, dim3 grid, int waves, size_t lds, hipStream_t s) {
  const dim3 block(64 * waves);
  if (combine) {
    if (sb_bf16) hipLaunchKernelGGL((down_kernel<NBW, true, true>), grid, block, lds, s, a);
    else hipLaunchKernelGGL((down_kernel<NBW, false, true>), grid, block, lds, s, a);
  } else {
    if (sb_bf16) hipLaunchKernelGGL((down_kernel<NBW, true, false>), grid, block, lds, s, a);
    else hipLaunchKernelGGL((down_kernel<NBW, false, false>), grid, block, lds, s, a);
  }
  return check_launch("q4_expert_gemv(down)");
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

int iterations(int K) { return (K / 32 + kLanesPerRow - 1) / kLanesPerRow; }

bool pool_ok(const moe_q4_pool* p, RecordOffsets* o, const char** why) {
  if (!p->base_dev) { *why = "pool base is NULL"; return false; }
  if (!record_offsets(p->d, p->F, p->sb_dtype, o)) { *why = "pool d/F not positive multiples of 64 or bad sb dtype"; return false; }
  if (p->d > kMaxK || p->F > kMaxK) { *why = "pool d/F above 8192"; return false; }
  if (p->record_bytes < o->total || p->record_bytes % 256) { *why = "record_bytes too small or not a multiple of 256"; return false; }
  if (!aligned(p->base_dev, 256)) { *why = "pool base not 256-byte aligned"; return false; }
  if (p->n_records < 1) { *why = "pool has no records"; return false; }
  return true;
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

}  // namespace
}  // namespace moeq4

using namespace moeq4;

extern "C" size_t q4_expert_gemv_workspace_bytes(const moe_q4_pool* routed, int32_t k, const moe_q4_pool* shared, int32_t T) {
  if (T < 1) return 0;
  size_t b = 0;
  if (routed && k > 0) b += align256((size_t)T * k * routed->F * 4);
  if (shared) b += align256((size_t)T * shared->F * 4);
  return b;
}

namespace moeq4 {
namespace {

// Validate the arguments shared by the three entry points and fill the launch arguments.
moe_status prepare(const char* who, const moe_q4_pool* routed, const int32_t* ids_dev, int32_t k, const moe_q4_pool* shared,
                   const void* x_dev, moe_dtype x_dtype, int32_t T, moe_act act, float* y_routed_dev, float* y_shared_dev,
                   void* workspace_dev, size_t workspace_bytes, bool need_x, bool need_y, GemvArgs* a, RecordOffsets* orr,
                   RecordOffsets* osh) {
  if (need_x && !x_dev) return fail(MOE_ERR_INVALID_ARG, "%s: x is NULL", who);
  if (need_x && x_dtype != MOE_F32 && x_dtype != MOE_BF16) return fail(MOE_ERR_INVALID_ARG, "%s: bad x_dtype", who);
  if (act != MOE_ACT_GELU_TANH && act != MOE_ACT_SILU) return fail(MOE_ERR_INVALID_ARG, "%s: bad act", who);
  if (T < 1 || T > 65535) return fail(MOE_ERR_INVALID_ARG, "%s: T=%d", who, T);
  if (k < 0 || k > 32) return fail(MOE_ERR_UNSUPPORTED, "%s: k=%d (0..32)", who, k);
  if (!routed && k > 0) return fail(MOE_ERR_INVALID_ARG, "%s: k=%d but routed pool is NULL", who, k);
  if (k == 0 && !shared) return fail(MOE_ERR_INVALID_ARG, "%s: nothing to compute (k=0, no shared expert)", who);
  const char* why = nullptr;
  const bool has_routed = routed && k > 0;
  if (has_routed) {
    if (!pool_ok(routed, orr, &why)) return fail(MOE_ERR_INVALID_ARG, "%s: routed %s", who, why);
    if (!ids_dev) return fail(MOE_ERR_INVALID_ARG, "%s: ids is NULL", who);
    if (need_y && !y_routed_dev) return fail(MOE_ERR_INVALID_ARG, "%s: y_routed is NULL", who);
  }
  if (shared) {
    if (!pool_ok(shared, osh, &why)) return fail(MOE_ERR_INVALID_ARG, "%s: shared %s", who, why);
    if (need_y && !y_shared_dev) return fail(MOE_ERR_INVALID_ARG, "%s: y_shared is NULL", who);
  }
  const int d = has_routed ? routed->d : shared->d;
  if (has_routed && shared) {
    if (shared->d != d) return fail(MOE_ERR_INVALID_ARG, "%s: routed d=%d != shared d=%d", who, d, shared->d);
    if (shared->sb_dtype != routed->sb_dtype)
      return fail(MOE_ERR_UNSUPPORTED, "%s: routed and shared scale/bias dtypes differ", who);
  }
  if (need_x && !aligned(x_dev, 16)) return fail(MOE_ERR_INVALID_ARG, "%s: x not 16-byte aligned", who);
  const size_t need = q4_expert_gemv_workspace_bytes(routed, k, shared, T);
  if (!workspace_dev || workspace_bytes < need)
    return fail(MOE_ERR_INVALID_ARG, "%s: workspace %zu bytes < %zu", who, workspace_bytes, need);
  if (!aligned(workspace_dev, 256)) return fail(MOE_ERR_INVALID_ARG, "%s: workspace not 256-byte aligned", who);
  const int Fr = has_routed ? routed->F : 0;
  const int Fs = shared ? shared->F : 0;
  *a = GemvArgs{};
  if (has_routed)
    a->routed = Pool{static_cast<const char*>(routed->base_dev), (int64_t)routed->record_bytes, routed->n_records, Fr, 0, 0};
  if (shared)
    a->shared = Pool{static_cast<const char*>(shared->base_dev), (int64_t)shared->record_bytes, shared->n_records, Fs, 0, 0};
  a->ids = ids_dev;
  a->k = has_routed ? k : 0;
  a->d = d;
  a->in = x_dev;
  char* ws = static_cast<char*>(workspace_dev);
  a->h_routed = has_routed ? reinterpret_cast<float*>(ws) : nullptr;
  a->h_shared = shared ? reinterpret_cast<float*>(ws + (has_routed ? align256((size_t)T * k * Fr * 4) : 0)) : nullptr;
  a->y_routed = y_routed_dev;
  a->y_shared = y_shared_dev;
  a->act = act;
  return MOE_OK;
}

// gate_up: 8 features per block; its waves split the iterations of rows of K = d
moe_status run_gate_up(GemvArgs a, const RecordOffsets& orr, const RecordOffsets& osh, moe_dtype x_dtype, bool sb_bf16,
                       int T, hipStream_t s) {
  a.routed.off_q = (int64_t)orr.gate_up_q;
  a.routed.off_sb = (int64_t)orr.gate_up_sb;
  a.shared.off_q = (int64_t)osh.gate_up_q;
  a.shared.off_sb = (int64_t)osh.gate_up_sb;
  a.nb_shared = a.shared.base ? a.shared.F / 8 : 0;
  a.nb_routed = a.routed.F / 8;
  const int nit = iterations(a.d);
  const int waves = nit < kMaxWaves ? nit : kMaxWaves;
  const int nbw = (nit + waves - 1) / waves;
  dim3 grid(a.nb_shared + a.k * a.nb_routed, T);
  return dispatch_nbw(nbw, [&](auto nb) {
    return launch_gate_up<decltype(nb)::value>(a, x_dtype, sb_bf16, grid, waves, lds_bytes(a.d), s);
  });
}

// down: 16 output rows per block; rows of K = F (routed) or S (shared)
moe_status run_down(GemvArgs a, const RecordOffsets& orr, const RecordOffsets& osh, bool sb_bf16, int T, hipStream_t s,
                    bool combine = false) {
  a.routed.off_q = (int64_t)orr.down_q;
  a.routed.off_sb = (int64_t)orr.down_sb;
  a.shared.off_q = (int64_t)osh.down_q;
  a.shared.off_sb = (int64_t)osh.down_sb;
  const bool has_routed = a.k > 0, has_shared = a.shared.base != nullptr;
  a.nb_shared = has_shared ? a.d / 16 : 0;
  a.nb_routed = a.d / 16;
  const int Fr = a.routed.F, Fs = a.shared.F;
  const int nit_r = has_routed ? iterations(Fr) : 0, nit_s = has_shared ? iterations(Fs) : 0;
  const int nit_lo = has_routed ? nit_r : nit_s, nit_hi = nit_r > nit_s ? nit_r : nit_s;
  const int waves = nit_lo < kMaxWaves ? nit_lo : kMaxWaves;
  const int nbw = (nit_hi + waves - 1) / waves;
  dim3 grid(a.nb_shared + a.k * a.nb_routed, T);
  return dispatch_nbw(nbw, [&](auto nb) {
    return launch_down<decltype(nb)::value>(a, sb_bf16, combine, grid, waves, lds_bytes(nit_r > nit_s ? Fr : Fs), s);
  });
}

bool sb_is_bf16(const moe_q4_pool* routed, int32_t k, const moe_q4_pool* shared) {
  return ((routed && k > 0) ? routed->sb_dtype : shared->sb_dtype) == MOE_BF16;
}

}  // namespace
}  // namespace moeq4

extern "C" moe_status q4_expert_gemv(const moe_q4_pool* routed, const int32_t* ids_dev, int32_t k,
                                     const moe_q4_pool* shared, const void* x_dev, moe_dtype x_dtype, int32_t T,
                                     moe_act act, float* y_routed_dev, float* y_shared_dev, void* workspace_dev,
                                     size_t workspace_bytes, void* stream) {
  GemvArgs a;
  RecordOffsets orr{}, osh{};
  moe_status st = prepare("q4_expert_gemv", routed, ids_dev, k, shared, x_dev, x_dtype, T, act, y_routed_dev, y_shared_dev,
                          workspace_dev, workspace_bytes, true, true, &a, &orr, &osh);
  if (st != MOE_OK) return st;
  const bool sb16 = sb_is_bf16(routed, k, shared);
  st = run_gate_up(a, orr, osh, x_dtype, sb16, T, as_stream(stream));
  if (st != MOE_OK) return st;
  return run_down(a, orr, osh, sb16, T, as_stream(stream));
}

extern "C" moe_status q4_expert_gate_up(const moe_q4_pool* routed, const int32_t* ids_dev, int32_t k,
                                        const moe_q4_pool* shared, const void* x_dev, moe_dtype x_dtype, int32_t T,
                                        moe_act act, void* workspace_dev, size_t workspace_bytes, void* stream) {
  GemvArgs a;
  RecordOffsets orr{}, osh{};
  moe_status st = prepare("q4_expert_gate_up", routed, ids_dev, k, shared, x_dev, x_dtype, T, act, nullptr, nullptr,
                          workspace_dev, workspace_bytes, true, false, &a, &orr, &osh);
  if (st != MOE_OK) return st;
  return run_gate_up(a, orr, osh, x_dtype, sb_is_bf16(routed, k, shared), T, as_stream(stream));
}

extern "C" moe_status q4_expert_down(const moe_q4_pool* routed, const int32_t* ids_dev, int32_t k, const moe_q4_pool* shared,
                                     int32_t T, float* y_routed_dev, float* y_shared_dev, void* workspace_dev,
                                     size_t workspace_bytes, void* stream) {
  GemvArgs a;
  RecordOffsets orr{}, osh{};
  moe_status st = prepare("q4_expert_down", routed, ids_dev, k, shared, nullptr, MOE_BF16, T, MOE_ACT_GELU_TANH, y_routed_dev,
                          y_shared_dev, workspace_dev, workspace_bytes, false, true, &a, &orr, &osh);
  if (st != MOE_OK) return st;
  return run_down(a, orr, osh, sb_is_bf16(routed, k, shared), T, as_stream(stream));
}

extern "C" size_t q4_expert_gemv_combine_workspace_bytes(const moe_q4_pool* routed, int32_t k, const moe_q4_pool* shared,
                                                         int32_t T) {
  if (T < 1 || (!shared && !(routed && k > 0))) return 0;
  const int d = (routed && k > 0) ? routed->d : shared->d;
  size_t b = q4_expert_gemv_workspace_bytes(routed, k, shared, T);
  if (routed && k > 0) b += align256((size_t)T * k * d * 4);
  if (shared) b += align256((size_t)T * d * 4);
  return b + align256((size_t)T * (d / 16) * 4);
}

extern "C" moe_status q4_expert_gemv_combine(const moe_q4_pool* routed, const int32_t* ids_dev, int32_t k,
                                             const moe_q4_pool* shared, const void* x_dev, moe_dtype x_dtype, int32_t T,
                                             moe_act act, const float* weights_dev, const void* residual_dev,
                                             moe_dtype residual_dtype, void* out_dev, moe_dtype out_dtype,
                                             void* workspace_dev, size_t workspace_bytes, void* stream) {
  const char* who = "q4_expert_gemv_combine";
  const bool has_routed = routed && k > 0;
  if (!out_dev) return fail(MOE_ERR_INVALID_ARG, "%s: out is NULL", who);
  if (has_routed && !weights_dev) return fail(MOE_ERR_INVALID_ARG, "%s: weights is NULL", who);
  if (out_dtype != MOE_F32 && out_dtype != MOE_BF16) return fail(MOE_ERR_INVALID_ARG, "%s: bad out_dtype", who);
  if (residual_dev && residual_dtype != MOE_F32 && residual_dtype != MOE_BF16)
    return fail(MOE_ERR_INVALID_ARG, "%s: bad residual_dtype", who);
  const size_t need = q4_expert_gemv_combine_workspace_bytes(routed, k, shared, T);
  if (workspace_dev && workspace_bytes < need)
    return fail(MOE_ERR_INVALID_ARG, "%s: workspace %zu bytes < %zu", who, workspace_bytes, need);
  // y_routed / y_shared / tile counters live in the workspace after the hidden activations; prepare() checks
  // the rest of the arguments with placeholder y pointers and fills in the hidden-activation layout
  const size_t hb = q4_expert_gemv_workspace_bytes(routed, k, shared, T);
  char* ws = static_cast<char*>(workspace_dev);
  const int d = has_routed ? routed->d : (shared ? shared->d : 0);
  float* y_r = has_routed && ws ? reinterpret_cast<float*>(ws + hb) : nullptr;
  const size_t yrb = has_routed ? align256((size_t)T * k * d * 4) : 0;
  float* y_s = shared && ws ? reinterpret_cast<float*>(ws + hb + yrb) : nullptr;
  const size_t ysb = shared ? align256((size_t)T * d * 4) : 0;
  GemvArgs a;
  RecordOffsets orr{}, osh{};
  moe_status st = prepare(who, routed, ids_dev, k, shared, x_dev, x_dtype, T, act, y_r, y_s, workspace_dev,
                          workspace_bytes, true, true, &a, &orr, &osh);
  if (st != MOE_OK) return st;
  a.weights = weights_dev;
  a.residual = residual_dev;
  a.res_bf16 = residual_dtype == MOE_BF16;
  a.out = out_dev;
  a.out_bf16 = out_dtype == MOE_BF16;
  a.tile_counters = reinterpret_cast<uint32_t*>(ws + hb + yrb + ysb);
  const bool sb16 = sb_is_bf16(routed, k, shared);
  hipStream_t s = as_stream(stream);
  st = run_gate_up(a, orr, osh, x_dtype, sb16, T, s);
  if (st != MOE_OK) return st;
  return run_down(a, orr, osh, sb16, T, s, true);
}
