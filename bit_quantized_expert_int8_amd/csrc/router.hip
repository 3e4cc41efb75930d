// moe_rmsnorm, moe_router_topk and moe_combine.
//
// Router: each block holds the token's activation in LDS as fp32 and each of its four wavefronts
// computes one expert's logit with 16-byte int8 loads (coalesced along the row) and a wave reduction.
// The last block to finish for a token (agent-scope ticket counter in the caller's workspace) reads the
// token's logits back into LDS, takes the k best in rank order (larger first, ties: lower id first) and
// the softmax over them.  It resets the counter, so the workspace is
// reusable.  Logits travel between blocks by device-coherent stores and loads.
#include "common.h"

namespace moeq4 {
namespace {

constexpr int kRouterWaves = 4;
// One ticket counter per token, 256 bytes apart: a token's E / 4 blocks take their tickets at once, and
// with the counters of all tokens in one line every ticket of a batch would queue on one L2 channel.
constexpr int kCounterStride = 64;
constexpr int kMaxExperts = 1024;
constexpr int kMaxK = 32;
constexpr int kRouterChunks = 8;    // 16-byte chunks per lane: rows of up to 8192 int8
// from this many tokens on, logits by (token, 16 experts) blocks; below, one launch of router_kernel
constexpr int kSplitRouterMinT = 2;
// up to this many tokens the last logit block of a token selects (ticket, one launch); above, a second launch
// selects (measured: 123.3 against 124.6 us per layer at 32 tokens, 180.1 against 179.3 at 128)
constexpr int kTicketRouterMaxT = 32;

template <typename T>
__device__ __forceinline__ float load_act(const T* p, int64_t i);
template <>
__device__ __forceinline__ float load_act<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_act<uint16_t>(const uint16_t* p, int64_t i) { return bf16_bits_to_f32(p[i]); }

// 8 consecutive activations (16- or 32-byte aligned) as fp32
__device__ __forceinline__ void load8(const uint16_t* p, float v[8]) {
  const uint4 r = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void load8(const float* p, float v[8]) {
  const float4 a = reinterpret_cast<const float4*>(p)[0], b = reinterpret_cast<const float4*>(p)[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

__device__ __forceinline__ void store_act(void* out, bool bf16, int64_t i, float v) {
  if (bf16)
    reinterpret_cast<uint16_t*>(out)[i] = (uint16_t)f32_to_bf16_bits(v);
  else
    reinterpret_cast<float*>(out)[i] = v;
}

// The normalized activation of a router block, from this thread's 8-value pieces v[p] (elements
// (threadIdx.x + 256 p) * 8 ..) and the gain g[p], into xs [d] (LDS) and, if u_out, to memory:
// u[j] = round_x((x[j] * gamma[j]) * rinv), rinv = 1 / sqrt(sum_j x[j]^2 / d + eps).  The sum runs in the
// order of the single-launch layer's norm (per thread an fma chain over its pieces in index order, the
// wavefront sum, then the four wavefronts' sums in order), so both compute the same u.  Ends with a barrier.
template <typename XT, int P>
__device__ __forceinline__ void router_norm(const float (&v)[P][8], const float (&g)[P][8], int d, float eps, float* xs,
                                            void* u_out, int64_t u_off, float* wsum) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float ss = 0.f;
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int j0 = (threadIdx.x + 256 * p) * 8;
    float si = ss;
#pragma unroll
    for (int i = 0; i < 8; ++i) si = fmaf(v[p][i], v[p][i], si);
    ss = j0 < d ? si : ss;
  }
  ss = wave_sum(ss);
  if (lane == 0) wsum[wave] = ss;
  __syncthreads();
  float tot = wsum[0];
#pragma unroll
  for (int w = 1; w < 4; ++w) tot += wsum[w];
  const float rinv = 1.0f / sqrtf(tot / (float)d + eps);
  constexpr bool bf16 = sizeof(XT) == 2;
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int j0 = (threadIdx.x + 256 * p) * 8;
    if (j0 < d) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float u = (v[p][i] * g[p][i]) * rinv;
        xs[j0 + i] = bf16 ? bf16_bits_to_f32(f32_to_bf16_bits(u)) : u;   // the norm output's rounding point
        if (u_out) store_act(u_out, bf16, u_off + j0 + i, u);
      }
    }
  }
  __syncthreads();
}

// The k best of lgs[0..E) (larger first, equal values -> lower id) into sel_i / sel_v in rank order, by the
// block: wavefront 0 takes them with topk_wave for E <= 256, every thread ranks its candidates against all E
// values otherwise (the same selection and order).  Ends with a barrier.
__device__ __forceinline__ void router_rank(const float* lgs, int E, int k, int* sel_i, float* sel_v) {
  if (E <= 256) {
    if (threadIdx.x < 64) {
      int id = -1;
      float val = 0.f;
      auto run = [&](auto per) {
        constexpr int PER = decltype(per)::value;
        float v[PER];
#pragma unroll
        for (int m = 0; m < PER; ++m) {
          const int e = threadIdx.x + 64 * m;
          v[m] = e < E ? lgs[e] : 0.f;
        }
        topk_wave<PER>(v, E, k, id, val);
      };
      if (E <= 64) run(std::integral_constant<int, 1>());
      else if (E <= 128) run(std::integral_constant<int, 2>());
      else if (E <= 192) run(std::integral_constant<int, 3>());
      else run(std::integral_constant<int, 4>());
      if ((int)threadIdx.x < k) {
        sel_i[threadIdx.x] = id;
        sel_v[threadIdx.x] = val;
      }
    }
  } else {
    for (int c = threadIdx.x; c < E; c += 256) {
      const float vc = lgs[c];
      int rank = 0;
      for (int e2 = 0; e2 < E; ++e2) {
        const float u = lgs[e2];
        rank += (u > vc) | ((u == vc) & (e2 < c));
      }
      if (rank < k) {
        sel_i[rank] = c;
        sel_v[rank] = vc;
      }
    }
  }
  __syncthreads();
}

// ------------------------------------------------------------------------------------------------
// RMSNorm: one block per token
// ------------------------------------------------------------------------------------------------
template <typename XT>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const XT* __restrict__ x, const float* __restrict__ gamma, float eps,
                                                      int d, void* __restrict__ out, bool out_bf16) {
  __shared__ float partial[4];
  const int64_t t = blockIdx.x;
  const XT* xt = x + t * d;
  // 8 elements per thread and pass, every load issued before the first use; values stay in registers
  constexpr int kPasses = 16384 / (8 * 256);
  float v[kPasses][8];
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    const int j0 = (threadIdx.x + 256 * p) * 8;
    if (j0 < d) load8(xt + j0, v[p]);
  }
  float g[kPasses][8];
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    const int j0 = (threadIdx.x + 256 * p) * 8;
    if (j0 < d) load8(gamma + j0, g[p]);
  }
  // the order of the single-launch layer's norm (router_norm): fma chain per thread, the wavefront sum,
  // the four wavefronts' sums in order; u = (x * gamma) * rinv
  float ss = 0.f;
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    const int j0 = (threadIdx.x + 256 * p) * 8;
    float si = ss;
#pragma unroll
    for (int i = 0; i < 8; ++i) si = fmaf(v[p][i], v[p][i], si);
    ss = j0 < d ? si : ss;
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) partial[threadIdx.x >> 6] = ss;
  __syncthreads();
  float tot = partial[0];
#pragma unroll
  for (int w = 1; w < 4; ++w) tot += partial[w];
  const float r = 1.0f / sqrtf(tot / (float)d + eps);
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    const int j0 = (threadIdx.x + 256 * p) * 8;
    if (j0 < d) {
#pragma unroll
      for (int i = 0; i < 8; ++i) store_act(out, out_bf16, t * d + j0 + i, (v[p][i] * g[p][i]) * r);
    }
  }
}

// ------------------------------------------------------------------------------------------------
// Router GEMV + last-block top-k
// ------------------------------------------------------------------------------------------------
struct RouterArgs {
  const void* x;
  int d, E, k;
  const int8_t* w;
  const float* scale;
  const int32_t* forced;
  int32_t* ids;
  float* weights;
  float* logits;         // [T][E]: caller's buffer or workspace
  uint32_t* counters;    // [T] at a stride of kCounterStride words, zero between calls
  const float* gamma;    // RMSNorm gain [d], or NULL: the router reads x as is
  float eps;
  void* u_out;           // [T][d] normalized activation (x dtype), written by block 0; NULL = not wanted
};

__device__ __forceinline__ bool better(float v, int i, float v2, int i2) { return v > v2 || (v == v2 && i < i2); }

template <typename XT>
__global__ __launch_bounds__(256) void router_kernel(RouterArgs a) {
  extern __shared__ float xs[];                      // [d] fp32 activation
  __shared__ uint32_t last_flag;
  const int64_t t = blockIdx.y;
  const XT* x = reinterpret_cast<const XT*>(a.x) + t * a.d;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int e = blockIdx.x * kRouterWaves + wave;
  const int nch = a.d / 16;                          // 16-byte chunks of one int8 row
  const int8_t* row = a.w + (int64_t)(e < a.E ? e : 0) * a.d;
  // every load of the block in one round trip: this wave's weight chunks, then the activation
  int4 q[kRouterChunks];
#pragma unroll
  for (int m = 0; m < kRouterChunks; ++m) {
    const int c = lane + 64 * m;
    if (c < nch) q[m] = *reinterpret_cast<const int4*>(row + c * 16);
  }
  // activation (and the norm gain): 8 elements per thread and pass, all issued before any is used
  constexpr int kPasses = 8192 / (8 * 256);
  float v[kPasses][8], g[kPasses][8];
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    const int j0 = (threadIdx.x + 256 * p) * 8;
    if (j0 < a.d) {
      load8(x + j0, v[p]);
      if (a.gamma) load8(a.gamma + j0, g[p]);
    }
  }
  if (!a.gamma) {
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
      const int j0 = (threadIdx.x + 256 * p) * 8;
      if (j0 < a.d) {
        *reinterpret_cast<float4*>(xs + j0) = make_float4(v[p][0], v[p][1], v[p][2], v[p][3]);
        *reinterpret_cast<float4*>(xs + j0 + 4) = make_float4(v[p][4], v[p][5], v[p][6], v[p][7]);
      }
    }
    __syncthreads();
  } else {
    // RMSNorm fused in: every block reduces x in the same fixed order, so all blocks obtain the same u
    __shared__ float wsum[4];
    router_norm<XT, kPasses>(v, g, a.d, a.eps, xs, blockIdx.x == 0 ? a.u_out : nullptr, t * a.d, wsum);
  }

  if (e < a.E) {
    float acc = 0.f;
#pragma unroll
    for (int m = 0; m < kRouterChunks; ++m) {
      const int c = lane + 64 * m;
      if (c >= nch) break;
      const float4* xv = reinterpret_cast<const float4*>(xs + c * 16);
      const int qw[4] = {q[m].x, q[m].y, q[m].z, q[m].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 xx = xv[i];
        acc += (float)(int8_t)(qw[i] & 0xff) * xx.x;
        acc += (float)(int8_t)((qw[i] >> 8) & 0xff) * xx.y;
        acc += (float)(int8_t)((qw[i] >> 16) & 0xff) * xx.z;
        acc += (float)(int8_t)((qw[i] >> 24) & 0xff) * xx.w;
      }
    }
    acc = wave_sum(acc);
    // device-coherent store (bypasses the non-coherent per-XCD L2 state), so no L2 writeback is needed
    if (lane == 0) __hip_atomic_store(a.logits + t * a.E + e, acc * a.scale[e], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // Publish this block's logits, then take a ticket; the last block selects.  Agent-scope fences would
  // write back and invalidate the whole L2 of every XCD from every wave; instead the logits travel by
  // device-coherent stores/loads and each wave waits for its stores to complete before the barrier.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t ticket = __hip_atomic_fetch_add(a.counters + t * kCounterStride, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last_flag = (ticket == gridDim.x - 1) ? 1u : 0u;
  }
  __syncthreads();
  if (!last_flag) return;

  // The last block selects: candidate e is kept iff fewer than k logits beat it (larger value, or equal
  // value and lower id), and its rank is its position in the output (router_rank).
  __shared__ float lgs[kMaxExperts];
  __shared__ float sel_v[kMaxK];
  __shared__ int sel_i[kMaxK];
  const float* lg = a.logits + t * a.E;
#pragma unroll
  for (int p = 0; p < kMaxExperts / 256; ++p) {
    const int e2 = threadIdx.x + 256 * p;
    if (e2 < a.E) lgs[e2] = __hip_atomic_load(lg + e2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (a.forced) {
    if (threadIdx.x < a.k) {
      const int i = a.forced[t * a.k + threadIdx.x];
      sel_i[threadIdx.x] = i;
      sel_v[threadIdx.x] = (i >= 0 && i < a.E) ? lgs[i] : NAN;
    }
    __syncthreads();
  } else {
    router_rank(lgs, a.E, a.k, sel_i, sel_v);
  }
  // softmax over the k kept logits; every lane sums the same terms in the same order
  if (threadIdx.x < a.k) {
    float mx = sel_v[0];
    for (int r = 1; r < a.k; ++r) mx = fmaxf(mx, sel_v[r]);
    float den = 0.f;
    for (int r = 0; r < a.k; ++r) den += expf(sel_v[r] - mx);
    a.ids[t * a.k + threadIdx.x] = sel_i[threadIdx.x];
    a.weights[t * a.k + threadIdx.x] = expf(sel_v[threadIdx.x] - mx) / den;
  }
  if (threadIdx.x == 0) __hip_atomic_store(a.counters + t * kCounterStride, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------------------------------------------
// Router for several tokens: logits by (token, 16 experts), then the selection
// ------------------------------------------------------------------------------------------------
// With a block per four experts and the selection in the last block to finish, a batch's tokens each
// gather E / 4 blocks' logits through device-coherent stores and a ticket counter that those blocks
// update one after another; for 32 or 128 tokens that hand-off dominates.  A block per token instead is
// bound by one compute unit's arithmetic (E dot products of d int8 values).  So the logits come from a
// block per (token, kLogitExperts experts).  With TICKET (up to kTicketRouterMaxT tokens) they go out by
// device-coherent stores and the last of a token's E / 16 blocks (ticket) selects, as router_kernel does;
// otherwise they go out with plain stores and a second launch selects, a block per token, after the kernel
// boundary has made them visible.  Every per-expert sum, the norm's reduction and the ranking run exactly
// as in router_kernel (same lanes, same order): the results agree bit for bit.  (Blocks that keep their
// rows for several tokens, the activations staged in LDS, were measured slower: a token's norm and dot
// products take a block about 3.5 us, so four tokens in turn cost more than the second round of blocks.)
constexpr int kLogitExperts = 16;   // experts per block: 4 per wavefront

// The dot products of a wavefront's kRows rows with the activation in LDS (xs, fp32): lane l takes the
// 16-value slices l, l + 64, ... of each row; the rows' sums run side by side (independent chains), each in
// the same order as alone; returns the wavefront sums.
template <int NCH, int kRows>
__device__ __forceinline__ void logit_rows(const int4 (&q)[kRows][NCH], const float* xs, int nch, float (&out)[kRows]) {
  const int lane = threadIdx.x & 63;
  // a lane's 16-value slices of the activation are the same for all of the wave's experts: read once
  float4 xr[NCH][4];
#pragma unroll
  for (int m = 0; m < NCH; ++m) {
    const int c = lane + 64 * m;
#pragma unroll
    for (int k4 = 0; k4 < 4; ++k4)
      xr[m][k4] = c < nch ? reinterpret_cast<const float4*>(xs + c * 16)[k4] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  float acc[kRows];
#pragma unroll
  for (int r = 0; r < kRows; ++r) acc[r] = 0.f;
#pragma unroll
  for (int m = 0; m < NCH; ++m) {
    const int c = lane + 64 * m;
    if (c >= nch) break;
#pragma unroll
    for (int k4 = 0; k4 < 4; ++k4) {
      const float4 xx = xr[m][k4];
#pragma unroll
      for (int r = 0; r < kRows; ++r) {
        const int qw = k4 == 0 ? q[r][m].x : k4 == 1 ? q[r][m].y : k4 == 2 ? q[r][m].z : q[r][m].w;
        acc[r] += (float)(int8_t)(qw & 0xff) * xx.x;
        acc[r] += (float)(int8_t)((qw >> 8) & 0xff) * xx.y;
        acc[r] += (float)(int8_t)((qw >> 16) & 0xff) * xx.z;
        acc[r] += (float)(int8_t)((qw >> 24) & 0xff) * xx.w;
      }
    }
  }
#pragma unroll
  for (int r = 0; r < kRows; ++r) out[r] = wave_sum(acc[r]);
}

// This wavefront's kRows rows of int8 weights (16-byte slices, as logit_rows reads them) and their scales
template <int NCH, int kRows>
__device__ __forceinline__ void load_logit_rows(const RouterArgs& a, int e0, int nch, int4 (&q)[kRows][NCH], float (&sc)[kRows]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    const int e = e0 + r;
    const int8_t* row = a.w + (int64_t)(e < a.E ? e : 0) * a.d;
    sc[r] = a.scale[e < a.E ? e : 0];
#pragma unroll
    for (int m = 0; m < NCH; ++m) {
      const int c = lane + 64 * m;
      if (c < nch) q[r][m] = *reinterpret_cast<const int4*>(row + c * 16);
    }
  }
}

template <typename XT, int NCH, bool TICKET>
__global__ __launch_bounds__(256) void router_logits_kernel(RouterArgs a) {
  extern __shared__ float xs[];   // [d] fp32 activation
  constexpr int kRows = kLogitExperts / 4;
  const int64_t t = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nch = a.d / 16;
  const int e0 = blockIdx.x * kLogitExperts + wave * kRows;
  // this wave's rows and scales first, then the activation (and the norm gain), all in one round trip
  int4 q[kRows][NCH];
  float sc[kRows];
  load_logit_rows<NCH, kRows>(a, e0, nch, q, sc);
  constexpr int kPasses = (NCH + 1) / 2;   // 8 values per thread and pass: rows of d <= 1024 NCH
  float v[kPasses][8], g[kPasses][8];
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    const int j0 = (threadIdx.x + 256 * p) * 8;
    if (j0 < a.d) {
      load8(reinterpret_cast<const XT*>(a.x) + t * a.d + j0, v[p]);
      if (a.gamma) load8(a.gamma + j0, g[p]);
    }
  }
  if (!a.gamma) {
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
      const int j0 = (threadIdx.x + 256 * p) * 8;
      if (j0 < a.d) {
        *reinterpret_cast<float4*>(xs + j0) = make_float4(v[p][0], v[p][1], v[p][2], v[p][3]);
        *reinterpret_cast<float4*>(xs + j0 + 4) = make_float4(v[p][4], v[p][5], v[p][6], v[p][7]);
      }
    }
    __syncthreads();
  } else {
    // the norm as in router_kernel
    __shared__ float wsum[4];
    router_norm<XT, kPasses>(v, g, a.d, a.eps, xs, blockIdx.x == 0 ? a.u_out : nullptr, t * a.d, wsum);
  }
  float lgt[kRows];
  logit_rows<NCH, kRows>(q, xs, nch, lgt);
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    const int e = e0 + r;
    if (lane == 0 && e < a.E) {
      if (TICKET) __hip_atomic_store(a.logits + t * a.E + e, lgt[r] * sc[r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      else a.logits[t * a.E + e] = lgt[r] * sc[r];
    }
  }
  if (!TICKET) return;
  __shared__ uint32_t last_flag;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t ticket = __hip_atomic_fetch_add(a.counters + t * kCounterStride, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last_flag = (ticket == gridDim.x - 1) ? 1u : 0u;
  }
  __syncthreads();
  if (!last_flag) return;
  __shared__ float lgs[kMaxExperts];
  __shared__ float sel_v[kMaxK];
  __shared__ int sel_i[kMaxK];
  const float* lg = a.logits + t * a.E;
  for (int e2 = threadIdx.x; e2 < a.E; e2 += 256) lgs[e2] = __hip_atomic_load(lg + e2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (a.forced) {
    if (threadIdx.x < a.k) {
      const int i = a.forced[t * a.k + threadIdx.x];
      sel_i[threadIdx.x] = i;
      sel_v[threadIdx.x] = (i >= 0 && i < a.E) ? lgs[i] : NAN;
    }
    __syncthreads();
  } else {
    router_rank(lgs, a.E, a.k, sel_i, sel_v);
  }
  if (threadIdx.x < a.k) {
    float mx = sel_v[0];
    for (int rr = 1; rr < a.k; ++rr) mx = fmaxf(mx, sel_v[rr]);
    float den = 0.f;
    for (int rr = 0; rr < a.k; ++rr) den += expf(sel_v[rr] - mx);
    a.ids[t * a.k + threadIdx.x] = sel_i[threadIdx.x];
    a.weights[t * a.k + threadIdx.x] = expf(sel_v[threadIdx.x] - mx) / den;
  }
  if (threadIdx.x == 0) __hip_atomic_store(a.counters + t * kCounterStride, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A block per token: the token's logits into LDS, top-k by rank and the softmax, as in router_kernel.
__global__ __launch_bounds__(256) void router_select_kernel(RouterArgs a) {
  __shared__ float lgs[kMaxExperts];
  __shared__ float sel_v[kMaxK];
  __shared__ int sel_i[kMaxK];
  const int64_t t = blockIdx.x;
  for (int e = threadIdx.x; e < a.E; e += 256) lgs[e] = a.logits[t * a.E + e];
  __syncthreads();
  if (a.forced) {
    if (threadIdx.x < a.k) {
      const int i = a.forced[t * a.k + threadIdx.x];
      sel_i[threadIdx.x] = i;
      sel_v[threadIdx.x] = (i >= 0 && i < a.E) ? lgs[i] : NAN;
    }
    __syncthreads();
  } else {
    router_rank(lgs, a.E, a.k, sel_i, sel_v);
  }
  if (threadIdx.x < a.k) {
    float mx = sel_v[0];
    for (int r = 1; r < a.k; ++r) mx = fmaxf(mx, sel_v[r]);
    float den = 0.f;
    for (int r = 0; r < a.k; ++r) den += expf(sel_v[r] - mx);
    a.ids[t * a.k + threadIdx.x] = sel_i[threadIdx.x];
    a.weights[t * a.k + threadIdx.x] = expf(sel_v[threadIdx.x] - mx) / den;
  }
}

// ------------------------------------------------------------------------------------------------
// combine
// ------------------------------------------------------------------------------------------------
template <typename RT, int KT>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y, const float* __restrict__ w,
                                                      const float* __restrict__ ys, const RT* __restrict__ res, int k,
                                                      int d, void* __restrict__ out, bool out_bf16) {
  const int64_t t = blockIdx.y;
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= d) return;
  // all loads first (one memory round trip), then the sum in the fixed order i = 0..k-1; loads past k
  // are clamped to a valid row and weighted by 0, so the code has no data-dependent branches
  float yv[KT], wv[KT];
  if (k > 0) {
#pragma unroll
    for (int i = 0; i < KT; ++i) {
      const int ic = i < k ? i : k - 1;
      yv[i] = y[(t * k + ic) * d + j];
      wv[i] = w[t * k + ic];
    }
  } else {
#pragma unroll
    for (int i = 0; i < KT; ++i) yv[i] = wv[i] = 0.f;
  }
  const float s = ys ? ys[t * d + j] : 0.f;
  const float r = res ? load_act(res, t * d + j) : 0.f;
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < KT; ++i) acc = __builtin_fmaf(i < k ? wv[i] : 0.f, yv[i], acc);
  acc += s;
  acc += r;
  store_act(out, out_bf16, t * d + j, acc);
}

}  // namespace
}  // namespace moeq4

using namespace moeq4;

extern "C" moe_status moe_rmsnorm(const void* x_dev, moe_dtype x_dtype, const float* gamma_dev, float eps, int32_t T,
                                  int32_t d, void* out_dev, moe_dtype out_dtype, void* stream) {
  if (!x_dev || !gamma_dev || !out_dev) return fail(MOE_ERR_INVALID_ARG, "moe_rmsnorm: NULL pointer");
  if (T < 1 || d < 8 || d % 8 || d > 16384) return fail(MOE_ERR_INVALID_ARG, "moe_rmsnorm: T=%d d=%d (multiple of 8, <= 16384)", T, d);
  if (!aligned(x_dev, 16) || !aligned(gamma_dev, 16)) return fail(MOE_ERR_INVALID_ARG, "moe_rmsnorm: x or gamma not 16-byte aligned");
  if ((x_dtype != MOE_F32 && x_dtype != MOE_BF16) || (out_dtype != MOE_F32 && out_dtype != MOE_BF16))
    return fail(MOE_ERR_INVALID_ARG, "moe_rmsnorm: bad dtype");
  if (!(eps >= 0.f)) return fail(MOE_ERR_INVALID_ARG, "moe_rmsnorm: eps must be >= 0");
  hipStream_t s = as_stream(stream);
  if (x_dtype == MOE_BF16)
    hipLaunchKernelGGL(rmsnorm_kernel<uint16_t>, dim3(T), dim3(256), 0, s, (const uint16_t*)x_dev, gamma_dev, eps, d,
                       out_dev, out_dtype == MOE_BF16);
  else
    hipLaunchKernelGGL(rmsnorm_kernel<float>, dim3(T), dim3(256), 0, s, (const float*)x_dev, gamma_dev, eps, d, out_dev,
                       out_dtype == MOE_BF16);
  return check_launch("moe_rmsnorm");
}

extern "C" size_t moe_router_workspace_bytes(int32_t T, int32_t E) {
  if (T < 1 || E < 1) return 0;
  const size_t counters = (size_t)T * kCounterStride * 4;
  return counters + (size_t)T * E * 4;
}

namespace {
moe_status router_launch(const char* who, const void* x_dev, moe_dtype x_dtype, int32_t T, int32_t d, const int8_t* w_dev,
                         const float* row_scale_dev, int32_t E, int32_t k, const int32_t* forced_ids_dev, int32_t* ids_dev,
                         float* weights_dev, float* logits_dev, void* workspace_dev, size_t workspace_bytes,
                         const float* gamma_dev, float eps, void* u_dev, void* stream);
}

extern "C" moe_status moe_router_topk(const void* x_dev, moe_dtype x_dtype, int32_t T, int32_t d, const int8_t* w_dev,
                                      const float* row_scale_dev, int32_t E, int32_t k, const int32_t* forced_ids_dev,
                                      int32_t* ids_dev, float* weights_dev, float* logits_dev, void* workspace_dev,
                                      size_t workspace_bytes, void* stream) {
  return router_launch("moe_router_topk", x_dev, x_dtype, T, d, w_dev, row_scale_dev, E, k, forced_ids_dev, ids_dev,
                       weights_dev, logits_dev, workspace_dev, workspace_bytes, nullptr, 0.f, nullptr, stream);
}

extern "C" moe_status moe_norm_router_topk(const void* x_dev, moe_dtype x_dtype, const float* gamma_dev, float eps, int32_t T,
                                           int32_t d, const int8_t* w_dev, const float* row_scale_dev, int32_t E, int32_t k,
                                           const int32_t* forced_ids_dev, int32_t* ids_dev, float* weights_dev,
                                           float* logits_dev, void* u_dev, void* workspace_dev, size_t workspace_bytes,
                                           void* stream) {
  if (!gamma_dev || !u_dev) return fail(MOE_ERR_INVALID_ARG, "moe_norm_router_topk: gamma or u is NULL");
  if (!(eps >= 0.f)) return fail(MOE_ERR_INVALID_ARG, "moe_norm_router_topk: eps must be >= 0");
  return router_launch("moe_norm_router_topk", x_dev, x_dtype, T, d, w_dev, row_scale_dev, E, k, forced_ids_dev, ids_dev,
                       weights_dev, logits_dev, workspace_dev, workspace_bytes, gamma_dev, eps, u_dev, stream);
}

namespace {
moe_status router_launch(const char* who, const void* x_dev, moe_dtype x_dtype, int32_t T, int32_t d, const int8_t* w_dev,
                         const float* row_scale_dev, int32_t E, int32_t k, const int32_t* forced_ids_dev, int32_t* ids_dev,
                         float* weights_dev, float* logits_dev, void* workspace_dev, size_t workspace_bytes,
                         const float* gamma_dev, float eps, void* u_dev, void* stream) {
  if (!x_dev || !w_dev || !row_scale_dev || !ids_dev || !weights_dev || !workspace_dev)
    return fail(MOE_ERR_INVALID_ARG, "%s: NULL pointer", who);
  if (x_dtype != MOE_F32 && x_dtype != MOE_BF16) return fail(MOE_ERR_INVALID_ARG, "%s: bad x_dtype", who);
  if (T < 1 || T > 65535) return fail(MOE_ERR_INVALID_ARG, "%s: T=%d", who, T);
  if (E < 1 || E > kMaxExperts || k < 1 || k > E || k > kMaxK)
    return fail(MOE_ERR_UNSUPPORTED, "%s: E=%d k=%d (need 1 <= k <= min(E, 32), E <= 1024)", who, E, k);
  if (d < 16 || d % 16 || d > 8192) return fail(MOE_ERR_UNSUPPORTED, "%s: d=%d (multiple of 16, <= 8192)", who, d);
  if (!aligned(w_dev, 16) || !aligned(x_dev, 16))
    return fail(MOE_ERR_INVALID_ARG, "%s: router weights or x not 16-byte aligned", who);
  const size_t need = moe_router_workspace_bytes(T, E);
  if (workspace_bytes < need)
    return fail(MOE_ERR_INVALID_ARG, "%s: workspace %zu bytes < %zu", who, workspace_bytes, need);
  if (!aligned(workspace_dev, 256)) return fail(MOE_ERR_INVALID_ARG, "%s: workspace not 256-byte aligned", who);
  RouterArgs a;
  a.x = x_dev;
  a.d = d;
  a.E = E;
  a.k = k;
  a.w = w_dev;
  a.scale = row_scale_dev;
  a.forced = forced_ids_dev;
  a.ids = ids_dev;
  a.weights = weights_dev;
  a.counters = static_cast<uint32_t*>(workspace_dev);
  a.logits = logits_dev ? logits_dev
                        : reinterpret_cast<float*>(static_cast<char*>(workspace_dev) + (size_t)T * kCounterStride * 4);
  a.gamma = gamma_dev;
  a.eps = eps;
  a.u_out = u_dev;
  if (gamma_dev && !aligned(u_dev, 16)) return fail(MOE_ERR_INVALID_ARG, "%s: u not 16-byte aligned", who);
  const size_t lds = (size_t)d * sizeof(float);
  hipStream_t s = as_stream(stream);
  if (T >= kSplitRouterMinT) {
    // logits by (token, 16 experts), then the selection by token (the same results as the kernel below)
    const int nch = (d / 16 + 63) / 64;
    const int ne = (E + kLogitExperts - 1) / kLogitExperts;
    auto go = [&](auto nc) {
      constexpr int NCH = decltype(nc)::value;
      if (T <= kTicketRouterMaxT) {
        if (x_dtype == MOE_BF16)
          hipLaunchKernelGGL((router_logits_kernel<uint16_t, NCH, true>), dim3(ne, T), dim3(256), lds, s, a);
        else
          hipLaunchKernelGGL((router_logits_kernel<float, NCH, true>), dim3(ne, T), dim3(256), lds, s, a);
        return check_launch(who);
      }
      if (x_dtype == MOE_BF16)
        hipLaunchKernelGGL((router_logits_kernel<uint16_t, NCH, false>), dim3(ne, T), dim3(256), lds, s, a);
      else
        hipLaunchKernelGGL((router_logits_kernel<float, NCH, false>), dim3(ne, T), dim3(256), lds, s, a);
      const moe_status st = check_launch(who);
      if (st != MOE_OK) return st;
      hipLaunchKernelGGL(router_select_kernel, dim3(T), dim3(256), 0, s, a);
      return check_launch(who);
    };
    if (nch <= 1) return go(std::integral_constant<int, 1>());
    if (nch <= 2) return go(std::integral_constant<int, 2>());
    if (nch <= 3) return go(std::integral_constant<int, 3>());
    if (nch <= 4) return go(std::integral_constant<int, 4>());
    return go(std::integral_constant<int, 8>());
  }
  dim3 grid((E + kRouterWaves - 1) / kRouterWaves, T);
  if (x_dtype == MOE_BF16)
    hipLaunchKernelGGL(router_kernel<uint16_t>, grid, dim3(256), lds, s, a);
  else
    hipLaunchKernelGGL(router_kernel<float>, grid, dim3(256), lds, s, a);
  return check_launch(who);
}
}  // namespace

extern "C" moe_status moe_combine(const float* y_routed_dev, const float* weights_dev, const float* y_shared_dev,
                                  const void* residual_dev, moe_dtype residual_dtype, int32_t T, int32_t k, int32_t d,
                                  void* out_dev, moe_dtype out_dtype, void* stream) {
  if (!out_dev || (k > 0 && (!y_routed_dev || !weights_dev))) return fail(MOE_ERR_INVALID_ARG, "moe_combine: NULL pointer");
  if (T < 1 || T > 65535 || k < 0 || k > kMaxK || d < 1) return fail(MOE_ERR_INVALID_ARG, "moe_combine: T=%d k=%d d=%d", T, k, d);
  if ((out_dtype != MOE_F32 && out_dtype != MOE_BF16) || (residual_dev && residual_dtype != MOE_F32 && residual_dtype != MOE_BF16))
    return fail(MOE_ERR_INVALID_ARG, "moe_combine: bad dtype");
  dim3 grid((d + 255) / 256, T);
  hipStream_t s = as_stream(stream);
  const bool rb = residual_dev && residual_dtype == MOE_BF16, ob = out_dtype == MOE_BF16;
  const uint16_t* r16 = (const uint16_t*)residual_dev;
  const float* r32 = (const float*)residual_dev;
  if (k <= 8) {
    if (rb) hipLaunchKernelGGL((combine_kernel<uint16_t, 8>), grid, dim3(256), 0, s, y_routed_dev, weights_dev, y_shared_dev, r16, k, d, out_dev, ob);
    else hipLaunchKernelGGL((combine_kernel<float, 8>), grid, dim3(256), 0, s, y_routed_dev, weights_dev, y_shared_dev, r32, k, d, out_dev, ob);
  } else {
    if (rb) hipLaunchKernelGGL((combine_kernel<uint16_t, kMaxK>), grid, dim3(256), 0, s, y_routed_dev, weights_dev, y_shared_dev, r16, k, d, out_dev, ob);
    else hipLaunchKernelGGL((combine_kernel<float, kMaxK>), grid, dim3(256), 0, s, y_routed_dev, weights_dev, y_shared_dev, r32, k, d, out_dev, ob);
  }
  return check_launch("moe_combine");
}
