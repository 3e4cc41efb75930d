// moe_decode_layer: one MoE layer of batch-1 decode in a single launch.
//
// The whole step ([G26] "Le pipeline de traitement": route with the 8-bit router, run the selected
// experts and the shared expert, combine; [G26] "Concurrence pour masquer la latence": the shared expert
// does not wait for the routing) as one grid whose blocks play five roles, laid out in dependency order:
//
//   [router | shared gate/up | routed gate/up | shared down | routed down]
//
//   router            one expert per wavefront: RMSNorm of x, int8 dot product, logit published, then
//                     that expert's rank among all logits (its routing entry if it is selected)
//   shared gate/up    8 features of the shared expert (needs only x: starts at once)
//   routed gate/up    8 features of the i-th selected expert: waits for its entry of the routing (or
//                     takes the forced ids: no wait at all)
//   shared down       16 rows of the shared expert, once all of its gate/up blocks are done
//   routed down       64 rows of the i-th selected expert, once that expert's gate/up blocks are done;
//                     its code words are loaded before the wait, so they stream while gate/up finishes
//
// Down blocks publish their rows tagged with the call; the block of the last routed slot keeps its own rows,
// polls the other k contributions to its 64 rows, and applies the routing-weighted combine and the
// residual, in the order of moe_combine.
//
// Apart from the router blocks (below), each block only waits on blocks with smaller indices, which the
// dispatcher starts first, so every wait is on work that is running or finished.  Waits are bounded: a
// wait that runs out sets the sticky status word of the workspace instead of hanging (results are then
// invalid).  Values cross blocks by device-coherent stores and loads and 32-bit relaxed device-scope
// counters.  Nothing waits for the end of the call: each counter is zeroed by the arrival that completes
// it, and flags and published values carry the call's tag, so the workspace is ready for the next call
// when the last block exits.
//
// The routing carries no counter.  Each logit is stored with the call's tag in the upper half of a 64-bit
// word (one store, single-copy atomic), in 8 replicas.  Every router wavefront then waits until all E tags match and
// counts the logits ranked before its own (larger, or equal with a smaller id); if that rank r is below
// k, it stores (id, logit), tagged, as entry r of each of 16 route replicas.  A block that needs the
// routing polls one replica until its k tags match and, if it needs the gate weights, takes the softmax
// of the k logits itself (every block the same way, so all agree).  The tag is the call number: each block
// keeps a count of calls in a workspace word of its own, read and advanced when the block starts.  The router
// blocks are the first 32 of the grid, all resident at once: they are the only blocks that wait on blocks
// with larger indices.
//
// The normalized activation is computed by every block that needs it with the same fixed-order
// reduction, so all of them (and the router) see the same u:
//   u[j] = round_x( (x[j] * gamma[j]) * rinv ),  rinv = 1 / sqrt(sum_j x[j]^2 / d + eps)
// The expert arithmetic is that of q4_expert_gemv (q4_device.h); the gate/up blocks split the row
// between their four wavefronts, the routed down blocks give each wavefront 16 whole rows.
#include <mutex>

#include "q4_device.h"

namespace moeq4 {
namespace {

constexpr int kThreads = 256;
constexpr int kLayerMaxE = 256;
constexpr int kLayerMaxD = 4096;
constexpr int kLayerMaxF = 1024;
constexpr int kLayerMaxK = 32;
constexpr int kSpinLimit = 1 << 18;       // polls (about 0.1 s); a legitimate wait takes tens of polls

// Synchronisation lives in 256-byte lines at the front of the workspace.  Many blocks polling one word
// while others increment it serialize at the memory-side atomic unit, so waiting blocks poll flag lines
// of their own: the arrival that completes a set writes the call's tag into each of its n_flags lines.  A
// set with many arrivals counts them on n_sub sub-counters first (each on its own line); the last arrival
// of a sub-counter bumps the top counter.  Small sets (n_sub = 1) save that second atomic round trip.
// The arrival that completes a counter sets it back to zero (no other block touches it again in the call),
// and flags hold the tag of the call that raised them, so nothing needs clearing between calls.
constexpr int kLW = 64;             // 32-bit words per line
struct SyncSet {
  uint32_t* base;                   // lines: [n_sub sub-counters][top][n_flags flags]
  int n_sub, n_flags;
  uint32_t total;                   // arrivals that complete the set (waiters on a set without flag lines
                                    // poll its counter for this value)
};
constexpr int kSharedSub = 16, kSharedFlags = 16;
constexpr int kSlotSub = 1, kSlotFlags = 8;
constexpr int kDoneSub = 1;         // the layer-done set counts combined 64-row blocks
// line 0: status word (sticky, bit 0 = a bounded wait ran out); then the sets shared, done, slots
constexpr int kXFlags = 64;      // flags announcing a layer's output to the next layer of the launch
constexpr int kLinesFixed = 1 + (kSharedSub + 1 + kSharedFlags) + (kDoneSub + 1 + kXFlags);
constexpr int kRouteReplicas = 16;   // copies of the tagged routing (pollers spread over them)
constexpr int kLgReplicas = 8;       // copies of the tagged logits (the router wavefronts poll them)
constexpr int kLinesPerSlot = kSlotSub + 1 + kSlotFlags;

struct LayerPool {
  const char* base;
  int64_t record_bytes;
  int32_t n_records, F;
  int64_t gu_q, gu_sb, dn_q, dn_sb;
};

struct LayerArgs {
  const void* x;
  const float* gamma;
  float eps;
  int32_t residual;
  const int8_t* rw;
  const float* rs;
  int32_t E, k, d, act;
  const int32_t* forced;
  const int32_t* gemv_ids;
  LayerPool routed, shared;
  int32_t has_shared;
  int32_t* ids_out;
  float* weights_out;
  float* logits_out;
  void* u_out;         // the normalized activation [d] in the activation dtype, or NULL
  void* out;
  int32_t x_ws, out_ws;    // activations exchanged through the workspace, in the activation dtype and read
                           // and written coherently (the layers between the first input and the last
                           // output of a launch)
  uint32_t* status;
  uint32_t tag;                          // this call's tag: 1 + the calls counted in this block's word
  SyncSet shared_h, done;                // done = this layer's output complete: counts combined 64-row
                                         // blocks (flags: the next layer of the launch)
  SyncSet prev_x;                        // the previous layer's done, or base == NULL
  uint32_t* slot_base;                   // per-slot sets, kLinesPerSlot lines apart
  uint32_t* prev_slot_base;              // the previous layer's per-slot sets, or NULL
  int32_t last_layer;                    // no later layer of the launch waits for this one
  uint64_t* lg_tag;    // [kLgReplicas][E] (tag << 32) | logit bits
  uint64_t* route;     // [kRouteReplicas][2][kLayerMaxK] (tag << 32) | id, (tag << 32) | weight bits
  float* h_routed;     // [k][F]
  float* h_shared;     // [S]
  uint64_t* y_routed;  // [k][d] (tag << 32) | row result bits
  uint64_t* y_shared;  // [d]    (tag << 32) | row result bits
  int32_t nR, nSG, nRG, nSD, nRD;
};

__device__ __forceinline__ SyncSet slot_set(const LayerArgs& a, int i) {
  return SyncSet{a.slot_base + (int64_t)i * kLinesPerSlot * kLW, kSlotSub, kSlotFlags, (uint32_t)(a.routed.F / 8)};
}

__device__ __forceinline__ float ld_c(const float* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ void st_c(float* p, float v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ void st_cu(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_cu(const uint32_t* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ void st_c64(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_c64(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// 16 bytes at byte offset `off` of the buffer `r` describes, loaded coherently at device scope (sc1)
__device__ __forceinline__ uint4 ld_c128(__amdgpu_buffer_rsrc_t r, int off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 16 /* sc1 */);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
// A raw buffer over n bytes at p (out-of-range loads return zero)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_buffer(const void* p, int n) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, n, 0x00020000);
}
__device__ __forceinline__ uint32_t add_cu(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Raise every flag of set `s` with this call's tag: called by a whole wavefront, lane f writes flag line f
// (n_flags <= 64).
__device__ __forceinline__ void raise_flags(const SyncSet& s, uint32_t tag) {
  const int lane = threadIdx.x & 63;
  if (lane < s.n_flags) st_cu(s.base + (s.n_sub + 1 + lane) * kLW, tag);
}

// One arrival (n units) out of `total` on set `s`, made by wavefront 0 of a block (all 64 lanes, after
// the block's published stores completed); `idx` in [0, total) picks the sub-counter.  Lane 0 makes the
// atomic round trips and zeroes each counter its arrival completed.  The arrival that completes the set
// raises its flags with `tag`.
__device__ __forceinline__ void arrive(const SyncSet& s, int idx, int total, uint32_t tag, uint32_t n = 1u) {
  uint32_t done = 0u;
  if ((threadIdx.x & 63) == 0) {
    if (s.n_sub > 1) {
      const int sub = idx % s.n_sub;
      const uint32_t expect = (uint32_t)((total - sub + s.n_sub - 1) / s.n_sub);
      const uint32_t subs_used = (uint32_t)(total < s.n_sub ? total : s.n_sub);
      if (add_cu(s.base + sub * kLW, 1u) == expect - 1) {
        st_cu(s.base + sub * kLW, 0u);
        if (add_cu(s.base + s.n_sub * kLW, 1u) == subs_used - 1) {
          st_cu(s.base + s.n_sub * kLW, 0u);
          done = 1u;
        }
      }
    } else if (add_cu(s.base, n) + n == (uint32_t)total) {
      st_cu(s.base, 0u);
      done = 1u;
    }
  }
  done = __builtin_amdgcn_readfirstlane(done);
  if (done) raise_flags(s, tag);
}

// Block-wide bounded wait for set `s` (n_flags > 0) to be completed by the call tagged `tag`: thread 0
// polls flag line `who` mod n_flags.  Ends with a block barrier.
__device__ __forceinline__ void wait_set(const SyncSet& s, int who, uint32_t tag, uint32_t* status) {
  if (threadIdx.x == 0) {
    uint32_t* f = s.base + (s.n_sub + 1 + who % s.n_flags) * kLW;
    uint32_t v = __hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    int n = 0;
    while (v != tag && n < kSpinLimit) {
      __builtin_amdgcn_s_sleep(1);
      v = __hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      ++n;
    }
    if (v != tag) __hip_atomic_fetch_or(status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
}

// Publish: every thread's coherent stores have completed before wavefront 0 arrives on the set.
__device__ __forceinline__ void publish(const SyncSet& s, int idx, int total, uint32_t tag) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x < 64) arrive(s, idx, total, tag);
}

// ------------------------------------------------------------------------------------------------
// the normalized activation
// ------------------------------------------------------------------------------------------------
struct NormLds {
  float wsum[kThreads / 64];
};

// u[j] from x[j] * gamma[j], rounded to the activation dtype (the norm output's rounding point)
template <typename XT>
__device__ __forceinline__ float u_of(float xg, float rinv) {
  const float u = xg * rinv;
  return sizeof(XT) == 2 ? bf16_bits_to_f32(f32_to_bf16_bits(u)) : u;
}

// u[0..d) into LDS: u[j] = round_x((x[j] * gamma[j]) * rinv), rinv = 1 / sqrt(sum_j x[j]^2 / d + eps), or
// u = x without gamma.  Fixed reduction order: per thread over its elements in index order, the wavefront
// sum, then the four waves in order (every thread adds the four partial sums itself, the same way).
// Every load of x and gamma is issued before the first use, without branches in between (an element
// index past d reads element 0, which is discarded): a conversion or a branch between two loads makes the
// compiler wait for the first before issuing the second.  The forms (x a previous layer's output in the
// workspace, read with coherent 16-byte loads; with or without gamma) are separate instantiations for the
// same reason.
template <typename XT, bool XWS, bool GAMMA>
__device__ __forceinline__ void norm_to_lds_impl(const LayerArgs& a, float* u, NormLds& nl) {
  constexpr int kIt = kLayerMaxD / (kThreads * 8);
  constexpr int kXw = sizeof(XT) == 4 ? 2 : 1;   // 16-byte words per 8 elements
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  bool live[kIt];
  uint4 xw[kIt][kXw];
  float4 gw[kIt][2];
#pragma unroll
  for (int it = 0; it < kIt; ++it) {
    const int j = (threadIdx.x + it * kThreads) * 8;
    live[it] = j < a.d;
    const int j0 = live[it] ? j : 0;
    if (XWS) {
      const __amdgpu_buffer_rsrc_t xr = raw_buffer(a.x, a.d * (int)sizeof(XT));
#pragma unroll
      for (int w = 0; w < kXw; ++w) xw[it][w] = ld_c128(xr, (j0 * (int)sizeof(XT)) + 16 * w);
    } else {
      const uint4* xp = reinterpret_cast<const uint4*>(reinterpret_cast<const XT*>(a.x) + j0);
#pragma unroll
      for (int w = 0; w < kXw; ++w) xw[it][w] = xp[w];
    }
    if (GAMMA) {
      gw[it][0] = reinterpret_cast<const float4*>(a.gamma + j0)[0];
      gw[it][1] = reinterpret_cast<const float4*>(a.gamma + j0)[1];
    }
  }
  float v[kIt][8];
#pragma unroll
  for (int it = 0; it < kIt; ++it) {
    if (kXw == 1) {
      const uint32_t q[4] = {xw[it][0].x, xw[it][0].y, xw[it][0].z, xw[it][0].w};
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        v[it][2 * m] = __uint_as_float(q[m] << 16);
        v[it][2 * m + 1] = __uint_as_float(q[m] & 0xffff0000u);
      }
    } else {
      const uint32_t q[8] = {xw[it][0].x, xw[it][0].y, xw[it][0].z, xw[it][0].w,
                             xw[it][kXw - 1].x, xw[it][kXw - 1].y, xw[it][kXw - 1].z, xw[it][kXw - 1].w};
#pragma unroll
      for (int i = 0; i < 8; ++i) v[it][i] = __uint_as_float(q[i]);
    }
  }
  float rinv = 1.0f;
  if (GAMMA) {
    float ss = 0.f;
#pragma unroll
    for (int it = 0; it < kIt; ++it) {
      float si = ss;
#pragma unroll
      for (int i = 0; i < 8; ++i) si = fmaf(v[it][i], v[it][i], si);
      ss = live[it] ? si : ss;
    }
    ss = wave_sum(ss);
    if (lane == 0) nl.wsum[wave] = ss;
    __syncthreads();
    float t = nl.wsum[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) t += nl.wsum[w];
    rinv = 1.0f / sqrtf(t / (float)a.d + a.eps);
  }
#pragma unroll
  for (int it = 0; it < kIt; ++it) {
    if (!live[it]) continue;
    const int j0 = (threadIdx.x + it * kThreads) * 8;
    float o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float gi = i < 4 ? (&gw[it][0].x)[i] : (&gw[it][1].x)[i - 4];
      o[i] = GAMMA ? u_of<XT>(v[it][i] * gi, rinv) : v[it][i];
    }
    reinterpret_cast<float4*>(u + j0)[0] = make_float4(o[0], o[1], o[2], o[3]);
    reinterpret_cast<float4*>(u + j0)[1] = make_float4(o[4], o[5], o[6], o[7]);
  }
  __syncthreads();
}

template <typename XT>
__device__ __forceinline__ void norm_to_lds(const LayerArgs& a, float* u, NormLds& nl) {
  if (a.x_ws) {
    if (a.gamma) norm_to_lds_impl<XT, true, true>(a, u, nl);
    else norm_to_lds_impl<XT, true, false>(a, u, nl);
  } else {
    if (a.gamma) norm_to_lds_impl<XT, false, true>(a, u, nl);
    else norm_to_lds_impl<XT, false, false>(a, u, nl);
  }
}

// u[0..d) (LDS, values already rounded to the activation dtype) to a.u_out, by the whole block
template <typename XT>
__device__ __forceinline__ void write_u(const LayerArgs& a, const float* u) {
  for (int j = threadIdx.x; j < a.d; j += kThreads) {
    if (sizeof(XT) == 2) reinterpret_cast<uint16_t*>(a.u_out)[j] = (uint16_t)(__float_as_uint(u[j]) >> 16);
    else reinterpret_cast<float*>(a.u_out)[j] = u[j];
  }
}

// ------------------------------------------------------------------------------------------------
// routing inside a block
// ------------------------------------------------------------------------------------------------
struct RouteLds {
  int sel_i[kLayerMaxK];
  float w[kLayerMaxK];
};

// Router wavefront of expert e < E, after publishing logit lgt: wait for all E logits of this call, rank
// lgt among them (larger logit first, equal logits -> lower id) and, if the rank is below k, publish
// (e, lgt) as that entry of every route replica.  With forced ids nothing is ranked.  A wait that runs out
// sets the status word and ranks whatever it read.
template <int PER>
__device__ __forceinline__ void rank_expert(const LayerArgs& a, int e, float lgt) {
  const int lane = threadIdx.x & 63;
  uint32_t key[PER];
  for (int n = 0;; ++n) {
    bool ok = true;
#pragma unroll
    for (int m = 0; m < PER; ++m) {
      key[m] = 0u;
      if (lane + 64 * m < a.E) {
        const uint64_t t = ld_c64(a.lg_tag + (int64_t)(e % kLgReplicas) * a.E + lane + 64 * m);
        ok = ok && (uint32_t)(t >> 32) == a.tag;
        key[m] = order_key(__uint_as_float((uint32_t)t));
      }
    }
    if (__ballot(!ok) == 0ull) break;
    if (n >= kSpinLimit) {
      if (lane == 0) __hip_atomic_fetch_or(a.status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  const uint32_t ke = order_key(lgt);
  int rank = 0;
#pragma unroll
  for (int m = 0; m < PER; ++m) {
    const int idx = lane + 64 * m;
    const bool before = idx < a.E && (key[m] > ke || (key[m] == ke && idx < e));
    rank += __popcll(__ballot(before));
  }
  if (rank < a.k && lane < kRouteReplicas) {
    uint64_t* rep_base = a.route + (int64_t)lane * 2 * kLayerMaxK;
    const uint64_t tg = (uint64_t)a.tag << 32;
    st_c64(rep_base + rank, tg | (uint32_t)e);
    st_c64(rep_base + kLayerMaxK + rank, tg | __float_as_uint(lgt));
  }
}

// sel_i[0..k) = the selected expert ids and, with weights, w[0..k) their gate weights (softmax over the k
// kept logits: one exp per kept logit, maximum and denominator taken in the order 0..k-1), in LDS for the
// whole block; wavefront 0 polls route replica blockIdx mod kRouteReplicas (with forced ids: the forced
// experts' logits).  With forced ids and no weights there is nothing to wait for.
__device__ __forceinline__ void get_route(const LayerArgs& a, RouteLds& r, bool weights) {
  if (a.forced && !weights) {
    if ((int)threadIdx.x < a.k) r.sel_i[threadIdx.x] = a.forced[threadIdx.x];
    __syncthreads();
    return;
  }
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const uint64_t* src = a.route + (int64_t)(blockIdx.x % kRouteReplicas) * 2 * kLayerMaxK;
    int id = -1;
    float v = __builtin_nanf("");
    const int fid = a.forced && lane < a.k ? a.forced[lane] : -1;
    const bool fvalid = fid >= 0 && fid < a.E;
    for (int n = 0;; ++n) {
      bool ok = true;
      if (lane < a.k) {
        if (a.forced) {
          id = fid;
          if (fvalid) {
            const uint64_t t = ld_c64(a.lg_tag + (int64_t)(blockIdx.x % kLgReplicas) * a.E + fid);
            ok = (uint32_t)(t >> 32) == a.tag;
            v = __uint_as_float((uint32_t)t);
          }
        } else {
          const uint64_t ti = ld_c64(src + lane), tv = ld_c64(src + kLayerMaxK + lane);
          ok = (uint32_t)(ti >> 32) == a.tag && (uint32_t)(tv >> 32) == a.tag;
          id = (int)(uint32_t)ti;
          v = __uint_as_float((uint32_t)tv);
        }
      }
      if (__ballot(!ok) == 0ull) break;
      if (n >= kSpinLimit) {
        if (lane == 0) __hip_atomic_fetch_or(a.status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    float w = 0.f;
    if (weights) {
      auto lane_f = [](float x, int i) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), i)); };
      float mx = lane_f(v, 0);
      for (int i = 1; i < a.k; ++i) mx = fmaxf(mx, lane_f(v, i));
      const float ex = lane < a.k ? expf(v - mx) : 0.f;
      float den = 0.f;
      for (int i = 0; i < a.k; ++i) den += lane_f(ex, i);
      w = ex / den;
    }
    if (lane < a.k) {
      r.sel_i[lane] = id;
      r.w[lane] = w;
    }
  }
  __syncthreads();
}

// ------------------------------------------------------------------------------------------------
// roles
// ------------------------------------------------------------------------------------------------
// Four experts per block, one per wavefront.  Lane l takes the 8-element pieces l, l + 64, ... of the row
// (8 int8 weights: one 8-byte load each, issued before the norm), so the reads of u are conflict-free.
template <typename XT>
__device__ __forceinline__ void router_block(const LayerArgs& a, int b, float* u, NormLds& nl) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int e = b * 4 + wave;
  const int np = a.d / 8;
  constexpr int kM = kLayerMaxD / 8 / 64;
  uint2 q[kM];
#pragma unroll
  for (int m = 0; m < kM; ++m) {
    const int p = lane + 64 * m;
    if (e < a.E && p < np) q[m] = *reinterpret_cast<const uint2*>(a.rw + (int64_t)e * a.d + p * 8);
  }
  // the row scale with the weights, not at its use after the dot product (the barriers of the norm keep
  // the compiler from moving it up there, and the logit would wait a memory round trip for it); the
  // expert is uniform over the wavefront, so it is a scalar load into a scalar register
  const float rse = a.rs[__builtin_amdgcn_readfirstlane(e < a.E ? e : a.E - 1)];
  if (a.prev_x.base) wait_set(a.prev_x, blockIdx.x, a.tag, a.status);
  norm_to_lds<XT>(a, u, nl);
  if (b == 0 && a.u_out && !a.has_shared) write_u<XT>(a, u);
  if (e < a.E) {
    float acc = 0.f;
    // three pieces at a time: their LDS reads are issued together
#pragma unroll
    for (int m0 = 0; m0 < kM; m0 += 3) {
      if (m0 * 64 >= np) break;
      float4 ub[3][2];
#pragma unroll
      for (int mm = 0; mm < 3; ++mm) {
        const int p = lane + 64 * (m0 + mm);
        const int pc = (m0 + mm < kM && p < np) ? p : 0;
        ub[mm][0] = reinterpret_cast<const float4*>(u + pc * 8)[0];
        ub[mm][1] = reinterpret_cast<const float4*>(u + pc * 8)[1];
      }
#pragma unroll
      for (int mm = 0; mm < 3; ++mm) {
        const int p = lane + 64 * (m0 + mm);
        if (m0 + mm >= kM || p >= np) continue;
        const float us[8] = {ub[mm][0].x, ub[mm][0].y, ub[mm][0].z, ub[mm][0].w,
                             ub[mm][1].x, ub[mm][1].y, ub[mm][1].z, ub[mm][1].w};
        const uint32_t w[2] = {q[m0 + mm].x, q[m0 + mm].y};
#pragma unroll
        for (int i = 0; i < 8; ++i) acc = fmaf((float)(int8_t)((w[i >> 2] >> (8 * (i & 3))) & 0xff), us[i], acc);
      }
    }
    acc = wave_sum(acc);
    const float lgt = acc * rse;
    if (lane < kLgReplicas) st_c64(a.lg_tag + (int64_t)lane * a.E + e, ((uint64_t)a.tag << 32) | __float_as_uint(lgt));
    if (lane == 0 && a.logits_out) a.logits_out[e] = lgt;
    if (!a.forced) {
      if (a.E <= 64) rank_expert<1>(a, e, lgt);
      else if (a.E <= 128) rank_expert<2>(a, e, lgt);
      else if (a.E <= 192) rank_expert<3>(a, e, lgt);
      else rank_expert<4>(a, e, lgt);
    }
  }
}

// 8 features (gate rows f, up rows F + f) of one expert; the four waves split the row.  Split in a load
// phase (this lane's code words and scale/bias) and a finish phase (stage u, dot products, publish h).
template <int NBW, bool SB_BF16>
struct GuRegs {
  SbWord<SB_BF16> sa[NBW], sb[NBW];
  u32x4 qa[NBW], qb[NBW];
};

template <int NBW, bool SB_BF16>
__device__ __forceinline__ void gu_load(const LayerArgs& a, const LayerPool& P, int rec_idx, bool valid, int tile,
                                        GuRegs<NBW, SB_BF16>& g) {
  const int K = a.d, lane = threadIdx.x & 63, wave = threadIdx.x >> 6, ra = lane >> 3, j = lane & 7;
  const int C = K / 32;
  const int f = tile * 8 + ra;
  const char* rec = P.base + (int64_t)(valid ? rec_idx : 0) * P.record_bytes;
  const int64_t rowb = K / 2, sbrow = (int64_t)(K / 64) * (SB_BF16 ? 4 : 8);
  const char* rowA = rec + P.gu_q + f * rowb;
  const char* rowB = rec + P.gu_q + (P.F + f) * rowb;
  const char* sbA = rec + P.gu_sb + f * sbrow;
  const char* sbB = rec + P.gu_sb + (P.F + f) * sbrow;
  if (!valid) return;
#pragma unroll
  for (int m = 0; m < NBW; ++m) {
    const int c = (wave + 4 * m) * kLanesPerRow + j;
    if (c < C) {
      g.sa[m] = load_sb<SB_BF16>(sbA, c >> 1);
      g.sb[m] = load_sb<SB_BF16>(sbB, c >> 1);
    }
  }
#pragma unroll
  for (int m = 0; m < NBW; ++m) {
    const int c = (wave + 4 * m) * kLanesPerRow + j;
    if (c < C) {
      g.qa[m] = load_nt(rowA + c * 16);
      g.qb[m] = load_nt(rowB + c * 16);
    }
  }
}

template <int NBW, bool SB_BF16>
__device__ __forceinline__ void gu_finish(const LayerArgs& a, const GuRegs<NBW, SB_BF16>& g, bool valid, int tile,
                                          float* hout, const SyncSet& done, int done_total, const float* u, Stage st) {
  const int K = a.d, lane = threadIdx.x & 63, wave = threadIdx.x >> 6, ra = lane >> 3, j = lane & 7;
  const int C = K / 32, nit = (C + kLanesPerRow - 1) / kLanesPerRow;
  const int f = tile * 8 + ra;
  // stage this wave's half-groups of u (the single-token kernel's slot mapping)
  constexpr int kPasses = (NBW * 32 + 63) / 64;
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    const int s = lane + 64 * p, m = s >> 5, jj = (s >> 2) & 7, qd = s & 3;
    const int it = wave + 4 * m;
    const int hg = it * kLanesPerRow + jj;
    const bool live = m < NBW && it < nit && hg < C;
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = live ? u[hg * 32 + qd * 8 + i] : 0.f;
    stage_word(v, live, hg, qd, st);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  float yA = 0.f, yB = 0.f;
  if (valid) {
    const Dequant dq = make_dequant();
#pragma unroll
    for (int m = 0; m < NBW; ++m) {
      const int c = (wave + 4 * m) * kLanesPerRow + j;
      if (c < C) {
        const u32x4* xv = reinterpret_cast<const u32x4*>(st.xw + c * kHgStride);
        const u32x4 x0 = xv[0], x1 = xv[1], x2 = xv[2], x3 = xv[3];
        const float4 h = st.hg[c];
        const float accA = chunk_dot(g.qa[m], x0, x1, x2, x3, dq, -h.y);
        const float accB = chunk_dot(g.qb[m], x0, x1, x2, x3, dq, -h.y);
        float s0, b0, s1, b1;
        sb_values<SB_BF16>(g.sa[m], s0, b0);
        sb_values<SB_BF16>(g.sb[m], s1, b1);
        yA = fmaf(h.x, fmaf(s0, accA, b0 * h.z), yA);
        yB = fmaf(h.x, fmaf(s1, accB, b1 * h.z), yB);
      }
    }
  }
  if (block_sum(yA, yB)) st_c(hout + f, valid ? activation(yA, a.act) * yB : __builtin_nanf(""));
  publish(done, tile, done_total, a.tag);
}

// Stage all half-groups of a published vector v[0..K) (coherent loads) into `st`, block-cooperatively.
__device__ __forceinline__ void stage_published(const float* v, int K, Stage st) {
  const int nhg = K / 32;
  for (int s = threadIdx.x; s < nhg * 4; s += kThreads) {
    const int hg = s >> 2, qd = s & 3;
    float w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = ld_c(v + hg * 32 + qd * 8 + i);
    stage_word(w, true, hg, qd, st);
  }
}

// The combine of rows [64 rb, 64 rb + 64), done by the block of the last routed slot for those rows once
// its own rows are in comb[k - 1][*]: it polls the other contributions (routed slots 0..k-2 and the shared
// expert, published tagged; all of one thread's loads in flight together) into comb, then thread t < 64
// stores out[64 rb + t] = round_x(sum_i w_i y_i (i = 0..k-1) + y_shared + residual), in moe_combine's
// order.  comb: LDS [k + 1][64] floats (index k: the shared expert).  Within a launch of several layers
// each combine but the last layer's counts on the layer's done set.
template <typename XT>
__device__ __forceinline__ void combine_rows(const LayerArgs& a, const RouteLds& r, int rb, float* comb) {
  constexpr int kPer = (kLayerMaxK + 1 + kThreads / 64 - 1) / (kThreads / 64);   // sources per thread, max
  const int t = threadIdx.x, rl = t & 63, row = rb * 64 + rl;
  const int nsrc = a.k - 1 + (a.has_shared ? 1 : 0);   // source s: routed slot s < k - 1, else shared
  float xr = 0.f;
  if (a.residual && t < 64) {
    const XT* x = reinterpret_cast<const XT*>(a.x);
    if (!a.x_ws)
      xr = sizeof(XT) == 2 ? bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(x)[row])
                           : reinterpret_cast<const float*>(x)[row];
    else if (sizeof(XT) == 2)   // the bf16 pair holding the row, read coherently
      xr = __uint_as_float((row & 1) ? ld_cu(reinterpret_cast<const uint32_t*>(x) + (row >> 1)) & 0xffff0000u
                                     : ld_cu(reinterpret_cast<const uint32_t*>(x) + (row >> 1)) << 16);
    else
      xr = ld_c(reinterpret_cast<const float*>(x) + row);
  }
  for (int n = 0;; ++n) {
    uint64_t v[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int sidx = (t >> 6) + i * (kThreads / 64);
      if (sidx < nsrc) v[i] = ld_c64((sidx < a.k - 1 ? a.y_routed + (int64_t)sidx * a.d : a.y_shared) + row);
    }
    bool ok = true;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int sidx = (t >> 6) + i * (kThreads / 64);
      if (sidx < nsrc) {
        ok = ok && (uint32_t)(v[i] >> 32) == a.tag;
        comb[(sidx < a.k - 1 ? sidx : a.k) * 64 + rl] = __uint_as_float((uint32_t)v[i]);
      }
    }
    if (!__syncthreads_or(!ok)) break;
    if (n >= kSpinLimit) {
      if (t == 0) __hip_atomic_fetch_or(a.status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  if (t < 64) {
    float acc = 0.f;
    for (int i = 0; i < a.k; ++i) acc = __builtin_fmaf(r.w[i], comb[i * 64 + rl], acc);
    if (a.has_shared) acc += comb[a.k * 64 + rl];
    if (a.residual) acc += xr;
    if (sizeof(XT) == 2) {   // the layer output's rounding
      const uint16_t o = (uint16_t)f32_to_bf16_bits(acc);
      if (a.out_ws) __hip_atomic_store(reinterpret_cast<uint16_t*>(a.out) + row, o, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      else reinterpret_cast<uint16_t*>(a.out)[row] = o;
    } else {
      if (a.out_ws) st_c(reinterpret_cast<float*>(a.out) + row, acc);
      else reinterpret_cast<float*>(a.out)[row] = acc;
    }
  }
  if (!a.last_layer) {
    // the next layer reads these rows once the count is complete: they are stored before the arrival
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (t < 64) arrive(a.done, 0, a.d / 64, a.tag);
  }
}

// 16 rows (r, r + 8 per lane group) of the shared expert's down matrix, waves split the row (K = S)
template <int NBW, typename XT, bool SB_BF16>
__device__ __forceinline__ void shared_down_block(const LayerArgs& a, int tile, Stage st) {
  const LayerPool& P = a.shared;
  const int K = P.F, lane = threadIdx.x & 63, wave = threadIdx.x >> 6, ra = lane >> 3, j = lane & 7;
  const int C = K / 32;
  const int row = tile * 16 + ra;
  const char* rec = P.base;
  const int64_t rowb = K / 2, sbrow = (int64_t)(K / 64) * (SB_BF16 ? 4 : 8);
  SbWord<SB_BF16> sa[NBW], sb[NBW];
  u32x4 qa[NBW], qb[NBW];
#pragma unroll
  for (int m = 0; m < NBW; ++m) {
    const int c = (wave + 4 * m) * kLanesPerRow + j;
    if (c < C) {
      sa[m] = load_sb<SB_BF16>(rec + P.dn_sb + row * sbrow, c >> 1);
      sb[m] = load_sb<SB_BF16>(rec + P.dn_sb + (row + 8) * sbrow, c >> 1);
    }
  }
#pragma unroll
  for (int m = 0; m < NBW; ++m) {
    const int c = (wave + 4 * m) * kLanesPerRow + j;
    if (c < C) {
      qa[m] = load_nt(rec + P.dn_q + row * rowb + c * 16);
      qb[m] = load_nt(rec + P.dn_q + (row + 8) * rowb + c * 16);
    }
  }
  wait_set(a.shared_h, blockIdx.x, a.tag, a.status);
  stage_published(a.h_shared, K, st);
  __syncthreads();
  float yA = 0.f, yB = 0.f;
  const Dequant dq = make_dequant();
#pragma unroll
  for (int m = 0; m < NBW; ++m) {
    const int c = (wave + 4 * m) * kLanesPerRow + j;
    if (c < C) {
      const u32x4* xv = reinterpret_cast<const u32x4*>(st.xw + c * kHgStride);
      const u32x4 x0 = xv[0], x1 = xv[1], x2 = xv[2], x3 = xv[3];
      const float4 h = st.hg[c];
      const float accA = chunk_dot(qa[m], x0, x1, x2, x3, dq, -h.y);
      const float accB = chunk_dot(qb[m], x0, x1, x2, x3, dq, -h.y);
      float s0, b0, s1, b1;
      sb_values<SB_BF16>(sa[m], s0, b0);
      sb_values<SB_BF16>(sb[m], s1, b1);
      yA = fmaf(h.x, fmaf(s0, accA, b0 * h.z), yA);
      yB = fmaf(h.x, fmaf(s1, accB, b1 * h.z), yB);
    }
  }
  if (block_sum(yA, yB)) {
    const uint64_t tg = (uint64_t)a.tag << 32;
    st_c64(a.y_shared + row, tg | __float_as_uint(yA));
    st_c64(a.y_shared + row + 8, tg | __float_as_uint(yB));
  }
}

// 64 rows of the i-th selected expert's down matrix: wave w takes rows 16w.. of the block, whole rows
template <int NBW, typename XT, bool SB_BF16>
__device__ __forceinline__ void routed_down_block(const LayerArgs& a, int slot, int rb, Stage st, RouteLds& r,
                                                  float* comb) {
  const LayerPool& P = a.routed;
  const int K = P.F, lane = threadIdx.x & 63, wave = threadIdx.x >> 6, ra = lane >> 3, j = lane & 7;
  const int C = K / 32;
  const int row = rb * 64 + wave * 16 + ra;
  const bool combiner = slot == a.k - 1;   // the last slot's block combines its 64 rows
  get_route(a, r, combiner || (slot == 0 && rb == 0 && a.weights_out));
  if (slot == 0 && rb == 0 && (int)threadIdx.x < a.k) {
    if (a.ids_out) a.ids_out[threadIdx.x] = r.sel_i[threadIdx.x];
    if (a.weights_out) a.weights_out[threadIdx.x] = r.w[threadIdx.x];
  }
  const int e = r.sel_i[slot];
  const int idx = a.gemv_ids ? a.gemv_ids[slot] : e;
  const bool valid = (unsigned)idx < (unsigned)P.n_records && (unsigned)e < (unsigned)a.E;
  const char* rec = P.base + (int64_t)(valid ? idx : 0) * P.record_bytes;
  const int64_t rowb = K / 2, sbrow = (int64_t)(K / 64) * (SB_BF16 ? 4 : 8);
  SbWord<SB_BF16> sa[NBW], sb[NBW];
  u32x4 qa[NBW], qb[NBW];
  if (valid) {
#pragma unroll
    for (int m = 0; m < NBW; ++m) {
      const int c = m * kLanesPerRow + j;
      if (c < C) {
        sa[m] = load_sb<SB_BF16>(rec + P.dn_sb + row * sbrow, c >> 1);
        sb[m] = load_sb<SB_BF16>(rec + P.dn_sb + (row + 8) * sbrow, c >> 1);
      }
    }
#pragma unroll
    for (int m = 0; m < NBW; ++m) {
      const int c = m * kLanesPerRow + j;
      if (c < C) {
        qa[m] = load_nt(rec + P.dn_q + row * rowb + c * 16);
        qb[m] = load_nt(rec + P.dn_q + (row + 8) * rowb + c * 16);
      }
    }
  }
  wait_set(slot_set(a, slot), blockIdx.x, a.tag, a.status);
  stage_published(a.h_routed + (int64_t)slot * K, K, st);
  __syncthreads();
  float yA = 0.f, yB = 0.f;
  if (valid) {
    const Dequant dq = make_dequant();
#pragma unroll
    for (int m = 0; m < NBW; ++m) {
      const int c = m * kLanesPerRow + j;
      if (c < C) {
        const u32x4* xv = reinterpret_cast<const u32x4*>(st.xw + c * kHgStride);
        const u32x4 x0 = xv[0], x1 = xv[1], x2 = xv[2], x3 = xv[3];
        const float4 h = st.hg[c];
        const float accA = chunk_dot(qa[m], x0, x1, x2, x3, dq, -h.y);
        const float accB = chunk_dot(qb[m], x0, x1, x2, x3, dq, -h.y);
        float s0, b0, s1, b1;
        sb_values<SB_BF16>(sa[m], s0, b0);
        sb_values<SB_BF16>(sb[m], s1, b1);
        yA = fmaf(h.x, fmaf(s0, accA, b0 * h.z), yA);
        yB = fmaf(h.x, fmaf(s1, accB, b1 * h.z), yB);
      }
    }
  }
  yA = reduce8(yA);
  yB = reduce8(yB);
  if (!valid) yA = yB = __builtin_nanf("");
  if (!combiner) {
    if (j == 0) {
      const uint64_t tg = (uint64_t)a.tag << 32;
      st_c64(a.y_routed + (int64_t)slot * a.d + row, tg | __float_as_uint(yA));
      st_c64(a.y_routed + (int64_t)slot * a.d + row + 8, tg | __float_as_uint(yB));
    }
    return;
  }
  __syncthreads();   // every wavefront is done with the staging area, which comb may overlay
  if (j == 0) {      // (combine_rows makes these visible to the block before it reads them)
    comb[(a.k - 1) * 64 + wave * 16 + ra] = yA;
    comb[(a.k - 1) * 64 + wave * 16 + ra + 8] = yB;
  }
  combine_rows<XT>(a, r, rb, comb);
}

// ------------------------------------------------------------------------------------------------
// launch: the layers of one launch one after the other in the grid, each laid out as above
// ------------------------------------------------------------------------------------------------
constexpr int kMaxStackLayers = 32;

struct StackLayer {           // what differs between the layers of a launch
  const int8_t* rw;
  const float* rs;
  const float* gamma;
  const char* routed_base;
  const char* shared_base;
  int32_t* ids_out;
  float* weights_out;
  float* logits_out;
  void* u_out;
};

struct WsLayout {
  size_t sync, calls, lg_tag, route, h_routed, h_shared, y_routed, y_shared, x_next, total;
};

struct StackArgs {
  StackLayer layer[kMaxStackLayers];
  LayerArgs base;             // fields common to all layers (per-layer ones are set by each block)
  char* ws;                   // layer l's region at ws + l * w.total
  WsLayout w;
  const void* x_in;
  void* out;
  uint32_t* status;           // the sticky status word (word 0 of the workspace, or the caller's word)
  int32_t n_layers, per_layer_blocks;
  // 0: the whole layer; 1: the router and the shared expert only; 2: the routed experts and the combine only
  // (the roles of part 2 after those of part 1 on the same workspace make one call)
  int32_t part;
};

__device__ __forceinline__ SyncSet layer_set(uint32_t* sync, int line, int n_sub, int n_flags, uint32_t total) {
  return SyncSet{sync + line * kLW, n_sub, n_flags, total};
}

// MULTI: the launch holds several layers.  A single-layer launch is its own instantiation, in which the
// previous-layer wait and the coherent fp32 activations are absent at compile time (no run-time branches
// around the first loads of a block).
template <int NBW, typename XT, bool SB_BF16, bool MULTI>
__global__ __launch_bounds__(kThreads) void decode_stack_kernel(const StackArgs sa) {
  extern __shared__ __align__(16) uint32_t lds[];
  __shared__ NormLds nl;
  __shared__ RouteLds r;
  const int l = MULTI ? (int)blockIdx.x / sa.per_layer_blocks : 0;
  int b = MULTI ? (int)blockIdx.x % sa.per_layer_blocks : (int)blockIdx.x;
  if (!MULTI && sa.part) {
    // a part's grid holds only its roles: map the block to its role index in the whole layer's layout
    // [router | shared gate/up | routed gate/up | shared down | routed down]
    const LayerArgs& c = sa.base;
    if (sa.part == 1) b = b < c.nR + c.nSG ? b : b + c.nRG;
    else b = b < c.nRG ? c.nR + c.nSG + b : c.nR + c.nSG + c.nRG + c.nSD + (b - c.nRG);
  }
  const bool last = !MULTI || l == sa.n_layers - 1;
  // this block's layer
  LayerArgs a = sa.base;
  const StackLayer& L = sa.layer[l];
  a.rw = L.rw;
  a.rs = L.rs;
  a.gamma = L.gamma;
  a.routed.base = L.routed_base;
  a.shared.base = L.shared_base;
  a.ids_out = L.ids_out;
  a.weights_out = L.weights_out;
  a.logits_out = L.logits_out;
  a.u_out = L.u_out;
  char* ws = sa.ws + (int64_t)l * sa.w.total;
  a.x = l == 0 ? sa.x_in : static_cast<const void*>(ws - sa.w.total + sa.w.x_next);
  a.x_ws = l > 0;
  a.out = last ? sa.out : static_cast<void*>(ws + sa.w.x_next);
  a.out_ws = !last;
  a.last_layer = last;
  a.status = sa.status;
  uint32_t* sync = reinterpret_cast<uint32_t*>(ws);
  int line = 1;
  // The call's tag, without a call-wide counter: every block counts the calls in a word of its own (no
  // other block reads or writes it), so all words of a workspace hold the same count.  Every thread reads
  // the word here; the block advances it when it ends.  Tag 0, the value of a zeroed workspace, is skipped
  // when the count wraps.
  uint32_t* const mine = reinterpret_cast<uint32_t*>(ws + sa.w.calls) + b;
  {
    const uint32_t t = ld_cu(mine) + 1u;
    a.tag = t != 0u ? t : 1u;
  }
  a.shared_h = layer_set(sync, line, kSharedSub, kSharedFlags, (uint32_t)a.nSG);
  line += kSharedSub + 1 + kSharedFlags;
  const int done_line = line;
  a.done = layer_set(sync, line, kDoneSub, last ? 0 : kXFlags, (uint32_t)(a.d / 64));
  line += kDoneSub + 1 + kXFlags;
  a.slot_base = sync + line * kLW;
  a.prev_slot_base = l > 0 ? a.slot_base - sa.w.total / 4 : nullptr;
  a.prev_x = l > 0 ? layer_set(sync - sa.w.total / 4, done_line, kDoneSub, kXFlags, (uint32_t)(a.d / 64))
                   : SyncSet{nullptr, 1, 0, 0u};
  a.lg_tag = reinterpret_cast<uint64_t*>(ws + sa.w.lg_tag);
  a.route = reinterpret_cast<uint64_t*>(ws + sa.w.route);
  a.h_routed = reinterpret_cast<float*>(ws + sa.w.h_routed);
  a.h_shared = reinterpret_cast<float*>(ws + sa.w.h_shared);
  a.y_routed = reinterpret_cast<uint64_t*>(ws + sa.w.y_routed);
  a.y_shared = reinterpret_cast<uint64_t*>(ws + sa.w.y_shared);
  float* u = reinterpret_cast<float*>(lds);                        // [d] the normalized activation
  uint32_t* stage_base = lds + a.d;                                 // staging area
  // staging area: [nhg][kHgStride] words then [nhg] float4; sized by the block's own K
  auto stage_for = [&](int K) {
    const int nhg = K / 32;
    return Stage{stage_base, reinterpret_cast<float4*>(stage_base + nhg * kHgStride)};
  };
  // Issue priority between the wavefronts sharing a SIMD: the router above every other role (all of them
  // wait for its routing or compete with it for the memory pipeline at the start); the other roles share
  // one level (measured: with the shared expert at a lower level the combine waited for its rows).
  if (b < a.nR) {
    __builtin_amdgcn_s_setprio(3);
    router_block<XT>(a, b, u, nl);
  } else {
    __builtin_amdgcn_s_setprio(2);
    b -= a.nR;
    const int nG = a.nSG + a.nRG, nD = nG + a.nSD;
    if (b < a.nSG) {
      // The shared expert needs only x.  In a launch of several layers its code words are requested before the
      // wait for the previous layer (they stream while that layer finishes); a single layer issues them after
      // the norm, whose loads go out with the router's (measured: 20.2 -> 18.9 us per layer over 30 layers in
      // one launch; the single launch is faster without, its registers otherwise cost occupancy).  They are
      // requested once the previous layer's routed gate/up blocks are all done (every slot's flag raised):
      // those rows are on that layer's critical path, and a compute unit serves its blocks' loads in order,
      // so code words requested earlier would be served first (measured: 18.85 -> 18.55 us per layer).
      GuRegs<NBW, SB_BF16> g;
      if (MULTI && a.prev_slot_base) {
        if ((int)threadIdx.x < a.k) {
          const uint32_t* f = a.prev_slot_base + (int64_t)threadIdx.x * kLinesPerSlot * kLW +
                              (kSlotSub + 1 + (int)(blockIdx.x % kSlotFlags)) * kLW;
          int n = 0;
          while (ld_cu(f) != a.tag && n < kSpinLimit) {
            __builtin_amdgcn_s_sleep(2);
            ++n;
          }
          if (n >= kSpinLimit) __hip_atomic_fetch_or(a.status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
      }
      if (MULTI) gu_load<NBW, SB_BF16>(a, a.shared, 0, true, b, g);
      if (a.prev_x.base) wait_set(a.prev_x, blockIdx.x, a.tag, a.status);
      norm_to_lds<XT>(a, u, nl);
      if (b == 0 && a.u_out) write_u<XT>(a, u);   // off the routing path: the first shared gate/up block
      if (!MULTI) gu_load<NBW, SB_BF16>(a, a.shared, 0, true, b, g);
      gu_finish<NBW, SB_BF16>(a, g, true, b, a.h_shared, a.shared_h, a.nSG, u, stage_for(a.d));
    } else if (b < nG) {
      const int per = a.routed.F / 8, slot = (b - a.nSG) / per, tile = (b - a.nSG) % per;
      // the norm needs only x: done while the router finishes
      if (a.prev_x.base) wait_set(a.prev_x, blockIdx.x, a.tag, a.status);
      norm_to_lds<XT>(a, u, nl);
      get_route(a, r, false);
      const int e = r.sel_i[slot];
      const int idx = a.gemv_ids ? a.gemv_ids[slot] : e;
      const bool valid = (unsigned)idx < (unsigned)a.routed.n_records && (unsigned)e < (unsigned)a.E;
      GuRegs<NBW, SB_BF16> g;
      gu_load<NBW, SB_BF16>(a, a.routed, idx, valid, tile, g);
      gu_finish<NBW, SB_BF16>(a, g, valid, tile, a.h_routed + (int64_t)slot * a.routed.F, slot_set(a, slot), per,
                              u, stage_for(a.d));
    } else if (b < nD) {
      shared_down_block<NBW, XT, SB_BF16>(a, b - nG, stage_for(a.shared.F));
    } else {
      const int per = a.d / 64, slot = (b - nD) / per, rb = (b - nD) % per;
      // the combine buffer of the last slot's blocks overlays the (then finished) staging area
      routed_down_block<NBW, XT, SB_BF16>(a, slot, rb, stage_for(a.routed.F), r, reinterpret_cast<float*>(lds));
    }
  }
  // count this call: every wavefront that uses the tag has read the word by now (a load still in flight
  // belongs to a wavefront that never uses its value)
  __syncthreads();
  if (threadIdx.x == 0) st_cu(mine, a.tag);
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// blocks of one layer: router, shared gate/up, routed gate/up, shared down, routed down
int layer_blocks(int d, int E, int k, int F, int S) {
  return (E + 3) / 4 + S / 8 + k * (F / 8) + (S > 0 ? d / 16 : 0) + k * (d / 64);
}

WsLayout ws_layout(int d, int E, int k, int F, int S) {
  WsLayout w;
  size_t o = 0;
  w.sync = o;       o += (size_t)(kLinesFixed + k * kLinesPerSlot) * kLW * 4;
  w.calls = o;      o += align256((size_t)layer_blocks(d, E, k, F, S) * 4);
  w.lg_tag = o;     o += align256((size_t)kLgReplicas * E * 8);
  w.route = o;      o += align256((size_t)kRouteReplicas * 2 * kLayerMaxK * 8);
  w.h_routed = o;   o += align256((size_t)k * F * 4);
  w.h_shared = o;   o += align256((size_t)(S > 0 ? S : 1) * 4);
  w.y_routed = o;   o += align256((size_t)k * d * 8);
  w.y_shared = o;   o += align256((size_t)d * 8);
  w.x_next = o;     o += align256((size_t)d * 4);
  w.total = o;
  return w;
}

bool layer_pool(const moe_q4_pool* p, LayerPool* out, const char** why) {
  RecordOffsets o;
  if (!p->base_dev) { *why = "pool base is NULL"; return false; }
  if (!record_offsets(p->d, p->F, p->sb_dtype, &o)) { *why = "pool d/F not positive multiples of 64 or bad sb dtype"; return false; }
  if (p->record_bytes < o.total || p->record_bytes % 256) { *why = "record_bytes too small or not a multiple of 256"; return false; }
  if (!aligned(p->base_dev, 256)) { *why = "pool base not 256-byte aligned"; return false; }
  if (p->n_records < 1) { *why = "pool has no records"; return false; }
  *out = LayerPool{static_cast<const char*>(p->base_dev), (int64_t)p->record_bytes, p->n_records, p->F,
                   (int64_t)o.gate_up_q, (int64_t)o.gate_up_sb, (int64_t)o.down_q, (int64_t)o.down_sb};
  return true;
}

// Checks shared by the one-layer and the stacked entry points; fills the common fields and the launch.
moe_status prepare_launch(const char* who, const void* x_dev, moe_dtype x_dtype, float eps, bool any_gamma,
                          int32_t residual, int32_t E, int32_t k, const moe_q4_pool* routed, const moe_q4_pool* shared,
                          moe_act act, void* out_dev, void* workspace_dev, size_t workspace_bytes, int n_layers,
                          StackArgs* sa, int* nbw, size_t* lds) {
  if (!x_dev || !routed || !out_dev || !workspace_dev) return fail(MOE_ERR_INVALID_ARG, "%s: NULL pointer", who);
  if (x_dtype != MOE_F32 && x_dtype != MOE_BF16) return fail(MOE_ERR_INVALID_ARG, "%s: bad x_dtype", who);
  if (act != MOE_ACT_GELU_TANH && act != MOE_ACT_SILU) return fail(MOE_ERR_INVALID_ARG, "%s: bad act", who);
  if (any_gamma && !(eps >= 0.f)) return fail(MOE_ERR_INVALID_ARG, "%s: eps must be >= 0", who);
  const char* why = nullptr;
  LayerArgs& a = sa->base;
  a = LayerArgs{};
  if (!layer_pool(routed, &a.routed, &why)) return fail(MOE_ERR_INVALID_ARG, "%s: routed %s", who, why);
  const int d = routed->d;
  if (shared) {
    if (!layer_pool(shared, &a.shared, &why)) return fail(MOE_ERR_INVALID_ARG, "%s: shared %s", who, why);
    if (shared->d != d) return fail(MOE_ERR_INVALID_ARG, "%s: routed d=%d != shared d=%d", who, d, shared->d);
    if (shared->sb_dtype != routed->sb_dtype) return fail(MOE_ERR_UNSUPPORTED, "%s: scale/bias dtypes differ", who);
  }
  if (d > kLayerMaxD || routed->F > kLayerMaxF || (shared && shared->F > kLayerMaxD))
    return fail(MOE_ERR_UNSUPPORTED, "%s: d=%d F=%d S=%d (need d, S <= %d, F <= %d)", who, d, routed->F,
                shared ? shared->F : 0, kLayerMaxD, kLayerMaxF);
  if (E < 1 || E > kLayerMaxE || k < 1 || k > kLayerMaxK || k > E)
    return fail(MOE_ERR_UNSUPPORTED, "%s: E=%d k=%d (need 1 <= k <= min(E, %d), E <= %d)", who, E, k, kLayerMaxK,
                kLayerMaxE);
  if (!aligned(x_dev, 16)) return fail(MOE_ERR_INVALID_ARG, "%s: x must be 16-byte aligned", who);
  const WsLayout w = ws_layout(d, E, k, routed->F, shared ? shared->F : 0);
  if (workspace_bytes < w.total * n_layers)
    return fail(MOE_ERR_INVALID_ARG, "%s: workspace %zu bytes < %zu", who, workspace_bytes, w.total * n_layers);
  if (!aligned(workspace_dev, 256)) return fail(MOE_ERR_INVALID_ARG, "%s: workspace not 256-byte aligned", who);
  a.eps = eps;
  a.residual = residual != 0;
  a.E = E;
  a.k = k;
  a.d = d;
  a.act = act;
  a.has_shared = shared != nullptr;
  a.nR = (E + 3) / 4;
  a.nSG = shared ? shared->F / 8 : 0;
  a.nRG = k * (routed->F / 8);
  a.nSD = shared ? d / 16 : 0;
  a.nRD = k * (d / 64);
  sa->ws = static_cast<char*>(workspace_dev);
  sa->status = static_cast<uint32_t*>(workspace_dev);
  sa->w = w;
  sa->x_in = x_dev;
  sa->out = out_dev;
  sa->n_layers = n_layers;
  sa->per_layer_blocks = a.nR + a.nSG + a.nRG + a.nSD + a.nRD;
  if (sa->per_layer_blocks != layer_blocks(d, E, k, routed->F, shared ? shared->F : 0))
    return fail(MOE_ERR_INVALID_ARG, "%s: inconsistent block count", who);   // (the call words are per block)
  // chunk iterations per lane: gate/up rows (K = d) and shared down rows (K = S) split over 4 waves,
  // routed down rows (K = F) whole per wave
  const int it_gu = (iterations(d) + 3) / 4, it_sd = shared ? (iterations(shared->F) + 3) / 4 : 1;
  const int it_rd = iterations(routed->F);
  int n = it_gu > it_sd ? it_gu : it_sd;
  n = n > it_rd ? n : it_rd;
  if (n > 4) return fail(MOE_ERR_UNSUPPORTED, "%s: rows too long for the single-launch layer", who);
  *nbw = n;
  int kmax = d > routed->F ? d : routed->F;
  if (shared && shared->F > kmax) kmax = shared->F;
  *lds = (size_t)d * 4 + (size_t)(kmax / 32) * (kHgStride * 4 + 16);
  if (*lds < (size_t)(k + 1) * 64 * 4) *lds = (size_t)(k + 1) * 64 * 4;   // the combine buffer
  return MOE_OK;
}

moe_status launch(const StackArgs& sa, moe_dtype x_dtype, bool sb16, int nbw, size_t lds, hipStream_t s,
                  const char* who) {
  const LayerArgs& c = sa.base;
  const dim3 grid(sa.part == 1 ? c.nR + c.nSG + c.nSD : sa.part == 2 ? c.nRG + c.nRD : sa.per_layer_blocks * sa.n_layers);
  if (grid.x == 0) return MOE_OK;
  return dispatch_nbw(nbw, [&](auto nb) {
    constexpr int N = decltype(nb)::value;
    if constexpr (N <= 4) {
      auto go = [&](auto multi) {
        constexpr bool M = decltype(multi)::value;
        if (x_dtype == MOE_BF16) {
          if (sb16) hipLaunchKernelGGL((decode_stack_kernel<N, uint16_t, true, M>), grid, dim3(kThreads), lds, s, sa);
          else hipLaunchKernelGGL((decode_stack_kernel<N, uint16_t, false, M>), grid, dim3(kThreads), lds, s, sa);
        } else {
          if (sb16) hipLaunchKernelGGL((decode_stack_kernel<N, float, true, M>), grid, dim3(kThreads), lds, s, sa);
          else hipLaunchKernelGGL((decode_stack_kernel<N, float, false, M>), grid, dim3(kThreads), lds, s, sa);
        }
      };
      if (sa.n_layers > 1) go(std::true_type());
      else go(std::false_type());
      return check_launch(who);
    } else {
      return fail(MOE_ERR_UNSUPPORTED, "%s: rows too long", who);
    }
  });
}

}  // namespace
}  // namespace moeq4

using namespace moeq4;

extern "C" size_t moe_decode_layer_sync_bytes(int32_t d, int32_t k) {
  if (d < 64 || k < 1 || k > kLayerMaxK) return 0;
  return ws_layout(d, 1, k, 64, 0).calls;   // the sync lines
}

extern "C" size_t moe_decode_layer_workspace_bytes(int32_t d, int32_t E, int32_t k, int32_t F, int32_t S) {
  if (d < 64 || E < 1 || k < 1 || F < 64) return 0;
  return ws_layout(d, E, k, F, S).total;
}

extern "C" size_t moe_decode_stack_workspace_bytes(int32_t n_layers, int32_t d, int32_t E, int32_t k, int32_t F,
                                                   int32_t S) {
  if (n_layers < 1 || n_layers > kMaxStackLayers) return 0;
  return moe_decode_layer_workspace_bytes(d, E, k, F, S) * (size_t)n_layers;
}

extern "C" moe_status moe_decode_layer(const void* x_dev, moe_dtype x_dtype, const float* gamma_dev, float eps,
                                       int32_t residual, const int8_t* router_w_dev, const float* router_scale_dev,
                                       int32_t E, int32_t k, const int32_t* forced_ids_dev, const moe_q4_pool* routed,
                                       const int32_t* gemv_ids_dev, const moe_q4_pool* shared, moe_act act,
                                       int32_t* ids_dev, float* weights_dev, float* logits_dev, void* u_dev,
                                       void* out_dev, void* workspace_dev, size_t workspace_bytes, void* stream) {
  const char* who = "moe_decode_layer";
  if (!router_w_dev || !router_scale_dev) return fail(MOE_ERR_INVALID_ARG, "%s: NULL pointer", who);
  if (!aligned(router_w_dev, 16) || (gamma_dev && !aligned(gamma_dev, 16)))
    return fail(MOE_ERR_INVALID_ARG, "%s: router weights and gamma must be 16-byte aligned", who);
  if (u_dev && (u_dev == x_dev || u_dev == out_dev)) return fail(MOE_ERR_INVALID_ARG, "%s: u must not alias x or out", who);
  StackArgs sa{};
  int nbw = 0;
  size_t lds = 0;
  moe_status st = prepare_launch(who, x_dev, x_dtype, eps, gamma_dev != nullptr, residual, E, k, routed, shared, act,
                                 out_dev, workspace_dev, workspace_bytes, 1, &sa, &nbw, &lds);
  if (st != MOE_OK) return st;
  sa.base.forced = forced_ids_dev;
  sa.base.gemv_ids = gemv_ids_dev;
  sa.layer[0] = StackLayer{router_w_dev, router_scale_dev, gamma_dev, static_cast<const char*>(routed->base_dev),
                           shared ? static_cast<const char*>(shared->base_dev) : nullptr, ids_dev, weights_dev,
                           logits_dev, u_dev};
  return launch(sa, x_dtype, routed->sb_dtype == MOE_BF16, nbw, lds, as_stream(stream), who);
}

extern "C" moe_status moe_decode_layer_part(int32_t part, const void* x_dev, moe_dtype x_dtype, const float* gamma_dev,
                                            float eps, int32_t residual, const int8_t* router_w_dev,
                                            const float* router_scale_dev, int32_t E, int32_t k,
                                            const int32_t* forced_ids_dev, const moe_q4_pool* routed,
                                            const int32_t* gemv_ids_dev, const moe_q4_pool* shared, moe_act act,
                                            int32_t* ids_dev, float* weights_dev, float* logits_dev, void* u_dev,
                                            void* out_dev, void* workspace_dev, size_t workspace_bytes, void* stream) {
  const char* who = "moe_decode_layer_part";
  if (part != 1 && part != 2) return fail(MOE_ERR_INVALID_ARG, "%s: part %d (1 or 2)", who, part);
  if (!router_w_dev || !router_scale_dev) return fail(MOE_ERR_INVALID_ARG, "%s: NULL pointer", who);
  if (!shared) return fail(MOE_ERR_INVALID_ARG, "%s: the parts split off the shared expert, which is NULL", who);
  if (!aligned(router_w_dev, 16) || (gamma_dev && !aligned(gamma_dev, 16)))
    return fail(MOE_ERR_INVALID_ARG, "%s: router weights and gamma must be 16-byte aligned", who);
  if (u_dev && (u_dev == x_dev || u_dev == out_dev)) return fail(MOE_ERR_INVALID_ARG, "%s: u must not alias x or out", who);
  StackArgs sa{};
  int nbw = 0;
  size_t lds = 0;
  moe_status st = prepare_launch(who, x_dev, x_dtype, eps, gamma_dev != nullptr, residual, E, k, routed, shared, act,
                                 out_dev, workspace_dev, workspace_bytes, 1, &sa, &nbw, &lds);
  if (st != MOE_OK) return st;
  sa.part = part;
  sa.base.forced = forced_ids_dev;
  sa.base.gemv_ids = gemv_ids_dev;
  sa.layer[0] = StackLayer{router_w_dev, router_scale_dev, gamma_dev, static_cast<const char*>(routed->base_dev),
                           static_cast<const char*>(shared->base_dev), ids_dev, weights_dev, logits_dev, u_dev};
  return launch(sa, x_dtype, routed->sb_dtype == MOE_BF16, nbw, lds, as_stream(stream), who);
}

extern "C" moe_status moe_decode_stack(const moe_stack_layer* layers_host, int32_t n_layers, const void* x_dev,
                                       moe_dtype x_dtype, float eps, int32_t residual, int32_t E, int32_t k,
                                       const moe_q4_pool* routed, const moe_q4_pool* shared, moe_act act,
                                       void* out_dev, void* workspace_dev, size_t workspace_bytes, void* stream) {
  const char* who = "moe_decode_stack";
  if (!layers_host) return fail(MOE_ERR_INVALID_ARG, "%s: layers is NULL", who);
  if (n_layers < 1 || n_layers > kMaxStackLayers)
    return fail(MOE_ERR_UNSUPPORTED, "%s: n_layers=%d (1..%d)", who, n_layers, kMaxStackLayers);
  if (x_dev == out_dev) return fail(MOE_ERR_INVALID_ARG, "%s: out must not alias x", who);
  bool any_gamma = false;
  for (int l = 0; l < n_layers; ++l) {
    const moe_stack_layer& L = layers_host[l];
    if (!L.router_w_dev || !L.router_scale_dev || !L.routed_base_dev || (shared && !L.shared_base_dev))
      return fail(MOE_ERR_INVALID_ARG, "%s: layer %d: NULL pointer", who, l);
    if (!aligned(L.router_w_dev, 16) || (L.gamma_dev && !aligned(L.gamma_dev, 16)) || !aligned(L.routed_base_dev, 256) ||
        (shared && !aligned(L.shared_base_dev, 256)))
      return fail(MOE_ERR_INVALID_ARG, "%s: layer %d: misaligned pointer", who, l);
    any_gamma |= L.gamma_dev != nullptr;
  }
  StackArgs sa{};
  int nbw = 0;
  size_t lds = 0;
  moe_status st = prepare_launch(who, x_dev, x_dtype, eps, any_gamma, residual, E, k, routed, shared, act, out_dev,
                                 workspace_dev, workspace_bytes, n_layers, &sa, &nbw, &lds);
  if (st != MOE_OK) return st;
  for (int l = 0; l < n_layers; ++l) {
    const moe_stack_layer& L = layers_host[l];
    sa.layer[l] = StackLayer{L.router_w_dev, L.router_scale_dev, L.gamma_dev, static_cast<const char*>(L.routed_base_dev),
                             static_cast<const char*>(L.shared_base_dev), L.ids_dev, L.weights_dev, L.logits_dev,
                             L.u_dev};
  }
  return launch(sa, x_dtype, routed->sb_dtype == MOE_BF16, nbw, lds, as_stream(stream), who);
}

// ------------------------------------------------------------------------------------------------
// moe_decode_layer_noalloc: moe_decode_layer with the workspace in a device array the library holds
// ------------------------------------------------------------------------------------------------
namespace moeq4 {
namespace {

constexpr size_t kScratchBytes = MOE_DECODE_LAYER_NOALLOC_MAX_BYTES;   // one layer's workspace
constexpr int kMaxDevices = 64;

// The workspace of moe_decode_layer_noalloc, one copy per GPU for the life of the process.  Host code never
// uses this name as an address (on the host it is a stand-in, not device memory): the address of each
// GPU's copy comes from hipGetSymbolAddress, once per device, and only that address reaches kernels.
static __device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

__global__ void zero_kernel(uint4* __restrict__ p, size_t n16) {
  const uint4 z = make_uint4(0u, 0u, 0u, 0u);
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x) p[i] = z;
}

// The current device's copy of `scratch`, looked up on the first call on that device.
moe_status scratch_for_current_device(void** out, const char* who) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "%s: hipGetDevice: %s", who, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(MOE_ERR_UNSUPPORTED, "%s: device %d (at most %d devices)", who, dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(MOE_ERR_HIP, "%s: hipGetSymbolAddress(scratch): %s", who, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace
}  // namespace moeq4

extern "C" moe_status moe_decode_layer_noalloc(const void* x_dev, moe_dtype x_dtype, const float* gamma_dev, float eps,
                                               int32_t residual, const int8_t* router_w_dev,
                                               const float* router_scale_dev, int32_t E, int32_t k,
                                               const int32_t* forced_ids_dev, const moe_q4_pool* routed,
                                               const int32_t* gemv_ids_dev, const moe_q4_pool* shared, moe_act act,
                                               int32_t* ids_dev, float* weights_dev, float* logits_dev, void* u_dev,
                                               void* out_dev, uint32_t* status_dev, void* stream) {
  const char* who = "moe_decode_layer_noalloc";
  if (!routed) return fail(MOE_ERR_INVALID_ARG, "%s: routed is NULL", who);
  const size_t need = moe_decode_layer_workspace_bytes(routed->d, E, k, routed->F, shared ? shared->F : 0);
  if (need == 0) return fail(MOE_ERR_INVALID_ARG, "%s: bad shape (d=%d E=%d k=%d F=%d)", who, routed->d, E, k, routed->F);
  if (need > kScratchBytes)
    return fail(MOE_ERR_UNSUPPORTED, "%s: this shape needs %zu bytes of workspace, more than the %zu bytes the library "
                "holds per device (use moe_decode_layer with a caller workspace)", who, need, kScratchBytes);
  if (!router_w_dev || !router_scale_dev) return fail(MOE_ERR_INVALID_ARG, "%s: NULL pointer", who);
  if (!aligned(router_w_dev, 16) || (gamma_dev && !aligned(gamma_dev, 16)))
    return fail(MOE_ERR_INVALID_ARG, "%s: router weights and gamma must be 16-byte aligned", who);
  if (u_dev && (u_dev == x_dev || u_dev == out_dev)) return fail(MOE_ERR_INVALID_ARG, "%s: u must not alias x or out", who);
  if (status_dev && !aligned(status_dev, 4)) return fail(MOE_ERR_INVALID_ARG, "%s: status not 4-byte aligned", who);
  void* ws = nullptr;
  moe_status st = scratch_for_current_device(&ws, who);
  if (st != MOE_OK) return st;
  StackArgs sa{};
  int nbw = 0;
  size_t lds = 0;
  st = prepare_launch(who, x_dev, x_dtype, eps, gamma_dev != nullptr, residual, E, k, routed, shared, act, out_dev, ws,
                      kScratchBytes, 1, &sa, &nbw, &lds);
  if (st != MOE_OK) return st;
  sa.base.forced = forced_ids_dev;
  sa.base.gemv_ids = gemv_ids_dev;
  sa.layer[0] = StackLayer{router_w_dev, router_scale_dev, gamma_dev, static_cast<const char*>(routed->base_dev),
                           shared ? static_cast<const char*>(shared->base_dev) : nullptr, ids_dev, weights_dev,
                           logits_dev, u_dev};
  if (status_dev) sa.status = status_dev;
  // The previous call on this device may have used another shape: start from a zeroed workspace (counters
  // and call words zero, no stale tagged value), with a fill kernel on the call's stream.
  hipStream_t s = as_stream(stream);
  const size_t n16 = (need + 15) / 16;
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)((n16 + 255) / 256 < 1024 ? (n16 + 255) / 256 : 1024)), dim3(256), 0, s,
                     static_cast<uint4*>(ws), n16);
  st = check_launch(who);
  if (st != MOE_OK) return st;
  return launch(sa, x_dtype, routed->sb_dtype == MOE_BF16, nbw, lds, s, who);
}
