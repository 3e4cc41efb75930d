// moe_decode_layer: one MoE layer of batch-1 decode in a single launch.
//
// The whole step ([G26] "Le pipeline de traitement": route with the 8-bit router, run the selected
// experts and the shared expert, combine; [G26] "Concurrence pour masquer la latence": the shared expert
// does not wait for the routing) as one grid whose blocks play five roles, laid out in dependency order:
//
//   [router | shared gate/up | routed gate/up | shared down | routed down]
//
//   router            one expert per wavefront: RMSNorm of x, int8 dot product, logit published
//   shared gate/up    8 features of the shared expert (needs only x: starts at once)
//   routed gate/up    8 features of the i-th selected expert: reads the published logits when all router
//                     blocks are done and ranks them itself (or takes the forced ids: no wait at all)
//   shared down       16 rows of the shared expert, once all of its gate/up blocks are done
//   routed down       64 rows of the i-th selected expert, once that expert's gate/up blocks are done;
//                     its code words are loaded before the wait, so they stream while gate/up finishes
//
// Down blocks publish their rows and take a ticket per 16-row tile; the last of the k + 1 contributions to
// a tile applies the routing-weighted combine and the residual, in the order of moe_combine.  Each block
// only waits on blocks with smaller indices, which the dispatcher starts first, so every wait is on work
// that is running or finished.  Waits are bounded: a wait that runs out sets the sticky status word of
// the workspace instead of hanging (results are then invalid).  Values cross blocks by device-coherent
// stores and loads and 32-bit relaxed device-scope counters; the block that combines the last tile resets
// every counter, so the workspace is ready for the next call when the kernel ends.
//
// The normalized activation is computed by every block that needs it with the same fixed-order
// reduction, so all of them (and the router) see the same u:
//   u[j] = round_x( (x[j] * gamma[j]) * rinv ),  rinv = 1 / sqrt(sum_j x[j]^2 / d + eps)
// The expert arithmetic is that of q4_expert_gemv (q4_device.h); the gate/up blocks split the row
// between their four wavefronts, the routed down blocks give each wavefront 16 whole rows.
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
// of their own: the arrival that completes a set writes a ready flag into each of its n_flags lines.  A
// set with many arrivals counts them on n_sub sub-counters first (each on its own line); the last arrival
// of a sub-counter bumps the top counter.  Small sets (n_sub = 1) save that second atomic round trip.
constexpr int kLW = 64;             // 32-bit words per line
struct SyncSet {
  uint32_t* base;                   // lines: [n_sub sub-counters][top][n_flags flags]
  int n_sub, n_flags;
  uint32_t total;                   // arrivals that complete the set (waiters on a set without flag lines
                                    // poll its counter for this value)
};
constexpr int kRouteSub = 1, kRouteFlags = 64;
constexpr int kSharedSub = 16, kSharedFlags = 16;
constexpr int kSlotSub = 1, kSlotFlags = 8;
constexpr int kTilesSub = 1;
// line 0: status word (sticky, bit 0 = a bounded wait ran out); then the sets route, shared, tiles, slots
constexpr int kLinesFixed = 1 + (kRouteSub + 1 + kRouteFlags) + (kSharedSub + 1 + kSharedFlags) + (kTilesSub + 1);
constexpr int kLinesPerSlot = kSlotSub + 1 + kSlotFlags;
constexpr int kTileStride = 16;     // words between two tile tickets

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
  void* out;
  uint32_t* status;
  SyncSet route, shared_h, tiles_done;
  SyncSet slot_h[kLayerMaxK];
  uint32_t* sync_base;  // all sync lines (reset by the block that combines the layer's last tile)
  int32_t sync_lines;
  uint32_t* tiles;     // [d/16] tickets, kTileStride words apart
  float* logits;       // [E]
  float* h_routed;     // [k][F]
  float* h_shared;     // [S]
  float* y_routed;     // [k][d]
  float* y_shared;     // [d]
  int32_t nR, nSG, nRG, nSD, nRD;
};

__device__ __forceinline__ float ld_c(const float* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ void st_c(float* p, float v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ void st_cu(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t add_cu(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One arrival (thread 0 of a block, after its published stores completed) out of `total` on set `s`;
// `idx` in [0, total) picks the sub-counter.  True for the arrival that completed the set, which has then
// raised every flag of the set.
__device__ __forceinline__ bool arrive(const SyncSet& s, int idx, int total, uint32_t n = 1u) {
  if (s.n_sub > 1) {
    const int sub = idx % s.n_sub;
    const uint32_t expect = (uint32_t)((total - sub + s.n_sub - 1) / s.n_sub);
    if (add_cu(s.base + sub * kLW, 1u) != expect - 1) return false;
    const uint32_t subs_used = (uint32_t)(total < s.n_sub ? total : s.n_sub);
    if (add_cu(s.base + s.n_sub * kLW, 1u) != subs_used - 1) return false;
  } else if (add_cu(s.base, n) + n != (uint32_t)total) {
    return false;
  }
  for (int f = 0; f < s.n_flags; ++f) st_cu(s.base + (s.n_sub + 1 + f) * kLW, 1u);
  return true;
}

// Block-wide bounded wait for set `s` to complete: thread 0 polls flag line `who` mod n_flags, or the
// counter of a single-counter set without flag lines.  Ends with a block barrier.
__device__ __forceinline__ void wait_set(const SyncSet& s, int who, uint32_t* status) {
  if (threadIdx.x == 0) {
    const bool flags = s.n_flags > 0;
    uint32_t* f = flags ? s.base + (s.n_sub + 1 + who % s.n_flags) * kLW : s.base;
    const uint32_t target = flags ? 1u : s.total;
    uint32_t v = __hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    int n = 0;
    while (v < target && n < kSpinLimit) {
      __builtin_amdgcn_s_sleep(1);
      v = __hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      ++n;
    }
    if (v < target) __hip_atomic_fetch_or(status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
}

// Publish: every thread's coherent stores have completed before thread 0 arrives on the set.
__device__ __forceinline__ void publish(const SyncSet& s, int idx, int total) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) arrive(s, idx, total);
}

// ------------------------------------------------------------------------------------------------
// the normalized activation
// ------------------------------------------------------------------------------------------------
struct NormLds {
  float wsum[kThreads / 64];
  float rinv;
};

// xg[j] = x[j] * gamma[j] (or x[j]) into LDS; returns rinv (1 without gamma).  Fixed reduction order:
// per thread over its elements in index order, the wavefront xor tree, then the four waves in order.
template <typename XT>
__device__ __forceinline__ float norm_to_lds(const LayerArgs& a, float* xg, NormLds& nl) {
  const XT* x = reinterpret_cast<const XT*>(a.x);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float ss = 0.f;
  for (int j0 = threadIdx.x * 8; j0 < a.d; j0 += kThreads * 8) {
    float v[8];
    if (sizeof(XT) == 2) {
      const uint4 w = *reinterpret_cast<const uint4*>(x + j0);
      const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        v[2 * m] = __uint_as_float(u[m] << 16);
        v[2 * m + 1] = __uint_as_float(u[m] & 0xffff0000u);
      }
    } else {
      const float4 p0 = reinterpret_cast<const float4*>(x + j0)[0], p1 = reinterpret_cast<const float4*>(x + j0)[1];
      v[0] = p0.x; v[1] = p0.y; v[2] = p0.z; v[3] = p0.w;
      v[4] = p1.x; v[5] = p1.y; v[6] = p1.z; v[7] = p1.w;
    }
    float g[8];
    if (a.gamma) {
      const float4 g0 = reinterpret_cast<const float4*>(a.gamma + j0)[0], g1 = reinterpret_cast<const float4*>(a.gamma + j0)[1];
      g[0] = g0.x; g[1] = g0.y; g[2] = g0.z; g[3] = g0.w;
      g[4] = g1.x; g[5] = g1.y; g[6] = g1.z; g[7] = g1.w;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      ss = fmaf(v[i], v[i], ss);
      xg[j0 + i] = a.gamma ? v[i] * g[i] : v[i];
    }
  }
  if (!a.gamma) {
    __syncthreads();
    return 1.0f;
  }
  ss = wave_sum(ss);
  if (lane == 0) nl.wsum[wave] = ss;
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = nl.wsum[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) t += nl.wsum[w];
    nl.rinv = 1.0f / sqrtf(t / (float)a.d + a.eps);
  }
  __syncthreads();
  return nl.rinv;
}

// u[j] from xg[j] (rounded to the activation dtype, the norm output's rounding point)
template <typename XT>
__device__ __forceinline__ float u_of(float xg, float rinv, bool norm) {
  if (!norm) return xg;
  const float u = xg * rinv;
  return sizeof(XT) == 2 ? bf16_bits_to_f32(f32_to_bf16_bits(u)) : u;
}

// ------------------------------------------------------------------------------------------------
// routing inside a block
// ------------------------------------------------------------------------------------------------
struct RouteLds {
  float lg[kLayerMaxE];
  float sel_v[kLayerMaxK];
  int sel_i[kLayerMaxK];
  float w[kLayerMaxK];
};

__device__ __forceinline__ void load_logits(const LayerArgs& a, RouteLds& r) {
  wait_set(a.route, blockIdx.x, a.status);
  if ((int)threadIdx.x < a.E) r.lg[threadIdx.x] = ld_c(a.logits + threadIdx.x);
  __syncthreads();
}

// sel_i[0..k) = the selected expert ids (top-k by rank: larger logit first, equal logits -> lower id),
// or the forced ids (no wait on the router).  sel_v = their logits when with_logits.
__device__ __forceinline__ void route_ids(const LayerArgs& a, RouteLds& r, bool with_logits) {
  if (a.forced) {
    if (with_logits) load_logits(a, r);
    if ((int)threadIdx.x < a.k) {
      const int i = a.forced[threadIdx.x];
      r.sel_i[threadIdx.x] = i;
      if (with_logits) r.sel_v[threadIdx.x] = (i >= 0 && i < a.E) ? r.lg[i] : __builtin_nanf("");
    }
    __syncthreads();
    return;
  }
  load_logits(a, r);
  if ((int)threadIdx.x < kLayerMaxK) {
    r.sel_i[threadIdx.x] = -1;
    r.sel_v[threadIdx.x] = __builtin_nanf("");
  }
  __syncthreads();
  const int c = threadIdx.x;
  if (c < a.E) {
    const float v = r.lg[c];
    int rank = 0;
    for (int e2 = 0; e2 < a.E; ++e2) {
      const float u = r.lg[e2];
      rank += (u > v) | ((u == v) & (e2 < c));
    }
    if (rank < a.k) {
      r.sel_i[rank] = c;
      r.sel_v[rank] = v;
    }
  }
  __syncthreads();
}

// w[0..k) = softmax of sel_v (after route_ids with logits); every thread sums the same terms in order
__device__ __forceinline__ void route_weights(const LayerArgs& a, RouteLds& r) {
  if ((int)threadIdx.x < a.k) {
    float mx = r.sel_v[0];
    for (int i = 1; i < a.k; ++i) mx = fmaxf(mx, r.sel_v[i]);
    float den = 0.f;
    for (int i = 0; i < a.k; ++i) den += expf(r.sel_v[i] - mx);
    r.w[threadIdx.x] = expf(r.sel_v[threadIdx.x] - mx) / den;
  }
  __syncthreads();
}

// ------------------------------------------------------------------------------------------------
// roles
// ------------------------------------------------------------------------------------------------
template <typename XT>
__device__ __forceinline__ void router_block(const LayerArgs& a, int b, float* xg, NormLds& nl) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int e = b * 4 + wave;
  const int nch = a.d / 16;
  int4 q[kLayerMaxD / 16 / 64];
#pragma unroll
  for (int m = 0; m < kLayerMaxD / 16 / 64; ++m) {
    const int c = lane + 64 * m;
    if (e < a.E && c < nch) q[m] = *reinterpret_cast<const int4*>(a.rw + (int64_t)e * a.d + c * 16);
  }
  const float rinv = norm_to_lds<XT>(a, xg, nl);
  // u in place (same rounding as the gate/up blocks)
  for (int j = threadIdx.x; j < a.d; j += kThreads) xg[j] = u_of<XT>(xg[j], rinv, a.gamma != nullptr);
  __syncthreads();
  if (e < a.E) {
    float acc = 0.f;
#pragma unroll
    for (int m = 0; m < kLayerMaxD / 16 / 64; ++m) {
      const int c = lane + 64 * m;
      if (c >= nch) break;
      const float4* xv = reinterpret_cast<const float4*>(xg + c * 16);
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
    if (lane == 0) {
      const float lgt = acc * a.rs[e];
      st_c(a.logits + e, lgt);
      if (a.logits_out) a.logits_out[e] = lgt;
    }
  }
  publish(a.route, b, a.nR);
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

template <int NBW, typename XT, bool SB_BF16>
__device__ __forceinline__ void gu_finish(const LayerArgs& a, const GuRegs<NBW, SB_BF16>& g, bool valid, int tile,
                                          float rinv, float* hout, const SyncSet& done, int done_total,
                                          const float* xg, Stage st) {
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
    for (int i = 0; i < 8; ++i) v[i] = live ? u_of<XT>(xg[hg * 32 + qd * 8 + i], rinv, a.gamma != nullptr) : 0.f;
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
  publish(done, tile, done_total);
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

// Combine tile `tile` (threads 0..15) with the block's routing (r.sel_i, r.w)
template <typename XT>
__device__ __forceinline__ void combine_one(const LayerArgs& a, const RouteLds& r, int tile) {
  const int row = tile * 16 + (int)threadIdx.x;
  float acc = 0.f;
  for (int i = 0; i < a.k; ++i) acc = __builtin_fmaf(r.w[i], ld_c(a.y_routed + (int64_t)i * a.d + row), acc);
  if (a.has_shared) acc += ld_c(a.y_shared + row);
  const XT* x = reinterpret_cast<const XT*>(a.x);
  if (a.residual) acc += sizeof(XT) == 2 ? bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(x)[row])
                                         : reinterpret_cast<const float*>(x)[row];
  if (sizeof(XT) == 2)
    reinterpret_cast<uint16_t*>(a.out)[row] = (uint16_t)f32_to_bf16_bits(acc);
  else
    reinterpret_cast<float*>(a.out)[row] = acc;
}

// After a down block published its rows: one ticket per covered tile; combine the tiles this block
// completed; the block that combines the last tile of the layer resets every counter.
template <typename XT>
__device__ __forceinline__ void tile_epilogue(const LayerArgs& a, int tile0, int ntiles, RouteLds& r, uint32_t* lastf,
                                              bool have_weights) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  const uint32_t units = (uint32_t)a.k + (a.has_shared ? 1u : 0u);
  if ((int)threadIdx.x < ntiles)
    lastf[threadIdx.x] = add_cu(a.tiles + (tile0 + threadIdx.x) * kTileStride, 1u) == units - 1;
  __syncthreads();
  bool any = false;
  for (int t = 0; t < ntiles; ++t) any |= lastf[t] != 0;
  if (!any) return;
  if (!have_weights) {
    route_ids(a, r, true);
    route_weights(a, r);
  }
  uint32_t n = 0;
  for (int t = 0; t < ntiles; ++t) {
    if (!lastf[t]) continue;
    ++n;
    if (threadIdx.x < 16) combine_one<XT>(a, r, tile0 + t);
    if (threadIdx.x == 0) st_cu(a.tiles + (tile0 + t) * kTileStride, 0u);
  }
  __shared__ uint32_t final_s;
  if (threadIdx.x == 0) final_s = arrive(a.tiles_done, 0, a.d / 16, n) ? 1u : 0u;
  __syncthreads();
  if (final_s) {
    // every other block has passed all of its waits: clear the sync lines (not the status line)
    for (int l = 1 + (int)threadIdx.x; l < a.sync_lines; l += kThreads) st_cu(a.sync_base + l * kLW, 0u);
  }
}

// 16 rows (r, r + 8 per lane group) of the shared expert's down matrix, waves split the row (K = S)
template <int NBW, typename XT, bool SB_BF16>
__device__ __forceinline__ void shared_down_block(const LayerArgs& a, int tile, Stage st, RouteLds& r, uint32_t* lastf) {
  const LayerPool& P = a.shared;
  const int K = P.F, lane = threadIdx.x & 63, wave = threadIdx.x >> 6, ra = lane >> 3, j = lane & 7;
  const int C = K / 32;
  const int row = tile * 16 + ra;
  __builtin_amdgcn_s_sleep(40);     // about 1 us: let the router blocks' first loads go ahead
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
  wait_set(a.shared_h, blockIdx.x, a.status);
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
    st_c(a.y_shared + row, yA);
    st_c(a.y_shared + row + 8, yB);
  }
  tile_epilogue<XT>(a, tile, 1, r, lastf, false);
}

// 64 rows of the i-th selected expert's down matrix: wave w takes rows 16w.. of the block, whole rows
template <int NBW, typename XT, bool SB_BF16>
__device__ __forceinline__ void routed_down_block(const LayerArgs& a, int slot, int rb, Stage st, RouteLds& r,
                                                  uint32_t* lastf) {
  const LayerPool& P = a.routed;
  const int K = P.F, lane = threadIdx.x & 63, wave = threadIdx.x >> 6, ra = lane >> 3, j = lane & 7;
  const int C = K / 32;
  const int row = rb * 64 + wave * 16 + ra;
  route_ids(a, r, true);      // with the weights: this block may combine tiles at the end
  route_weights(a, r);
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
  wait_set(a.slot_h[slot], blockIdx.x, a.status);
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
  if (j == 0) {
    float* y = a.y_routed + (int64_t)slot * a.d;
    st_c(y + row, valid ? yA : __builtin_nanf(""));
    st_c(y + row + 8, valid ? yB : __builtin_nanf(""));
  }
  tile_epilogue<XT>(a, rb * 4, 4, r, lastf, true);
}

template <int NBW, typename XT, bool SB_BF16>
__global__ __launch_bounds__(kThreads) void decode_layer_kernel(LayerArgs a) {
  extern __shared__ __align__(16) uint32_t lds[];
  __shared__ NormLds nl;
  __shared__ RouteLds r;
  __shared__ uint32_t lastf[4];
  float* xg = reinterpret_cast<float*>(lds);                       // [d]
  uint32_t* stage_base = lds + a.d;                                 // staging area
  int b = blockIdx.x;
  // staging area: [nhg][kHgStride] words then [nhg] float4; sized by the block's own K
  auto stage_for = [&](int K) {
    const int nhg = K / 32;
    return Stage{stage_base, reinterpret_cast<float4*>(stage_base + nhg * kHgStride)};
  };
  if (b < a.nR) {
    router_block<XT>(a, b, xg, nl);
    return;
  }
  b -= a.nR;
  if (b < a.nSG) {
    // the shared expert needs only x: code words first, then the norm while they are in flight
    __builtin_amdgcn_s_sleep(40);   // about 1 us: let the router blocks' first loads go ahead
    GuRegs<NBW, SB_BF16> g;
    gu_load<NBW, SB_BF16>(a, a.shared, 0, true, b, g);
    const float rinv = norm_to_lds<XT>(a, xg, nl);
    gu_finish<NBW, XT, SB_BF16>(a, g, true, b, rinv, a.h_shared, a.shared_h, a.nSG, xg, stage_for(a.d));
    return;
  }
  b -= a.nSG;
  if (b < a.nRG) {
    const int per = a.routed.F / 8, slot = b / per, tile = b % per;
    const bool designated = b == 0 && (a.ids_out || a.weights_out);
    // the norm needs only x: done while the router finishes
    const float rinv = norm_to_lds<XT>(a, xg, nl);
    route_ids(a, r, designated);
    if (designated) {
      route_weights(a, r);
      if ((int)threadIdx.x < a.k) {
        if (a.ids_out) a.ids_out[threadIdx.x] = r.sel_i[threadIdx.x];
        if (a.weights_out) a.weights_out[threadIdx.x] = r.w[threadIdx.x];
      }
    }
    const int e = r.sel_i[slot];
    const int idx = a.gemv_ids ? a.gemv_ids[slot] : e;
    const bool valid = (unsigned)idx < (unsigned)a.routed.n_records && (unsigned)e < (unsigned)a.E;
    GuRegs<NBW, SB_BF16> g;
    gu_load<NBW, SB_BF16>(a, a.routed, idx, valid, tile, g);
    gu_finish<NBW, XT, SB_BF16>(a, g, valid, tile, rinv, a.h_routed + (int64_t)slot * a.routed.F,
                                a.slot_h[slot], per, xg, stage_for(a.d));
    return;
  }
  b -= a.nRG;
  if (b < a.nSD) {
    shared_down_block<NBW, XT, SB_BF16>(a, b, stage_for(a.shared.F), r, lastf);
    return;
  }
  b -= a.nSD;
  const int per = a.d / 64, slot = b / per, rb = b % per;
  routed_down_block<NBW, XT, SB_BF16>(a, slot, rb, stage_for(a.routed.F), r, lastf);
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

struct WsLayout {
  size_t tiles, logits, h_routed, h_shared, y_routed, y_shared, total;
};

WsLayout ws_layout(int d, int E, int k, int F, int S) {
  WsLayout w;
  size_t o = (size_t)(kLinesFixed + k * kLinesPerSlot) * kLW * 4;
  w.tiles = o;      o += align256((size_t)(d / 16) * kTileStride * 4);
  w.logits = o;     o += align256((size_t)E * 4);
  w.h_routed = o;   o += align256((size_t)k * F * 4);
  w.h_shared = o;   o += align256((size_t)(S > 0 ? S : 1) * 4);
  w.y_routed = o;   o += align256((size_t)k * d * 4);
  w.y_shared = o;   o += align256((size_t)d * 4);
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

}  // namespace
}  // namespace moeq4

using namespace moeq4;

extern "C" size_t moe_decode_layer_sync_bytes(int32_t d, int32_t k) {
  if (d < 64 || k < 1 || k > kLayerMaxK) return 0;
  return ws_layout(d, 1, k, 64, 0).tiles + align256((size_t)(d / 16) * kTileStride * 4);
}

extern "C" size_t moe_decode_layer_workspace_bytes(int32_t d, int32_t E, int32_t k, int32_t F, int32_t S) {
  if (d < 64 || E < 1 || k < 1 || F < 64) return 0;
  return ws_layout(d, E, k, F, S).total;
}

extern "C" moe_status moe_decode_layer(const void* x_dev, moe_dtype x_dtype, const float* gamma_dev, float eps,
                                       int32_t residual, const int8_t* router_w_dev, const float* router_scale_dev,
                                       int32_t E, int32_t k, const int32_t* forced_ids_dev, const moe_q4_pool* routed,
                                       const int32_t* gemv_ids_dev, const moe_q4_pool* shared, moe_act act,
                                       int32_t* ids_dev, float* weights_dev, float* logits_dev, void* out_dev,
                                       void* workspace_dev, size_t workspace_bytes, void* stream) {
  const char* who = "moe_decode_layer";
  if (!x_dev || !router_w_dev || !router_scale_dev || !routed || !out_dev || !workspace_dev)
    return fail(MOE_ERR_INVALID_ARG, "%s: NULL pointer", who);
  if (x_dtype != MOE_F32 && x_dtype != MOE_BF16) return fail(MOE_ERR_INVALID_ARG, "%s: bad x_dtype", who);
  if (act != MOE_ACT_GELU_TANH && act != MOE_ACT_SILU) return fail(MOE_ERR_INVALID_ARG, "%s: bad act", who);
  if (gamma_dev && !(eps >= 0.f)) return fail(MOE_ERR_INVALID_ARG, "%s: eps must be >= 0", who);
  const char* why = nullptr;
  LayerArgs a{};
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
    return fail(MOE_ERR_UNSUPPORTED, "%s: E=%d k=%d (need 1 <= k <= min(E, 32), E <= %d)", who, E, k, kLayerMaxE);
  if (!aligned(x_dev, 16) || !aligned(router_w_dev, 16) || (gamma_dev && !aligned(gamma_dev, 16)))
    return fail(MOE_ERR_INVALID_ARG, "%s: x, router weights and gamma must be 16-byte aligned", who);
  const WsLayout w = ws_layout(d, E, k, routed->F, shared ? shared->F : 0);
  if (workspace_bytes < w.total) return fail(MOE_ERR_INVALID_ARG, "%s: workspace %zu bytes < %zu", who, workspace_bytes, w.total);
  if (!aligned(workspace_dev, 256)) return fail(MOE_ERR_INVALID_ARG, "%s: workspace not 256-byte aligned", who);
  char* ws = static_cast<char*>(workspace_dev);
  a.x = x_dev;
  a.gamma = gamma_dev;
  a.eps = eps;
  a.residual = residual != 0;
  a.rw = router_w_dev;
  a.rs = router_scale_dev;
  a.E = E;
  a.k = k;
  a.d = d;
  a.act = act;
  a.forced = forced_ids_dev;
  a.gemv_ids = gemv_ids_dev;
  a.has_shared = shared != nullptr;
  a.ids_out = ids_dev;
  a.weights_out = weights_dev;
  a.logits_out = logits_dev;
  a.out = out_dev;
  uint32_t* sync = reinterpret_cast<uint32_t*>(ws);
  a.status = sync;
  a.sync_base = sync;
  a.sync_lines = kLinesFixed + k * kLinesPerSlot;
  int line = 1;
  a.route = SyncSet{sync + line * kLW, kRouteSub, kRouteFlags, (uint32_t)((E + 3) / 4)};
  line += kRouteSub + 1 + kRouteFlags;
  a.shared_h = SyncSet{sync + line * kLW, kSharedSub, kSharedFlags, (uint32_t)(shared ? shared->F / 8 : 0)};
  line += kSharedSub + 1 + kSharedFlags;
  a.tiles_done = SyncSet{sync + line * kLW, kTilesSub, 0, (uint32_t)(d / 16)};
  line += kTilesSub + 1;
  for (int i = 0; i < k; ++i) {
    a.slot_h[i] = SyncSet{sync + line * kLW, kSlotSub, kSlotFlags, (uint32_t)(routed->F / 8)};
    line += kLinesPerSlot;
  }
  a.tiles = reinterpret_cast<uint32_t*>(ws + w.tiles);
  a.logits = reinterpret_cast<float*>(ws + w.logits);
  a.h_routed = reinterpret_cast<float*>(ws + w.h_routed);
  a.h_shared = reinterpret_cast<float*>(ws + w.h_shared);
  a.y_routed = reinterpret_cast<float*>(ws + w.y_routed);
  a.y_shared = reinterpret_cast<float*>(ws + w.y_shared);
  a.nR = (E + 3) / 4;
  a.nSG = shared ? shared->F / 8 : 0;
  a.nRG = k * (routed->F / 8);
  a.nSD = shared ? d / 16 : 0;
  a.nRD = k * (d / 64);
  // chunk iterations per lane: gate/up rows (K = d) and shared down rows (K = S) split over 4 waves,
  // routed down rows (K = F) whole per wave
  const int it_gu = (iterations(d) + 3) / 4, it_sd = shared ? (iterations(shared->F) + 3) / 4 : 1;
  const int it_rd = iterations(routed->F);
  int nbw = it_gu > it_sd ? it_gu : it_sd;
  nbw = nbw > it_rd ? nbw : it_rd;
  if (nbw > 4) return fail(MOE_ERR_UNSUPPORTED, "%s: rows too long for the single-launch layer", who);
  int kmax = d > routed->F ? d : routed->F;
  if (shared && shared->F > kmax) kmax = shared->F;
  const size_t lds = (size_t)d * 4 + (size_t)(kmax / 32) * (kHgStride * 4 + 16);
  const dim3 grid(a.nR + a.nSG + a.nRG + a.nSD + a.nRD);
  const bool sb16 = routed->sb_dtype == MOE_BF16;
  hipStream_t s = as_stream(stream);
  return dispatch_nbw(nbw, [&](auto nb) {
    constexpr int N = decltype(nb)::value;
    if constexpr (N <= 4) {
      if (x_dtype == MOE_BF16) {
        if (sb16) hipLaunchKernelGGL((decode_layer_kernel<N, uint16_t, true>), grid, dim3(kThreads), lds, s, a);
        else hipLaunchKernelGGL((decode_layer_kernel<N, uint16_t, false>), grid, dim3(kThreads), lds, s, a);
      } else {
        if (sb16) hipLaunchKernelGGL((decode_layer_kernel<N, float, true>), grid, dim3(kThreads), lds, s, a);
        else hipLaunchKernelGGL((decode_layer_kernel<N, float, false>), grid, dim3(kThreads), lds, s, a);
      }
      return check_launch("moe_decode_layer");
    } else {
      return fail(MOE_ERR_UNSUPPORTED, "moe_decode_layer: rows too long");
    }
  });
}
