// Batched decode (T > 1 tokens per call): the T*k (token, slot) pairs are grouped by expert so that
// each selected expert's rows are streamed from HBM once per call, for all of the tokens routed to it
// ([G26] "Le pipeline de traitement" and [REMIO] "Mac Gemma 4 26B tient en mémoire...": a prompt's
// tokens are processed together, sharing each expert's weights).
//
// 1. group_pairs_kernel (one block): counting sort of the pairs by expert id.  Counts per expert, an
//    exclusive scan over experts, then a stable placement (pairs of one expert keep ascending pair
//    order) into perm; non-empty experts are listed in `groups`.  Ids outside the routed pool form one
//    extra group whose outputs are NaN, as in the single-token kernels.
// 2. grouped gate_up: one block per (group, 8 features), and per (8 shared features, chunk of up to 8
//    tokens).  The block loads its rows' codes and scale/bias into registers once, then walks its tokens:
//    each wave stages the token's activation half-groups it consumes (the staging of the single-token
//    kernel), computes the same dot2 chains, and the block adds the waves' partial sums in the same fixed
//    order.  One token per pass: staging several at once made the compiler keep every token's LDS
//    addresses live (193 VGPRs at 4 tokens, 2 blocks per CU, measured slower).  The token loop is
//    pipelined: the list's pair indices are read 64 at a time into a lane register, and the next token's
//    activation words are loaded before the current token's dot products.
// 3. grouped down: routed blocks take 64 output rows of a group's expert, wave w rows 16w.. whole (the
//    mapping of the single-launch layer's down blocks): per token the block stages h once, each wave
//    reduces its rows within itself, no block-wide sum.  Shared blocks take 16 rows of the shared expert
//    (waves split the long row) for a chunk of up to 8 tokens.
// Every token's result is bit-identical to the single-token kernels'; the codes cross HBM once for all of
// the group's tokens (the shared expert's once per 8 tokens, the rest from the caches).
// The problem is bound by HBM (about 12 flops per weight byte at 32 tokens), so the dot products stay on
// the vector ALUs; see q4_device.h for the dequantization.
#include "q4_device.h"

namespace moeq4 {
namespace {

constexpr int kGroupThreads = 256;

__device__ __forceinline__ int bucket_of(int32_t e, int n_valid) { return (unsigned)e < (unsigned)n_valid ? e : n_valid; }

// Exclusive scan of two counters over the block (blockDim.x == kGroupThreads); *total gets the sums.
__device__ __forceinline__ int2 block_exclusive_scan2(int2 v, int2* total) {
  __shared__ int2 wsum[kGroupThreads / 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int2 inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int x = __shfl_up(inc.x, o, 64), y = __shfl_up(inc.y, o, 64);
    if (lane >= o) {
      inc.x += x;
      inc.y += y;
    }
  }
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  int2 base = make_int2(0, 0), tot = make_int2(0, 0);
#pragma unroll
  for (int w = 0; w < kGroupThreads / 64; ++w) {
    if (w < wave) {
      base.x += wsum[w].x;
      base.y += wsum[w].y;
    }
    tot.x += wsum[w].x;
    tot.y += wsum[w].y;
  }
  *total = tot;
  return make_int2(base.x + inc.x - v.x, base.y + inc.y - v.y);
}

__global__ __launch_bounds__(kGroupThreads) void group_pairs_kernel(const int32_t* __restrict__ ids, int P, int n_valid,
                                                                    int32_t* __restrict__ n_groups, int4* __restrict__ groups,
                                                                    int32_t* __restrict__ perm) {
  __shared__ int cnt[kMaxGroupedRecords + 1];
  __shared__ int cur[kMaxGroupedRecords + 1];
  __shared__ int keys[kGroupThreads];
  const int tid = threadIdx.x, nb = n_valid + 1;
  for (int b = tid; b < nb; b += kGroupThreads) cnt[b] = 0;
  __syncthreads();
  for (int p = tid; p < P; p += kGroupThreads) atomicAdd(&cnt[bucket_of(ids[p], n_valid)], 1);   // integer counts
  __syncthreads();
  // buckets [b0, b1) per thread; scan of (pairs, non-empty buckets)
  const int per = (nb + kGroupThreads - 1) / kGroupThreads;
  const int b0 = min(nb, tid * per), b1 = min(nb, b0 + per);
  int2 loc = make_int2(0, 0);
  for (int b = b0; b < b1; ++b) {
    loc.x += cnt[b];
    loc.y += cnt[b] > 0;
  }
  int2 tot;
  int2 base = block_exclusive_scan2(loc, &tot);
  for (int b = b0; b < b1; ++b) {
    cur[b] = base.x;
    if (cnt[b] > 0) groups[base.y++] = make_int4(b, base.x, cnt[b], 0);
    base.x += cnt[b];
  }
  if (tid == 0) *n_groups = tot.y;
  __syncthreads();
  // stable placement, kGroupThreads pairs per round: rank among the round's earlier pairs of the same expert
  for (int p0 = 0; p0 < P; p0 += kGroupThreads) {
    const int p = p0 + tid;
    const int key = p < P ? bucket_of(ids[p], n_valid) : -1;
    keys[tid] = key;
    __syncthreads();
    int r = 0;
    bool last = true;
    if (p < P) {
      for (int u = 0; u < kGroupThreads; ++u) {
        const bool same = keys[u] == key;
        r += same && u < tid;
        last = last && !(same && u > tid);
      }
      perm[cur[key] + r] = p;
    }
    __syncthreads();
    if (p < P && last) cur[key] += r + 1;
    __syncthreads();
  }
}

// ------------------------------------------------------------------------------------------------
// grouped GEMV blocks
// ------------------------------------------------------------------------------------------------
struct GroupSlot {
  bool shared, valid;
  int tile, e, start, count;
};

// The block's matrix and token list; false for blocks past the last non-empty group.
__device__ __forceinline__ bool group_slot(const GemvArgs& a, GroupSlot& s) {
  int u = blockIdx.x;
  const int nsb = a.nb_shared * ((a.T + kSharedTokens - 1) / kSharedTokens);
  s.shared = u < nsb;
  s.valid = true;
  s.e = 0;
  s.start = 0;
  if (s.shared) {
    s.tile = u % a.nb_shared;
    s.start = (u / a.nb_shared) * kSharedTokens;
    s.count = min(kSharedTokens, a.T - s.start);
    return true;
  }
  u -= nsb;
  const int j = u / a.nb_routed;
  s.tile = u % a.nb_routed;
  if (j >= *a.n_groups) return false;
  const int4 g = a.groups[j];
  s.valid = (unsigned)g.x < (unsigned)a.routed.n_records;
  s.e = s.valid ? g.x : 0;
  s.start = g.y;
  s.count = g.z;
  return true;
}

template <int NBW, bool SB_BF16>
struct RowPairRegs {
  SbWord<SB_BF16> sa[NBW], sb[NBW];
  u32x4 qa[NBW], qb[NBW];
};

// Steps 2-3 of the single-token row-pair routine: this lane's scale/bias words and code chunks.
template <int NBW, bool SB_BF16>
__device__ __forceinline__ void load_rowpair(const char* rowA, const char* rowB, const char* sbA, const char* sbB, int K,
                                             bool valid, RowPairRegs<NBW, SB_BF16>& r, int W) {
  const int wave = threadIdx.x >> 6, j = threadIdx.x & 7;
  const int C = K / 32;
  if (!valid) return;
#pragma unroll
  for (int m = 0; m < NBW; ++m) {
    const int c = (wave + W * m) * kLanesPerRow + j;
    if (c < C) {
      r.sa[m] = load_sb<SB_BF16>(sbA, c >> 1);
      r.sb[m] = load_sb<SB_BF16>(sbB, c >> 1);
    }
  }
#pragma unroll
  for (int m = 0; m < NBW; ++m) {
    const int c = (wave + W * m) * kLanesPerRow + j;
    if (c < C) {
      r.qa[m] = load_nt(rowA + c * 16);
      r.qb[m] = load_nt(rowB + c * 16);
    }
  }
}

// The block's token list: entry c is pair pair_at(c) (t*k + i; the token itself for the shared expert).
// Routed lists are read from perm 64 entries at a time into a lane register, so a token's pair index is a
// lane broadcast instead of a dependent load.
struct TokenList {
  const int32_t* perm;   // NULL for the shared expert
  int start, count, base, lanes;
  __device__ __forceinline__ int pair_at(int c) {
    if (!perm) return start + c;
    if (c - base >= 64 || c < base) {   // uniform over the block
      base = c & ~63;
      const int lane = threadIdx.x & 63;
      lanes = base + lane < count ? perm[start + base + lane] : 0;
    }
    return __builtin_amdgcn_readlane(lanes, c - base);
  }
};

__device__ __forceinline__ TokenList token_list(const GemvArgs& a, const GroupSlot& s) {
  return TokenList{s.shared ? nullptr : a.perm, s.start, s.count, -64, 0};
}

// Step 1 of the single-token row-pair routine for one token: this wave's activation words (the slots are
// the same for every token).
template <int NBW>
struct TokSlots {
  static constexpr int kPasses = (NBW * 32 + 63) / 64;
  int hgp[kPasses];
  bool livep[kPasses];
  __device__ __forceinline__ TokSlots(int K, int W) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int C = K / 32, nit = (C + kLanesPerRow - 1) / kLanesPerRow;
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
      const int s = lane + 64 * p, m = s >> 5, jj = (s >> 2) & 7;
      const int it = wave + W * m;
      hgp[p] = it * kLanesPerRow + jj;
      livep[p] = m < NBW && it < nit && hgp[p] < C;
    }
  }
};

template <int NBW, typename XT>
__device__ __forceinline__ void load_token(const XT* x, const TokSlots<NBW>& ts, XWord<XT> (&xw)[TokSlots<NBW>::kPasses]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int p = 0; p < TokSlots<NBW>::kPasses; ++p)
    if (ts.livep[p]) load_word<XT>(x, ts.hgp[p], (lane + 64 * p) & 3, xw[p]);
}

// Step 4: stage this wave's half-groups of the loaded token (wave-local).
template <int NBW, typename XT>
__device__ __forceinline__ void stage_token(const XWord<XT> (&xw)[TokSlots<NBW>::kPasses], const TokSlots<NBW>& ts,
                                            Stage st) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int p = 0; p < TokSlots<NBW>::kPasses; ++p) {
    float v[8];
    if (ts.livep[p]) word_to_f32<XT>(xw[p], v);
    else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = 0.f;
    }
    stage_word(v, ts.livep[p], ts.hgp[p], (lane + 64 * p) & 3, st);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Step 5: chunk_dot on the staged activation (the codes are dequantized again per token: a few extra VALU
// operations instead of 32 more live registers per chunk).
template <int NBW, bool SB_BF16>
__device__ __forceinline__ void rowpair_dots(const RowPairRegs<NBW, SB_BF16>& r, int K, Stage st, bool valid, float& yA,
                                             float& yB, int W) {
  const int wave = threadIdx.x >> 6, j = threadIdx.x & 7;
  const int C = K / 32;
  yA = yB = 0.f;
  if (!valid) return;
  const Dequant dq = opaque_dequant();
#pragma unroll
  for (int m = 0; m < NBW; ++m) {
    const int c = (wave + W * m) * kLanesPerRow + j;
    if (c >= C) continue;
    float s0, b0, s1, b1;
    sb_values<SB_BF16>(r.sa[m], s0, b0);
    sb_values<SB_BF16>(r.sb[m], s1, b1);
    const u32x4* xv = reinterpret_cast<const u32x4*>(st.xw + c * kHgStride);
    const u32x4 x0 = xv[0], x1 = xv[1], x2 = xv[2], x3 = xv[3];
    const float4 h = st.hg[c];
    const float accA = chunk_dot(r.qa[m], x0, x1, x2, x3, dq, -h.y);
    const float accB = chunk_dot(r.qb[m], x0, x1, x2, x3, dq, -h.y);
    yA = fmaf(h.x, fmaf(s0, accA, b0 * h.z), yA);
    yB = fmaf(h.x, fmaf(s1, accB, b1 * h.z), yB);
  }
}

// block_sum over the first W waves (same order: 8 lanes, then waves 0..W-1).  The caller must pass a block
// barrier before the next call (the LDS partials are reused).
__device__ __forceinline__ bool block_sum_waves(float& yA, float& yB, int W) {
  __shared__ float red[kMaxWaves][16];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, ra = lane >> 3, j = lane & 7;
  yA = reduce8(yA);
  yB = reduce8(yB);
  if (W == 1 && blockDim.x == 64) return j == 0;
  if (j == 0 && wave < W) {
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

// The token loop of the row-pair blocks (gate_up, shared down): rows in registers, each token staged by
// the waves that use it; the next token's words are loaded before the current token's dot products.
// emit(pair, yA, yB) runs on the lanes holding the totals.
template <int NBW, typename XT, bool SB_BF16, typename Row, typename Emit>
__device__ __forceinline__ void rowpair_token_loop(const RowPairRegs<NBW, SB_BF16>& w, TokenList tl, int K, Stage st,
                                                   bool valid, bool active, int W, Row row_of, Emit emit) {
  const TokSlots<NBW> ts(K, W);
  XWord<XT> cur[TokSlots<NBW>::kPasses], nxt[TokSlots<NBW>::kPasses];
  int pair = tl.count > 0 ? tl.pair_at(0) : 0;
  if (active && tl.count > 0) load_token<NBW, XT>(row_of(pair), ts, cur);
  for (int c = 0; c < tl.count; ++c) {
    if (active) stage_token<NBW, XT>(cur, ts, st);
    const int next = c + 1 < tl.count ? tl.pair_at(c + 1) : 0;
    if (active && c + 1 < tl.count) load_token<NBW, XT>(row_of(next), ts, nxt);
    float yA, yB;
    rowpair_dots<NBW, SB_BF16>(w, K, st, valid && active, yA, yB, W);
    if (block_sum_waves(yA, yB, W)) emit(pair, yA, yB);
    __syncthreads();   // the staging area and the partials are rewritten for the next token
#pragma unroll
    for (int p = 0; p < TokSlots<NBW>::kPasses; ++p) cur[p] = nxt[p];
    pair = next;
  }
}

template <int NBW, typename XT, bool SB_BF16>
__global__ __launch_bounds__(64 * kMaxWaves) void gate_up_grouped_kernel(GemvArgs a) {
  extern __shared__ __align__(16) uint32_t lds[];
  GroupSlot sl;
  if (!group_slot(a, sl)) return;
  const Pool& P = sl.shared ? a.shared : a.routed;
  const int K = a.d, nhg = K / 32, W = blockDim.x >> 6;
  const int ra = (threadIdx.x & 63) >> 3;
  const int F = P.F, f = sl.tile * 8 + ra;
  const char* rec = P.base + (int64_t)sl.e * P.record_bytes;
  const int64_t rowb = K / 2, sbrow = (int64_t)(K / 64) * (SB_BF16 ? 4 : 8);
  RowPairRegs<NBW, SB_BF16> w;
  load_rowpair<NBW, SB_BF16>(rec + P.off_q + f * rowb, rec + P.off_q + (F + f) * rowb, rec + P.off_sb + f * sbrow,
                             rec + P.off_sb + (F + f) * sbrow, K, sl.valid, w, W);
  const Stage st{lds, reinterpret_cast<float4*>(lds + nhg * kHgStride)};
  const XT* x = reinterpret_cast<const XT*>(a.in);
  float* hbase = sl.shared ? a.h_shared : a.h_routed;
  const bool shared = sl.shared, valid = sl.valid;
  const int k = a.k, act = a.act;
  rowpair_token_loop<NBW, XT, SB_BF16>(
      w, token_list(a, sl), K, st, valid, true, W,
      [=](int pair) { return x + (int64_t)(shared ? pair : pair / k) * K; },
      [=](int pair, float yA, float yB) {
        hbase[(int64_t)pair * F + f] = valid ? activation(yA, act) * yB : __builtin_nanf("");
      });
}

// The 64-row routed block: lane (ra, j) of wave w takes rows r = tile * 64 + 16 w + ra and r + 8, chunks
// m * 8 + j of the whole row (NBW >= the row's chunk iterations).
template <int NBW, bool SB_BF16>
__device__ __forceinline__ void down_routed_rows(const GemvArgs& a, const GroupSlot& sl, uint32_t* lds) {
  const Pool& P = a.routed;
  const int W = a.down_waves;
  const int d = a.d, K = P.F, nhg = K / 32, C = K / 32;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, ra = lane >> 3, j = lane & 7;
  const int r = sl.tile * 64 + wave * 16 + ra;
  const char* rec = P.base + (int64_t)sl.e * P.record_bytes;
  const int64_t rowb = K / 2, sbrow = (int64_t)(K / 64) * (SB_BF16 ? 4 : 8);
  SbWord<SB_BF16> sa[NBW], sb[NBW];
  u32x4 qa[NBW], qb[NBW];
  if (sl.valid) {
#pragma unroll
    for (int m = 0; m < NBW; ++m) {
      const int c = m * kLanesPerRow + j;
      if (c < C) {
        sa[m] = load_sb<SB_BF16>(rec + P.off_sb + r * sbrow, c >> 1);
        sb[m] = load_sb<SB_BF16>(rec + P.off_sb + (r + 8) * sbrow, c >> 1);
      }
    }
#pragma unroll
    for (int m = 0; m < NBW; ++m) {
      const int c = m * kLanesPerRow + j;
      if (c < C) {
        qa[m] = load_nt(rec + P.off_q + r * rowb + c * 16);
        qb[m] = load_nt(rec + P.off_q + (r + 8) * rowb + c * 16);
      }
    }
  }
  const Stage st{lds, reinterpret_cast<float4*>(lds + nhg * kHgStride)};
  // the token's h is staged by the block, one (half-group, quarter) item per thread (K <= 1024 with 256
  // threads: one item each); the next token's h is loaded before the current token's dot products
  TokenList tl = token_list(a, sl);
  const int item = threadIdx.x, hg_i = item >> 2, qd_i = item & 3;
  const bool has_item = item < nhg * 4;
  float4 hc0 = make_float4(0.f, 0.f, 0.f, 0.f), hc1 = hc0, hn0 = hc0, hn1 = hc0;
  int pair = tl.count > 0 ? tl.pair_at(0) : 0;
  if (has_item && tl.count > 0) {
    const float4* hv = reinterpret_cast<const float4*>(a.h_routed + (int64_t)pair * K + hg_i * 32 + qd_i * 8);
    hc0 = hv[0];
    hc1 = hv[1];
  }
  for (int c0 = 0; c0 < tl.count; ++c0) {
    const Dequant dq = opaque_dequant();
    {
      const float v[8] = {hc0.x, hc0.y, hc0.z, hc0.w, hc1.x, hc1.y, hc1.z, hc1.w};
      stage_word(v, has_item, hg_i, qd_i, st);
    }
    const int next = c0 + 1 < tl.count ? tl.pair_at(c0 + 1) : 0;
    if (has_item && c0 + 1 < tl.count) {
      const float4* hv = reinterpret_cast<const float4*>(a.h_routed + (int64_t)next * K + hg_i * 32 + qd_i * 8);
      hn0 = hv[0];
      hn1 = hv[1];
    }
    __syncthreads();
    // chunk iteration m belongs to wave m % W of the one-token launch: one partial per such wave, each
    // summed over its 8 lanes, then added in wave order (that launch's association, bit for bit)
    float pa[kMaxWaves], pb[kMaxWaves];
#pragma unroll
    for (int w = 0; w < kMaxWaves; ++w) pa[w] = pb[w] = 0.f;
    if (sl.valid) {
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
#pragma unroll
          for (int w = 0; w < kMaxWaves; ++w)
            if (m % W == w) {
              pa[w] = fmaf(h.x, fmaf(s0, accA, b0 * h.z), pa[w]);
              pb[w] = fmaf(h.x, fmaf(s1, accB, b1 * h.z), pb[w]);
            }
        }
      }
    }
    float yA = reduce8(pa[0]), yB = reduce8(pb[0]);
#pragma unroll
    for (int w = 1; w < kMaxWaves; ++w)
      if (w < W) {
        yA += reduce8(pa[w]);
        yB += reduce8(pb[w]);
      }
    if (j == 0) {
      float* y = a.y_routed + (int64_t)pair * d;
      y[r] = sl.valid ? yA : __builtin_nanf("");
      y[r + 8] = sl.valid ? yB : __builtin_nanf("");
    }
    __syncthreads();   // the staging area is rewritten for the next token
    hc0 = hn0;
    hc1 = hn1;
    pair = next;
  }
}

template <int NBW, bool SB_BF16>
__global__ __launch_bounds__(64 * kMaxWaves) void down_grouped_kernel(GemvArgs a) {
  extern __shared__ __align__(16) uint32_t lds[];
  GroupSlot sl;
  if (!group_slot(a, sl)) return;
  if (!sl.shared) {
    down_routed_rows<NBW, SB_BF16>(a, sl, lds);
    return;
  }
  // 16 rows of the shared expert, the first down_waves waves split the row (K = S), as in the one-token
  // launch; the others only take part in the block's barriers
  const int W = a.down_waves;
  const bool active = (int)(threadIdx.x >> 6) < W;
  const Pool& P = a.shared;
  const int d = a.d, K = P.F, nhg = K / 32;
  const int ra = (threadIdx.x & 63) >> 3;
  const int r = sl.tile * 16 + ra;
  const char* rec = P.base;
  const int64_t rowb = K / 2, sbrow = (int64_t)(K / 64) * (SB_BF16 ? 4 : 8);
  RowPairRegs<NBW, SB_BF16> w;
  load_rowpair<NBW, SB_BF16>(rec + P.off_q + r * rowb, rec + P.off_q + (r + 8) * rowb, rec + P.off_sb + r * sbrow,
                             rec + P.off_sb + (r + 8) * sbrow, K, active, w, W);
  const Stage st{lds, reinterpret_cast<float4*>(lds + nhg * kHgStride)};
  const float* hs = a.h_shared;
  float* ys = a.y_shared;
  rowpair_token_loop<NBW, float, SB_BF16>(
      w, token_list(a, sl), K, st, true, active, W, [=](int pair) { return hs + (int64_t)pair * K; },
      [=](int pair, float yA, float yB) {
        ys[(int64_t)pair * d + r] = yA;
        ys[(int64_t)pair * d + r + 8] = yB;
      });
}

}  // namespace

moe_status launch_group_pairs(const int32_t* ids, int P, int n_valid, int32_t* n_groups, int4* groups, int32_t* perm,
                              hipStream_t s) {
  hipLaunchKernelGGL(group_pairs_kernel, dim3(1), dim3(kGroupThreads), 0, s, ids, P, n_valid, n_groups, groups, perm);
  return check_launch("group_pairs");
}

moe_status launch_gate_up_grouped(const GemvArgs& a, moe_dtype x_dtype, bool sb_bf16, int nbw, int waves, dim3 grid,
                                  hipStream_t s) {
  const dim3 block(64 * waves);
  const size_t lds = lds_bytes(a.d);
  return dispatch_nbw(nbw, [&](auto nb) {
    constexpr int N = decltype(nb)::value;
    if (x_dtype == MOE_BF16) {
      if (sb_bf16) hipLaunchKernelGGL((gate_up_grouped_kernel<N, uint16_t, true>), grid, block, lds, s, a);
      else hipLaunchKernelGGL((gate_up_grouped_kernel<N, uint16_t, false>), grid, block, lds, s, a);
    } else {
      if (sb_bf16) hipLaunchKernelGGL((gate_up_grouped_kernel<N, float, true>), grid, block, lds, s, a);
      else hipLaunchKernelGGL((gate_up_grouped_kernel<N, float, false>), grid, block, lds, s, a);
    }
    return check_launch("q4_expert_gemv(gate_up, grouped)");
  });
}

moe_status launch_down_grouped(const GemvArgs& a, bool sb_bf16, int nbw, dim3 grid, int K_lds, hipStream_t s) {
  const dim3 block(64 * kMaxWaves);
  const size_t lds = lds_bytes(K_lds);
  return dispatch_nbw(nbw, [&](auto nb) {
    constexpr int N = decltype(nb)::value;
    if (sb_bf16) hipLaunchKernelGGL((down_grouped_kernel<N, true>), grid, block, lds, s, a);
    else hipLaunchKernelGGL((down_grouped_kernel<N, false>), grid, block, lds, s, a);
    return check_launch("q4_expert_gemv(down, grouped)");
  });
}

}  // namespace moeq4

using namespace moeq4;

extern "C" int32_t moe_group_pairs_max_groups(int32_t T, int32_t k, int32_t n_valid) {
  if (T < 1 || k < 1 || n_valid < 1) return 0;
  const long long pairs = (long long)T * k, buckets = (long long)n_valid + 1;
  return (int32_t)(pairs < buckets ? pairs : buckets);
}

extern "C" moe_status moe_group_pairs(const int32_t* ids_dev, int32_t T, int32_t k, int32_t n_valid, int32_t* n_groups_dev,
                                      int32_t* groups_dev, int32_t* perm_dev, void* stream) {
  if (!ids_dev || !n_groups_dev || !groups_dev || !perm_dev) return fail(MOE_ERR_INVALID_ARG, "moe_group_pairs: NULL pointer");
  if (T < 1 || T > 65535 || k < 1 || k > 32)
    return fail(MOE_ERR_INVALID_ARG, "moe_group_pairs: T=%d k=%d (1..65535, 1..32)", T, k);
  if (n_valid < 1 || n_valid > kMaxGroupedRecords)
    return fail(MOE_ERR_UNSUPPORTED, "moe_group_pairs: n_valid=%d (1..%d)", n_valid, kMaxGroupedRecords);
  if (!aligned(groups_dev, 16)) return fail(MOE_ERR_INVALID_ARG, "moe_group_pairs: groups not 16-byte aligned");
  return launch_group_pairs(ids_dev, T * k, n_valid, n_groups_dev, reinterpret_cast<int4*>(groups_dev), perm_dev,
                            as_stream(stream));
}
