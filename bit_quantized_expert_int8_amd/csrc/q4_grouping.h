// Device code of the grouping of a batch's (token, slot) pairs by expert (see q4_grouped.hip), shared by
// the grouping launch and the launch that groups the pairs and stages the tokens together.
#pragma once
#include "q4_device.h"

namespace moeq4 {

// Groups the pairs (as launch_group_pairs, with the chunk table) and stages the T token rows (as
// launch_stage_rows) in one launch (q4_mfma.hip).
struct SplitShape;
moe_status launch_group_and_stage(const int32_t* ids, int P, int n_valid, int32_t* n_groups, int4* groups,
                                  int32_t* perm, int32_t* n_chunks, int4* chunks, const void* x, bool x_bf16, int rows,
                                  int K, const StagedRows& out, hipStream_t s, int4* plan0, const SplitShape* shape0,
                                  int4* plan1, const SplitShape* shape1);

constexpr int kGroupThreads = 256;

// ------------------------------------------------------------------------------------------------
// How the persistent blocks of a ring-kernel launch (q4_mfma.hip) split its work, given the routed chunk
// count ng (known on the device once the pairs are grouped).  The shared matrix gets blocks in proportion
// to its steps times its token chunks (tc = ceil(T / 16)) against the routed steps of the ng chunks; its
// rs = nsb / tc step ranges each take tc blocks, one per token chunk, placed so that the chunks of a range
// share an XCD (block b runs on XCD b mod 8): ranges in octets, chunk c of range 8 o + x at block
// 8 tc o + 8 c + x; the L ranges after the last full octet take 8 / L XCDs each when that divides evenly.
// The R remaining blocks split the routed chunks: with ng <= R each chunk gets R / ng or R / ng + 1 blocks,
// each an equal part of its steps; with more chunks than blocks, block b takes chunks b, b + R, ... whole.
// Host and device share this arithmetic: the grouping launch writes one descriptor per block from it (when
// the host has checked that no block needs more than one item), or the blocks run it themselves.
// ------------------------------------------------------------------------------------------------
struct SplitShape {
  int nb;   // blocks of the launch
  int T;    // tokens
  int ss;   // steps of the shared matrix (0: none)
  int sr;   // steps per routed chunk (0: none)
};
struct SplitItem {
  bool shared;
  int j;        // routed chunk, or the shared token chunk
  int s0, s1;   // step range
};

// floor(a / b) for 0 <= a < 2^53, 0 < b: a double division and an exact integer correction (a 64-bit integer
// division is a long instruction sequence on the device)
__host__ __device__ inline int64_t div_floor(int64_t a, int64_t b) {
  int64_t q = (int64_t)((double)a / (double)b);
  while (q > 0 && q * b > a) --q;
  while ((q + 1) * b <= a) ++q;
  return q;
}
// floor(a * m / d) for non-negative ints: 32-bit unsigned arithmetic when the product fits
__host__ __device__ inline int muldiv(int a, int m, int d) {
  const uint64_t p = (uint64_t)(uint32_t)a * (uint32_t)m;
  return p >> 32 ? (int)div_floor((int64_t)p, d) : (int)((uint32_t)p / (uint32_t)d);
}

// shared blocks nsb and step ranges rs for ng routed chunks
__host__ __device__ inline void split_counts(const SplitShape& sh, int ng, int* nsb_out, int* rs_out) {
  ng = sh.sr > 0 ? ng : 0;
  const int tc = (sh.T + 15) / 16;
  int nsb = 0, rs = 1;
  if (sh.ss > 0) {
    if (ng <= 0) {
      nsb = sh.nb;
    } else {
      const int64_t us = (int64_t)sh.ss * tc, ur = (int64_t)sh.sr * ng;
      nsb = (int)div_floor(sh.nb * us + (us + ur) / 2, us + ur);
      nsb = nsb < 1 ? 1 : (nsb > sh.nb - 1 ? sh.nb - 1 : nsb);
    }
    rs = nsb / tc > 1 ? nsb / tc : 1;
    nsb = nsb < tc ? nsb : rs * tc;
  }
  *nsb_out = nsb;
  *rs_out = rs;
}

// item `it` of block b (false: none), given split_counts' nsb and rs
__host__ __device__ inline bool split_item_at(const SplitShape& sh, int ng, int nsb, int rs, int b, int it, SplitItem& x) {
  ng = sh.sr > 0 ? ng : 0;
  const int tc = (sh.T + 15) / 16;
  if (b < nsb) {
    if (nsb < tc) {
      // fewer blocks than token chunks: block b takes chunks b, b + nsb, ... over all steps
      const int c = b + it * nsb;
      if (c >= tc) return false;
      x = SplitItem{true, c, 0, sh.ss};
      return true;
    }
    if (it > 0) return false;
    const int full = (rs / 8) * 8, L = rs - full;
    int c, r;
    if (b < full * tc) {
      const int o = b / (8 * tc), w = b % (8 * tc);
      c = w / 8;
      r = 8 * o + w % 8;
    } else {
      const int b2 = b - full * tc, g = 8 / L;
      if (8 % L == 0 && tc % g == 0) {
        const int m = b2 / 8, xx = b2 % 8;
        r = full + xx % L;
        c = (xx / L) * (tc / g) + m;
      } else {
        c = b2 % tc;
        r = full + b2 / tc;
      }
    }
    x = SplitItem{true, c, muldiv(r, sh.ss, rs), muldiv(r + 1, sh.ss, rs)};
    return true;
  }
  if (ng <= 0) return false;
  const int o = b - nsb, R = sh.nb - nsb, steps = sh.sr;
  int j, s0 = 0, s1 = steps;
  if (ng <= R) {
    if (it > 0) return false;
    const int q = R / ng, rem = R % ng;
    int part, parts;
    if (o < rem * (q + 1)) {
      j = o / (q + 1);
      part = o % (q + 1);
      parts = q + 1;
    } else {
      const int o2 = o - rem * (q + 1);
      j = rem + o2 / q;
      part = o2 % q;
      parts = q;
    }
    s0 = muldiv(part, steps, parts);
    s1 = muldiv(part + 1, steps, parts);
  } else {
    j = o + it * R;
    if (j >= ng) return false;
  }
  x = SplitItem{false, j, s0, s1};
  return true;
}

__host__ __device__ inline bool split_item(const SplitShape& sh, int ng, int b, int it, SplitItem& x) {
  int nsb, rs;
  split_counts(sh, ng, &nsb, &rs);
  return split_item_at(sh, ng, nsb, rs, b, it, x);
}


// No block holds more than one item for any chunk count 1..ng_max (the host's check before it asks the
// grouping launch for descriptors).
inline bool split_single_item(const SplitShape& sh, int ng_max) {
  const int tc = (sh.T + 15) / 16;
  for (int ng = sh.sr > 0 ? 1 : 0; ng <= (sh.sr > 0 ? ng_max : 0); ++ng) {
    int nsb, rs;
    split_counts(sh, ng, &nsb, &rs);
    if (sh.ss > 0 && nsb < tc && tc > 1) return false;
    if (ng > sh.nb - nsb) return false;
  }
  return true;
}

// A block's work descriptor: (record, first index into perm or first token, count, steps and flags); w holds
// s0 in bits 0-14, s1 in bits 15-29, bit 30 shared, bit 31 valid.  An all-zero entry is no work.
__host__ __device__ inline uint32_t plan_word(int s0, int s1, bool shared, bool valid) {
  return (uint32_t)s0 | ((uint32_t)s1 << 15) | (shared ? 1u << 30 : 0u) | (valid ? 1u << 31 : 0u);
}
constexpr int kPlanMaxSteps = 1 << 15;
constexpr int kPlanMaxBlocks = 4096;   // descriptors reserved per launch in a grouped call's workspace

// The split shape of a grouped launch run from descriptors (the blocks of its descriptor instantiation); false
// when the launch would not use the ring kernel, or its shape does not fit the descriptors.
bool mfma_plan_shape(MfmaArgs a, bool has_shared, bool has_routed, bool sb_bf16, SplitShape* out);



__device__ __forceinline__ int bucket_of(int32_t e, int n_valid) { return (unsigned)e < (unsigned)n_valid ? e : n_valid; }

// Exclusive scan of three counters over the block (blockDim.x == kGroupThreads); *total gets the sums.
__device__ __forceinline__ int3 block_exclusive_scan3(int3 v, int3* total) {
  __shared__ int3 wsum[kGroupThreads / 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int3 inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int x = __shfl_up(inc.x, o, 64), y = __shfl_up(inc.y, o, 64), z = __shfl_up(inc.z, o, 64);
    if (lane >= o) {
      inc.x += x;
      inc.y += y;
      inc.z += z;
    }
  }
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  int3 base = make_int3(0, 0, 0), tot = make_int3(0, 0, 0);
#pragma unroll
  for (int w = 0; w < kGroupThreads / 64; ++w) {
    if (w < wave) {
      base.x += wsum[w].x;
      base.y += wsum[w].y;
      base.z += wsum[w].z;
    }
    tot.x += wsum[w].x;
    tot.y += wsum[w].y;
    tot.z += wsum[w].z;
  }
  *total = tot;
  return make_int3(base.x + inc.x - v.x, base.y + inc.y - v.y, base.z + inc.z - v.z);
}

// Descriptors of the two product launches that follow a grouping (plan[i] NULL: none; the host has checked that
// every block of them holds one item).  Written by the blocks that stage the tokens, each a share of them,
// beside the block that groups the pairs and without waiting for it: each rebuilds the chunk count and the
// chunk table from the ids in LDS (per expert the pairs counted, scanned, cut in runs of 16 in expert order:
// the grouping's table) and writes its blocks' items as split_item gives them.
struct PlanOut {
  int4* plan[2];
  SplitShape shape[2];
};

// part of nparts: this block's share of the descriptors
__device__ __forceinline__ void plan_share(const PlanOut& po, const int32_t* __restrict__ ids, int P, int n_valid,
                                           int part, int nparts) {
  __shared__ int pcnt[kMaxGroupedRecords + 1];   // pairs per expert (bucket n_valid: ids outside the pool)
  __shared__ int pre_x[kMaxGroupedRecords + 1];  // first pair of the bucket in the grouped order
  __shared__ int pre_z[kMaxGroupedRecords + 2];  // first chunk of the bucket
  const int tid = threadIdx.x, nbk = n_valid + 1;
  for (int b = tid; b < nbk; b += kGroupThreads) pcnt[b] = 0;
  __syncthreads();
  for (int p = tid; p < P; p += kGroupThreads) atomicAdd(&pcnt[bucket_of(ids[p], n_valid)], 1);
  __syncthreads();
  const int per = (nbk + kGroupThreads - 1) / kGroupThreads;
  const int b0 = min(nbk, tid * per), b1 = min(nbk, b0 + per);
  int3 loc = make_int3(0, 0, 0);
  for (int b = b0; b < b1; ++b) {
    loc.x += pcnt[b];
    loc.z += (pcnt[b] + kChunkPairs - 1) / kChunkPairs;
  }
  int3 tot;
  int3 base = block_exclusive_scan3(loc, &tot);
  for (int b = b0; b < b1; ++b) {
    pre_x[b] = base.x;
    pre_z[b] = base.z;
    base.x += pcnt[b];
    base.z += (pcnt[b] + kChunkPairs - 1) / kChunkPairs;
  }
  if (tid == 0) pre_z[nbk] = tot.z;
  __syncthreads();
  const int ng = tot.z;
  for (int i = 0; i < 2; ++i) {
    if (!po.plan[i]) continue;
    const SplitShape& sh = po.shape[i];
    int nsb, rs;
    split_counts(sh, ng, &nsb, &rs);
    const int lo = muldiv(part, sh.nb, nparts), hi = muldiv(part + 1, sh.nb, nparts);
    for (int b = lo + tid; b < hi; b += kGroupThreads) {
      SplitItem x;
      int4 p = make_int4(0, 0, 0, 0);
      if (split_item_at(sh, ng, nsb, rs, b, 0, x) && x.s0 < x.s1) {
        if (x.shared) {
          const int cnt = sh.T - 16 * x.j < 16 ? sh.T - 16 * x.j : 16;
          p = make_int4(0, 16 * x.j, cnt, (int)plan_word(x.s0, x.s1, true, true));
        } else {
          // the bucket holding chunk j: the last with pre_z <= j
          int lo_b = 0, hi_b = nbk - 1;
          while (lo_b < hi_b) {
            const int mid = (lo_b + hi_b + 1) >> 1;
            if (pre_z[mid] <= x.j) lo_b = mid;
            else hi_b = mid - 1;
          }
          while (lo_b + 1 < nbk && pre_z[lo_b + 1] <= x.j) ++lo_b;   // skip empty buckets at the same start
          const int k0 = (x.j - pre_z[lo_b]) * kChunkPairs;
          const int cnt = pcnt[lo_b] - k0 < kChunkPairs ? pcnt[lo_b] - k0 : kChunkPairs;
          const bool valid = lo_b < n_valid;
          p = make_int4(valid ? lo_b : 0, pre_x[lo_b] + k0, cnt, (int)plan_word(x.s0, x.s1, false, valid));
        }
      }
      po.plan[i][b] = p;
    }
  }
}

// The whole grouping, by one block of kGroupThreads threads.
__device__ __forceinline__ int group_pairs_block(const int32_t* __restrict__ ids, int P, int n_valid,
                                                  int32_t* __restrict__ n_groups, int4* __restrict__ groups,
                                                  int32_t* __restrict__ perm, int32_t* __restrict__ n_chunks,
                                                  int4* __restrict__ chunks) {
  __shared__ int cnt[kMaxGroupedRecords + 1];
  __shared__ int cur[kMaxGroupedRecords + 1];
  const int tid = threadIdx.x, nb = n_valid + 1;
  for (int b = tid; b < nb; b += kGroupThreads) cnt[b] = 0;
  __syncthreads();
  for (int p = tid; p < P; p += kGroupThreads) atomicAdd(&cnt[bucket_of(ids[p], n_valid)], 1);   // integer counts
  __syncthreads();
  // buckets [b0, b1) per thread; scan of (pairs, non-empty buckets, chunks of 16 pairs)
  const int per = (nb + kGroupThreads - 1) / kGroupThreads;
  const int b0 = min(nb, tid * per), b1 = min(nb, b0 + per);
  int3 loc = make_int3(0, 0, 0);
  for (int b = b0; b < b1; ++b) {
    loc.x += cnt[b];
    loc.y += cnt[b] > 0;
    loc.z += (cnt[b] + kChunkPairs - 1) / kChunkPairs;
  }
  int3 tot;
  int3 base = block_exclusive_scan3(loc, &tot);
  for (int b = b0; b < b1; ++b) {
    cur[b] = base.x;
    if (cnt[b] > 0) groups[base.y++] = make_int4(b, base.x, cnt[b], 0);
    if (chunks)
      for (int c = 0; c < cnt[b]; c += kChunkPairs) chunks[base.z++] = make_int4(b, base.x + c, min(kChunkPairs, cnt[b] - c), 0);
    base.x += cnt[b];
  }
  if (tid == 0) {
    *n_groups = tot.y;
    if (n_chunks) *n_chunks = tot.z;
  }
  __syncthreads();
  // stable placement, kGroupThreads pairs per round.  Within a wave, the lanes holding the same bucket are
  // found by one ballot per bit of the bucket number; a pair's place is its bucket's cursor plus the number
  // of earlier lanes with that bucket.  The waves then take their places in wave order, the last lane of
  // each bucket advancing the cursor, so the order is the pairs' order.
  const int lane = tid & 63, wave = tid >> 6;
  const int nbits = 32 - __builtin_clz((unsigned)n_valid);   // buckets 0 .. n_valid
  const uint64_t below = (1ull << lane) - 1ull, above = ~((2ull << lane) - 1ull);
  for (int p0 = 0; p0 < P; p0 += kGroupThreads) {
    const int p = p0 + tid;
    const bool live = p < P;
    const int key = live ? bucket_of(ids[p], n_valid) : 0;
    uint64_t same = __ballot(live);
    for (int bit = 0; bit < nbits; ++bit) {
      const bool set = (key >> bit) & 1;
      const uint64_t m = __ballot(set);
      same &= set ? m : ~m;
    }
    const int rank = __popcll(same & below), n_same = __popcll(same);
    const bool last = (same & above) == 0;
    for (int w = 0; w < kGroupThreads / 64; ++w) {
      if (wave == w && live) {
        const int base = cur[key];   // read by every lane of the wave before any lane advances it
        perm[base + rank] = p;
        if (last) cur[key] = base + n_same;
      }
      __syncthreads();
    }
  }
  return tot.z;
}


}  // namespace moeq4
