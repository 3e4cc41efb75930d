// Device code of the grouping of a batch's (token, slot) pairs by expert (see q4_grouped.hip), shared by
// the grouping launch and the launch that groups the pairs and stages the tokens together.
#pragma once
#include "q4_device.h"

namespace moeq4 {

// Groups the pairs (as launch_group_pairs, with the chunk table) and stages the T token rows (as
// launch_stage_rows) in one launch (q4_mfma.hip).
moe_status launch_group_and_stage(const int32_t* ids, int P, int n_valid, int32_t* n_groups, int4* groups,
                                  int32_t* perm, int32_t* n_chunks, int4* chunks, const void* x, bool x_bf16, int rows,
                                  int K, const StagedRows& out, hipStream_t s);

constexpr int kGroupThreads = 256;

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

// The whole grouping, by one block of kGroupThreads threads.
__device__ __forceinline__ void group_pairs_block(const int32_t* __restrict__ ids, int P, int n_valid,
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
}


}  // namespace moeq4
