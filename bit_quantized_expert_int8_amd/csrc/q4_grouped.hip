// Batched decode (T > 1 tokens per call): the T*k (token, slot) pairs are grouped by expert so that
// each selected expert's rows are streamed from HBM once per call, for all of the tokens routed to it
// ([G26] "Le pipeline de traitement" and [REMIO] "Mac Gemma 4 26B tient en mémoire...": a prompt's
// tokens are processed together, sharing each expert's weights).
//
// group_pairs_kernel (one block): counting sort of the pairs by expert id.  Counts per expert, an
// exclusive scan over experts, then a stable placement (pairs of one expert keep ascending pair order)
// into perm; non-empty experts are listed in `groups`, and (for the grouped products) every group's runs
// of at most 16 consecutive pairs in `chunks`, the unit of work of the matrix-core kernel.  Ids outside the routed pool form one extra group
// whose outputs are NaN, as in the single-token kernels.  The grouped products themselves run on the
// matrix cores (q4_mfma.hip).
#include "q4_device.h"

namespace moeq4 {
namespace {

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

__global__ __launch_bounds__(kGroupThreads) void group_pairs_kernel(const int32_t* __restrict__ ids, int P, int n_valid,
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

}  // namespace

moe_status launch_group_pairs(const int32_t* ids, int P, int n_valid, int32_t* n_groups, int4* groups, int32_t* perm,
                              hipStream_t s, int32_t* n_chunks, int4* chunks) {
  hipLaunchKernelGGL(group_pairs_kernel, dim3(1), dim3(kGroupThreads), 0, s, ids, P, n_valid, n_groups, groups, perm,
                     n_chunks, chunks);
  return check_launch("group_pairs");
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
