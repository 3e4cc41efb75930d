// Batched decode (T > 1 tokens per call): the T*k (token, slot) pairs are grouped by expert so that
// each selected expert's rows are streamed from HBM once per call, for all of the tokens routed to it
// ([G26] "Le pipeline de traitement" and [REMIO] "Mac Gemma 4 26B tient en mémoire...": a prompt's
// tokens are processed together, sharing each expert's weights).
//
// group_pairs_kernel (one block): counting sort of the pairs by expert id.  Counts per expert, an
// exclusive scan over experts, then a stable placement (pairs of one expert keep ascending pair order)
// into perm; non-empty experts are listed in `groups`.  Ids outside the routed pool form one extra group
// whose outputs are NaN, as in the single-token kernels.  The grouped products themselves run on the
// matrix cores (q4_mfma.hip).
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

}  // namespace

moe_status launch_group_pairs(const int32_t* ids, int P, int n_valid, int32_t* n_groups, int4* groups, int32_t* perm,
                              hipStream_t s) {
  hipLaunchKernelGGL(group_pairs_kernel, dim3(1), dim3(kGroupThreads), 0, s, ids, P, n_valid, n_groups, groups, perm);
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
