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
#include "q4_grouping.h"

namespace moeq4 {
namespace {

__global__ __launch_bounds__(kGroupThreads) void group_pairs_kernel(const int32_t* __restrict__ ids, int P, int n_valid,
                                                                    int32_t* __restrict__ n_groups, int4* __restrict__ groups,
                                                                    int32_t* __restrict__ perm, int32_t* __restrict__ n_chunks,
                                                                    int4* __restrict__ chunks) {
  group_pairs_block(ids, P, n_valid, n_groups, groups, perm, n_chunks, chunks);
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
