// q4_expert_gemv and its halves: the single-token (decode) kernels and the C entry points.  The
// arithmetic, the work mapping and the dequantization are described in q4_device.h; batches of more
// than one token go through the grouped kernels of q4_grouped.hip.
#include <map>
#include <mutex>
#include <tuple>

#include "q4_grouping.h"

namespace moeq4 {
namespace {

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
  combine_tile(a, t, sl.tile);
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

// Upper bound on the non-empty expert groups of a grouped call (ids outside the pool share one group).
int groups_max(int n_records, int T, int k) {
  const long long pairs = (long long)T * k, buckets = (long long)n_records + 1;
  return (int)(pairs < buckets ? pairs : buckets);
}

// Bytes of the grouping tables of a grouped call: group count, groups, pair permutation.
int chunks_max(int n_records, int T, int k) { return groups_max(n_records, T, k) + T * k / kChunkPairs; }
// the group count and chunk count (one 256-byte slot), groups, chunks, perm, then the work descriptors of the
// grouped gate/up and down launches
size_t group_table_bytes(int n_records, int T, int k) {
  return 256 + align256((size_t)groups_max(n_records, T, k) * 16) + align256((size_t)chunks_max(n_records, T, k) * 16) +
         align256((size_t)T * k * 4) + 2 * (size_t)kPlanMaxBlocks * 16;
}

}  // namespace
}  // namespace moeq4

using namespace moeq4;

// T > 1: the activations staged for the matrix cores, the tokens' (gate_up) or the hidden vectors (down)
size_t stage_region_bytes(const moe_q4_pool* routed, int32_t k, const moe_q4_pool* shared, int32_t T) {
  const bool has_routed = routed && k > 0;
  const int d = has_routed ? routed->d : shared->d;
  const size_t gu = moeq4::staged_rows_bytes(T, d);
  const size_t dn = (has_routed ? moeq4::staged_rows_bytes((int64_t)T * k, routed->F) : 0) +
                    (shared ? moeq4::staged_rows_bytes(T, shared->F) : 0);
  return gu > dn ? gu : dn;
}

extern "C" size_t q4_expert_gemv_workspace_bytes(const moe_q4_pool* routed, int32_t k, const moe_q4_pool* shared, int32_t T) {
  if (T < 1) return 0;
  size_t b = 0;
  if (routed && k > 0) b += align256((size_t)T * k * routed->F * 4);
  if (shared) b += align256((size_t)T * shared->F * 4);
  if (routed && k > 0 && T > 1) b += group_table_bytes(routed->n_records, T, k);
  if (T > 1 && ((routed && k > 0) || shared)) b += stage_region_bytes(routed, k, shared, T);
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
    if (T > 1 && routed->n_records > kMaxGroupedRecords)
      return fail(MOE_ERR_UNSUPPORTED, "%s: T > 1 supports routed pools of at most %d records (got %d)", who,
                  kMaxGroupedRecords, routed->n_records);
  }
  if (shared) {
    if (!pool_ok(shared, osh, &why)) return fail(MOE_ERR_INVALID_ARG, "%s: shared %s", who, why);
    if (need_y && !y_shared_dev) return fail(MOE_ERR_INVALID_ARG, "%s: y_shared is NULL", who);
  }
  const int d = has_routed ? routed->d : shared->d;
  if (T > 1) {
    // the matrix-core kernels address staged rows with 32-bit byte offsets
    const int64_t rows = has_routed ? (int64_t)T * k : T;
    const int64_t kmax = std::max<int64_t>(d, std::max<int64_t>(has_routed ? routed->F : 0, shared ? shared->F : 0));
    if (rows * kmax * 2 >= (int64_t(1) << 31))
      return fail(MOE_ERR_UNSUPPORTED, "%s: T=%d: %lld staged rows of %lld values exceed 2 GiB", who, T, (long long)rows,
                  (long long)kmax);
  }
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
  a->T = T;
  char* g = ws + (has_routed ? align256((size_t)T * k * Fr * 4) : 0) + (shared ? align256((size_t)T * Fs * 4) : 0);
  if (has_routed && T > 1) {
    const size_t gb = align256((size_t)groups_max(routed->n_records, T, k) * 16);
    const size_t cb = align256((size_t)chunks_max(routed->n_records, T, k) * 16);
    a->n_groups = reinterpret_cast<int32_t*>(g);
    a->n_chunks = reinterpret_cast<int32_t*>(g) + 1;
    a->groups = reinterpret_cast<int4*>(g + 256);
    a->chunks = reinterpret_cast<int4*>(g + 256 + gb);
    a->perm = reinterpret_cast<int32_t*>(g + 256 + gb + cb);
    char* pl = g + 256 + gb + cb + align256((size_t)T * k * 4);
    a->plan_gu = reinterpret_cast<int4*>(pl);
    a->plan_dn = reinterpret_cast<int4*>(pl + (size_t)kPlanMaxBlocks * 16);
    g += group_table_bytes(routed->n_records, T, k);
  }
  a->stage = T > 1 ? g : nullptr;
  return MOE_OK;
}

// The grouped products' arguments that fix their launch shapes (T > 1).
MfmaArgs gate_up_mfma(const GemvArgs& a, int T) {
  MfmaArgs m{};
  m.routed = a.routed;
  m.shared = a.shared;
  m.K_routed = m.K_shared = a.d;
  m.wk_routed = m.wk_shared = mfma_waves_per_tile(a.d);
  m.gate_up = 1;
  m.act = a.act;
  m.T = T;
  m.k = a.k;
  m.tiles_shared = a.shared.base ? a.shared.F / 8 : 0;   // 8 features a tile
  m.tiles_routed = a.routed.F / 8;
  return m;
}
MfmaArgs down_mfma(const GemvArgs& a, int T) {
  MfmaArgs m{};
  m.routed = a.routed;
  m.shared = a.shared;
  m.K_routed = a.routed.F;
  m.K_shared = a.shared.F;
  m.wk_routed = a.k > 0 ? mfma_waves_per_tile(a.routed.F) : 1;
  m.wk_shared = a.shared.base ? mfma_waves_per_tile(a.shared.F) : 1;
  m.T = T;
  m.k = a.k;
  m.tiles_shared = m.tiles_routed = a.d / 16;   // 16 rows a tile
  return m;
}
// Whether a grouped launch runs from descriptors the grouping launch writes: the ring kernel, and no block
// with more than one item for any chunk count the call can produce.  Both the gate/up call (which asks the
// grouping for them) and the down call (which reads them) decide the same way.
bool use_plan(const MfmaArgs& m, bool has_shared, bool has_routed, bool sb_bf16, int n_records, int T, int k,
              SplitShape* sh) {
  if (!has_routed || !mfma_plan_shape(m, has_shared, has_routed, sb_bf16, sh)) return false;
  static std::mutex mu;
  static std::map<std::tuple<int, int, int, int, int>, bool> cache;
  const int cmax = chunks_max(n_records, T, k);
  const auto key = std::make_tuple(sh->nb, sh->T, sh->ss, sh->sr, cmax);
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  const bool ok = split_single_item(*sh, cmax);
  cache.emplace(key, ok);
  return ok;
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
  if (T > 1) {
    // grouped on the matrix cores: sort the pairs by expert and stage the T tokens (one launch), then the
    // products, every selected expert's and the shared expert's rows streamed once per chunk of tokens
    const StagedRows xs = staged_rows_at(a.stage, T, a.d);
    MfmaArgs m = gate_up_mfma(a, T);
    // the work descriptors of this launch and of the down launch that follows, written by the grouping
    SplitShape shg{}, shd{};
    const bool pg = use_plan(m, a.nb_shared > 0, a.k > 0, sb_bf16, a.routed.n_records, T, a.k, &shg);
    const bool pd = use_plan(down_mfma(a, T), a.shared.base != nullptr, a.k > 0, sb_bf16, a.routed.n_records, T, a.k, &shd);
    const moe_status st =
        a.k > 0 ? launch_group_and_stage(a.ids, T * a.k, a.routed.n_records, a.n_groups, a.groups, a.perm, a.n_chunks,
                                         a.chunks, a.in, x_dtype == MOE_BF16, T, a.d, xs, s, pg ? a.plan_gu : nullptr,
                                         &shg, pd ? a.plan_dn : nullptr, &shd)
                : launch_stage_rows(a.in, x_dtype == MOE_BF16, T, a.d, xs, s);
    if (st != MOE_OK) return st;
    if (pg) m.plan = a.plan_gu;
    m.n_chunks = a.n_chunks;
    m.chunks = a.chunks;
    m.perm = a.perm;
    m.xs_routed = m.xs_shared = xs;
    m.out_routed = a.h_routed;
    m.out_shared = a.h_shared;
    m.out_len_routed = a.routed.F;
    m.out_len_shared = a.shared.F;
    return launch_grouped_mfma(m, a.nb_shared > 0, a.k > 0, sb_bf16, s);
  }
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
  if (T > 1) {
    // grouped on the matrix cores: stage the hidden vectors (one row per pair, one per token for the shared
    // expert), then one launch for both matrices: tiles of 16 rows of d with all of a group's pairs (routed,
    // row length F) or all T tokens (shared, row length S)
    if (combine) return fail(MOE_ERR_UNSUPPORTED, "q4_expert_gemv: the combine of several tokens is its own launch");
    const int P = T * a.k;
    char* base = a.stage;
    StagedRows xr{}, xsh{};
    if (has_routed) {
      xr = staged_rows_at(base, P, Fr);
      base += staged_rows_bytes(P, Fr);
    }
    if (has_shared) xsh = staged_rows_at(base, T, Fs);
    const moe_status st =
        launch_stage_rows2(a.h_routed, has_routed ? P : 0, Fr, xr, a.h_shared, has_shared ? T : 0, Fs, xsh, s);
    if (st != MOE_OK) return st;
    MfmaArgs m = down_mfma(a, T);
    SplitShape shd{};
    if (use_plan(m, has_shared, has_routed, sb_bf16, a.routed.n_records, T, a.k, &shd)) m.plan = a.plan_dn;
    m.n_chunks = a.n_chunks;
    m.chunks = a.chunks;
    m.perm = a.perm;
    m.xs_routed = xr;
    m.xs_shared = xsh;
    m.out_routed = a.y_routed;
    m.out_shared = a.y_shared;
    m.out_len_routed = m.out_len_shared = a.d;
    return launch_grouped_mfma(m, has_shared, has_routed, sb_bf16, s);
  }
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
  if (T == 1) return run_down(a, orr, osh, sb16, T, s, true);
  // several tokens: per-tile tickets would cost T * d / 16 atomics per contribution, so the grouped down
  // GEMV publishes its rows and the combine runs as its own launch
  st = run_down(a, orr, osh, sb16, T, s, false);
  if (st != MOE_OK) return st;
  return moe_combine(y_r, weights_dev, y_s, residual_dev, residual_dtype, T, has_routed ? k : 0, d, out_dev, out_dtype,
                     stream);
}

// ------------------------------------------------------------------------------------------------
// q4_gemv: one 4-bit affine matrix [N][K] times T vectors, with the row-pair routine of the expert
// kernels (same staging, dequantization and fixed-order wave sum), so its results are those of one
// expert matrix inside q4_expert_gemv.  A block owns 16 rows; rows past N in a ragged last tile read row
// N - 1 and are not stored.
// ------------------------------------------------------------------------------------------------
namespace moeq4 {
namespace {

constexpr int kGemvBlocksPerCu = 4;   // persistent blocks of q4_gemv per compute unit

struct MatArgs {
  const void* x;      // x dtype [T][K]
  const char* q;      // uint32 [N][K/8]
  const char* sb;     // sb dtype [N][K/64][2]
  float* y;           // [T][N]
  int32_t N, K, sb_row_bytes;
};

// One tile = 16 rows (rows r and r + 8 per 8-lane group of a wave, the waves splitting the row's chunk
// iterations): this lane's code words and scale/bias words of a tile, loaded in one go.
template <int NBW, bool SB_BF16>
struct TileRegs {
  SbWord<SB_BF16> sa[NBW], sb[NBW];
  u32x4 qa[NBW], qb[NBW];
};

template <int NBW, bool SB_BF16>
__device__ __forceinline__ void load_tile(const MatArgs& m, int tile, TileRegs<NBW, SB_BF16>& g) {
  const int W = blockDim.x >> 6, wave = threadIdx.x >> 6, lane = threadIdx.x & 63, ra = lane >> 3, j = lane & 7;
  const int C = m.K / 32;
  const int rA = min(tile * 16 + ra, m.N - 1), rB = min(tile * 16 + ra + 8, m.N - 1);
  const char* qA = m.q + (int64_t)rA * (m.K / 2);
  const char* qB = m.q + (int64_t)rB * (m.K / 2);
  const char* sA = m.sb + (int64_t)rA * m.sb_row_bytes;
  const char* sB = m.sb + (int64_t)rB * m.sb_row_bytes;
#pragma unroll
  for (int i = 0; i < NBW; ++i) {
    const int c = (wave + W * i) * kLanesPerRow + j;
    if (c < C) {
      g.sa[i] = load_sb<SB_BF16>(sA, c >> 1);
      g.sb[i] = load_sb<SB_BF16>(sB, c >> 1);
    }
  }
#pragma unroll
  for (int i = 0; i < NBW; ++i) {
    const int c = (wave + W * i) * kLanesPerRow + j;
    if (c < C) {
      g.qa[i] = load_nt(qA + c * 16);
      g.qb[i] = load_nt(qB + c * 16);
    }
  }
}

// The tile's two row sums of this lane (before the 8-lane and the wave reductions), in rowpair_partial's order.
template <int NBW, bool SB_BF16>
__device__ __forceinline__ void tile_dot(const MatArgs& m, const TileRegs<NBW, SB_BF16>& g, Stage st, float& yA, float& yB) {
  const int W = blockDim.x >> 6, wave = threadIdx.x >> 6, j = threadIdx.x & 7;
  const int C = m.K / 32;
  yA = 0.f;
  yB = 0.f;
  const Dequant dq = opaque_dequant();
#pragma unroll
  for (int i = 0; i < NBW; ++i) {
    const int c = (wave + W * i) * kLanesPerRow + j;
    if (c < C) {
      const u32x4* xv = reinterpret_cast<const u32x4*>(st.xw + c * kHgStride);
      const u32x4 x0 = xv[0], x1 = xv[1], x2 = xv[2], x3 = xv[3];
      const float4 h = st.hg[c];
      const float accA = chunk_dot(g.qa[i], x0, x1, x2, x3, dq, -h.y);
      const float accB = chunk_dot(g.qb[i], x0, x1, x2, x3, dq, -h.y);
      float s0, b0, s1, b1;
      sb_values<SB_BF16>(g.sa[i], s0, b0);
      sb_values<SB_BF16>(g.sb[i], s1, b1);
      yA = fmaf(h.x, fmaf(s0, accA, b0 * h.z), yA);
      yB = fmaf(h.x, fmaf(s1, accB, b1 * h.z), yB);
    }
  }
}

// Sum the tile's row pair over the block's waves in wave order (block_sum's order), with a reduction buffer
// per parity of the tile count so that the next tile's writes never meet this tile's reads.
__device__ __forceinline__ bool tile_sum(float& yA, float& yB, float (*red)[kMaxWaves][16], int parity) {
  const int W = blockDim.x >> 6, wave = threadIdx.x >> 6, lane = threadIdx.x & 63, ra = lane >> 3, j = lane & 7;
  yA = reduce8(yA);
  yB = reduce8(yB);
  if (W == 1) return j == 0;
  if (j == 0) {
    red[parity][wave][ra] = yA;
    red[parity][wave][8 + ra] = yB;
  }
  __syncthreads();
  if (wave != 0 || j != 0) return false;
  yA = red[parity][0][ra];
  yB = red[parity][0][8 + ra];
  for (int w = 1; w < W; ++w) {
    yA += red[parity][w][ra];
    yB += red[parity][w][8 + ra];
  }
  return true;
}

// A persistent grid over the matrix's 16-row tiles for token blockIdx.y: every block stages the token's
// activation once (each wave its own half-groups, as rowpair_partial does), then walks the tiles
// blockIdx.x, + gridDim.x, ... with the next tile's code words in flight while the current one is reduced
// and stored.  Each row's arithmetic and summation order are those of rowpair_partial + block_sum, so the
// results equal the expert kernels' row routine bit for bit.
template <int NBW, typename XT, bool SB_BF16>
__global__ __launch_bounds__(64 * kMaxWaves) void matrix_gemv_kernel(MatArgs m, int n_tiles) {
  extern __shared__ __align__(16) uint32_t lds[];
  __shared__ float red[2][kMaxWaves][16];
  const int W = blockDim.x >> 6, wave = threadIdx.x >> 6, lane = threadIdx.x & 63, ra = lane >> 3;
  const int C = m.K / 32, nit = (C + kLanesPerRow - 1) / kLanesPerRow, t = blockIdx.y;
  const Stage st{lds, reinterpret_cast<float4*>(lds + C * kHgStride)};
  const XT* x = reinterpret_cast<const XT*>(m.x) + (int64_t)t * m.K;
  int tile = blockIdx.x;
  TileRegs<NBW, SB_BF16> g0, g1;
  if (tile < n_tiles) load_tile<NBW, SB_BF16>(m, tile, g0);
  // stage this wave's half-groups (slot mapping of rowpair_partial) while the first tile is in flight
  constexpr int kPasses = (NBW * 32 + 63) / 64;
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    const int s = lane + 64 * p, mi = s >> 5, jj = (s >> 2) & 7, q = s & 3;
    const int it = wave + W * mi;
    const int hg = it * kLanesPerRow + jj;
    const bool live = mi < NBW && it < nit && hg < C;
    XWord<XT> xw;
    float v[8];
    if (live) {
      load_word<XT>(x, hg, q, xw);
      word_to_f32<XT>(xw, v);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = 0.f;
    }
    stage_word(v, live, hg, q, st);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  float* y = m.y + (int64_t)t * m.N;
  int parity = 0;
  auto finish = [&](const TileRegs<NBW, SB_BF16>& g, int tl) {
    float yA, yB;
    tile_dot<NBW, SB_BF16>(m, g, st, yA, yB);
    if (tile_sum(yA, yB, red, parity)) {
      const int rA = tl * 16 + ra, rB = rA + 8;
      if (rA < m.N) y[rA] = yA;
      if (rB < m.N) y[rB] = yB;
    }
    parity ^= 1;
  };
  // two register sets alternate: the next tile loads into one while the other is computed
  while (tile < n_tiles) {
    const int t1 = tile + (int)gridDim.x;
    if (t1 < n_tiles) load_tile<NBW, SB_BF16>(m, t1, g1);
    finish(g0, tile);
    if (t1 >= n_tiles) break;
    const int t2 = t1 + (int)gridDim.x;
    if (t2 < n_tiles) load_tile<NBW, SB_BF16>(m, t2, g0);
    finish(g1, t1);
    tile = t2;
  }
}

}  // namespace
}  // namespace moeq4

extern "C" moe_status q4_gemv(const void* x_dev, moe_dtype x_dtype, int32_t T, const uint32_t* codes_dev,
                              const void* sb_dev, moe_dtype sb_dtype, int32_t N, int32_t K, float* y_dev, void* stream) {
  const char* who = "q4_gemv";
  if (!x_dev || !codes_dev || !sb_dev || !y_dev) return fail(MOE_ERR_INVALID_ARG, "%s: NULL pointer", who);
  if (x_dtype != MOE_F32 && x_dtype != MOE_BF16) return fail(MOE_ERR_INVALID_ARG, "%s: bad x_dtype", who);
  if (sb_dtype != MOE_F32 && sb_dtype != MOE_BF16) return fail(MOE_ERR_INVALID_ARG, "%s: bad sb_dtype", who);
  if (T < 1 || T > 65535 || N < 1 || K < 64 || K % 64 != 0 || K > kMaxK)
    return fail(MOE_ERR_INVALID_ARG, "%s: T=%d N=%d K=%d (need 1 <= T <= 65535, N >= 1, K a multiple of 64, <= %d)",
                who, T, N, K, kMaxK);
  if (!aligned(x_dev, 16) || !aligned(codes_dev, 16) || !aligned(sb_dev, 8))
    return fail(MOE_ERR_INVALID_ARG, "%s: x and codes must be 16-byte aligned, sb 8-byte aligned", who);
  const int nit = iterations(K);
  const int waves = nit < kMaxWaves ? nit : kMaxWaves;
  const int nbw = (nit + waves - 1) / waves;
  const int sb_elem = sb_dtype == MOE_BF16 ? 2 : 4;
  const moeq4::MatArgs m{x_dev, reinterpret_cast<const char*>(codes_dev), reinterpret_cast<const char*>(sb_dev),
                         y_dev, N, K, (K / 64) * 2 * sb_elem};
  const int n_tiles = (N + 15) / 16;
  int dev = 0, cus = 0;
  (void)hipGetDevice(&dev);
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 256;
  const int per_cu = kGemvBlocksPerCu;
  const dim3 grid(n_tiles < cus * per_cu ? n_tiles : cus * per_cu, T), block(64 * waves);
  const size_t lds = lds_bytes(K);
  hipStream_t s = as_stream(stream);
  return dispatch_nbw(nbw, [&](auto nb) {
    constexpr int NB = decltype(nb)::value;
    if (x_dtype == MOE_BF16) {
      if (sb_dtype == MOE_BF16) hipLaunchKernelGGL((moeq4::matrix_gemv_kernel<NB, uint16_t, true>), grid, block, lds, s, m, n_tiles);
      else hipLaunchKernelGGL((moeq4::matrix_gemv_kernel<NB, uint16_t, false>), grid, block, lds, s, m, n_tiles);
    } else {
      if (sb_dtype == MOE_BF16) hipLaunchKernelGGL((moeq4::matrix_gemv_kernel<NB, float, true>), grid, block, lds, s, m, n_tiles);
      else hipLaunchKernelGGL((moeq4::matrix_gemv_kernel<NB, float, false>), grid, block, lds, s, m, n_tiles);
    }
    return check_launch(who);
  });
}
