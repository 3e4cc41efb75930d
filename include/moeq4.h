/*
 * moeq4.h — C ABI of libmoeq4.so: the per-token Mixture-of-Experts decode step on MI355X (gfx950).
 *
 * The step, as the pages describe it for Gemma 4 26B-A4B: per token and per layer an 8-bit router picks
 * the top 8 of 128 experts, the selected experts run as quantized matrix-vector products on 4-bit
 * MLX-style affine weights, a shared expert runs for every token, and the two branches are combined;
 * routed experts live in a small per-layer LFU cache fed from slower storage.
 *
 * Pages cited (by title):
 *   [G26]   "Gemma 4 26B : Comment faire tourner un LLM en 2 Go de RAM" (lhusser.fr)
 *   [LEAF]  romain.leaflet.pub article on TurboFieldfare (untitled page)
 *   [DAILY] "TurboFieldfare" event page, daily.steinslab.io
 *   [REMIO] "TurboFieldfare exécute Mac Gemma 4 26B dans 2 Go, mais la vitesse du SSD devient le compromis"
 *   [DEVT]  "Een model met 26 miljard parameters uitvoeren in twee gigabyte geheugen op een gewone Mac"
 *
 * Conventions for every entry point:
 *   - Pointers named *_dev are device pointers (hipMalloc'd or torch CUDA tensors); *_host are host pointers.
 *   - The caller owns every buffer.  The library allocates no device memory inside these calls; scratch
 *     space comes from a caller workspace sized by the matching *_workspace_bytes() query.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Compute calls only enqueue work.
 *   - Arguments are validated on the host before anything is enqueued; a non-MOE_OK status means nothing
 *     was enqueued (except MOE_ERR_HIP, raised by a failed launch).  moe_last_error() then returns a
 *     thread-local message.  Device-side data errors (an expert id outside the pool) cannot be checked on
 *     the host: the affected outputs are written as NaN.
 *   - Results are deterministic: fixed reduction orders, no floating-point atomics.
 */
#ifndef MOEQ4_H
#define MOEQ4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,   /* null pointer, bad size, bad enum */
  MOE_ERR_UNSUPPORTED = 2,   /* shape outside what the kernels support (see each call) */
  MOE_ERR_OUT_OF_RANGE = 3,  /* a host-visible id or index is outside its range */
  MOE_ERR_CACHE = 4,         /* cache policy refused the request (duplicate ids, more ids than slots) */
  MOE_ERR_HIP = 5            /* a HIP runtime call or launch failed */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Gated activation of the expert FFN.  The pages name no activation; GELU (tanh form) is the reading for
 * Gemma-style experts, SiLU the common alternative. */
typedef enum { MOE_ACT_GELU_TANH = 0, MOE_ACT_SILU = 1 } moe_act;

/* ---------------------------------------------------------------------------------------------------
 * Expert record format ([REMIO] "L'affirmation des 2 Go fait de la bande passante SSD la nouvelle
 * contrainte": experts in MLX affine 4-bit layout; [DAILY] "1. Compression par 4").
 *
 * One expert (hidden size d, FFN width F) is one contiguous record — the unit the expert cache copies.
 * Sections, each starting on a 256-byte boundary, record size rounded up to 256 bytes:
 *   gate_up codes   uint32 [2F][d/8]       rows 0..F-1 = gate matrix, rows F..2F-1 = up matrix
 *   gate_up scale/bias  sb [2F][d/64][2]   (scale, bias) per group of 64 input columns
 *   down codes      uint32 [d][F/8]
 *   down scale/bias     sb [d][F/64][2]
 * Code of column c of a row: word c/8 of that row, bits 4*(c%8) .. 4*(c%8)+3 (low nibble first).
 * Dequantized weight: w = scale * code + bias, code in 0..15.  sb is bf16 or fp32 (moe_dtype).
 * d and F must be multiples of 64.
 * ------------------------------------------------------------------------------------------------- */

/* Byte size of one expert record; 0 if d or F is not a positive multiple of 64 or sb_dtype is invalid. */
size_t moe_record_bytes(int32_t d, int32_t F, moe_dtype sb_dtype);

/* Byte offsets of the four sections (gate_up codes, gate_up s/b, down codes, down s/b) into offsets[4]. */
moe_status moe_record_layout(int32_t d, int32_t F, moe_dtype sb_dtype, size_t offsets[4]);

/* A pool of expert records in device memory: record i at base + i * record_bytes. */
typedef struct {
  const void* base_dev;    /* device pointer to record 0 (256-byte aligned) */
  size_t record_bytes;     /* stride between records, >= moe_record_bytes(d, F, sb_dtype), multiple of 256 */
  int32_t n_records;       /* experts in the pool (or cache slots) */
  int32_t d;               /* hidden size, multiple of 64, <= 8192 */
  int32_t F;               /* FFN width, multiple of 64, <= 8192 */
  moe_dtype sb_dtype;      /* scale/bias dtype */
} moe_q4_pool;

/* ---------------------------------------------------------------------------------------------------
 * q4_quantize — encode fp32 weights W [N][K] (row-major, device) into 4-bit codes and scale/bias.
 * The pages list quantization among the engine's own GPU kernels ([DEVT] "Geen afhankelijkheden van
 * llama.cpp en MLX").  Min-max per group of 64 along K (the plainest affine reading):
 *   scale = (max - min)/15 (fp32), bias = min, both rounded to sb_dtype (round-to-nearest-even);
 *   code = clamp(round_half_even((w - bias) / scale), 0, 15) in IEEE fp32; code = 0 when scale == 0.
 * codes_dev: uint32 [N][K/8]; sb_dev: sb_dtype [N][K/64][2].  K % 64 == 0, N >= 1.
 * ------------------------------------------------------------------------------------------------- */
moe_status q4_quantize(const float* w_dev, int32_t N, int32_t K, moe_dtype sb_dtype,
                       uint32_t* codes_dev, void* sb_dev, void* stream);

/* Encode one expert record from fp32 gate_up [2F][d] and down [d][F] weights (device) into record_dev
 * (moe_record_bytes(d, F, sb_dtype) bytes, 256-byte aligned).  Padding bytes are left untouched. */
moe_status q4_pack_expert(const float* w_gate_up_dev, const float* w_down_dev, int32_t d, int32_t F,
                          moe_dtype sb_dtype, void* record_dev, void* stream);

/* ---------------------------------------------------------------------------------------------------
 * q4_gemv — one 4-bit affine matrix times T vectors, no activation ([LEAF] "Du code sur-mesure sans
 * dépendance externe": fused dequantize + matrix-vector kernels; [REMIO] "L'affirmation des 2 Go fait de
 * la bande passante SSD la nouvelle contrainte": MLX affine 4-bit weights):
 *   y[t][r] = sum_c (scale[r][c/64] * code[r][c] + bias[r][c/64]) * x[t][c]        fp32
 * Uses the row routine of q4_expert_gemv (same dequantization, accumulation and summation order), so a
 * result equals that of the same matrix inside an expert record; with x = e_j it is column j of the
 * dequantized matrix.
 * x_dev: x_dtype [T][K] (fp32 or bf16), 16-byte aligned; codes_dev: uint32 [N][K/8], 16-byte aligned,
 * code of column c in word c/8, bits 4*(c%8) (q4_quantize's output); sb_dev: sb_dtype [N][K/64][2]
 * (scale, bias), 8-byte aligned; y_dev: fp32 [T][N].  All device memory owned by the caller.
 * Limits: 1 <= T <= 65535, N >= 1, K a multiple of 64 with 64 <= K <= 8192 (MOE_ERR_INVALID_ARG otherwise;
 * nothing is launched).  Asynchronous on `stream`.
 * ------------------------------------------------------------------------------------------------- */
moe_status q4_gemv(const void* x_dev, moe_dtype x_dtype, int32_t T, const uint32_t* codes_dev, const void* sb_dev,
                   moe_dtype sb_dtype, int32_t N, int32_t K, float* y_dev, void* stream);

/* ---------------------------------------------------------------------------------------------------
 * moe_rmsnorm — u[t] = (x[t] * gamma) * (1 / sqrt(mean(x[t]^2) + eps)), fp32 math, rounded to out_dtype
 * (RNE).  The sum of squares runs in one fixed order (each thread an fma chain over its 8-value pieces
 * (thread + 256 p) * 8, the wavefront sums, then the four wavefronts' sums in order), the order of
 * moe_norm_router_topk and of the single-launch layer, so all three produce the same u.
 * The pages list a normalisation (RMSNorm) kernel ([LEAF] "Du code sur-mesure sans dépendance externe";
 * [DEVT] "Geen afhankelijkheden van llama.cpp en MLX"); it precedes each MoE block in the stacked decode.
 * x_dev: x_dtype [T][d]; gamma_dev: fp32 [d]; out_dev: out_dtype [T][d].  d % 8 == 0, d <= 16384, T >= 1;
 * x and gamma 16-byte aligned.
 * ------------------------------------------------------------------------------------------------- */
moe_status moe_rmsnorm(const void* x_dev, moe_dtype x_dtype, const float* gamma_dev, float eps,
                       int32_t T, int32_t d, void* out_dev, moe_dtype out_dtype, void* stream);

/* ---------------------------------------------------------------------------------------------------
 * moe_router_topk — the 8-bit router and top-k selection ([G26] "Le pipeline de traitement": an 8-bit
 * router picks the 8 experts a token needs; [DAILY] "L'atout caché des modèles MoE": 8 of 128 active).
 *   logit[t][e] = row_scale[e] * sum_j w[e][j] * x[t][j]      (int8 x activation, fp32 accumulate)
 *   ids[t]      = the k largest logits, descending; equal logits -> lower expert id first
 *   weights[t]  = softmax of logit[t][ids[t][i]] over i < k   (sums to 1)
 * With forced_ids_dev != NULL the selection is skipped: ids are copied from forced_ids_dev [T][k] (a routing
 * trace) and weights are the softmax of the logits at those ids, in that order.
 * x_dev: x_dtype [T][d]; w_dev: int8 [E][d] row-major; row_scale_dev: fp32 [E];
 * ids_dev: int32 [T][k]; weights_dev: fp32 [T][k]; logits_dev: fp32 [T][E] or NULL.
 * Limits: 1 <= k <= min(E, 32), E <= 1024, d % 16 == 0, d <= 8192.
 * Workspace: moe_router_workspace_bytes(T, E) bytes of device memory that must be ZERO before its first
 * use; every completed call leaves it zero again, so one workspace serves any number of calls ordered
 * on one stream (and graph replays).  Calls that overlap in time need separate workspaces.
 * ------------------------------------------------------------------------------------------------- */
size_t moe_router_workspace_bytes(int32_t T, int32_t E);
moe_status moe_router_topk(const void* x_dev, moe_dtype x_dtype, int32_t T, int32_t d,
                           const int8_t* w_dev, const float* row_scale_dev, int32_t E, int32_t k,
                           const int32_t* forced_ids_dev, int32_t* ids_dev, float* weights_dev,
                           float* logits_dev, void* workspace_dev, size_t workspace_bytes, void* stream);

/* moe_norm_router_topk — moe_rmsnorm fused into moe_router_topk for the stacked decode, where the norm
 * output feeds both the router and the expert GEMVs ([LEAF] "Du code sur-mesure sans dépendance externe":
 * the RMSNorm and router kernels of the engine).  Every router block normalizes x itself:
 *   u[t] = round_x( x[t] / sqrt(mean(x[t]^2) + eps) * gamma )      (fp32 math, RNE to x_dtype)
 * and routes u[t] exactly as moe_router_topk routes its x; block 0 also writes u to u_dev (x_dtype [T][d],
 * 16-byte aligned) for the expert GEMVs.  The norm is moe_rmsnorm's, in the same order: u equals
 * moe_rmsnorm's output bit for bit, and a token's logits, ids and weights do not depend on T.  gamma_dev:
 * fp32 [d], 16-byte aligned; eps >= 0.  Other arguments, limits and the workspace rule as moe_router_topk. */
moe_status moe_norm_router_topk(const void* x_dev, moe_dtype x_dtype, const float* gamma_dev, float eps, int32_t T,
                                int32_t d, const int8_t* w_dev, const float* row_scale_dev, int32_t E, int32_t k,
                                const int32_t* forced_ids_dev, int32_t* ids_dev, float* weights_dev,
                                float* logits_dev, void* u_dev, void* workspace_dev, size_t workspace_bytes,
                                void* stream);

/* ---------------------------------------------------------------------------------------------------
 * q4_expert_gemv — the selected experts' FFNs and the shared expert's FFN on 4-bit affine weights
 * ([LEAF] "Du code sur-mesure sans dépendance externe": quantized matrix-vector kernels; [REMIO]
 * "Mac Gemma 4 26B tient en mémoire...": one shared expert for every token besides the 8 routed ones).
 * For each token t and each i < k with e = ids[t][i] (an index into `routed`):
 *   y_routed[t][i] = W_down,e ( act(W_gate,e x[t]) * (W_up,e x[t]) )          fp32 [d]
 * and, if shared != NULL (a pool whose record 0 is the shared expert, width shared->F):
 *   y_shared[t]    = W_down,s ( act(W_gate,s x[t]) * (W_up,s x[t]) )          fp32 [d]
 * Weights are dequantized on the fly; accumulation is fp32.  Both experts kinds run in the same launches.
 * x_dev: x_dtype [T][d]; ids_dev: int32 [T][k] (device, e.g. straight from moe_router_topk or cache slot
 * ids from expert_cache_stage); y_routed_dev: fp32 [T][k][d]; y_shared_dev: fp32 [T][d] (needed iff shared).
 * T == 1 is the decode GEMV (vector ALUs, dot2).  T > 1 first groups the T*k (token, slot) pairs by
 * expert on the device (moe_group_pairs, below), then streams each selected expert's rows once for all of
 * its tokens, and the shared expert's rows once for all T tokens, as small dense products on the matrix
 * cores (fp16 inputs: codes exactly, activations scaled by a power of two per token row; fp32 sums).
 * The two paths round differently: a token's T > 1 result matches its T == 1 result within the fp32/fp16
 * rounding of the activations (tested to max relative error 1e-2 with the oracle), not bit for bit.
 * Limits: k <= 32; routed and shared share d; routed may be NULL (k == 0) to run only the shared expert;
 * with T > 1 the routed pool has at most 4096 records, and T*k rows (T without routed experts) of the longest
 * row length among d, F and S take less than 2 GiB in fp16 (MOE_ERR_UNSUPPORTED otherwise).
 * Workspace: q4_expert_gemv_workspace_bytes(...) bytes of device memory (contents need no initial value).
 * An id outside [0, routed->n_records) makes that expert's y_routed row NaN.
 * ------------------------------------------------------------------------------------------------- */
size_t q4_expert_gemv_workspace_bytes(const moe_q4_pool* routed, int32_t k, const moe_q4_pool* shared, int32_t T);
moe_status q4_expert_gemv(const moe_q4_pool* routed, const int32_t* ids_dev, int32_t k,
                          const moe_q4_pool* shared, const void* x_dev, moe_dtype x_dtype, int32_t T,
                          moe_act act, float* y_routed_dev, float* y_shared_dev,
                          void* workspace_dev, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------------------------
 * moe_group_pairs — the batch's (token, slot) pairs grouped by expert, the first step of a T > 1
 * q4_expert_gemv ([G26] "Le pipeline de traitement": a prompt's tokens processed together share each
 * expert's weights).  Pair p = t*k + i carries expert ids[t][i]; ids outside [0, n_valid) form one bucket
 * after all valid experts.  The pairs are sorted stably by bucket:
 *   perm[0 .. T*k)      pair indices, bucket-ascending, pair-ascending within a bucket
 *   groups[j] = (bucket, first index into perm, count, 0) for the non-empty buckets, bucket-ascending
 *   *n_groups           number of non-empty buckets (<= moe_group_pairs_max_groups(T, k, n_valid))
 * ids_dev: int32 [T][k]; n_groups_dev: int32 [1]; groups_dev: int32 [max_groups][4], 16-byte aligned;
 * perm_dev: int32 [T*k] (all device).  Limits: 1 <= T <= 65535, 1 <= k <= 32, 1 <= n_valid <= 4096.
 * One block; deterministic (integer work only).
 * ------------------------------------------------------------------------------------------------- */
int32_t moe_group_pairs_max_groups(int32_t T, int32_t k, int32_t n_valid);
moe_status moe_group_pairs(const int32_t* ids_dev, int32_t T, int32_t k, int32_t n_valid, int32_t* n_groups_dev,
                           int32_t* groups_dev, int32_t* perm_dev, void* stream);

/* The two halves of q4_expert_gemv, for callers that schedule them separately (and for timing one
 * launch).  q4_expert_gate_up computes h = act(W_gate x) * (W_up x) for the routed and shared experts
 * into the workspace (fp32 [T][k][F] then [T][S]); q4_expert_down reads h from the same workspace and
 * writes y_routed / y_shared.  Between the two calls the caller must pass the same pools, ids, k, T and
 * workspace, in stream order.  Same limits and errors as q4_expert_gemv. */
moe_status q4_expert_gate_up(const moe_q4_pool* routed, const int32_t* ids_dev, int32_t k, const moe_q4_pool* shared,
                             const void* x_dev, moe_dtype x_dtype, int32_t T, moe_act act, void* workspace_dev,
                             size_t workspace_bytes, void* stream);
moe_status q4_expert_down(const moe_q4_pool* routed, const int32_t* ids_dev, int32_t k, const moe_q4_pool* shared,
                          int32_t T, float* y_routed_dev, float* y_shared_dev, void* workspace_dev,
                          size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------------------------
 * moe_combine — merge the branches ([G26] "Concurrence pour masquer la latence": the shared-expert output
 * and the routed outputs are combined once the routed experts are in; [REMIO] "L'affirmation des 2 Go...").
 *   out[t] = round_out( sum_{i<k} weights[t][i] * y_routed[t][i] + y_shared[t] + residual[t] )
 * summed in fp32 in the order i = 0..k-1, then shared, then residual; y_shared and residual may be NULL.
 * y_routed_dev: fp32 [T][k][d]; weights_dev: fp32 [T][k]; y_shared_dev: fp32 [T][d]; residual_dev:
 * residual_dtype [T][d]; out_dev: out_dtype [T][d] (may alias residual_dev when the dtypes match).
 * ------------------------------------------------------------------------------------------------- */
moe_status moe_combine(const float* y_routed_dev, const float* weights_dev, const float* y_shared_dev,
                       const void* residual_dev, moe_dtype residual_dtype, int32_t T, int32_t k, int32_t d,
                       void* out_dev, moe_dtype out_dtype, void* stream);

/* q4_expert_gemv_combine — q4_expert_gemv followed by moe_combine.  With T == 1 in two launches instead of
 * three: the down GEMV's blocks publish their rows and the last block to finish a 16-row tile applies the
 * combine to it ([G26] "Concurrence pour masquer la latence": routed and shared outputs merged once all
 * are in); with T > 1 the grouped down products and the combine are separate launches (per-tile tickets
 * for every token would cost more than the launch they save).  Computes, for every token t,
 *   out[t] = round_out( sum_{i<k} weights[t][i] * y_routed[t][i] + y_shared[t] + residual[t] )
 * with y_routed / y_shared as q4_expert_gemv defines them, summed in the same order as moe_combine; the
 * result is bit-identical to q4_expert_gemv + moe_combine on the same inputs.  y_routed and y_shared stay
 * internal (in the workspace).  weights_dev: fp32 [T][k] (e.g. from moe_router_topk; may be NULL iff
 * k == 0); residual_dev: residual_dtype [T][d] or NULL; out_dev: out_dtype [T][d] (may alias residual_dev
 * when the dtypes match).  Pools, ids, x, act, limits and errors as q4_expert_gemv.
 * Workspace: q4_expert_gemv_combine_workspace_bytes(...) bytes of device memory, 256-byte aligned, that
 * must be ZERO before its first use (its last T*d/16 words are per-tile counters that every completed
 * call leaves zero again).  Calls that overlap in time need separate workspaces. */
size_t q4_expert_gemv_combine_workspace_bytes(const moe_q4_pool* routed, int32_t k, const moe_q4_pool* shared,
                                              int32_t T);
moe_status q4_expert_gemv_combine(const moe_q4_pool* routed, const int32_t* ids_dev, int32_t k,
                                  const moe_q4_pool* shared, const void* x_dev, moe_dtype x_dtype, int32_t T,
                                  moe_act act, const float* weights_dev, const void* residual_dev,
                                  moe_dtype residual_dtype, void* out_dev, moe_dtype out_dtype,
                                  void* workspace_dev, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------------------------
 * moe_decode_layer — one whole MoE layer of batch-1 decode in a single launch: RMSNorm, 8-bit router and
 * top-k, the k selected experts and the shared expert, combine and residual ([G26] "Le pipeline de
 * traitement"; [G26] "Concurrence pour masquer la latence": the shared expert runs without waiting for the
 * routing, the branches are merged once the routed experts are in).  For the single token x:
 *   u       = gamma ? round_x((x * gamma) * rsqrt(mean(x^2) + eps)) : x
 *   logits  = row_scale[e] * (w[e] . u);  ids = top-k (or forced ids);  weights = softmax over ids
 *   out     = round_x( sum_i weights[i] * FFN_{ids[i]}(u) + FFN_shared(u) + (residual ? x : 0) )
 * with the selection rule, weights and expert arithmetic of moe_router_topk / q4_expert_gemv.  u equals
 * moe_rmsnorm's bit for bit (the same summation order); the router's dot products use an order of their own,
 * so the logits may differ from moe_router_topk's in the last bits.
 * x_dev, out_dev: x_dtype [d] (16-byte aligned, must not alias); gamma_dev: fp32 [d] or NULL;
 * router as moe_router_topk; forced_ids_dev: int32 [k] or NULL; routed: pool of experts, indexed by the
 * selected ids, or by gemv_ids_dev[i] (int32 [k], e.g. cache slots from expert_cache_stage) when that is
 * non-NULL; shared: pool whose record 0 is the shared expert, or NULL; ids_dev / weights_dev / logits_dev:
 * optional outputs (int32 [k], fp32 [k], fp32 [E]); u_dev: optional output x_dtype [d], the normalized
 * activation u that the router and the experts consumed (must not alias x or out).
 * Limits: d <= 4096, shared width <= 4096, routed F <= 1024, E <= 256, 1 <= k <= min(E, 32).
 * Workspace: moe_decode_layer_workspace_bytes(d, E, k, F, S) bytes (S = 0 without shared expert), 256-byte
 * aligned, ZERO before its first use, and used with one shape (d, E, k, F, S and shared or not).  Its first
 * moe_decode_layer_sync_bytes(d, k) bytes hold the counters and flags the blocks synchronise with: every
 * completed call leaves each counter zero and each flag zero or at the number of calls made on the
 * workspace; 32-bit word 0 is a sticky error flag, nonzero if a wait inside the kernel ran out (the results
 * of that call are invalid; zero the workspace before reusing it).  After them come one call counter per
 * block of the grid, each advanced by one per call (flags and the values published during a call carry
 * the call number, so nothing needs clearing between calls), and the call's intermediate values.  Calls
 * that overlap in time need separate workspaces.
 * ------------------------------------------------------------------------------------------------- */
size_t moe_decode_layer_workspace_bytes(int32_t d, int32_t E, int32_t k, int32_t F, int32_t S);
size_t moe_decode_layer_sync_bytes(int32_t d, int32_t k);
moe_status moe_decode_layer(const void* x_dev, moe_dtype x_dtype, const float* gamma_dev, float eps, int32_t residual,
                            const int8_t* router_w_dev, const float* router_scale_dev, int32_t E, int32_t k,
                            const int32_t* forced_ids_dev, const moe_q4_pool* routed, const int32_t* gemv_ids_dev,
                            const moe_q4_pool* shared, moe_act act, int32_t* ids_dev, float* weights_dev,
                            float* logits_dev, void* u_dev, void* out_dev, void* workspace_dev,
                            size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------------------------
 * moe_decode_layer_part — moe_decode_layer as two launches, so that the routed experts' weights can arrive
 * in between ([G26] "Concurrence pour masquer la latence": the shared expert computes while the missing
 * experts are fetched, the two branches are merged once they are in; [DAILY] "3. Cache intelligent +
 * Chevauchement temporel").  part 1 runs the router (logits, top-k) and the whole shared expert and leaves
 * them in the workspace; part 2 runs the routed experts and the combine (with the residual) and writes
 * out, ids and weights.  Arguments, limits and errors as moe_decode_layer; shared must not be NULL; logits
 * and u are written by part 1, ids, weights and out by part 2.  A call of part 1 followed by part 2 with the
 * same arguments on the same workspace (part 2 ordered after part 1, e.g. on the same stream) equals one
 * moe_decode_layer call bit for bit; a workspace may alternate such pairs with whole calls, but every part 1
 * must be followed by its part 2 before anything else uses the workspace.  The routed pool and gemv ids
 * are read only by part 2: an expert cache may fill its slots between the parts (expert_cache_stage's
 * ready event waited on before part 2).
 * ------------------------------------------------------------------------------------------------- */
moe_status moe_decode_layer_part(int32_t part, const void* x_dev, moe_dtype x_dtype, const float* gamma_dev,
                                 float eps, int32_t residual, const int8_t* router_w_dev,
                                 const float* router_scale_dev, int32_t E, int32_t k, const int32_t* forced_ids_dev,
                                 const moe_q4_pool* routed, const int32_t* gemv_ids_dev, const moe_q4_pool* shared,
                                 moe_act act, int32_t* ids_dev, float* weights_dev, float* logits_dev, void* u_dev,
                                 void* out_dev, void* workspace_dev, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------------------------
 * moe_decode_layer_noalloc — moe_decode_layer for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the same computation, kernels
 * and results, with the workspace in a device array the library holds instead of a caller workspace.
 * Arguments, outputs, limits and errors as moe_decode_layer, without workspace_dev / workspace_bytes, and:
 *   status_dev: optional uint32 (device, caller-owned, 4-byte aligned) into which the call ORs 1 if a wait
 *   inside the kernel ran out (the results of that call are then invalid); NULL = not reported.
 * The library's array holds MOE_DECODE_LAYER_NOALLOC_MAX_BYTES (1 MiB) per GPU, allocated with the library's
 * code object and kept until the process ends; a shape whose moe_decode_layer_workspace_bytes(d, E, k, F, S)
 * exceeds it is rejected with MOE_ERR_UNSUPPORTED before anything is enqueued (d = 2816, 128 experts, top-8,
 * F = 704, S = 2816 needs about 317 KB).  Each call first clears the part of the array its shape uses (a
 * fill kernel on `stream`, no memset node), then launches the layer kernel, so consecutive calls may use
 * different shapes.  Every call on a GPU shares that GPU's array: calls that overlap in time on one GPU (on
 * different streams, or from several threads) race and give undefined results.  The call allocates nothing:
 * no hipMalloc, hipFree or allocating library routine; the array's device address is looked up once per
 * device with hipGetSymbolAddress on the first call made with that device current.
 * ------------------------------------------------------------------------------------------------- */
#define MOE_DECODE_LAYER_NOALLOC_MAX_BYTES (1u << 20)
moe_status moe_decode_layer_noalloc(const void* x_dev, moe_dtype x_dtype, const float* gamma_dev, float eps,
                                    int32_t residual, const int8_t* router_w_dev, const float* router_scale_dev,
                                    int32_t E, int32_t k, const int32_t* forced_ids_dev, const moe_q4_pool* routed,
                                    const int32_t* gemv_ids_dev, const moe_q4_pool* shared, moe_act act,
                                    int32_t* ids_dev, float* weights_dev, float* logits_dev, void* u_dev,
                                    void* out_dev, uint32_t* status_dev, void* stream);

/* ---------------------------------------------------------------------------------------------------
 * moe_decode_stack — n_layers consecutive layers of moe_decode_layer for one token in a single launch
 * (the stacked decode: RMSNorm and the MoE block per layer, residual stream between them).  Layer l + 1's
 * blocks load their router rows and shared-expert weights while layer l finishes, then wait for layer l's
 * output; intermediate activations stay in the workspace in x_dtype, so the result equals n_layers chained
 * moe_decode_layer calls bit for bit.
 * layers_host: host array of n_layers descriptors (copied into the launch; the device buffers they point to
 * must stay valid until the work completes).  routed / shared: the pools' shape (d, F, record_bytes,
 * n_records, sb_dtype; base_dev is ignored, every layer gives its own); shared may be NULL.
 * x_dev: x_dtype [d] input of layer 0; out_dev: x_dtype [d] output of the last layer (must not alias x_dev).
 * Per layer: router as moe_router_topk; gamma_dev fp32 [d] or NULL (no norm); ids/weights/logits/u optional
 * outputs (u: the layer's normalized activation, x_dtype [d]).  Limits as moe_decode_layer, and 1 <= n_layers <= 32.
 * Workspace: moe_decode_stack_workspace_bytes(...) bytes, 256-byte aligned, ZERO before first use; the
 * region of layer l is moe_decode_layer_workspace_bytes(d, E, k, F, S) bytes at offset l times that size,
 * laid out as moe_decode_layer's (word 0 of the whole workspace is the sticky error flag), with the same
 * state after every completed call: counters zero, flags zero or at the number of calls made.  A workspace
 * is bound to one n_layers and one shape for its life: every block of every layer counts the calls made on
 * it and waits for the values tagged with that count, so a call with another n_layers, or a
 * moe_decode_layer call on one layer's region, leaves the counts unequal and the next calls' waits run out
 * (the sticky flag is set; nothing hangs).  Zero it before using it for another n_layers or shape.
 * ------------------------------------------------------------------------------------------------- */
typedef struct {
  const int8_t* router_w_dev;      /* int8 [E][d] */
  const float* router_scale_dev;   /* fp32 [E] */
  const float* gamma_dev;          /* fp32 [d] or NULL */
  const void* routed_base_dev;     /* this layer's routed pool (n_records records) */
  const void* shared_base_dev;     /* this layer's shared expert record, or NULL without shared pool */
  int32_t* ids_dev;                /* int32 [k] or NULL */
  float* weights_dev;              /* fp32 [k] or NULL */
  float* logits_dev;               /* fp32 [E] or NULL */
  void* u_dev;                     /* x_dtype [d] or NULL: the normalized activation of this layer */
} moe_stack_layer;

size_t moe_decode_stack_workspace_bytes(int32_t n_layers, int32_t d, int32_t E, int32_t k, int32_t F, int32_t S);
moe_status moe_decode_stack(const moe_stack_layer* layers_host, int32_t n_layers, const void* x_dev,
                            moe_dtype x_dtype, float eps, int32_t residual, int32_t E, int32_t k,
                            const moe_q4_pool* routed, const moe_q4_pool* shared, moe_act act, void* out_dev,
                            void* workspace_dev, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------------------------
 * Expert cache — 16-slot-per-layer least-frequently-used cache of expert records ([DAILY] "Cache
 * d'experts"; [DEVT] "Wat is de belangrijkste architectuurtruuc"; [REMIO] "Mac Gemma 4 26B tient en
 * mémoire..."), fed on demand from slower memory while the shared expert computes ([G26] "Concurrence
 * pour masquer la latence").  Here the slow tier is pinned host memory and the fast tier is HBM; misses
 * are copied with hipMemcpyAsync on a caller-provided copy stream.
 *
 * Policy (readings of "LFU"): in-cache LFU — a slot's use count starts at 1 on load and is forgotten on
 * eviction; a request first marks every requested expert already resident (count += 1, last use = now)
 * and pins it for the request; each miss, in request order, takes the lowest empty slot, else evicts the
 * unpinned slot with the smallest (count, last use, slot index).  The cache starts empty.
 *
 * moe_expert_cache_create: n_layers x n_slots slots of record_bytes each.  host_pool_host[l] points to
 * layer l's n_experts records in pinned host memory (hipHostMalloc); slot_pool_dev[l] points to layer l's
 * n_slots slot records in device memory.  Both arrays of pointers are copied; the memory stays the
 * caller's and must outlive the cache.  flags: 0, or MOE_CACHE_HOST_ONLY (slot pools and slot-id outputs
 * are host memory, copies are memcpy, streams/events are ignored: the policy without a GPU).
 * ------------------------------------------------------------------------------------------------- */
typedef struct moe_expert_cache moe_expert_cache;
#define MOE_CACHE_HOST_ONLY 1u

moe_status moe_expert_cache_create(int32_t n_layers, int32_t n_experts, int32_t n_slots, size_t record_bytes,
                                   const void* const* host_pool_host, void* const* slot_pool_dev,
                                   uint32_t flags, moe_expert_cache** out);
void moe_expert_cache_destroy(moe_expert_cache* cache);

/* expert_cache_stage — make the n experts ids_host[0..n) of `layer` resident.
 * Runs the policy on the host, enqueues one hipMemcpyAsync per miss (pinned host record -> HBM slot) on
 * copy_stream after waiting on wait_event (if not NULL: the event recorded after the last kernel that read
 * this layer's slots, so a slot is never overwritten while it is read; an event already complete at the
 * call is not waited on, the copies then start without a device-side wait), writes the slot index of each id
 * to slot_ids_dev (int32 [n], copied on copy_stream), then records ready_event (if not NULL) on
 * copy_stream.  Kernels that read the slots must wait on ready_event.
 * Errors: duplicate ids or n > n_slots -> MOE_ERR_CACHE; id outside [0, n_experts) -> MOE_ERR_OUT_OF_RANGE;
 * a failed copy -> MOE_ERR_HIP.  On any error the policy state is left as it was before the call
 * (transactional) and the affected slots are marked empty if a copy may have been partially enqueued. */
moe_status expert_cache_stage(moe_expert_cache* cache, int32_t layer, const int32_t* ids_host, int32_t n,
                              int32_t* slot_ids_dev, void* copy_stream, void* wait_event, void* ready_event);

/* Counters of one layer, or of all layers when layer == -1. Any output pointer may be NULL. */
moe_status moe_expert_cache_stats(const moe_expert_cache* cache, int32_t layer, uint64_t* hits,
                                  uint64_t* misses, uint64_t* bytes_copied);

/* Expert held by each slot of a layer (-1 = empty): experts_host int32 [n_slots]. */
moe_status moe_expert_cache_slots(const moe_expert_cache* cache, int32_t layer, int32_t* experts_host);

/* Test hook: make the copy number `after_n_copies` (counted from this call, 0-based) fail with
 * MOE_ERR_HIP without copying; -1 disables.  Used to force the failure path from the host. */
moe_status moe_expert_cache_inject_copy_failure(moe_expert_cache* cache, int32_t after_n_copies);

/* moe_hbm_read_probe — measurement aid, not a step of the layer: reads `bytes` of device memory once with
 * 16-byte nontemporal loads spread over every compute unit (the plain streaming read that the 4-bit GEMVs'
 * achieved bandwidth is compared with).  buf_dev: 16-byte aligned, bytes a nonzero multiple of 16; sink_dev:
 * uint32 [1024] the kernel may write (it writes nothing in practice; the folded words only keep the loads).
 * MOE_ERR_INVALID_ARG on bad arguments (nothing launched).  Asynchronous on `stream`. */
moe_status moe_hbm_read_probe(const void* buf_dev, size_t bytes, uint32_t* sink_dev, void* stream);

/* Thread-local message describing the last non-MOE_OK status returned on this thread. */
const char* moe_last_error(void);

/* Library version string. */
const char* moe_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOEQ4_H */
