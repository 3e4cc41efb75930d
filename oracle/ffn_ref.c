/* CPU oracle, C part: the expert feed-forward network of the MoE decode step on 4-bit affine weights.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, __graft_entry__.smoke() and bench.py's cpu_baseline leg load
 * this library (oracle/liboracle_ffn.so, built with gcc by the package's build step).  It shares no code,
 * header, table or constant generator with the HIP path.
 *
 * It is the same definition as oracle/moe.py (quantize_affine_q4, dequantize, expert_ffn), written in
 * plain C so that a full-size stack of layers can be checked token by token in seconds instead of hours:
 *   - the 4-bit affine encoding ("MLX affine 4-bit" weights: [REMIO] "L'affirmation des 2 Go fait de la
 *     bande passante SSD la nouvelle contrainte"; [DAILY] "1. Compression par 4"), read as plain min-max per
 *     group of 64 columns, with its integer decisions taken in IEEE fp32 like the numpy oracle;
 *   - the dequantized weight w_hat = scale * code + bias in float64;
 *   - the expert: y = W_down (act(W_gate u) * (W_up u)), float64, every dot product summed in column
 *     order ([LEAF] "Du code sur-mesure sans dépendance externe": quantized matrix-vector kernels; the
 *     gated structure is the reading for Gemma-style experts).
 * Nothing is blocked, fused or reordered beyond evaluating several input rows in the same pass over a
 * weight row (each output still sums its products in column order).
 *
 * Pages cited (by title):
 *   [REMIO] "TurboFieldfare exécute Mac Gemma 4 26B dans 2 Go, mais la vitesse du SSD devient le compromis"
 *   [DAILY] "TurboFieldfare" event page, daily.steinslab.io
 *   [LEAF]  romain.leaflet.pub article on TurboFieldfare (untitled page)
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define GROUP 64

/* float32 -> nearest bfloat16 (ties to even), returned as float32 (finite inputs) */
static float round_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  u = (u + 0x7fffu + ((u >> 16) & 1u)) & 0xffff0000u;
  memcpy(&f, &u, 4);
  return f;
}

/* Encode w [N][K] (fp32, K a multiple of 64): per row and group of 64 columns, mn and mx of the group,
 * scale = (mx - mn) / 15 and bias = mn (each rounded to bf16 when sb_bf16), code = clamp(round half to
 * even((w - bias) / scale), 0, 15), code = 0 when scale == 0.  All in fp32.
 * codes uint8 [N][K]; scale, bias fp32 [N][K/64]. */
void orc_quantize_q4(const float* w, int N, int K, int sb_bf16, uint8_t* codes, float* scale, float* bias) {
  const int G = K / GROUP;
  for (int r = 0; r < N; ++r) {
    for (int g = 0; g < G; ++g) {
      const float* wg = w + (int64_t)r * K + g * GROUP;
      float mn = wg[0], mx = wg[0];
      for (int i = 1; i < GROUP; ++i) {
        if (wg[i] < mn) mn = wg[i];
        if (wg[i] > mx) mx = wg[i];
      }
      float s = (mx - mn) / 15.0f;
      float b = mn;
      if (sb_bf16) {
        s = round_bf16(s);
        b = round_bf16(b);
      }
      scale[(int64_t)r * G + g] = s;
      bias[(int64_t)r * G + g] = b;
      uint8_t* cg = codes + (int64_t)r * K + g * GROUP;
      for (int i = 0; i < GROUP; ++i) {
        if (s == 0.0f) {
          cg[i] = 0;
          continue;
        }
        float t = rintf((wg[i] - b) / s);   /* default rounding mode: to nearest, ties to even */
        if (t < 0.0f) t = 0.0f;
        if (t > 15.0f) t = 15.0f;
        cg[i] = (uint8_t)t;
      }
    }
  }
}

static double gelu_tanh(double z) {
  return 0.5 * z * (1.0 + tanh(sqrt(2.0 / M_PI) * (z + 0.044715 * z * z * z)));
}

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* out[t][r] = sum_c w_hat[r][c] * x[t][c] for the rows r of one quantized matrix [N][K] and n input
 * rows x [n][K]; the sum over c runs in column order for every output. */
static void dequant_matvec(const uint8_t* codes, const float* scale, const float* bias, int N, int K,
                           const double* x, int n, double* out /* [n][N] */, double* acc /* [n] */) {
  const int G = K / GROUP;
  for (int r = 0; r < N; ++r) {
    for (int t = 0; t < n; ++t) acc[t] = 0.0;
    for (int g = 0; g < G; ++g) {
      const double s = scale[(int64_t)r * G + g], b = bias[(int64_t)r * G + g];
      for (int i = 0; i < GROUP; ++i) {
        const int c = g * GROUP + i;
        const double w = s * (double)codes[(int64_t)r * K + c] + b;
        for (int t = 0; t < n; ++t) acc[t] += w * x[(int64_t)t * K + c];
      }
    }
    for (int t = 0; t < n; ++t) out[(int64_t)t * N + r] = acc[t];
  }
}

/* The expert FFN for n input rows: w_gu fp32 [2F][d] (gate rows 0..F-1, up rows F..2F-1), w_down fp32
 * [d][F], both encoded as above; u float64 [n][d] -> y float64 [n][d], and h float64 [n][F] if h != NULL.
 * act: 0 = GELU (tanh form), 1 = SiLU.  Returns 0, or -1 if memory runs out. */
int orc_expert_ffn(const float* w_gu, const float* w_down, int d, int F, int sb_bf16, int act, const double* u, int n,
                   double* y, double* h_out) {
  int rc = -1;
  uint8_t* cgu = malloc((size_t)2 * F * d);
  float* sgu = malloc((size_t)2 * F * (d / GROUP) * sizeof(float));
  float* bgu = malloc((size_t)2 * F * (d / GROUP) * sizeof(float));
  uint8_t* cd = malloc((size_t)d * F);
  float* sd = malloc((size_t)d * (F / GROUP) * sizeof(float));
  float* bd = malloc((size_t)d * (F / GROUP) * sizeof(float));
  double* gu = malloc((size_t)n * 2 * F * sizeof(double));
  double* h = malloc((size_t)n * F * sizeof(double));
  double* acc = malloc((size_t)n * sizeof(double));
  if (!cgu || !sgu || !bgu || !cd || !sd || !bd || !gu || !h || !acc) goto out;
  orc_quantize_q4(w_gu, 2 * F, d, sb_bf16, cgu, sgu, bgu);
  orc_quantize_q4(w_down, d, F, sb_bf16, cd, sd, bd);
  /* gate and up: g = W_gate u, v = W_up u; h = act(g) * v */
  dequant_matvec(cgu, sgu, bgu, 2 * F, d, u, n, gu, acc);
  for (int t = 0; t < n; ++t)
    for (int f = 0; f < F; ++f) {
      const double g = gu[(int64_t)t * 2 * F + f], v = gu[(int64_t)t * 2 * F + F + f];
      h[(int64_t)t * F + f] = (act == 1 ? silu(g) : gelu_tanh(g)) * v;
    }
  /* down: y = W_down h */
  dequant_matvec(cd, sd, bd, d, F, h, n, y, acc);
  if (h_out) memcpy(h_out, h, (size_t)n * F * sizeof(double));
  rc = 0;
out:
  free(cgu);
  free(sgu);
  free(bgu);
  free(cd);
  free(sd);
  free(bd);
  free(gu);
  free(h);
  free(acc);
  return rc;
}
