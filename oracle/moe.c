/*
 * moe.c -- plain fp64 CPU oracle of Flint's MoE sublayer at decode: router,
 * top-k selection, the routed and shared expert FFNs.
 *
 * TEST INFRASTRUCTURE, like oracle.c: only the tests, the smoke check and the
 * bench may load it, and it shares nothing with the HIP library.
 *
 * Sources (page titles and sections):
 *   "Day-0 Support for Flint on vLLM" (hnkhoi.com), "Model architecture":
 *       hidden size 2048; 256 experts with sigmoid top-6 routing plus a
 *       shared expert.
 *   "How to Run Recursive Flint Locally with SGLang" (mindstudio.ai): 256
 *       routed experts, 6 selected per token, one always-active shared
 *       expert.
 *   "Day-0 Support for Flint on vLLM" (newruntime.com), "What happened":
 *       small-batch MoE and dense GEMV kernels on the optimised decode path.
 * Readings where the pages are silent (each restated at its use):
 *   - router logits z_e = <x, w_e>, no bias; score s_e = 1 / (1 + e^{-z_e});
 *   - the top_k experts by score, i.e. in the order of the exact (fp64) z,
 *     ties to the lower index (the definition; a kernel that ranks rounded
 *     logits agrees wherever the top-k boundary is not within its rounding);
 *   - routing weights s_sel / sum(s_sel) over the selected experts;
 *   - every expert, routed or shared, is a SwiGLU FFN of width `inter`:
 *     E(x) = W_down (silu(W_gate x) * (W_up x)), silu(g) = g / (1 + e^{-g});
 *   - the shared expert joins with weight 1:
 *     y = sum_k w_k E_{id_k}(x) + sum_shared E_shared(x).
 * Weights are bf16 bit patterns in the library's layout:
 *   w_router  [experts][hidden]
 *   w_gate_up [experts + shared][2][inter][hidden]  (gate rows, then up rows)
 *   w_down    [experts + shared][hidden][inter]
 * with the shared experts after the routed ones.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"

static double bfv(uint16_t b) { return orc_bf16_value(b); }

/* O9: routing of one token. */
int orc_moe_route(const orc_moe* M, const float* x, const uint16_t* w_router, int32_t* ids,
                  double* weights) {
  if (M->top_k < 1 || M->top_k > M->experts) return -1;
  double* z = (double*)malloc(sizeof(double) * (size_t)M->experts);
  char* taken = (char*)calloc((size_t)M->experts, 1);
  for (int e = 0; e < M->experts; ++e) {
    const uint16_t* w = w_router + (int64_t)e * M->hidden;
    double acc = 0.0;
    for (int i = 0; i < M->hidden; ++i) acc += (double)x[i] * bfv(w[i]);
    z[e] = acc;
  }
  /* top_k by repeated selection of the largest remaining fp64 logit; a
   * strict comparison keeps the lower index on ties */
  double ssum = 0.0;
  for (int k = 0; k < M->top_k; ++k) {
    int best = -1;
    for (int e = 0; e < M->experts; ++e)
      if (!taken[e] && (best < 0 || z[e] > z[best])) best = e;
    taken[best] = 1;
    ids[k] = best;
    weights[k] = 1.0 / (1.0 + exp(-z[best]));
    ssum += weights[k];
  }
  for (int k = 0; k < M->top_k; ++k) weights[k] /= ssum;
  free(z);
  free(taken);
  return 0;
}

/* One SwiGLU expert (index e in the weight arrays) on one token, added to y
 * with weight w. */
static void expert_add(const orc_moe* M, int e, const float* x, const uint16_t* w_gate_up,
                       const uint16_t* w_down, double w, double* y) {
  const int H = M->hidden, I = M->inter;
  const uint16_t* wg = w_gate_up + (int64_t)e * 2 * I * H;
  const uint16_t* wu = wg + (int64_t)I * H;
  const uint16_t* wd = w_down + (int64_t)e * H * I;
  double* h = (double*)malloc(sizeof(double) * (size_t)I);
  for (int j = 0; j < I; ++j) {
    double g = 0.0, u = 0.0;
    for (int i = 0; i < H; ++i) {
      g += (double)x[i] * bfv(wg[(int64_t)j * H + i]);
      u += (double)x[i] * bfv(wu[(int64_t)j * H + i]);
    }
    h[j] = g / (1.0 + exp(-g)) * u;
  }
  for (int r = 0; r < H; ++r) {
    double acc = 0.0;
    for (int j = 0; j < I; ++j) acc += bfv(wd[(int64_t)r * I + j]) * h[j];
    y[r] += w * acc;
  }
  free(h);
}

/* O10: the MoE sublayer for T tokens.  ids [T][top_k], weights [T][top_k],
 * y [T][hidden]. */
int orc_moe_forward(const orc_moe* M, int T, const float* x, const uint16_t* w_router,
                    const uint16_t* w_gate_up, const uint16_t* w_down, int32_t* ids,
                    double* weights, double* y, int nthreads) {
  if (nthreads <= 0) nthreads = orc_default_threads();
  int bad = 0;
  for (int t = 0; t < T; ++t)
    bad |= orc_moe_route(M, x + (int64_t)t * M->hidden, w_router, ids + (int64_t)t * M->top_k,
                         weights + (int64_t)t * M->top_k);
  if (bad) return -1;
  memset(y, 0, sizeof(double) * (size_t)T * M->hidden);
  const int per = M->top_k + M->shared;
  /* one work item per (token, expert slot); each adds into its own buffer */
  double* part = (double*)calloc((size_t)T * per * M->hidden, sizeof(double));
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
  for (int64_t it = 0; it < (int64_t)T * per; ++it) {
    const int t = (int)(it / per), k = (int)(it % per);
    const float* xt = x + (int64_t)t * M->hidden;
    const int e = k < M->top_k ? ids[(int64_t)t * M->top_k + k] : M->experts + (k - M->top_k);
    const double w = k < M->top_k ? weights[(int64_t)t * M->top_k + k] : 1.0;
    expert_add(M, e, xt, w_gate_up, w_down, w, part + it * M->hidden);
  }
  for (int64_t it = 0; it < (int64_t)T * per; ++it) {
    double* yt = y + (it / per) * M->hidden;
    for (int r = 0; r < M->hidden; ++r) yt[r] += part[it * M->hidden + r];
  }
  free(part);
  return 0;
}
