/*
 * CPU oracle of the fused Mixture-of-Experts layer forward pass.
 *
 * TEST INFRASTRUCTURE ONLY. It exists to check the HIP library, not to serve
 * it: only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * load it. It shares no code, header, table or helper with the HIP library.
 *
 * Everything is plain loops in the order the definitions are written:
 * dot products accumulate in double in ascending index order; the only
 * parallelism is an OpenMP loop over independent tokens, which does not
 * change any per-element result.
 *
 * What it computes (citations name the page and the passage):
 *  - Gate scores G = A . W_router, an S x E affinity matrix
 *    (FlashMoE review, "Core formulas": G_phi in R^{S x E}, produced by the
 *    gate; Algorithm 1 step "FusedGate(A)").
 *  - Softmax top-k routing: per token the k largest scores, and router weights
 *    from a softmax (vLLM fused_moe note, op table "topk_softmax"; Mixture-of-
 *    Kittens, "Overlapping compute and communication in MoE": the router picks
 *    the top-k routed experts and gives each a router weight).
 *  - Capacity: the routing table T_phi in (N x R)^{E x C}, slot c of expert e
 *    holding (token i, weight w) (FlashMoE review, "Core formulas"; capacity
 *    factor 1.0 in "Experimental setup").
 *  - moe_align_block_size: per-expert counts, block padding, exclusive cumsum,
 *    block-padded sorted ids and one expert id per block (vLLM fused_moe note,
 *    op table; vLLM PR 53280 summary, "Implementation", steps 2-3; size_t
 *    offsets from step 3).
 *  - The layer x' = W_shared(x) + sum_{e in top-k} w_e W_down^e
 *    SwiGLU(W_up^e x, W_gate^e x), SwiGLU(u, g) = SiLU(u) * g
 *    (Mixture-of-Kittens, "Overlapping compute and communication in MoE",
 *    the layer equation and the SwiGLU definition under it).
 *
 * Readings where the pages leave a step open:
 *  - top-k ties go to the lower expert index; slots are ordered by descending
 *    score;
 *  - renormalize=1: w_j = exp(G_j - m) / sum_{j'<k} exp(G_j' - m), the softmax
 *    over all E scores restricted to the chosen k and rescaled to sum to 1;
 *    renormalize=0: the full softmax over all E scores, at the chosen ids;
 *  - capacity C: an expert keeps its assignments in ascending token order
 *    and drops those at slot c >= C; dropped weights are not renormalised;
 *  - inside an expert, sorted ids ascend by flat index f = token*k + slot;
 *    padding entries hold the sentinel S*k;
 *  - weight layouts: W_up, W_gate [E][H][D], W_down [E][D][H], W_router
 *    [H][E], shared [H][Ds], [H][Ds], [Ds][H], all row-major.
 *
 * Precision: inputs are fp32 or bf16 (widened exactly); the gate scores are
 * rounded once to fp32 (the routing decision is taken on fp32 scores, as the
 * library's score tensor is fp32); the router weights are computed in double
 * and rounded once to fp32; the expert FFN and the combine stay in double.
 *
 * ORACLE_PLANT_* macros build deliberately wrong variants for the pin
 * self-test only (each must be caught by at least one pin).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OR_F32 0
#define OR_BF16 1

static double elem(const void* p, int dtype, size_t i) {
  if (dtype == OR_F32) return (double)((const float*)p)[i];
  uint32_t u = ((uint32_t)((const uint16_t*)p)[i]) << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* G[s][e] = fp32( sum_h A[s][h] * Wr[h][e] ) (+ bias[e], an fp32 add). */
void oracle_gate_logits(int64_t S, int64_t H, int64_t E, int dtype, const void* A,
                        const void* Wr, const float* bias, float* G) {
#pragma omp parallel for schedule(static)
  for (int64_t s = 0; s < S; ++s) {
    double* acc = (double*)calloc((size_t)E, sizeof(double));
    for (int64_t h = 0; h < H; ++h) {
      double a = elem(A, dtype, (size_t)s * H + h);
      for (int64_t e = 0; e < E; ++e) acc[e] += a * elem(Wr, dtype, (size_t)h * E + e);
    }
    for (int64_t e = 0; e < E; ++e) {
      float g = (float)acc[e];
      if (bias) g = g + bias[e];
      G[(size_t)s * E + e] = g;
    }
    free(acc);
  }
}

typedef struct {
  float v;
  int32_t e;
} scored;

/* Total order: larger score first, lower expert index first on equal score. */
static int by_score(const void* pa, const void* pb) {
  const scored* a = (const scored*)pa;
  const scored* b = (const scored*)pb;
  if (a->v > b->v) return -1;
  if (a->v < b->v) return 1;
#ifdef ORACLE_PLANT_TIE_HIGH
  return (a->e > b->e) ? -1 : (a->e < b->e);
#else
  return (a->e < b->e) ? -1 : (a->e > b->e);
#endif
}

/* Top-k of each row of G, then router weights (see header for the formula). */
void oracle_topk_softmax(int64_t S, int64_t E, int64_t k, int renormalize, const float* G,
                         int32_t* ids, float* w) {
#pragma omp parallel for schedule(static)
  for (int64_t s = 0; s < S; ++s) {
    const float* g = G + (size_t)s * E;
    scored* order = (scored*)malloc((size_t)E * sizeof(scored));
    for (int64_t e = 0; e < E; ++e) {
      order[e].v = g[e];
      order[e].e = (int32_t)e;
    }
    qsort(order, (size_t)E, sizeof(scored), by_score);
    double m = (double)order[0].v;
    double den = 0.0;
    if (renormalize) {
      for (int64_t j = 0; j < k; ++j) den += exp((double)order[j].v - m);
    } else {
      for (int64_t e = 0; e < E; ++e) den += exp((double)g[e] - m);
    }
    for (int64_t j = 0; j < k; ++j) {
      ids[(size_t)s * k + j] = order[j].e;
#ifdef ORACLE_PLANT_WEIGHT_NO_EXP
      w[(size_t)s * k + j] = (float)(((double)order[j].v - m + 1.0) / den);
#else
      w[(size_t)s * k + j] = (float)(exp((double)order[j].v - m) / den);
#endif
    }
    free(order);
  }
}

/* kept[f] = 1 when assignment f = s*k + j (expert ids[f]) gets a slot c < C,
 * slots being handed out in ascending f; C = 0 keeps everything. */
void oracle_capacity_mask(int64_t S, int64_t k, int64_t E, int64_t C, const int32_t* ids,
                          uint8_t* kept) {
  int64_t F = S * k;
  int64_t* seen = (int64_t*)calloc((size_t)(E > 0 ? E : 1), sizeof(int64_t));
  for (int64_t f = 0; f < F; ++f) {
    int64_t c = seen[ids[f]]++;
#ifdef ORACLE_PLANT_CAP_OFF_BY_ONE
    kept[f] = (C <= 0 || c <= C) ? 1 : 0;
#else
    kept[f] = (C <= 0 || c < C) ? 1 : 0;
#endif
  }
  free(seen);
}

/* moe_align_block_size over the flat ids (F = S*k entries):
 * cnt_e, kept_e = min(cnt_e, C), pad_e = ceil(kept_e/BM)*BM,
 * off_e = sum_{e'<e} pad_e', sorted_ids[off_e + c] = c-th kept f of expert e
 * (ascending f), padding = F, expert_ids[b] = e for the blocks of expert e,
 * ntpp = sum pad_e, counts[e] = kept_e. */
void oracle_align(int64_t S, int64_t k, int64_t E, int64_t BM, int64_t C, const int32_t* ids,
                  int32_t* sorted_ids, int32_t* expert_ids, int32_t* ntpp, int32_t* counts) {
  int64_t F = S * k;
  int64_t* cnt = (int64_t*)calloc((size_t)E, sizeof(int64_t));
  int64_t* keep = (int64_t*)calloc((size_t)E, sizeof(int64_t));
  int64_t* off = (int64_t*)calloc((size_t)E, sizeof(int64_t));
  int64_t* seen = (int64_t*)calloc((size_t)E, sizeof(int64_t));
  for (int64_t f = 0; f < F; ++f) cnt[ids[f]]++;
  int64_t total = 0;
  for (int64_t e = 0; e < E; ++e) {
    keep[e] = (C > 0 && cnt[e] > C) ? C : cnt[e];
    int64_t pad = (keep[e] + BM - 1) / BM * BM;
    off[e] = total;
    total += pad;
    for (int64_t i = off[e]; i < total; ++i) sorted_ids[i] = (int32_t)F;
    for (int64_t b = off[e] / BM; b < total / BM; ++b) expert_ids[b] = (int32_t)e;
  }
  for (int64_t f = 0; f < F; ++f) {
    int64_t e = ids[f];
    int64_t c = seen[e]++;
#ifdef ORACLE_PLANT_ALIGN_REVERSED
    if (c < keep[e]) sorted_ids[off[e] + keep[e] - 1 - c] = (int32_t)f;
#else
    if (c < keep[e]) sorted_ids[off[e] + c] = (int32_t)f;
#endif
  }
  *ntpp = (int32_t)total;
  for (int64_t e = 0; e < E; ++e) counts[e] = (int32_t)keep[e];
  free(cnt);
  free(keep);
  free(off);
  free(seen);
}

static double silu(double x) { return x / (1.0 + exp(-x)); }

/* y[H] += scale * W_down^T SwiGLU(W_up^T a, W_gate^T a) for one token row a[H];
 * Wu, Wg are [H][Dx], Wd is [Dx][H]. */
static void ffn_accumulate(int64_t H, int64_t Dx, int dtype, const void* A, size_t a_off,
                           const void* Wu, const void* Wg, const void* Wd, size_t w_off_up,
                           size_t w_off_down, double scale, double* y) {
  double* u = (double*)calloc((size_t)Dx, sizeof(double));
  double* g = (double*)calloc((size_t)Dx, sizeof(double));
  for (int64_t h = 0; h < H; ++h) {
    double a = elem(A, dtype, a_off + (size_t)h);
    for (int64_t d = 0; d < Dx; ++d) {
      u[d] += a * elem(Wu, dtype, w_off_up + (size_t)h * Dx + d);
      g[d] += a * elem(Wg, dtype, w_off_up + (size_t)h * Dx + d);
    }
  }
  for (int64_t d = 0; d < Dx; ++d) {
#ifdef ORACLE_PLANT_SILU_ON_GATE
    double hd = silu(g[d]) * u[d];
#else
    double hd = silu(u[d]) * g[d];
#endif
    for (int64_t n = 0; n < H; ++n) {
#ifdef ORACLE_PLANT_DOWN_TRANSPOSED
      y[n] += scale * hd * elem(Wd, dtype, w_off_down + (size_t)n * Dx + d);
#else
      y[n] += scale * hd * elem(Wd, dtype, w_off_down + (size_t)d * H + n);
#endif
    }
  }
  free(u);
  free(g);
}

/* Output rows of the layer for the listed tokens, given the routing:
 * O[i][:] = sum_{j<k, kept} w[t*k+j] * FFN_{ids[t*k+j]}(A_t) + FFN_shared(A_t),
 * t = tokens[i]. kept may be NULL (all kept); Ds = 0 means no shared expert. */
void oracle_layer_rows(int64_t H, int64_t D, int64_t E, int64_t k, int64_t Ds, int dtype,
                       const void* A, const void* W_up, const void* W_gate, const void* W_down,
                       const void* Ws_up, const void* Ws_gate, const void* Ws_down,
                       const int32_t* ids, const float* w, const uint8_t* kept, int64_t n_rows,
                       const int64_t* tokens, double* O) {
  (void)E;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t i = 0; i < n_rows; ++i) {
    int64_t t = tokens[i];
    double* y = O + (size_t)i * H;
    for (int64_t n = 0; n < H; ++n) y[n] = 0.0;
    for (int64_t j = 0; j < k; ++j) {
#ifdef ORACLE_PLANT_ROW_INDEX
      size_t f = (size_t)i * k + j;
#else
      size_t f = (size_t)t * k + j;
#endif
      if (kept && !kept[f]) continue;
      int64_t e = ids[f];
#ifdef ORACLE_PLANT_WEIGHT_SLOT0
      double wt = (double)w[(size_t)t * k];
#else
      double wt = (double)w[f];
#endif
      ffn_accumulate(H, D, dtype, A, (size_t)t * H, W_up, W_gate, W_down, (size_t)e * H * D,
                     (size_t)e * D * H, wt, y);
    }
#ifndef ORACLE_PLANT_DROP_SHARED
    if (Ds > 0) ffn_accumulate(H, Ds, dtype, A, (size_t)t * H, Ws_up, Ws_gate, Ws_down, 0, 0, 1.0, y);
#endif
  }
}

/* Threads the OpenMP loops above run on. */
int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
