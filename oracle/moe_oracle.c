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
 * MXFP8 mode (the functions at the end): the same layer with FP8 E4M3
 * operands in MX blocks of 32 sharing an E8M0 scale, quantised by the OCP
 * Microscaling rule; products of the dequantised values accumulate in double
 * and the SwiGLU rows are requantised before the down projection.
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

/* ------------------------------------------------------------------ MXFP8
 * MXFP8 expert weights and activations (the Mixture-of-Kittens page names
 * MXFP8 as the low-precision format of its MoE kernels; the format is the OCP
 * Microscaling (MX) specification's): blocks of 32 consecutive values along
 * the reduction dimension share one E8M0 scale 2^(x - 127); each value is an
 * FP8 E4M3 number (1 sign, 4 exponent bits with bias 7, 3 mantissa bits;
 * subnormals below 2^-6; largest magnitude 448; no infinities; S.1111.111 is
 * NaN). A block's scale is 2^(floor(log2(max |v|)) - 8), 8 being the E4M3
 * exponent of its largest binade, clamped to 2^-127 .. 2^127 (2^-127 for an
 * all-zero block); each element is v / scale rounded to the nearest E4M3
 * value, ties to the even code, magnitudes past 448 saturating to 448. */

/* The value of an E4M3 code. */
double oracle_e4m3_value(uint8_t c) {
  const int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
  if (e == 15 && m == 7) return NAN;
  /* normal: (1 + m/8) 2^(e-7) = (8 + m) 2^(e-10); subnormal: (m/8) 2^-6 = m 2^-9 */
  const double v = e ? ldexp(8.0 + m, e - 10) : ldexp((double)m, -9);
  return s ? -v : v;
}

/* The E4M3 code nearest to x (ties to the even code; |x| >= 448 gives +-448;
 * a result of zero keeps x's sign). */
uint8_t oracle_e4m3_encode(double x) {
  const uint8_t sign = signbit(x) ? 0x80 : 0;
  double a = fabs(x);
#ifdef ORACLE_PLANT_E4M3_NO_SATURATE
  if (a >= 480.0) return sign | 0x7F;
#endif
  if (a >= 448.0) return sign | 0x7E;
  if (a == 0.0) return sign;
  int e2;
  frexp(a, &e2);
  const int E = e2 - 1;                    /* a in [2^E, 2^(E+1)) */
  const int step = E < -6 ? -9 : E - 3;    /* spacing of E4M3 values around a */
#ifdef ORACLE_PLANT_E4M3_TIES_AWAY
  const double q = round(ldexp(a, -step));
#else
  const double q = nearbyint(ldexp(a, -step));  /* default rounding: ties to even */
#endif
  if (E < -6) return sign | (uint8_t)q;   /* subnormal m = q (q = 8 is 2^-6, code 0x08) */
  if (q >= 16.0) return sign | (uint8_t)((E + 8) << 3);   /* rounded up to 2^(E+1) */
  return sign | (uint8_t)(((E + 7) << 3) | ((int)q - 8));
}

/* Element-wise forms of the two above, over n codes or values. */
void oracle_e4m3_values(int64_t n, const uint8_t* c, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_value(c[i]);
}
void oracle_e4m3_encode_array(int64_t n, const double* x, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_encode(x[i]);
}

/* Scale exponent of a block whose largest magnitude is amax. */
static int mx_scale_exp(double amax) {
  if (amax == 0.0) return -127;
  int e2;
  frexp(amax, &e2);
#ifdef ORACLE_PLANT_MX_EMAX7
  int se = (e2 - 1) - 7;
#else
  int se = (e2 - 1) - 8;
#endif
  return se < -127 ? -127 : (se > 127 ? 127 : se);
}

/* MX blocks along the rows of a [R][K] matrix (K a multiple of 32):
 * codes [R][K], scales [R][K/32]. */
void oracle_mx_quantize_rows(int64_t R, int64_t K, int dtype, const void* V, uint8_t* codes,
                             uint8_t* scales) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < R; ++r)
    for (int64_t b = 0; b < K / 32; ++b) {
      double amax = 0.0;
      for (int64_t i = 0; i < 32; ++i) {
        const double v = fabs(elem(V, dtype, (size_t)r * K + b * 32 + i));
        if (v > amax) amax = v;
      }
      const int se = mx_scale_exp(amax);
      scales[(size_t)r * (K / 32) + b] = (uint8_t)(se + 127);
      for (int64_t i = 0; i < 32; ++i)
        codes[(size_t)r * K + b * 32 + i] =
            oracle_e4m3_encode(ldexp(elem(V, dtype, (size_t)r * K + b * 32 + i), -se));
    }
}

/* MX blocks along the columns of a [K][N] matrix (K a multiple of 32): block
 * b of column n holds rows 32b .. 32b + 31. codes [K][N], scales [K/32][N]. */
void oracle_mx_quantize_cols(int64_t K, int64_t N, int dtype, const void* V, uint8_t* codes,
                             uint8_t* scales) {
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n)
    for (int64_t b = 0; b < K / 32; ++b) {
      double amax = 0.0;
      for (int64_t i = 0; i < 32; ++i) {
        const double v = fabs(elem(V, dtype, (size_t)(b * 32 + i) * N + n));
        if (v > amax) amax = v;
      }
      const int se = mx_scale_exp(amax);
      scales[(size_t)b * N + n] = (uint8_t)(se + 127);
      for (int64_t i = 0; i < 32; ++i)
        codes[(size_t)(b * 32 + i) * N + n] =
            oracle_e4m3_encode(ldexp(elem(V, dtype, (size_t)(b * 32 + i) * N + n), -se));
    }
}

/* The value an MX element stands for: its code's value times its block's scale. */
static double mx_value(const uint8_t* codes, const uint8_t* scales, size_t i, size_t si) {
  return ldexp(oracle_e4m3_value(codes[i]), (int)scales[si] - 127);
}

/* y[H] += scale * W_down^T q(SwiGLU(W_up^T a, W_gate^T a)) for one token with
 * MXFP8 operands: the token's row (codes a_q[H], scales a_s[H/32]); W_up,
 * W_gate [H][Dx] with scales [H/32][Dx]; W_down [Dx][H] with scales
 * [Dx/32][H]. u and g are exact sums of the dequantised products (double),
 * rounded to fp32 as the GPU holds them; the SwiGLU value is rounded to fp32
 * and q() quantises the Dx of them to MX blocks of 32 (the down projection's
 * reduction runs over Dx) before the down projection. */
static void ffn_accumulate_mx(int64_t H, int64_t Dx, const uint8_t* a_q, const uint8_t* a_s,
                              const uint8_t* wu_q, const uint8_t* wu_s, const uint8_t* wg_q,
                              const uint8_t* wg_s, const uint8_t* wd_q, const uint8_t* wd_s,
                              double scale, double* y) {
  double* u = (double*)calloc((size_t)Dx, sizeof(double));
  double* g = (double*)calloc((size_t)Dx, sizeof(double));
  float* hv = (float*)malloc((size_t)Dx * sizeof(float));
  uint8_t* h_q = (uint8_t*)malloc((size_t)Dx);
  uint8_t* h_s = (uint8_t*)malloc((size_t)(Dx / 32));
  for (int64_t h = 0; h < H; ++h) {
    const double a = mx_value(a_q, a_s, (size_t)h, (size_t)(h / 32));
    for (int64_t d = 0; d < Dx; ++d) {
#ifdef ORACLE_PLANT_MX_WEIGHT_UNSCALED
      u[d] += a * oracle_e4m3_value(wu_q[(size_t)h * Dx + d]);
#else
      u[d] += a * mx_value(wu_q, wu_s, (size_t)h * Dx + d, (size_t)(h / 32) * Dx + d);
#endif
      g[d] += a * mx_value(wg_q, wg_s, (size_t)h * Dx + d, (size_t)(h / 32) * Dx + d);
    }
  }
  for (int64_t d = 0; d < Dx; ++d) {
    const float u32 = (float)u[d], g32 = (float)g[d];
    hv[d] = (float)(silu((double)u32) * (double)g32);
  }
#ifdef ORACLE_PLANT_MX_NO_H_QUANT
  for (int64_t d = 0; d < Dx; ++d)
    for (int64_t n = 0; n < H; ++n)
      y[n] += scale * (double)hv[d] * mx_value(wd_q, wd_s, (size_t)d * H + n, (size_t)(d / 32) * H + n);
#else
  oracle_mx_quantize_rows(1, Dx, OR_F32, hv, h_q, h_s);
  for (int64_t d = 0; d < Dx; ++d) {
    const double hd = mx_value(h_q, h_s, (size_t)d, (size_t)(d / 32));
    for (int64_t n = 0; n < H; ++n)
      y[n] += scale * hd * mx_value(wd_q, wd_s, (size_t)d * H + n, (size_t)(d / 32) * H + n);
  }
#endif
  free(u);
  free(g);
  free(hv);
  free(h_q);
  free(h_s);
}

/* Output rows of the layer with MXFP8 operands, for the listed tokens, given
 * the routing (as oracle_layer_rows): A_q [S][H] with A_s [S][H/32] (the MX
 * blocks of each token row); W_up_q, W_gate_q [E][H][D] with scales
 * [E][H/32][D]; W_down_q [E][D][H] with scales [E][D/32][H]; the shared
 * expert's [H][Ds], [H/32][Ds] and [Ds][H], [Ds/32][H] (Ds = 0: none). */
void oracle_layer_rows_mx(int64_t H, int64_t D, int64_t E, int64_t k, int64_t Ds,
                          const uint8_t* A_q, const uint8_t* A_s, const uint8_t* Wu_q,
                          const uint8_t* Wu_s, const uint8_t* Wg_q, const uint8_t* Wg_s,
                          const uint8_t* Wd_q, const uint8_t* Wd_s, const uint8_t* Wsu_q,
                          const uint8_t* Wsu_s, const uint8_t* Wsg_q, const uint8_t* Wsg_s,
                          const uint8_t* Wsd_q, const uint8_t* Wsd_s, const int32_t* ids,
                          const float* w, const uint8_t* kept, int64_t n_rows,
                          const int64_t* tokens, double* O) {
  (void)E;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t i = 0; i < n_rows; ++i) {
    const int64_t t = tokens[i];
    double* y = O + (size_t)i * H;
    for (int64_t n = 0; n < H; ++n) y[n] = 0.0;
    const uint8_t* a_q = A_q + (size_t)t * H;
    const uint8_t* a_s = A_s + (size_t)t * (H / 32);
    for (int64_t j = 0; j < k; ++j) {
      const size_t f = (size_t)t * k + j;
      if (kept && !kept[f]) continue;
      const size_t e = (size_t)ids[f];
      ffn_accumulate_mx(H, D, a_q, a_s, Wu_q + e * H * D, Wu_s + e * (H / 32) * D,
                        Wg_q + e * H * D, Wg_s + e * (H / 32) * D, Wd_q + e * D * H,
                        Wd_s + e * (D / 32) * H, (double)w[f], y);
    }
    if (Ds > 0)
      ffn_accumulate_mx(H, Ds, a_q, a_s, Wsu_q, Wsu_s, Wsg_q, Wsg_s, Wsd_q, Wsd_s, 1.0, y);
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
