// Softmax top-k of one token's gate scores (used by the top-k kernel and by
// the fused gate + top-k kernel).
#pragma once

#include "moe_common.h"

namespace moe {

// One wave64 per token; lane l holds the scores of experts l, l+64, ... (E <=
// 1024 -> at most 16 per lane; the code is instantiated per count). The
// order is (score descending, expert index ascending), NaN ranking as -inf. Each of the k rounds:
//   1. lane-local maximum over the lane's untaken scores;
//   2. wave maximum M: DPP exchanges inside each row of 16 lanes (quad
//      permutes, half-row and row mirrors), then the four row maxima read
//      into scalars;
//   3. the winner is the lowest expert index holding M among the untaken
//      ones: expert l + 64 i ranks below every expert of a larger i, so the
//      first non-empty ballot over i = 0, 1, ... gives it (its lowest lane);
//   4. the owning lane marks it taken.
// No shuffles through LDS and no index comparisons across lanes. The router
// weights are then computed in double from the chosen fp32 scores and rounded
// once to fp32.
__device__ __forceinline__ float dpp_max_step(float x, int ctrl) {
  // ctrl is a DPP control code: quad_perm, row_half_mirror, row_mirror
  int y;
  switch (ctrl) {
    case 0xB1: y = __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, true); break;
    case 0x4E: y = __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, true); break;
    case 0x141: y = __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x141, 0xF, 0xF, true); break;
    default: y = __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x140, 0xF, 0xF, true); break;
  }
  return fmaxf(x, __builtin_bit_cast(float, y));
}

// Maximum of x over the 64 lanes (every lane gets it; wave-uniform).
__device__ __forceinline__ float wave_max(float x) {
  x = dpp_max_step(x, 0xB1);   // quad_perm [1,0,3,2]: pairs
  x = dpp_max_step(x, 0x4E);   // quad_perm [2,3,0,1]: quads
  x = dpp_max_step(x, 0x141);  // row_half_mirror: the two quads of a half-row
  x = dpp_max_step(x, 0x140);  // row_mirror: the two half-rows of a row
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

__device__ __forceinline__ double readlane_f64(double x, int l) {
  const uint64_t b = __builtin_bit_cast(uint64_t, x);
  const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)b, l);
  const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(b >> 32), l);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// The k choices of one token: g = its E scores (global or LDS), NPL >=
// ceil(E / 64) scores per lane, k <= 64. Every lane of the wave calls it;
// lane j < k gets the j-th choice's score and expert, every lane the top
// score m0.
template <int NPL, typename GPtr>
__device__ __forceinline__ void topk_select_n(GPtr g, int E, int k, int lane, float& my_sel,
                                              int& my_id, float& m0) {
  float v[NPL];
  uint32_t live = 0;  // bit i: expert lane + 64 i exists and is not taken
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int e = lane + 64 * i;
    const float x = (e < E) ? g[e] : -INFINITY;
    v[i] = (x != x) ? -INFINITY : x;
    if (e < E) live |= 1u << i;
  }
  my_sel = 0.f;  // lane j: score of the j-th choice
  my_id = 0;     // lane j: expert of the j-th choice
  m0 = 0.f;
  for (int j = 0; j < k; ++j) {
    float lm = -INFINITY;
#pragma unroll
    for (int i = 0; i < NPL; ++i)
      if ((live >> i) & 1u) lm = fmaxf(lm, v[i]);
    const float M = wave_max(lm);
    int e_win = 0;
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const uint64_t b = __ballot(((live >> i) & 1u) && v[i] == M);
      if (b) {
        e_win = 64 * i + (int)__builtin_ctzll(b);
        break;
      }
    }
    if ((e_win & 63) == lane) live &= ~(1u << (e_win >> 6));
    if (lane == j) {
      my_sel = M;
      my_id = e_win;
    }
    if (j == 0) m0 = M;
  }
}

// One token: g = its E scores (global or LDS), ids / w = its k outputs
// (k <= 64), NPL >= ceil(E / 64) scores per lane. Every lane of the wave
// calls it.
template <int NPL, typename GPtr>
__device__ __forceinline__ void topk_one_n(GPtr g, int E, int k, int renormalize, int32_t* ids,
                                           float* w, int lane) {
  float my_sel, m0;
  int my_id;
  topk_select_n<NPL>(g, E, k, lane, my_sel, my_id, m0);
  const double m = (double)m0;
  if (renormalize) {
    // lane j < k computes exp(G_j - G_0); the denominator adds them in slot
    // order (the same sum, in the same order, as a serial loop)
    const double ej = lane < k ? exp((double)my_sel - m) : 0.0;
    double den = 0.0;
    for (int j = 0; j < k; ++j) den += readlane_f64(ej, j);
    if (lane < k) {
      ids[lane] = my_id;
      w[lane] = (float)(ej / den);
    }
  } else {
    // full softmax denominator: each lane sums its experts in index order,
    // then the lane sums are added in lane order
    double part = 0.0;
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const int e = lane + 64 * i;
      if (e < E) part += exp((double)g[e] - m);
    }
    double den = 0.0;
    for (int l = 0; l < 64; ++l) den += readlane_f64(part, l);
    if (lane < k) {
      ids[lane] = my_id;
      w[lane] = (float)(exp((double)my_sel - m) / den);
    }
  }
}

// topk_select_n dispatched on the scores per lane (E <= 1024).
template <typename GPtr>
__device__ __forceinline__ void topk_select(GPtr g, int E, int k, int lane, float& my_sel,
                                            int& my_id, float& m0) {
  if (E <= 64)
    topk_select_n<1>(g, E, k, lane, my_sel, my_id, m0);
  else if (E <= 128)
    topk_select_n<2>(g, E, k, lane, my_sel, my_id, m0);
  else if (E <= 256)
    topk_select_n<4>(g, E, k, lane, my_sel, my_id, m0);
  else if (E <= 512)
    topk_select_n<8>(g, E, k, lane, my_sel, my_id, m0);
  else
    topk_select_n<16>(g, E, k, lane, my_sel, my_id, m0);
}

// Renormalised router weights of nt tokens, token t being s0 + t * stride
// (one wave): sel = their chosen scores, k per token in slot order, in LDS;
// e = LDS room for nt * k doubles; w = the [S][k] weights. The same arithmetic as topk_one_n's renormalised weights
// (exp(G_j - G_0) in double, the denominator added in slot order, the
// quotient rounded once), but with the exponentials of all nt tokens spread
// over the lanes instead of k lanes per token: the double exp is the
// costly part, so one pass over nt * k lanes replaces nt passes.
__device__ __forceinline__ void topk_weights_renorm(const float* sel, double* e, int nt, int k,
                                                    int64_t s0, int64_t stride, float* w,
                                                    int lane) {
  const int n = nt * k;
  for (int p = lane; p < n; p += 64) {
    const int t = p / k;
    e[p] = exp((double)sel[p] - (double)sel[t * k]);
  }
  // other lanes' exponentials are read below: wait for this wave's LDS
  // writes (one wave, so no workgroup barrier)
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
  for (int p = lane; p < n; p += 64) {
    const int t = p / k;
    double den = 0.0;
    for (int j = 0; j < k; ++j) den += e[t * k + j];
    w[(s0 + t * stride) * k + (p - t * k)] = (float)(e[p] / den);
  }
}

// Dispatch on the scores per lane (E <= 1024).
template <typename GPtr>
__device__ __forceinline__ void topk_one(GPtr g, int64_t E_, int64_t k_, int renormalize,
                                         int32_t* ids, float* w, int lane) {
  const int E = (int)E_;
  const int k = (int)k_;
  if (E <= 64)
    topk_one_n<1>(g, E, k, renormalize, ids, w, lane);
  else if (E <= 128)
    topk_one_n<2>(g, E, k, renormalize, ids, w, lane);
  else if (E <= 256)
    topk_one_n<4>(g, E, k, renormalize, ids, w, lane);
  else if (E <= 512)
    topk_one_n<8>(g, E, k, renormalize, ids, w, lane);
  else
    topk_one_n<16>(g, E, k, renormalize, ids, w, lane);
}

}  // namespace moe
