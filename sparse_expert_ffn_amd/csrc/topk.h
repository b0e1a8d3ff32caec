// Softmax top-k of one token's gate scores (used by the top-k kernel and by
// the fused gate + top-k kernel).
#pragma once

#include "moe_common.h"

namespace moe {

// One wave64 per token; lane l holds the scores of experts l, l+64, ... (E <=
// 1024 -> at most 16 per lane). k rounds of: lane-local best, then a 6-step
// butterfly over the wave; the order is (score descending, expert index
// ascending), NaN ranking as -inf. The router weights are then computed in
// double from the chosen fp32 scores and rounded once to fp32.
constexpr int kTopkMaxPerLane = 16;

__device__ __forceinline__ bool topk_better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

// One token: g = its E scores (global or LDS), ids / w = its k outputs.
// sel: 32 floats of wave-private scratch.
template <typename GPtr>
__device__ __forceinline__ void topk_one(GPtr g, int64_t E_, int64_t k_, int renormalize,
                                         int32_t* ids, float* w, int lane, float* sel) {
  const int E = (int)E_;
  const int k = (int)k_;
  float v[kTopkMaxPerLane];
  uint32_t taken = 0;
#pragma unroll
  for (int i = 0; i < kTopkMaxPerLane; ++i) {
    const int e = lane + 64 * i;
    float x = (e < E) ? g[e] : -INFINITY;
    v[i] = (x != x) ? -INFINITY : x;
  }
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < kTopkMaxPerLane; ++i) {
      const int e = lane + 64 * i;
      if (e < E && !((taken >> i) & 1u) && topk_better(v[i], e, bv, bi)) {
        bv = v[i];
        bi = e;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oi = __shfl_xor(bi, off);
      if (topk_better(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    if (lane == 0) {
      ids[j] = bi;
      sel[j] = bv;
    }
  }
  __builtin_amdgcn_wave_barrier();
  const double m = (double)sel[0];
  if (renormalize) {
    // lane j < k computes exp(G_j - G_0); every lane then adds them in slot
    // order (the same sum, in the same order, as a serial loop)
    const double ej = lane < k ? exp((double)sel[lane] - m) : 0.0;
    double den = 0.0;
    for (int j = 0; j < k; ++j) den += __shfl(ej, j);
    if (lane < k) w[lane] = (float)(ej / den);
  } else if (lane == 0) {
    double den = 0.0;
    for (int e = 0; e < E; ++e) den += exp((double)g[e] - m);
    for (int j = 0; j < k; ++j) w[j] = (float)(exp((double)sel[j] - m) / den);
  }
}

}  // namespace moe
