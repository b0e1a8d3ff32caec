// Routing kernels: softmax top-k over the gate scores, and the
// moe_align_block_size counting sort.
#include <float.h>

#include "moe_common.h"
#include "topk.h"

namespace moe {

// ------------------------------------------------------------------ top-k
// (per-token selection in topk.h, shared with the fused gate kernel)
__global__ __launch_bounds__(256) void topk_softmax_kernel(TopkParams p) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  // each wave handles tokens s, s + 4 * gridDim.x, ... (no block barrier below)
  for (int64_t s = (int64_t)blockIdx.x * 4 + wave; s < p.S; s += (int64_t)gridDim.x * 4)
    topk_one(p.G + (size_t)s * p.E, p.E, p.k, p.renormalize, p.ids + (size_t)s * p.k,
             p.w + (size_t)s * p.k, lane);
}

hipError_t launch_topk(const TopkParams& p, hipStream_t st) {
  if (p.S == 0) return hipSuccess;
  int64_t want = (p.S + 3) / 4;
  const unsigned blocks = (unsigned)(want < 1024 ? want : 1024);
  hipLaunchKernelGGL(topk_softmax_kernel, dim3(blocks), dim3(256), 0, st, p);
  return hipGetLastError();
}

// ------------------------------------------------------------------ align
// Stable counting sort of the F flat assignments by expert, in three launches:
//  1. count: each wave takes one segment of kAlignSeg consecutive assignments
//     and histograms it in LDS -> seg_counts[seg][E];
//  2. scan (one workgroup): per expert, the exclusive prefix of its counts over
//     segments (in place), the total, the capacity clip, the block padding,
//     the exclusive cumsum over experts (64-bit), expert_counts,
//     num_tokens_post_padded, the sentinel padding and the per-block expert ids;
//  3. scatter: each wave walks its segment again 64 assignments at a time; a
//     lane's rank among equal experts in the step comes from ballots over the
//     expert id bits, so positions follow ascending flat index within an
//     expert and the result is deterministic.

__global__ __launch_bounds__(256) void align_count_kernel(AlignParams p) {
  __shared__ int hist[4][1024];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t seg = (int64_t)blockIdx.x * 4 + wave;
  const int E = (int)p.E;
  for (int e = lane; e < E; e += 64) hist[wave][e] = 0;
  __syncthreads();
  if (seg < p.nseg) {
    const int64_t f0 = seg * kAlignSeg;
    const int64_t f1 = min(f0 + kAlignSeg, p.F);
    for (int64_t f = f0 + lane; f < f1; f += 64) atomicAdd(&hist[wave][p.ids[f]], 1);
  }
  __syncthreads();
  if (seg < p.nseg)
    for (int e = lane; e < E; e += 64) p.seg_counts[(size_t)seg * E + e] = hist[wave][e];
}

__global__ __launch_bounds__(1024) void align_scan_kernel(AlignParams p) {
  __shared__ int64_t s_scan[1024];
  __shared__ int64_t s_off[1024];
  const int e = threadIdx.x;
  const int E = (int)p.E;
  int64_t cnt = 0;
  if (e < E) {
    // exclusive prefix over segments, in place; loads issued 16 at a time so
    // they overlap (each thread walks one expert's column)
    constexpr int kBatch = 16;
    int* col = p.seg_counts + e;
    for (int64_t s0 = 0; s0 < p.nseg; s0 += kBatch) {
      int v[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) v[u] = (s0 + u < p.nseg) ? col[(size_t)(s0 + u) * E] : 0;
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        if (s0 + u < p.nseg) col[(size_t)(s0 + u) * E] = (int)cnt;
        cnt += v[u];
      }
    }
  }
  const int64_t kept = (p.C > 0 && cnt > p.C) ? p.C : cnt;
  const int64_t pad = (kept + p.BM - 1) / p.BM * p.BM;
  // inclusive Hillis-Steele scan of pad over the 1024 threads
  s_scan[e] = pad;
  __syncthreads();
  for (int d = 1; d < 1024; d <<= 1) {
    const int64_t add = (e >= d) ? s_scan[e - d] : 0;
    __syncthreads();
    s_scan[e] += add;
    __syncthreads();
  }
  const int64_t off = s_scan[e] - pad;
  const int64_t total = s_scan[1023];
  s_off[e] = (e < E) ? off : total;
  if (e < E) {
    p.counts[e] = (int32_t)kept;
    p.offsets[e] = off;
    p.kept[e] = (int32_t)kept;
    for (int64_t i = kept; i < pad; ++i) p.sorted_ids[off + i] = (int32_t)p.F;
  }
  if (e == 0) *p.ntpp = (int32_t)total;
  __syncthreads();
  const int64_t nblocks = total / p.BM;
  for (int64_t b = e; b < nblocks; b += 1024) {
    const int64_t pos = b * p.BM;
    int lo = 0, hi = E - 1;  // last expert whose offset is <= pos
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_off[mid] <= pos)
        lo = mid;
      else
        hi = mid - 1;
    }
    p.expert_ids[b] = lo;
  }
}

__global__ __launch_bounds__(256) void align_scatter_kernel(AlignParams p) {
  __shared__ int base[4][1024];
  __shared__ int s_kept[1024];
  __shared__ int64_t s_offs[1024];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t seg = (int64_t)blockIdx.x * 4 + wave;
  const int E = (int)p.E;
  for (int e = threadIdx.x; e < E; e += 256) {
    s_kept[e] = p.kept[e];
    s_offs[e] = p.offsets[e];
  }
  if (seg < p.nseg)
    for (int e = lane; e < E; e += 64) base[wave][e] = p.seg_counts[(size_t)seg * E + e];
  __syncthreads();
  if (seg >= p.nseg) return;
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int64_t f0 = seg * kAlignSeg;
  for (int step = 0; step < kAlignSeg / 64; ++step) {
    const int64_t f = f0 + step * 64 + lane;
    const bool valid = f < p.F && f < f0 + kAlignSeg;
    const int e = valid ? p.ids[f] : 0;
    uint64_t m = __ballot(valid);
    for (int bit = 0; bit < nbits; ++bit) {
      const bool on = (e >> bit) & 1;
      const uint64_t bb = __ballot(valid && on);
      m &= on ? bb : ~bb;
    }
    int cur = 0;
    if (valid) {
      cur = base[wave][e];
      const int pos = cur + __popcll(m & below);
      if (pos < s_kept[e]) p.sorted_ids[s_offs[e] + pos] = (int32_t)f;
    }
    __builtin_amdgcn_wave_barrier();
    if (valid && lane == 63 - __clzll(m)) base[wave][e] = cur + __popcll(m);
    __builtin_amdgcn_wave_barrier();
  }
}

hipError_t launch_align(const AlignParams& p, hipStream_t st) {
  const unsigned wg = (unsigned)((p.nseg + 3) / 4);
  if (wg > 0) {
    hipLaunchKernelGGL(align_count_kernel, dim3(wg), dim3(256), 0, st, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(align_scan_kernel, dim3(1), dim3(1024), 0, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (wg > 0) {
    hipLaunchKernelGGL(align_scatter_kernel, dim3(wg), dim3(256), 0, st, p);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace moe
