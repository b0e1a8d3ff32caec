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
// Stable counting sort of the F flat assignments by expert. Up to
// kAlignSmallF assignments: one workgroup does everything (align_small_kernel).
// Beyond, three launches:
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

// Inclusive prefix sum over the 64 lanes of a wave (64-bit values).
__device__ __forceinline__ int64_t wave_inclusive_scan(int64_t x, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int64_t y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  return x;
}

// Steps common to both align paths, for one workgroup of 1024 threads whose
// thread e < E holds expert e's total count cnt: the capacity clip, the block
// padding, the exclusive cumsum of the padded counts (wave scans, then the
// wave totals), the outputs counts / offsets / kept / num_tokens_post_padded,
// the sentinel slots and the expert of every block. Leaves the offsets
// (s_off[E..1023] = total), the kept and the padded counts in LDS.
__device__ __forceinline__ void align_layout(const AlignParams& p, int64_t cnt, int64_t* s_off,
                                             int* s_kept, int* s_pad, int64_t* s_wsum) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int E = (int)p.E;
  const int64_t BM = p.BM;
  const int64_t kept = (tid < E) ? ((p.C > 0 && cnt > p.C) ? p.C : cnt) : 0;
  const int64_t pad = (kept + BM - 1) / BM * BM;
  const int64_t incl = wave_inclusive_scan(pad, lane);
  if (lane == 63) s_wsum[wave] = incl;
  __syncthreads();
  int64_t before = 0;
  for (int w = 0; w < wave; ++w) before += s_wsum[w];
  int64_t total = 0;
  for (int w = 0; w < 16; ++w) total += s_wsum[w];
  const int64_t off = before + incl - pad;
  s_off[tid] = (tid < E) ? off : total;
  s_kept[tid] = (int)kept;
  s_pad[tid] = (int)pad;
  if (tid < E) {
    p.counts[tid] = (int32_t)kept;
    p.offsets[tid] = off;
    p.kept[tid] = (int32_t)kept;
  }
  if (tid == 0) *p.ntpp = (int32_t)total;
  __syncthreads();
  // sentinels: slots kept .. pad-1 of every expert; wave w fills experts
  // w, w + 16, ..., its lanes consecutive slots (every padded count fits in
  // 32 bits: the sorted array's capacity does)
  for (int ex = wave; ex < E; ex += 16) {
    const int kx = s_kept[ex];
    const int px = s_pad[ex];
    int32_t* dst = p.sorted_ids + s_off[ex];
    for (int r = kx + lane; r < px; r += 64) dst[r] = (int32_t)p.F;
  }
  // expert of every block: the last expert whose offset is <= the block start
  const int64_t nblocks = total / BM;
  for (int64_t b = tid; b < nblocks; b += 1024) {
    const int64_t pos = b * BM;
    int lo = 0, hi = E - 1;
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

// Position of this lane's assignment (expert e, valid) among the wave's 64:
// lanes with the same expert (ballots over the expert id bits) and a lower
// lane index come first. Returns the match mask.
__device__ __forceinline__ uint64_t match_expert(int e, bool valid, int nbits) {
  uint64_t m = __ballot(valid);
  for (int bit = 0; bit < nbits; ++bit) {
    const bool on = (e >> bit) & 1;
    const uint64_t bb = __ballot(valid && on);
    m &= on ? bb : ~bb;
  }
  return m;
}

__global__ __launch_bounds__(1024) void align_scan_kernel(AlignParams p) {
  __shared__ int s_part[1024];      // per (chunk, expert) segment-count sums
  __shared__ int64_t s_wsum[16];
  __shared__ int64_t s_off[1024];
  __shared__ int s_kept[1024];
  __shared__ int s_pad[1024];
  const int tid = threadIdx.x;
  const int E = (int)p.E;
  const int64_t nseg = p.nseg;
  // per expert, exclusive prefix of its counts over the segments, in place.
  // Expert e's column is cut into T contiguous chunks of segments, one
  // thread each (thread (t, e) = t * EP + e, EP = E rounded up to a power of
  // two, T = 1024 / EP).
  int EP = 1;
  while (EP < E) EP <<= 1;
  const int T = 1024 / EP;
  const int e = tid & (EP - 1);
  const int t = tid / EP;
  const int64_t chunk = (nseg + T - 1) / T;
  const int64_t s0 = (int64_t)t * chunk;
  const int64_t s1 = min(nseg, s0 + chunk);
  int* col = p.seg_counts + e;
  constexpr int kBatch = 16;
  int local = 0;
  if (e < E) {
    for (int64_t sb = s0; sb < s1; sb += kBatch) {
      int v[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) v[u] = (sb + u < s1) ? col[(size_t)(sb + u) * E] : 0;
#pragma unroll
      for (int u = 0; u < kBatch; ++u) local += v[u];
    }
  }
  s_part[tid] = local;
  __syncthreads();
  int64_t cnt = 0;  // expert total, held by thread (0, e) = e
  if (t == 0 && e < E) {
    int run = 0;
    for (int c = 0; c < T; ++c) {
      const int x = s_part[c * EP + e];
      s_part[c * EP + e] = run;  // exclusive prefix of the chunk sums
      run += x;
    }
    cnt = run;
  }
  __syncthreads();
  if (e < E) {
    int run = s_part[tid];
    for (int64_t sb = s0; sb < s1; sb += kBatch) {
      int v[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) v[u] = (sb + u < s1) ? col[(size_t)(sb + u) * E] : 0;
#pragma unroll
      for (int u = 0; u < kBatch; ++u)
        if (sb + u < s1) {
          col[(size_t)(sb + u) * E] = run;
          run += v[u];
        }
    }
  }
  align_layout(p, cnt, s_off, s_kept, s_pad, s_wsum);
}

// The whole align in one workgroup for small F: the 16 waves take 16
// contiguous segments of the assignments, histogram them in LDS, the
// per-expert prefix over the segments stays in LDS, then each wave scatters
// its segment as the three-launch path does.
__global__ __launch_bounds__(1024) void align_small_kernel(AlignParams p) {
  __shared__ int hist[16][1024];
  __shared__ int64_t s_wsum[16];
  __shared__ int64_t s_off[1024];
  __shared__ int s_kept[1024];
  __shared__ int s_pad[1024];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int E = (int)p.E;
  const int F = (int)p.F;
  const int segw = ((F + 15) / 16 + 63) / 64 * 64;  // assignments per wave
  const int f0 = wave * segw;
  const int f1 = min(F, f0 + segw);
  for (int i = tid; i < 16 * 1024; i += 1024) (&hist[0][0])[i] = 0;
  __syncthreads();
  for (int f = f0 + lane; f < f1; f += 64) atomicAdd(&hist[wave][p.ids[f]], 1);
  __syncthreads();
  int64_t cnt = 0;
  if (tid < E) {
    int run = 0;
    for (int w = 0; w < 16; ++w) {
      const int x = hist[w][tid];
      hist[w][tid] = run;
      run += x;
    }
    cnt = run;
  }
  align_layout(p, cnt, s_off, s_kept, s_pad, s_wsum);  // ends with every LDS write visible
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int fb = f0; fb < f1; fb += 64) {
    const int f = fb + lane;
    const bool valid = f < f1;
    const int e = valid ? p.ids[f] : 0;
    const uint64_t m = match_expert(e, valid, nbits);
    int cur = 0;
    if (valid) {
      cur = hist[wave][e];
      const int pos = cur + __popcll(m & below);
      if (pos < s_kept[e]) p.sorted_ids[s_off[e] + pos] = (int32_t)f;
    }
    __builtin_amdgcn_wave_barrier();
    if (valid && lane == 63 - __clzll(m)) hist[wave][e] = cur + __popcll(m);
    __builtin_amdgcn_wave_barrier();
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
    const uint64_t m = match_expert(e, valid, nbits);
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
  if (p.F <= kAlignSmallF) {
    hipLaunchKernelGGL(align_small_kernel, dim3(1), dim3(1024), 0, st, p);
    return hipGetLastError();
  }
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
