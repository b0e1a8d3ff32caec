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
// Beyond, two launches (the vLLM align PR's multi-block form, "Implementation"
// steps 2-3, with the layout computed where it is used):
//  1. count: each wave takes one segment of kAlignSeg consecutive assignments
//     and histograms it in LDS -> seg_counts[seg][E];
//  2. layout and scatter: every workgroup (4 waves, 4 segments) reads all
//     segment counts and computes, itself, each expert's total, the
//     capacity clip, the block padding and the exclusive cumsum over experts
//     (the same values in every workgroup), and its segments' exclusive
//     prefix over the earlier segments. It writes its share of the outputs
//     that do not depend on the segments (expert_counts and
//     num_tokens_post_padded from workgroup 0, a slice of the sentinel padding
//     and of the per-block expert ids from each), then each wave scatters its
//     segment 64 assignments at a time; a lane's rank among equal experts in
//     the step comes from ballots over the expert id bits, so positions follow
//     ascending flat index within an expert and the result is deterministic.
// No workgroup waits for another, and nothing in the workspace needs a
// reset between calls (a grid-wide barrier or a look-back over workgroups
// would need device state that starts at zero on every call, graph replays
// included).

constexpr int kAlignPer = kAlignSeg / 64;  // assignments per lane and segment

// This wave's segment of the assignments, kAlignPer per lane (lane l holds
// assignments f0 + 64 u + l), loaded at once; -1 past the end.
__device__ __forceinline__ void load_segment(const AlignParams& p, int64_t seg, int lane,
                                             int (&v)[kAlignPer]) {
  const int64_t f0 = seg * kAlignSeg;
#pragma unroll
  for (int u = 0; u < kAlignPer; ++u) {
    const int64_t f = f0 + u * 64 + lane;
    v[u] = (seg < p.nseg && f < p.F) ? p.ids[f] : -1;
  }
}

__global__ __launch_bounds__(256) void align_count_kernel(AlignParams p) {
  __shared__ int hist[4][1024];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t seg = (int64_t)blockIdx.x * 4 + wave;
  const int E = (int)p.E;
  int v[kAlignPer];
  load_segment(p, seg, lane, v);
  for (int e = lane; e < E; e += 64) hist[wave][e] = 0;
  __syncthreads();
#pragma unroll
  for (int u = 0; u < kAlignPer; ++u)
    if (v[u] >= 0) atomicAdd(&hist[wave][v[u]], 1);
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
// NBITS (the bits of the largest expert id) is a compile-time count, so the
// ballots unroll into straight-line code (measured: with a loop over a run-time
// bit count, the ranks of a 512-assignment segment took 3.2 µs).
template <int NBITS>
__device__ __forceinline__ uint64_t match_expert(int e, bool valid) {
  uint64_t m = __ballot(valid);
#pragma unroll
  for (int bit = 0; bit < NBITS; ++bit) {
    const bool on = (e >> bit) & 1;
    const uint64_t bb = __ballot(valid && on);
    m &= on ? bb : ~bb;
  }
  return m;
}

// Bits needed for expert ids 0 .. E-1.
inline int expert_bits(int64_t E) {
  int nbits = 0;
  while (((int64_t)1 << nbits) < E) ++nbits;
  return nbits;
}

// The whole align in one workgroup for small F: the 16 waves take 16
// contiguous segments of the assignments, histogram them in LDS, the
// per-expert prefix over the segments stays in LDS, then each wave scatters
// its segment as the three-launch path does.
template <int NBITS>
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
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int fb = f0; fb < f1; fb += 64) {
    const int f = fb + lane;
    const bool valid = f < f1;
    const int e = valid ? p.ids[f] : 0;
    const uint64_t m = match_expert<NBITS>(e, valid);
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

// Launch 2 of the multi-workgroup align (see above). Workgroup g holds
// segments 4g .. 4g+3, one per wave.
template <int NBITS>
__global__ __launch_bounds__(256) void align_scatter_kernel(AlignParams p) {
  __shared__ int s_part[4][1024];   // per quarter of the segments: counts summed
  __shared__ int s_bef[4][1024];    // ... over the segments before this workgroup's
  __shared__ int s_base[4][1024];   // per wave: expert's assignments before its segment
  __shared__ int s_kept[1024];
  __shared__ int64_t s_off[1024];
  __shared__ int64_t s_wsum[4];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int E = (int)p.E;
  const int64_t nseg = p.nseg;
  const int64_t seg0 = (int64_t)blockIdx.x * 4;
  int v[kAlignPer];
  load_segment(p, seg0 + wave, lane, v);  // in flight while the layout is computed
  // per expert, its counts summed over Q parts of the segments (Q = 4, 2 or
  // 1 as E allows): thread (q, e) = q * EP + e, EP = E rounded up to a power
  // of two; with EP >= 256 one part, thread t taking experts t, t + 256, ...
  int EP = 1;
  while (EP < E) EP <<= 1;
  const int Q = EP >= 256 ? 1 : (256 / EP < 4 ? 256 / EP : 4);
  const int q = EP >= 256 ? 0 : tid / EP;
  const int64_t per = (nseg + Q - 1) / Q;
  const int64_t s0 = (int64_t)q * per;
  const int64_t s1 = min(nseg, s0 + per);
  const int e_first = EP >= 256 ? tid : (q < Q ? tid % EP : E);
  const int e_step = EP >= 256 ? 256 : E;  // one expert per thread below 256
  for (int e = e_first; e < E; e += e_step) {
    int tot = 0, bef = 0;
    constexpr int kBatch = 16;
    for (int64_t sb = s0; sb < s1; sb += kBatch) {
      int c[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u)
        c[u] = (sb + u < s1) ? p.seg_counts[(size_t)(sb + u) * E + e] : 0;
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int64_t sg = sb + u;
        tot += c[u];
        if (sg < seg0) bef += c[u];
        if (sg >= seg0 && sg < seg0 + 4 && sg < s1) s_base[sg - seg0][e] = c[u];
      }
    }
    s_part[q][e] = tot;
    s_bef[q][e] = bef;
  }
  __syncthreads();
  // totals, the capacity clip, the padding, and the exclusive padded cumsum
  // over experts: thread t holds experts 4t .. 4t+3
  // (32-bit arithmetic: a count and its padding fit, as the sorted array's
  // capacity does; 64-bit division is a long software routine on the GPU)
  const uint32_t bm = (uint32_t)p.BM;
  int64_t pad4[4], kept4[4], sum = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = 4 * tid + j;
    int64_t cnt = 0;
    if (e < E)
      for (int qq = 0; qq < Q; ++qq) cnt += s_part[qq][e];
    kept4[j] = (p.C > 0 && cnt > p.C) ? p.C : cnt;
    pad4[j] = (int64_t)(((uint32_t)kept4[j] + bm - 1) / bm * bm);
    sum += pad4[j];
  }
  const int64_t incl = wave_inclusive_scan(sum, lane);
  if (lane == 63) s_wsum[wave] = incl;
  __syncthreads();
  int64_t run = incl - sum;
  for (int w = 0; w < wave; ++w) run += s_wsum[w];
  const int64_t total = s_wsum[0] + s_wsum[1] + s_wsum[2] + s_wsum[3];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = 4 * tid + j;
    if (e < E) {
      s_off[e] = run;
      s_kept[e] = (int)kept4[j];
      if (blockIdx.x == 0) p.counts[e] = (int32_t)kept4[j];
    }
    run += pad4[j];
  }
  if (blockIdx.x == 0 && tid == 0) *p.ntpp = (int32_t)total;
  // each wave's base: the expert's assignments in all segments before its own
  for (int e = tid; e < E; e += 256) {
    int b = 0;
    for (int qq = 0; qq < Q; ++qq) b += s_bef[qq][e];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int c = (seg0 + w < nseg) ? s_base[w][e] : 0;
      s_base[w][e] = b;
      b += c;
    }
  }
  __syncthreads();
  // this workgroup's share of the sentinels (experts e = g, g + G, ...) and of
  // the block experts (blocks g, g + G, ...)
  const int64_t G = gridDim.x;
  for (int64_t ex = blockIdx.x + G * wave; ex < E; ex += 4 * G) {
    const uint32_t kx = (uint32_t)s_kept[ex];
    const uint32_t px = (kx + bm - 1) / bm * bm;
    int32_t* dst = p.sorted_ids + s_off[ex];
    for (uint32_t r = kx + lane; r < px; r += 64) dst[r] = (int32_t)p.F;
  }
  const int64_t nblocks = (int64_t)((uint64_t)total / bm);
  for (int64_t b = blockIdx.x + G * tid; b < nblocks; b += 256 * G) {
    const int64_t pos = b * (int64_t)bm;
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
  // scatter this wave's segment. The steps' ballot ranks and the experts'
  // offsets do not depend on each other: all first; the only serial chain
  // left is the per-expert running base in LDS.
  const int64_t seg = seg0 + wave;
  if (seg >= nseg) return;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int64_t f0 = seg * kAlignSeg;
  int rank[kAlignPer], nrun[kAlignPer], kept[kAlignPer];
  bool lead[kAlignPer];
  int64_t off[kAlignPer];
#pragma unroll
  for (int u = 0; u < kAlignPer; ++u) {
    const bool valid = v[u] >= 0;
    const int e = valid ? v[u] : 0;
    const uint64_t m = match_expert<NBITS>(e, valid);
    rank[u] = __popcll(m & below);
    nrun[u] = __popcll(m);
    lead[u] = valid && lane == 63 - __clzll(m);
    off[u] = s_off[e];
    kept[u] = valid ? s_kept[e] : 0;
  }
  int pos[kAlignPer];
#pragma unroll
  for (int u = 0; u < kAlignPer; ++u) {
    const int e = v[u] >= 0 ? v[u] : 0;
    const int cur = s_base[wave][e];
    pos[u] = cur + rank[u];
    __builtin_amdgcn_wave_barrier();
    if (lead[u]) s_base[wave][e] = cur + nrun[u];
    __builtin_amdgcn_wave_barrier();
  }
#pragma unroll
  for (int u = 0; u < kAlignPer; ++u)
    if (pos[u] < kept[u]) p.sorted_ids[off[u] + pos[u]] = (int32_t)(f0 + u * 64 + lane);
}

template <int NBITS>
static hipError_t launch_align_t(const AlignParams& p, hipStream_t st) {
  if (p.F <= kAlignSmallF) {
    hipLaunchKernelGGL(align_small_kernel<NBITS>, dim3(1), dim3(1024), 0, st, p);
    return hipGetLastError();
  }
  // F > kAlignSmallF >= 1: at least one segment
  const unsigned wg = (unsigned)((p.nseg + 3) / 4);
  hipLaunchKernelGGL(align_count_kernel, dim3(wg), dim3(256), 0, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(align_scatter_kernel<NBITS>, dim3(wg), dim3(256), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_align(const AlignParams& p, hipStream_t st) {
  switch (expert_bits(p.E)) {  // E <= kMaxE = 1024
    case 0: return launch_align_t<0>(p, st);
    case 1: return launch_align_t<1>(p, st);
    case 2: return launch_align_t<2>(p, st);
    case 3: return launch_align_t<3>(p, st);
    case 4: return launch_align_t<4>(p, st);
    case 5: return launch_align_t<5>(p, st);
    case 6: return launch_align_t<6>(p, st);
    case 7: return launch_align_t<7>(p, st);
    case 8: return launch_align_t<8>(p, st);
    case 9: return launch_align_t<9>(p, st);
    default: return launch_align_t<10>(p, st);
  }
}

}  // namespace moe
