// GEMM kernels of the MoE layer: gate scores (with the top-k fused, or split
// along H), the two persistent grouped GEMMs of the expert FFN (up/gate with
// a SwiGLU epilogue; down writing each kept row to its fp32 slot, or adding
// it with atomics), the streaming down kernel for decode-sized tiles, both
// GEMMs in one launch (MOE_FUSED_LAUNCH), the setup fill, the ordered slot
// combine and the output cast.
//
// Persistent scheduling (Weave review, sections 2.1-2.2 and 5.1): the work of
// a grouped GEMM is cut into tile tasks (m-block of BM sorted rows, n-tile of
// BN output columns); a grid of about one workgroup per CU claims tasks with
// an atomic counter until none are left, instead of a fixed share of CUs per
// expert. Task count depends on the routing and is read on the device (no
// host synchronisation). On MI355X the task list is cut into 8 contiguous
// ranges, one per XCD (workgroup i runs on XCD i % 8); a workgroup claims from
// its own XCD's range first, so tasks that share weight and activation tiles
// run on CUs that share one L2, and moves on to the other ranges when its
// own is empty (work stealing keeps the tail balanced).
//
// Inside a range the tasks of a group of kGroupBlocks consecutive m-blocks are
// ordered n-tile-major: tasks running side by side share both the A rows of
// a few m-blocks and the weight strips of a few n-tiles. With about one
// m-block per expert (nothing to share across m-blocks) each m-block's
// n-tiles run back to back instead.
#include <algorithm>
#include <type_traits>

#include "gemm_direct.h"
#include "gemm_tile.h"
#include "moe_sched.h"
#include "topk.h"

namespace moe {

// Tile core of the persistent grouped GEMMs: bf16 loads straight into LDS
// (gemm_direct.h); fp32 stages through registers (gemm_tile.h).
// BS (bf16 core only): the weights are streamed once (non-temporal loads).
template <typename T, int BM, int NB, int STAGING, bool BS = false>
struct TileSel {
  using type = TileGemm<T, BM, 128, NB, false, STAGING>;
};
// Stage K: 32 for 256-row tiles (four 32 KB stages, three in flight), 64
// otherwise (measured). MOE_STAGE_K overrides it for all tiles.
#ifndef MOE_STAGE_K
#define MOE_STAGE_K 0
#endif
template <int BM>
constexpr int stage_k() {
  return MOE_STAGE_K > 0 ? MOE_STAGE_K : (BM >= 256 ? 32 : 64);
}
// MFMA shape of the persistent GEMMs' cores for tiles of BM rows (and of
// their half tiles, which must add in the same order).
template <int BM>
constexpr int mfma_shape() {
  return MOE_MFMA32 && BM >= 128 ? 32 : 16;
}
// A in 64-K stages (whole 128-byte lines of the gathered token rows) for the
// up/gate tiles of 256 rows (STAGING 2 marks the up/gate GEMM): 1 for the
// tiles that stream their weights (measured faster there, slower where the
// weights stay in the caches), 2 for every such tile, 0 for none.
#ifndef MOE_A64
#define MOE_A64 1
#endif
template <int BM, int NB, int STAGING, bool BS>
constexpr bool a64_tile() {
  return STAGING == 2 && BM >= 256 && stage_k<BM>() == 32 && (MOE_A64 == 2 || (MOE_A64 == 1 && BS));
}
template <int BM, int NB, int STAGING, bool BS>
struct TileSel<bf16_t, BM, NB, STAGING, BS> {
  using type = TileGemmDirect<BM, NB, 8, stage_k<BM>(), 144 * 1024, BS, false, mfma_shape<BM>(),
                              a64_tile<BM, NB, STAGING, BS>()>;
};

template <typename TG>
constexpr bool is_direct() {
  return TG::DIRECT;
}

// Run the K loop of tile core TG. The direct core gets the static LDS ring
// and skips each wave's row blocks past the last row for which valid(r)
// holds; the register-staged core uses the dynamic buffer and computes every
// row.
template <typename TG, typename Valid>
__device__ __forceinline__ void run_mainloop(TG& g, char* dyn, int64_t K, Valid valid) {
  trace_stamp(1);
  if constexpr (is_direct<TG>()) {
    g.mainloop(lds_ring<TG>(), K, g.active_blocks(valid));
  } else {
    g.mainloop(dyn, K);
  }
  trace_stamp(2);
}

constexpr int kGateBM = 64;
constexpr int kGateBN = 64;

// ------------------------------------------------------------------ gate GEMM
// G[s][e] = sum_h A[s][h] * Wr[h][e] (+ bias[e]), fp32 out. One tile per
// workgroup (not persistent: the gate has no routing-dependent imbalance).
template <typename T, bool RAGGED>
__global__ __launch_bounds__(256) void gate_gemm_kernel(GateParams p) {
  using TG = TileGemm<T, kGateBM, kGateBN, 1, RAGGED>;
  __shared__ __align__(16) char smem[TG::LDS_BYTES];
  const int64_t n_tiles = (p.E + kGateBN - 1) / kGateBN;
  const int64_t m0 = (int64_t)(blockIdx.x / n_tiles) * kGateBM;
  const int64_t n0 = (int64_t)(blockIdx.x % n_tiles) * kGateBN;
  TG g;
  const char* Bm[1] = {reinterpret_cast<const char*>(p.Wr)};
  const int64_t S = p.S, H = p.H;
  const uint32_t bb[1] = {(uint32_t)(H * p.E * sizeof(T))};
  const int64_t nc[1] = {p.E - n0};
  g.setup(p.A, (uint32_t)(S * H * sizeof(T)), [&](int r) -> uint32_t {
    const int64_t s = m0 + r;
    return s < S ? (uint32_t)(s * H * sizeof(T)) : kOob;
  }, Bm, bb, p.E, n0, nc);
  g.mainloop(smem, p.H);
  g.for_each([&](int, int row, int col, float v) {
    const int64_t s = m0 + row, e = n0 + col;
    if (s < p.S && e < p.E) {
      float out = v;
      if (p.bias) out = out + p.bias[e];
      p.G[(size_t)s * p.E + e] = out;
    }
  });
}

// bf16 gate scores on the LDS-direct core (E a multiple of 8): BMG-row tiles,
// 128 experts per tile, 72 KB of LDS so two workgroups share a CU.
template <int BMG>
__global__ __launch_bounds__(512, 2) void gate_gemm_direct_kernel(GateParams p) {
  using TG = TileGemmDirect<BMG, 1, 8, 64, 72 * 1024>;
  __shared__ __align__(16) char ring[TG::LDS_BYTES];
  const int64_t n_tiles = (p.E + TG::BN - 1) / TG::BN;
  const int64_t m0 = (int64_t)(blockIdx.x / n_tiles) * BMG;
  const int64_t n0 = (int64_t)(blockIdx.x % n_tiles) * TG::BN;
  TG g;
  const char* Bm[1] = {reinterpret_cast<const char*>(p.Wr)};
  const int64_t S = p.S, H = p.H;
  const uint32_t bb[1] = {(uint32_t)(H * p.E * sizeof(bf16_t))};
  const int64_t nc[1] = {p.E - n0};
  g.setup(p.A, (uint32_t)(S * H * sizeof(bf16_t)), [&](int r) -> uint32_t {
    const int64_t s = m0 + r;
    return s < S ? (uint32_t)(s * H * sizeof(bf16_t)) : kOob;
  }, Bm, bb, p.E, n0, nc);
  g.mainloop(ring, p.H);
  g.for_each([&](int, int row, int col, float v) {
    const int64_t s = m0 + row, e = n0 + col;
    if (s < p.S && e < p.E) {
      float out = v;
      if (p.bias) out = out + p.bias[e];
      p.G[(size_t)s * p.E + e] = out;
    }
  });
}

template <int BMG>
static hipError_t launch_gate_direct(const GateParams& p, hipStream_t st) {
  const int64_t tiles = ((p.S + BMG - 1) / BMG) * ((p.E + 127) / 128);
  hipLaunchKernelGGL(gate_gemm_direct_kernel<BMG>, dim3((unsigned)tiles), dim3(512), 0, st, p);
  return hipGetLastError();
}

// Fused gate + top-k (the gate producing the routing table directly): one
// workgroup computes the scores of BMG tokens for all E <= NB * 128 experts
// on the LDS-direct core, stages the fp32 score tile (bias added) in LDS,
// writes it to G coalesced, and each wave ranks its tokens from LDS.
// Largest k whose weights the fused gate computes in one pass per wave.
constexpr int kTopkBatchK = 8;

template <int BMG, int NB>
__global__ __launch_bounds__(512, 1) void gate_topk_kernel(GateParams gp, TopkParams tp) {
  using TG = TileGemmDirect<BMG, NB, 8, 64, 120 * 1024>;
  static_assert(TG::LDS_BYTES >= BMG * NB * 128 * (int)sizeof(float), "score tile fits the ring");
  __shared__ __align__(16) char ring[TG::LDS_BYTES];
  const int64_t m0 = (int64_t)blockIdx.x * BMG;
  const int64_t S = gp.S, H = gp.H, E = gp.E;
  TG g;
  const char* Bm[NB];
  uint32_t bb[NB];
  int64_t nc[NB];
#pragma unroll
  for (int m = 0; m < NB; ++m) {
    Bm[m] = reinterpret_cast<const char*>(gp.Wr) + (size_t)m * 128 * sizeof(bf16_t);
    bb[m] = (uint32_t)(H * E * sizeof(bf16_t)) - (uint32_t)(m * 128 * sizeof(bf16_t));
    nc[m] = E - m * 128;
  }
  g.setup(gp.A, (uint32_t)(S * H * sizeof(bf16_t)), [&](int r) -> uint32_t {
    const int64_t s = m0 + r;
    return s < S ? (uint32_t)(s * H * sizeof(bf16_t)) : kOob;
  }, Bm, bb, E, 0, nc);
  g.mainloop(ring, H);
  __syncthreads();  // every wave is done with the LDS ring
  float* tile = reinterpret_cast<float*>(ring);  // [BMG][E] fp32 scores
  g.for_each([&](int m, int row, int col, float v) {
    const int64_t e = m * 128 + col;
    if (e < E) tile[row * E + e] = gp.bias ? v + gp.bias[e] : v;
  });
  __syncthreads();
  const int rows = (int)min<int64_t>(BMG, S - m0);
  for (int i = threadIdx.x; i < rows * E; i += 512) gp.G[(size_t)m0 * E + i] = tile[i];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  if (tp.renormalize && tp.k <= kTopkBatchK) {
    // choices token by token, then the weights of all the wave's tokens in one
    // pass (topk_weights_renorm)
    constexpr int NT = BMG / 8;  // tokens per wave
    __shared__ float s_sel[8][NT * kTopkBatchK];
    __shared__ double s_e[8][NT * kTopkBatchK];
    const int k = (int)tp.k;
    int nt = 0;
    for (int r = wave; r < rows; r += 8, ++nt) {
      float my_sel, top;
      int my_id;
      topk_select(tile + r * E, (int)E, k, lane, my_sel, my_id, top);
      if (lane < k) {
        tp.ids[(m0 + r) * k + lane] = my_id;
        s_sel[wave][nt * k + lane] = my_sel;
      }
    }
    topk_weights_renorm(s_sel[wave], s_e[wave], nt, k, m0 + wave, 8, tp.w, lane);
  } else {
    for (int r = wave; r < rows; r += 8) {
      const int64_t s = m0 + r;
      topk_one(tile + r * E, E, tp.k, tp.renormalize, tp.ids + s * tp.k, tp.w + s * tp.k, lane);
    }
  }
}

template <int BMG, int NB>
static hipError_t launch_gate_topk_t(const GateParams& gp, const TopkParams& tp,
                                     hipStream_t st) {
  const int64_t tiles = (gp.S + BMG - 1) / BMG;
  hipLaunchKernelGGL((gate_topk_kernel<BMG, NB>), dim3((unsigned)tiles), dim3(512), 0, st, gp,
                     tp);
  return hipGetLastError();
}

bool gate_topk_fusable(const GateParams& gp, int dtype) {
  return dtype == 1 && gp.E % 8 == 0 && gp.E <= 256;
}

hipError_t launch_gate_topk(const GateParams& gp, const TopkParams& tp, hipStream_t st) {
  if (gp.S == 0) return hipSuccess;
  const bool two = gp.E > 128;
  // enough row tiles to cover the CUs, else smaller ones
  if (gp.S >= 64 * 256) return two ? launch_gate_topk_t<64, 2>(gp, tp, st)
                                   : launch_gate_topk_t<64, 1>(gp, tp, st);
  if (gp.S >= 32 * 256) return two ? launch_gate_topk_t<32, 2>(gp, tp, st)
                                   : launch_gate_topk_t<32, 1>(gp, tp, st);
  return two ? launch_gate_topk_t<16, 2>(gp, tp, st) : launch_gate_topk_t<16, 1>(gp, tp, st);
}

// Split gate (bf16, E <= 256, E % 8 == 0): when the fused kernel would have
// few row tiles, or a long K loop per tile, the H loop is cut into `splits`
// ranges of kc elements. gate_split_kernel writes each range's fp32 partial
// scores to part[split][S][E]; gate_reduce_topk_kernel adds them in split
// order (a fixed order: the same scores on every call), adds the bias,
// writes G and ranks each token from LDS.
GateSplit gate_split_plan(int64_t S, int64_t H, int64_t E, int dtype) {
  GateSplit g{0, 1, 0};
  if (dtype != 1 || E % 8 != 0 || E > 256 || S < 1 || H < 1) return g;
  // the fused kernel's row tiles (see launch_gate_topk)
  const int64_t bm_fused = S >= 64 * 256 ? 64 : (S >= 32 * 256 ? 32 : 16);
  const int64_t fused_tiles = (S + bm_fused - 1) / bm_fused;
  const int64_t stages = (H + 63) / 64;
  if (fused_tiles >= 256 && stages <= 64) return g;  // fused kernel fills the GPU
  const int bmg = S >= 4096 ? 64 : 16;
  const int64_t tiles = (S + bmg - 1) / bmg * ((E + 127) / 128);
  int64_t splits = std::max<int64_t>(1, 512 / tiles);
  splits = std::min<int64_t>(splits, std::max<int64_t>(1, stages / 2));  // >= 2 stages each
  splits = std::min<int64_t>(splits, 64);
  if (splits < 2) return g;
  const int64_t kc = (stages + splits - 1) / splits * 64;
  g.bmg = bmg;
  g.splits = (int)((H + kc - 1) / kc);  // no empty split
  g.kc = kc;
  return g.splits >= 2 ? g : GateSplit{0, 1, 0};
}

template <int BMG>
__global__ __launch_bounds__(512, 2) void gate_split_kernel(GateParams p, float* part,
                                                            int64_t kc) {
  using TG = TileGemmDirect<BMG, 1, 8, 64, 72 * 1024>;
  __shared__ __align__(16) char ring[TG::LDS_BYTES];
  const int64_t n_tiles = (p.E + TG::BN - 1) / TG::BN;
  const int64_t tiles = (p.S + BMG - 1) / BMG * n_tiles;
  const int64_t sp = blockIdx.x / tiles;  // split (tiles of one split share W_router rows)
  const int64_t tile = blockIdx.x - sp * tiles;
  const int64_t m0 = (tile / n_tiles) * BMG;
  const int64_t n0 = (tile % n_tiles) * TG::BN;
  const int64_t k0 = sp * kc;
  const int64_t K = min(kc, p.H - k0);
  const int64_t S = p.S, H = p.H, E = p.E;
  TG g;
  const char* Bm[1] = {reinterpret_cast<const char*>(p.Wr) + (size_t)k0 * E * sizeof(bf16_t)};
  const uint32_t bb[1] = {(uint32_t)((H - k0) * E * sizeof(bf16_t))};
  const int64_t nc[1] = {E - n0};
  const bf16_t* a0 = reinterpret_cast<const bf16_t*>(p.A) + k0;
  g.setup(a0, (uint32_t)((S * H - k0) * sizeof(bf16_t)), [&](int r) -> uint32_t {
    const int64_t s = m0 + r;
    return s < S ? (uint32_t)(s * H * sizeof(bf16_t)) : kOob;
  }, Bm, bb, E, n0, nc);
  g.mainloop(ring, K);
  float* out = part + (size_t)sp * S * E;
  g.for_each([&](int, int row, int col, float v) {
    const int64_t s = m0 + row, e = n0 + col;
    if (s < S && e < E) out[(size_t)s * E + e] = v;
  });
}

__global__ __launch_bounds__(256) void gate_reduce_topk_kernel(const float* part, int splits,
                                                               GateParams gp, TopkParams tp) {
  __shared__ float s_row[4][256];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t S = gp.S, E = gp.E;
  // a uniform loop (the block barriers below): 4 tokens per step
  for (int64_t base = (int64_t)blockIdx.x * 4; base < S; base += (int64_t)gridDim.x * 4) {
    const int64_t s = base + wave;
    if (s < S) {
      // lane: experts lane + 64 i (i < 4); the partials of 8 splits are
      // loaded together, then added in split order
      float acc[4];
      const float* p0 = part + (size_t)s * E + lane;
      const size_t step = (size_t)S * E;  // one split
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = (lane + 64 * i < E) ? p0[64 * i] : 0.f;
      for (int j0 = 1; j0 < splits; j0 += 8) {
        float v[8][4];
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            v[u][i] = (j0 + u < splits && lane + 64 * i < E) ? p0[(j0 + u) * step + 64 * i] : 0.f;
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (j0 + u < splits)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] += v[u][i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t e = lane + 64 * i;
        if (e < E) {
          const float x = gp.bias ? acc[i] + gp.bias[e] : acc[i];
          s_row[wave][e] = x;
          gp.G[(size_t)s * E + e] = x;
        }
      }
    }
    __syncthreads();
    if (s < S)
      topk_one(s_row[wave], E, tp.k, tp.renormalize, tp.ids + s * tp.k, tp.w + s * tp.k, lane);
    __syncthreads();
  }
}

hipError_t launch_gate_split(const GateParams& gp, const TopkParams& tp, const GateSplit& plan,
                             float* part, hipStream_t st) {
  const int64_t tiles = (gp.S + plan.bmg - 1) / plan.bmg * ((gp.E + 127) / 128);
  const unsigned grid = (unsigned)(tiles * plan.splits);
  if (plan.bmg == 64)
    hipLaunchKernelGGL(gate_split_kernel<64>, dim3(grid), dim3(512), 0, st, gp, part, plan.kc);
  else
    hipLaunchKernelGGL(gate_split_kernel<16>, dim3(grid), dim3(512), 0, st, gp, part, plan.kc);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t want = (gp.S + 3) / 4;
  const unsigned blocks = (unsigned)(want < 1024 ? want : 1024);
  hipLaunchKernelGGL(gate_reduce_topk_kernel, dim3(blocks), dim3(256), 0, st, part, plan.splits,
                     gp, tp);
  return hipGetLastError();
}

hipError_t launch_gate(const GateParams& p, int dtype, hipStream_t st) {
  if (p.S == 0) return hipSuccess;
  const bool ragged = (p.E % 8) != 0;
  if (dtype == 1 && !ragged) {
    // enough row tiles to cover the CUs, else smaller ones
    const int64_t ntile = (p.E + 127) / 128;
    if (((p.S + 63) / 64) * ntile >= 256) return launch_gate_direct<64>(p, st);
    if (((p.S + 31) / 32) * ntile >= 128) return launch_gate_direct<32>(p, st);
    return launch_gate_direct<16>(p, st);
  }
  const int64_t tiles = ((p.S + kGateBM - 1) / kGateBM) * ((p.E + kGateBN - 1) / kGateBN);
  if (dtype == 1) {
    hipLaunchKernelGGL((gate_gemm_kernel<bf16_t, true>), dim3((unsigned)tiles), dim3(256), 0, st, p);
  } else {
    if (ragged)
      hipLaunchKernelGGL((gate_gemm_kernel<float, true>), dim3((unsigned)tiles), dim3(256), 0, st, p);
    else
      hipLaunchKernelGGL((gate_gemm_kernel<float, false>), dim3((unsigned)tiles), dim3(256), 0, st, p);
  }
  return hipGetLastError();
}

// The half-tile core of a persistent kernel with BM-row tiles: the LDS-direct
// core at BM/2 rows, where BM/2 still gives each SIMD one wave of each row
// group (bf16, BM >= 64); void where tasks are not split.
template <typename T, int BM, int NB, int STAGING, bool BS>
struct HalfSel {
  using type = void;
};
template <int BM, int NB, int STAGING, bool BS>
struct HalfSel<bf16_t, BM, NB, STAGING, BS> {
  using type = std::conditional_t<(BM >= 64),
                                  TileGemmDirect<BM / 2, NB, 8, stage_k<BM / 2>(), 144 * 1024, BS,
                                                 false, mfma_shape<BM>()>,
                                  void>;
};

// ---------------------------------------------------- quota scheduler
// Ablation baseline (the Weave review's comparator, sections 1.2-1.3: a fixed
// number of SMs per expert): workgroup g serves only the experts
// [g*E/grid, max(g*E/grid + 1, (g+1)*E/grid)), so each expert gets about
// grid/E workgroups whatever its load, and claims that expert's tasks from a
// per-expert counter; afterwards, shared-expert tasks from one counter. The
// returned task ids are those of the queue scheduler (same tiles, same
// results).
struct QuotaState {
  int e, e_hi;
  int64_t b0, nblk;  // current expert's blocks; b0 < 0: not looked up yet
  int phase;         // 0 routed, 1 shared, 2 done
};

__device__ __forceinline__ QuotaState quota_init(int64_t E) {
  QuotaState st;
  const int64_t g = blockIdx.x, G = gridDim.x;
  st.e = (int)(g * E / G);
  st.e_hi = (int)max(g * E / G + 1, (g + 1) * E / G);
  st.b0 = -1;
  st.nblk = 0;
  st.phase = 0;
  return st;
}

// first block of the sorted expert ids with expert >= e (expert_ids ascend)
__device__ __forceinline__ int64_t first_block(const int32_t* expert_ids, int64_t nb, int e) {
  int64_t lo = 0, hi = nb;
  while (lo < hi) {
    const int64_t mid = (lo + hi) >> 1;
    if (expert_ids[mid] < e)
      lo = mid + 1;
    else
      hi = mid;
  }
  return lo;
}

// Task id of (m-block b, n-tile j) in the queue scheduler's order (the
// inverse of decode_task).
__device__ __forceinline__ int64_t encode_task(int64_t b, int64_t j, int64_t nb, int64_t nn,
                                               int64_t gb) {
  const int64_t grp = b / gb;
  const int64_t b0 = grp * gb;
  const int64_t gsz = min(gb, nb - b0);
  return grp * gb * nn + j * gsz + (b - b0);
}

__device__ __forceinline__ int64_t claim_quota(const ForwardParams& p, const TaskSpace& ts,
                                               int* ctr, QuotaState& st) {
  for (;;) {
    if (st.phase == 0) {
      if (st.e >= st.e_hi) {
        st.phase = 1;
        continue;
      }
      if (st.b0 < 0) {
        st.b0 = first_block(p.expert_ids, ts.nb_r, st.e);
        st.nblk = first_block(p.expert_ids, ts.nb_r, st.e + 1) - st.b0;
      }
      const int64_t u = atomicAdd(&ctr[st.e], 1);
      if (u < st.nblk * ts.nn_r)
        return encode_task(st.b0 + u / ts.nn_r, u % ts.nn_r, ts.nb_r, ts.nn_r, ts.gb_r);
      ++st.e;
      st.b0 = -1;
      continue;
    }
    if (st.phase == 1) {
      st.phase = 2;
      if (ts.total > ts.t_r) {
        const int64_t u = atomicAdd(&ctr[kQuotaStride - 1], 1);
        if (ts.t_r + u < ts.total) {
          st.phase = 1;
          return ts.t_r + u;
        }
      }
    }
    return -1;
  }
}

// ---------------------------------------------------- up/gate GEMM + SwiGLU
// Routed task (m-block b of expert e = expert_ids[b], n-tile j):
//   h[b*BM + r][n] = SiLU(A_t . W_up^e[:, n]) * (A_t . W_gate^e[:, n]),
//   t = sorted_ids[b*BM + r] / k; sentinel rows are skipped.
// Shared task (m-block b over tokens b*BM + r < S): the same with Ws_up,
// Ws_gate into hs.
template <typename T, int BM, int NB, int STAGING>
constexpr int tile_threads() {
  return TileSel<T, BM, NB, STAGING>::type::THREADS;
}

// One up/gate task t of the task space ts (m-blocks of BMB rows), run by
// the whole workgroup on tile core TG: a whole block (TG::BM = BMB, row0 = 0)
// or the rows row0 .. row0 + TG::BM of it. Returns the readiness index of its
// m-block (b routed, nb_r + b shared).
template <typename T, int BMB, int BN, typename TG>
__device__ __forceinline__ int64_t upgate_task(const ForwardParams& p, const TaskSpace& ts,
                                               int64_t t, int row0, TG& g, char* smem,
                                               int* s_tok) {
  static_assert(TG::BN == BN, "tile width");
  constexpr int BM = TG::BM;  // tile rows
  {
    const bool shared = t >= ts.t_r;
    int64_t b, j;
    if (!shared)
      decode_task(t, ts.nb_r, ts.nn_r, ts.gb_r, b, j);
    else
      decode_task(t - ts.t_r, ts.nb_s, ts.nn_s, kGroupBlocks, b, j);
    // the block's expert, loaded before the row barrier so that its latency
    // overlaps the sorted ids' (it does not depend on them)
    const int64_t e_blk = shared ? -1 : (int64_t)__builtin_amdgcn_readfirstlane(p.expert_ids[b]);
    if (threadIdx.x < BM) {
      const int r = threadIdx.x;
      int tok;
      if (!shared) {
        const int f = p.sorted_ids[b * BMB + row0 + r];
        tok = f < p.F ? (int)(f / p.k) : -1;
        // slot combine: the first n-tile's task of a block marks its kept
        // assignments (the flags were cleared by the setup kernel)
        if (!p.atomic_combine && j == 0 && f < p.F) p.kept[f] = 1;
      } else {
        const int64_t s = b * BMB + row0 + r;
        tok = s < p.S ? (int)s : -1;
      }
      s_tok[r] = tok;
    }
    __syncthreads();
    const int64_t N = shared ? p.Ds : p.D;
    const int64_t n0 = j * BN;
    const char* Bm[2];
    if (!shared) {
      const size_t off = (size_t)e_blk * p.H * p.D * sizeof(T);
      Bm[0] = reinterpret_cast<const char*>(p.Wu) + off;
      Bm[1] = reinterpret_cast<const char*>(p.Wg) + off;
    } else {
      Bm[0] = reinterpret_cast<const char*>(p.Wsu);
      Bm[1] = reinterpret_cast<const char*>(p.Wsg);
    }
    const int64_t H = p.H;
    const uint32_t bb[2] = {(uint32_t)(H * N * sizeof(T)), (uint32_t)(H * N * sizeof(T))};
    const int64_t nc[2] = {N - n0, N - n0};
    g.setup(p.A, (uint32_t)(p.S * H * sizeof(T)), [&](int r) -> uint32_t {
      const int tok = s_tok[r];
      return tok >= 0 ? (uint32_t)((int64_t)tok * H * sizeof(T)) : kOob;
    }, Bm, bb, N, n0, nc);
    run_mainloop(g, smem, p.H, [&](int r) { return s_tok[r] >= 0; });
    T* out = reinterpret_cast<T*>(shared ? p.hs : p.h);
    g.for_each_pair([&](int row, int c, float u, float gv) {
      const int64_t col = n0 + c;
      if (s_tok[row] >= 0 && col < N) {
        const int brow = row0 + row;  // row in the block
        const size_t o = p.h_blocked ? (size_t)b * BMB * N + (size_t)(col >> 5) * (BMB * 32) +
                                           brow * 32 + (col & 31)
                                     : (size_t)(b * BMB + brow) * N + col;
        out[o] = from_f32<T>(silu_f32(u) * gv);
      }
    });
    return shared ? ts.nb_r + b : b;
  }
}

// HALVES: the instance with the half-row core, for the long-tail split
// (p.split_tail); the other holds whole tiles only (the second core costs the
// whole tiles about 2% where nothing is split).
template <typename T, int BM, int BN, bool BS, bool HALVES>
__global__ __launch_bounds__((tile_threads<T, BM, 2, 2>()), 1) void upgate_kernel(ForwardParams p) {
  using TG = typename TileSel<T, BM, 2, 2, BS>::type;
  extern __shared__ __align__(16) char smem[];
  __shared__ int64_t s_task;
  __shared__ int s_tok[BM];
  const TaskSpace ts = task_space(p, BM, BN, p.D, p.Ds);
  Claimer cs(blockIdx.x % kXcds);
  QuotaState qs = quota_init(p.E);
  using TH = typename HalfSel<T, BM, 2, 2, BS>::type;
  constexpr bool kHalves = HALVES && !std::is_void<TH>::value;
  const bool split = kHalves && !p.sched_quota;
  TG g;
  for (;;) {
    if (threadIdx.x == 0) {
      if (p.sched_quota) {
        const int64_t t = claim_quota(p, ts, p.counters + kQuotaBase, qs);
        s_task = t < 0 ? -1 : t << 2;
      } else {
        s_task = claim_checked(p, 0, ts.total, split, cs);
      }
    }
    trace_stamp(0);
    __syncthreads();
    const int64_t c = uniform64(s_task);
    if (c < 0) {
      trace_record(p, kTraceUpgate, -1);
      break;
    }
    const int part = (int)(c & 3);
    if constexpr (kHalves) {
      if (part != 0) {
        TH gh;
        upgate_task<T, BM, BN>(p, ts, c >> 2, (part - 1) * (BM / 2), gh, smem, s_tok);
        trace_record(p, kTraceUpgate, c);
        continue;
      }
    }
    upgate_task<T, BM, BN>(p, ts, c >> 2, 0, g, smem, s_tok);
    trace_record(p, kTraceUpgate, c);
  }
}

// ---------------------------------------------------- down GEMM + combine
// Routed task: y = h[b*BM + r] . W_down^e[:, n-tile];
//   O_acc[t][n] += topk_weights[f] * y for f = sorted_ids[b*BM + r] != F.
// Shared task: y = hs[b*BM + r] . Ws_down[:, n-tile]; O_acc[s][n] += y.
// An n-tile is 2 x 128 columns: two adjacent column strips of the down
// weights run as the tile core's two matrices, sharing the h rows.
constexpr int kDownStrips = 2;

// ------------------------------------- the combine in the down epilogue
// (MOE_COMBINE_FUSED). A token's output tile (256 columns) is complete once
// every kept slot of the token, and the shared expert's row, has been
// computed, by down tasks that may run on any XCD. Each task:
//  1. writes its rows to their slots (Y[f], or Ys[token] for the shared
//     expert) with device-scope stores, which write through the XCD's L2 to
//     the level the XCDs share; a release fence and a barrier follow;
//  2. counts one arrival per row in arrivals[token][tile] (device-scope
//     atomic); a row whose count reaches the token's kept slots (+1 with a
//     shared expert) was the token's last to arrive, and goes on a list;
//  3. for the listed tokens the whole workgroup adds the token's rows in slot
//     order, w * y each product rounded to fp32, then the shared row, and
//     writes O, 256 columns per row; the rows are read back with device-scope
//     loads (which do not take stale lines from the XCD's L2). The
//     arithmetic is the slot combine pass's: the same output, bit for bit.
// No task waits for another; the counters are cleared by the setup kernel.
// Measured about 3x the down kernel's time at prefill sizes (the per-task
// read-back of the other slots is latency-bound inside the epilogue, where
// the separate pass streams the slots with the whole GPU), so it is an
// option, not the default.
template <int BM, int BN, typename TG>
__device__ __forceinline__ void fused_combine_epilogue(const ForwardParams& p, TG& g, bool shared,
                                                       int64_t j, int64_t n0, const int* s_tok,
                                                       const int* s_f) {
  constexpr int NT = kDownStrips * BN;  // columns per task
  __shared__ int s_n;                   // tokens completed by this task
  __shared__ int s_list[BM];            // their tile rows
  __shared__ uint32_t s_mask[BM];       // the token's kept slots, per tile row
  const int64_t H = p.H;
  const int64_t k = p.k;
  float* Yb = shared ? p.Ys : p.Y;
  g.for_each([&](int m, int row, int col, float v) {
    const int f = s_f[row];
    const int64_t n = n0 + m * BN + col;
    if (f >= 0 && n < H)
      __hip_atomic_store(Yb + (size_t)f * H + n, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  });
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  if (threadIdx.x == 0) s_n = 0;
  __syncthreads();
  if (threadIdx.x < BM) {
    const int r = threadIdx.x;
    const int tok = s_tok[r];
    if (tok >= 0 && s_f[r] >= 0) {
      uint32_t mask = 0;
      int need = p.Ds > 0 ? 1 : 0;
      for (int64_t jj = 0; jj < k; ++jj)
        if (p.kept[(int64_t)tok * k + jj]) {
          mask |= 1u << jj;
          ++need;
        }
      s_mask[r] = mask;
      const int old = __hip_atomic_fetch_add(p.arrivals + (int64_t)tok * p.arr_tiles + j, 1,
                                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (old == need - 1) s_list[atomicAdd(&s_n, 1)] = r;
    }
  }
  __syncthreads();
  const int nl = s_n;
  for (int q = threadIdx.x; q < nl * NT; q += TG::THREADS) {
    const int r = s_list[q / NT];
    const int64_t n = n0 + q % NT;
    if (n >= H) continue;
    const int64_t tok = s_tok[r];
    const uint32_t mask = s_mask[r];
    float a = 0.f;
    for (int64_t jj = 0; jj < k; ++jj) {
      if (!((mask >> jj) & 1u)) continue;
      const int64_t f2 = tok * k + jj;
      const float y =
          __hip_atomic_load(p.Y + f2 * H + n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      a = a + __fmul_rn(p.topk_w[f2], y);  // the product rounded, not fused
    }
    if (p.Ds > 0)
      a += __hip_atomic_load(p.Ys + tok * H + n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (p.out_bf16)
      reinterpret_cast<bf16_t*>(p.O)[tok * H + n] = f32_to_bf16(a);
    else
      reinterpret_cast<float*>(p.O)[tok * H + n] = a;
  }
  (void)shared;
}

// One down task t of the task space ts, run by the whole workgroup.
// before_rows(rb, shared) runs on every thread once the m-block is known and
// before the barrier that precedes the task's first read of h (rb: the
// m-block's readiness index, as upgate_task returns it). SLOT_NT: honour
// p.slots_nt (a second copy of the slot epilogue; the one-launch kernel
// leaves it out, its SGPR budget has no room for it).
// As upgate_task, the tile is a whole m-block of BMB rows or the rows row0 ..
// row0 + TG::BM of it.
// WAITS: before_rows may give up a bounded wait for the m-block's SwiGLU
// rows (it then returns true on thread 0): the task writes NaN to its output
// rows instead of its product with whatever h held.
// FCOMB: the combine runs here (p.fused_combine; see fused_combine_epilogue).
template <typename T, int BMB, int BN, bool SLOT_NT, bool WAITS, bool FCOMB = false, typename TG,
          typename BeforeRows>
__device__ __forceinline__ void down_task(const ForwardParams& p, const TaskSpace& ts, int64_t t,
                                          int row0, TG& g, char* smem, int* s_tok, int* s_f,
                                          float* s_w, BeforeRows before_rows) {
  static_assert(TG::BN == BN, "tile width");
  constexpr int BM = TG::BM;            // tile rows
  constexpr int NT = kDownStrips * BN;  // columns per task
  {
    const bool shared = t >= ts.t_r;
    int64_t b, j;
    if (!shared)
      decode_task(t, ts.nb_r, ts.nn_r, ts.gb_r, b, j);
    else
      decode_task(t - ts.t_r, ts.nb_s, ts.nn_s, kGroupBlocks, b, j);
    __shared__ int s_gave_up;
    const bool gave_up = before_rows(shared ? ts.nb_r + b : b, shared);
    if (WAITS && threadIdx.x == 0) s_gave_up = gave_up ? 1 : 0;
    // the block's expert, loaded before the row barrier (its latency overlaps
    // the sorted ids'); the router weights only where the epilogue applies
    // them (atomic combine: the slot rows are unweighted)
    const int64_t e_blk = shared ? -1 : (int64_t)__builtin_amdgcn_readfirstlane(p.expert_ids[b]);
    if (threadIdx.x < BM) {
      const int r = threadIdx.x;
      if (!shared) {
        const int f = p.sorted_ids[b * BMB + row0 + r];
        if (f < p.F) {
          s_tok[r] = (int)(f / p.k);
          s_f[r] = f;
          s_w[r] = p.atomic_combine ? p.topk_w[f] : 0.f;
        } else {
          s_tok[r] = -1;
          s_f[r] = -1;
          s_w[r] = 0.f;
        }
      } else {
        const int64_t s = b * BMB + row0 + r;
        s_tok[r] = s < p.S ? (int)s : -1;
        s_f[r] = s_tok[r];
        s_w[r] = 1.f;
      }
    }
    __syncthreads();
    const int64_t K = shared ? p.Ds : p.D;
    const int64_t n0 = j * NT;
    const char* Wb;
    if (!shared) {
      Wb = reinterpret_cast<const char*>(p.Wd) + (size_t)e_blk * p.D * p.H * sizeof(T);
    } else {
      Wb = reinterpret_cast<const char*>(p.Wsd);
    }
    const uint32_t wbytes = (uint32_t)(K * p.H * sizeof(T));
    const char* Bm[kDownStrips];
    uint32_t bb[kDownStrips];
    int64_t nc[kDownStrips];
#pragma unroll
    for (int m = 0; m < kDownStrips; ++m) {
      // strip m: columns n0 + m*BN .. of the [K][H] down weights
      Bm[m] = Wb + (size_t)m * BN * sizeof(T);
      bb[m] = wbytes - (uint32_t)(m * BN * sizeof(T));
      nc[m] = p.H - n0 - m * BN;
    }
    // this m-block's BMB rows of h (or hs); the tile's row r is block row
    // row0 + r
    const char* Ab = reinterpret_cast<const char*>(shared ? p.hs : p.h) +
                     (size_t)b * BMB * K * sizeof(T);
    if constexpr (is_direct<TG>()) {
      const bool hb = p.h_blocked;
      g.setup(Ab, (uint32_t)(BMB * K * sizeof(T)), [&](int r) -> uint32_t {
        const int br = row0 + r;
        return s_tok[r] >= 0 ? (uint32_t)(hb ? br * 64 : br * K * sizeof(T)) : kOob;
      }, Bm, bb, p.H, n0, nc, hb ? BMB : 0);
    } else {
      g.setup(Ab, (uint32_t)(BMB * K * sizeof(T)), [&](int r) -> uint32_t {
        return s_tok[r] >= 0 ? (uint32_t)((row0 + r) * K * sizeof(T)) : kOob;
      }, Bm, bb, p.H, n0, nc);
    }
    run_mainloop(g, smem, K, [&](int r) { return s_tok[r] >= 0; });
    const int64_t H = p.H;
    if (WAITS && s_gave_up) {
      // the rows this task would have computed from unpublished h: NaN
      const float nan = __builtin_nanf("");
      if (p.atomic_combine)
        g.for_each([&](int m, int row, int col, float) {
          const int tok = s_tok[row];
          const int64_t n = n0 + m * BN + col;
          if (tok >= 0 && n < H) atomicAdd(p.Oacc + (size_t)tok * H + n, nan);
        });
      else
        g.for_each([&](int m, int row, int col, float) {
          const int f = s_f[row];
          const int64_t n = n0 + m * BN + col;
          if (f >= 0 && n < H) (shared ? p.Ys : p.Y)[(size_t)f * H + n] = nan;
        });
      return;
    }
    if (p.atomic_combine) {
      float* O = p.Oacc;
      g.for_each([&](int m, int row, int col, float v) {
        const int tok = s_tok[row];
        const int64_t n = n0 + m * BN + col;
        if (tok >= 0 && n < H) atomicAdd(O + (size_t)tok * H + n, s_w[row] * v);
      });
    } else if constexpr (FCOMB) {
      fused_combine_epilogue<BM, BN>(p, g, shared, j, n0, s_tok, s_f);
    } else {
      // the row into its own slot: routed -> Y[f], shared -> Ys[token]; the
      // combine applies the router weight
      float* Yb = shared ? p.Ys : p.Y;
      if (SLOT_NT && p.slots_nt)
        g.for_each([&](int m, int row, int col, float v) {
          const int f = s_f[row];
          const int64_t n = n0 + m * BN + col;
          if (f >= 0 && n < H) __builtin_nontemporal_store(v, Yb + (size_t)f * H + n);
        });
      else
        g.for_each([&](int m, int row, int col, float v) {
          const int f = s_f[row];
          const int64_t n = n0 + m * BN + col;
          if (f >= 0 && n < H) Yb[(size_t)f * H + n] = v;
        });
    }
  }
}

// The down kernel's tile core; with the fused combine (FC) the LDS-direct core
// takes the wait-state form of its loads (the larger epilogue raises the SGPR
// pressure until the compiler restores descriptors from VGPR lanes next to
// the loads).
template <typename T, int BM, bool BS, bool FC, bool DIRECT = TileSel<T, BM, 2, 1, BS>::type::DIRECT>
struct DownTile {
  using type = typename TileSel<T, BM, 2, 1, BS>::type;
};
template <typename T, int BM, bool BS>
struct DownTile<T, BM, BS, true, true> {
  using type = TileGemmDirect<BM, 2, 8, stage_k<BM>(), 144 * 1024, BS, true, mfma_shape<BM>()>;
};

// LEAN: the instance for the default options (task queues, slot combine),
// with the quota scheduler's claims and the atomic epilogue compiled out
// (measured: down -1 to -2.5% at prefill sizes; the code the kernel carries
// changes how its main loop is built).
template <typename T, int BM, int BN, bool BS, bool FC = false, bool LEAN = false>
__global__ __launch_bounds__((tile_threads<T, BM, kDownStrips, 1>()), 1) void down_kernel(
    ForwardParams pk) {
  ForwardParams p = pk;
  if constexpr (LEAN) {
    p.sched_quota = 0;
    p.atomic_combine = 0;
  }
  static_assert(kDownStrips == 2, "two strips per down task");
  using TG = typename DownTile<T, BM, BS, FC>::type;
  extern __shared__ __align__(16) char smem[];
  __shared__ int64_t s_task;
  __shared__ int s_tok[BM];
  __shared__ int s_f[BM];   // output row: slot f (routed) or token (shared)
  __shared__ float s_w[BM];
  const TaskSpace ts = task_space(p, BM, kDownStrips * BN, p.H, p.H);
  Claimer cs(blockIdx.x % kXcds);
  QuotaState qs = quota_init(p.E);
  TG g;
  for (;;) {
    if (threadIdx.x == 0) {
      if (p.sched_quota) {
        const int64_t t = claim_quota(p, ts, p.counters + kQuotaBase + kQuotaStride, qs);
        s_task = t < 0 ? -1 : t << 2;
      } else {
        // whole tiles only: split into halves, the down tasks measured no
        // faster, and the half-tile code slowed the whole-tile path (prefill
        // down +3 to +5%)
        s_task = claim_checked(p, 1, ts.total, false, cs);
      }
    }
    trace_stamp(0);
    __syncthreads();
    const int64_t c = uniform64(s_task);
    if (c < 0) {
      trace_record(p, kTraceDown, -1);
      break;
    }
    down_task<T, BM, BN, !FC, false, FC>(p, ts, c >> 2, 0, g, smem, s_tok, s_f, s_w,
                                         [](int64_t, bool) { return false; });
    trace_record(p, kTraceDown, c);
  }
}

// ------------------------------------------ up/gate and down in one launch
// The FlashMoE review's single persistent kernel (Algorithm 1 and the task
// graph of its "Technical details"): one grid runs both GEMMs' tasks. A
// workgroup first claims up/gate tasks (own XCD's range, then the others);
// once every up/gate queue is empty it claims down tasks the same way. A down
// task of m-block b needs all of b's h columns, so it waits until the
// m-block's readiness counter has counted every up/gate n-tile of b; each
// up/gate task publishes its h stores (release at device scope) and then
// adds one to that counter.
// No wait can deadlock: a workgroup waits only after every up/gate task has
// been claimed, and a claimed up/gate task runs to its end without waiting
// (its workgroup is running, whatever the other workgroups do). As a guard
// the wait is still bounded by the constant-rate clock (kReadyWaitTicks), so
// the kernel always ends. A task that gives up sets the call's status word
// (counters[kStatusWord], cleared by the setup kernel) and writes NaN to its
// output rows: a wrong result is never silent.
constexpr uint64_t kReadyWaitTicks = (uint64_t)1 << 28;  // about 2.7 s at 100 MHz

// true when the count reached `need`, false when the wait gave up
__device__ __forceinline__ bool wait_count(const int* ctr, int need) {
  const uint64_t t0 = wall_clock64();
  bool ok = true;
  while (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < need) {
    __builtin_amdgcn_s_sleep(2);
    if (wall_clock64() - t0 > kReadyWaitTicks) {
      ok = false;
      break;
    }
  }
  // one acquire after the spin (not per poll: each acquire invalidates caches)
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  return ok;
}

// The one-launch kernel's tile core: the persistent kernels' core in the
// wait-state form of its loads (both GEMMs' task code in one kernel leaves the
// compiler short of SGPRs; it restores descriptors from VGPR lanes right
// before loads).
template <int BM, bool BS>
using FusedTile = TileGemmDirect<BM, 2, 8, stage_k<BM>(), 144 * 1024, BS, true, mfma_shape<BM>()>;

template <int BM, int BN, bool BS>
__global__ __launch_bounds__((tile_threads<bf16_t, BM, 2, 2>()), 1) void fused_kernel(
    ForwardParams p) {
  using TG = FusedTile<BM, BS>;
  static_assert(kDownStrips == 2, "one tile core (and one LDS ring) for both GEMMs");
  extern __shared__ __align__(16) char smem[];
  __shared__ int64_t s_task;
  __shared__ int s_tok[BM];
  __shared__ int s_f[BM];
  __shared__ float s_w[BM];
  const TaskSpace tu = task_space(p, BM, BN, p.D, p.Ds);
  const TaskSpace td = task_space(p, BM, kDownStrips * BN, p.H, p.H);
  int q = blockIdx.x % kXcds, tried = 0, phase = 0;  // thread 0 only
  TG g;
  for (;;) {
    if (threadIdx.x == 0) {
      int64_t t = -1;
      if (phase == 0) {
        t = claim_task(p.counters, tu.total, q, tried);
        if (t < 0) {
          phase = 1;
          q = blockIdx.x % kXcds;
          tried = 0;
        }
      }
      if (phase == 1) {
        t = claim_task(p.counters + kXcds, td.total, q, tried);
        if (t >= 0) t += tu.total;
      }
      s_task = t;
    }
    trace_stamp(0);
    __syncthreads();
    const int64_t t = uniform64(s_task);
    if (t < 0) {
      trace_record(p, kTraceFusedDown, -1);
      break;
    }
    if (t < tu.total) {
      const int64_t rb = upgate_task<bf16_t, BM, BN>(p, tu, t, 0, g, smem, s_tok);
      // Publish: each wave waits until its h stores have completed (vmcnt
      // 0: they are in this XCD's L2), then one device-scope release by
      // thread 0 writes the L2 back and the task is counted. A release fence
      // in every wave would write the L2 back once per wave: measured 35%
      // slower at prefill sizes, twice as slow at decode sizes.
      wait_vmcnt<0>();
      __syncthreads();
      if (threadIdx.x == 0) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        __hip_atomic_fetch_add(p.ready + rb, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      trace_record(p, kTraceFusedUp, t << 2);
    } else {
      // (the task's t_rows stamp follows the wait for its m-block's h rows)
      down_task<bf16_t, BM, BN, false, true>(
          p, td, t - tu.total, 0, g, smem, s_tok, s_f, s_w, [&](int64_t rb, bool shared) {
            if (threadIdx.x != 0) return false;
            if (wait_count(p.ready + rb, (int)(shared ? tu.nn_s : tu.nn_r))) return false;
            atomicOr(p.counters + kStatusWord, kStatusReadyTimeout);
            return true;
          });
      trace_record(p, kTraceFusedDown, (t - tu.total) << 2);
    }
  }
}

// ------------------------------------------ streaming down GEMM (bf16)
// The persistent kernels above refill the LDS ring at every task: claim,
// row metadata, the first stages' latency, then the epilogue's stores drain
// before the next task's loads go out. With a short K loop (decode: 12
// stages of the down projection) that is a large share of each task. Here
// the ring streams across tasks instead:
//  - each workgroup's tasks are fixed in advance (static_tasks: the XCD's
//    contiguous range, one task per workgroup per round, the position in the
//    round rotating with the round so that full and partial m-blocks spread
//    evenly), so the next task is known without an atomic whose result would
//    have to be waited for;
//  - its row metadata (the m-block's sorted ids and expert) is copied into
//    LDS by LDS-direct loads when the compute side starts the task before it;
//  - the issue side moves on to the next task's stages NSTAGE-1 stages
//    before the compute side finishes the current one, whose epilogue stores
//    then drain behind loads already in flight.
// Every iteration issues exactly one stage (zeros past the last task), so the
// per-wave vmcnt waits of the direct core stay exact; extra loads and stores
// only make them stricter. Requires at least 2*NSTAGE-1 K stages per task (the
// metadata of task i+1 has then landed before the issue side reaches it).
// Measured against the queue kernel: faster for short K loops over small
// tiles (decode down, 16-row tiles, 12 stages: -10%), slower for long K
// loops, for the up/gate projection and for tiles of uneven cost (skewed
// routing at 128 rows: +26%, the static order loses the queue's balancing),
// so the launcher uses it only there. Slot combine only (the epilogue writes
// unweighted rows; no gather of weights).

struct StaticTasks {
  int64_t lo, n, R, r;  // XCD range start / size, its workgroups, this one's rank
  __device__ __forceinline__ int64_t at(int64_t i) const {
    const int64_t pos = i * R + (r + i) % R;
    return pos < n ? lo + pos : -1;
  }
};

__device__ __forceinline__ StaticTasks static_tasks(int64_t total) {
  const int64_t G = gridDim.x, g = blockIdx.x;
  const int64_t X = G < kXcds ? G : kXcds;
  const int64_t x = g % X;
  StaticTasks st;
  st.lo = total * x / X;
  st.n = total * (x + 1) / X - st.lo;
  st.R = (G - x + X - 1) / X;
  st.r = g / X;
  return st;
}

struct StreamTask {
  int64_t t, b, j, K, nk;  // t < 0: none
  bool shared;
};

__device__ __forceinline__ StreamTask stream_task(const TaskSpace& ts, int64_t t, int64_t KR,
                                                  int64_t KS, int BK) {
  StreamTask k;
  k.t = t;
  k.shared = t >= ts.t_r;
  k.b = k.j = 0;
  k.K = k.nk = 0;
  if (t < 0) return k;
  if (!k.shared)
    decode_task(t, ts.nb_r, ts.nn_r, ts.gb_r, k.b, k.j);
  else
    decode_task(t - ts.t_r, ts.nb_s, ts.nn_s, kGroupBlocks, k.b, k.j);
  k.K = k.shared ? KS : KR;
  k.nk = (k.K + BK - 1) / BK;
  return k;
}

// Row metadata of one task in LDS (routed tasks): the m-block's sorted ids
// (F = sentinel) and its expert.
struct StreamMeta {
  int32_t f[256];
  int32_t e[4];
};

template <int BM>
__device__ __forceinline__ void stream_meta_direct(const ForwardParams& p, const StreamTask& k,
                                                   StreamMeta& m) {
  if (k.t < 0 || k.shared) return;
  if (threadIdx.x < BM) m.f[threadIdx.x] = p.sorted_ids[k.b * BM + threadIdx.x];
  if (threadIdx.x == 0) m.e[0] = p.expert_ids[k.b];
}

template <int BM>
__device__ __forceinline__ void stream_meta_dma(const ForwardParams& p, const TaskSpace& ts,
                                                const StreamTask& k, StreamMeta& m) {
  if (k.t < 0 || k.shared) return;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (wave != 0) return;
  const int lane = threadIdx.x & 63;
  const i32x4_t srd_s = make_srd(p.sorted_ids, (uint32_t)(ts.nb_r * BM * sizeof(int32_t)));
  const i32x4_t srd_e = make_srd(p.expert_ids, (uint32_t)(ts.nb_r * sizeof(int32_t)));
  // (the descriptors may come back from VGPR lanes: the wait-state form)
  if (lane < BM / 4) dma16<true>(srd_s, (uint32_t)(k.b * BM * 4 + lane * 16), m.f);
  if (lane == 0) dma4(srd_e, (uint32_t)(k.b * 4), m.e);
}

// Row r of a task holds a row: routed, a sorted id below F; shared, a token.
__device__ __forceinline__ bool stream_row_valid(const ForwardParams& p, const StreamTask& k,
                                                 const StreamMeta& m, int BM, int r) {
  return k.shared ? (k.b * BM + r < p.S) : (m.f[r] < p.F);
}

// Issue-side setup of task k (the expert's down strips, the h rows).
template <typename TG>
__device__ __forceinline__ void stream_setup(TG& g, const ForwardParams& p, const StreamTask& k,
                                             const StreamMeta& m) {
  constexpr int BM = TG::BM;
  const int64_t H = p.H;
  const int64_t K = k.K;
  const int e = k.shared ? -1 : __builtin_amdgcn_readfirstlane(m.e[0]);
  const int64_t n0 = k.j * kDownStrips * TG::BN;
  const char* Wb = k.shared ? reinterpret_cast<const char*>(p.Wsd)
                            : reinterpret_cast<const char*>(p.Wd) +
                                  (size_t)e * p.D * p.H * sizeof(bf16_t);
  const uint32_t wbytes = (uint32_t)(K * H * sizeof(bf16_t));
  const char* Bm[kDownStrips];
  uint32_t bb[kDownStrips];
  int64_t nc[kDownStrips];
#pragma unroll
  for (int mm = 0; mm < kDownStrips; ++mm) {
    Bm[mm] = Wb + (size_t)mm * TG::BN * sizeof(bf16_t);
    bb[mm] = wbytes - (uint32_t)(mm * TG::BN * sizeof(bf16_t));
    nc[mm] = H - n0 - mm * TG::BN;
  }
  const char* Ab = reinterpret_cast<const char*>(k.shared ? p.hs : p.h) +
                   (size_t)k.b * BM * K * sizeof(bf16_t);
  const bool hb = p.h_blocked;
  g.setup(Ab, (uint32_t)(BM * K * sizeof(bf16_t)), [&](int r) -> uint32_t {
    return stream_row_valid(p, k, m, BM, r) ? (uint32_t)(hb ? r * 64 : r * K * sizeof(bf16_t))
                                            : kOob;
  }, Bm, bb, H, n0, nc, hb ? BM : 0);
  g.set_k(K);
}

template <typename TG>
__device__ __forceinline__ void stream_epilogue(const TG& g, const ForwardParams& p,
                                                const StreamTask& k, const StreamMeta& m) {
  constexpr int BM = TG::BM;
  const int64_t H = p.H;
  const int64_t n0 = k.j * kDownStrips * TG::BN;
  float* Yb = k.shared ? p.Ys : p.Y;
  g.for_each([&](int mm, int row, int col, float v) {
    const int64_t n = n0 + mm * TG::BN + col;
    if (stream_row_valid(p, k, m, BM, row) && n < H) {
      const int64_t orow = k.shared ? k.b * BM + row : m.f[row];
      Yb[(size_t)orow * H + n] = v;
    }
  });
}

template <int BM, bool BS>
__global__ __launch_bounds__(512, 1) void down_stream_kernel(ForwardParams p) {
  using TG = typename TileSel<bf16_t, BM, kDownStrips, 1, BS>::type;
  static_assert(TG::DIRECT, "the streaming kernel runs on the LDS-direct core");
  constexpr int NSTAGE = TG::NSTAGE;
  __shared__ __align__(16) char ring[TG::LDS_BYTES];
  __shared__ StreamMeta meta[2];
  const TaskSpace ts = task_space(p, BM, kDownStrips * TG::BN, p.H, p.H);
  const StaticTasks st = static_tasks(ts.total);
  auto task = [&](int64_t i) { return stream_task(ts, st.at(i), p.D, p.Ds, TG::BK); };
  StreamTask c = task(0);  // the task the compute side works on
  if (c.t < 0) return;
  stream_meta_direct<BM>(p, c, meta[0]);
  stream_meta_direct<BM>(p, task(1), meta[1]);
  __syncthreads();
  TG g;
  int64_t ii = 0;         // task the issue side is on
  StreamTask is = c;
  int64_t ikt = 0;        // its next stage
  stream_setup(g, p, is, meta[0]);
  auto issue_next = [&](int slot) {
    if (ikt >= is.nk) {
      const StreamTask nx = task(ii + 1);
      if (nx.t >= 0) {  // its metadata landed at least NSTAGE iterations ago
        ++ii;
        is = nx;
        ikt = 0;
        stream_setup(g, p, is, meta[ii & 1]);
      }
    }
    // (the wait-state form: under this kernel's SGPR pressure the compiler
    // may restore the descriptors from VGPR lanes right before the loads)
    g.template issue_stage<true>(ring + slot * TG::STAGE, (int)ikt);  // past the last task: zeros
    ++ikt;
  };
  g.zero_acc();
#pragma unroll
  for (int sl = 0; sl + 1 < NSTAGE; ++sl) issue_next(sl);
  int64_t ci = 0;         // compute task index
  int slot_c = 0, slot_i = NSTAGE - 1;
  int nact_c = g.active_blocks([&](int r) { return stream_row_valid(p, c, meta[0], BM, r); });
  for (;;) {
    for (int64_t ckt = 0; ckt < c.nk; ++ckt) {
      wait_vmcnt<(NSTAGE - 2) * TG::MIN_PW>();  // this wave's loads of the stage have landed
      __syncthreads();                          // ... every wave's; the previous stage's reads done
      issue_next(slot_i);
      slot_i = slot_i + 1 == NSTAGE ? 0 : slot_i + 1;
      if (ckt == 0 && ci >= 1) stream_meta_dma<BM>(p, ts, task(ci + 1), meta[(ci + 1) & 1]);
      g.compute_stage_n(ring + slot_c * TG::STAGE, nact_c);
      slot_c = slot_c + 1 == NSTAGE ? 0 : slot_c + 1;
    }
    stream_epilogue(g, p, c, meta[ci & 1]);
    ++ci;
    c = task(ci);
    if (c.t < 0) break;
    g.zero_acc();
    nact_c = g.active_blocks([&](int r) { return stream_row_valid(p, c, meta[ci & 1], BM, r); });
  }
  wait_vmcnt<0>();  // no LDS-direct load may land after the workgroup ends
}

// dynamic LDS bytes of a persistent kernel (the direct core's stage buffers
// are static)
template <typename T, int BM, int NB, int STAGING>
static int lds_bytes() {
  using TG = typename TileSel<T, BM, NB, STAGING>::type;
  return is_direct<TG>() ? 0 : TG::LDS_BYTES;
}

// Output tile width per weight matrix (up/gate: 2 matrices share the A tile).
template <int BM>
constexpr int upgate_bn() { return 128; }
template <int BM>
constexpr int down_bn() { return 128; }

// The streaming down kernel: bf16, slot combine, the queue scheduler (the
// quota ablation keeps the kernels it compares), tiles of at most 32 rows
// (a task's cost is then its weight stream, the same for every task: the
// static order cannot fall out of balance) and 2*NSTAGE-1 .. 16 K stages per
// task (routed and shared).
template <int BM>
static bool down_stream_ok(const ForwardParams& p) {
  using TG = typename TileSel<bf16_t, BM, kDownStrips, 1>::type;
  if (BM > 32) return false;
  const int64_t kmin = p.Ds > 0 ? std::min(p.D, p.Ds) : p.D;
  const int64_t kmax = p.Ds > 0 ? std::max(p.D, p.Ds) : p.D;
  return !p.atomic_combine && !p.sched_quota && !p.fused_combine &&
         (kmin + TG::BK - 1) / TG::BK >= 2 * TG::NSTAGE - 1 &&
         (kmax + TG::BK - 1) / TG::BK <= 16;
}

// The weights are read once per call when the routing leaves about one
// m-block per expert: under half a block of assignments per expert on
// average (decode; DeepSeek-V3's 256 experts at 256-row blocks). The task
// order then runs each m-block's n-tiles back to back and no task reuses
// another's weight strip, so the weight loads take the non-temporal hint
// (measured: decode -9% per step, dsv3 -1%; with several m-blocks per expert
// sharing each strip in L2, prefill, the hint cost 1-2%). The 256-row up/gate
// tiles then also load A in 64-K stages (a64_tile). Cache hint and load
// shape only: the results are the same either way.
static bool weights_streamed(const ForwardParams& p, int BM) {
  return p.E > 0 && 2 * ((p.F + p.E - 1) / p.E) <= BM;
}

template <typename T, int BM, bool BS>
static hipError_t launch_upgate_bs(const ForwardParams& p, hipStream_t st) {
  constexpr int BN = upgate_bn<BM>();
  constexpr bool kHas = !std::is_void<typename HalfSel<T, BM, 2, 2, BS>::type>::value;
  if constexpr (kHas) {
    if (p.split_tail && !p.sched_quota)
      return launch_persistent(upgate_kernel<T, BM, BN, BS, true>, lds_bytes<T, BM, 2, 2>(),
                               tile_threads<T, BM, 2, 2>(), p, st);
  }
  return launch_persistent(upgate_kernel<T, BM, BN, BS, false>, lds_bytes<T, BM, 2, 2>(),
                           tile_threads<T, BM, 2, 2>(), p, st);
}

template <typename T, int BM>
static hipError_t launch_upgate_t(const ForwardParams& p, hipStream_t st) {
  if constexpr (sizeof(T) == 2) {
    if (weights_streamed(p, BM)) return launch_upgate_bs<T, BM, true>(p, st);
  }
  return launch_upgate_bs<T, BM, false>(p, st);
}

template <typename T, int BM>
static hipError_t launch_down_t(const ForwardParams& p, hipStream_t st) {
  if (p.fused_combine) {
    constexpr int BN = down_bn<BM>();
    if constexpr (sizeof(T) == 2) {
      if (weights_streamed(p, BM))
        return launch_persistent(down_kernel<T, BM, BN, true, true>,
                                 lds_bytes<T, BM, kDownStrips, 1>(),
                                 tile_threads<T, BM, kDownStrips, 1>(), p, st);
    }
    return launch_persistent(down_kernel<T, BM, BN, false, true>, lds_bytes<T, BM, kDownStrips, 1>(),
                             tile_threads<T, BM, kDownStrips, 1>(), p, st);
  }
  const bool lean = !p.sched_quota && !p.atomic_combine;
  constexpr int BN = down_bn<BM>();
  if constexpr (sizeof(T) == 2) {
    const bool bs = weights_streamed(p, BM);
    if (down_stream_ok<BM>(p))
      return bs ? launch_persistent(down_stream_kernel<BM, true>, 0, 512, p, st)
                : launch_persistent(down_stream_kernel<BM, false>, 0, 512, p, st);
    if (bs)
      return lean ? launch_persistent(down_kernel<T, BM, BN, true, false, true>,
                                      lds_bytes<T, BM, kDownStrips, 1>(),
                                      tile_threads<T, BM, kDownStrips, 1>(), p, st)
                  : launch_persistent(down_kernel<T, BM, BN, true>,
                                      lds_bytes<T, BM, kDownStrips, 1>(),
                                      tile_threads<T, BM, kDownStrips, 1>(), p, st);
  }
  return lean ? launch_persistent(down_kernel<T, BM, BN, false, false, true>,
                                  lds_bytes<T, BM, kDownStrips, 1>(),
                                  tile_threads<T, BM, kDownStrips, 1>(), p, st)
              : launch_persistent(down_kernel<T, BM, BN, false>, lds_bytes<T, BM, kDownStrips, 1>(),
                                  tile_threads<T, BM, kDownStrips, 1>(), p, st);
}

template <typename T>
static hipError_t dispatch_bm(const ForwardParams& p, int BM, bool up, hipStream_t st) {
  switch (BM) {
    case 16: return up ? launch_upgate_t<T, 16>(p, st) : launch_down_t<T, 16>(p, st);
    case 32: return up ? launch_upgate_t<T, 32>(p, st) : launch_down_t<T, 32>(p, st);
    case 64: return up ? launch_upgate_t<T, 64>(p, st) : launch_down_t<T, 64>(p, st);
    case 128: return up ? launch_upgate_t<T, 128>(p, st) : launch_down_t<T, 128>(p, st);
    case 256:
      if constexpr (sizeof(T) == 2)
        return up ? launch_upgate_t<T, 256>(p, st) : launch_down_t<T, 256>(p, st);
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

template <int BM>
static hipError_t launch_fused_t(const ForwardParams& p, hipStream_t st) {
  if (weights_streamed(p, BM))
    return launch_persistent(fused_kernel<BM, upgate_bn<BM>(), true>, 0,
                             tile_threads<bf16_t, BM, 2, 2>(), p, st);
  return launch_persistent(fused_kernel<BM, upgate_bn<BM>(), false>, 0,
                           tile_threads<bf16_t, BM, 2, 2>(), p, st);
}

hipError_t launch_forward_fused(const ForwardParams& p, int BM, hipStream_t st) {
  switch (BM) {
    case 16: return launch_fused_t<16>(p, st);
    case 32: return launch_fused_t<32>(p, st);
    case 64: return launch_fused_t<64>(p, st);
    case 128: return launch_fused_t<128>(p, st);
    case 256: return launch_fused_t<256>(p, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_forward_upgate(const ForwardParams& p, int dtype, int BM, hipStream_t st) {
  return dtype == 1 ? dispatch_bm<bf16_t>(p, BM, true, st) : dispatch_bm<float>(p, BM, true, st);
}

hipError_t launch_forward_down(const ForwardParams& p, int dtype, int BM, hipStream_t st) {
  return dtype == 1 ? dispatch_bm<bf16_t>(p, BM, false, st) : dispatch_bm<float>(p, BM, false, st);
}

int forward_lds_ok(int dtype, int BM) {
  return BM == 16 || BM == 32 || BM == 64 || BM == 128 || (BM == 256 && dtype == 1);
}

// ------------------------------------------------------- setup and combine
// Clear what must start at zero with a fill kernel rather than a memset node,
// so the whole call can be captured in a HIP graph: the task counters, and
// either the fp32 accumulator (atomic combine) or the kept flags (slot combine).
// keep_queues (testing): leave the queue counters [0, 2 kXcds) as they are.
__global__ __launch_bounds__(256) void setup_kernel(float* acc, int64_t n, uint8_t* flags,
                                                    int64_t nflags, int* counters, int* ready,
                                                    int64_t nready, int keep_queues, int* arrivals,
                                                    int64_t narr) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t i0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (acc != nullptr) {
    const int64_t n4 = n / 4;
    float4* a4 = reinterpret_cast<float4*>(acc);
    for (int64_t i = i0; i < n4; i += stride) a4[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int64_t i = n4 * 4 + i0; i < n; i += stride) acc[i] = 0.f;
  }
  if (flags != nullptr) {
    const int64_t n16 = nflags / 16;
    uint4* f16 = reinterpret_cast<uint4*>(flags);
    for (int64_t i = i0; i < n16; i += stride) f16[i] = make_uint4(0, 0, 0, 0);
    for (int64_t i = n16 * 16 + i0; i < nflags; i += stride) flags[i] = 0;
  }
  for (int64_t i = i0; i < kCounterInts; i += stride)
    if (!keep_queues || i >= 2 * kXcds) counters[i] = 0;
  for (int64_t i = i0; i < nready; i += stride) ready[i] = 0;
  for (int64_t i = i0; i < narr; i += stride) arrivals[i] = 0;
}

hipError_t launch_forward_setup(const ForwardParams& p, hipStream_t st) {
  float* acc = p.atomic_combine ? p.Oacc : nullptr;
  const int64_t n = acc ? p.S * p.H : 0;
  uint8_t* flags = p.atomic_combine ? nullptr : p.kept;
  const int64_t nf = flags ? p.F : 0;
  const int64_t narr = p.fused_combine ? p.S * p.arr_tiles : 0;
  int64_t blocks = (std::max(std::max(n / 4, nf / 16), narr) + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(setup_kernel, dim3((unsigned)blocks), dim3(256), 0, st, acc, n, flags, nf,
                     p.counters, p.ready, p.fused ? p.n_ready : (int64_t)0, p.keep_counters,
                     p.arrivals, narr);
  return hipGetLastError();
}

// Slot combine: O[t][:] = sum_{j<k, kept} w[f] * Y[f][:] (f = t*k + j) (+ Ys[t][:]):
// each product rounded to fp32, summed in slot order in fp32, rounded once
// into O.
// 8 consecutive fp32 of a slot row; NT: with the non-temporal hint.
template <bool NT>
__device__ __forceinline__ void load8(const float* src, float (&y)[8]) {
  typedef float f32x4v __attribute__((ext_vector_type(4)));
  const f32x4v* s = reinterpret_cast<const f32x4v*>(src);
  f32x4v a, b;
  if constexpr (NT) {
    a = __builtin_nontemporal_load(s);
    b = __builtin_nontemporal_load(s + 1);
  } else {
    a = s[0];
    b = s[1];
  }
  y[0] = a.x; y[1] = a.y; y[2] = a.z; y[3] = a.w;
  y[4] = b.x; y[5] = b.y; y[6] = b.z; y[7] = b.w;
}

template <bool OUT_BF16, bool NT>
__global__ __launch_bounds__(256) void combine_kernel(const float* Y, const float* Ys,
                                                      const uint8_t* kept, const float* w,
                                                      void* O, int64_t S, int64_t H,
                                                      int64_t k) {
  // 8 columns per thread step. A token's k slot rows are loaded whether or
  // not the slot was kept (the rows exist in the workspace; an unkept one
  // holds stale data that is never added), so the loads do not wait on the
  // kept flags; the sum is the same as adding only the kept slots, in slot
  // order.
  const int64_t h8 = H / 8;
  const int64_t total = S * h8;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    const int64_t t = i / h8;
    const int64_t c = (i - t * h8) * 8;
    float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int64_t j = 0; j < k; ++j) {
      const int64_t f = t * k + j;
      float y[8];
      load8<NT>(Y + f * H + c, y);
      const bool use = kept[f] != 0;
      const float wf = w[f];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float s = a[e] + __fmul_rn(wf, y[e]);  // the product rounded, not fused
        a[e] = use ? s : a[e];
      }
    }
    if (Ys != nullptr) {
      float y[8];
      load8<NT>(Ys + t * H + c, y);
#pragma unroll
      for (int e = 0; e < 8; ++e) a[e] += y[e];
    }
    if constexpr (OUT_BF16) {
      uint32_t q[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        q[e] = f32_to_bf16(a[2 * e]) | ((uint32_t)f32_to_bf16(a[2 * e + 1]) << 16);
      *reinterpret_cast<uint4*>(reinterpret_cast<bf16_t*>(O) + t * H + c) =
          make_uint4(q[0], q[1], q[2], q[3]);
    } else {
      float* o = reinterpret_cast<float*>(O) + t * H + c;
      *reinterpret_cast<float4*>(o) = make_float4(a[0], a[1], a[2], a[3]);
      *reinterpret_cast<float4*>(o + 4) = make_float4(a[4], a[5], a[6], a[7]);
    }
  }
}

hipError_t launch_forward_combine(const ForwardParams& p, hipStream_t st) {
  const int64_t total = p.S * (p.H / 8);
  if (total == 0) return hipSuccess;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  const float* Ys = p.Ds > 0 ? p.Ys : nullptr;
  const bool nt = p.slots_nt != 0;
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(256), 0, st, p.Y, Ys, p.kept,
                       p.topk_w, p.O, p.S, p.H, p.k);
  };
  if (p.out_bf16)
    nt ? go(combine_kernel<true, true>) : go(combine_kernel<true, false>);
  else
    nt ? go(combine_kernel<false, true>) : go(combine_kernel<false, false>);
  return hipGetLastError();
}

// With the fused combine and no shared expert: tokens with no kept slot
// (every choice dropped by the capacity) get the zero row the combine pass
// would write. One wave per token: its lanes test the k kept flags.
__global__ __launch_bounds__(256) void zero_unrouted_kernel(const uint8_t* kept, void* O, int64_t S,
                                                            int64_t H, int64_t k, int out_bf16) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= S) return;
  bool any = false;
  for (int64_t j = lane; j < k; j += 64) any = any || kept[t * k + j] != 0;
  if (__ballot(any)) return;
  for (int64_t c = lane; c < H; c += 64) {
    if (out_bf16)
      reinterpret_cast<bf16_t*>(O)[t * H + c] = 0;
    else
      reinterpret_cast<float*>(O)[t * H + c] = 0.f;
  }
}

hipError_t launch_zero_unrouted(const ForwardParams& p, hipStream_t st) {
  if (p.S == 0) return hipSuccess;
  hipLaunchKernelGGL(zero_unrouted_kernel, dim3((unsigned)((p.S + 3) / 4)), dim3(256), 0, st,
                     p.kept, p.O, p.S, p.H, p.k, p.out_bf16);
  return hipGetLastError();
}

// O = bf16_rne(O_acc), 8 elements per thread step.
__global__ __launch_bounds__(256) void finalize_kernel(const float* acc, bf16_t* out, int64_t n) {
  const int64_t n8 = n / 8;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t i0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (int64_t i = i0; i < n8; i += stride) {
    const float4 a = reinterpret_cast<const float4*>(acc)[2 * i];
    const float4 b = reinterpret_cast<const float4*>(acc)[2 * i + 1];
    const uint32_t w0 = f32_to_bf16(a.x) | ((uint32_t)f32_to_bf16(a.y) << 16);
    const uint32_t w1 = f32_to_bf16(a.z) | ((uint32_t)f32_to_bf16(a.w) << 16);
    const uint32_t w2 = f32_to_bf16(b.x) | ((uint32_t)f32_to_bf16(b.y) << 16);
    const uint32_t w3 = f32_to_bf16(b.z) | ((uint32_t)f32_to_bf16(b.w) << 16);
    reinterpret_cast<uint4*>(out)[i] = make_uint4(w0, w1, w2, w3);
  }
  for (int64_t i = n8 * 8 + i0; i < n; i += stride) out[i] = f32_to_bf16(acc[i]);
}

hipError_t launch_forward_finalize(const ForwardParams& p, hipStream_t st) {
  const int64_t n = p.S * p.H;
  if (n == 0) return hipSuccess;
  int64_t blocks = (n / 8 + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(finalize_kernel, dim3((unsigned)blocks), dim3(256), 0, st, p.Oacc,
                     reinterpret_cast<bf16_t*>(p.O), n);
  return hipGetLastError();
}

}  // namespace moe
