// Internal definitions shared by the HIP sources of the MoE library.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

typedef uint16_t bf16_t;
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kXcds = 8;          // MI355X: 8 XCDs, workgroups dispatched round-robin
// Task counters at the head of the forward workspace: per-XCD queues of the
// two grouped GEMMs at [0, 16); with the per-expert quota scheduler, one
// counter per expert plus one for the shared expert's tasks per GEMM at
// kQuotaBase + g * kQuotaStride.
constexpr int kQuotaBase = 64;
constexpr int kQuotaStride = 1024 + 16;
constexpr int kCounterInts = kQuotaBase + 2 * kQuotaStride;
// The call's status word, an int inside the counter block (so cleared by
// every call's setup kernel) at the byte offset the public header names
// (MOE_FORWARD_STATUS_OFFSET); bits as MOE_STATUS_* there.
constexpr int kStatusWord = 32;
constexpr int kStatusReadyTimeout = 1;
constexpr int kStatusTasksLost = 2;
constexpr int kStatusQueueCount = 4;
// Queue bookkeeping of the two-launch grouped GEMMs, also in the counter
// block: per GEMM g (0 up/gate, 1 down) the task parts handed out
// (kDoneBase + 2 g) and the workgroups that found no task left
// (kDoneBase + 2 g + 1).
constexpr int kDoneBase = 16;
// Tasks claimed per queue atomic with the batched-claims flag.
constexpr int kClaimBatch = 4;

__device__ __forceinline__ float bf16_to_f32(bf16_t x) {
  return __uint_as_float(((uint32_t)x) << 16);
}

__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  // round to nearest even (v_cvt_pk_bf16_f32 on gfx950)
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(bf16_t, b);
}

template <typename T>
__device__ __forceinline__ float to_f32(T x);
template <>
__device__ __forceinline__ float to_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ float to_f32<bf16_t>(bf16_t x) { return bf16_to_f32(x); }

template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) { return f32_to_bf16(x); }

// SiLU(u) = u / (1 + exp(-u)); v_exp_f32 and v_rcp_f32 (about 1 ulp each).
// exp overflows to +inf for u < -88, where rcp(inf) = 0 gives the -0 limit.
__device__ __forceinline__ float silu_f32(float u) {
  return u * __builtin_amdgcn_rcpf(1.0f + __expf(-u));
}

// ---------------------------------------------------------------- launchers
// Host-side launch helpers implemented in the .hip sources; each returns the
// hipError_t of its launch.

struct GateParams {
  const void* A;          // [S][H]
  const void* Wr;         // [H][E]
  const float* bias;      // [E] or null
  float* G;               // [S][E]
  int64_t S, H, E;
};

struct TopkParams {
  const float* G;         // [S][E]
  int32_t* ids;           // [S][k]
  float* w;               // [S][k]
  int64_t S, E, k;
  int renormalize;
};

struct AlignParams {
  const int32_t* ids;     // [F]
  int32_t* sorted_ids;
  int32_t* expert_ids;
  int32_t* ntpp;
  int32_t* counts;
  int32_t* seg_counts;    // workspace [nseg][E]
  int64_t* offsets;       // workspace [E]
  int32_t* kept;          // workspace [E]
  int64_t F, E, BM, C;
  int64_t nseg;
};

struct ForwardParams {
  const void* A;
  const void* Wu;
  const void* Wg;
  const void* Wd;
  const void* Wsu;
  const void* Wsg;
  const void* Wsd;
  const float* topk_w;
  const int32_t* sorted_ids;
  const int32_t* expert_ids;
  const int32_t* ntpp;
  void* O;                // [S][H] dtype (fp32 with out_f32)
  float* Oacc;            // atomic combine: [S][H] fp32 accumulator (may be O)
  float* Y;               // slot combine: [F][H] fp32 weighted rows
  float* Ys;              // slot combine: [S][H] fp32 shared-expert rows
  uint8_t* kept;          // slot combine: [F] 1 = assignment has a slot
  void* h;                // [cap_rows][D] (layout: h_blocked)
  void* hs;               // [round_up(S, BM)][Ds] (layout: h_blocked)
  int* counters;          // kCounterInts ints
  int* ready;             // one launch: per m-block count of finished up/gate tasks
                          // (routed blocks, then shared blocks)
  int64_t n_ready;        // entries of ready
  int64_t S, H, D, E, k, Ds, F;
  int atomic_combine;     // 1: atomics into Oacc; 0: slots Y / Ys + combine pass
  int sched_quota;        // 1: static per-expert workgroup quota (ablation baseline)
  int out_bf16;           // O is bf16 (else fp32)
  int h_blocked;          // 1: h and hs hold each BM-row block as slabs of 32 columns
                          // (row r, column c of block b at b*BM*N + (c/32)*BM*32 + r*32 + c%32)
                          // so that each down-projection K stage is contiguous; 0: row-major
  int grid;               // persistent workgroups
  int fused;              // 1: up/gate and down in one launch (bf16)
  int slots_nt;           // 1: the slot rows Y / Ys are written and read with the
                          // non-temporal hint (they far exceed the MALL)
  int fused_combine;      // 1: the combine in the down epilogue (arrival counts)
  int* arrivals;          // fused combine: [S][arr_tiles] rows arrived per token and tile
  int64_t arr_tiles;      // 256-column tiles of H
  int claim_batch;        // task parts claimed per queue atomic (1, or kClaimBatch)
  int split_tail;         // 1: the up/gate queues' last tasks run as two row halves
  int keep_counters;      // testing: the setup kernel leaves the queue counters as they are
  void* a_blk;            // MXFP8: stage-blocked quantised rows of the routed m-blocks
  void* as_blk;           // MXFP8: the same for the shared expert's m-blocks
  void* trace;            // per-task timing records (libraries built with MOE_TRACE), or null
  int64_t trace_cap;      // records that fit the trace buffer
};

// Per-task timing records of the persistent GEMM kernels (compile with
// -DMOE_TRACE=1). The trace buffer starts with a 64-byte header whose first
// uint64 counts the records written (an atomic cursor); records of
// kTraceRecBytes follow. Times are the GPU's constant 100 MHz clock.
#ifndef MOE_TRACE
#define MOE_TRACE 0
#endif
struct TraceRec {
  uint32_t kernel;      // kTraceUpgate, kTraceDown, kTraceFusedUp, kTraceFusedDown
  uint32_t workgroup;
  int64_t task;         // claimed task id << 2 | part (part 1, 2: row halves); -1: the
                        // workgroup found no task left (t_claim is then its exit time)
  uint64_t t_claim;     // the claim's result arrived
  uint64_t t_rows;      // row metadata in LDS, tile set up: the K loop starts
  uint64_t t_kloop;     // the K loop ended: the epilogue starts
  uint64_t t_end;       // the epilogue's stores were issued
};
constexpr int kTraceHeaderBytes = 64;
constexpr int kTraceRecBytes = (int)sizeof(TraceRec);
enum { kTraceUpgate = 1, kTraceDown = 2, kTraceFusedUp = 3, kTraceFusedDown = 4 };

constexpr int kAlignSeg = 512;   // assignments per wave segment in the align kernels
#ifndef MOE_ALIGN_SMALL_F
#define MOE_ALIGN_SMALL_F 16384
#endif
// Up to this many assignments the one-workgroup align; the crossover with the
// three-launch path was measured between 16K and 32K assignments (E = 64, 256).
constexpr int64_t kAlignSmallF = MOE_ALIGN_SMALL_F;

// The split gate: bmg rows per tile, the H loop cut into `splits` ranges of
// kc elements (splits == 1: not split).
struct GateSplit {
  int bmg;
  int splits;
  int64_t kc;
};
GateSplit gate_split_plan(int64_t S, int64_t H, int64_t E, int dtype);
hipError_t launch_gate_split(const GateParams& gp, const TopkParams& tp, const GateSplit& plan,
                             float* part, hipStream_t st);
hipError_t launch_gate(const GateParams& p, int dtype, hipStream_t st);
bool gate_topk_fusable(const GateParams& gp, int dtype);
hipError_t launch_gate_topk(const GateParams& gp, const TopkParams& tp, hipStream_t st);
hipError_t launch_topk(const TopkParams& p, hipStream_t st);
hipError_t launch_align(const AlignParams& p, hipStream_t st);
hipError_t launch_forward_setup(const ForwardParams& p, hipStream_t st);
hipError_t launch_forward_upgate(const ForwardParams& p, int dtype, int BM, hipStream_t st);
hipError_t launch_forward_down(const ForwardParams& p, int dtype, int BM, hipStream_t st);
hipError_t launch_forward_fused(const ForwardParams& p, int BM, hipStream_t st);
hipError_t launch_forward_finalize(const ForwardParams& p, hipStream_t st);
hipError_t launch_forward_combine(const ForwardParams& p, hipStream_t st);
hipError_t launch_zero_unrouted(const ForwardParams& p, hipStream_t st);
int forward_lds_ok(int dtype, int BM);
// MXFP8 mode (moe_mx.hip)
hipError_t launch_mx_quantize_rows(const void* X, int dtype, int64_t R, int64_t K, uint8_t* codes,
                                   uint8_t* scales, hipStream_t st);
hipError_t launch_mx_pack_weights(const void* W, int64_t E, int64_t K, int64_t N, void* packed,
                                  hipStream_t st);
hipError_t launch_mx_gather(const ForwardParams& p, int BM, int64_t cap_rows, int64_t s_rows,
                            hipStream_t st);
hipError_t launch_forward_mx(const ForwardParams& p, int BM, bool up, hipStream_t st);

}  // namespace moe
