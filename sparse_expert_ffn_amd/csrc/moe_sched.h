// Scheduling pieces shared by the persistent GEMM kernels (bf16 / fp32 and
// MXFP8): the LDS ring of the LDS-direct tile cores, per-task timing records,
// the task space of a grouped GEMM (routed m-blocks x n-tiles, then the shared
// expert's), the per-XCD atomic task queues, and the persistent launch.
#pragma once

#include "moe_common.h"

namespace moe {

constexpr int kGroupBlocks = 4;

// The direct cores' static LDS ring: one buffer for every core type, so a
// kernel that runs tiles of several shapes (whole and half tiles, or both
// GEMMs) holds a single ring.
constexpr int kRingBytes = 144 * 1024;

__device__ __forceinline__ char* lds_ring_bytes() {
  __shared__ __align__(16) char ring[kRingBytes];
  return ring;
}

template <typename TG>
__device__ __forceinline__ char* lds_ring() {
  static_assert(TG::LDS_BYTES <= kRingBytes, "ring size");
  return lds_ring_bytes();
}

// ------------------------------------------------------- per-task timing
// With MOE_TRACE, thread 0 of a persistent kernel stamps each task's phases
// into LDS and writes one TraceRec per task to the caller's trace buffer;
// without it these are empty.
__device__ __forceinline__ uint64_t* trace_stamps() {
  __shared__ uint64_t s[4];
  return s;
}
__device__ __forceinline__ void trace_stamp(int i) {
  if constexpr (MOE_TRACE) {
    if (threadIdx.x == 0) trace_stamps()[i] = wall_clock64();
  }
}
__device__ __forceinline__ void trace_record(const ForwardParams& p, uint32_t kernel,
                                             int64_t task) {
  if constexpr (MOE_TRACE) {
    if (threadIdx.x != 0 || p.trace == nullptr) return;
    uint64_t* s = trace_stamps();
    const uint64_t now = wall_clock64();
    if (task < 0) s[0] = now;
    unsigned long long* cur = reinterpret_cast<unsigned long long*>(p.trace);
    const unsigned long long i = atomicAdd(cur, 1ull);
    if ((int64_t)i >= p.trace_cap) return;
    TraceRec* r = reinterpret_cast<TraceRec*>(reinterpret_cast<char*>(p.trace) +
                                              kTraceHeaderBytes + i * kTraceRecBytes);
    r->kernel = kernel;
    r->workgroup = blockIdx.x;
    r->task = task;
    r->t_claim = s[0];
    r->t_rows = task < 0 ? now : s[1];
    r->t_kloop = task < 0 ? now : s[2];
    r->t_end = now;
  }
}

// ------------------------------------------------------------ task scheduling

// Task t of a space of nb m-blocks x nn n-tiles -> (m-block b, n-tile j),
// n-tile-major inside each group of gb consecutive m-blocks.
__device__ __forceinline__ void decode_task(int64_t t, int64_t nb, int64_t nn, int64_t gb,
                                            int64_t& b, int64_t& j) {
  const int64_t per = gb * nn;
  const int64_t grp = t / per;
  const int64_t b0 = grp * gb;
  const int64_t gsz = min(gb, nb - b0);
  const int64_t w = t - grp * per;
  j = w / gsz;
  b = b0 + w % gsz;
}

// Claim the next task of [0, total): own XCD's range first, then the others.
// q / tried persist across calls of one workgroup (thread 0 only).
// A value every lane of the wave holds, made visibly wave-uniform (SGPR).
__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ int64_t claim_task(int* counters, int64_t total, int& q, int& tried) {
  while (tried < kXcds) {
    const int64_t lo = total * q / kXcds;
    const int64_t hi = total * (q + 1) / kXcds;
    if (lo < hi) {
      const int c = atomicAdd(&counters[q], 1);
      if (lo + c < hi) return lo + c;
    }
    q = (q + 1) % kXcds;
    ++tried;
  }
  return -1;
}

// Workgroups per XCD of this grid.
__device__ __forceinline__ int64_t wgs_per_xcd() {
  return gridDim.x >= kXcds ? gridDim.x / kXcds : 1;
}

// Thread 0's claim state in one persistent workgroup: the queue it claims
// from, how many queues it has found empty, and the claims left of its last
// batch on queue q.
struct Claimer {
  int q, tried;
  int64_t c_next, c_end;
  __device__ explicit Claimer(int q0) : q(q0), tried(0), c_next(0), c_end(0) {}
};

// Long-tail splitting (the Weave review's tail handling, section 5.1). Tasks
// cost about the same, so when a queue's n tasks are not a multiple of its R
// workgroups, n mod R of them form a last round that only some workgroups
// run while the others wait for the kernel's end (measured: 13% of the
// up/gate kernel's workgroup time idle at prefill_skew, about 1,080 tasks on
// 256 workgroups). Those last n mod R tasks of each queue are claimed as two
// halves, rows [0, BM/2) and [BM/2, BM) of the tile, each run by a whole
// workgroup on the BM/2-row tile core, so a half takes about half a task.
// The half core adds the same 32-wide K chunks in the same order into each
// output element as the whole-tile core, so the result is the same, bit for
// bit. Claimed ids are (task << 2) | part: part 0 = whole tile, 1 = the first
// half of the rows, 2 = the second. R = workgroups per XCD; split = false
// keeps every task whole.
//
// Batched claims (the Weave review's two-level claiming, section 5.2): with
// batch > 1 one atomic takes `batch` consecutive claims of the queue, which
// the workgroup then runs one after the other. Fewer atomics, coarser
// balance at the end of each queue.
//
// done (or null) counts the claims handed out, for the end-of-kernel check
// (queue_check).
__device__ __forceinline__ int64_t claim_task_split(int* counters, int64_t total, int64_t R,
                                                    bool split, int batch, Claimer& cs,
                                                    int* done) {
  while (cs.tried < kXcds) {
    const int q = cs.q;
    const int64_t lo = total * q / kXcds;
    const int64_t n = total * (q + 1) / kXcds - lo;
    if (n > 0) {
      const int64_t k = split ? n % R : 0;  // tasks cut in two
      int64_t c;
      if (cs.c_next < cs.c_end) {
        c = cs.c_next++;
      } else {
        c = atomicAdd(&counters[q], batch);
        if (c < n + k) {
          cs.c_next = c + 1;
          cs.c_end = c + batch < n + k ? c + batch : n + k;
          if (done) atomicAdd(done, (int)(cs.c_end - c));
        }
      }
      if (c < n + k) {
        const int64_t whole = n - k;
        if (c < whole) return (lo + c) << 2;
        const int64_t v = c - whole;
        return ((lo + whole + v / 2) << 2) | (1 + (v & 1));
      }
    }
    cs.q = (q + 1) % kXcds;
    ++cs.tried;
  }
  return -1;
}

// The end-of-kernel check of one grouped GEMM's queues, run by thread 0 of
// each workgroup once it has found every queue empty. The last workgroup to
// get there checks what the claims must have left:
//  - the claims handed out (`done`) equal the task parts of the task space;
//    fewer means tasks never ran, as when the counters did not start at zero
//    (kStatusTasksLost);
//  - each queue with tasks ends at batch * (its successful atomics + one
//    failed atomic per workgroup), an empty queue at 0 (kStatusQueueCount).
// A failure sets its bit in the call's status word.
__device__ __forceinline__ void queue_check(const int* queues, const int* done, int* exits,
                                            int* status, int64_t total, int64_t R, bool split,
                                            int batch) {
  const int grid = (int)gridDim.x;
  const int prev = __hip_atomic_fetch_add(exits, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
  if (prev != grid - 1) return;
  int64_t parts = 0;
  bool counts_ok = true;
  for (int q = 0; q < kXcds; ++q) {
    const int64_t lo = total * q / kXcds;
    const int64_t n = total * (q + 1) / kXcds - lo;
    const int64_t k = split ? n % R : 0;
    parts += n + k;
    const int64_t want = n > 0 ? (int64_t)batch * ((n + k + batch - 1) / batch + grid) : 0;
    const int got = __hip_atomic_load(&queues[q], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
    if ((int64_t)got != want) counts_ok = false;
  }
  const int d = __hip_atomic_load(done, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
  int bits = 0;
  if ((int64_t)d != parts) bits |= kStatusTasksLost;
  if (!counts_ok) bits |= kStatusQueueCount;
  if (bits) atomicOr(status, bits);
}

// Claim with the call's batching and bookkeeping for grouped GEMM g (0
// up/gate, 1 down), whose queues are at counters + g * kXcds; on finding
// every queue empty, run the end-of-kernel check. Thread 0 only.
__device__ __forceinline__ int64_t claim_checked(const ForwardParams& p, int g, int64_t total,
                                                 bool split, Claimer& cs) {
  int* queues = p.counters + g * kXcds;
  int* done = p.counters + kDoneBase + 2 * g;
  const int64_t R = wgs_per_xcd();
  const int64_t c = claim_task_split(queues, total, R, split, p.claim_batch, cs, done);
  if (c < 0)
    queue_check(queues, done, done + 1, p.counters + kStatusWord, total, R, split, p.claim_batch);
  return c;
}

struct TaskSpace {
  int64_t nb_r, nn_r, nb_s, nn_s, t_r, total;
  int64_t gb_r;  // routed m-blocks per group (the shared expert's: kGroupBlocks)
};

__device__ __forceinline__ TaskSpace task_space(const ForwardParams& p, int BM, int BN,
                                                int64_t n_routed_cols, int64_t n_shared_cols) {
  TaskSpace ts;
  ts.nb_r = (int64_t)(*p.ntpp) / BM;
  ts.nn_r = (n_routed_cols + BN - 1) / BN;
  ts.nb_s = p.Ds > 0 ? (p.S + BM - 1) / BM : 0;
  ts.nn_s = (n_shared_cols + BN - 1) / BN;
  ts.t_r = ts.nb_r * ts.nn_r;
  ts.total = ts.t_r + ts.nb_s * ts.nn_s;
  // About one m-block per expert (decode, many experts): the m-blocks share
  // no weights, so each m-block's n-tiles run back to back and the XCD's
  // concurrent tasks stream whole weight rows (measured: dsv3 -2%). Several
  // m-blocks per expert: groups of kGroupBlocks share each weight strip.
  ts.gb_r = ts.nb_r <= p.E + p.E / 4 ? 1 : kGroupBlocks;
  return ts;
}

// ------------------------------------------------------------ host launch
inline int num_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
      v = 256;
    cus[dev] = v;
  }
  return cus[dev];
}

template <typename K>
inline hipError_t launch_persistent(K kernel, int lds, int threads, const ForwardParams& p,
                                    hipStream_t st) {
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  int per_cu = 0;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, lds);
  if (e != hipSuccess) return e;
  if (per_cu < 1) per_cu = 1;
  const int grid = num_cus() * per_cu;
  hipLaunchKernelGGL(kernel, dim3(grid), dim3(threads), lds, st, p);
  return hipGetLastError();
}

}  // namespace moe
