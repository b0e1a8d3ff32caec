// Host side of the C ABI declared in include/moe.h: argument validation,
// workspace layout, kernel launches and the optional per-stage timing.
#include <mutex>
#include <vector>

#include "moe.h"
#include "moe_common.h"

using namespace moe;

namespace {

constexpr int64_t kMaxE = 1024;
constexpr int64_t kMaxK = 32;
constexpr size_t kAlignUp = 256;

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// below 2 GiB: addressable by one raw buffer resource
bool fits_buffer(int64_t bytes) { return bytes >= 0 && bytes < ((int64_t)1 << 31); }

moe_status check_routing_dims(const moe_shape* s) {
  if (s == nullptr) return MOE_ERR_INVALID_ARGUMENT;
  if ((s->flags & ~(MOE_OUTPUT_F32 | MOE_COMBINE_ATOMIC | MOE_SCHED_QUOTA | MOE_FUSED_LAUNCH |
                    MOE_SCHED_BATCH | MOE_TEST_SKIP_QUEUE_RESET | MOE_COMBINE_FUSED |
                    MOE_SPLIT_TAIL)) != 0)
    return MOE_ERR_INVALID_ARGUMENT;
  if (s->dtype != MOE_F32 && s->dtype != MOE_BF16 && s->dtype != MOE_MXFP8)
    return MOE_ERR_INVALID_ARGUMENT;
  if (s->S < 0 || s->E < 1 || s->k < 1 || s->k > s->E) return MOE_ERR_INVALID_ARGUMENT;
  if (s->E > kMaxE || s->k > kMaxK) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

moe_status check_align_dims(const moe_shape* s) {
  moe_status st = check_routing_dims(s);
  if (st != MOE_OK) return st;
  if (s->block_size < 1 || s->capacity < 0) return MOE_ERR_INVALID_ARGUMENT;
  // every stored index (flat ids, the sentinel S*k, padded positions) is int32
  if (s->S > (int64_t)INT32_MAX / s->k) return MOE_ERR_UNSUPPORTED;
  const int64_t cap = s->S * s->k + s->E * ((int64_t)s->block_size - 1);
  if (cap > (int64_t)INT32_MAX) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// Bytes of a stage-blocked MXFP8 matrix of `rows` rows and K columns
// (64 code bytes and 2 scale bytes per row and stage of 64 K values).
int64_t mx_blocked_bytes(int64_t rows, int64_t K) { return rows * (K / 64) * 66; }

// MXFP8 forward: H, D, D_shared multiples of 128 (whole n-tiles and K
// stages), 64/128/256-row blocks, the slot combine, two launches.
moe_status check_mx_forward_dims(const moe_shape* s) {
  if (s->H % 128 || s->D % 128 || s->D_shared % 128) return MOE_ERR_UNSUPPORTED;
  if (s->block_size != 64 && s->block_size != 128 && s->block_size != 256)
    return MOE_ERR_UNSUPPORTED;
  if (s->flags & (MOE_COMBINE_ATOMIC | MOE_SCHED_QUOTA | MOE_FUSED_LAUNCH | MOE_COMBINE_FUSED))
    return MOE_ERR_UNSUPPORTED;
  const int64_t BM = s->block_size;
  const int64_t cap_rows = (s->S * s->k + s->E * (BM - 1) + BM - 1) / BM * BM;
  const int64_t s_rows = (s->S + BM - 1) / BM * BM;
  if (!fits_buffer(mx_blocked_bytes(cap_rows, s->H)) || !fits_buffer(mx_blocked_bytes(s_rows, s->H)) ||
      !fits_buffer(mx_blocked_bytes(cap_rows, s->D)) ||
      !fits_buffer(mx_blocked_bytes(s_rows, s->D_shared)) ||
      !fits_buffer(mx_blocked_bytes(s->D, s->H)) || !fits_buffer(mx_blocked_bytes(s->H, s->D)) ||
      !fits_buffer(mx_blocked_bytes(s->D_shared, s->H)) ||
      !fits_buffer(mx_blocked_bytes(s->H, s->D_shared)))
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

moe_status check_forward_dims(const moe_shape* s) {
  moe_status st = check_align_dims(s);
  if (st != MOE_OK) return st;
  if (s->H < 1 || s->D < 1 || s->D_shared < 0) return MOE_ERR_INVALID_ARGUMENT;
  if (s->H % 8 || s->D % 8 || s->D_shared % 8) return MOE_ERR_UNSUPPORTED;
  if (s->dtype == MOE_MXFP8) return check_mx_forward_dims(s);
  if (!forward_lds_ok(s->dtype, s->block_size)) return MOE_ERR_UNSUPPORTED;
  if ((s->flags & MOE_FUSED_LAUNCH) &&
      (s->dtype != MOE_BF16 || (s->flags & MOE_SCHED_QUOTA)))
    return MOE_ERR_UNSUPPORTED;
  // the fused combine replaces the slot combine pass of the two-launch path
  if ((s->flags & MOE_COMBINE_FUSED) && (s->flags & (MOE_COMBINE_ATOMIC | MOE_FUSED_LAUNCH)))
    return MOE_ERR_UNSUPPORTED;
  // batching and the queue-reset test hook act on the two-launch queues
  if ((s->flags & (MOE_SCHED_BATCH | MOE_TEST_SKIP_QUEUE_RESET)) &&
      (s->flags & (MOE_SCHED_QUOTA | MOE_FUSED_LAUNCH)))
    return MOE_ERR_UNSUPPORTED;
  // the kernels address A, each expert's weight matrices and the SwiGLU rows
  // through 32-bit buffer offsets: each must stay below 2 GiB
  const int64_t es = s->dtype == MOE_BF16 ? 2 : 4;
  const int64_t BM = s->block_size;
  const int64_t cap_rows = (s->S * s->k + s->E * (BM - 1) + BM - 1) / BM * BM;
  if (!fits_buffer(s->S * s->H * es) || !fits_buffer(s->H * s->D * es) ||
      !fits_buffer(s->H * s->D_shared * es) || !fits_buffer(cap_rows * s->D * es) ||
      !fits_buffer(((s->S + BM - 1) / BM * BM) * s->D_shared * es))
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

int64_t align_nseg(const moe_shape* s) { return (s->S * s->k + kAlignSeg - 1) / kAlignSeg; }

struct AlignLayout {
  size_t seg_counts, offsets, kept, total;
};

AlignLayout align_layout(const moe_shape* s) {
  AlignLayout L;
  L.seg_counts = 0;
  L.offsets = round_up((size_t)align_nseg(s) * s->E * sizeof(int32_t), kAlignUp);
  L.kept = L.offsets + round_up((size_t)s->E * sizeof(int64_t), kAlignUp);
  L.total = L.kept + round_up((size_t)s->E * sizeof(int32_t), kAlignUp);
  return L;
}

bool out_bf16(const moe_shape* s) {
  return s->dtype != MOE_F32 && (s->flags & MOE_OUTPUT_F32) == 0;
}

bool atomic_combine(const moe_shape* s) { return (s->flags & MOE_COMBINE_ATOMIC) != 0; }

struct ForwardLayout {
  size_t counters, ready, arr, oacc, y, ys, kept, h, hs, a_blk, as_blk, total;
  int64_t n_ready, n_arr;
};

bool fused_combine(const moe_shape* s) { return (s->flags & MOE_COMBINE_FUSED) != 0; }

// 256-column tiles of H (a down task's width)
int64_t arrival_tiles(const moe_shape* s) { return (s->H + 255) / 256; }

ForwardLayout forward_layout(const moe_shape* s) {
  const size_t es = s->dtype == MOE_BF16 ? 2 : 4;
  const int64_t BM = s->block_size;
  const int64_t F = s->S * s->k;
  const int64_t cap_rows = (F + s->E * (BM - 1) + BM - 1) / BM * BM;
  const int64_t s_rows = (s->S + BM - 1) / BM * BM;
  const bool atom = atomic_combine(s);
  ForwardLayout L;
  L.counters = 0;
  L.ready = round_up(kCounterInts * sizeof(int), kAlignUp);
  // one readiness counter per routed and per shared m-block (one launch only)
  L.n_ready = (s->flags & MOE_FUSED_LAUNCH) ? cap_rows / BM + s_rows / BM : 0;
  L.arr = L.ready + round_up((size_t)L.n_ready * sizeof(int), kAlignUp);
  // fused combine: one arrival counter per token and 256-column tile
  L.n_arr = fused_combine(s) ? s->S * arrival_tiles(s) : 0;
  L.oacc = L.arr + round_up((size_t)L.n_arr * sizeof(int), kAlignUp);
  // atomic combine: fp32 accumulator unless O itself is fp32
  const size_t oacc_bytes = (atom && out_bf16(s)) ? (size_t)s->S * s->H * sizeof(float) : 0;
  L.y = L.oacc + round_up(oacc_bytes, kAlignUp);
  const size_t y_bytes = atom ? 0 : (size_t)F * s->H * sizeof(float);
  L.ys = L.y + round_up(y_bytes, kAlignUp);
  const size_t ys_bytes = (atom || s->D_shared == 0) ? 0 : (size_t)s->S * s->H * sizeof(float);
  L.kept = L.ys + round_up(ys_bytes, kAlignUp);
  L.h = L.kept + round_up(atom ? 0 : (size_t)F, kAlignUp);
  if (s->dtype == MOE_MXFP8) {
    // stage-blocked quantised rows: h and hs, then the activation rows the
    // GEMMs read (routed in sorted order, shared in token order)
    L.hs = L.h + round_up((size_t)mx_blocked_bytes(cap_rows, s->D), kAlignUp);
    L.a_blk = L.hs + round_up((size_t)mx_blocked_bytes(s_rows, s->D_shared), kAlignUp);
    L.as_blk = L.a_blk + round_up((size_t)mx_blocked_bytes(cap_rows, s->H), kAlignUp);
    L.total = L.as_blk +
              round_up(s->D_shared > 0 ? (size_t)mx_blocked_bytes(s_rows, s->H) : 0, kAlignUp);
    return L;
  }
  L.hs = L.h + round_up((size_t)cap_rows * s->D * es, kAlignUp);
  L.total = L.hs + round_up((size_t)s_rows * s->D_shared * es, kAlignUp);
  L.a_blk = L.as_blk = L.total;
  return L;
}

// ------------------------------------------------------------ stage timing
struct ProfileRecord {
  int stage;
  hipEvent_t start, stop;
};

// per-task timing records (libraries built with MOE_TRACE)
void* g_trace = nullptr;
int64_t g_trace_cap = 0;

std::mutex g_prof_mu;
bool g_prof_on = false;
unsigned g_prof_mask = 0;  // bit s: time stage s
int g_prof_calls = 0;
std::vector<ProfileRecord> g_prof;
std::vector<hipEvent_t> g_event_pool;

hipEvent_t take_event() {
  if (!g_event_pool.empty()) {
    hipEvent_t e = g_event_pool.back();
    g_event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Launch one stage, bracketed by events when timing is on.
template <typename F>
hipError_t run_stage(int stage, hipStream_t st, F launch) {
  if (!g_prof_on || !((g_prof_mask >> stage) & 1u)) return launch();
  std::lock_guard<std::mutex> lk(g_prof_mu);
  ProfileRecord r{stage, take_event(), take_event()};
  if (r.start == nullptr || r.stop == nullptr) return hipErrorOutOfMemory;
  hipError_t e = hipEventRecord(r.start, st);
  if (e != hipSuccess) return e;
  e = launch();
  if (e != hipSuccess) return e;
  e = hipEventRecord(r.stop, st);
  if (e != hipSuccess) return e;
  g_prof.push_back(r);
  return hipSuccess;
}

// ------------------------------------------------ allocation-free workspace
// The workspace of moe_forward_noalloc: one array per GPU in the library's
// device image, held from the module's load until the process ends. In host
// code `scratch` names a host-side stand-in, not the device array: the
// device address comes from hipGetSymbolAddress, taken once per device with
// that device current, and only that address is passed to kernels.
constexpr size_t kScratchBytes = (size_t)MOE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {nullptr};

// The current device's scratch address (looked up on its first use).
moe_status scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_dev[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return MOE_ERR_HIP;
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return MOE_OK;
}

// moe_forward on a given workspace. timing = false: no stage events (the
// allocation-free entry point creates none).
moe_status forward_impl(const moe_shape* shape, const void* A, const void* W_up,
                        const void* W_gate, const void* W_down, const void* Ws_up,
                        const void* Ws_gate, const void* Ws_down, const float* topk_weights,
                        const int32_t* sorted_ids, const int32_t* expert_ids,
                        const int32_t* num_tokens_post_padded, void* O, void* workspace,
                        size_t workspace_bytes, void* stream, bool timing) {
  moe_status st = check_forward_dims(shape);
  if (st != MOE_OK) return st;
  const bool has_shared = shape->D_shared > 0;
  if ((Ws_up != nullptr) != has_shared || (Ws_gate != nullptr) != has_shared ||
      (Ws_down != nullptr) != has_shared)
    return MOE_ERR_INVALID_ARGUMENT;
  if (shape->S == 0) return MOE_OK;
  if (A == nullptr || W_up == nullptr || W_gate == nullptr || W_down == nullptr ||
      topk_weights == nullptr || sorted_ids == nullptr || expert_ids == nullptr ||
      num_tokens_post_padded == nullptr || O == nullptr || workspace == nullptr)
    return MOE_ERR_INVALID_ARGUMENT;
  const void* vec_ptrs[] = {A, W_up, W_gate, W_down, O, workspace};
  for (const void* q : vec_ptrs)
    if (!aligned16(q)) return MOE_ERR_UNSUPPORTED;
  if (has_shared && (!aligned16(Ws_up) || !aligned16(Ws_gate) || !aligned16(Ws_down)))
    return MOE_ERR_UNSUPPORTED;
  const ForwardLayout L = forward_layout(shape);
  if (workspace_bytes < L.total) return MOE_ERR_WORKSPACE_TOO_SMALL;

  char* ws = static_cast<char*>(workspace);
  ForwardParams p;
  p.A = A;
  p.Wu = W_up;
  p.Wg = W_gate;
  p.Wd = W_down;
  p.Wsu = Ws_up;
  p.Wsg = Ws_gate;
  p.Wsd = Ws_down;
  p.topk_w = topk_weights;
  p.sorted_ids = sorted_ids;
  p.expert_ids = expert_ids;
  p.ntpp = num_tokens_post_padded;
  p.O = O;
  p.atomic_combine = atomic_combine(shape) ? 1 : 0;
  p.out_bf16 = out_bf16(shape) ? 1 : 0;
  p.sched_quota = (shape->flags & MOE_SCHED_QUOTA) ? 1 : 0;
  p.Oacc = (p.atomic_combine && p.out_bf16) ? reinterpret_cast<float*>(ws + L.oacc)
                                            : reinterpret_cast<float*>(O);
  p.Y = reinterpret_cast<float*>(ws + L.y);
  p.Ys = reinterpret_cast<float*>(ws + L.ys);
  p.kept = reinterpret_cast<uint8_t*>(ws + L.kept);
  p.h = ws + L.h;
  p.hs = ws + L.hs;
  p.counters = reinterpret_cast<int*>(ws + L.counters);
  p.ready = reinterpret_cast<int*>(ws + L.ready);
  p.n_ready = L.n_ready;
  p.fused = (shape->flags & MOE_FUSED_LAUNCH) ? 1 : 0;
  p.fused_combine = fused_combine(shape) ? 1 : 0;
  p.arrivals = reinterpret_cast<int*>(ws + L.arr);
  p.arr_tiles = arrival_tiles(shape);
  p.claim_batch = (shape->flags & MOE_SCHED_BATCH) ? kClaimBatch : 1;
  p.split_tail = (shape->flags & MOE_SPLIT_TAIL) ? 1 : 0;
  p.keep_counters = (shape->flags & MOE_TEST_SKIP_QUEUE_RESET) ? 1 : 0;
  // Slot rows far larger than the 256 MB MALL (DeepSeek-V3 sizes: 0.94 GB)
  // go to HBM and come back from it anyway: the down kernel stores them and
  // the combine loads them with the non-temporal hint (measured: down -3%,
  // combine -15% there). Rows about the MALL's size (prefill, 0.27 GB) are
  // partly served from it, and the hint measured 8% slower for both.
  const double slot_bytes =
      (double)(shape->S * shape->k + (shape->D_shared > 0 ? shape->S : 0)) * shape->H * 4.0;
  p.slots_nt = (!atomic_combine(shape) && slot_bytes > 512.0 * (1 << 20)) ? 1 : 0;
  p.S = shape->S;
  p.H = shape->H;
  p.D = shape->D;
  p.E = shape->E;
  p.k = shape->k;
  p.Ds = shape->D_shared;
  p.F = shape->S * shape->k;
  p.grid = 0;
  p.a_blk = ws + L.a_blk;
  p.as_blk = ws + L.as_blk;
  p.trace = g_trace;
  p.trace_cap = g_trace_cap;
  // bf16 h in 32-column slabs per block (the down kernel's K stages then read
  // one contiguous block each); the fp32 path and other widths stay row-major
  p.h_blocked = (shape->dtype == MOE_BF16 && p.D % 32 == 0 && p.Ds % 32 == 0) ? 1 : 0;
  const int dt = shape->dtype;
  const int BM = shape->block_size;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  if (timing && g_prof_on) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    ++g_prof_calls;
  }
  auto run_stage = [&](int stage, hipStream_t st, auto launch) {
    return timing ? ::run_stage(stage, st, launch) : launch();
  };
  if (run_stage(0, hs, [&] { return launch_forward_setup(p, hs); }) != hipSuccess)
    return MOE_ERR_HIP;
  if (dt == MOE_MXFP8) {
    // activation rows quantised into the stage-blocked layout the GEMMs read,
    // then the two MXFP8 GEMMs
    const int64_t cap_rows = (p.F + p.E * (BM - 1) + BM - 1) / BM * BM;
    const int64_t s_rows = p.Ds > 0 ? (p.S + BM - 1) / BM * BM : 0;
    if (run_stage(4, hs, [&] { return launch_mx_gather(p, BM, cap_rows, s_rows, hs); }) !=
        hipSuccess)
      return MOE_ERR_HIP;
    if (run_stage(1, hs, [&] { return launch_forward_mx(p, BM, true, hs); }) != hipSuccess)
      return MOE_ERR_HIP;
    if (run_stage(2, hs, [&] { return launch_forward_mx(p, BM, false, hs); }) != hipSuccess)
      return MOE_ERR_HIP;
  } else if (p.fused) {
    if (run_stage(1, hs, [&] { return launch_forward_fused(p, BM, hs); }) != hipSuccess)
      return MOE_ERR_HIP;
  } else {
    if (run_stage(1, hs, [&] { return launch_forward_upgate(p, dt, BM, hs); }) != hipSuccess)
      return MOE_ERR_HIP;
    if (run_stage(2, hs, [&] { return launch_forward_down(p, dt, BM, hs); }) != hipSuccess)
      return MOE_ERR_HIP;
  }
  if (p.atomic_combine) {
    if (p.out_bf16 &&
        run_stage(3, hs, [&] { return launch_forward_finalize(p, hs); }) != hipSuccess)
      return MOE_ERR_HIP;
  } else if (p.fused_combine) {
    // the combine ran in the down epilogue; tokens no task reached get zeros
    if (p.Ds == 0 &&
        run_stage(3, hs, [&] { return launch_zero_unrouted(p, hs); }) != hipSuccess)
      return MOE_ERR_HIP;
  } else if (run_stage(3, hs, [&] { return launch_forward_combine(p, hs); }) != hipSuccess) {
    return MOE_ERR_HIP;
  }
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARGUMENT: return "MOE_ERR_INVALID_ARGUMENT";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "MOE_ERR_WORKSPACE_TOO_SMALL";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
  }
  return "MOE_ERR_UNKNOWN";
}

size_t moe_gate_workspace_bytes(const moe_shape* shape) {
  if (check_routing_dims(shape) != MOE_OK) return 0;
  const GateSplit g = gate_split_plan(shape->S, shape->H, shape->E,
                                      shape->dtype == MOE_MXFP8 ? MOE_BF16 : shape->dtype);
  if (g.splits < 2) return 0;
  return round_up((size_t)g.splits * shape->S * shape->E * sizeof(float), kAlignUp);
}

moe_status moe_gate_topk(const moe_shape* shape, const void* A, const void* W_router,
                         const float* router_bias, const float* logits_in, float* logits_out,
                         int32_t* topk_ids, float* topk_weights, void* workspace,
                         size_t workspace_bytes, void* stream) {
  moe_status st = check_routing_dims(shape);
  if (st != MOE_OK) return st;
  if (shape->renormalize != 0 && shape->renormalize != 1) return MOE_ERR_INVALID_ARGUMENT;
  if (shape->S == 0) return MOE_OK;
  if (topk_ids == nullptr || topk_weights == nullptr) return MOE_ERR_INVALID_ARGUMENT;
  const float* G = logits_in;
  // the MXFP8 layer's activations and router weights are bf16
  const int gdt = shape->dtype == MOE_MXFP8 ? MOE_BF16 : shape->dtype;
  if (logits_in == nullptr) {
    if (A == nullptr || W_router == nullptr || logits_out == nullptr) return MOE_ERR_INVALID_ARGUMENT;
    if (shape->H < 1) return MOE_ERR_INVALID_ARGUMENT;
    if (shape->H % 8 || !aligned16(A) || !aligned16(W_router)) return MOE_ERR_UNSUPPORTED;
    const int64_t es = gdt == MOE_BF16 ? 2 : 4;
    if (!fits_buffer(shape->S * shape->H * es) || !fits_buffer(shape->H * shape->E * es))
      return MOE_ERR_UNSUPPORTED;
    G = logits_out;
  }
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  TopkParams tp{G, topk_ids, topk_weights, shape->S, shape->E, shape->k, shape->renormalize};
  if (logits_in == nullptr) {
    GateParams gp{A, W_router, router_bias, logits_out, shape->S, shape->H, shape->E};
    const GateSplit plan = gate_split_plan(shape->S, shape->H, shape->E, gdt);
    if (plan.splits >= 2) {  // H split: partial scores, then sum + routing
      if (workspace == nullptr || workspace_bytes < moe_gate_workspace_bytes(shape))
        return MOE_ERR_WORKSPACE_TOO_SMALL;
      if (!aligned16(workspace)) return MOE_ERR_UNSUPPORTED;
      return launch_gate_split(gp, tp, plan, static_cast<float*>(workspace), hs) == hipSuccess
                 ? MOE_OK
                 : MOE_ERR_HIP;
    }
    if (gate_topk_fusable(gp, gdt))  // one kernel: scores and routing
      return launch_gate_topk(gp, tp, hs) == hipSuccess ? MOE_OK : MOE_ERR_HIP;
    if (launch_gate(gp, gdt, hs) != hipSuccess) return MOE_ERR_HIP;
  } else if (logits_out != nullptr && logits_out != logits_in) {
    if (hipMemcpyAsync(logits_out, logits_in, (size_t)shape->S * shape->E * sizeof(float),
                       hipMemcpyDeviceToDevice, hs) != hipSuccess)
      return MOE_ERR_HIP;
  }
  if (launch_topk(tp, hs) != hipSuccess) return MOE_ERR_HIP;
  return MOE_OK;
}

size_t moe_align_workspace_bytes(const moe_shape* shape) {
  if (check_align_dims(shape) != MOE_OK) return 0;
  return align_layout(shape).total;
}

moe_status moe_align_block_size(const moe_shape* shape, const int32_t* topk_ids,
                                int32_t* sorted_ids, int32_t* expert_ids,
                                int32_t* num_tokens_post_padded, int32_t* expert_counts,
                                void* workspace, size_t workspace_bytes, void* stream) {
  moe_status st = check_align_dims(shape);
  if (st != MOE_OK) return st;
  if ((topk_ids == nullptr && shape->S > 0) || sorted_ids == nullptr || expert_ids == nullptr ||
      num_tokens_post_padded == nullptr || expert_counts == nullptr || workspace == nullptr)
    return MOE_ERR_INVALID_ARGUMENT;
  const AlignLayout L = align_layout(shape);
  if (workspace_bytes < L.total) return MOE_ERR_WORKSPACE_TOO_SMALL;
  char* ws = static_cast<char*>(workspace);
  AlignParams p;
  p.ids = topk_ids;
  p.sorted_ids = sorted_ids;
  p.expert_ids = expert_ids;
  p.ntpp = num_tokens_post_padded;
  p.counts = expert_counts;
  p.seg_counts = reinterpret_cast<int32_t*>(ws + L.seg_counts);
  p.offsets = reinterpret_cast<int64_t*>(ws + L.offsets);
  p.kept = reinterpret_cast<int32_t*>(ws + L.kept);
  p.F = shape->S * shape->k;
  p.E = shape->E;
  p.BM = shape->block_size;
  p.C = shape->capacity;
  p.nseg = align_nseg(shape);
  if (launch_align(p, reinterpret_cast<hipStream_t>(stream)) != hipSuccess) return MOE_ERR_HIP;
  return MOE_OK;
}

size_t moe_forward_workspace_bytes(const moe_shape* shape) {
  if (check_forward_dims(shape) != MOE_OK) return 0;
  return forward_layout(shape).total;
}

moe_status moe_forward(const moe_shape* shape, const void* A, const void* W_up,
                       const void* W_gate, const void* W_down, const void* Ws_up,
                       const void* Ws_gate, const void* Ws_down, const float* topk_weights,
                       const int32_t* sorted_ids, const int32_t* expert_ids,
                       const int32_t* num_tokens_post_padded, void* O, void* workspace,
                       size_t workspace_bytes, void* stream) {
  return forward_impl(shape, A, W_up, W_gate, W_down, Ws_up, Ws_gate, Ws_down, topk_weights,
                      sorted_ids, expert_ids, num_tokens_post_padded, O, workspace,
                      workspace_bytes, stream, true);
}

moe_status moe_forward_noalloc(const moe_shape* shape, const void* A, const void* W_up,
                               const void* W_gate, const void* W_down, const void* Ws_up,
                               const void* Ws_gate, const void* Ws_down,
                               const float* topk_weights, const int32_t* sorted_ids,
                               const int32_t* expert_ids, const int32_t* num_tokens_post_padded,
                               void* O, void* stream) {
  moe_status st = check_forward_dims(shape);
  if (st != MOE_OK) return st;
  if (forward_layout(shape).total > sizeof(scratch)) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if (shape->S == 0)
    return forward_impl(shape, A, W_up, W_gate, W_down, Ws_up, Ws_gate, Ws_down, topk_weights,
                        sorted_ids, expert_ids, num_tokens_post_padded, O, nullptr, 0, stream,
                        false);
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != MOE_OK) return st;
  return forward_impl(shape, A, W_up, W_gate, W_down, Ws_up, Ws_gate, Ws_down, topk_weights,
                      sorted_ids, expert_ids, num_tokens_post_padded, O, ws, sizeof(scratch),
                      stream, false);
}


size_t moe_mxfp8_weight_bytes(int64_t E, int64_t K, int64_t N) {
  if (E < 1 || K < 64 || N < 128 || K % 64 || N % 128) return 0;
  return (size_t)(E * mx_blocked_bytes(N, K));
}

moe_status moe_pack_mxfp8_weights(const void* W, int64_t E, int64_t K, int64_t N, void* packed,
                                  void* stream) {
  if (W == nullptr || packed == nullptr) return MOE_ERR_INVALID_ARGUMENT;
  if (E < 1 || K < 1 || N < 1) return MOE_ERR_INVALID_ARGUMENT;
  if (K % 64 || N % 128 || !aligned16(W) || !aligned16(packed)) return MOE_ERR_UNSUPPORTED;
  return launch_mx_pack_weights(W, E, K, N, packed, reinterpret_cast<hipStream_t>(stream)) ==
                 hipSuccess
             ? MOE_OK
             : MOE_ERR_HIP;
}

moe_status moe_quantize_mxfp8(const void* X, int64_t R, int64_t K, int32_t dtype, uint8_t* codes,
                              uint8_t* scales, void* stream) {
  if (R < 0 || K < 1 || (dtype != MOE_F32 && dtype != MOE_BF16)) return MOE_ERR_INVALID_ARGUMENT;
  if (R == 0) return MOE_OK;
  if (X == nullptr || codes == nullptr || scales == nullptr) return MOE_ERR_INVALID_ARGUMENT;
  if (K % 32 || !aligned16(X) || !aligned16(codes)) return MOE_ERR_UNSUPPORTED;
  return launch_mx_quantize_rows(X, dtype, R, K, codes, scales,
                                 reinterpret_cast<hipStream_t>(stream)) == hipSuccess
             ? MOE_OK
             : MOE_ERR_HIP;
}

moe_status moe_trace_attach(void* buffer, size_t bytes) {
  if (!MOE_TRACE) return MOE_ERR_UNSUPPORTED;
  if (buffer == nullptr) {
    g_trace = nullptr;
    g_trace_cap = 0;
    return MOE_OK;
  }
  if (bytes < (size_t)kTraceHeaderBytes || (reinterpret_cast<uintptr_t>(buffer) & 63) != 0)
    return MOE_ERR_INVALID_ARGUMENT;
  g_trace = buffer;
  g_trace_cap = (int64_t)((bytes - kTraceHeaderBytes) / kTraceRecBytes);
  return MOE_OK;
}

moe_status moe_device_query(int* cu_count, int* max_clock_khz, char* name, size_t name_bytes) {
  if (name != nullptr && name_bytes == 0) return MOE_ERR_INVALID_ARGUMENT;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (cu_count != nullptr &&
      hipDeviceGetAttribute(cu_count, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return MOE_ERR_HIP;
  if (max_clock_khz != nullptr &&
      hipDeviceGetAttribute(max_clock_khz, hipDeviceAttributeClockRate, dev) != hipSuccess)
    return MOE_ERR_HIP;
  if (name != nullptr) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MOE_ERR_HIP;
    size_t i = 0;
    for (; i + 1 < name_bytes && i < sizeof(prop.name) && prop.name[i] != 0; ++i)
      name[i] = prop.name[i];
    name[i] = 0;
  }
  return MOE_OK;
}

moe_status moe_profile_enable(int stage_mask) {
  if (stage_mask < 0 || stage_mask > 31) return MOE_ERR_INVALID_ARGUMENT;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_on = stage_mask != 0;
  g_prof_mask = (unsigned)stage_mask;
  return MOE_OK;
}

moe_status moe_profile_collect(float* stage_ms, int max_stages, int* n_calls) {
  if (max_stages < 0 || (max_stages > 0 && stage_ms == nullptr)) return MOE_ERR_INVALID_ARGUMENT;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  moe_status st = MOE_OK;
  for (const ProfileRecord& r : g_prof) {
    float ms = 0.f;
    if (hipEventSynchronize(r.stop) != hipSuccess ||
        hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess) {
      st = MOE_ERR_HIP;
    } else if (r.stage < max_stages) {
      stage_ms[r.stage] += ms;
    }
    g_event_pool.push_back(r.start);
    g_event_pool.push_back(r.stop);
  }
  g_prof.clear();
  if (n_calls) *n_calls = g_prof_calls;
  g_prof_calls = 0;
  return st;
}

}  // extern "C"
