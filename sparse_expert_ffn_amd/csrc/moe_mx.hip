// MXFP8 mode of the MoE layer: FP8 E4M3 operands in blocks of 32 sharing an
// E8M0 scale (the OCP Microscaling format; the Mixture-of-Kittens page names
// MXFP8 as the low-precision format of its MoE kernels).
//
//  - mx_quantize_rows_kernel: plain row-major quantisation of any [R][K]
//    matrix (codes [R][K], scales [R][K/32]).
//  - mx_pack_weights_kernel: an expert weight tensor [E][K][N] (bf16, the
//    layer's layout, K the reduction dimension) into the stage-blocked
//    layout of the MXFP8 tile core: per expert, per n-tile of 128 columns,
//    per stage of 64 K values, the 128 columns' 64 codes (K-contiguous), then
//    their two scales.
//  - mx_gather_kernel: the token rows each m-block's tasks read (routed rows
//    in sorted order, shared-expert rows in token order), quantised into the
//    same stage-blocked layout: every K stage of an m-block is one
//    contiguous stretch.
//  - upgate_mx_kernel / down_mx_kernel: the persistent grouped GEMMs of the
//    expert FFN on the MXFP8 core (gemm_mx.h), with the task scheduling of
//    the bf16 kernels; the up/gate epilogue quantises each SwiGLU row's 32-
//    column blocks straight into the stage-blocked h the down kernel reads.
//
// Quantisation rule (one block of 32 values v): scale 2^e with e =
// floor(log2 max |v|) - 8 clamped to [-127, 127] (-127 for an all-zero
// block), stored as e + 127; elements v / 2^e rounded to the nearest E4M3
// value, ties to the even code, magnitudes past 448 saturating to 448.
#include "gemm_mx.h"
#include "moe_sched.h"

namespace moe {

// ------------------------------------------------------------- the format
// Scale exponent of a block whose largest magnitude is amax (fp32).
__device__ __forceinline__ int mx_scale_exp(float amax) {
  const uint32_t b = __float_as_uint(amax);
  const int be = (int)((b >> 23) & 0xFF);  // biased exponent; 0: zero or subnormal
  if (be == 0) return -127;               // below 2^-126: the smallest scale
  const int e = be - 127 - 8;
  return e < -127 ? -127 : e;             // be <= 254 keeps e <= 119
}

// E4M3 codes (bytes 0, 1 of the result; bytes 2, 3 from `old`, or with
// HIGH, bytes 2, 3 = the codes and bytes 0, 1 from `old`) of the finite
// values x0, x1: the code nearest to the value, ties to the even code, a
// magnitude of 448 or more giving 448 and a zero result keeping the sign.
// v_cvt_pk_fp8_f32 rounds to nearest even into the OCP E4M3 format; with its
// inputs clamped to +-448 it saturates as the rule asks. (Checked on the GPU
// against a software encoder of the same rule, for every float of magnitude
// up to 1024, both signs: no difference.)
template <bool HIGH = false>
__device__ __forceinline__ uint32_t e4m3_pair(float x0, float x1, uint32_t old = 0) {
  x0 = fminf(fmaxf(x0, -448.0f), 448.0f);
  x1 = fminf(fmaxf(x1, -448.0f), 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, (int)old, HIGH);
}

// The largest of v over each group of 32 lanes (lanes 0-31, 32-63), in every
// lane of the group. Quad swaps (xor 1, xor 2) and the half-row and row
// mirrors run on DPP (a max is its own all-reduce under any pairing that
// joins the halves), then one swizzle joins the two 16-lane rows.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float max32_lanes(float v) {
  v = fmaxf(v, dpp_f32<0xB1>(v));   // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp_f32<0x4E>(v));   // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp_f32<0x141>(v));  // row_half_mirror
  v = fmaxf(v, dpp_f32<0x140>(v));  // row_mirror
  // lane ^ 16 within each 32 (bitmask swizzle: and 0x1F, xor 0x10)
  return fmaxf(v, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F)));
}

// Quantise 32 values (one block) to codes packed 4 per uint32 and the scale.
__device__ __forceinline__ uint32_t mx_block(const float (&v)[32], uint32_t (&codes)[8]) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const int e = mx_scale_exp(amax);
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    const uint32_t lo = e4m3_pair(ldexpf(v[4 * w], -e), ldexpf(v[4 * w + 1], -e));
    codes[w] = e4m3_pair<true>(ldexpf(v[4 * w + 2], -e), ldexpf(v[4 * w + 3], -e), lo);
  }
  return (uint32_t)(e + 127);
}

template <typename T>
__device__ __forceinline__ void load32(const T* p, float (&v)[32]);
template <>
__device__ __forceinline__ void load32<bf16_t>(const bf16_t* p, float (&v)[32]) {
  const uint4* q = reinterpret_cast<const uint4*>(p);
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint4 x = q[w];
    const uint32_t u[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[8 * w + 2 * j] = __uint_as_float(u[j] << 16);
      v[8 * w + 2 * j + 1] = __uint_as_float(u[j] & 0xFFFF0000u);
    }
  }
}
template <>
__device__ __forceinline__ void load32<float>(const float* p, float (&v)[32]) {
  const float4* q = reinterpret_cast<const float4*>(p);
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    const float4 x = q[w];
    v[4 * w] = x.x;
    v[4 * w + 1] = x.y;
    v[4 * w + 2] = x.z;
    v[4 * w + 3] = x.w;
  }
}

// ------------------------------------------------- plain row quantisation
// One thread per block of 32: X [R][K] (bf16 or fp32) -> codes [R][K],
// scales [R][K/32].
template <typename T>
__global__ __launch_bounds__(256) void mx_quantize_rows_kernel(const T* X, int64_t R, int64_t K,
                                                               uint8_t* codes, uint8_t* scales) {
  const int64_t nb = K / 32;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= R * nb) return;
  const int64_t r = i / nb, b = i - r * nb;
  float v[32];
  load32<T>(X + r * K + b * 32, v);
  uint32_t c[8];
  scales[i] = (uint8_t)mx_block(v, c);
  uint4* dst = reinterpret_cast<uint4*>(codes + r * K + b * 32);
  dst[0] = make_uint4(c[0], c[1], c[2], c[3]);
  dst[1] = make_uint4(c[4], c[5], c[6], c[7]);
}

hipError_t launch_mx_quantize_rows(const void* X, int dtype, int64_t R, int64_t K, uint8_t* codes,
                                   uint8_t* scales, hipStream_t st) {
  const int64_t n = R * (K / 32);
  if (n == 0) return hipSuccess;
  const unsigned grid = (unsigned)((n + 255) / 256);
  if (dtype == 0)
    hipLaunchKernelGGL(mx_quantize_rows_kernel<float>, dim3(grid), dim3(256), 0, st,
                       static_cast<const float*>(X), R, K, codes, scales);
  else
    hipLaunchKernelGGL(mx_quantize_rows_kernel<bf16_t>, dim3(grid), dim3(256), 0, st,
                       static_cast<const bf16_t*>(X), R, K, codes, scales);
  return hipGetLastError();
}

// ------------------------------------------------------- weight packing
// Stage-blocked weights: expert e, n-tile j (128 columns), stage s (64 K):
// block (e * NT + j) * KS + s of mx_stage_bytes(128) bytes, NT = N / 128,
// KS = K / 64; inside, column c's 64 codes at c * 64, its two scales at
// 128 * 64 + 2 c.
// One thread per (expert, column, block of 32 K): reads the 32 values of its
// column (strided by N; neighbouring threads read neighbouring columns).
__global__ __launch_bounds__(256) void mx_pack_weights_kernel(const bf16_t* W, int64_t E,
                                                              int64_t K, int64_t N,
                                                              uint8_t* packed) {
  const int64_t kb = K / 32;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // ((e * kb) + b) * N + n
  if (i >= E * kb * N) return;
  const int64_t n = i % N;
  const int64_t b = (i / N) % kb;
  const int64_t e = i / (N * kb);
  const bf16_t* src = W + (e * K + b * 32) * N + n;
  float v[32];
#pragma unroll
  for (int t = 0; t < 32; ++t) v[t] = bf16_to_f32(src[(int64_t)t * N]);
  uint32_t c[8];
  const uint32_t sc = mx_block(v, c);
  const int64_t NT = N / 128, KS = K / 64;
  const int64_t j = n / 128, col = n % 128, s = b / 2, half = b % 2;
  uint8_t* blk = packed + ((e * NT + j) * KS + s) * (int64_t)mx_stage_bytes(128);
  uint4* dst = reinterpret_cast<uint4*>(blk + col * 64 + half * 32);
  dst[0] = make_uint4(c[0], c[1], c[2], c[3]);
  dst[1] = make_uint4(c[4], c[5], c[6], c[7]);
  blk[128 * 64 + col * 2 + half] = (uint8_t)sc;
}

hipError_t launch_mx_pack_weights(const void* W, int64_t E, int64_t K, int64_t N, void* packed,
                                  hipStream_t st) {
  const int64_t n = E * (K / 32) * N;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(mx_pack_weights_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                     st, static_cast<const bf16_t*>(W), E, K, N, static_cast<uint8_t*>(packed));
  return hipGetLastError();
}

}  // namespace moe

namespace moe {

// ------------------------------------------------- activation rows, blocked
// Stage-blocked activation rows: m-block b of BM rows holds K/64 stages of
// mx_stage_bytes(BM) bytes at (b * (K/64) + s) * mx_stage_bytes(BM); inside,
// row r's 64 codes at r * 64 and its two scales at BM * 64 + 2 r.
// Routed rows: row p of the sorted order is token sorted_ids[p] / k (a
// sentinel: a zero row), for p < num_tokens_post_padded; shared rows: row r is
// token r (past S: a zero row). One thread per (row, block of 32 K values).
__global__ __launch_bounds__(256) void mx_gather_kernel(const bf16_t* A, int64_t S, int64_t H,
                                                        int64_t k, int64_t F,
                                                        const int32_t* sorted_ids,
                                                        const int32_t* ntpp, int64_t cap_rows,
                                                        int64_t s_rows, int BM, uint8_t* a_blk,
                                                        uint8_t* as_blk) {
  const int64_t kb = H / 32;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (cap_rows + s_rows) * kb) return;
  const int64_t row = i / kb, b32 = i - row * kb;
  int64_t rr, tok;
  uint8_t* base;
  if (row < cap_rows) {
    if (row >= (int64_t)*ntpp) return;  // past the used blocks
    const int32_t f = sorted_ids[row];
    tok = f < F ? f / k : -1;
    rr = row;
    base = a_blk;
  } else {
    rr = row - cap_rows;
    tok = rr < S ? rr : -1;
    base = as_blk;
  }
  const int64_t b = rr / BM, r = rr - b * BM, s = b32 / 2, half = b32 & 1;
  uint8_t* blk = base + (b * (H / 64) + s) * (int64_t)mx_stage_bytes(BM);
  uint32_t c[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  uint32_t sc = 0;
  if (tok >= 0) {
    float v[32];
    load32<bf16_t>(A + tok * H + b32 * 32, v);
    sc = mx_block(v, c);
  }
  uint4* dst = reinterpret_cast<uint4*>(blk + r * 64 + half * 32);
  dst[0] = make_uint4(c[0], c[1], c[2], c[3]);
  dst[1] = make_uint4(c[4], c[5], c[6], c[7]);
  blk[BM * 64 + r * 2 + half] = (uint8_t)sc;
}

hipError_t launch_mx_gather(const ForwardParams& p, int BM, int64_t cap_rows, int64_t s_rows,
                            hipStream_t st) {
  const int64_t n = (cap_rows + s_rows) * (p.H / 32);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(mx_gather_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                     static_cast<const bf16_t*>(p.A), p.S, p.H, p.k, p.F, p.sorted_ids, p.ntpp,
                     cap_rows, s_rows, BM, static_cast<uint8_t*>(p.a_blk),
                     static_cast<uint8_t*>(p.as_blk));
  return hipGetLastError();
}

// ----------------------------------------------------- the grouped GEMMs
// Bytes of one expert's packed weights [K][N] and of one n-tile's stages.
__device__ __forceinline__ int64_t mx_tile_bytes(int64_t K) {
  return (K / kMxK) * (int64_t)mx_stage_bytes(128);
}

// Rows of a task's m-block (routed: sorted ids; shared: tokens) into LDS;
// the up/gate kernel's first n-tile task of a routed block marks its kept
// assignments for the slot combine.
__device__ __forceinline__ void mx_rows(const ForwardParams& p, bool shared, int64_t b, int BM,
                                        bool mark_kept, int* s_tok, int* s_f, float* s_w) {
  if (threadIdx.x < BM) {
    const int r = threadIdx.x;
    if (!shared) {
      const int f = p.sorted_ids[b * BM + r];
      const bool real = f < p.F;
      s_tok[r] = real ? (int)(f / p.k) : -1;
      if (s_f) s_f[r] = real ? f : -1;
      if (mark_kept && real) p.kept[f] = 1;
    } else {
      const int64_t s = b * BM + r;
      s_tok[r] = s < p.S ? (int)s : -1;
      if (s_f) s_f[r] = s_tok[r];
    }
  }
  (void)s_w;
  __syncthreads();
}

// Up/gate task (m-block b, n-tile j of 128 columns of D): h = SiLU(u) * g,
// quantised per row and 32-column block into the stage-blocked h.
template <int BM, typename TG>
__device__ __forceinline__ void upgate_mx_task(const ForwardParams& p, const TaskSpace& ts,
                                               int64_t t, TG& g, int* s_tok) {
  const bool shared = t >= ts.t_r;
  int64_t b, j;
  if (!shared)
    decode_task(t, ts.nb_r, ts.nn_r, ts.gb_r, b, j);
  else
    decode_task(t - ts.t_r, ts.nb_s, ts.nn_s, kGroupBlocks, b, j);
  mx_rows(p, shared, b, BM, !p.atomic_combine && j == 0 && !shared, s_tok, nullptr, nullptr);
  const int64_t N = shared ? p.Ds : p.D;
  const int64_t KS = p.H / kMxK;
  const int64_t nblk = shared ? ts.nb_s : ts.nb_r;
  const char* Bm[2];
  uint32_t bb[2], bo[2];
  const int64_t wbytes = (N / 128) * mx_tile_bytes(p.H);
  if (!shared) {
    const int64_t e = __builtin_amdgcn_readfirstlane(p.expert_ids[b]);
    Bm[0] = static_cast<const char*>(p.Wu) + e * wbytes;
    Bm[1] = static_cast<const char*>(p.Wg) + e * wbytes;
  } else {
    Bm[0] = static_cast<const char*>(p.Wsu);
    Bm[1] = static_cast<const char*>(p.Wsg);
  }
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    bb[m] = (uint32_t)wbytes;
    bo[m] = (uint32_t)(j * mx_tile_bytes(p.H));
  }
  const int64_t a_stage_set = KS * (int64_t)TG::A_BYTES;  // one m-block
  g.setup(shared ? p.as_blk : p.a_blk, (uint32_t)(nblk * a_stage_set), (uint32_t)(b * a_stage_set),
          Bm, bb, bo, (int)KS);
  trace_stamp(1);
  g.mainloop(lds_ring<TG>(), g.active_blocks([&](int r) { return s_tok[r] >= 0; }));
  trace_stamp(2);
  // epilogue: the wave's 32 columns of a row form one MX block of h
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  int lrow = (wave / TG::WN) * (BM / TG::WM) + 4 * (lane >> 5);
  int lcol = (wave % TG::WN) * 32 + (lane & 31);
  asm volatile("" : "+v"(lrow), "+v"(lcol));
  const int64_t col = j * 128 + lcol;          // column of h (N a multiple of 128)
  const int64_t s = col / kMxK, half = (col % kMxK) / 32;
  uint8_t* blk = static_cast<uint8_t*>(shared ? p.hs : p.h) +
                 (b * (N / kMxK) + s) * (int64_t)TG::A_BYTES;
#pragma unroll
  for (int i = 0; i < TG::MI; ++i) {
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int r = 0; r < 16; r += 2) {  // two rows per conversion
      float x[2];
      int e[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const float h = silu_f32(g.acc[0][i][r + q]) * g.acc[1][i][r + q];
        e[q] = mx_scale_exp(max32_lanes(fabsf(h)));
        x[q] = ldexpf(h, -e[q]);
      }
      const uint32_t c = e4m3_pair(x[0], x[1]);
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int row = lrow + i * 32 + 8 * ((r + q) >> 2) + ((r + q) & 3);
        if (s_tok[row] >= 0) {
          blk[row * 64 + (col % kMxK)] = (uint8_t)(c >> (8 * q));
          if ((lane & 31) == 0) blk[BM * 64 + row * 2 + half] = (uint8_t)(e[q] + 127);
        }
      }
    }
  }
}

template <int BM, bool BS>
__global__ __launch_bounds__(512, 1) void upgate_mx_kernel(ForwardParams p) {
  using TG = TileGemmMx<BM, 2, BS, true>;  // the wait-state form of the loads: the
                                           // kernels restore descriptors from VGPR lanes
  __shared__ int64_t s_task;
  __shared__ int s_tok[BM];
  const TaskSpace ts = task_space(p, BM, 128, p.D, p.Ds);
  Claimer cs(blockIdx.x % kXcds);
  TG g;
  for (;;) {
    if (threadIdx.x == 0) s_task = claim_checked(p, 0, ts.total, false, cs) >> 2;
    trace_stamp(0);
    __syncthreads();
    const int64_t t = uniform64(s_task);
    if (t < 0) {
      trace_record(p, kTraceUpgate, -1);
      break;
    }
    upgate_mx_task<BM>(p, ts, t, g, s_tok);
    trace_record(p, kTraceUpgate, t << 2);
  }
}

// Down task (m-block b, column strips 2j and 2j + 1 of 128 columns of H):
// y = h . W_down for each kept row into its fp32 slot (as the bf16 kernel).
template <int BM, typename TG>
__device__ __forceinline__ void down_mx_task(const ForwardParams& p, const TaskSpace& ts,
                                             int64_t t, TG& g, int* s_tok, int* s_f) {
  const bool shared = t >= ts.t_r;
  int64_t b, j;
  if (!shared)
    decode_task(t, ts.nb_r, ts.nn_r, ts.gb_r, b, j);
  else
    decode_task(t - ts.t_r, ts.nb_s, ts.nn_s, kGroupBlocks, b, j);
  mx_rows(p, shared, b, BM, false, s_tok, s_f, nullptr);
  const int64_t K = shared ? p.Ds : p.D;
  const int64_t KS = K / kMxK;
  const int64_t NT = p.H / 128;
  const int64_t nblk = shared ? ts.nb_s : ts.nb_r;
  const int64_t wbytes = NT * mx_tile_bytes(K);
  const char* Wb;
  if (!shared) {
    const int64_t e = __builtin_amdgcn_readfirstlane(p.expert_ids[b]);
    Wb = static_cast<const char*>(p.Wd) + e * wbytes;
  } else {
    Wb = static_cast<const char*>(p.Wsd);
  }
  const char* Bm[2] = {Wb, Wb};
  uint32_t bb[2], bo[2];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int64_t strip = 2 * j + m;
    bb[m] = (uint32_t)wbytes;
    bo[m] = strip < NT ? (uint32_t)(strip * mx_tile_bytes(K)) : kOob;
  }
  const int64_t a_stage_set = KS * (int64_t)TG::A_BYTES;
  g.setup(shared ? p.hs : p.h, (uint32_t)(nblk * a_stage_set), (uint32_t)(b * a_stage_set), Bm,
          bb, bo, (int)KS);
  trace_stamp(1);
  g.mainloop(lds_ring<TG>(), g.active_blocks([&](int r) { return s_tok[r] >= 0; }));
  trace_stamp(2);
  const int64_t H = p.H;
  const int64_t n0 = j * 256;
  float* Yb = shared ? p.Ys : p.Y;
  if (p.slots_nt)
    g.for_each([&](int m, int row, int c, float v) {
      const int f = s_f[row];
      const int64_t n = n0 + m * 128 + c;
      if (f >= 0 && n < H) __builtin_nontemporal_store(v, Yb + (size_t)f * H + n);
    });
  else
    g.for_each([&](int m, int row, int c, float v) {
      const int f = s_f[row];
      const int64_t n = n0 + m * 128 + c;
      if (f >= 0 && n < H) Yb[(size_t)f * H + n] = v;
    });
}

template <int BM, bool BS>
__global__ __launch_bounds__(512, 1) void down_mx_kernel(ForwardParams p) {
  using TG = TileGemmMx<BM, 2, BS, true>;  // the wait-state form of the loads: the
                                           // kernels restore descriptors from VGPR lanes
  __shared__ int64_t s_task;
  __shared__ int s_tok[BM];
  __shared__ int s_f[BM];
  const TaskSpace ts = task_space(p, BM, 256, p.H, p.H);
  Claimer cs(blockIdx.x % kXcds);
  TG g;
  for (;;) {
    if (threadIdx.x == 0) s_task = claim_checked(p, 1, ts.total, false, cs) >> 2;
    trace_stamp(0);
    __syncthreads();
    const int64_t t = uniform64(s_task);
    if (t < 0) {
      trace_record(p, kTraceDown, -1);
      break;
    }
    down_mx_task<BM>(p, ts, t, g, s_tok, s_f);
    trace_record(p, kTraceDown, t << 2);
  }
}

template <int BM>
static hipError_t launch_mx_bm(const ForwardParams& p, bool up, bool bs, hipStream_t st) {
  if (up)
    return bs ? launch_persistent(upgate_mx_kernel<BM, true>, 0, 512, p, st)
              : launch_persistent(upgate_mx_kernel<BM, false>, 0, 512, p, st);
  return bs ? launch_persistent(down_mx_kernel<BM, true>, 0, 512, p, st)
            : launch_persistent(down_mx_kernel<BM, false>, 0, 512, p, st);
}

hipError_t launch_forward_mx(const ForwardParams& p, int BM, bool up, hipStream_t st) {
  // the weights are read once per call when the routing leaves about one
  // m-block per expert (as the bf16 kernels)
  const bool bs = p.E > 0 && 2 * ((p.F + p.E - 1) / p.E) <= BM;
  switch (BM) {
    case 64: return launch_mx_bm<64>(p, up, bs, st);
    case 128: return launch_mx_bm<128>(p, up, bs, st);
    case 256: return launch_mx_bm<256>(p, up, bs, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace moe
