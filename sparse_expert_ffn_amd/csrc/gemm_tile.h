// One workgroup's output tile of C_m = A . B_m (m < NB) on gfx950 MFMA.
//
// 256 threads (4 wave64s). A rows are gathered through per-row byte offsets
// into one buffer (an out-of-range offset is a zero row) and are
// K-contiguous; each B_m is K x N, N-contiguous (row-major), with leading
// dimension ldb. NB weight matrices share the A tile (the up and gate
// projections of one expert). All global loads are raw buffer loads: rows
// past K, columns past N and zero rows get an offset past the buffer's end,
// which the hardware turns into zeros, so the K loop has no branches.
//
// Data path per K stage (128 bytes of K per row: 64 bf16 or 32 fp32):
//  - global -> registers: A as 8-element units (16 B bf16 / 32 B fp32) with 8
//    consecutive threads per row; B as 8 x 8 element blocks (8 consecutive K
//    rows of one 8-column strip), which each thread transposes in registers;
//  - registers -> LDS: A rows and B columns both stored K-contiguous with a
//    16-byte pad per row, so the MFMA operand reads (16 rows at one K
//    offset) and the transposed B writes (8 K-units of one row) are free of
//    bank conflicts;
//  - LDS -> MFMA: one 16-byte (bf16) or 32-byte (fp32) read per lane per
//    16x16 operand block; v_mfma_f32_16x16x32_bf16, or eight
//    v_mfma_f32_16x16x4_f32 for fp32. Lane l holds row (or column) l % 16
//    and K elements 8*(l/16) .. 8*(l/16)+7 of the 32-wide K step, the same
//    assignment for both operands, so each MFMA sums the right products.
//  - Two LDS stages, one barrier per stage; register staging as selected by
//    MOE_STAGING below.
// The accumulator of a 16x16 block: lane l holds column l % 16 and rows
// 4*(l/16) .. 4*(l/16)+3.
#pragma once

#include "moe_common.h"

namespace moe {

constexpr uint32_t kOob = 0xF0000000u;  // offset past every buffer: loads return 0

// K-loop structure (compile-time; chosen by measurement):
//  STAGING 1 (template argument): one register staging set; the next
//    stage's loads are issued before the current stage's MFMAs and stored to
//    LDS after them.
//  STAGING 2: two sets; loads run two stages ahead and the LDS stores of the
//    next stage sit between the two halves of the current stage's MFMAs
//    (pays off when a stage carries enough MFMA work per wave: the up/gate
//    tile with two weight matrices; the down tile does better with 1).
//  MOE_FRAG_ORDER 0: all A and B operand fragments of a 32-wide K step are
//    read first; 1: B fragments stay resident, A fragments are read one
//    16-row block at a time.
#ifndef MOE_FRAG_ORDER
#define MOE_FRAG_ORDER 0
#endif

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // gfx9 buffer resource: raw (stride 0), num_records = bytes, dword3 0x00020000
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

template <typename T, int BM_, int BN_, int NB_, bool RAGGED_B = false, int STAGING = 1>
struct TileGemm {
  static constexpr int BM = BM_, BN = BN_, NB = NB_;
  static constexpr bool DIRECT = false;  // register-staged core (vs gemm_direct.h)
  static constexpr int THREADS = 256;
  static constexpr int ES = sizeof(T);
  static constexpr int BK = 128 / ES;   // K elements per stage
  static constexpr int KB = BK / 8;     // 8-element units per row per stage
  static constexpr int UB = 8 * ES;     // bytes per unit
  static constexpr int UV = UB / 16;    // uint4 per unit
  static constexpr int ROWB = 128 + 16; // LDS bytes per row (16 B pad)
  static constexpr int WM = BM >= 32 ? 2 : 1;
  static constexpr int WN = 4 / WM;
  static constexpr int MI = BM / WM / 16;
  static constexpr int NI = BN / WN / 16;
  static constexpr int A_UNITS = BM * KB;
  static constexpr int A_PT = (A_UNITS + 255) / 256;
  static constexpr int NBLK = BN / 8;
  static constexpr int B_BLOCKS = NB * KB * NBLK;
  static constexpr int B_PT = (B_BLOCKS + 255) / 256;
  static constexpr int A_LDS = BM * ROWB;
  static constexpr int B_LDS = NB * BN * ROWB;
  static constexpr int STAGE = A_LDS + B_LDS;
  static constexpr int LDS_BYTES = 2 * STAGE;
  static constexpr int KSTEPS = BK / 32;
  static_assert(MI >= 1 && NI >= 1, "tile too small for four waves");
  static_assert(BM % (16 * WM) == 0 && BN % (16 * WN) == 0, "tile shape");

  static_assert(NB == 1 || (KB * NBLK) % 64 == 0, "each wave must load blocks of one B matrix");

  struct Unit {
    uint4 v[UV];
  };

  f32x4_t acc[NB][MI][NI];
  // staging registers (MOE_STAGING sets): a stage lives there from its
  // global loads until its LDS store
  Unit areg[STAGING][A_PT];
  Unit breg[STAGING][B_PT][8];
  // byte offsets of this thread's loads inside the A / B buffer resources;
  // kOob marks a zero row / column strip (the buffer load returns zeros)
  uint32_t aoff[A_PT];
  uint32_t boff[B_PT];
  int bcols[B_PT];  // valid columns of the strip (RAGGED_B only)
  __amdgpu_buffer_rsrc_t rsrc_a;
  __amdgpu_buffer_rsrc_t rsrc_b[NB];
  int64_t ldb_bytes;

  __device__ __forceinline__ void zero_acc() {
#pragma unroll
    for (int m = 0; m < NB; ++m)
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j) acc[m][i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  // A: buffer of a_bytes bytes at a_base; row_off(r) = byte offset of row r
  //    (K-contiguous) or kOob for a zero row.
  // B[m]: base of the K x ldb matrix m (row-major) with b_bytes[m] bytes;
  //    this tile covers columns n0 .. n0 + BN of it, ncols_m[m] valid.
  template <typename RowOff>
  __device__ __forceinline__ void setup(const void* a_base, uint32_t a_bytes, RowOff row_off,
                                        const char* const* B, const uint32_t* b_bytes,
                                        int64_t ldb, int64_t n0, const int64_t* ncols_m) {
    const int tid = threadIdx.x;
    rsrc_a = make_rsrc(a_base, a_bytes);
#pragma unroll
    for (int m = 0; m < NB; ++m) rsrc_b[m] = make_rsrc(B[m], b_bytes[m]);
    ldb_bytes = ldb * ES;
#pragma unroll
    for (int i = 0; i < A_PT; ++i) {
      const int c = tid + i * 256;
      uint32_t o = kOob;
      if (c < A_UNITS) {
        const uint32_t r = row_off(c / KB);
        if (r != kOob) o = r + (c % KB) * UB;
      }
      aoff[i] = o;
    }
#pragma unroll
    for (int i = 0; i < B_PT; ++i) {
      const int c = tid + i * 256;
      const int nb = (c / KB) % NBLK;
      const int kb = c % KB;
      const int64_t ncols = c < B_BLOCKS ? ncols_m[c / (KB * NBLK)] : 0;
      const bool ok = c < B_BLOCKS && (int64_t)nb * 8 + (RAGGED_B ? 1 : 8) <= ncols;
      boff[i] = ok ? (uint32_t)((n0 + nb * 8) * ES + (int64_t)kb * 8 * ldb_bytes) : kOob;
      bcols[i] = RAGGED_B ? (int)min<int64_t>(8, ncols - (int64_t)nb * 8) : 8;
    }
  }

  __device__ __forceinline__ static void load_unit(Unit& u, __amdgpu_buffer_rsrc_t r,
                                                   uint32_t off) {
#pragma unroll
    for (int q = 0; q < UV; ++q)
      u.v[q] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                             r, off + q * 16, 0, 0));
  }

  template <int P>
  __device__ __forceinline__ void load_stage(int kt, int64_t K) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < A_PT; ++i) {
      const int c = tid + i * 256;
      const int64_t k = (int64_t)kt * BK + (c % KB) * 8;
      const uint32_t o = (aoff[i] != kOob && k < K) ? aoff[i] + (uint32_t)(kt * BK * ES) : kOob;
      load_unit(areg[P][i], rsrc_a, o);
    }
    const int wm = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
    for (int i = 0; i < B_PT; ++i) {
      // all lanes of a wave load blocks of the same matrix (static_assert above):
      // pick its resource with a wave-uniform select
      const int m = (wm * 64 + i * 256) / (KB * NBLK);
      __amdgpu_buffer_rsrc_t rb = rsrc_b[0];
      if constexpr (NB > 1) {
        if (m == 1) rb = rsrc_b[1];
      }
      const uint32_t o = boff[i] == kOob ? kOob
                                         : boff[i] + (uint32_t)((int64_t)kt * BK * ldb_bytes);
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const uint32_t orow = o == kOob ? kOob : o + (uint32_t)(r * ldb_bytes);
        if constexpr (!RAGGED_B) {
          load_unit(breg[P][i][r], rb, orow);
        } else {
          // unaligned rows or a partial strip: element by element
          T tmp[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint32_t oe = (orow == kOob || e >= bcols[i]) ? kOob : orow + e * ES;
            if constexpr (ES == 2)
              tmp[e] = __builtin_amdgcn_raw_buffer_load_b16(rb, oe, 0, 0);
            else
              tmp[e] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rb, oe, 0, 0));
          }
          __builtin_memcpy(&breg[P][i][r], tmp, sizeof(tmp));
        }
      }
    }
  }

  __device__ __forceinline__ static uint32_t word(const uint4& v, int i) {
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
  }

  // Transpose an 8 (K) x 8 (N) block held as 8 K-rows into 8 N-columns.
  __device__ __forceinline__ static void transpose8(const Unit (&in)[8], Unit (&out)[8]) {
    if constexpr (ES == 2) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        uint32_t w[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t lo = word(in[2 * q].v[0], j / 2);
          const uint32_t hi = word(in[2 * q + 1].v[0], j / 2);
          w[q] = (j & 1) ? ((lo >> 16) | (hi & 0xFFFF0000u)) : ((lo & 0xFFFFu) | (hi << 16));
        }
        out[j].v[0] = make_uint4(w[0], w[1], w[2], w[3]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        uint32_t w[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) w[r] = word(in[r].v[j / 4], j % 4);
        out[j].v[0] = make_uint4(w[0], w[1], w[2], w[3]);
        out[j].v[1] = make_uint4(w[4], w[5], w[6], w[7]);
      }
    }
  }

  template <int P>
  __device__ __forceinline__ void store_stage(char* lds, int s) {
    const int tid = threadIdx.x;
    char* base = lds + s * STAGE;
#pragma unroll
    for (int i = 0; i < A_PT; ++i) {
      const int c = tid + i * 256;
      if (c < A_UNITS) {
        char* dst = base + (c / KB) * ROWB + (c % KB) * UB;
#pragma unroll
        for (int q = 0; q < UV; ++q) *reinterpret_cast<uint4*>(dst + q * 16) = areg[P][i].v[q];
      }
    }
#pragma unroll
    for (int i = 0; i < B_PT; ++i) {
      const int c = tid + i * 256;
      if (c < B_BLOCKS) {
        const int kb = c % KB;
        const int nb = (c / KB) % NBLK;
        const int m = c / (KB * NBLK);
        Unit t[8];
        transpose8(breg[P][i], t);
        char* dst = base + A_LDS + (m * BN + nb * 8) * ROWB + kb * UB;
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
          for (int q = 0; q < UV; ++q)
            *reinterpret_cast<uint4*>(dst + j * ROWB + q * 16) = t[j].v[q];
      }
    }
  }

  __device__ __forceinline__ void mfma(f32x4_t& c, const Unit& a, const Unit& b) {
    if constexpr (ES == 2) {
      c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a.v[0]),
                                                  __builtin_bit_cast(bf16x8_t, b.v[0]), c, 0, 0,
                                                  0);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(
            __builtin_bit_cast(float, word(a.v[e / 4], e % 4)),
            __builtin_bit_cast(float, word(b.v[e / 4], e % 4)), c, 0, 0, 0);
    }
  }

  // One LDS stage, K steps [ks_lo, ks_hi) of 32 elements each.
  __device__ __forceinline__ void compute_stage(const char* lds, int s, int ks_lo, int ks_hi) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm0 = (wave / WN) * (BM / WM);
    const int wn0 = (wave % WN) * (BN / WN);
    const char* base = lds + s * STAGE;
    const int lr = lane & 15;
    const int lk = (lane >> 4) * 8 * ES;  // byte offset of this lane's K group
#pragma unroll
    for (int ks = ks_lo; ks < ks_hi; ++ks) {
      Unit b[NB][NI];
#pragma unroll
      for (int m = 0; m < NB; ++m)
#pragma unroll
        for (int j = 0; j < NI; ++j) {
          const char* p = base + A_LDS + (m * BN + wn0 + j * 16 + lr) * ROWB + ks * 32 * ES + lk;
#pragma unroll
          for (int q = 0; q < UV; ++q) b[m][j].v[q] = *reinterpret_cast<const uint4*>(p + q * 16);
        }
#if MOE_FRAG_ORDER == 0
      Unit a[MI];
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const char* p = base + (wm0 + i * 16 + lr) * ROWB + ks * 32 * ES + lk;
#pragma unroll
        for (int q = 0; q < UV; ++q) a[i].v[q] = *reinterpret_cast<const uint4*>(p + q * 16);
      }
#pragma unroll
      for (int m = 0; m < NB; ++m)
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int j = 0; j < NI; ++j) mfma(acc[m][i][j], a[i], b[m][j]);
#else
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        Unit a;
        const char* p = base + (wm0 + i * 16 + lr) * ROWB + ks * 32 * ES + lk;
#pragma unroll
        for (int q = 0; q < UV; ++q) a.v[q] = *reinterpret_cast<const uint4*>(p + q * 16);
#pragma unroll
        for (int m = 0; m < NB; ++m)
#pragma unroll
          for (int j = 0; j < NI; ++j) mfma(acc[m][i][j], a, b[m][j]);
      }
#endif
    }
  }

  // ---- STAGING == 2
  // One K iteration on parity P (= kt % 2): LDS buffer P holds stage kt,
  // staging set 1-P holds stage kt+1 (loads issued one iteration ago). The
  // loads of stage kt+2 go into set P; stage kt+1 is written to LDS buffer
  // 1-P between the two halves of stage kt's MFMAs. Loads and stores are
  // issued unconditionally (stages past the end of K load zeros through
  // out-of-range offsets, without memory traffic), so the wait before the LDS
  // stores covers only the older set of loads.
  template <int P>
  __device__ __forceinline__ void iteration(char* lds, int kt, int64_t K) {
    load_stage<P>(kt + 2, K);
    constexpr int half = KSTEPS > 1 ? KSTEPS / 2 : 1;
    compute_stage(lds, P, 0, half);
    store_stage<1 - P>(lds, 1 - P);
    if (half < KSTEPS) compute_stage(lds, P, half, KSTEPS);
    __syncthreads();
  }

  __device__ __forceinline__ void mainloop2(char* lds, int64_t K) {
    zero_acc();
    const int nk = (int)((K + BK - 1) / BK);
    if (nk <= 0) return;
    load_stage<0>(0, K);
    load_stage<1>(1, K);
    store_stage<0>(lds, 0);
    __syncthreads();
    int kt = 0;
    for (; kt + 1 < nk; kt += 2) {
      iteration<0>(lds, kt, K);
      iteration<1>(lds, kt + 1, K);
    }
    if (kt < nk) iteration<0>(lds, kt, K);
  }

  // ---- STAGING == 1
  // Stage kt is multiplied from LDS buffer kt % 2 while the loads of stage
  // kt+1 are in flight; they are stored to the other buffer afterwards.
  __device__ __forceinline__ void mainloop1(char* lds, int64_t K) {
    zero_acc();
    const int nk = (int)((K + BK - 1) / BK);
    if (nk <= 0) return;
    load_stage<0>(0, K);
    store_stage<0>(lds, 0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const bool more = kt + 1 < nk;
      if (more) load_stage<0>(kt + 1, K);
      compute_stage(lds, kt & 1, 0, KSTEPS);
      if (more) store_stage<0>(lds, (kt + 1) & 1);
      __syncthreads();
    }
  }

  // Full K loop for the current tile.
  __device__ __forceinline__ void mainloop(char* lds, int64_t K) {
    if constexpr (STAGING == 2)
      mainloop2(lds, K);
    else
      mainloop1(lds, K);
  }

  // Visit every accumulator element: f(m, row, col, value), row < BM, col < BN.
  template <typename F>
  __device__ __forceinline__ void for_each(F f) const {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm0 = (wave / WN) * (BM / WM);
    const int wn0 = (wave % WN) * (BN / WN);
#pragma unroll
    for (int m = 0; m < NB; ++m)
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j)
          if (__builtin_amdgcn_sched_barrier(0), true)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            f(m, wm0 + i * 16 + (lane >> 4) * 4 + r, wn0 + j * 16 + (lane & 15), acc[m][i][j][r]);
  }

  // f(tile row, tile column, value of matrix 0, value of matrix 1) for each
  // element of a two-matrix tile, one 16-row block at a time.
  template <typename F>
  __device__ __forceinline__ void for_each_pair(F f) const {
    static_assert(NB == 2, "two matrices");
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    int lrow = (wave / WN) * (BM / WM) + (lane >> 4) * 4;
    int lcol = (wave % WN) * (BN / WN) + (lane & 15);
    asm volatile("" : "+v"(lrow), "+v"(lcol));
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < NI; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          f(lrow + i * 16 + r, lcol + j * 16, acc[0][i][j][r], acc[1][i][j][r]);
    }
  }
};

}  // namespace moe
