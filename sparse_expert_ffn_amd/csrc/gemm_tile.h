// One workgroup's output tile of C_m = A . B_m (m < NB) on gfx950 MFMA.
//
// 256 threads (4 wave64s). A rows are gathered through per-row pointers
// (a null pointer is a zero row) and are K-contiguous; each B_m is K x N,
// N-contiguous (row-major), with leading dimension ldb. NB weight matrices
// share the A tile (the up and gate projections of one expert).
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
//  - Two LDS stages: the next stage's global loads are in flight while the
//    current stage is multiplied (one barrier per stage).
// The accumulator of a 16x16 block: lane l holds column l % 16 and rows
// 4*(l/16) .. 4*(l/16)+3.
#pragma once

#include "moe_common.h"

namespace moe {

template <typename T, int BM_, int BN_, int NB_>
struct TileGemm {
  static constexpr int BM = BM_, BN = BN_, NB = NB_;
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

  struct Unit {
    uint4 v[UV];
  };

  f32x4_t acc[NB][MI][NI];
  Unit areg[A_PT];
  Unit breg[B_PT][8];
  const char* aptr[A_PT];
  const char* bptr[B_PT];
  bool bvec[B_PT];

  __device__ __forceinline__ void zero_acc() {
#pragma unroll
    for (int m = 0; m < NB; ++m)
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j) acc[m][i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  // rowptr(r): byte pointer to row r of A (K-contiguous), or null for a zero row.
  // B[m]: byte pointer to B_m at column n0. ldb, N in elements; ncols = N - n0.
  template <typename RowPtr>
  __device__ __forceinline__ void setup(RowPtr rowptr, const char* const* B, int64_t ldb,
                                        int64_t ncols) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < A_PT; ++i) {
      const int c = tid + i * 256;
      aptr[i] = (c < A_UNITS) ? rowptr(c / KB) : nullptr;
    }
#pragma unroll
    for (int i = 0; i < B_PT; ++i) {
      const int c = tid + i * 256;
      const int nb = (c / KB) % NBLK;
      const int m = c / (KB * NBLK);
      bptr[i] = nullptr;
      bvec[i] = false;
      if (c < B_BLOCKS && (int64_t)nb * 8 < ncols) {
        bptr[i] = B[m] + (size_t)nb * 8 * ES;
        bvec[i] = ((int64_t)nb * 8 + 8 <= ncols) && ((ldb % 8) == 0) &&
                  ((((uintptr_t)bptr[i]) & 15) == 0);
      }
    }
  }

  __device__ __forceinline__ static void load_unit(Unit& u, const char* p) {
#pragma unroll
    for (int q = 0; q < UV; ++q) u.v[q] = *reinterpret_cast<const uint4*>(p + q * 16);
  }

  __device__ __forceinline__ static void zero_unit(Unit& u) {
#pragma unroll
    for (int q = 0; q < UV; ++q) u.v[q] = make_uint4(0, 0, 0, 0);
  }

  __device__ __forceinline__ void load_stage(int kt, int64_t K, int64_t ldb, int64_t ncols) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < A_PT; ++i) {
      const int c = tid + i * 256;
      const int64_t k = (int64_t)kt * BK + (c % KB) * 8;
      if (aptr[i] != nullptr && k < K)
        load_unit(areg[i], aptr[i] + (size_t)k * ES);
      else
        zero_unit(areg[i]);
    }
#pragma unroll
    for (int i = 0; i < B_PT; ++i) {
      const int c = tid + i * 256;
      const int64_t k0 = (int64_t)kt * BK + (c % KB) * 8;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int64_t k = k0 + r;
        if (bptr[i] == nullptr || k >= K) {
          zero_unit(breg[i][r]);
        } else if (bvec[i]) {
          load_unit(breg[i][r], bptr[i] + (size_t)k * ldb * ES);
        } else {
          // ragged column strip or unaligned rows: element by element
          const int nb = (c / KB) % NBLK;
          const int64_t left = ncols - (int64_t)nb * 8;
          const T* src = reinterpret_cast<const T*>(bptr[i] + (size_t)k * ldb * ES);
          T tmp[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) tmp[e] = (e < left) ? src[e] : T(0);
          __builtin_memcpy(&breg[i][r], tmp, sizeof(tmp));
        }
      }
    }
  }

  // Transpose an 8 (K) x 8 (N) block held as 8 K-rows into 8 N-columns.
  __device__ __forceinline__ static void transpose8(const Unit (&in)[8], Unit (&out)[8]) {
    if constexpr (ES == 2) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        uint32_t w[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t lo = reinterpret_cast<const uint32_t*>(&in[2 * q].v[0])[j / 2];
          const uint32_t hi = reinterpret_cast<const uint32_t*>(&in[2 * q + 1].v[0])[j / 2];
          w[q] = (j & 1) ? ((lo >> 16) | (hi & 0xFFFF0000u)) : ((lo & 0xFFFFu) | (hi << 16));
        }
        out[j].v[0] = make_uint4(w[0], w[1], w[2], w[3]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        uint32_t w[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) w[r] = reinterpret_cast<const uint32_t*>(&in[r].v[0])[j];
        out[j].v[0] = make_uint4(w[0], w[1], w[2], w[3]);
        out[j].v[1] = make_uint4(w[4], w[5], w[6], w[7]);
      }
    }
  }

  __device__ __forceinline__ void store_stage(char* lds, int s) {
    const int tid = threadIdx.x;
    char* base = lds + s * STAGE;
#pragma unroll
    for (int i = 0; i < A_PT; ++i) {
      const int c = tid + i * 256;
      if (c < A_UNITS) {
        char* dst = base + (c / KB) * ROWB + (c % KB) * UB;
#pragma unroll
        for (int q = 0; q < UV; ++q) *reinterpret_cast<uint4*>(dst + q * 16) = areg[i].v[q];
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
        transpose8(breg[i], t);
        char* dst = base + A_LDS + (m * BN + nb * 8) * ROWB + kb * UB;
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
          for (int q = 0; q < UV; ++q)
            *reinterpret_cast<uint4*>(dst + j * ROWB + q * 16) = t[j].v[q];
      }
    }
  }

  __device__ __forceinline__ void compute_stage(const char* lds, int s) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm0 = (wave / WN) * (BM / WM);
    const int wn0 = (wave % WN) * (BN / WN);
    const char* base = lds + s * STAGE;
    const int lr = lane & 15;
    const int lk = (lane >> 4) * 8 * ES;  // byte offset of this lane's K group
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      Unit a[MI];
      Unit b[NB][NI];
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const char* p = base + (wm0 + i * 16 + lr) * ROWB + ks * 32 * ES + lk;
#pragma unroll
        for (int q = 0; q < UV; ++q) a[i].v[q] = *reinterpret_cast<const uint4*>(p + q * 16);
      }
#pragma unroll
      for (int m = 0; m < NB; ++m)
#pragma unroll
        for (int j = 0; j < NI; ++j) {
          const char* p = base + A_LDS + (m * BN + wn0 + j * 16 + lr) * ROWB + ks * 32 * ES + lk;
#pragma unroll
          for (int q = 0; q < UV; ++q) b[m][j].v[q] = *reinterpret_cast<const uint4*>(p + q * 16);
        }
#pragma unroll
      for (int m = 0; m < NB; ++m)
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int j = 0; j < NI; ++j) {
            if constexpr (ES == 2) {
              acc[m][i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  __builtin_bit_cast(bf16x8_t, a[i].v[0]), __builtin_bit_cast(bf16x8_t, b[m][j].v[0]),
                  acc[m][i][j], 0, 0, 0);
            } else {
              const float* af = reinterpret_cast<const float*>(&a[i].v[0]);
              const float* bf = reinterpret_cast<const float*>(&b[m][j].v[0]);
#pragma unroll
              for (int e = 0; e < 8; ++e)
                acc[m][i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[e], bf[e], acc[m][i][j], 0, 0, 0);
            }
          }
    }
  }

  // Full K loop for the current tile.
  __device__ __forceinline__ void mainloop(char* lds, int64_t K, int64_t ldb, int64_t ncols) {
    zero_acc();
    const int nk = (int)((K + BK - 1) / BK);
    if (nk <= 0) return;
    load_stage(0, K, ldb, ncols);
    store_stage(lds, 0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const bool more = kt + 1 < nk;
      if (more) load_stage(kt + 1, K, ldb, ncols);
      compute_stage(lds, kt & 1);
      if (more) store_stage(lds, (kt + 1) & 1);
      __syncthreads();
    }
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
#pragma unroll
          for (int r = 0; r < 4; ++r)
            f(m, wm0 + i * 16 + (lane >> 4) * 4 + r, wn0 + j * 16 + (lane & 15), acc[m][i][j][r]);
  }
};

}  // namespace moe
