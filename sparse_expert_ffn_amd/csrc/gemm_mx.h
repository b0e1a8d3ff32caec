// One workgroup's tile of C_m = A . B_m (m < NB) with MXFP8 operands on gfx950
// (FP8 E4M3 elements, one E8M0 scale per 32 consecutive K values), on the
// scaled matrix instruction v_mfma_scale_f32_32x32x64_f8f6f4, fp32
// accumulation.
//
// Operands in memory are "stage-blocked": for a set of R rows (activation
// rows of an m-block, or the 128 output columns of a weight n-tile, each
// stored K-contiguous), one stage of 64 K values is R rows x 64 code bytes
// followed by R x 2 scale bytes (the row's two blocks of 32), R * 66 bytes
// in all; the stages follow one another. A stage of either operand is thus
// one contiguous stretch, loaded straight into LDS with 16-byte-per-lane
// LDS-direct loads (the last load of a stretch with only the lanes it needs).
//
//  - Lane layout of the instruction (found on the GPU with probes): A lane l
//    holds row l % 32 and, with h = l / 32, the K values 16 h .. 16 h + 15
//    (bytes 0-15) and 32 + 16 h .. 32 + 16 h + 15 (bytes 16-31): each half of
//    the wave holds a quarter of each 32-value block. The scale of lane
//    r + 32 h applies to row r's block h (K 32 h .. 32 h + 31), whichever
//    lanes hold its values. B lane l holds column l % 32 with the same K
//    values and its scale likewise; the 16 accumulators of lane l are rows
//    8 (r / 4) + 4 (l / 32) + r % 4 of column l % 32.
//  - LDS: each 64-byte row of codes keeps its four 16-byte chunks XOR-
//    swizzled by (row >> 2) & 3, so the 16-byte fragment reads of 16
//    consecutive rows cover all banks; scales stay linear.
//  - 8 wave64s: 2 row groups x 4 column groups; a wave computes BM/2 rows x
//    32 columns of each of the NB matrices (BM/64 row blocks of 32).
//  - Pipeline as the bf16 core (gemm_direct.h): NSTAGE-1 stages in flight,
//    each wave waits (vmcnt) for its own loads of a stage, one barrier per
//    stage.
#pragma once

#include "gemm_direct.h"

namespace moe {

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// Row blocks whose A fragments are read ahead of the MFMAs (all of the
// stage's by default: a row block has only NB MFMAs to cover a read).
#ifndef MOE_MX_ADIST
#define MOE_MX_ADIST 4
#endif

constexpr int kMxK = 64;          // K values per stage
constexpr int kMxRowBytes = 66;   // per row and stage: 64 codes + 2 scales

// Bytes of one stage-blocked stage of R rows.
__host__ __device__ constexpr int mx_stage_bytes(int R) { return R * kMxRowBytes; }

// 16 bytes per lane from `srd` at voff into LDS at lds_dst + 16 * lane, for
// the lanes below `active` only (the tail of a stretch).
template <bool SGPR_FROM_VALU, bool NT>
__device__ __forceinline__ void dma16_lanes(i32x4_t srd, uint32_t voff, const void* lds_dst,
                                            int active) {
  if ((int)(threadIdx.x & 63) < active) dma16<SGPR_FROM_VALU, NT>(srd, voff, lds_dst);
}

template <int BM_, int NB_, bool B_STREAM = false, bool VALU_SGPR = false>
struct TileGemmMx {
  static constexpr bool DIRECT = true;
  static constexpr int BM = BM_, BN = 128, NB = NB_;
  static constexpr int NW = 8;
  static constexpr int THREADS = 64 * NW;
  static constexpr int BK = kMxK;
  static_assert(BM == 64 || BM == 128 || BM == 256, "MXFP8 tiles of 64, 128 or 256 rows");
  static constexpr int WM = 2, WN = 4;
  static constexpr int MI = BM / WM / 32;             // 32-row blocks per wave
  static constexpr int A_BYTES = mx_stage_bytes(BM);  // one stage of A in memory
  static constexpr int B_BYTES = mx_stage_bytes(BN);  // one stage of one B matrix
  static constexpr int A_INSTR = (A_BYTES + 1023) / 1024;
  static constexpr int B_INSTR = (B_BYTES + 1023) / 1024;
  static constexpr int A_LDS = A_INSTR * 1024;
  static constexpr int B_LDS = B_INSTR * 1024;
  static constexpr int STAGE = A_LDS + NB * B_LDS;
  static constexpr int NSTAGE = (144 * 1024) / STAGE > 6 ? 6 : (144 * 1024) / STAGE;
  static constexpr int LDS_BYTES = NSTAGE * STAGE;
  static_assert(NSTAGE >= 2, "at least two LDS stages");
  static constexpr int N_INSTR = A_INSTR + NB * B_INSTR;  // load instructions per stage
  static constexpr int PW = (N_INSTR + NW - 1) / NW;       // per wave (upper bound)
  static constexpr int MIN_PW = N_INSTR / NW;              // every wave issues at least
  static_assert((NSTAGE - 2) * PW < 64, "vmcnt range");

  f32x16_t acc[NB][MI];
  uint32_t a_base;          // byte offset of the tile's stage 0 of A in rsrc_a
  uint32_t b_base[NB];      // byte offset of stage 0 of matrix m in rsrc_b[m]
  i32x4_t rsrc_a;
  i32x4_t rsrc_b[NB];
  int nk_;

  // chunk position of 16-byte chunk c of row r in LDS
  __device__ __forceinline__ static int cswz(int r) { return (r >> 2) & 3; }

  __device__ __forceinline__ void zero_acc() {
#pragma unroll
    for (int m = 0; m < NB; ++m)
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[m][i][r] = 0.f;
  }

  // A: stage-blocked rows of this tile, stage kt at a_off + kt * A_BYTES of a
  // buffer of a_bytes; B[m]: stage-blocked n-tile of matrix m, stage kt at
  // b_off[m] + kt * B_BYTES of a buffer of b_bytes[m].
  __device__ __forceinline__ void setup(const void* a_buf, uint32_t a_bytes, uint32_t a_off,
                                        const char* const* b_buf, const uint32_t* b_bytes,
                                        const uint32_t* b_off, int nk) {
    rsrc_a = make_srd(a_buf, a_bytes);
    a_base = a_off;
#pragma unroll
    for (int m = 0; m < NB; ++m) {
      rsrc_b[m] = make_srd(b_buf[m], b_bytes[m]);
      b_base[m] = b_off[m];
    }
    nk_ = nk;
  }

  // The global byte offset (within its stage) that lane `lane` of load
  // instruction q of an R-row stretch reads, so that the row's chunks land
  // swizzled: LDS byte q * 1024 + 16 lane holds, for codes, row
  // (q * 1024 + 16 lane) / 64, chunk position ((..) / 16) % 4.
  template <int R>
  __device__ __forceinline__ static uint32_t src_off(int q, int lane) {
    const int p = q * 1024 + lane * 16;
    if (p >= R * 64) return (uint32_t)p;  // scales: linear
    const int r = p >> 6;
    const int pos = (p >> 4) & 3;
    return (uint32_t)(r * 64 + ((pos ^ cswz(r)) << 4));
  }

  // Load instruction idx (0 <= idx < N_INSTR) of stage kt into stage buffer `base`.
  // Stages past the last (kt >= nk) load zeros with no memory traffic, so
  // every K step has the same loads in flight.
  template <bool SGPR_FROM_VALU = VALU_SGPR>
  __device__ __forceinline__ void issue_instr(char* base, int kt, int idx) {
    const int lane = threadIdx.x & 63;
    const bool past = kt >= nk_;
    if (idx < A_INSTR) {
      const int tail = A_BYTES - idx * 1024;
      const uint32_t o = past ? kOob : a_base + (uint32_t)kt * A_BYTES + src_off<BM>(idx, lane);
      if (tail >= 1024)
        dma16<SGPR_FROM_VALU, false>(rsrc_a, o, base + idx * 1024);
      else
        dma16_lanes<SGPR_FROM_VALU, false>(rsrc_a, o, base + idx * 1024, tail / 16);
    } else {
      const int j = idx - A_INSTR;
      const int m = j / B_INSTR;  // wave-uniform
      const int q = j - m * B_INSTR;
      const int tail = B_BYTES - q * 1024;
      const uint32_t o0 = (uint32_t)kt * B_BYTES + src_off<BN>(q, lane);
      i32x4_t rb = rsrc_b[0];
      uint32_t o = b_base[0] + o0;
      if constexpr (NB > 1) {
        if (m == 1) {
          rb = rsrc_b[1];
          o = b_base[1] + o0;
        }
      }
      if (past) o = kOob;
      char* dst = base + A_LDS + m * B_LDS + q * 1024;
      if (tail >= 1024)
        dma16<SGPR_FROM_VALU, B_STREAM>(rb, o, dst);
      else
        dma16_lanes<SGPR_FROM_VALU, B_STREAM>(rb, o, dst, tail / 16);
    }
  }

  // This wave's loads of stage kt (instructions wave, wave + NW, ...).
  template <bool SGPR_FROM_VALU = VALU_SGPR>
  __device__ __forceinline__ void issue_stage(char* base, int kt) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
    for (int t = 0; t < PW; ++t) {
      const int idx = wave + NW * t;
      if (idx < N_INSTR) issue_instr<SGPR_FROM_VALU>(base, kt, idx);
    }
  }

  // The MFMA operand of lane half h for row r of a codes region: the 16-byte
  // chunks h and 2 + h of the row's 64 K bytes (see the lane layout above).
  __device__ __forceinline__ static i32x8_t read_frag(const char* codes, int r, int h) {
    const int s = cswz(r);
    const uint4 lo = *reinterpret_cast<const uint4*>(codes + r * 64 + ((h ^ s) << 4));
    const uint4 hi = *reinterpret_cast<const uint4*>(codes + r * 64 + (((2 + h) ^ s) << 4));
    i32x8_t v;
    v[0] = (int)lo.x; v[1] = (int)lo.y; v[2] = (int)lo.z; v[3] = (int)lo.w;
    v[4] = (int)hi.x; v[5] = (int)hi.y; v[6] = (int)hi.z; v[7] = (int)hi.w;
    return v;
  }

  // MFMAs of one stage for this wave's row blocks [0, NA), software-
  // pipelined: the B fragments and the first MOE_MX_ADIST row blocks' A
  // fragments are read first, then the read of block i + MOE_MX_ADIST goes
  // out ahead of block i's MFMAs, so the matrix core works while later
  // fragments come back from LDS. between(i)
  // runs after block i's MFMAs (the next stage's loads go out one at a time
  // there). The instruction order is pinned with scheduling-group barriers.
  template <int NA, typename Between>
  __device__ __forceinline__ void compute_stage(const char* base, Between between) {
    if constexpr (NA > 0) {
      const int lane = threadIdx.x & 63;
      const int wave = threadIdx.x >> 6;
      const int h = lane >> 5;
      const int wm0 = (wave / WN) * (BM / WM);
      const int col = (wave % WN) * 32 + (lane & 31);
      i32x8_t b[NB];
      int sb[NB];
#pragma unroll
      for (int m = 0; m < NB; ++m) {
        const char* bm = base + A_LDS + m * B_LDS;
        b[m] = read_frag(bm, col, h);
        sb[m] = *reinterpret_cast<const unsigned char*>(bm + BN * 64 + col * 2 + h);
      }
      constexpr int D = MOE_MX_ADIST < NA ? MOE_MX_ADIST : NA;  // blocks read ahead
      i32x8_t a[NA];
      int sa[NA];
      auto read_a = [&](int i) {
        const int r = wm0 + i * 32 + (lane & 31);
        a[i] = read_frag(base, r, h);
        sa[i] = *reinterpret_cast<const unsigned char*>(base + BM * 64 + r * 2 + h);
      };
#pragma unroll
      for (int i = 0; i < D; ++i) read_a(i);
      __builtin_amdgcn_sched_group_barrier(0x100, 3 * NB + 3 * D, 0);
#pragma unroll
      for (int i = 0; i < NA; ++i) {
        if (i + D < NA) read_a(i + D);
#pragma unroll
        for (int m = 0; m < NB; ++m)
          acc[m][i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              a[i], b[m], acc[m][i], 0, 0, 0, sa[i], 0, sb[m]);
        if (i + D < NA) __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, NB, 0);
        between(i);
      }
    }
  }

  // Number of this wave's 32-row blocks up to its last row for which
  // valid(r) holds (r = tile row).
  template <typename Valid>
  __device__ __forceinline__ int active_blocks(Valid valid) const {
    constexpr int R = BM / WM;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm0 = (wave / WN) * R;
    int last = -1;
#pragma unroll
    for (int b = 0; b < R; b += 64) {
      const int r = b + lane;
      const uint64_t msk = __ballot(r < R && valid(wm0 + r));
      if (msk) last = b + 63 - __clzll(msk);
    }
    return __builtin_amdgcn_readfirstlane((last + 32) / 32);
  }

  // This wave's load t (0 <= t < PW) of stage kt into the stage buffer `base`.
  __device__ __forceinline__ void issue_one(char* base, int kt, int t) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int idx = wave + NW * t;
    if (idx < N_INSTR) issue_instr(base, kt, idx);
  }

  template <int NA>
  __device__ __forceinline__ void kloop(char* lds, int nk) {
    int slot = 0, slot_next = NSTAGE - 1;
    for (int kt = 0; kt < nk; ++kt) {
      wait_vmcnt<(NSTAGE - 2) * MIN_PW>();  // this wave's stage-kt loads have landed
      __syncthreads();                      // ... every wave's; stage kt-1 reads done
      char* nxt = lds + slot_next * STAGE;
      const int knx = kt + NSTAGE - 1;
      // the next stage's loads between the row blocks' MFMAs
      compute_stage<NA>(lds + slot * STAGE, [&](int i) {
        if (i < PW) issue_one(nxt, knx, i);
      });
#pragma unroll
      for (int t = NA; t < PW; ++t) issue_one(nxt, knx, t);
      slot = slot + 1 == NSTAGE ? 0 : slot + 1;
      slot_next = slot_next + 1 == NSTAGE ? 0 : slot_next + 1;
    }
  }

  template <int NA = MI>
  __device__ __forceinline__ void kloop_n(char* lds, int nk, int nact) {
    if constexpr (NA == 0) {
      kloop<0>(lds, nk);
    } else if (nact >= NA) {
      kloop<NA>(lds, nk);
    } else {
      kloop_n<NA - 1>(lds, nk, nact);
    }
  }

  __device__ __forceinline__ void mainloop(char* lds, int nact = MI) {
    zero_acc();
    const int nk = nk_;
    if (nk <= 0) return;
    __syncthreads();  // every wave is done with the ring
#pragma unroll
    for (int s = 0; s + 1 < NSTAGE; ++s) issue_stage(lds + s * STAGE, s);
    kloop_n(lds, nk, nact);
    wait_vmcnt<0>();
  }

  // f(matrix, tile row, tile column, value) for each accumulator element.
  template <typename F>
  __device__ __forceinline__ void for_each(F f) const {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    int lrow = (wave / WN) * (BM / WM) + 4 * (lane >> 5);
    int lcol = (wave % WN) * 32 + (lane & 31);
    asm volatile("" : "+v"(lrow), "+v"(lcol));
#pragma unroll
    for (int m = 0; m < NB; ++m)
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          f(m, lrow + i * 32 + 8 * (r >> 2) + (r & 3), lcol, acc[m][i][r]);
  }
};

}  // namespace moe
