// One workgroup's bf16 output tile of C_m = A . B_m (m < NB) on gfx950, with
// both operands loaded straight from global memory into LDS.
//
// NW wave64s (8: two per SIMD, so one wave's MFMAs cover the other's LDS
// and barrier waits), tile BM rows x BN (= 128) columns per weight matrix,
// K stages of BK (32 or 64) elements in a ring of as many LDS stage slots as
// fit the budget.
//
//  - global -> LDS: buffer_load_dwordx4 with the lds bit (16 bytes per lane;
//    lane l's bytes land at the LDS base in M0 + 16 l). No staging registers,
//    no register transpose, no LDS store instructions.
//    Zero rows, rows past K and columns past N use out-of-range offsets: the
//    hardware writes zeros.
//  - A in LDS: BM rows of 2*BK bytes, 16-byte chunk c of row r stored in slot
//    c ^ key(r) (see aswz), the key chosen by measurement so the fragment
//    reads (ds_read_b128) are free of bank conflicts.
//  - B in LDS: each matrix as [BK k-rows][BN columns], N-contiguous as in
//    memory (256 bytes per row); its 32-byte column pairs are XOR-swizzled by
//    g(k) = (k & 3) | ((k >> 3) & 1) << 2 so the 16 k-rows one transposed read
//    touches fall in 8 different pair slots.
//  - A operand: one ds_read_b128 per 16x32 block (lane l: row l % 16, K
//    elements 8 (l / 16) .. +7).
//  - B operand: two ds_read_b64_tr_b16 per 32x16 block. Within each 16-lane
//    group, lane i receives element i % 4 of the 8-byte chunks addressed by
//    lanes i/4, i/4 + 4, i/4 + 8, i/4 + 12 of its group. With lane i of group
//    g addressing k-row k0 + 8g + i/4 and columns n0 + 4 (i % 4) .. +3, lane i
//    receives column n0 + i at k-rows k0 + 8g .. +3: the MFMA B operand layout
//    (column l % 16, K elements 8 (l / 16) .. +7) after the second read at
//    k-rows + 4.
//  - v_mfma_f32_16x16x32_bf16, fp32 accumulators (lane l: column l % 16, rows
//    4 (l / 16) .. +3 of each 16x16 block).
//  - Pipeline: NSTAGE-1 stages in flight; each wave waits (vmcnt) only for
//    its own stage-kt loads, then one barrier per stage.
#pragma once

#include <type_traits>

#include "gemm_tile.h"

namespace moe {

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// Schedule knobs (compile time, chosen by measurement):
//  MOE_PINGPONG   1: the two waves of each SIMD alternate between reading
//                 fragments and running MFMAs (kloop_pp).
//  MOE_MFMA_PRIO  1: raise the wave's issue priority around its MFMA block.
#ifndef MOE_PINGPONG
#define MOE_PINGPONG 0
#endif
//  MOE_A_DIST     A fragment reads in flight ahead of their MFMAs.
#ifndef MOE_A_DIST
#define MOE_A_DIST 3
#endif
#ifndef MOE_MFMA_PRIO
#define MOE_MFMA_PRIO 0
#endif
//  MOE_MFMA32     1: the persistent GEMMs' cores (tiles of 128 rows or more
//                 and their half tiles) use v_mfma_f32_32x32x16_bf16.
#ifndef MOE_MFMA32
#define MOE_MFMA32 0
#endif

// Raw buffer descriptor (gfx9): base[47:0], stride 0, num_records = bytes,
// dword3 0x00020000. Built from wave-uniform values so it lives in SGPRs.
__device__ __forceinline__ i32x4_t make_srd(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4_t r;
  r.x = (int)(uint32_t)a;
  r.y = (int)((a >> 32) & 0xFFFFu);
  r.z = (int)bytes;
  r.w = 0x00020000;
  return r;
}

// 16 bytes per lane from buffer `srd` at byte offset voff into LDS at
// lds_dst + 16 * lane (lds_dst wave-uniform, set through M0). Written as a
// one-instruction asm block so that the compiler does not add a wait for it in
// front of later LDS reads of other stage buffers: the K loop orders these
// loads itself (vmcnt wait on the issuing wave, then a workgroup barrier).
// The instruction has no register result. NT = true sets the non-temporal
// hint (data read once: do not keep it in the caches at the expense of data
// that is reused).
//
// The compiler does not look inside the asm, so it does not insert the wait
// states a vector memory instruction needs after a VALU op wrote one of its
// SGPRs (5 on gfx9: v_readlane / v_readfirstlane results, or SGPRs restored
// from VGPR lanes under SGPR pressure). SGPR_FROM_VALU = true puts them in the
// asm (s_nop 4); the default form relies on the descriptor being built by
// scalar code, which a test checks on the compiled kernels.
template <bool SGPR_FROM_VALU = false, bool NT = false>
__device__ __forceinline__ void dma16(i32x4_t srd, uint32_t voff, const void* lds_dst) {
  const uint32_t m0v = (uint32_t)reinterpret_cast<uintptr_t>(
      (const __attribute__((address_space(3))) char*)lds_dst);
  if constexpr (SGPR_FROM_VALU && NT)
    asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen nt lds" ::"v"(voff), "s"(srd),
                 "{m0}"(m0v)
                 : "memory");
  else if constexpr (SGPR_FROM_VALU)
    asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(srd),
                 "{m0}"(m0v)
                 : "memory");
  else if constexpr (NT)
    asm volatile("buffer_load_dwordx4 %0, %1, 0 offen nt lds" ::"v"(voff), "s"(srd), "{m0}"(m0v)
                 : "memory");
  else
    asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(srd), "{m0}"(m0v)
                 : "memory");
}

// 4 bytes per lane from buffer `srd` at byte offset voff into LDS at
// lds_dst + 4 * lane (same form as dma16, with the wait states).
__device__ __forceinline__ void dma4(i32x4_t srd, uint32_t voff, const void* lds_dst) {
  const uint32_t m0v = (uint32_t)reinterpret_cast<uintptr_t>(
      (const __attribute__((address_space(3))) char*)lds_dst);
  asm volatile("s_nop 4\n\tbuffer_load_dword %0, %1, 0 offen lds" ::"v"(voff), "s"(srd),
               "{m0}"(m0v)
               : "memory");
}

// s_waitcnt with vmcnt <= n, expcnt and lgkmcnt unconstrained (gfx9 encoding:
// vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt[5:4] in bits [15:14]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// B_STREAM: the B operand (the weights) is read once per call, no other task
// reuses it from the caches; its loads carry the non-temporal hint.
// VALU_SGPR: every LDS-direct load takes the wait-state form of dma16 (for
// kernels whose SGPR pressure makes the compiler restore the buffer
// descriptors from VGPR lanes next to the loads; the asm hazard test finds
// the sites).
// MF: the MFMA shape, 16 (v_mfma_f32_16x16x32_bf16) or 32
// (v_mfma_f32_32x32x16_bf16). With 32, a row block is 32 rows, a column
// block 32 columns, and a K step 16 elements:
//  - A operand: lane l holds row l % 32, K elements 8 (l / 32) .. +7 of the
//    step (one ds_read_b128);
//  - B operand: lane l holds column l % 32, the same K elements (two
//    ds_read_b64_tr_b16: 16-lane group g addresses k-rows 8 (g / 2) + i / 4
//    (+4 for the second read) and columns 16 (g % 2) + 4 (i % 4) .. +3);
//  - accumulators: lane l, register r holds row 8 (r / 4) + 4 (l / 32) +
//    r % 4, column l % 32;
//  - B's column pairs are swizzled by ((k & 3) << 1) | ((k >> 3) & 1), so that
//    the two column halves a read's 32 lanes address at the same k-rows, and
//    the k-rows 8 apart, fall in different 32-byte slots.
// A64: A is loaded in 64-K stages of its own (128 bytes, a whole cache line,
// of each gathered row per load) while B keeps 32-K stages (BK = 32). LDS slot
// s holds A stage s and B stage s side by side; B stage kt sits in slot
// kt % NSTAGE and A stage kt / 2 in slot (kt / 2) % NSTAGE. Each 32-K step
// issues B stage kt + NSTAGE - 1 and one half of the loads of A stage
// kt / 2 + NSTAGE - 1, so every step issues the same number of loads and one
// vmcnt bound covers both rings.
// Each 32-column step of K adds its products in the same order for any BM, so
// a half tile reproduces the whole tile's sums bit for bit (for the same MF).
template <int BM_, int NB_, int NW_ = 8, int BK_ = 64, int LDS_BUDGET = 144 * 1024,
          bool B_STREAM = false, bool VALU_SGPR = false, int MF = 16, bool A64 = false>
struct TileGemmDirect {
  static constexpr bool DIRECT = true;  // the LDS-direct core (vs gemm_tile.h)
  static constexpr int BM = BM_, BN = 128, NB = NB_;
  static constexpr int NW = NW_;              // waves per workgroup (2 per SIMD at 8)
  static constexpr int THREADS = 64 * NW;
  static constexpr int ES = 2;
  static constexpr int BK = BK_;              // 32 or 64 K elements per stage
  static constexpr int A_BK = A64 ? 64 : BK;  // K elements per A stage
  static constexpr int ACH = A_BK / 8;        // 16-byte chunks per A row
  static constexpr int A_ROWB = A_BK * ES;
  static constexpr int B_ROWB = BN * ES;      // 256
  static constexpr int A_LDS = BM * A_ROWB;
  static constexpr int B_MAT = BK * B_ROWB;   // per matrix per stage
  static constexpr int B_LDS = NB * B_MAT;
  static constexpr int STAGE = A_LDS + B_LDS;
  // as many stages as fit the budget (one LDS array, stage kt in slot kt % NSTAGE)
  static constexpr int NSTAGE = LDS_BUDGET / STAGE > 8 ? 8 : LDS_BUDGET / STAGE;
  static constexpr int LDS_BYTES = NSTAGE * STAGE;
  static_assert(NSTAGE >= 2, "at least two LDS stages");
  static_assert(BK == 32 || BK == 64, "stage K");
  static_assert(MF == 16 || MF == 32, "MFMA shape");
  static constexpr int WM = BM >= 32 ? 2 : 1;
  static constexpr int WN = NW / WM;
  static constexpr int MI = BM / WM / MF;     // row blocks per wave
  static constexpr int NI = BN / WN / MF;     // column blocks per wave and matrix
  static constexpr int KS = 512 / MF;         // K elements per MFMA step (32 or 16)
  static constexpr int KSTEPS = BK / KS;
  static constexpr int ADIST = MOE_A_DIST;
  // 1 KB (one wave instruction) units per stage
  static constexpr int A_INSTR = A_LDS / 1024;
  static constexpr int B_INSTR = B_LDS / 1024;
  static constexpr int A_PW = (A_INSTR + NW - 1) / NW;   // per wave (upper bound)
  static constexpr int B_PW = B_INSTR / NW;
  static constexpr int A_HPW = A_PW / 2;  // A64: A loads per wave and 32-K step
  // loads every wave issues per stage (waves with fewer A units wait for less)
  static constexpr int MIN_PW = A64 ? A_HPW + B_PW : A_INSTR / NW + B_PW;
  static_assert((NSTAGE - 2) * (A_PW + B_PW) < 64, "vmcnt range");
  static_assert(!A64 || (BK == 32 && A_INSTR % NW == 0 && A_PW % 2 == 0),
                "A64: 32-K B stages, A loads split evenly over waves and steps");
  static_assert(B_INSTR % NW == 0, "B loads split evenly over the waves");
  static_assert(MI >= 1 && NI >= 1, "tile too small for the waves");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");

  using acc_t = std::conditional_t<MF == 32, f32x16_t, f32x4_t>;
  static constexpr int ACC_N = MF == 32 ? 16 : 4;
  acc_t acc[NB][MI][NI];
  uint32_t aoff[A_PW];   // per-lane A row byte offset + logical chunk (kOob = zero)
  uint32_t boff[B_PW];   // per-lane B offset at k-stage 0 (kOob = zero column strip)
  i32x4_t rsrc_a;
  i32x4_t rsrc_b[NB];
  uint32_t b_stage_bytes;  // BK * ldb * ES
  uint32_t a_stage_bytes;  // A bytes from one K stage to the next (see setup)
  int64_t K_;

  __device__ __forceinline__ static int bswz(int k) {
    if constexpr (MF == 32)
      return ((k & 3) << 1) | ((k >> 3) & 1);
    else
      return (k & 3) | (((k >> 3) & 1) << 2);
  }
  // A chunk swizzle (8 chunks per 128-byte row, or 4 per 64-byte row). Chosen
  // by measurement, with an LDS probe of exactly the fragment-read pattern on
  // 256 workgroups: these keys sustain 234 B/clk per CU; the keys that spread
  // one read's 16 rows over 16 different 16-byte bank windows ((r & 7) ^
  // ((r >> 3) & 1) and (r >> 2) & 3) ran at 128 B/clk, half of the LDS
  // cycles stalled on bank conflicts (the hardware does not serve a read's
  // 64 lanes as four groups of 16 consecutive lanes).
  __device__ __forceinline__ static int aswz(int r) {
    if constexpr (ACH == 8)
      return (r >> 1) & 7;
    else if constexpr (MF == 32)
      return ((r >> 2) & 1) | (((r >> 3) & 1) << 1);
    else
      return ((r >> 2) & 1) << 1;
  }

  __device__ __forceinline__ void zero_acc() {
#pragma unroll
    for (int m = 0; m < NB; ++m)
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j) acc[m][i][j] = acc_t{};
  }

  // A: buffer of a_bytes at a_base, row_off(r) = byte offset of row r or kOob.
  // a_slab_rows = 0: rows K-contiguous (element k of row r at row_off(r) +
  // 2k). a_slab_rows = R > 0: a block of R rows stored as slabs of 32
  // columns, slab by slab (element k of block row r at (k / 32) * R * 64 +
  // r * 64 + 2 (k % 32); the caller's row_off(r) is then the row's r * 64),
  // so each stage of A is one contiguous block. R is the tile's BM, or
  // larger when the tile covers part of a block's rows.
  // B[m]: base of weight matrix m (K x ldb, row-major) with b_bytes[m] bytes;
  // the tile covers its columns n0 .. n0 + BN, of which ncols[m] are valid.
  template <typename RowOff>
  __device__ __forceinline__ void setup(const void* a_base, uint32_t a_bytes, RowOff row_off,
                                        const char* const* B, const uint32_t* b_bytes,
                                        int64_t ldb, int64_t n0, const int64_t* ncols,
                                        int a_slab_rows = 0) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    rsrc_a = make_srd(a_base, a_bytes);
#pragma unroll
    for (int m = 0; m < NB; ++m) rsrc_b[m] = make_srd(B[m], b_bytes[m]);
    a_stage_bytes =
        a_slab_rows ? (uint32_t)(A_BK / 32 * a_slab_rows * 64) : (uint32_t)(A_BK * ES);
    b_stage_bytes = (uint32_t)(BK * ldb * ES);
#pragma unroll
    for (int t = 0; t < A_PW; ++t) {
      const int q = wave + NW * t;  // A instruction index: 1 KB of consecutive rows
      uint32_t o = kOob;
      if (q < A_INSTR) {
        const int r = q * (1024 / A_ROWB) + lane / ACH;
        const int c = (lane % ACH) ^ aswz(r);  // logical chunk stored in this lane's slot
        const uint32_t ro = row_off(r);
        if (ro != kOob)
          o = a_slab_rows ? ro + (c >> 2) * (a_slab_rows * 64) + (c & 3) * 16 : ro + c * 16;
      }
      aoff[t] = o;
    }
#pragma unroll
    for (int t = 0; t < B_PW; ++t) {
      const int q = wave + NW * t;                // B instruction index
      const int kr = (q % (B_MAT / 1024)) * 4 + (lane >> 4);  // k-row in the stage
      const int pc = lane & 15;                   // physical 16-byte chunk in the row
      const int c = (((pc >> 1) ^ bswz(kr)) << 1) | (pc & 1);  // logical chunk
      const bool ok = (int64_t)c * 8 + 8 <= ncols[q / (B_MAT / 1024)];
      boff[t] = ok ? (uint32_t)(((int64_t)kr * ldb + n0 + c * 8) * ES) : kOob;
    }
  }

  // LDS-direct load number idx (0 <= idx < NPIECE: this wave's A loads, then
  // its B loads) of K stage kt into the stage buffer `base`.
  // SGPR_FROM_VALU: the caller cannot rule out that the compiler restores the
  // buffer descriptors from VGPR lanes right before (see dma16).
  static constexpr int NPIECE = A64 ? A_HPW + B_PW : A_PW + B_PW;  // loads per wave and step
  // This wave's A load t (0 <= t < A_PW) of A stage ka into the A buffer abuf;
  // t = t0, or t0 + A_HPW if hi (t0 a compile-time index after unrolling,
  // so that aoff stays in registers).
  template <bool SGPR_FROM_VALU = VALU_SGPR>
  __device__ __forceinline__ void issue_a(char* abuf, int ka, int t0, bool hi = false) {
    // wave-uniform (scalar) so the buffer resources stay in SGPRs
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int t = t0;
    uint32_t ao = aoff[t0];
    if constexpr (A64) {
      // select between the two values, not their addresses (a select of
      // addresses would index aoff at run time and move it to memory)
      uint32_t ao_hi = aoff[t0 + A_HPW < A_PW ? t0 + A_HPW : 0];
      asm("" : "+v"(ao), "+v"(ao_hi));
      if (hi) {
        t = t0 + A_HPW;
        ao = ao_hi;
      }
    }
    const int q = wave + NW * t;
    if (q < A_INSTR) {  // wave-uniform
      const int64_t k0 = (int64_t)ka * A_BK;
      const int lane = threadIdx.x & 63;
      const int r = q * (1024 / A_ROWB) + lane / ACH;
      const int c = (lane % ACH) ^ aswz(r);
      const uint32_t o = (ao != kOob && k0 + c * 8 < K_) ? ao + (uint32_t)ka * a_stage_bytes : kOob;
      dma16<SGPR_FROM_VALU>(rsrc_a, o, abuf + q * 1024);
    }
  }
  // This wave's B load t (0 <= t < B_PW) of B stage kt into the B buffer bbuf.
  template <bool SGPR_FROM_VALU = VALU_SGPR>
  __device__ __forceinline__ void issue_b(char* bbuf, int kt, int t) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int q = wave + NW * t;
    const int m = q / (B_MAT / 1024);  // wave-uniform
    const uint32_t o = boff[t] == kOob ? kOob : boff[t] + (uint32_t)kt * b_stage_bytes;
    i32x4_t rb = rsrc_b[0];
    if constexpr (NB > 1) {
      if (m == 1) rb = rsrc_b[1];
    }
    dma16<SGPR_FROM_VALU, B_STREAM>(rb, o, bbuf + q * 1024);
  }
  template <bool SGPR_FROM_VALU = VALU_SGPR>
  __device__ __forceinline__ void issue_piece(char* base, int kt, int idx) {
    if (idx < A_PW)
      issue_a<SGPR_FROM_VALU>(base, kt, idx);
    else
      issue_b<SGPR_FROM_VALU>(base + A_LDS, kt, idx - A_PW);
  }
  // A64: load idx (0 <= idx < NPIECE) of 32-K step kt's share: half kt & 1 of
  // A stage kt / 2 + NSTAGE - 1 into anext, then B stage kt + NSTAGE - 1 into
  // bnext (both stage slots).
  __device__ __forceinline__ void issue_piece64(char* anext, char* bnext, int kt, int idx) {
    const int d = NSTAGE - 1;
    if (idx < A_HPW)
      issue_a(anext, (kt >> 1) + d, idx, kt & 1);
    else
      issue_b(bnext + A_LDS, kt + d, idx - A_HPW);
  }

  // All LDS-direct loads of K stage kt into the stage buffer `base`.
  template <bool SGPR_FROM_VALU = VALU_SGPR>
  __device__ __forceinline__ void issue_stage(char* base, int kt) {
#pragma unroll
    for (int i = 0; i < NPIECE; ++i) issue_piece<SGPR_FROM_VALU>(base, kt, i);
  }

  struct Frags {
    uint4 b[NB][NI];
  };
  Frags fb_[KSTEPS];  // the stage's B fragments, one set per 32-wide K step

  __device__ __forceinline__ void read_frags_b(const char* base, int ks, Frags& f) const {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wn0 = (wave % WN) * (BN / WN);
    const int lr = lane & 15;
    const int lg = lane >> 4;
#pragma unroll
    for (int m = 0; m < NB; ++m)
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        i16x4_t h[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int k = MF == 32 ? ks * 16 + 8 * (lg >> 1) + 4 * hh + (lr >> 2)
                                 : ks * 32 + 8 * lg + 4 * hh + (lr >> 2);
          const int n = MF == 32 ? wn0 + j * 32 + 16 * (lg & 1) + 4 * (lr & 3)
                                 : wn0 + j * 16 + 4 * (lr & 3);
          const int c = n >> 3;
          const int pc = ((((c >> 1) ^ bswz(k)) << 1) | (c & 1));
          const char* p = base + A_LDS + m * B_MAT + k * B_ROWB + (pc << 4) + ((n & 4) << 1);
          h[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4_t*)(p));
        }
        f.b[m][j] = __builtin_bit_cast(uint4, h);
      }
  }

  // A fragment of row block i at K step ks of the A stage at base, plus ak
  // chunks (A64: 4 for the second 32-K half of an A stage).
  __device__ __forceinline__ uint4 read_a(const char* base, int ks, int i, int ak = 0) const {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm0 = (wave / WN) * (BM / WM);
    const int r = MF == 32 ? wm0 + i * 32 + (lane & 31) : wm0 + i * 16 + (lane & 15);
    const int c = (MF == 32 ? ks * 2 + (lane >> 5) : ks * 4 + (lane >> 4)) + ak;
    return *reinterpret_cast<const uint4*>(base + r * A_ROWB + ((c ^ aswz(r)) << 4));
  }

  __device__ __forceinline__ void mfma_row(int i, const uint4& a, const uint4 (&b)[NB][NI]) {
#pragma unroll
    for (int m = 0; m < NB; ++m)
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        if constexpr (MF == 32)
          acc[m][i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b[m][j]),
              acc[m][i][j], 0, 0, 0);
        else
          acc[m][i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b[m][j]),
              acc[m][i][j], 0, 0, 0);
      }
  }

  // MFMAs of this wave's row blocks [LO, HI) over one stage, as straight-line
  // code whose instruction order is pinned with scheduling-group barriers
  // (the compiler's own schedule, at this register pressure, reads one A
  // fragment at a time and waits for it before its MFMAs). Each K step reads
  // its B fragments (READ_B; else they are in fb_ from an earlier call) and
  // the first ADIST A fragments, then alternates the MFMAs of block i with
  // the read of block i + ADIST: ADIST LDS reads stay in flight behind the
  // matrix work.
  // A64: the A fragments come from abase at chunk offset ak instead of base.
  template <int LO, int HI, bool READ_B, typename Between>
  __device__ __forceinline__ void compute_range(const char* base, Between between,
                                                const char* abase = nullptr, int ak = 0) {
    const char* ab = A64 ? abase : base;
    if constexpr (HI > LO) {
      constexpr int NBLK = HI - LO;
      constexpr int D = ADIST < NBLK ? ADIST : NBLK;
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        if constexpr (READ_B) read_frags_b(base, ks, fb_[ks]);
        uint4 a[NBLK];
#pragma unroll
        for (int i = 0; i < D; ++i) a[i] = read_a(ab, ks, LO + i, ak);
        __builtin_amdgcn_sched_group_barrier(0x100, (READ_B ? 2 * NB * NI : 0) + D, 0);
#pragma unroll
        for (int i = 0; i < NBLK; ++i) {
          if (i + D < NBLK) a[i + D] = read_a(ab, ks, LO + i + D, ak);
          mfma_row(LO + i, a[i], fb_[ks].b);
          __builtin_amdgcn_sched_group_barrier(0x008, NB * NI, 0);
          if (i + D < NBLK) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          between(ks * NBLK + i);
        }
      }
    }
  }
  template <int LO, int HI, bool READ_B>
  __device__ __forceinline__ void compute_range(const char* base) {
    compute_range<LO, HI, READ_B>(base, [](int) {});
  }

  // Row blocks [0, nact) of one stage (0 <= nact <= MI): blocks after the
  // wave's last real row hold only padding, contribute nothing and are
  // skipped (their accumulators stay zero).
  template <int NA = MI>
  __device__ __forceinline__ void compute_stage_n(const char* base, int nact) {
    if constexpr (NA > 0) {
      if (nact >= NA)
        compute_range<0, NA, true>(base);
      else
        compute_stage_n<NA - 1>(base, nact);
    }
  }

  // Number of this wave's row blocks (MF rows) up to the last row for which
  // valid(r) holds (r = tile row); blocks after it are padding only.
  template <typename Valid>
  __device__ __forceinline__ int active_blocks(Valid valid) const {
    constexpr int R = BM / WM;  // rows per wave
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm0 = (wave / WN) * R;
    int last = -1;
#pragma unroll
    for (int b = 0; b < R; b += 64) {
      const int r = b + lane;
      const uint64_t m = __ballot(r < R && valid(wm0 + r));
      if (m) last = b + 63 - __clzll(m);
    }
    return __builtin_amdgcn_readfirstlane((last + MF) / MF);
  }

  // K loop over a ring of NSTAGE stage slots in one LDS array for a wave
  // with NA active row blocks: NSTAGE-1 stages are in flight; stage
  // kt+NSTAGE-1 is issued right after the barrier that makes stage kt
  // visible (and ends every read of the slot it reuses). Stages past the end
  // of K are issued too (zeros, no memory traffic) so every step has the same
  // loads in flight.
  template <int NA>
  __device__ __forceinline__ void kloop(char* lds, int nk) {
    int slot = 0;                 // slot of stage kt
    int slot_next = NSTAGE - 1;   // slot of stage kt + NSTAGE - 1
    for (int kt = 0; kt < nk; ++kt) {
      wait_vmcnt<(NSTAGE - 2) * MIN_PW>();  // this wave's stage-kt loads have landed
      __syncthreads();                      // ... every wave's; stage kt-1 reads done
      // the stage kt+NSTAGE-1 loads go out one at a time between the row
      // blocks' MFMAs (all of them at once would hold the wave at the
      // memory issue while its MFMAs wait)
      char* nxt = lds + slot_next * STAGE;
      const int knx = kt + NSTAGE - 1;
      compute_range<0, NA, true>(lds + slot * STAGE, [&](int i) {
        if (i < NPIECE) issue_piece(nxt, knx, i);
      });
#pragma unroll
      for (int i = NA * KSTEPS; i < NPIECE; ++i) issue_piece(nxt, knx, i);
      slot = slot + 1 == NSTAGE ? 0 : slot + 1;
      slot_next = slot_next + 1 == NSTAGE ? 0 : slot_next + 1;
    }
  }

  // A64 K loop: 32-K step kt reads B stage kt (slot kt % NSTAGE) and half
  // kt & 1 of A stage kt / 2 (slot (kt / 2) % NSTAGE). At the top of step kt
  // every load issued up to step kt - NSTAGE + 1 must have landed: B stage kt
  // was issued in step kt - NSTAGE + 1 and the second half of A stage kt / 2
  // in step 2 (kt / 2) - 2 NSTAGE + 3 at the latest, both no later. A stage
  // kt / 2 + NSTAGE - 1 goes into the slot of A stage kt / 2 - 1, whose last
  // reader was step kt - 1 at the latest (done at this step's barrier), and B
  // stage kt + NSTAGE - 1 into the slot of B stage kt - 1.
  template <int NA>
  __device__ __forceinline__ void kloop64(char* lds, int nk) {
    int bslot = 0, bnext = NSTAGE - 1;
    int aslot = 0, anext = NSTAGE - 1;
    for (int kt = 0; kt < nk; ++kt) {
      wait_vmcnt<(NSTAGE - 2) * MIN_PW>();
      __syncthreads();
      char* an = lds + anext * STAGE;
      char* bn = lds + bnext * STAGE;
      compute_range<0, NA, true>(
          lds + bslot * STAGE, [&](int i) {
            if (i < NPIECE) issue_piece64(an, bn, kt, i);
          },
          lds + aslot * STAGE, (kt & 1) * (BK / 8));
#pragma unroll
      for (int i = NA * KSTEPS; i < NPIECE; ++i) issue_piece64(an, bn, kt, i);
      bslot = bslot + 1 == NSTAGE ? 0 : bslot + 1;
      bnext = bnext + 1 == NSTAGE ? 0 : bnext + 1;
      if (kt & 1) {
        aslot = aslot + 1 == NSTAGE ? 0 : aslot + 1;
        anext = anext + 1 == NSTAGE ? 0 : anext + 1;
      }
    }
  }

  // ---- ping-pong schedule (two waves per SIMD alternate roles)
  // Waves 0 .. NW/2-1 form group 0, waves NW/2 .. NW-1 group 1; waves are
  // placed on SIMDs round-robin, so each SIMD holds one wave of each group.
  // The K loop runs in phases separated by workgroup barriers. In each phase
  // one group runs the MFMAs of a whole stage from fragments already in its
  // registers while the other group reads the fragments of its next stage
  // from LDS and issues its share of a later stage's LDS-direct loads; the
  // groups swap roles every phase. On every SIMD one wave feeds the matrix
  // core while the other waits on LDS, instead of both doing the same thing
  // at the same time.
  //
  // Phase q (q = -1 .. 2nk-1; group 0 = G0, group 1 = G1):
  //   q = 2s:   G0 computes stage s; G1 reads stage s (and, for s >= 1,
  //             issues its part of stage s-1+NSTAGE);
  //   q = 2s+1: G0 reads stage s+1 and issues its part of stage s+NSTAGE;
  //             G1 computes stage s.
  // The prologue has stages 0 .. NSTAGE-1 in flight, one per slot.
  //  - stage X is read first by G0 in phase 2X-1; every wave waits for its
  //    own loads of stage X before the barrier that ends phase 2X-2, so the
  //    stage is complete and visible when either group reads it;
  //  - the slot of stage s is read by G0 in phase 2s-1 and by G1 in phase
  //    2s; its next stage (s+NSTAGE) is loaded from phase 2s+1 on;
  //  - every wave passes the same barriers (no barrier depends on the group).
  static constexpr bool PP_OK = MOE_PINGPONG && NW == 8 && MI >= 2 && NSTAGE >= 3 && !A64;
  uint4 fa_[PP_OK ? KSTEPS : 1][PP_OK ? MI : 1];  // A fragments of one stage

  template <int NA>
  __device__ __forceinline__ void pp_read(const char* base) {
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      if constexpr (NA > 0) read_frags_b(base, ks, fb_[ks]);
#pragma unroll
      for (int i = 0; i < NA; ++i) fa_[ks][i] = read_a(base, ks, i);
    }
  }

  template <int NA>
  __device__ __forceinline__ void pp_compute() {
#if MOE_MFMA_PRIO
    __builtin_amdgcn_s_setprio(1);
#endif
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks)
#pragma unroll
      for (int i = 0; i < NA; ++i) mfma_row(i, fa_[ks][i], fb_[ks].b);
#if MOE_MFMA_PRIO
    __builtin_amdgcn_s_setprio(0);
#endif
  }

  template <int NA>
  __device__ __forceinline__ void kloop_pp(char* lds, int nk) {
    const bool g1 = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) >= NW / 2;
    auto slot_of = [](int st) { return st % NSTAGE; };
    // a phase boundary: nothing is scheduled across it (the compiler would
    // otherwise move MFMAs over the barrier into the other phase)
    auto phase_end = [] {
      __builtin_amdgcn_sched_barrier(0);
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
    };
    // the prologue issued stages 0 .. NSTAGE-2; the last slot's stage here
    issue_stage(lds + (NSTAGE - 1) * STAGE, NSTAGE - 1);
    wait_vmcnt<(NSTAGE - 1) * MIN_PW>();  // this wave's stage-0 loads have landed
    __syncthreads();
    // one loop per group (each straight-line; the fragments have a single
    // writer and a single reader per iteration), with the same barriers
    if (!g1) {
      pp_read<NA>(lds);  // phase -1: read stage 0
      phase_end();
      for (int s = 0; s < nk; ++s) {
        pp_compute<NA>();                     // phase 2s
        wait_vmcnt<(NSTAGE - 2) * MIN_PW>();  // this wave's stage-(s+1) loads have landed
        phase_end();
        if (s + 1 < nk) pp_read<NA>(lds + slot_of(s + 1) * STAGE);  // phase 2s+1
        issue_stage(lds + slot_of(s) * STAGE, s + NSTAGE);
        phase_end();
      }
    } else {
      phase_end();  // phase -1
      for (int s = 0; s < nk; ++s) {
        pp_read<NA>(lds + slot_of(s) * STAGE);  // phase 2s
        if (s >= 1) issue_stage(lds + slot_of(s - 1) * STAGE, s - 1 + NSTAGE);
        wait_vmcnt<(NSTAGE - 2) * MIN_PW>();  // this wave's stage-(s+1) loads have landed
        phase_end();
        pp_compute<NA>();  // phase 2s+1
        phase_end();
      }
    }
    // G1's part of stage nk-1+NSTAGE was never issued and nothing waits for
    // it; the tail past K is zeros either way
  }

  // The K loop for this wave's number of active row blocks (one
  // instantiation per count, so that each is straight-line code).
  template <int NA = MI>
  __device__ __forceinline__ void kloop_n(char* lds, int nk, int nact) {
    if constexpr (NA == 0) {
      if constexpr (A64)
        kloop64<0>(lds, nk);
      else if constexpr (PP_OK)
        kloop_pp<0>(lds, nk);
      else
        kloop<0>(lds, nk);
    } else if (nact >= NA) {
      if constexpr (A64)
        kloop64<NA>(lds, nk);
      else if constexpr (PP_OK)
        kloop_pp<NA>(lds, nk);
      else
        kloop<NA>(lds, nk);
    } else {
      kloop_n<NA - 1>(lds, nk, nact);
    }
  }

  // K of the tile set up last (the streaming kernels set it per task).
  __device__ __forceinline__ void set_k(int64_t K) { K_ = K; }

  __device__ __forceinline__ void mainloop(char* lds, int64_t K, int nact = MI) {
    zero_acc();
    K_ = K;
    const int nk = (int)((K + BK - 1) / BK);
    if (nk <= 0) return;
    // No wait for this wave's earlier memory operations here: an earlier
    // tile's loads all landed before its mainloop returned, and what may
    // still be in flight are an epilogue's global stores. vmcnt retires in
    // issue order, so the first stage's wait below covers them, and their
    // latency overlaps the first stages' loads (measured: up/gate -1% at
    // prefill sizes).
    __syncthreads();  // every wave is done with the ring
    if constexpr (A64) {
      // the loads steps -2 (NSTAGE - 1) .. -1 would have issued, in order: A
      // stages 0 .. NSTAGE - 2 and B stages 0 .. NSTAGE - 2
#pragma unroll
      for (int v = -2 * (NSTAGE - 1); v < 0; ++v) {
        const int ka = (v >> 1) + NSTAGE - 1;  // arithmetic shift: floor(v / 2)
        const int kb = v + NSTAGE - 1;
        if (ka >= 0)
#pragma unroll
          for (int t = 0; t < A_HPW; ++t) issue_a(lds + ka * STAGE, ka, t, v & 1);
        if (kb >= 0)
#pragma unroll
          for (int t = 0; t < B_PW; ++t) issue_b(lds + kb * STAGE + A_LDS, kb, t);
      }
    } else {
#pragma unroll
      for (int s = 0; s + 1 < NSTAGE; ++s) issue_stage(lds + s * STAGE, s);
    }
    kloop_n(lds, nk, nact);
    wait_vmcnt<0>();
  }

  // f(matrix, tile row, tile column, value) for each accumulator element.
  template <typename F>
  __device__ __forceinline__ void for_each(F f) const {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    // this lane's first row and column, opaque to the optimiser: the row and
    // column indices are formed here rather than hoisted out of a caller's
    // task loop and held in registers through its K loop
    int lrow = (wave / WN) * (BM / WM) + (MF == 32 ? (lane >> 5) : (lane >> 4)) * 4;
    int lcol = (wave % WN) * (BN / WN) + (lane & (MF - 1));
    asm volatile("" : "+v"(lrow), "+v"(lcol));
#pragma unroll
    for (int m = 0; m < NB; ++m)
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        // one row block at a time (its row indices and addresses are not
        // all formed ahead and held in registers)
        if constexpr (MF == 32) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < NI; ++j)
#pragma unroll
          for (int r = 0; r < ACC_N; ++r)
            f(m, lrow + i * MF + acc_row(r), lcol + j * MF, acc[m][i][j][r]);
      }
  }

  // Row offset of accumulator register r within its block, relative to the
  // lane's first row.
  __device__ __forceinline__ static constexpr int acc_row(int r) {
    return MF == 32 ? 8 * (r >> 2) + (r & 3) : r;
  }

  // f(tile row, tile column, value of matrix 0, value of matrix 1) for each
  // element of a two-matrix tile, one row block at a time (the accumulator
  // reads of a block are not hoisted into VGPRs ahead of the others).
  template <typename F>
  __device__ __forceinline__ void for_each_pair(F f) const {
    static_assert(NB == 2, "two matrices");
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    int lrow = (wave / WN) * (BM / WM) + (MF == 32 ? (lane >> 5) : (lane >> 4)) * 4;
    int lcol = (wave % WN) * (BN / WN) + (lane & (MF - 1));
    asm volatile("" : "+v"(lrow), "+v"(lcol));
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < NI; ++j)
#pragma unroll
        for (int r = 0; r < ACC_N; ++r)
          f(lrow + i * MF + acc_row(r), lcol + j * MF, acc[0][i][j][r], acc[1][i][j][r]);
    }
  }
};

}  // namespace moe
