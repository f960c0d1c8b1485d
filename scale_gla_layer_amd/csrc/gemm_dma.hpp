// MFMA GEMM core for gfx950 with asynchronous operand copies:
// C = A * B^T, both operands read along K ("NT"), fp32 accumulation.
//
// A workgroup of WGM x WGN waves computes a BM x BN tile; each wave owns a
// (16 WM) x (16 WN) sub-tile of v_mfma 16 x 16 tiles.  K advances in segments
// of KSEG bytes (64 or 128) per operand row; the problem class supplies, per
// row and segment, where that segment starts in memory (which makes gathers
// such as the causal hold free).  Every segment of both operands is copied
// global -> LDS with global_load_lds_dwordx4 (one instruction = 1 KB: 8 rows
// of 128 bytes or 16 rows of 64 bytes, no VGPRs) into one of NST rotating
// stages, NST-1 segments ahead of the MFMAs, with one LDS-only barrier per
// segment.  The copies of later segments stay in flight while earlier ones are
// multiplied: the vmcnt wait at segment kt allows exactly the copies of the
// segments issued after it.  Inside a stage, 16-byte piece p of row r is
// XOR-swizzled (KSEG 128: p ^ (r & 7); KSEG 64: p ^ ((r >> 2) & 3)) so that the
// fragment reads of 16 consecutive rows spread over all banks.
//
// Problem class interface (Cfg::a_row / b_row give the tile row a lane's copy
// slot j holds):
//   void setup(int wave, int lane)      precompute the lane's row sources
//   void started(char* lds)             after the first segments are in flight
//                                        (may fill LDS beyond Cfg::LDS)
//   void prep(int kt)                    once per copied segment, before a_row/b_row
//   const char* a_row(int j, int kt)    byte address of segment kt of slot j's row
//   const char* b_row(int j, int kt)    (valid memory even for rows outside the
//                                        problem: their results are discarded)
//   int  nk()                           number of K segments
//   bool seg_end(int kt)                true if segment kt closes a group of K
//                                        segments after which fold() is called
//   void fold(acc, wr, wc, lane)        consume and clear acc
//   void finish(acc, wr, wc, lane)      final accumulators into acc
//   void store(acc, wr, wc, lane, lds)  write the tile out (LDS may be reused)
#pragma once
#include <type_traits>

#include "async_copy.hpp"
#include "device_common.hpp"

// Optional timing hook: a build may define MSGLA_TILE_MARK(stage) to record
// when a tile starts (0), finishes its K loop (1) and finishes its store (2).
#ifndef MSGLA_TILE_MARK
#define MSGLA_TILE_MARK(stage) ((void)0)
#endif

namespace msgla {

template <int WM_, int WN_, int WGM_, int WGN_, int KSEG_, int NST_>
struct GemmCfg {
  static constexpr int WM = WM_, WN = WN_;      // 16 x 16 tiles per wave
  static constexpr int WGM = WGM_, WGN = WGN_;  // wave grid (row-major)
  static constexpr int NW = WGM * WGN, THREADS = 64 * NW;
  static constexpr int BM = 16 * WM * WGM, BN = 16 * WN * WGN;
  static constexpr int KSEG = KSEG_, NSL = KSEG_ / 64, NST = NST_;
  static constexpr int A_BYTES = BM * KSEG, B_BYTES = BN * KSEG, STAGE = A_BYTES + B_BYTES;
  static constexpr int LDS = NST * STAGE;
  static constexpr int RPI = 1024 / KSEG;       // rows per copy instruction
  static constexpr int A_SLOTS = BM / (RPI * NW), B_SLOTS = BN / (RPI * NW);
  static constexpr int COPIES = A_SLOTS + B_SLOTS;  // copy instructions per wave and segment
  static constexpr int LDC = BN + 4;            // fp32 staging row stride of gd_stage_tile
  static constexpr int LDS_STAGED = LDS > BM * LDC * 4 ? LDS : BM * LDC * 4;
  static_assert(KSEG == 64 || KSEG == 128, "segment");
  static_assert(NST >= 2 && NST <= 8, "stages");
  static_assert(A_SLOTS >= 1 && B_SLOTS >= 1 && A_SLOTS * RPI * NW == BM && B_SLOTS * RPI * NW == BN,
                "copy slots");
  static_assert((NST - 2) * COPIES < 64, "vmcnt range");

  // tile row held by copy slot j of a lane
  __device__ static int a_row(int j, int wave, int lane) { return RPI * (A_SLOTS * wave + j) + lane / (KSEG / 16); }
  __device__ static int b_row(int j, int wave, int lane) { return RPI * (B_SLOTS * wave + j) + lane / (KSEG / 16); }
  // LDS byte offset of 16-byte piece p of row r inside an operand block
  __device__ static int off(int r, int p) {
    if constexpr (KSEG == 128)
      return r * 128 + ((p ^ (r & 7)) << 4);
    else
      return r * 64 + ((p ^ ((r >> 2) & 3)) << 4);
  }
  // byte offset inside the row segment of the piece a lane copies (its LDS
  // slot is 16 * lane of the instruction; the swizzle is an involution)
  __device__ static int cp_piece(int lane) {
    if constexpr (KSEG == 128)
      return ((lane & 7) ^ (lane >> 3)) << 4;
    else
      return ((lane & 3) ^ ((lane >> 4) & 3)) << 4;
  }
};

// s_waitcnt vmcnt(n * COPIES) for a wave-uniform n in [0, MAXN]
template <int COPIES, int MAXN>
__device__ __forceinline__ void wait_stages(int n) {
  if constexpr (MAXN <= 0) {
    wait_vmcnt<0>();
  } else {
    if (n >= MAXN)
      wait_vmcnt<MAXN * COPIES>();
    else
      wait_stages<COPIES, MAXN - 1>(n);
  }
}

template <typename T, class Cfg, class Prob>
__device__ __forceinline__ void gemm_dma_tile(Prob& prob, int n_valid, char* lds) {
  constexpr int WM = Cfg::WM, WN = Cfg::WN, NST = Cfg::NST;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wave / Cfg::WGN, wc = wave % Cfg::WGN;
  const int lrow = lane & 15, lgrp = lane >> 4;
  const int nk = prob.nk();
  MSGLA_TILE_MARK(0);
  prob.setup(wave, lane);

  const int cpp = Cfg::cp_piece(lane);
  auto issue = [&](int kt) {
    char* st = lds + (kt % NST) * Cfg::STAGE;
    prob.prep(kt);
#pragma unroll
    for (int j = 0; j < Cfg::A_SLOTS; ++j)
      dma16(prob.a_row(j, kt) + cpp, st + 1024 * (Cfg::A_SLOTS * wave + j));
#pragma unroll
    for (int j = 0; j < Cfg::B_SLOTS; ++j)
      dma16(prob.b_row(j, kt) + cpp, st + Cfg::A_BYTES + 1024 * (Cfg::B_SLOTS * wave + j));
  };

  // fragment offsets inside a stage (the same for every segment): rows of a
  // 16-row tile differ by multiples of 16, which leave the swizzle key alone
  int offA[Cfg::NSL], offB[Cfg::NSL];
#pragma unroll
  for (int sl = 0; sl < Cfg::NSL; ++sl) {
    offA[sl] = Cfg::off(wr * 16 * WM + lrow, sl * 4 + lgrp);
    offB[sl] = Cfg::A_BYTES + Cfg::off(wc * 16 * WN + lrow, sl * 4 + lgrp);
  }

  f32x4 acc[WM][WN];
#pragma unroll
  for (int a = 0; a < WM; ++a)
#pragma unroll
    for (int b = 0; b < WN; ++b) acc[a][b] = zero4();

  int nb_valid = 0;
#pragma unroll
  for (int b = 0; b < WN; ++b) nb_valid += (wc * 16 * WN + 16 * b < n_valid) ? 1 : 0;

  for (int kt = 0; kt < NST - 1 && kt < nk; ++kt) issue(kt);
  prob.started(lds);

  // FULL: every 16-column tile of this wave is inside the problem, so the MFMA
  // block has no branches and its LDS reads can be scheduled freely
  auto kloop = [&](auto full) {
    for (int kt = 0; kt < nk; ++kt) {
      // segment kt has landed once only the copies of later segments remain
      wait_stages<Cfg::COPIES, NST - 2>(min(NST - 2, nk - 1 - kt));
      lds_barrier();
      if (kt + NST - 1 < nk) issue(kt + NST - 1);
      const char* st = lds + (kt % NST) * Cfg::STAGE;
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int sl = 0; sl < Cfg::NSL; ++sl) {
        u32x4 fa[WM], fb[WN];
#pragma unroll
        for (int a = 0; a < WM; ++a) fa[a] = ld16(st + offA[sl] + a * 16 * Cfg::KSEG);
#pragma unroll
        for (int b = 0; b < WN; ++b) fb[b] = ld16(st + offB[sl] + b * 16 * Cfg::KSEG);
#pragma unroll
        for (int b = 0; b < WN; ++b) {
          if (decltype(full)::value || b < nb_valid) {
#pragma unroll
            for (int a = 0; a < WM; ++a) acc[a][b] = mma_slab<T>(fa[a], fb[b], acc[a][b]);
          }
        }
      }
      __builtin_amdgcn_s_setprio(0);
      if (prob.seg_end(kt)) prob.fold(acc, wr, wc, lane);
    }
  };
  if (nb_valid == WN)
    kloop(std::integral_constant<bool, true>());
  else
    kloop(std::integral_constant<bool, false>());
  MSGLA_TILE_MARK(1);
  prob.finish(acc, wr, wc, lane);
  lds_barrier();  // all waves are done with the stages
  prob.store(acc, wr, wc, lane, lds);
  MSGLA_TILE_MARK(2);
}

// Whole-tile fp32 staging for epilogues that route values by row and column:
// C[r][c] at C + r * Cfg::LDC + c.  Call after gemm_dma_tile's final barrier
// (the stages are free), then lds_barrier() before reading other waves' values.
// The stores are volatile so that they stay single ds_write_b32: the ROCm 7.2
// compiler, pairing these stores into ds_write2_b32 around a re-based address
// (offsets beyond the 8-bit dword range), has emitted a wrong offset for one of
// the pair in this very pattern.
template <class Cfg>
__device__ __forceinline__ void gd_stage_tile(const f32x4 (&acc)[Cfg::WM][Cfg::WN], int wr, int wc,
                                              int lane, float* C) {
  const int lrow = lane & 15, lgrp = lane >> 4;
  typedef __attribute__((address_space(3))) volatile float lds_vfloat;
  lds_vfloat* base = (lds_vfloat*)(C + (wr * 16 * Cfg::WM + 4 * lgrp) * Cfg::LDC + wc * 16 * Cfg::WN + lrow);
#pragma unroll
  for (int a = 0; a < Cfg::WM; ++a)
#pragma unroll
    for (int b = 0; b < Cfg::WN; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) base[(16 * a + i) * Cfg::LDC + 16 * b] = acc[a][b][i];
}

}  // namespace msgla
