// MFMA GEMM core for gfx950 with asynchronous operand copies:
// C = A * B^T, both operands read along K ("NT"), fp32 accumulation.
//
// Four waves in a 2 x 2 grid; each wave owns a (16 WM) x (16 WN) sub-tile
// (WM x WN v_mfma 16 x 16 tiles), so the workgroup tile is BM x BN with
// BM = 32 WM, BN = 32 WN.  Every operand row is a 128-byte K segment of some
// global row; the problem class supplies, per row, where it starts (which
// makes gathers such as the causal hold free).  Each K segment of both
// operands is copied global -> LDS with global_load_lds_dwordx4 (one
// instruction = 8 rows x 128 bytes, without VGPRs) into one of NST rotating
// stages, NST-1 segments ahead of the MFMAs; one LDS-only barrier per segment.
// Inside a stage, 16-byte piece p of row r lives at r * 128 + ((p ^ (r & 7)) << 4),
// so the fragment reads of 8 consecutive rows hit distinct banks.
//
// Problem class interface (A slot j of a lane copies tile row
// ra_j = (BM / 4) wave + 8 j + lane / 8, B slot j row rb_j likewise with BN):
//   void setup(int wave, int lane)      precompute the lane's row sources
//   void started(char* lds)             after the first segments are in flight
//                                        (may fill LDS beyond the NST stages)
//   void prep(int kt)                    once per copied segment, before a_row/b_row
//   const char* a_row(int j, int kt)    byte address of slot j's row, K segment kt
//   const char* b_row(int j, int kt)    (valid memory even for rows outside the
//                                        problem: their results are discarded)
//   int  nk()                           number of K segments
//   bool seg_end(int kt)                true if segment kt closes a group of K
//                                        segments after which fold() is called
//   void fold(acc, wr, wc, lane)        consume and clear acc
//   void finish(acc, wr, wc, lane)      final accumulators into acc
//   void store(acc, wr, wc, lane, lds)  write the tile out (LDS may be reused)
#pragma once
#include "async_copy.hpp"
#include "device_common.hpp"

namespace msgla {

constexpr int GD_THREADS = 256;

template <int WM, int WN>
struct GemmShape {
  static constexpr int BM = 32 * WM, BN = 32 * WN;
  static constexpr int A_BYTES = BM * 128, B_BYTES = BN * 128, STAGE = A_BYTES + B_BYTES;
  static constexpr int A_SLOTS = BM / 32, B_SLOTS = BN / 32;  // copy instructions per wave
};

template <int WM, int WN, int NST>
constexpr int gd_lds_bytes() {
  return NST * GemmShape<WM, WN>::STAGE;
}

template <typename T, int WM, int WN, int NST, class Prob>
__device__ __forceinline__ void gemm_dma_tile(Prob& prob, int n_valid, char* lds) {
  static_assert(NST == 2 || NST == 3, "2 or 3 pipeline stages");
  using S = GemmShape<WM, WN>;
  constexpr int COPIES = S::A_SLOTS + S::B_SLOTS;  // copy instructions per wave per segment
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wave >> 1, wc = wave & 1;
  const int lrow = lane & 15, lgrp = lane >> 4;
  const int nk = prob.nk();
  prob.setup(wave, lane);

  // this lane's copy slots: piece (lane & 7) ^ (lane >> 3) of rows 8 k + lane / 8
  const int cp_piece = ((lane & 7) ^ (lane >> 3)) << 4;
  auto issue = [&](int kt) {
    char* st = lds + (kt % NST) * S::STAGE;
    prob.prep(kt);
#pragma unroll
    for (int j = 0; j < S::A_SLOTS; ++j) {
      const int k = S::A_SLOTS * wave + j;
      __builtin_amdgcn_global_load_lds(prob.a_row(j, kt) + cp_piece, (lds_void_t*)(st + 1024 * k),
                                       16, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < S::B_SLOTS; ++j) {
      const int k = S::B_SLOTS * wave + j;
      __builtin_amdgcn_global_load_lds(prob.b_row(j, kt) + cp_piece,
                                       (lds_void_t*)(st + S::A_BYTES + 1024 * k), 16, 0, 0);
    }
  };

  // fragment offsets inside a stage (the same for every segment)
  int offA[WM][2], offB[WN][2];
#pragma unroll
  for (int sl = 0; sl < 2; ++sl) {
    const int p = sl * 4 + lgrp;
#pragma unroll
    for (int a = 0; a < WM; ++a) {
      const int r = wr * 16 * WM + 16 * a + lrow;
      offA[a][sl] = r * 128 + ((p ^ (r & 7)) << 4);
    }
#pragma unroll
    for (int b = 0; b < WN; ++b) {
      const int r = wc * 16 * WN + 16 * b + lrow;
      offB[b][sl] = S::A_BYTES + r * 128 + ((p ^ (r & 7)) << 4);
    }
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

  for (int kt = 0; kt < nk; ++kt) {
    // segment kt has landed once only the copies of later segments remain
    if (NST == 3 && kt + 1 < nk)
      wait_vmcnt<COPIES>();
    else
      wait_vmcnt<0>();
    lds_barrier();
    if (kt + NST - 1 < nk) issue(kt + NST - 1);
    const char* st = lds + (kt % NST) * S::STAGE;
#pragma unroll
    for (int sl = 0; sl < 2; ++sl) {
      u32x4 fa[WM], fb[WN];
#pragma unroll
      for (int a = 0; a < WM; ++a) fa[a] = ld16(st + offA[a][sl]);
#pragma unroll
      for (int b = 0; b < WN; ++b) fb[b] = ld16(st + offB[b][sl]);
#pragma unroll
      for (int b = 0; b < WN; ++b) {
        if (b < nb_valid) {
#pragma unroll
          for (int a = 0; a < WM; ++a) acc[a][b] = mma_slab<T>(fa[a], fb[b], acc[a][b]);
        }
      }
    }
    if (prob.seg_end(kt)) prob.fold(acc, wr, wc, lane);
  }
  prob.finish(acc, wr, wc, lane);
  lds_barrier();  // all waves are done with the stages
  prob.store(acc, wr, wc, lane, lds);
}

// Whole-tile fp32 staging for epilogues that route values by row and column:
// C[r][c] at C + r * (BN + 4) + c.  Call after gemm_dma_tile's final barrier
// (the stages are free), then lds_barrier() before reading other waves' values.
template <int WM, int WN>
constexpr int gd_ldc() {
  return 32 * WN + 4;
}
template <int WM, int WN, int NST>
constexpr int gd_lds_bytes_staged() {
  return gd_lds_bytes<WM, WN, NST>() > 32 * WM * gd_ldc<WM, WN>() * 4
             ? gd_lds_bytes<WM, WN, NST>()
             : 32 * WM * gd_ldc<WM, WN>() * 4;
}
template <int WM, int WN>
__device__ __forceinline__ void gd_stage_tile(const f32x4 (&acc)[WM][WN], int wr, int wc, int lane,
                                              float* C) {
  constexpr int LDC = gd_ldc<WM, WN>();
  const int lrow = lane & 15, lgrp = lane >> 4;
#pragma unroll
  for (int a = 0; a < WM; ++a)
#pragma unroll
    for (int b = 0; b < WN; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        C[(wr * 16 * WM + 16 * a + 4 * lgrp + i) * LDC + wc * 16 * WN + 16 * b + lrow] = acc[a][b][i];
}

// Writes a wave's accumulators through a per-wave LDS staging area in row
// blocks of 16 (one MFMA row tile across all its columns) and hands each
// staged block to emit(row0, C, ldc), C = 16 x (16 WN) fp32 starting at row
// row0 of the wave's sub-tile.  `stage` holds 4 * 16 * (16 WN + 4) floats.
template <int WM, int WN, class Emit>
__device__ __forceinline__ void stage_rows16(f32x4 (&acc)[WM][WN], int wave, int lane,
                                             float* stage, Emit&& emit) {
  constexpr int LDC = 16 * WN + 4;
  float* C = stage + wave * 16 * LDC;
  const int lrow = lane & 15, lgrp = lane >> 4;
#pragma unroll
  for (int a = 0; a < WM; ++a) {
#pragma unroll
    for (int b = 0; b < WN; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) C[(4 * lgrp + i) * LDC + 16 * b + lrow] = acc[a][b][i];
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (0 << 8));  // own LDS writes done
    asm volatile("" ::: "memory");
    emit(16 * a, C, LDC);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (0 << 8));  // reads done before reuse
    asm volatile("" ::: "memory");
  }
}

}  // namespace msgla
