// 128 x 128 output-tile MFMA GEMM core for gfx950, C = A * B^T with both
// operands read along K ("NT"), fp32 accumulation.
//
// 256 threads = 4 wave64s in a 2 x 2 grid; each wave owns a 64 x 64 sub-tile
// (4 x 4 MFMA tiles of 16 x 16).  K advances in 128-byte row segments
// (64 bf16 or 32 fp32 values = two 64-byte k-slabs) staged through LDS with
// double buffering.  Each iteration issues the global loads of the next
// segment, runs the MFMAs of the current one, and only then combines the
// loaded data (pooling sums, fusion scaling) and writes it to the other LDS
// stage, so memory latency overlaps the MFMAs; one barrier per segment.
// LDS rows are padded to 144 bytes so the 16-byte fragment reads of 8
// consecutive lanes hit distinct banks.
//
// The operand loaders and the epilogue come from a problem class:
//   void a_setup(int i, int row) / void a_fetch(int i, int kt, int c16) / u32x4 a_get(int i)
//   void b_setup(int i, int row) / void b_fetch(int i, int kt, int c16) / u32x4 b_get(int i)
//   void epilogue(const float* C, int ldc)   (C = the 128 x 128 fp32 tile in LDS)
// a_fetch issues the loads of piece i (row = t/8 + 32 i, c16 = t % 8) of
// segment kt into the problem's registers; a_get, called after the MFMAs,
// returns the 16 bytes to stage.  Loaders return zeros outside the problem.
#pragma once
#include "device_common.hpp"

namespace msgla {

constexpr int GEMM_BM = 128;
constexpr int GEMM_BN = 128;
constexpr int GEMM_THREADS = 256;
constexpr int GEMM_ROWB = 144;                        // padded LDS row (bytes)
constexpr int GEMM_STAGE = (GEMM_BM + GEMM_BN) * GEMM_ROWB;
constexpr int GEMM_LDC = GEMM_BN + 4;                 // fp32 epilogue tile row
constexpr int GEMM_LDS_BYTES =
    (2 * GEMM_STAGE > GEMM_BM * GEMM_LDC * 4) ? 2 * GEMM_STAGE : GEMM_BM * GEMM_LDC * 4;

template <typename T, class Prob>
__device__ __forceinline__ void gemm_tile_128(Prob& prob, int nk, int n_valid, char* lds) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  const int lrow = lane & 15, lgrp = lane >> 4;
  const int c16 = tid & 7;

#pragma unroll
  for (int i = 0; i < 4; ++i) {
    prob.a_setup(i, (tid >> 3) + 32 * i);
    prob.b_setup(i, (tid >> 3) + 32 * i);
  }

  f32x4 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = zero4();

  // column tiles of this wave that hold at least one valid column
  int nb_valid = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b) nb_valid += (wc * 64 + 16 * b < n_valid) ? 1 : 0;

  auto fetch = [&](int kt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      prob.a_fetch(i, kt, c16);
      prob.b_fetch(i, kt, c16);
    }
  };
  auto stage = [&](int st) {
    char* sa = lds + st * GEMM_STAGE;
    char* sb = sa + GEMM_BM * GEMM_ROWB;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = (tid >> 3) + 32 * i;
      st16(sa + row * GEMM_ROWB + c16 * 16, prob.a_get(i));
      st16(sb + row * GEMM_ROWB + c16 * 16, prob.b_get(i));
    }
  };

  fetch(0);
  stage(0);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const bool more = kt + 1 < nk;
    if (more) fetch(kt + 1);
    const char* sa = lds + (kt & 1) * GEMM_STAGE;
    const char* sb = sa + GEMM_BM * GEMM_ROWB;
#pragma unroll
    for (int sl = 0; sl < 2; ++sl) {
      u32x4 fa[4], fb[4];
#pragma unroll
      for (int a = 0; a < 4; ++a)
        fa[a] = ld16(sa + (wr * 64 + 16 * a + lrow) * GEMM_ROWB + sl * 64 + lgrp * 16);
#pragma unroll
      for (int b = 0; b < 4; ++b)
        fb[b] = ld16(sb + (wc * 64 + 16 * b + lrow) * GEMM_ROWB + sl * 64 + lgrp * 16);
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        if (b < nb_valid) {
#pragma unroll
          for (int a = 0; a < 4; ++a) acc[a][b] = mma_slab<T>(fa[a], fb[b], acc[a][b]);
        }
      }
    }
    if (more) stage((kt + 1) & 1);
    __syncthreads();
  }

  // stage the fp32 tile in LDS (the operand stages are free after the last barrier)
  float* C = reinterpret_cast<float*>(lds);
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        C[(wr * 64 + 16 * a + 4 * lgrp + i) * GEMM_LDC + wc * 64 + 16 * b + lrow] = acc[a][b][i];
  __syncthreads();
  prob.epilogue(C, GEMM_LDC);
}

}  // namespace msgla
