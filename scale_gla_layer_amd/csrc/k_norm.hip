// Optional per-head RMS normalisation of each branch's GLA output before its
// output projection.  The MS-GLA notes (Sec. 3.2) name a per-branch
// normalisation without giving its form; the form taken is
//   y_c <- y_c / sqrt(mean_c' y_c'^2 + eps) * g_c   over the d_v channels of a head,
// with fp32 gains g per branch and eps = 1e-6.  Rows (b, head, j) of a
// branch's y [B][h][np][d_v] are normalised in place (or into a second buffer of
// the same layout, for the backward's recompute), between the chunk-state
// kernel that writes y and the output projections that read it.  HBM-bound:
// reads and writes y once.
#include "device_common.hpp"
#include "layout.hpp"

namespace msgla {

// A row takes LPR lanes (32 when it has at most 32 pieces of 16 bytes, so a
// wave holds two rows side by side, else 64), and each wave takes NORM_NR such
// row groups, issuing all their loads before the first reduction.
constexpr int NORM_NR = 4;

template <typename T, int LPR>
__global__ __launch_bounds__(256) void k_norm_rows(const NormParams P) {
  constexpr int PER = per16<T>(), RPS = 64 / LPR, PPL = LPR == 64 ? 2 : 1;  // rows per slot, pieces per lane
  const int lane = threadIdx.x & 63, sub = lane / LPR, l = lane % LPR;
  const int row0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * NORM_NR * RPS;
  if (row0 >= P.total_rows) return;  // the same for the whole wave
  const int pieces = P.dv / PER;     // 16-byte pieces of a row: at most LPR * PPL
  T* yr[NORM_NR];
  T* yw[NORM_NR];
  const float* gr[NORM_NR];
  bool ok[NORM_NR];
#pragma unroll
  for (int u = 0; u < NORM_NR; ++u) {
    const int want = row0 + u * RPS + sub;
    const int row = min(want, P.total_rows - 1);  // rows past the end redo the last one, unstored
    ok[u] = want < P.total_rows;
    int bi = 0;
    while (bi + 1 < P.nbranch && row >= P.br[bi + 1].row_begin) ++bi;
    const NormBranch& Br = P.br[bi];
    const int local = row - Br.row_begin;
    const int bh = local / Br.n, j = local - bh * Br.n;
    yr[u] = reinterpret_cast<T*>(Br.y) + ((size_t)bh * Br.np + j) * P.dv;
    yw[u] = reinterpret_cast<T*>(Br.yo ? Br.yo : Br.y) + ((size_t)bh * Br.np + j) * P.dv;
    gr[u] = Br.g + (bh % Br.h) * P.dv;
  }
  u32x4 raw[NORM_NR][PPL];
#pragma unroll
  for (int u = 0; u < NORM_NR; ++u)
#pragma unroll
    for (int k = 0; k < PPL; ++k) raw[u][k] = ld16(yr[u] + min(l + LPR * k, pieces - 1) * PER);
#pragma unroll
  for (int u = 0; u < NORM_NR; ++u) {
    float v[PPL][PER];
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < PPL; ++k) {
      unpack16<T>(raw[u][k], v[k]);
      if (l + LPR * k < pieces) {
#pragma unroll
        for (int e = 0; e < PER; ++e) ss += v[k][e] * v[k][e];
      }
    }
#pragma unroll
    for (int off = LPR / 2; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
    const float rs = 1.0f / sqrtf(ss / (float)P.dv + NORM_EPS);
#pragma unroll
    for (int k = 0; k < PPL; ++k) {
      const int pc = l + LPR * k;
      if (ok[u] && pc < pieces) {
        float f[PER];
#pragma unroll
        for (int e = 0; e < PER; e += 4) {
          float g4[4];
          unpack16<float>(ld16(gr[u] + pc * PER + e), g4);
#pragma unroll
          for (int i = 0; i < 4; ++i) f[e + i] = v[k][e + i] * rs * g4[i];
        }
        st16(yw[u] + pc * PER, pack16<T>(f));
      }
    }
  }
}

template <typename T>
static void launch_norm_t(const NormParams& P, hipStream_t st) {
  const bool half = P.dv / per16<T>() <= 32;
  const int rows_per_block = 4 * NORM_NR * (half ? 2 : 1);
  const dim3 grid((P.total_rows + rows_per_block - 1) / rows_per_block), block(256);
  if (half)
    hipLaunchKernelGGL((k_norm_rows<T, 32>), grid, block, 0, st, P);
  else
    hipLaunchKernelGGL((k_norm_rows<T, 64>), grid, block, 0, st, P);
}

hipError_t launch_norm(const NormParams& P, bool bf16_path, hipStream_t st) {
  if (P.total_rows == 0) return hipSuccess;
  if (bf16_path)
    launch_norm_t<bf16>(P, st);
  else
    launch_norm_t<float>(P, st);
  return hipGetLastError();
}

}  // namespace msgla
