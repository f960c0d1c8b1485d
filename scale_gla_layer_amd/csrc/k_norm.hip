// Optional per-head RMS normalisation of each branch's GLA output before its
// output projection.  The MS-GLA notes (Sec. 3.2) name a per-branch
// normalisation without giving its form; the form taken is
//   y_c <- y_c / sqrt(mean_c' y_c'^2 + eps) * g_c   over the d_v channels of a head,
// with fp32 gains g per branch and eps = 1e-6.  Rows (b, head, j) of a
// branch's y [B][h][np][d_v] are normalised in place, between the chunk-state kernel
// that writes y and the output projections that read it.  HBM-bound: reads and
// writes y once.
#include "device_common.hpp"
#include "layout.hpp"

namespace msgla {

// Each wave takes NR consecutive rows and issues all their loads before the
// first reduction, so several rows per wave are in flight.
constexpr int NORM_NR = 4;

template <typename T>
__global__ __launch_bounds__(256) void k_norm_rows(const NormParams P) {
  constexpr int PER = per16<T>();
  const int row0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * NORM_NR;
  const int lane = threadIdx.x & 63;
  if (row0 >= P.total_rows) return;  // the same for the whole wave
  const int pieces = P.dv / PER;     // 16-byte pieces of a row, at most 128
  T* yr[NORM_NR];
  const float* gr[NORM_NR];
  bool ok[NORM_NR];
#pragma unroll
  for (int u = 0; u < NORM_NR; ++u) {
    const int row = min(row0 + u, P.total_rows - 1);  // rows past the end redo the last one, unstored
    ok[u] = row0 + u < P.total_rows;
    int bi = 0;
    while (bi + 1 < P.nbranch && row >= P.br[bi + 1].row_begin) ++bi;
    const NormBranch& Br = P.br[bi];
    const int local = row - Br.row_begin;
    const int bh = local / Br.n, j = local - bh * Br.n;
    yr[u] = reinterpret_cast<T*>(Br.y) + ((size_t)bh * Br.np + j) * P.dv;
    gr[u] = Br.g + (bh % Br.h) * P.dv;
  }
  u32x4 raw[NORM_NR][2];
#pragma unroll
  for (int u = 0; u < NORM_NR; ++u)
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int pc = min(lane + 64 * k, pieces - 1);
      raw[u][k] = ld16(yr[u] + pc * PER);
    }
#pragma unroll
  for (int u = 0; u < NORM_NR; ++u) {
    float v[2][PER];
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      unpack16<T>(raw[u][k], v[k]);
      if (lane + 64 * k < pieces) {
#pragma unroll
        for (int e = 0; e < PER; ++e) ss += v[k][e] * v[k][e];
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
    const float rs = 1.0f / sqrtf(ss / (float)P.dv + NORM_EPS);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int pc = lane + 64 * k;
      if (ok[u] && pc < pieces) {
        float f[PER];
#pragma unroll
        for (int e = 0; e < PER; e += 4) {
          float g4[4];
          unpack16<float>(ld16(gr[u] + pc * PER + e), g4);
#pragma unroll
          for (int i = 0; i < 4; ++i) f[e + i] = v[k][e + i] * rs * g4[i];
        }
        st16(yr[u] + pc * PER, pack16<T>(f));
      }
    }
  }
}

hipError_t launch_norm(const NormParams& P, bool bf16_path, hipStream_t st) {
  if (P.total_rows == 0) return hipSuccess;
  const dim3 grid((P.total_rows + 4 * NORM_NR - 1) / (4 * NORM_NR)), block(256);
  if (bf16_path)
    hipLaunchKernelGGL(k_norm_rows<bf16>, grid, block, 0, st, P);
  else
    hipLaunchKernelGGL(k_norm_rows<float>, grid, block, 0, st, P);
  return hipGetLastError();
}

}  // namespace msgla
