// Pooling prepass: the non-overlapping block means of Eq. (8) (MS-GLA notes,
// Sec. 3.1) for every coarse branch, rounded once to the storage type.
//
// X is read once for all scales that divide the largest coarse scale s_max:
// a thread sums one 16-byte column piece over a block of s_max rows in fp32
// and emits the block means of every such scale (a partial tail block is not
// pooled: it never reaches the recurrence).  Scales that do not divide s_max
// take a second pass of their own.  HBM-bound: reads B L d elements per pass,
// writes sum_s B floor(L/s) d.
#include "device_common.hpp"
#include "layout.hpp"

namespace msgla {

// One thread per (row block, 16-byte column piece), consecutive threads on
// consecutive pieces of the same rows.  The rows of a block are loaded U at a
// time before any of them is summed, so each thread keeps U loads in flight.
template <typename T>
__global__ __launch_bounds__(256) void k_pool(const PoolParams P) {
  constexpr int PER = per16<T>();
  constexpr int U = 8;
  const int pieces = P.d / PER;
  const int nblk = (P.L + P.smax - 1) / P.smax;
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long)P.B * nblk * pieces) return;
  const int grp = (int)(idx / pieces), piece = (int)(idx - (long)grp * pieces);
  const int b = grp / nblk, q = grp - b * nblk;
  const T* x = reinterpret_cast<const T*>(P.x) + ((size_t)b * P.L + (size_t)q * P.smax) * P.d +
               piece * PER;
  const int rows = min(P.smax, P.L - q * P.smax);
  float acc[MSGLA_MAX_BRANCHES][PER];
  int cnt[MSGLA_MAX_BRANCHES], jout[MSGLA_MAX_BRANCHES];
#pragma unroll
  for (int i = 0; i < MSGLA_MAX_BRANCHES; ++i) {
    cnt[i] = 0;
    jout[i] = i < P.nout ? q * (P.smax / P.out[i].s) : 0;  // s divides smax
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[i][e] = 0.f;
  }
  for (int u0 = 0; u0 < rows; u0 += U) {
    u32x4 raw[U];
#pragma unroll
    for (int k = 0; k < U; ++k) raw[k] = (u0 + k < rows) ? ld16(x + (size_t)(u0 + k) * P.d) : zero16();
#pragma unroll
    for (int k = 0; k < U; ++k) {
      if (u0 + k >= rows) break;
      float v[PER];
      unpack16<T>(raw[k], v);
#pragma unroll
      for (int i = 0; i < MSGLA_MAX_BRANCHES; ++i) {
        if (i < P.nout) {
          const PoolOut& o = P.out[i];
#pragma unroll
          for (int e = 0; e < PER; ++e) acc[i][e] += v[e];
          if (++cnt[i] == o.s) {  // a block of this scale is complete
            if (jout[i] < o.n) {
              float m[PER];
#pragma unroll
              for (int e = 0; e < PER; ++e) m[e] = acc[i][e] * o.inv_s;
              st16(reinterpret_cast<T*>(o.xp) + ((size_t)b * o.n + jout[i]) * P.d + piece * PER,
                   pack16<T>(m));
            }
            ++jout[i];
            cnt[i] = 0;
#pragma unroll
            for (int e = 0; e < PER; ++e) acc[i][e] = 0.f;
          }
        }
      }
    }
  }
}

hipError_t launch_pool(const PoolParams& P, bool bf16_path, hipStream_t st) {
  const int per = bf16_path ? 8 : 4;
  const long threads = (long)P.B * ((P.L + P.smax - 1) / P.smax) * (P.d / per);
  const dim3 grid((unsigned)((threads + 255) / 256));
  if (bf16_path)
    hipLaunchKernelGGL(k_pool<bf16>, grid, dim3(256), 0, st, P);
  else
    hipLaunchKernelGGL(k_pool<float>, grid, dim3(256), 0, st, P);
  return hipGetLastError();
}

}  // namespace msgla
