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

// grid: (ceil(d / (8 per16)), B * ceil(L / smax)); block 8 x 32 threads of 16-byte pieces
template <typename T>
__global__ __launch_bounds__(256) void k_pool(const PoolParams P) {
  constexpr int PER = per16<T>();
  const int pieces = P.d / PER;
  const int piece = blockIdx.x * 256 + threadIdx.x;
  if (piece >= pieces) return;
  const int nblk = (P.L + P.smax - 1) / P.smax;
  const int b = blockIdx.y / nblk, q = blockIdx.y - b * nblk;
  const T* x = reinterpret_cast<const T*>(P.x) + ((size_t)b * P.L + (size_t)q * P.smax) * P.d +
               piece * PER;
  const int rows = min(P.smax, P.L - q * P.smax);
  float acc[MSGLA_MAX_BRANCHES][PER];
#pragma unroll
  for (int i = 0; i < MSGLA_MAX_BRANCHES; ++i)
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[i][e] = 0.f;
  for (int u = 0; u < rows; ++u) {
    float v[PER];
    unpack16<T>(ld16(x + (size_t)u * P.d), v);
#pragma unroll
    for (int i = 0; i < MSGLA_MAX_BRANCHES; ++i) {
      if (i < P.nout) {
        const PoolOut& o = P.out[i];
#pragma unroll
        for (int e = 0; e < PER; ++e) acc[i][e] += v[e];
        if ((u + 1) % o.s == 0) {  // a block of this scale is complete
          const int j = (q * P.smax + u + 1) / o.s - 1;
          if (j < o.n) {
            float m[PER];
#pragma unroll
            for (int e = 0; e < PER; ++e) m[e] = acc[i][e] * o.inv_s;
            st16(reinterpret_cast<T*>(o.xp) + ((size_t)b * o.n + j) * P.d + piece * PER,
                 pack16<T>(m));
          }
#pragma unroll
          for (int e = 0; e < PER; ++e) acc[i][e] = 0.f;
        }
      }
    }
  }
}

hipError_t launch_pool(const PoolParams& P, bool bf16_path, hipStream_t st) {
  const int per = bf16_path ? 8 : 4;
  const dim3 grid((P.d / per + 255) / 256, P.B * ((P.L + P.smax - 1) / P.smax));
  if (bf16_path)
    hipLaunchKernelGGL(k_pool<bf16>, grid, dim3(256), 0, st, P);
  else
    hipLaunchKernelGGL(k_pool<float>, grid, dim3(256), 0, st, P);
  return hipGetLastError();
}

}  // namespace msgla
