// K3 — causal hold, softmax fusion and the per-branch output projections as
// one GEMM.
//
// MS-GLA notes, Sec. 3.2 (each branch projects back to the common d space with
// its own output projection) and Sec. 3.3 (causal upsampling: coarse output j
// of branch s is usable from position (j+1)s-1 until block j+1 completes, zero
// before the first block; Eqs. (10)-(11): O_t = sum_i w_{t,i} Yhat^{(i)}_t).
// Because W_o^{(i)} is linear,
//   O_t = sum_i w_{t,i} y^{(i)}_{j_i(t)} W_o^{(i)}
//       = [w_{t,1} y^{(1)}_{j_1(t)} | ... | w_{t,m} y^{(m)}_{j_m(t)}] [W_o^{(1)}; ...; W_o^{(m)}],
// with j_i(t) = floor((t+1)/s_i) - 1 (a zero row when negative).  The A-operand
// loader gathers the held coarse rows and applies the fusion weight, B is the
// stacked W_o^T, and the epilogue writes O row-major.  Each 128-byte K segment
// lies inside one branch (branch K ranges are padded to 128 bytes).
#include "device_common.hpp"
#include "gemm_engine.hpp"
#include "layout.hpp"

namespace msgla {

template <typename T>
struct K3Prob {
  const K3Params& P;
  int m0, n0;
  int ab[4], at[4];  // sequence and position of each loaded A row (-1: none)
  const T* brow[4];
  u32x4 ra[4], rb[4];
  float wv[4];

  __device__ K3Prob(const K3Params& p, int m0_, int n0_) : P(p), m0(m0_), n0(n0_) {}

  __device__ void a_setup(int i, int row) {
    const int m = m0 + row;
    if (m < P.B * P.L) {
      ab[i] = m / P.L;
      at[i] = m - ab[i] * P.L;
    } else {
      ab[i] = -1;
      at[i] = 0;
    }
  }
  // gather the held coarse row (Sec. 3.3) and its fusion weight; scaled in a_get
  __device__ void a_fetch(int i, int kt, int c16) {
    ra[i] = zero16();
    wv[i] = 0.f;
    if (ab[i] < 0) return;
    constexpr int E128 = 128 / sizeof(T);
    const int k0 = kt * E128;
    int bi = 0;
    while (bi + 1 < MSGLA_MAX_BRANCHES && bi + 1 < P.m && k0 >= P.br[bi + 1].ko) ++bi;
    const K3Branch& Br = P.br[bi];
    const int j = (at[i] + 1) / Br.s - 1;
    const int kk = k0 - Br.ko + c16 * per16<T>();
    if (j < 0 || kk >= Br.h * P.dv) return;
    const int hh = kk / P.dv, v = kk - hh * P.dv;
    ra[i] = ld16(reinterpret_cast<const T*>(Br.y) + (((size_t)ab[i] * Br.h + hh) * Br.np + j) * P.dv + v);
    wv[i] = (P.m > 1) ? P.w[((size_t)ab[i] * P.L + at[i]) * FUSION_STRIDE + bi] : 1.f;
  }
  __device__ u32x4 a_get(int i) {
    if (P.m == 1) return ra[i];
    float f[per16<T>()];
    unpack16<T>(ra[i], f);
#pragma unroll
    for (int e = 0; e < per16<T>(); ++e) f[e] *= wv[i];
    return pack16<T>(f);
  }
  __device__ void b_setup(int i, int row) {
    const int n = n0 + row;
    brow[i] = (n < P.d) ? reinterpret_cast<const T*>(P.WoT) + (size_t)n * P.Ktot : nullptr;
  }
  __device__ void b_fetch(int i, int kt, int c16) {
    rb[i] = brow[i] ? ld16(brow[i] + kt * (128 / sizeof(T)) + c16 * per16<T>()) : zero16();
  }
  __device__ u32x4 b_get(int i) { return rb[i]; }
  __device__ void epilogue(const float* C, int ldc) {
    const int tid = threadIdx.x;
    T* out = reinterpret_cast<T*>(P.out);
    for (int it = tid; it < GEMM_BM * (GEMM_BN / 8); it += GEMM_THREADS) {
      const int r = it >> 4, cg = it & 15;
      const int m = m0 + r, col = n0 + cg * 8;
      if (m >= P.B * P.L || col >= P.d) continue;
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = C[r * ldc + cg * 8 + e];
      T* dst = out + (size_t)m * P.d + col;
      if constexpr (sizeof(T) == 2) {
        st16(dst, pack16<T>(v));
      } else {
        st16(dst, pack16<T>(v));
        st16(dst + 4, pack16<T>(v + 4));
      }
    }
  }
};

template <typename T>
__global__ __launch_bounds__(GEMM_THREADS) void k3_hold_fuse(const K3Params P) {
  __shared__ __attribute__((aligned(16))) char lds[GEMM_LDS_BYTES];
  const int tile = remap_xcd(blockIdx.x, P.per_xcd);
  if (tile >= P.total_tiles) return;
  const int tm = tile / P.tiles_n, tn = tile - tm * P.tiles_n;
  K3Prob<T> prob(P, tm * GEMM_BM, tn * GEMM_BN);
  gemm_tile_128<T>(prob, P.Ktot * (int)sizeof(T) / 128, P.d - tn * GEMM_BN, lds);
}

hipError_t launch_k3(const K3Params& P, bool bf16_path, hipStream_t stream) {
  const dim3 grid(P.per_xcd * N_XCD), block(GEMM_THREADS);
  if (bf16_path)
    hipLaunchKernelGGL(k3_hold_fuse<bf16>, grid, block, 0, stream, P);
  else
    hipLaunchKernelGGL(k3_hold_fuse<float>, grid, block, 0, stream, P);
  return hipGetLastError();
}

}  // namespace msgla
