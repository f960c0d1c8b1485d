// K1 — pooled projection GEMM over all branches in one launch.
//
// MS-GLA notes, Sec. 3.1 (Eq. (8), non-overlapping mean pooling) and Sec. 3.2
// (independent q, k, v and low-rank gate projections per branch), plus the
// fusion logits of Eq. (10) from the unpooled x_t.
//
// For branch i (scale s): C_i = P_s(X) * Wp_i^T, where row (b, j) of P_s(X) is
// the mean of X rows b*L + j*s .. + s-1 (only complete blocks), computed in
// fp32 inside the A-operand loader and rounded once to the storage type, so
// the pooled sequence never touches HBM (the s raw loads are issued before the
// MFMAs of the previous K segment and summed after them).  Wp_i stacks the transposed q, k, v,
// first-gate-factor and (for the branch that carries them) fusion-logit
// weights; the epilogue routes each column range to its consumer layout:
// q, k head-major fp32 rows, v transposed per chunk, the gate factor in fp32, and
// the fusion logits turned into softmax weights (Eq. (10)) with the bias.
// The work list is every (group, m-tile, n-tile), n fastest, laid out so each
// XCD walks a contiguous range (tiles that share an A tile share an L2).
#include "device_common.hpp"
#include "gemm_engine.hpp"
#include "layout.hpp"

namespace msgla {

template <typename T, int SMAX>
struct K1Prob {
  const K1Params& P;
  const K1Group& G;
  int m0, n0;
  const T* arow[4];
  const T* brow[4];
  const T* apos[4];        // first raw row of the piece being fetched
  u32x4 raw[4][SMAX];      // raw 16-byte pieces of the s rows of a pooled block
  u32x4 rb[4];
  float inv_s;

  __device__ K1Prob(const K1Params& p, const K1Group& g, int m0_, int n0_)
      : P(p), G(g), m0(m0_), n0(n0_), inv_s(1.0f / (float)g.s) {}

  __device__ void a_setup(int i, int row) {
    const int m = m0 + row;
    if (m < G.M) {
      const int b = m / G.n, j = m - b * G.n;
      arow[i] = reinterpret_cast<const T*>(P.x) + ((size_t)b * P.L + (size_t)j * G.s) * P.d;
    } else {
      arow[i] = nullptr;
    }
  }
  // issue the loads of the s raw rows (consumed after the MFMAs in a_get)
  __device__ void a_fetch(int i, int kt, int c16) {
    if (!arow[i]) return;
    const T* p = arow[i] + kt * (128 / sizeof(T)) + c16 * per16<T>();
    apos[i] = p;
#pragma unroll
    for (int u = 0; u < SMAX; ++u)
      if (u < G.s) raw[i][u] = ld16(p + (size_t)u * P.d);
  }
  __device__ u32x4 a_get(int i) {
    if (!arow[i]) return zero16();
    if (SMAX == 1 || G.s == 1) return raw[i][0];
    float sum[per16<T>()], tmp[per16<T>()];
    unpack16<T>(raw[i][0], sum);
#pragma unroll
    for (int u = 1; u < SMAX; ++u) {
      if (u < G.s) {
        unpack16<T>(raw[i][u], tmp);
#pragma unroll
        for (int e = 0; e < per16<T>(); ++e) sum[e] += tmp[e];
      }
    }
    for (int u = SMAX; u < G.s; ++u) {  // blocks longer than SMAX: remaining rows now
      unpack16<T>(ld16(apos[i] + (size_t)u * P.d), tmp);
#pragma unroll
      for (int e = 0; e < per16<T>(); ++e) sum[e] += tmp[e];
    }
#pragma unroll
    for (int e = 0; e < per16<T>(); ++e) sum[e] *= inv_s;
    return pack16<T>(sum);
  }
  __device__ void b_setup(int i, int row) {
    const int n = n0 + row;
    brow[i] = (n < G.N) ? reinterpret_cast<const T*>(G.Wp) + (size_t)n * P.d : nullptr;
  }
  __device__ void b_fetch(int i, int kt, int c16) {
    rb[i] = brow[i] ? ld16(brow[i] + kt * (128 / sizeof(T)) + c16 * per16<T>()) : zero16();
  }
  __device__ u32x4 b_get(int i) { return rb[i]; }

  __device__ void store8(T* dst, const float* v) {
    if constexpr (sizeof(T) == 2) {
      st16(dst, pack16<T>(v));
    } else {
      st16(dst, pack16<T>(v));
      st16(dst + 4, pack16<T>(v + 4));
    }
  }

  __device__ void epilogue(const float* C, int ldc) {
    const int tid = threadIdx.x;
    // (1) row-major destinations: q, k, gate factor, fusion weights
    for (int it = tid; it < GEMM_BM * (GEMM_BN / 8); it += GEMM_THREADS) {
      const int r = it >> 4, cg = it & 15;
      const int m = m0 + r, col = n0 + cg * 8;
      if (m >= G.M || col >= G.N) continue;
      if (col >= G.col_v && col < G.col_g) continue;  // v: transposed pass below
      const int b = m / G.n, j = m - b * G.n;
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = C[r * ldc + cg * 8 + e];
      if (col < G.col_v) {
        const bool isq = col < G.col_k;
        const int c = isq ? col : col - G.col_k;
        const int hh = c / P.dk, ch = c - hh * P.dk;
        float* dst = (isq ? G.q : G.k) + (((size_t)b * G.h + hh) * G.np + j) * P.dk + ch;
        st16(dst, pack16<float>(v));
        st16(dst + 4, pack16<float>(v + 4));
      } else if (col < (G.col_z >= 0 ? G.col_z : G.col_end)) {
        float* dst = G.g + ((size_t)b * G.np + j) * P.rp + (col - G.col_g);
        st16(dst, pack16<float>(v));
        st16(dst + 4, pack16<float>(v + 4));
      } else if (G.col_z >= 0 && col == G.col_z) {
        // softmax over the m fusion logits of this (unpooled) position, Eq. (10)
        float z[8], mx = -INFINITY, sum = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          z[e] = (e < P.m) ? v[e] + P.bf[e] : -INFINITY;
          mx = fmaxf(mx, z[e]);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          z[e] = (e < P.m) ? __expf(z[e] - mx) : 0.f;
          sum += z[e];
        }
        const float inv = 1.0f / sum;
#pragma unroll
        for (int e = 0; e < 8; ++e) z[e] *= inv;
        float* dst = P.w + ((size_t)b * P.L + j) * FUSION_STRIDE;
        st16(dst, pack16<float>(z));
        st16(dst + 4, pack16<float>(z + 4));
      }
    }
    // (2) v, written transposed per chunk: vT[b][hh][chunk][v][tau]
    if (G.col_g > G.col_v && n0 < G.col_g && n0 + GEMM_BN > G.col_v) {
      for (int it = tid; it < GEMM_BN * (GEMM_BM / 8); it += GEMM_THREADS) {
        const int cl = it & (GEMM_BN - 1), rg = it >> 7;
        const int col = n0 + cl;
        if (col < G.col_v || col >= G.col_g) continue;
        const int cv = col - G.col_v;
        const int hh = cv / P.dv, vch = cv - hh * P.dv;
        const int mA = m0 + rg * 8;
        if (mA >= G.M) continue;
        const int b0 = mA / G.n, j0 = mA - b0 * G.n;
        T* vT = reinterpret_cast<T*>(G.vT);
        if (mA + 7 < G.M && j0 + 7 < G.n && (j0 & 7) == 0) {
          float v[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = C[(rg * 8 + e) * ldc + cl];
          const int chunk = j0 / P.C, tau = j0 - chunk * P.C;
          store8(vT + ((((size_t)b0 * G.h + hh) * G.nch + chunk) * P.dv + vch) * P.C + tau, v);
        } else {
          for (int e = 0; e < 8; ++e) {
            const int m = mA + e;
            if (m >= G.M) break;
            const int b = m / G.n, j = m - b * G.n;
            const int chunk = j / P.C, tau = j - chunk * P.C;
            vT[((((size_t)b * G.h + hh) * G.nch + chunk) * P.dv + vch) * P.C + tau] =
                from_f32<T>(C[(rg * 8 + e) * ldc + cl]);
          }
        }
      }
    }
  }
};

template <typename T, int SMAX>
__global__ __launch_bounds__(GEMM_THREADS) void k1_pool_proj(const K1Params P) {
  __shared__ __attribute__((aligned(16))) char lds[GEMM_LDS_BYTES];
  const int tile = remap_xcd(blockIdx.x, P.per_xcd);
  if (tile >= P.total_tiles) return;
  int gi = 0;
  while (gi + 1 < P.ngroups && tile >= P.g[gi + 1].tile_begin) ++gi;
  const K1Group& G = P.g[gi];
  const int local = tile - G.tile_begin;
  const int tm = local / G.tiles_n, tn = local - tm * G.tiles_n;
  K1Prob<T, SMAX> prob(P, G, tm * GEMM_BM, tn * GEMM_BN);
  gemm_tile_128<T>(prob, P.d * (int)sizeof(T) / 128, G.N - tn * GEMM_BN, lds);
}

template <typename T>
static void launch_k1_t(const K1Params& P, dim3 grid, hipStream_t stream) {
  int smax = 1;
  for (int g = 0; g < P.ngroups; ++g) smax = smax > P.g[g].s ? smax : P.g[g].s;
  const dim3 block(GEMM_THREADS);
  if (smax <= 1)
    hipLaunchKernelGGL((k1_pool_proj<T, 1>), grid, block, 0, stream, P);
  else if (smax <= 2)
    hipLaunchKernelGGL((k1_pool_proj<T, 2>), grid, block, 0, stream, P);
  else if (smax <= 4)
    hipLaunchKernelGGL((k1_pool_proj<T, 4>), grid, block, 0, stream, P);
  else
    hipLaunchKernelGGL((k1_pool_proj<T, 8>), grid, block, 0, stream, P);
}

hipError_t launch_k1(const K1Params& P, bool bf16_path, hipStream_t stream) {
  const dim3 grid(P.per_xcd * N_XCD);
  if (bf16_path)
    launch_k1_t<bf16>(P, grid, stream);
  else
    launch_k1_t<float>(P, grid, stream);
  return hipGetLastError();
}

}  // namespace msgla
