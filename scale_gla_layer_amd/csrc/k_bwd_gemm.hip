// Layer backward: the activation-gradient products of every branch as grouped
// GEMMs on the forward's MFMA core (gemm_dma.hpp), and the weight transposes
// they read.
//
// MS-GLA notes, Sec. 3.2 (each branch's input projections and output projection)
// and Sec. 3.4 (training paragraph).  Two grouped launches per backward:
//   dLoss/do of every branch: dO W_o^T (scale 1) and dY_j W_o^T (coarse branches),
//   dLoss/d(pooled input) of every branch: dP Wp^T, dP = [dq | dk | dv | dg1].
// Both are C = A B^T with K contiguous in A and B (dLoss/do in fp32, the pooled
// inputs' gradient in the storage type): B is W_o as [h d_v][d] rows
// and Wp transposed to [d][NP], made by k_bwd_transpose from the packed
// weights (which hold W_o^T and Wp for the forward's products).
#include "device_common.hpp"
#include "gemm_dma.hpp"
#include "layout.hpp"

namespace msgla {

using BgCfg = GemmCfg<2, 4, 4, 2, 128, 2>;  // 128 x 128 tiles, 8 waves, double-buffered 128-byte K segments

namespace {

// OT: the type C is written in (fp32, or the storage type T)
template <typename T, typename OT>
struct BwdGemmRows {
  const BwdGemmGroup& G;
  int m0, n0;
  const char* arow[BgCfg::A_SLOTS];
  const char* brow[BgCfg::B_SLOTS];

  __device__ BwdGemmRows(const BwdGemmGroup& g, int m0_, int n0_) : G(g), m0(m0_), n0(n0_) {}
  __device__ int nk() const { return G.K * (int)sizeof(T) / BgCfg::KSEG; }
  // rows outside the problem read row 0 (their results are not stored)
  __device__ void setup(int wave, int lane) {
#pragma unroll
    for (int j = 0; j < BgCfg::A_SLOTS; ++j) {
      const int m = m0 + BgCfg::a_row(j, wave, lane);
      arow[j] = reinterpret_cast<const char*>(G.A) + (size_t)(m < G.M ? m : 0) * G.lda * sizeof(T);
    }
#pragma unroll
    for (int j = 0; j < BgCfg::B_SLOTS; ++j) {
      const int n = n0 + BgCfg::b_row(j, wave, lane);
      brow[j] = reinterpret_cast<const char*>(G.B) + (size_t)(n < G.N ? n : 0) * G.ldb * sizeof(T);
    }
  }
  __device__ void started(char*) {}
  __device__ void prep(int) {}
  __device__ const char* a_row(int j, int kt) const { return arow[j] + kt * BgCfg::KSEG; }
  __device__ const char* b_row(int j, int kt) const { return brow[j] + kt * BgCfg::KSEG; }
  __device__ bool seg_end(int) const { return false; }
  template <class Acc> __device__ void fold(Acc&, int, int, int) {}
  template <class Acc> __device__ void finish(Acc&, int, int, int) {}
  template <class Acc>
  __device__ void store(const Acc& acc, int wr, int wc, int lane, char* lds) {
    float* C = reinterpret_cast<float*>(lds);
    gd_stage_tile<BgCfg>(acc, wr, wc, lane, C);
    lds_barrier();
    for (int it = threadIdx.x; it < BgCfg::BM * (BgCfg::BN / 8); it += BgCfg::THREADS) {
      const int r = it / (BgCfg::BN / 8), cg = it % (BgCfg::BN / 8);
      const int m = m0 + r, col = n0 + cg * 8;
      if (m >= G.M || col >= G.N) continue;
      OT* dst = reinterpret_cast<OT*>(G.C) + (size_t)m * G.ldc + col;
      const float* src = C + r * BgCfg::LDC + cg * 8;
      if constexpr (sizeof(OT) == 4) {
        st16(dst, ld16(src));
        st16(dst + 4, ld16(src + 4));
      } else {
        float v[8];
        unpack16<float>(ld16(src), v);
        unpack16<float>(ld16(src + 4), v + 4);
        st16(dst, pack16<OT>(v));
      }
    }
  }
};

template <typename T, typename OT>
__global__ __launch_bounds__(BgCfg::THREADS) void k_bwd_gemm(const BwdGemm P) {
  __shared__ __attribute__((aligned(16))) char lds[BgCfg::LDS_STAGED];
  // XCD x (block id mod 8 under the hardware's round-robin dispatch) takes the
  // x-th eighth of every group's tiles, the groups in order: each XCD gets the
  // same mix of long and short K loops, and consecutive tiles of one group
  // (which share A rows) share its L2
  const int x = blockIdx.x % N_XCD;
  int li = blockIdx.x / N_XCD, gi = 0, local = -1;
  for (; gi < P.ngroups; ++gi) {
    const int nt = P.g[gi].total;
    const int lo = (int)((int64_t)nt * x / N_XCD), cnt = (int)((int64_t)nt * (x + 1) / N_XCD) - lo;
    if (li < cnt) {
      local = lo + li;
      break;
    }
    li -= cnt;
  }
  if (local < 0) return;
  const BwdGemmGroup& G = P.g[gi];
  const int tm = local / G.tiles_n, tn = local - tm * G.tiles_n;
  BwdGemmRows<T, OT> prob(G, tm * BgCfg::BM, tn * BgCfg::BN);
  gemm_dma_tile<T, BgCfg>(prob, G.N - tn * BgCfg::BN, lds);
}

// 64 x 64 tiles through LDS; one launch for every job
template <typename T>
__global__ __launch_bounds__(256) void k_bwd_transpose(const BwdTranspose P) {
  __shared__ T tl[64][65];
  int ji = 0;
  while (ji + 1 < P.njobs && (int)blockIdx.x >= P.j[ji + 1].tile_begin) ++ji;
  const BwdTransposeJob& J = P.j[ji];
  const int local = blockIdx.x - J.tile_begin;
  const int tr = local / J.tiles_c, tc = local - tr * J.tiles_c;
  const int r0 = tr * 64, c0 = tc * 64;
  const T* in = reinterpret_cast<const T*>(J.in);
  T* out = reinterpret_cast<T*>(J.out);
  const int x = threadIdx.x & 63, y0 = threadIdx.x >> 6;
  T v[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int r = r0 + y0 + 4 * k, c = c0 + x;
    const bool ok = r < J.R && c < J.C;
    v[k] = in[(size_t)(ok ? r : 0) * J.ldi + (ok ? c : 0)];
    if (!ok) v[k] = T(0.f);
  }
#pragma unroll
  for (int k = 0; k < 16; ++k) tl[y0 + 4 * k][x] = v[k];
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int c = c0 + y0 + 4 * k, r = r0 + x;
    if (c < J.C && r < J.Rp) out[(size_t)c * J.ldo + r] = tl[x][y0 + 4 * k];
  }
}

}  // namespace

// out_storage: C in the storage type (else fp32)
hipError_t launch_bwd_gemm(const BwdGemm& P, bool bf16_path, bool out_storage, hipStream_t st) {
  if (P.per_xcd == 0) return hipSuccess;
  const dim3 grid(P.per_xcd * N_XCD), block(BgCfg::THREADS);
  if (bf16_path && out_storage) hipLaunchKernelGGL((k_bwd_gemm<bf16, bf16>), grid, block, 0, st, P);
  else if (bf16_path) hipLaunchKernelGGL((k_bwd_gemm<bf16, float>), grid, block, 0, st, P);
  else hipLaunchKernelGGL((k_bwd_gemm<float, float>), grid, block, 0, st, P);
  return hipGetLastError();
}

hipError_t launch_bwd_transpose(const BwdTranspose& P, bool bf16_path, hipStream_t st) {
  if (P.total_tiles == 0) return hipSuccess;
  if (bf16_path) hipLaunchKernelGGL(k_bwd_transpose<bf16>, dim3(P.total_tiles), dim3(256), 0, st, P);
  else hipLaunchKernelGGL(k_bwd_transpose<float>, dim3(P.total_tiles), dim3(256), 0, st, P);
  return hipGetLastError();
}

}  // namespace msgla
