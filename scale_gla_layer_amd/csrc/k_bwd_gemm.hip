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



// ---- weight gradients: C = A^T B over the position axis, bf16 storage ----
// MS-GLA notes, Sec. 3.4 (training paragraph): the gradient of every weight
// matrix of the layer is a sum over positions of outer products of its input
// rows and its output's gradient rows, C [M][N] = sum_k A[k][m] B[k][n], with
// both operands position-major.  The matrix cores read operands with K
// contiguous, so each 64-position step of a 128 x 128 tile is copied into LDS
// transposed: a thread loads four positions' 16-byte pieces (eight m, or eight
// n) and writes each m as one 8-byte run of four positions.  The 16-byte
// K chunks of an LDS row are XOR-swizzled by (row / 8) % 8, which spreads the
// transposing writes and the fragment reads over the banks.  Four waves of
// 64 x 64 (4 x 4 bf16 MFMA tiles) per workgroup; the next step's pieces are
// loaded into registers while the current step is multiplied.  The K range is
// cut into slices (work items = (job, slice, tile)) whose fp32 partials are
// summed by k_bwd_splitk_reduce.
namespace {

constexpr int WG_T = 128, WG_K = 64;

// byte offset of element k of LDS row r (rows of WG_K bf16, 16-byte chunks swizzled)
__device__ __forceinline__ int wg_off(int r, int k) {
  return r * (WG_K * 2) + ((((k >> 3) ^ ((r >> 3) & 7))) << 4) + ((k & 7) << 1);
}

__global__ __launch_bounds__(256) void k_bwd_wgrad(const Wgrad P) {
  __shared__ __attribute__((aligned(16))) char at[WG_T * WG_K * 2];  // A^T [m][k]
  __shared__ __attribute__((aligned(16))) char bt[WG_T * WG_K * 2];  // B^T [n][k]
  const int item = remap_xcd(blockIdx.x, (P.items + N_XCD - 1) / N_XCD);
  if (item >= P.items) return;
  int ji = 0;
  while (ji + 1 < P.njobs && item >= P.j[ji + 1].item_begin) ++ji;
  const WgradJob& J = P.j[ji];
  const int local = item - J.item_begin;
  // slices outermost: consecutive items are tiles of one slice, which share the
  // slice's rows of A (along a tile row) and of B
  const int sl = local / J.tiles, tile = local - sl * J.tiles;
  const int tm = tile / J.tiles_n, tn = tile - tm * J.tiles_n;
  const int m0 = tm * WG_T, n0 = tn * WG_T;
  const int k0 = sl * J.Ks, k1 = min(J.K, k0 + J.Ks);
  const bf16* A = reinterpret_cast<const bf16*>(J.A);
  const bf16* B = reinterpret_cast<const bf16*>(J.B);
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, lr = l & 15, lg = l >> 4;
  const int wm = w & 1, wn = w >> 1;
  // the thread's pieces: columns 8 g .. 8 g + 7 of the tile, positions 4 q .. 4 q + 3
  const int g = tid & 15, q = tid >> 4;
  const bool am = m0 + 8 * g < J.M, bn = n0 + 8 * g < J.N;
  const bf16* pa = A + (am ? m0 + 8 * g : 0);
  const bf16* pb = B + (bn ? n0 + 8 * g : 0);
  u32x4 ra[4], rb[4];
  auto load = [&](int kb) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int k = kb + 4 * q + r;
      const bool ok = k < k1;
      const size_t kk = ok ? k : k0;
      ra[r] = ld16(pa + kk * J.lda);
      rb[r] = ld16(pb + kk * J.ldb);
      if (!ok || !am) ra[r] = zero16();
      if (!ok || !bn) rb[r] = zero16();
    }
  };
  // element e of the four pieces, as one 8-byte run of four positions
  auto quad = [&](const u32x4 (&v)[4], int e) {
    const int wd = e >> 1, hi = e & 1;
    uint32_t h[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) h[r] = hi ? (v[r][wd] >> 16) : (v[r][wd] & 0xffffu);
    return u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
  };
  auto stage = [&]() {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      st8(at + wg_off(8 * g + e, 4 * q), quad(ra, e));
      st8(bt + wg_off(8 * g + e, 4 * q), quad(rb, e));
    }
  };
  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) acc[i][jt] = zero4();
  if (k0 < k1) load(k0);
  for (int kb = k0; kb < k1; kb += WG_K) {
    lds_barrier();  // the previous step's fragments are read
    stage();
    lds_barrier();
    if (kb + WG_K < k1) load(kb + WG_K);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      u32x4 fa[4], fb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) fa[i] = ld16(at + wg_off(64 * wm + 16 * i + lr, 32 * s + 8 * lg));
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) fb[jt] = ld16(bt + wg_off(64 * wn + 16 * jt + lr, 32 * s + 8 * lg));
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) acc[i][jt] = mma_slab<bf16>(fa[i], fb[jt], acc[i][jt]);
    }
  }
  float* C = J.C + (size_t)sl * J.M * J.N;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int m = m0 + 64 * wm + 16 * i + 4 * lg + e;
      if (m >= J.M) continue;
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) {
        const int n = n0 + 64 * wn + 16 * jt + lr;
        if (n < J.N) C[(size_t)m * J.N + n] = acc[i][jt][e];
      }
    }
}

}  // namespace

hipError_t launch_bwd_wgrad(const Wgrad& P, hipStream_t st) {
  if (P.items == 0) return hipSuccess;
  const int per = (P.items + N_XCD - 1) / N_XCD;
  hipLaunchKernelGGL(k_bwd_wgrad, dim3(per * N_XCD), dim3(256), 0, st, P);
  return hipGetLastError();
}

}  // namespace msgla
