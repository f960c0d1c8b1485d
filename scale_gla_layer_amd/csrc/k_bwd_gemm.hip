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
// both operands position-major.  A workgroup forms a 128 x 128 tile with four
// waves of 64 x 64 (4 x 4 bf16 MFMA tiles).  Each step of WG_KS positions
// copies both operands global -> LDS asynchronously, one 256-byte row per
// position (the tile's 128 columns), into one of WG_NST rotating stages,
// WG_NST - 1 steps ahead of the products, with one LDS-only barrier per step.
// The matrix cores want each lane's operand K-contiguous; the LDS transpose
// read (ds_read_b64_tr_b16) supplies that from the position-major rows: in
// each 16-lane group, lane i receives element i % 4 of the 8-byte reads of
// lanes 4 e + i / 4 (e = 0 .. 3).  So a lane that reads the four columns
// 4 q .. 4 q + 3 of position row 4 h + e of its group's eight (lane = 16 g +
// 4 e + q) hands every lane of the group one column's four consecutive
// positions, and two such reads (h = 0, 1) make the eight positions of a
// 16 x 16 x 32 operand.  The 16-byte pieces of row r sit XOR-swizzled by
// (r % 4) + 4 ((r / 8) % 4), which gives the 16 rows of one read 16 distinct
// keys: the read's 32 pieces cover each bank pair twice (the minimum).  The
// K range is cut into slices (work items = (job, slice, tile)) whose fp32
// partials are summed by k_bwd_splitk_reduce.
namespace {

constexpr int WG_T = 128;                      // output tile edge
// 32 positions per step in two stages (32 KB of LDS, three workgroups per CU at
// 131 registers): measured against 64-position steps in two stages (2 per CU)
// and 32-position steps in three or four stages, and against a cap of 128
// registers for a fourth workgroup, all slower
constexpr int WG_KS = 32;                      // positions per step
constexpr int WG_NST = 2;                      // LDS stages
constexpr int WG_ROW = WG_T * 2;               // bytes of one position row of an operand tile
constexpr int WG_OPB = WG_KS * WG_ROW;         // bytes of one operand per stage
constexpr int WG_STAGE = 2 * WG_OPB;
constexpr int WG_CP = WG_OPB / 1024 / 4;       // copy instructions per wave, operand and step
static_assert(WG_KS % 32 == 0 && WG_CP >= 1 && (WG_NST - 2) * 2 * WG_CP < 64, "weight-gradient pipeline");

__device__ __forceinline__ int wg_key(int r) { return (r & 3) | (((r >> 3) & 3) << 2); }

typedef short wg_v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) wg_v4s lds_v4s;

// 8 bf16 operand values: positions 8 g .. 8 g + 7 of the lane's column, from
// the two transpose reads at byte offsets off and off + 4 rows
__device__ __forceinline__ u32x4 wg_frag(const char* p) {
  const wg_v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(p));
  const wg_v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(p + 4 * WG_ROW));
  const u32x2 a = __builtin_bit_cast(u32x2, lo), b = __builtin_bit_cast(u32x2, hi);
  return u32x4{a[0], a[1], b[0], b[1]};
}

// zero the operand values of positions >= valid (slab-local position of value
// j: 8 g + j)
__device__ __forceinline__ u32x4 wg_mask(u32x4 v, int g, int valid) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const int k = 8 * g + 2 * w;
    const uint32_t lo = k < valid ? 0xffffu : 0u, hi = k + 1 < valid ? 0xffff0000u : 0u;
    v[w] &= lo | hi;
  }
  return v;
}

__global__ __launch_bounds__(256) void k_bwd_wgrad(const Wgrad P) {
  __shared__ __attribute__((aligned(16))) char lds[WG_NST * WG_STAGE];
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
  const char* A = reinterpret_cast<const char*>(J.A);
  const char* B = reinterpret_cast<const char*>(J.B);
  const int tid = threadIdx.x, l = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w & 1, wn = w >> 1;

  // copy slots: instruction j of this wave fills rows 4 (WG_CP w + j) .. + 3 of
  // a stage's operand block; the lane's 16 bytes land in row 4 (WG_CP w + j) +
  // l / 16, physical piece l % 16, and carry the logical piece (columns)
  // (l % 16) ^ key(row).  Pieces past the problem's columns read column 0
  // (their results are not stored).
  const int crow = 4 * WG_CP * w + (l >> 4);
  int acol[WG_CP], bcol[WG_CP];
#pragma unroll
  for (int j = 0; j < WG_CP; ++j) {
    const int lp = (l & 15) ^ wg_key(crow + 4 * j);
    const int ma = m0 + 8 * lp, nb = n0 + 8 * lp;
    acol[j] = (ma < J.M ? ma : 0) * 2;
    bcol[j] = (nb < J.N ? nb : 0) * 2;
  }
  const size_t lda = (size_t)J.lda * 2, ldb = (size_t)J.ldb * 2;
  const int nsteps = (k1 - k0 + WG_KS - 1) / WG_KS;
  // positions past the slice's end read its first row (their values are zeroed
  // after the transpose reads)
  auto issue = [&](int t) {
    char* st = lds + (t % WG_NST) * WG_STAGE;
#pragma unroll
    for (int j = 0; j < WG_CP; ++j) {
      const int k = k0 + t * WG_KS + crow + 4 * j;
      const size_t kk = k < k1 ? k : k0;
      dma16(A + kk * lda + acol[j], st + 1024 * (WG_CP * w + j));
      dma16(B + kk * ldb + bcol[j], st + WG_OPB + 1024 * (WG_CP * w + j));
    }
  };

  // transpose-read offsets: lane 16 g + 4 e + q reads columns 4 q .. 4 q + 3 of
  // 16-column tile i, position row 8 g + e (+ 4 for the second read) of a slab
  const int g = l >> 4, e = (l >> 2) & 3, q = l & 3;
  const int key = e | (g << 2);
  int offA[4], offB[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int base = (8 * g + e) * WG_ROW + 8 * (q & 1);
    offA[i] = base + 16 * (((8 * wm + 2 * i) + (q >> 1)) ^ key);
    offB[i] = WG_OPB + base + 16 * (((8 * wn + 2 * i) + (q >> 1)) ^ key);
  }

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) acc[i][jt] = zero4();

  for (int t = 0; t < WG_NST - 1 && t < nsteps; ++t) issue(t);
  for (int t = 0; t < nsteps; ++t) {
    // step t has landed once only the copies of later steps remain
    wait_stages<2 * WG_CP, WG_NST - 2>(min(WG_NST - 2, nsteps - 1 - t));
    lds_barrier();
    if (t + WG_NST - 1 < nsteps) issue(t + WG_NST - 1);
    const char* st = lds + (t % WG_NST) * WG_STAGE;
    const int valid = k1 - k0 - t * WG_KS;  // positions of this step inside the slice
#pragma unroll
    for (int s = 0; s < WG_KS / 32; ++s) {
      u32x4 fa[4], fb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        fa[i] = wg_frag(st + offA[i] + 32 * s * WG_ROW);
        fb[i] = wg_frag(st + offB[i] + 32 * s * WG_ROW);
      }
      if (valid < WG_KS) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          fa[i] = wg_mask(fa[i], g, valid - 32 * s);
          fb[i] = wg_mask(fb[i], g, valid - 32 * s);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) acc[i][jt] = mma_slab<bf16>(fa[i], fb[jt], acc[i][jt]);
    }
  }
  float* C = J.C + (size_t)sl * J.M * J.N;
  const int lr = l & 15, lg = l >> 4;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = m0 + 64 * wm + 16 * i + 4 * lg + r;
      if (m >= J.M) continue;
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) {
        const int n = n0 + 64 * wn + 16 * jt + lr;
        if (n < J.N) C[(size_t)m * J.N + n] = acc[i][jt][r];
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
