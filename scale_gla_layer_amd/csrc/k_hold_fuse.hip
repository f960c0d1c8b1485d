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
// with j_i(t) = floor((t+1)/s_i) - 1 (a zero row when negative).  The A rows are
// gathered straight from the held coarse rows by the asynchronous copies of
// gemm_dma.hpp (a per-row source address; zeros come from a zero block), B is
// the stacked W_o^T.  Each 128-byte K segment lies inside one head of one
// branch, so the fusion weight is applied once per branch instead of per
// element: the accumulators of branch i are folded into the total as
// total += w_{t,i} * acc at the branch's last K segment.  The epilogue writes O
// row-major.
#include "device_common.hpp"
#include "gemm_dma.hpp"
#include "layout.hpp"

namespace msgla {

using K3Cfg = GemmCfg<4, 4, 2, 2, 128, 2>;  // 128 x 128 tiles, 4 waves, double-buffered 128-byte K segments
constexpr int K3_WM = K3Cfg::WM, K3_WN = K3Cfg::WN;
constexpr int K3_BM = K3Cfg::BM, K3_BN = K3Cfg::BN;
// the tile's fusion weights [BM][FUSION_STRIDE] fp32 live in LDS after the stages
constexpr int K3_W_OFF = K3Cfg::LDS;
constexpr int K3_LDS = K3Cfg::LDS_STAGED > K3_W_OFF + K3_BM * FUSION_STRIDE * 4
                           ? K3Cfg::LDS_STAGED
                           : K3_W_OFF + K3_BM * FUSION_STRIDE * 4;
static_assert(K3_BM * FUSION_STRIDE * 4 == K3Cfg::THREADS * 16, "one 16-byte piece per thread");

template <typename T>
struct K3Prob {
  const K3Params& P;
  int m0, n0;
  int rb[K3Cfg::A_SLOTS], rt[K3Cfg::A_SLOTS];  // sequence / position of the lane's copy rows (-1: none)
  const char* brow[K3Cfg::B_SLOTS];
  const char* arow[K3Cfg::A_SLOTS];            // row base of the branch currently being copied
  int ib_issue = -1;           // branch of the K segments being copied
  int ib_fold = 0;             // branch of the K segments being multiplied
  f32x4 total[K3_WM][K3_WN];
  const float* wl = nullptr;   // LDS copy of the tile's fusion weights

  __device__ K3Prob(const K3Params& p, int m0_, int n0_) : P(p), m0(m0_), n0(n0_) {}

  __device__ int nk() const { return P.Ktot * (int)sizeof(T) / K3Cfg::KSEG; }
  __device__ int seg_begin(int i) const { return P.br[i].ko * (int)sizeof(T) / K3Cfg::KSEG; }
  __device__ int branch_of(int kt) const {
    int bi = 0;
    while (bi + 1 < P.m && kt >= seg_begin(bi + 1)) ++bi;
    return bi;
  }
  __device__ void setup(int wave, int lane) {
#pragma unroll
    for (int j = 0; j < K3Cfg::A_SLOTS; ++j) {
      const int m = m0 + K3Cfg::a_row(j, wave, lane);
      rb[j] = (m < P.B * P.L) ? m / P.L : -1;
      rt[j] = (m < P.B * P.L) ? m - rb[j] * P.L : 0;
    }
#pragma unroll
    for (int j = 0; j < K3Cfg::B_SLOTS; ++j) {
      const int n = n0 + K3Cfg::b_row(j, wave, lane);
      brow[j] = reinterpret_cast<const char*>(P.WoT) + (size_t)(n < P.d ? n : 0) * P.Ktot * sizeof(T);
    }
    if (P.m > 1) {
#pragma unroll
      for (int a = 0; a < K3_WM; ++a)
#pragma unroll
        for (int b = 0; b < K3_WN; ++b) total[a][b] = zero4();
    }
  }
  // stage the tile's fusion weights (consumed by fold, which runs after at
  // least one LDS barrier of the K loop; the final staging of the output
  // overwrites them only after the last fold)
  __device__ void started(char* lds) {
    float* w = reinterpret_cast<float*>(lds + K3_W_OFF);
    if (P.m > 1) {
      const int tid = threadIdx.x;
      const int r = tid / (FUSION_STRIDE / 4), m = m0 + r;
      st16(w + 4 * tid, m < P.B * P.L ? ld16(P.w + (size_t)m * FUSION_STRIDE + 4 * (tid % (FUSION_STRIDE / 4)))
                                       : zero16());
    }
    wl = w;
  }
  // held coarse row of each copy row for branch bi (zero block before the first block)
  __device__ void enter_branch(int bi) {
    const K3Branch& Br = P.br[bi];
#pragma unroll
    for (int j = 0; j < K3Cfg::A_SLOTS; ++j) {
      const int jr = (rt[j] + 1) / Br.s - 1;
      arow[j] = (rb[j] < 0 || jr < 0)
                    ? nullptr
                    : reinterpret_cast<const char*>(Br.y) +
                          ((size_t)rb[j] * Br.h * Br.np + jr) * P.dv * sizeof(T);
    }
    ib_issue = bi;
  }
  // per copied segment: branch (switching the held rows when it changes) and the
  // byte offset of the segment inside a held row of that branch
  size_t seg_off = 0;
  __device__ void prep(int kt) {
    const int bi = branch_of(kt);
    if (bi != ib_issue) enter_branch(bi);
    const int head_bytes = P.dv * (int)sizeof(T);
    const int kb = (kt - seg_begin(bi)) * K3Cfg::KSEG;  // bytes into the branch's K range
    const int hh = kb / head_bytes;             // head of this segment
    seg_off = (size_t)hh * P.br[bi].np * head_bytes + (kb - hh * head_bytes);
  }
  __device__ const char* a_row(int j, int) const {
    return arow[j] ? arow[j] + seg_off : reinterpret_cast<const char*>(P.zero);
  }
  __device__ const char* b_row(int j, int kt) const { return brow[j] + kt * K3Cfg::KSEG; }
  __device__ bool seg_end(int kt) const {
    return P.m > 1 && (ib_fold + 1 >= P.m ? kt + 1 == nk() : kt + 1 == seg_begin(ib_fold + 1));
  }
  // total += w_{row, branch} * acc for the 16 rows this lane holds; acc = 0
  __device__ void fold(f32x4 (&acc)[K3_WM][K3_WN], int wr, int wc, int lane) {
    const int lgrp = lane >> 4;
#pragma unroll
    for (int a = 0; a < K3_WM; ++a)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float w = wl[(wr * 16 * K3_WM + 16 * a + 4 * lgrp + e) * FUSION_STRIDE + ib_fold];
#pragma unroll
        for (int b = 0; b < K3_WN; ++b) {
          total[a][b][e] += w * acc[a][b][e];
          acc[a][b][e] = 0.f;
        }
      }
    ++ib_fold;
    (void)wc;
  }
  __device__ void finish(f32x4 (&acc)[K3_WM][K3_WN], int, int, int) {
    if (P.m > 1) {
#pragma unroll
      for (int a = 0; a < K3_WM; ++a)
#pragma unroll
        for (int b = 0; b < K3_WN; ++b) acc[a][b] = total[a][b];
    }
  }
  __device__ void store(const f32x4 (&acc)[K3_WM][K3_WN], int wr, int wc, int lane, char* lds) {
    float* C = reinterpret_cast<float*>(lds);
    gd_stage_tile<K3Cfg>(acc, wr, wc, lane, C);
    lds_barrier();
    epilogue(C, K3Cfg::LDC);
  }
  __device__ void epilogue(const float* C, int ldc) {
    const int tid = threadIdx.x;
    T* out = reinterpret_cast<T*>(P.out);
    for (int it = tid; it < K3_BM * (K3_BN / 8); it += K3Cfg::THREADS) {
      const int r = it / (K3_BN / 8), cg = it % (K3_BN / 8);
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
__global__ __launch_bounds__(K3Cfg::THREADS) __attribute__((amdgpu_waves_per_eu(2))) void k3_hold_fuse(const K3Params P) {
  __shared__ __attribute__((aligned(16))) char lds[K3_LDS];
  const int tile = remap_xcd(blockIdx.x, P.per_xcd);
  if (tile >= P.total_tiles) return;
  const int tm = tile / P.tiles_n, tn = tile - tm * P.tiles_n;
  K3Prob<T> prob(P, tm * K3_BM, tn * K3_BN);
  gemm_dma_tile<T, K3Cfg>(prob, P.d - tn * K3_BN, lds);
}

hipError_t launch_k3(const K3Params& P, bool bf16_path, hipStream_t stream) {
  const dim3 grid(P.per_xcd * N_XCD), block(K3Cfg::THREADS);
  if (bf16_path)
    hipLaunchKernelGGL(k3_hold_fuse<bf16>, grid, block, 0, stream, P);
  else
    hipLaunchKernelGGL(k3_hold_fuse<float>, grid, block, 0, stream, P);
  return hipGetLastError();
}

}  // namespace msgla
