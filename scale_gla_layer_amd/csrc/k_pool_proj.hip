// K1 — pooled projection GEMM over all branches in one launch.
//
// MS-GLA notes, Sec. 3.1 (Eq. (8), non-overlapping mean pooling), Sec. 3.2
// (independent q, k, v and low-rank gate projections per branch) and Sec. 3.3
// (Eq. (10), fusion logits from the unpooled x_t).
//
// For branch i (scale s): C_i = P_s(X) * Wp_i^T, where row (b, j) of P_s(X) is
// the mean of X rows b*L + j*s .. + s-1 (only complete blocks): X itself for
// s = 1, otherwise the block means written by the pooling prepass (summed in
// fp32, rounded once; with a token mask and bf16 storage the q and k columns
// also take the means' rounding residuals through a second pass over K).
// Wp_i stacks the transposed q, k and v weights; the epilogue writes q, k
// head-major fp32 rows and v transposed per chunk.
// One more group, the small projection X [W_g1^(1) | ... | W_g1^(m) | W_f]
// over the unpooled rows, gives every branch's gate first factor at every
// position (by linearity mean(x) W_g1 = mean(x W_g1), so the recurrence
// kernel averages it over each block) and the fusion weights: softmax of the
// logits plus bias (Eq. (10)).  Keeping those few columns out of the branch
// groups keeps every branch tile full width.
// Both operands stream global -> LDS asynchronously (gemm_dma.hpp), so the K
// loop issues no address or conversion arithmetic.  Every XCD walks an equal
// share of every group's row tiles (the groups in the host's order), each row
// tile's column tiles one after another, so tiles that share an A tile share
// an L2 and every XCD gets the same mix of work.
#include "device_common.hpp"
#include "gemm_dma.hpp"
#include "layout.hpp"

namespace msgla {

using K1Cfg = GemmCfg<2, 4, 4, 2, 128, 2>;  // 128 x 128 tiles, 8 waves (32 x 64 each), double-buffered 128-byte K segments
constexpr int K1_BM = K1Cfg::BM, K1_BN = K1Cfg::BN;

// MASKED: a token mask is given (rows of masked positions of the scale-1 group are zeroed)
template <typename T, bool MASKED>
struct K1Prob {
  const K1Params& P;
  const K1Group& G;
  int m0, n0;
  bool small;  // the small-projection group
  // Masked bf16 calls: the q / k column tiles of a pooled group run K twice,
  // first over the rounded block means, then over their residuals (the same
  // weight rows), so q and k see each mean at fp32 accuracy
  bool lo_pass;
  int nk0;     // K segments of one pass over d
  const char* arow[K1Cfg::A_SLOTS];
  const char* arow_lo[MASKED ? K1Cfg::A_SLOTS : 1];
  const char* brow[K1Cfg::B_SLOTS];

  __device__ K1Prob(const K1Params& p, const K1Group& g, int m0_, int n0_, bool small_)
      : P(p), G(g), m0(m0_), n0(n0_), small(small_) {
    nk0 = P.d * (int)sizeof(T) / K1Cfg::KSEG;
    lo_pass = MASKED && !small && G.A_lo != nullptr && n0 < G.col_v;
  }

  __device__ int nk() const { return lo_pass ? 2 * nk0 : nk0; }
  // 0 for row m of the scale-1 group at a masked position (its pooled input
  // M_t x_t of Eq. (8) is zero, so are q, k and v), else 1
  __device__ float keep(int m) const {
    if constexpr (!MASKED)
      return 1.f;
    else
      return (!small && G.s == 1) ? (P.mask[m] ? 1.f : 0.f) : 1.f;
  }
  __device__ void setup(int wave, int lane) {
    const size_t row_bytes = (size_t)P.d * sizeof(T);
#pragma unroll
    for (int j = 0; j < K1Cfg::A_SLOTS; ++j) {
      const int m = m0 + K1Cfg::a_row(j, wave, lane);
      arow[j] = reinterpret_cast<const char*>(G.A) + (size_t)(m < G.M ? m : 0) * row_bytes;
      if constexpr (MASKED)
        arow_lo[j] = lo_pass ? reinterpret_cast<const char*>(G.A_lo) + (size_t)(m < G.M ? m : 0) * row_bytes
                             : arow[j];
    }
#pragma unroll
    for (int j = 0; j < K1Cfg::B_SLOTS; ++j) {
      const int n = n0 + K1Cfg::b_row(j, wave, lane);
      if (!small) {
        brow[j] = reinterpret_cast<const char*>(G.Wp) + (size_t)(n < G.N ? n : 0) * row_bytes;
      } else {
        const char* src = reinterpret_cast<const char*>(P.sm.seg[0].W);  // columns past Ns: any row
        for (int q = 0; q < P.sm.nseg; ++q)
          if (n >= P.sm.seg[q].col0 && n < P.sm.seg[q].col0 + P.sm.seg[q].cnt)
            src = reinterpret_cast<const char*>(P.sm.seg[q].W) + (size_t)(n - P.sm.seg[q].col0) * row_bytes;
        brow[j] = src;
      }
    }
  }
  __device__ void started(char*) {}
  __device__ void prep(int) {}
  __device__ const char* a_row(int j, int kt) const {
    if constexpr (MASKED)
      if (kt >= nk0) return arow_lo[j] + (kt - nk0) * K1Cfg::KSEG;
    return arow[j] + kt * K1Cfg::KSEG;
  }
  __device__ const char* b_row(int j, int kt) const {
    if constexpr (MASKED)
      if (kt >= nk0) return brow[j] + (kt - nk0) * K1Cfg::KSEG;
    return brow[j] + kt * K1Cfg::KSEG;
  }
  __device__ bool seg_end(int) const { return false; }
  __device__ void fold(f32x4 (&)[K1Cfg::WM][K1Cfg::WN], int, int, int) {}
  __device__ void finish(f32x4 (&)[K1Cfg::WM][K1Cfg::WN], int, int, int) {}
  __device__ void store(const f32x4 (&acc)[K1Cfg::WM][K1Cfg::WN], int wr, int wc, int lane, char* lds) {
    if (!small && n0 + K1_BN <= G.col_v) {
      store_qk(acc, wr, wc, lane);
      return;
    }
    if (!small && n0 >= G.col_v && G.n % 4 == 0) {
      store_v(acc, wr, wc, lane);
      return;
    }
    float* C = reinterpret_cast<float*>(lds);
    gd_stage_tile<K1Cfg>(acc, wr, wc, lane, C);
    lds_barrier();
    if (small)
      epilogue_small(C, K1Cfg::LDC);
    else
      epilogue(C, K1Cfg::LDC);
  }

  // q / k tiles go straight from the accumulators to their head-major fp32 rows:
  // each store instruction writes 16 consecutive channels of 4 rows
  __device__ void store_qk(const f32x4 (&acc)[K1Cfg::WM][K1Cfg::WN], int wr, int wc, int lane) {
    const int lrow = lane & 15, lgrp = lane >> 4;
    float* dstc[K1Cfg::WN];
#pragma unroll
    for (int bb = 0; bb < K1Cfg::WN; ++bb) {
      const int col = n0 + wc * 16 * K1Cfg::WN + 16 * bb + lrow;
      const bool isq = col < G.col_k;
      const int c = isq ? col : col - G.col_k;
      const int hh = c / P.dk, ch = c - hh * P.dk;
      dstc[bb] = (isq ? G.q : G.k) + (size_t)hh * G.np * P.dk + ch;
    }
#pragma unroll
    for (int a = 0; a < K1Cfg::WM; ++a) {
      const int ma = m0 + wr * 16 * K1Cfg::WM + 16 * a;  // wave-uniform
      const int ba = ma / G.n, ja = ma - ba * G.n;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * lgrp + i;
        if (ma + r >= G.M) continue;
        int b = ba, j = ja + r;
        while (j >= G.n) {
          j -= G.n;
          ++b;
        }
        const size_t roff = ((size_t)b * G.h * G.np + j) * P.dk;
        const float kp = keep(ma + r);
#pragma unroll
        for (int bb = 0; bb < K1Cfg::WN; ++bb) dstc[bb][roff] = kp * acc[a][bb][i];
      }
    }
  }

  // v tiles go straight from the accumulators to vT[b][hh][chunk][v][tau]: a
  // lane's 4 consecutive rows are 4 consecutive positions of one channel, in
  // one chunk of one sequence (n and the chunk length are multiples of 4)
  __device__ void store_v(const f32x4 (&acc)[K1Cfg::WM][K1Cfg::WN], int wr, int wc, int lane) {
    const int lrow = lane & 15, lgrp = lane >> 4;
    T* vT = reinterpret_cast<T*>(G.vT);
    size_t cbase[K1Cfg::WN];
    bool cok[K1Cfg::WN];
#pragma unroll
    for (int bb = 0; bb < K1Cfg::WN; ++bb) {
      const int col = n0 + wc * 16 * K1Cfg::WN + 16 * bb + lrow;
      cok[bb] = col < G.N;
      const int cv = cok[bb] ? col - G.col_v : 0;
      const int hh = cv / P.dv, vch = cv - hh * P.dv;
      cbase[bb] = ((size_t)hh * G.nch * P.dv + vch) * P.C;
    }
#pragma unroll
    for (int a = 0; a < K1Cfg::WM; ++a) {
      const int m = m0 + wr * 16 * K1Cfg::WM + 16 * a + 4 * lgrp;
      if (m >= G.M) continue;
      const int b = m / G.n, j = m - b * G.n;
      const int chunk = j / P.C, tau = j - chunk * P.C;
      const size_t roff = (((size_t)b * G.h * G.nch + chunk) * P.dv) * P.C + tau;
      const float kp[4] = {keep(m), keep(m + 1), keep(m + 2), keep(m + 3)};
#pragma unroll
      for (int bb = 0; bb < K1Cfg::WN; ++bb) {
        if (!cok[bb]) continue;
        const float f[4] = {kp[0] * acc[a][bb][0], kp[1] * acc[a][bb][1], kp[2] * acc[a][bb][2],
                            kp[3] * acc[a][bb][3]};
        T* dst = vT + roff + cbase[bb];
        if constexpr (sizeof(T) == 2)
          st8(dst, pack8<T>(f));
        else
          st16(dst, pack16<T>(f));
      }
    }
  }

  // gate first factors (fp32 rows of rp) and fusion weights, per unpooled position m
  __device__ void epilogue_small(const float* C, int ldc) {
    const K1Small& S = P.sm;
    const int gcols = S.gm * S.rp;
    for (int it = threadIdx.x; it < K1_BM * (K1_BN / 8); it += K1Cfg::THREADS) {
      const int r = it / (K1_BN / 8), cg = it % (K1_BN / 8);
      const int m = m0 + r, col = n0 + cg * 8;
      if (m >= G.M || col >= G.N) continue;
      const float* src = C + r * ldc + cg * 8;
      if (col < gcols) {
        const int i = col / S.rp, c = col - i * S.rp;
        float* dst = S.g[i] + (size_t)m * S.rp + c;
        st16(dst, ld16(src));
        st16(dst + 4, ld16(src + 4));
      } else if (col == S.zcol) {
        // softmax over the m fusion logits of this position (Eq. (10))
        float z[8], mx = -INFINITY, sum = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          z[e] = (e < S.m) ? src[e] + S.bf[e] : -INFINITY;
          mx = fmaxf(mx, z[e]);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          z[e] = (e < S.m) ? __expf(z[e] - mx) : 0.f;
          sum += z[e];
        }
        const float inv = 1.0f / sum;
#pragma unroll
        for (int e = 0; e < 8; ++e) z[e] *= inv;
        float* dst = S.w + (size_t)m * FUSION_STRIDE;
        st16(dst, pack16<float>(z));
        st16(dst + 4, pack16<float>(z + 4));
      }
    }
  }

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
    // (1) row-major destinations: q, k
    for (int it = tid; it < K1_BM * (K1_BN / 8); it += K1Cfg::THREADS) {
      const int r = it / (K1_BN / 8), cg = it % (K1_BN / 8);
      const int m = m0 + r, col = n0 + cg * 8;
      if (m >= G.M || col >= G.col_v) continue;  // v: transposed pass below
      const int b = m / G.n, j = m - b * G.n;
      const float kp = keep(m);
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = kp * C[r * ldc + cg * 8 + e];
      const bool isq = col < G.col_k;
      const int c = isq ? col : col - G.col_k;
      const int hh = c / P.dk, ch = c - hh * P.dk;
      float* dst = (isq ? G.q : G.k) + (((size_t)b * G.h + hh) * G.np + j) * P.dk + ch;
      st16(dst, pack16<float>(v));
      st16(dst + 4, pack16<float>(v + 4));
    }
    // (2) v, written transposed per chunk: vT[b][hh][chunk][v][tau]
    if (n0 + K1_BN > G.col_v) {
      for (int it = tid; it < K1_BN * (K1_BM / 8); it += K1Cfg::THREADS) {
        const int cl = it % K1_BN, rg = it / K1_BN;
        const int col = n0 + cl;
        if (col < G.col_v || col >= G.N) continue;
        const int cv = col - G.col_v;
        const int hh = cv / P.dv, vch = cv - hh * P.dv;
        const int mA = m0 + rg * 8;
        if (mA >= G.M) continue;
        const int b0 = mA / G.n, j0 = mA - b0 * G.n;
        T* vT = reinterpret_cast<T*>(G.vT);
        if (mA + 7 < G.M && j0 + 7 < G.n && (j0 & 7) == 0) {
          float v[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = keep(mA + e) * C[(rg * 8 + e) * ldc + cl];
          const int chunk = j0 / P.C, tau = j0 - chunk * P.C;
          store8(vT + ((((size_t)b0 * G.h + hh) * G.nch + chunk) * P.dv + vch) * P.C + tau, v);
        } else {
          for (int e = 0; e < 8; ++e) {
            const int m = mA + e;
            if (m >= G.M) break;
            const int b = m / G.n, j = m - b * G.n;
            const int chunk = j / P.C, tau = j - chunk * P.C;
            vT[((((size_t)b * G.h + hh) * G.nch + chunk) * P.dv + vch) * P.C + tau] =
                from_f32<T>(keep(m) * C[(rg * 8 + e) * ldc + cl]);
          }
        }
      }
    }
  }
};

template <typename T, bool MASKED>
__global__ __launch_bounds__(K1Cfg::THREADS) void k1_pool_proj(const K1Params P) {
  __shared__ __attribute__((aligned(16))) char lds[K1Cfg::LDS_STAGED];
  // consecutive workgroups go to the eight XCDs in turn: this one is the j-th
  // of XCD x, which walks its share of every group's row tiles in group order
  const int x = blockIdx.x % N_XCD;
  int j = blockIdx.x / N_XCD, gi = -1, tm = 0, tn = 0;
  for (int o = 0; o < P.ngroups; ++o) {
    const int g = P.order[o];
    const int cnt = (P.mt_begin[g][x + 1] - P.mt_begin[g][x]) * P.g[g].tiles_n;
    if (j < cnt) {
      gi = g;
      tm = P.mt_begin[g][x] + j / P.g[g].tiles_n;
      tn = j % P.g[g].tiles_n;
      break;
    }
    j -= cnt;
  }
  if (gi < 0) return;
  const K1Group& G = P.g[gi];
  K1Prob<T, MASKED> prob(P, G, tm * K1_BM, tn * K1_BN, gi == P.sm.group);
  gemm_dma_tile<T, K1Cfg>(prob, G.N - tn * K1_BN, lds);
}

hipError_t launch_k1(const K1Params& P, bool bf16_path, hipStream_t stream) {
  const dim3 grid(P.per_xcd * N_XCD), block(K1Cfg::THREADS);
  if (bf16_path)
    hipLaunchKernelGGL((P.mask ? k1_pool_proj<bf16, true> : k1_pool_proj<bf16, false>), grid, block, 0, stream, P);
  else
    hipLaunchKernelGGL((P.mask ? k1_pool_proj<float, true> : k1_pool_proj<float, false>), grid, block, 0, stream, P);
  return hipGetLastError();
}

}  // namespace msgla
