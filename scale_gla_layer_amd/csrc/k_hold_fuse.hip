// K3 — per-branch output projections, causal hold and softmax fusion.
//
// MS-GLA notes, Sec. 3.2 (each branch projects back to the common d space with
// its own output projection) and Sec. 3.3 (causal upsampling: coarse output j
// of branch s is usable from position (j+1)s-1 until block j+1 completes, zero
// before the first block; Eqs. (10)-(11): O_t = sum_i w_{t,i} Yhat^{(i)}_t).
//
// Two launches:
//  K3c  Y^{(i)} = y^{(i)} W_o^{(i)} at the coarse length for every branch with
//       s > 1 (one grouped GEMM), written in the storage type.  Projecting
//       before the hold costs 2 (BL/s) h d_v d flops instead of s times that.
//  K3f  the scale-1 branch's projection y^{(1)} W_o^{(1)} (if there is one) as
//       a GEMM whose epilogue forms
//         O_t = w_{t,1} (y^{(1)} W_o^{(1)})_t + sum_{s_i > 1} w_{t,i} Y^{(i)}_{j_i(t)},
//       j_i(t) = floor((t+1)/s_i) - 1 (the term is absent while negative), and
//       writes O row-major.  Without a scale-1 branch the GEMM part is empty.
// The A rows of both GEMMs are the per-head y rows of one coarse position,
// gathered by the asynchronous copies of gemm_dma.hpp (each K segment of
// 128 bytes lies inside one head); B is the branch's slice of the stacked
// W_o^T.
#include "device_common.hpp"
#include "gemm_dma.hpp"
#include "layout.hpp"

namespace msgla {

using K3Cfg = GemmCfg<2, 4, 4, 2, 128, 2>;  // 128 x 128 tiles, 8 waves (32 x 64 each), double-buffered 128-byte K segments
constexpr int K3_BM = K3Cfg::BM, K3_BN = K3Cfg::BN;
using K3Acc = f32x4[K3Cfg::WM][K3Cfg::WN];

// A operand: rows (b, j) of one branch's y, K = the branch's h d_v columns;
// B operand: the branch's rows of W_o^T.
template <typename T>
struct K3Rows {
  const K3Params& P;
  const K3Branch& Br;
  int m0, n0;
  const char* arow[K3Cfg::A_SLOTS];  // head-0 segment of the lane's copy rows (nullptr: zero row)
  const char* brow[K3Cfg::B_SLOTS];
  size_t seg_off = 0;

  __device__ K3Rows(const K3Params& p, const K3Branch& br, int m0_, int n0_)
      : P(p), Br(br), m0(m0_), n0(n0_) {}

  __device__ int nk() const { return Br.h * P.dv * (int)sizeof(T) / K3Cfg::KSEG; }
  // rows: (b, j) = (m / rows_per_seq, m % rows_per_seq), M = B * rows_per_seq
  __device__ void setup_rows(int wave, int lane, int rows_per_seq) {
    const int M = P.B * rows_per_seq;
#pragma unroll
    for (int j = 0; j < K3Cfg::A_SLOTS; ++j) {
      const int m = m0 + K3Cfg::a_row(j, wave, lane);
      const int b = m / rows_per_seq, r = m - b * rows_per_seq;
      arow[j] = (m < M) ? reinterpret_cast<const char*>(Br.y) +
                              ((size_t)b * Br.h * Br.np + r) * P.dv * sizeof(T)
                        : nullptr;
    }
#pragma unroll
    for (int j = 0; j < K3Cfg::B_SLOTS; ++j) {
      const int n = n0 + K3Cfg::b_row(j, wave, lane);
      brow[j] = reinterpret_cast<const char*>(P.WoT) +
                ((size_t)(n < P.d ? n : 0) * P.Ktot + Br.ko) * sizeof(T);
    }
  }
  __device__ void started(char*) {}
  // byte offset of K segment kt inside the branch's head-major y rows
  __device__ void prep(int kt) {
    const int head_bytes = P.dv * (int)sizeof(T);
    const int kb = kt * K3Cfg::KSEG;
    const int hh = kb / head_bytes;
    seg_off = (size_t)hh * Br.np * head_bytes + (kb - hh * head_bytes);
  }
  __device__ const char* a_row(int j, int) const {
    return arow[j] ? arow[j] + seg_off : reinterpret_cast<const char*>(P.zero);
  }
  __device__ const char* b_row(int j, int kt) const { return brow[j] + kt * K3Cfg::KSEG; }
  __device__ bool seg_end(int) const { return false; }
  __device__ void fold(K3Acc&, int, int, int) {}
  __device__ void finish(K3Acc&, int, int, int) {}
};

template <typename T>
__device__ __forceinline__ void k3_store8(T* dst, const float* v) {
  if constexpr (sizeof(T) == 2) {
    st16(dst, pack16<T>(v));
  } else {
    st16(dst, pack16<T>(v));
    st16(dst + 4, pack16<T>(v + 4));
  }
}

template <typename T>
__device__ __forceinline__ void k3_load8(const T* src, float* v) {
  if constexpr (sizeof(T) == 2) {
    unpack16<T>(ld16(src), v);
  } else {
    unpack16<T>(ld16(src), v);
    unpack16<T>(ld16(src + 4), v + 4);
  }
}

// ---- K3c: coarse projections, Y^{(i)} [B][n_i][d] ----
template <typename T>
struct K3Coarse : K3Rows<T> {
  using K3Rows<T>::K3Rows;
  __device__ void setup(int wave, int lane) { this->setup_rows(wave, lane, this->Br.n); }
  __device__ void store(const K3Acc& acc, int wr, int wc, int lane, char* lds) {
    float* C = reinterpret_cast<float*>(lds);
    gd_stage_tile<K3Cfg>(acc, wr, wc, lane, C);
    lds_barrier();
    const K3Params& P = this->P;
    const int M = P.B * this->Br.n;
    T* yc = reinterpret_cast<T*>(this->Br.yc);
    for (int it = threadIdx.x; it < K3_BM * (K3_BN / 8); it += K3Cfg::THREADS) {
      const int r = it / (K3_BN / 8), cg = it % (K3_BN / 8);
      const int m = this->m0 + r, col = this->n0 + cg * 8;
      if (m >= M || col >= P.d) continue;
      k3_store8(yc + (size_t)m * P.d + col, C + r * K3Cfg::LDC + cg * 8);
    }
  }
};

template <typename T>
__global__ __launch_bounds__(K3Cfg::THREADS) void k3c_coarse(const K3Params P) {
  __shared__ __attribute__((aligned(16))) char lds[K3Cfg::LDS_STAGED];
  const int tile = remap_xcd(blockIdx.x, P.c_per_xcd);
  if (tile >= P.c_total) return;
  int ci = 0;
  while (ci + 1 < P.ncoarse && tile >= P.br[P.coarse[ci + 1]].tile_begin) ++ci;
  const K3Branch& Br = P.br[P.coarse[ci]];
  const int local = tile - Br.tile_begin;
  const int tm = local / P.tiles_n, tn = local - tm * P.tiles_n;
  K3Coarse<T> prob(P, Br, tm * K3_BM, tn * K3_BN);
  gemm_dma_tile<T, K3Cfg>(prob, P.d - tn * K3_BN, lds);
}

// ---- K3f: scale-1 projection + hold + fusion -> O [B][L][d] ----
// The tile's fusion weights are staged in LDS behind the output staging area
// when the GEMM starts; the epilogue walks the tile a few row pieces at a
// time, issuing all gathered loads of the NC coarse branches for those pieces
// before using any of them.
constexpr int K3F_W_OFF = K3Cfg::LDS_STAGED;
constexpr int K3F_LDS = K3F_W_OFF + K3_BM * FUSION_STRIDE * 4;
static_assert(K3_BM * FUSION_STRIDE * 4 <= K3Cfg::THREADS * 16, "one 16-byte piece per thread");

template <typename T, int NC, bool HELD>
struct K3Fine : K3Rows<T> {
  bool has_fine;
  __device__ K3Fine(const K3Params& p, const K3Branch& br, bool fine, int m0_, int n0_)
      : K3Rows<T>(p, br, m0_, n0_), has_fine(fine) {}
  __device__ int nk() const { return has_fine ? K3Rows<T>::nk() : 0; }
  __device__ void setup(int wave, int lane) {
    if (has_fine) this->setup_rows(wave, lane, this->P.L);
  }
  __device__ void started(char* lds) {
    const K3Params& P = this->P;
    const int tid = threadIdx.x;
    if (P.m > 1 && tid < K3_BM * FUSION_STRIDE / 4) {
      const int m = this->m0 + tid / (FUSION_STRIDE / 4);
      st16(lds + K3F_W_OFF + 16 * tid,
           m < P.B * P.L ? ld16(P.w + (size_t)m * FUSION_STRIDE + 4 * (tid % (FUSION_STRIDE / 4)))
                         : zero16());
    }
  }
  __device__ void store(const K3Acc& acc, int wr, int wc, int lane, char* lds) {
    float* C = reinterpret_cast<float*>(lds);
    const float* wl = reinterpret_cast<const float*>(lds + K3F_W_OFF);
    const K3Params& P = this->P;
    T* out = reinterpret_cast<T*>(P.out);
    // pieces in flight per thread, fewer when many coarse rows are gathered per piece
    constexpr int PIECES = K3_BM * (K3_BN / 8), U = NC <= 2 ? 4 : (NC <= 4 ? 2 : 1);
    static_assert(PIECES % (U * K3Cfg::THREADS) == 0, "epilogue batches");
    constexpr int PER = per16<T>();
    constexpr int NP = 8 / PER;  // 16-byte pieces per 8 outputs
    // the first batch's gathered coarse rows are requested before the tile is
    // staged, so their latency overlaps the staging and its barrier
    int it0 = threadIdx.x;
    int r[U], col[U];
    bool ok[U], held[U][NC > 0 ? NC : 1];
    u32x4 raw[U][NC > 0 ? NC : 1][NP];
    // every lane issues all loads of a batch (pieces outside the problem and
    // positions before a branch's first block read a valid row and drop it).
    // Continuing from a state whose header failed its check, the entry outputs
    // are not read (a valid word of the packed weights stands in for them)
    // and the whole output is NaN.
    const bool entry_ok = !HELD || state_in_ok(P.chk);
    auto gather = [&](int it_first) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int it = it_first + u * K3Cfg::THREADS;
        r[u] = it / (K3_BN / 8);
        col[u] = this->n0 + (it % (K3_BN / 8)) * 8;
        const int m = this->m0 + r[u];
        ok[u] = m < P.B * P.L && col[u] < P.d;
        const int b = ok[u] ? m / P.L : 0;
        const int t = ok[u] ? m - b * P.L : 0;
        const int cc = ok[u] ? col[u] : 0;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const K3Branch& Bi = P.br[P.coarse[c]];
          // held coarse row (none before the call's first block; continuing
          // from a state, the blocks start r = entry position mod s early)
          const int j = (t + 1 + (HELD ? entry_offset(P.chk, P.coarse[c]) : 0)) / Bi.s - 1;
          held[u][c] = j >= 0;
          // a branch without a block in this call has no coarse rows: read a
          // valid word of its entry output instead (dropped)
          const T* src = !HELD || Bi.n > 0
                             ? reinterpret_cast<const T*>(Bi.yc) + ((size_t)b * Bi.n + max(j, 0)) * P.d + cc
                             : (entry_ok ? reinterpret_cast<const T*>(Bi.held_in) : reinterpret_cast<const T*>(P.WoT)) + cc;
#pragma unroll
          for (int q = 0; q < NP; ++q) raw[u][c][q] = ld16(src + q * PER);
        }
      }
    };
    gather(it0);
    if (has_fine) gd_stage_tile<K3Cfg>(acc, wr, wc, lane, C);
    lds_barrier();  // staged tile and fusion weights visible to all waves
#pragma unroll 1
    for (;;) {
      // all gathered values are in registers before the first store, so the
      // stores are not serialised behind waits for the loads
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
          for (int q = 0; q < NP; ++q) asm volatile("" : "+v"(raw[u][c][q])::"memory");
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (!ok[u]) continue;
        const float* wr_ = wl + r[u] * FUSION_STRIDE;
        float v[8];
        if (has_fine) {
          const float wf = P.m > 1 ? wr_[P.fine] : 1.f;
          const float* crow = C + r[u] * K3Cfg::LDC + (col[u] - this->n0);
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = wf * crow[e];
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = 0.f;
        }
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const K3Branch& Bi = P.br[P.coarse[c]];
          const float wi = P.m > 1 ? wr_[P.coarse[c]] : 1.f;
          float y[8];
#pragma unroll
          for (int q = 0; q < NP; ++q) unpack16<T>(held[u][c] ? raw[u][c][q] : zero16(), y + q * PER);
          if (HELD && entry_ok && !held[u][c]) {
            // before this call's first block: the output held on entry (fp32)
            const float* hp = Bi.held_in + (size_t)((this->m0 + r[u]) / P.L) * P.d + col[u];
            unpack16<float>(ld16(hp), y);
            unpack16<float>(ld16(hp + 4), y + 4);
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] += wi * y[e];
        }
        if (!entry_ok)
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = __builtin_nanf("");
        k3_store8(out + (size_t)(this->m0 + r[u]) * P.d + col[u], v);
      }
      it0 += U * K3Cfg::THREADS;
      if (it0 >= PIECES) break;
      gather(it0);
    }
  }
};

// HELD: the call continues from a state, so positions before a coarse
// branch's first block take the output that branch held on entry.
template <typename T, int NC, bool HELD>
__global__ __launch_bounds__(K3Cfg::THREADS) void k3f_fine_fuse(const K3Params P) {
  __shared__ __attribute__((aligned(16))) char lds[K3F_LDS];
  const int tile = remap_xcd(blockIdx.x, P.f_per_xcd);
  if (tile >= P.f_total) return;
  const int tm = tile / P.tiles_n, tn = tile - tm * P.tiles_n;
  const bool fine = P.fine >= 0;
  K3Fine<T, NC, HELD> prob(P, P.br[fine ? P.fine : 0], fine, tm * K3_BM, tn * K3_BN);
  gemm_dma_tile<T, K3Cfg>(prob, P.d - tn * K3_BN, lds);
}

hipError_t launch_k3c(const K3Params& P, bool bf16_path, hipStream_t stream) {
  if (P.c_total == 0) return hipSuccess;
  const dim3 grid(P.c_per_xcd * N_XCD), block(K3Cfg::THREADS);
  if (bf16_path)
    hipLaunchKernelGGL(k3c_coarse<bf16>, grid, block, 0, stream, P);
  else
    hipLaunchKernelGGL(k3c_coarse<float>, grid, block, 0, stream, P);
  return hipGetLastError();
}

template <typename T, bool HELD>
static void launch_k3f_th(const K3Params& P, dim3 grid, dim3 block, hipStream_t stream) {
  switch (P.ncoarse) {
    case 0: hipLaunchKernelGGL((k3f_fine_fuse<T, 0, HELD>), grid, block, 0, stream, P); break;
    case 1: hipLaunchKernelGGL((k3f_fine_fuse<T, 1, HELD>), grid, block, 0, stream, P); break;
    case 2: hipLaunchKernelGGL((k3f_fine_fuse<T, 2, HELD>), grid, block, 0, stream, P); break;
    case 3: hipLaunchKernelGGL((k3f_fine_fuse<T, 3, HELD>), grid, block, 0, stream, P); break;
    case 4: hipLaunchKernelGGL((k3f_fine_fuse<T, 4, HELD>), grid, block, 0, stream, P); break;
    case 5: hipLaunchKernelGGL((k3f_fine_fuse<T, 5, HELD>), grid, block, 0, stream, P); break;
    case 6: hipLaunchKernelGGL((k3f_fine_fuse<T, 6, HELD>), grid, block, 0, stream, P); break;
    case 7: hipLaunchKernelGGL((k3f_fine_fuse<T, 7, HELD>), grid, block, 0, stream, P); break;
    default: hipLaunchKernelGGL((k3f_fine_fuse<T, 8, HELD>), grid, block, 0, stream, P); break;
  }
}

template <typename T>
static void launch_k3f_t(const K3Params& P, dim3 grid, dim3 block, hipStream_t stream) {
  if (P.held_in)
    launch_k3f_th<T, true>(P, grid, block, stream);
  else
    launch_k3f_th<T, false>(P, grid, block, stream);
}

hipError_t launch_k3f(const K3Params& P, bool bf16_path, hipStream_t stream) {
  const dim3 grid(P.f_per_xcd * N_XCD), block(K3Cfg::THREADS);
  if (bf16_path)
    launch_k3f_t<bf16>(P, grid, block, stream);
  else
    launch_k3f_t<float>(P, grid, block, stream);
  return hipGetLastError();
}

}  // namespace msgla
