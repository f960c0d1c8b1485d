// Streaming decode step (MS-GLA notes, paragraph on token-by-token inference:
// per branch the cache holds the GLA state, the pending partial block and the
// latest output; a new token is accumulated, and when s tokens have arrived
// they are pooled, the state takes one step of S = Diag(alpha) S + k^T v,
// o = q S, and the held output is replaced; the branches are fused with
// softmax weights from the unpooled token, Eqs. (10)-(11)).
//
// Four launches per token, all enqueued without host synchronisation; each
// kernel reads the token count from the state header on the device and a
// branch whose block is not complete skips its work:
//   D0 pool:   psum += x_t; on completion xp = psum / s, psum = 0;
//              plus the fusion weights of x_t (one block per sequence)
//   D1 proj:   [q | k | v | g] = xp Wp^T for completing branches (MFMA, 16 sequences x
//              16 columns per wave)
//   D2 state:  gate, state update and o = q S per (branch, sequence, head, d_v tile)
//   D3 out:    held = o W_o for completing branches (MFMA as D1), out = sum_i w_i
//              held_i, header position + 1
#include "device_common.hpp"
#include "layout.hpp"

namespace msgla {

constexpr int DEC_THREADS = 256;

__device__ __forceinline__ int64_t dec_pos(const void* state) {
  return reinterpret_cast<const StateHeader*>(state)->pos;
}
__device__ __forceinline__ bool completes(int64_t pos, int s) { return ((pos + 1) % s) == 0; }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, WAVE);
  return v;
}

// grid (ceil(d/256), B, m + 1): z == m computes the fusion weights of sequence y
template <typename T>
__global__ __launch_bounds__(DEC_THREADS) void k_dec_pool(const DecParams P) {
  const int b = blockIdx.y, i = blockIdx.z;
  const int64_t pos = dec_pos(P.state);
  const T* x = reinterpret_cast<const T*>(P.x) + (size_t)b * P.d;
  if (i < P.nbranch) {
    const DecBranch& Br = P.br[i];
    const int col = blockIdx.x * DEC_THREADS + threadIdx.x;
    if (col < P.d) {
      const float ps = Br.psum[(size_t)b * P.d + col] + to_f32(x[col]);
      if (completes(pos, Br.s)) {
        Br.xp[(size_t)b * P.d + col] = ps / (float)Br.s;
        Br.psum[(size_t)b * P.d + col] = 0.f;
      } else {
        Br.psum[(size_t)b * P.d + col] = ps;
      }
    }
    if (blockIdx.x == 0 && b == 0 && i == 0 && threadIdx.x == 0) *P.pos_ws = pos;
    return;
  }
  if (blockIdx.x != 0) return;
  // fusion weights of this token (Eq. (10)); m == 1 -> weight 1
  __shared__ float red[DEC_THREADS / WAVE][FUSION_STRIDE];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const T* wz = reinterpret_cast<const T*>(P.Wz);
  float z[FUSION_STRIDE];
  for (int e = 0; e < P.m; ++e) {
    float acc = 0.f;
    if (P.m > 1)
      for (int c = threadIdx.x; c < P.d; c += DEC_THREADS) acc += to_f32(x[c]) * to_f32(wz[(size_t)e * P.d + c]);
    acc = wave_sum(acc);
    if (lane == 0) red[wave][e] = acc;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float mx = -INFINITY, sum = 0.f;
    for (int e = 0; e < P.m; ++e) {
      z[e] = red[0][e] + red[1][e] + red[2][e] + red[3][e] + P.bf[e];
      mx = fmaxf(mx, z[e]);
    }
    for (int e = 0; e < P.m; ++e) {
      z[e] = __expf(z[e] - mx);
      sum += z[e];
    }
    for (int e = 0; e < FUSION_STRIDE; ++e) P.w[(size_t)b * FUSION_STRIDE + e] = (e < P.m) ? z[e] / sum : 0.f;
  }
}

// Batched row-times-matrix products of the step as MFMA tiles: the (up to)
// 16 sequences of a batch tile are the 16 rows of the A operand, 16 weight
// rows the B operand, and K runs in 64-byte k-slabs (one MFMA each), so a
// wave forms 16 x 16 outputs and every weight is read once per batch tile.
// A-operand rows come from fp32 vectors rounded to the storage type, as the
// forward rounds its pooled rows and its y.  The slabs of a wave's K range
// are loaded NS at a time before any is used (a decode step is latency-bound).
template <typename T>
__device__ __forceinline__ f32x4 dec_rows_times_cols(const float* xrow, bool xok, const T* wrow, int K,
                                                     f32x4 acc) {
  constexpr int PER = per16<T>(), SLAB = 4 * PER, NS = 8;
  for (int k0 = 0; k0 < K; k0 += NS * SLAB) {
    u32x4 wf[NS], xf[NS * PER / 4];
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      const bool in = k0 + u * SLAB < K;
      wf[u] = in ? ld16(wrow + k0 + u * SLAB) : zero16();
#pragma unroll
      for (int q = 0; q < PER / 4; ++q)
        xf[u * (PER / 4) + q] = in && xok ? ld16(xrow + k0 + u * SLAB + 4 * q) : zero16();
    }
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      float xv[PER];
#pragma unroll
      for (int q = 0; q < PER / 4; ++q) unpack16<float>(xf[u * (PER / 4) + q], xv + 4 * q);
      acc = mma_slab<T>(pack16<T>(xv), wf[u], acc);
    }
  }
  return acc;
}

// Sum of the four waves' 16 x 16 partial tiles through LDS; wave 0 returns it.
__device__ __forceinline__ f32x4 dec_reduce4(f32x4 acc, float* red, int wave, int lane) {
  if (wave > 0) {
    const float t[4] = {acc[0], acc[1], acc[2], acc[3]};
    st16(red + ((wave - 1) * 64 + lane) * 4, pack16<float>(t));
  }
  __syncthreads();
  if (wave == 0)
#pragma unroll
    for (int w = 0; w < 3; ++w) {
      float t[4];
      unpack16<float>(ld16(red + (w * 64 + lane) * 4), t);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] += t[e];
    }
  return acc;
}

// grid (ceil(Nmax / 16), m, ceil(B / 16)): projection columns 16 x .. 16 x + 15
// for sequences 16 z .. 16 z + 15; the four waves take a quarter of K each
template <typename T>
__global__ __launch_bounds__(DEC_THREADS) void k_dec_proj(const DecParams P) {
  const DecBranch& Br = P.br[blockIdx.y];
  if (!completes(dec_pos(P.state), Br.s)) return;
  __shared__ __attribute__((aligned(16))) float red[3 * 64 * 4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int n0 = blockIdx.x * 16, b0 = blockIdx.z * 16;
  if (n0 >= Br.N) return;
  constexpr int PER = per16<T>(), SLAB = 4 * PER;
  const int n = min(n0 + lr, Br.N - 1), b = b0 + lr;  // B-operand row, A-operand row
  // wave w: k-slabs [w nsl / 4, (w + 1) nsl / 4) of the nsl = d / SLAB
  const int nsl = P.d / SLAB, k_lo = wave * nsl / 4 * SLAB, k_hi = (wave + 1) * nsl / 4 * SLAB;
  const T* wrow = reinterpret_cast<const T*>(Br.Wp) + (size_t)n * P.d + k_lo + PER * lg;
  const float* xrow = Br.xp + (size_t)(b < P.B ? b : 0) * P.d + k_lo + PER * lg;
  f32x4 acc = dec_rows_times_cols<T>(xrow, b < P.B, wrow, k_hi - k_lo, zero4());
  acc = dec_reduce4(acc, red, wave, lane);
  if (wave != 0) return;
  // acc[e]: sequence b0 + 4 lg + e, column n0 + lr
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int bb = b0 + 4 * lg + e;
    if (bb < P.B && n0 + lr < Br.N) Br.proj[(size_t)bb * Br.N + n0 + lr] = acc[e];
  }
}

// grid (B * hmax, ceil(dv / 64), m); 256 threads: lane -> v column, wave -> quarter of d_k
__global__ __launch_bounds__(DEC_THREADS) void k_dec_state(const DecParams P) {
  const DecBranch& Br = P.br[blockIdx.z];
  if (!completes(dec_pos(P.state), Br.s)) return;
  const int bh = blockIdx.x;
  if (bh >= P.B * Br.h) return;
  const int b = bh / Br.h, hh = bh - b * Br.h;
  extern __shared__ float sh[];
  float* alpha = sh;             // [dk]
  float* kk = sh + P.dk;         // [dk]
  float* qq = sh + 2 * P.dk;     // [dk]
  float* part = sh + 3 * P.dk;   // [4][64]
  const float* pr = Br.proj + (size_t)b * Br.N;
  for (int c = threadIdx.x; c < P.dk; c += DEC_THREADS) {
    float z = Br.bg[hh * P.dk + c];
    for (int r = 0; r < P.r; ++r) z = fmaf(pr[Br.col_g + r], Br.W2[(size_t)r * Br.h * P.dk + hh * P.dk + c], z);
    alpha[c] = __expf(logsigmoid_f(z) * P.inv_gamma);
    kk[c] = pr[Br.col_k + hh * P.dk + c];
    qq[c] = pr[hh * P.dk + c] * P.q_scale;
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int v = blockIdx.y * 64 + lane;
  float acc = 0.f;
  if (v < P.dv) {
    const float vv = pr[Br.col_v + hh * P.dv + v];
    float* S = Br.S + (size_t)bh * P.dk * P.dv;
    const int cq = (P.dk + 3) / 4;
    for (int c = wave * cq; c < min(P.dk, (wave + 1) * cq); ++c) {
      const float s = fmaf(alpha[c], S[(size_t)c * P.dv + v], kk[c] * vv);
      S[(size_t)c * P.dv + v] = s;
      acc = fmaf(qq[c], s, acc);
    }
  }
  part[wave * 64 + lane] = acc;
  __syncthreads();
  if (wave == 0 && v < P.dv)
    Br.y[(size_t)b * Br.h * P.dv + hh * P.dv + v] = part[lane] + part[64 + lane] + part[128 + lane] + part[192 + lane];
}

// grid (d / 16, ceil(B / 16)): output columns 16 x .. 16 x + 15 for sequences
// 16 y .. 16 y + 15.  Wave w takes branches w, w + 4, ...: a completing branch
// replaces its held output by y W_o (MFMA over K = h d_v), the others keep
// theirs; the waves' weighted sums meet in LDS and out = sum_i w_i held_i.
template <typename T>
__global__ __launch_bounds__(DEC_THREADS) void k_dec_out(const DecParams P) {
  __shared__ __attribute__((aligned(16))) float red[3 * 64 * 4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int n0 = blockIdx.x * 16, b0 = blockIdx.y * 16;
  const int64_t pos = *P.pos_ws;
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0)
    reinterpret_cast<StateHeader*>(P.state)->pos = pos + 1;
  constexpr int PER = per16<T>();
  const int n = n0 + lr;  // d is a multiple of 64
  f32x4 o = zero4();
  for (int i = wave; i < P.nbranch; i += 4) {
    const DecBranch& Br = P.br[i];
    float held[4];
    if (completes(pos, Br.s)) {
      const int K = Br.h * P.dv, b = b0 + lr;
      const T* wrow = reinterpret_cast<const T*>(P.WoT) + (size_t)n * P.Ktot + Br.ko + PER * lg;
      const float* yrow = Br.y + (size_t)(b < P.B ? b : 0) * K + PER * lg;
      const f32x4 acc = dec_rows_times_cols<T>(yrow, b < P.B, wrow, K, zero4());
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        held[e] = acc[e];
        const int bb = b0 + 4 * lg + e;
        if (bb < P.B) Br.held[(size_t)bb * P.d + n] = held[e];
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int bb = b0 + 4 * lg + e;
        held[e] = bb < P.B ? Br.held[(size_t)bb * P.d + n] : 0.f;
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int bb = b0 + 4 * lg + e;
      o[e] += (P.m > 1 && bb < P.B ? P.w[(size_t)bb * FUSION_STRIDE + i] : 1.f) * held[e];
    }
  }
  o = dec_reduce4(o, red, wave, lane);
  if (wave != 0) return;
  T* out = reinterpret_cast<T*>(P.out);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int bb = b0 + 4 * lg + e;
    if (bb < P.B) out[(size_t)bb * P.d + n] = from_f32<T>(o[e]);
  }
}

hipError_t launch_decode(const DecParams& P, int Nmax, int hmax, bool bf16_path, hipStream_t st) {
  const dim3 blk(DEC_THREADS);
  const dim3 g0((P.d + DEC_THREADS - 1) / DEC_THREADS, P.B, P.nbranch + 1);
  const int btiles = (P.B + 15) / 16;
  const dim3 g1((Nmax + 15) / 16, P.nbranch, btiles);
  const dim3 g2(P.B * hmax, (P.dv + 63) / 64, P.nbranch);
  const dim3 g3(P.d / 16, btiles);
  const size_t lds2 = (size_t)(3 * P.dk + 4 * 64) * sizeof(float);
  if (bf16_path) {
    hipLaunchKernelGGL(k_dec_pool<bf16>, g0, blk, 0, st, P);
    hipLaunchKernelGGL(k_dec_proj<bf16>, g1, blk, 0, st, P);
  } else {
    hipLaunchKernelGGL(k_dec_pool<float>, g0, blk, 0, st, P);
    hipLaunchKernelGGL(k_dec_proj<float>, g1, blk, 0, st, P);
  }
  hipLaunchKernelGGL(k_dec_state, g2, blk, lds2, st, P);
  if (bf16_path)
    hipLaunchKernelGGL(k_dec_out<bf16>, g3, blk, 0, st, P);
  else
    hipLaunchKernelGGL(k_dec_out<float>, g3, blk, 0, st, P);
  return hipGetLastError();
}

}  // namespace msgla
