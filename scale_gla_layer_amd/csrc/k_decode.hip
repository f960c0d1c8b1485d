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
//   D1 proj:   [q | k | v | g] = xp Wp^T for completing branches (one wave per column)
//   D2 state:  gate, state update and o = q S per (branch, sequence, head, d_v tile)
//   D3 out:    held = o W_o for completing branches, out = sum_i w_i held_i,
//              header position + 1
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

// grid (ceil(Nmax / 4), m): each wave computes one projection column for all B
template <typename T>
__global__ __launch_bounds__(DEC_THREADS) void k_dec_proj(const DecParams P) {
  const DecBranch& Br = P.br[blockIdx.y];
  if (!completes(dec_pos(P.state), Br.s)) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = blockIdx.x * 4 + wave;
  if (n >= Br.N) return;
  const T* w = reinterpret_cast<const T*>(Br.Wp) + (size_t)n * P.d;
  for (int b = 0; b < P.B; ++b) {
    const float* xp = Br.xp + (size_t)b * P.d;
    float acc = 0.f;
    for (int c = lane; c < P.d; c += WAVE) acc = fmaf(xp[c], to_f32(w[c]), acc);
    acc = wave_sum(acc);
    if (lane == 0) Br.proj[(size_t)b * Br.N + n] = acc;
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

// grid (ceil(d / 4)); each wave produces one output column for all B
template <typename T>
__global__ __launch_bounds__(DEC_THREADS) void k_dec_out(const DecParams P) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = blockIdx.x * 4 + wave;
  const int64_t pos = *P.pos_ws;
  if (blockIdx.x == 0 && threadIdx.x == 0) reinterpret_cast<StateHeader*>(P.state)->pos = pos + 1;
  if (n >= P.d) return;
  const T* wo = reinterpret_cast<const T*>(P.WoT) + (size_t)n * P.Ktot;
  T* out = reinterpret_cast<T*>(P.out);
  for (int b = 0; b < P.B; ++b) {
    float o = 0.f;
    for (int i = 0; i < P.nbranch; ++i) {
      const DecBranch& Br = P.br[i];
      float held;
      if (completes(pos, Br.s)) {
        const int K = Br.h * P.dv;
        const float* y = Br.y + (size_t)b * K;
        float acc = 0.f;
        for (int k = lane; k < K; k += WAVE) acc = fmaf(y[k], to_f32(wo[Br.ko + k]), acc);
        held = wave_sum(acc);
        if (lane == 0) Br.held[(size_t)b * P.d + n] = held;
      } else {
        held = Br.held[(size_t)b * P.d + n];
      }
      o += (P.m > 1 ? P.w[(size_t)b * FUSION_STRIDE + i] : 1.f) * held;
    }
    if (lane == 0) out[(size_t)b * P.d + n] = from_f32<T>(o);
  }
}

hipError_t launch_decode(const DecParams& P, int Nmax, int hmax, bool bf16_path, hipStream_t st) {
  const dim3 blk(DEC_THREADS);
  const dim3 g0((P.d + DEC_THREADS - 1) / DEC_THREADS, P.B, P.nbranch + 1);
  const dim3 g1((Nmax + 3) / 4, P.nbranch);
  const dim3 g2(P.B * hmax, (P.dv + 63) / 64, P.nbranch);
  const dim3 g3((P.d + 3) / 4);
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
