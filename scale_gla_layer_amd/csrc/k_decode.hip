// Streaming decode step (MS-GLA notes, paragraph on token-by-token inference:
// per branch the cache holds the GLA state, the pending partial block and the
// latest output; a new token is accumulated, and when s tokens have arrived
// they are pooled, the state takes one step of S = Diag(alpha) S + k^T v,
// o = q S, and the held output is replaced; the branches are fused with
// softmax weights from the unpooled token, Eqs. (10)-(11)).
//
// Three launches per token, all enqueued without host synchronisation; the
// first kernel reads the token count from the state header on the device
// (checking that the header describes this configuration and batch; otherwise
// the step changes nothing and outputs NaN), and a branch whose block is not
// complete skips its work:
//   D1 proj:   [q | k | v | g] = xp Wp^T for completing branches, where the
//              pooled row xp = (pending sum + x_t) / (pending tokens + 1) is
//              formed as the MFMA operand is loaded, plus the fusion logits x_t W_f
//              (MFMA, 16 sequences x 16 columns per block)
//   D2 state:  gate, state update and o = q S per (branch, sequence, head, d_v tile)
//   D3 out:    held = o W_o for completing branches (MFMA as D1), the fusion
//              softmax, out = sum_i w_i held_i, the pending sums and token
//              counts (reset or accumulate x_t), header position + 1
#include "device_common.hpp"
#include "layout.hpp"

namespace msgla {

constexpr int DEC_THREADS = 256;

// The step's position from the state header, or -1 when the header does not
// describe this configuration and batch or records an error: the step then
// changes nothing and its output is NaN.
__device__ __forceinline__ int64_t dec_pos(const DecParams& P) {
  const StateHeader* h = reinterpret_cast<const StateHeader*>(P.state);
  const bool ok = h->magic == STATE_MAGIC && h->version == STATE_VERSION && h->B == P.B &&
                  h->m == P.m && h->status == 0 && h->pos >= 0;
  return ok ? h->pos : -1;
}
__device__ __forceinline__ bool completes(int64_t pos, int s) { return ((pos + 1) % s) == 0; }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, WAVE);
  return v;
}

// Batched row-times-matrix products of the step as MFMA tiles: the (up to)
// 16 sequences of a batch tile are the 16 rows of the A operand, 16 weight
// rows the B operand, and K runs in 64-byte k-slabs (one MFMA each), so a
// wave forms 16 x 16 outputs and every weight is read once per batch tile.
// A-operand row k is (F ? frow[k] : 0) + (X ? trow[k] : 0), times `scale`, in
// fp32, rounded to the storage type as the forward rounds its pooled rows and
// its y.  The slabs of a wave's K range are loaded NS at a time before any is
// used (a decode step is latency-bound).
template <typename T, bool F, bool X>
__device__ __forceinline__ f32x4 dec_rows_times_cols(const float* frow, const T* trow, float scale,
                                                     bool rok, const T* wrow, int K, f32x4 acc) {
  constexpr int PER = per16<T>(), SLAB = 4 * PER, NS = 8, NF = PER / 4;
  for (int k0 = 0; k0 < K; k0 += NS * SLAB) {
    u32x4 wf[NS], ff[NS * NF], tf[NS];
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      const int k = k0 + u * SLAB;
      const bool in = k < K;
      wf[u] = in ? ld16(wrow + k) : zero16();
      if constexpr (F) {
#pragma unroll
        for (int q = 0; q < NF; ++q) ff[u * NF + q] = in && rok ? ld16(frow + k + 4 * q) : zero16();
      }
      if constexpr (X) tf[u] = in && rok ? ld16(trow + k) : zero16();
    }
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      float xv[PER];
#pragma unroll
      for (int e = 0; e < PER; ++e) xv[e] = 0.f;
      if constexpr (F) {
#pragma unroll
        for (int q = 0; q < NF; ++q) unpack16<float>(ff[u * NF + q], xv + 4 * q);
      }
      if constexpr (X) {
        float tv[PER];
        unpack16<T>(tf[u], tv);
#pragma unroll
        for (int e = 0; e < PER; ++e) xv[e] += tv[e];
      }
#pragma unroll
      for (int e = 0; e < PER; ++e) xv[e] *= scale;
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

// grid (ceil(Nmax / 16), m + 1, ceil(B / 16)): projection columns 16 x .. 16 x
// + 15 of branch y (y == m: the fusion logits) for sequences 16 z .. 16 z + 15;
// the four waves take a quarter of K each
template <typename T>
__global__ __launch_bounds__(DEC_THREADS) void k_dec_proj(const DecParams P) {
  // the header is read first but used only after the block's loads and
  // products, which do not depend on it, so its round trip overlaps theirs
  // (a block whose branch does not complete this step discards its result)
  const int64_t pos = dec_pos(P);
  const bool logits = blockIdx.y == P.nbranch;
  const DecBranch& Br = P.br[logits ? 0 : blockIdx.y];
  const int N = logits ? P.m : Br.N;
  const int n0 = blockIdx.x * 16, b0 = blockIdx.z * 16;
  const bool block0 = blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0;
  if ((logits && P.m == 1) || n0 >= N) {
    if (block0 && threadIdx.x == 0) *P.pos_ws = pos;
    return;
  }
  __shared__ __attribute__((aligned(16))) float red[3 * 64 * 4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  constexpr int PER = per16<T>(), SLAB = 4 * PER;
  const int n = min(n0 + lr, N - 1), b = b0 + lr;  // B-operand row, A-operand row
  const int bc = b < P.B ? b : 0;
  // wave w: k-slabs [w nsl / 4, (w + 1) nsl / 4) of the nsl = d / SLAB
  const int nsl = P.d / SLAB, k_lo = wave * nsl / 4 * SLAB, k_hi = (wave + 1) * nsl / 4 * SLAB;
  const T* wrow = reinterpret_cast<const T*>(logits ? P.Wz : Br.Wp) + (size_t)n * P.d + k_lo + PER * lg;
  const T* trow = reinterpret_cast<const T*>(P.x) + (size_t)bc * P.d + k_lo + PER * lg;
  f32x4 acc;
  if (logits) {
    acc = dec_rows_times_cols<T, false, true>(nullptr, trow, 1.f, b < P.B, wrow, k_hi - k_lo, zero4());
  } else {
    // the completed block: (pending sum + x_t) / its tokens (s, unless a
    // masked forward left masked positions in it; Eq. (8))
    const float* frow = Br.psum + (size_t)bc * P.d + k_lo + PER * lg;
    const float inv = 1.0f / fmaxf(1.f, Br.tok[bc] + 1.f);
    acc = dec_rows_times_cols<T, true, true>(frow, trow, inv, b < P.B, wrow, k_hi - k_lo, zero4());
  }
  if (block0 && threadIdx.x == 0) *P.pos_ws = pos;  // this step's position, for the later kernels
  if (pos < 0 || (!logits && !completes(pos, Br.s))) return;  // block-uniform
  acc = dec_reduce4(acc, red, wave, lane);
  if (wave != 0) return;
  // acc[e]: sequence b0 + 4 lg + e, column n0 + lr
  float* dst = logits ? P.w : Br.proj;
  const int ld = logits ? FUSION_STRIDE : N;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int bb = b0 + 4 * lg + e;
    if (bb < P.B && n0 + lr < N) dst[(size_t)bb * ld + n0 + lr] = acc[e];
  }
}

// grid (B * hmax, ceil(dv / 64), m); 256 threads: lane -> v column, wave -> quarter of d_k
__global__ __launch_bounds__(DEC_THREADS) void k_dec_state(const DecParams P) {
  const DecBranch& Br = P.br[blockIdx.z];
  const int bh = blockIdx.x;
  if (bh >= P.B * Br.h) return;
  // the position is read first and used after the gate, which does not
  // depend on it (a branch that does not complete discards the gate)
  const int64_t pos = *P.pos_ws;
  const int b = bh / Br.h, hh = bh - b * Br.h;
  extern __shared__ float sh[];
  float* alpha = sh;             // [dk]
  float* kk = sh + P.dk;         // [dk]
  float* qq = sh + 2 * P.dk;     // [dk]
  float* part = sh + 3 * P.dk;   // [4][64]
  const float* pr = Br.proj + (size_t)b * Br.N;
  for (int c = threadIdx.x; c < P.dk; c += DEC_THREADS) {
    float z = Br.bg[hh * P.dk + c];
    // z = b_g + g1 W_g2: the rank loop 16 terms at a time, all their loads in
    // flight before the first product (same summation order)
    const float* w2 = Br.W2 + hh * P.dk + c;
    const size_t w2s = (size_t)Br.h * P.dk;
    for (int r0 = 0; r0 < P.r; r0 += 16) {
      float pv[16], wv[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int rr = min(r0 + u, P.r - 1);
        pv[u] = pr[Br.col_g + rr];
        wv[u] = w2[(size_t)rr * w2s];
      }
#pragma unroll
      for (int u = 0; u < 16; ++u)
        if (r0 + u < P.r) z = fmaf(pv[u], wv[u], z);
    }
    alpha[c] = __expf(logsigmoid_f(z) * P.inv_gamma);
    kk[c] = pr[Br.col_k + hh * P.dk + c];
    qq[c] = pr[hh * P.dk + c] * P.q_scale;
  }
  __syncthreads();
  if (pos < 0 || !completes(pos, Br.s)) return;  // block-uniform
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int v = blockIdx.y * 64 + lane;
  float acc = 0.f;
  if (v < P.dv) {
    const float vv = pr[Br.col_v + hh * P.dv + v];
    float* S = Br.S + (size_t)bh * P.dk * P.dv + v;
    const int cq = (P.dk + 3) / 4, c1 = min(P.dk, (wave + 1) * cq);
    // rows of S 32 at a time, all 32 loads in flight before the updates
    for (int c0 = wave * cq; c0 < c1; c0 += 32) {
      float sv[32];
#pragma unroll
      for (int u = 0; u < 32; ++u) sv[u] = S[(size_t)min(c0 + u, c1 - 1) * P.dv];
#pragma unroll
      for (int u = 0; u < 32; ++u) {
        const int c = c0 + u;
        if (c < c1) {
          const float sn = fmaf(alpha[c], sv[u], kk[c] * vv);
          S[(size_t)c * P.dv] = sn;
          acc = fmaf(qq[c], sn, acc);
        }
      }
    }
  }
  part[wave * 64 + lane] = acc;
  __syncthreads();
  if (wave == 0 && v < P.dv)
    Br.y[(size_t)b * Br.h * P.dv + hh * P.dv + v] = part[lane] + part[64 + lane] + part[128 + lane] + part[192 + lane];
}

// grid (B * hmax, m), one wave: the per-head RMS normalisation of a completing
// branch's new y row (gains and eps as in the forward), before the output kernel
__global__ __launch_bounds__(64) void k_dec_norm(const DecParams P) {
  const DecBranch& Br = P.br[blockIdx.y];
  const int64_t pos = *P.pos_ws;
  if (!Br.gn || pos < 0 || !completes(pos, Br.s)) return;
  const int bh = blockIdx.x;
  if (bh >= P.B * Br.h) return;
  const int b = bh / Br.h, hh = bh - b * Br.h;
  const int lane = threadIdx.x;
  float* y = Br.y + (size_t)b * Br.h * P.dv + hh * P.dv;
  float v[8];
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int c = lane + 64 * k;
    v[k] = c < P.dv ? y[c] : 0.f;
    ss += v[k] * v[k];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
  const float rs = 1.0f / sqrtf(ss / (float)P.dv + NORM_EPS);
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int c = lane + 64 * k;
    if (c < P.dv) y[c] = v[k] * rs * Br.gn[hh * P.dv + c];
  }
}

// grid (d / 16, ceil(B / 16)): output columns 16 x .. 16 x + 15 for sequences
// 16 y .. 16 y + 15.  Wave w takes branches w, w + 4, ...: a completing branch
// replaces its held output by y W_o (MFMA over K = h d_v), the others keep
// theirs; the waves' weighted sums meet in LDS and out = sum_i w_i held_i, with
// w the softmax of the logits + b_f (Eq. (10)).  The block then moves its 16 x
// 16 entries of every branch's pending sum on (reset after a completed block,
// else + x_t), after the projection kernel has read them.
template <typename T>
__global__ __launch_bounds__(DEC_THREADS) void k_dec_out(const DecParams P) {
  __shared__ __attribute__((aligned(16))) float red[3 * 64 * 4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int n0 = blockIdx.x * 16, b0 = blockIdx.y * 16;
  const int64_t pos = *P.pos_ws;
  constexpr int PER = per16<T>();
  const int n = n0 + lr;  // d is a multiple of 64
  // fusion logits of this lane's four sequences, loaded with the position
  float zl[4][FUSION_STRIDE];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float* wr = P.w + (size_t)min(b0 + 4 * lg + e, P.B - 1) * FUSION_STRIDE;
#pragma unroll
    for (int q = 0; q < FUSION_STRIDE; q += 4) unpack16<float>(ld16(wr + q), zl[e] + q);
  }
  if (pos < 0) {  // unusable state: NaN output, nothing else changes
    if (wave == 0) {
      T* out = reinterpret_cast<T*>(P.out);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int bb = b0 + 4 * lg + e;
        if (bb < P.B) out[(size_t)bb * P.d + n] = from_f32<T>(__builtin_nanf(""));
      }
    }
    return;
  }
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0)
    reinterpret_cast<StateHeader*>(P.state)->pos = pos + 1;
  // the softmax's maximum and sum
  float zmax[4], zsum[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    zmax[e] = -INFINITY;
    zsum[e] = 0.f;
    if (P.m > 1) {
#pragma unroll
      for (int i = 0; i < FUSION_STRIDE; ++i)
        if (i < P.m) zmax[e] = fmaxf(zmax[e], zl[e][i] + P.bf[i]);
#pragma unroll
      for (int i = 0; i < FUSION_STRIDE; ++i)
        if (i < P.m) zsum[e] += __expf(zl[e][i] + P.bf[i] - zmax[e]);
    }
  }
  f32x4 o = zero4();
  for (int i = wave; i < P.nbranch; i += 4) {
    const DecBranch& Br = P.br[i];
    float held[4];
    if (completes(pos, Br.s)) {
      const int K = Br.h * P.dv, b = b0 + lr;
      const T* wrow = reinterpret_cast<const T*>(P.WoT) + (size_t)n * P.Ktot + Br.ko + PER * lg;
      const float* yrow = Br.y + (size_t)(b < P.B ? b : 0) * K + PER * lg;
      const f32x4 acc = dec_rows_times_cols<T, true, false>(yrow, nullptr, 1.f, b < P.B, wrow, K, zero4());
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
      float zi = 0.f;  // branch i's logit (register select, no dynamic index)
#pragma unroll
      for (int q = 0; q < FUSION_STRIDE; ++q) zi = q == i ? zl[e][q] : zi;
      const float wi = P.m > 1 ? __expf(zi + P.bf[i] - zmax[e]) / zsum[e] : 1.f;
      o[e] += wi * held[e];
    }
  }
  o = dec_reduce4(o, red, wave, lane);
  if (wave == 0) {
    T* out = reinterpret_cast<T*>(P.out);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int bb = b0 + 4 * lg + e;
      if (bb < P.B) out[(size_t)bb * P.d + n] = from_f32<T>(o[e]);
    }
  }
  // pending sums of this block's entries (the projection kernel has read them)
  {
    const int bb = b0 + (threadIdx.x >> 4), nn = n0 + (threadIdx.x & 15);
    if (bb < P.B) {
      const float xv = to_f32(reinterpret_cast<const T*>(P.x)[(size_t)bb * P.d + nn]);
      for (int i = 0; i < P.nbranch; ++i) {
        float* ps = P.br[i].psum + (size_t)bb * P.d + nn;
        *ps = completes(pos, P.br[i].s) ? 0.f : *ps + xv;
        if (nn == 0) {
          float* tk = P.br[i].tok + bb;
          *tk = completes(pos, P.br[i].s) ? 0.f : *tk + 1.f;
        }
      }
    }
  }
}

hipError_t launch_decode(const DecParams& P, int Nmax, int hmax, bool bf16_path, hipStream_t st) {
  const dim3 blk(DEC_THREADS);
  const int btiles = (P.B + 15) / 16;
  const int ncols = Nmax > P.m ? Nmax : P.m;
  const dim3 g1((ncols + 15) / 16, P.nbranch + 1, btiles);
  const dim3 g2(P.B * hmax, (P.dv + 63) / 64, P.nbranch);
  const dim3 g3(P.d / 16, btiles);
  const size_t lds2 = (size_t)(3 * P.dk + 4 * 64) * sizeof(float);
  if (bf16_path)
    hipLaunchKernelGGL(k_dec_proj<bf16>, g1, blk, 0, st, P);
  else
    hipLaunchKernelGGL(k_dec_proj<float>, g1, blk, 0, st, P);
  hipLaunchKernelGGL(k_dec_state, g2, blk, lds2, st, P);
  if (P.norm) hipLaunchKernelGGL(k_dec_norm, dim3(P.B * hmax, P.nbranch), dim3(64), 0, st, P);
  if (bf16_path)
    hipLaunchKernelGGL(k_dec_out<bf16>, g3, blk, 0, st, P);
  else
    hipLaunchKernelGGL(k_dec_out<float>, g3, blk, 0, st, P);
  return hipGetLastError();
}

}  // namespace msgla
