// Layer backward (training): the vector-Jacobian product of the forward.
//
// MS-GLA notes, Sec. 3.4 (training paragraph: every branch is trained with
// GLA's chunkwise-parallel algorithm) and Sec. 5.5, Table 4 (training
// throughput).  For loss gradients dO of the layer output, the chain rule
// through the forward's steps in reverse:
//
//  fusion and hold (Sec. 3.3, Eqs. (10)-(11)), O_t = sum_i w_{t,i} Yhat^(i)_t:
//    dw_{t,i} = dO_t . Yhat^(i)_t,  dz_t = w_t * (dw_t - sum_i w_{t,i} dw_{t,i}),
//    dY^(i)_j = sum of w_{t,i} dO_t over the positions t that hold block j
//    (t = (j+1)s - 1 .. (j+2)s - 2); the scale-1 branch's dO W_o^T is scaled
//    by w_{t,1} (k_bwd_out, k_bwd_hold);
//  the recurrence (Sec. 2.1), S_t = Diag(alpha_t) S_{t-1} + k_t^T v_t,
//  o_t = q_t S_t, per chunk of C positions with b_t the chunk-local cumulative
//  log alpha (all factors exp(b_t - b_i), t >= i, are <= 1):
//    S_prev of every chunk by a forward scan of the chunks' k-hat^T V,
//    dS_end (what the loss receives through a chunk's last state from later
//    chunks) by a reverse scan of q-tilde^T dO            (k_bwd_outer, k_bwd_scan)
//    A_ti = sum_c q_tc k_ic e^{b_tc - b_ic},  D_ti = do_t . v_i   (t >= i)   (k_bwd_AD)
//    dv_i = sum_{t>=i} A_ti do_t + (k_i * e^{b_last - b_i}) dS_end         (k_bwd_dv)
//    dq_t = e^{b_t} * (do_t S_prev^T) + sum_{i<=t} D_ti k_i * e^{b_t - b_i}
//    dk_i = e^{b_last - b_i} * (v_i dS_end^T) + sum_{t>=i} D_ti q_t * e^{b_t - b_i}
//                                                                      (k_bwd_dqdk)
//    and, from a zero initial state, dlog alpha_u = sum_{t>=u} (q_t dq_t - k_t dk_t)
//    per channel: in-chunk suffix sums plus the totals of later chunks;
//  the gate (Sec. 2.1), log alpha = logsigmoid(z) / gamma, z = g1 W_g2 + b_g:
//    dz = dlog alpha sigmoid(-z) / gamma, dg1 = dz W_g2^T        (k_bwd_dzg, k_bwd_dg1);
//  the pooling (Sec. 3.1, Eq. (8)): dx_t += dxp_j / s for t in complete block j,
//  plus the fusion logits' dz_t W_f^T                                   (k_bwd_dx).
// The plain products around these (dY W_o^T, the weight gradients and the
// pooled inputs' gradient) are left to the host's GEMM calls.
#include "device_common.hpp"
#include "layout.hpp"

namespace msgla {

namespace {

struct UnitPos {
  int bi, b, head, ch, sq;  // branch, batch row, head, chunk, (b, head) sequence
};

__device__ __forceinline__ UnitPos unit_pos(const BwdParams& P, int unit) {
  int bi = 0;
  while (bi + 1 < P.nbranch && unit >= P.br[bi + 1].unit_begin) ++bi;
  const BwdBranch& Br = P.br[bi];
  const int local = unit - Br.unit_begin;
  UnitPos u;
  u.bi = bi;
  u.sq = local / Br.nch;
  u.ch = local - u.sq * Br.nch;
  u.b = u.sq / Br.h;
  u.head = u.sq - u.b * Br.h;
  return u;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, WAVE);
  return v;
}

template <typename T>
__device__ __forceinline__ void load8(const T* p, float* v) {
  if constexpr (sizeof(T) == 2) {
    unpack16<T>(ld16(p), v);
  } else {
    unpack16<T>(ld16(p), v);
    unpack16<T>(ld16(p + 4), v + 4);
  }
}

template <typename T>
__device__ __forceinline__ void store8(T* p, const float* v) {
  if constexpr (sizeof(T) == 2) {
    st16(p, pack16<T>(v));
  } else {
    st16(p, pack16<T>(v));
    st16(p + 4, pack16<T>(v + 4));
  }
}

// Stages a ROWS x COLS fp32 tile into LDS: element (row, col) = f(row, col)
// goes to lds[row * LS + col] (TR: lds[col * LS + row]).  Threads take
// consecutive columns (COL_FAST) or consecutive rows, whichever keeps the
// source reads coalesced.  Every load of a thread is issued before its LDS
// stores, so a staging pass costs one memory round trip; f must load
// unconditionally (from a clamped address) and select the value afterwards.
template <int ROWS, int COLS, int LS, bool COL_FAST, bool TR, class F>
__device__ __forceinline__ void stage(float* lds, F&& f) {
  static_assert((ROWS * COLS) % 256 == 0, "whole rounds of 256 threads");
  constexpr int N = ROWS * COLS / 256;
  float v[N];
#pragma unroll
  for (int k = 0; k < N; ++k) {
    const int idx = threadIdx.x + 256 * k;
    const int row = COL_FAST ? idx / COLS : idx % ROWS, col = COL_FAST ? idx % COLS : idx / ROWS;
    v[k] = f(row, col);
  }
#pragma unroll
  for (int k = 0; k < N; ++k) {
    const int idx = threadIdx.x + 256 * k;
    const int row = COL_FAST ? idx / COLS : idx % ROWS, col = COL_FAST ? idx % COLS : idx / ROWS;
    lds[TR ? col * LS + row : row * LS + col] = v[k];
  }
}

}  // namespace

// ---- gate recompute: b (chunk-local cumulative log alpha), sigmoid(-z)/gamma, g1 ----
// One workgroup of d_k threads per (branch, b, head, chunk); thread = key channel.
// Dynamic LDS: the chunk's block means g1s [C][r] (at least 256 floats: the part
// totals reuse them), the head's W_g2 slice [r][d_k], and log alpha [C][d_k].
__global__ __launch_bounds__(256) void k_bwd_gate(const BwdParams P) {
  extern __shared__ float gate_lds[];
  float* g1s = gate_lds;
  float* w2s = gate_lds + max(P.C * P.r, 256);
  const UnitPos u = unit_pos(P, blockIdx.x);
  const BwdBranch& Br = P.br[u.bi];
  const int j0 = u.ch * P.C;
  const int hdk = Br.h * P.dk;
  for (int idx = threadIdx.x; idx < P.C * P.r; idx += blockDim.x) {
    const int jj = idx / P.r, rr = idx - jj * P.r;
    const int j = j0 + jj;
    float acc = 0.f;
    if (j < Br.n) {
      const float* gp = Br.g + ((size_t)u.b * P.L + (size_t)j * Br.s) * P.rp + rr;
      for (int v = 0; v < Br.s; ++v) acc += gp[(size_t)v * P.rp];
      acc /= (float)Br.s;
      if (u.head == 0) Br.g1c[((size_t)u.b * Br.n + j) * P.rp + rr] = acc;
    }
    g1s[jj * P.r + rr] = acc;
  }
  for (int idx = threadIdx.x; idx < P.r * P.dk; idx += blockDim.x) {
    const int rr = idx / P.dk, c = idx - rr * P.dk;
    w2s[rr * P.dk + c] = Br.W2[(size_t)rr * hdk + u.head * P.dk + c];
  }
  __syncthreads();
  // thread = (channel, part): the chunk's positions are cut into 256 / d_k
  // parts scanned side by side, then each part adds the totals of the parts
  // before it
  const int parts = 256 / P.dk;
  const int c = threadIdx.x % P.dk, part = threadIdx.x / P.dk;
  const int len = (P.C + parts - 1) / parts, jb = part * len, je = min(P.C, jb + len);
  const float bgc = Br.bg[u.head * P.dk + c];
  float* las = w2s + P.r * P.dk;  // log alpha [C][d_k]
  float bsum = 0.f;
  for (int jj = jb; jj < je; ++jj) {
    const bool valid = j0 + jj < Br.n;
    float z = bgc;
    for (int rr = 0; rr < P.r; ++rr) z += g1s[jj * P.r + rr] * w2s[rr * P.dk + c];
    const float la = valid ? logsigmoid_f(z) * P.inv_gamma : 0.f;
    las[jj * P.dk + c] = la;
    bsum += la;
    Br.sg[((size_t)u.sq * Br.np + j0 + jj) * P.dk + c] = valid ? __expf(logsigmoid_f(-z)) * P.inv_gamma : 0.f;
  }
  __syncthreads();  // the block means are no longer needed: their space takes the part totals
  float* tot = g1s;
  tot[part * P.dk + c] = bsum;
  __syncthreads();
  float run = 0.f;
  for (int q = 0; q < part; ++q) run += tot[q * P.dk + c];
  for (int jj = jb; jj < je; ++jj) {
    run += las[jj * P.dk + c];
    Br.lb[((size_t)u.sq * Br.np + j0 + jj) * P.dk + c] = run;
  }
}

// ---- per-chunk outer products (X * F)^T Y  [d_k][64-column slice of d_v] ----
// REV = false: X = k, F = e^{b_last - b}, Y = v     (the chunk's state increment)
// REV = true:  X = q_scale q, F = e^{b}, Y = dLoss/do  (its state-gradient increment)
template <typename T, int DK, bool REV>
__global__ __launch_bounds__(256) void k_bwd_outer(const BwdParams P) {
  __shared__ float xs[64 * DK];
  __shared__ __attribute__((aligned(16))) float ys[64 * 64];
  const UnitPos u = unit_pos(P, blockIdx.x);
  const BwdBranch& Br = P.br[u.bi];
  const int j0 = u.ch * P.C, e0 = blockIdx.y * 64;
  const int nvalid = min(P.C, Br.n - j0);
  const size_t row0 = (size_t)u.sq * Br.np + j0;
  stage<64, DK, DK, true, false>(xs, [&](int t, int c) {
    const bool ok = t < nvalid;
    const size_t o = (row0 + (ok ? t : 0)) * DK + c;
    float val;
    if constexpr (REV)
      val = P.q_scale * Br.q[o] * __expf(Br.lb[o]);
    else
      val = Br.k[o] * __expf(Br.lb[(row0 + P.C - 1) * DK + c] - Br.lb[o]);
    return ok ? val : 0.f;
  });
  if constexpr (REV)
    stage<64, 64, 64, true, false>(ys, [&](int t, int e) {
      const bool ok = t < nvalid;
      const float val = Br.dob[((size_t)(u.b * Br.n + j0 + (ok ? t : 0)) * Br.h + u.head) * P.dv + e0 + e];
      return ok ? val : 0.f;
    });
  else
    stage<64, 64, 64, false, false>(ys, [&](int t, int e) {
      const bool ok = t < nvalid;
      const float val = to_f32(reinterpret_cast<const T*>(Br.vT)[(((size_t)u.sq * Br.nch + u.ch) * P.dv + e0 + e) * P.C + (ok ? t : 0)]);
      return ok ? val : 0.f;
    });
  __syncthreads();
  constexpr int NA = DK >= 32 ? DK / 32 : 1;
  const int cr = threadIdx.x & 31, er = threadIdx.x >> 5;
  float acc[NA][8];
#pragma unroll
  for (int a = 0; a < NA; ++a)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[a][e] = 0.f;
  const int crc = DK >= 32 ? cr : (cr & (DK - 1));
  for (int t = 0; t < nvalid; ++t) {
    const f32x4 y0 = *reinterpret_cast<const f32x4*>(ys + t * 64 + er * 8);
    const f32x4 y1 = *reinterpret_cast<const f32x4*>(ys + t * 64 + er * 8 + 4);
#pragma unroll
    for (int a = 0; a < NA; ++a) {
      const float xv = xs[t * DK + crc + 32 * a];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[a][e] += xv * y0[e];
        acc[a][e + 4] += xv * y1[e];
      }
    }
  }
  if (DK < 32 && cr >= DK) return;
  float* out = REV ? Br.dSt : Br.Sst;
#pragma unroll
  for (int a = 0; a < NA; ++a) {
    float* o = out + (((size_t)u.sq * Br.nch + u.ch) * DK + crc + 32 * a) * P.dv + e0 + er * 8;
    *reinterpret_cast<f32x4*>(o) = f32x4{acc[a][0], acc[a][1], acc[a][2], acc[a][3]};
    *reinterpret_cast<f32x4*>(o + 4) = f32x4{acc[a][4], acc[a][5], acc[a][6], acc[a][7]};
  }
}

// ---- scan over chunks, in place: buf[c] <- carried value entering chunk c ----
// forward: S_prev(c+1) = Diag(lambda_c) S_prev(c) + dS_c, S_prev(0) = 0
// reverse: G(c-1)      = Diag(lambda_c) G(c) + dG_c,     G(last) = 0
// lambda_c = e^{b_last} of chunk c (per key channel).  One thread per element.
__global__ __launch_bounds__(256) void k_bwd_scan(float* buf, const float* lb, int seqs, int nch,
                                                  int np, int C, int dk, int dv, int rev) {
  const size_t total = (size_t)seqs * dk * dv;
  for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (size_t)gridDim.x * blockDim.x) {
    const size_t sq = idx / ((size_t)dk * dv);
    const int rem = (int)(idx - sq * dk * dv);
    const int c = rem / dv, e = rem - c * dv;
    float S = 0.f;
#pragma unroll 4
    for (int it = 0; it < nch; ++it) {
      const int ch = rev ? nch - 1 - it : it;
      const size_t o = ((sq * nch + ch) * dk + c) * dv + e;
      const float lam = __expf(lb[(sq * np + (size_t)ch * C + C - 1) * dk + c]);
      const float t = buf[o];
      buf[o] = S;
      S = lam * S + t;
    }
  }
}

// ---- A and D of a chunk (t >= i, zero above the diagonal and outside the call) ----
// thread: t = lane, i in 16 * wave .. 16 * wave + 15
template <typename T, int DK>
__global__ __launch_bounds__(256) void k_bwd_AD(const BwdParams P) {
  __shared__ float sm[3 * 64 * 33 > 2 * 64 * 65 ? 3 * 64 * 33 : 2 * 64 * 65];
  const UnitPos u = unit_pos(P, blockIdx.x);
  const BwdBranch& Br = P.br[u.bi];
  const int j0 = u.ch * P.C;
  const int nvalid = min(P.C, Br.n - j0);
  const size_t row0 = (size_t)u.sq * Br.np + j0;
  const int t = threadIdx.x & 63, ig = threadIdx.x >> 6;
  float accA[16], accD[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) accA[v] = accD[v] = 0.f;
  float* qs = sm;
  float* ks = sm + 64 * 33;
  float* bs = sm + 2 * 64 * 33;
  constexpr int CW = DK < 32 ? DK : 32;
  for (int c0 = 0; c0 < DK; c0 += CW) {
    auto at_ = [&](int tt, int cc) { return (row0 + (tt < nvalid ? tt : 0)) * DK + c0 + cc; };
    stage<64, CW, 33, true, false>(qs, [&](int tt, int cc) {
      const float v = P.q_scale * Br.q[at_(tt, cc)];
      return tt < nvalid ? v : 0.f;
    });
    stage<64, CW, 33, true, false>(ks, [&](int tt, int cc) {
      const float v = Br.k[at_(tt, cc)];
      return tt < nvalid ? v : 0.f;
    });
    stage<64, CW, 33, true, false>(bs, [&](int tt, int cc) {
      const float v = Br.lb[at_(tt, cc)];
      return tt < nvalid ? v : 0.f;
    });
    __syncthreads();
    for (int cc = 0; cc < CW; ++cc) {
      const float qv = qs[t * 33 + cc], bt = bs[t * 33 + cc];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int i = ig * 16 + v;
        accA[v] += qv * ks[i * 33 + cc] * __expf(fminf(bt - bs[i * 33 + cc], 0.f));
      }
    }
    __syncthreads();
  }
  float* ds = sm;
  float* vs = sm + 64 * 65;
  for (int e0 = 0; e0 < P.dv; e0 += 64) {
    stage<64, 64, 65, true, false>(ds, [&](int tt, int e) {
      const bool ok = tt < nvalid;
      const float v = Br.dob[((size_t)(u.b * Br.n + j0 + (ok ? tt : 0)) * Br.h + u.head) * P.dv + e0 + e];
      return ok ? v : 0.f;
    });
    // v^T per chunk [d_v][C]: consecutive threads take consecutive positions
    stage<64, 64, 65, false, false>(vs, [&](int tt, int e) {
      const bool ok = tt < nvalid;
      const float v = to_f32(reinterpret_cast<const T*>(Br.vT)[(((size_t)u.sq * Br.nch + u.ch) * P.dv + e0 + e) * P.C + (ok ? tt : 0)]);
      return ok ? v : 0.f;
    });
    __syncthreads();
    for (int e = 0; e < 64; ++e) {
      const float dv_ = ds[t * 65 + e];
#pragma unroll
      for (int v = 0; v < 16; ++v) accD[v] += dv_ * vs[(ig * 16 + v) * 65 + e];
    }
    __syncthreads();
  }
  float* A = Br.AD + ((size_t)u.sq * Br.nch + u.ch) * 2 * 64 * 64;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int i = ig * 16 + v;
    const bool keep = i <= t && t < nvalid;
    A[t * 64 + i] = keep ? accA[v] : 0.f;
    A[64 * 64 + t * 64 + i] = keep ? accD[v] : 0.f;
  }
}

// ---- dv_i = sum_{t>=i} A_ti do_t + k-hat_i dS_end, into the v columns of dP ----
// thread: i = lane, 16 columns 16 * wave .. of the block's 64-column slice
template <typename T, int DK>
__global__ __launch_bounds__(256) void k_bwd_dv(const BwdParams P) {
  __shared__ float as[64 * 65];
  __shared__ __attribute__((aligned(16))) float dos[64 * 64];
  __shared__ float khs[64 * 65];
  __shared__ __attribute__((aligned(16))) float dss[64 * 64];
  const UnitPos u = unit_pos(P, blockIdx.x);
  const BwdBranch& Br = P.br[u.bi];
  const int j0 = u.ch * P.C, e0 = blockIdx.y * 64;
  const int nvalid = min(P.C, Br.n - j0);
  const size_t row0 = (size_t)u.sq * Br.np + j0;
  const int i = threadIdx.x & 63, eg = threadIdx.x >> 6;
  const float* A = Br.AD + ((size_t)u.sq * Br.nch + u.ch) * 2 * 64 * 64;
  stage<64, 64, 65, true, false>(as, [&](int tt, int i) { return A[tt * 64 + i]; });
  stage<64, 64, 64, true, false>(dos, [&](int tt, int e) {
    const bool ok = tt < nvalid;
    const float v = Br.dob[((size_t)(u.b * Br.n + j0 + (ok ? tt : 0)) * Br.h + u.head) * P.dv + e0 + e];
    return ok ? v : 0.f;
  });
  __syncthreads();
  float acc[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.f;
  for (int tt = 0; tt < 64; ++tt) {
    const float a = as[tt * 65 + i];
#pragma unroll
    for (int v = 0; v < 16; v += 4) {
      const f32x4 d4 = *reinterpret_cast<const f32x4*>(dos + tt * 64 + eg * 16 + v);
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[v + q] += a * d4[q];
    }
  }
  constexpr int CW = DK < 64 ? DK : 64;
  for (int c0 = 0; c0 < DK; c0 += CW) {
    __syncthreads();
    stage<64, CW, 65, true, false>(khs, [&](int tt, int cc) {
      const bool ok = tt < nvalid;
      const size_t o = (row0 + (ok ? tt : 0)) * DK + c0 + cc;
      const float v = Br.k[o] * __expf(Br.lb[(row0 + P.C - 1) * DK + c0 + cc] - Br.lb[o]);
      return ok ? v : 0.f;
    });
    stage<CW, 64, 64, true, false>(dss, [&](int cc, int e) {
      return Br.dSt[(((size_t)u.sq * Br.nch + u.ch) * DK + c0 + cc) * P.dv + e0 + e];
    });
    __syncthreads();
    for (int cc = 0; cc < CW; ++cc) {
      const float kv = khs[i * 65 + cc];
#pragma unroll
      for (int v = 0; v < 16; v += 4) {
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(dss + cc * 64 + eg * 16 + v);
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[v + q] += kv * d4[q];
      }
    }
  }
  if (i >= nvalid) return;
  T* dst = reinterpret_cast<T*>(Br.dP) + (size_t)(u.b * Br.n + j0 + i) * Br.NP + Br.col_v + u.head * P.dv + e0 + eg * 16;
  store8<T>(dst, acc);
  store8<T>(dst + 8, acc + 8);
}

// ---- dq and dk of a chunk's 32-channel slice; in-chunk suffix sums of q dq - k dk ----
// thread: t = lane, channels c0 + 8 * wave .. + 7
template <typename T, int DK>
__global__ __launch_bounds__(256) void k_bwd_dqdk(const BwdParams P) {
  constexpr int CS = DK < 32 ? DK : 32;  // channels per block
  __shared__ __attribute__((aligned(16))) float sm[2 * 64 * 65 + 2 * 64 * 32];
  __shared__ float rs[64 * 33];
  const UnitPos u = unit_pos(P, blockIdx.x);
  const BwdBranch& Br = P.br[u.bi];
  const int j0 = u.ch * P.C, c0 = blockIdx.y * CS;
  const int nvalid = min(P.C, Br.n - j0);
  const size_t row0 = (size_t)u.sq * Br.np + j0;
  const int t = threadIdx.x & 63, cg = threadIdx.x >> 6;
  const bool live = cg * 8 < CS;  // DK 16: two waves of channels
  const size_t sbase = ((size_t)u.sq * Br.nch + u.ch) * DK;
  float aq[8], ak[8], iq[8], ik[8], bt[8];
#pragma unroll
  for (int v = 0; v < 8; ++v) aq[v] = ak[v] = iq[v] = ik[v] = 0.f;
  // inter-chunk terms: do_t S_prev^T and v_t dS_end^T over d_v in 64-column steps
  {
    float* dos = sm;
    float* vs = sm + 64 * 65;
    float* sT = sm + 2 * 64 * 65;            // [64 e][32 c]
    float* dsT = sm + 2 * 64 * 65 + 64 * 32;
    for (int e0 = 0; e0 < P.dv; e0 += 64) {
      stage<64, 64, 65, true, false>(dos, [&](int tt, int e) {
        const bool ok = tt < nvalid;
        const float v = Br.dob[((size_t)(u.b * Br.n + j0 + (ok ? tt : 0)) * Br.h + u.head) * P.dv + e0 + e];
        return ok ? v : 0.f;
      });
      stage<64, 64, 65, false, false>(vs, [&](int tt, int e) {
        const bool ok = tt < nvalid;
        const float v = to_f32(reinterpret_cast<const T*>(Br.vT)[(((size_t)u.sq * Br.nch + u.ch) * P.dv + e0 + e) * P.C + (ok ? tt : 0)]);
        return ok ? v : 0.f;
      });
      stage<CS, 64, 32, true, true>(sT, [&](int cc, int e) { return Br.Sst[(sbase + c0 + cc) * P.dv + e0 + e]; });
      stage<CS, 64, 32, true, true>(dsT, [&](int cc, int e) { return Br.dSt[(sbase + c0 + cc) * P.dv + e0 + e]; });
      __syncthreads();
      if (live) {
        for (int e = 0; e < 64; ++e) {
          const float dv_ = dos[t * 65 + e], vv = vs[t * 65 + e];
          const f32x4 s0 = *reinterpret_cast<const f32x4*>(sT + e * 32 + cg * 8);
          const f32x4 s1 = *reinterpret_cast<const f32x4*>(sT + e * 32 + cg * 8 + 4);
          const f32x4 g0 = *reinterpret_cast<const f32x4*>(dsT + e * 32 + cg * 8);
          const f32x4 g1 = *reinterpret_cast<const f32x4*>(dsT + e * 32 + cg * 8 + 4);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            aq[q] += dv_ * s0[q];
            aq[q + 4] += dv_ * s1[q];
            ak[q] += vv * g0[q];
            ak[q + 4] += vv * g1[q];
          }
        }
      }
      __syncthreads();
    }
  }
  // intra-chunk terms with e^{-|b_t - b_i|} (b is non-increasing along the chunk)
  float* ds = sm;                  // D[t][i], stride 65
  float* qs = sm + 64 * 65;        // q_scale q, stride 33
  float* ks = qs + 64 * 33;
  float* bs = ks + 64 * 33;
  const float* D = Br.AD + ((size_t)u.sq * Br.nch + u.ch) * 2 * 64 * 64 + 64 * 64;
  stage<64, 64, 65, true, false>(ds, [&](int tt, int i) { return D[tt * 64 + i]; });
  auto at_ = [&](int tt, int cc) { return (row0 + (tt < nvalid ? tt : 0)) * DK + c0 + cc; };
  stage<64, CS, 33, true, false>(qs, [&](int tt, int cc) {
    const float v = P.q_scale * Br.q[at_(tt, cc)];
    return tt < nvalid ? v : 0.f;
  });
  stage<64, CS, 33, true, false>(ks, [&](int tt, int cc) {
    const float v = Br.k[at_(tt, cc)];
    return tt < nvalid ? v : 0.f;
  });
  // rows past the chunk keep its last b (the gate adds nothing past the call's end)
  stage<64, CS, 33, true, false>(bs, [&](int tt, int cc) { return Br.lb[(row0 + min(tt, P.C - 1)) * DK + c0 + cc]; });
  __syncthreads();
  float blast[8];
#pragma unroll
  for (int v = 0; v < 8; ++v) {
    const int cc = live ? cg * 8 + v : 0;
    bt[v] = bs[t * 33 + cc];
    blast[v] = bs[(P.C - 1) * 33 + cc];
  }
  if (live) {
    for (int i = 0; i < 64; ++i) {
      const float dti = ds[t * 65 + i];  // D_ti, zero unless i <= t
      const float dit = ds[i * 65 + t];  // D_it, zero unless i >= t
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        const int cc = cg * 8 + v;
        const float E = __expf(-fabsf(bt[v] - bs[i * 33 + cc]));
        iq[v] += dti * ks[i * 33 + cc] * E;
        ik[v] += dit * qs[i * 33 + cc] * E;
      }
    }
  }
  float dq[8], dk[8];
#pragma unroll
  for (int v = 0; v < 8; ++v) {
    dq[v] = __expf(bt[v]) * aq[v] + iq[v];
    dk[v] = __expf(blast[v] - bt[v]) * ak[v] + ik[v];
    if (t >= nvalid) dq[v] = dk[v] = 0.f;
  }
  if (live) {
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      const int cc = cg * 8 + v;
      rs[t * 33 + cc] = qs[t * 33 + cc] * dq[v] - ks[t * 33 + cc] * dk[v];
    }
    if (t < nvalid) {
      const size_t prow = (size_t)(u.b * Br.n + j0 + t) * Br.NP + u.head * DK + c0 + cg * 8;
      float sq8[8];
#pragma unroll
      for (int v = 0; v < 8; ++v) sq8[v] = P.q_scale * dq[v];
      store8<T>(reinterpret_cast<T*>(Br.dP) + prow, sq8);
      store8<T>(reinterpret_cast<T*>(Br.dP) + prow + Br.col_k, dk);
    }
  }
  __syncthreads();
  if (threadIdx.x < CS) {
    const int cc = threadIdx.x;
    float run = 0.f;
    for (int tt = P.C - 1; tt >= 0; --tt) {
      run += rs[tt * 33 + cc];
      Br.rsum[(row0 + tt) * DK + c0 + cc] = run;
    }
    Br.rtot[((size_t)u.sq * Br.nch + u.ch) * DK + c0 + cc] = run;
  }
}

// ---- dz of the gate: (suffix of q dq - k dk) * sigmoid(-z) / gamma, position-major ----
__global__ __launch_bounds__(256) void k_bwd_dzg(const BwdParams P, int bi) {
  const BwdBranch& Br = P.br[bi];
  const size_t total = (size_t)P.B * Br.h * Br.nch * P.dk;
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int c = (int)(idx % P.dk);
  const size_t sc = idx / P.dk;
  const int ch = (int)(sc % Br.nch);
  const int sq = (int)(sc / Br.nch);
  const int b = sq / Br.h, head = sq - b * Br.h;
  float suffix = 0.f;
  for (int c2 = ch + 1; c2 < Br.nch; ++c2) suffix += Br.rtot[((size_t)sq * Br.nch + c2) * P.dk + c];
  const int nvalid = min(P.C, Br.n - ch * P.C);
  for (int t0 = 0; t0 < nvalid; t0 += 8) {
    float rv[8], sv[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const size_t o = ((size_t)sq * Br.np + ch * P.C + min(t0 + k, nvalid - 1)) * P.dk + c;
      rv[k] = Br.rsum[o];
      sv[k] = Br.sg[o];
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int j = ch * P.C + t0 + k;
      if (t0 + k < nvalid) Br.dzg[((size_t)(b * Br.n + j) * Br.h + head) * P.dk + c] = (rv[k] + suffix) * sv[k];
    }
  }
}

// ---- dg1 = dz W_g2^T into the gate columns of dP: one wave per pooled position ----
template <typename T, int RP>
__global__ __launch_bounds__(256) void k_bwd_dg1(const BwdParams P, int bi) {
  const BwdBranch& Br = P.br[bi];
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= P.B * Br.n) return;
  const int hdk = Br.h * P.dk;
  float acc[RP];
#pragma unroll
  for (int r = 0; r < RP; ++r) acc[r] = 0.f;
  const float* dz = Br.dzg + (size_t)row * hdk;
  for (int c = lane; c < hdk; c += 64) {
    const float z = dz[c];
#pragma unroll
    for (int r = 0; r < RP; ++r) acc[r] += z * Br.W2[(size_t)r * hdk + c];
  }
#pragma unroll
  for (int r = 0; r < RP; ++r) acc[r] = wave_sum(acc[r]);
  T* dst = reinterpret_cast<T*>(Br.dP) + (size_t)row * Br.NP + Br.col_g;
#pragma unroll
  for (int r = 0; r < RP; ++r)
    if (lane == r) dst[r] = from_f32<T>(acc[r]);
}

// ---- fusion and hold, per position (one wave each) ----
// dw of every branch, dz = w (dw - sum w dw); the scale-1 branch's
// dLoss/do (its G = dO W_o^T rows, scaled in place by w_1) and w_1 y rows.
template <typename T>
__global__ __launch_bounds__(256) void k_bwd_out(const BwdParams P) {
  const int pos = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (pos >= P.B * P.L) return;
  const int b = pos / P.L, t = pos - b * P.L;
  const T* dO = reinterpret_cast<const T*>(P.dout) + (size_t)pos * P.d;
  float w[MSGLA_MAX_BRANCHES], dw[MSGLA_MAX_BRANCHES];
#pragma unroll
  for (int i = 0; i < MSGLA_MAX_BRANCHES; ++i) {
    w[i] = (P.m > 1 && i < P.m) ? P.w[(size_t)pos * FUSION_STRIDE + i] : (i == 0 ? 1.f : 0.f);
    dw[i] = 0.f;
  }
#pragma unroll
  for (int i = 0; i < MSGLA_MAX_BRANCHES; ++i) {
    if (i >= P.nbranch) break;
    const BwdBranch& Br = P.br[i];
    float part = 0.f;
    if (Br.s == 1) {
      if (Br.n == 0) continue;
      const int hdv = Br.h * P.dv;
      float* G = Br.dob + (size_t)pos * hdv;
      T* yc = reinterpret_cast<T*>(Br.ycat) + (size_t)pos * hdv;
      for (int p = lane * 8; p < hdv; p += 64 * 8) {
        const int hh = p / P.dv, e = p - hh * P.dv;
        float y8[8], g8[8];
        load8<T>(reinterpret_cast<const T*>(Br.y) + (((size_t)b * Br.h + hh) * Br.np + t) * P.dv + e, y8);
        const f32x4 ga = *reinterpret_cast<const f32x4*>(G + p);
        const f32x4 gb = *reinterpret_cast<const f32x4*>(G + p + 4);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          g8[q] = ga[q];
          g8[q + 4] = gb[q];
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          part += g8[q] * y8[q];
          g8[q] *= w[i];
          y8[q] *= w[i];
        }
        *reinterpret_cast<f32x4*>(G + p) = f32x4{g8[0], g8[1], g8[2], g8[3]};
        *reinterpret_cast<f32x4*>(G + p + 4) = f32x4{g8[4], g8[5], g8[6], g8[7]};
        store8<T>(yc + p, y8);
      }
    } else {
      const int j = (t + 1) / Br.s - 1;
      if (j < 0) continue;
      const T* Y = reinterpret_cast<const T*>(Br.yc) + ((size_t)b * Br.n + j) * P.d;
      for (int p = lane * 8; p < P.d; p += 64 * 8) {
        float a8[8], y8[8];
        load8<T>(dO + p, a8);
        load8<T>(Y + p, y8);
#pragma unroll
        for (int q = 0; q < 8; ++q) part += a8[q] * y8[q];
      }
    }
    dw[i] = wave_sum(part);
  }
  if (P.m <= 1) return;
  float S = 0.f;
#pragma unroll
  for (int i = 0; i < MSGLA_MAX_BRANCHES; ++i) S += w[i] * dw[i];
#pragma unroll
  for (int i = 0; i < FUSION_STRIDE; ++i)
    if (lane == i) P.dz[(size_t)pos * FUSION_STRIDE + i] = i < P.m ? w[i] * (dw[i] - S) : 0.f;
}

// ---- coarse branch: dY_j = sum over the positions holding block j of w dO; y rows ----
template <typename T>
__global__ __launch_bounds__(256) void k_bwd_hold(const BwdParams P, int bi) {
  const BwdBranch& Br = P.br[bi];
  const int rows = P.B * Br.n;
  const int pd = P.d / 8, py = Br.h * P.dv / 8;
  const size_t n1 = (size_t)rows * pd, total = n1 + (size_t)rows * py;
  for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (size_t)gridDim.x * blockDim.x) {
    if (idx < n1) {
      const int row = (int)(idx / pd), col = (int)(idx - (size_t)row * pd) * 8;
      const int b = row / Br.n, j = row - b * Br.n;
      const int t0 = (j + 1) * Br.s - 1, t1 = min((j + 2) * Br.s - 2, P.L - 1);
      float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      for (int t = t0; t <= t1; ++t) {
        const size_t pos = (size_t)b * P.L + t;
        const float wt = P.m > 1 ? P.w[pos * FUSION_STRIDE + bi] : 1.f;
        float a8[8];
        load8<T>(reinterpret_cast<const T*>(P.dout) + pos * P.d + col, a8);
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] += wt * a8[q];
      }
      store8<T>(reinterpret_cast<T*>(Br.dY) + (size_t)row * P.d + col, acc);
    } else {
      const size_t k = idx - n1;
      const int row = (int)(k / py), p = (int)(k - (size_t)row * py) * 8;
      const int b = row / Br.n, j = row - b * Br.n;
      const int hh = p / P.dv, e = p - hh * P.dv;
      const T* src = reinterpret_cast<const T*>(Br.y) + (((size_t)b * Br.h + hh) * Br.np + j) * P.dv + e;
      T* dst = reinterpret_cast<T*>(Br.ycat) + (size_t)row * Br.h * P.dv + p;
      st16(dst, ld16(src));
      if constexpr (sizeof(T) == 4) st16(dst + 4, ld16(src + 4));
    }
  }
}

// ---- dx = sum over branches of the pooled gradient / s + dz W_f^T ----
template <typename T>
__global__ __launch_bounds__(256) void k_bwd_dx(const BwdParams P) {
  const int pd = P.d / 8;
  const size_t total = (size_t)P.B * P.L * pd;
  for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (size_t)gridDim.x * blockDim.x) {
    const size_t pos = idx / pd;
    const int col = (int)(idx - pos * pd) * 8;
    const int b = (int)(pos / P.L), t = (int)(pos - (size_t)b * P.L);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int i = 0; i < P.nbranch; ++i) {
      const BwdBranch& Br = P.br[i];
      if (t >= Br.n * Br.s) continue;
      const float* src = Br.dxp + ((size_t)b * Br.n + t / Br.s) * P.d + col;
      const float inv = 1.f / (float)Br.s;
      const f32x4 a = *reinterpret_cast<const f32x4*>(src);
      const f32x4 c = *reinterpret_cast<const f32x4*>(src + 4);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[q] += a[q] * inv;
        acc[q + 4] += c[q] * inv;
      }
    }
    if (P.m > 1) {
      for (int i = 0; i < P.m; ++i) {
        const float z = P.dz[pos * FUSION_STRIDE + i];
        float f8[8];
        load8<T>(reinterpret_cast<const T*>(P.Wf) + (size_t)i * P.d + col, f8);
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] += z * f8[q];
      }
    }
    store8<T>(reinterpret_cast<T*>(P.dx) + pos * P.d + col, acc);
  }
}

// ---- column sums and x^T dz, in two deterministic passes ----
// partial[rb][col] = sum over row block rb of src[row][col] (src fp32, ld);
// a block is 64 columns x 4 row lanes, its row block cut into the lanes
__global__ __launch_bounds__(256) void k_bwd_colsum_partial(const float* src, int rows, int cols, int ld,
                                                            int rows_per_block, float* partial) {
  __shared__ float red[4][64];
  const int cc = threadIdx.x & 63, lane4 = threadIdx.x >> 6;
  const int col = blockIdx.x * 64 + cc;
  const int r0 = blockIdx.y * rows_per_block, r1 = min(rows, r0 + rows_per_block);
  const int colc = min(col, cols - 1);
  float acc = 0.f;
  for (int r = r0 + lane4; r < r1; r += 32) {
    float v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = src[(size_t)min(r + 4 * k, r1 - 1) * ld + colc];
#pragma unroll
    for (int k = 0; k < 8; ++k) acc += (r + 4 * k < r1) ? v[k] : 0.f;
  }
  red[lane4][cc] = acc;
  __syncthreads();
  if (lane4 == 0 && col < cols)
    partial[(size_t)blockIdx.y * cols + col] = red[0][cc] + red[1][cc] + red[2][cc] + red[3][cc];
}

// out[col] = sum_rb partial[rb][col]
__global__ __launch_bounds__(256) void k_bwd_colsum_finish(const float* partial, int nrb, int cols, float* out,
                                                           int out_stride) {
  const int col = blockIdx.x * 256 + threadIdx.x;
  if (col >= cols) return;
  float acc = 0.f;
  for (int rb0 = 0; rb0 < nrb; rb0 += 8) {
    float v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = partial[(size_t)min(rb0 + k, nrb - 1) * cols + col];
#pragma unroll
    for (int k = 0; k < 8; ++k) acc += (rb0 + k < nrb) ? v[k] : 0.f;
  }
  out[(size_t)col * out_stride] = acc;
}

// partial[rb][col][i] = sum over row block rb of x[row][col] dz[row][i], i < 8
template <typename T>
__global__ __launch_bounds__(256) void k_bwd_wf_partial(const BwdParams P, int rows_per_block, float* partial) {
  __shared__ float red[4][64][FUSION_STRIDE];
  const int cc = threadIdx.x & 63, tg = threadIdx.x >> 6;
  const int col = blockIdx.x * 64 + cc;
  const int rows = P.B * P.L;
  const int r0 = blockIdx.y * rows_per_block, r1 = min(rows, r0 + rows_per_block);
  float acc[FUSION_STRIDE];
#pragma unroll
  for (int i = 0; i < FUSION_STRIDE; ++i) acc[i] = 0.f;
#pragma unroll 4
  for (int r = r0 + tg; r < r1; r += 4) {
    const float xv = to_f32(reinterpret_cast<const T*>(P.x)[(size_t)r * P.d + col]);
    const f32x4 z0 = *reinterpret_cast<const f32x4*>(P.dz + (size_t)r * FUSION_STRIDE);
    const f32x4 z1 = *reinterpret_cast<const f32x4*>(P.dz + (size_t)r * FUSION_STRIDE + 4);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc[q] += xv * z0[q];
      acc[q + 4] += xv * z1[q];
    }
  }
#pragma unroll
  for (int i = 0; i < FUSION_STRIDE; ++i) red[tg][cc][i] = acc[i];
  __syncthreads();
  if (tg == 0) {
#pragma unroll
    for (int i = 0; i < FUSION_STRIDE; ++i) {
      const float v = red[0][cc][i] + red[1][cc][i] + red[2][cc][i] + red[3][cc][i];
      partial[((size_t)blockIdx.y * P.d + col) * FUSION_STRIDE + i] = v;
    }
  }
}

// ---------------- launchers ----------------

template <typename T, int DK>
static void launch_chunk_kernels_t(const BwdParams& P, int which, hipStream_t st) {
  const int slices = P.dv / 64;
  switch (which) {
    case 0: hipLaunchKernelGGL((k_bwd_outer<T, DK, false>), dim3(P.total_units, slices), dim3(256), 0, st, P); break;
    case 1: hipLaunchKernelGGL((k_bwd_outer<T, DK, true>), dim3(P.total_units, slices), dim3(256), 0, st, P); break;
    case 2: hipLaunchKernelGGL((k_bwd_AD<T, DK>), dim3(P.total_units), dim3(256), 0, st, P); break;
    case 3: hipLaunchKernelGGL((k_bwd_dv<T, DK>), dim3(P.total_units, slices), dim3(256), 0, st, P); break;
    default: {
      const int cs = DK < 32 ? 1 : DK / 32;
      hipLaunchKernelGGL((k_bwd_dqdk<T, DK>), dim3(P.total_units, cs), dim3(256), 0, st, P);
    }
  }
}

template <typename T>
static hipError_t launch_chunk_kernels_dk(const BwdParams& P, int which, hipStream_t st) {
  switch (P.dk) {
    case 16: launch_chunk_kernels_t<T, 16>(P, which, st); break;
    case 32: launch_chunk_kernels_t<T, 32>(P, which, st); break;
    case 64: launch_chunk_kernels_t<T, 64>(P, which, st); break;
    case 128: launch_chunk_kernels_t<T, 128>(P, which, st); break;
    case 256: launch_chunk_kernels_t<T, 256>(P, which, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// which: 0 state increments, 1 state-gradient increments, 2 A and D, 3 dv, 4 dq and dk
hipError_t launch_bwd_chunk(const BwdParams& P, int which, bool bf16_path, hipStream_t st) {
  if (P.total_units == 0) return hipSuccess;
  return bf16_path ? launch_chunk_kernels_dk<bf16>(P, which, st) : launch_chunk_kernels_dk<float>(P, which, st);
}

hipError_t launch_bwd_gate(const BwdParams& P, hipStream_t st) {
  if (P.total_units == 0) return hipSuccess;
  // block means, W_g2 slice, log alpha; the part totals (256 floats) reuse the first
  const size_t lds = (size_t)(std::max(P.C * P.r, 256) + P.r * P.dk + P.C * P.dk) * sizeof(float);
  hipLaunchKernelGGL(k_bwd_gate, dim3(P.total_units), dim3(256), lds, st, P);
  return hipGetLastError();
}

hipError_t launch_bwd_scan(float* buf, const float* lb, int seqs, int nch, int np, int C, int dk, int dv,
                           bool rev, hipStream_t st) {
  const size_t total = (size_t)seqs * dk * dv;
  if (total == 0) return hipSuccess;
  const unsigned grid = (unsigned)std::min<size_t>((total + 255) / 256, 65536);
  hipLaunchKernelGGL(k_bwd_scan, dim3(grid), dim3(256), 0, st, buf, lb, seqs, nch, np, C, dk, dv, rev ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_bwd_dzg(const BwdParams& P, int bi, hipStream_t st) {
  const size_t total = (size_t)P.B * P.br[bi].h * P.br[bi].nch * P.dk;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(k_bwd_dzg, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, P, bi);
  return hipGetLastError();
}

hipError_t launch_bwd_dg1(const BwdParams& P, int bi, bool bf16_path, hipStream_t st) {
  const int rows = P.B * P.br[bi].n;
  if (rows == 0) return hipSuccess;
  const dim3 grid((rows + 3) / 4);
  if (P.rp == 16) {
    if (bf16_path) hipLaunchKernelGGL((k_bwd_dg1<bf16, 16>), grid, dim3(256), 0, st, P, bi);
    else hipLaunchKernelGGL((k_bwd_dg1<float, 16>), grid, dim3(256), 0, st, P, bi);
  } else {
    if (bf16_path) hipLaunchKernelGGL((k_bwd_dg1<bf16, 64>), grid, dim3(256), 0, st, P, bi);
    else hipLaunchKernelGGL((k_bwd_dg1<float, 64>), grid, dim3(256), 0, st, P, bi);
  }
  return hipGetLastError();
}

hipError_t launch_bwd_out(const BwdParams& P, bool bf16_path, hipStream_t st) {
  const dim3 grid((unsigned)((P.B * P.L + 3) / 4));
  if (bf16_path) hipLaunchKernelGGL(k_bwd_out<bf16>, grid, dim3(256), 0, st, P);
  else hipLaunchKernelGGL(k_bwd_out<float>, grid, dim3(256), 0, st, P);
  return hipGetLastError();
}

hipError_t launch_bwd_hold(const BwdParams& P, int bi, bool bf16_path, hipStream_t st) {
  const size_t total = (size_t)P.B * P.br[bi].n * (P.d / 8 + P.br[bi].h * P.dv / 8);
  if (total == 0) return hipSuccess;
  const unsigned grid = (unsigned)std::min<size_t>((total + 255) / 256, 65536);
  if (bf16_path) hipLaunchKernelGGL(k_bwd_hold<bf16>, dim3(grid), dim3(256), 0, st, P, bi);
  else hipLaunchKernelGGL(k_bwd_hold<float>, dim3(grid), dim3(256), 0, st, P, bi);
  return hipGetLastError();
}

hipError_t launch_bwd_dx(const BwdParams& P, bool bf16_path, hipStream_t st) {
  const size_t total = (size_t)P.B * P.L * (P.d / 8);
  const unsigned grid = (unsigned)std::min<size_t>((total + 255) / 256, 65536);
  if (bf16_path) hipLaunchKernelGGL(k_bwd_dx<bf16>, dim3(grid), dim3(256), 0, st, P);
  else hipLaunchKernelGGL(k_bwd_dx<float>, dim3(grid), dim3(256), 0, st, P);
  return hipGetLastError();
}

// out[c * out_stride] = sum over rows of src[row][c]; partial holds nrb * cols floats
hipError_t launch_bwd_colsum(const float* src, int rows, int cols, int ld, float* partial, int nrb,
                             float* out, int out_stride, hipStream_t st) {
  if (cols == 0) return hipSuccess;
  const int rpb = (rows + nrb - 1) / nrb;
  hipLaunchKernelGGL(k_bwd_colsum_partial, dim3((cols + 63) / 64, nrb), dim3(256), 0, st, src, rows, cols, ld,
                     rpb, partial);
  hipLaunchKernelGGL(k_bwd_colsum_finish, dim3((cols + 255) / 256), dim3(256), 0, st, partial, nrb, cols, out,
                     out_stride);
  return hipGetLastError();
}

// partial [nrb][d][8]: x^T dz per row block; the host sums them with colsum_finish
hipError_t launch_bwd_wf_partial(const BwdParams& P, float* partial, int nrb, bool bf16_path, hipStream_t st) {
  const int rpb = (P.B * P.L + nrb - 1) / nrb;
  const dim3 grid(P.d / 64, nrb);
  if (bf16_path) hipLaunchKernelGGL(k_bwd_wf_partial<bf16>, grid, dim3(256), 0, st, P, rpb, partial);
  else hipLaunchKernelGGL(k_bwd_wf_partial<float>, grid, dim3(256), 0, st, P, rpb, partial);
  return hipGetLastError();
}

// dW_f [d][m] = sum over row blocks of the partials [nrb][d][8]
__global__ __launch_bounds__(256) void k_bwd_wf_finish(const float* partial, int nrb, int d, int m, float* out) {
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= d * m) return;
  const int c = idx / m, i = idx - c * m;
  float acc = 0.f;
  for (int rb0 = 0; rb0 < nrb; rb0 += 8) {
    float v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = partial[((size_t)min(rb0 + k, nrb - 1) * d + c) * FUSION_STRIDE + i];
#pragma unroll
    for (int k = 0; k < 8; ++k) acc += (rb0 + k < nrb) ? v[k] : 0.f;
  }
  out[idx] = acc;
}

hipError_t launch_bwd_wf_finish(const float* partial, int nrb, int d, int m, float* out, hipStream_t st) {
  hipLaunchKernelGGL(k_bwd_wf_finish, dim3((d * m + 255) / 256), dim3(256), 0, st, partial, nrb, d, m, out);
  return hipGetLastError();
}

}  // namespace msgla

namespace msgla {

// Sum of S partial products [S][M][N] (fp32) into up to four destinations,
// each owning a column range of the product: out_k[row][col - c0_k].

__global__ __launch_bounds__(256) void k_bwd_splitk_reduce(const float* part, int S, int M, int N, SplitDst D) {
  const size_t total = (size_t)M * N;
  for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (size_t)gridDim.x * blockDim.x) {
    float acc = 0.f;
    for (int s = 0; s < S; ++s) acc += part[(size_t)s * total + idx];
    const int row = (int)(idx / N), col = (int)(idx - (size_t)row * N);
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (k < D.n && col >= D.c0[k] && col < D.c0[k] + D.nc[k]) D.p[k][(size_t)row * D.nc[k] + col - D.c0[k]] = acc;
  }
}

hipError_t launch_bwd_splitk_reduce(const float* part, int S, int M, int N, const SplitDst& D, hipStream_t st) {
  const size_t total = (size_t)M * N;
  if (total == 0) return hipSuccess;
  const unsigned grid = (unsigned)std::min<size_t>((total + 255) / 256, 65536);
  hipLaunchKernelGGL(k_bwd_splitk_reduce, dim3(grid), dim3(256), 0, st, part, S, M, N, D);
  return hipGetLastError();
}

}  // namespace msgla
