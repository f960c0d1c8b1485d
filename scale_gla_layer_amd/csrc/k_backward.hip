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
//    A_ti = sum_c q_tc k_ic e^{b_tc - b_ic} (the forward's), D_ti = do_t . v_i
//    (t >= i)                                                            (k_bwd_mm1)
//    dv_i = sum_{t>=i} A_ti do_t + (k_i * e^{b_last - b_i}) dS_end         (k_bwd_dv)
//    dq_t = e^{b_t} * (do_t S_prev^T) + sum_{i<=t} D_ti k_i * e^{b_t - b_i}
//    dk_i = e^{b_last - b_i} * (v_i dS_end^T) + sum_{t>=i} D_ti q_t * e^{b_t - b_i}
//                                                                      (k_bwd_dqdk)
//    and, from a zero initial state, dlog alpha_u = sum_{t>=u} (q_t dq_t - k_t dk_t)
//    per channel: in-chunk suffix sums plus the totals of later chunks;
//  the gate (Sec. 2.1), log alpha = logsigmoid(z) / gamma, z = g1 W_g2 + b_g:
//    dz = dlog alpha sigmoid(-z) / gamma, dg1 = dz W_g2^T, dW_g2 = g1^T dz and
//    db_g = sum of dz                              (k_bwd_gate_grads, k_bwd_mcolsum_*);
//  the pooling (Sec. 3.1, Eq. (8)): dx_t += dxp_j / s for t in complete block j,
//  plus the fusion logits' dz_t W_f^T                                   (k_bwd_dx).
// The plain products around these (dO W_o^T and dY W_o^T, the pooled inputs'
// gradient, the weight gradients) run in k_bwd_gemm.hip.
#include "async_copy.hpp"
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

// The work item (unit, slice) of this block when the launch has 8 * per blocks
// for nwork = units * inner items, unit-major: each XCD (block id mod 8) takes
// one contiguous range of items, so the slices of one unit, which read its
// operands, share that XCD's L2.  False for blocks past the end.
__device__ __forceinline__ bool xcd_item(int nwork, int inner, int& unit, int& slice) {
  const int wk = remap_xcd(blockIdx.x, (nwork + N_XCD - 1) / N_XCD);
  if (wk >= nwork) return false;
  unit = wk / inner;
  slice = wk - unit * inner;
  return true;
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

// The two halves of stage(), for tiles whose loads should share one round trip
// (or be issued a step ahead): load_tile fills v[] in registers, store_tile
// writes it to LDS with the same element order.
template <int ROWS, int COLS, bool COL_FAST, class F>
__device__ __forceinline__ void load_tile(float (&v)[ROWS * COLS / 256], F&& f) {
  static_assert((ROWS * COLS) % 256 == 0, "whole rounds of 256 threads");
#pragma unroll
  for (int k = 0; k < ROWS * COLS / 256; ++k) {
    const int idx = threadIdx.x + 256 * k;
    const int row = COL_FAST ? idx / COLS : idx % ROWS, col = COL_FAST ? idx % COLS : idx / ROWS;
    v[k] = f(row, col);
  }
}
template <int ROWS, int COLS, int LS, bool COL_FAST, bool TR>
__device__ __forceinline__ void store_tile(float* lds, const float (&v)[ROWS * COLS / 256]) {
#pragma unroll
  for (int k = 0; k < ROWS * COLS / 256; ++k) {
    const int idx = threadIdx.x + 256 * k;
    const int row = COL_FAST ? idx / COLS : idx % ROWS, col = COL_FAST ? idx % COLS : idx / ROWS;
    lds[TR ? col * LS + row : row * LS + col] = v[k];
  }
}

// One 16 x 16 fp32 tile on the matrix cores: acc += A B^T over 16 * ns k-values,
// A and B rows of fp32 in LDS (16 rows each from a and b, row strides lda and
// ldb floats, 16-byte aligned).  Lane l holds rows 4 (l / 16) + i, i = 0..3, of
// column l % 16 of the tile.
__device__ __forceinline__ f32x4 tile_f32(const float* a, int lda, const float* b, int ldb, int ns, f32x4 acc) {
  const int l = threadIdx.x & 63;
  const float* pa = a + (l & 15) * lda + 4 * (l >> 4);
  const float* pb = b + (l & 15) * ldb + 4 * (l >> 4);
  for (int s = 0; s < ns; ++s) acc = mma_slab<float>(ld16(pa + 16 * s), ld16(pb + 16 * s), acc);
  return acc;
}

}  // namespace

// ---- gate recompute: b (chunk-local cumulative log alpha), sigmoid(-z)/gamma, g1 ----
// One workgroup of d_k threads per (branch, b, head, chunk); thread = key channel.
// Dynamic LDS: the chunk's block means g1s [C][RP] (ranks >= r zero; at least 256
// floats: the part totals reuse them), the head's W_g2 slice [r][d_k], and
// log alpha [C][d_k].  With E = e^{-|z|}: log alpha = (min(z, 0) - log1p(E)) / gamma
// and sigmoid(-z) = (z > 0 ? E : 1) / (1 + E), both from one reciprocal of 1 + E.
template <int RP>
__global__ __launch_bounds__(256) void k_bwd_gate(const BwdParams P) {
  extern __shared__ __attribute__((aligned(16))) float gate_lds[];
  float* g1s = gate_lds;
  float* w2s = gate_lds + max(P.C * RP, 256);
  const UnitPos u = unit_pos(P, blockIdx.x);
  const BwdBranch& Br = P.br[u.bi];
  const int j0 = u.ch * P.C;
  const int hdk = Br.h * P.dk;
  // the block means of x W_g1 (Eq. (8): over the block's tokens when masked);
  // four entries per thread and round, their rows' loads issued together
  for (int base = 0; base < P.C * RP; base += 4 * 256) {
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    int cnt[4] = {0, 0, 0, 0};
    for (int v0 = 0; v0 < Br.s; v0 += 4) {
      float gv[4][4];
      bool tok[4][4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int idx = min(base + threadIdx.x + 256 * k, P.C * RP - 1);
        const int jj = idx / RP, rr = min(idx - jj * RP, P.r - 1);
        const int j = min(j0 + jj, Br.n - 1);
        const size_t t0 = (size_t)u.b * P.L + (size_t)j * Br.s;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int v = min(v0 + q, Br.s - 1);
          gv[k][q] = Br.g[(t0 + v) * P.rp + rr];
          tok[k][q] = v0 + q < Br.s && (!P.mask || P.mask[t0 + v] != 0);
        }
      }
#pragma unroll
      for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[k] += tok[k][q] ? gv[k][q] : 0.f;
          cnt[k] += tok[k][q] ? 1 : 0;
        }
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int idx = base + threadIdx.x + 256 * k;
      if (idx >= P.C * RP) continue;
      const int jj = idx / RP, rr = idx - jj * RP;
      const int j = j0 + jj;
      const float mean =
          (j < Br.n && rr < P.r) ? acc[k] / (float)(P.mask ? max(cnt[k], 1) : Br.s) : 0.f;
      if (j < Br.n && rr < P.r && u.head == 0) Br.g1c[((size_t)u.b * Br.n + j) * P.rp + rr] = mean;
      g1s[jj * RP + rr] = mean;
    }
  }
  for (int base = 0; base < P.r * P.dk; base += 8 * 256) {
    float wv[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int idx = min(base + threadIdx.x + 256 * k, P.r * P.dk - 1);
      const int rr = idx / P.dk, c = idx - rr * P.dk;
      wv[k] = Br.W2[(size_t)rr * hdk + u.head * P.dk + c];
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int idx = base + threadIdx.x + 256 * k;
      if (idx < P.r * P.dk) w2s[idx] = wv[k];
    }
  }
  __syncthreads();
  // thread = (channel, part): the chunk's positions are cut into 256 / d_k
  // parts scanned side by side, then each part adds the totals of the parts
  // before it
  const int parts = 256 / P.dk;
  const int c = threadIdx.x % P.dk, part = threadIdx.x / P.dk;
  const int len = (P.C + parts - 1) / parts, jb = part * len, je = min(P.C, jb + len);
  const float bgc = Br.bg[u.head * P.dk + c];
  float w2r[RP];
#pragma unroll
  for (int rr = 0; rr < RP; ++rr) w2r[rr] = rr < P.r ? w2s[rr * P.dk + c] : 0.f;
  float* las = w2s + P.r * P.dk;  // log alpha [C][d_k]
  float bsum = 0.f;
#pragma unroll 4
  for (int jj = jb; jj < je; ++jj) {
    const bool valid = j0 + jj < Br.n;
    float z = bgc;
#pragma unroll
    for (int q = 0; q < RP / 4; ++q) {
      float g4[4];
      unpack16<float>(ld16(g1s + jj * RP + 4 * q), g4);
#pragma unroll
      for (int i = 0; i < 4; ++i) z += g4[i] * w2r[4 * q + i];
    }
    // log1p(E) as log(v) for v = 1 + E rounded, plus the first-order correction
    // (E - (v - 1)) / v for that rounding
    const float E = __expf(-fabsf(z)), v = 1.f + E, rv = __frcp_rn(v);
    const float L1 = __logf(v) + (E - (v - 1.f)) * rv;
    const float la = valid ? (fminf(z, 0.f) - L1) * P.inv_gamma : 0.f;
    las[jj * P.dk + c] = la;
    bsum += la;
    Br.sg[((size_t)u.sq * Br.np + j0 + jj) * P.dk + c] = valid ? (z > 0.f ? E : 1.f) * rv * P.inv_gamma : 0.f;
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
// On the matrix cores: A = (X * F)^T [d_k][64 positions], B = Y^T [64 columns][64
// positions]; wave w takes columns 16 w .. 16 w + 15 and every row tile.
template <typename T, int DK, bool REV>
__global__ __launch_bounds__(256) void k_bwd_outer(const BwdParams P) {
  constexpr int LD = 68, NT = DK / 16;
  __shared__ __attribute__((aligned(16))) float xt[DK * LD];
  __shared__ __attribute__((aligned(16))) float yt[64 * LD];
  int unit, slice;
  if (!xcd_item(P.total_units * (P.dv / 64), P.dv / 64, unit, slice)) return;
  const UnitPos u = unit_pos(P, unit);
  const BwdBranch& Br = P.br[u.bi];
  const int j0 = u.ch * P.C, e0 = slice * 64;
  const int nvalid = min(P.C, Br.n - j0);
  const size_t row0 = (size_t)u.sq * Br.np + j0;
  {
    float rx[64 * DK / 256], ry[16];
    load_tile<64, DK, true>(rx, [&](int t, int c) {
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
      load_tile<64, 64, true>(ry, [&](int t, int e) {
        const bool ok = t < nvalid;
        const float val = Br.dob[((size_t)(u.b * Br.n + j0 + (ok ? t : 0)) * Br.h + u.head) * P.dv + e0 + e];
        return ok ? val : 0.f;
      });
    else
      load_tile<64, 64, true>(ry, [&](int e, int t) {
        const bool ok = t < nvalid;
        const float val = to_f32(reinterpret_cast<const T*>(Br.vT)[(((size_t)u.sq * Br.nch + u.ch) * P.dv + e0 + e) * P.C + (ok ? t : 0)]);
        return ok ? val : 0.f;
      });
    store_tile<64, DK, LD, true, true>(xt, rx);
    if constexpr (REV)
      store_tile<64, 64, LD, true, true>(yt, ry);
    else
      store_tile<64, 64, LD, true, false>(yt, ry);
  }
  __syncthreads();
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  f32x4 acc[NT];
#pragma unroll
  for (int ct = 0; ct < NT; ++ct) acc[ct] = tile_f32(xt + 16 * ct * LD, LD, yt + 16 * w * LD, LD, 4, zero4());
  float* out = REV ? Br.dSt : Br.Sst;
  const size_t base = ((size_t)u.sq * Br.nch + u.ch) * DK;
#pragma unroll
  for (int ct = 0; ct < NT; ++ct)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      out[(base + 16 * ct + 4 * (l >> 4) + i) * P.dv + e0 + 16 * w + (l & 15)] = acc[ct][i];
}

// ---- the same increments for bf16 storage, on bf16 matrix cores ----
// X * F is carried as hi + lo bf16; Y = v is exact in bf16, Y = dLoss/do is
// split like X (products hi.hi + hi.lo + lo.hi; see k_bwd_mm1_split).  X^T and
// Y^T are staged as bf16 rows over the chunk's 64 positions (two k-slabs);
// wave w takes columns 16 w .. 16 w + 15 and every row tile.
__device__ __forceinline__ f32x4 slab_bf(const bf16* a, int lda, const bf16* b, int ldb, f32x4 acc) {
  const int l = threadIdx.x & 63;
  return mma_slab<bf16>(ld16(a + (l & 15) * lda + 8 * (l >> 4)), ld16(b + (l & 15) * ldb + 8 * (l >> 4)), acc);
}

// 8 positions of a column of a position-major fp32 matrix (rows t0 .. t0 + 7 at
// src + t * ld, zero from nvalid on), split into hi and lo bf16 packets
__device__ __forceinline__ void col8_split(const float* src, size_t ld, int t0, int nvalid, u32x4& hi, u32x4& lo) {
  float v[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) v[k] = src[(size_t)min(t0 + k, max(nvalid - 1, 0)) * ld];
#pragma unroll
  for (int k = 0; k < 8; ++k) v[k] = t0 + k < nvalid ? v[k] : 0.f;
  split_bf16(v, hi, lo);
}

template <int DK, bool REV>
__global__ __launch_bounds__(256) void k_bwd_outer_split(const BwdParams P) {
  constexpr int LB = 64 + 8, NT = DK / 16;
  constexpr int TPC = 256 / DK;              // threads per channel
  constexpr int GPT = (8 + TPC - 1) / TPC;   // 8-position groups per thread
  __shared__ __attribute__((aligned(16))) bf16 xh[DK * LB], xl[DK * LB];       // (X * F)^T [c][t]
  __shared__ __attribute__((aligned(16))) bf16 yh[64 * LB], yl[(REV ? 64 : 1) * LB];  // Y^T [e][t]
  int unit, slice;
  if (!xcd_item(P.total_units * (P.dv / 64), P.dv / 64, unit, slice)) return;
  const UnitPos u = unit_pos(P, unit);
  const BwdBranch& Br = P.br[u.bi];
  const int j0 = u.ch * P.C, e0 = slice * 64;
  const int nvalid = min(P.C, Br.n - j0);
  const size_t row0 = (size_t)u.sq * Br.np + j0;
  const int tid = threadIdx.x;
  {
    // X^T: thread = channel c (loads coalesced over channels), groups of 8 positions
    const int c = tid % DK;
    const float lastb = Br.lb[(row0 + P.C - 1) * DK + c];
#pragma unroll
    for (int gi = 0; gi < GPT; ++gi) {
      const int g = tid / DK + gi * TPC;
      if (g >= 8) break;
      float xv[8], lv[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const size_t o = (row0 + min(8 * g + k, nvalid - 1)) * DK + c;
        xv[k] = REV ? Br.q[o] : Br.k[o];
        lv[k] = Br.lb[o];
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float f = REV ? P.q_scale * xv[k] * __expf(lv[k]) : xv[k] * __expf(lastb - lv[k]);
        xv[k] = 8 * g + k < nvalid ? f : 0.f;
      }
      u32x4 hi, lo;
      split_bf16(xv, hi, lo);
      st16(xh + c * LB + 8 * g, hi);
      st16(xl + c * LB + 8 * g, lo);
    }
  }
  if constexpr (REV) {
    // dLoss/do^T: thread = column e (coalesced), position groups tid / 64 and + 4
    const int e = tid & 63;
    const float* src = Br.dob + ((size_t)(u.b * Br.n + j0) * Br.h + u.head) * P.dv + e0 + e;
#pragma unroll
    for (int gi = 0; gi < 2; ++gi) {
      const int g = (tid >> 6) + 4 * gi;
      u32x4 hi, lo;
      col8_split(src, (size_t)Br.h * P.dv, 8 * g, nvalid, hi, lo);
      st16(yh + e * LB + 8 * g, hi);
      st16(yl + e * LB + 8 * g, lo);
    }
  } else {
    // v^T rows straight from the chunk's v^T (exact in bf16), zero past the call's end
    const bf16* vT = reinterpret_cast<const bf16*>(Br.vT) + ((size_t)u.sq * Br.nch + u.ch) * P.dv * P.C;
    const int e = tid >> 2;
#pragma unroll
    for (int gi = 0; gi < 2; ++gi) {
      const int g = (tid & 3) + 4 * gi;
      const bool inc = 8 * g < P.C;
      float v8[8];
      unpack16<bf16>(ld16(vT + (size_t)(e0 + e) * P.C + (inc ? 8 * g : 0)), v8);
#pragma unroll
      for (int k = 0; k < 8; ++k) v8[k] = inc && 8 * g + k < nvalid ? v8[k] : 0.f;
      st16(yh + e * LB + 8 * g, pack16<bf16>(v8));
    }
  }
  __syncthreads();
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  f32x4 acc[NT];
#pragma unroll
  for (int ct = 0; ct < NT; ++ct) {
    acc[ct] = zero4();
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const bf16* a = xh + 16 * ct * LB + 32 * s;
      const bf16* al = xl + 16 * ct * LB + 32 * s;
      const bf16* b = yh + 16 * w * LB + 32 * s;
      acc[ct] = slab_bf(a, LB, b, LB, acc[ct]);
      acc[ct] = slab_bf(al, LB, b, LB, acc[ct]);
      if constexpr (REV) acc[ct] = slab_bf(a, LB, yl + 16 * w * LB + 32 * s, LB, acc[ct]);
    }
  }
  float* out = REV ? Br.dSt : Br.Sst;
  const size_t base = ((size_t)u.sq * Br.nch + u.ch) * DK;
#pragma unroll
  for (int ct = 0; ct < NT; ++ct)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      out[(base + 16 * ct + 4 * (l >> 4) + i) * P.dv + e0 + 16 * w + (l & 15)] = acc[ct][i];
}

// ---- chunk states by a walk over the chunks (bf16 storage) ----
// REV = false: Sst[c] = S entering chunk c:  S(0) = 0,    S(c+1) = Diag(lambda_c) S(c) + k-hat_c^T V_c;
// REV = true:  dSt[c] = G reaching c's end:  G(last) = 0, G(c-1) = Diag(lambda_c) G(c) + q-tilde_c^T dO_c;
// lambda_c = e^{b_last} of chunk c per key channel (the same values the increments
// and scans of the fp32 layer produce).  One workgroup per (branch, b, head,
// 64-column slice of d_v, 32-channel part of d_k) walks its sequence's chunks
// and keeps its 32 x 64 slice of the state in the accumulators of its four
// waves (wave w: columns 16 w .. 16 w + 15, both 16-channel tiles).  Per chunk
// it writes the slice, scales its rows by lambda and adds the chunk's increment
// on bf16 matrix cores (hi + lo operands, see k_bwd_mm1_split); the operands of
// the next two chunks are loaded while the current one is multiplied (the
// barriers wait for LDS only).  Block ids go round-robin over the XCDs, which
// spreads the long walks of the scale-1 branch over all of them.
template <int DK, bool REV, int CP>
__global__ __launch_bounds__(256) void k_bwd_walk(const BwdParams P) {
  constexpr int LB = 64 + 8, NCP = DK / CP, NCT = CP / 16, XG = CP * 64 / 8 / 256;
  __shared__ __attribute__((aligned(16))) bf16 xh[CP * LB], xl[CP * LB];              // (X * F)^T [c][t]
  __shared__ __attribute__((aligned(16))) bf16 yh[64 * LB], yl[(REV ? 64 : 1) * LB];  // Y^T [e][t]
  const int wunit = blockIdx.x;
  if (wunit >= P.walk_units) return;
  int bi = 0;
  while (bi + 1 < P.nbranch && wunit >= P.br[bi + 1].walk_begin) ++bi;
  const BwdBranch& Br = P.br[bi];
  const int ns = P.dv / 64;
  int local = wunit - Br.walk_begin;
  const int cp = local % NCP;
  local /= NCP;
  const int es = local % ns, sq = local / ns;
  const int c0 = CP * cp, e0 = 64 * es;
  const int b = sq / Br.h, head = sq - b * Br.h;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int nch = Br.nch;
  // staging pieces.  X: channel xc, positions 8 xg .. 8 xg + 7.  Y: v^T row
  // e = tid / 4 with positions 8 (tid % 4) and + 32 (forward), or dLoss/do
  // column e = tid % 64 with positions 8 (tid / 64) and + 32 (reverse)
  const int xc = tid % CP, xg0 = tid / CP;
  struct Regs {
    float xv[XG][8], lv[XG][8], lastb, lam[NCT][4];
    float dv8[2][8];
    u32x4 vv[2];
  };
  auto load = [&](Regs& R, int ch) {
    const int j0 = ch * P.C, nvalid = min(P.C, Br.n - j0);
    const size_t row0 = (size_t)sq * Br.np + j0;
#pragma unroll
    for (int gi = 0; gi < XG; ++gi) {
      const int xg = xg0 + (256 / CP) * gi;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const size_t o = (row0 + min(8 * xg + k, nvalid - 1)) * DK + c0 + xc;
        R.xv[gi][k] = REV ? Br.q[o] : Br.k[o];
        R.lv[gi][k] = Br.lb[o];
      }
    }
    R.lastb = Br.lb[(row0 + P.C - 1) * DK + c0 + xc];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) R.lam[ct][i] = Br.lb[(row0 + P.C - 1) * DK + c0 + 16 * ct + 4 * (l >> 4) + i];
    if constexpr (REV) {
      const float* src = Br.dob + ((size_t)(b * Br.n + j0) * Br.h + head) * P.dv + e0 + (tid & 63);
      const size_t ld = (size_t)Br.h * P.dv;
#pragma unroll
      for (int gi = 0; gi < 2; ++gi) {
        const int g = (tid >> 6) + 4 * gi;
#pragma unroll
        for (int k = 0; k < 8; ++k) R.dv8[gi][k] = src[(size_t)min(8 * g + k, nvalid - 1) * ld];
      }
    } else {
      const bf16* vT = reinterpret_cast<const bf16*>(Br.vT) + (((size_t)sq * nch + ch) * P.dv + e0 + (tid >> 2)) * P.C;
#pragma unroll
      for (int gi = 0; gi < 2; ++gi) {
        const int g = (tid & 3) + 4 * gi;
        R.vv[gi] = ld16(vT + (8 * g < P.C ? 8 * g : 0));
      }
    }
  };
  auto stage = [&](Regs& R, int ch) {
    const int nvalid = min(P.C, Br.n - ch * P.C);
    u32x4 hi, lo;
#pragma unroll
    for (int gi = 0; gi < XG; ++gi) {
      const int xg = xg0 + (256 / CP) * gi;
      float f[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float v = REV ? P.q_scale * R.xv[gi][k] * __expf(R.lv[gi][k]) : R.xv[gi][k] * __expf(R.lastb - R.lv[gi][k]);
        f[k] = 8 * xg + k < nvalid ? v : 0.f;
      }
      split_bf16(f, hi, lo);
      st16(xh + xc * LB + 8 * xg, hi);
      st16(xl + xc * LB + 8 * xg, lo);
    }
    if constexpr (REV) {
#pragma unroll
      for (int gi = 0; gi < 2; ++gi) {
        const int g = (tid >> 6) + 4 * gi;
        float d8[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) d8[k] = 8 * g + k < nvalid ? R.dv8[gi][k] : 0.f;
        split_bf16(d8, hi, lo);
        st16(yh + (tid & 63) * LB + 8 * g, hi);
        st16(yl + (tid & 63) * LB + 8 * g, lo);
      }
    } else {
#pragma unroll
      for (int gi = 0; gi < 2; ++gi) {
        const int g = (tid & 3) + 4 * gi;
        u32x4 v = R.vv[gi];
        if (8 * g + 8 > nvalid) {  // a position past the call's end (or the chunk) in this piece
          float v8[8];
          unpack16<bf16>(v, v8);
#pragma unroll
          for (int k = 0; k < 8; ++k) v8[k] = 8 * g + k < nvalid ? v8[k] : 0.f;
          v = pack16<bf16>(v8);
        }
        st16(yh + (tid >> 2) * LB + 8 * g, v);
      }
    }
  };
  float* out = REV ? Br.dSt : Br.Sst;
  f32x4 acc[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) acc[ct] = zero4();
  auto chunk = [&](int it) { return REV ? nch - 1 - it : it; };
  // one walk step: the operands of step it (in R) go to LDS and R takes those
  // of step it + 2
  auto step = [&](Regs& R, int it) {
    const int ch = chunk(it);
    float lc[NCT][4];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) lc[ct][i] = __expf(R.lam[ct][i]);
    lds_barrier();  // the previous chunk's products are done with the LDS tiles
    stage(R, ch);
    lds_barrier();
    if (it + 2 < nch) load(R, chunk(it + 2));
    const size_t base = ((size_t)sq * nch + ch) * DK + c0;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        out[(base + 16 * ct + 4 * (l >> 4) + i) * P.dv + e0 + 16 * w + (l & 15)] = acc[ct][i];
        acc[ct][i] *= lc[ct][i];
      }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const bf16* bh = yh + 16 * w * LB + 32 * s;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const bf16* ah = xh + 16 * ct * LB + 32 * s;
        acc[ct] = slab_bf(ah, LB, bh, LB, acc[ct]);
        acc[ct] = slab_bf(xl + 16 * ct * LB + 32 * s, LB, bh, LB, acc[ct]);
        if constexpr (REV) acc[ct] = slab_bf(ah, LB, yl + 16 * w * LB + 32 * s, LB, acc[ct]);
      }
    }
  };
  Regs ra, rb;
  if (nch > 0) load(ra, chunk(0));
  if (nch > 1) load(rb, chunk(1));
  for (int it = 0; it < nch; it += 2) {
    step(ra, it);
    if (it + 1 < nch) step(rb, it + 1);
  }
}

// ---- scan over chunks, in place: buf[c] <- carried value entering chunk c ----
// forward (S):  S_prev(c+1) = Diag(lambda_c) S_prev(c) + dS_c, S_prev(0) = 0
// reverse (dS): G(c-1)      = Diag(lambda_c) G(c) + dG_c,     G(last) = 0
// lambda_c = e^{b_last} of chunk c (per key channel).  One thread per element;
// blockIdx.y = branch, so every branch scans in one launch.
__global__ __launch_bounds__(256) void k_bwd_scan(const BwdParams P, int rev) {
  const BwdBranch& Br = P.br[blockIdx.y];
  float* buf = rev ? Br.dSt : Br.Sst;
  const int nch = Br.nch;
  const size_t total = (size_t)P.B * Br.h * P.dk * P.dv;
  for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (size_t)gridDim.x * blockDim.x) {
    const size_t sq = idx / ((size_t)P.dk * P.dv);
    const int rem = (int)(idx - sq * P.dk * P.dv);
    const int c = rem / P.dv, e = rem - c * P.dv;
    float S = 0.f;
#pragma unroll 4
    for (int it = 0; it < nch; ++it) {
      const int ch = rev ? nch - 1 - it : it;
      const size_t o = ((sq * nch + ch) * P.dk + c) * P.dv + e;
      const float lam = __expf(Br.lb[(sq * Br.np + (size_t)ch * P.C + P.C - 1) * P.dk + c]);
      const float t = buf[o];
      buf[o] = S;
      S = lam * S + t;
    }
  }
}

// ---- the chunk's dense products on the matrix cores: do S_prev^T, v dS_end^T, D ----
// Over d_v in 32-column steps (do, v, S and dS staged in LDS): wave w takes rows
// 16 w .. 16 w + 15 of do S^T and v dS^T (every column tile) and of
// D = do v^T (D_ti for t >= i, zero elsewhere and outside the call).
template <typename T, int DK>
__global__ __launch_bounds__(256) void k_bwd_mm1(const BwdParams P) {
  constexpr int EC = 32, LD = EC + 4, NT = DK / 16;
  __shared__ __attribute__((aligned(16))) float dos[64 * LD];
  __shared__ __attribute__((aligned(16))) float vs[64 * LD];
  __shared__ __attribute__((aligned(16))) float ss[DK * LD];
  __shared__ __attribute__((aligned(16))) float dss[DK * LD];
  const UnitPos u = unit_pos(P, blockIdx.x);
  const BwdBranch& Br = P.br[u.bi];
  const int j0 = u.ch * P.C;
  const int nvalid = min(P.C, Br.n - j0);
  const size_t sbase = ((size_t)u.sq * Br.nch + u.ch) * DK;
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  f32x4 aq[NT], ak[NT], ad[4];
#pragma unroll
  for (int ct = 0; ct < NT; ++ct) aq[ct] = ak[ct] = zero4();
#pragma unroll
  for (int j = 0; j < 4; ++j) ad[j] = zero4();
  // the next step's four tiles are loaded into registers while this step's
  // products run, and stored to LDS after them
  float rd[64 * EC / 256], rv[64 * EC / 256], rs_[DK * EC / 256], rds[DK * EC / 256];
  auto load_step = [&](int e0) {
    load_tile<64, EC, true>(rd, [&](int t, int e) {
      const bool ok = t < nvalid;
      const float v = Br.dob[((size_t)(u.b * Br.n + j0 + (ok ? t : 0)) * Br.h + u.head) * P.dv + e0 + e];
      return ok ? v : 0.f;
    });
    load_tile<64, EC, false>(rv, [&](int t, int e) {
      const bool ok = t < nvalid;
      const float v = to_f32(reinterpret_cast<const T*>(Br.vT)[(((size_t)u.sq * Br.nch + u.ch) * P.dv + e0 + e) * P.C + (ok ? t : 0)]);
      return ok ? v : 0.f;
    });
    load_tile<DK, EC, true>(rs_, [&](int c, int e) { return Br.Sst[(sbase + c) * P.dv + e0 + e]; });
    load_tile<DK, EC, true>(rds, [&](int c, int e) { return Br.dSt[(sbase + c) * P.dv + e0 + e]; });
  };
  load_step(0);
  for (int e0 = 0; e0 < P.dv; e0 += EC) {
    store_tile<64, EC, LD, true, false>(dos, rd);
    store_tile<64, EC, LD, false, false>(vs, rv);
    store_tile<DK, EC, LD, true, false>(ss, rs_);
    store_tile<DK, EC, LD, true, false>(dss, rds);
    __syncthreads();
    if (e0 + EC < P.dv) load_step(e0 + EC);
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) {
      aq[ct] = tile_f32(dos + 16 * w * LD, LD, ss + 16 * ct * LD, LD, EC / 16, aq[ct]);
      ak[ct] = tile_f32(vs + 16 * w * LD, LD, dss + 16 * ct * LD, LD, EC / 16, ak[ct]);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) ad[j] = tile_f32(dos + 16 * w * LD, LD, vs + 16 * j * LD, LD, EC / 16, ad[j]);
    __syncthreads();
  }
  float* QK = Br.QKi + ((size_t)u.sq * Br.nch + u.ch) * 2 * 64 * DK;
  float* D = Br.AD + ((size_t)u.sq * Br.nch + u.ch) * 64 * 64;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = 16 * w + 4 * (l >> 4) + i;
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) {
      QK[t * DK + 16 * ct + (l & 15)] = aq[ct][i];
      QK[64 * DK + t * DK + 16 * ct + (l & 15)] = ak[ct][i];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = 16 * j + (l & 15);
      D[t * 64 + c] = (c <= t && t < nvalid) ? ad[j][i] : 0.f;
    }
  }
}

// ---- the same products for bf16 storage, on bf16 matrix cores ----
// Each fp32 operand (do, S, dS) is carried as hi + lo bf16 (hi = bf16(x),
// lo = bf16(x - hi)) and a product as hi.hi + hi.lo + lo.hi, fp32 accumulate:
// the dropped lo.lo term and lo's rounding leave about 2^-16 of each product.
// v is exact in bf16 (its storage type), so its products take two terms.
// Over d_v in 32-column steps (one bf16 k-slab): LDS planes of bf16 rows; wave w
// takes rows 16 w .. 16 w + 15 as in the fp32 kernel.
template <int DK>
__global__ __launch_bounds__(256) void k_bwd_mm1_split(const BwdParams P) {
  constexpr int EC = 32, LB = EC + 8, NT = DK / 16;
  constexpr int SG = (DK * EC / 8 + 255) / 256;  // 8-column groups of S (and dS) per thread
  __shared__ __attribute__((aligned(16))) bf16 doh[64 * LB], dol[64 * LB], vh[64 * LB];
  __shared__ __attribute__((aligned(16))) bf16 sh[DK * LB], sl[DK * LB], dsh[DK * LB], dsl[DK * LB];
  const UnitPos u = unit_pos(P, blockIdx.x);
  const BwdBranch& Br = P.br[u.bi];
  const int j0 = u.ch * P.C;
  const int nvalid = min(P.C, Br.n - j0);
  const size_t sbase = ((size_t)u.sq * Br.nch + u.ch) * DK;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const bf16* vT = reinterpret_cast<const bf16*>(Br.vT) + ((size_t)u.sq * Br.nch + u.ch) * P.dv * P.C;
  f32x4 aq[NT], ak[NT], ad[4];
#pragma unroll
  for (int ct = 0; ct < NT; ++ct) aq[ct] = ak[ct] = zero4();
#pragma unroll
  for (int j = 0; j < 4; ++j) ad[j] = zero4();
  // thread's pieces: do row tid / 4, columns 8 (tid % 4) ..; v column e = tid / 8
  // (of the step), positions 8 (tid % 8) ..; S and dS rows tid / 4 + 64 g
  const int dr = tid >> 2, dc = 8 * (tid & 3);
  const int ve = tid >> 3, vt = 8 * (tid & 7);
  const bool dok = dr < nvalid, vok = vt < P.C;
  const float* dsrc = Br.dob + ((size_t)(u.b * Br.n + j0 + (dok ? dr : 0)) * Br.h + u.head) * P.dv + dc;
  float rd[8], rs_[SG][8], rds[SG][8];
  u32x4 rv;
  auto load_step = [&](int e0) {
    unpack16<float>(ld16(dsrc + e0), rd);
    unpack16<float>(ld16(dsrc + e0 + 4), rd + 4);
    rv = ld16(vT + (size_t)(e0 + ve) * P.C + (vok ? vt : 0));
#pragma unroll
    for (int g = 0; g < SG; ++g) {
      const int c = min(dr + 64 * g, DK - 1);
      const float* ps = Br.Sst + (sbase + c) * P.dv + e0 + dc;
      const float* pd = Br.dSt + (sbase + c) * P.dv + e0 + dc;
      unpack16<float>(ld16(ps), rs_[g]);
      unpack16<float>(ld16(ps + 4), rs_[g] + 4);
      unpack16<float>(ld16(pd), rds[g]);
      unpack16<float>(ld16(pd + 4), rds[g] + 4);
    }
  };
  auto store_step = [&]() {
    u32x4 hi, lo;
    if (!dok)
#pragma unroll
      for (int k = 0; k < 8; ++k) rd[k] = 0.f;
    split_bf16(rd, hi, lo);
    st16(doh + dr * LB + dc, hi);
    st16(dol + dr * LB + dc, lo);
    {
      // every row is written: zero past the call's end and past the chunk (C < 64)
      float v8[8];
      unpack16<bf16>(rv, v8);
#pragma unroll
      for (int k = 0; k < 8; ++k) vh[(vt + k) * LB + ve] = (bf16)(vok && vt + k < nvalid ? v8[k] : 0.f);
    }
#pragma unroll
    for (int g = 0; g < SG; ++g) {
      const int c = dr + 64 * g;
      if (c < DK) {
        split_bf16(rs_[g], hi, lo);
        st16(sh + c * LB + dc, hi);
        st16(sl + c * LB + dc, lo);
        split_bf16(rds[g], hi, lo);
        st16(dsh + c * LB + dc, hi);
        st16(dsl + c * LB + dc, lo);
      }
    }
  };
  load_step(0);
  for (int e0 = 0; e0 < P.dv; e0 += EC) {
    store_step();
    lds_barrier();  // LDS only: the next step's loads below stay in flight past the barriers
    if (e0 + EC < P.dv) load_step(e0 + EC);
    const bf16* ra = doh + 16 * w * LB;
    const bf16* rl = dol + 16 * w * LB;
    const bf16* rvv = vh + 16 * w * LB;
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) {
      aq[ct] = slab_bf(ra, LB, sh + 16 * ct * LB, LB, aq[ct]);
      aq[ct] = slab_bf(ra, LB, sl + 16 * ct * LB, LB, aq[ct]);
      aq[ct] = slab_bf(rl, LB, sh + 16 * ct * LB, LB, aq[ct]);
      ak[ct] = slab_bf(rvv, LB, dsh + 16 * ct * LB, LB, ak[ct]);
      ak[ct] = slab_bf(rvv, LB, dsl + 16 * ct * LB, LB, ak[ct]);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ad[j] = slab_bf(ra, LB, vh + 16 * j * LB, LB, ad[j]);
      ad[j] = slab_bf(rl, LB, vh + 16 * j * LB, LB, ad[j]);
    }
    lds_barrier();
  }
  float* QK = Br.QKi + ((size_t)u.sq * Br.nch + u.ch) * 2 * 64 * DK;
  float* D = Br.AD + ((size_t)u.sq * Br.nch + u.ch) * 64 * 64;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = 16 * w + 4 * (l >> 4) + i;
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) {
      QK[t * DK + 16 * ct + (l & 15)] = aq[ct][i];
      QK[64 * DK + t * DK + 16 * ct + (l & 15)] = ak[ct][i];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = 16 * j + (l & 15);
      D[t * 64 + c] = (c <= t && t < nvalid) ? ad[j][i] : 0.f;
    }
  }
}

// ---- dv_i = sum_{t>=i} A_ti do_t + k-hat_i dS_end, into the v columns of dP ----
// On the matrix cores: rows i, columns e of the block's 64-column slice; wave w
// takes rows 16 w .. 16 w + 15.  A is the forward's (K2a's, in the storage
// type); A^T and do^T are staged with positions along k; then k-hat and
// dS_end^T in 32-channel steps.
template <typename T, int DK>
__global__ __launch_bounds__(256) void k_bwd_dv(const BwdParams P) {
  constexpr int LD = 68, CW = DK < 32 ? DK : 32, LDC = CW + 4;
  __shared__ __attribute__((aligned(16))) float at[64 * LD];   // A^T [i][t]
  __shared__ __attribute__((aligned(16))) float dt[64 * LD];   // do^T [e][t]
  __shared__ __attribute__((aligned(16))) float kh[64 * LDC];  // k-hat [i][c]
  __shared__ __attribute__((aligned(16))) float dst[64 * LDC]; // dS_end^T [e][c]
  int unit, slice;
  if (!xcd_item(P.total_units * (P.dv / 64), P.dv / 64, unit, slice)) return;
  const UnitPos u = unit_pos(P, unit);
  const BwdBranch& Br = P.br[u.bi];
  const int j0 = u.ch * P.C, e0 = slice * 64;
  const int nvalid = min(P.C, Br.n - j0);
  const size_t row0 = (size_t)u.sq * Br.np + j0;
  const size_t sbase = ((size_t)u.sq * Br.nch + u.ch) * DK;
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const T* A = reinterpret_cast<const T*>(Br.A) + ((size_t)u.sq * Br.nch + u.ch) * P.C * P.C;
  float rk[64 * CW / 256], rd[CW * 64 / 256];
  auto load_step = [&](int c0) {
    load_tile<64, CW, true>(rk, [&](int tt, int cc) {
      const bool ok = tt < nvalid;
      const size_t o = (row0 + (ok ? tt : 0)) * DK + c0 + cc;
      const float v = Br.k[o] * __expf(Br.lb[(row0 + P.C - 1) * DK + c0 + cc] - Br.lb[o]);
      return ok ? v : 0.f;
    });
    load_tile<CW, 64, true>(rd, [&](int cc, int e) { return Br.dSt[(sbase + c0 + cc) * P.dv + e0 + e]; });
  };
  {
    float ra[16], rt[16];
    // rows past the call's end hold no position (and no defined A): zero
    load_tile<64, 64, true>(ra, [&](int tt, int i) {
      const bool ok = tt < nvalid && i < P.C;
      const float v = to_f32(A[(ok ? tt : 0) * P.C + (ok ? i : 0)]);
      return ok ? v : 0.f;
    });
    load_tile<64, 64, true>(rt, [&](int tt, int e) {
      const bool ok = tt < nvalid;
      const float v = Br.dob[((size_t)(u.b * Br.n + j0 + (ok ? tt : 0)) * Br.h + u.head) * P.dv + e0 + e];
      return ok ? v : 0.f;
    });
    load_step(0);
    store_tile<64, 64, LD, true, true>(at, ra);
    store_tile<64, 64, LD, true, true>(dt, rt);
  }
  __syncthreads();
  f32x4 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = tile_f32(at + 16 * w * LD, LD, dt + 16 * j * LD, LD, 4, zero4());
  for (int c0 = 0; c0 < DK; c0 += CW) {
    __syncthreads();
    store_tile<64, CW, LDC, true, false>(kh, rk);
    store_tile<CW, 64, LDC, true, true>(dst, rd);
    __syncthreads();
    if (c0 + CW < DK) load_step(c0 + CW);
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = tile_f32(kh + 16 * w * LDC, LDC, dst + 16 * j * LDC, LDC, CW / 16, acc[j]);
  }
  T* dP = reinterpret_cast<T*>(Br.dP);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 16 * w + 4 * (l >> 4) + i;
    if (r >= nvalid) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      dP[(size_t)(u.b * Br.n + j0 + r) * Br.NP + Br.col_v + u.head * P.dv + e0 + 16 * j + (l & 15)] =
          from_f32<T>(acc[j][i]);
  }
}

// ---- dv for bf16 storage, on bf16 matrix cores ----
// A^T do over the chunk's positions (A exact in bf16, do as hi + lo), then
// k-hat dS_end^T over the key channels in 64-channel steps (both as hi + lo);
// see k_bwd_mm1_split.  Wave w takes rows 16 w .. 16 w + 15, every column tile
// of the block's 64-column slice.  d_k >= 32 (one bf16 k-slab per 32 channels).
template <int DK>
__global__ __launch_bounds__(256) void k_bwd_dv_split(const BwdParams P) {
  constexpr int LB = 64 + 8, CW = DK < 64 ? DK : 64, LC = CW + 8, NS = CW / 32;
  constexpr int KG = 64 * CW / 8 / 256;  // k-hat 8-channel groups per thread
  static_assert(DK >= 32 && DK % 32 == 0, "whole bf16 k-slabs of channels");
  __shared__ __attribute__((aligned(16))) bf16 at[64 * LB];                   // A^T [i][t]
  __shared__ __attribute__((aligned(16))) bf16 dth[64 * LB], dtl[64 * LB];    // do^T [e][t]
  __shared__ __attribute__((aligned(16))) bf16 kh[64 * LC], kl[64 * LC];      // k-hat [i][c]
  __shared__ __attribute__((aligned(16))) bf16 sh[64 * LC], sl[64 * LC];      // dS_end^T [e][c]
  int unit, slice;
  if (!xcd_item(P.total_units * (P.dv / 64), P.dv / 64, unit, slice)) return;
  const UnitPos u = unit_pos(P, unit);
  const BwdBranch& Br = P.br[u.bi];
  const int j0 = u.ch * P.C, e0 = slice * 64;
  const int nvalid = min(P.C, Br.n - j0);
  const size_t row0 = (size_t)u.sq * Br.np + j0;
  const size_t sbase = ((size_t)u.sq * Br.nch + u.ch) * DK;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  {
    // A^T: thread = (row t, 8-column group), two rows; written transposed
    const bf16* A = reinterpret_cast<const bf16*>(Br.A) + ((size_t)u.sq * Br.nch + u.ch) * P.C * P.C;
    const int ig = tid & 7;
#pragma unroll
    for (int gi = 0; gi < 2; ++gi) {
      const int t = (tid >> 3) + 32 * gi;
      const bool ok = t < nvalid && 8 * ig < P.C;
      float a8[8];
      unpack16<bf16>(ld16(A + (size_t)(ok ? t : 0) * P.C + (ok ? 8 * ig : 0)), a8);
#pragma unroll
      for (int k = 0; k < 8; ++k) at[(8 * ig + k) * LB + t] = (bf16)(ok ? a8[k] : 0.f);
    }
    // do^T: thread = column e (coalesced), position groups tid / 64 and + 4
    const int e = tid & 63;
    const float* src = Br.dob + ((size_t)(u.b * Br.n + j0) * Br.h + u.head) * P.dv + e0 + e;
#pragma unroll
    for (int gi = 0; gi < 2; ++gi) {
      const int g = (tid >> 6) + 4 * gi;
      u32x4 hi, lo;
      col8_split(src, (size_t)Br.h * P.dv, 8 * g, nvalid, hi, lo);
      st16(dth + e * LB + 8 * g, hi);
      st16(dtl + e * LB + 8 * g, lo);
    }
  }
  f32x4 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = zero4();
  for (int c0 = 0; c0 < DK; c0 += CW) {
    // k-hat [i][c0 .. c0 + CW): thread = (row i, 8-channel group)
#pragma unroll
    for (int gi = 0; gi < KG; ++gi) {
      const int idx = tid + 256 * gi, i = idx / (CW / 8), cg = 8 * (idx % (CW / 8));
      const size_t o = (row0 + min(i, nvalid - 1)) * DK + c0 + cg;
      float k8[8], b8[8], bl8[8];
      unpack16<float>(ld16(Br.k + o), k8);
      unpack16<float>(ld16(Br.k + o + 4), k8 + 4);
      unpack16<float>(ld16(Br.lb + o), b8);
      unpack16<float>(ld16(Br.lb + o + 4), b8 + 4);
      const float* pl = Br.lb + (row0 + P.C - 1) * DK + c0 + cg;
      unpack16<float>(ld16(pl), bl8);
      unpack16<float>(ld16(pl + 4), bl8 + 4);
#pragma unroll
      for (int k = 0; k < 8; ++k) k8[k] = i < nvalid ? k8[k] * __expf(bl8[k] - b8[k]) : 0.f;
      u32x4 hi, lo;
      split_bf16(k8, hi, lo);
      st16(kh + i * LC + cg, hi);
      st16(kl + i * LC + cg, lo);
    }
    // dS_end^T [e][c]: thread = column e (coalesced over e), 8-channel groups
    {
      const int e = tid & 63;
#pragma unroll
      for (int g = tid >> 6; g < CW / 8; g += 4) {
        u32x4 hi, lo;
        col8_split(Br.dSt + (sbase + c0) * P.dv + e0 + e, P.dv, 8 * g, CW, hi, lo);
        st16(sh + e * LC + 8 * g, hi);
        st16(sl + e * LC + 8 * g, lo);
      }
    }
    __syncthreads();
    if (c0 == 0) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const bf16* a = at + 16 * w * LB + 32 * s;
          acc[j] = slab_bf(a, LB, dth + 16 * j * LB + 32 * s, LB, acc[j]);
          acc[j] = slab_bf(a, LB, dtl + 16 * j * LB + 32 * s, LB, acc[j]);
        }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const bf16* a = kh + 16 * w * LC + 32 * s;
        const bf16* al = kl + 16 * w * LC + 32 * s;
        const bf16* b = sh + 16 * j * LC + 32 * s;
        acc[j] = slab_bf(a, LC, b, LC, acc[j]);
        acc[j] = slab_bf(a, LC, sl + 16 * j * LC + 32 * s, LC, acc[j]);
        acc[j] = slab_bf(al, LC, b, LC, acc[j]);
      }
    __syncthreads();
  }
  bf16* dP = reinterpret_cast<bf16*>(Br.dP);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 16 * w + 4 * (l >> 4) + i;
    if (r >= nvalid) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      dP[(size_t)(u.b * Br.n + j0 + r) * Br.NP + Br.col_v + u.head * P.dv + e0 + 16 * j + (l & 15)] =
          (bf16)acc[j][i];
  }
}

// ---- dq and dk of a chunk's 32-channel slice; in-chunk suffix sums of q dq - k dk ----
// The dense parts (do S_prev^T and v dS_end^T) come from k_bwd_mm1; here the
// intra-chunk terms.  The chunk's positions form four blocks of 16, with e_J =
// 16 J + 15 the last position of block J.  b is non-increasing along the chunk,
// so for i in block J and t in a later block, e^{b_t - b_i} = e^{b_t - b_eJ}
// e^{b_eJ - b_i} with both factors <= 1:
//   dq_t (block w) += sum_{J<w} e^{b_t - b_eJ} * (D[t, block J] K~J),
//       K~J_ic = k_ic e^{b_eJ,c - b_ic};
//   dk_i (block w) += sum_{J>=w} e^{b_eJ - b_i} * (D[block J+1, i]^T Q~J),
//       Q~J_tc = q_tc e^{b_tc - b_eJ,c}, t in block J + 1;
// those products run on the matrix cores (fp32); the four diagonal blocks take
// one factor e^{-|b_t - b_i|} per pair.  Thread elements follow the MFMA
// accumulator layout: wave w, rows 16 w + 4 (lane / 16) + i, channel tiles ct,
// channel 16 ct + lane % 16.
template <typename T, int DK>
__global__ __launch_bounds__(256) void k_bwd_dqdk(const BwdParams P) {
  constexpr int CS = DK < 32 ? DK : 32;  // channels per block
  constexpr int NCT = CS / 16, LDD = 68, LQ = CS + 4, LT = 20, LR = CS + 1;
  __shared__ __attribute__((aligned(16))) float ds[64 * LDD];   // D[t][i]
  __shared__ __attribute__((aligned(16))) float qs[64 * LQ];    // q_scale q
  __shared__ __attribute__((aligned(16))) float ks[64 * LQ];
  __shared__ __attribute__((aligned(16))) float bs[64 * LQ];
  __shared__ __attribute__((aligned(16))) float kt[3 * CS * LT];  // K~J^T [J][c][i in block J]
  __shared__ __attribute__((aligned(16))) float qt[3 * CS * LT];  // Q~J^T [J][c][t in block J + 1]
  __shared__ float rs[64 * LR];
  int unit, slice;
  if (!xcd_item(P.total_units * (DK / CS), DK / CS, unit, slice)) return;
  const UnitPos u = unit_pos(P, unit);
  const BwdBranch& Br = P.br[u.bi];
  const int j0 = u.ch * P.C, c0 = slice * CS;
  const int nvalid = min(P.C, Br.n - j0);
  const size_t row0 = (size_t)u.sq * Br.np + j0;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, lr = l & 15, lg = l >> 4;
  const float* D = Br.AD + ((size_t)u.sq * Br.nch + u.ch) * 64 * 64;
  const float* QK = Br.QKi + ((size_t)u.sq * Br.nch + u.ch) * 2 * 64 * DK;
  {
    // one round trip for the four tiles
    auto at_ = [&](int tt, int cc) { return (row0 + (tt < nvalid ? tt : 0)) * DK + c0 + cc; };
    float r0[16], r1[64 * CS / 256], r2[64 * CS / 256], r3[64 * CS / 256];
    load_tile<64, 64, true>(r0, [&](int tt, int i) { return D[tt * 64 + i]; });
    load_tile<64, CS, true>(r1, [&](int tt, int cc) {
      const float v = P.q_scale * Br.q[at_(tt, cc)];
      return tt < nvalid ? v : 0.f;
    });
    load_tile<64, CS, true>(r2, [&](int tt, int cc) {
      const float v = Br.k[at_(tt, cc)];
      return tt < nvalid ? v : 0.f;
    });
    // rows past the chunk keep its last b (the gate adds nothing past the call's end)
    load_tile<64, CS, true>(r3, [&](int tt, int cc) { return Br.lb[(row0 + min(tt, P.C - 1)) * DK + c0 + cc]; });
    store_tile<64, 64, LDD, true, false>(ds, r0);
    store_tile<64, CS, LQ, true, false>(qs, r1);
    store_tile<64, CS, LQ, true, false>(ks, r2);
    store_tile<64, CS, LQ, true, false>(bs, r3);
  }
  // the inter-chunk parts of this thread's elements
  float aq[NCT][4], ak[NCT][4];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 16 * w + 4 * lg + i, c = c0 + 16 * ct + lr;
      aq[ct][i] = QK[t * DK + c];
      ak[ct][i] = QK[64 * DK + t * DK + c];
    }
  __syncthreads();
  for (int idx = tid; idx < 3 * CS * 16; idx += 256) {
    const int J = idx / (CS * 16), rem = idx - J * CS * 16, c = rem >> 4, i = rem & 15;
    const int tk = 16 * J + i, tq = tk + 16;
    const float be = bs[(16 * J + 15) * LQ + c];
    kt[(J * CS + c) * LT + i] = ks[tk * LQ + c] * __expf(be - bs[tk * LQ + c]);
    qt[(J * CS + c) * LT + i] = qs[tq * LQ + c] * __expf(bs[tq * LQ + c] - be);
  }
  __syncthreads();
  float bt[NCT][4], iq[NCT][4], ik[NCT][4];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      bt[ct][i] = bs[(16 * w + 4 * lg + i) * LQ + 16 * ct + lr];
      iq[ct][i] = ik[ct][i] = 0.f;
    }
  // off-diagonal blocks (wave-uniform loops)
  for (int J = 0; J < w; ++J)
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const f32x4 p = tile_f32(ds + 16 * w * LDD + 16 * J, LDD, kt + (J * CS + 16 * ct) * LT, LT, 1, zero4());
      const float be = bs[(16 * J + 15) * LQ + 16 * ct + lr];
#pragma unroll
      for (int i = 0; i < 4; ++i) iq[ct][i] += p[i] * __expf(bt[ct][i] - be);
    }
  for (int J = w; J < 3; ++J)
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      // A[i][t] = D[16 (J + 1) + t][16 w + i], four positions per lane
      f32x4 a;
#pragma unroll
      for (int j = 0; j < 4; ++j) a[j] = ds[(16 * (J + 1) + 4 * lg + j) * LDD + 16 * w + lr];
      const f32x4 p = mma_slab<float>(__builtin_bit_cast(u32x4, a),
                                      ld16(qt + (J * CS + 16 * ct + lr) * LT + 4 * lg), zero4());
      const float be = bs[(16 * J + 15) * LQ + 16 * ct + lr];
#pragma unroll
      for (int i = 0; i < 4; ++i) ik[ct][i] += p[i] * __expf(be - bt[ct][i]);
    }
  // the diagonal block, pair by pair
  for (int i2 = 16 * w; i2 < 16 * w + 16; ++i2) {
    float bi[NCT], ki[NCT], qi[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      bi[ct] = bs[i2 * LQ + 16 * ct + lr];
      ki[ct] = ks[i2 * LQ + 16 * ct + lr];
      qi[ct] = qs[i2 * LQ + 16 * ct + lr];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 16 * w + 4 * lg + i;
      const float dti = ds[t * LDD + i2];  // D_t,i2: zero unless i2 <= t
      const float dit = ds[i2 * LDD + t];  // D_i2,t: zero unless i2 >= t
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const float E = __expf(-fabsf(bt[ct][i] - bi[ct]));
        iq[ct][i] += dti * ki[ct] * E;
        ik[ct][i] += dit * qi[ct] * E;
      }
    }
  }
  T* dPq = reinterpret_cast<T*>(Br.dP) + (size_t)(u.b * Br.n + j0) * Br.NP + u.head * DK + c0;
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    const float blast = bs[(P.C - 1) * LQ + 16 * ct + lr];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 16 * w + 4 * lg + i, c = 16 * ct + lr;
      float dq = __expf(bt[ct][i]) * aq[ct][i] + iq[ct][i];
      float dk = __expf(blast - bt[ct][i]) * ak[ct][i] + ik[ct][i];
      if (t >= nvalid) dq = dk = 0.f;
      rs[t * LR + c] = qs[t * LQ + c] * dq - ks[t * LQ + c] * dk;
      if (t < nvalid) {
        dPq[(size_t)t * Br.NP + c] = from_f32<T>(P.q_scale * dq);
        dPq[(size_t)t * Br.NP + Br.col_k + c] = from_f32<T>(dk);
      }
    }
  }
  __syncthreads();
  if (tid < CS) {
    const int cc = tid;
    float run = 0.f;
    for (int tt = P.C - 1; tt >= 0; --tt) {
      run += rs[tt * LR + cc];
      Br.rsum[(row0 + tt) * DK + c0 + cc] = run;
    }
    Br.rtot[((size_t)u.sq * Br.nch + u.ch) * DK + c0 + cc] = run;
  }
}

// ---- the gate's gradients over one (branch, b, chunk) ----
// dz_tc = (sum over positions u >= t of q dq - k dk in channel c) * sigmoid(-z_tc) / gamma:
// the in-chunk suffix (rsum) plus the later chunks' totals (rtot).  From dz:
//   dg1 = dz W_g2^T into the gate columns of dP (fp32 MFMA over 128-channel
//   slices of dz staged in LDS),
//   and per (chunk, half of its rows) the sums of g1 dz (toward dW_g2 = g1^T dz)
//   and of dz (toward db_g) into gpart, summed over chunks by k_bwd_mcolsum_*.
// thread = (channel of the slice, half of the chunk's rows); wave w takes the
// dg1 tiles w, w + 4, ... of the chunk's (C / 16) x (RP / 16) tiles.
template <typename T, int RP>
__global__ __launch_bounds__(256) void k_bwd_gate_grads(const BwdParams P) {
  constexpr int SW = 128, LDZ = SW + 4, LDG = RP + 4;
  __shared__ __attribute__((aligned(16))) float dzs[64 * LDZ];   // dz [t][channel]
  __shared__ __attribute__((aligned(16))) float w2s[RP * LDZ];   // W_g2 [rank][channel]
  __shared__ __attribute__((aligned(16))) float g1s[64 * LDG];   // block means [t][rank]
  int bi = 0;
  while (bi + 1 < P.nbranch && (int)blockIdx.x >= P.br[bi + 1].gg_begin) ++bi;
  const BwdBranch& Br = P.br[bi];
  const int local = blockIdx.x - Br.gg_begin;
  const int b = local / Br.nch, ch = local - b * Br.nch;
  const int j0 = ch * P.C, nvalid = min(P.C, Br.n - j0);
  const int hdk = Br.h * P.dk, r = P.r;
  const int tid = threadIdx.x, cs = tid & (SW - 1), half = tid >> 7;
  const int w = tid >> 6, l = tid & 63;
  const size_t row0 = (size_t)b * Br.n + j0;  // the chunk's first pooled position row
  {
    // the block means of the chunk's rows; zero past the call's end and for ranks >= r
    constexpr int NG = 64 * RP / 256;
    float gv[NG];
#pragma unroll
    for (int k = 0; k < NG; ++k) {
      const int idx = tid + 256 * k, t = idx / RP, rr = idx - t * RP;
      const bool ok = t < nvalid && rr < r;
      gv[k] = Br.g1c[(row0 + (ok ? t : 0)) * P.rp + (ok ? rr : 0)];
    }
#pragma unroll
    for (int k = 0; k < NG; ++k) {
      const int idx = tid + 256 * k, t = idx / RP, rr = idx - t * RP;
      g1s[t * LDG + rr] = (t < nvalid && rr < r) ? gv[k] : 0.f;
    }
  }
  const int MT = P.C / 16, ntile = MT * (RP / 16);
  f32x4 acc[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) acc[k] = zero4();
  const int hr = P.C / 2, t0 = half * hr;
  __syncthreads();  // g1s
  for (int hc0 = 0; hc0 < hdk; hc0 += SW) {
    const int hc = hc0 + cs;
    const bool act = hc < hdk;
    const int hcc = act ? hc : hdk - 1;
    const int head = hcc / P.dk, c = hcc - head * P.dk;
    const size_t sq = (size_t)b * Br.h + head;
    {
      // the slice of W_g2 (its rows >= r are zero in the packed weights)
      constexpr int NW = RP * SW / 256;
      float wv[NW];
#pragma unroll
      for (int k = 0; k < NW; ++k) {
        const int idx = tid + 256 * k, rr = idx / SW, col = idx - rr * SW;
        wv[k] = Br.W2[(size_t)rr * hdk + min(hc0 + col, hdk - 1)];
      }
#pragma unroll
      for (int k = 0; k < NW; ++k) {
        const int idx = tid + 256 * k, rr = idx / SW, col = idx - rr * SW;
        w2s[rr * LDZ + col] = hc0 + col < hdk ? wv[k] : 0.f;
      }
    }
    // the later chunks' totals of this channel
    float suf = 0.f;
    for (int c2 = ch + 1; c2 < Br.nch; c2 += 8) {
      float v[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = Br.rtot[(sq * Br.nch + min(c2 + k, Br.nch - 1)) * P.dk + c];
#pragma unroll
      for (int k = 0; k < 8; ++k) suf += c2 + k < Br.nch ? v[k] : 0.f;
    }
    float bs = 0.f, aw[RP];
#pragma unroll
    for (int rr = 0; rr < RP; ++rr) aw[rr] = 0.f;
    for (int tb = 0; tb < hr; tb += 8) {
      float rv[8], sv[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const size_t o = (sq * Br.np + j0 + min(t0 + tb + k, nvalid - 1)) * P.dk + c;
        rv[k] = Br.rsum[o];
        sv[k] = Br.sg[o];
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int t = t0 + tb + k;
        const float dz = (act && t < nvalid) ? (rv[k] + suf) * sv[k] : 0.f;
        dzs[t * LDZ + cs] = dz;
        bs += dz;
#pragma unroll
        for (int q = 0; q < RP / 4; ++q) {
          float g4[4];
          unpack16<float>(ld16(g1s + t * LDG + 4 * q), g4);
#pragma unroll
          for (int i = 0; i < 4; ++i) aw[4 * q + i] += g4[i] * dz;
        }
      }
    }
    if (act) {
      float* gp = Br.gpart + (size_t)(2 * local + half) * (r + 1) * hdk + hc;
#pragma unroll
      for (int rr = 0; rr < RP; ++rr)
        if (rr < r) gp[(size_t)rr * hdk] = aw[rr];
      gp[(size_t)r * hdk] = bs;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int tt = w + 4 * k;
      if (tt < ntile) {
        const int mt = tt % MT, rt = tt / MT;
        acc[k] = tile_f32(dzs + 16 * mt * LDZ, LDZ, w2s + 16 * rt * LDZ, LDZ, SW / 16, acc[k]);
      }
    }
    __syncthreads();  // before the next slice overwrites dzs and w2s
  }
  T* dP = reinterpret_cast<T*>(Br.dP);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int tt = w + 4 * k;
    if (tt >= ntile) continue;
    const int mt = tt % MT, rt = tt / MT, rr = 16 * rt + (l & 15);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 16 * mt + 4 * (l >> 4) + i;
      if (t < nvalid && rr < r) dP[(row0 + t) * Br.NP + Br.col_g + rr] = from_f32<T>(acc[k][i]);
    }
  }
  // the columns past the rank (padding to whole K segments of the input-gradient
  // product) are zero
  const int pad0 = Br.col_g + r, npad = Br.NP - pad0;
  for (int idx = tid; idx < nvalid * npad; idx += 256) {
    const int t = idx / npad;
    dP[(row0 + t) * Br.NP + pad0 + (idx - t * npad)] = from_f32<T>(0.f);
  }
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
        load8<T>(reinterpret_cast<const T*>(Br.yv) + (((size_t)b * Br.h + hh) * Br.np + t) * P.dv + e, y8);
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
      const T* src = reinterpret_cast<const T*>(Br.yv) + (((size_t)b * Br.h + hh) * Br.np + j) * P.dv + e;
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
    const uint8_t* Mrow = P.mask ? P.mask + (size_t)b * P.L : nullptr;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int i = 0; i < P.nbranch; ++i) {
      const BwdBranch& Br = P.br[i];
      if (t >= Br.n * Br.s) continue;
      const int j = t / Br.s;
      const T* src = reinterpret_cast<const T*>(Br.dxp) + ((size_t)b * Br.n + j) * P.d + col;
      // Eq. (8): the block mean is sum M x / max(1, sum M)
      float inv = 1.f / (float)Br.s;
      if (Mrow) {
        if (!Mrow[t]) continue;
        int cnt = 0;
        for (int v = j * Br.s; v < (j + 1) * Br.s; ++v) cnt += Mrow[v] != 0;
        inv = 1.f / (float)max(cnt, 1);
      }
      float a[8];
      load8<T>(src, a);
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] += a[q] * inv;
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

// ---- the normalisation (config norm): dLoss/do from dLoss/d(normalised row) ----
// y = o g / r per head row, r = sqrt(mean o^2 + eps):
//   do_c = g_c dy_c / r - o_c (sum_c' g_c' dy_c' o_c') / (d_v r^3),
// written over dy in place; o_c dy_c / r goes to ngt for the gains' gradient.
// One wave per (pooled position, head).
template <typename T>
__global__ __launch_bounds__(256) void k_bwd_norm(const BwdParams P, int bi) {
  const BwdBranch& Br = P.br[bi];
  const int rh = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (rh >= P.B * Br.n * Br.h) return;
  const int row = rh / Br.h, hh = rh - row * Br.h;
  const int b = row / Br.n, j = row - b * Br.n;
  const T* o = reinterpret_cast<const T*>(Br.y) + (((size_t)b * Br.h + hh) * Br.np + j) * P.dv;
  float* dy = Br.dob + (size_t)rh * P.dv;
  const float* g = Br.gn + hh * P.dv;
  float ss = 0.f, inner = 0.f;
  for (int c = lane; c < P.dv; c += 64) {
    const float oc = to_f32(o[c]);
    ss += oc * oc;
    inner += g[c] * dy[c] * oc;
  }
  ss = wave_sum(ss);
  inner = wave_sum(inner);
  const float r = sqrtf(ss / (float)P.dv + NORM_EPS);
  const float ir = 1.f / r, k3 = inner / ((float)P.dv * r * r * r);
  for (int c = lane; c < P.dv; c += 64) {
    const float oc = to_f32(o[c]), dyc = dy[c];
    dy[c] = g[c] * dyc * ir - oc * k3;
    Br.ngt[(size_t)rh * P.dv + c] = oc * dyc * ir;
  }
}

// ---- a masked call's scale-1 branch: its pooled input is M_t x_t, so the rows
// of dP at masked positions carry nothing to x or to the weights: zero them ----
template <typename T>
__global__ __launch_bounds__(256) void k_bwd_mask_rows(const BwdParams P, int bi) {
  const BwdBranch& Br = P.br[bi];
  const int pieces = Br.NP / 8;
  const size_t total = (size_t)P.B * P.L * pieces;
  for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (size_t)gridDim.x * blockDim.x) {
    const size_t row = idx / pieces;
    if (P.mask[row]) continue;
    const float z[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    store8<T>(reinterpret_cast<T*>(Br.dP) + row * Br.NP + (idx - row * pieces) * 8, z);
  }
}

// ---- column sums and x^T dz, in two deterministic passes ----
// Several column sums in one pair of launches (ColsumJobs): the partial pass
// writes part[pofs + rb * cols + col] = sum over row block rb of src[row][col]
// (a block is 64 columns x 4 row lanes); the finishing pass adds the row blocks.
__global__ __launch_bounds__(256) void k_bwd_mcolsum_partial(const ColsumJobs J, float* part) {
  __shared__ float red[4][64];
  int j = 0;
  while (j + 1 < J.n && (int)blockIdx.x >= J.cb[j + 1]) ++j;
  if ((int)blockIdx.y >= J.nrb[j]) return;  // the whole block
  const int cc = threadIdx.x & 63, lane4 = threadIdx.x >> 6;
  const int rows = J.rows[j], cols = J.cols[j], ld = J.ld[j];
  const int col = ((int)blockIdx.x - J.cb[j]) * 64 + cc;
  const int rpb = (rows + J.nrb[j] - 1) / J.nrb[j];
  const int r0 = blockIdx.y * rpb, r1 = min(rows, r0 + rpb);
  const int colc = min(col, cols - 1);
  const float* src = J.src[j];
  float acc = 0.f;
  for (int rw = r0 + lane4; rw < r1; rw += 32) {
    float v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = src[(size_t)min(rw + 4 * k, r1 - 1) * ld + colc];
#pragma unroll
    for (int k = 0; k < 8; ++k) acc += (rw + 4 * k < r1) ? v[k] : 0.f;
  }
  red[lane4][cc] = acc;
  __syncthreads();
  if (lane4 == 0 && col < cols)
    part[J.pofs[j] + (size_t)blockIdx.y * cols + col] = red[0][cc] + red[1][cc] + red[2][cc] + red[3][cc];
}

__global__ __launch_bounds__(256) void k_bwd_mcolsum_finish(const ColsumJobs J, const float* part) {
  int j = 0;
  while (j + 1 < J.n && (int)blockIdx.x >= J.fb[j + 1]) ++j;
  const int cols = J.cols[j], nrb = J.nrb[j];
  const int col = ((int)blockIdx.x - J.fb[j]) * 256 + threadIdx.x;
  if (col >= cols) return;
  const float* p = part + J.pofs[j];
  float acc = 0.f;
  for (int rb0 = 0; rb0 < nrb; rb0 += 8) {
    float v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = p[(size_t)min(rb0 + k, nrb - 1) * cols + col];
#pragma unroll
    for (int k = 0; k < 8; ++k) acc += (rb0 + k < nrb) ? v[k] : 0.f;
  }
  J.dst[j][col] = acc;
}

// partial[rb][col][i] = sum over row block rb of x[row][col] dz[row][i], i < 8
template <typename T>
__global__ __launch_bounds__(256) void k_bwd_wf_partial(const BwdParams P, int rows_per_block, float* partial) {
  // 64 columns per block: lane = (8-column group, row lane); 32 row lanes, 8 per wave
  __shared__ float red[4][64][FUSION_STRIDE];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int cg = lane & 7, rl = (lane >> 3) + 8 * wv;
  const int col0 = blockIdx.x * 64 + 8 * cg;
  const int rows = P.B * P.L;
  const int r0 = blockIdx.y * rows_per_block, r1 = min(rows, r0 + rows_per_block);
  float acc[8][FUSION_STRIDE];
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int i = 0; i < FUSION_STRIDE; ++i) acc[c][i] = 0.f;
#pragma unroll 2
  for (int r = r0 + rl; r < r1; r += 32) {
    float xv[8];
    load8<T>(reinterpret_cast<const T*>(P.x) + (size_t)r * P.d + col0, xv);
    const f32x4 z0 = *reinterpret_cast<const f32x4*>(P.dz + (size_t)r * FUSION_STRIDE);
    const f32x4 z1 = *reinterpret_cast<const f32x4*>(P.dz + (size_t)r * FUSION_STRIDE + 4);
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[c][q] += xv[c] * z0[q];
        acc[c][q + 4] += xv[c] * z1[q];
      }
  }
  // the wave's 8 row lanes (lane bits 3..5), then its 4 waves through LDS
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int i = 0; i < FUSION_STRIDE; ++i)
      if (i < P.m) {
        float v = acc[c][i];
        v += __shfl_xor(v, 8, WAVE);
        v += __shfl_xor(v, 16, WAVE);
        v += __shfl_xor(v, 32, WAVE);
        acc[c][i] = v;
      }
  if (lane < 8)
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
      for (int i = 0; i < FUSION_STRIDE; ++i) red[wv][8 * cg + c][i] = acc[c][i];
  __syncthreads();
  if (tid < 64) {
    const int col = blockIdx.x * 64 + tid;
#pragma unroll
    for (int i = 0; i < FUSION_STRIDE; ++i)
      if (i < P.m)
        partial[((size_t)blockIdx.y * P.d + col) * FUSION_STRIDE + i] =
            red[0][tid][i] + red[1][tid][i] + red[2][tid][i] + red[3][tid][i];
  }
}

// ---------------- launchers ----------------

template <typename T, int DK>
static void launch_chunk_kernels_t(const BwdParams& P, int which, hipStream_t st) {
  const int slices = P.dv / 64;
  // a flat grid over (unit, slice) items, 8 * ceil(items / 8) blocks (see xcd_item)
  auto xg = [&](int inner) { return dim3((unsigned)(((int64_t)P.total_units * inner + N_XCD - 1) / N_XCD * N_XCD)); };
  switch (which) {
    case 0:
      if constexpr (sizeof(T) == 2)
        hipLaunchKernelGGL((k_bwd_outer_split<DK, false>), xg(slices), dim3(256), 0, st, P);
      else
        hipLaunchKernelGGL((k_bwd_outer<T, DK, false>), xg(slices), dim3(256), 0, st, P);
      break;
    case 1:
      if constexpr (sizeof(T) == 2)
        hipLaunchKernelGGL((k_bwd_outer_split<DK, true>), xg(slices), dim3(256), 0, st, P);
      else
        hipLaunchKernelGGL((k_bwd_outer<T, DK, true>), xg(slices), dim3(256), 0, st, P);
      break;
    case 5:
      if constexpr (sizeof(T) == 2)
        hipLaunchKernelGGL((k_bwd_mm1_split<DK>), dim3(P.total_units), dim3(256), 0, st, P);
      else
        hipLaunchKernelGGL((k_bwd_mm1<T, DK>), dim3(P.total_units), dim3(256), 0, st, P);
      break;
    case 3:
      if constexpr (sizeof(T) == 2 && DK >= 32)
        hipLaunchKernelGGL((k_bwd_dv_split<DK>), xg(slices), dim3(256), 0, st, P);
      else
        hipLaunchKernelGGL((k_bwd_dv<T, DK>), xg(slices), dim3(256), 0, st, P);
      break;
    default: {
      const int cs = DK < 32 ? 1 : DK / 32;
      hipLaunchKernelGGL((k_bwd_dqdk<T, DK>), xg(cs), dim3(256), 0, st, P);
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

// which: 0 state increments, 1 state-gradient increments, 3 dv, 4 dq and dk,
// 5 the dense products do S^T, v dS^T and D
hipError_t launch_bwd_chunk(const BwdParams& P, int which, bool bf16_path, hipStream_t st) {
  if (P.total_units == 0) return hipSuccess;
  return bf16_path ? launch_chunk_kernels_dk<bf16>(P, which, st) : launch_chunk_kernels_dk<float>(P, which, st);
}

hipError_t launch_bwd_gate(const BwdParams& P, hipStream_t st) {
  if (P.total_units == 0) return hipSuccess;
  // block means, W_g2 slice, log alpha; the part totals (256 floats) reuse the first
  if (P.rp != 16 && P.rp != 64) return hipErrorInvalidValue;
  const size_t lds = (size_t)(std::max(P.C * P.rp, 256) + P.r * P.dk + P.C * P.dk) * sizeof(float);
  if (P.rp == 16) hipLaunchKernelGGL(k_bwd_gate<16>, dim3(P.total_units), dim3(256), lds, st, P);
  else hipLaunchKernelGGL(k_bwd_gate<64>, dim3(P.total_units), dim3(256), lds, st, P);
  return hipGetLastError();
}

// the state walks of every branch in one launch (bf16 storage), 32 channels per
// walk (64-channel walks, with half the restaging of the shared V or dO tile,
// took 1.5x as long: one workgroup per CU leaves each walk's latency exposed)
#define WALK_CP(DKV) 32
hipError_t launch_bwd_walk(const BwdParams& P, bool rev, hipStream_t st) {
  if (P.walk_units == 0) return hipSuccess;
  const dim3 grid(P.walk_units), block(256);
  switch (P.dk) {
#define MSGLA_WALK(DKV)                                                                         \
  case DKV:                                                                                     \
    if (rev) hipLaunchKernelGGL((k_bwd_walk<DKV, true, WALK_CP(DKV)>), grid, block, 0, st, P);  \
    else hipLaunchKernelGGL((k_bwd_walk<DKV, false, WALK_CP(DKV)>), grid, block, 0, st, P);     \
    break;
    MSGLA_WALK(32)
    MSGLA_WALK(64)
    MSGLA_WALK(128)
    MSGLA_WALK(256)
#undef MSGLA_WALK
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
#undef WALK_CP

// every branch's scan in one launch (blockIdx.y = branch)
hipError_t launch_bwd_scan(const BwdParams& P, bool rev, hipStream_t st) {
  size_t most = 0;
  for (int i = 0; i < P.nbranch; ++i) most = std::max(most, (size_t)P.B * P.br[i].h * P.dk * P.dv);
  if (most == 0 || P.nbranch == 0) return hipSuccess;
  const unsigned grid = (unsigned)std::min<size_t>((most + 255) / 256, 65536);
  hipLaunchKernelGGL(k_bwd_scan, dim3(grid, P.nbranch), dim3(256), 0, st, P, rev ? 1 : 0);
  return hipGetLastError();
}

// dz, dg1 and the dW_g2 / db_g partials of every branch in one launch
hipError_t launch_bwd_gate_grads(const BwdParams& P, bool bf16_path, hipStream_t st) {
  if (P.gate_units == 0) return hipSuccess;
  if (P.C % 16 != 0 || P.C > 64 || P.r > P.rp || (P.rp != 16 && P.rp != 64)) return hipErrorInvalidValue;
  const dim3 grid(P.gate_units);
  if (P.rp == 16) {
    if (bf16_path) hipLaunchKernelGGL((k_bwd_gate_grads<bf16, 16>), grid, dim3(256), 0, st, P);
    else hipLaunchKernelGGL((k_bwd_gate_grads<float, 16>), grid, dim3(256), 0, st, P);
  } else {
    if (bf16_path) hipLaunchKernelGGL((k_bwd_gate_grads<bf16, 64>), grid, dim3(256), 0, st, P);
    else hipLaunchKernelGGL((k_bwd_gate_grads<float, 64>), grid, dim3(256), 0, st, P);
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

hipError_t launch_bwd_mask_rows(const BwdParams& P, int bi, bool bf16_path, hipStream_t st) {
  const size_t total = (size_t)P.B * P.L * (P.br[bi].NP / 8);
  if (total == 0 || !P.mask) return hipSuccess;
  const unsigned grid = (unsigned)std::min<size_t>((total + 255) / 256, 65536);
  if (bf16_path) hipLaunchKernelGGL(k_bwd_mask_rows<bf16>, dim3(grid), dim3(256), 0, st, P, bi);
  else hipLaunchKernelGGL(k_bwd_mask_rows<float>, dim3(grid), dim3(256), 0, st, P, bi);
  return hipGetLastError();
}

hipError_t launch_bwd_norm(const BwdParams& P, int bi, bool bf16_path, hipStream_t st) {
  const int n = P.B * P.br[bi].n * P.br[bi].h;
  if (n == 0) return hipSuccess;
  const dim3 grid((n + 3) / 4);
  if (bf16_path) hipLaunchKernelGGL(k_bwd_norm<bf16>, grid, dim3(256), 0, st, P, bi);
  else hipLaunchKernelGGL(k_bwd_norm<float>, grid, dim3(256), 0, st, P, bi);
  return hipGetLastError();
}

hipError_t launch_bwd_dx(const BwdParams& P, bool bf16_path, hipStream_t st) {
  const size_t total = (size_t)P.B * P.L * (P.d / 8);
  const unsigned grid = (unsigned)std::min<size_t>((total + 255) / 256, 65536);
  if (bf16_path) hipLaunchKernelGGL(k_bwd_dx<bf16>, dim3(grid), dim3(256), 0, st, P);
  else hipLaunchKernelGGL(k_bwd_dx<float>, dim3(grid), dim3(256), 0, st, P);
  return hipGetLastError();
}

// every job of J (partials at part, J.pofs) in one pair of launches
hipError_t launch_bwd_mcolsum(const ColsumJobs& J, float* part, hipStream_t st) {
  if (J.n == 0 || J.cb[J.n] == 0) return hipSuccess;
  int nrb = 1;
  for (int j = 0; j < J.n; ++j) nrb = std::max(nrb, J.nrb[j]);
  hipLaunchKernelGGL(k_bwd_mcolsum_partial, dim3(J.cb[J.n], nrb), dim3(256), 0, st, J, part);
  hipLaunchKernelGGL(k_bwd_mcolsum_finish, dim3(J.fb[J.n]), dim3(256), 0, st, J, static_cast<const float*>(part));
  return hipGetLastError();
}

// partial [nrb][d][8]: x^T dz per row block, summed by k_bwd_wf_finish
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
// each owning a column range of the product: out_k[row][col - c0_k]; every
// split-K product of a backward in one launch.

__global__ __launch_bounds__(256) void k_bwd_splitk_reduce(const SplitJobs J) {
  // blockIdx.y = job; a grid-stride walk over its M x N sums
  const int j = blockIdx.y;
  if (j >= J.n) return;
  const int S = J.S[j], N = J.N[j];
  const size_t total = (size_t)J.M[j] * N;
  const float* part = J.part[j];
  const SplitDst& D = J.dst[j];
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

hipError_t launch_bwd_splitk_reduce(const SplitJobs& J, hipStream_t st) {
  if (J.n == 0) return hipSuccess;
  size_t most = 0;
  for (int j = 0; j < J.n; ++j) most = std::max(most, (size_t)J.M[j] * J.N[j]);
  const unsigned grid = (unsigned)std::min<size_t>((most + 255) / 256, 1024);
  hipLaunchKernelGGL(k_bwd_splitk_reduce, dim3(grid, J.n), dim3(256), 0, st, J);
  return hipGetLastError();
}

}  // namespace msgla
