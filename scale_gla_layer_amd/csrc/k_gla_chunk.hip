// K2a — chunk-local part of the gated linear recurrence, one workgroup per
// (branch, sequence, head, chunk), all chunks in parallel.
//
// MS-GLA notes, Sec. 2.1 (S_t = Diag(alpha_t) S_{t-1} + k_t^T v_t, o_t = q_t S_t,
// alpha from a low-rank projection through a sigmoid-type map) and Sec. 3.4
// (each branch reuses the chunkwise-parallel GLA algorithm; the chunk is a
// schedule, distinct from the pooling block).
//
// Within a chunk of C positions starting at c0, with b_t = sum_{c0<=u<=t} log alpha_u
// (per key channel, fp32), the recurrence unrolls to
//   o_t = q_t S_{c0-1} ⊙ e^{b_t} + sum_{c0<=i<=t} (sum_c q_tc k_ic e^{b_tc - b_ic}) v_i
//   S_{c0+C-1} = Diag(e^{b_last}) S_{c0-1} + sum_i (k_i ⊙ e^{b_last - b_i})^T v_i .
// This kernel computes everything that does not need the carried state:
//   lam   = e^{b_last}                          (per channel)
//   qt    = q ⊙ e^{b}          (inter-chunk query)
//   kT    = (k ⊙ e^{b_last - b})^T             (state-update key, transposed)
//   A     = [sum_c q_tc k_ic e^{b_tc - b_ic}]_{t >= i}   (zero above the diagonal)
// b is kept in base-2 units (log2 alpha), so every decay factor is one exp2.
// q and k arrive in fp32 (a single q_t . k_i can cancel strongly, and A scales
// whole output rows); A is formed from the fp32 operands (fp32 MFMA, or for
// bf16 storage three bf16 MFMA products of their hi/lo split) and rounded once
// to the storage type.
// Every stored factor has an exponent <= 0.  With e_J = 16 J + 15 the last
// position of 16-position tile J, the key side is referenced at the end of
// its own tile, kb_i = k_i e^{b_{e_J} - b_i} (<= |k_i|), so kT = kb e^{b_last -
// b_{e_J}} and every off-diagonal block A[T][J], J < T, is
// (q_t e^{b_t - b_16T}) . (kb_i D_TJ) with D_TJ = e^{b_16T - b_{e_J}} <= 1.
// The diagonal block A[T][T] has one growing factor, C_T = e^{b_16T - b_{e_T}}
// (the tile's own total decay, inverted): kb_i C_T.  It is used only while
// C_T <= 2^32 and kb C_T is finite for every channel of the tile (so |k| up
// to 2^96); otherwise that block is formed pair by pair, A[t][i] =
// sum_c q_tc k_ic prod_{u=i+1..t} alpha_uc, from the per-step decays alpha <= 1
// (exact for any gate, and some 8x slower, so it is reserved for tiles that
// decay by more than 2^-32).  Rows beyond the sequence end are treated as
// q = k = 0 and log alpha = 0, which leaves the state untouched.
//
// Work layout: wave w owns the 16 positions 16w .. 16w+15 of the chunk and all
// key channels.  Its gate pre-activations z^T = W_g2^T (xp W_g1)^T come from
// fp32 MFMA, so lane l holds channels 16 rt + 4 (l/16) + i of position
// 16 w + l % 16 for every channel tile rt.  The cumulative sum over positions
// is a DPP prefix scan inside each 16-lane row; the waves then exchange their
// totals (and first values) through LDS.  The key side of A (fp32, referenced
// at the end of its tile) goes to LDS; the query side stays in registers,
// referenced at the wave's first position, so it is formed once; wave w
// scales the key side of tile J by D_wJ (J < w, a per-channel table it fills
// in LDS) or C_w (J = w) and forms the blocks A[w][J] with MFMA as
// (key side)(query side)^T so that each lane holds 4 consecutive keys of one
// query row.  All shapes are compile-time (chunk C, key width DK, padded gate
// rank RP), so every loop unrolls.
#include "async_copy.hpp"
#include "device_common.hpp"
#include "layout.hpp"

namespace msgla {

template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL,
                                                               0xf, 0xf, true));
}

// inclusive prefix sum inside each row of 16 lanes (DPP row_shr 1, 2, 4, 8)
__device__ __forceinline__ float row_scan16(float x) {
  x += dpp_f<0x111>(x);
  x += dpp_f<0x112>(x);
  x += dpp_f<0x114>(x);
  x += dpp_f<0x118>(x);
  return x;
}

constexpr float K2A_LOG2E = 1.4426950408889634f;

// log2(sigmoid(z)) = min(z, 0) log2(e) - log2(1 + u), u = e^{-|z|} in (0, 1].
// log2(1 + u) is taken as log2(v) with v = 1 + u rounded, plus the first-order
// correction (u - (v - 1)) log2(e) for that rounding (the exact factor 1 / v
// differs from 1 by at most u, which leaves a relative error below 2^-23), so
// small u keep their relative accuracy.
__device__ __forceinline__ float log2sigmoid(float z) {
  const float u = __builtin_amdgcn_exp2f(-fabsf(z) * K2A_LOG2E);
  const float v = 1.f + u;
  return (fminf(z, 0.f) - (u - (v - 1.f))) * K2A_LOG2E - __builtin_amdgcn_logf(v);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// log2 of the largest growing factor the diagonal block may use (C_w <= 2^32)
constexpr float K2A_DIAG_LOG2_BOUND = 32.f;

template <typename T, int C, int DK>
struct K2aGeom {
  static constexpr int NW = C / 16;            // waves, one per 16-position tile
  static constexpr int NT = DK / 16;           // 16-channel tiles
  static constexpr int THREADS = 64 * NW;
  static constexpr bool BF = sizeof(T) == 2;
  // key-side rows in LDS (fp32), padded by 16 bytes against bank conflicts between rows
  static constexpr int KROW = DK * 4 + 16;
  static constexpr int XCH = 5 * NW * DK * 4;  // wave totals, first values, three factor tables
  static constexpr int KS = C * KROW;
  static constexpr int DT = NW * (NW - 1) * DK * 4;  // per wave: D_wJ for J < w
  static constexpr int LDS = XCH + KS + DT;  // 49 KB at C 64, d_k 128: three workgroups per CU
  static_assert(C == 16 || C == 32 || C == 64, "chunk");
  static_assert(BF ? (DK >= 32 && DK % 32 == 0) : (DK >= 16 && DK % 16 == 0), "key width");
};

template <typename T, int C, int DK, int RP>
__global__ __launch_bounds__(256) void k2a_gla_chunk(const K2Params P) {
  using G = K2aGeom<T, C, DK>;
  constexpr int NW = G::NW, NT = G::NT;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int unit = blockIdx.x;
  int bi = 0;
  while (bi + 1 < P.nbranch && unit >= P.br[bi + 1].unit_begin) ++bi;
  const K2Branch& Bb = P.br[bi];
  const int local = unit - Bb.unit_begin;
  const int chunk = local % Bb.nch;
  const int bh = local / Bb.nch;  // b * h + head
  const int b = bh / Bb.h, hh = bh - b * Bb.h;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  const int row0 = chunk * C;                  // first pooled row of the chunk
  // real rows in this chunk: the blocks this call completes (continuing from
  // a state, floor((L + r) / s) with r positions of block 0 pending on entry)
  const int valid = min(C, blocks_in_call(P.chk, bi, Bb.n) - row0);
  const int p = 16 * w + lr;                   // this lane's position in the chunk
  const bool live = p < valid;

  float* tot = reinterpret_cast<float*>(smem);  // [NW][DK] wave totals of log2 alpha
  float* first = tot + NW * DK;                 // [NW][DK] value at each wave's first row
  float* Ew = first + NW * DK + w * 3 * DK;     // [NW][3][DK] e^{b_16w}, e^{b_last - b_e}, C_w
  char* ks = smem + G::XCH;                     // key side [C][KROW] fp32
  float* Dw = reinterpret_cast<float*>(smem + G::XCH + G::KS) + w * (NW - 1) * DK;  // [J][DK]

  const size_t seq_row = (size_t)bh * Bb.np + row0;  // row index in [B][h][np]

  // ---- operands of this lane's position: q, k (4 channels per tile), gate factor ----
  // The head's W_g2 slice [RP][DK] and gate bias [DK] are copied global -> LDS
  // (into the key-side area, which is written only after the gate is formed)
  // while q and k load, so the gate MFMAs read them without a memory round
  // trip each; configurations where they do not fit read them from global.
  constexpr bool STAGE_W = RP * DK * 4 + 1024 <= G::KS;
  const int hdk = Bb.h * DK;
  float* w2s = reinterpret_cast<float*>(ks);  // [RP][DK]
  float* bgs = w2s + RP * DK;                 // [DK] (+ padding to 1 KB)
  if constexpr (STAGE_W) {
    constexpr int NI = RP * DK / 256;  // 1 KB copy instructions for W_g2
    const float* w2g = Bb.W2 + hh * DK;
    for (int k = w; k <= NI; k += NW) {
      const int q4 = 64 * k + lane;  // 16-byte piece
      const float* src;
      if (k < NI) {
        const int r = q4 / (DK / 4), c4 = q4 - r * (DK / 4);
        src = w2g + (size_t)r * hdk + 4 * c4;
      } else {
        src = Bb.bg + hh * DK + 4 * min(lane, DK / 4 - 1);
      }
      dma16(src, reinterpret_cast<char*>(w2s) + 1024 * k);
    }
  }

  // The gate factor loads first and q, k after it: the gate, its scan and the
  // waves' exchange need only the gate factor, so they run while q and k are
  // still in flight.  Every lane issues the same loads (dead positions load a
  // valid row and discard it), so the copies and the gate factor have landed
  // once only the 2 NT q / k loads remain.
  const int pl = live ? p : 0;
  // the gate's first factor of this lane's position (4 of its RP values per lane)
  auto load_gate_factor = [&](float (&gb)[RP / 4]) {
    // x W_g1 is given per unpooled position: the block's mean is this row's value
    const float* gr = Bb.g + ((size_t)b * P.L + (size_t)(row0 + pl) * Bb.s) * RP + lg;
    if (P.mask || P.chk) {
      // Eq. (8) in general: the block's mean over its tokens, sum M x W_g1 /
      // max(1, sum M) (for s = 1: M_t x_t W_g1; without a mask every
      // position is a token).  Continuing from a state, block j covers call
      // positions [j s - r, (j + 1) s - r): block 0 starts with the entry
      // state's pending positions, whose x W_g1 sum and token count it holds.
      const int t_lo = (row0 + pl) * Bb.s - entry_offset(P.chk, bi);
      const float* gq = Bb.g + (size_t)b * P.L * RP + lg;
      const uint8_t* mr = P.mask ? P.mask + (size_t)b * P.L : nullptr;
      float den = 0.f;
#pragma unroll
      for (int k4 = 0; k4 < RP / 4; ++k4) gb[k4] = 0.f;
      if (t_lo < 0 && Bb.psumg && state_in_ok(P.chk)) {
#pragma unroll
        for (int k4 = 0; k4 < RP / 4; ++k4) gb[k4] = Bb.psumg[(size_t)b * RP + 4 * k4 + lg];
        den = Bb.tok_in[b];
      }
      for (int u = 0; u < Bb.s; ++u) {
        const int t = t_lo + u;
        if (t < 0 || t >= P.L) continue;
        const float w = mr ? (mr[t] ? 1.f : 0.f) : 1.f;
        den += w;
#pragma unroll
        for (int k4 = 0; k4 < RP / 4; ++k4) gb[k4] += w * gq[(size_t)t * RP + 4 * k4];
      }
      const float sc = 1.0f / fmaxf(1.f, den);
#pragma unroll
      for (int k4 = 0; k4 < RP / 4; ++k4) gb[k4] *= sc;
    } else {
#pragma unroll
      for (int k4 = 0; k4 < RP / 4; ++k4) gb[k4] = gr[4 * k4];
      if (Bb.s > 1) {
        // three rows per round trip (dead slots reload the last row and are dropped)
        for (int u0 = 1; u0 < Bb.s; u0 += 3) {
          float t[3][RP / 4];
#pragma unroll
          for (int j = 0; j < 3; ++j) {
            const int u = min(u0 + j, Bb.s - 1);
#pragma unroll
            for (int k4 = 0; k4 < RP / 4; ++k4) t[j][k4] = gr[(size_t)u * RP + 4 * k4];
          }
#pragma unroll
          for (int j = 0; j < 3; ++j)
#pragma unroll
            for (int k4 = 0; k4 < RP / 4; ++k4) gb[k4] += u0 + j < Bb.s ? t[j][k4] : 0.f;
        }
        const float inv_s = 1.0f / (float)Bb.s;
#pragma unroll
        for (int k4 = 0; k4 < RP / 4; ++k4) gb[k4] *= inv_s;
      }
    }
#pragma unroll
    for (int k4 = 0; k4 < RP / 4; ++k4) gb[k4] = live ? gb[k4] : 0.f;
  };
  // log2 alpha of channel tile rt at this lane's position (z from fp32 MFMA) and
  // its inclusive scan over the wave's 16 positions
  auto gate_scan = [&](const float (&gb)[RP / 4], const float* w2, int w2stride, const float* bgp,
                       int rt, float (&xo)[4]) {
    f32x4 acc = __builtin_bit_cast(f32x4, ld16(bgp + 16 * rt + 4 * lg));  // gate bias
#pragma unroll
    for (int k4 = 0; k4 < RP / 4; ++k4)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(w2[(4 * k4 + lg) * w2stride + 16 * rt], gb[k4], acc, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float la = live ? log2sigmoid(acc[i]) * P.inv_gamma : 0.f;
      xo[i] = row_scan16(la);
    }
  };
  float gb[RP / 4];
  load_gate_factor(gb);
  asm volatile("" ::: "memory");  // keep the q / k loads behind the copies and the gate factor
  u32x4 qraw[NT], kraw[NT];
  {
    const float* qg = Bb.q + (seq_row + pl) * DK + 4 * lg;
    const float* kg = Bb.k + (seq_row + pl) * DK + 4 * lg;
#pragma unroll
    for (int rt = 0; rt < NT; ++rt) {
      qraw[rt] = ld16(qg + 16 * rt);
      kraw[rt] = ld16(kg + 16 * rt);
    }
  }
  asm volatile("" ::: "memory");

  // ---- z^T[c][t] = sum_r W2[r][c] g[t][r] (fp32 MFMA), then log2 alpha and its scan ----
  float x[NT][4];
  if constexpr (STAGE_W) {
    wait_vmcnt<2 * NT>();  // copies and gate factor landed; q, k may still be in flight
    lds_barrier();         // (a full fence here would wait for q and k too)
  }
  {
    const float* w2 = STAGE_W ? w2s + lr : Bb.W2 + hh * DK + lr;
    const int w2stride = STAGE_W ? DK : hdk;
    const float* bgp = STAGE_W ? bgs : Bb.bg + hh * DK;
#pragma unroll
    for (int rt = 0; rt < NT; ++rt) {
      gate_scan(gb, w2, w2stride, bgp, rt, x[rt]);
      if (lr == 15) st16(tot + w * DK + 16 * rt + 4 * lg, pack16<float>(x[rt]));
      if (lr == 0) st16(first + w * DK + 16 * rt + 4 * lg, pack16<float>(x[rt]));
    }
  }
  lds_barrier();  // the exchange is through LDS only; q and k may still be loading

  // ---- per channel (lane owns channels lane, lane + 64, ...): b at this wave's
  // first position b_16w = (totals of the earlier waves) + (first value) and at
  // its last b_e = (totals up to this wave); the factors e^{b_16w},
  // e^{b_last - b_e} and C_w = e^{b_16w - b_e} (LDS), D_wJ = e^{b_16w - b_{e_J}}
  // for J < w (LDS) and, from wave 0, lam = e^{b_last} (global).  A tile whose
  // decay e^{b_e - b_16w} is below 2^-32 in some channel forms its diagonal
  // block pair by pair ----
  bool exact_diag = false;
  {
    float* lamg = Bb.lam + ((size_t)bh * Bb.nch + chunk) * DK;
#pragma unroll
    for (int u = 0; u < (DK + 63) / 64; ++u) {
      const int ch = lane + 64 * u;
      if (ch < DK) {
        float carry = 0.f, blast = 0.f;
#pragma unroll
        for (int v = 0; v < NW; ++v) {
          const float tv = tot[v * DK + ch];
          blast += tv;
          if (v < w) carry += tv;
        }
        const float bw = carry + first[w * DK + ch];
        const float be = carry + tot[w * DK + ch];
        const float growth = first[w * DK + ch] - tot[w * DK + ch];  // log2 C_w >= 0
        exact_diag |= !(growth <= K2A_DIAG_LOG2_BOUND);
        Ew[ch] = exp2_fast(bw);
        Ew[DK + ch] = exp2_fast(blast - be);
        Ew[2 * DK + ch] = exp2_fast(fminf(growth, K2A_DIAG_LOG2_BOUND));
        if (w == 0) lamg[ch] = exp2_fast(blast);
        float cj = 0.f;
#pragma unroll
        for (int J = 0; J < NW - 1; ++J) {
          cj += tot[J * DK + ch];  // b at the end of tile J
          if (J < w) Dw[J * DK + ch] = exp2_fast(bw - cj);
        }
      }
    }
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (0 << 8));  // own LDS writes done
    asm volatile("" ::: "memory");
  }

  // ---- per element, with d = b_t - b_16w <= 0 and d_e = b_e - b_t <= 0 (this
  // lane's scan against the wave's first and last values): query side of A
  // q e^d (registers, in place of q), key side kb = k e^{d_e} (LDS),
  // qt = q e^{b_t} = (q e^d) e^{b_16w} and kT = k e^{b_last - b_t} =
  // kb e^{b_last - b_e} (global); kb C_w is checked for overflow ----
  float qv[NT][4], kv[NT][4];
#pragma unroll
  for (int rt = 0; rt < NT; ++rt) {
    unpack16<float>(live ? qraw[rt] : zero16(), qv[rt]);
    unpack16<float>(live ? kraw[rt] : zero16(), kv[rt]);
  }
  {
    T* qtg = reinterpret_cast<T*>(Bb.qt) + (seq_row + p) * DK + 4 * lg;
    T* kTg = reinterpret_cast<T*>(Bb.kT) + ((size_t)bh * Bb.nch + chunk) * DK * C;
    const int odd = lr & 1;
    char* krow = ks + p * G::KROW + 16 * lg;
#pragma unroll
    for (int rt = 0; rt < NT; ++rt) {
      float f4[4], t4[4], e1[4], e2[4], cw[4], qo[4], kb[4], kt[4];
      unpack16<float>(ld16(first + w * DK + 16 * rt + 4 * lg), f4);
      unpack16<float>(ld16(tot + w * DK + 16 * rt + 4 * lg), t4);
      unpack16<float>(ld16(Ew + 16 * rt + 4 * lg), e1);
      unpack16<float>(ld16(Ew + DK + 16 * rt + 4 * lg), e2);
      unpack16<float>(ld16(Ew + 2 * DK + 16 * rt + 4 * lg), cw);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float qs = qv[rt][i] * P.q_scale * exp2_fast(x[rt][i] - f4[i]);  // <= |q|
        qv[rt][i] = qs;
        qo[i] = qs * e1[i];
        kb[i] = kv[rt][i] * exp2_fast(t4[i] - x[rt][i]);  // <= |k|
        kt[i] = kb[i] * e2[i];
        exact_diag |= __builtin_isinf(kb[i] * cw[i]);
      }
      if constexpr (G::BF)
        st8(qtg + 16 * rt, pack8<T>(qo));
      else
        st16(qtg + 16 * rt, pack16<T>(qo));
      st16(krow + 64 * rt, pack16<float>(kb));
      // kT[c][t]: neighbouring lanes (positions p, p ^ 1) swap one value so that
      // the even lane stores channel c at (p, p + 1) and the odd lane channel
      // c + 1 at (p - 1, p), two consecutive elements per store
#pragma unroll
      for (int i = 0; i < 4; i += 2) {
        const float recv = dpp_f<0xB1>(odd ? kt[i] : kt[i + 1]);  // quad_perm [1, 0, 3, 2]
        const float pr[4] = {odd ? recv : kt[i], odd ? kt[i + 1] : recv, 0.f, 0.f};
        T* dst = kTg + (size_t)(16 * rt + 4 * lg + i + odd) * C + (p - odd);
        if constexpr (G::BF)
          *reinterpret_cast<uint32_t*>(dst) = pack8<T>(pr)[0];
        else
          st8(dst, pack8<T>(pr));
      }
    }
  }

  const bool exact = __builtin_amdgcn_ballot_w64(exact_diag) != 0;
  lds_barrier();  // key side in LDS; the qt, kT stores drain meanwhile

  // ---- A[w][J] for J <= w (zero blocks above the diagonal) ----
  // fp32 storage: fp32 MFMA.  bf16 storage: each fp32 operand is split into
  // bf16 hi + lo and the product taken as hi.hi + hi.lo + lo.hi with bf16
  // MFMA over 32 channels at a time (two channel tiles per packet, the same
  // channel order on both sides); the dropped lo.lo term is below 2^-16 of
  // each product.
  {
    T* Ag = reinterpret_cast<T*>(Bb.A) + (((size_t)bh * Bb.nch + chunk) * C + p) * C + 4 * lg;
    constexpr int NP = G::BF ? NT / 2 : 1;  // channel-tile pairs
    u32x4 qh[NP], ql[NP];
    if constexpr (G::BF) {
#pragma unroll
      for (int rp = 0; rp < NP; ++rp) {
        const float f[8] = {qv[2 * rp][0], qv[2 * rp][1], qv[2 * rp][2], qv[2 * rp][3],
                            qv[2 * rp + 1][0], qv[2 * rp + 1][1], qv[2 * rp + 1][2], qv[2 * rp + 1][3]};
        split_bf16(f, qh[rp], ql[rp]);
      }
    }
#pragma unroll
    for (int J = 0; J < NW; ++J) {
      if (J == w && exact) continue;  // formed pair by pair below
      float out[4] = {0.f, 0.f, 0.f, 0.f};
      if (J <= w) {
        const char* krow = ks + (16 * J + lr) * G::KROW + 16 * lg;
        // the key side (referenced at the end of tile J) moved onto this wave's
        // first position: D_wJ <= 1 for J < w, the bounded C_w for J = w
        const float* fac = J < w ? Dw + J * DK : Ew + 2 * DK;
        f32x4 acc = zero4();
        if constexpr (G::BF) {
#pragma unroll
          for (int rp = 0; rp < NP; ++rp) {
            float k8[8], d8[8];
            unpack16<float>(ld16(krow + 64 * (2 * rp)), k8);
            unpack16<float>(ld16(krow + 64 * (2 * rp + 1)), k8 + 4);
            unpack16<float>(ld16(fac + 16 * (2 * rp) + 4 * lg), d8);
            unpack16<float>(ld16(fac + 16 * (2 * rp + 1) + 4 * lg), d8 + 4);
#pragma unroll
            for (int i = 0; i < 8; ++i) k8[i] *= d8[i];
            u32x4 kh, kl;
            split_bf16(k8, kh, kl);
            acc = mma_slab<bf16>(kh, qh[rp], acc);
            acc = mma_slab<bf16>(kh, ql[rp], acc);
            acc = mma_slab<bf16>(kl, qh[rp], acc);
          }
        } else {
#pragma unroll
          for (int rt = 0; rt < NT; ++rt) {
            float k4[4], d4[4];
            unpack16<float>(ld16(krow + 64 * rt), k4);
            unpack16<float>(ld16(fac + 16 * rt + 4 * lg), d4);
#pragma unroll
            for (int i = 0; i < 4; ++i) k4[i] *= d4[i];
            acc = mma_slab<float>(pack16<float>(k4), pack16<float>(qv[rt]), acc);
          }
        }
        // acc[e] = A[16 w + lr][16 J + 4 lg + e]; causal mask on the diagonal block
#pragma unroll
        for (int e = 0; e < 4; ++e) out[e] = (J < w || 4 * lg + e <= lr) ? acc[e] : 0.f;
      }
      if constexpr (G::BF)
        st8(Ag + 16 * J, pack8<T>(out));
      else
        st16(Ag + 16 * J, pack16<T>(out));
    }

    // ---- exact diagonal block (wave-uniform): A[t][t - dl] = sum_c q_tc k_(t-dl)c
    // prod_{u = t-dl+1..t} alpha_uc for dl = 0..15, every factor <= 1.  Each lane
    // sums over its own channels (row shifts bring the earlier positions' key
    // and per-step decay, alpha_t = 2^{x_t - x_(t-1)}, of the same channels),
    // then the four lanes holding a position's channels add their sums.  The
    // gate and its scan are formed again, one channel tile at a time (W_g2 from
    // global memory: its LDS copy is gone), so nothing stays live across the
    // blocks above and the channel loop need not unroll ----
    if (exact) {
      float gx[RP / 4];
      load_gate_factor(gx);
      float part[16];
#pragma unroll
      for (int dl = 0; dl < 16; ++dl) part[dl] = 0.f;
      const float* qg = Bb.q + (seq_row + pl) * DK + 4 * lg;
      const float* kg = Bb.k + (seq_row + pl) * DK + 4 * lg;
#pragma unroll 1
      for (int rt = 0; rt < NT; ++rt) {
        float x4[4], q4[4], k4[4];
        gate_scan(gx, Bb.W2 + hh * DK + lr, hdk, Bb.bg + hh * DK, rt, x4);
        unpack16<float>(live ? ld16(qg + 16 * rt) : zero16(), q4);
        unpack16<float>(live ? ld16(kg + 16 * rt) : zero16(), k4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float qc = q4[i] * P.q_scale;
          float kc = k4[i];
          float ac = exp2_fast(x4[i] - dpp_f<0x111>(x4[i]));  // row_shr 1 (0 before the tile)
          float pr = 1.f;
          part[0] += qc * kc;
#pragma unroll
          for (int dl = 1; dl < 16; ++dl) {
            kc = dpp_f<0x111>(kc);  // key of position t - dl (0 before the tile)
            pr *= ac;               // prod of alpha over t-dl+1 .. t
            ac = dpp_f<0x111>(ac);
            part[dl] += (qc * pr) * kc;
          }
        }
      }
#pragma unroll
      for (int dl = 0; dl < 16; ++dl) {
        part[dl] += __shfl_xor(part[dl], 16);
        part[dl] += __shfl_xor(part[dl], 32);
      }
      float out[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int dl = lr - 4 * lg - e;  // key 16w + 4 lg + e of query 16w + lr
        out[e] = 0.f;
#pragma unroll
        for (int j = 0; j < 16; ++j) out[e] = dl == j ? part[j] : out[e];
      }
      if constexpr (G::BF)
        st8(Ag + 16 * w, pack8<T>(out));
      else
        st16(Ag + 16 * w, pack16<T>(out));
    }
  }
}

template <typename T, int C, int DK, int RP>
static void launch_k2a_cdr(const K2Params& P, hipStream_t stream) {
  using G = K2aGeom<T, C, DK>;
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&k2a_gla_chunk<T, C, DK, RP>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, G::LDS);
  hipLaunchKernelGGL((k2a_gla_chunk<T, C, DK, RP>), dim3(P.total_units), dim3(G::THREADS), G::LDS,
                     stream, P);
}

template <typename T, int C, int DK>
static void launch_k2a_cd(const K2Params& P, hipStream_t stream) {
  if (P.rp == 16)
    launch_k2a_cdr<T, C, DK, 16>(P, stream);
  else
    launch_k2a_cdr<T, C, DK, 64>(P, stream);
}

template <typename T, int C>
static bool launch_k2a_c(const K2Params& P, hipStream_t stream) {
  switch (P.dk) {
    case 16: if constexpr (sizeof(T) == 4) { launch_k2a_cd<T, C, 16>(P, stream); return true; } return false;
    case 32: launch_k2a_cd<T, C, 32>(P, stream); return true;
    case 64: launch_k2a_cd<T, C, 64>(P, stream); return true;
    case 128: launch_k2a_cd<T, C, 128>(P, stream); return true;
    case 256: launch_k2a_cd<T, C, 256>(P, stream); return true;
    default: return false;
  }
}

template <typename T>
static bool launch_k2a_t(const K2Params& P, hipStream_t stream) {
  switch (P.C) {
    case 16: if constexpr (sizeof(T) == 4) return launch_k2a_c<T, 16>(P, stream); return false;
    case 32: return launch_k2a_c<T, 32>(P, stream);
    case 64: return launch_k2a_c<T, 64>(P, stream);
    default: return false;
  }
}

hipError_t launch_k2a(const K2Params& P, bool bf16_path, hipStream_t stream) {
  const bool ok = bf16_path ? launch_k2a_t<bf16>(P, stream) : launch_k2a_t<float>(P, stream);
  if (!ok) return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace msgla
