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
// q and k arrive in fp32 (a single q_t . k_i can cancel strongly, and A scales
// whole output rows), A is formed with a split-bf16 product (hi*hi + hi*lo +
// lo*hi, ~16 mantissa bits) and rounded once to the storage type.
// Every exponent used is <= 0 except one bounded by 15 positions of decay:
// A is built from 16-row sub-blocks with the reference point at the first row
// 16T of the query sub-block T:  q_t e^{b_t - b_16T} (<= 1), k_i e^{b_16J - b_i}
// (growth over < 16 positions inside key sub-block J) and
// D_TJ = e^{b_16T - b_16J} (<= 1) for J < T; on the diagonal D = 1 and the mask
// selects t >= i.  Rows beyond the sequence end are treated as q = k = 0 and
// log alpha = 0, which leaves the state untouched.
//
// Layout of the work: the gate pre-activation z^T = W_g2^T (xp W_g1)^T of the
// chunk comes from fp32 MFMA, so lane l of a wave holds channels 4(l/16)+i of a
// 16-channel tile for position 16 ct + l%16 of each 16-position tile ct.  The
// cumulative sum over positions is then a DPP prefix scan inside each 16-lane
// row plus a carry across the position tiles, all in registers; the decay
// factors and the scaled q / k are formed in the same layout.  Wave J then
// computes the 16 x 16 blocks A[T][J], T >= J, with MFMA as (k-side)(q-side)^T
// so that each lane holds 4 consecutive keys of one query row.
#include "device_common.hpp"
#include "layout.hpp"

namespace msgla {

constexpr int K2A_THREADS = 256;

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

// value of lane (l & ~15) | src of the caller's 16-lane row
__device__ __forceinline__ float row_bcast(float x, int lane, int src) {
  return __shfl(x, (lane & ~15) | src, WAVE);
}

constexpr int K2A_SRT = 4;  // channel tiles per wave (d_k <= 256)
constexpr int K2A_PT = 4;   // position tiles (C <= 64)

template <typename T, int RP>
__global__ __launch_bounds__(K2A_THREADS) void k2a_gla_chunk(const K2Params P) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int unit = blockIdx.x;
  int bi = 0;
  while (bi + 1 < P.nbranch && unit >= P.br[bi + 1].unit_begin) ++bi;
  const K2Branch& Bb = P.br[bi];
  const int local = unit - Bb.unit_begin;
  const int chunk = local % Bb.nch;
  const int bh = local / Bb.nch;  // b * h + head
  const int b = bh / Bb.h, hh = bh - b * Bb.h;

  const int C = P.C, dk = P.dk;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  const int row0 = chunk * C;                       // first pooled row of the chunk
  const int valid = min(C, Bb.n - row0);            // real rows in this chunk
  const int nsub = C / 16;                          // 16-position tiles
  const int nrt = dk / 16;                          // 16-channel tiles

  // LDS: qs, ks fp32 [C][dk+4] | D fp32 [4][4][dk] | kTs T [dk][C+pad]
  //      (phase 0 keeps the gate factor [C][RP] and W2 [RP][dk] where kTs goes)
  const int ldq = dk + 4;
  const int ldt = C + 16 / (int)sizeof(T);
  float* qs = reinterpret_cast<float*>(smem);
  float* ks = qs + (size_t)C * ldq;
  float* Dm = ks + (size_t)C * ldq;
  T* kTs = reinterpret_cast<T*>(Dm + 16 * dk);
  float* gs = reinterpret_cast<float*>(kTs);
  float* w2s = gs + C * RP;

  const size_t seq_row = (size_t)bh * Bb.np + row0;  // row index in [B][h][np]
  const float* qg = Bb.q + seq_row * dk;
  const float* kg = Bb.k + seq_row * dk;
  T* qtg = reinterpret_cast<T*>(Bb.qt) + seq_row * dk;
  T* kTg = reinterpret_cast<T*>(Bb.kT) + ((size_t)bh * Bb.nch + chunk) * dk * C;
  float* lamg = Bb.lam + ((size_t)bh * Bb.nch + chunk) * dk;
  const int hdk = Bb.h * dk;

  // ---- phase 0: stage the gate factor rows and this head's W2 slice ----
  {
    const float* gsrc = Bb.g + ((size_t)b * Bb.np + row0) * RP;
    for (int p = tid; p < C * RP / 4; p += K2A_THREADS) {
      const int t = (p * 4) / RP;
      st16(gs + p * 4, t < valid ? ld16(gsrc + p * 4) : zero16());
    }
    for (int p = tid; p < RP * dk / 4; p += K2A_THREADS) {
      const int r = (p * 4) / dk, c = p * 4 - r * dk;
      st16(w2s + p * 4, ld16(Bb.W2 + (size_t)r * hdk + hh * dk + c));
    }
  }
  __syncthreads();

  // ---- phase 1a: z^T[c][t] = sum_r W2[r][c] g[t][r] (fp32 MFMA), then log alpha ----
  // register z[a][ct][i]: channel c = 16 (wave + 4a) + 4 lg + i, position t = 16 ct + lr
  float x[K2A_SRT][K2A_PT][4];
#pragma unroll
  for (int a = 0; a < K2A_SRT; ++a) {
    const int rt = wave + 4 * a;
#pragma unroll
    for (int ct = 0; ct < K2A_PT; ++ct) {
      f32x4 acc = zero4();
      if (rt < nrt && ct < nsub) {
#pragma unroll
        for (int k4 = 0; k4 < RP; k4 += 4) {
          const float wa = w2s[(k4 + lg) * dk + 16 * rt + lr];
          const float gb = gs[(16 * ct + lr) * RP + k4 + lg];
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(wa, gb, acc, 0, 0, 0);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) x[a][ct][i] = acc[i];
    }
  }
  __syncthreads();  // gs / w2s are overwritten by kTs below

  float blast[K2A_SRT][4];
#pragma unroll
  for (int a = 0; a < K2A_SRT; ++a) {
    const int rt = wave + 4 * a;
    if (rt >= nrt) continue;
    const int c0 = 16 * rt + 4 * lg;  // first of this lane's 4 channels
    const f32x4 bgv = __builtin_bit_cast(f32x4, ld16(Bb.bg + hh * dk + c0));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float carry = 0.f;
#pragma unroll
      for (int ct = 0; ct < K2A_PT; ++ct) {
        if (ct < nsub) {
          const int t = 16 * ct + lr;
          const float la = (t < valid) ? logsigmoid_f(x[a][ct][i] + bgv[i]) * P.inv_gamma : 0.f;
          const float v = row_scan16(la) + carry;  // b_t = sum_{u <= t} log alpha_u
          carry = row_bcast(v, lane, 15);
          x[a][ct][i] = v;
        }
      }
      blast[a][i] = carry;  // b at the last position of the chunk
    }

    // ---- phase 1b: decay factors and scaled operands, same register layout ----
    float bref[K2A_PT][4];
#pragma unroll
    for (int ct = 0; ct < K2A_PT; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) bref[ct][i] = (ct < nsub) ? row_bcast(x[a][ct][i], lane, 0) : 0.f;
    if (lr == 0) {
      // D_TJ = exp(b_16T - b_16J), J < T;  lam = exp(b_last)
#pragma unroll
      for (int T_ = 1; T_ < K2A_PT; ++T_)
#pragma unroll
        for (int J = 0; J < T_; ++J)
          if (T_ < nsub) {
            float dv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) dv[i] = __expf(bref[T_][i] - bref[J][i]);
            st16(Dm + (T_ * 4 + J) * dk + c0, pack16<float>(dv));
          }
      float lv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) lv[i] = __expf(blast[a][i]);
      st16(lamg + c0, pack16<float>(lv));
    }
#pragma unroll
    for (int ct = 0; ct < K2A_PT; ++ct) {
      if (ct >= nsub) continue;
      const int t = 16 * ct + lr;
      float qv[4] = {0.f, 0.f, 0.f, 0.f}, kv[4] = {0.f, 0.f, 0.f, 0.f};
      if (t < valid) {
        unpack16<float>(ld16(qg + (size_t)t * dk + c0), qv);
        unpack16<float>(ld16(kg + (size_t)t * dk + c0), kv);
      }
      float qsv[4], ksv[4], qo[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float bt = x[a][ct][i];
        qv[i] *= P.q_scale;
        qsv[i] = qv[i] * __expf(bt - bref[ct][i]);   // query side of A, <= |q|
        ksv[i] = kv[i] * __expf(bref[ct][i] - bt);   // key side of A (growth < 16 steps)
        qo[i] = qv[i] * __expf(bt);                  // inter-chunk query
        kTs[(size_t)(c0 + i) * ldt + t] = from_f32<T>(kv[i] * __expf(blast[a][i] - bt));
      }
      st16(qs + (size_t)t * ldq + c0, pack16<float>(qsv));
      st16(ks + (size_t)t * ldq + c0, pack16<float>(ksv));
      if constexpr (sizeof(T) == 2)
        st8(qtg + (size_t)t * dk + c0, pack8<T>(qo));
      else
        st16(qtg + (size_t)t * dk + c0, pack16<T>(qo));
    }
  }
  __syncthreads();
  // ---- phase 2: A = masked decayed q k^T from 16 x 16 sub-blocks (wave J) ----
  const int J = wave;
  if (J < nsub) {
    const int lr = lane & 15, lg = lane >> 4;
    T* Ag = reinterpret_cast<T*>(Bb.A) + ((size_t)bh * Bb.nch + chunk) * C * C;
    for (int T_ = 0; T_ < nsub; ++T_) {
      float out[4] = {0.f, 0.f, 0.f, 0.f};
      if (T_ >= J) {
        f32x4 acc = zero4();
        const int i_row = 16 * J + lr;   // key row for the A-operand
        const int t_row = 16 * T_ + lr;  // query row for the B-operand
        for (int c0 = 0; c0 < dk; c0 += slab_elems<T>()) {
          const int cc = c0 + lg * per16<T>();
          float kf[per16<T>()], qf[per16<T>()];
#pragma unroll
          for (int e = 0; e < per16<T>(); e += 4) {
            unpack16<float>(ld16(ks + (size_t)i_row * ldq + cc + e), kf + e);
            unpack16<float>(ld16(qs + (size_t)t_row * ldq + cc + e), qf + e);
          }
          if (T_ > J) {
#pragma unroll
            for (int e = 0; e < per16<T>(); ++e) qf[e] *= Dm[(T_ * 4 + J) * dk + cc + e];
          }
          if constexpr (sizeof(T) == 2) {
            // split-bf16 product (hi*hi + hi*lo + lo*hi): A is a scalar weight of
            // whole output rows, so it is formed to ~16 mantissa bits.
            u32x4 kh, kl, qh, ql;
            split_bf16(kf, kh, kl);
            split_bf16(qf, qh, ql);
            acc = mma_slab<bf16>(kh, qh, acc);
            acc = mma_slab<bf16>(kh, ql, acc);
            acc = mma_slab<bf16>(kl, qh, acc);
          } else {
            acc = mma_slab<float>(pack16<float>(kf), pack16<float>(qf), acc);
          }
        }
        // acc[e] = A[16T + lr][16J + 4 lg + e]
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool keep = (T_ > J) || (4 * lg + e <= lr);
          out[e] = keep ? acc[e] : 0.f;
        }
      }
      T* dst = Ag + (size_t)(16 * T_ + lr) * C + 16 * J + 4 * lg;
      if constexpr (sizeof(T) == 2) {
        st8(dst, pack8<T>(out));
      } else {
        st16(dst, pack16<T>(out));
      }
    }
  }

  // ---- phase 3: the transposed state-update key, coalesced ----
  constexpr int PER = per16<T>();
  for (int p = tid; p < dk * C / PER; p += K2A_THREADS) {
    const int c = (p * PER) / C, t0 = p * PER - c * C;
    st16(kTg + (size_t)c * C + t0, ld16(kTs + (size_t)c * ldt + t0));
  }
}

size_t k2a_lds_bytes(int C, int dk, int rp, bool bf16_path) {
  const int es = bf16_path ? 2 : 4;
  const size_t kts = (size_t)dk * (C + 16 / es) * es;
  const size_t gw = (size_t)(C * rp + rp * dk) * 4;
  return (size_t)2 * C * (dk + 4) * 4 + (size_t)16 * dk * 4 + (kts > gw ? kts : gw);
}

template <typename T, int RP>
static void launch_k2a_rp(const K2Params& P, size_t lds, hipStream_t stream) {
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&k2a_gla_chunk<T, RP>),
                      hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  hipLaunchKernelGGL((k2a_gla_chunk<T, RP>), dim3(P.total_units), dim3(K2A_THREADS), lds, stream, P);
}

template <typename T>
static void launch_k2a_t(const K2Params& P, size_t lds, hipStream_t stream) {
  if (P.rp == 16)
    launch_k2a_rp<T, 16>(P, lds, stream);
  else
    launch_k2a_rp<T, 64>(P, lds, stream);
}

hipError_t launch_k2a(const K2Params& P, bool bf16_path, hipStream_t stream) {
  const size_t lds = k2a_lds_bytes(P.C, P.dk, P.rp, bf16_path);
  if (bf16_path)
    launch_k2a_t<bf16>(P, lds, stream);
  else
    launch_k2a_t<float>(P, lds, stream);
  return hipGetLastError();
}

}  // namespace msgla
