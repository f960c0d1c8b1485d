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
// Layout of the work: lane = position t in the chunk for the gate, the
// cumulative-sum wavefront scan and the scalings (wave w owns a quarter of the
// key channels), then wave J computes the 16 x 16 blocks A[T][J], T >= J, with
// MFMA as (k-side)(q-side)^T so that each lane holds 4 consecutive keys of one
// query row and stores them as one packet.
#include "device_common.hpp"
#include "layout.hpp"

namespace msgla {

constexpr int K2A_THREADS = 256;

__device__ __forceinline__ float wave_inclusive_scan(float x, int lane) {
#pragma unroll
  for (int off = 1; off < WAVE; off <<= 1) {
    const float t = __shfl_up(x, off, WAVE);
    if (lane >= off) x += t;
  }
  return x;
}

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
  const int row0 = chunk * C;                       // first pooled row of the chunk
  const int valid = min(C, Bb.n - row0);            // real rows in this chunk
  const int nsub = C / 16;

  // LDS: qs fp32 [C][dk+4] | ks fp32 [C][dk+4] | D fp32 [4][4][dk]
  const int ldq = dk + 4;
  float* qs = reinterpret_cast<float*>(smem);
  float* ks = qs + (size_t)C * ldq;
  float* Dm = ks + (size_t)C * ldq;

  const size_t seq_row = (size_t)bh * Bb.np + row0;  // row index in [B][h][np]
  const float* qg = Bb.q + seq_row * dk;
  const float* kg = Bb.k + seq_row * dk;
  T* qtg = reinterpret_cast<T*>(Bb.qt) + seq_row * dk;
  T* kTg = reinterpret_cast<T*>(Bb.kT) + ((size_t)bh * Bb.nch + chunk) * dk * C;
  float* lamg = Bb.lam + ((size_t)bh * Bb.nch + chunk) * dk;
  const int hdk = Bb.h * dk;

  // ---- phase 1: gate, wavefront scan of log alpha, scalings (lane = position) ----
  const int t = lane;
  const bool live = t < C;
  const bool real = t < valid;
  float gr[RP];
#pragma unroll
  for (int r = 0; r < RP; ++r) gr[r] = 0.f;
  if (real) {
    const float* gp = Bb.g + ((size_t)b * Bb.np + row0 + t) * RP;
#pragma unroll
    for (int q4 = 0; q4 < RP; q4 += 4) unpack16<float>(ld16(gp + q4), gr + q4);
  }
  // channels of this wave, in groups of 8 (d_k < 32 leaves some waves idle)
  const int cw = ((dk / 4 + 7) / 8) * 8;
  const int cbeg = wave * cw;
  const int cend = min(dk, cbeg + cw);
  for (int c8 = cbeg; c8 < cend; c8 += 8) {
    float qv[8], kv[8], bsum[8];
    if (real) {
      unpack16<float>(ld16(qg + (size_t)t * dk + c8), qv);
      unpack16<float>(ld16(qg + (size_t)t * dk + c8 + 4), qv + 4);
      unpack16<float>(ld16(kg + (size_t)t * dk + c8), kv);
      unpack16<float>(ld16(kg + (size_t)t * dk + c8 + 4), kv + 4);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) qv[e] = kv[e] = 0.f;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int ch = hh * dk + c8 + e;  // channel within the branch
      float z = Bb.bg[ch];
#pragma unroll
      for (int r = 0; r < RP; ++r) z = fmaf(gr[r], Bb.W2[(size_t)r * hdk + ch], z);
      const float la = real ? logsigmoid_f(z) * P.inv_gamma : 0.f;
      bsum[e] = wave_inclusive_scan(la, lane);
      qv[e] *= P.q_scale;
    }
    float blast[8], bref[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      blast[e] = __shfl(bsum[e], C - 1, WAVE);
      bref[e] = __shfl(bsum[e], lane & ~15, WAVE);
    }
    // D_TJ = exp(b_16T - b_16J) for J < T
    for (int J = 0; J + 1 < nsub; ++J) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float bJ = __shfl(bsum[e], 16 * J, WAVE);
        const int T_ = lane >> 4;
        if ((lane & 15) == 0 && T_ > J && T_ < nsub)
          Dm[(T_ * 4 + J) * dk + c8 + e] = __expf(bsum[e] - bJ);
      }
    }
    if (live) {
      float qo[8], ko[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        qs[t * ldq + c8 + e] = qv[e] * __expf(bsum[e] - bref[e]);
        ks[t * ldq + c8 + e] = kv[e] * __expf(bref[e] - bsum[e]);
        qo[e] = qv[e] * __expf(bsum[e]);
        ko[e] = kv[e] * __expf(blast[e] - bsum[e]);
      }
      if constexpr (sizeof(T) == 2) {
        st16(qtg + (size_t)t * dk + c8, pack16<T>(qo));
      } else {
        st16(qtg + (size_t)t * dk + c8, pack16<T>(qo));
        st16(qtg + (size_t)t * dk + c8 + 4, pack16<T>(qo + 4));
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) kTg[(size_t)(c8 + e) * C + t] = from_f32<T>(ko[e]);
      if (t == 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) lamg[c8 + e] = __expf(blast[e]);
      }
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
}

size_t k2a_lds_bytes(int C, int dk, bool /*bf16_path*/) {
  return (size_t)2 * C * (dk + 4) * 4 + (size_t)16 * dk * 4;
}

template <typename T, int RP>
static void launch_k2a_rp(const K2Params& P, size_t lds, hipStream_t stream) {
  hipFuncSetAttribute(reinterpret_cast<const void*>(&k2a_gla_chunk<T, RP>),
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
  const size_t lds = k2a_lds_bytes(P.C, P.dk, bf16_path);
  if (bf16_path)
    launch_k2a_t<bf16>(P, lds, stream);
  else
    launch_k2a_t<float>(P, lds, stream);
  return hipGetLastError();
}

}  // namespace msgla
