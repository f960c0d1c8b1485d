// K2b — carried-state part of the gated linear recurrence.
//
// MS-GLA notes, Sec. 2.1 (S_t = Diag(alpha_t) S_{t-1} + k_t^T v_t, o_t = q_t S_t)
// in its chunkwise form (Sec. 3.4).  With the chunk-local quantities of K2a
// (A, qt = q ⊙ e^b, kT = (k ⊙ e^{b_last - b})^T, lam = e^{b_last}), chunk c
// entering with state S_c produces
//   y_c     = A_c V_c + qt_c S_c
//   S_{c+1} = Diag(lam_c) S_c + kT_c V_c .
// One workgroup owns one (branch, sequence, head) and a 32-wide slice of d_v
// and walks its chunks in order; the slices of one sequence run on the same
// XCD (they read the same A / qt / kT, which then stay in that XCD's L2).
// The state slice lives in fp32 MFMA accumulators across the whole walk —
// wave w keeps rows c of S with (c / 16) % 4 == w — and after each update it
// is published to LDS in the storage type (transposed, [v][c]) as the
// B-operand of the next chunk's qt S.  Wave w also produces output rows
// 16w .. 16w+15 of each chunk.  V of the chunk is staged in LDS (positions
// beyond the sequence end are zeroed there) and serves both products.
// After the last chunk the fp32 state is optionally written out.
#include "device_common.hpp"
#include "layout.hpp"

namespace msgla {

constexpr int K2B_THREADS = 256;
constexpr int K2B_DVT = 32;  // d_v columns per workgroup

template <typename T, int SRT>
__global__ __launch_bounds__(K2B_THREADS) void k2b_gla_state(const K2Params P) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int g = blockIdx.x;
  const int slot = g / N_XCD, xcd = g % N_XCD;
  const int qseq = (slot / P.n_dvt) * N_XCD + xcd;
  const int tile = slot % P.n_dvt;
  if (qseq >= P.total_seqs) return;
  int bi = P.order[0];
  for (int o = 1; o < P.nbranch; ++o)
    if (qseq >= P.br[P.order[o]].seq_begin) bi = P.order[o];
  const K2Branch& Bb = P.br[bi];
  const int bh = qseq - Bb.seq_begin;  // b * h + head

  const int C = P.C, dk = P.dk, dv = P.dv;
  const int v0 = tile * K2B_DVT;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  const int nrt = dk / 16;  // state row tiles

  // LDS: ST[2][DVT][dk + pad] (T) | VT[2][DVT][C + pad] (T)
  const int lds_s = dk + 16 / (int)sizeof(T);
  const int lds_v = C + 16 / (int)sizeof(T);
  T* ST = reinterpret_cast<T*>(smem);
  T* VS = ST + 2 * K2B_DVT * lds_s;

  const size_t chunk0 = (size_t)bh * Bb.nch;
  const T* Ag = reinterpret_cast<const T*>(Bb.A);
  const T* qtg = reinterpret_cast<const T*>(Bb.qt) + (size_t)bh * Bb.np * dk;
  const T* kTg = reinterpret_cast<const T*>(Bb.kT);
  const T* vTg = reinterpret_cast<const T*>(Bb.vT);
  T* yg = reinterpret_cast<T*>(Bb.y) + (size_t)bh * Bb.np * dv;

  // state accumulators: [SRT row tiles][2 col tiles]
  f32x4 S[SRT][2];
#pragma unroll
  for (int a = 0; a < SRT; ++a) S[a][0] = S[a][1] = zero4();

  // S_0 = 0 published to LDS buffer 0
  for (int i = tid; i < K2B_DVT * lds_s; i += K2B_THREADS) ST[i] = from_f32<T>(0.f);

  // stage V of chunk c (positions >= valid zeroed) into buffer c & 1
  auto stage_v = [&](int c) {
    const int valid = min(C, Bb.n - c * C);
    const T* src = vTg + ((chunk0 + c) * dv + v0) * C;
    T* dst = VS + (c & 1) * K2B_DVT * lds_v;
    const int per_row = C / per16<T>();
    for (int p = tid; p < K2B_DVT * per_row; p += K2B_THREADS) {
      const int vr = p / per_row, tp = (p - vr * per_row) * per16<T>();
      u32x4 x = ld16(src + (size_t)vr * C + tp);
      if (tp + per16<T>() > valid) {
        float f[per16<T>()];
        unpack16<T>(x, f);
#pragma unroll
        for (int e = 0; e < per16<T>(); ++e)
          if (tp + e >= valid) f[e] = 0.f;
        x = pack16<T>(f);
      }
      st16(dst + vr * lds_v + tp, x);
    }
  };
  if (Bb.nch > 0) stage_v(0);
  __syncthreads();

  for (int c = 0; c < Bb.nch; ++c) {
    const T* Sb = ST + (c & 1) * K2B_DVT * lds_s;
    const T* Vb = VS + (c & 1) * K2B_DVT * lds_v;
    // ---- y rows of this wave: y = A V + qt S ----
    if (wave < C / 16) {
      const int rt = wave;
      f32x4 y[2] = {zero4(), zero4()};
      const T* Arow = Ag + ((chunk0 + c) * C + 16 * rt + lr) * C;
      for (int i0 = 0; i0 < C; i0 += slab_elems<T>()) {
        const u32x4 a = ld16(Arow + i0 + lg * per16<T>());
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          const u32x4 bv = ld16(Vb + (16 * ct + lr) * lds_v + i0 + lg * per16<T>());
          y[ct] = mma_slab<T>(a, bv, y[ct]);
        }
      }
      const T* qrow = qtg + ((size_t)c * C + 16 * rt + lr) * dk;
      for (int c0 = 0; c0 < dk; c0 += slab_elems<T>()) {
        const u32x4 a = ld16(qrow + c0 + lg * per16<T>());
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          const u32x4 bs = ld16(Sb + (16 * ct + lr) * lds_s + c0 + lg * per16<T>());
          y[ct] = mma_slab<T>(a, bs, y[ct]);
        }
      }
      const int valid = min(C, Bb.n - c * C);
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int tau = 16 * rt + 4 * lg + e;
          if (tau < valid) yg[((size_t)c * C + tau) * dv + v0 + 16 * ct + lr] = from_f32<T>(y[ct][e]);
        }
    }
    // ---- state update: S = Diag(lam) S + kT V, rows owned by this wave ----
    const float* lam = Bb.lam + (chunk0 + c) * dk;
    T* Sn = ST + ((c + 1) & 1) * K2B_DVT * lds_s;
#pragma unroll
    for (int a = 0; a < SRT; ++a) {
      const int rt = wave + 4 * a;
      if (rt < nrt) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float l = lam[16 * rt + 4 * lg + e];
          S[a][0][e] *= l;
          S[a][1][e] *= l;
        }
        const T* krow = kTg + ((chunk0 + c) * dk + 16 * rt + lr) * C;
        for (int t0 = 0; t0 < C; t0 += slab_elems<T>()) {
          const u32x4 ak = ld16(krow + t0 + lg * per16<T>());
#pragma unroll
          for (int ct = 0; ct < 2; ++ct) {
            const u32x4 bv = ld16(Vb + (16 * ct + lr) * lds_v + t0 + lg * per16<T>());
            S[a][ct] = mma_slab<T>(ak, bv, S[a][ct]);
          }
        }
        // publish S_{c+1}: ST[v][c], 4 consecutive c per lane
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          float f[4] = {S[a][ct][0], S[a][ct][1], S[a][ct][2], S[a][ct][3]};
          T* dst = Sn + (16 * ct + lr) * lds_s + 16 * rt + 4 * lg;
          if constexpr (sizeof(T) == 2)
            st8(dst, pack8<T>(f));
          else
            st16(dst, pack16<T>(f));
        }
      }
    }
    if (c + 1 < Bb.nch) stage_v(c + 1);
    __syncthreads();
  }

  if (Bb.S_out) {
    float* So = Bb.S_out + (size_t)bh * dk * dv;
#pragma unroll
    for (int a = 0; a < SRT; ++a) {
      const int rt = wave + 4 * a;
      if (rt < nrt) {
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            So[(size_t)(16 * rt + 4 * lg + e) * dv + v0 + 16 * ct + lr] = S[a][ct][e];
      }
    }
  }
}

size_t k2b_lds_bytes(int C, int dk, bool bf16_path) {
  const int es = bf16_path ? 2 : 4;
  return (size_t)2 * K2B_DVT * (dk + 16 / es) * es + (size_t)2 * K2B_DVT * (C + 16 / es) * es;
}

int k2b_dvt() { return K2B_DVT; }

template <typename T>
static void launch_k2b_t(const K2Params& P, dim3 grid, size_t lds, hipStream_t stream) {
  const int nrt = P.dk / 16;
  if (nrt <= 4)
    hipLaunchKernelGGL((k2b_gla_state<T, 1>), grid, dim3(K2B_THREADS), lds, stream, P);
  else if (nrt <= 8)
    hipLaunchKernelGGL((k2b_gla_state<T, 2>), grid, dim3(K2B_THREADS), lds, stream, P);
  else
    hipLaunchKernelGGL((k2b_gla_state<T, 4>), grid, dim3(K2B_THREADS), lds, stream, P);
}

hipError_t launch_k2b(const K2Params& P, bool bf16_path, hipStream_t stream) {
  const size_t lds = k2b_lds_bytes(P.C, P.dk, bf16_path);
  const dim3 grid(((P.total_seqs + N_XCD - 1) / N_XCD) * N_XCD * P.n_dvt);
  if (bf16_path)
    launch_k2b_t<bf16>(P, grid, lds, stream);
  else
    launch_k2b_t<float>(P, grid, lds, stream);
  return hipGetLastError();
}

}  // namespace msgla
