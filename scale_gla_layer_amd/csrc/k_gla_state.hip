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
// 16w .. 16w+15 of each chunk.  The walk is latency-bound unless the inputs
// of later chunks are already in flight: A, qt, kT, the chunk's V slice and
// lam are copied global -> LDS asynchronously (global_load_lds_dwordx4, no
// VGPRs) into NST rotating stages, NST-1 chunks ahead of the compute, with
// vmcnt waits and one barrier per chunk.  V positions beyond the sequence end
// are zeroed in the fragments (the workspace there is never written).
// After the last chunk the fp32 state is optionally written out.
#include "async_copy.hpp"
#include "device_common.hpp"
#include "layout.hpp"

namespace msgla {

constexpr int K2B_THREADS = 256;
constexpr int K2B_DVT = 32;  // d_v columns per workgroup

struct K2bStage {  // byte offsets of one pipeline stage (each a multiple of 1 KB)
  int A, Q, K, V, L, bytes;
};

__host__ __device__ inline int k2b_kb(int b) { return (b + 1023) & ~1023; }

__host__ __device__ inline K2bStage k2b_stage(int C, int dk, int es) {
  K2bStage g;
  g.A = 0;
  g.Q = g.A + k2b_kb(C * C * es);
  g.K = g.Q + k2b_kb(C * dk * es);
  g.V = g.K + k2b_kb(dk * C * es);
  g.L = g.V + k2b_kb(K2B_DVT * C * es);
  g.bytes = g.L + k2b_kb(dk * 4);
  return g;
}

// Per-lane source offset of copy instruction k for a contiguous block stored
// as swizzled 128-byte virtual rows (async_copy.hpp): source = block + 1024 k
// + off.  The swizzle key of instruction k is ((8 k + lane / 8) >> hs) & 7;
// rows of up to 512 bytes (hs <= 2) make it depend on k mod 4 only and rows of
// 1024 bytes (hs = 3) on k mod 8, so wave w (instructions k = w, w + 4, ...)
// needs one offset for its even-numbered and one for its odd-numbered copies.
__device__ __forceinline__ int k2b_lane_off(int lg, int k, int lane) {
  const int hs = blk_hs(lg);
  const int vrow = 8 * k + (lane >> 3);
  return 128 * (lane >> 3) + 16 * ((lane & 7) ^ ((vrow >> hs) & 7));
}

template <typename T, int SRT, int NST>
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

  constexpr int es = sizeof(T);
  constexpr int PER = per16<T>();
  const int C = P.C, dk = P.dk, dv = P.dv;
  const int v0 = tile * K2B_DVT;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lgp = lane >> 4;
  const int nrt = dk / 16;                  // state row tiles
  const int lgC = 31 - __builtin_clz(C * es);   // log2 bytes of an A / kT / V row
  const int lgQ = 31 - __builtin_clz(dk * es);  // log2 bytes of a qt row
  const int lgL = 31 - __builtin_clz(dk * 4);   // lam: one row of dk floats
  const int nslab_c = C * es / 64;          // 64-byte k-slabs over positions
  const int nslab_k = dk * es / 64;         // 64-byte k-slabs over key channels

  // LDS: NST stages | ST[2][DVT][dk + pad] (published state) | per-wave y staging
  const K2bStage sg = k2b_stage(C, dk, es);
  const int lds_s = dk + 16 / es;
  T* ST = reinterpret_cast<T*>(smem + (size_t)NST * sg.bytes);
  const int ldy = K2B_DVT + 16 / es;
  T* ys = ST + 2 * K2B_DVT * lds_s + wave * 16 * ldy;

  const size_t chunk0 = (size_t)bh * Bb.nch;
  const int bA = C * C * es, bQ = C * dk * es, bV = K2B_DVT * C * es, bL = dk * 4;
  const char* Ag = reinterpret_cast<const char*>(Bb.A) + chunk0 * bA;
  const char* Qg = reinterpret_cast<const char*>(Bb.qt) + (size_t)bh * Bb.np * dk * es;
  const char* Kg = reinterpret_cast<const char*>(Bb.kT) + chunk0 * bQ;
  const char* Vg = reinterpret_cast<const char*>(Bb.vT) + (chunk0 * dv + v0) * C * es;
  const char* Lg = reinterpret_cast<const char*>(Bb.lam + chunk0 * dk);
  T* yg = reinterpret_cast<T*>(Bb.y) + (size_t)bh * Bb.np * dv + v0;

  // hoisted copy offsets (one per block) and copy counts (per wave)
  // (A, kT and V rows hold C <= 64 elements, at most 256 bytes; qt rows up to 1 KB)
  const int oA = k2b_lane_off(lgC, wave, lane);
  const int oQ0 = k2b_lane_off(lgQ, wave, lane), oQ1 = k2b_lane_off(lgQ, wave + 4, lane);
  const int oL = 16 * lane;  // lam: one partial instruction, unswizzled row (key 0)
  const int nA = (bA / 1024 + 3 - wave) / 4, nQ = (bQ / 1024 + 3 - wave) / 4;
  const int nV = (bV / 1024 + 3 - wave) / 4;
  const int K = nA + 2 * nQ + nV + (wave == 0 ? 1 : 0);  // copies per chunk of this wave
  auto issue = [&](int c) {
    char* st = smem + (size_t)(c % NST) * sg.bytes;
    const char* a = Ag + (size_t)c * bA;
    const char* q = Qg + (size_t)c * bQ;
    const char* kk = Kg + (size_t)c * bQ;
    const char* v = Vg + (size_t)c * dv * C * es;
    for (int i = 0; i < nA; ++i) {
      const int k = wave + 4 * i;
      __builtin_amdgcn_global_load_lds(a + 1024 * k + oA, (lds_void_t*)(st + sg.A + 1024 * k), 16, 0, 0);
    }
    for (int i = 0; i < nQ; ++i) {
      const int k = wave + 4 * i;
      __builtin_amdgcn_global_load_lds(q + 1024 * k + ((i & 1) ? oQ1 : oQ0),
                                       (lds_void_t*)(st + sg.Q + 1024 * k), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(kk + 1024 * k + oA, (lds_void_t*)(st + sg.K + 1024 * k), 16, 0, 0);
    }
    for (int i = 0; i < nV; ++i) {
      const int k = wave + 4 * i;
      __builtin_amdgcn_global_load_lds(v + 1024 * k + oA, (lds_void_t*)(st + sg.V + 1024 * k), 16, 0, 0);
    }
    if (wave == 0) {
      if (oL < bL)
        __builtin_amdgcn_global_load_lds(Lg + (size_t)c * bL + oL, (lds_void_t*)(st + sg.L), 16, 0, 0);
    }
  };

  // hoisted LDS fragment offsets (inside a stage)
  int offV[4][2], offA[4], offK[SRT][4], offQ[16];
#pragma unroll
  for (int sl = 0; sl < 4; ++sl) {
    offV[sl][0] = sg.V + tile_off(lr, sl * 4 + lgp, lgC);
    offV[sl][1] = sg.V + tile_off(16 + lr, sl * 4 + lgp, lgC);
    offA[sl] = sg.A + tile_off(16 * wave + lr, sl * 4 + lgp, lgC);
#pragma unroll
    for (int a = 0; a < SRT; ++a) offK[a][sl] = sg.K + tile_off(16 * (wave + 4 * a) + lr, sl * 4 + lgp, lgC);
  }
#pragma unroll
  for (int sl = 0; sl < 16; ++sl) offQ[sl] = sg.Q + tile_off(16 * wave + lr, sl * 4 + lgp, lgQ);
  int offL[SRT];
#pragma unroll
  for (int a = 0; a < SRT; ++a) offL[a] = sg.L + tile_off(0, (16 * (wave + 4 * a) + 4 * lgp) >> 2, lgL);

  f32x4 S[SRT][2];
#pragma unroll
  for (int a = 0; a < SRT; ++a) S[a][0] = S[a][1] = zero4();

  for (int c = 0; c < NST - 1 && c < Bb.nch; ++c) issue(c);
  for (int i = tid; i < K2B_DVT * lds_s; i += K2B_THREADS) ST[i] = from_f32<T>(0.f);

  for (int c = 0; c < Bb.nch; ++c) {
    // stage c must have landed: with one later stage in flight at most K more
    // copies may be outstanding (stores issued since only add to that count)
    if (NST > 2 && c + 1 < Bb.nch && K >= 8)
      wait_vmcnt<8>();
    else
      wait_vmcnt<0>();
    lds_barrier();
    if (c + NST - 1 < Bb.nch) issue(c + NST - 1);

    const char* st = smem + (size_t)(c % NST) * sg.bytes;
    const T* Sb = ST + (c & 1) * K2B_DVT * lds_s;
    T* Sn = ST + ((c + 1) & 1) * K2B_DVT * lds_s;
    const int valid = min(C, Bb.n - c * C);

    // V fragments (B-operand of both products); positions >= valid zeroed
    u32x4 vf[4][2];
#pragma unroll
    for (int sl = 0; sl < 4; ++sl)
      if (sl < nslab_c) {
        vf[sl][0] = ld16(st + offV[sl][0]);
        vf[sl][1] = ld16(st + offV[sl][1]);
      }
    if (valid < C) {
#pragma unroll
      for (int sl = 0; sl < 4; ++sl)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          if (sl < nslab_c) {
            const int tau0 = (sl * 4 + lgp) * PER;
            float u[PER];
            unpack16<T>(vf[sl][ct], u);
#pragma unroll
            for (int e = 0; e < PER; ++e)
              if (tau0 + e >= valid) u[e] = 0.f;
            vf[sl][ct] = pack16<T>(u);
          }
        }
    }

    // ---- y rows 16w .. 16w+15: y = A V + qt S, staged for 16-byte stores ----
    if (wave < C / 16) {
      const int rt = wave;
      f32x4 y[2] = {zero4(), zero4()};
#pragma unroll
      for (int sl = 0; sl < 4; ++sl) {
        if (sl < nslab_c) {
          const u32x4 a = ld16(st + offA[sl]);
          y[0] = mma_slab<T>(a, vf[sl][0], y[0]);
          y[1] = mma_slab<T>(a, vf[sl][1], y[1]);
        }
      }
#pragma unroll
      for (int sl = 0; sl < 16; ++sl) {
        if (sl < nslab_k) {
          const u32x4 a = ld16(st + offQ[sl]);
          const T* srow = Sb + lr * lds_s + sl * slab_elems<T>() + lgp * PER;
          y[0] = mma_slab<T>(a, ld16(srow), y[0]);
          y[1] = mma_slab<T>(a, ld16(srow + 16 * lds_s), y[1]);
        }
      }
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e) ys[(4 * lgp + e) * ldy + 16 * ct + lr] = from_f32<T>(y[ct][e]);
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (0 << 8));  // own LDS writes done
      asm volatile("" ::: "memory");
      // 16 rows x DVT values of this wave -> 16-byte global stores
      constexpr int PR = K2B_DVT / PER;  // pieces per row
#pragma unroll
      for (int p0 = 0; p0 < 16 * PR; p0 += 64) {
        const int p = p0 + lane;
        const int row = p / PR, pc = p - row * PR;
        if (p < 16 * PR && 16 * rt + row < valid)
          st16(yg + ((size_t)c * C + 16 * rt + row) * dv + pc * PER, ld16(ys + row * ldy + pc * PER));
      }
    }
    // ---- state update: S = Diag(lam) S + kT V for the rows this wave owns ----
#pragma unroll
    for (int a = 0; a < SRT; ++a) {
      const int rt = wave + 4 * a;
      if (rt < nrt) {
        const f32x4 l4 = __builtin_bit_cast(f32x4, ld16(st + offL[a]));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          S[a][0][e] *= l4[e];
          S[a][1][e] *= l4[e];
        }
#pragma unroll
        for (int sl = 0; sl < 4; ++sl) {
          if (sl < nslab_c) {
            const u32x4 ak = ld16(st + offK[a][sl]);
            S[a][0] = mma_slab<T>(ak, vf[sl][0], S[a][0]);
            S[a][1] = mma_slab<T>(ak, vf[sl][1], S[a][1]);
          }
        }
        // publish S_{c+1}: ST[v][c], 4 consecutive c per lane
        const int c4 = 16 * rt + 4 * lgp;
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          float f[4] = {S[a][ct][0], S[a][ct][1], S[a][ct][2], S[a][ct][3]};
          T* dst = Sn + (16 * ct + lr) * lds_s + c4;
          if constexpr (sizeof(T) == 2)
            st8(dst, pack8<T>(f));
          else
            st16(dst, pack16<T>(f));
        }
      }
    }
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
            So[(size_t)(16 * rt + 4 * lgp + e) * dv + v0 + 16 * ct + lr] = S[a][ct][e];
      }
    }
  }
}

static size_t k2b_lds(int C, int dk, int es, int nst) {
  return (size_t)nst * k2b_stage(C, dk, es).bytes + (size_t)2 * K2B_DVT * (dk + 16 / es) * es +
         (size_t)4 * 16 * (K2B_DVT + 16 / es) * es;
}

size_t k2b_lds_bytes(int C, int dk, bool bf16_path) {
  const int es = bf16_path ? 2 : 4;
  return k2b_lds(C, dk, es, k2b_lds(C, dk, es, 3) <= 160 * 1024 ? 3 : 2);
}

int k2b_dvt() { return K2B_DVT; }

template <typename T, int SRT, int NST>
static void launch_k2b_n(const K2Params& P, dim3 grid, size_t lds, hipStream_t stream) {
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&k2b_gla_state<T, SRT, NST>),
                      hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  hipLaunchKernelGGL((k2b_gla_state<T, SRT, NST>), grid, dim3(K2B_THREADS), lds, stream, P);
}

template <typename T, int SRT>
static void launch_k2b_s(const K2Params& P, dim3 grid, hipStream_t stream) {
  const int es = sizeof(T);
  if (k2b_lds(P.C, P.dk, es, 3) <= 160 * 1024)
    launch_k2b_n<T, SRT, 3>(P, grid, k2b_lds(P.C, P.dk, es, 3), stream);
  else
    launch_k2b_n<T, SRT, 2>(P, grid, k2b_lds(P.C, P.dk, es, 2), stream);
}

template <typename T>
static void launch_k2b_t(const K2Params& P, dim3 grid, hipStream_t stream) {
  const int nrt = P.dk / 16;
  if (nrt <= 4)
    launch_k2b_s<T, 1>(P, grid, stream);
  else if (nrt <= 8)
    launch_k2b_s<T, 2>(P, grid, stream);
  else
    launch_k2b_s<T, 4>(P, grid, stream);
}

hipError_t launch_k2b(const K2Params& P, bool bf16_path, hipStream_t stream) {
  const dim3 grid(((P.total_seqs + N_XCD - 1) / N_XCD) * N_XCD * P.n_dvt);
  if (bf16_path)
    launch_k2b_t<bf16>(P, grid, stream);
  else
    launch_k2b_t<float>(P, grid, stream);
  return hipGetLastError();
}

}  // namespace msgla
