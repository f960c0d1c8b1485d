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
// The eight waves split the two products of a chunk: waves 0-3 ("output
// waves") form y rows 16w .. 16w+15 from S_c, waves 4-7 ("state waves") keep
// 16-row tiles of S in fp32 MFMA accumulators across the whole walk
// (rows c with (c / 16) % 4 == w - 4), form S_{c+1} and publish it to LDS in
// the storage type (transposed, [v][c], double-buffered by chunk parity) as
// the B-operand of the next chunk's qt S.  On each SIMD one output and one
// state wave run side by side.  The walk is latency-bound unless the inputs
// of later chunks are already in flight: A, qt, kT, the chunk's V slice and
// lam are copied global -> LDS asynchronously (global_load_lds_dwordx4, no
// VGPRs) into NST rotating stages, NST-1 chunks ahead of the compute, by two
// more waves that do nothing else and take the copy instructions in turn (the
// copies of one chunk keep the CU's vector-memory path busy for about as long
// as the chunk's products take, and a compute wave that issued them would
// wait that long), with vmcnt waits on the copy waves and one barrier per
// chunk.  V positions beyond the sequence end
// are zeroed in the fragments (the workspace there is never written).
// After the last chunk the fp32 state is optionally written out.
#include <type_traits>

#include "async_copy.hpp"
#include "device_common.hpp"
#include "layout.hpp"

namespace msgla {

constexpr int K2B_COPY_WAVES = 2;
constexpr int K2B_THREADS = 64 * (8 + K2B_COPY_WAVES);  // 4 output waves + 4 state waves + the copy waves
constexpr int K2B_DVT = 32;  // d_v columns per workgroup

constexpr int k2b_kb(int b) { return (b + 1023) & ~1023; }
constexpr int k2b_ilog2(int x) { return x <= 1 ? 0 : 1 + k2b_ilog2(x / 2); }

// Compile-time geometry for chunk length C and key width DK (powers of two).
// A pipeline stage holds, 1 KB aligned: A [C][C], qt [C][DK], kT [DK][C],
// the chunk's V slice [DVT][C] (storage type) and lam [DK] (fp32).
template <typename T, int C, int DK>
struct K2bGeom {
  static constexpr int es = sizeof(T);
  static constexpr int NSC = C * es / 64;   // 64-byte k-slabs over positions
  static constexpr int NSK = DK * es / 64;  // 64-byte k-slabs over key channels
  static constexpr int NRT = DK / 16;       // 16-row tiles of the state
  static constexpr int SRT = (NRT + 3) / 4; // state row tiles per state wave
  static constexpr int bA = C * C * es, bQ = C * DK * es, bV = K2B_DVT * C * es, bL = DK * 4;
  static constexpr int oA = 0, oQ = k2b_kb(bA), oK = oQ + k2b_kb(bQ), oV = oK + k2b_kb(bQ),
                       oL = oV + k2b_kb(bV), STAGE = oL + k2b_kb(bL);
  static constexpr int nA = bA / 1024, nQ = bQ / 1024, nV = bV / 1024;  // copy instructions
  static constexpr int lgC = k2b_ilog2(C * es), lgQ = k2b_ilog2(DK * es), lgL = k2b_ilog2(DK * 4);
  static constexpr int LDS_S = DK + 16 / es;       // published-state row stride (elements)
  static constexpr int EXTRA = 2 * K2B_DVT * LDS_S * es;
  static constexpr int NST = 3 * STAGE + EXTRA <= 160 * 1024 ? 3 : 2;
  static constexpr int LDS = NST * STAGE + EXTRA;
  // copy instructions per chunk (all issued by the copy waves)
  static constexpr int NCOPY = nA + 2 * nQ + nV + (bL <= 1024 ? 1 : 0);
  static constexpr int NCOPY_S = nQ + nV + (bL <= 1024 ? 1 : 0);  // state-only walk: kT, V, lam
  static_assert(bA % 1024 == 0 && bQ % 1024 == 0 && bV % 1024 == 0 && bL <= 1024, "block sizes");
  static_assert(NSC >= 1 && NSC <= 4 && NSK >= 1 && NSK <= 16, "slab counts");
};

// Per-lane source offset of copy instruction k for a contiguous block stored
// as swizzled 128-byte virtual rows (async_copy.hpp): source = block + 1024 k
// + off.  The swizzle key of instruction k is ((8 k + lane / 8) >> hs) & 7,
// which for rows of up to 1 KB (hs <= 3) depends on k mod 8 only, so wave w
// (instructions k = w, w + 8, ...) needs one offset per block.
__device__ __forceinline__ int k2b_lane_off(int lg, int k, int lane) {
  const int hs = blk_hs(lg);
  const int vrow = 8 * k + (lane >> 3);
  return 128 * (lane >> 3) + 16 * ((lane & 7) ^ ((vrow >> hs) & 7));
}

// SONLY: the state-only pass of the segmented walk (no A, qt or y; the
// segment's local final state from zero goes to Sseg).
template <typename T, int C, int DK, bool SONLY>
__global__ __launch_bounds__(K2B_THREADS) void k2b_gla_state(const K2Params P) {
  using G = K2bGeom<T, C, DK>;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int seg = blockIdx.x / P.seg_base;
  const int g = blockIdx.x - seg * P.seg_base;
  const int slot = g / N_XCD, xcd = g % N_XCD;
  const int qseq = (slot / P.n_dvt) * N_XCD + xcd;
  const int tile = slot % P.n_dvt;
  if (qseq >= P.total_seqs) return;
  int bi = P.order[0];
  for (int o = 1; o < P.nbranch; ++o)
    if (qseq >= P.br[P.order[o]].seq_begin) bi = P.order[o];
  const K2Branch& Bb = P.br[bi];
  const int bh = qseq - Bb.seq_begin;  // b * h + head
  // this workgroup's chunks [cb, cb + cnt) and its start / end states
  const int seg_len = (Bb.nch + P.nseg - 1) / max(P.nseg, 1);
  const int cb = seg * seg_len;
  const int cnt = max(0, min(Bb.nch, cb + seg_len) - cb);
  const bool last_seg = P.nseg == 1 || seg == max(0, (Bb.nch - 1) / max(seg_len, 1));
  if (P.nseg > 1 && cnt == 0 && (SONLY || !last_seg)) return;  // the whole workgroup
  float* Sseg_slot = P.Sseg ? P.Sseg + (size_t)(qseq * P.nseg + seg) * DK * P.dv : nullptr;
  const float* S_in = Bb.S_in && state_in_ok(P.chk) ? Bb.S_in : nullptr;
  const float* S_start = SONLY ? nullptr : (P.nseg > 1 ? Sseg_slot : (S_in ? S_in + (size_t)bh * DK * P.dv : nullptr));
  float* S_end = SONLY ? Sseg_slot : (last_seg && Bb.S_out ? Bb.S_out + (size_t)bh * DK * P.dv : nullptr);

  constexpr int es = G::es;
  constexpr int PER = per16<T>();
  constexpr int NST = G::NST;
  const int dv = P.dv;
  const int v0 = tile * K2B_DVT;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool out_wave = wave < 4;
  const int w4 = wave & 3;  // index among the output waves or among the state waves
  const int lr = lane & 15, lgp = lane >> 4;

  // LDS: NST stages | ST[2][DVT][DK + pad] (published state)
  T* ST = reinterpret_cast<T*>(smem + NST * G::STAGE);

  const size_t chunk0 = (size_t)bh * Bb.nch;
  const char* Ag = reinterpret_cast<const char*>(Bb.A) + chunk0 * G::bA;
  const char* Qg = reinterpret_cast<const char*>(Bb.qt) + (size_t)bh * Bb.np * DK * es;
  const char* Kg = reinterpret_cast<const char*>(Bb.kT) + chunk0 * G::bQ;
  const char* Vg = reinterpret_cast<const char*>(Bb.vT) + (chunk0 * dv + v0) * C * es;
  const char* Lg = reinterpret_cast<const char*>(Bb.lam + chunk0 * DK);
  T* yg = reinterpret_cast<T*>(Bb.y) + (size_t)bh * Bb.np * dv + v0;

  // Waves 8 and up issue every copy, taking a chunk's copy instructions in turn
  // (a chunk's ~45 copy instructions occupy the CU's vector-memory path for
  // about as long as the chunk's products take, and one wave alone issues them
  // slower than the path takes them): the compute waves never queue behind
  // copy instructions, and a copy wave's vmcnt holds nothing but its own
  // copies, so its waits are exact.
  const int oL = 16 * lane;  // lam: one partial instruction of one virtual row (key 0)
  auto issue = [&](int i, int cw) {
    int n = 0;  // copy instructions of the chunk so far (wave-uniform)
    auto cp = [&](const char* src, char* dst, bool lane_on) {
      if (n++ % K2B_COPY_WAVES == cw && lane_on) dma16(src, dst);
    };
    const int c = cb + i;
    char* st = smem + (i % NST) * G::STAGE;
    const char* a = Ag + (size_t)c * G::bA;
    const char* q = Qg + (size_t)c * G::bQ;
    const char* kk = Kg + (size_t)c * G::bQ;
    const char* v = Vg + (size_t)c * dv * C * es;
    // the V slice first: the one block that comes from HBM rather than L2
#pragma unroll
    for (int k = 0; k < G::nV; ++k) cp(v + 1024 * k + k2b_lane_off(G::lgC, k, lane), st + G::oV + 1024 * k, true);
    cp(Lg + (size_t)c * G::bL + oL, st + G::oL, oL < G::bL);
#pragma unroll
    for (int k = 0; k < G::nQ; ++k) {
      cp(kk + 1024 * k + k2b_lane_off(G::lgC, k, lane), st + G::oK + 1024 * k, true);
      if constexpr (!SONLY) cp(q + 1024 * k + k2b_lane_off(G::lgQ, k, lane), st + G::oQ + 1024 * k, true);
    }
    if constexpr (!SONLY) {
#pragma unroll
      for (int k = 0; k < G::nA; ++k) cp(a + 1024 * k + k2b_lane_off(G::lgC, k, lane), st + G::oA + 1024 * k, true);
    }
  };
  constexpr int NCP = SONLY ? G::NCOPY_S : G::NCOPY;
  if (wave >= 8) {
    const int cw = wave - 8;
    // copy wave cw's instructions per chunk: every K2B_COPY_WAVES-th from the cw-th
    auto copy_loop = [&](auto per_chunk) {
      constexpr int W = decltype(per_chunk)::value;
      for (int i = 0; i < NST - 1 && i < cnt; ++i) issue(i, cw);
      for (int i = 0; i < cnt; ++i) {
        // stage i has landed once only the copies of later stages remain
        if (NST > 2 && i + 1 < cnt)
          wait_vmcnt<(W < 63 ? W : 63)>();
        else
          wait_vmcnt<0>();
        lds_barrier();
        if (i + NST - 1 < cnt) issue(i + NST - 1, cw);
      }
    };
    static_assert(K2B_COPY_WAVES == 2, "copy-wave split");
    if (cw == 0)
      copy_loop(std::integral_constant<int, (NCP + 1) / 2>());
    else
      copy_loop(std::integral_constant<int, NCP / 2>());
    return;
  }

  // LDS fragment offsets inside a stage
  int offV[G::NSC][2], offA[G::NSC], offK[G::SRT][G::NSC], offQ[G::NSK], offL[G::SRT];
#pragma unroll
  for (int sl = 0; sl < G::NSC; ++sl) {
    offV[sl][0] = G::oV + tile_off(lr, sl * 4 + lgp, G::lgC);
    offV[sl][1] = G::oV + tile_off(16 + lr, sl * 4 + lgp, G::lgC);
    offA[sl] = G::oA + tile_off(16 * w4 + lr, sl * 4 + lgp, G::lgC);
#pragma unroll
    for (int a = 0; a < G::SRT; ++a) offK[a][sl] = G::oK + tile_off(16 * (w4 + 4 * a) + lr, sl * 4 + lgp, G::lgC);
  }
#pragma unroll
  for (int sl = 0; sl < G::NSK; ++sl) offQ[sl] = G::oQ + tile_off(16 * w4 + lr, sl * 4 + lgp, G::lgQ);
#pragma unroll
  for (int a = 0; a < G::SRT; ++a) offL[a] = G::oL + tile_off(0, (16 * (w4 + 4 * a) + 4 * lgp) >> 2, G::lgL);

  f32x4 S[G::SRT][2];
#pragma unroll
  for (int a = 0; a < G::SRT; ++a) S[a][0] = S[a][1] = zero4();

  if (!S_start) {
    for (int i = tid; i < K2B_DVT * G::LDS_S; i += 512) ST[i] = from_f32<T>(0.f);
  } else if (!out_wave) {
    // continuing from a state: each state wave loads its rows of S and
    // publishes them for chunk 0 as it would a carried state
    const float* Si = S_start;
#pragma unroll
    for (int a = 0; a < G::SRT; ++a) {
      const int rt = w4 + 4 * a;
      if (rt < G::NRT) {
        const int c4 = 16 * rt + 4 * lgp;
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
#pragma unroll
          for (int e = 0; e < 4; ++e) S[a][ct][e] = Si[(size_t)(c4 + e) * dv + v0 + 16 * ct + lr];
          const float f[4] = {S[a][ct][0], S[a][ct][1], S[a][ct][2], S[a][ct][3]};
          T* dst = ST + (16 * ct + lr) * G::LDS_S + c4;
          if constexpr (sizeof(T) == 2)
            st8(dst, pack8<T>(f));
          else
            st16(dst, pack16<T>(f));
        }
      }
    }
  }

  for (int i = 0; i < cnt; ++i) {
    const int c = cb + i;
    lds_barrier();  // stage i has landed (the copy wave waited for it)

    const char* st = smem + (i % NST) * G::STAGE;
    const int valid = min(C, blocks_in_call(P.chk, bi, Bb.n) - c * C);

    // V fragments (B-operand of both products); positions >= valid zeroed
    u32x4 vf[G::NSC][2];
#pragma unroll
    for (int sl = 0; sl < G::NSC; ++sl) {
      vf[sl][0] = ld16(st + offV[sl][0]);
      vf[sl][1] = ld16(st + offV[sl][1]);
    }
    if (valid < C) {
#pragma unroll
      for (int sl = 0; sl < G::NSC; ++sl)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          const int tau0 = (sl * 4 + lgp) * PER;
          float u[PER];
          unpack16<T>(vf[sl][ct], u);
#pragma unroll
          for (int e = 0; e < PER; ++e)
            if (tau0 + e >= valid) u[e] = 0.f;
          vf[sl][ct] = pack16<T>(u);
        }
    }

    if (SONLY && out_wave) {
      // state-only pass: the output waves only keep the barriers
    } else if (out_wave) {
      // ---- y rows 16w .. 16w+15 as y^T = V^T A^T + S_c^T qt^T: with V (and the
      // published S^T) as the A-operand, lane l holds 4 consecutive v of
      // position 16w + l % 16, which go straight to global memory ----
      if (w4 < C / 16) {
        const T* Sb = ST + (i & 1) * K2B_DVT * G::LDS_S;
        u32x4 af[G::NSC], qf[G::NSK], sf[G::NSK][2];
#pragma unroll
        for (int sl = 0; sl < G::NSC; ++sl) af[sl] = ld16(st + offA[sl]);
#pragma unroll
        for (int sl = 0; sl < G::NSK; ++sl) {
          qf[sl] = ld16(st + offQ[sl]);
          const T* srow = Sb + lr * G::LDS_S + sl * slab_elems<T>() + lgp * PER;
          sf[sl][0] = ld16(srow);
          sf[sl][1] = ld16(srow + 16 * G::LDS_S);
        }
        // two accumulators per column tile (intra-chunk, inter-chunk) keep the
        // dependent MFMA chains short
        f32x4 yi[2] = {zero4(), zero4()}, yo[2] = {zero4(), zero4()};
#pragma unroll
        for (int sl = 0; sl < G::NSC; ++sl) {
          yi[0] = mma_slab<T>(vf[sl][0], af[sl], yi[0]);
          yi[1] = mma_slab<T>(vf[sl][1], af[sl], yi[1]);
        }
#pragma unroll
        for (int sl = 0; sl < G::NSK; ++sl) {
          yo[0] = mma_slab<T>(sf[sl][0], qf[sl], yo[0]);
          yo[1] = mma_slab<T>(sf[sl][1], qf[sl], yo[1]);
        }
        const int t = 16 * w4 + lr;
        if (t < valid) {
          T* dst = yg + ((size_t)c * C + t) * dv + 4 * lgp;
#pragma unroll
          for (int ct = 0; ct < 2; ++ct) {
            float f[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) f[e] = yi[ct][e] + yo[ct][e];
            if constexpr (sizeof(T) == 2)
              st8(dst + 16 * ct, pack8<T>(f));
            else
              st16(dst + 16 * ct, pack16<T>(f));
          }
        }
      }
    } else {
      // ---- state rows: S_{c+1} = Diag(lam) S_c + kT V, published for chunk c+1 ----
      T* Sn = ST + ((i + 1) & 1) * K2B_DVT * G::LDS_S;
#pragma unroll
      for (int a = 0; a < G::SRT; ++a) {
        const int rt = w4 + 4 * a;
        if (rt < G::NRT) {
          u32x4 kf[G::NSC];
#pragma unroll
          for (int sl = 0; sl < G::NSC; ++sl) kf[sl] = ld16(st + offK[a][sl]);
          const f32x4 l4 = __builtin_bit_cast(f32x4, ld16(st + offL[a]));
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            S[a][0][e] *= l4[e];
            S[a][1][e] *= l4[e];
          }
#pragma unroll
          for (int sl = 0; sl < G::NSC; ++sl) {
            S[a][0] = mma_slab<T>(kf[sl], vf[sl][0], S[a][0]);
            S[a][1] = mma_slab<T>(kf[sl], vf[sl][1], S[a][1]);
          }
          // publish S_{c+1}: ST[v][c], 4 consecutive c per lane
          const int c4 = 16 * rt + 4 * lgp;
#pragma unroll
          for (int ct = 0; ct < 2; ++ct) {
            float f[4] = {S[a][ct][0], S[a][ct][1], S[a][ct][2], S[a][ct][3]};
            T* dst = Sn + (16 * ct + lr) * G::LDS_S + c4;
            if constexpr (sizeof(T) == 2)
              st8(dst, pack8<T>(f));
            else
              st16(dst, pack16<T>(f));
          }
        }
      }
    }
  }

  if (!out_wave && S_end) {
    float* So = S_end;
#pragma unroll
    for (int a = 0; a < G::SRT; ++a) {
      const int rt = w4 + 4 * a;
      if (rt < G::NRT) {
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            So[(size_t)(16 * rt + 4 * lgp + e) * dv + v0 + 16 * ct + lr] = S[a][ct][e];
      }
    }
  }
}

template <typename T, int C, int DK>
static void launch_k2b_cd(const K2Params& P, dim3 grid, hipStream_t stream, bool sonly) {
  using G = K2bGeom<T, C, DK>;
  if (sonly) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&k2b_gla_state<T, C, DK, true>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, G::LDS);
    hipLaunchKernelGGL((k2b_gla_state<T, C, DK, true>), grid, dim3(K2B_THREADS), G::LDS, stream, P);
  } else {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&k2b_gla_state<T, C, DK, false>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, G::LDS);
    hipLaunchKernelGGL((k2b_gla_state<T, C, DK, false>), grid, dim3(K2B_THREADS), G::LDS, stream, P);
  }
}

template <typename T, int C>
static bool launch_k2b_c(const K2Params& P, dim3 grid, hipStream_t stream, bool sonly) {
  switch (P.dk) {
    case 16: if constexpr (sizeof(T) == 4) { launch_k2b_cd<T, C, 16>(P, grid, stream, sonly); return true; } return false;
    case 32: launch_k2b_cd<T, C, 32>(P, grid, stream, sonly); return true;
    case 64: launch_k2b_cd<T, C, 64>(P, grid, stream, sonly); return true;
    case 128: launch_k2b_cd<T, C, 128>(P, grid, stream, sonly); return true;
    case 256: launch_k2b_cd<T, C, 256>(P, grid, stream, sonly); return true;
    default: return false;
  }
}

template <typename T>
static bool launch_k2b_t(const K2Params& P, dim3 grid, hipStream_t stream, bool sonly) {
  switch (P.C) {
    case 16: if constexpr (sizeof(T) == 4) return launch_k2b_c<T, 16>(P, grid, stream, sonly); return false;
    case 32: return launch_k2b_c<T, 32>(P, grid, stream, sonly);
    case 64: return launch_k2b_c<T, 64>(P, grid, stream, sonly);
    default: return false;
  }
}

// Segmented walk, between the two passes: per (sequence, key channel c) and
// every d_v column, the start state of segment p is
//   S_start(0) = S_in (or 0),  S_start(p + 1) = Diag(Lam_p) S_start(p) + S_local(p),
// Lam_p = the product of the segment's per-chunk decays lam (row c).  Sseg
// holds S_local on entry and S_start on exit.
__global__ __launch_bounds__(256) void k2b_seg_scan(const K2Params P) {
  constexpr int NCH_LDS = 8192;
  __shared__ float lam_seg[64];
  __shared__ float lam_all[NCH_LDS];
  const int qseq = blockIdx.x / P.dk, c = blockIdx.x - qseq * P.dk;
  int bi = P.order[0];
  for (int o = 1; o < P.nbranch; ++o)
    if (qseq >= P.br[P.order[o]].seq_begin) bi = P.order[o];
  const K2Branch& Bb = P.br[bi];
  const int bh = qseq - Bb.seq_begin;
  const int seg_len = (Bb.nch + P.nseg - 1) / P.nseg;
  const float* lam = Bb.lam + (size_t)bh * Bb.nch * P.dk + c;  // chunk ch at lam[ch * dk]
  const bool staged = Bb.nch <= NCH_LDS;
  if (staged) {
    // every chunk's decay of channel c, loaded by all threads at once
    for (int ch = threadIdx.x; ch < Bb.nch; ch += 256) lam_all[ch] = lam[(size_t)ch * P.dk];
    __syncthreads();
  }
  if (threadIdx.x < P.nseg) {
    const int p = threadIdx.x;
    const int c1 = min(Bb.nch, (p + 1) * seg_len);
    float prod = 1.f;
    for (int ch = p * seg_len; ch < c1; ++ch) prod *= staged ? lam_all[ch] : lam[(size_t)ch * P.dk];
    lam_seg[p] = prod;
  }
  __syncthreads();
  const float* S_in = Bb.S_in && state_in_ok(P.chk) ? Bb.S_in : nullptr;
  for (int v = threadIdx.x; v < P.dv; v += 256) {
    float cur = S_in ? S_in[((size_t)bh * P.dk + c) * P.dv + v] : 0.f;
    for (int p = 0; p < P.nseg; ++p) {
      float* slot = P.Sseg + ((size_t)(qseq * P.nseg + p) * P.dk + c) * P.dv + v;
      const float loc = *slot;
      *slot = cur;
      cur = lam_seg[p] * cur + loc;
    }
  }
}

int k2b_dvt() { return K2B_DVT; }

// LDS bytes one workgroup of the state kernel needs (0: shape not instantiated)
template <typename T, int C>
static int k2b_lds_c(int dk) {
  switch (dk) {
    case 16: if constexpr (sizeof(T) == 4) return K2bGeom<T, C, 16>::LDS; return 0;
    case 32: return K2bGeom<T, C, 32>::LDS;
    case 64: return K2bGeom<T, C, 64>::LDS;
    case 128: return K2bGeom<T, C, 128>::LDS;
    case 256: return K2bGeom<T, C, 256>::LDS;
    default: return 0;
  }
}

int k2b_lds_bytes(bool bf16_path, int C, int dk) {
  if (bf16_path) {
    if (C == 32) return k2b_lds_c<bf16, 32>(dk);
    if (C == 64) return k2b_lds_c<bf16, 64>(dk);
    return 0;
  }
  if (C == 16) return k2b_lds_c<float, 16>(dk);
  if (C == 32) return k2b_lds_c<float, 32>(dk);
  if (C == 64) return k2b_lds_c<float, 64>(dk);
  return 0;
}

hipError_t launch_k2b(const K2Params& P, bool bf16_path, hipStream_t stream) {
  const dim3 grid(P.seg_base * P.nseg);
  auto walk = [&](bool sonly) {
    return bf16_path ? launch_k2b_t<bf16>(P, grid, stream, sonly) : launch_k2b_t<float>(P, grid, stream, sonly);
  };
  if (P.nseg > 1) {
    if (!walk(true)) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k2b_seg_scan, dim3(P.total_seqs * P.dk), dim3(256), 0, stream, P);
  }
  if (!walk(false)) return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace msgla
