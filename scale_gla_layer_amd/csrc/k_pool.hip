// Pooling prepass: the non-overlapping block means of Eq. (8) (MS-GLA notes,
// Sec. 3.1) for every coarse branch, rounded once to the storage type.
//
// X is read once for all scales that divide the largest coarse scale s_max:
// a thread sums one 16-byte column piece over a block of s_max rows in fp32
// and emits the block means of every such scale (a partial tail block is not
// pooled: it never reaches the recurrence).  Scales that do not divide s_max
// take a second pass of their own.  HBM-bound: reads B L d elements per pass,
// writes sum_s B floor(L/s) d.  With a token mask M the mean of a block is
// sum M x / max(1, sum M) (Eq. (8)): a block without tokens pools to zero.
// Masked bf16 calls also write each mean's residual m - bf16(m) (xp_lo), so
// the projection can take the mean at fp32 accuracy as hi + lo.
#include "device_common.hpp"
#include "layout.hpp"

namespace msgla {

// Stores the means m (PER values) at element offset off of the block-mean
// buffer and, where a residual buffer is given (bf16 storage), m - bf16(m).
template <typename T>
__device__ __forceinline__ void store_mean(const PoolOut& o, size_t off, const float* m) {
  constexpr int PER = per16<T>();
  const u32x4 hi = pack16<T>(m);
  st16(reinterpret_cast<T*>(o.xp) + off, hi);
  if constexpr (sizeof(T) == 2) {
    if (o.xp_lo) {
      float h[PER], r[PER];
      unpack16<T>(hi, h);
#pragma unroll
      for (int e = 0; e < PER; ++e) r[e] = m[e] - h[e];
      st16(reinterpret_cast<T*>(o.xp_lo) + off, pack16<T>(r));
    }
  }
}

// One thread per (row block, 16-byte column piece), consecutive threads on
// consecutive pieces of the same rows.  The rows of a block are loaded U at a
// time before any of them is summed, so each thread keeps U loads in flight.
template <typename T>
__global__ __launch_bounds__(256) void k_pool(const PoolParams P) {
  constexpr int PER = per16<T>();
  constexpr int U = 8;
  const int pieces = P.d / PER;
  const int nblk = (P.L + P.smax - 1) / P.smax;
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long)P.B * nblk * pieces) return;
  const int grp = (int)(idx / pieces), piece = (int)(idx - (long)grp * pieces);
  const int b = grp / nblk, q = grp - b * nblk;
  const T* x = reinterpret_cast<const T*>(P.x) + ((size_t)b * P.L + (size_t)q * P.smax) * P.d +
               piece * PER;
  const int rows = min(P.smax, P.L - q * P.smax);
  const uint8_t* mk = P.mask ? P.mask + (size_t)b * P.L + (size_t)q * P.smax : nullptr;
  float acc[MSGLA_MAX_BRANCHES][PER], den[MSGLA_MAX_BRANCHES];
  int cnt[MSGLA_MAX_BRANCHES], jout[MSGLA_MAX_BRANCHES];
#pragma unroll
  for (int i = 0; i < MSGLA_MAX_BRANCHES; ++i) {
    cnt[i] = 0;
    den[i] = 0.f;
    jout[i] = i < P.nout ? q * (P.smax / P.out[i].s) : 0;  // s divides smax
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[i][e] = 0.f;
  }
  for (int u0 = 0; u0 < rows; u0 += U) {
    u32x4 raw[U];
    float wt[U];
#pragma unroll
    for (int k = 0; k < U; ++k) {
      raw[k] = (u0 + k < rows) ? ld16(x + (size_t)(u0 + k) * P.d) : zero16();
      wt[k] = (mk && u0 + k < rows) ? (mk[u0 + k] ? 1.f : 0.f) : 1.f;
    }
#pragma unroll
    for (int k = 0; k < U; ++k) {
      if (u0 + k >= rows) break;
      float v[PER];
      unpack16<T>(raw[k], v);
#pragma unroll
      for (int i = 0; i < MSGLA_MAX_BRANCHES; ++i) {
        if (i < P.nout) {
          const PoolOut& o = P.out[i];
#pragma unroll
          for (int e = 0; e < PER; ++e) acc[i][e] += wt[k] * v[e];
          den[i] += wt[k];
          if (++cnt[i] == o.s) {  // a block of this scale is complete
            if (jout[i] < o.n) {
              const float sc = mk ? 1.0f / fmaxf(1.f, den[i]) : o.inv_s;
              float m[PER];
#pragma unroll
              for (int e = 0; e < PER; ++e) m[e] = acc[i][e] * sc;
              store_mean<T>(o, ((size_t)b * o.n + jout[i]) * P.d + piece * PER, m);
            }
            ++jout[i];
            cnt[i] = 0;
            den[i] = 0.f;
#pragma unroll
            for (int e = 0; e < PER; ++e) acc[i][e] = 0.f;
          }
        }
      }
    }
  }
}

// Power-of-two s_max (every pooled scale is then a power of two dividing it):
// the thread loads all S = 2^LS rows of its block at once, then forms the block
// sums level by level, pairs of the previous level, and emits the means of
// each requested scale as its level completes.  The loads are unconditional (a
// short tail block re-reads its last row; blocks it does not complete are not
// emitted), so the S loads of a thread are in flight together.
template <typename T, int LS>
__global__ __launch_bounds__(256) void k_pool_pow2(const PoolParams P) {
  constexpr int PER = per16<T>(), S = 1 << LS;
  const int pieces = P.d / PER;
  const int nblk = (P.L + S - 1) / S;
  const int idx = blockIdx.x * 256 + threadIdx.x;  // the launcher keeps the count below 2^31
  if (idx >= P.B * nblk * pieces) return;
  const int grp = idx / pieces, piece = idx - grp * pieces;
  const int b = grp / nblk, q = grp - b * nblk;
  const T* x = reinterpret_cast<const T*>(P.x) + ((size_t)b * P.L + (size_t)q * S) * P.d + piece * PER;
  const int last = min(S, P.L - q * S) - 1;
  u32x4 raw[S];
#pragma unroll
  for (int u = 0; u < S; ++u) raw[u] = ld16(x + (size_t)min(u, last) * P.d);
  // token weights and counts of Eq. (8) with a mask (a tail block's missing
  // rows re-read the last row; the blocks they would join are not emitted)
  const uint8_t* mk = P.mask ? P.mask + (size_t)b * P.L + (size_t)q * S : nullptr;
  float c[S];
#pragma unroll
  for (int u = 0; u < S; ++u) c[u] = mk ? (mk[min(u, last)] ? 1.f : 0.f) : 1.f;
  // every load is issued before the first one is used (the scheduler would
  // otherwise start unpacking between them and wait on the early ones)
#pragma unroll
  for (int u = 0; u < S; ++u) asm volatile("" : "+v"(raw[u])::"memory");
  float v[S][PER];
#pragma unroll
  for (int u = 0; u < S; ++u) unpack16<T>(raw[u], v[u]);
  if (mk) {
#pragma unroll
    for (int u = 0; u < S; ++u)
#pragma unroll
      for (int e = 0; e < PER; ++e) v[u][e] *= c[u];
  }
#pragma unroll
  for (int l = 1; l <= LS; ++l) {
#pragma unroll
    for (int j = 0; j < (S >> l); ++j) {
#pragma unroll
      for (int e = 0; e < PER; ++e) v[j][e] = v[2 * j][e] + v[2 * j + 1][e];
      c[j] = c[2 * j] + c[2 * j + 1];
    }
    const int i = P.lvl[l];
    if (i >= 0) {
      const PoolOut& o = P.out[i];
#pragma unroll
      for (int j = 0; j < (S >> l); ++j) {
        const int jo = q * (S >> l) + j;
        if (jo < o.n) {
          const float sc = mk ? 1.0f / fmaxf(1.f, c[j]) : o.inv_s;
          float m[PER];
#pragma unroll
          for (int e = 0; e < PER; ++e) m[e] = v[j][e] * sc;
          store_mean<T>(o, ((size_t)b * o.n + jo) * P.d + piece * PER, m);
        }
      }
    }
  }
}

// A forward continuing from a state: branch s's blocks start r = (entry
// position mod s) positions before the call (block 0 completes the entry
// state's pending block, whose masked sum and token count the state holds),
// so they no longer line up across scales.  One thread per (branch, b, block
// j, 16-byte column piece) sums the block's positions in the call, [j s - r,
// (j + 1) s - r) within [0, L), plus for block 0 the pending sum, and divides
// by the token count: Eq. (8), where positions of the call without a mask
// count as tokens.  Rows j >= floor((L + r) / s) are not written.
template <typename T>
__global__ __launch_bounds__(256) void k_pool_cont(const PoolParams P) {
  constexpr int PER = per16<T>();
  const int pieces = P.d / PER;
  long idx = (long)blockIdx.x * 256 + threadIdx.x;
  int i = 0;
  for (; i < P.nout; ++i) {
    const long cnt = (long)P.B * P.out[i].n * pieces;
    if (idx < cnt) break;
    idx -= cnt;
  }
  if (i >= P.nout) return;
  const PoolOut& o = P.out[i];
  const int piece = (int)(idx % pieces);
  const long bj = idx / pieces;
  const int j = (int)(bj % o.n), b = (int)(bj / o.n);
  const int r = entry_offset(P.chk, o.branch), nv = blocks_in_call(P.chk, o.branch, o.n);
  if (j >= nv) return;
  const int t_lo = j * o.s - r, t_hi = min(t_lo + o.s, P.L);
  float acc[PER], den = 0.f;
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  if (t_lo < 0 && o.psum_in && state_in_ok(P.chk)) {
    // the entry state's pending positions (block 0 only)
    const float* ps = o.psum_in + (size_t)b * P.d + piece * PER;
#pragma unroll
    for (int e = 0; e < PER; e += 4) unpack16<float>(ld16(ps + e), acc + e);
    den = o.tok_in[b];
  }
  const T* x = reinterpret_cast<const T*>(P.x) + (size_t)b * P.L * P.d + piece * PER;
  const uint8_t* mk = P.mask ? P.mask + (size_t)b * P.L : nullptr;
  for (int t = max(t_lo, 0); t < t_hi; ++t) {
    const float w = mk ? (mk[t] ? 1.f : 0.f) : 1.f;
    float v[PER];
    unpack16<T>(ld16(x + (size_t)t * P.d), v);
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] += w * v[e];
    den += w;
  }
  const float sc = 1.0f / fmaxf(1.f, den);
  float m[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) m[e] = acc[e] * sc;
  store_mean<T>(o, ((size_t)b * o.n + j) * P.d + piece * PER, m);
}

template <typename T>
static void launch_pool_t(const PoolParams& P, hipStream_t st) {
  if (P.chk) {
    long threads = 0;
    for (int i = 0; i < P.nout; ++i) threads += (long)P.B * P.out[i].n * (P.d / per16<T>());
    if (threads == 0) return;
    hipLaunchKernelGGL(k_pool_cont<T>, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st, P);
    return;
  }
  const long threads = (long)P.B * ((P.L + P.smax - 1) / P.smax) * (P.d / per16<T>());
  const dim3 grid((unsigned)((threads + 255) / 256)), block(256);
  switch (threads + 255 < (1L << 31) ? P.smax : 0) {
    case 2: hipLaunchKernelGGL((k_pool_pow2<T, 1>), grid, block, 0, st, P); return;
    case 4: hipLaunchKernelGGL((k_pool_pow2<T, 2>), grid, block, 0, st, P); return;
    case 8: hipLaunchKernelGGL((k_pool_pow2<T, 3>), grid, block, 0, st, P); return;
    case 16: hipLaunchKernelGGL((k_pool_pow2<T, 4>), grid, block, 0, st, P); return;
    default: hipLaunchKernelGGL(k_pool<T>, grid, block, 0, st, P); return;
  }
}

hipError_t launch_pool(const PoolParams& P0, bool bf16_path, hipStream_t st) {
  PoolParams P = P0;
  for (int l = 0; l < 8; ++l) P.lvl[l] = -1;
  for (int i = 0; i < P.nout; ++i)
    for (int l = 1; l < 8; ++l)
      if (P.out[i].s == (1 << l)) P.lvl[l] = i;
  if (bf16_path)
    launch_pool_t<bf16>(P, st);
  else
    launch_pool_t<float>(P, st);
  return hipGetLastError();
}

}  // namespace msgla
