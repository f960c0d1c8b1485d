// Streaming-state header and the end-of-forward export of the per-branch cache.
//
// MS-GLA notes, paragraph on token-by-token inference (the author's cache):
// each branch keeps its GLA state, the not-yet-complete block of hidden
// states and its most recent output.  A forward over L tokens that starts
// with r positions of branch s's block already pending (r = entry position
// mod s, 0 for a fresh call) completes n = floor((L + r)/s) blocks, block j
// covering call positions [j s - r, (j + 1) s - r) (block 0 with the pending
// ones).  The state kernel writes the GLA state directly; this kernel adds the
// sum and the count of the tokens among the pending positions after the call
// (all of them without a token mask; with no complete block, the entry
// state's pending sum and count as well) and the held output
// Y_{n-1} = y_{n-1} W_o (the entry's held output when n = 0), and sets the
// position in the header.  A forward continuing from a state first checks
// that state's header on the device (k_state_check); the readers of the entry
// state use it only if the check passed.
#include "device_common.hpp"
#include "layout.hpp"

namespace msgla {

// Header of a state written after `pos` more tokens: position = entry position
// (from the forward's check of its state_in, else 0) + pos; a failed check
// gives status = that check's code and position -1, which later calls reject.
__global__ void k_state_header(void* state, int B, int m, int64_t pos, const StateCheck* chk) {
  if (threadIdx.x == 0 && blockIdx.x == 0) {
    StateHeader* h = reinterpret_cast<StateHeader*>(state);
    const int32_t status = chk ? chk->status : 0;
    h->magic = STATE_MAGIC;
    h->version = STATE_VERSION;
    h->B = B;
    h->m = m;
    h->pos = status != 0 ? -1 : (chk ? chk->pos : 0) + pos;
    h->status = status;
    h->pad = 0;
  }
}

// Check of a forward's state_in header against its configuration and batch
// (one thread): status 0, or 1 (MSGLA_ERR_INVALID_ARG: not a state of this
// configuration and batch, or a state that records an error).  On success it
// also gives every branch's entry offset r = position mod s and the number of
// blocks the call completes, floor((L + r) / s).
__global__ void k_state_check(const StateCheckParams P) {
  if (threadIdx.x == 0 && blockIdx.x == 0) {
    const StateHeader* h = reinterpret_cast<const StateHeader*>(P.state_in);
    const bool ok = h->magic == STATE_MAGIC && h->version == STATE_VERSION && h->B == P.B &&
                    h->m == P.m && h->status == 0 && h->pos >= 0;
    P.out->status = ok ? 0 : 1;
    P.out->pad = 0;
    P.out->pos = ok ? h->pos : 0;
    for (int i = 0; i < MSGLA_MAX_BRANCHES; ++i) {
      const int r = ok && i < P.m ? (int)(h->pos % P.scale[i]) : 0;
      P.out->r[i] = r;
      P.out->nv[i] = i < P.m ? (P.L + r) / P.scale[i] : 0;
    }
  }
}

// Continuing from a state: each branch's pending block enters block 0 of the
// call, whose gate first factor averages x W_g1 over the block's tokens, so
// the pending part needs its sum psum W_g1 (by linearity).  grid (m, B), one
// workgroup of 256 threads per (branch, sequence): out[i][b][c] = sum_k
// psum[i][b][k] W_g1^(i)[k][c] for c < rp, in fp32 (W_g1 as packed: row c of
// the branch's transposed projection block).
template <typename T>
__global__ __launch_bounds__(256) void k_pending_gate(const PendingGateParams P) {
  const int i = blockIdx.x, b = blockIdx.y;
  const PendingGateBranch& Br = P.br[i];
  __shared__ float part[4][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const bool ok = state_in_ok(P.chk);
  const float* ps = Br.psum + (size_t)b * P.d;
  for (int c = 0; c < P.rp; ++c) {
    const T* w = reinterpret_cast<const T*>(Br.Wg1) + (size_t)c * P.d;
    float acc = 0.f;
    if (ok)
      for (int k = threadIdx.x; k < P.d; k += 256) acc = fmaf(ps[k], to_f32(w[k]), acc);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
    if (lane == 0) part[wave][c & 63] = acc;
    __syncthreads();
    if (threadIdx.x == 0)
      Br.out[(size_t)b * P.rp + c] = part[0][c & 63] + part[1][c & 63] + part[2][c & 63] + part[3][c & 63];
    __syncthreads();
  }
}

// grid: (ceil(d / 256), B, m)
template <typename T>
__global__ void k_state_export(const StateParams P) {
  const int col = blockIdx.x * blockDim.x + threadIdx.x;
  const int b = blockIdx.y, i = blockIdx.z;
  const StateBranch& Br = P.br[i];
  const uint8_t* mk = P.mask ? P.mask + (size_t)b * P.L : nullptr;
  const bool entry = state_in_ok(P.chk) && P.chk;  // a checked entry state
  const int r = entry_offset(P.chk, i), n = blocks_in_call(P.chk, i, Br.n);
  // the incomplete block after the call: call positions [n s - r, L), and the
  // entry state's pending positions too when no block completed
  const int t0 = n * Br.s - r;
  const bool carry = entry && n == 0 && Br.psum_in;
  // tokens and token sum are read before either is written (state_in may be
  // state_out): each thread reads and writes only its own entries
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    // tokens of the incomplete block (Eq. (8): its pooling divides by them)
    float c = carry ? Br.tok_in[b] : 0.f;
    for (int t = max(t0, 0); t < P.L; ++t) c += mk ? (mk[t] ? 1.f : 0.f) : 1.f;
    Br.tok[b] = c;
  }
  if (col < P.d) {
    // sum of the tokens of the incomplete block
    const T* x = reinterpret_cast<const T*>(P.x);
    float s = carry ? Br.psum_in[(size_t)b * P.d + col] : 0.f;
    for (int t = max(t0, 0); t < P.L; ++t)
      if (!mk || mk[t]) s += to_f32(x[((size_t)b * P.L + t) * P.d + col]);
    Br.psum[(size_t)b * P.d + col] = s;
    // held output of the last complete block (or, without one, the output
    // held on entry)
    float acc = Br.held_in && state_in_ok(P.chk) ? Br.held_in[(size_t)b * P.d + col] : 0.f;
    if (n > 0) {
      acc = 0.f;
      const T* y = reinterpret_cast<const T*>(Br.y);
      const T* wo = reinterpret_cast<const T*>(P.WoT) + (size_t)col * P.Ktot + Br.ko;
      for (int hh = 0; hh < Br.h; ++hh) {
        const T* yr = y + (((size_t)b * Br.h + hh) * Br.np + (n - 1)) * P.dv;
        for (int v = 0; v < P.dv; ++v) acc = fmaf(to_f32(yr[v]), to_f32(wo[hh * P.dv + v]), acc);
      }
    }
    Br.held[(size_t)b * P.d + col] = acc;
  }
  // a branch that saw no complete block keeps its GLA state: zero, or the
  // entry state, which the state kernel has already copied to the output
  if (n == 0 && !(Br.S_in && state_in_ok(P.chk))) {
    const size_t per_b = (size_t)Br.h * P.dk * P.dv;
    for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < per_b;
         e += (size_t)gridDim.x * blockDim.x)
      Br.S[(size_t)b * per_b + e] = 0.f;
  }
}

hipError_t launch_state_header(void* state, int B, int m, int64_t pos, const StateCheck* chk,
                               hipStream_t st) {
  hipLaunchKernelGGL(k_state_header, dim3(1), dim3(64), 0, st, state, B, m, pos, chk);
  return hipGetLastError();
}

hipError_t launch_state_check(const StateCheckParams& P, hipStream_t st) {
  hipLaunchKernelGGL(k_state_check, dim3(1), dim3(64), 0, st, P);
  return hipGetLastError();
}

hipError_t launch_pending_gate(const PendingGateParams& P, bool bf16_path, hipStream_t st) {
  const dim3 grid(P.m, P.B);
  if (bf16_path)
    hipLaunchKernelGGL(k_pending_gate<bf16>, grid, dim3(256), 0, st, P);
  else
    hipLaunchKernelGGL(k_pending_gate<float>, grid, dim3(256), 0, st, P);
  return hipGetLastError();
}

hipError_t launch_state_export(const StateParams& P, bool bf16_path, hipStream_t st) {
  const dim3 grid((P.d + 255) / 256, P.B, P.m);
  if (bf16_path)
    hipLaunchKernelGGL(k_state_export<bf16>, grid, dim3(256), 0, st, P);
  else
    hipLaunchKernelGGL(k_state_export<float>, grid, dim3(256), 0, st, P);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  return launch_state_header(P.state, P.B, P.m, P.pos, P.chk, st);
}

}  // namespace msgla
