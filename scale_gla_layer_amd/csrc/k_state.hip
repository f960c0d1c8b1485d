// Streaming-state header and the end-of-forward export of the per-branch cache.
//
// MS-GLA notes, paragraph on token-by-token inference (the author's cache):
// each branch keeps its GLA state, the not-yet-complete block of hidden
// states and its most recent output.  After a forward over L tokens branch s
// has consumed n = floor(L/s) blocks: its GLA state is written by the state
// kernel directly; this kernel adds the sum and the count of the tokens among
// the L - n s pending positions (all of them without a token mask) and the
// held output Y_{n-1} = y_{n-1} W_o (zero when n = 0), and sets the token
// count in the header.  A forward continuing from a state first checks that
// state's header on the device (k_state_check); the readers of the entry state
// use it only if the check passed.
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
// (one thread): the codes are those of msgla_status (1 = invalid argument:
// not a state of this configuration and batch, or a state that records an
// error; 2 = unsupported: a position inside a block of some scale).
__global__ void k_state_check(const StateCheckParams P) {
  if (threadIdx.x == 0 && blockIdx.x == 0) {
    const StateHeader* h = reinterpret_cast<const StateHeader*>(P.state_in);
    int32_t status = 0;
    if (h->magic != STATE_MAGIC || h->version != STATE_VERSION || h->B != P.B || h->m != P.m ||
        h->status != 0 || h->pos < 0) {
      status = 1;
    } else {
      for (int i = 0; i < P.m; ++i)
        if (h->pos % P.scale[i] != 0) status = 2;
    }
    P.out->status = status;
    P.out->pad = 0;
    P.out->pos = status == 0 ? h->pos : 0;
  }
}

// grid: (ceil(d / 256), B, m)
template <typename T>
__global__ void k_state_export(const StateParams P) {
  const int col = blockIdx.x * blockDim.x + threadIdx.x;
  const int b = blockIdx.y, i = blockIdx.z;
  const StateBranch& Br = P.br[i];
  const uint8_t* mk = P.mask ? P.mask + (size_t)b * P.L : nullptr;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    // tokens of the incomplete block (Eq. (8): its pooling divides by them)
    float c = 0.f;
    for (int t = Br.n * Br.s; t < P.L; ++t) c += mk ? (mk[t] ? 1.f : 0.f) : 1.f;
    Br.tok[b] = c;
  }
  if (col < P.d) {
    // sum of the tokens of the incomplete block
    const T* x = reinterpret_cast<const T*>(P.x);
    float s = 0.f;
    for (int t = Br.n * Br.s; t < P.L; ++t)
      if (!mk || mk[t]) s += to_f32(x[((size_t)b * P.L + t) * P.d + col]);
    Br.psum[(size_t)b * P.d + col] = s;
    // held output of the last complete block (or, without one, the output
    // held on entry)
    float acc = Br.held_in && state_in_ok(P.chk) ? Br.held_in[(size_t)b * P.d + col] : 0.f;
    if (Br.n > 0) {
      acc = 0.f;
      const T* y = reinterpret_cast<const T*>(Br.y);
      const T* wo = reinterpret_cast<const T*>(P.WoT) + (size_t)col * P.Ktot + Br.ko;
      for (int hh = 0; hh < Br.h; ++hh) {
        const T* yr = y + (((size_t)b * Br.h + hh) * Br.np + (Br.n - 1)) * P.dv;
        for (int v = 0; v < P.dv; ++v) acc = fmaf(to_f32(yr[v]), to_f32(wo[hh * P.dv + v]), acc);
      }
    }
    Br.held[(size_t)b * P.d + col] = acc;
  }
  // a branch that saw no complete block keeps its GLA state: zero, or the
  // entry state, which the state kernel has already copied to the output
  if (Br.n == 0 && !(Br.S_in && state_in_ok(P.chk))) {
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
