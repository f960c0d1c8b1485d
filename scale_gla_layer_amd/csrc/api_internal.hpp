// Host-side geometry shared by the forward, decode and backward entry points:
// validation, the packed-weight / workspace / state layouts, the K1 tile
// schedule and the kernel launchers.  Internal to the library.
#pragma once
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>

#include "../../include/msgla.h"
#include "layout.hpp"

namespace msgla {
// launchers (one per kernel file)
hipError_t launch_pool(const PoolParams& P, bool bf16_path, hipStream_t st);
hipError_t launch_k1(const K1Params& P, bool bf16_path, hipStream_t stream);
hipError_t launch_k2a(const K2Params& P, bool bf16_path, hipStream_t stream);
hipError_t launch_k2b(const K2Params& P, bool bf16_path, hipStream_t stream);
hipError_t launch_k3c(const K3Params& P, bool bf16_path, hipStream_t stream);
hipError_t launch_k3f(const K3Params& P, bool bf16_path, hipStream_t stream);
hipError_t launch_state_export(const StateParams& P, bool bf16_path, hipStream_t st);
hipError_t launch_state_header(void* state, int B, int m, int64_t pos, const StateCheck* chk,
                               hipStream_t st);
hipError_t launch_state_check(const StateCheckParams& P, hipStream_t st);
hipError_t launch_pending_gate(const PendingGateParams& P, bool bf16_path, hipStream_t st);
hipError_t launch_decode(const DecParams& P, int Nmax, int hmax, bool bf16_path, hipStream_t st);
hipError_t launch_norm(const NormParams& P, bool bf16_path, hipStream_t st);
hipError_t pack_transpose(bool bf16_path, const void* src, int R, int Cn, void* dst,
                          size_t dst_ld, hipStream_t st);
hipError_t pack_to_f32(bool src_bf16, const void* src, size_t n, float* dst, hipStream_t st);
hipError_t fill_zero(void* p, size_t bytes, hipStream_t st);
int k2b_dvt();
int k2b_lds_bytes(bool bf16_path, int C, int dk);
}  // namespace msgla


namespace msgla {
namespace host {


constexpr int GEMM_TILE = 128;

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline int cdiv(int a, int b) { return (a + b - 1) / b; }

// K1's tile schedule: every group's row tiles are split evenly over the eight
// XCDs (each keeps the column tiles of its row tiles together, which share the
// A rows in its L2), so each XCD gets the same mix of work.  Groups whose tiles
// run K twice (the q / k tiles of pooled groups in a masked bf16 call) are
// walked first, so the longest tiles start first on every XCD.
inline void k1_schedule(K1Params& p) {
  int n = 0;
  for (int pass = 0; pass < 2; ++pass)
    for (int g = 0; g < p.ngroups; ++g) {
      const bool heavy = p.g[g].A_lo != nullptr;
      if (heavy == (pass == 0)) p.order[n++] = g;
    }
  int longest = 0;
  for (int x = 0; x < N_XCD; ++x) {
    int cnt = 0;
    for (int g = 0; g < p.ngroups; ++g) {
      const int mt = cdiv(p.g[g].M, GEMM_TILE);
      p.mt_begin[g][x] = (int)((int64_t)mt * x / N_XCD);
      p.mt_begin[g][x + 1] = (int)((int64_t)mt * (x + 1) / N_XCD);
      cnt += (p.mt_begin[g][x + 1] - p.mt_begin[g][x]) * p.g[g].tiles_n;
    }
    longest = std::max(longest, cnt);
  }
  p.per_xcd = longest;
}

struct BranchGeom {
  int s, h;
  int col_k, col_v, col_g, col_z, N;  // projection columns
  int ko, kp;                         // stacked W_o^T K range
  size_t off_Wp, off_W2, off_bg;      // packed offsets
  size_t off_gn;                      // normalisation gains [h dv] fp32 (config norm)
};

struct PackGeom {
  bool bf16, norm;
  int es, m, d, dk, dv, r, rp, C, Ktot, carrier;
  size_t off_Wz;  // 0 if none (fusion carried by a branch or m == 1)
  bool has_Wz;
  size_t off_bf, off_zero, off_WoT, total;
  BranchGeom br[MSGLA_MAX_BRANCHES];
};

inline msgla_status check_config(const msgla_config* c) {
  if (!c) return MSGLA_ERR_INVALID_ARG;
  if (c->n_branches < 1 || c->n_branches > MSGLA_MAX_BRANCHES) return MSGLA_ERR_INVALID_ARG;
  if (c->dtype != MSGLA_F32 && c->dtype != MSGLA_BF16) return MSGLA_ERR_INVALID_ARG;
  const bool bf = c->dtype == MSGLA_BF16;
  for (int i = 0; i < c->n_branches; ++i) {
    if (c->scale[i] < 1 || c->heads[i] < 1 || c->heads[i] > 64) return MSGLA_ERR_INVALID_ARG;
    for (int j = 0; j < i; ++j)
      if (c->scale[j] == c->scale[i]) return MSGLA_ERR_INVALID_ARG;
  }
  if (c->d_model < 64 || c->d_model % 64 != 0 || c->d_model > 65536) return MSGLA_ERR_INVALID_ARG;
  // d_k: a power of two, 32 .. 256 (bf16) or 16 .. 256 (fp32)
  if (c->d_k < (bf ? 32 : 16) || c->d_k > 256 || (c->d_k & (c->d_k - 1)) != 0) return MSGLA_ERR_INVALID_ARG;
  // a 128-byte K segment of the output projection must lie inside one head
  if (c->d_v < 32 || c->d_v > 512 || c->d_v % (bf ? 64 : 32) != 0) return MSGLA_ERR_INVALID_ARG;
  if (c->gate_rank < 1 || c->gate_rank > 64) return MSGLA_ERR_INVALID_ARG;
  if (bf ? (c->chunk != 32 && c->chunk != 64)
         : (c->chunk != 16 && c->chunk != 32 && c->chunk != 64))
    return MSGLA_ERR_INVALID_ARG;
  if (!(c->gate_normalizer > 0.f) || !(c->q_scale == c->q_scale)) return MSGLA_ERR_INVALID_ARG;
  if (c->norm != 0 && c->norm != 1) return MSGLA_ERR_INVALID_ARG;
  // the state kernel keeps three (or two) chunks of A, qt, kT and V in LDS:
  // shapes whose stages do not fit the CU's 160 KB are not implemented
  const int lds = k2b_lds_bytes(bf, c->chunk, c->d_k);
  if (lds <= 0 || lds > 160 * 1024) return MSGLA_ERR_UNSUPPORTED;
  return MSGLA_OK;
}

inline PackGeom pack_geom(const msgla_config* c) {
  PackGeom g{};
  g.bf16 = c->dtype == MSGLA_BF16;
  g.norm = c->norm == 1;
  g.es = g.bf16 ? 2 : 4;
  g.m = c->n_branches;
  g.d = c->d_model;
  g.dk = c->d_k;
  g.dv = c->d_v;
  g.r = c->gate_rank;
  g.rp = c->gate_rank <= 16 ? 16 : 64;
  g.C = c->chunk;
  g.carrier = -1;
  if (g.m > 1)
    for (int i = 0; i < g.m; ++i)
      if (c->scale[i] == 1) {
        g.carrier = i;
        break;
      }
  const int e128 = 128 / g.es;
  size_t cur = 0;
  int ko = 0;
  for (int i = 0; i < g.m; ++i) {
    BranchGeom& b = g.br[i];
    b.s = c->scale[i];
    b.h = c->heads[i];
    b.col_k = b.h * g.dk;
    b.col_v = 2 * b.h * g.dk;
    b.col_g = b.col_v + b.h * g.dv;
    b.col_z = (i == g.carrier) ? b.col_g + g.rp : -1;
    b.N = b.col_g + g.rp + ((i == g.carrier) ? 16 : 0);
    b.off_Wp = cur;
    cur += align256((size_t)b.N * g.d * g.es);
    b.off_W2 = cur;
    cur += align256((size_t)g.rp * b.h * g.dk * 4);
    b.off_bg = cur;
    cur += align256((size_t)b.h * g.dk * 4);
    b.off_gn = cur;
    if (g.norm) cur += align256((size_t)b.h * g.dv * 4);
    b.ko = ko;
    b.kp = cdiv(b.h * g.dv, e128) * e128;
    ko += b.kp;
  }
  g.Ktot = ko;
  g.has_Wz = g.m > 1 && g.carrier < 0;
  g.off_Wz = cur;
  if (g.has_Wz) cur += align256((size_t)16 * g.d * g.es);
  g.off_bf = cur;
  cur += 256;
  g.off_zero = cur;  // 256 zero bytes (the whole blob is zero-filled before packing)
  cur += 256;
  g.off_WoT = cur;
  cur += align256((size_t)g.d * g.Ktot * g.es);
  g.total = cur;
  return g;
}

// forward workspace
struct WsBranch {
  int n, nch, np;
  size_t xp, xp_lo, q, k, qt, kT, vT, g, A, lam, y;
};
struct WsGeom {
  WsBranch br[MSGLA_MAX_BRANCHES];
  size_t w, chk, psumg, total;
  int nseg;        // segments of the chunk-state walk (1: one walk per sequence)
  int seg_base;    // workgroups of one segment
  size_t Sseg;     // segment states, when nseg > 1
};

// cont: the call continues from a state, whose blocks may start before the
// call, so a branch of scale s can complete ceil(L / s) blocks, not floor.
inline WsGeom ws_geom(const PackGeom& g, int64_t B, int64_t L, bool cont) {
  WsGeom w{};
  size_t cur = 0;
  auto take = [&](size_t bytes) {
    const size_t o = cur;
    cur += align256(bytes);
    return o;
  };
  for (int i = 0; i < g.m; ++i) {
    const BranchGeom& bg = g.br[i];
    WsBranch& b = w.br[i];
    b.n = (int)(cont ? (L + bg.s - 1) / bg.s : L / bg.s);
    b.nch = cdiv(b.n, g.C);
    b.np = b.nch * g.C;
    const size_t rows = (size_t)B * bg.h * b.np;
    b.xp = bg.s > 1 ? take((size_t)B * b.n * g.d * g.es) : 0;  // block means
    // their bf16 rounding residuals, which a masked call's projection adds back
    b.xp_lo = bg.s > 1 && g.bf16 ? take((size_t)B * b.n * g.d * g.es) : 0;
    b.q = take(rows * g.dk * 4);
    b.k = take(rows * g.dk * 4);
    b.qt = take(rows * g.dk * g.es);
    b.kT = take(rows * g.dk * g.es);
    b.vT = take(rows * g.dv * g.es);
    b.g = take((size_t)B * L * g.rp * 4);  // x W_g1 at every unpooled position
    b.A = take(rows * g.C * g.es);
    b.lam = take((size_t)B * bg.h * b.nch * g.dk * 4);
    b.y = take(rows * g.dv * g.es);
  }
  w.w = take((size_t)B * L * FUSION_STRIDE * 4);
  w.chk = take(sizeof(StateCheck));  // the device-side check of state_in
  w.psumg = take((size_t)g.m * B * g.rp * 4);  // pending gate sums of a continuing call
  // The chunk-state walk runs one workgroup per (sequence, 32-wide d_v slice).
  // With few of them (small batches of long sequences) the sequential walk over
  // the chunks leaves most CUs idle, so each walk is cut into segments (at least
  // 8 chunks each) walked in parallel in two passes around a scan over segments.
  {
    int seqs = 0, nch_max = 0;
    for (int i = 0; i < g.m; ++i) {
      seqs += (int)B * g.br[i].h;
      nch_max = std::max(nch_max, w.br[i].nch);
    }
    w.seg_base = cdiv(seqs, N_XCD) * N_XCD * (g.dv / k2b_dvt());
    w.nseg = 1;
    if (w.seg_base < 128) w.nseg = std::max(1, std::min({256 / std::max(w.seg_base, 1), nch_max / 8, 64}));
    w.Sseg = w.nseg > 1 ? take((size_t)seqs * w.nseg * g.dk * g.dv * 4) : 0;
  }
  w.total = cur;
  return w;
}

struct StGeom {
  size_t S[MSGLA_MAX_BRANCHES], psum[MSGLA_MAX_BRANCHES], held[MSGLA_MAX_BRANCHES],
      tok[MSGLA_MAX_BRANCHES];
  size_t total;
};

inline StGeom st_geom(const PackGeom& g, int64_t B) {
  StGeom s{};
  size_t cur = STATE_HEADER;
  for (int i = 0; i < g.m; ++i) {
    s.S[i] = cur;
    cur += align256((size_t)B * g.br[i].h * g.dk * g.dv * 4);
    s.psum[i] = cur;
    cur += align256((size_t)B * g.d * 4);
    s.held[i] = cur;
    cur += align256((size_t)B * g.d * 4);
    s.tok[i] = cur;
    cur += align256((size_t)B * 4);
  }
  s.total = cur;
  return s;
}

struct DecGeom {
  size_t proj[MSGLA_MAX_BRANCHES], y[MSGLA_MAX_BRANCHES];
  size_t w, pos, total;
};

inline DecGeom dec_geom(const PackGeom& g, int64_t B) {
  DecGeom d{};
  size_t cur = 0;
  for (int i = 0; i < g.m; ++i) {
    d.proj[i] = cur;
    cur += align256((size_t)B * g.br[i].N * 4);
    d.y[i] = cur;
    cur += align256((size_t)B * g.br[i].h * g.dv * 4);
  }
  d.w = cur;
  cur += align256((size_t)B * FUSION_STRIDE * 4);
  d.pos = cur;
  cur += 256;
  d.total = cur;
  return d;
}

template <typename P> P* at(void* base, size_t off) {
  return reinterpret_cast<P*>(static_cast<char*>(base) + off);
}
template <typename P> const P* at(const void* base, size_t off) {
  return reinterpret_cast<const P*>(static_cast<const char*>(base) + off);
}

#define HIP_TRY(expr)                               \
  do {                                              \
    if ((expr) != hipSuccess) return MSGLA_ERR_HIP; \
  } while (0)

inline bool batch_ok(int64_t B, int64_t L) {
  return B >= 1 && L >= 1 && B <= (1 << 20) && L <= (1 << 24) && B * L <= ((int64_t)1 << 31) / 8;
}


// Internal hooks of the forward launch sequence for the backward (its recompute,
// and the training forward): coarse outputs Y = y W_o go to yc[i] (instead of
// the dead block-mean buffer, which the backward still needs), normalised rows
// to yn[i] (keeping the GLA outputs); the fused output launch runs only when
// an output is given.
struct FwdHooks {
  void* yc[MSGLA_MAX_BRANCHES];
  void* yn[MSGLA_MAX_BRANCHES];  // configs with the normalisation: normalised rows go here
};

msgla_status forward_impl(const msgla_config* cfg, const void* packed, const void* x,
                          const uint8_t* mask, int64_t B, int64_t L, void* out,
                          const void* state_in, void* state_out, void* workspace,
                          size_t workspace_bytes, void* stream,
                          const msgla_stage_events* events, const FwdHooks* hooks);

}  // namespace host
}  // namespace msgla
