// Host side of the C ABI declared in include/msgla.h: validation, the packed /
// workspace / state layouts, and the launch sequence of the forward and the
// decode step.  No allocation, no global state, and no synchronisation except
// in msgla_state_query, which exists to read a state's header on the host.
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

using namespace msgla;

static_assert(sizeof(msgla_status) == sizeof(int32_t), "status codes travel as 32-bit ints");

namespace {

constexpr int GEMM_TILE = 128;

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
int cdiv(int a, int b) { return (a + b - 1) / b; }

// K1's tile schedule: every group's row tiles are split evenly over the eight
// XCDs (each keeps the column tiles of its row tiles together, which share the
// A rows in its L2), so each XCD gets the same mix of work.  Groups whose tiles
// run K twice (the q / k tiles of pooled groups in a masked bf16 call) are
// walked first, so the longest tiles start first on every XCD.
void k1_schedule(K1Params& p) {
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

msgla_status check_config(const msgla_config* c) {
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

PackGeom pack_geom(const msgla_config* c) {
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
WsGeom ws_geom(const PackGeom& g, int64_t B, int64_t L, bool cont) {
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

StGeom st_geom(const PackGeom& g, int64_t B) {
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

DecGeom dec_geom(const PackGeom& g, int64_t B) {
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

bool batch_ok(int64_t B, int64_t L) {
  return B >= 1 && L >= 1 && B <= (1 << 20) && L <= (1 << 24) && B * L <= ((int64_t)1 << 31) / 8;
}

}  // namespace

extern "C" {

const char* msgla_status_str(msgla_status s) {
  // a C caller may pass any int: read the bits, not the enum value
  int32_t v;
  std::memcpy(&v, &s, sizeof(v));
  switch (v) {
    case MSGLA_OK: return "ok";
    case MSGLA_ERR_INVALID_ARG: return "invalid argument";
    case MSGLA_ERR_UNSUPPORTED: return "unsupported";
    case MSGLA_ERR_WORKSPACE: return "workspace or buffer too small";
    case MSGLA_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

msgla_status msgla_validate_config(const msgla_config* cfg) { return check_config(cfg); }

size_t msgla_packed_weights_bytes(const msgla_config* cfg) {
  if (check_config(cfg) != MSGLA_OK) return 0;
  return pack_geom(cfg).total;
}

size_t msgla_workspace_bytes(const msgla_config* cfg, int64_t B, int64_t L) {
  if (check_config(cfg) != MSGLA_OK || !batch_ok(B, L)) return 0;
  // the larger of the two layouts (a continuing call may pool one more block)
  return ws_geom(pack_geom(cfg), B, L, true).total;
}

size_t msgla_state_bytes(const msgla_config* cfg, int64_t B) {
  if (check_config(cfg) != MSGLA_OK || !batch_ok(B, 1)) return 0;
  return st_geom(pack_geom(cfg), B).total;
}

size_t msgla_decode_workspace_bytes(const msgla_config* cfg, int64_t B) {
  if (check_config(cfg) != MSGLA_OK || !batch_ok(B, 1)) return 0;
  return dec_geom(pack_geom(cfg), B).total;
}

msgla_status msgla_pack_weights(const msgla_config* cfg, const msgla_weights* w, void* packed,
                                size_t packed_bytes, void* stream) {
  if (msgla_status st = check_config(cfg); st != MSGLA_OK) return st;
  if (!w || !packed || !aligned16(packed)) return MSGLA_ERR_INVALID_ARG;
  const PackGeom g = pack_geom(cfg);
  if (packed_bytes < g.total) return MSGLA_ERR_WORKSPACE;
  for (int i = 0; i < g.m; ++i) {
    const msgla_branch_weights& b = w->br[i];
    if (!b.W_q || !b.W_k || !b.W_v || !b.W_g1 || !b.W_g2 || !b.b_g || !b.W_o)
      return MSGLA_ERR_INVALID_ARG;
    if (g.norm && !b.norm_g) return MSGLA_ERR_INVALID_ARG;
  }
  if (g.m > 1 && (!w->W_f || !w->b_f)) return MSGLA_ERR_INVALID_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  HIP_TRY(fill_zero(packed, g.total, st));
  for (int i = 0; i < g.m; ++i) {
    const BranchGeom& b = g.br[i];
    const msgla_branch_weights& s = w->br[i];
    void* Wp = at<char>(packed, b.off_Wp);
    const size_t rowb = (size_t)g.d * g.es;
    HIP_TRY(pack_transpose(g.bf16, s.W_q, g.d, b.h * g.dk, Wp, g.d, st));
    HIP_TRY(pack_transpose(g.bf16, s.W_k, g.d, b.h * g.dk, at<char>(Wp, b.col_k * rowb), g.d, st));
    HIP_TRY(pack_transpose(g.bf16, s.W_v, g.d, b.h * g.dv, at<char>(Wp, b.col_v * rowb), g.d, st));
    HIP_TRY(pack_transpose(g.bf16, s.W_g1, g.d, g.r, at<char>(Wp, b.col_g * rowb), g.d, st));
    if (b.col_z >= 0)
      HIP_TRY(pack_transpose(g.bf16, w->W_f, g.d, g.m, at<char>(Wp, b.col_z * rowb), g.d, st));
    HIP_TRY(pack_to_f32(g.bf16, s.W_g2, (size_t)g.r * b.h * g.dk, at<float>(packed, b.off_W2), st));
    HIP_TRY(hipMemcpyAsync(at<char>(packed, b.off_bg), s.b_g, (size_t)b.h * g.dk * 4,
                           hipMemcpyDeviceToDevice, st));
    if (g.norm)
      HIP_TRY(hipMemcpyAsync(at<char>(packed, b.off_gn), s.norm_g, (size_t)b.h * g.dv * 4,
                             hipMemcpyDeviceToDevice, st));
    // W_o [h dv][d] -> WoT[n][ko + k]
    HIP_TRY(pack_transpose(g.bf16, s.W_o, b.h * g.dv, g.d, at<char>(packed, g.off_WoT + (size_t)b.ko * g.es),
                           g.Ktot, st));
  }
  if (g.has_Wz) HIP_TRY(pack_transpose(g.bf16, w->W_f, g.d, g.m, at<char>(packed, g.off_Wz), g.d, st));
  if (g.m > 1)
    HIP_TRY(hipMemcpyAsync(at<char>(packed, g.off_bf), w->b_f, (size_t)g.m * 4,
                           hipMemcpyDeviceToDevice, st));
  return MSGLA_OK;
}

msgla_status msgla_state_init(const msgla_config* cfg, int64_t B, void* state, size_t state_bytes,
                              void* stream) {
  if (msgla_status st = check_config(cfg); st != MSGLA_OK) return st;
  if (!batch_ok(B, 1) || !state || !aligned16(state)) return MSGLA_ERR_INVALID_ARG;
  const PackGeom g = pack_geom(cfg);
  const StGeom s = st_geom(g, B);
  if (state_bytes < s.total) return MSGLA_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  HIP_TRY(fill_zero(state, s.total, st));
  HIP_TRY(launch_state_header(state, (int)B, g.m, 0, nullptr, st));
  return MSGLA_OK;
}

msgla_status msgla_state_query(const void* state, msgla_state_info* info, void* stream) {
  if (!state || !info || !aligned16(state)) return MSGLA_ERR_INVALID_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  StateHeader h{};
  HIP_TRY(hipMemcpyAsync(&h, state, sizeof h, hipMemcpyDeviceToHost, st));
  HIP_TRY(hipStreamSynchronize(st));
  if (h.magic != STATE_MAGIC || h.version != STATE_VERSION) return MSGLA_ERR_INVALID_ARG;
  info->status = h.status;
  info->B = h.B;
  info->m = h.m;
  info->position = h.pos;
  return MSGLA_OK;
}

msgla_status msgla_forward_timed(const msgla_config* cfg, const void* packed, const void* x,
                                 const uint8_t* mask, int64_t B, int64_t L, void* out,
                                 const void* state_in, void* state_out, void* workspace,
                                 size_t workspace_bytes, void* stream,
                                 const msgla_stage_events* events) {
  if (msgla_status st = check_config(cfg); st != MSGLA_OK) return st;
  if (!batch_ok(B, L)) return MSGLA_ERR_INVALID_ARG;
  if (!packed || !x || !out || !workspace) return MSGLA_ERR_INVALID_ARG;
  if (!aligned16(packed) || !aligned16(x) || !aligned16(out) || !aligned16(workspace) ||
      (state_out && !aligned16(state_out)) || (state_in && !aligned16(state_in)))
    return MSGLA_ERR_INVALID_ARG;
  const PackGeom g = pack_geom(cfg);
  const WsGeom W = ws_geom(g, B, L, state_in != nullptr);
  if (workspace_bytes < W.total) return MSGLA_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const StGeom S = st_geom(g, B);
  // Continuing from a state: its header is checked on the device (this
  // configuration and batch, no recorded error); the check also gives every
  // branch's entry offset r = position mod s (block 0 of the call completes
  // the state's pending block) and the number of blocks the call completes.
  // Every kernel that reads the state, or depends on the offsets, reads the
  // check's result; the state itself only if the check passed.  The pending
  // block's gate first factors are summed here, as psum W_g1.
  const StateCheck* chk = nullptr;
  if (state_in) {
    StateCheckParams pc{};
    pc.state_in = state_in;
    pc.out = at<StateCheck>(workspace, W.chk);
    pc.B = (int)B;
    pc.m = g.m;
    pc.L = (int)L;
    for (int i = 0; i < g.m; ++i) pc.scale[i] = g.br[i].s;
    HIP_TRY(launch_state_check(pc, st));
    chk = pc.out;
    PendingGateParams pg{};
    pg.B = (int)B;
    pg.d = g.d;
    pg.rp = g.rp;
    pg.m = g.m;
    pg.chk = chk;
    for (int i = 0; i < g.m; ++i) {
      pg.br[i].Wg1 = at<char>(packed, g.br[i].off_Wp + (size_t)g.br[i].col_g * g.d * g.es);
      pg.br[i].psum = at<float>(state_in, S.psum[i]);
      pg.br[i].out = at<float>(workspace, W.psumg) + (size_t)i * B * g.rp;
    }
    HIP_TRY(launch_pending_gate(pg, g.bf16, st));
  }

  auto ev = [&](int stage, bool start) -> hipError_t {
    if (!events) return hipSuccess;
    void* e = start ? events->start[stage] : events->stop[stage];
    return e ? hipEventRecord(static_cast<hipEvent_t>(e), st) : hipSuccess;
  };

  // ---------------- K1 ----------------
  K1Params p1{};
  p1.B = (int)B;
  p1.mask = mask;
  p1.d = g.d;
  p1.dk = g.dk;
  p1.dv = g.dv;
  p1.C = g.C;
  int tiles = 0, ng = 0;
  for (int i = 0; i < g.m; ++i) {
    const BranchGeom& b = g.br[i];
    const WsBranch& wb = W.br[i];
    if (wb.n == 0) continue;
    K1Group& G = p1.g[ng++];
    G.Wp = at<char>(packed, b.off_Wp);
    G.A = b.s == 1 ? x : static_cast<const void*>(at<char>(workspace, wb.xp));
    G.A_lo = (mask && b.s > 1 && g.bf16) ? static_cast<const void*>(at<char>(workspace, wb.xp_lo)) : nullptr;
    G.s = b.s;
    G.n = wb.n;
    G.M = (int)B * wb.n;
    G.N = b.col_g;  // q, k and v columns
    G.tiles_n = cdiv(G.N, GEMM_TILE);
    tiles += cdiv(G.M, GEMM_TILE) * G.tiles_n;
    G.h = b.h;
    G.col_k = b.col_k;
    G.col_v = b.col_v;
    G.np = wb.np;
    G.nch = wb.nch;
    G.q = at<float>(workspace, wb.q);
    G.k = at<float>(workspace, wb.k);
    G.vT = at<char>(workspace, wb.vT);
  }
  {
    // the small projection over the unpooled rows: gate first factors, fusion logits
    K1Small& S = p1.sm;
    S.m = g.m;
    S.rp = g.rp;
    S.gm = g.m;
    int Ns = 0;
    for (int i = 0; i < g.m; ++i) {
      const BranchGeom& b = g.br[i];
      S.seg[S.nseg++] = XSeg{at<char>(packed, b.off_Wp + (size_t)b.col_g * g.d * g.es), Ns, g.rp};
      S.g[i] = at<float>(workspace, W.br[i].g);
      Ns += g.rp;
    }
    S.zcol = -1;
    if (g.m > 1) {
      const size_t zoff = g.carrier >= 0
                              ? g.br[g.carrier].off_Wp + (size_t)g.br[g.carrier].col_z * g.d * g.es
                              : g.off_Wz;
      S.seg[S.nseg++] = XSeg{at<char>(packed, zoff), Ns, 16};
      S.zcol = Ns;
      Ns += 16;
    }
    S.bf = at<float>(packed, g.off_bf);
    S.w = at<float>(workspace, W.w);
    S.group = ng;
    K1Group& G = p1.g[ng++];
    G.A = x;
    G.s = 1;
    G.n = (int)L;
    G.M = (int)(B * L);
    G.N = Ns;
    G.tiles_n = cdiv(Ns, GEMM_TILE);
    tiles += cdiv(G.M, GEMM_TILE) * G.tiles_n;
  }
  p1.ngroups = ng;
  p1.total_tiles = tiles;
  k1_schedule(p1);

  // ---------------- K2 ----------------
  K2Params p2{};
  p2.B = (int)B;
  p2.L = (int)L;
  p2.dk = g.dk;
  p2.dv = g.dv;
  p2.r = g.r;
  p2.rp = g.rp;
  p2.C = g.C;
  p2.inv_gamma = 1.0f / cfg->gate_normalizer;
  p2.q_scale = cfg->q_scale;
  p2.mask = mask;
  p2.nbranch = g.m;
  int units = 0;
  for (int i = 0; i < g.m; ++i) {
    const BranchGeom& b = g.br[i];
    const WsBranch& wb = W.br[i];
    K2Branch& k = p2.br[i];
    k.h = b.h;
    k.s = b.s;
    k.n = wb.n;
    k.nch = wb.nch;
    k.np = wb.np;
    k.unit_begin = units;
    units += (int)B * b.h * wb.nch;
    k.q = at<float>(workspace, wb.q);
    k.k = at<float>(workspace, wb.k);
    k.g = at<float>(workspace, wb.g);
    k.W2 = at<float>(packed, b.off_W2);
    k.bg = at<float>(packed, b.off_bg);
    k.qt = at<char>(workspace, wb.qt);
    k.kT = at<char>(workspace, wb.kT);
    k.vT = at<char>(workspace, wb.vT);
    k.A = at<char>(workspace, wb.A);
    k.lam = at<float>(workspace, wb.lam);
    k.y = at<char>(workspace, wb.y);
    k.S_out = state_out ? at<float>(state_out, S.S[i]) : nullptr;
    k.S_in = state_in ? at<float>(state_in, S.S[i]) : nullptr;
    k.psumg = state_in ? at<float>(workspace, W.psumg) + (size_t)i * B * g.rp : nullptr;
    k.tok_in = state_in ? at<float>(state_in, S.tok[i]) : nullptr;
  }
  p2.total_units = units;
  // K2b: sequences ordered by decreasing chunk count (longest walks start first)
  int order[MSGLA_MAX_BRANCHES];
  for (int i = 0; i < g.m; ++i) order[i] = i;
  std::stable_sort(order, order + g.m, [&](int a, int b) { return W.br[a].nch > W.br[b].nch; });
  int seqs = 0;
  for (int o = 0; o < g.m; ++o) {
    p2.order[o] = order[o];
    p2.br[order[o]].seq_begin = seqs;
    seqs += (int)B * g.br[order[o]].h;
  }
  p2.total_seqs = seqs;
  p2.n_dvt = g.dv / k2b_dvt();
  p2.nseg = W.nseg;
  p2.seg_base = W.seg_base;
  p2.Sseg = W.nseg > 1 ? at<float>(workspace, W.Sseg) : nullptr;
  p2.chk = chk;

  // ---------------- K3 ----------------
  // coarse outputs Y = y W_o reuse the block-mean buffers of their branch
  // (same [B][n][d] shape, dead once the projection GEMM has run)
  K3Params p3{};
  p3.B = (int)B;
  p3.L = (int)L;
  p3.d = g.d;
  p3.dv = g.dv;
  p3.m = g.m;
  p3.Ktot = g.Ktot;
  p3.fine = -1;
  p3.tiles_n = cdiv(g.d, GEMM_TILE);
  p3.WoT = at<char>(packed, g.off_WoT);
  p3.zero = at<char>(packed, g.off_zero);
  p3.w = at<float>(workspace, W.w);
  p3.out = out;
  int ctiles = 0;
  for (int i = 0; i < g.m; ++i) {
    K3Branch& k = p3.br[i];
    k.y = at<char>(workspace, W.br[i].y);
    k.s = g.br[i].s;
    k.h = g.br[i].h;
    k.np = W.br[i].np;
    k.n = W.br[i].n;
    k.ko = g.br[i].ko;
    k.held_in = state_in ? at<float>(state_in, S.held[i]) : nullptr;
    if (k.s == 1) {
      p3.fine = i;
    } else if (k.n > 0) {
      k.yc = at<char>(workspace, W.br[i].xp);
      k.tile_begin = ctiles;
      ctiles += cdiv((int)B * k.n, GEMM_TILE) * p3.tiles_n;
      p3.coarse[p3.ncoarse++] = i;
    }
  }
  // a coarse branch with no complete block in this call still contributes the
  // output it held on entry: fused only (no K3c tiles), after the others
  for (int i = 0; i < g.m; ++i) {
    K3Branch& k = p3.br[i];
    if (k.s > 1 && k.n == 0 && k.held_in) {
      k.tile_begin = ctiles;
      p3.coarse[p3.ncoarse++] = i;
    }
  }
  p3.held_in = state_in != nullptr;
  p3.chk = chk;
  p3.c_total = ctiles;
  p3.c_per_xcd = cdiv(ctiles, N_XCD);
  p3.f_total = cdiv((int)(B * L), GEMM_TILE) * p3.tiles_n;
  p3.f_per_xcd = cdiv(p3.f_total, N_XCD);

  // pooling prepass: one pass for the scales dividing the largest coarse scale,
  // one more per remaining coarse scale
  PoolParams pp[MSGLA_MAX_BRANCHES];
  int npass = 0;
  {
    bool done[MSGLA_MAX_BRANCHES] = {};
    for (;;) {
      int smax = 0;
      for (int i = 0; i < g.m; ++i)
        if (!done[i] && g.br[i].s > 1 && W.br[i].n > 0) smax = std::max(smax, g.br[i].s);
      if (smax == 0) break;
      PoolParams& q = pp[npass++];
      q = PoolParams{};
      q.x = x;
      q.mask = mask;
      q.chk = chk;
      q.B = (int)B;
      q.L = (int)L;
      q.d = g.d;
      q.smax = smax;
      for (int i = 0; i < g.m; ++i) {
        const int s = g.br[i].s;
        if (done[i] || s <= 1 || W.br[i].n == 0 || smax % s != 0) continue;
        PoolOut& o = q.out[q.nout++];
        o.xp = at<char>(workspace, W.br[i].xp);
        o.xp_lo = (mask && g.bf16) ? at<char>(workspace, W.br[i].xp_lo) : nullptr;
        o.s = s;
        o.n = W.br[i].n;
        o.inv_s = 1.0f / (float)s;
        o.branch = i;
        o.psum_in = state_in ? at<float>(state_in, S.psum[i]) : nullptr;
        o.tok_in = state_in ? at<float>(state_in, S.tok[i]) : nullptr;
        done[i] = true;
      }
    }
  }

  HIP_TRY(ev(0, true));
  for (int i = 0; i < npass; ++i) HIP_TRY(launch_pool(pp[i], g.bf16, st));
  HIP_TRY(ev(0, false));
  HIP_TRY(ev(1, true));
  if (p1.total_tiles > 0) HIP_TRY(launch_k1(p1, g.bf16, st));
  HIP_TRY(ev(1, false));
  HIP_TRY(ev(2, true));
  if (p2.total_units > 0) HIP_TRY(launch_k2a(p2, g.bf16, st));
  HIP_TRY(ev(2, false));
  HIP_TRY(ev(3, true));
  if (p2.total_seqs > 0) HIP_TRY(launch_k2b(p2, g.bf16, st));
  if (g.norm) {
    // the branches' y rows, normalised in place before the output projections
    NormParams pn{};
    pn.dv = g.dv;
    int rows = 0;
    for (int i = 0; i < g.m; ++i) {
      if (W.br[i].n == 0) continue;
      NormBranch& nb = pn.br[pn.nbranch++];
      nb.y = at<char>(workspace, W.br[i].y);
      nb.g = at<float>(packed, g.br[i].off_gn);
      nb.h = g.br[i].h;
      nb.n = W.br[i].n;
      nb.np = W.br[i].np;
      nb.row_begin = rows;
      rows += (int)B * nb.h * nb.n;
    }
    pn.total_rows = rows;
    HIP_TRY(launch_norm(pn, g.bf16, st));
  }
  HIP_TRY(ev(3, false));
  HIP_TRY(ev(4, true));
  HIP_TRY(launch_k3c(p3, g.bf16, st));
  HIP_TRY(ev(4, false));
  HIP_TRY(ev(5, true));
  HIP_TRY(launch_k3f(p3, g.bf16, st));
  HIP_TRY(ev(5, false));

  if (state_out) {
    StateParams ps{};
    ps.B = (int)B;
    ps.L = (int)L;
    ps.d = g.d;
    ps.dk = g.dk;
    ps.dv = g.dv;
    ps.m = g.m;
    ps.Ktot = g.Ktot;
    ps.pos = L;
    ps.chk = chk;
    ps.x = x;
    ps.mask = mask;
    ps.WoT = p3.WoT;
    ps.state = state_out;
    for (int i = 0; i < g.m; ++i) {
      StateBranch& b = ps.br[i];
      b.s = g.br[i].s;
      b.h = g.br[i].h;
      b.n = W.br[i].n;
      b.np = W.br[i].np;
      b.ko = g.br[i].ko;
      b.S = at<float>(state_out, S.S[i]);
      b.psum = at<float>(state_out, S.psum[i]);
      b.held = at<float>(state_out, S.held[i]);
      b.tok = at<float>(state_out, S.tok[i]);
      b.y = at<char>(workspace, W.br[i].y);
      b.S_in = state_in ? at<float>(state_in, S.S[i]) : nullptr;
      b.held_in = state_in ? at<float>(state_in, S.held[i]) : nullptr;
      b.psum_in = state_in ? at<float>(state_in, S.psum[i]) : nullptr;
      b.tok_in = state_in ? at<float>(state_in, S.tok[i]) : nullptr;
    }
    HIP_TRY(launch_state_export(ps, g.bf16, st));
  }
  return MSGLA_OK;
}

msgla_status msgla_forward(const msgla_config* cfg, const void* packed, const void* x,
                           const uint8_t* mask, int64_t B, int64_t L, void* out,
                           const void* state_in, void* state_out, void* workspace,
                           size_t workspace_bytes, void* stream) {
  return msgla_forward_timed(cfg, packed, x, mask, B, L, out, state_in, state_out, workspace,
                             workspace_bytes, stream, nullptr);
}

msgla_status msgla_fusion_weights(const msgla_config* cfg, const void* packed, const void* x,
                                  int64_t B, int64_t L, float* w_out, void* stream) {
  if (msgla_status st = check_config(cfg); st != MSGLA_OK) return st;
  if (!batch_ok(B, L)) return MSGLA_ERR_INVALID_ARG;
  if (!packed || !x || !w_out || !aligned16(packed) || !aligned16(x) || !aligned16(w_out))
    return MSGLA_ERR_INVALID_ARG;
  const PackGeom g = pack_geom(cfg);
  if (g.m < 2) return MSGLA_ERR_INVALID_ARG;  // one branch has no fusion weights
  // the projection kernel with its small group alone, holding only the fusion logits
  K1Params p1{};
  p1.B = (int)B;
  p1.d = g.d;
  p1.dk = g.dk;
  p1.dv = g.dv;
  p1.C = g.C;
  K1Small& S = p1.sm;
  S.m = g.m;
  S.rp = g.rp;
  S.gm = 0;
  const size_t zoff = g.carrier >= 0
                          ? g.br[g.carrier].off_Wp + (size_t)g.br[g.carrier].col_z * g.d * g.es
                          : g.off_Wz;
  S.seg[S.nseg++] = XSeg{at<char>(packed, zoff), 0, 16};
  S.zcol = 0;
  S.bf = at<float>(packed, g.off_bf);
  S.w = w_out;
  S.group = 0;
  K1Group& G = p1.g[0];
  G.A = x;
  G.s = 1;
  G.n = (int)L;
  G.M = (int)(B * L);
  G.N = 16;
  G.tiles_n = 1;
  p1.ngroups = 1;
  p1.total_tiles = cdiv(G.M, GEMM_TILE);
  k1_schedule(p1);
  HIP_TRY(launch_k1(p1, g.bf16, static_cast<hipStream_t>(stream)));
  return MSGLA_OK;
}

msgla_status msgla_decode_step(const msgla_config* cfg, const void* packed, const void* x_t,
                               int64_t B, void* state, void* out_t, void* workspace,
                               size_t workspace_bytes, void* stream) {
  if (msgla_status st = check_config(cfg); st != MSGLA_OK) return st;
  if (!batch_ok(B, 1) || !packed || !x_t || !state || !out_t || !workspace)
    return MSGLA_ERR_INVALID_ARG;
  if (!aligned16(packed) || !aligned16(x_t) || !aligned16(state) || !aligned16(out_t) ||
      !aligned16(workspace))
    return MSGLA_ERR_INVALID_ARG;
  const PackGeom g = pack_geom(cfg);
  const DecGeom D = dec_geom(g, B);
  if (workspace_bytes < D.total) return MSGLA_ERR_WORKSPACE;
  const StGeom S = st_geom(g, B);
  DecParams p{};
  p.B = (int)B;
  p.d = g.d;
  p.dk = g.dk;
  p.dv = g.dv;
  p.r = g.r;
  p.m = g.m;
  p.Ktot = g.Ktot;
  p.inv_gamma = 1.0f / cfg->gate_normalizer;
  p.q_scale = cfg->q_scale;
  p.x = x_t;
  p.out = out_t;
  p.state = state;
  p.pos_ws = at<int64_t>(workspace, D.pos);
  p.w = at<float>(workspace, D.w);
  p.bf = at<float>(packed, g.off_bf);
  p.WoT = at<char>(packed, g.off_WoT);
  if (g.has_Wz)
    p.Wz = at<char>(packed, g.off_Wz);
  else if (g.carrier >= 0)
    p.Wz = at<char>(packed, g.br[g.carrier].off_Wp + (size_t)g.br[g.carrier].col_z * g.d * g.es);
  else
    p.Wz = nullptr;
  p.nbranch = g.m;
  p.norm = g.norm ? 1 : 0;
  int Nmax = 0, hmax = 0;
  for (int i = 0; i < g.m; ++i) {
    const BranchGeom& b = g.br[i];
    DecBranch& k = p.br[i];
    k.s = b.s;
    k.h = b.h;
    k.N = b.N;
    k.col_k = b.col_k;
    k.col_v = b.col_v;
    k.col_g = b.col_g;
    k.col_z = b.col_z;
    k.ko = b.ko;
    k.Wp = at<char>(packed, b.off_Wp);
    k.W2 = at<float>(packed, b.off_W2);
    k.bg = at<float>(packed, b.off_bg);
    k.S = at<float>(state, S.S[i]);
    k.psum = at<float>(state, S.psum[i]);
    k.held = at<float>(state, S.held[i]);
    k.tok = at<float>(state, S.tok[i]);
    k.proj = at<float>(workspace, D.proj[i]);
    k.y = at<float>(workspace, D.y[i]);
    k.gn = g.norm ? at<float>(packed, b.off_gn) : nullptr;
    Nmax = std::max(Nmax, b.N);
    hmax = std::max(hmax, b.h);
  }
  HIP_TRY(launch_decode(p, Nmax, hmax, g.bf16, static_cast<hipStream_t>(stream)));
  return MSGLA_OK;
}

}  // extern "C"
