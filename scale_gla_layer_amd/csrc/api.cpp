// Host side of the C ABI declared in include/msgla.h: validation, the packed /
// workspace / state layouts, and the launch sequence of the forward and the
// decode step.  No allocation, no global state, and no synchronisation except
// in msgla_state_query, which exists to read a state's header on the host.
#include "api_internal.hpp"

using namespace msgla;
using namespace msgla::host;

static_assert(sizeof(msgla_status) == sizeof(int32_t), "status codes travel as 32-bit ints");


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

}  // extern "C"

msgla_status msgla::host::forward_impl(const msgla_config* cfg, const void* packed, const void* x,
                                       const uint8_t* mask, int64_t B, int64_t L, void* out,
                                       const void* state_in, void* state_out, void* workspace,
                                       size_t workspace_bytes, void* stream,
                                       const msgla_stage_events* events, const FwdHooks* hooks) {
  if (msgla_status st = check_config(cfg); st != MSGLA_OK) return st;
  if (!batch_ok(B, L)) return MSGLA_ERR_INVALID_ARG;
  if (!packed || !x || (!out && !hooks) || !workspace) return MSGLA_ERR_INVALID_ARG;
  if (!aligned16(packed) || !aligned16(x) || (out && !aligned16(out)) || !aligned16(workspace) ||
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
    k.y = (hooks && hooks->yn[i]) ? static_cast<const void*>(hooks->yn[i]) : at<char>(workspace, W.br[i].y);
    k.s = g.br[i].s;
    k.h = g.br[i].h;
    k.np = W.br[i].np;
    k.n = W.br[i].n;
    k.ko = g.br[i].ko;
    k.held_in = state_in ? at<float>(state_in, S.held[i]) : nullptr;
    if (k.s == 1) {
      p3.fine = i;
    } else if (k.n > 0) {
      k.yc = hooks ? hooks->yc[i] : at<char>(workspace, W.br[i].xp);
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
      nb.yo = hooks ? hooks->yn[i] : nullptr;
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
  if (!hooks || out) HIP_TRY(launch_k3f(p3, g.bf16, st));
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

extern "C" {

msgla_status msgla_forward_timed(const msgla_config* cfg, const void* packed, const void* x,
                                 const uint8_t* mask, int64_t B, int64_t L, void* out,
                                 const void* state_in, void* state_out, void* workspace,
                                 size_t workspace_bytes, void* stream,
                                 const msgla_stage_events* events) {
  return forward_impl(cfg, packed, x, mask, B, L, out, state_in, state_out, workspace,
                      workspace_bytes, stream, events, nullptr);
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
