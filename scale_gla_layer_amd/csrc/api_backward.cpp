// Host side of msgla_backward: the layer's vector-Jacobian product (see
// k_backward.hip for the chain rule it follows).  The call recomputes the
// forward's intermediates with the forward's own kernels (keeping the coarse
// outputs Y beside the block means), then walks the layer in reverse: fusion
// and hold, the output projections, the chunkwise recurrence, the gate, the
// input projections and the pooling.  Every step runs in the library's
// kernels, the plain products too (grouped GEMMs for the activation gradients,
// the weight-gradient kernel); only the fp32 layer's weight gradients go to
// rocBLAS.
#include <rocblas/rocblas.h>

#include <mutex>

#include "api_internal.hpp"

namespace msgla {
hipError_t launch_bwd_gate(const BwdParams& P, hipStream_t st);
hipError_t launch_bwd_chunk(const BwdParams& P, int which, bool bf16_path, hipStream_t st);
hipError_t launch_bwd_scan(const BwdParams& P, bool rev, hipStream_t st);
hipError_t launch_bwd_walk(const BwdParams& P, bool rev, hipStream_t st);
hipError_t launch_bwd_gate_grads(const BwdParams& P, bool bf16_path, hipStream_t st);
hipError_t launch_bwd_out(const BwdParams& P, bool bf16_path, hipStream_t st);
hipError_t launch_bwd_hold(const BwdParams& P, int bi, bool bf16_path, hipStream_t st);
hipError_t launch_bwd_dx(const BwdParams& P, bool bf16_path, hipStream_t st);
hipError_t launch_bwd_mask_rows(const BwdParams& P, int bi, bool bf16_path, hipStream_t st);
hipError_t launch_bwd_norm(const BwdParams& P, int bi, bool bf16_path, hipStream_t st);
hipError_t launch_bwd_mcolsum(const ColsumJobs& J, float* part, hipStream_t st);
hipError_t launch_bwd_wf_partial(const BwdParams& P, float* partial, int nrb, bool bf16_path, hipStream_t st);
hipError_t launch_bwd_wf_finish(const float* partial, int nrb, int d, int m, float* out, hipStream_t st);
hipError_t launch_bwd_splitk_reduce(const SplitJobs& J, hipStream_t st);
hipError_t launch_bwd_gemm(const BwdGemm& P, bool bf16_path, bool out_storage, hipStream_t st);
hipError_t launch_bwd_transpose(const BwdTranspose& P, bool bf16_path, hipStream_t st);
hipError_t launch_bwd_wgrad(const Wgrad& P, hipStream_t st);
}  // namespace msgla

using namespace msgla;
using namespace msgla::host;

namespace {

constexpr int BWD_NRB_MAX = 64;   // row blocks of the deterministic column sums
constexpr int BWD_WF_NRB = 64;    // row blocks of x^T dz
constexpr int BWD_SPLIT_MAX = 16; // K slices of a weight-gradient product

// row blocks of a column sum over `rows` rows (at least 128 rows each)
int colsum_blocks(int rows) { return std::max(1, std::min(BWD_NRB_MAX, (rows + 127) / 128)); }

struct BwdBranchGeom {
  size_t lb, sg, g1c, Sst, dSt, AD, QKi, rsum, rtot, dob, gpart, dP, dY, Yc, ycat, dxp, yn, ngt, WpT;
  int NP;
};

struct BwdGeom {
  WsGeom W;
  BwdBranchGeom br[MSGLA_MAX_BRANCHES];
  size_t dz, partial, mcol, mcol_floats, splitk, splitk_floats, Wo, total;
};

bool bwd_supported(const msgla_config* cfg) { return cfg->d_v % 64 == 0; }

// K slices of a weight-gradient product C [M][N] over K positions (see gemm_wgrad).
// bf16 storage (the library's kernel): slices of about 4096 positions (whole
// 64-position multiples), which give the main workload's six products 680 work
// items, about three workgroups per CU in one round (measured against 2048,
// 3072 and 8192 positions: the kernel plus the reduction took 163, 154 and 254
// us against 151 us).  fp32 storage (rocBLAS): slices double while the batch
// stays within 192 output tiles of 128 x 128 (measured on the main workload's
// bf16 backward when rocBLAS ran it: caps 768 and 1536 cost 15 and 40 us more,
// 96 and below 60 us and more).
int wgrad_ks(int K) {
  const int S = std::max(1, std::min(BWD_SPLIT_MAX, K / 4096));
  return ((K + S - 1) / S + 63) & ~63;
}
int wgrad_slices(bool bf16, int M, int N, int K) {
  if (bf16) {
    const int Ks = wgrad_ks(K);
    return (K + Ks - 1) / Ks;
  }
  const int tiles = ((M + 127) / 128) * ((N + 127) / 128);
  int S = 1;
  while (S < BWD_SPLIT_MAX && tiles * S * 2 <= 192 && K % (2 * S) == 0 && K / (2 * S) >= 256) S *= 2;
  return S;
}

// fp32 partials a weight-gradient product leaves for the reduction (0: written directly)
size_t wgrad_part_floats(bool bf16, int M, int N, int K, bool one_full_dst) {
  const int S = wgrad_slices(bf16, M, N, K);
  return (S == 1 && one_full_dst) ? 0 : (size_t)S * M * N;
}

BwdGeom bwd_geom(const PackGeom& g, int64_t B, int64_t L) {
  BwdGeom G{};
  G.W = ws_geom(g, B, L, false);
  size_t cur = G.W.total;
  auto take = [&](size_t bytes) {
    const size_t o = cur;
    cur += align256(bytes);
    return o;
  };
  size_t gate_cols = 0, norm_cols = 0, part = 0;
  for (int i = 0; i < g.m; ++i) {
    const BranchGeom& bg = g.br[i];
    const WsBranch& w = G.W.br[i];
    BwdBranchGeom& o = G.br[i];
    const size_t rows = (size_t)B * bg.h * w.np;  // per-head positions, chunk padded
    const size_t prow = (size_t)B * w.n;          // pooled positions
    const size_t chunks = (size_t)B * bg.h * w.nch;
    o.lb = take(rows * g.dk * 4);
    o.sg = take(rows * g.dk * 4);
    o.g1c = take(prow * g.rp * 4);
    o.Sst = take(chunks * g.dk * g.dv * 4);
    o.dSt = take(chunks * g.dk * g.dv * 4);
    o.AD = take(chunks * 64 * 64 * 4);
    o.QKi = take(chunks * 2 * 64 * g.dk * 4);
    o.rsum = take(rows * g.dk * 4);
    o.rtot = take(chunks * g.dk * 4);
    o.dob = take(prow * bg.h * g.dv * 4);
    o.gpart = take((size_t)B * w.nch * 2 * (g.r + 1) * bg.h * g.dk * 4);
    // whole 128-byte K segments for the grouped products (the pad columns are zero)
    const int seg = 128 / g.es;
    o.NP = (bg.col_g + g.r + seg - 1) / seg * seg;
    o.dP = take(prow * o.NP * g.es);
    if (bg.s > 1) {
      o.dY = take(prow * g.d * g.es);
      o.Yc = take(prow * g.d * g.es);
    }
    o.ycat = take(prow * bg.h * g.dv * g.es);
    o.dxp = take(prow * g.d * g.es);
    o.WpT = take((size_t)g.d * o.NP * g.es);  // Wp^T [d][NP]
    if (g.norm) {
      o.yn = take(rows * g.dv * g.es);         // normalised rows, laid out as y
      o.ngt = take(prow * bg.h * g.dv * 4);    // per-row terms of the gains' gradient
    }
    gate_cols += (size_t)(g.r + 1) * bg.h * g.dk;
    norm_cols += (size_t)bg.h * g.dv;
    // the partials of its two weight-gradient products, each in a region of its own
    const int K = (int)prow;
    if (K > 0) {
      part += wgrad_part_floats(g.bf16, bg.h * g.dv, g.d, K, true);       // W_o
      part += wgrad_part_floats(g.bf16, g.d, bg.col_g + g.r, K, false);  // q | k | v | W_g1
    }
  }
  G.dz = take((size_t)B * L * FUSION_STRIDE * 4);
  G.partial = take((size_t)BWD_WF_NRB * g.d * FUSION_STRIDE * 4);
  // column-sum partials: the gate's dW_g2 and db_g with db_f, or the gains' gradients
  G.mcol_floats = (size_t)BWD_NRB_MAX * std::max(gate_cols + g.m, norm_cols);
  G.mcol = take(G.mcol_floats * 4);
  G.Wo = take((size_t)g.Ktot * g.d * g.es);  // W_o rows [Ktot][d]
  G.splitk_floats = part;
  G.splitk = take(std::max<size_t>(part, 1) * 4);
  G.total = cur;
  return G;
}

rocblas_datatype storage_type(bool bf16) { return bf16 ? rocblas_datatype_bf16_r : rocblas_datatype_f32_r; }

// Weight gradient C[M][N] = A^T B with A row-major [K][M] (lda) and B row-major
// [K][N] (ldb), K the long reduction over positions, written to the column
// ranges of `dst`.  With few output tiles the K range is cut into S slices
// computed as one strided batch into its own region `part` [S][M][N] (the
// cursor advances past it), to be summed by one reduction launch for every
// product (`jobs`), so that the product fills the chip.  S doubles while the batch stays within
// 192 output tiles of 128 x 128: measured on the main workload's backward
// against caps of 0 (no split) to 1536, more slices cost more in partial
// traffic and summing than they gain in occupancy (caps 768 and 1536: +15 and
// +40 us; 96 and below: +60 us and more).
bool gemm_wgrad(rocblas_handle h, int M, int N, int K, const void* A, rocblas_datatype ta, int lda,
                const void* Bm, rocblas_datatype tb, int ldb, const SplitDst& dst, float*& part, const float* part_end,
                SplitJobs& jobs, Wgrad* wg) {
  if (M == 0 || N == 0) return true;
  const bool bf16 = wg != nullptr;
  const int S = wgrad_slices(bf16, M, N, K);
  const bool direct = S == 1 && dst.n == 1 && dst.c0[0] == 0 && dst.nc[0] == N;
  float* C = direct ? dst.p[0] : part;
  if (!direct && (part + (size_t)S * M * N > part_end || jobs.n >= SplitJobs::MAX)) return false;
  if (bf16) {
    // the library's kernel, launched once for every product (launch_bwd_wgrad)
    if (wg->njobs >= 2 * MSGLA_MAX_BRANCHES) return false;
    WgradJob& j = wg->j[wg->njobs++];
    j.A = A;
    j.B = Bm;
    j.C = C;
    j.M = M;
    j.N = N;
    j.K = K;
    j.lda = lda;
    j.ldb = ldb;
    j.S = S;
    j.Ks = wgrad_ks(K);
    j.tiles_n = (N + 127) / 128;
    j.tiles = (M + 127) / 128 * j.tiles_n;
    j.item_begin = wg->items;
    wg->items += j.tiles * S;
  } else {
    const float alpha = 1.f, beta = 0.f;
    const int Ks = K / S;
    const rocblas_stride sA = (rocblas_stride)Ks * lda, sB = (rocblas_stride)Ks * ldb,
                         sC = (rocblas_stride)M * N;
    if (rocblas_gemm_strided_batched_ex(h, rocblas_operation_none, rocblas_operation_transpose, N, M, Ks, &alpha,
                                        Bm, tb, ldb, sB, A, ta, lda, sA, &beta, C, rocblas_datatype_f32_r, N, sC, C,
                                        rocblas_datatype_f32_r, N, sC, S, rocblas_datatype_f32_r,
                                        rocblas_gemm_algo_standard, 0, 0) != rocblas_status_success)
      return false;
  }
  if (!direct) {
    // summed with the other products' partials by one launch at the end
    const int jn = jobs.n++;
    jobs.part[jn] = part;
    jobs.S[jn] = S;
    jobs.M[jn] = M;
    jobs.N[jn] = N;
    jobs.dst[jn] = dst;
    part += (size_t)S * M * N;
  }
  return true;
}

// Appends a column sum of src [rows][cols] (row stride ld) into dst[cols].
bool add_colsum(ColsumJobs& J, size_t& used, size_t cap, const float* src, int rows, int cols, int ld,
                float* dst) {
  if (J.n >= ColsumJobs::MAX) return false;
  const int j = J.n++;
  J.src[j] = src;
  J.dst[j] = dst;
  J.rows[j] = rows;
  J.cols[j] = cols;
  J.ld[j] = ld;
  J.nrb[j] = colsum_blocks(rows);
  J.pofs[j] = used;
  used += (size_t)J.nrb[j] * cols;
  J.cb[j + 1] = J.cb[j] + (cols + 63) / 64;
  J.fb[j + 1] = J.fb[j] + (cols + 255) / 256;
  return used <= cap;
}

// Appends the group C [M][N] (ldc) = A [M][K] B [N][K]^T to a grouped product.
void add_group(BwdGemm& Gm, const void* A, int lda, const void* Bm, int ldb, void* C, int ldc, int M, int N,
               int K) {
  if (M == 0 || N == 0 || K == 0) return;
  BwdGemmGroup& gg = Gm.g[Gm.ngroups++];
  gg.A = A;
  gg.B = Bm;
  gg.C = C;
  gg.M = M;
  gg.N = N;
  gg.K = K;
  gg.lda = lda;
  gg.ldb = ldb;
  gg.ldc = ldc;
  gg.tiles_n = (N + 127) / 128;
  gg.total = (M + 127) / 128 * gg.tiles_n;
  // XCD x receives the x-th eighth of every group
  int most = 0;
  for (int x = 0; x < N_XCD; ++x) {
    int n = 0;
    for (int i = 0; i < Gm.ngroups; ++i) {
      const int T = Gm.g[i].total;
      n += (int)((int64_t)T * (x + 1) / N_XCD) - (int)((int64_t)T * x / N_XCD);
    }
    most = std::max(most, n);
  }
  Gm.per_xcd = most;
}

// Appends out [C][Rp] (ldo) = in [R][C]^T (ldi), rows R .. Rp of out zero.
void add_transpose(BwdTranspose& T, const void* in, int R, int C, int ldi, void* out, int Rp, int ldo) {
  BwdTransposeJob& j = T.j[T.njobs++];
  j.in = in;
  j.out = out;
  j.R = R;
  j.C = C;
  j.Rp = Rp;
  j.ldi = ldi;
  j.ldo = ldo;
  j.tile_begin = T.total_tiles;
  j.tiles_c = (C + 63) / 64;
  T.total_tiles += (Rp + 63) / 64 * j.tiles_c;
}

SplitDst one_dst(float* p, int n) {
  SplitDst d{};
  d.p[0] = p;
  d.c0[0] = 0;
  d.nc[0] = n;
  d.n = 1;
  return d;
}

// one rocBLAS handle per device, created on first use; calls are serialised
std::mutex g_blas_mu;
rocblas_handle g_blas[64] = {};

rocblas_handle blas_handle() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  if (!g_blas[dev]) {
    rocblas_handle h = nullptr;
    if (rocblas_create_handle(&h) != rocblas_status_success) return nullptr;
    // no atomic accumulation inside the library's kernels: the gradients are the
    // same bits from call to call
    if (rocblas_set_atomics_mode(h, rocblas_atomics_not_allowed) != rocblas_status_success) {
      rocblas_destroy_handle(h);
      return nullptr;
    }
    g_blas[dev] = h;
  }
  return g_blas[dev];
}

#define BLAS_TRY(expr)                              \
  do {                                              \
    if (!(expr)) return MSGLA_ERR_HIP;              \
  } while (0)

}  // namespace

extern "C" {

size_t msgla_backward_workspace_bytes(const msgla_config* cfg, int64_t B, int64_t L) {
  if (check_config(cfg) != MSGLA_OK || !batch_ok(B, L) || !bwd_supported(cfg)) return 0;
  return bwd_geom(pack_geom(cfg), B, L).total;
}

}  // extern "C"

namespace {

// The hooks that keep the forward's intermediates where the backward reads them.
FwdHooks bwd_hooks(const PackGeom& g, const BwdGeom& G, void* workspace) {
  FwdHooks hooks{};
  for (int i = 0; i < g.m; ++i) {
    if (g.br[i].s > 1) hooks.yc[i] = at<char>(workspace, G.br[i].Yc);
    if (g.norm) hooks.yn[i] = at<char>(workspace, G.br[i].yn);
  }
  return hooks;
}

// recompute: run the forward's launches first (msgla_backward); otherwise the
// workspace holds them from msgla_forward_train (msgla_backward_saved)
msgla_status backward_impl(const msgla_config* cfg, const void* packed, const void* x, const void* dout,
                           const uint8_t* mask, int64_t B, int64_t L, void* dx, const msgla_grads* grads,
                           void* workspace, size_t workspace_bytes, void* stream, bool recompute) {
  if (msgla_status st = check_config(cfg); st != MSGLA_OK) return st;
  if (!bwd_supported(cfg)) return MSGLA_ERR_UNSUPPORTED;
  if (!batch_ok(B, L)) return MSGLA_ERR_INVALID_ARG;
  if (!packed || !x || !dout || !dx || !grads || !workspace) return MSGLA_ERR_INVALID_ARG;
  if (!aligned16(packed) || !aligned16(x) || !aligned16(dout) || !aligned16(dx) || !aligned16(workspace))
    return MSGLA_ERR_INVALID_ARG;
  const PackGeom g = pack_geom(cfg);
  for (int i = 0; i < g.m; ++i) {
    const msgla_branch_grads& b = grads->br[i];
    if (!b.W_q || !b.W_k || !b.W_v || !b.W_g1 || !b.W_g2 || !b.b_g || !b.W_o) return MSGLA_ERR_INVALID_ARG;
    if (g.norm && !b.norm_g) return MSGLA_ERR_INVALID_ARG;
  }
  if (g.m > 1 && (!grads->W_f || !grads->b_f)) return MSGLA_ERR_INVALID_ARG;
  const BwdGeom G = bwd_geom(g, B, L);
  if (workspace_bytes < G.total) return MSGLA_ERR_WORKSPACE;
  const WsGeom& W = G.W;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const rocblas_datatype ST = storage_type(g.bf16);

  // forward intermediates (q, k, v^T, x W_g1, y, A, fusion weights, block means, Y)
  if (recompute) {
    const FwdHooks hooks = bwd_hooks(g, G, workspace);
    if (msgla_status s = forward_impl(cfg, packed, x, mask, B, L, nullptr, nullptr, nullptr, workspace,
                                      workspace_bytes, stream, nullptr, &hooks);
        s != MSGLA_OK)
      return s;
  }

  // rocBLAS (the fp32 layer's weight gradients only): the device's handle, one caller at a time
  std::unique_lock<std::mutex> lock(g_blas_mu, std::defer_lock);
  rocblas_handle hb = nullptr;
  if (!g.bf16) {
    lock.lock();
    hb = blas_handle();
    if (!hb || rocblas_set_stream(hb, st) != rocblas_status_success) return MSGLA_ERR_HIP;
  }

  BwdParams P{};
  P.B = (int)B;
  P.L = (int)L;
  P.d = g.d;
  P.dk = g.dk;
  P.dv = g.dv;
  P.C = g.C;
  P.r = g.r;
  P.rp = g.rp;
  P.m = g.m;
  P.inv_gamma = 1.0f / cfg->gate_normalizer;
  P.q_scale = cfg->q_scale;
  P.nbranch = g.m;
  P.fine = -1;
  P.x = x;
  P.mask = mask;
  P.dout = dout;
  P.dx = dx;
  P.w = at<float>(workspace, W.w);
  P.dz = at<float>(workspace, G.dz);
  P.Wf = g.m > 1 ? (g.carrier >= 0 ? at<char>(packed, g.br[g.carrier].off_Wp +
                                                          (size_t)g.br[g.carrier].col_z * g.d * g.es)
                                   : at<char>(packed, g.off_Wz))
                 : nullptr;
  int units = 0, gunits = 0, wunits = 0;
  for (int i = 0; i < g.m; ++i) {
    const BranchGeom& bg = g.br[i];
    const WsBranch& wb = W.br[i];
    const BwdBranchGeom& o = G.br[i];
    BwdBranch& Br = P.br[i];
    Br.s = bg.s;
    Br.h = bg.h;
    Br.n = wb.n;
    Br.nch = wb.nch;
    Br.np = wb.np;
    Br.unit_begin = units;
    units += (int)B * bg.h * wb.nch;
    Br.gg_begin = gunits;
    gunits += (int)B * wb.nch;
    Br.walk_begin = wunits;
    if (wb.nch > 0) wunits += (int)B * bg.h * (g.dv / 64) * (g.dk / 32);
    Br.col_k = bg.col_k;
    Br.col_v = bg.col_v;
    Br.col_g = bg.col_g;
    Br.NP = o.NP;
    Br.q = at<float>(workspace, wb.q);
    Br.k = at<float>(workspace, wb.k);
    Br.vT = at<char>(workspace, wb.vT);
    Br.g = at<float>(workspace, wb.g);
    Br.y = at<char>(workspace, wb.y);
    Br.yv = g.norm ? at<char>(workspace, o.yn) : Br.y;
    Br.gn = g.norm ? at<float>(packed, bg.off_gn) : nullptr;
    Br.ngt = g.norm ? at<float>(workspace, o.ngt) : nullptr;
    Br.A = at<char>(workspace, wb.A);
    Br.yc = bg.s > 1 ? at<char>(workspace, o.Yc) : nullptr;
    Br.W2 = at<float>(packed, bg.off_W2);
    Br.bg = at<float>(packed, bg.off_bg);
    Br.lb = at<float>(workspace, o.lb);
    Br.sg = at<float>(workspace, o.sg);
    Br.g1c = at<float>(workspace, o.g1c);
    Br.Sst = at<float>(workspace, o.Sst);
    Br.dSt = at<float>(workspace, o.dSt);
    Br.AD = at<float>(workspace, o.AD);
    Br.QKi = at<float>(workspace, o.QKi);
    Br.rsum = at<float>(workspace, o.rsum);
    Br.rtot = at<float>(workspace, o.rtot);
    Br.dob = at<float>(workspace, o.dob);
    Br.gpart = at<float>(workspace, o.gpart);
    Br.dP = at<char>(workspace, o.dP);
    Br.dY = bg.s > 1 ? at<char>(workspace, o.dY) : nullptr;
    Br.ycat = at<char>(workspace, o.ycat);
    Br.dxp = at<char>(workspace, o.dxp);
    if (bg.s == 1) P.fine = i;
  }
  P.total_units = units;
  P.gate_units = gunits;
  P.walk_units = wunits;
  float* partial = at<float>(workspace, G.partial);
  float* mcol = at<float>(workspace, G.mcol);
  float* sk = at<float>(workspace, G.splitk);
  const float* sk_end = sk + G.splitk_floats;
  SplitJobs sjobs{};
  Wgrad wgrad{};  // bf16 storage: the weight-gradient products, one launch
  Wgrad* wgp = g.bf16 ? &wgrad : nullptr;
  const char* WoT = at<char>(packed, g.off_WoT);

  // ---- the weights as the grouped products read them: W_o rows, Wp^T ----
  {
    BwdTranspose T{};
    add_transpose(T, WoT, g.d, g.Ktot, g.Ktot, at<char>(workspace, G.Wo), g.d, g.d);
    for (int i = 0; i < g.m; ++i)
      if (P.br[i].n > 0)
        add_transpose(T, at<char>(packed, g.br[i].off_Wp), g.br[i].col_g + g.r, g.d, g.d,
                      at<char>(workspace, G.br[i].WpT), P.br[i].NP, P.br[i].NP);
    HIP_TRY(launch_bwd_transpose(T, g.bf16, st));
  }
  const char* Wo = at<char>(workspace, G.Wo);

  // ---- fusion, hold and the output projections ----
  // dY of the coarse branches, then every branch's dLoss/do = dO W_o^T (scale 1,
  // scaled by w_1 in k_bwd_out) or dY W_o^T as one grouped product
  for (int i = 0; i < g.m; ++i)
    if (P.br[i].n > 0 && P.br[i].s > 1) HIP_TRY(launch_bwd_hold(P, i, g.bf16, st));
  {
    BwdGemm Gm{};
    for (int i = 0; i < g.m; ++i) {
      const BwdBranch& Br = P.br[i];
      const int hdv = Br.h * g.dv;
      add_group(Gm, Br.s == 1 ? dout : Br.dY, g.d, Wo + (size_t)g.br[i].ko * g.d * g.es, g.d, Br.dob, hdv,
                (int)B * Br.n, hdv, g.d);
    }
    HIP_TRY(launch_bwd_gemm(Gm, g.bf16, false, st));
  }
  HIP_TRY(launch_bwd_out(P, g.bf16, st));
  for (int i = 0; i < g.m; ++i) {
    const BwdBranch& Br = P.br[i];
    const int hdv = Br.h * g.dv, rows = (int)B * Br.n;
    if (Br.n == 0) {
      HIP_TRY(fill_zero(grads->br[i].W_o, (size_t)hdv * g.d * 4, st));
      continue;
    }
    const void* dYi = Br.s == 1 ? dout : Br.dY;
    BLAS_TRY(gemm_wgrad(hb, hdv, g.d, rows, Br.ycat, ST, hdv, dYi, ST, g.d, one_dst(grads->br[i].W_o, g.d), sk,
                        sk_end, sjobs, wgp));
  }

  // ---- the normalisation: dLoss/d(normalised rows) -> dLoss/do, and the gains' gradient ----
  if (g.norm) {
    ColsumJobs J{};
    size_t used = 0;
    for (int i = 0; i < g.m; ++i) {
      const BwdBranch& Br = P.br[i];
      const int hdv = Br.h * g.dv, rows = (int)B * Br.n;
      if (Br.n == 0) {
        HIP_TRY(fill_zero(grads->br[i].norm_g, (size_t)hdv * 4, st));
        continue;
      }
      HIP_TRY(launch_bwd_norm(P, i, g.bf16, st));
      if (!add_colsum(J, used, G.mcol_floats, Br.ngt, rows, hdv, hdv, grads->br[i].norm_g)) return MSGLA_ERR_HIP;
    }
    HIP_TRY(launch_bwd_mcolsum(J, mcol, st));
  }

  // ---- the chunkwise recurrence and the gate ----
  HIP_TRY(launch_bwd_gate(P, st));
  if (g.bf16) {
    // the states entering each chunk and the state gradients reaching each chunk's end
    HIP_TRY(launch_bwd_walk(P, false, st));
    HIP_TRY(launch_bwd_walk(P, true, st));
  } else {
    // the same as per-chunk increments and scans over the chunks
    HIP_TRY(launch_bwd_chunk(P, 0, g.bf16, st));
    HIP_TRY(launch_bwd_scan(P, false, st));
    HIP_TRY(launch_bwd_chunk(P, 1, g.bf16, st));
    HIP_TRY(launch_bwd_scan(P, true, st));
  }
  HIP_TRY(launch_bwd_chunk(P, 5, g.bf16, st));
  HIP_TRY(launch_bwd_chunk(P, 3, g.bf16, st));
  HIP_TRY(launch_bwd_chunk(P, 4, g.bf16, st));
  // the gate: dz, dg1 into dP, and dW_g2, db_g (with db_f) as column sums
  HIP_TRY(launch_bwd_gate_grads(P, g.bf16, st));
  {
    ColsumJobs J{};
    size_t used = 0;
    for (int i = 0; i < g.m; ++i) {
      const BwdBranch& Br = P.br[i];
      const int hdk = Br.h * g.dk;
      if (Br.n == 0) {
        HIP_TRY(fill_zero(grads->br[i].W_g2, (size_t)g.r * hdk * 4, st));
        HIP_TRY(fill_zero(grads->br[i].b_g, (size_t)hdk * 4, st));
        continue;
      }
      const int parts = 2 * (int)B * Br.nch, ld = (g.r + 1) * hdk;
      if (!add_colsum(J, used, G.mcol_floats, Br.gpart, parts, g.r * hdk, ld, grads->br[i].W_g2) ||
          !add_colsum(J, used, G.mcol_floats, Br.gpart + (size_t)g.r * hdk, parts, hdk, ld, grads->br[i].b_g))
        return MSGLA_ERR_HIP;
    }
    if (g.m > 1 && !add_colsum(J, used, G.mcol_floats, P.dz, (int)(B * L), g.m, FUSION_STRIDE, grads->b_f))
      return MSGLA_ERR_HIP;
    HIP_TRY(launch_bwd_mcolsum(J, mcol, st));
  }

  // ---- the input projections and the pooling ----
  // dLoss/d(pooled input) of every branch as one grouped product dP Wp^T, then
  // the weight gradients of the q | k | v | x W_g1 columns, one product per branch
  if (mask && P.fine >= 0 && P.br[P.fine].n > 0) HIP_TRY(launch_bwd_mask_rows(P, P.fine, g.bf16, st));
  {
    BwdGemm Gm{};
    for (int i = 0; i < g.m; ++i) {
      const BwdBranch& Br = P.br[i];
      add_group(Gm, Br.dP, Br.NP, at<char>(workspace, G.br[i].WpT), Br.NP, const_cast<void*>(Br.dxp), g.d,
                (int)B * Br.n, g.d, Br.NP);
    }
    HIP_TRY(launch_bwd_gemm(Gm, g.bf16, true, st));
  }
  for (int i = 0; i < g.m; ++i) {
    const BwdBranch& Br = P.br[i];
    const BranchGeom& bg = g.br[i];
    const msgla_branch_grads& gr = grads->br[i];
    const int hdk = Br.h * g.dk, hdv = Br.h * g.dv, rows = (int)B * Br.n;
    if (Br.n == 0) {
      HIP_TRY(fill_zero(gr.W_q, (size_t)g.d * hdk * 4, st));
      HIP_TRY(fill_zero(gr.W_k, (size_t)g.d * hdk * 4, st));
      HIP_TRY(fill_zero(gr.W_v, (size_t)g.d * hdv * 4, st));
      HIP_TRY(fill_zero(gr.W_g1, (size_t)g.d * g.r * 4, st));
      continue;
    }
    const char* dP = static_cast<const char*>(Br.dP);
    const void* xp = bg.s == 1 ? x : static_cast<const void*>(at<char>(workspace, W.br[i].xp));
    // one product for the q | k | v | x W_g1 columns, scattered into the four gradients
    SplitDst dw{};
    dw.n = 4;
    dw.p[0] = gr.W_q, dw.c0[0] = 0, dw.nc[0] = hdk;
    dw.p[1] = gr.W_k, dw.c0[1] = bg.col_k, dw.nc[1] = hdk;
    dw.p[2] = gr.W_v, dw.c0[2] = bg.col_v, dw.nc[2] = hdv;
    dw.p[3] = gr.W_g1, dw.c0[3] = bg.col_g, dw.nc[3] = g.r;
    BLAS_TRY(gemm_wgrad(hb, g.d, bg.col_g + g.r, rows, xp, ST, g.d, dP, ST, Br.NP, dw, sk, sk_end, sjobs, wgp));
  }
  if (wgp) HIP_TRY(launch_bwd_wgrad(wgrad, st));
  HIP_TRY(launch_bwd_splitk_reduce(sjobs, st));
  HIP_TRY(launch_bwd_dx(P, g.bf16, st));
  if (g.m > 1) {
    HIP_TRY(launch_bwd_wf_partial(P, partial, BWD_WF_NRB, g.bf16, st));
    HIP_TRY(launch_bwd_wf_finish(partial, BWD_WF_NRB, g.d, g.m, grads->W_f, st));
  }
  return MSGLA_OK;
}

}  // namespace

extern "C" {

msgla_status msgla_backward(const msgla_config* cfg, const void* packed, const void* x, const void* dout,
                            const uint8_t* mask, int64_t B, int64_t L, void* dx, const msgla_grads* grads,
                            void* workspace, size_t workspace_bytes, void* stream) {
  return backward_impl(cfg, packed, x, dout, mask, B, L, dx, grads, workspace, workspace_bytes, stream, true);
}

msgla_status msgla_backward_saved(const msgla_config* cfg, const void* packed, const void* x, const void* dout,
                                  const uint8_t* mask, int64_t B, int64_t L, void* dx, const msgla_grads* grads,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  return backward_impl(cfg, packed, x, dout, mask, B, L, dx, grads, workspace, workspace_bytes, stream, false);
}

msgla_status msgla_forward_train(const msgla_config* cfg, const void* packed, const void* x, const uint8_t* mask,
                                 int64_t B, int64_t L, void* out, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  if (msgla_status st = check_config(cfg); st != MSGLA_OK) return st;
  if (!bwd_supported(cfg)) return MSGLA_ERR_UNSUPPORTED;
  if (!batch_ok(B, L)) return MSGLA_ERR_INVALID_ARG;
  if (!out || !workspace) return MSGLA_ERR_INVALID_ARG;
  const PackGeom g = pack_geom(cfg);
  const BwdGeom G = bwd_geom(g, B, L);
  if (workspace_bytes < G.total) return MSGLA_ERR_WORKSPACE;
  const FwdHooks hooks = bwd_hooks(g, G, workspace);
  return forward_impl(cfg, packed, x, mask, B, L, out, nullptr, nullptr, workspace, workspace_bytes, stream,
                      nullptr, &hooks);
}

}  // extern "C"
