// Kernel parameter blocks and memory layouts shared by the host API and the
// kernels.  Everything here is plain data passed to kernels by value.
//
// Memory layouts (T = storage type: bf16 or fp32; C = chunk length):
//
// Packed weights, per branch i (h heads, scale s):
//   Wp_i  [Np_i][d]  T   rows = output columns of the pooled projection:
//                        [ q: h d_k | k: h d_k | v: h d_v | g: rp | z: 16 if
//                        this branch carries the fusion logits ]
//                        (transposed so the GEMM reads both operands along d;
//                        rp = 16 if r <= 16 else 64, unused rows are zero)
//   W2_i  [rp][h d_k] fp32 (rows >= r zero),  bg_i [h d_k] fp32
// then, if fusion logits need their own pass (m > 1 and no scale-1 branch),
//   Wz [16][d] T (W_f^T, zero padded),
// then bf [16] fp32 (fusion bias, zero padded) and
//   WoT [d][Ktot] T   stacked W_o^T of all branches along K; branch i occupies
//                     columns [ko_i, ko_i + kp_i), kp_i = h_i d_v rounded up to
//                     a 128-byte multiple (zero padded).
//
// Forward workspace, per branch i (n = floor(L/s) pooled rows, nch = ceil(n/C),
// np = nch C):
//   q, k        [B][h][np][d_k]   fp32  projections (kept in fp32: the intra-chunk
//                                       products q_t . k_i can cancel strongly)
//   qt          [B][h][np][d_k]   T     q ⊙ exp(b) (chunk-local)
//   kT          [B][h][nch][d_k][C] T   (k ⊙ exp(b_last - b))^T per chunk
//   vT          [B][h][nch][d_v][C] T   v^T per chunk
//   g           [B][L][rp]        fp32  first gate factor x W_g1 at every position
//   A           [B][h][nch][C][C] T     masked decayed q k^T per chunk
//   lam         [B][h][nch][d_k]  fp32  exp(b_last) per chunk
//   y           [B][h][np][d_v]   T     GLA outputs o_t
//   xp, xp_lo   [B][n][d]         T     block means of a coarse branch (s > 1) and,
//                                       bf16 only, their residuals (masked calls)
// plus the fusion weights w [B L][8] fp32.  Rows >= n of a chunk are never
// written by the projection and are masked by every reader.
//
// State (fp32 except the header): 256-byte header {magic, version, B, m, pos,
// status}, then per branch S [B][h][d_k][d_v], psum [B][d], held [B][d] and
// tok [B] (tokens in the incomplete block: its positions, unless a masked
// forward left masked positions in it; psum sums only its tokens).
#pragma once
#include <stdint.h>
#include <stddef.h>

#ifndef MSGLA_MAX_BRANCHES
#define MSGLA_MAX_BRANCHES 8
#endif

namespace msgla {

constexpr uint32_t STATE_MAGIC = 0x4C47534Du;  // "MSGL"
constexpr uint32_t STATE_VERSION = 2;
constexpr size_t STATE_HEADER = 256;
constexpr int FUSION_STRIDE = 8;  // floats per row of the fusion-weight buffer
constexpr int N_XCD = 8;          // XCDs (separate L2 caches) of an MI355X

struct StateHeader {
  uint32_t magic;
  uint32_t version;
  int32_t B;
  int32_t m;
  int64_t pos;
  int32_t status;   // 0, or the msgla_status of the call that wrote it (then pos = -1)
  int32_t pad;
};

// A forward's check of its state_in header, made on the device (forward
// workspace): status 0 if the header describes this configuration and batch
// and records no error; pos = its position.  Every kernel that reads
// state_in reads it only when status is 0.
struct StateCheck {
  int32_t status;
  int32_t pad;
  int64_t pos;
  // per branch: positions of the block in progress on entry (pos mod s), and
  // the blocks that complete in this call, floor((L + r) / s); block j of the
  // call covers call positions [j s - r, (j + 1) s - r)
  int32_t r[MSGLA_MAX_BRANCHES];
  int32_t nv[MSGLA_MAX_BRANCHES];
};

struct StateCheckParams {
  const void* state_in;
  StateCheck* out;
  int B, m, L;
  int scale[MSGLA_MAX_BRANCHES];
};

// The entry offset r and complete-block count of branch i for a forward's
// kernels: from the device-side check when the call continues from a state
// that passed it, else (a fresh call) 0 and n.
__host__ __device__ inline int entry_offset(const StateCheck* chk, int i) {
  return chk && chk->status == 0 ? chk->r[i] : 0;
}
__host__ __device__ inline int blocks_in_call(const StateCheck* chk, int i, int n) {
  return chk && chk->status == 0 ? chk->nv[i] : n;
}

// ---------------- pooling prepass ------------------------------------------------
struct PoolOut {
  void* xp;         // [B][n][d] block means of scale s
  void* xp_lo;      // [B][n][d] bf16 residuals m - bf16(m) of the means, or null
  int s, n;
  float inv_s;
  int branch;       // index of the branch (its entry offset in StateCheck)
  const float* psum_in;  // continuing: the entry state's pending sum [B][d] and
  const float* tok_in;   // token count [B] of this branch (block 0 of the call)
};

struct PoolParams {
  const void* x;    // [B][L][d]
  const uint8_t* mask;  // [B][L] token mask of Eq. (8) (nonzero = token), or null
  const StateCheck* chk;  // continuing from a state: its check (entry offsets), else null
  int B, L, d, smax, nout;
  PoolOut out[MSGLA_MAX_BRANCHES];
  int lvl[8];       // power-of-two smax: out index of scale 2^l, or -1 (set by the launcher)
};

// ---------------- K1: pooled projection GEMM ----------------------------------
// B-operand rows [col0, col0 + cnt) of the small projection start at W (row
// stride d elements): each branch's gate first factor, then the fusion logits.
struct XSeg {
  const void* W;
  int col0, cnt;
};

struct K1Group {
  const void* Wp;   // [N][d]: the transposed q, k and v projections (branch groups)
  const void* A;    // A rows: x (scale 1 and the small group) or the block means [M][d]
  const void* A_lo; // residuals of the block means [M][d] (masked bf16 calls), or null:
                    // the q / k column tiles then run K over [A | A_lo] against [W | W]
  int s;            // pooling factor
  int n;            // pooled rows per sequence
  int M;            // B * n
  int N;            // GEMM columns: h (2 dk + dv), or Ns for the small group
  int tiles_n;      // ceil(N / BN)
  int h;            // heads
  int col_k, col_v; // column ranges: q [0, col_k), k [col_k, col_v), v [col_v, N)
  int np, nch;      // padded rows and chunks per (b, head)
  float* q;         // outputs (see layout)
  float* k;
  void* vT;
};

// The small projection x [W_g1^(1) | ... | W_g1^(m) | W_f] over the unpooled
// rows: each branch's gate first factor at every position and the fusion weights.
struct K1Small {
  int group;        // index of its group in K1Params::g, -1 if none
  int m, rp;
  int gm;           // branches whose gate first factors lead the columns (m, or 0 for the weights alone)
  int nseg;
  XSeg seg[MSGLA_MAX_BRANCHES + 1];
  float* g[MSGLA_MAX_BRANCHES];  // per branch [B L][rp] fp32
  int zcol;         // first fusion-logit column, -1 if none
  const float* bf;  // fusion bias [m]
  float* w;         // fusion weights [B L][FUSION_STRIDE]
};

struct K1Params {
  int B, d, dk, dv, C;
  const uint8_t* mask;  // [B][L] token mask, or null: rows of masked positions of the scale-1 group are zero
  int ngroups, total_tiles, per_xcd;
  K1Group g[MSGLA_MAX_BRANCHES + 1];
  K1Small sm;
  // Tile schedule: XCD x takes m-tiles [mt_begin[g][x], mt_begin[g][x + 1]) of
  // every group g (all their column tiles), the groups in the order `order`;
  // per_xcd is the longest of the eight lists
  int order[MSGLA_MAX_BRANCHES + 1];
  int mt_begin[MSGLA_MAX_BRANCHES + 1][N_XCD + 1];
};

// ---------------- K2a: chunk-local gate, decay and intra-chunk matrix ----------
struct K2Branch {
  int h, n, nch, np;
  int s;            // pooling factor
  int unit_begin;   // first flattened (b, head, chunk) unit of this branch (K2a)
  int seq_begin;    // first flattened (b, head) sequence of this branch (K2b)
  const float* q;
  const float* k;
  const float* g;   // x W_g1 at every unpooled position [B L][rp] (averaged over each block here)
  const float* W2;  // [rp][h dk], rows >= r are zero
  const float* bg;  // [h dk]
  void* qt;
  void* kT;
  const void* vT;
  void* A;
  float* lam;
  void* y;
  float* S_out;     // state S of this branch [B][h][dk][dv] or null
  const float* S_in;  // state S the walk starts from [B][h][dk][dv], null: zero
  // continuing: block 0 of the call completes the entry state's pending block,
  // whose gate first factors sum to psumg [B][rp] (its pending sum times W_g1)
  // over tok_in [B] tokens
  const float* psumg;
  const float* tok_in;
};

struct K2Params {
  int B, L, dk, dv, r, rp, C;
  float inv_gamma;
  float q_scale;
  const uint8_t* mask;  // [B][L] token mask: the gate factor is averaged over a block's tokens, or null
  int nbranch;
  int total_units;  // K2a grid
  int total_seqs;   // K2b: number of (branch, b, head) sequences
  int n_dvt;        // K2b: d_v tiles per sequence
  int per_xcd;      // K2b block remap
  int order[MSGLA_MAX_BRANCHES];  // K2b: branches by decreasing chunk count
  // K2b segmented walk (few sequences, long chains): each sequence's chunks are
  // cut into nseg segments walked in parallel, first for their local states
  // (state-only pass from zero), then, after a scan over the segments, again
  // from their true start states.  nseg = 1: one walk per sequence.
  int nseg;
  int seg_base;     // workgroups of one segment (the plain walk's grid)
  float* Sseg;      // [total_seqs][nseg][dk][dv] fp32: local, then start states
  const StateCheck* chk;  // check of state_in (S_in is read only if it passed), or null
  K2Branch br[MSGLA_MAX_BRANCHES];
};

// ---------------- K3: output projections, hold and fusion ---------------------
struct K3Branch {
  const void* y;    // [B][h][np][dv]
  void* yc;         // coarse outputs y W_o [B][n][d] (branches with s > 1)
  int s, h, np, n;
  int ko;           // K offset of the branch in the stacked W_o^T
  int tile_begin;   // first tile of the branch in the coarse work list
  const float* held_in;  // output held from before this call [B][d] fp32, null: zero
};

struct K3Params {
  int B, L, d, dv, m, Ktot;
  int fine;                           // branch with scale 1, or -1
  int ncoarse;                        // branches with s > 1, in work-list order
  int coarse[MSGLA_MAX_BRANCHES];
  int tiles_n;                        // column tiles of d
  int c_total, c_per_xcd;             // coarse GEMM work list (K3c)
  int f_total, f_per_xcd;             // fine GEMM + fusion work list (K3f)
  int held_in;                        // the call continues from a state
  const StateCheck* chk;              // its check (held_in read only if it passed), or null
  const void* zero; // >= 128 zero bytes (rows outside the problem)
  const void* WoT;  // [d][Ktot]
  const float* w;   // fusion weights [B L][8]
  void* out;        // [B][L][d]
  K3Branch br[MSGLA_MAX_BRANCHES];
};

// ---------------- backward ------------------------------------------------------
// Backward workspace, per branch (n, nch, np as in the forward; T = storage type;
// rows >= n of a chunk hold no position and are zero or ignored):
//   lb, sg      [B][h][np][d_k]        fp32  chunk-local cumulative log alpha, and
//                                            sigmoid(-z) / gamma (the gate's slope)
//   g1c         [B n][rp]              fp32  block means of x W_g1
//   Sst, dSt    [B][h][nch][d_k][d_v]  fp32  state entering each chunk, and the
//                                            loss gradient reaching each chunk's
//                                            last state from later chunks
//   AD          [B][h][nch][64][64]    fp32  D (do v^T, t >= i) of each chunk
//   QKi         [B][h][nch][2][64][d_k] fp32 do S_prev^T and v dS_end^T of each chunk
//   rsum, rtot  [B][h][np][d_k], [B][h][nch][d_k]  fp32  in-chunk suffix sums of
//                                            q dq - k dk, and their chunk totals
//   dob         [B n][h d_v]           fp32  dLoss/d(GLA output o)
//   gpart       [B nch][2][r + 1][h d_k]  fp32  per (chunk, half of its rows):
//                                            sums of g1 dz (rows 0..r-1) and of dz
//                                            (row r), dz = dLoss/d(gate pre-activation)
//   dP          [B n][NP]              T     dLoss/d[q | k | v | x W_g1] columns
//                                            (q_scale folded into q); NP = col_g + r
//                                            rounded up to whole 128-byte segments,
//                                            the columns past col_g + r zero
//   dY, Yc      [B n][d]               T     coarse branches: dLoss/dY and Y = y W_o
//   ycat        [B n][h d_v]           T     y rows position-major (scale 1: w_1 y)
//   dxp         [B n][d]               T     dLoss/d(pooled input)
// plus dz [B L][8] fp32 (dLoss/d fusion logits) and reduction partials.
struct BwdBranch {
  int s, h, n, nch, np;
  int unit_begin;             // first (b, head, chunk) unit of the branch
  int gg_begin;               // first (b, chunk) unit of the branch's gate gradients
  int walk_begin;             // first (b, head, d_v slice, d_k part) unit of its state walks
  int col_k, col_v, col_g, NP;
  const float* q;             // forward workspace: projections (q unscaled)
  const float* k;
  const void* vT;
  const float* g;             // x W_g1 at every unpooled position [B L][rp]
  const void* y;              // GLA outputs [B][h][np][d_v]
  const void* yv;             // the rows the output projection read: y, or y normalised
  const float* gn;            // normalisation gains [h d_v] (config norm), or null
  float* ngt;                 // per-row terms of the gains' gradient [B n][h d_v], or null
  const void* A;              // the forward's decayed q k^T per chunk [B][h][nch][C][C] (T)
  const void* yc;             // coarse outputs [B n][d] (s > 1)
  const float* W2;            // packed gate factor [rp][h d_k] and bias [h d_k]
  const float* bg;
  float* lb;
  float* sg;
  float* g1c;
  float* Sst;
  float* dSt;
  float* AD;
  float* QKi;                 // [B][h][nch][2][64][d_k] do S^T and v dS^T of each chunk
  float* rsum;
  float* rtot;
  float* dob;
  float* gpart;
  void* dP;
  void* dY;
  void* ycat;
  const void* dxp;
};

struct BwdParams {
  int B, L, d, dk, dv, C, r, rp, m;
  float inv_gamma, q_scale;
  int nbranch, total_units, gate_units, walk_units;
  int fine;                   // branch with scale 1, or -1
  const void* x;              // [B][L][d] T
  const uint8_t* mask;        // [B][L] token mask of the forward, or null
  const void* dout;           // [B][L][d] T
  void* dx;                   // [B][L][d] T
  const float* w;             // fusion weights [B L][8]
  float* dz;                  // [B L][8]
  const void* Wf;             // fusion logit rows [m][d] T (packed), null when m == 1
  BwdBranch br[MSGLA_MAX_BRANCHES];
};

// Column sums of several row-major fp32 matrices in one pair of launches
// (k_bwd_mcolsum_*): job j sums rows x cols of src[j] (row stride ld) into
// dst[j][cols] through nrb[j] row blocks of partials at part + pofs[j].
struct ColsumJobs {
  static constexpr int MAX = 2 * MSGLA_MAX_BRANCHES + 1;
  int n;
  const float* src[MAX];
  float* dst[MAX];
  int rows[MAX], cols[MAX], ld[MAX], nrb[MAX];
  int cb[MAX + 1];   // first 64-column block of each job (partial pass)
  int fb[MAX + 1];   // first 256-column block of each job (finishing pass)
  size_t pofs[MAX];
};

// Grouped products on the matrix cores (k_bwd_gemm): per group g,
// C_g [M][N] (ldc) = A_g [M][K] B_g [N][K]^T, A and B in the storage type
// with K contiguous (lda, ldb elements); K a multiple of 128 bytes of elements.
struct BwdGemmGroup {
  const void* A;
  const void* B;
  void* C;                  // fp32 or the storage type (per launch)
  int M, N, K, lda, ldb, ldc;
  int total, tiles_n;       // 128 x 128 tiles of the group, column tiles
};
struct BwdGemm {
  int ngroups, per_xcd;     // per_xcd: the most tiles any XCD receives
  BwdGemmGroup g[MSGLA_MAX_BRANCHES];
};

// Transposes with zero padding (k_bwd_transpose): out[c][r] (ldo) = in[r][c]
// (ldi) for r < R, c < C; out[c][r] = 0 for R <= r < Rp.
struct BwdTransposeJob {
  const void* in;
  void* out;
  int R, C, Rp, ldi, ldo;
  int tile_begin, tiles_c;  // first 64 x 64 tile, tiles along C
};
struct BwdTranspose {
  int njobs, total_tiles;
  BwdTransposeJob j[MSGLA_MAX_BRANCHES + 1];
};

// Destinations of a split-K weight-gradient product (k_bwd_splitk_reduce).
struct SplitDst {
  float* p[4];
  int c0[4], nc[4];
  int n;
};

// Weight-gradient products on the matrix cores (k_bwd_wgrad), bf16 storage:
// per job C_s [M][N] fp32 = sum over positions k in slice s of A[k][m] B[k][n],
// A [K][lda] and B [K][ldb] position-major (m and n contiguous), for the
// slices s < S of Ks positions each; C_s at C + s M N.
struct WgradJob {
  const void* A;
  const void* B;
  float* C;
  int M, N, K, lda, ldb, S, Ks;
  int tiles_n, tiles;  // 128 x 128 output tiles: along N, in all
  int item_begin;      // first work item (tile, slice) of the job
};
struct Wgrad {
  int njobs, items;
  WgradJob j[2 * MSGLA_MAX_BRANCHES];
};

// Every split-K product of a backward, summed by one launch: job j adds the S[j]
// slices part[j] [S][M][N] into its destinations.
struct SplitJobs {
  static constexpr int MAX = 2 * MSGLA_MAX_BRANCHES;
  int n;
  const float* part[MAX];
  int S[MAX], M[MAX], N[MAX];
  SplitDst dst[MAX];
};

// ---------------- packing ------------------------------------------------------
struct PackSrc {
  const void* W_q; const void* W_k; const void* W_v; const void* W_g1; const void* W_g2;
  const float* b_g; const void* W_o;
};

// ---------------- state export / init ------------------------------------------
struct StateBranch {
  int s, h, n, np, ko;
  float* S; float* psum; float* held; float* tok;
  const void* y;    // forward workspace y (export only)
  const float* S_in;     // state the forward started from (kept when n == 0), or null
  const float* held_in;
  const float* psum_in;  // the entry state's pending sum and token count, or null
  const float* tok_in;
};

// Pending-gate sums of a continuing forward (k_pending_gate).
struct PendingGateBranch {
  const void* Wg1;  // [rp][d] the branch's W_g1, transposed (rows of its packed block)
  const float* psum;  // entry state's pending sum [B][d]
  float* out;       // [B][rp]
};
struct PendingGateParams {
  int B, d, rp, m;
  const StateCheck* chk;
  PendingGateBranch br[MSGLA_MAX_BRANCHES];
};

struct StateParams {
  int B, L, d, dk, dv, m, Ktot;
  int64_t pos;      // tokens of this call (added to the entry position)
  const StateCheck* chk;  // check of the entry state (S_in / held_in read only if it passed), or null
  const void* x;    // forward input (export only)
  const uint8_t* mask;  // the forward's token mask [B][L], or null
  const void* WoT;
  void* state;      // header
  StateBranch br[MSGLA_MAX_BRANCHES];
};

// ---------------- decode ---------------------------------------------------------
struct DecBranch {
  int s, h, N, col_k, col_v, col_g, col_z, ko;
  const void* Wp;   // [N][d]
  const float* W2;
  const float* bg;
  float* S;         // state [B][h][dk][dv]
  float* psum;      // [B][d]
  float* held;      // [B][d]
  float* tok;       // [B] tokens in the incomplete block
  float* proj;      // workspace [B][N]
  float* y;         // workspace [B][h dv]
  const float* gn;  // normalisation gains [h dv], or null (no normalisation)
};

struct DecParams {
  int B, d, dk, dv, r, m, Ktot;
  float inv_gamma, q_scale;
  const void* x;    // [B][d]
  void* out;        // [B][d]
  void* state;      // header (pos)
  int64_t* pos_ws;  // workspace copy of pos for this step
  float* w;         // fusion logits x_t W_f [B][8] of this step (projection kernel)
  const void* Wz;   // fusion-logit weights W_f^T [m][d] (inside a branch's Wp or separate)
  const float* bf;
  const void* WoT;
  int nbranch;
  int norm;         // the branches' outputs are normalised before W_o
  DecBranch br[MSGLA_MAX_BRANCHES];
};

// ---------------- optional per-head RMS normalisation of the branch outputs ---
constexpr float NORM_EPS = 1e-6f;

struct NormBranch {
  void* y;          // [B][h][np][dv] storage type, normalised in place
  void* yo;         // or, when set, written here (same layout) and y kept
  const float* g;   // gains [h dv] fp32
  int h, n, np;     // heads, rows per (b, head), padded row stride
  int row_begin;    // first flattened row (b, head, j) of this branch
};

struct NormParams {
  int dv, nbranch, total_rows;
  NormBranch br[MSGLA_MAX_BRANCHES];
};

}  // namespace msgla
