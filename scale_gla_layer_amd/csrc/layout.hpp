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
//   g           [B][np][rp]       fp32  first gate factor xp W_g1
//   A           [B][h][nch][C][C] T     masked decayed q k^T per chunk
//   lam         [B][h][nch][d_k]  fp32  exp(b_last) per chunk
//   y           [B][h][np][d_v]   T     GLA outputs o_t
// plus the fusion weights w [B L][8] fp32.  Rows >= n of a chunk are never
// written by the projection and are masked by every reader.
//
// State (fp32 except the header): 256-byte header {magic, version, B, m, pos},
// then per branch S [B][h][d_k][d_v], psum [B][d], held [B][d].
#pragma once
#include <stdint.h>
#include <stddef.h>

#ifndef MSGLA_MAX_BRANCHES
#define MSGLA_MAX_BRANCHES 8
#endif

namespace msgla {

constexpr uint32_t STATE_MAGIC = 0x4C47534Du;  // "MSGL"
constexpr uint32_t STATE_VERSION = 1;
constexpr size_t STATE_HEADER = 256;
constexpr int FUSION_STRIDE = 8;  // floats per row of the fusion-weight buffer
constexpr int N_XCD = 8;          // XCDs (separate L2 caches) of an MI355X

struct StateHeader {
  uint32_t magic;
  uint32_t version;
  int32_t B;
  int32_t m;
  int64_t pos;
};

// ---------------- pooling prepass ------------------------------------------------
struct PoolOut {
  void* xp;         // [B][n][d] block means of scale s
  int s, n;
  float inv_s;
};

struct PoolParams {
  const void* x;    // [B][L][d]
  const uint8_t* mask;  // [B][L] token mask of Eq. (8) (nonzero = token), or null
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
  int s;            // pooling factor
  int n;            // pooled rows per sequence
  int M;            // B * n
  int N;            // GEMM columns: h (2 dk + dv), or Ns for the small group
  int tiles_n;      // ceil(N / BN)
  int tile_begin;   // first flattened tile of this group
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
  const void* zero; // >= 128 zero bytes (rows outside the problem)
  const void* WoT;  // [d][Ktot]
  const float* w;   // fusion weights [B L][8]
  void* out;        // [B][L][d]
  K3Branch br[MSGLA_MAX_BRANCHES];
};

// ---------------- packing ------------------------------------------------------
struct PackSrc {
  const void* W_q; const void* W_k; const void* W_v; const void* W_g1; const void* W_g2;
  const float* b_g; const void* W_o;
};

// ---------------- state export / init ------------------------------------------
struct StateBranch {
  int s, h, n, np, ko;
  float* S; float* psum; float* held;
  const void* y;    // forward workspace y (export only)
  const float* S_in;     // state the forward started from (kept when n == 0), or null
  const float* held_in;
};

struct StateParams {
  int B, L, d, dk, dv, m, Ktot;
  int64_t pos;
  const void* x;    // forward input (export only)
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
  const float* g;   // gains [h dv] fp32
  int h, n, np;     // heads, rows per (b, head), padded row stride
  int row_begin;    // first flattened row (b, head, j) of this branch
};

struct NormParams {
  int dv, nbranch, total_rows;
  NormBranch br[MSGLA_MAX_BRANCHES];
};

}  // namespace msgla
