/*
 * msgla.h — C ABI of the MS-GLA token-mixing layer forward for AMD MI355X (gfx950).
 *
 * The layer (reading notes "MS-GLA：多时间尺度门控线性注意力研读笔记" on
 * arXiv:2609.35664, "MS-GLA: Multi-Scale Gated Linear Attention ...", Sec. 3,
 * Eqs. (8)-(11)): for every scale s of the branch set, average-pool the hidden
 * states X [L x d] over non-overlapping blocks of s tokens (Sec. 3.1, Eq. (8)),
 * project the pooled states to q, k, v and a low-rank forget gate with
 * per-branch weights (Sec. 3.2, Eq. (9)), run gated linear attention
 *     S_t = Diag(alpha_t) S_{t-1} + k_t^T v_t,   o_t = q_t S_t
 * (Sec. 2.1), project back to d, causally hold each coarse output from
 * position (j+1)s-1 until the next block completes (Sec. 3.3), and fuse the
 * branches per position with softmax weights computed from the unpooled x_t
 * (Sec. 3.3, Eqs. (10)-(11)).
 *
 * Conventions shared by every entry point:
 *  - All tensor pointers are DEVICE pointers unless stated otherwise, row-major,
 *    16-byte aligned.  The caller owns every buffer (inputs, outputs, packed
 *    weights, workspace, state); the library allocates nothing, keeps no
 *    global state and, except msgla_state_query, never synchronises: work is
 *    enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *    completes asynchronously.  Calls with distinct workspaces may run
 *    concurrently.
 *  - Weights reach msgla_forward and msgla_decode_step as ONE packed device
 *    blob (msgla_pack_weights, once per set of weights), not as the struct of
 *    per-matrix pointers (msgla_weights) that the packing reads: the blob holds
 *    them transposed and concatenated in the order the kernels stream them,
 *    so no call re-lays out a weight.
 *  - Errors in arguments are detected on the host before anything is enqueued
 *    and are returned synchronously; a failed kernel launch returns
 *    MSGLA_ERR_HIP.  NaN and Inf in the data are not checked; they propagate.
 *  - Element type: `dtype` of the config.  MSGLA_BF16 stores x, weights and
 *    outputs as bfloat16 and accumulates in fp32 (the recurrent state, the
 *    cumulative log-decay and all accumulators are fp32); MSGLA_F32 stores and
 *    computes everything in fp32.  Biases are always fp32.
 */
#ifndef MSGLA_H
#define MSGLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MSGLA_OK = 0,
  MSGLA_ERR_INVALID_ARG = 1,  /* bad config, NULL or misaligned pointer, bad size */
  MSGLA_ERR_UNSUPPORTED = 2,  /* valid request this build does not implement      */
  MSGLA_ERR_WORKSPACE = 3,    /* workspace / buffer smaller than the size query    */
  MSGLA_ERR_HIP = 4           /* a HIP runtime call or kernel launch failed        */
} msgla_status;

typedef enum { MSGLA_F32 = 0, MSGLA_BF16 = 1 } msgla_dtype;

#define MSGLA_MAX_BRANCHES 8

/*
 * Layer configuration.  Branch i pools over blocks of scale[i] tokens and owns
 * heads[i] heads of key width d_k and value width d_v (Sec. 3.2: the total head
 * count H = sum heads[i] is what a single-scale GLA layer would have).
 * gate_rank r: rank of the forget-gate projection W_g1 [d x r] W_g2 [r x h d_k];
 * log(alpha) = logsigmoid(xp W_g1 W_g2 + b_g) / gate_normalizer.
 * chunk: length of the GPU chunk schedule; the result does not depend on it
 * beyond rounding (Sec. 3.4 separates it from the pooling block).
 * q_scale multiplies q (1.0 reproduces the notes' recurrence).
 * norm: the notes name a per-branch normalisation without giving its form.
 * 0 leaves it out (identity); 1 applies, before the branch's W_o (in the
 * forward and in the streaming step), a per-head RMS normalisation over d_v
 * with gains: y_c / sqrt(mean_c' y_c'^2 + 1e-6) * norm_g[head d_v + c].
 * Other values are invalid.
 * Requirements (MSGLA_ERR_INVALID_ARG otherwise): 1 <= n_branches <= 8; scales
 * positive and distinct; 1 <= heads <= 64; d_model a multiple of 64 up to
 * 65536; 1 <= gate_rank <= 64; gate_normalizer > 0; and, by storage type,
 *   bf16: d_k in {32, 64, 128, 256}, d_v a multiple of 64 in [64, 512],
 *         chunk 32 or 64;
 *   fp32: d_k in {16, 32, 64, 128, 256}, d_v a multiple of 32 in [32, 512],
 *         chunk 16, 32 or 64.
 * Valid shapes whose chunk-state stages exceed a CU's 160 KB of LDS are not
 * implemented (MSGLA_ERR_UNSUPPORTED): bf16 d_k 256 with chunk 64; fp32 d_k
 * 256 with chunk 32 or 64; fp32 d_k 128 with chunk 64.
 */
typedef struct {
  int32_t n_branches;
  int32_t scale[MSGLA_MAX_BRANCHES];
  int32_t heads[MSGLA_MAX_BRANCHES];
  int32_t d_model;
  int32_t d_k;
  int32_t d_v;
  int32_t gate_rank;
  int32_t chunk;
  float gate_normalizer;
  float q_scale;
  int32_t dtype; /* msgla_dtype */
  int32_t norm;  /* 0: none; 1: per-head RMS normalisation of each branch's output (below) */
} msgla_config;

/*
 * Unpacked weights of one branch, in the notes' row-vector convention
 * (y = x W, W stored [in][out] row-major), element type = config dtype
 * except the fp32 bias.  Head j of the branch owns column slice j of W_q, W_k,
 * W_v, W_g2, b_g and row slice j of W_o.
 *   W_q, W_k [d][h d_k]   W_v [d][h d_v]   W_g1 [d][r]   W_g2 [r][h d_k]
 *   b_g [h d_k] (fp32)    W_o [h d_v][d]   (per-branch output projection, no bias)
 */
typedef struct {
  const void* W_q;
  const void* W_k;
  const void* W_v;
  const void* W_g1;
  const void* W_g2;
  const float* b_g;
  const void* W_o;
  const float* norm_g; /* [h d_v] fp32 gains of the normalisation (config norm = 1), else unused */
} msgla_branch_weights;

/* All weights.  W_f [d][m] (config dtype) and b_f [m] (fp32) give the fusion
 * logits z_t = x_t W_f + b_f over the m = n_branches branches (Eq. (10)); both
 * are ignored (and may be NULL) when m == 1. */
typedef struct {
  msgla_branch_weights br[MSGLA_MAX_BRANCHES];
  const void* W_f;
  const float* b_f;
} msgla_weights;

/* Human-readable name of a status code (static string). */
const char* msgla_status_str(msgla_status s);

/* Host-only check of a configuration against the requirements above. */
msgla_status msgla_validate_config(const msgla_config* cfg);

/*
 * Packed weights: one device blob in the layout the kernels read (per branch
 * the concatenated, transposed [q|k|v|g1|fusion] projection, the fp32 gate
 * factor and bias, and the stacked transposed output projections).  Packing is
 * done once per set of weights; `msgla_forward` and `msgla_decode_step` read
 * only the packed blob.  Returns 0 for an invalid config.
 */
size_t msgla_packed_weights_bytes(const msgla_config* cfg);

/* Packs `w` (device pointers, layout above) into `packed` (device,
 * >= msgla_packed_weights_bytes bytes) on `stream`.  `w` is read during the
 * call's execution on the stream; the struct itself is copied at call time. */
msgla_status msgla_pack_weights(const msgla_config* cfg, const msgla_weights* w, void* packed,
                                size_t packed_bytes, void* stream);

/* Device workspace needed by msgla_forward for batch B and length L (bytes). */
size_t msgla_workspace_bytes(const msgla_config* cfg, int64_t B, int64_t L);

/*
 * Streaming state ("cache" of the notes' paragraph on token-by-token
 * inference): per branch the fp32 GLA state S [B][h][d_k][d_v], the fp32 sum
 * of the tokens of the not-yet-complete pooling block [B][d] and their count
 * [B] (the block's positions, unless a masked forward left padding in it),
 * and the fp32 held output (the branch's latest coarse output after W_o)
 * [B][d], plus the number of positions consumed so far.  Opaque, versioned
 * blob; its recurrent part is sum_s h_s d_k d_v fp32 elements per sequence.
 */
size_t msgla_state_bytes(const msgla_config* cfg, int64_t B);

/* Writes an empty state (position 0, zero state, empty blocks, zero held
 * outputs) into `state` (device, >= msgla_state_bytes). */
msgla_status msgla_state_init(const msgla_config* cfg, int64_t B, void* state, size_t state_bytes,
                              void* stream);

/*
 * Layer forward over a batch of B sequences of L tokens from an empty state.
 *   x [B][L][d] (dtype) -> out [B][L][d] (dtype).
 *   mask: NULL (every position is a token), or a device array [B][L] of
 *         bytes, nonzero for a token and 0 for padding.  It enters the pooling
 *         only (Eq. (8)): every branch pools each complete block as
 *         sum M x / max(1, sum M), so at scale 1 a padded position is a zero
 *         input (the recurrence still decays its state there) and a block
 *         without tokens pools to zero; the fusion weights still come from the
 *         unpooled x_t.  A masked call may continue from state_in and
 *         export state_out: the incomplete block it leaves keeps the sum and
 *         the count of its tokens, and the decode steps that complete it pool
 *         it as sum / max(1, tokens).
 *   state_in: NULL (start from an empty state), or a state of the same
 *         config and B (written by msgla_forward's state_out,
 *         msgla_state_init or msgla_decode_step) to continue from, at any
 *         position: its GLA states seed the recurrences, each branch's block
 *         in progress (r = position mod s positions, kept as their sum and
 *         token count) is completed by the first s - r positions of this
 *         call, and its held outputs fill the positions before each coarse
 *         branch's first completed block.  The result equals one forward
 *         over the concatenated tokens.  Its header is checked on the
 *         device, in stream order (the call does not synchronise and can be
 *         captured in a graph): when it does not describe this config and B
 *         or records an error, nothing past the header is read, every
 *         element of out is NaN, and state_out (if given) records the error
 *         (MSGLA_ERR_INVALID_ARG) with position -1; msgla_state_query reads
 *         it.  The call itself then still returns MSGLA_OK.  state_in may
 *         equal state_out.
 *   state_out: NULL, or a buffer of msgla_state_bytes(cfg, B) that receives
 *         the streaming state after the L tokens (for msgla_decode_step).
 *   workspace: >= msgla_workspace_bytes(cfg, B, L) bytes of device memory;
 *         its contents on entry are irrelevant.
 * L may be any value >= 1; branches with s > L contribute zero.
 */
msgla_status msgla_forward(const msgla_config* cfg, const void* packed, const void* x,
                           const uint8_t* mask, int64_t B, int64_t L, void* out,
                           const void* state_in, void* state_out, void* workspace,
                           size_t workspace_bytes, void* stream);

/*
 * Optional per-stage timing: hipEvent_t handles recorded on `stream`
 * immediately before (start[i]) and after (stop[i]) stage i of the forward:
 * 0 = pooling prepass (block means of the coarse scales; empty when every
 * branch has scale 1), 1 = projection GEMM, 2 = chunk-local
 * gate/decay/intra-chunk kernel, 3 = chunk-state recurrence kernel,
 * 4 = output projections of the coarse branches (empty without one),
 * 5 = scale-1 output projection + causal hold + fusion.  NULL entries are
 * skipped.  Events are recorded, never waited on.
 */
#define MSGLA_N_STAGES 6
typedef struct {
  void* start[MSGLA_N_STAGES];
  void* stop[MSGLA_N_STAGES];
} msgla_stage_events;

/* msgla_forward with optional stage events (NULL = none). */
msgla_status msgla_forward_timed(const msgla_config* cfg, const void* packed, const void* x,
                                 const uint8_t* mask, int64_t B, int64_t L, void* out,
                                 const void* state_in, void* state_out, void* workspace,
                                 size_t workspace_bytes, void* stream,
                                 const msgla_stage_events* events);

/*
 * Fusion weights alone (Eq. (10)): w_t = softmax(x_t W_f + b_f) for every
 * position, the quantity whose means over the first, middle and last tenth of
 * long sequences the notes use to judge routing stability (Sec. 5.4, Table 3).
 *   x [B][L][d] (dtype) -> w_out [B][L][8] fp32 (device, 16-byte aligned),
 *   row t holding w_t in its first m = n_branches entries and zeros after.
 * Same arithmetic as the weights msgla_forward applies.  Needs no workspace.
 * n_branches must be at least 2 (MSGLA_ERR_INVALID_ARG otherwise: one branch
 * has weight 1).
 */
msgla_status msgla_fusion_weights(const msgla_config* cfg, const void* packed, const void* x,
                                  int64_t B, int64_t L, float* w_out, void* stream);

/*
 * What a state's header records (msgla_state_query).  status is MSGLA_OK for
 * a usable state, else the error of the forward that wrote it (a state_in it
 * could not continue from; position is then -1).
 */
typedef struct {
  int32_t status;   /* msgla_status */
  int32_t B;        /* batch the state was written for */
  int32_t m;        /* branches */
  int64_t position; /* tokens consumed, or -1 */
} msgla_state_info;

/*
 * Reads the header of `state` (device) after the work already enqueued on
 * `stream`: this call waits for that work (the only call that synchronises).
 * Returns MSGLA_ERR_INVALID_ARG if `state` does not hold a state header.
 */
msgla_status msgla_state_query(const void* state, msgla_state_info* info, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the layer
 * forward of msgla_forward (same arguments and results, without the
 * workspace), its workspace being a device array of
 * MSGLA_NOALLOC_WORKSPACE_BYTES that the library holds on every GPU it runs on
 * until the process ends.  The call allocates nothing.  A call whose
 * msgla_workspace_bytes(cfg, B, L) exceeds that size returns
 * MSGLA_ERR_WORKSPACE and enqueues nothing (192 MiB holds the B = 8,
 * L = 2048 and B = 1, L = 16384 workloads at d = 1024).  Every call on one
 * GPU uses that GPU's one array: calls that overlap on one GPU (several
 * streams or threads) race, and the caller must serialise them.  The first
 * call on a device looks the array's address up (no allocation).
 */
#define MSGLA_NOALLOC_WORKSPACE_BYTES (192u << 20)
msgla_status msgla_forward_noalloc(const msgla_config* cfg, const void* packed, const void* x,
                                   const uint8_t* mask, int64_t B, int64_t L, void* out,
                                   const void* state_in, void* state_out, void* stream);

/* Device workspace needed by msgla_decode_step for batch B (bytes). */
size_t msgla_decode_workspace_bytes(const msgla_config* cfg, int64_t B);

/*
 * One streaming step for B sequences (the notes' per-branch cache): every
 * branch adds x_t to its pending block; a branch whose block completes (s
 * positions) pools it (sum of its tokens over their count, Eq. (8)), takes
 * one recurrence step and replaces its held output;
 * the others keep theirs; the held outputs are fused with weights from the
 * unpooled x_t.  The result equals msgla_forward's output at the same
 * position (up to rounding).
 *   x_t [B][d] (dtype) -> out_t [B][d] (dtype); state: in/out (device,
 *   produced by msgla_state_init or msgla_forward's state_out with the same B).
 *   The state's header is checked on the device: a state of another config
 *   or B, or one that records an error, is left unchanged and out_t is NaN.
 */
msgla_status msgla_decode_step(const msgla_config* cfg, const void* packed, const void* x_t,
                               int64_t B, void* state, void* out_t, void* workspace,
                               size_t workspace_bytes, void* stream);

/*
 * Layer backward, for training.  The notes train every branch with GLA's
 * chunkwise-parallel algorithm (Sec. 3.4, training paragraph) and compare
 * training throughput with single-scale GLA (Sec. 5.5, Table 4); what training
 * needs from the layer is its vector-Jacobian product.  For the forward of x
 * from a fresh state (what msgla_forward computes with state_in NULL and the
 * same mask: NULL, or the [B][L] token mask of Eq. (8), which enters the
 * pooling only), given dout = dLoss/dO, msgla_backward writes dx = dLoss/dx
 * and the gradient of the loss with respect to every weight.
 *
 * Gradients are fp32, laid out as the weights of msgla_weights are, [in][out]
 * row-major, and are overwritten (not accumulated):
 *   per branch  W_q, W_k [d][h d_k]  W_v [d][h d_v]  W_g1 [d][r]
 *               W_g2 [r][h d_k]  b_g [h d_k]  W_o [h d_v][d]
 *   fusion      W_f [d][m], b_f [m]   (ignored, may be NULL, when m == 1)
 * x, dout, dx: [B][L][d] in the config's storage type.  The call recomputes
 * the forward's intermediates itself (it needs no saved activations), keeps
 * every intermediate gradient of the recurrence in fp32, and rounds the
 * operands of its large products (the weight and input gradients) to the
 * storage type, accumulating in fp32.  Everything runs in the library's
 * kernels (the hold and fusion, the chunkwise recurrence, the gate, the
 * pooling, and the plain products as grouped GEMMs), except the weight
 * gradients of fp32 configurations, which run on rocBLAS.
 * With the per-branch normalisation (config norm = 1) the gains' gradient is
 * written too (norm_g required).  d_v must be a multiple of 64
 * (MSGLA_ERR_UNSUPPORTED otherwise: fp32 configurations with d_v 32 or 96).
 * Pointers are device memory, 16-byte aligned.
 * Asynchronous on `stream`.  For fp32 configurations the library's rocBLAS
 * handle for the device is created on the first call (not under graph
 * capture), and such calls from several host threads are serialised by the
 * library.
 */
typedef struct {
  float* W_q;
  float* W_k;
  float* W_v;
  float* W_g1;
  float* W_g2;
  float* b_g;
  float* W_o;
  float* norm_g; /* [h d_v] gradient of the normalisation gains (config norm = 1), else unused */
} msgla_branch_grads;

typedef struct {
  msgla_branch_grads br[MSGLA_MAX_BRANCHES];
  float* W_f;
  float* b_f;
} msgla_grads;

/* Device workspace needed by msgla_backward for batch B and length L (bytes);
 * 0 for an invalid configuration or size, or one msgla_backward does not
 * support. */
size_t msgla_backward_workspace_bytes(const msgla_config* cfg, int64_t B, int64_t L);

msgla_status msgla_backward(const msgla_config* cfg, const void* packed, const void* x,
                            const void* dout, const uint8_t* mask, int64_t B, int64_t L,
                            void* dx, const msgla_grads* grads, void* workspace,
                            size_t workspace_bytes, void* stream);

/*
 * A training step without the backward's recompute (Sec. 3.4, training
 * paragraph; Sec. 5.5, Table 4): the forward's intermediates are kept from the
 * step's own forward instead of being computed twice.
 *
 * msgla_forward_train computes what msgla_forward computes from a fresh state
 * (out [B][L][d], the same values: the same launches), in a workspace of at
 * least msgla_backward_workspace_bytes(cfg, B, L) bytes, where it leaves every
 * intermediate the backward reads.  msgla_backward_saved then takes the same
 * arguments as msgla_backward and returns the same gradients (bit for bit),
 * reading those intermediates instead of recomputing them.  The caller keeps
 * the contract of such a saved workspace: the same cfg, packed weights, x,
 * mask, B and L in both calls, and the workspace unchanged in between; a
 * mismatch is not detected and gives wrong gradients.  msgla_backward_saved
 * leaves the saved intermediates unchanged, so several backward calls (other
 * dout) may follow one training forward.  Errors as msgla_backward; both are
 * asynchronous on `stream`.
 */
msgla_status msgla_forward_train(const msgla_config* cfg, const void* packed, const void* x,
                                 const uint8_t* mask, int64_t B, int64_t L, void* out,
                                 void* workspace, size_t workspace_bytes, void* stream);

msgla_status msgla_backward_saved(const msgla_config* cfg, const void* packed, const void* x,
                                  const void* dout, const uint8_t* mask, int64_t B, int64_t L,
                                  void* dx, const msgla_grads* grads, void* workspace,
                                  size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MSGLA_H */
