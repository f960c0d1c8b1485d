// Host-side exercise of the C ABI for a build whose host code carries
// AddressSanitizer and UndefinedBehaviorSanitizer: validation and every size
// query over a grid of valid and invalid configurations and batch shapes
// (including the largest accepted and the first rejected ones), and the
// argument-error paths of every entry point that take data pointers.  No call
// here reaches the GPU: each returns before its first HIP call.  Exit status
// 0 means every expectation held and no sanitizer reported anything.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "msgla.h"

static int failures = 0;
#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      std::fprintf(stderr, "expectation failed at line %d: %s\n", __LINE__, #cond); \
      ++failures;                                                      \
    }                                                                  \
  } while (0)

static msgla_config make(int nb, const int* sc, const int* hd, int d, int dk, int dv, int r, int C,
                         float gamma, int dtype, int norm) {
  msgla_config c;
  std::memset(&c, 0, sizeof(c));
  c.n_branches = nb;
  for (int i = 0; sc && hd && i < nb && i < MSGLA_MAX_BRANCHES; ++i) {
    c.scale[i] = sc[i];
    c.heads[i] = hd[i];
  }
  c.d_model = d;
  c.d_k = dk;
  c.d_v = dv;
  c.gate_rank = r;
  c.chunk = C;
  c.gate_normalizer = gamma;
  c.q_scale = 1.f;
  c.dtype = dtype;
  c.norm = norm;
  return c;
}

// every size query on one configuration: consistent with its validation
static void sizes(const msgla_config& c) {
  const msgla_status v = msgla_validate_config(&c);
  const size_t pw = msgla_packed_weights_bytes(&c);
  EXPECT((v == MSGLA_OK) == (pw > 0));
  const int64_t Bs[] = {-1, 0, 1, 3, 16, 1 << 20, (1 << 20) + 1};
  const int64_t Ls[] = {-5, 0, 1, 7, 64, 2049, 1 << 24, (1 << 24) + 1, INT64_MAX};
  for (int64_t B : Bs) {
    const size_t st = msgla_state_bytes(&c, B);
    const size_t dw = msgla_decode_workspace_bytes(&c, B);
    if (v != MSGLA_OK || B < 1) {
      EXPECT(st == 0);
      EXPECT(dw == 0);
    }
    for (int64_t L : Ls) {
      const size_t ws = msgla_workspace_bytes(&c, B, L);
      if (v != MSGLA_OK || B < 1 || L < 1) EXPECT(ws == 0);
      // accepted shapes: the workspace at least holds the fp32 q and k rows
      if (ws > 0) EXPECT(ws >= (size_t)B * (size_t)L / 4);
      // the backward's workspace holds at least its fusion-logit gradients (8 fp32 per position)
      const size_t bw = msgla_backward_workspace_bytes(&c, B, L);
      if (ws == 0) EXPECT(bw == 0);
      if (bw > 0) EXPECT(bw >= (size_t)B * (size_t)L * 32);
    }
  }
}

int main() {
  // a grid of configurations, valid and invalid
  const int dks[] = {8, 16, 32, 48, 64, 128, 256, 512};
  const int dvs[] = {16, 32, 64, 96, 128, 256, 512, 576};
  const int Cs[] = {8, 16, 32, 48, 64, 128};
  const int ds[] = {32, 64, 96, 1024, 65536, 65600};
  const int rs[] = {0, 1, 16, 17, 64, 65};
  int n = 0;
  for (int dtype = 0; dtype < 2; ++dtype)
    for (int dk : dks)
      for (int dv : dvs)
        for (int C : Cs) {
          const int sc[3] = {1, 2, 4}, hd[3] = {2, 1, 1};
          sizes(make(3, sc, hd, 1024, dk, dv, 16, C, 16.f, dtype, 0));
          ++n;
        }
  for (int d : ds)
    for (int r : rs)
      for (int norm = -1; norm < 3; ++norm) {
        const int sc[4] = {1, 2, 4, 8}, hd[4] = {1, 1, 1, 1};
        sizes(make(4, sc, hd, d, 128, 256, r, 64, 16.f, 1, norm));
        ++n;
      }
  {
    // branch sets: 0, 1 and 8 branches, 9 (too many), duplicate and bad scales / heads
    const int sc8[8] = {1, 2, 3, 4, 5, 6, 7, 8}, hd8[8] = {1, 1, 1, 1, 1, 1, 1, 1};
    for (int nb = -1; nb <= 8; ++nb) sizes(make(nb, sc8, hd8, 256, 64, 64, 16, 32, 16.f, 1, 0));
    msgla_config c9 = make(8, sc8, hd8, 256, 64, 64, 16, 32, 16.f, 1, 0);
    c9.n_branches = 9;
    sizes(c9);
    const int dup[2] = {2, 2}, zero[2] = {0, 2}, neg[2] = {-4, 2}, h1[2] = {1, 1}, h0[2] = {1, 0},
              hbig[2] = {1, 65}, big[2] = {1, 1 << 30};
    sizes(make(2, dup, h1, 256, 64, 64, 16, 32, 16.f, 1, 0));
    sizes(make(2, zero, h1, 256, 64, 64, 16, 32, 16.f, 1, 0));
    sizes(make(2, neg, h1, 256, 64, 64, 16, 32, 16.f, 1, 0));
    sizes(make(2, big, h1, 256, 64, 64, 16, 32, 16.f, 1, 0));
    const int s2[2] = {1, 2};
    sizes(make(2, s2, h0, 256, 64, 64, 16, 32, 16.f, 1, 0));
    sizes(make(2, s2, hbig, 256, 64, 64, 16, 32, 16.f, 1, 0));
    // gate normaliser: zero, negative, NaN; q_scale NaN; unknown dtype
    sizes(make(2, s2, h1, 256, 64, 64, 16, 32, 0.f, 1, 0));
    sizes(make(2, s2, h1, 256, 64, 64, 16, 32, -1.f, 1, 0));
    sizes(make(2, s2, h1, 256, 64, 64, 16, 32, __builtin_nanf(""), 1, 0));
    msgla_config cq = make(2, s2, h1, 256, 64, 64, 16, 32, 16.f, 1, 0);
    cq.q_scale = __builtin_nanf("");
    sizes(cq);
    sizes(make(2, s2, h1, 256, 64, 64, 16, 32, 16.f, 7, 0));
    n += 20;
  }
  sizes(make(1, nullptr, nullptr, 0, 0, 0, 0, 0, 0.f, 0, 0));
  EXPECT(msgla_validate_config(nullptr) != MSGLA_OK);
  EXPECT(msgla_packed_weights_bytes(nullptr) == 0);
  EXPECT(msgla_workspace_bytes(nullptr, 1, 1) == 0);
  EXPECT(msgla_state_bytes(nullptr, 1) == 0);
  EXPECT(msgla_decode_workspace_bytes(nullptr, 1) == 0);

  // argument errors of the data entry points, with fake aligned addresses
  // that are never dereferenced
  const int sc[3] = {1, 2, 4}, hd[3] = {2, 1, 1};
  const msgla_config c = make(3, sc, hd, 128, 32, 64, 16, 64, 16.f, 1, 0);
  EXPECT(msgla_validate_config(&c) == MSGLA_OK);
  char* f = reinterpret_cast<char*>(uintptr_t(1) << 20);
  const size_t ws = msgla_workspace_bytes(&c, 2, 64);
  const size_t st = msgla_state_bytes(&c, 2);
  const size_t dws = msgla_decode_workspace_bytes(&c, 2);
  EXPECT(msgla_forward(&c, f, nullptr, nullptr, 2, 64, f, nullptr, nullptr, f, ws, nullptr) == MSGLA_ERR_INVALID_ARG);
  EXPECT(msgla_forward(&c, f, f + 2, nullptr, 2, 64, f, nullptr, nullptr, f, ws, nullptr) == MSGLA_ERR_INVALID_ARG);
  EXPECT(msgla_forward(&c, f, f, nullptr, 0, 64, f, nullptr, nullptr, f, ws, nullptr) == MSGLA_ERR_INVALID_ARG);
  EXPECT(msgla_forward(&c, f, f, nullptr, 2, -3, f, nullptr, nullptr, f, ws, nullptr) == MSGLA_ERR_INVALID_ARG);
  EXPECT(msgla_forward(&c, f, f, nullptr, INT64_MAX, INT64_MAX, f, nullptr, nullptr, f, ws, nullptr) ==
         MSGLA_ERR_INVALID_ARG);
  EXPECT(msgla_forward(&c, f, f, nullptr, 2, 64, f, f + 8, nullptr, f, ws, nullptr) == MSGLA_ERR_INVALID_ARG);
  EXPECT(msgla_forward(&c, f, f, nullptr, 2, 64, f, nullptr, f + 4, f, ws, nullptr) == MSGLA_ERR_INVALID_ARG);
  EXPECT(msgla_forward(&c, f, f, nullptr, 2, 64, f, nullptr, nullptr, nullptr, ws, nullptr) != MSGLA_OK);
  EXPECT(msgla_forward(&c, f, f, nullptr, 2, 64, f, nullptr, nullptr, f, ws - 1, nullptr) == MSGLA_ERR_WORKSPACE);
  EXPECT(msgla_forward(nullptr, f, f, nullptr, 2, 64, f, nullptr, nullptr, f, ws, nullptr) != MSGLA_OK);
  EXPECT(msgla_forward_timed(&c, f, f, nullptr, 2, 64, f, nullptr, nullptr, f, ws - 1, nullptr, nullptr) ==
         MSGLA_ERR_WORKSPACE);
  EXPECT(msgla_forward_noalloc(&c, f, nullptr, nullptr, 2, 64, f, nullptr, nullptr, nullptr) != MSGLA_OK);
  EXPECT(msgla_forward_noalloc(&c, f, f, nullptr, 1 << 20, 1 << 8, f, nullptr, nullptr, nullptr) ==
         MSGLA_ERR_WORKSPACE);
  EXPECT(msgla_decode_step(&c, f, nullptr, 2, f, f, f, dws, nullptr) == MSGLA_ERR_INVALID_ARG);
  EXPECT(msgla_decode_step(&c, f, f, 0, f, f, f, dws, nullptr) == MSGLA_ERR_INVALID_ARG);
  EXPECT(msgla_decode_step(&c, f, f, 2, f, f, f, dws - 1, nullptr) == MSGLA_ERR_WORKSPACE);
  EXPECT(msgla_decode_step(&c, f, f, 2, f + 4, f, f, dws, nullptr) == MSGLA_ERR_INVALID_ARG);
  EXPECT(msgla_state_init(&c, 2, f, st - 1, nullptr) == MSGLA_ERR_WORKSPACE);
  EXPECT(msgla_state_init(&c, 2, nullptr, st, nullptr) == MSGLA_ERR_INVALID_ARG);
  EXPECT(msgla_state_init(&c, 0, f, st, nullptr) != MSGLA_OK);
  EXPECT(msgla_fusion_weights(&c, f, f, 2, 64, nullptr, nullptr) == MSGLA_ERR_INVALID_ARG);
  EXPECT(msgla_fusion_weights(&c, f, f, 0, 64, reinterpret_cast<float*>(f), nullptr) == MSGLA_ERR_INVALID_ARG);
  msgla_weights w;
  std::memset(&w, 0, sizeof(w));
  EXPECT(msgla_pack_weights(&c, &w, f, msgla_packed_weights_bytes(&c), nullptr) == MSGLA_ERR_INVALID_ARG);
  EXPECT(msgla_pack_weights(&c, nullptr, f, msgla_packed_weights_bytes(&c), nullptr) == MSGLA_ERR_INVALID_ARG);
  EXPECT(msgla_pack_weights(&c, &w, f, msgla_packed_weights_bytes(&c) - 1, nullptr) != MSGLA_OK);
  msgla_state_info info;
  EXPECT(msgla_state_query(nullptr, &info, nullptr) == MSGLA_ERR_INVALID_ARG);
  EXPECT(msgla_state_query(f + 8, &info, nullptr) == MSGLA_ERR_INVALID_ARG);
  EXPECT(msgla_state_query(f, nullptr, nullptr) == MSGLA_ERR_INVALID_ARG);
  for (int s = -1; s < 7; ++s) EXPECT(msgla_status_str((msgla_status)s) != nullptr);
  // backward argument errors
  {
    const size_t bws = msgla_backward_workspace_bytes(&c, 2, 64);
    EXPECT(bws > ws);
    msgla_grads gr;
    std::memset(&gr, 0, sizeof(gr));
    for (int i = 0; i < c.n_branches; ++i) {
      float* p = reinterpret_cast<float*>(f);
      gr.br[i] = msgla_branch_grads{p, p, p, p, p, p, p};
    }
    gr.W_f = gr.b_f = reinterpret_cast<float*>(f);
    EXPECT(msgla_backward(&c, f, f, nullptr, nullptr, 2, 64, f, &gr, f, bws, nullptr) == MSGLA_ERR_INVALID_ARG);
    EXPECT(msgla_backward(&c, f, f, f, nullptr, 2, 64, f + 4, &gr, f, bws, nullptr) == MSGLA_ERR_INVALID_ARG);
    EXPECT(msgla_backward(&c, f, f, f, nullptr, 2, 64, f, nullptr, f, bws, nullptr) == MSGLA_ERR_INVALID_ARG);
    EXPECT(msgla_backward(&c, f, f, f, nullptr, INT64_MAX, 64, f, &gr, f, bws, nullptr) == MSGLA_ERR_INVALID_ARG);
    EXPECT(msgla_backward(&c, f, f, f, nullptr, 2, 64, f, &gr, f, bws - 1, nullptr) == MSGLA_ERR_WORKSPACE);
    EXPECT(msgla_backward(nullptr, f, f, f, nullptr, 2, 64, f, &gr, f, bws, nullptr) != MSGLA_OK);
    gr.br[2].W_g2 = nullptr;
    EXPECT(msgla_backward(&c, f, f, f, nullptr, 2, 64, f, &gr, f, bws, nullptr) == MSGLA_ERR_INVALID_ARG);
    gr.br[2].W_g2 = reinterpret_cast<float*>(f);
    msgla_config cn = c;
    cn.norm = 1;
    const size_t bwn = msgla_backward_workspace_bytes(&cn, 2, 64);
    EXPECT(bwn > bws);
    EXPECT(msgla_backward(&cn, f, f, f, nullptr, 2, 64, f, &gr, f, bwn, nullptr) == MSGLA_ERR_INVALID_ARG);
    // the training pair: the forward needs the backward's workspace, the saved backward
    // validates as the backward does
    EXPECT(msgla_forward_train(&c, f, f, nullptr, 2, 64, nullptr, f, bws, nullptr) == MSGLA_ERR_INVALID_ARG);
    EXPECT(msgla_forward_train(&c, f, f, nullptr, 2, 64, f, f, ws, nullptr) == MSGLA_ERR_WORKSPACE);
    EXPECT(msgla_forward_train(&c, f, f + 4, nullptr, 2, 64, f, f, bws, nullptr) == MSGLA_ERR_INVALID_ARG);
    EXPECT(msgla_backward_saved(&c, f, f, nullptr, nullptr, 2, 64, f, &gr, f, bws, nullptr) == MSGLA_ERR_INVALID_ARG);
    EXPECT(msgla_backward_saved(&c, f, f, f, nullptr, 2, 64, f, &gr, f, bws - 1, nullptr) == MSGLA_ERR_WORKSPACE);
  }

  std::printf("configurations %d, failures %d\n", n, failures);
  return failures == 0 ? 0 : 1;
}
