// Host-side argument checks of the C ABI, built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code (tests/test_host_sanitizers.py).
// No GPU is needed: every call below fails validation, or only sizes a
// workspace, before any HIP call.  Exits 0 when every return code is the
// documented one; a sanitizer report aborts with a nonzero status.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <vector>

#include "llama_mi355x.h"

static int g_failures = 0;

#define EXPECT(cond)                                                  \
  do {                                                                \
    if (!(cond)) {                                                    \
      fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond); \
      ++g_failures;                                                   \
    }                                                                 \
  } while (0)

static llama_args args8b(int max_batch, int max_seq) {
  llama_args a;
  memset(&a, 0, sizeof a);
  a.dim = 4096; a.n_layers = 2; a.n_heads = 32; a.n_kv_heads = 8; a.vocab_size = 128256;
  a.multiple_of = 1024; a.ffn_dim_multiplier = 1.3f; a.norm_eps = 1e-5f; a.rope_theta = 500000.f;
  a.max_batch_size = max_batch; a.max_seq_len = max_seq; a.dtype = LLAMA_BF16;
  return a;
}

static llama_args args_small() {
  llama_args a;
  memset(&a, 0, sizeof a);
  a.dim = 512; a.n_layers = 2; a.n_heads = 8; a.n_kv_heads = 4; a.vocab_size = 68;
  a.multiple_of = 256; a.ffn_dim_multiplier = -1.f; a.norm_eps = 1e-5f; a.rope_theta = 500000.f;
  a.max_batch_size = 4; a.max_seq_len = 64; a.dtype = LLAMA_BF16;
  return a;
}

static void expect_error(int rc, int code) {
  EXPECT(rc == code);
  EXPECT(strlen(llama_last_error()) > 0);
}

int main() {
  void *fake = reinterpret_cast<void *>(0x1000);  // never dereferenced: validation returns first
  const size_t huge = (size_t)1 << 40;

  // model validation over a grid of shapes (divisibility, head sizes, overflow)
  const int dims[] = {0, 64, 500, 512, 640, 768, 4096, 8192, 16384};
  const int heads[] = {0, 1, 3, 4, 8, 32, 64};
  for (int D : dims)
    for (int H : heads)
      for (int G : heads) {
        llama_args a = args_small();
        a.dim = D; a.n_heads = H; a.n_kv_heads = G;
        const size_t n = llama_workspace_bytes(&a, 2, 16);
        const int32_t f = llama_ffn_hidden_dim(&a);
        if (D > 0) EXPECT(f > 0);
        const bool ok = D > 0 && H > 0 && G > 0 && D % H == 0 && H % G == 0 && ((D / H) == 64 || (D / H) == 96 ||
                        (D / H) == 128) && D % 64 == 0 && D <= 8192 && (H / G) <= 16 && ((H / G) & (H / G - 1)) == 0;
        EXPECT((n > 0) == ok);
      }
  {
    llama_args a = args_small();
    a.multiple_of = 0;
    EXPECT(llama_ffn_hidden_dim(&a) == LLAMA_ERR_ARG);
    a = args_small();
    a.dim = 0x7fffff00; a.ffn_dim_multiplier = 1e30f;
    EXPECT(llama_ffn_hidden_dim(&a) == LLAMA_ERR_ARG);  // overflows int32
    EXPECT(llama_ffn_hidden_dim(nullptr) == LLAMA_ERR_ARG);
    a = args_small();
    a.dtype = (llama_dtype)7;
    EXPECT(llama_workspace_bytes(&a, 1, 1) == 0);
  }

  // workspace sizes grow with tokens and batch; generation workspace covers decode
  {
    llama_args a = args8b(64, 4224);
    const size_t p1 = llama_workspace_bytes(&a, 1, 8192), p2 = llama_workspace_bytes(&a, 1, 16384);
    EXPECT(p1 > 0 && p2 > p1);
    EXPECT(llama_workspace_bytes(&a, 64, 1) > 0);
    EXPECT(llama_generate_workspace_bytes(&a, 64, 160) >= llama_workspace_bytes(&a, 64, 1));
    EXPECT(llama_generate_workspace_bytes(&a, 65, 160) == 0);
    EXPECT(llama_workspace_bytes(&a, 0, 8) == 0 && llama_workspace_bytes(&a, 1, 0) == 0);
  }

  llama_args a = args_small();
  llama_layer_w lw;
  void **lp = reinterpret_cast<void **>(&lw);
  for (size_t i = 0; i < sizeof lw / sizeof(void *); ++i) lp[i] = fake;
  std::vector<llama_layer_w> layers(2, lw);
  llama_model_w model = {fake, layers.data(), fake, fake};
  llama_kv kvs[2] = {{fake, fake}, {fake, fake}};
  const float *xf = static_cast<const float *>(fake);
  float *yf = static_cast<float *>(fake);
  const int32_t *ids = static_cast<const int32_t *>(fake);
  int32_t *out = static_cast<int32_t *>(fake);

  // layer forward
  expect_error(llama_layer_forward(&a, &lw, nullptr, yf, 1, 8, 0, nullptr, fake, huge, nullptr), LLAMA_ERR_ARG);
  expect_error(llama_layer_forward(&a, &lw, xf, yf, 1, 8, 3, nullptr, fake, huge, nullptr), LLAMA_ERR_ARG);
  expect_error(llama_layer_forward(&a, &lw, xf, yf, 5, 8, 0, kvs, fake, huge, nullptr), LLAMA_ERR_SHAPE);
  expect_error(llama_layer_forward(&a, &lw, xf, yf, 1, 8, 60, kvs, fake, huge, nullptr), LLAMA_ERR_SHAPE);
  expect_error(llama_layer_forward(&a, &lw, xf, yf, 1, 8, 0, nullptr, fake, 64, nullptr), LLAMA_ERR_WORKSPACE);
  expect_error(llama_layer_forward(&a, &lw, xf, yf, 1, 8, 0x7fffffff, kvs, fake, huge, nullptr), LLAMA_ERR_SHAPE);
  {
    llama_layer_w bad = lw;
    bad.w2 = nullptr;
    expect_error(llama_layer_forward(&a, &bad, xf, yf, 1, 8, 0, nullptr, fake, huge, nullptr), LLAMA_ERR_ARG);
  }
  expect_error(llama_layer_forward_docs(&a, &lw, xf, yf, 0, 8, 0, nullptr, ids, fake, huge, nullptr), LLAMA_ERR_ARG);

  // prefill
  expect_error(llama_prefill(&a, &model, nullptr, 1, 8, nullptr, nullptr, nullptr, out, fake, huge, nullptr),
               LLAMA_ERR_ARG);
  expect_error(llama_prefill(&a, &model, ids, 5, 8, kvs, nullptr, nullptr, out, fake, huge, nullptr),
               LLAMA_ERR_SHAPE);
  expect_error(llama_prefill(&a, &model, ids, 1, 8, nullptr, nullptr, nullptr, out, fake, 16, nullptr),
               LLAMA_ERR_WORKSPACE);
  expect_error(llama_prefill_docs(&a, &model, ids, ids, 1, 0, nullptr, nullptr, nullptr, out, fake, huge, nullptr),
               LLAMA_ERR_ARG);
  {
    llama_model_w m2 = model;
    m2.layers = nullptr;
    expect_error(llama_prefill(&a, &m2, ids, 1, 8, nullptr, nullptr, nullptr, out, fake, huge, nullptr),
                 LLAMA_ERR_ARG);
  }

  // decode
  expect_error(llama_decode_step(&a, &model, ids, nullptr, 2, kvs, nullptr, out, fake, huge, nullptr), LLAMA_ERR_ARG);
  expect_error(llama_decode_step(&a, &model, ids, ids, 9, kvs, nullptr, out, fake, huge, nullptr), LLAMA_ERR_SHAPE);
  expect_error(llama_decode_step(&a, &model, ids, ids, 2, kvs, nullptr, out, fake, 64, nullptr), LLAMA_ERR_WORKSPACE);
  expect_error(llama_decode_step(&a, &model, ids, ids, 2, nullptr, nullptr, out, fake, huge, nullptr), LLAMA_ERR_ARG);
  expect_error(llama_decode_step_docs(&a, &model, ids, ids, ids, 0, kvs, nullptr, out, fake, huge, nullptr),
               LLAMA_ERR_ARG);
  expect_error(llama_decode_step_noalloc(&a, &model, ids, nullptr, 2, kvs, nullptr, out, nullptr), LLAMA_ERR_ARG);
  {
    llama_args big = args8b(64, 131072);
    llama_kv kv8[2] = {{fake, fake}, {fake, fake}};
    expect_error(llama_decode_step_noalloc(&big, &model, ids, ids, 64, kv8, nullptr, out, nullptr),
                 LLAMA_ERR_WORKSPACE);
    EXPECT(llama_decode_noalloc_max_bytes() == ((size_t)96 << 20));
  }

  // head, sampler, generation
  expect_error(lm_head_argmax(&a, xf, nullptr, fake, 0, nullptr, out, fake, huge, nullptr), LLAMA_ERR_ARG);
  expect_error(lm_head_argmax(&a, xf, nullptr, fake, 4, nullptr, out, fake, 8, nullptr), LLAMA_ERR_WORKSPACE);
  const float *lg = static_cast<const float *>(fake);
  expect_error(llama_sample_top_p(lg, 2, 100, 0.f, 0.9f, lg, out, nullptr), LLAMA_ERR_ARG);
  expect_error(llama_sample_top_p(lg, 2, 200000, 0.6f, 0.9f, lg, out, nullptr), LLAMA_ERR_UNSUPPORTED);
  {
    int32_t lens[4] = {3, 70, 2, 2};
    int32_t steps = -1;
    expect_error(llama_generate(&a, &model, ids, 80, lens, 4, 4, -1, 0.f, 0.9f, nullptr, kvs, out, out, 0, &steps,
                                fake, huge, nullptr),
                 LLAMA_ERR_ARG);  // prompt_len above max_seq_len
    lens[1] = 5;
    expect_error(llama_generate(&a, &model, ids, 4, lens, 4, 4, -1, 0.f, 0.9f, nullptr, kvs, out, out, 0, &steps,
                                fake, huge, nullptr),
                 LLAMA_ERR_ARG);  // stride shorter than a prompt
    expect_error(llama_generate(&a, &model, ids, 8, lens, 4, 4, -1, 0.5f, 0.9f, nullptr, kvs, out, out, 0, &steps,
                                fake, huge, nullptr),
                 LLAMA_ERR_ARG);  // sampling without uniforms
    expect_error(llama_generate(&a, &model, ids, 8, lens, 65, 4, -1, 0.f, 0.9f, nullptr, kvs, out, out, 0, &steps,
                                fake, huge, nullptr),
                 LLAMA_ERR_UNSUPPORTED);
    expect_error(llama_generate(&a, &model, ids, 8, lens, 4, 4, -1, 0.f, 0.9f, nullptr, kvs, out, out, 0, &steps,
                                fake, 32, nullptr),
                 LLAMA_ERR_WORKSPACE);
    EXPECT(steps == -1);
  }

  // timing record without a device: enabling and reporting an empty record
  EXPECT(llama_timing_enable(1) == LLAMA_OK);
  char buf[64];
  EXPECT(llama_timing_report(buf, sizeof buf) == 1 && buf[0] == 0);
  EXPECT(llama_timing_enable(0) == LLAMA_OK);

  if (g_failures) {
    fprintf(stderr, "%d expectation(s) failed\n", g_failures);
    return 1;
  }
  printf("host checks passed\n");
  return 0;
}
