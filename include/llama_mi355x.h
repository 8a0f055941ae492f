/*
 * llama_mi355x.h - C ABI of the MI355X (gfx950) Llama-3 decoder forward pass.
 *
 * The library computes the dense decoder-only forward pass described on the
 * pages cited below: RMSNorm, Q/K/V projections, rotary position embedding
 * (RoPE), causal grouped-query attention (GQA), output projection, SwiGLU
 * feed-forward, final RMSNorm, LM-head logits and argmax.
 *
 * Pages (cited by title and section):
 *   [P1] "机器学习 | 从0开发大模型—译llama3-from-scratch" (sunaigc.com translation
 *        of the llama3-from-scratch notebook)
 *   [P2] "Build your own Llama 3 architecture from scratch" notes (gitcode.csdn.net)
 *   [P3] "大语言模型实现llama3-from-scratch：输出层与预测" (agent.csdn.net)
 *   [P4] joto.ai blog post on the Llama architecture (GQA, RoPE, RMSNorm)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Ownership: the caller owns every buffer (weights, activations, KV cache,
 *   logits, ids, workspace).  Pointers marked "device" are HIP device
 *   pointers; the library allocates nothing and keeps no pointer after it
 *   returns.  All work is enqueued asynchronously on `stream` (a hipStream_t
 *   passed as void*; NULL is the null stream); outputs are valid once the
 *   stream has completed.  Nothing synchronises the host, except
 *   llama_generate, which waits on its stream to stop early.
 * Layouts: contiguous row-major, device pointers 16-byte aligned.  Linear
 *   weights are [out, in] as in nn.Linear [P2 3.4, 3.5; P1 6.2].  Head h of
 *   wq occupies rows [h*hd, (h+1)*hd) [P1 6.3]; wo's input columns are the
 *   heads concatenated in order [P1 8].
 * Number types: `dtype` (llama_args.dtype) is the storage type of weights,
 *   norm weights, embeddings and the KV cache: LLAMA_F32 or LLAMA_BF16.
 *   Hidden states passed in and out (the residual stream) are always fp32;
 *   logits are always fp32 [P2 4 `logits.float()`; P3 numerics]; token ids
 *   are int32.  bf16 contractions accumulate in fp32.
 * Errors: every entry point returns LLAMA_OK (0) or a negative llama_status.
 *   Arguments are validated before any HIP call; on error nothing has been
 *   enqueued and llama_last_error() describes the cause (thread-local).
 *   LLAMA_ERR_HIP reports a failed launch or runtime call; work enqueued
 *   before the failure may have run.  Token ids outside [0, vocab) are a
 *   caller error: their embedding rows are filled with NaN.
 */
#ifndef LLAMA_MI355X_H
#define LLAMA_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LLAMA_OK = 0,
  LLAMA_ERR_ARG = -1,         /* null pointer or invalid scalar argument */
  LLAMA_ERR_SHAPE = -2,       /* inconsistent shapes (see each function) */
  LLAMA_ERR_UNSUPPORTED = -3, /* a shape the kernels do not specialise */
  LLAMA_ERR_WORKSPACE = -4,   /* workspace smaller than llama_workspace_bytes() */
  LLAMA_ERR_HIP = -5          /* HIP launch or runtime failure */
} llama_status;

typedef enum { LLAMA_F32 = 0, LLAMA_BF16 = 1 } llama_dtype;

/* Model hyper-parameters; mirrors ModelArgs [P2 1.2] and params.json [P1 2].
 * ffn_dim_multiplier <= 0 encodes None.  max_batch_size / max_seq_len give
 * the KV-cache capacity [P2 3.3]. */
typedef struct {
  int32_t dim, n_layers, n_heads, n_kv_heads, vocab_size;
  int32_t multiple_of;
  float ffn_dim_multiplier;
  float norm_eps;
  float rope_theta;
  int32_t max_batch_size, max_seq_len;
  int32_t dtype; /* llama_dtype */
} llama_args;

/* One decoder layer's weights (device, dtype).  Names follow the checkpoint
 * keys [P1 2]: attention_norm [D], wq [H*hd, D], wk [G*hd, D], wv [G*hd, D],
 * wo [D, H*hd], ffn_norm [D], w1 [F, D], w2 [D, F], w3 [F, D]. */
typedef struct {
  const void *attention_norm, *wq, *wk, *wv, *wo, *ffn_norm, *w1, *w2, *w3;
} llama_layer_w;

/* Whole model: tok_embeddings [V, D], layers (HOST array of n_layers
 * llama_layer_w), norm [D], output [V, D]; tensors on the device. */
typedef struct {
  const void *tok_embeddings;
  const llama_layer_w *layers;
  const void *norm, *output;
} llama_model_w;

/* One layer's KV cache (device, dtype): k and v each
 * [max_batch_size][max_seq_len][n_kv_heads][head_dim].  Keys are stored
 * after RoPE [P2 3.3-3.4]. */
typedef struct {
  void *k, *v;
} llama_kv;

/* SwiGLU hidden size F [P2 3.5]: int(2*(4*dim)/3), times ffn_dim_multiplier
 * (truncated) when set, rounded up to a multiple of multiple_of.  Returns a
 * negative llama_status on invalid arguments. */
int32_t llama_ffn_hidden_dim(const llama_args *a);

/* Bytes of device workspace that llama_layer_forward and llama_prefill need
 * for (batch, seq_len) and that llama_decode_step and lm_head_argmax need
 * for `batch` rows.  Returns 0 on invalid arguments.  Pass the workspace as
 * `ws`, at least 256-byte aligned. */
size_t llama_workspace_bytes(const llama_args *a, int32_t batch, int32_t seq_len);

/* One pre-norm decoder block [P2 3.6; P1 6-10] on hidden states
 *   x[batch][seq_len][dim] (fp32, device) at positions start_pos + s:
 *     h1 = x  + wo( GQA( rope(q), rope(k), v ) ),  q,k,v = rmsnorm(x) W^T
 *     y  = h1 + w2( silu(w1 xn2) * w3 xn2 ),        xn2  = rmsnorm(h1)
 * y[batch][seq_len][dim] (fp32, device) may alias x.
 * kv (nullable): when given, the new keys/values are written to
 *   kv->k/v[b][start_pos + s] and queries attend to cache positions
 *   0..start_pos+s (chunked prefill); when NULL, start_pos must be 0 and
 *   attention runs over the chunk itself [P2 3.4 training branch].
 * Errors: ERR_ARG (null x/y/w/ws, start_pos < 0, start_pos > 0 without kv),
 *   ERR_SHAPE (dim % n_heads, n_heads % n_kv_heads, odd head_dim,
 *   batch > max_batch_size with kv, start_pos + seq_len > max_seq_len [P2 6
 *   assert]), ERR_UNSUPPORTED (head_dim not in {64, 96, 128}, dim or F not a
 *   multiple of 64, n_heads/n_kv_heads not a power of two <= 16),
 *   ERR_WORKSPACE. */
int llama_layer_forward(const llama_args *a, const llama_layer_w *w, const float *x, float *y,
                        int32_t batch, int32_t seq_len, int32_t start_pos, const llama_kv *kv,
                        void *ws, size_t ws_bytes, void *stream);

/* llama_layer_forward with the document-level attention mask [P2 appendix,
 * item 1 (document-level attention mask); P2 1 (the cross-document mask among
 * Llama 3's changes)]: when several documents are concatenated into one
 * sequence, a token attends only to earlier tokens of its own document.
 *   doc_ids [batch][start_pos + seq_len] int32 (device, nullable): a
 *     document id per position, cache positions included; a document is a
 *     maximal run of equal ids, so key j is visible to the query at position
 *     p iff j <= p and positions j..p all carry the same id.  RoPE positions
 *     stay the positions in the concatenated sequence.  NULL: plain causal
 *     mask (llama_layer_forward).
 * Errors: as llama_layer_forward. */
int llama_layer_forward_docs(const llama_args *a, const llama_layer_w *w, const float *x, float *y,
                             int32_t batch, int32_t seq_len, int32_t start_pos, const llama_kv *kv,
                             const int32_t *doc_ids, void *ws, size_t ws_bytes, void *stream);

/* Prefill of `batch` sequences of `seq_len` tokens from position 0
 * [P2 4 Transformer.forward; P1 4-12]: embedding lookup, n_layers blocks,
 * final RMSNorm of each sequence's last position, LM head, argmax.
 *   ids     [batch][seq_len] int32 (device)
 *   kv      nullable HOST array of n_layers llama_kv; when given the caches
 *           are filled at positions 0..seq_len-1
 *   hidden  nullable; receives the residual stream after the last layer,
 *           [batch][seq_len][dim] fp32 (device)
 *   logits  nullable; receives last-position logits [batch][vocab] fp32
 *   next_id [batch] int32 (device): argmax of each row of the logits, the
 *           smallest index on ties [P1 12; P3 4]
 * Errors: as llama_layer_forward, plus ERR_ARG for null ids/next_id. */
int llama_prefill(const llama_args *a, const llama_model_w *w, const int32_t *ids, int32_t batch,
                  int32_t seq_len, const llama_kv *kv, float *hidden, float *logits, int32_t *next_id,
                  void *ws, size_t ws_bytes, void *stream);

/* llama_prefill with the document-level attention mask (see
 * llama_layer_forward_docs): doc_ids [batch][seq_len] int32 (device,
 * nullable; NULL = llama_prefill).  Errors: as llama_prefill. */
int llama_prefill_docs(const llama_args *a, const llama_model_w *w, const int32_t *ids, const int32_t *doc_ids,
                       int32_t batch, int32_t seq_len, const llama_kv *kv, float *hidden, float *logits,
                       int32_t *next_id, void *ws, size_t ws_bytes, void *stream);

/* One decode step: one new token per sequence [P2 3.3, 6 generate].
 *   ids [batch] int32 (device): the new tokens
 *   pos [batch] int32 (device): each sequence's current cache length; the
 *       new key/value go to cache slot pos[b] and the token attends to
 *       positions 0..pos[b] [P2 3.4 inference branch].  Each pos[b] must lie
 *       in [0, max_seq_len); out-of-range entries are clamped by the kernels
 *       so no access leaves the cache.  The cache stores the new key/value
 *       in `dtype`; the token's own attention uses them unrounded (fp32).
 *   kv  HOST array of n_layers llama_kv (required)
 *   logits nullable [batch][vocab] fp32; next_id [batch] int32 (device).
 * Errors: ERR_ARG (null ids/pos/kv/next_id), ERR_SHAPE (batch >
 *   max_batch_size), ERR_UNSUPPORTED, ERR_WORKSPACE. */
int llama_decode_step(const llama_args *a, const llama_model_w *w, const int32_t *ids, const int32_t *pos,
                      int32_t batch, const llama_kv *kv, float *logits, int32_t *next_id, void *ws,
                      size_t ws_bytes, void *stream);

/* llama_decode_step with the document-level attention mask (see
 * llama_layer_forward_docs): the new token continues the document that
 * starts at cache position doc_start[b] and attends to positions
 * doc_start[b]..pos[b] only.
 *   doc_start [batch] int32 (device, nullable; NULL = llama_decode_step);
 *     values are clamped to [0, pos[b]].
 * Errors: as llama_decode_step. */
int llama_decode_step_docs(const llama_args *a, const llama_model_w *w, const int32_t *ids, const int32_t *pos,
                           const int32_t *doc_start, int32_t batch, const llama_kv *kv, float *logits,
                           int32_t *next_id, void *ws, size_t ws_bytes, void *stream);

/* llama_decode_step without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  It computes exactly what
 * llama_decode_step computes (same kernels, bit-identical outputs) and
 * allocates nothing: its scratch (the decode workspace) is a static device
 * array of llama_decode_noalloc_max_bytes() = 96 MiB inside the library,
 * one per GPU, held by every GPU the library runs on until the process ends.
 * The scratch of the current device is used (its address is looked up once
 * per device, on the first call there); `stream` must belong to that device.
 * Every call on a GPU shares that GPU's scratch and leaves its contents
 * behind: calls that overlap on one GPU (on different streams, or from
 * different threads without ordering) race and must not be issued.  Nothing
 * in the scratch needs to start at zero: every value the step reads is
 * written earlier in the same step.
 * Arguments: as llama_decode_step, minus ws/ws_bytes.
 * Errors: as llama_decode_step; ERR_WORKSPACE when the step needs more
 *   scratch than the static array holds (llama_workspace_bytes(a, batch, 1)
 *   gives the need; e.g. 8B shapes at 64 sequences fit up to a max_seq_len
 *   of about 11000); ERR_HIP when the scratch's address cannot be obtained. */
int llama_decode_step_noalloc(const llama_args *a, const llama_model_w *w, const int32_t *ids, const int32_t *pos,
                              int32_t batch, const llama_kv *kv, float *logits, int32_t *next_id, void *stream);

/* Size in bytes of the static scratch of llama_decode_step_noalloc. */
size_t llama_decode_noalloc_max_bytes(void);

/* Output head on M hidden rows [P1 11-12; P3 1-4]:
 *   h [M][dim] fp32 (device); final_norm_w (nullable, dtype) applies the
 *   final RMSNorm first; w_out [vocab][dim] (dtype).
 *   logits (nullable) [M][vocab] fp32; argmax [M] int32, smallest index on
 *   ties.  Errors: ERR_ARG (null h/w_out/argmax, M < 1), ERR_UNSUPPORTED
 *   (dim not a multiple of 64), ERR_WORKSPACE (needs
 *   llama_workspace_bytes(a, M, 1)). */
int lm_head_argmax(const llama_args *a, const float *h, const void *final_norm_w, const void *w_out, int32_t M,
                   float *logits, int32_t *argmax, void *ws, size_t ws_bytes, void *stream);

/* Temperature / top-p sampling of one token per row [P2 6 sample_top_p;
 * P3 temperature softmax]:
 *   p = softmax(logits[r] / temperature); the nucleus is the longest prefix
 *   of the tokens sorted by descending p (ties by ascending id) whose mass
 *   before each member is at most top_p; out_id[r] is drawn from the
 *   renormalised nucleus with u[r] in [0, 1) by inverse CDF over the kept
 *   tokens in ascending id order (the smallest id whose cumulative kept mass
 *   exceeds u[r] times the kept total).  top_p >= 1 keeps every token.
 *   Probabilities are carried as floor(2^40 z) with z computed in fp32, and
 *   every sum is exact, so the choice does not depend on summation order.
 *   logits [M][V] fp32 (device, finite), u [M] fp32 (device),
 *   out_id [M] int32 (device).
 * Errors: ERR_ARG (null pointers, M < 1, V < 1, temperature <= 0, top_p < 0
 *   or NaN), ERR_UNSUPPORTED (V > 131072). */
int llama_sample_top_p(const float *logits, int32_t M, int32_t V, float temperature, float top_p, const float *u,
                       int32_t *out_id, void *stream);

/* Workspace bytes llama_generate needs for `batch` sequences whose prompts
 * hold at most max_prompt_len tokens; 0 on invalid arguments. */
size_t llama_generate_workspace_bytes(const llama_args *a, int32_t batch, int32_t max_prompt_len);

#define LLAMA_GEN_GRAPH 2

/* Autoregressive generation [P2 6 generate; P3 4]: each sequence's prompt,
 * then one model choice per position.
 *   prompt      [batch][prompt_stride] int32 (device); sequence b's prompt
 *               is prompt[b][0, prompt_len[b])
 *   prompt_len  HOST [batch], 1 <= prompt_len[b] <= max_seq_len
 *   max_gen_len tokens to generate at most per sequence (>= 0); sequence b
 *               ends at total_b = min(prompt_len[b] + max_gen_len,
 *               max_seq_len) positions, or right after it produces eos_id
 *               (eos_id < 0: no end-of-text stop)
 *   temperature 0: greedy, the argmax with the smallest id on ties;
 *               > 0: llama_sample_top_p with top_p, drawing the g-th
 *               generated token of sequence b with uniforms[g][b]
 *   uniforms    [max_gen_len][batch] fp32 in [0, 1) (device); required when
 *               temperature > 0, else ignored
 *   kv          HOST array of n_layers llama_kv (caches of at least `batch`
 *               rows); rows [0, batch) are overwritten
 *   tokens      [batch][max_seq_len] int32 (device, out): the prompt and the
 *               generated tokens, -1 after each sequence's last position
 *   out_len     [batch] int32 (device, out): the number of tokens before the
 *               first eos_id in tokens[b] (the pages cut the output there),
 *               else the sequence's length
 *   flags       LLAMA_GEN_GRAPH: capture one step (decode, choice, state
 *               update) as a HIP graph and replay it, instead of launching
 *               its kernels one by one (needs a stream other than the null
 *               stream; on this stack the two measure alike at 8B shapes and
 *               the graph is slightly slower on small models).  A stream that
 *               is itself being captured is not supported.
 *   steps_run   HOST (nullable): decode steps run
 * The prompts are right-padded to the longest one and prefilled together
 * (at most 16384 tokens per call), each sequence's first token taken from its
 * own last prompt row; then every decode step advances all sequences at
 * once, each at its own position; a finished sequence keeps its position and
 * its output no longer changes.  The host waits on the stream every 8 steps and stops once
 * every sequence has finished.
 * Errors: ERR_ARG (null pointers, prompt_len out of range, max_gen_len < 0,
 *   temperature < 0, temperature > 0 without uniforms, prompt_stride <
 *   max prompt_len), ERR_SHAPE (batch > max_batch_size), ERR_UNSUPPORTED
 *   (batch > 64, vocab > 131072 when sampling), ERR_WORKSPACE, and the
 *   errors of llama_prefill / llama_decode_step. */
int llama_generate(const llama_args *a, const llama_model_w *w, const int32_t *prompt, int32_t prompt_stride,
                   const int32_t *prompt_len, int32_t batch, int32_t max_gen_len, int32_t eos_id, float temperature,
                   float top_p, const float *uniforms, const llama_kv *kv, int32_t *tokens, int32_t *out_len,
                   int32_t flags, int32_t *steps_run, void *ws, size_t ws_bytes, void *stream);

/* Message describing the last non-OK return on the calling thread. */
const char *llama_last_error(void);

/* Per-kernel timing for measurement.  llama_timing_enable(1) clears the
 * record and makes every later launch (from any entry point) record a HIP
 * event before and after it on its stream; llama_timing_enable(0) stops
 * recording.  llama_timing_report() waits for the recorded events, writes
 * one line "kernel_name launches total_ms" per kernel into buf (up to len
 * bytes, NUL-terminated, may be NULL), clears the record and returns the
 * bytes the full report needs (or a negative llama_status).  The events are
 * created on first use and reused; timing adds host work per launch, so
 * time whole steps with it off. */
int llama_timing_enable(int on);
int64_t llama_timing_report(char *buf, size_t len);

#ifdef __cplusplus
}
#endif
#endif /* LLAMA_MI355X_H */
