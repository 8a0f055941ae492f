// Internal launcher interface between the C ABI (api.hip) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace llk {

struct NormArgs {
  float *h;            // fp32 rows (input; also receives the partial sums)
  int64_t in_offset;   // element offset of logical row 0
  int64_t in_stride;   // elements between logical rows
  const float *part;   // split-K partials [nsplit][rows][D] or nullptr
  int nsplit;
  int64_t part_stride; // elements between partial planes
  const void *w;       // norm weight [D] (dtype) or nullptr (no normalisation)
  float eps;
  int D;
  void *out;           // output rows [rows][D]
  int64_t out_plane;   // elements between hi and lo planes (mode 2)
};

struct RopeQkvArgs {
  const float *part;   // [nsplit][rows][(H+2G)*hd] fp32
  int nsplit;
  int64_t part_stride;
  int rows, S;         // rows = B*S tokens
  int H, G, hd;
  const float2 *tab;   // RoPE (cos, sin) table
  int tab_mod;         // table row = r % tab_mod (prefill) or r (tab_mod == 0)
  const int32_t *pos;  // per-sequence start positions or nullptr
  int start_pos;
  int cap;             // cache capacity (positions per sequence)
  float *qout;         // [rows][H*hd] fp32 (or nullptr)
  uint16_t *qhl;       // optional: q * qscale as bf16 hi/lo planes [2][rows][H*hd]
  uint16_t *qbf;       // optional: q as bf16 [rows][H*hd] (prefill attention operand)
  float qscale;
  void *kc, *vc;       // [B][cap][G][hd] (dtype)
  float *knew, *vnew;  // optional: rotated k and v of each row in fp32, [rows][G*hd]
};

// Dense bf16 GEMM C = A * B^T on MFMA with fused epilogues (prefill).
enum GemmEpi { EPI_STORE_F32 = 0, EPI_RESID = 1, EPI_QKV_ROPE = 2, EPI_SWIGLU = 3, EPI_STORE_BF16 = 4 };
struct GemmArgs {
  const uint16_t *A; int64_t lda;   // [M][K] bf16
  // [N][K] bf16 weights: B1 = w3 for SwiGLU; for EPI_QKV_ROPE the B-rows
  // [0, nq) come from B0 (wq), [nq, nq+nk) from B1 (wk), the rest from B2 (wv).
  const uint16_t *B0; const uint16_t *B1; const uint16_t *B2; int64_t ldb;
  int nq, nk;
  int M, N, K;                       // N counts output columns of A*B^T (SwiGLU: 2*F B-rows)
  // EPI_STORE_F32 / EPI_STORE_BF16 / EPI_RESID / EPI_SWIGLU
  void *C; int64_t ldc;
  const float *R; int64_t ldr;       // residual (EPI_RESID), may alias C
  // EPI_QKV_ROPE
  int S, H, G, hd, start_pos, cap;
  const float2 *tab;                 // rows indexed by s = row % S
  uint16_t *q; void *kc; void *vc;   // q [M][H*hd]; caches [B][cap][G][hd]
};

// Skinny bf16 GEMM for M <= 64 rows (decode, LM head): A given as hi/lo bf16
// planes, weights streamed once.
enum SkinnyEpi { SK_PARTIAL = 0, SK_SWIGLU_HILO = 1, SK_LOGITS = 2 };
struct SkinnyArgs {
  const uint16_t *A; int64_t a_plane; int lda;  // [2][M][K] (hi, lo) bf16
  int use_lo;                                   // 0: hi only
  // [N][K] bf16 weights.  SwiGLU: B0 = w1, B1 = w3.  SK_PARTIAL with nq > 0:
  // B-rows [0, nq) from B0, [nq, nq+nk) from B1, the rest from B2.
  const uint16_t *B0; const uint16_t *B1; const uint16_t *B2;
  int nq, nk;
  int M, N, K;                                  // N: B-rows (SwiGLU: 2*F)
  int ksplit;                                   // K slices (grid.y)
  void *C; int64_t c_plane;                     // SK_PARTIAL: [ksplit][M][N] fp32; SWIGLU: [2][M][F]
  float *logits;                                // SK_LOGITS: [M][N] fp32 or nullptr
  float *pval; int32_t *pidx; int nblk;         // SK_LOGITS argmax partials [M][nblk]
};

// Flash-style causal GQA attention, bf16 operands, fp32 softmax (prefill).
struct AttnArgs {
  const void *q; int64_t q_stride;        // [B*S][H*hd] rows
  const void *k; const void *v;           // [B][kcap][G][hd]
  int kcap;
  void *o;                                // [B*S][H*hd]
  int B, S, H, G, hd;
  int start_pos;                          // absolute position of query s = start_pos + s
  float scale;                            // 1/sqrt(hd)
  // optional [B][S] int32: the lowest key position query s may attend to
  // (document mask); keys below it get zero weight.  nullptr: 0.
  const int32_t *kv_lo;
};

// Decode attention over the cache (split over key chunks, then combined).
struct DecodeAttnArgs {
  const float *q;                         // [B][H*hd] fp32 (rotated)
  const uint16_t *qhl;                    // q * scale * log2(e) as bf16 hi/lo planes [2][B][H*hd] (bf16 path)
  const void *k; const void *v;           // [B][cap][G][hd] (dtype)
  const int32_t *pos;                     // [B] query positions (inclusive key range 0..pos)
  // optional [B][G][hd] fp32 key/value of the query's own position: when set,
  // the chunk kernels cover cached keys 0..pos-1 and the combine kernel adds
  // the query's own term from these unrounded values
  const float *knew; const float *vnew;
  int cap, B, H, G, hd, chunk, nchunk;
  float scale;
  float *pm; float *pl; float *po;        // partials [B][H][nchunk] (m, l), [B][H][nchunk][hd]
  void *out; int out_mode; int64_t out_plane;  // [B][H*hd]: 0 fp32, 2 bf16 hi/lo planes
  // optional [B]: the lowest visible cache position of each sequence (the
  // first position of its current document); keys below it get zero weight
  const int32_t *kv_lo;
};

// Token generation: per-sequence lengths (passed by value) and device state.
constexpr int kGenMaxBatch = 64;
struct GenLens {
  int32_t L[kGenMaxBatch];      // prompt length
  int32_t total[kGenMaxBatch];  // min(prompt + max_gen, max_seq_len)
};
struct RowList {                // row indices passed by value
  int32_t r[kGenMaxBatch];
};
struct GenState {              // each [B] int32 in device memory
  int32_t *cur, *pos;          // token and position the next decode step feeds
  int32_t *done, *end;         // finished flag; one past the last written position
  int32_t *next;               // the step's choice (argmax or sample)
  int32_t *gidx;               // index of the token the next step produces
  int32_t *active;             // [1] number of running sequences
};

hipError_t launch_embed(int dtype, const int32_t *ids, const void *E, float *h, int rows, int D, int V, hipStream_t s);
hipError_t launch_rmsnorm(int dtype, int mode, const NormArgs &a, int rows, hipStream_t s);
hipError_t launch_rope_table(float2 *tab, const int32_t *pos, int start_pos, int pos_max, int rows, int hd,
                             double theta, hipStream_t s);
hipError_t launch_rope_qkv(int dtype, const RopeQkvArgs &a, hipStream_t s);
hipError_t launch_swiglu(const float *gate, const float *up, float *u, int64_t n, hipStream_t s);
hipError_t launch_argmax_reduce(const float *pv, const int32_t *pi, int rows, int nblk, int32_t *out, hipStream_t s);
hipError_t launch_argmax_partial(const float *x, int rows, int n, int chunk, float *pv, int32_t *pi, int nblk,
                                 hipStream_t s);

hipError_t launch_gen_fill(const int32_t *prompt, int64_t pstride, int32_t *tokens, int64_t tstride,
                           const GenLens &lens, int B, hipStream_t s);
hipError_t launch_gen_stage_ids(const int32_t *prompt, int64_t pstride, const GenLens &lens, int b0, int g, int S,
                                int32_t *ids, hipStream_t s);
// D must be a multiple of 4
hipError_t launch_gather_rows(const float *h, int D, const RowList &rows, int n, float *out, hipStream_t s);
hipError_t launch_gen_step(const GenState &st, const GenLens &lens, int B, int eos, const int32_t *prompt,
                           int64_t pstride, int32_t *tokens, int64_t tstride, int first, hipStream_t s);
hipError_t launch_gen_finish(const GenState &st, int B, int eos, const int32_t *tokens, int64_t tstride,
                             int32_t *out_len, hipStream_t s);
// One block per row; requires V <= 131072.
hipError_t launch_sample_top_p(const float *logits, int64_t ld, int M, int V, float temperature, float top_p,
                               const float *u, int urows, const int32_t *gidx, int32_t *out, hipStream_t s);

hipError_t launch_gemm_bf16(int epi, const GemmArgs &a, hipStream_t s);
// fp32 path: C = A*B^T (+R), all fp32; epi is EPI_STORE_F32 or EPI_RESID.
hipError_t launch_gemm_f32(int epi, const float *A, const float *B, float *C, int64_t ldc, const float *R,
                           int64_t ldr, int M, int N, int K, hipStream_t s);

// Weight rows per block (64 or 128), row blocks (grid.x) and, for SK_PARTIAL,
// K slices (grid.y): workspace sizing and the launch use the same rule.
int skinny_rows(int N, int K, int epi);
int skinny_nblk(int N, int K, int epi);
int skinny_ksplit(int N, int K);
hipError_t launch_skinny(int epi, const SkinnyArgs &a, hipStream_t s);

hipError_t launch_attn_prefill(int dtype, const AttnArgs &a, hipStream_t s);
// kv_lo[b][s] = first position of the document (maximal run of equal ids in
// doc[b][0, start_pos + S)) that holds position start_pos + s.
hipError_t launch_doc_starts(const int32_t *doc, int B, int start_pos, int S, int32_t *kv_lo, hipStream_t s);
hipError_t launch_attn_decode(int dtype, const DecodeAttnArgs &a, hipStream_t s);
hipError_t launch_attn_combine(const DecodeAttnArgs &a, hipStream_t s);

}  // namespace llk
