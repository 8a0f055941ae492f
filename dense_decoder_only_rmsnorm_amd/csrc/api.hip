// C ABI of the Llama-3 decoder forward pass (declared in include/llama_mi355x.h):
// argument validation, workspace carving and the launch sequence of each
// entry point.  Everything is enqueued on the caller's stream; nothing here
// allocates device memory or synchronises the host.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "kernels.h"
#include "llama_mi355x.h"

using namespace llk;
using u16 = uint16_t;

namespace {

thread_local std::string g_err;

int fail(int code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

#define HIPCHK(expr)                                                                        \
  do {                                                                                      \
    hipError_t e_ = (expr);                                                                 \
    if (e_ != hipSuccess) return fail(LLAMA_ERR_HIP, "%s: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

// ---------------------------------------------------------------------------
// Optional per-kernel timing (llama_timing_enable / llama_timing_report): when
// on, every launch is bracketed by two hipEvents recorded on its stream.
// ---------------------------------------------------------------------------
struct TimingRec {
  const char *name;
  hipEvent_t start, stop;
};
struct Timing {
  std::mutex mu;
  bool on = false;
  std::vector<TimingRec> recs;
  std::vector<hipEvent_t> pool;
  size_t used = 0;
  hipEvent_t get() {
    if (used == pool.size()) {
      hipEvent_t e = nullptr;
      if (hipEventCreate(&e) != hipSuccess) return nullptr;
      pool.push_back(e);
    }
    return pool[used++];
  }
};
Timing g_timing;

struct TimingScope {
  const char *name;
  hipStream_t s;
  hipEvent_t start = nullptr;
  TimingScope(const char *n, hipStream_t st) : name(n), s(st) {
    if (!g_timing.on) return;
    std::lock_guard<std::mutex> lk(g_timing.mu);
    start = g_timing.get();
    if (start) hipEventRecord(start, s);
  }
  ~TimingScope() {
    if (!start) return;
    std::lock_guard<std::mutex> lk(g_timing.mu);
    hipEvent_t stop = g_timing.get();
    if (!stop) return;
    hipEventRecord(stop, s);
    g_timing.recs.push_back({name, start, stop});
  }
};

// launch with a timing tag; returns LLAMA_ERR_HIP from the enclosing function on failure
#define LAUNCH(tag, expr)         \
  do {                            \
    TimingScope ts_((tag), s);    \
    HIPCHK(expr);                 \
  } while (0)

constexpr int kDecodeChunk = 256;  // keys per decode-attention chunk
constexpr int kSkinnyRows = 64;    // rows per skinny GEMM launch

// Model dimensions derived from llama_args.
struct Dims {
  int D, L, H, G, hd, F, V, nrep, dt, esz;
  int Hq() const { return H * hd; }
  int Hk() const { return G * hd; }
  int Nqkv() const { return (H + 2 * G) * hd; }
};

int32_t ffn_hidden(const llama_args *a) {
  // [P2 3.5]: hidden = int(2 * (4 * dim) / 3); times the multiplier when set
  // (truncated); rounded up to a multiple of multiple_of.
  int64_t hidden = (int64_t)(2.0 * (4.0 * a->dim) / 3.0);
  if (a->ffn_dim_multiplier > 0.f) {
    const double scaled = (double)a->ffn_dim_multiplier * (double)hidden;
    if (!(scaled < 2147483648.0)) return -1;  // also keeps the conversion below defined
    hidden = (int64_t)scaled;
  }
  const int64_t m = a->multiple_of;
  const int64_t f = m * ((hidden + m - 1) / m);
  return f > INT32_MAX ? -1 : (int32_t)f;
}

int check_model(const llama_args *a, Dims &d) {
  if (!a) return fail(LLAMA_ERR_ARG, "args is NULL");
  if (a->dim <= 0 || a->n_heads <= 0 || a->n_kv_heads <= 0 || a->n_layers < 0 || a->vocab_size <= 0 ||
      a->multiple_of <= 0)
    return fail(LLAMA_ERR_ARG, "non-positive dimension in llama_args");
  if (a->dtype != LLAMA_F32 && a->dtype != LLAMA_BF16) return fail(LLAMA_ERR_ARG, "dtype %d is not F32/BF16", a->dtype);
  if (!(a->norm_eps >= 0.f) || !(a->rope_theta > 0.f)) return fail(LLAMA_ERR_ARG, "norm_eps/rope_theta out of range");
  if (a->dim % a->n_heads) return fail(LLAMA_ERR_SHAPE, "dim %d not divisible by n_heads %d", a->dim, a->n_heads);
  if (a->n_heads % a->n_kv_heads)
    return fail(LLAMA_ERR_SHAPE, "n_heads %d not divisible by n_kv_heads %d", a->n_heads, a->n_kv_heads);
  d.D = a->dim;
  d.L = a->n_layers;
  d.H = a->n_heads;
  d.G = a->n_kv_heads;
  d.hd = a->dim / a->n_heads;
  d.nrep = d.H / d.G;
  d.V = a->vocab_size;
  d.dt = a->dtype;
  d.esz = a->dtype == LLAMA_BF16 ? 2 : 4;
  d.F = ffn_hidden(a);
  if (d.F <= 0) return fail(LLAMA_ERR_ARG, "ffn hidden size overflows");
  if (d.hd % 2) return fail(LLAMA_ERR_SHAPE, "head_dim %d is odd (RoPE rotates pairs)", d.hd);
  if (d.hd != 64 && d.hd != 96 && d.hd != 128)
    return fail(LLAMA_ERR_UNSUPPORTED, "head_dim %d not in {64, 96, 128}", d.hd);
  if (d.D % 64 || d.F % 64) return fail(LLAMA_ERR_UNSUPPORTED, "dim %d / ffn hidden %d not multiples of 64", d.D, d.F);
  if (d.D > 8192) return fail(LLAMA_ERR_UNSUPPORTED, "dim %d above 8192", d.D);
  if (d.nrep > 16 || (d.nrep & (d.nrep - 1)))
    return fail(LLAMA_ERR_UNSUPPORTED, "n_heads/n_kv_heads = %d is not a power of two <= 16", d.nrep);
  return LLAMA_OK;
}

// Bump allocator over the caller's workspace; with base == nullptr it only
// measures.
struct Carver {
  char *base;
  size_t off = 0;
  explicit Carver(void *b) : base(static_cast<char *>(b)) {}
  template <typename T>
  T *take(size_t count) {
    off = (off + 255) & ~(size_t)255;
    T *p = base ? reinterpret_cast<T *>(base + off) : nullptr;
    off += count * sizeof(T);
    return p;
  }
};

// ------------------------------- prefill layout ------------------------------
struct PrefillWs {
  float *h;        // residual stream [T][D] fp32 (llama_prefill only)
  void *xn;        // [T][D] dtype
  float2 *tab;     // [S][hd/2]
  void *q;         // [T][Hq] dtype
  void *k, *v;     // [B][S][G][hd] dtype (no-cache path)
  void *o;         // [T][Hq] dtype
  void *u;         // [T][F] dtype
  float *qkv;      // fp32 path: [T][Nqkv]
  float *gate, *up;  // fp32 path: [T][F]
  // output head (rows = B)
  u16 *hf;         // bf16: [2][B][D]; fp32 path uses hf32
  float *hf32;
  float *logits;   // fp32 path scratch logits [B][V]
  float *pval;
  int32_t *pidx;
  int nblk;
  int32_t *kv_lo;  // [B][S] lowest visible key per query (document mask)
  // bf16 layers on at most kSkinnyRows tokens run on the skinny (weight
  // streaming) kernels: hi/lo activations and split-K partials
  u16 *xhl;        // [2][T][D]
  float *qkv_part; // [ks1][T][Nqkv]
  float *wo_part;  // [ks2][T][D]
  u16 *uhl;        // [2][T][F]
  float *w2_part;  // [ks3][T][D]
  int ks1, ks2, ks3;
};

PrefillWs carve_prefill(Carver &c, const Dims &d, int B, int S) {
  PrefillWs w{};
  const size_t T = (size_t)B * S;
  w.kv_lo = c.take<int32_t>(T);
  w.h = c.take<float>(T * d.D);
  w.tab = c.take<float2>((size_t)S * (d.hd / 2));
  if (d.dt == LLAMA_BF16) {
    w.xn = c.take<u16>(T * d.D);
    w.q = c.take<u16>(T * d.Hq());
    w.k = c.take<u16>(T * d.Hk());
    w.v = c.take<u16>(T * d.Hk());
    w.o = c.take<u16>(T * d.Hq());
    w.u = c.take<u16>(T * d.F);
    if (T <= (size_t)kSkinnyRows) {
      w.ks1 = skinny_ksplit(d.Nqkv(), d.D);
      w.ks2 = skinny_ksplit(d.D, d.Hq());
      w.ks3 = skinny_ksplit(d.D, d.F);
      w.xhl = c.take<u16>(2 * T * d.D);
      w.qkv_part = c.take<float>((size_t)w.ks1 * T * d.Nqkv());
      w.wo_part = c.take<float>((size_t)w.ks2 * T * d.D);
      w.uhl = c.take<u16>(2 * T * d.F);
      w.w2_part = c.take<float>((size_t)w.ks3 * T * d.D);
    }
  } else {
    w.xn = c.take<float>(T * d.D);
    w.qkv = c.take<float>(T * d.Nqkv());
    w.q = c.take<float>(T * d.Hq());
    w.k = c.take<float>(T * d.Hk());
    w.v = c.take<float>(T * d.Hk());
    w.o = c.take<float>(T * d.Hq());
    w.gate = c.take<float>(T * d.F);
    w.up = c.take<float>(T * d.F);
    w.u = c.take<float>(T * d.F);
  }
  return w;
}

struct HeadWs {
  float *last;     // [M][D] fp32: gathered last rows (ragged prompts)
  u16 *hf;
  float *hf32;
  float *logits;
  float *pval;
  int32_t *pidx;
  int nblk;
};

HeadWs carve_head(Carver &c, const Dims &d, int M) {
  HeadWs w{};
  w.last = c.take<float>((size_t)M * d.D);
  if (d.dt == LLAMA_BF16) {
    w.hf = c.take<u16>((size_t)2 * M * d.D);
    w.nblk = skinny_nblk(d.V, d.D, SK_LOGITS);
  } else {
    w.hf32 = c.take<float>((size_t)M * d.D);
    w.logits = c.take<float>((size_t)M * d.V);
    w.nblk = (d.V + 4095) / 4096;
  }
  w.pval = c.take<float>((size_t)M * w.nblk);
  w.pidx = c.take<int32_t>((size_t)M * w.nblk);
  return w;
}

// ------------------------------- decode layout -------------------------------
struct DecodeWs {
  float *h;         // [B][D]
  float2 *tab;      // [B][hd/2]
  void *xn;         // bf16 hi/lo [2][B][D] or fp32 [B][D]
  float *qkv_part;  // bf16: [ks1][B][Nqkv]; fp32: [B][Nqkv]
  float *q;         // [B][Hq]
  u16 *qhl;         // bf16 path: [2][B][Hq] (q scaled into log2 units)
  float *knew, *vnew;  // [B][G*hd] fp32: the new token's rotated key and value
  float *pm, *pl, *po;
  void *o;          // bf16 hi/lo [2][B][Hq] or fp32 [B][Hq]
  float *wo_part;   // [ks2][B][D]
  void *u;          // bf16 hi/lo [2][B][F] or fp32 [B][F]
  float *w2_part;   // [ks3][B][D]
  float *gate, *up; // fp32 path
  int ks1, ks2, ks3, nchunk;
};

DecodeWs carve_decode(Carver &c, const Dims &d, int B, int cap) {
  DecodeWs w{};
  w.ks1 = skinny_ksplit(d.Nqkv(), d.D);
  w.ks2 = skinny_ksplit(d.D, d.Hq());
  w.ks3 = skinny_ksplit(d.D, d.F);
  w.nchunk = (cap + kDecodeChunk - 1) / kDecodeChunk;
  const size_t Bz = (size_t)B;
  w.h = c.take<float>(Bz * d.D);
  w.tab = c.take<float2>(Bz * (d.hd / 2));
  w.q = c.take<float>(Bz * d.Hq());
  w.qhl = c.take<u16>(2 * Bz * d.Hq());
  w.knew = c.take<float>(Bz * d.Hk());
  w.vnew = c.take<float>(Bz * d.Hk());
  w.pm = c.take<float>(Bz * d.H * w.nchunk);
  w.pl = c.take<float>(Bz * d.H * w.nchunk);
  w.po = c.take<float>(Bz * d.H * w.nchunk * d.hd);
  if (d.dt == LLAMA_BF16) {
    w.xn = c.take<u16>(2 * Bz * d.D);
    w.qkv_part = c.take<float>((size_t)w.ks1 * Bz * d.Nqkv());
    w.o = c.take<u16>(2 * Bz * d.Hq());
    w.wo_part = c.take<float>((size_t)w.ks2 * Bz * d.D);
    w.u = c.take<u16>(2 * Bz * d.F);
    w.w2_part = c.take<float>((size_t)w.ks3 * Bz * d.D);
  } else {
    w.xn = c.take<float>(Bz * d.D);
    w.qkv_part = c.take<float>(Bz * d.Nqkv());
    w.o = c.take<float>(Bz * d.Hq());
    w.gate = c.take<float>(Bz * d.F);
    w.up = c.take<float>(Bz * d.F);
    w.u = c.take<float>(Bz * d.F);
  }
  return w;
}

size_t prefill_bytes(const Dims &d, int B, int S) {
  Carver c(nullptr);
  carve_prefill(c, d, B, S);
  carve_head(c, d, B);
  return c.off;
}
size_t decode_bytes(const Dims &d, int B, int cap) {
  Carver c(nullptr);
  carve_decode(c, d, B, cap);
  carve_head(c, d, B);
  return c.off;
}

// ------------------------------- building blocks -----------------------------
int rmsnorm(const Dims &d, int mode, float *h, int64_t in_off, int64_t in_stride, const float *part, int nsplit,
            int64_t part_stride, const void *w, float eps, void *out, int64_t out_plane, int rows, hipStream_t s) {
  NormArgs na{};
  na.h = h;
  na.in_offset = in_off;
  na.in_stride = in_stride;
  na.part = part;
  na.nsplit = nsplit;
  na.part_stride = part_stride;
  na.w = w;
  na.eps = eps;
  na.D = d.D;
  na.out = out;
  na.out_plane = out_plane;
  LAUNCH("rmsnorm", launch_rmsnorm(d.dt, mode, na, rows, s));
  return LLAMA_OK;
}

// Final head on M rows already normalised into ws (hi/lo planes or fp32).
int run_head(const Dims &d, const HeadWs &hw, const void *w_out, int M, float *logits, int32_t *ids, hipStream_t s) {
  if (d.dt == LLAMA_BF16) {
    for (int r0 = 0; r0 < M; r0 += kSkinnyRows) {
      const int m = std::min(kSkinnyRows, M - r0);
      SkinnyArgs sa{};
      sa.A = hw.hf + (int64_t)r0 * d.D;
      sa.a_plane = (int64_t)M * d.D;
      sa.lda = d.D;
      sa.use_lo = 1;
      sa.B0 = static_cast<const u16 *>(w_out);
      sa.M = m;
      sa.N = d.V;
      sa.K = d.D;
      sa.ksplit = 1;
      sa.logits = logits ? logits + (int64_t)r0 * d.V : nullptr;
      sa.pval = hw.pval + (int64_t)r0 * hw.nblk;
      sa.pidx = hw.pidx + (int64_t)r0 * hw.nblk;
      sa.nblk = hw.nblk;
      LAUNCH("lm_head", launch_skinny(SK_LOGITS, sa, s));
    }
  } else {
    float *lg = logits ? logits : hw.logits;
    LAUNCH("lm_head", launch_gemm_f32(EPI_STORE_F32, hw.hf32, static_cast<const float *>(w_out), lg, d.V, nullptr, 0, M, d.V, d.D,
                           s));
    LAUNCH("argmax_partial", launch_argmax_partial(lg, M, d.V, 4096, hw.pval, hw.pidx, hw.nblk, s));
  }
  LAUNCH("argmax_reduce", launch_argmax_reduce(hw.pval, hw.pidx, M, hw.nblk, ids, s));
  return LLAMA_OK;
}

// One bf16 layer on T <= kSkinnyRows tokens: every projection streams its
// weights once through the skinny kernels (the tiled GEMMs would leave most of
// a 256-row tile empty and most compute units idle), with hi/lo activations
// as in the decode step; RoPE and the cache write run in rope_qkv_kernel,
// attention in the prefill attention kernel.  h = y may alias x_in.
int run_layer_prefill_skinny(const llama_args *a, const Dims &d, const llama_layer_w *lw, const float *x_in,
                             float *h, int B, int S, int start_pos, void *kc, void *vc, int cap,
                             const PrefillWs &w, const int32_t *kv_lo, hipStream_t s) {
  const int T = B * S;
  const int64_t TD = (int64_t)T * d.D;
  auto skinny = [&](const char *tag, int epi, const u16 *A, int64_t a_plane, int lda, int use_lo, const void *B0,
                    const void *B1, const void *B2, int nq, int nk, int N, int K, int ks, void *C,
                    int64_t c_plane) -> int {
    SkinnyArgs sa{};
    sa.A = A;
    sa.a_plane = a_plane;
    sa.lda = lda;
    sa.use_lo = use_lo;
    sa.B0 = static_cast<const u16 *>(B0);
    sa.B1 = static_cast<const u16 *>(B1);
    sa.B2 = static_cast<const u16 *>(B2);
    sa.nq = nq;
    sa.nk = nk;
    sa.M = T;
    sa.N = N;
    sa.K = K;
    sa.ksplit = ks;
    sa.C = C;
    sa.c_plane = c_plane;
    LAUNCH(tag, launch_skinny(epi, sa, s));
    return LLAMA_OK;
  };
  // a2: attention_norm -> hi/lo
  if (int e = rmsnorm(d, 2, const_cast<float *>(x_in), 0, d.D, nullptr, 0, 0, lw->attention_norm, a->norm_eps, w.xhl,
                      TD, T, s))
    return e;
  // a3: QKV partials
  if (int e = skinny("skinny_qkv", SK_PARTIAL, w.xhl, TD, d.D, 1, lw->wq, lw->wk, lw->wv, d.Hq(), d.Hk(), d.Nqkv(),
                     d.D, w.ks1, w.qkv_part, (int64_t)T * d.Nqkv()))
    return e;
  // a4-a5: sum of the partials, RoPE at start_pos + s, q as bf16, K/V to the cache
  RopeQkvArgs ra{};
  ra.part = w.qkv_part;
  ra.nsplit = w.ks1;
  ra.part_stride = (int64_t)T * d.Nqkv();
  ra.rows = T;
  ra.S = S;
  ra.H = d.H;
  ra.G = d.G;
  ra.hd = d.hd;
  ra.tab = w.tab;
  ra.tab_mod = S;
  ra.pos = nullptr;
  ra.start_pos = start_pos;
  ra.cap = cap;
  ra.qbf = static_cast<u16 *>(w.q);
  ra.kc = kc;
  ra.vc = vc;
  LAUNCH("rope_qkv", launch_rope_qkv(d.dt, ra, s));
  // a6: causal GQA attention (bf16 output o)
  AttnArgs at{};
  at.q = w.q;
  at.q_stride = d.Hq();
  at.k = kc;
  at.v = vc;
  at.kcap = cap;
  at.o = w.o;
  at.B = B;
  at.S = S;
  at.H = d.H;
  at.G = d.G;
  at.hd = d.hd;
  at.start_pos = start_pos;
  at.scale = (float)(1.0 / sqrt((double)d.hd));
  at.kv_lo = kv_lo;
  LAUNCH("attn_prefill", launch_attn_prefill(d.dt, at, s));
  // a8: wo partials, folded into h = x_in + o wo^T by the ffn_norm kernel
  if (int e = skinny("skinny_wo", SK_PARTIAL, static_cast<const u16 *>(w.o), 0, d.Hq(), 0, lw->wo, nullptr, nullptr, 0,
                     0, d.D, d.Hq(), w.ks2, w.wo_part, TD))
    return e;
  if (h != x_in) HIPCHK(hipMemcpyAsync(h, x_in, (size_t)TD * sizeof(float), hipMemcpyDeviceToDevice, s));
  if (int e = rmsnorm(d, 2, h, 0, d.D, w.wo_part, w.ks2, TD, lw->ffn_norm, a->norm_eps, w.xhl, TD, T, s)) return e;
  // a9: u = silu(xn2 w1^T) * (xn2 w3^T) as hi/lo
  if (int e = skinny("skinny_w1w3_swiglu", SK_SWIGLU_HILO, w.xhl, TD, d.D, 1, lw->w1, lw->w3, nullptr, 0, 0, 2 * d.F,
                     d.D, 1, w.uhl, (int64_t)T * d.F))
    return e;
  // a10: h += u w2^T (partials folded in place; w == nullptr: no normalisation)
  if (int e = skinny("skinny_w2", SK_PARTIAL, w.uhl, (int64_t)T * d.F, d.F, 1, lw->w2, nullptr, nullptr, 0, 0, d.D,
                     d.F, w.ks3, w.w2_part, TD))
    return e;
  return rmsnorm(d, 0, h, 0, d.D, w.w2_part, w.ks3, TD, nullptr, a->norm_eps, h, 0, T, s);
}

// One prefill layer.  h [T][D] fp32 is updated in place (h == y after the
// copy-free residual epilogues); x_in is the layer input (may equal h).
int run_layer_prefill(const llama_args *a, const Dims &d, const llama_layer_w *lw, const float *x_in, float *h,
                      int B, int S, int start_pos, const llama_kv *kv, const PrefillWs &w, bool table_ready,
                      const int32_t *kv_lo, hipStream_t s) {
  const int T = B * S;
  const int cap = kv ? a->max_seq_len : S;
  void *kc = kv ? kv->k : w.k;
  void *vc = kv ? kv->v : w.v;
  if (!table_ready) LAUNCH("rope_table", launch_rope_table(w.tab, nullptr, start_pos, INT32_MAX, S, d.hd, a->rope_theta, s));
  if (d.dt == LLAMA_BF16 && T <= kSkinnyRows)
    return run_layer_prefill_skinny(a, d, lw, x_in, h, B, S, start_pos, kc, vc, cap, w, kv_lo, s);

  if (d.dt == LLAMA_BF16) {
    // a2: attention_norm -> bf16
    if (int e = rmsnorm(d, 1, const_cast<float *>(x_in), 0, d.D, nullptr, 0, 0, lw->attention_norm, a->norm_eps,
                        w.xn, 0, T, s))
      return e;
    // a3-a5: fused QKV projection + RoPE + K/V write
    GemmArgs g{};
    g.A = static_cast<const u16 *>(w.xn);
    g.lda = d.D;
    g.B0 = static_cast<const u16 *>(lw->wq);
    g.B1 = static_cast<const u16 *>(lw->wk);
    g.B2 = static_cast<const u16 *>(lw->wv);
    g.ldb = d.D;
    g.nq = d.Hq();
    g.nk = d.Hk();
    g.M = T;
    g.N = d.Nqkv();
    g.K = d.D;
    g.S = S;
    g.H = d.H;
    g.G = d.G;
    g.hd = d.hd;
    g.start_pos = start_pos;
    g.cap = cap;
    g.tab = w.tab;
    g.q = static_cast<u16 *>(w.q);
    g.kc = kc;
    g.vc = vc;
    LAUNCH("gemm_qkv_rope", launch_gemm_bf16(EPI_QKV_ROPE, g, s));
  } else {
    if (int e = rmsnorm(d, 0, const_cast<float *>(x_in), 0, d.D, nullptr, 0, 0, lw->attention_norm, a->norm_eps,
                        w.xn, 0, T, s))
      return e;
    const float *xn = static_cast<const float *>(w.xn);
    LAUNCH("gemm_qkv", launch_gemm_f32(EPI_STORE_F32, xn, static_cast<const float *>(lw->wq), w.qkv, d.Nqkv(), nullptr, 0, T,
                           d.Hq(), d.D, s));
    LAUNCH("gemm_qkv", launch_gemm_f32(EPI_STORE_F32, xn, static_cast<const float *>(lw->wk), w.qkv + d.Hq(), d.Nqkv(), nullptr,
                           0, T, d.Hk(), d.D, s));
    LAUNCH("gemm_qkv", launch_gemm_f32(EPI_STORE_F32, xn, static_cast<const float *>(lw->wv), w.qkv + d.Hq() + d.Hk(), d.Nqkv(),
                           nullptr, 0, T, d.Hk(), d.D, s));
    RopeQkvArgs ra{};
    ra.part = w.qkv;
    ra.nsplit = 1;
    ra.part_stride = 0;
    ra.rows = T;
    ra.S = S;
    ra.H = d.H;
    ra.G = d.G;
    ra.hd = d.hd;
    ra.tab = w.tab;
    ra.tab_mod = S;
    ra.pos = nullptr;
    ra.start_pos = start_pos;
    ra.cap = cap;
    ra.qout = static_cast<float *>(w.q);
    ra.kc = kc;
    ra.vc = vc;
    LAUNCH("rope_qkv", launch_rope_qkv(d.dt, ra, s));
  }
  // a6: causal GQA attention
  AttnArgs at{};
  at.q = w.q;
  at.q_stride = d.Hq();
  at.k = kc;
  at.v = vc;
  at.kcap = cap;
  at.o = w.o;
  at.B = B;
  at.S = S;
  at.H = d.H;
  at.G = d.G;
  at.hd = d.hd;
  at.start_pos = start_pos;
  at.scale = (float)(1.0 / sqrt((double)d.hd));
  at.kv_lo = kv_lo;
  LAUNCH("attn_prefill", launch_attn_prefill(d.dt, at, s));

  if (d.dt == LLAMA_BF16) {
    // a8: h = x + o wo^T
    GemmArgs g{};
    g.A = static_cast<const u16 *>(w.o);
    g.lda = d.Hq();
    g.B0 = static_cast<const u16 *>(lw->wo);
    g.ldb = d.Hq();
    g.M = T;
    g.N = d.D;
    g.K = d.Hq();
    g.C = h;
    g.ldc = d.D;
    g.R = x_in;
    g.ldr = d.D;
    LAUNCH("gemm_wo_resid", launch_gemm_bf16(EPI_RESID, g, s));
    // a2: ffn_norm
    if (int e = rmsnorm(d, 1, h, 0, d.D, nullptr, 0, 0, lw->ffn_norm, a->norm_eps, w.xn, 0, T, s)) return e;
    // a9: u = silu(xn2 w1^T) * (xn2 w3^T)
    GemmArgs f{};
    f.A = static_cast<const u16 *>(w.xn);
    f.lda = d.D;
    f.B0 = static_cast<const u16 *>(lw->w1);
    f.B1 = static_cast<const u16 *>(lw->w3);
    f.ldb = d.D;
    f.M = T;
    f.N = 2 * d.F;
    f.K = d.D;
    f.C = w.u;
    f.ldc = d.F;
    LAUNCH("gemm_w1w3_swiglu", launch_gemm_bf16(EPI_SWIGLU, f, s));
    // a10: h += u w2^T
    GemmArgs g2{};
    g2.A = static_cast<const u16 *>(w.u);
    g2.lda = d.F;
    g2.B0 = static_cast<const u16 *>(lw->w2);
    g2.ldb = d.F;
    g2.M = T;
    g2.N = d.D;
    g2.K = d.F;
    g2.C = h;
    g2.ldc = d.D;
    g2.R = h;
    g2.ldr = d.D;
    LAUNCH("gemm_w2_resid", launch_gemm_bf16(EPI_RESID, g2, s));
  } else {
    LAUNCH("gemm_wo_resid", launch_gemm_f32(EPI_RESID, static_cast<const float *>(w.o), static_cast<const float *>(lw->wo), h, d.D,
                           x_in, d.D, T, d.D, d.Hq(), s));
    if (int e = rmsnorm(d, 0, h, 0, d.D, nullptr, 0, 0, lw->ffn_norm, a->norm_eps, w.xn, 0, T, s)) return e;
    const float *xn = static_cast<const float *>(w.xn);
    LAUNCH("gemm_w1w3", launch_gemm_f32(EPI_STORE_F32, xn, static_cast<const float *>(lw->w1), w.gate, d.F, nullptr, 0, T, d.F, d.D,
                           s));
    LAUNCH("gemm_w1w3", launch_gemm_f32(EPI_STORE_F32, xn, static_cast<const float *>(lw->w3), w.up, d.F, nullptr, 0, T, d.F, d.D,
                           s));
    LAUNCH("swiglu", launch_swiglu(w.gate, w.up, static_cast<float *>(w.u), (int64_t)T * d.F, s));
    LAUNCH("gemm_w2_resid", launch_gemm_f32(EPI_RESID, static_cast<const float *>(w.u), static_cast<const float *>(lw->w2), h, d.D, h,
                           d.D, T, d.D, d.F, s));
  }
  return LLAMA_OK;
}

int check_layer_w(const llama_layer_w *lw) {
  if (!lw || !lw->attention_norm || !lw->wq || !lw->wk || !lw->wv || !lw->wo || !lw->ffn_norm || !lw->w1 || !lw->w2 ||
      !lw->w3)
    return fail(LLAMA_ERR_ARG, "layer weight pointer is NULL");
  return LLAMA_OK;
}

// ------------------------------- generation layout ---------------------------
constexpr int64_t kGenPrefillTokens = 16384;  // tokens per prefill call inside generation
constexpr int kGenCheckEvery = 8;             // decode steps between early-stop checks
constexpr int kSampleMaxVocab = 131072;       // 1024 threads x 128 ids per sampler block

struct GenWs {
  GenState st;
  float *logits;   // [B][V] fp32 (sampling)
  int32_t *ids;    // staged prompt rows of one prefill call
  void *rest;      // prefill / decode workspace
  size_t rest_bytes;
};

int gen_rows_per_call(int L, int B) {
  return (int)std::max<int64_t>(1, std::min<int64_t>(B, kGenPrefillTokens / L));
}

// Prefill (prompts padded to Lmax, gen_rows_per_call rows at a time) or
// decode workspace, whichever is larger.
size_t gen_inner_bytes(const Dims &d, int B, int Lmax, int cap) {
  return std::max(decode_bytes(d, B, cap), prefill_bytes(d, gen_rows_per_call(Lmax, B), Lmax));
}

GenWs carve_gen(Carver &c, const Dims &d, int B, int Lmax, int cap) {
  GenWs w{};
  w.st.cur = c.take<int32_t>(B);
  w.st.pos = c.take<int32_t>(B);
  w.st.done = c.take<int32_t>(B);
  w.st.end = c.take<int32_t>(B);
  w.st.next = c.take<int32_t>(B);
  w.st.gidx = c.take<int32_t>(B);
  w.st.active = c.take<int32_t>(1);
  w.logits = c.take<float>((size_t)B * d.V);
  w.ids = c.take<int32_t>((size_t)B * Lmax);
  w.rest_bytes = gen_inner_bytes(d, B, Lmax, cap);
  w.rest = c.take<char>(w.rest_bytes);
  return w;
}


// Prefill of `batch` sequences; with last_rows (HOST, batch <= 64) the logits
// of sequence b come from its row last_rows[b] instead of seq_len - 1.
int prefill_impl(const llama_args *a, const llama_model_w *w, const int32_t *ids, const int32_t *doc_ids,
                 int batch, int seq_len, const llama_kv *kv, float *hidden, float *logits, int32_t *next_id,
                 const int32_t *last_rows, void *ws, size_t ws_bytes, void *stream) {
  Dims d;
  if (int e = check_model(a, d)) return e;
  if (!w || !w->tok_embeddings || !w->norm || !w->output || (d.L > 0 && !w->layers))
    return fail(LLAMA_ERR_ARG, "model weight pointer is NULL");
  for (int l = 0; l < d.L; ++l)
    if (int e = check_layer_w(&w->layers[l])) return e;
  if (!ids || !next_id || !ws) return fail(LLAMA_ERR_ARG, "ids, next_id or ws is NULL");
  if (batch < 1 || seq_len < 1) return fail(LLAMA_ERR_ARG, "batch and seq_len must be >= 1");
  if (batch > kSkinnyRows * 1024) return fail(LLAMA_ERR_UNSUPPORTED, "batch %d too large", batch);
  if (kv) {
    for (int l = 0; l < d.L; ++l)
      if (!kv[l].k || !kv[l].v) return fail(LLAMA_ERR_ARG, "kv[%d] has a NULL pointer", l);
    if (batch > a->max_batch_size) return fail(LLAMA_ERR_SHAPE, "batch %d > max_batch_size %d", batch, a->max_batch_size);
    if (seq_len > a->max_seq_len) return fail(LLAMA_ERR_SHAPE, "seq_len %d > max_seq_len %d", seq_len, a->max_seq_len);
  }
  if (last_rows) {
    if (batch > kGenMaxBatch) return fail(LLAMA_ERR_UNSUPPORTED, "ragged batch %d above %d", batch, kGenMaxBatch);
    for (int b = 0; b < batch; ++b)
      if (last_rows[b] < 0 || last_rows[b] >= seq_len) return fail(LLAMA_ERR_ARG, "last row %d out of range", b);
  }
  const size_t need = prefill_bytes(d, batch, seq_len);
  if (ws_bytes < need) return fail(LLAMA_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  if ((uintptr_t)ws % 256) return fail(LLAMA_ERR_ARG, "workspace not 256-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  Carver c(ws);
  PrefillWs pw = carve_prefill(c, d, batch, seq_len);
  HeadWs hw = carve_head(c, d, batch);
  float *h = hidden ? hidden : pw.h;
  const int T = batch * seq_len;
  // a1: embedding rows
  LAUNCH("embed", launch_embed(d.dt, ids, w->tok_embeddings, h, T, d.D, d.V, s));
  LAUNCH("rope_table", launch_rope_table(pw.tab, nullptr, 0, INT32_MAX, seq_len, d.hd, a->rope_theta, s));
  if (doc_ids) LAUNCH("doc_starts", launch_doc_starts(doc_ids, batch, 0, seq_len, pw.kv_lo, s));
  // a2-a11: layers
  for (int l = 0; l < d.L; ++l) {
    if (int e = run_layer_prefill(a, d, &w->layers[l], h, h, batch, seq_len, 0, kv ? &kv[l] : nullptr, pw, true,
                                  doc_ids ? pw.kv_lo : nullptr, s))
      return e;
  }
  // a12: final norm of each sequence's last row -> hi/lo (bf16) or fp32
  float *hl = h;
  int64_t l_off = (int64_t)(seq_len - 1) * d.D, l_stride = (int64_t)seq_len * d.D;
  if (last_rows) {
    // ragged prompts padded to seq_len: gather each sequence's own last row
    RowList rl{};
    for (int b = 0; b < batch; ++b) rl.r[b] = b * seq_len + last_rows[b];
    LAUNCH("gather_rows", launch_gather_rows(h, d.D, rl, batch, hw.last, s));
    hl = hw.last;
    l_off = 0;
    l_stride = d.D;
  }
  if (d.dt == LLAMA_BF16) {
    if (int e = rmsnorm(d, 2, hl, l_off, l_stride, nullptr, 0, 0, w->norm, a->norm_eps, hw.hf, (int64_t)batch * d.D,
                        batch, s))
      return e;
  } else {
    if (int e = rmsnorm(d, 0, hl, l_off, l_stride, nullptr, 0, 0, w->norm, a->norm_eps, hw.hf32, 0, batch, s))
      return e;
  }
  // a13-a14: LM head + argmax
  return run_head(d, hw, w->output, batch, logits, next_id, s);
}

}  // namespace

extern "C" {

int32_t llama_ffn_hidden_dim(const llama_args *a) {
  if (!a || a->dim <= 0 || a->multiple_of <= 0) return fail(LLAMA_ERR_ARG, "invalid llama_args");
  const int32_t f = ffn_hidden(a);
  return f > 0 ? f : fail(LLAMA_ERR_ARG, "ffn hidden size overflows");
}

size_t llama_workspace_bytes(const llama_args *a, int32_t batch, int32_t seq_len) {
  Dims d;
  if (check_model(a, d) != LLAMA_OK || batch < 1 || seq_len < 1) return 0;
  const int cap = std::max(a->max_seq_len, 1);
  return std::max(prefill_bytes(d, batch, seq_len), decode_bytes(d, batch, cap)) + 256;
}

int llama_layer_forward(const llama_args *a, const llama_layer_w *w, const float *x, float *y, int32_t batch,
                        int32_t seq_len, int32_t start_pos, const llama_kv *kv, void *ws, size_t ws_bytes,
                        void *stream) {
  return llama_layer_forward_docs(a, w, x, y, batch, seq_len, start_pos, kv, nullptr, ws, ws_bytes, stream);
}

int llama_layer_forward_docs(const llama_args *a, const llama_layer_w *w, const float *x, float *y, int32_t batch,
                             int32_t seq_len, int32_t start_pos, const llama_kv *kv, const int32_t *doc_ids, void *ws,
                             size_t ws_bytes, void *stream) {
  Dims d;
  if (int e = check_model(a, d)) return e;
  if (int e = check_layer_w(w)) return e;
  if (!x || !y || !ws) return fail(LLAMA_ERR_ARG, "x, y or ws is NULL");
  if (batch < 1 || seq_len < 1) return fail(LLAMA_ERR_ARG, "batch and seq_len must be >= 1");
  if (start_pos < 0) return fail(LLAMA_ERR_ARG, "start_pos < 0");
  if (!kv && start_pos != 0) return fail(LLAMA_ERR_ARG, "start_pos > 0 needs a KV cache");
  if (kv) {
    if (!kv->k || !kv->v) return fail(LLAMA_ERR_ARG, "kv->k or kv->v is NULL");
    if (batch > a->max_batch_size) return fail(LLAMA_ERR_SHAPE, "batch %d > max_batch_size %d", batch, a->max_batch_size);
    if ((int64_t)start_pos + seq_len > a->max_seq_len)
      return fail(LLAMA_ERR_SHAPE, "start_pos + seq_len = %lld > max_seq_len %d", (long long)start_pos + seq_len,
                  a->max_seq_len);
  }
  const size_t need = prefill_bytes(d, batch, seq_len);
  if (ws_bytes < need) return fail(LLAMA_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  if ((uintptr_t)ws % 256) return fail(LLAMA_ERR_ARG, "workspace not 256-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  Carver c(ws);
  PrefillWs pw = carve_prefill(c, d, batch, seq_len);
  if (doc_ids) LAUNCH("doc_starts", launch_doc_starts(doc_ids, batch, start_pos, seq_len, pw.kv_lo, s));
  return run_layer_prefill(a, d, w, x, y, batch, seq_len, start_pos, kv, pw, false, doc_ids ? pw.kv_lo : nullptr,
                           s);
}

int llama_prefill(const llama_args *a, const llama_model_w *w, const int32_t *ids, int32_t batch, int32_t seq_len,
                  const llama_kv *kv, float *hidden, float *logits, int32_t *next_id, void *ws, size_t ws_bytes,
                  void *stream) {
  return llama_prefill_docs(a, w, ids, nullptr, batch, seq_len, kv, hidden, logits, next_id, ws, ws_bytes, stream);
}

int llama_prefill_docs(const llama_args *a, const llama_model_w *w, const int32_t *ids, const int32_t *doc_ids,
                       int32_t batch, int32_t seq_len, const llama_kv *kv, float *hidden, float *logits,
                       int32_t *next_id, void *ws, size_t ws_bytes, void *stream) {
  return prefill_impl(a, w, ids, doc_ids, batch, seq_len, kv, hidden, logits, next_id, nullptr, ws, ws_bytes, stream);
}


int llama_decode_step(const llama_args *a, const llama_model_w *w, const int32_t *ids, const int32_t *pos,
                      int32_t batch, const llama_kv *kv, float *logits, int32_t *next_id, void *ws, size_t ws_bytes,
                      void *stream) {
  return llama_decode_step_docs(a, w, ids, pos, nullptr, batch, kv, logits, next_id, ws, ws_bytes, stream);
}

}  // extern "C"

namespace {

// Argument checks of a decode step (everything but the workspace).
int check_decode(const llama_args *a, const llama_model_w *w, const int32_t *ids, const int32_t *pos, int32_t batch,
                 const llama_kv *kv, int32_t *next_id, Dims &d) {
  if (int e = check_model(a, d)) return e;
  if (!w || !w->tok_embeddings || !w->norm || !w->output || (d.L > 0 && !w->layers))
    return fail(LLAMA_ERR_ARG, "model weight pointer is NULL");
  for (int l = 0; l < d.L; ++l)
    if (int e = check_layer_w(&w->layers[l])) return e;
  if (!ids || !pos || !next_id || (d.L > 0 && !kv)) return fail(LLAMA_ERR_ARG, "ids, pos, kv or next_id is NULL");
  for (int l = 0; l < d.L; ++l)
    if (!kv[l].k || !kv[l].v) return fail(LLAMA_ERR_ARG, "kv[%d] has a NULL pointer", l);
  if (batch < 1) return fail(LLAMA_ERR_ARG, "batch must be >= 1");
  if (batch > a->max_batch_size) return fail(LLAMA_ERR_SHAPE, "batch %d > max_batch_size %d", batch, a->max_batch_size);
  if (a->max_seq_len < 1) return fail(LLAMA_ERR_SHAPE, "max_seq_len < 1");
  if (d.dt == LLAMA_BF16 && batch > kSkinnyRows)
    return fail(LLAMA_ERR_UNSUPPORTED, "decode batch %d above %d rows", batch, kSkinnyRows);
  return LLAMA_OK;
}

// ---------------------------------------------------------------------------
// Scratch of the allocation-free decode step (llama_decode_step_noalloc): a
// file-scope device array that every GPU the library runs on holds until the
// process ends.  Host code never uses the array's name as an address: its
// device address is taken once per device with hipGetSymbolAddress and kept.
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = (size_t)96 << 20;
constexpr int kMaxDevices = 64;
__device__ __align__(256) unsigned char scratch[kScratchBytes];
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch (looked up on its first use).
int scratch_on_current_device(void **out) {
  int dev = -1;
  const hipError_t eg = hipGetDevice(&dev);
  if (eg != hipSuccess) return fail(LLAMA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(eg));
  if (dev < 0 || dev >= kMaxDevices) return fail(LLAMA_ERR_UNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return fail(LLAMA_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return LLAMA_OK;
}

}  // namespace

extern "C" {

int llama_decode_step_docs(const llama_args *a, const llama_model_w *w, const int32_t *ids, const int32_t *pos,
                           const int32_t *doc_start, int32_t batch, const llama_kv *kv, float *logits,
                           int32_t *next_id, void *ws, size_t ws_bytes, void *stream) {
  Dims d;
  if (int e = check_decode(a, w, ids, pos, batch, kv, next_id, d)) return e;
  if (!ws) return fail(LLAMA_ERR_ARG, "ws is NULL");
  const int cap = a->max_seq_len;
  const size_t need = decode_bytes(d, batch, cap);
  if (ws_bytes < need) return fail(LLAMA_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  if ((uintptr_t)ws % 256) return fail(LLAMA_ERR_ARG, "workspace not 256-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  Carver c(ws);
  DecodeWs dw = carve_decode(c, d, batch, cap);
  HeadWs hw = carve_head(c, d, batch);
  const int B = batch;
  const bool bf = d.dt == LLAMA_BF16;

  LAUNCH("embed", launch_embed(d.dt, ids, w->tok_embeddings, dw.h, B, d.D, d.V, s));
  LAUNCH("rope_table", launch_rope_table(dw.tab, pos, 0, cap - 1, B, d.hd, a->rope_theta, s));
  const float *pend = nullptr;  // w2 partials of the previous layer still to fold into h
  int pend_n = 0;
  for (int l = 0; l < d.L; ++l) {
    const llama_layer_w *lw = &w->layers[l];
    // a2 (+ previous layer's a10 residual)
    if (int e = rmsnorm(d, bf ? 2 : 0, dw.h, 0, d.D, pend, pend_n, (int64_t)B * d.D, lw->attention_norm, a->norm_eps,
                        dw.xn, (int64_t)B * d.D, B, s))
      return e;
    // a3: QKV
    if (bf) {
      SkinnyArgs sa{};
      sa.A = static_cast<const u16 *>(dw.xn);
      sa.a_plane = (int64_t)B * d.D;
      sa.lda = d.D;
      sa.use_lo = 1;
      sa.B0 = static_cast<const u16 *>(lw->wq);
      sa.B1 = static_cast<const u16 *>(lw->wk);
      sa.B2 = static_cast<const u16 *>(lw->wv);
      sa.nq = d.Hq();
      sa.nk = d.Hk();
      sa.M = B;
      sa.N = d.Nqkv();
      sa.K = d.D;
      sa.ksplit = dw.ks1;
      sa.C = dw.qkv_part;
      sa.c_plane = (int64_t)B * d.Nqkv();
      LAUNCH("skinny_qkv", launch_skinny(SK_PARTIAL, sa, s));
    } else {
      const float *xn = static_cast<const float *>(dw.xn);
      LAUNCH("gemm_qkv", launch_gemm_f32(EPI_STORE_F32, xn, static_cast<const float *>(lw->wq), dw.qkv_part, d.Nqkv(), nullptr, 0,
                             B, d.Hq(), d.D, s));
      LAUNCH("gemm_qkv", launch_gemm_f32(EPI_STORE_F32, xn, static_cast<const float *>(lw->wk), dw.qkv_part + d.Hq(), d.Nqkv(),
                             nullptr, 0, B, d.Hk(), d.D, s));
      LAUNCH("gemm_qkv", launch_gemm_f32(EPI_STORE_F32, xn, static_cast<const float *>(lw->wv), dw.qkv_part + d.Hq() + d.Hk(),
                             d.Nqkv(), nullptr, 0, B, d.Hk(), d.D, s));
    }
    // a4-a5: RoPE + cache write at pos[b]
    RopeQkvArgs ra{};
    ra.part = dw.qkv_part;
    ra.nsplit = bf ? dw.ks1 : 1;
    ra.part_stride = (int64_t)B * d.Nqkv();
    ra.rows = B;
    ra.S = 1;
    ra.H = d.H;
    ra.G = d.G;
    ra.hd = d.hd;
    ra.tab = dw.tab;
    ra.tab_mod = 0;
    ra.pos = pos;
    ra.start_pos = 0;
    ra.cap = cap;
    ra.qout = dw.q;
    ra.qhl = bf ? dw.qhl : nullptr;
    ra.qscale = (float)(1.4426950408889634 / sqrt((double)d.hd));
    ra.kc = kv[l].k;
    ra.vc = kv[l].v;
    ra.knew = dw.knew;
    ra.vnew = dw.vnew;
    LAUNCH("rope_qkv", launch_rope_qkv(d.dt, ra, s));
    // a7: attention over the cache; the token's own key and value enter
    // unrounded (fp32) through the combine step, the cache keeps them in the
    // storage type for later steps
    DecodeAttnArgs da{};
    da.q = dw.q;
    da.qhl = bf ? dw.qhl : nullptr;
    da.k = kv[l].k;
    da.v = kv[l].v;
    da.pos = pos;
    da.knew = dw.knew;
    da.vnew = dw.vnew;
    da.cap = cap;
    da.B = B;
    da.H = d.H;
    da.G = d.G;
    da.hd = d.hd;
    da.chunk = kDecodeChunk;
    da.nchunk = dw.nchunk;
    da.scale = (float)(1.0 / sqrt((double)d.hd));
    da.pm = dw.pm;
    da.pl = dw.pl;
    da.po = dw.po;
    da.out = dw.o;
    da.out_mode = bf ? 2 : 0;
    da.out_plane = (int64_t)B * d.Hq();
    da.kv_lo = doc_start;
    LAUNCH("attn_decode", launch_attn_decode(d.dt, da, s));
    LAUNCH("attn_combine", launch_attn_combine(da, s));
    if (bf) {
      // a8: wo partials, folded into h by the ffn_norm kernel
      SkinnyArgs sa{};
      sa.A = static_cast<const u16 *>(dw.o);
      sa.a_plane = (int64_t)B * d.Hq();
      sa.lda = d.Hq();
      sa.use_lo = 1;
      sa.B0 = static_cast<const u16 *>(lw->wo);
      sa.M = B;
      sa.N = d.D;
      sa.K = d.Hq();
      sa.ksplit = dw.ks2;
      sa.C = dw.wo_part;
      sa.c_plane = (int64_t)B * d.D;
      LAUNCH("skinny_wo", launch_skinny(SK_PARTIAL, sa, s));
      if (int e = rmsnorm(d, 2, dw.h, 0, d.D, dw.wo_part, dw.ks2, (int64_t)B * d.D, lw->ffn_norm, a->norm_eps, dw.xn,
                          (int64_t)B * d.D, B, s))
        return e;
      // a9: SwiGLU
      SkinnyArgs fa{};
      fa.A = static_cast<const u16 *>(dw.xn);
      fa.a_plane = (int64_t)B * d.D;
      fa.lda = d.D;
      fa.use_lo = 1;
      fa.B0 = static_cast<const u16 *>(lw->w1);
      fa.B1 = static_cast<const u16 *>(lw->w3);
      fa.M = B;
      fa.N = 2 * d.F;
      fa.K = d.D;
      fa.ksplit = 1;
      fa.C = dw.u;
      fa.c_plane = (int64_t)B * d.F;
      LAUNCH("skinny_w1w3_swiglu", launch_skinny(SK_SWIGLU_HILO, fa, s));
      // a10: w2 partials (folded by the next norm)
      SkinnyArgs sb{};
      sb.A = static_cast<const u16 *>(dw.u);
      sb.a_plane = (int64_t)B * d.F;
      sb.lda = d.F;
      sb.use_lo = 1;
      sb.B0 = static_cast<const u16 *>(lw->w2);
      sb.M = B;
      sb.N = d.D;
      sb.K = d.F;
      sb.ksplit = dw.ks3;
      sb.C = dw.w2_part;
      sb.c_plane = (int64_t)B * d.D;
      LAUNCH("skinny_w2", launch_skinny(SK_PARTIAL, sb, s));
      pend = dw.w2_part;
      pend_n = dw.ks3;
    } else {
      LAUNCH("gemm_wo_resid", launch_gemm_f32(EPI_RESID, static_cast<const float *>(dw.o), static_cast<const float *>(lw->wo), dw.h,
                             d.D, dw.h, d.D, B, d.D, d.Hq(), s));
      if (int e = rmsnorm(d, 0, dw.h, 0, d.D, nullptr, 0, 0, lw->ffn_norm, a->norm_eps, dw.xn, 0, B, s)) return e;
      const float *xn = static_cast<const float *>(dw.xn);
      LAUNCH("gemm_w1w3", launch_gemm_f32(EPI_STORE_F32, xn, static_cast<const float *>(lw->w1), dw.gate, d.F, nullptr, 0, B, d.F,
                             d.D, s));
      LAUNCH("gemm_w1w3", launch_gemm_f32(EPI_STORE_F32, xn, static_cast<const float *>(lw->w3), dw.up, d.F, nullptr, 0, B, d.F,
                             d.D, s));
      LAUNCH("swiglu", launch_swiglu(dw.gate, dw.up, static_cast<float *>(dw.u), (int64_t)B * d.F, s));
      LAUNCH("gemm_w2_resid", launch_gemm_f32(EPI_RESID, static_cast<const float *>(dw.u), static_cast<const float *>(lw->w2), dw.h,
                             d.D, dw.h, d.D, B, d.D, d.F, s));
    }
  }
  // a12: final norm (folding the last w2 partials)
  if (bf) {
    if (int e = rmsnorm(d, 2, dw.h, 0, d.D, pend, pend_n, (int64_t)B * d.D, w->norm, a->norm_eps, hw.hf,
                        (int64_t)B * d.D, B, s))
      return e;
  } else {
    if (int e = rmsnorm(d, 0, dw.h, 0, d.D, nullptr, 0, 0, w->norm, a->norm_eps, hw.hf32, 0, B, s)) return e;
  }
  return run_head(d, hw, w->output, B, logits, next_id, s);
}

size_t llama_decode_noalloc_max_bytes(void) { return kScratchBytes; }

int llama_decode_step_noalloc(const llama_args *a, const llama_model_w *w, const int32_t *ids, const int32_t *pos,
                              int32_t batch, const llama_kv *kv, float *logits, int32_t *next_id, void *stream) {
  Dims d;
  if (int e = check_decode(a, w, ids, pos, batch, kv, next_id, d)) return e;
  const size_t need = decode_bytes(d, batch, a->max_seq_len);
  if (need > kScratchBytes)
    return fail(LLAMA_ERR_WORKSPACE,
                "decode step of %d sequences with max_seq_len %d needs %zu bytes of scratch; the library's static "
                "scratch holds %zu",
                batch, a->max_seq_len, need, kScratchBytes);
  void *ws = nullptr;
  if (int e = scratch_on_current_device(&ws)) return e;
  return llama_decode_step_docs(a, w, ids, pos, nullptr, batch, kv, logits, next_id, ws, kScratchBytes, stream);
}

int lm_head_argmax(const llama_args *a, const float *h, const void *final_norm_w, const void *w_out, int32_t M,
                   float *logits, int32_t *argmax, void *ws, size_t ws_bytes, void *stream) {
  Dims d;
  if (int e = check_model(a, d)) return e;
  if (!h || !w_out || !argmax || !ws) return fail(LLAMA_ERR_ARG, "h, w_out, argmax or ws is NULL");
  if (M < 1) return fail(LLAMA_ERR_ARG, "M must be >= 1");
  Carver probe(nullptr);
  carve_head(probe, d, M);
  if (ws_bytes < probe.off) return fail(LLAMA_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, probe.off);
  if ((uintptr_t)ws % 256) return fail(LLAMA_ERR_ARG, "workspace not 256-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  Carver c(ws);
  HeadWs hw = carve_head(c, d, M);
  if (d.dt == LLAMA_BF16) {
    if (int e = rmsnorm(d, 2, const_cast<float *>(h), 0, d.D, nullptr, 0, 0, final_norm_w, a->norm_eps, hw.hf,
                        (int64_t)M * d.D, M, s))
      return e;
  } else {
    if (int e = rmsnorm(d, 0, const_cast<float *>(h), 0, d.D, nullptr, 0, 0, final_norm_w, a->norm_eps, hw.hf32, 0, M,
                        s))
      return e;
  }
  return run_head(d, hw, w_out, M, logits, argmax, s);
}

int llama_sample_top_p(const float *logits, int32_t M, int32_t V, float temperature, float top_p, const float *u,
                       int32_t *out_id, void *stream) {
  if (!logits || !u || !out_id) return fail(LLAMA_ERR_ARG, "logits, u or out_id is NULL");
  if (M < 1 || V < 1) return fail(LLAMA_ERR_ARG, "M and V must be >= 1");
  if (!(temperature > 0.f)) return fail(LLAMA_ERR_ARG, "temperature must be > 0");
  if (!(top_p >= 0.f)) return fail(LLAMA_ERR_ARG, "top_p must be >= 0");
  if (V > kSampleMaxVocab) return fail(LLAMA_ERR_UNSUPPORTED, "vocab %d above %d", V, kSampleMaxVocab);
  hipStream_t s = static_cast<hipStream_t>(stream);
  LAUNCH("sample_top_p", launch_sample_top_p(logits, V, M, V, temperature, top_p, u, 1, nullptr, out_id, s));
  return LLAMA_OK;
}

size_t llama_generate_workspace_bytes(const llama_args *a, int32_t batch, int32_t max_prompt_len) {
  Dims d;
  if (check_model(a, d) != LLAMA_OK || batch < 1 || batch > kGenMaxBatch || max_prompt_len < 1 ||
      a->max_seq_len < 1)
    return 0;
  Carver c(nullptr);
  carve_gen(c, d, batch, max_prompt_len, a->max_seq_len);
  return c.off + 256;
}

int llama_generate(const llama_args *a, const llama_model_w *w, const int32_t *prompt, int32_t prompt_stride,
                   const int32_t *prompt_len, int32_t batch, int32_t max_gen_len, int32_t eos_id, float temperature,
                   float top_p, const float *uniforms, const llama_kv *kv, int32_t *tokens, int32_t *out_len,
                   int32_t flags, int32_t *steps_run, void *ws, size_t ws_bytes, void *stream) {
  Dims d;
  if (int e = check_model(a, d)) return e;
  if (!w || !w->tok_embeddings || !w->norm || !w->output || (d.L > 0 && !w->layers))
    return fail(LLAMA_ERR_ARG, "model weight pointer is NULL");
  for (int l = 0; l < d.L; ++l)
    if (int e = check_layer_w(&w->layers[l])) return e;
  if (!prompt || !prompt_len || !tokens || !out_len || !ws || (d.L > 0 && !kv))
    return fail(LLAMA_ERR_ARG, "prompt, prompt_len, kv, tokens, out_len or ws is NULL");
  for (int l = 0; l < d.L; ++l)
    if (!kv[l].k || !kv[l].v) return fail(LLAMA_ERR_ARG, "kv[%d] has a NULL pointer", l);
  if (batch < 1) return fail(LLAMA_ERR_ARG, "batch must be >= 1");
  if (batch > kGenMaxBatch) return fail(LLAMA_ERR_UNSUPPORTED, "generation batch %d above %d", batch, kGenMaxBatch);
  if (batch > a->max_batch_size) return fail(LLAMA_ERR_SHAPE, "batch %d > max_batch_size %d", batch, a->max_batch_size);
  if (max_gen_len < 0) return fail(LLAMA_ERR_ARG, "max_gen_len < 0");
  if (!(temperature >= 0.f)) return fail(LLAMA_ERR_ARG, "temperature must be >= 0");
  const bool samp = temperature > 0.f;
  if (samp) {
    if (!uniforms) return fail(LLAMA_ERR_ARG, "sampling needs uniforms");
    if (!(top_p >= 0.f)) return fail(LLAMA_ERR_ARG, "top_p must be >= 0");
    if (d.V > kSampleMaxVocab) return fail(LLAMA_ERR_UNSUPPORTED, "vocab %d above %d", d.V, kSampleMaxVocab);
  }
  const int cap = a->max_seq_len;
  if (cap < 1) return fail(LLAMA_ERR_SHAPE, "max_seq_len < 1");
  GenLens lens{};
  int Lmax = 0, steps = 0;
  for (int b = 0; b < batch; ++b) {
    const int L = prompt_len[b];
    if (L < 1 || L > cap) return fail(LLAMA_ERR_ARG, "prompt_len[%d] = %d outside [1, %d]", b, L, cap);
    lens.L[b] = L;
    lens.total[b] = (int32_t)std::min<int64_t>((int64_t)L + max_gen_len, cap);
    Lmax = std::max(Lmax, L);
    steps = std::max(steps, lens.total[b] - L - 1);  // decode steps after the prefill's choice
  }
  if (prompt_stride < Lmax) return fail(LLAMA_ERR_ARG, "prompt_stride %d < longest prompt %d", prompt_stride, Lmax);
  Carver probe(nullptr);
  carve_gen(probe, d, batch, Lmax, cap);
  if (ws_bytes < probe.off) return fail(LLAMA_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, probe.off);
  if ((uintptr_t)ws % 256) return fail(LLAMA_ERR_ARG, "workspace not 256-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  Carver c(ws);
  GenWs gw = carve_gen(c, d, batch, Lmax, cap);
  const int B = batch;
  bool any = false;
  for (int b = 0; b < B; ++b) any |= lens.total[b] > lens.L[b];

  LAUNCH("gen_fill", launch_gen_fill(prompt, prompt_stride, tokens, cap, lens, B, s));
  int32_t ran = 0;
  if (any) {
    // prompts: right-padded to the longest and prefilled together (at most
    // kGenPrefillTokens tokens per call); each sequence's first token comes
    // from its own last prompt row.  Padded positions repeat the prompt's
    // last token; no prompt row attends to them, and the decode step at
    // position p writes cache slot p before any later step reads it.
    std::vector<llama_kv> kvg(std::max(d.L, 1));
    const int gmax = gen_rows_per_call(Lmax, B);
    const size_t row_bytes = (size_t)cap * d.Hk() * d.esz;
    for (int b0 = 0; b0 < B; b0 += gmax) {
      const int g = std::min(gmax, B - b0);
      LAUNCH("gen_stage_ids", launch_gen_stage_ids(prompt, prompt_stride, lens, b0, g, Lmax, gw.ids, s));
      for (int l = 0; l < d.L; ++l) {
        kvg[l].k = static_cast<char *>(kv[l].k) + (size_t)b0 * row_bytes;
        kvg[l].v = static_cast<char *>(kv[l].v) + (size_t)b0 * row_bytes;
      }
      int32_t last[kGenMaxBatch];
      for (int i = 0; i < g; ++i) last[i] = lens.L[b0 + i] - 1;
      if (int e = prefill_impl(a, w, gw.ids, nullptr, g, Lmax, d.L > 0 ? kvg.data() : nullptr, nullptr,
                               samp ? gw.logits + (int64_t)b0 * d.V : nullptr, gw.st.next + b0, last, gw.rest,
                               gw.rest_bytes, stream))
        return e;
    }
    if (samp)
      LAUNCH("sample_top_p", launch_sample_top_p(gw.logits, d.V, B, d.V, temperature, top_p, uniforms,
                                                 std::max(max_gen_len, 1), nullptr, gw.st.next, s));
  }
  // the prefill's choice becomes each sequence's first generated token (a
  // sequence with nothing to generate parks on its last prompt position)
  LAUNCH("gen_step", launch_gen_step(gw.st, lens, B, eos_id, prompt, prompt_stride, tokens, cap, 1, s));
  if (any) {
    // one step: decode at each sequence's position, choose, append
    auto one_step = [&]() -> int {
      if (int e = llama_decode_step(a, w, gw.st.cur, gw.st.pos, B, kv, samp ? gw.logits : nullptr, gw.st.next,
                                    gw.rest, gw.rest_bytes, stream))
        return e;
      if (samp)
        LAUNCH("sample_top_p", launch_sample_top_p(gw.logits, d.V, B, d.V, temperature, top_p, uniforms,
                                                   std::max(max_gen_len, 1), gw.st.gidx, gw.st.next, s));
      LAUNCH("gen_step", launch_gen_step(gw.st, lens, B, eos_id, prompt, prompt_stride, tokens, cap, 0, s));
      return LLAMA_OK;
    };
    bool timing_on;
    {
      std::lock_guard<std::mutex> lk(g_timing.mu);
      timing_on = g_timing.on;
    }
    const bool use_graph = steps > 0 && (flags & LLAMA_GEN_GRAPH) && s != nullptr && !timing_on;
    hipGraphExec_t ge = nullptr;
    if (use_graph) {
      HIPCHK(hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal));
      const int e = one_step();
      hipGraph_t graph = nullptr;
      const hipError_t ec = hipStreamEndCapture(s, &graph);
      if (e) {
        if (graph) (void)hipGraphDestroy(graph);
        return e;
      }
      if (ec != hipSuccess) return fail(LLAMA_ERR_HIP, "hipStreamEndCapture: %s", hipGetErrorString(ec));
      const hipError_t ei = hipGraphInstantiate(&ge, graph, nullptr, nullptr, 0);
      (void)hipGraphDestroy(graph);
      if (ei != hipSuccess) return fail(LLAMA_ERR_HIP, "hipGraphInstantiate: %s", hipGetErrorString(ei));
    }
    int rc = LLAMA_OK;
    int32_t active = 1;
    for (int t = 0; t < steps && rc == LLAMA_OK; ++t) {
      if (t % kGenCheckEvery == 0) {
        hipError_t e1 = hipMemcpyAsync(&active, gw.st.active, sizeof active, hipMemcpyDeviceToHost, s);
        if (e1 == hipSuccess) e1 = hipStreamSynchronize(s);
        if (e1 != hipSuccess) {
          rc = fail(LLAMA_ERR_HIP, "reading the active count: %s", hipGetErrorString(e1));
          break;
        }
        if (!active) break;
      }
      if (ge) {
        const hipError_t e2 = hipGraphLaunch(ge, s);
        if (e2 != hipSuccess) rc = fail(LLAMA_ERR_HIP, "hipGraphLaunch: %s", hipGetErrorString(e2));
      } else {
        rc = one_step();
      }
      if (rc == LLAMA_OK) ++ran;
    }
    if (ge) {
      const hipError_t e3 = hipStreamSynchronize(s);
      (void)hipGraphExecDestroy(ge);
      if (rc == LLAMA_OK && e3 != hipSuccess) rc = fail(LLAMA_ERR_HIP, "hipStreamSynchronize: %s", hipGetErrorString(e3));
    }
    if (rc) return rc;
  }
  LAUNCH("gen_finish", launch_gen_finish(gw.st, B, eos_id, tokens, cap, out_len, s));
  if (steps_run) *steps_run = ran;
  return LLAMA_OK;
}

const char *llama_last_error(void) { return g_err.c_str(); }

int llama_timing_enable(int on) {
  std::lock_guard<std::mutex> lk(g_timing.mu);
  g_timing.on = on != 0;
  g_timing.recs.clear();
  g_timing.used = 0;
  return LLAMA_OK;
}

int64_t llama_timing_report(char *buf, size_t len) {
  std::lock_guard<std::mutex> lk(g_timing.mu);
  struct Agg {
    int64_t n = 0;
    double ms = 0.0;
  };
  std::map<std::string, Agg> agg;
  for (const TimingRec &r : g_timing.recs) {
    if (hipEventSynchronize(r.stop) != hipSuccess) return fail(LLAMA_ERR_HIP, "hipEventSynchronize failed");
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess) return fail(LLAMA_ERR_HIP, "hipEventElapsedTime failed");
    Agg &a = agg[r.name];
    a.n += 1;
    a.ms += ms;
  }
  std::string out;
  char line[256];
  for (const auto &kv : agg) {
    snprintf(line, sizeof line, "%s %lld %.6f\n", kv.first.c_str(), (long long)kv.second.n, kv.second.ms);
    out += line;
  }
  if (buf && len) {
    const size_t n = std::min(len - 1, out.size());
    memcpy(buf, out.data(), n);
    buf[n] = 0;
  }
  g_timing.recs.clear();
  g_timing.used = 0;
  return (int64_t)out.size() + 1;
}

}  // extern "C"
