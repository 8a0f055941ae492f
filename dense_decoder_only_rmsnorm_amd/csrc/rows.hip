// Row-wise kernels: embedding gather, RMSNorm (with optional split-K partial
// accumulation into the residual stream), RoPE table, RoPE + KV-cache write,
// SwiGLU gate (fp32 path), argmax reduction.
//
// Pages: [P1] llama3-from-scratch translation (sections 4, 5, 6.6-6.9, 9.3, 12);
//        [P2] "Build your own Llama 3" notes (sections 3.1-3.5);
//        [P3] llama3-from-scratch output layer page (steps 1-4).
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace llk {

// ---------------------------------------------------------------------------
// Embedding lookup [P1 4; P2 4 tok_embeddings]: h[r, :] = E[ids[r], :] as fp32.
// Ids outside [0, V) produce NaN rows instead of an out-of-bounds read.
// One block per row; each thread moves 16-byte pieces: 8 bf16 (or 4 fp32)
// table elements per load, written as fp32 with 16-byte stores.  D must be a
// multiple of 8 (bf16) or 4 (fp32); rows are 16-byte aligned.
// ---------------------------------------------------------------------------
template <typename TW>
__global__ __launch_bounds__(256) void embed_kernel(const int32_t *__restrict__ ids, const TW *__restrict__ E,
                                                    float *__restrict__ h, int D, int V) {
  constexpr int EPL = 16 / sizeof(TW);  // table elements per 16-byte load
  const int r = blockIdx.x;
  const int id = ids[r];
  float *dst = h + (int64_t)r * D;
  const bool ok = id >= 0 && id < V;
  const TW *src = E + (int64_t)(ok ? id : 0) * D;
  const float qnan = __int_as_float(0x7fc00000);
  // every piece of the row is loaded before the first store (D <= 8192)
  constexpr int MAXP = 8192 / (256 * EPL);
  uint4 raws[MAXP];
#pragma unroll
  for (int k = 0; k < MAXP; ++k) {
    const int i = (k * 256 + threadIdx.x) * EPL;
    raws[k] = make_uint4(0, 0, 0, 0);
    if (i < D) raws[k] = *reinterpret_cast<const uint4 *>(src + i);
  }
#pragma unroll
  for (int k = 0; k < MAXP; ++k) {
    const int i = (k * 256 + threadIdx.x) * EPL;
    if (i >= D) break;
    const uint4 raw = raws[k];
    if (EPL == 8) {
      const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
      float4 lo, hi;
      lo.x = __uint_as_float(w[0] << 16); lo.y = __uint_as_float(w[0] & 0xffff0000u);
      lo.z = __uint_as_float(w[1] << 16); lo.w = __uint_as_float(w[1] & 0xffff0000u);
      hi.x = __uint_as_float(w[2] << 16); hi.y = __uint_as_float(w[2] & 0xffff0000u);
      hi.z = __uint_as_float(w[3] << 16); hi.w = __uint_as_float(w[3] & 0xffff0000u);
      if (!ok) lo = hi = make_float4(qnan, qnan, qnan, qnan);
      *reinterpret_cast<float4 *>(dst + i) = lo;
      *reinterpret_cast<float4 *>(dst + i + 4) = hi;
    } else {
      float4 v = make_float4(__uint_as_float(raw.x), __uint_as_float(raw.y), __uint_as_float(raw.z),
                             __uint_as_float(raw.w));
      if (!ok) v = make_float4(qnan, qnan, qnan, qnan);
      *reinterpret_cast<float4 *>(dst + i) = v;
    }
  }
}

// ---------------------------------------------------------------------------
// RMSNorm [P1 5; P2 3.1; P3 step 1]: y = x / sqrt(mean(x^2) + eps) * w, with
// the mean over the model dimension, eps inside the root and the weight
// applied after normalising.  fp32 arithmetic, one rounding at the store.
//
// Optionally first folds split-K partial sums into the residual stream:
//   x[r] += sum_s part[s][r]   (written back to x).
// w == nullptr skips the normalisation (pure conversion of x).
// Output modes: 0 fp32, 1 bf16, 2 bf16 hi/lo planes (hi at out, lo at
// out + out_plane).  One block of NT threads per row; D <= 8192.  Few rows
// (decode) use NT = 1024 so that the partial planes stream with enough
// loads in flight.
// ---------------------------------------------------------------------------
template <typename TW, int MODE, int NT, int NV>
__global__ __launch_bounds__(NT) void rmsnorm_kernel(NormArgs a) {
  // NV > 0: D is exactly NV * NT * 4, every lane holds NV pieces and no
  // piece needs a guard (the guards' branches make the compiler wait for
  // each store before the next); NV == 0: any D <= 8192
  constexpr int MAXV = NV > 0 ? NV : 8192 / (NT * 4);
  const int r = blockIdx.x;
  const int D = a.D;
  float *x = a.h + a.in_offset + (int64_t)r * a.in_stride;
  float4 v[MAXV];
  float ss = 0.f;
  // the row's loads and the weight loads first, all in flight together (a
  // store the compiler cannot tell apart from the weights would make every
  // later load wait for it); then the folds and sums
  const TW *w = static_cast<const TW *>(a.w);
  using WRaw = typename std::conditional<std::is_same<TW, float>::value, float4, uint2>::type;
  WRaw wraw[MAXV];  // raw 4-element pieces, converted at their use
#pragma unroll
  for (int j = 0; j < MAXV; ++j) {
    const int i = (j * NT + threadIdx.x) * 4;
    v[j] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (NV > 0 || i < D) v[j] = *reinterpret_cast<const float4 *>(x + i);
    // (without weights the row itself is read in their place and ignored, so
    // the load is not behind a branch that would wait for it)
    const WRaw *wp = w != nullptr ? reinterpret_cast<const WRaw *>(w + i) : reinterpret_cast<const WRaw *>(x + i);
    wraw[j] = WRaw{};
    if (NV > 0 || i < D) wraw[j] = *wp;
  }
  // Split-K partials in groups of 8: a group's loads (clamped to a valid
  // plane, the extra ones weighted 0) are issued together instead of one
  // latency per plane.  The few-row (decode) variants issue the first group
  // with the row loads above, ahead of the loop.
  constexpr int PG = NT == 1024 ? MAXV : 1;
  float4 p0[PG][8];
  if (NT == 1024 && a.nsplit > 0) {
#pragma unroll
    for (int j = 0; j < PG; ++j) {
      const int i = (j * NT + threadIdx.x) * 4;
      if (NV > 0 || i < D) {
#pragma unroll
        for (int u = 0; u < 8; ++u)
          p0[j][u] = *reinterpret_cast<const float4 *>(a.part + min(u, a.nsplit - 1) * a.part_stride + (int64_t)r * D + i);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < MAXV; ++j) {
    const int i = (j * NT + threadIdx.x) * 4;
    if (NV > 0 || i < D) {
      float4 t = v[j];
      if (a.nsplit > 0) {
        for (int s0 = 0; s0 < a.nsplit; s0 += 8) {
          float4 p[8];
          if (NT == 1024 && s0 == 0) {
#pragma unroll
            for (int u = 0; u < 8; ++u) p[u] = p0[j < PG ? j : 0][u];
          } else {
#pragma unroll
            for (int u = 0; u < 8; ++u)
              p[u] = *reinterpret_cast<const float4 *>(a.part + min(s0 + u, a.nsplit - 1) * a.part_stride + (int64_t)r * D + i);
          }
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const float m = s0 + u < a.nsplit ? 1.f : 0.f;
            t.x += m * p[u].x; t.y += m * p[u].y; t.z += m * p[u].z; t.w += m * p[u].w;
          }
        }
        *reinterpret_cast<float4 *>(x + i) = t;
      }
      v[j] = t;
      ss += t.x * t.x + t.y * t.y + t.z * t.z + t.w * t.w;
    }
  }
  float scale = 1.f;
  if (a.w != nullptr) {
    __shared__ float red[NT / 64];
    ss = wave_sum(ss);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) tot += red[w];
    scale = 1.0f / sqrtf(tot / (float)D + a.eps);
  }
  // the outputs are formed before the guarded stores (the empty asm keeps
  // the compiler from sinking them into the branches, where each would wait
  // for the loads and for the previous store again)
  float yv[MAXV][4];
#pragma unroll
  for (int j = 0; j < MAXV; ++j) {
    yv[j][0] = v[j].x * scale;
    yv[j][1] = v[j].y * scale;
    yv[j][2] = v[j].z * scale;
    yv[j][3] = v[j].w * scale;
    if (w != nullptr) {
      const TW *we = reinterpret_cast<const TW *>(&wraw[j]);
#pragma unroll
      for (int e = 0; e < 4; ++e) yv[j][e] *= Elem<TW>::load(we + e);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) asm volatile("" : "+v"(yv[j][e]));
  }
#pragma unroll
  for (int j = 0; j < MAXV; ++j) {
    const int i = (j * NT + threadIdx.x) * 4;
    if (NV > 0 || i < D) {
      const float *y = yv[j];
      const int64_t o = (int64_t)r * D + i;
      if (MODE == 0) {
        *reinterpret_cast<float4 *>(static_cast<float *>(a.out) + o) = make_float4(y[0], y[1], y[2], y[3]);
      } else if (MODE == 1) {
        u16 *p = static_cast<u16 *>(a.out) + o;
        uint2 pk;
        pk.x = (uint32_t)f2bf(y[0]) | ((uint32_t)f2bf(y[1]) << 16);
        pk.y = (uint32_t)f2bf(y[2]) | ((uint32_t)f2bf(y[3]) << 16);
        *reinterpret_cast<uint2 *>(p) = pk;
      } else {
        u16 hi[4], lo[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) split_hilo(y[e], hi[e], lo[e]);
        u16 *p = static_cast<u16 *>(a.out) + o;
        uint2 ph, pl;
        ph.x = (uint32_t)hi[0] | ((uint32_t)hi[1] << 16);
        ph.y = (uint32_t)hi[2] | ((uint32_t)hi[3] << 16);
        pl.x = (uint32_t)lo[0] | ((uint32_t)lo[1] << 16);
        pl.y = (uint32_t)lo[2] | ((uint32_t)lo[3] << 16);
        *reinterpret_cast<uint2 *>(p) = ph;
        *reinterpret_cast<uint2 *>(p + a.out_plane) = pl;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// RoPE table [P2 3.2 precompute_freqs_cis; P1 6.7]: for table row r at
// position p_r and pair i < hd/2, tab[r][i] = (cos, sin)(p_r * theta_i) with
// theta_i = rope_theta^(-2i/hd).  The angle and its cosine/sine are evaluated
// in fp64 and rounded once to fp32, so large positions keep full accuracy.
// p_r = pos[r] (clamped to [0, pos_max]) when pos != nullptr, else
// start_pos + r.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void rope_table_kernel(float2 *__restrict__ tab, const int32_t *__restrict__ pos,
                                                         int start_pos, int pos_max, int rows, int half,
                                                         double log2_theta) {
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= rows * half) return;
  const int r = idx / half, i = idx % half;
  int p = pos ? pos[r] : start_pos + r;
  p = p < 0 ? 0 : (p > pos_max ? pos_max : p);
  const double inv_freq = exp2(-(2.0 * i / (2.0 * half)) * log2_theta);
  double s, c;
  sincos((double)p * inv_freq, &s, &c);
  tab[idx] = make_float2((float)c, (float)s);
}

// ---------------------------------------------------------------------------
// RoPE + KV-cache write for Q/K/V rows held in fp32 (split-K partials summed
// first) [P2 3.2 apply_rotary_emb, 3.3-3.4 cache write; P1 6.8-6.10].
//   qkv row r = [q (H*hd) | k (G*hd) | v (G*hd)], sum over nsplit partials.
//   q, k: adjacent pairs rotated by the table row of r; v copied.
//   q -> qout[r][H*hd] (fp32), qbf (bf16) and/or qhl (scaled hi/lo planes);
//   k, v -> cache[b][p][g][hd] (TC), where
//   b = r / S, s = r % S and p = (pos ? clamp(pos[b]) : start_pos) + s.
// One thread per pair.
// ---------------------------------------------------------------------------
template <typename TC>
__global__ __launch_bounds__(256) void rope_qkv_kernel(RopeQkvArgs a) {
  const int npair = (a.H + 2 * a.G) * a.hd / 2;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)a.rows * npair) return;
  const int r = (int)(idx / npair);
  const int j = (int)(idx % npair) * 2;  // even column
  const int N = (a.H + 2 * a.G) * a.hd;
  const int Hq = a.H * a.hd, Hk = a.G * a.hd;
  const int b = r / a.S, sidx = r % a.S;
  // the loads that do not depend on the partial sums go out first: the
  // sequence's position and the table entry (v columns read a valid entry
  // and keep their values)
  int p0 = a.pos ? a.pos[b] : a.start_pos;
  const int tr = a.tab_mod > 0 ? (r % a.tab_mod) : r;
  const bool rot = j < Hq + Hk;
  const int dcol = (j < Hq ? j : (rot ? j - Hq : 0)) % a.hd;
  const float2 cs = a.tab[(int64_t)tr * (a.hd / 2) + dcol / 2];
  float x0 = 0.f, x1 = 0.f;
  for (int s0 = 0; s0 < a.nsplit; s0 += 8) {  // loads of 8 partials at a time (see rmsnorm_kernel)
    float2 t[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      t[u] = *reinterpret_cast<const float2 *>(a.part + min(s0 + u, a.nsplit - 1) * a.part_stride + (int64_t)r * N + j);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float m = s0 + u < a.nsplit ? 1.f : 0.f;
      x0 += m * t[u].x;
      x1 += m * t[u].y;
    }
  }
  p0 = p0 < 0 ? 0 : (p0 > a.cap - 1 ? a.cap - 1 : p0);
  int p = p0 + sidx;
  p = p > a.cap - 1 ? a.cap - 1 : p;
  {
    const float2 y = rotate_pair(x0, x1, cs.x, cs.y);
    x0 = rot ? y.x : x0;
    x1 = rot ? y.y : x1;
  }
  if (j < Hq) {
    if (a.qout) *reinterpret_cast<float2 *>(a.qout + (int64_t)r * Hq + j) = make_float2(x0, x1);
    if (a.qbf)
      *reinterpret_cast<uint32_t *>(a.qbf + (int64_t)r * Hq + j) = (uint32_t)f2bf(x0) | ((uint32_t)f2bf(x1) << 16);
    if (a.qhl) {
      u16 h0, l0, h1, l1;
      split_hilo(x0 * a.qscale, h0, l0);
      split_hilo(x1 * a.qscale, h1, l1);
      const int64_t o = (int64_t)r * Hq + j;
      *reinterpret_cast<uint32_t *>(a.qhl + o) = (uint32_t)h0 | ((uint32_t)h1 << 16);
      *reinterpret_cast<uint32_t *>(a.qhl + (int64_t)a.rows * Hq + o) = (uint32_t)l0 | ((uint32_t)l1 << 16);
    }
  } else {
    const bool isk = j < Hq + Hk;
    const int c = isk ? j - Hq : j - Hq - Hk;
    const int g = c / a.hd, d = c % a.hd;
    TC *base = static_cast<TC *>(isk ? a.kc : a.vc);
    TC *dst = base + (((int64_t)b * a.cap + p) * a.G + g) * a.hd + d;
    Elem<TC>::store(dst, x0);
    Elem<TC>::store(dst + 1, x1);
    float *fn = isk ? a.knew : a.vnew;
    if (fn) *reinterpret_cast<float2 *>(fn + (int64_t)r * Hk + c) = make_float2(x0, x1);
  }
}

// SwiGLU gate for the fp32 path [P2 3.5; P1 9.3]: u = silu(gate) * up.
__global__ __launch_bounds__(256) void swiglu_kernel(const float *__restrict__ gate, const float *__restrict__ up,
                                                     float *__restrict__ u, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) u[i] = silu(gate[i]) * up[i];
}

// ---------------------------------------------------------------------------
// Argmax over per-block partial maxima [P1 12; P3 4]: for each row pick the
// largest value, and among equal values the smallest index.
// part_val/part_idx: [rows][nblk].
// ---------------------------------------------------------------------------
__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

__global__ __launch_bounds__(256) void argmax_reduce_kernel(const float *__restrict__ part_val,
                                                            const int32_t *__restrict__ part_idx, int nblk,
                                                            int32_t *__restrict__ out) {
  const int r = blockIdx.x;
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  for (int j = threadIdx.x; j < nblk; j += 256) {
    const float v = part_val[(int64_t)r * nblk + j];
    const int i = part_idx[(int64_t)r * nblk + j];
    if (better(v, i, bv, bi)) { bv = v; bi = i; }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float v = __shfl_xor(bv, o, kWave);
    const int i = __shfl_xor(bi, o, kWave);
    if (better(v, i, bv, bi)) { bv = v; bi = i; }
  }
  __shared__ float sv[4];
  __shared__ int si[4];
  if ((threadIdx.x & 63) == 0) { sv[threadIdx.x >> 6] = bv; si[threadIdx.x >> 6] = bi; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < 4; ++w)
      if (better(sv[w], si[w], bv, bi)) { bv = sv[w]; bi = si[w]; }
    out[r] = bi == 0x7fffffff ? 0 : bi;
  }
}

// Row-wise argmax of a dense fp32 [rows][n] matrix into per-block partials
// (fp32 path LM head).  Block (r, j) scans columns [j*chunk, (j+1)*chunk).
__global__ __launch_bounds__(256) void argmax_partial_kernel(const float *__restrict__ x, int n, int chunk,
                                                             float *__restrict__ part_val,
                                                             int32_t *__restrict__ part_idx, int nblk) {
  const int r = blockIdx.y, j = blockIdx.x;
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  const int c1 = min(n, (j + 1) * chunk);
  for (int c = j * chunk + threadIdx.x; c < c1; c += 256) {
    const float v = x[(int64_t)r * n + c];
    if (better(v, c, bv, bi)) { bv = v; bi = c; }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float v = __shfl_xor(bv, o, kWave);
    const int i = __shfl_xor(bi, o, kWave);
    if (better(v, i, bv, bi)) { bv = v; bi = i; }
  }
  __shared__ float sv[4];
  __shared__ int si[4];
  if ((threadIdx.x & 63) == 0) { sv[threadIdx.x >> 6] = bv; si[threadIdx.x >> 6] = bi; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < 4; ++w)
      if (better(sv[w], si[w], bv, bi)) { bv = sv[w]; bi = si[w]; }
    part_val[(int64_t)r * nblk + j] = bv;
    part_idx[(int64_t)r * nblk + j] = bi;
  }
}

// ---------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------
hipError_t launch_embed(int dtype, const int32_t *ids, const void *E, float *h, int rows, int D, int V,
                        hipStream_t s) {
  if (dtype == 0)
    hipLaunchKernelGGL(embed_kernel<float>, dim3(rows), dim3(256), 0, s, ids, (const float *)E, h, D, V);
  else
    hipLaunchKernelGGL(embed_kernel<u16>, dim3(rows), dim3(256), 0, s, ids, (const u16 *)E, h, D, V);
  return hipGetLastError();
}

hipError_t launch_rmsnorm(int dtype, int mode, const NormArgs &a, int rows, hipStream_t s) {
#define LLK_NORM(TW, M)                                                                           \
  do {                                                                                            \
    if (rows < 512 && a.D == 4096)                                                                \
      hipLaunchKernelGGL((rmsnorm_kernel<TW, M, 1024, 1>), dim3(rows), dim3(1024), 0, s, a);     \
    else if (rows < 512)                                                                          \
      hipLaunchKernelGGL((rmsnorm_kernel<TW, M, 1024, 0>), dim3(rows), dim3(1024), 0, s, a);     \
    else if (a.D == 4096)                                                                         \
      hipLaunchKernelGGL((rmsnorm_kernel<TW, M, 256, 4>), dim3(rows), dim3(256), 0, s, a);       \
    else                                                                                          \
      hipLaunchKernelGGL((rmsnorm_kernel<TW, M, 256, 0>), dim3(rows), dim3(256), 0, s, a);       \
  } while (0)
  if (dtype == 0) {
    if (mode == 0) LLK_NORM(float, 0);
    else if (mode == 1) LLK_NORM(float, 1);
    else LLK_NORM(float, 2);
  } else {
    if (mode == 0) LLK_NORM(u16, 0);
    else if (mode == 1) LLK_NORM(u16, 1);
    else LLK_NORM(u16, 2);
  }
#undef LLK_NORM
  return hipGetLastError();
}

hipError_t launch_rope_table(float2 *tab, const int32_t *pos, int start_pos, int pos_max, int rows, int hd,
                             double theta, hipStream_t s) {
  const int n = rows * (hd / 2);
  hipLaunchKernelGGL(rope_table_kernel, dim3((n + 255) / 256), dim3(256), 0, s, tab, pos, start_pos, pos_max, rows,
                     hd / 2, log2(theta));
  return hipGetLastError();
}

hipError_t launch_rope_qkv(int dtype, const RopeQkvArgs &a, hipStream_t s) {
  const int64_t n = (int64_t)a.rows * ((a.H + 2 * a.G) * a.hd / 2);
  const dim3 grid((unsigned)((n + 255) / 256));
  if (dtype == 0)
    hipLaunchKernelGGL(rope_qkv_kernel<float>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(rope_qkv_kernel<u16>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_swiglu(const float *gate, const float *up, float *u, int64_t n, hipStream_t s) {
  hipLaunchKernelGGL(swiglu_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, gate, up, u, n);
  return hipGetLastError();
}

hipError_t launch_argmax_reduce(const float *pv, const int32_t *pi, int rows, int nblk, int32_t *out,
                                hipStream_t s) {
  hipLaunchKernelGGL(argmax_reduce_kernel, dim3(rows), dim3(256), 0, s, pv, pi, nblk, out);
  return hipGetLastError();
}

hipError_t launch_argmax_partial(const float *x, int rows, int n, int chunk, float *pv, int32_t *pi, int nblk,
                                 hipStream_t s) {
  hipLaunchKernelGGL(argmax_partial_kernel, dim3(nblk, rows), dim3(256), 0, s, x, n, chunk, pv, pi, nblk);
  return hipGetLastError();
}

}  // namespace llk
