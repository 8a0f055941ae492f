// Token-generation loop state and the temperature / top-p sampler.
//
// Generation (P2 "Inference" section, the generate loop): after each
// sequence's prompt, every step appends the model's choice for the next
// position until the sequence has produced its end-of-text token or reached
// its total length min(prompt + max_gen, max_seq_len).  The per-sequence
// state lives in device memory so that a whole step (decode + this update)
// can be replayed as one captured graph without host round trips.
//
// Sampling (P2 "Inference", sample_top_p; P3 temperature softmax): the
// probabilities softmax(logits / T) are cut to the nucleus (the longest
// prefix of the descending-probability order whose mass before each member
// is at most top_p, ties ordered by token id), renormalised, and one token is
// drawn with a caller-supplied uniform u in [0, 1) by inverse CDF over the
// kept tokens in token-id order.
//
// Exactness of the sampler's decisions: each probability is carried as the
// fixed-point integer q_i = floor(2^40 * z_i), z_i = 2^((l_i - max) * log2e / T)
// in fp32.  Every sum (total, nucleus mass, prefix mass) is an exact u64 sum,
// so the nucleus cut and the draw are independent of summation order: the
// kernel's choice is a deterministic function of the logits, T, top_p and u.
// The nucleus threshold is found by a 4-pass radix select (8 bits per pass)
// over the fp32 bit pattern of z (monotone for z >= 0), with mass-weighted
// histograms.
#include "common.h"
#include "kernels.h"

namespace llk {

// ---------------------------------------------------------------------------
// generation state
// ---------------------------------------------------------------------------
// tokens[b][j] = prompt[b][j] for j < L[b], -1 after.  Grid (ceil(tstride/256), B).
__global__ __launch_bounds__(256) void gen_fill_kernel(const int32_t *__restrict__ prompt, int64_t pstride,
                                                       int32_t *__restrict__ tokens, int64_t tstride, GenLens lens) {
  const int b = blockIdx.y;
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (j >= tstride) return;
  tokens[(int64_t)b * tstride + j] = j < lens.L[b] ? prompt[(int64_t)b * pstride + j] : -1;
}

// One block of 64 threads (B <= 64).  first = 1: take the prefill's choice
// (next[b]) as the token at position L[b]; first = 0: append next[b] at
// pos[b] + 1 for sequences still running.  Afterwards cur/pos hold the token
// and position the next decode step feeds, gidx the index (0-based, counted
// from the first generated token) of the token that step will produce, and
// active[0] the number of running sequences.
__global__ __launch_bounds__(64) void gen_step_kernel(GenState st, GenLens lens, int B, int eos,
                                                      const int32_t *__restrict__ prompt, int64_t pstride,
                                                      int32_t *__restrict__ tokens, int64_t tstride, int first) {
  const int b = threadIdx.x;
  int running = 0;
  if (b < B) {
    const int L = lens.L[b], tot = lens.total[b];
    if (first) {
      if (L >= tot) {
        // nothing to generate: park on the prompt's last position (the decode
        // steps of other sequences recompute it without effect on the output)
        st.done[b] = 1;
        st.pos[b] = L - 1;
        st.cur[b] = prompt[(int64_t)b * pstride + L - 1];
        st.end[b] = L;
        st.gidx[b] = 0;
      } else {
        const int tok = st.next[b];
        tokens[(int64_t)b * tstride + L] = tok;
        st.end[b] = L + 1;
        st.done[b] = (eos >= 0 && tok == eos) || L + 1 >= tot;
        st.cur[b] = tok;
        st.pos[b] = L;
        st.gidx[b] = 1;
      }
    } else if (!st.done[b]) {
      const int p = st.pos[b] + 1;
      const int tok = st.next[b];
      tokens[(int64_t)b * tstride + p] = tok;
      st.end[b] = p + 1;
      st.done[b] = (eos >= 0 && tok == eos) || p + 1 >= tot;
      st.cur[b] = tok;
      st.pos[b] = p;
      st.gidx[b] = p + 1 - L;
    }
    running = !st.done[b];
  }
  const uint64_t m = __ballot(running);
  if (b == 0) st.active[0] = __popcll(m);
}

// Prompt rows for one padded prefill: ids[i][j] = prompt[b0 + i][j] for
// j < L, else the prompt's last token (the padded positions are never
// attended to by the prompt's own rows and are overwritten by decode
// before they are read).  Grid (ceil(S/256), g).
__global__ __launch_bounds__(256) void gen_stage_ids_kernel(const int32_t *__restrict__ prompt, int64_t pstride,
                                                            GenLens lens, int b0, int S, int32_t *__restrict__ ids) {
  const int i = blockIdx.y;
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= S) return;
  const int L = lens.L[b0 + i];
  ids[(int64_t)i * S + j] = prompt[(int64_t)(b0 + i) * pstride + min(j, L - 1)];
}

// out[i][:] = h[rows.r[i]][:] (D floats).  Grid n.
__global__ __launch_bounds__(256) void gather_rows_kernel(const float *__restrict__ h, int D, RowList rows,
                                                          float *__restrict__ out) {
  const int i = blockIdx.x;
  const float4 *src = reinterpret_cast<const float4 *>(h + (int64_t)rows.r[i] * D);
  float4 *dst = reinterpret_cast<float4 *>(out + (int64_t)i * D);
  for (int c = threadIdx.x; c < D / 4; c += 256) dst[c] = src[c];
}

// out_len[b] = index of the first end-of-text token in tokens[b][0, end[b]),
// else end[b] (the output is cut at the first end-of-text token).  Grid B.
__global__ __launch_bounds__(256) void gen_finish_kernel(GenState st, int eos, const int32_t *__restrict__ tokens,
                                                         int64_t tstride, int32_t *__restrict__ out_len) {
  const int b = blockIdx.x;
  const int end = st.end[b];
  int first = end;
  if (eos >= 0)
    for (int j = threadIdx.x; j < end; j += 256)
      if (tokens[(int64_t)b * tstride + j] == eos) { first = min(first, j); break; }
  __shared__ int sm[4];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) first = min(first, __shfl_xor(first, o, kWave));
  if ((threadIdx.x & 63) == 0) sm[threadIdx.x >> 6] = first;
  __syncthreads();
  if (threadIdx.x == 0) out_len[b] = min(min(sm[0], sm[1]), min(sm[2], sm[3]));
}

// ---------------------------------------------------------------------------
// sampler
// ---------------------------------------------------------------------------
constexpr int kSampThreads = 1024;
constexpr int kSampWaves = kSampThreads / kWave;
constexpr float kFix = 1099511627776.0f;  // 2^40

__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Block-wide u64 sum; every thread gets the result.  red: kSampWaves slots.
__device__ __forceinline__ uint64_t block_sum_u64(uint64_t v, uint64_t *red) {
  v = wave_sum_u64(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  uint64_t t = 0;
#pragma unroll
  for (int w = 0; w < kSampWaves; ++w) t += red[w];
  return t;
}

// Radix digits of the 32-bit key, most significant first.  Bits 31..30 are
// zero for every z in [0, 1] (sign 0, exponent at most 127), so the first
// digit is bits 29..22: the exponent spread over ~80 buckets instead of the
// ~20 the top byte would use, which keeps the histogram atomics apart.
__device__ __forceinline__ int digit_shift(int pass) { return pass < 3 ? 22 - 8 * pass : 0; }
__device__ __forceinline__ int digit_bits(int pass) { return pass < 3 ? 8 : 6; }

// One block per row.  logits [M][ld] fp32; u [urows][M] (row of each logits
// row chosen by gidx[r], clamped to urows - 1, or row 0 when gidx is null).
__global__ __launch_bounds__(kSampThreads) void sample_top_p_kernel(const float *__restrict__ logits, int64_t ld,
                                                                    int V, float k2, float top_p,
                                                                    const float *__restrict__ u, int M, int urows,
                                                                    const int32_t *__restrict__ gidx,
                                                                    int32_t *__restrict__ out) {
  const int r = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const float *x = logits + (int64_t)r * ld;
  __shared__ uint64_t hist[kSampWaves][256];  // one histogram per wave (fewer colliding atomics)
  __shared__ uint64_t red[kSampWaves];
  __shared__ float redf[kSampWaves];
  __shared__ uint64_t sel_mass;   // mass of keys above the selected prefix
  __shared__ uint32_t sel_digit;
  __shared__ uint64_t wmass[kSampWaves];
  __shared__ uint32_t wties[kSampWaves];
  __shared__ int picked;
  if (tid == 0) picked = 0;

  // max
  float mx = -INFINITY;
  for (int i = tid; i < V; i += kSampThreads) mx = fmaxf(mx, x[i]);
  mx = wave_max(mx);
  if (lane == 0) redf[wv] = mx;
  __syncthreads();
  mx = redf[0];
#pragma unroll
  for (int w = 1; w < kSampWaves; ++w) mx = fmaxf(mx, redf[w]);

  auto zkey = [&](int i, uint64_t &q) -> uint32_t {
    const float z = exp2f((x[i] - mx) * k2);
    q = (z > 0.f && z <= 1.f) ? (uint64_t)(z * kFix) : 0ull;  // NaN (non-finite logits) carries no mass
    return __float_as_uint(z);
  };
  uint64_t *hflat = &hist[0][0];
  // merge the per-wave histograms into hist[0] (thread t owns bucket t)
  auto merge_hist = [&]() {
    __syncthreads();
    if (tid < 256) {
      uint64_t t = 0;
#pragma unroll
      for (int w = 0; w < kSampWaves; ++w) t += hist[w][tid];
      hist[0][tid] = t;
    }
    __syncthreads();
  };

  // total mass + first histogram
  for (int i = tid; i < kSampWaves * 256; i += kSampThreads) hflat[i] = 0;
  __syncthreads();
  uint64_t tot = 0;
  for (int i = tid; i < V; i += kSampThreads) {
    uint64_t q;
    const uint32_t key = zkey(i, q);
    if (q) {
      tot += q;
      atomicAdd((unsigned long long *)&hist[wv][(key >> 22) & 255], (unsigned long long)q);
    }
  }
  const uint64_t Z = block_sum_u64(tot, red);

  // threshold key t* = the largest key with mass(keys >= t*) > top_p * Z,
  // and the number of tokens with key == t* that stay in the nucleus
  uint32_t thr = 0;
  uint64_t above = 0;  // mass of keys > t*
  uint64_t take = 0xFFFFFFFFull;
  const bool keep_all = !(top_p < 1.0f);
  if (!keep_all) {
    const uint64_t R = (uint64_t)((double)top_p * (double)Z);
    uint32_t prefix = 0;
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = digit_shift(pass), nb = 1 << digit_bits(pass);
      if (pass > 0) {
        __syncthreads();
        for (int i = tid; i < kSampWaves * 256; i += kSampThreads) hflat[i] = 0;
        __syncthreads();
        const int hi = shift + digit_bits(pass);  // bits at and above hi are fixed by the prefix
        for (int i = tid; i < V; i += kSampThreads) {
          uint64_t q;
          const uint32_t key = zkey(i, q);
          if (q && (key >> hi) == (prefix >> hi))
            atomicAdd((unsigned long long *)&hist[wv][(key >> shift) & (nb - 1)], (unsigned long long)q);
        }
      }
      merge_hist();
      // wave 0: the largest digit d with above + sum(hist[d..]) > R
      if (tid < 64) {
        const uint64_t h0 = hist[0][4 * tid], h1 = hist[0][4 * tid + 1], h2 = hist[0][4 * tid + 2],
                       h3 = hist[0][4 * tid + 3];
        const uint64_t mine = h0 + h1 + h2 + h3;  // buckets past nb are zero
        uint64_t suf = mine;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const uint64_t t = __shfl_down(suf, o, kWave);
          if (tid + o < 64) suf += t;
        }
        const uint64_t base = above + (suf - mine);  // mass of the digits above this lane's four
        int d = -1;
        uint64_t dm = 0;
        if (base + h3 > R) { d = 4 * tid + 3; dm = base; }
        else if (base + h3 + h2 > R) { d = 4 * tid + 2; dm = base + h3; }
        else if (base + h3 + h2 + h1 > R) { d = 4 * tid + 1; dm = base + h3 + h2; }
        else if (base + mine > R) { d = 4 * tid; dm = base + h3 + h2 + h1; }
        // the crossing lies in exactly one lane (the suffix mass is monotone)
        const uint64_t hit = __ballot(d >= 0);
        const int src = hit ? 63 - __clzll(hit) : 0;
        if (tid == src) {
          sel_digit = d >= 0 ? (uint32_t)d : 0u;
          sel_mass = d >= 0 ? dm : above;
        }
      }
      __syncthreads();
      prefix |= sel_digit << shift;
      above = sel_mass;
    }
    thr = prefix;
    // tokens with key == t* all carry q* = floor(2^40 * z(t*)); the first j of
    // them (by id) are kept, j = floor((R - above) / q*) + 1
    const uint64_t qs = (uint64_t)(__uint_as_float(thr) * kFix);
    take = qs ? (R - above) / qs + 1 : 0;
  }
  const uint64_t qs = keep_all ? 0 : (uint64_t)(__uint_as_float(thr) * kFix);

  // kept mass and ties per wave over contiguous id ranges (coalesced, 64 ids a step)
  const int chunk = (((V + kSampWaves - 1) / kSampWaves) + 63) & ~63;
  const int w0 = wv * chunk, w1 = min(V, w0 + chunk);
  uint64_t m_gt = 0;
  uint32_t n_tie = 0;
  for (int i = w0 + lane; i < w1; i += 64) {
    uint64_t q;
    const uint32_t key = zkey(i, q);
    if (!q) continue;
    if (keep_all || key > thr) m_gt += q;
    else if (key == thr) ++n_tie;
  }
  m_gt = wave_sum_u64(m_gt);
  uint32_t nt = n_tie;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) nt += __shfl_xor(nt, o, kWave);
  if (lane == 0) {
    wmass[wv] = m_gt;
    wties[wv] = nt;
  }
  __syncthreads();
  // per wave: ties before it (in id order), its kept mass (its ties stay
  // while their rank is below take); prefix over the waves before this one
  uint32_t tp = 0, tie0 = 0;
  uint64_t pre = 0, Mk = 0, mine = 0;
  for (int w = 0; w < kSampWaves; ++w) {
    const uint64_t kt = keep_all ? 0 : min((uint64_t)wties[w], take > tp ? take - tp : 0ull);
    const uint64_t mw = wmass[w] + kt * qs;
    if (w < wv) pre += mw;
    if (w == wv) {
      tie0 = tp;
      mine = mw;
    }
    Mk += mw;
    tp += wties[w];
  }

  const int urow = gidx ? min(max(gidx[r], 0), urows - 1) : 0;
  const float uu = u[(int64_t)urow * M + r];
  uint64_t target = (uint64_t)((double)uu * (double)Mk);
  if (Mk && target >= Mk) target = Mk - 1;
  // the wave whose kept range [pre, pre + mine) holds the target walks it in
  // id order, 64 ids a step, with a wave-wide inclusive scan of the kept mass
  if (mine && target >= pre && target < pre + mine) {
    uint64_t acc = pre;
    uint32_t rank = tie0;
    for (int i0 = w0; i0 < w1; i0 += 64) {
      const int i = i0 + lane;
      uint64_t q = 0;
      uint32_t key = 0;
      if (i < w1) key = zkey(i, q);
      const bool tie = q && !keep_all && key == thr;
      const uint64_t tmask = __ballot(tie);
      const uint32_t my_rank = rank + __popcll(tmask & ((1ull << lane) - 1ull));
      bool kept = false;
      if (q) kept = keep_all || key > thr || (tie && (uint64_t)my_rank < take);
      uint64_t v = kept ? q : 0;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint64_t t = __shfl_up(v, o, kWave);
        if (lane >= o) v += t;
      }
      const uint64_t hitm = __ballot(kept && acc + v > target);
      if (hitm) {
        const int first = __ffsll((long long)hitm) - 1;
        if (lane == first) {
          out[r] = i;
          picked = 1;
        }
        break;
      }
      acc += __shfl(v, 63, kWave);
      rank += __popcll(tmask);
    }
  }
  // only non-finite logits leave the target outside every kept range: fall
  // back to the first maximum (or 0) so the output is always a valid id
  __syncthreads();
  if (!picked) {
    int first = V;
    for (int i = tid; i < V; i += kSampThreads)
      if (x[i] == mx) { first = i; break; }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) first = min(first, __shfl_xor(first, o, kWave));
    if (lane == 0) wties[wv] = (uint32_t)first;
    __syncthreads();
    if (tid == 0) {
      int f = V;
      for (int w = 0; w < kSampWaves; ++w) f = min(f, (int)wties[w]);
      out[r] = f < V ? f : 0;
    }
  }
}

hipError_t launch_gen_fill(const int32_t *prompt, int64_t pstride, int32_t *tokens, int64_t tstride,
                           const GenLens &lens, int B, hipStream_t s) {
  hipLaunchKernelGGL(gen_fill_kernel, dim3((unsigned)((tstride + 255) / 256), B), dim3(256), 0, s, prompt, pstride,
                     tokens, tstride, lens);
  return hipGetLastError();
}

hipError_t launch_gen_stage_ids(const int32_t *prompt, int64_t pstride, const GenLens &lens, int b0, int g, int S,
                                int32_t *ids, hipStream_t s) {
  hipLaunchKernelGGL(gen_stage_ids_kernel, dim3((S + 255) / 256, g), dim3(256), 0, s, prompt, pstride, lens, b0, S, ids);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const float *h, int D, const RowList &rows, int n, float *out, hipStream_t s) {
  hipLaunchKernelGGL(gather_rows_kernel, dim3(n), dim3(256), 0, s, h, D, rows, out);
  return hipGetLastError();
}

hipError_t launch_gen_step(const GenState &st, const GenLens &lens, int B, int eos, const int32_t *prompt,
                           int64_t pstride, int32_t *tokens, int64_t tstride, int first, hipStream_t s) {
  hipLaunchKernelGGL(gen_step_kernel, dim3(1), dim3(64), 0, s, st, lens, B, eos, prompt, pstride, tokens, tstride,
                     first);
  return hipGetLastError();
}

hipError_t launch_gen_finish(const GenState &st, int B, int eos, const int32_t *tokens, int64_t tstride,
                             int32_t *out_len, hipStream_t s) {
  hipLaunchKernelGGL(gen_finish_kernel, dim3(B), dim3(256), 0, s, st, eos, tokens, tstride, out_len);
  return hipGetLastError();
}

hipError_t launch_sample_top_p(const float *logits, int64_t ld, int M, int V, float temperature, float top_p,
                               const float *u, int urows, const int32_t *gidx, int32_t *out, hipStream_t s) {
  const float k2 = (float)(1.4426950408889634 / (double)temperature);
  hipLaunchKernelGGL(sample_top_p_kernel, dim3(M), dim3(kSampThreads), 0, s, logits, ld, V, k2, top_p, u, M, urows,
                     gidx, out);
  return hipGetLastError();
}

}  // namespace llk
