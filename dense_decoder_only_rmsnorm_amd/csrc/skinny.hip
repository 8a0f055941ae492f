// Skinny bf16 GEMM for at most 64 activation rows: the batched decode step's
// projections and the LM head, where the weight stream from HBM is the cost
// [P3 "内存效率": the output matrix is read in full for every prediction].
//
// C = A * B^T with B [N][K] an nn.Linear weight (bf16) read exactly once.
// A arrives as two bf16 planes (hi, lo) of an fp32 activation, hi + lo
// carrying ~16 significant bits; both planes are multiplied against the same
// weight fragment (two MFMAs), so the weight bytes do not change.
//
// A block of 8*NR threads owns NR = 64 or 128 B-rows and one K slice
// (grid.y).  The K slice streams through two LDS stages of 64 k: weights and
// both activation planes arrive with global_load_lds_dwordx4 in fully
// coalesced 1 KB pieces (8 rows x 128 bytes), stored with the 16-byte chunk
// swizzle c ^ ((row >> 1) & 7) so the MFMA fragment reads of 16 consecutive
// rows are bank-conflict free.  The activations are shared by all waves
// through LDS.  Waves w and w + NR/16 own the same 16 B-rows and split each
// 64-k stage into its two 32-k halves; their partial sums meet in LDS at the
// end.  Small stages leave room for three 64-row or two 128-row blocks per
// compute unit: the weight stream is latency-bound, and resident waves, more
// than a deeper pipeline per block, keep enough loads in flight.  The
// activation pieces are two thirds of a 64-row stage; 128-row blocks halve
// that share, which pays wherever it still leaves enough blocks (the LM head,
// and split-K products whose K slices stay at 512 or more).
// MFMA 16x16x32 (v_mfma_f32_16x16x32_bf16): lane l supplies row/column
// (l % 16) and eight consecutive k at 8*(l / 16); output register r of lane
// l holds row 4*(l/16) + r, column l % 16.
//
// Epilogues:
//   SK_PARTIAL       fp32 split-K partial [ks][M][N] (summed by the consumer)
//   SK_SWIGLU_HILO   B-rows interleave w1/w3 (16 each, twice per block);
//                    u = silu(gate) * up written as hi/lo planes [P2 3.5]
//   SK_LOGITS        fp32 logits (optional) + per-block (max, argmax)
//                    partials, smallest index on ties [P1 12; P3 4]
#include "common.h"
#include "kernels.h"

namespace llk {

namespace {

constexpr int SK_KCH = 64;     // k per LDS stage
constexpr int SK_STAGES = 2;
constexpr int SK_ROWB = SK_KCH * 2;  // bytes per tile row (128)

template <int NR, int RW, int MB, int EPI>
__global__ __launch_bounds__((NR / RW) * 128) void skinny_kernel(SkinnyArgs a) {
  constexpr int NG = NR / RW;               // row groups of RW B-rows
  constexpr int NW = 2 * NG, NT = NW * 64;  // waves (a row group and a 32-k half each), threads
  constexpr int NB = RW / 16;               // 16-row MFMA blocks per wave
  // stage layout (bf16): A hi [64][64], A lo [64][64], B [NR][64]
  constexpr int ST_ELEMS = (128 + NR) * SK_KCH;
  extern __shared__ __align__(16) u16 sm[];  // [SK_STAGES][ST_ELEMS]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rg = wave % NG, khalf = wave / NG;
  const int nblk0 = blockIdx.x;
  const int ks = blockIdx.y;
  const int Kc = a.K / a.ksplit;
  const int kbeg = ks * Kc;
  const int nchunk = Kc / SK_KCH;

  // Loader: 16 + NR/8 pieces of 1 KB per stage (A hi 8, A lo 8, B NR/8),
  // piece p at stage offset 512*p; wave w issues pieces w, w + NW, ...
  // Piece p covers rows 8*(p%8) .. +7 of A hi (p < 8) or A lo (p < 16), else
  // rows 8*(p-16) .. +7 of B; lane L -> row 8*(piece row) + L/8, physical
  // chunk L%8 holding logical chunk (L%8) ^ ((row >> 1) & 7).  Rows past M or
  // past the weight read a clamped valid row: they only feed outputs that are
  // never stored.
  static_assert((16 + NR / 8) % NW == 0, "pieces spread evenly over the waves");
  constexpr int NP = (16 + NR / 8) / NW;
  const int lr = lane >> 3, lq = lane & 7;
  const u16 *src[NP];
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int p = wave + NW * i;
    const int mat = p < 16 ? (p >> 3) : 2;  // 0: A hi, 1: A lo, 2: B
    const int row = mat < 2 ? (p & 7) * 8 + lr : (p - 16) * 8 + lr;  // row of its matrix
    const int c = lq ^ ((row >> 1) & 7);
    const u16 *base;
    int64_t ld;
    int grow;
    if (mat < 2) {
      grow = min(row, a.M - 1);
      base = a.A + (mat == 1 && a.use_lo ? a.a_plane : 0);
      ld = a.lda;
    } else {
      int wr;
      if (EPI == SK_SWIGLU_HILO) {
        // tile rows: [gate 0-15 | up 0-15 | gate 16-31 | up 16-31] of this block's 32 output columns
        const int F = a.N / 2;
        wr = min(nblk0 * (NR / 2) + (row >> 5) * 16 + (row & 15), F - 1);
        base = ((row >> 4) & 1) ? a.B1 : a.B0;
      } else {
        const int n = min(nblk0 * NR + row, a.N - 1);
        if (a.nq > 0) {
          base = n < a.nq ? a.B0 : (n < a.nq + a.nk ? a.B1 : a.B2);
          wr = n < a.nq ? n : (n < a.nq + a.nk ? n - a.nq : n - a.nq - a.nk);
        } else {
          base = a.B0;
          wr = n;
        }
      }
      grow = wr;
      ld = a.K;
    }
    src[i] = base + (int64_t)grow * ld + kbeg + c * 8;
  }
  auto issue = [&](int stage, int chunk) {
    u16 *st = sm + stage * ST_ELEMS;
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int p = __builtin_amdgcn_readfirstlane(wave + NW * i);
      // activation rows from MB*16 on are never read by the MFMAs (few rows:
      // the prefill LM head, small decode batches): their pieces are skipped
      if (p < 16 && (p & 7) * 8 >= MB * 16) continue;
      if (p >= 8 && p < 16 && !a.use_lo) continue;  // one activation plane: the lo pieces are never read
      u16 *dst = st + p * 8 * SK_KCH;
      __builtin_amdgcn_global_load_lds((const void *)(src[i] + chunk * SK_KCH),
                                       (__attribute__((address_space(3))) void *)dst, 16, 0, 0);
    }
  };

  // fragment offsets: row (lane % 16) of a 16-row block, logical chunk 4*kk + lane/16
  const int frow = lane & 15;
  const int sw = (frow >> 1) & 7;
  f32x4 acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  issue(0, 0);
  for (int ch = 0; ch < nchunk; ++ch) {
    // this wave's pieces of stage ch have landed; after the barrier every
    // wave's have, and every wave is done reading the stage refilled next
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    asm volatile("s_barrier" ::: "memory");
    if (ch + 1 < nchunk) issue((ch + 1) % SK_STAGES, ch + 1);
    const u16 *st = sm + (ch % SK_STAGES) * ST_ELEMS;
    // this wave's 32-k half of the stage, rows rg*RW + 16 j of B (the row
    // swizzle is the same for every 16-row block)
    const int co = ((4 * khalf + (lane >> 4)) ^ sw) * 8;
    bf16x8 bb[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j)
      bb[j] = *reinterpret_cast<const bf16x8 *>(st + 2 * 64 * SK_KCH + (rg * RW + j * 16 + frow) * SK_KCH + co);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const u16 *ap = st + (mb * 16 + frow) * SK_KCH + co;
      const bf16x8 ah = *reinterpret_cast<const bf16x8 *>(ap);
#pragma unroll
      for (int j = 0; j < NB; ++j) acc[mb][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bb[j], acc[mb][j], 0, 0, 0);
      if (a.use_lo) {
        const bf16x8 al = *reinterpret_cast<const bf16x8 *>(ap + 64 * SK_KCH);
#pragma unroll
        for (int j = 0; j < NB; ++j)
          acc[mb][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bb[j], acc[mb][j], 0, 0, 0);
      }
    }
  }
  __syncthreads();  // stages are reused for the epilogue

  // waves (rg, 0) and (rg, 1) hold B-rows rg*RW .. +RW-1 over the two k
  // halves: acc[mb][j][r] = partial C[mb*16 + 4*(lane/16) + r][rg*RW + 16j + lane%16]
  float *red = reinterpret_cast<float *>(sm);  // [MB*16 rows][NR cols]
  if (khalf == 0) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          red[(mb * 16 + 4 * (lane >> 4) + r) * NR + rg * RW + j * 16 + frow] = acc[mb][j][r];
  }
  __syncthreads();
  if (khalf == 1) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          red[(mb * 16 + 4 * (lane >> 4) + r) * NR + rg * RW + j * 16 + frow] += acc[mb][j][r];
  }
  __syncthreads();
  constexpr int ROWS = MB * 16;

  if (EPI == SK_PARTIAL) {
    float *C = static_cast<float *>(a.C) + (int64_t)ks * a.c_plane;
    for (int e = tid; e < ROWS * NR; e += NT) {
      const int row = e / NR, col = nblk0 * NR + e % NR;
      if (row < a.M && col < a.N) C[(int64_t)row * a.N + col] = red[e];
    }
  } else if (EPI == SK_SWIGLU_HILO) {
    const int F = a.N / 2;
    u16 *C = static_cast<u16 *>(a.C);
    for (int e = tid; e < ROWS * (NR / 2); e += NT) {
      const int row = e / (NR / 2), uc = e % (NR / 2);
      const int gc = (uc >> 4) * 32 + (uc & 15);  // gate column in the tile; up is 16 further
      const int col = nblk0 * (NR / 2) + uc;
      if (row < a.M && col < F) {
        const float g = red[row * NR + gc], up = red[row * NR + gc + 16];
        const float u = silu(g) * up;
        const int64_t o = (int64_t)row * F + col;
        u16 hi, lo;
        split_hilo(u, hi, lo);
        C[o] = hi;
        C[a.c_plane + o] = lo;
      }
    }
  } else {  // SK_LOGITS
    if (a.logits) {
      for (int e = tid; e < ROWS * NR; e += NT) {
        const int row = e / NR, col = nblk0 * NR + e % NR;
        if (row < a.M && col < a.N) a.logits[(int64_t)row * a.N + col] = red[e];
      }
    }
    if (tid < ROWS) {
      const int row = tid;
      float bv = -INFINITY;
      int bi = 0x7fffffff;
      for (int c = 0; c < NR; ++c) {
        const int col = nblk0 * NR + c;
        if (col >= a.N) break;
        const float v = red[row * NR + c];
        if (v > bv) { bv = v; bi = col; }  // ascending columns: first maximum kept
      }
      if (row < a.M) {
        a.pval[(int64_t)row * a.nblk + nblk0] = bv;
        a.pidx[(int64_t)row * a.nblk + nblk0] = bi;
      }
    }
  }
}

template <int NR, int RW, int MB, int EPI>
hipError_t launch_one(const SkinnyArgs &a, dim3 grid, hipStream_t s) {
  // two stages; the epilogue's MB*16 x NR floats fit in the same space
  constexpr size_t lds = (size_t)SK_STAGES * (128 + NR) * SK_KCH * sizeof(u16);
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void *>(&skinny_kernel<NR, RW, MB, EPI>), hipFuncAttributeMaxDynamicSharedMemorySize,
      (int)lds);
  (void)attr;
  hipLaunchKernelGGL((skinny_kernel<NR, RW, MB, EPI>), grid, dim3((NR / RW) * 128), lds, s, a);
  return hipGetLastError();
}

template <int NR, int RW, int MB>
hipError_t launch_mb(int epi, const SkinnyArgs &a, dim3 grid, hipStream_t s) {
  switch (epi) {
    case SK_PARTIAL: return launch_one<NR, RW, MB, SK_PARTIAL>(a, grid, s);
    case SK_SWIGLU_HILO: return launch_one<NR, RW, MB, SK_SWIGLU_HILO>(a, grid, s);
    case SK_LOGITS: return launch_one<NR, RW, MB, SK_LOGITS>(a, grid, s);
  }
  return hipErrorInvalidValue;
}

template <int NR, int RW>
hipError_t launch_nr(int epi, const SkinnyArgs &a, dim3 grid, hipStream_t s) {
  switch ((a.M + 15) / 16) {
    case 1: return launch_mb<NR, RW, 1>(epi, a, grid, s);
    case 2: return launch_mb<NR, RW, 2>(epi, a, grid, s);
    case 3: return launch_mb<NR, RW, 3>(epi, a, grid, s);
    case 4: return launch_mb<NR, RW, 4>(epi, a, grid, s);
  }
  return hipErrorInvalidValue;
}

// K slices for nblk row blocks: enough blocks to cover the 256 compute units
// about 1.5 times, slices remaining multiples of 128
int ksplit_rule(int nblk, int K) {
  int ks = 1;
  while (nblk * ks < 384 && ks < 16 && K % (ks * 2 * 128) == 0) ks *= 2;
  return ks;
}
}  // namespace

int skinny_rows(int N, int K, int epi) {
  if (epi == SK_SWIGLU_HILO) return 64;  // 128 would leave CUs without a block
  if (epi == SK_LOGITS) return 128;
  return K / ksplit_rule((N + 127) / 128, K) >= 512 ? 128 : 64;
}

int skinny_nblk(int N, int K, int epi) {
  const int nr = skinny_rows(N, K, epi);
  return epi == SK_SWIGLU_HILO ? (N / 2 + nr / 2 - 1) / (nr / 2) : (N + nr - 1) / nr;
}

int skinny_ksplit(int N, int K) { return ksplit_rule(skinny_nblk(N, K, SK_PARTIAL), K); }

hipError_t launch_skinny(int epi, const SkinnyArgs &a, hipStream_t s) {
  const dim3 grid(skinny_nblk(a.N, a.K, epi), a.ksplit);
  return skinny_rows(a.N, a.K, epi) == 128 ? launch_nr<128, 16>(epi, a, grid, s) : launch_nr<64, 16>(epi, a, grid, s);
}

}  // namespace llk
