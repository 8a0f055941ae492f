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
// and split-K products whose K slices stay at 256 or more).
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
constexpr int SK_ROWB = SK_KCH * 2;  // bytes per tile row (128)

// s_waitcnt vmcnt(n) for a wave-uniform n <= 15 (the count must be an immediate)
__device__ __forceinline__ void wait_vmcnt(int n) {
  switch (n) {
#define LLK_VM(i) \
  case i: __builtin_amdgcn_s_waitcnt(0x0F70 | i); break;
    LLK_VM(0) LLK_VM(1) LLK_VM(2) LLK_VM(3) LLK_VM(4) LLK_VM(5) LLK_VM(6) LLK_VM(7)
    LLK_VM(8) LLK_VM(9) LLK_VM(10) LLK_VM(11) LLK_VM(12) LLK_VM(13) LLK_VM(14)
#undef LLK_VM
    default: __builtin_amdgcn_s_waitcnt(0x0F70 | 15); break;
  }
}

template <int NR, int RW, int NS, int MB, int EPI>
__global__ __launch_bounds__((NR / RW) * 128) void skinny_kernel(SkinnyArgs a) {
  constexpr int NG = NR / RW;               // row groups of RW B-rows
  constexpr int NW = 2 * NG, NT = NW * 64;  // waves (a row group and a 32-k half each), threads
  constexpr int NB = RW / 16;               // 16-row MFMA blocks per wave
  // stage layout (bf16): A hi [64][64], A lo [64][64], B [NR][64]
  constexpr int ST_ELEMS = (128 + NR) * SK_KCH;
  extern __shared__ __align__(16) u16 sm[];  // [NS][ST_ELEMS]
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

  // loads this wave issues per stage (the same for every stage)
  int nper = 0;
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int p = wave + NW * i;
    nper += !((p < 16 && (p & 7) * 8 >= MB * 16) || (p >= 8 && p < 16 && !a.use_lo));
  }
  // NS stages: chunks ch+1 .. ch+NS-1 are in flight while chunk ch is computed
#pragma unroll
  for (int c = 0; c < NS - 1; ++c)
    if (c < nchunk) issue(c, c);
  for (int ch = 0; ch < nchunk; ++ch) {
    // this wave's pieces of stage ch have landed (loads complete in order;
    // the later chunks' pieces may stay in flight); after the barrier every
    // wave's have, and every wave is done reading the stage refilled next
    wait_vmcnt(nper * max(0, min(NS - 2, nchunk - 1 - ch)));
    asm volatile("s_barrier" ::: "memory");
    if (ch + NS - 1 < nchunk) issue((ch + NS - 1) % NS, ch + NS - 1);
    const u16 *st = sm + (ch % NS) * ST_ELEMS;
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

template <int NR, int RW, int NS, int MB, int EPI>
hipError_t launch_one(const SkinnyArgs &a, dim3 grid, hipStream_t s) {
  // NS stages; the epilogue's MB*16 x NR floats fit in the same space
  constexpr size_t lds = (size_t)NS * (128 + NR) * SK_KCH * sizeof(u16);
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void *>(&skinny_kernel<NR, RW, NS, MB, EPI>), hipFuncAttributeMaxDynamicSharedMemorySize,
      (int)lds);
  (void)attr;
  hipLaunchKernelGGL((skinny_kernel<NR, RW, NS, MB, EPI>), grid, dim3((NR / RW) * 128), lds, s, a);
  return hipGetLastError();
}

template <int NR, int RW, int NS, int MB>
hipError_t launch_mb(int epi, const SkinnyArgs &a, dim3 grid, hipStream_t s) {
  switch (epi) {
    case SK_PARTIAL: return launch_one<NR, RW, NS, MB, SK_PARTIAL>(a, grid, s);
    case SK_SWIGLU_HILO: return launch_one<NR, RW, NS, MB, SK_SWIGLU_HILO>(a, grid, s);
    case SK_LOGITS: return launch_one<NR, RW, NS, MB, SK_LOGITS>(a, grid, s);
  }
  return hipErrorInvalidValue;
}

template <int NR, int RW, int NS = 2>
hipError_t launch_nr(int epi, const SkinnyArgs &a, dim3 grid, hipStream_t s) {
  switch ((a.M + 15) / 16) {
    case 1: return launch_mb<NR, RW, NS, 1>(epi, a, grid, s);
    case 2: return launch_mb<NR, RW, NS, 2>(epi, a, grid, s);
    case 3: return launch_mb<NR, RW, NS, 3>(epi, a, grid, s);
    case 4: return launch_mb<NR, RW, NS, 4>(epi, a, grid, s);
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

// Launch plan of one product: rows per block, rows per wave, LDS stages and
// K slices.  Measured at 64 activation rows on the 8B decode shapes with the
// weights rotating beyond the Infinity Cache: one block of 128 rows per
// compute unit with four stages in flight (three chunks loading while one is
// computed) streams fastest when the blocks fill one round of the chip
// (w1/w3 70 -> 58.5 us, w2 30.9 -> 27.8 us, wo 14.5 -> 12.5 us); products
// with more row blocks than that keep two stages and about 1.5 blocks per
// compute unit, as does the LM head (1002 blocks).
struct Plan {
  int nr, rw, ns, ks;
};

Plan skinny_plan(int N, int K, int epi) {
  if (epi == SK_LOGITS) return {128, 16, 2, 1};
  if (epi == SK_SWIGLU_HILO) return {128, 32, 4, 1};
  const int nb = (N + 127) / 128;
  int ks = 1;
  while (nb * ks * 2 <= 256 && K % (ks * 2 * SK_KCH) == 0 && K / (ks * 2) >= 256) ks *= 2;
  if (nb * ks >= 192) return {128, 32, 4, ks};
  const int nr = K / ksplit_rule(nb, K) >= 256 ? 128 : 64;
  return {nr, 16, 2, ksplit_rule((N + nr - 1) / nr, K)};
}
}  // namespace

int skinny_rows(int N, int K, int epi) { return skinny_plan(N, K, epi).nr; }

int skinny_nblk(int N, int K, int epi) {
  const int nr = skinny_rows(N, K, epi);
  return epi == SK_SWIGLU_HILO ? (N / 2 + nr / 2 - 1) / (nr / 2) : (N + nr - 1) / nr;
}

int skinny_ksplit(int N, int K) { return skinny_plan(N, K, SK_PARTIAL).ks; }

hipError_t launch_skinny(int epi, const SkinnyArgs &a, hipStream_t s) {
  const Plan p = skinny_plan(a.N, a.K, epi);
  if (epi == SK_PARTIAL && a.ksplit != p.ks) return hipErrorInvalidValue;  // partial planes sized for p.ks
  const dim3 grid(skinny_nblk(a.N, a.K, epi), a.ksplit);
  if (p.nr == 128 && p.rw == 32 && p.ns == 4) return launch_nr<128, 32, 4>(epi, a, grid, s);
  if (p.nr == 128) return launch_nr<128, 16, 2>(epi, a, grid, s);
  return launch_nr<64, 16, 2>(epi, a, grid, s);
}

}  // namespace llk
