// Skinny bf16 GEMM for at most 64 activation rows: the batched decode step's
// projections and the LM head, where the weight stream from HBM is the cost
// [P3 "内存效率": the output matrix is read in full for every prediction].
//
// C = A * B^T with B [N][K] an nn.Linear weight (bf16) read exactly once.
// A arrives as two bf16 planes (hi, lo) of an fp32 activation, hi + lo
// carrying ~16 significant bits; both planes are multiplied against the same
// weight fragment (two MFMAs), so the weight bytes do not change.
//
// A block of 512 threads owns 64 B-rows and one K slice (grid.y).  The K
// slice streams through two LDS stages of 64 k: weights and both activation
// planes arrive with global_load_lds_dwordx4 in fully coalesced 1 KB pieces
// (8 rows x 128 bytes), stored with the 16-byte chunk swizzle
// c ^ ((row >> 1) & 7) so the MFMA fragment reads of 16 consecutive rows are
// bank-conflict free.  The activations are shared by all waves through LDS.
// Waves w and w+4 own the same 16 B-rows and split each 64-k stage into its
// two 32-k halves; their partial sums meet in LDS at the end.  Small stages
// and eight waves per block leave room for three blocks per compute unit:
// the weight stream is latency-bound, and resident waves, more than a deeper
// pipeline per block, are what keep enough loads in flight.
// MFMA 16x16x32 (v_mfma_f32_16x16x32_bf16): lane l supplies row/column
// (l % 16) and eight consecutive k at 8*(l / 16); output register r of lane
// l holds row 4*(l/16) + r, column l % 16.
//
// Epilogues:
//   SK_PARTIAL       fp32 split-K partial [ks][M][N] (summed by the consumer)
//   SK_SWIGLU_HILO   B-rows interleave w1/w3 (16 each, twice per block);
//                    u = silu(gate) * up written as hi/lo planes [P2 3.5]
//   SK_SWIGLU_BF16   same, one bf16 plane
//   SK_LOGITS        fp32 logits (optional) + per-block (max, argmax)
//                    partials, smallest index on ties [P1 12; P3 4]
#include "common.h"
#include "kernels.h"

namespace llk {

namespace {

constexpr int SK_KCH = 64;     // k per LDS stage
constexpr int SK_STAGES = 2;
constexpr int SK_ROWB = SK_KCH * 2;  // bytes per tile row (128)

template <int MB, int EPI>
__global__ __launch_bounds__(512) void skinny_kernel(SkinnyArgs a) {
  // stage layout (bf16): A hi [64][64], A lo [64][64], B [64][64]
  constexpr int ST_ELEMS = 3 * 64 * SK_KCH;
  extern __shared__ __align__(16) u16 sm[];  // [SK_STAGES][ST_ELEMS]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wcol = wave & 3, khalf = wave >> 2;
  const int nblk0 = blockIdx.x;
  const int ks = blockIdx.y;
  const int Kc = a.K / a.ksplit;
  const int kbeg = ks * Kc;
  const int nchunk = Kc / SK_KCH;

  // Loader: 24 pieces of 1 KB per stage (A hi 8, A lo 8, B 8); wave w issues
  // pieces w, w+8, w+16.  Piece p covers tile rows 8*(p%8) .. +7 of its matrix;
  // lane L -> row 8*(p%8) + L/8, physical chunk L%8 holding logical chunk
  // (L%8) ^ ((row >> 1) & 7).  Rows past M or past the weight read a clamped
  // valid row: they only feed outputs that are never stored.
  const int lr = lane >> 3, lq = lane & 7;
  const u16 *src[3];
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const int p = wave + 8 * i;        // 0..23
    const int mat = p >> 3;            // 0: A hi, 1: A lo, 2: B
    const int row = (p & 7) * 8 + lr;  // tile row 0..63
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
      if (EPI == SK_SWIGLU_HILO || EPI == SK_SWIGLU_BF16) {
        // tile rows: [gate 0-15 | up 0-15 | gate 16-31 | up 16-31] of this block's 32 output columns
        const int F = a.N / 2;
        wr = min(nblk0 * 32 + (row >> 5) * 16 + (row & 15), F - 1);
        base = ((row >> 4) & 1) ? a.B1 : a.B0;
      } else {
        const int n = min(nblk0 * 64 + row, a.N - 1);
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
    for (int i = 0; i < 3; ++i) {
      const int p = __builtin_amdgcn_readfirstlane(wave + 8 * i);
      u16 *dst = st + (p >> 3) * 64 * SK_KCH + (p & 7) * 8 * SK_KCH;
      __builtin_amdgcn_global_load_lds((const void *)(src[i] + chunk * SK_KCH),
                                       (__attribute__((address_space(3))) void *)dst, 16, 0, 0);
    }
  };

  // fragment offsets: row (lane % 16) of a 16-row block, logical chunk 4*kk + lane/16
  const int frow = lane & 15;
  const int sw = (frow >> 1) & 7;
  f32x4 acc[MB];
#pragma unroll
  for (int i = 0; i < MB; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  issue(0, 0);
  for (int ch = 0; ch < nchunk; ++ch) {
    // this wave's pieces of stage ch have landed; after the barrier every
    // wave's have, and every wave is done reading the stage refilled next
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    asm volatile("s_barrier" ::: "memory");
    if (ch + 1 < nchunk) issue((ch + 1) % SK_STAGES, ch + 1);
    const u16 *st = sm + (ch % SK_STAGES) * ST_ELEMS;
    const u16 *bp = st + 2 * 64 * SK_KCH + (wcol * 16 + frow) * SK_KCH;
    {
      const int kk = khalf;  // this wave's 32-k half of the stage
      const int co = ((4 * kk + (lane >> 4)) ^ sw) * 8;
      const bf16x8 bb = *reinterpret_cast<const bf16x8 *>(bp + co);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const u16 *ap = st + (mb * 16 + frow) * SK_KCH + co;
        acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const bf16x8 *>(ap), bb, acc[mb], 0, 0, 0);
        if (a.use_lo)
          acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const bf16x8 *>(ap + 64 * SK_KCH), bb,
                                                            acc[mb], 0, 0, 0);
      }
    }
  }
  __syncthreads();  // stages are reused for the epilogue

  // wave pair (w, w+4) holds column block w%4: acc[mb][r] = partial
  // C[mb*16 + 4*(lane/16) + r][16*(w%4) + lane%16] over its k halves
  float *red = reinterpret_cast<float *>(sm);  // [MB*16 rows][64 cols]
  if (khalf == 0) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[(mb * 16 + 4 * (lane >> 4) + r) * 64 + wcol * 16 + frow] = acc[mb][r];
  }
  __syncthreads();
  if (khalf == 1) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[(mb * 16 + 4 * (lane >> 4) + r) * 64 + wcol * 16 + frow] += acc[mb][r];
  }
  __syncthreads();
  constexpr int ROWS = MB * 16;

  if (EPI == SK_PARTIAL) {
    float *C = static_cast<float *>(a.C) + (int64_t)ks * a.c_plane;
    for (int e = tid; e < ROWS * 64; e += 512) {
      const int row = e >> 6, col = nblk0 * 64 + (e & 63);
      if (row < a.M && col < a.N) C[(int64_t)row * a.N + col] = red[e];
    }
  } else if (EPI == SK_SWIGLU_HILO || EPI == SK_SWIGLU_BF16) {
    const int F = a.N / 2;
    u16 *C = static_cast<u16 *>(a.C);
    for (int e = tid; e < ROWS * 32; e += 512) {
      const int row = e >> 5, uc = e & 31;
      const int gc = (uc >> 4) * 32 + (uc & 15);  // gate column in the tile; up is 16 further
      const int col = nblk0 * 32 + uc;
      if (row < a.M && col < F) {
        const float g = red[row * 64 + gc], up = red[row * 64 + gc + 16];
        const float u = silu(g) * up;
        const int64_t o = (int64_t)row * F + col;
        if (EPI == SK_SWIGLU_HILO) {
          u16 hi, lo;
          split_hilo(u, hi, lo);
          C[o] = hi;
          C[a.c_plane + o] = lo;
        } else {
          C[o] = f2bf(u);
        }
      }
    }
  } else {  // SK_LOGITS
    if (a.logits) {
      for (int e = tid; e < ROWS * 64; e += 512) {
        const int row = e >> 6, col = nblk0 * 64 + (e & 63);
        if (row < a.M && col < a.N) a.logits[(int64_t)row * a.N + col] = red[e];
      }
    }
    if (tid < ROWS) {
      const int row = tid;
      float bv = -INFINITY;
      int bi = 0x7fffffff;
      for (int c = 0; c < 64; ++c) {
        const int col = nblk0 * 64 + c;
        if (col >= a.N) break;
        const float v = red[row * 64 + c];
        if (v > bv) { bv = v; bi = col; }  // ascending columns: first maximum kept
      }
      if (row < a.M) {
        a.pval[(int64_t)row * a.nblk + nblk0] = bv;
        a.pidx[(int64_t)row * a.nblk + nblk0] = bi;
      }
    }
  }
}

template <int MB, int EPI>
hipError_t launch_one(const SkinnyArgs &a, dim3 grid, size_t lds, hipStream_t s) {
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void *>(&skinny_kernel<MB, EPI>),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  (void)attr;
  hipLaunchKernelGGL((skinny_kernel<MB, EPI>), grid, dim3(512), lds, s, a);
  return hipGetLastError();
}

template <int MB>
hipError_t launch_mb(int epi, const SkinnyArgs &a, hipStream_t s) {
  const int nblk = (epi == SK_SWIGLU_HILO || epi == SK_SWIGLU_BF16) ? (a.N / 2 + 31) / 32 : (a.N + 63) / 64;
  dim3 grid(nblk, a.ksplit);
  const size_t lds = (size_t)SK_STAGES * 3 * 64 * SK_KCH * sizeof(u16);  // >= the epilogue's 64 x 64 floats
  switch (epi) {
    case SK_PARTIAL: return launch_one<MB, SK_PARTIAL>(a, grid, lds, s);
    case SK_SWIGLU_HILO: return launch_one<MB, SK_SWIGLU_HILO>(a, grid, lds, s);
    case SK_SWIGLU_BF16: return launch_one<MB, SK_SWIGLU_BF16>(a, grid, lds, s);
    case SK_LOGITS: return launch_one<MB, SK_LOGITS>(a, grid, lds, s);
  }
  return hipErrorInvalidValue;
}
}  // namespace

int skinny_nblk(int N, int epi) {
  return (epi == SK_SWIGLU_HILO || epi == SK_SWIGLU_BF16) ? (N / 2 + 31) / 32 : (N + 63) / 64;
}

hipError_t launch_skinny(int epi, const SkinnyArgs &a, hipStream_t s) {
  const int mb = (a.M + 15) / 16;
  switch (mb) {
    case 1: return launch_mb<1>(epi, a, s);
    case 2: return launch_mb<2>(epi, a, s);
    case 3: return launch_mb<3>(epi, a, s);
    case 4: return launch_mb<4>(epi, a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace llk
