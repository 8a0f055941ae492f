// Skinny bf16 GEMM for at most 64 activation rows: the batched decode step's
// projections and the LM head, where the weight stream from HBM is the cost
// [P3 "内存效率": the output matrix is read in full for every prediction].
//
// C = A * B^T with B [N][K] an nn.Linear weight (bf16) read exactly once.
// A arrives as two bf16 planes (hi, lo) of an fp32 activation, hi + lo
// carrying ~16 significant bits; both planes are multiplied against the same
// weight fragment (two MFMAs), so the weight bytes do not change.
//
// A block of 256 threads owns 64 B-rows (four 16-column MFMA blocks) and one
// K slice (grid.y); its four waves take interleaved 32-wide K steps and are
// summed through LDS at the end.  MFMA 16x16x32 (v_mfma_f32_16x16x32_bf16):
// lane l supplies row/column (l % 16) and eight consecutive k at 8*(l / 16);
// output register r of lane l holds row 4*(l/16) + r, column l % 16.
//
// Epilogues:
//   SK_PARTIAL       fp32 split-K partial [ks][M][N] (summed by the consumer)
//   SK_SWIGLU_HILO   B-rows interleave w1/w3 (32 each per block);
//                    u = silu(gate) * up written as hi/lo planes [P2 3.5]
//   SK_SWIGLU_BF16   same, one bf16 plane
//   SK_LOGITS        fp32 logits (optional) + per-block (max, argmax)
//                    partials, smallest index on ties [P1 12; P3 4]
#include "common.h"
#include "kernels.h"

namespace llk {

namespace {

template <int MB, int EPI>
__global__ __launch_bounds__(256) void skinny_kernel(SkinnyArgs a) {
  extern __shared__ __align__(16) float red[];  // [4 waves][MB][4][4][64]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nblk0 = blockIdx.x;
  const int ks = blockIdx.y;
  const int Kc = a.K / a.ksplit;
  const int kbeg = ks * Kc;
  const int l16 = lane & 15, lk = (lane >> 4) * 8;

  // weight rows of this lane for each of the four 16-column blocks
  const u16 *brow[4];
  bool bok[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    int wr;
    const u16 *base;
    bool ok;
    if (EPI == SK_SWIGLU_HILO || EPI == SK_SWIGLU_BF16) {
      const int F = a.N / 2;
      wr = nblk0 * 32 + (nb & 1) * 16 + l16;
      base = nb < 2 ? a.B0 : a.B1;
      ok = wr < F;
    } else {
      const int n = nblk0 * 64 + nb * 16 + l16;
      ok = n < a.N;
      if (a.nq > 0) {
        base = n < a.nq ? a.B0 : (n < a.nq + a.nk ? a.B1 : a.B2);
        wr = n < a.nq ? n : (n < a.nq + a.nk ? n - a.nq : n - a.nq - a.nk);
      } else {
        base = a.B0;
        wr = n;
      }
    }
    bok[nb] = ok;
    brow[nb] = base + (int64_t)(ok ? wr : 0) * a.K + kbeg + lk;
  }
  const u16 *arow[MB];
  bool aok[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int r = mb * 16 + l16;
    aok[mb] = r < a.M;
    arow[mb] = a.A + (int64_t)(aok[mb] ? r : 0) * a.lda + kbeg + lk;
  }

  f32x4 acc[MB][4];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nsteps = Kc / 32;
  const uint4 z = make_uint4(0, 0, 0, 0);
  for (int st = wave; st < nsteps; st += 4) {
    const int k = st * 32;
    uint4 bv[4], ah[MB], al[MB];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) bv[nb] = bok[nb] ? *reinterpret_cast<const uint4 *>(brow[nb] + k) : z;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      ah[mb] = aok[mb] ? *reinterpret_cast<const uint4 *>(arow[mb] + k) : z;
      al[mb] = (aok[mb] && a.use_lo) ? *reinterpret_cast<const uint4 *>(arow[mb] + a.a_plane + k) : z;
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<bf16x8 *>(&ah[mb]),
                                                              *reinterpret_cast<bf16x8 *>(&bv[nb]), acc[mb][nb], 0, 0, 0);
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<bf16x8 *>(&al[mb]),
                                                              *reinterpret_cast<bf16x8 *>(&bv[nb]), acc[mb][nb], 0, 0, 0);
      }
    }
  }

  // cross-wave reduction through LDS: red[w][mb][nb][r][lane]
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[(((wave * MB + mb) * 4 + nb) * 4 + r) * 64 + lane] = acc[mb][nb][r];
  __syncthreads();
  constexpr int PER_W = MB * 4 * 4 * 64;
  auto total = [&](int e) { return red[e] + red[PER_W + e] + red[2 * PER_W + e] + red[3 * PER_W + e]; };

  if (EPI == SK_PARTIAL) {
    float *C = static_cast<float *>(a.C) + (int64_t)ks * a.c_plane;
    for (int e = tid; e < PER_W; e += 256) {
      const int ln = e & 63, r = (e >> 6) & 3, nb = (e >> 8) & 3, mb = e >> 10;
      const int row = mb * 16 + 4 * (ln >> 4) + r, col = nblk0 * 64 + nb * 16 + (ln & 15);
      if (row < a.M && col < a.N) C[(int64_t)row * a.N + col] = total(e);
    }
  } else if (EPI == SK_SWIGLU_HILO || EPI == SK_SWIGLU_BF16) {
    const int F = a.N / 2;
    u16 *C = static_cast<u16 *>(a.C);
    for (int e = tid; e < PER_W; e += 256) {
      const int ln = e & 63, r = (e >> 6) & 3, nb = (e >> 8) & 3, mb = e >> 10;
      if (nb >= 2) continue;
      const int row = mb * 16 + 4 * (ln >> 4) + r, col = nblk0 * 32 + nb * 16 + (ln & 15);
      if (row < a.M && col < F) {
        const float g = total(e), up = total(e + 2 * 256);
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
    __syncthreads();
    // fold the four waves into red[0 .. PER_W) first
    for (int e = tid; e < PER_W; e += 256) red[e] = total(e);
    __syncthreads();
    if (a.logits) {
      for (int e = tid; e < PER_W; e += 256) {
        const int ln = e & 63, r = (e >> 6) & 3, nb = (e >> 8) & 3, mb = e >> 10;
        const int row = mb * 16 + 4 * (ln >> 4) + r, col = nblk0 * 64 + nb * 16 + (ln & 15);
        if (row < a.M && col < a.N) a.logits[(int64_t)row * a.N + col] = red[e];
      }
    }
    if (tid < MB * 16) {
      const int row = tid;
      const int mb = row >> 4, q = (row & 15) >> 2, r = row & 3;
      float bv = -INFINITY;
      int bi = 0x7fffffff;
      for (int c = 0; c < 64; ++c) {
        const int nb = c >> 4, cl = c & 15;
        const int col = nblk0 * 64 + c;
        if (col >= a.N) break;
        const float v = red[((mb * 4 + nb) * 4 + r) * 64 + q * 16 + cl];
        if (v > bv) { bv = v; bi = col; }  // ascending columns: first maximum kept
      }
      if (row < a.M) {
        a.pval[(int64_t)row * a.nblk + nblk0] = bv;
        a.pidx[(int64_t)row * a.nblk + nblk0] = bi;
      }
    }
  }
}

template <int MB>
hipError_t launch_mb(int epi, const SkinnyArgs &a, hipStream_t s) {
  const int nblk = (epi == SK_SWIGLU_HILO || epi == SK_SWIGLU_BF16) ? (a.N / 2 + 31) / 32 : (a.N + 63) / 64;
  dim3 grid(nblk, a.ksplit);
  const size_t lds = (size_t)4 * MB * 4 * 4 * 64 * sizeof(float);
  switch (epi) {
    case SK_PARTIAL: hipLaunchKernelGGL((skinny_kernel<MB, SK_PARTIAL>), grid, dim3(256), lds, s, a); break;
    case SK_SWIGLU_HILO: hipLaunchKernelGGL((skinny_kernel<MB, SK_SWIGLU_HILO>), grid, dim3(256), lds, s, a); break;
    case SK_SWIGLU_BF16: hipLaunchKernelGGL((skinny_kernel<MB, SK_SWIGLU_BF16>), grid, dim3(256), lds, s, a); break;
    case SK_LOGITS: hipLaunchKernelGGL((skinny_kernel<MB, SK_LOGITS>), grid, dim3(256), lds, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
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
