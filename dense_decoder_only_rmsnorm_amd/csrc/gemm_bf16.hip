// Dense bf16 GEMM on gfx950 MFMA (v_mfma_f32_32x32x16_bf16), C = A * B^T with
// A [M][K] activations and B [N][K] an nn.Linear weight, fp32 accumulation,
// LDS double buffering and fused epilogues for the prefill path:
//   EPI_QKV_ROPE  Q/K/V projection + RoPE on q and k + KV write
//                 [P2 3.2 apply_rotary_emb, 3.3-3.4; P1 6.5-6.10]
//   EPI_RESID     output projection / w2 with the residual add [P2 3.6; P1 9.1, 10]
//   EPI_SWIGLU    w1 and w3 in one pass, u = silu(x w1^T) * (x w3^T) [P2 3.5; P1 9.3]
//   EPI_STORE_*   plain stores
//
// Tiling: a block of 256 threads (4 waves in a 2x2 grid) owns a BM x BN
// output tile; each wave owns (BM/2) x (BN/2) as 32x32 MFMA blocks.  The K
// loop steps by 64: the next A/B tiles are fetched into registers with 16-byte
// loads while the MFMAs consume the current LDS buffer, then written to the
// other buffer.  LDS rows are padded by 16 bytes so the 16-byte fragment reads
// of 32 consecutive rows spread over all banks.
//
// MFMA 32x32x16 operand layout (lane l): A supplies row (l % 32) and eight
// consecutive k at 8*(l / 32); B likewise for output column (l % 32).  Output
// register r of lane l holds row 8*(r/4) + 4*(l/32) + (r%4), column l % 32.
#include "common.h"
#include "kernels.h"

namespace llk {

namespace {
constexpr int BK = 64;
constexpr int PADK = 8;
constexpr int LDK = BK + PADK;  // bf16 elements per LDS row

struct Chunk16 {
  uint4 v;
};

template <int BM, int BN, int EPI>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(GemmArgs a) {
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int FM = WM / 32, FN = WN / 32;
  constexpr int ACH = BM * (BK / 8) / 256;  // 16-byte chunks per thread (A)
  constexpr int BCH = BN * (BK / 8) / 256;
  extern __shared__ __align__(16) u16 smem[];
  u16 *As = smem;                      // [2][BM][LDK]
  u16 *Bs = smem + 2 * BM * LDK;       // [2][BN][LDK]

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.x * BM;
  const int n0 = blockIdx.y * BN;
  const int K = a.K;

  // global source rows for this thread's chunks
  const u16 *asrc[ACH];
  bool aok[ACH];
  int acol[ACH], arow[ACH];
#pragma unroll
  for (int i = 0; i < ACH; ++i) {
    const int c = tid + i * 256;
    arow[i] = c / (BK / 8);
    acol[i] = (c % (BK / 8)) * 8;
    const int gr = m0 + arow[i];
    aok[i] = gr < a.M;
    asrc[i] = a.A + (int64_t)(aok[i] ? gr : 0) * a.lda + acol[i];
  }
  const u16 *bsrc[BCH];
  bool bok[BCH];
  int bcol[BCH], brow[BCH];
#pragma unroll
  for (int i = 0; i < BCH; ++i) {
    const int c = tid + i * 256;
    brow[i] = c / (BK / 8);
    bcol[i] = (c % (BK / 8)) * 8;
    const int t = brow[i];
    const u16 *base;
    int wr;
    bool ok;
    if (EPI == EPI_SWIGLU) {
      const int F = a.N / 2;
      wr = n0 / 2 + (t >> 6) * 32 + (t & 31);
      base = ((t >> 5) & 1) ? a.B1 : a.B0;
      ok = wr < F;
    } else if (EPI == EPI_QKV_ROPE) {
      const int n = n0 + t;
      ok = n < a.N;
      base = n < a.nq ? a.B0 : (n < a.nq + a.nk ? a.B1 : a.B2);
      wr = n < a.nq ? n : (n < a.nq + a.nk ? n - a.nq : n - a.nq - a.nk);
    } else {
      wr = n0 + t;
      base = a.B0;
      ok = wr < a.N;
    }
    bok[i] = ok;
    bsrc[i] = base + (int64_t)(ok ? wr : 0) * a.ldb + bcol[i];
  }

  uint4 ra[ACH], rb[BCH];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < ACH; ++i) ra[i] = aok[i] ? *reinterpret_cast<const uint4 *>(asrc[i] + k0) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < BCH; ++i) rb[i] = bok[i] ? *reinterpret_cast<const uint4 *>(bsrc[i] + k0) : make_uint4(0, 0, 0, 0);
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < ACH; ++i) *reinterpret_cast<uint4 *>(As + (buf * BM + arow[i]) * LDK + acol[i]) = ra[i];
#pragma unroll
    for (int i = 0; i < BCH; ++i) *reinterpret_cast<uint4 *>(Bs + (buf * BN + brow[i]) * LDK + bcol[i]) = rb[i];
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int KT = K / BK;
  gload(0);
  lstore(0);
  __syncthreads();
  const int lrow = lane & 31, lk = (lane >> 5) * 8;
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KT) gload((kt + 1) * BK);
    const u16 *Ab = As + (buf * BM + wm * WM + lrow) * LDK + lk;
    const u16 *Bb = Bs + (buf * BN + wn * WN + lrow) * LDK + lk;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8 af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) af[i] = *reinterpret_cast<const bf16x8 *>(Ab + i * 32 * LDK + kk * 16);
#pragma unroll
      for (int j = 0; j < FN; ++j) bfr[j] = *reinterpret_cast<const bf16x8 *>(Bb + j * 32 * LDK + kk * 16);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < KT) lstore(buf ^ 1);
    __syncthreads();
  }

  // ---------------- epilogue ----------------
  const int col_l = lane & 31;
  const int rbase = m0 + wm * WM + 4 * (lane >> 5);
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int col = n0 + wn * WN + j * 32 + col_l;
      if (EPI == EPI_SWIGLU) {
        if (j & 1) continue;  // odd blocks (up) are consumed with their gate block
        const int ucol = n0 / 2 + (wn * WN / 64 + j / 2) * 32 + col_l;
        const int F = a.N / 2;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = rbase + i * 32 + 8 * (r / 4) + (r % 4);
          if (row < a.M && ucol < F) {
            const float g = acc[i][j][r], up = acc[i][j + 1][r];
            static_cast<u16 *>(a.C)[(int64_t)row * a.ldc + ucol] = f2bf(silu(g) * up);
          }
        }
      } else if (EPI == EPI_QKV_ROPE) {
        const int Hq = a.H * a.hd, Hk = a.G * a.hd;
        const bool rot = col < Hq + Hk;
        const int c = col < Hq ? col : (col < Hq + Hk ? col - Hq : col - Hq - Hk);
        const int d = c % a.hd;
        const bool odd = col & 1;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = rbase + i * 32 + 8 * (r / 4) + (r % 4);
          float v = acc[i][j][r];
          const float pv = __shfl_xor(v, 1, kWave);
          const int rr = row < a.M ? row : a.M - 1;
          const int b = rr / a.S, s = rr % a.S;
          if (rot) {
            const float2 cs = a.tab[(int64_t)s * (a.hd / 2) + d / 2];
            const float2 y = odd ? rotate_pair(pv, v, cs.x, cs.y) : rotate_pair(v, pv, cs.x, cs.y);
            v = odd ? y.y : y.x;
          }
          if (row < a.M && col < a.N) {
            if (col < Hq) {
              a.q[(int64_t)row * Hq + col] = f2bf(v);
            } else {
              const int g = c / a.hd;
              const int p = a.start_pos + s;
              u16 *dst = static_cast<u16 *>(col < Hq + Hk ? a.kc : a.vc);
              dst[(((int64_t)b * a.cap + p) * a.G + g) * a.hd + d] = f2bf(v);
            }
          }
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = rbase + i * 32 + 8 * (r / 4) + (r % 4);
          if (row < a.M && col < a.N) {
            const float v = acc[i][j][r];
            if (EPI == EPI_RESID) {
              float *C = static_cast<float *>(a.C);
              C[(int64_t)row * a.ldc + col] = a.R[(int64_t)row * a.ldr + col] + v;
            } else if (EPI == EPI_STORE_F32) {
              static_cast<float *>(a.C)[(int64_t)row * a.ldc + col] = v;
            } else {
              static_cast<u16 *>(a.C)[(int64_t)row * a.ldc + col] = f2bf(v);
            }
          }
        }
      }
    }
  }
}

template <int BM, int BN, int EPI>
hipError_t launch_tile(const GemmArgs &a, hipStream_t s) {
  dim3 grid((a.M + BM - 1) / BM, (a.N + BN - 1) / BN);  // a.N counts B-rows
  const size_t lds = (size_t)2 * (BM + BN) * LDK * sizeof(u16);
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void *>(&gemm_bf16_kernel<BM, BN, EPI>),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  (void)attr;
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, EPI>), grid, dim3(256), lds, s, a);
  return hipGetLastError();
}

template <int EPI>
hipError_t launch_epi(const GemmArgs &a, hipStream_t s) {
  const long tiles256 = (long)((a.M + 255) / 256) * ((a.N + 255) / 256);
  if (tiles256 >= 512) return launch_tile<256, 256, EPI>(a, s);
  return launch_tile<128, 128, EPI>(a, s);
}
}  // namespace

hipError_t launch_gemm_bf16(int epi, const GemmArgs &a, hipStream_t s) {
  switch (epi) {
    case EPI_STORE_F32: return launch_epi<EPI_STORE_F32>(a, s);
    case EPI_RESID: return launch_epi<EPI_RESID>(a, s);
    case EPI_QKV_ROPE: return launch_epi<EPI_QKV_ROPE>(a, s);
    case EPI_SWIGLU: return launch_epi<EPI_SWIGLU>(a, s);
    case EPI_STORE_BF16: return launch_epi<EPI_STORE_BF16>(a, s);
  }
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// fp32 GEMM for the fp32 configuration: C = A * B^T (+R).  64x64 tiles,
// 16-deep K steps staged through LDS, 4x4 outputs per thread, fp32 FMA.
// ---------------------------------------------------------------------------
namespace {
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float *__restrict__ A, const float *__restrict__ B,
                                                       float *C, int64_t ldc, const float *R, int64_t ldr, int M,
                                                       int N, int K) {
  __shared__ float As[16][64 + 4];
  __shared__ float Bs[16][64 + 4];
  const int tid = threadIdx.x;
  const int m0 = blockIdx.x * 64, n0 = blockIdx.y * 64;
  const int tr = tid / 16, tc = tid % 16;  // 16x16 threads, 4x4 outputs each
  float acc[4][4] = {};
  const int lr = tid / 4, lk = (tid % 4) * 4;  // loader: row lr (0..63), k lk..lk+3
  for (int k0 = 0; k0 < K; k0 += 16) {
    float4 av = make_float4(0, 0, 0, 0), bv = make_float4(0, 0, 0, 0);
    if (m0 + lr < M) av = *reinterpret_cast<const float4 *>(A + (int64_t)(m0 + lr) * K + k0 + lk);
    if (n0 + lr < N) bv = *reinterpret_cast<const float4 *>(B + (int64_t)(n0 + lr) * K + k0 + lk);
    As[lk + 0][lr] = av.x; As[lk + 1][lr] = av.y; As[lk + 2][lr] = av.z; As[lk + 3][lr] = av.w;
    Bs[lk + 0][lr] = bv.x; Bs[lk + 1][lr] = bv.y; Bs[lk + 2][lr] = bv.z; Bs[lk + 3][lr] = bv.w;
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float a4[4], b4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a4[i] = As[kk][tr * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b4[j] = Bs[kk][tc * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a4[i], b4[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = m0 + tr * 4 + i;
    if (row >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + tc * 4 + j;
      if (col >= N) continue;
      const float v = acc[i][j];
      C[(int64_t)row * ldc + col] = R ? R[(int64_t)row * ldr + col] + v : v;
    }
  }
}
}  // namespace

hipError_t launch_gemm_f32(int epi, const float *A, const float *B, float *C, int64_t ldc, const float *R,
                           int64_t ldr, int M, int N, int K, hipStream_t s) {
  dim3 grid((M + 63) / 64, (N + 63) / 64);
  hipLaunchKernelGGL(gemm_f32_kernel, grid, dim3(256), 0, s, A, B, C, ldc, epi == EPI_RESID ? R : nullptr, ldr, M, N,
                     K);
  return hipGetLastError();
}

}  // namespace llk
