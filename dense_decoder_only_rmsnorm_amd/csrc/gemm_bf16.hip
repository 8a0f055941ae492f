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
// loop steps by 64 through two LDS stages.  Tiles move global -> LDS with
// global_load_lds_dwordx4 (no staging registers): one wave instruction fills
// 1 KB = 8 tile rows of 128 bytes, lane L landing at 16-byte slot L.  Each
// lane fetches the global piece that belongs in its slot under an XOR
// swizzle (16-byte chunk c of row r lives at chunk c ^ ((r >> 1) & 7)), so
// the 16-byte fragment reads of 16 consecutive rows hit 16 distinct bank
// groups.  The next stage is loading while the MFMAs consume the current
// one; operand fragments are double-buffered in registers across k-steps.
//
// MFMA 32x32x16 operand layout (lane l): A supplies row (l % 32) and eight
// consecutive k at 8*(l / 32); B likewise for output column (l % 32).  Output
// register r of lane l holds row 8*(r/4) + 4*(l/32) + (r%4), column l % 32.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace llk {

namespace {
constexpr int BK = 64;

template <int BM, int BN, int EPI>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(GemmArgs a) {
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int FM = WM / 32, FN = WN / 32;
  constexpr int RS = BK;                  // LDS row stride (bf16), 128 bytes, unpadded
  constexpr int AI = BM / 32, BI = BN / 32;  // 8-row load instructions per wave (A, B)
  extern __shared__ __align__(16) u16 smem[];
  u16 *As = smem;                         // [2][BM][RS]
  u16 *Bs = smem + 2 * BM * RS;           // [2][BN][RS]

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  // Tile order.  Workgroups go to the eight XCDs round-robin by linear id.
  // When both tile counts are multiples of 16, each run of 256 consecutive
  // ids covers a 16 x 16 block of tiles (M-blocks first), and the 32 tiles
  // one XCD receives from it form a 4 x 8 rectangle, so each XCD's L2 sees
  // four A row-blocks and eight B row-blocks per k-chunk, and the chip as a
  // whole works through the operands one 16 x 16 block at a time.
  int bm = blockIdx.x, bn = blockIdx.y;
  if ((gridDim.x & 15) == 0 && (gridDim.y & 15) == 0) {
    const int L = blockIdx.x + blockIdx.y * gridDim.x;
    const int sr = L >> 8, i = L & 255, x = i & 7, j = i >> 3;
    const int smt = gridDim.x >> 4;
    bm = 16 * (sr % smt) + 4 * (x & 3) + (j & 3);
    bn = 16 * (sr / smt) + 8 * (x >> 2) + (j >> 2);
  }
  const int m0 = bm * BM;
  const int n0 = bn * BN;
  const int K = a.K;

  // Loader: wave w fills tile rows 8j..8j+7 for j = w*AI + i (A) and w*BI + i
  // (B).  Lane L writes slot L of that 1 KB block: row 8j + L/8, physical
  // chunk L%8, which holds logical chunk (L%8) ^ ((row >> 1) & 7).  Rows past
  // M (A) or past the weight's rows (B) read a clamped valid row: they only
  // feed outputs that are never stored.
  const int lr = lane >> 3, lq = lane & 7;
  const u16 *asrc[AI];
#pragma unroll
  for (int i = 0; i < AI; ++i) {
    const int t = (wave * AI + i) * 8 + lr;
    const int c = lq ^ ((t >> 1) & 7);
    asrc[i] = a.A + (int64_t)min(m0 + t, a.M - 1) * a.lda + c * 8;
  }
  const u16 *bsrc[BI];
#pragma unroll
  for (int i = 0; i < BI; ++i) {
    const int t = (wave * BI + i) * 8 + lr;
    const int c = lq ^ ((t >> 1) & 7);
    const u16 *base;
    int wr, nrows;
    if (EPI == EPI_SWIGLU) {
      wr = n0 / 2 + (t >> 6) * 32 + (t & 31);  // 64 tile rows = 32 gate rows (w1) + 32 up rows (w3)
      base = ((t >> 5) & 1) ? a.B1 : a.B0;
      nrows = a.N / 2;
    } else if (EPI == EPI_QKV_ROPE) {
      const int n = n0 + t;
      base = n < a.nq ? a.B0 : (n < a.nq + a.nk ? a.B1 : a.B2);
      wr = n < a.nq ? n : (n < a.nq + a.nk ? n - a.nq : n - a.nq - a.nk);
      nrows = n < a.nq ? a.nq : (n < a.nq + a.nk ? a.nk : a.N - a.nq - a.nk);
    } else {
      wr = n0 + t;
      base = a.B0;
      nrows = a.N;
    }
    bsrc[i] = base + (int64_t)min(wr, nrows - 1) * a.ldb + c * 8;
  }
  // one load instruction of a stage refill: l < AI for A, then B
  auto issue_one = [&](int stage, int k0, int l) {
    if (l < AI) {
      const int j = __builtin_amdgcn_readfirstlane(wave * AI + l);
      __builtin_amdgcn_global_load_lds((const void *)(asrc[l] + k0),
                                       (__attribute__((address_space(3))) void *)(As + stage * BM * RS + j * 8 * RS), 16, 0, 0);
    } else {
      const int j = __builtin_amdgcn_readfirstlane(wave * BI + (l - AI));
      __builtin_amdgcn_global_load_lds((const void *)(bsrc[l - AI] + k0),
                                       (__attribute__((address_space(3))) void *)(Bs + stage * BN * RS + j * 8 * RS), 16, 0, 0);
    }
  };
  auto issue = [&](int stage, int k0) {
    u16 *ad = As + stage * BM * RS;
    u16 *bd = Bs + stage * BN * RS;
#pragma unroll
    for (int i = 0; i < AI; ++i) {
      const int j = __builtin_amdgcn_readfirstlane(wave * AI + i);
      __builtin_amdgcn_global_load_lds((const void *)(asrc[i] + k0), (__attribute__((address_space(3))) void *)(ad + j * 8 * RS), 16, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < BI; ++i) {
      const int j = __builtin_amdgcn_readfirstlane(wave * BI + i);
      __builtin_amdgcn_global_load_lds((const void *)(bsrc[i] + k0), (__attribute__((address_space(3))) void *)(bd + j * 8 * RS), 16, 0, 0);
    }
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // fragment read offsets: row (lane & 31) of a 32-row block, logical chunk
  // 2*kk + (lane >> 5), swizzled with ((row >> 1) & 7)
  const int frow = lane & 31;
  const int sw = (frow >> 1) & 7;
  int koff[BK / 16];
#pragma unroll
  for (int kk = 0; kk < BK / 16; ++kk) koff[kk] = (((2 * kk + (lane >> 5)) ^ sw) * 8);

  // Two stages.  Chunk kt is computed from stage kt&1 in four k-steps; the
  // fragments of step kk+1 are read during the MFMAs of step kk.  In the last
  // step of a chunk the wave waits for its loads of chunk kt+1, meets the
  // others at the barrier, and then refills the stage it just finished with
  // chunk kt+2 while it runs the step's remaining MFMAs: the refill loads and
  // the first fragment reads of chunk kt+1 are spread between those MFMAs, so
  // the address unit drains them while the matrix core stays busy.
  const int KT = K / BK;
  constexpr int KS = BK / 16;
  issue(0, 0);
  __syncthreads();
  if (KT > 1) issue(1, BK);
  bf16x8 af[2][FM], bfr[2][FN];
  {
    const u16 *Ab = As + (wm * WM + frow) * RS;
    const u16 *Bb = Bs + (wn * WN + frow) * RS;
#pragma unroll
    for (int i = 0; i < FM; ++i) af[0][i] = *reinterpret_cast<const bf16x8 *>(Ab + i * 32 * RS + koff[0]);
#pragma unroll
    for (int j = 0; j < FN; ++j) bfr[0][j] = *reinterpret_cast<const bf16x8 *>(Bb + j * 32 * RS + koff[0]);
  }
  auto run_chunk = [&](int kt, auto boundary) {
    constexpr bool BOUNDARY = decltype(boundary)::value;
    const int cur = kt & 1;
    const u16 *Ab = As + (cur * BM + wm * WM + frow) * RS;
    const u16 *Bb = Bs + (cur * BN + wn * WN + frow) * RS;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      const int cb = kk & 1;
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[0][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[cb][0], bfr[cb][j], acc[0][j], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      if (kk + 1 < KS) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
          af[cb ^ 1][i] = *reinterpret_cast<const bf16x8 *>(Ab + i * 32 * RS + koff[kk + 1]);
#pragma unroll
        for (int j = 0; j < FN; ++j)
          bfr[cb ^ 1][j] = *reinterpret_cast<const bf16x8 *>(Bb + j * 32 * RS + koff[kk + 1]);
        __builtin_amdgcn_sched_barrier(0);
      } else if (BOUNDARY) {
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's loads of chunk kt+1 have landed
        __syncthreads();                      // everyone's have, and everyone is done reading stage cur
        // Refill (past the last chunk the last chunk is loaded again into
        // this dead stage, which keeps the step free of branches), spread
        // between the step's remaining MFMAs together with the first
        // fragment reads of chunk kt+1.
        const int k0 = min(kt + 2, KT - 1) * BK;
        const u16 *An = As + ((cur ^ 1) * BM + wm * WM + frow) * RS;
        const u16 *Bn = Bs + ((cur ^ 1) * BN + wn * WN + frow) * RS;
        constexpr int NM = (FM - 1) * FN, NL = AI + BI, NR = FM + FN;
#pragma unroll
        for (int q = 0; q < NM; ++q) {
          const int i = 1 + q / FN, j = q % FN;
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[cb][i], bfr[cb][j], acc[i][j], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int l = q * NL / NM; l < (q + 1) * NL / NM; ++l) issue_one(cur, k0, l);
#pragma unroll
          for (int r = q * NR / NM; r < (q + 1) * NR / NM; ++r) {
            if (r < FM) af[cb ^ 1][r] = *reinterpret_cast<const bf16x8 *>(An + r * 32 * RS + koff[0]);
            else bfr[cb ^ 1][r - FM] = *reinterpret_cast<const bf16x8 *>(Bn + (r - FM) * 32 * RS + koff[0]);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        continue;
      }
#pragma unroll
      for (int i = 1; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[cb][i], bfr[cb][j], acc[i][j], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  for (int kt = 0; kt + 1 < KT; ++kt) run_chunk(kt, std::true_type{});
  run_chunk(KT - 1, std::false_type{});
  __builtin_amdgcn_s_waitcnt(0x0F70);  // the refill of the dead stage has landed before LDS is reused
  __syncthreads();  // every wave is done with the stages before the epilogue reuses them

  // ---------------- epilogue ----------------
  const int col_l = lane & 31;
  const int rloc = wm * WM + 4 * (lane >> 5);  // tile-local row base of this lane
  if (EPI == EPI_RESID || EPI == EPI_STORE_F32) {
    // fp32 outputs: each store instruction writes 32 consecutive floats of a
    // row.  The residual loads of one 32-row block (FN x 16 per lane) are
    // issued together from clamped, always valid addresses, so they overlap
    // instead of each waiting for the previous one; only stores are guarded.
    float *C = static_cast<float *>(a.C);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      float rv[FN][16];
      if (EPI == EPI_RESID) {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int col = min(n0 + wn * WN + j * 32 + col_l, a.N - 1);
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = min(m0 + rloc + i * 32 + 8 * (r / 4) + (r % 4), a.M - 1);
            rv[j][r] = a.R[(int64_t)row * a.ldr + col];
          }
        }
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int col = n0 + wn * WN + j * 32 + col_l;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = m0 + rloc + i * 32 + 8 * (r / 4) + (r % 4);
          const float v = EPI == EPI_RESID ? rv[j][r] + acc[i][j][r] : acc[i][j][r];
          if (row < a.M && col < a.N) C[(int64_t)row * a.ldc + col] = v;
        }
      }
    }
    return;
  }

  // bf16 outputs: finish the values in registers, stage the tile in LDS as
  // bf16, then write it out in 16-byte pieces of 8 consecutive columns.
  constexpr int CN = (EPI == EPI_SWIGLU) ? BN / 2 : BN;  // output columns of the tile
  constexpr int LDC = CN + 8;
  u16 *Cs = smem;  // [BM][LDC], reuses the operand buffers (loop ended with a barrier)
  if (EPI == EPI_QKV_ROPE) {
    // Table row offsets of this lane's 16 rows of row block i.  Rows past the
    // matrix are clamped to its last row so every lookup stays inside the
    // table; their values are not stored.
    const int pbase = m0 % a.S;  // sequence position of tile row 0 (table row = row % S)
    auto row_offsets = [&](int i, int *toff) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int x = min(rloc + i * 32 + 8 * (r / 4) + (r % 4), a.M - 1 - m0);
        int p = pbase + x;
        // sequences of at least BM rows wrap at most once within a tile (a
        // select); shorter ones take the (uniform) modulo path
        if (a.S >= BM)
          p = p >= a.S ? p - a.S : p;
        else
          p %= a.S;
        toff[r] = p * (a.hd / 2);
      }
    };
    // A 32-column block lies inside one head of one of q, k, v (the head size
    // is a multiple of 32, checked at launch), so whether it rotates and its
    // table column are the same for the whole block.  v blocks read a valid
    // table entry and apply the identity.
    const int Hq = a.H * a.hd, Hk = a.G * a.hd;
    int dh[FN];
    bool rot[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int col0 = n0 + wn * WN + j * 32;
      rot[j] = col0 < Hq + Hk;
      dh[j] = rot[j] ? (((col0 < Hq ? col0 : col0 - Hq) % a.hd) + col_l) >> 1 : 0;
    }
    // pair (2t, 2t+1) sits in lanes (2t, 2t+1) of one row:
    //   even: x0 cos - x1 sin,  odd: x1 cos + x0 sin
    const float sgn = (lane & 1) ? 1.f : -1.f;
    // the table entries of block q+1 are loaded while block q is rotated
    // (row offsets of row blocks i and i+1 live at a time)
    constexpr int NQ = FM * FN;
    int toff[2][16];
    row_offsets(0, toff[0]);
    float2 cs[2][16];
    // (32-bit byte offsets from the table base: loads take a scalar base)
    const char *tab = reinterpret_cast<const char *>(a.tab);
    auto tab_at = [&](int e) { return *reinterpret_cast<const float2 *>(tab + (uint32_t)e * 8u); };
#pragma unroll
    for (int r = 0; r < 16; ++r) cs[0][r] = tab_at(toff[0][r] + dh[0]);
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int i = q / FN, j = q % FN;
      if (j == 0 && i + 1 < FM) row_offsets(i + 1, toff[(i + 1) & 1]);
      if (q + 1 < NQ) {
#pragma unroll
        for (int r = 0; r < 16; ++r) cs[(q + 1) & 1][r] = tab_at(toff[((q + 1) / FN) & 1][r] + dh[(q + 1) % FN]);
      }
      const int ccol = wn * WN + j * 32 + col_l;
      if (rot[j]) {  // wave-uniform
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rr = rloc + i * 32 + 8 * (r / 4) + (r % 4);
          const float v = acc[i][j][r];
          const float pv = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
          Cs[rr * LDC + ccol] = f2bf(fmaf(pv, sgn * cs[q & 1][r].y, v * cs[q & 1][r].x));
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rr = rloc + i * 32 + 8 * (r / 4) + (r % 4);
          Cs[rr * LDC + ccol] = f2bf(acc[i][j][r]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);  // keeps the loads one block ahead, not all hoisted
    }
  } else {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        if (EPI == EPI_SWIGLU) {
          if (j & 1) continue;  // the up block j+1 is consumed with its gate block j
          const int ccol = (wn * WN / 64 + j / 2) * 32 + col_l;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int rr = rloc + i * 32 + 8 * (r / 4) + (r % 4);
            Cs[rr * LDC + ccol] = f2bf(silu(acc[i][j][r]) * acc[i][j + 1][r]);
          }
        } else {
          const int ccol = wn * WN + j * 32 + col_l;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int rr = rloc + i * 32 + 8 * (r / 4) + (r % 4);
            Cs[rr * LDC + ccol] = f2bf(acc[i][j][r]);
          }
        }
      }
  }
  __syncthreads();
  constexpr int CPR = CN / 8;  // 16-byte pieces per tile row
  static_assert(256 % CPR == 0, "a thread keeps one column piece for the whole copy");
  // Each thread copies the same 8 columns of every (256 / CPR)-th row, so
  // everything that depends on the column is computed once.
  const int c8 = (tid % CPR) * 8;
  const int col = (EPI == EPI_SWIGLU ? n0 / 2 : n0) + c8;
  if (col >= (EPI == EPI_SWIGLU ? a.N / 2 : a.N)) return;
  if (EPI == EPI_QKV_ROPE) {
    const int Hq = a.H * a.hd, Hk = a.G * a.hd;
    if (col < Hq) {
      for (int rr = tid / CPR; rr < BM && m0 + rr < a.M; rr += 256 / CPR)
        *reinterpret_cast<uint4 *>(a.q + (int64_t)(m0 + rr) * Hq + col) =
            *reinterpret_cast<const uint4 *>(Cs + rr * LDC + c8);
      return;
    }
    // k or v: row m0 + rr is (batch b, position p) of the cache
    const bool isk = col < Hq + Hk;
    const int cc = isk ? col - Hq : col - Hq - Hk;
    const int g = cc / a.hd, d = cc % a.hd;
    u16 *dst = static_cast<u16 *>(isk ? a.kc : a.vc) + (int64_t)g * a.hd + d;
    const int b0 = m0 / a.S, p0 = m0 % a.S;
    for (int rr = tid / CPR; rr < BM && m0 + rr < a.M; rr += 256 / CPR) {
      int b = b0, p = p0 + rr;
      if (a.S >= BM) {  // at most one wrap within a tile (selects)
        const bool w = p >= a.S;
        p = w ? p - a.S : p;
        b = w ? b + 1 : b;
      } else {
        b += p / a.S;
        p %= a.S;
      }
      *reinterpret_cast<uint4 *>(dst + ((int64_t)b * a.cap + p + a.start_pos) * a.G * a.hd) =
          *reinterpret_cast<const uint4 *>(Cs + rr * LDC + c8);
    }
    return;
  }
  u16 *C = static_cast<u16 *>(a.C) + col;
  for (int rr = tid / CPR; rr < BM && m0 + rr < a.M; rr += 256 / CPR)
    *reinterpret_cast<uint4 *>(C + (int64_t)(m0 + rr) * a.ldc) = *reinterpret_cast<const uint4 *>(Cs + rr * LDC + c8);
}

template <int BM, int BN, int EPI>
hipError_t launch_tile(const GemmArgs &a, hipStream_t s) {
  dim3 grid((a.M + BM - 1) / BM, (a.N + BN - 1) / BN);  // a.N counts B-rows
  constexpr int CN = (EPI == EPI_SWIGLU) ? BN / 2 : BN;
  const size_t lds = std::max((size_t)2 * (BM + BN) * BK * sizeof(u16), (size_t)BM * (CN + 8) * sizeof(u16));
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
    case EPI_QKV_ROPE:
      if (a.hd % 32) return hipErrorInvalidValue;  // the epilogue takes 32-column blocks inside one head
      return launch_epi<EPI_QKV_ROPE>(a, s);
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
