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
// loop steps through chunks of BK = 32 or 64 held in NS LDS stages (the
// launches use BK = 64 in two stages).  Tiles move global -> LDS with raw
// buffer loads straight into LDS (buffer_load_dwordx4 ... lds, no staging
// registers): one wave instruction fills 1 KB = 1024 / (2 BK) tile rows,
// lane L landing at 16-byte slot L.  Each lane fetches the global piece that
// belongs in its slot under an XOR swizzle (16-byte chunk c of row r lives at
// chunk c ^ ((r >> SH) & (BK/8 - 1)), SH = 1 for 128-byte rows and 2 for
// 64-byte rows), so the 16-byte fragment reads of 16 consecutive rows hit 16
// distinct bank groups.  While chunk kt is computed, chunks kt+1 .. kt+NS-1
// are in flight or landed.  Operand fragments are double-buffered in
// registers across k-steps.
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
// s_waitcnt operand: vmcnt <= n (n < 64) and lgkmcnt = 0, expcnt not waited on
constexpr int vm_lgkm_wait(int n) { return (n & 15) | ((n >> 4) << 14) | 0x70; }

// One 1 KB load into LDS: lane L's 16 bytes at byte voff + soff of the raw
// buffer [base, base + bytes) (clamped to 4 GiB - 1; reads past the end
// return zero) land at LDS slot L of dst.
__device__ __forceinline__ void buffer_load_lds16(const u16 *base, int64_t bytes, u16 *dst, uint32_t voff, uint32_t soff) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<u16 *>(base), (short)0, (int)(uint32_t)(bytes < 0xFFFFFFFFll ? bytes : 0xFFFFFFFFll),
      0x00020000);  // untyped, 32-bit data format, no stride
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)dst, 16, voff, soff, 0, 0);
}

// One float of the raw buffer [base, base + bytes) at byte voff + soff.
__device__ __forceinline__ float buffer_load_f32(const float *base, int64_t bytes, uint32_t voff, uint32_t soff) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float *>(base), (short)0, (int)(uint32_t)(bytes < 0xFFFFFFFFll ? bytes : 0xFFFFFFFFll), 0x00020000);
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}
__device__ __forceinline__ void buffer_store_f32(float v, float *base, int64_t bytes, uint32_t voff, uint32_t soff) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
      base, (short)0, (int)(uint32_t)(bytes < 0xFFFFFFFFll ? bytes : 0xFFFFFFFFll), 0x00020000);
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, voff, soff, 0);
}

// Copy-out of a whole staged tile: thread tid moves the 16-byte piece at
// column c8 of every (256 / CPR)-th row from LDS to dst + row * ld.  The LDS
// reads go out in batches of eight before their stores (one read-wait-store
// per row otherwise; the empty asm keeps the stores behind the batch).
template <int BM, int CPR, int LDC>
__device__ __forceinline__ void copy_whole_tile(const u16 *Cs, int tid, int c8, u16 *dst, int64_t ld) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  constexpr int STEP = 256 / CPR, NIT = BM / STEP, NB = NIT < 8 ? NIT : 8;
  const int r0 = tid / CPR;
  u16 *dr = dst + r0 * ld;
  const int64_t rstep = STEP * ld;
#pragma unroll
  for (int i0 = 0; i0 < NIT; i0 += NB) {
    u32x4 v[NB];
#pragma unroll
    for (int u = 0; u < NB; ++u) v[u] = *reinterpret_cast<const u32x4 *>(Cs + (r0 + (i0 + u) * STEP) * LDC + c8);
#pragma unroll
    for (int u = 0; u < NB; ++u) asm volatile("" : "+v"(v[u]));
#pragma unroll
    for (int u = 0; u < NB; ++u) *reinterpret_cast<u32x4 *>(dr + (i0 + u) * rstep) = v[u];
  }
}

template <int BM, int BN, int BK, int NS, int EPI>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(GemmArgs a) {
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int FM = WM / 32, FN = WN / 32;
  constexpr int RS = BK;                     // LDS row stride (bf16): 64 or 128 bytes, unpadded
  constexpr int CH = BK / 8;                 // 16-byte chunks per row
  constexpr int RPI = 64 / CH;               // tile rows one 1 KB load instruction fills
  constexpr int SH = CH == 8 ? 1 : 2;        // swizzle shift
  constexpr int AI = BM / RPI / 4, BI = BN / RPI / 4;  // load instructions per wave and stage (A, B)
  constexpr int NL = AI + BI;
  static_assert(BK == 32 || BK == 64, "rows of 64 or 128 bytes");
  static_assert(NS >= 2 && NS * NL <= 63, "the outstanding loads of all stages fit the vmcnt counter");
  extern __shared__ __align__(16) u16 smem[];
  u16 *As = smem;                         // [NS][BM][RS]
  u16 *Bs = smem + NS * BM * RS;          // [NS][BN][RS]

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

  // Loader: wave w fills the RPI-row groups j = w*AI + i (A) and w*BI + i
  // (B).  Lane L writes slot L of that 1 KB block: row RPI*j + L/CH,
  // physical chunk L%CH, which holds logical chunk (L%CH) ^ swizzle(row).
  // The loads are raw buffer loads: A's resource starts at the tile's first
  // row, each weight matrix's covers the whole matrix (below 4 GiB, checked
  // at launch); a lane's 32-bit offset is its row times the row pitch plus
  // its 16-byte chunk, and the k position of the chunk goes in the scalar
  // offset, so a refill costs no vector address arithmetic.  Rows past M
  // (A) or past a weight's rows (B) read a clamped valid row: they only feed
  // outputs that are never stored.
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int lr = lane / CH, lq = lane % CH;
  const u16 *abase = a.A + (int64_t)m0 * a.lda;
  const int64_t abytes = (int64_t)(a.M - m0) * a.lda * 2;
  uint32_t aoff[AI];
#pragma unroll
  for (int i = 0; i < AI; ++i) {
    const int t = (wave * AI + i) * RPI + lr;
    const int c = lq ^ ((t >> SH) & (CH - 1));
    aoff[i] = (uint32_t)((min(m0 + t, a.M - 1) - m0) * a.lda * 2 + c * 16);
  }
  // weight matrices: B0 alone, w1 / w3 (SwiGLU), or wq / wk / wv (QKV)
  const int nq = EPI == EPI_QKV_ROPE ? a.nq : (EPI == EPI_SWIGLU ? a.N / 2 : a.N);
  const int nk = EPI == EPI_QKV_ROPE ? a.nk : (EPI == EPI_SWIGLU ? a.N / 2 : 0);
  uint32_t boff[BI];
  const u16 *bbase[BI];  // the matrix load i reads (uniform: a row group never straddles two)
  int64_t bbytes[BI];
#pragma unroll
  for (int i = 0; i < BI; ++i) {
    const int t = (wave * BI + i) * RPI + lr;
    const int tg = (wv * BI + i) * RPI;  // the group's first tile row
    const int c = lq ^ ((t >> SH) & (CH - 1));
    int wr, nrows, sel;
    if (EPI == EPI_SWIGLU) {
      wr = n0 / 2 + (t >> 6) * 32 + (t & 31);  // 64 tile rows = 32 gate rows (w1) + 32 up rows (w3)
      sel = (tg >> 5) & 1;
      nrows = a.N / 2;
    } else if (EPI == EPI_QKV_ROPE) {
      const int n = n0 + t, ng = n0 + tg;
      sel = ng < a.nq ? 0 : (ng < a.nq + a.nk ? 1 : 2);
      wr = n < a.nq ? n : (n < a.nq + a.nk ? n - a.nq : n - a.nq - a.nk);
      nrows = n < a.nq ? a.nq : (n < a.nq + a.nk ? a.nk : a.N - a.nq - a.nk);
    } else {
      wr = n0 + t;
      sel = 0;
      nrows = a.N;
    }
    boff[i] = (uint32_t)(min(wr, nrows - 1) * a.ldb * 2 + c * 16);
    // the matrix as an offset from B0 in arithmetic (a select between the
    // pointer fields would become a scalar load of the argument block with a
    // computed offset, and its wait, in every refill)
    const int64_t d1 = a.B1 - a.B0, d2 = a.B2 - a.B0;
    bbase[i] = a.B0 + (sel == 1 ? d1 : 0) + (sel == 2 ? d2 : 0);
    bbytes[i] = (int64_t)(sel == 0 ? nq : (sel == 1 ? nk : a.N - nq - nk)) * a.ldb * 2;
  }
  // one load instruction of a stage refill: l < AI for A, then B
  auto issue_one = [&](int stage, int k0, int l) {
    if (l < AI) {
      buffer_load_lds16(abase, abytes, As + stage * BM * RS + (wv * AI + l) * RPI * RS, aoff[l], k0 * 2);
    } else {
      const int i = l - AI;
      buffer_load_lds16(bbase[i], bbytes[i], Bs + stage * BN * RS + (wv * BI + i) * RPI * RS, boff[i], k0 * 2);
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
  // 2*kk + (lane >> 5), swizzled
  const int frow = lane & 31;
  const int sw = (frow >> SH) & (CH - 1);
  int koff[BK / 16];
#pragma unroll
  for (int kk = 0; kk < BK / 16; ++kk) koff[kk] = (((2 * kk + (lane >> 5)) ^ sw) * 8);

  // Chunk kt is computed from stage kt % NS in BK/16 k-steps; the fragments
  // of step kk+1 are read during the MFMAs of step kk.  In the last step of a
  // chunk the wave waits until its own loads of chunk kt+1 have landed (loads
  // complete in order; those of chunks kt+2 .. kt+NS-1 stay in flight),
  // meets the others at the barrier (after it every wave's part of chunk
  // kt+1 is in LDS and every wave is done reading stage kt % NS), and then
  // refills that stage with chunk kt+NS while it runs the step's remaining
  // MFMAs: the refill loads and the first fragment reads of chunk kt+1 are
  // spread between those MFMAs, so the address unit drains them while the
  // matrix core stays busy.  Chunks past the last one load the last chunk
  // again into a dead stage, which keeps the count of loads in flight, and
  // so every wait, the same in every step.
  const int KT = K / BK;
  constexpr int KS = BK / 16;
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int l = 0; l < NL; ++l) issue_one(s, min(s, KT - 1) * BK, l);
  __builtin_amdgcn_s_waitcnt(vm_lgkm_wait((NS - 1) * NL));  // this wave's part of chunk 0 has landed
  asm volatile("s_barrier" ::: "memory");                      // and everyone's
  bf16x8 af[2][FM], bfr[2][FN];
  {
    const u16 *Ab = As + (wm * WM + frow) * RS;
    const u16 *Bb = Bs + (wn * WN + frow) * RS;
#pragma unroll
    for (int i = 0; i < FM; ++i) af[0][i] = *reinterpret_cast<const bf16x8 *>(Ab + i * 32 * RS + koff[0]);
#pragma unroll
    for (int j = 0; j < FN; ++j) bfr[0][j] = *reinterpret_cast<const bf16x8 *>(Bb + j * 32 * RS + koff[0]);
  }
  int cur = 0;  // stage of chunk kt
  auto run_chunk = [&](int kt, auto boundary) {
    constexpr bool BOUNDARY = decltype(boundary)::value;
    const int nxt = cur + 1 == NS ? 0 : cur + 1;
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
        __builtin_amdgcn_s_waitcnt(vm_lgkm_wait((NS - 2) * NL));
        asm volatile("s_barrier" ::: "memory");
        const int k0 = min(kt + NS, KT - 1) * BK;
        const u16 *An = As + (nxt * BM + wm * WM + frow) * RS;
        const u16 *Bn = Bs + (nxt * BN + wn * WN + frow) * RS;
        constexpr int NM = (FM - 1) * FN, NR = FM + FN;
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
    cur = nxt;
  };
  for (int kt = 0; kt + 1 < KT; ++kt) run_chunk(kt, std::true_type{});
  run_chunk(KT - 1, std::false_type{});
  __builtin_amdgcn_s_waitcnt(vm_lgkm_wait(0));  // the refills of dead stages have landed before LDS is reused
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
    if (m0 + BM <= a.M && n0 + BN <= a.N) {
      // A whole tile: raw buffer accesses from the tile's first element, the
      // lane's column and row-within-group in a vector offset, the row of
      // each accumulator register in the scalar offset; no guards and no
      // per-element address arithmetic.
      const int wmu = wv >> 1, wnu = wv & 1;
      const float *Rt = a.R + (int64_t)m0 * a.ldr + n0;
      float *Ct = C + (int64_t)m0 * a.ldc + n0;
      const int64_t rbytes = ((int64_t)(a.M - m0) * a.ldr - n0) * 4, cbytes = ((int64_t)(a.M - m0) * a.ldc - n0) * 4;
      // The residual rows of 32-row block i+1 are loaded before block i is
      // stored: the output may be the residual itself, so a load placed
      // after a store would wait for that store to complete.
      float rv[2][FN][16];
      auto load_block = [&](int i, auto buf_c) {
        constexpr int BUF = decltype(buf_c)::value;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const uint32_t vo = (uint32_t)((4 * (lane >> 5)) * a.ldr + wnu * WN + j * 32 + col_l) * 4u;
#pragma unroll
          for (int r = 0; r < 16; ++r)
            rv[BUF][j][r] = buffer_load_f32(Rt, rbytes, vo, (uint32_t)((wmu * WM + i * 32 + 8 * (r / 4) + (r % 4)) * a.ldr) * 4u);
        }
      };
      if (EPI == EPI_RESID) load_block(0, std::integral_constant<int, 0>());
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        if (EPI == EPI_RESID && i + 1 < FM) {
          if (i & 1) load_block(i + 1, std::integral_constant<int, 0>());
          else load_block(i + 1, std::integral_constant<int, 1>());
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const uint32_t vo = (uint32_t)((4 * (lane >> 5)) * a.ldc + wnu * WN + j * 32 + col_l) * 4u;
#pragma unroll
          for (int r = 0; r < 16; ++r)
            buffer_store_f32(EPI == EPI_RESID ? rv[i & 1][j][r] + acc[i][j][r] : acc[i][j][r], Ct, cbytes, vo,
                             (uint32_t)((wmu * WM + i * 32 + 8 * (r / 4) + (r % 4)) * a.ldc) * 4u);
        }
      }
      return;
    }
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
      if (m0 + BM <= a.M) {
        copy_whole_tile<BM, CPR, LDC>(Cs, tid, c8, a.q + (int64_t)m0 * Hq + col, Hq);
        return;
      }
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
  if (m0 + BM <= a.M) {
    copy_whole_tile<BM, CPR, LDC>(Cs, tid, c8, C + (int64_t)m0 * a.ldc, a.ldc);
    return;
  }
  for (int rr = tid / CPR; rr < BM && m0 + rr < a.M; rr += 256 / CPR)
    *reinterpret_cast<uint4 *>(C + (int64_t)(m0 + rr) * a.ldc) = *reinterpret_cast<const uint4 *>(Cs + rr * LDC + c8);
}

template <int BM, int BN, int BK, int NS, int EPI>
hipError_t launch_tile(const GemmArgs &a, hipStream_t s) {
  dim3 grid((a.M + BM - 1) / BM, (a.N + BN - 1) / BN);  // a.N counts B-rows
  constexpr int CN = (EPI == EPI_SWIGLU) ? BN / 2 : BN;
  const size_t lds = std::max((size_t)NS * (BM + BN) * BK * sizeof(u16), (size_t)BM * (CN + 8) * sizeof(u16));
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void *>(&gemm_bf16_kernel<BM, BN, BK, NS, EPI>),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, BK, NS, EPI>), grid, dim3(256), lds, s, a);
  return hipGetLastError();
}

template <int EPI>
hipError_t launch_epi(const GemmArgs &a, hipStream_t s) {
  const long tiles256 = (long)((a.M + 255) / 256) * ((a.N + 255) / 256);
  if (tiles256 >= 512) return launch_tile<256, 256, 64, 2, EPI>(a, s);
  return launch_tile<128, 128, 64, 2, EPI>(a, s);
}
}  // namespace

hipError_t launch_gemm_bf16(int epi, const GemmArgs &a, hipStream_t s) {
  // the loads and fp32 stores take 32-bit byte offsets: every weight matrix
  // and any 256 rows of the activations, the output and the residual stay
  // below 4 GiB
  if ((int64_t)a.N * a.ldb * 2 > 0xFFFFFFFFll || (int64_t)256 * a.lda * 2 > 0xFFFFFFFFll ||
      (int64_t)256 * a.ldc * 4 > 0xFFFFFFFFll || (int64_t)256 * a.ldr * 4 > 0xFFFFFFFFll)
    return hipErrorInvalidValue;
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
// fp32 GEMM for the fp32 configuration: C = A * B^T (+R), A [M][K] and B [N][K]
// row-major fp32, K a multiple of 64.  fp32 matrix cores
// (v_mfma_f32_32x32x2_f32: lane l supplies A[l % 32][l / 32] and
// B^T[l / 32][l % 32]; output register r of lane l holds row
// 8*(r/4) + 4*(l/32) + r%4, column l % 32).  A block of 256 threads owns a
// 64 x 64 tile, each wave 32 x 32; K steps by 64 through LDS (rows padded to
// 66 floats: the 32 rows x 2 k a fragment read touches fall in distinct
// banks), the next step's operands (four 16-byte loads per matrix and
// thread) prefetched into registers; even and odd k pairs accumulate in
// separate chains so consecutive MFMAs are independent.  Rows past M or N
// read a clamped valid row and are not stored.
// ---------------------------------------------------------------------------
namespace {
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float *__restrict__ A, const float *__restrict__ B,
                                                       float *C, int64_t ldc, const float *R, int64_t ldr, int M,
                                                       int N, int K) {
  constexpr int BKF = 64, LD = BKF + 2, NL = 64 * BKF / 4 / 256;  // 16-byte loads per matrix and thread
  __shared__ float As[64 * LD];
  __shared__ float Bs[64 * LD];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.x * 64, n0 = blockIdx.y * 64;
  // loader: load i of thread t covers row (t + 256 i) / 16, k 4 * (t % 16) .. +3
  const int lk = (tid & 15) * 4;
  const float *ap[NL], *bp[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int r = (tid + 256 * i) >> 4;
    ap[i] = A + (int64_t)min(m0 + r, M - 1) * K + lk;
    bp[i] = B + (int64_t)min(n0 + r, N - 1) * K + lk;
  }
  f32x16 acc0, acc1;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc0[r] = acc1[r] = 0.f;
  float4 ra[NL], rb[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    ra[i] = *reinterpret_cast<const float4 *>(ap[i]);
    rb[i] = *reinterpret_cast<const float4 *>(bp[i]);
  }
  const int fr = lane & 31, fk = lane >> 5;
  const float *af = As + (wm * 32 + fr) * LD + fk;
  const float *bf = Bs + (wn * 32 + fr) * LD + fk;
  for (int k0 = 0; k0 < K; k0 += BKF) {
    __syncthreads();  // every wave is done with the previous step's tiles
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int o = ((tid + 256 * i) >> 4) * LD + lk;
      *reinterpret_cast<float2 *>(As + o) = make_float2(ra[i].x, ra[i].y);
      *reinterpret_cast<float2 *>(As + o + 2) = make_float2(ra[i].z, ra[i].w);
      *reinterpret_cast<float2 *>(Bs + o) = make_float2(rb[i].x, rb[i].y);
      *reinterpret_cast<float2 *>(Bs + o + 2) = make_float2(rb[i].z, rb[i].w);
    }
    __syncthreads();
    if (k0 + BKF < K) {
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        ra[i] = *reinterpret_cast<const float4 *>(ap[i] + k0 + BKF);
        rb[i] = *reinterpret_cast<const float4 *>(bp[i] + k0 + BKF);
      }
    }
#pragma unroll
    for (int kk = 0; kk < BKF; kk += 4) {
      acc0 = __builtin_amdgcn_mfma_f32_32x32x2f32(af[kk], bf[kk], acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x2f32(af[kk + 2], bf[kk + 2], acc1, 0, 0, 0);
    }
  }
  const int col = n0 + wn * 32 + fr;
  // the residual loads (from clamped, valid rows and columns) all before the
  // first store: the output may be the residual itself
  float rv[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = m0 + wm * 32 + 8 * (r >> 2) + 4 * fk + (r & 3);
    rv[r] = R ? R[(int64_t)min(row, M - 1) * ldr + min(col, N - 1)] : 0.f;
  }
  // the sums formed before the guarded stores (the empty asm keeps the
  // compiler from sinking them into the branches), so that no store's branch
  // waits for the loads again
  float out[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const float v = acc0[r] + acc1[r];
    out[r] = R ? rv[r] + v : v;
    asm volatile("" : "+v"(out[r]));
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = m0 + wm * 32 + 8 * (r >> 2) + 4 * fk + (r & 3);
    if (row < M && col < N) C[(int64_t)row * ldc + col] = out[r];
  }
}
}  // namespace

hipError_t launch_gemm_f32(int epi, const float *A, const float *B, float *C, int64_t ldc, const float *R,
                           int64_t ldr, int M, int N, int K, hipStream_t s) {
  if (K % 64) return hipErrorInvalidValue;
  dim3 grid((M + 63) / 64, (N + 63) / 64);
  hipLaunchKernelGGL(gemm_f32_kernel, grid, dim3(256), 0, s, A, B, C, ldc, epi == EPI_RESID ? R : nullptr, ldr, M, N,
                     K);
  return hipGetLastError();
}

}  // namespace llk
