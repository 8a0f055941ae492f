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
// (grid.y).  The K slice streams through NS LDS stages of 64 k: weights and
// both activation planes arrive with raw buffer loads straight into LDS
// (buffer_load_dwordx4 ... lds) in fully coalesced 1 KB pieces (8 rows x 128
// bytes), stored with the 16-byte chunk swizzle c ^ ((row >> 1) & 7) so the
// MFMA fragment reads of 16 consecutive rows are bank-conflict free.  The activations are shared by all waves
// through LDS.  Waves w and w + NR/RW own the same RW B-rows and split each
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
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace llk {

namespace {

constexpr int SK_KCH = 64;     // k per LDS stage
constexpr int SK_ROWB = SK_KCH * 2;  // bytes per tile row (128)

// s_waitcnt vmcnt(n) for a wave-uniform n <= 63 (the count must be an
// immediate: vmcnt bits 3:0 and 15:14, expcnt and lgkmcnt not waited on)
__device__ __forceinline__ void wait_vmcnt(int n) {
  switch (n) {
#define LLK_VM(i) \
  case i: __builtin_amdgcn_s_waitcnt(0x0F70 | ((i) & 15) | (((i) >> 4) << 14)); break;
#define LLK_VM8(i) LLK_VM(i) LLK_VM(i + 1) LLK_VM(i + 2) LLK_VM(i + 3) LLK_VM(i + 4) LLK_VM(i + 5) LLK_VM(i + 6) LLK_VM(i + 7)
    LLK_VM8(0) LLK_VM8(8) LLK_VM8(16) LLK_VM8(24) LLK_VM8(32) LLK_VM8(40) LLK_VM8(48) LLK_VM8(56)
#undef LLK_VM8
#undef LLK_VM
    default: __builtin_amdgcn_s_waitcnt(0x0F70); break;  // vmcnt(0)
  }
}

// One 1 KB load into LDS: lane L's 16 bytes at byte voff + soff of the raw
// buffer [base, base + bytes) (clamped to 4 GiB - 1; reads past the end
// return zero) land at LDS slot L of dst.
__device__ __forceinline__ void sk_load_lds(const u16 *base, int64_t bytes, u16 *dst, uint32_t voff, uint32_t soff) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<u16 *>(base), (short)0, (int)(uint32_t)(bytes < 0xFFFFFFFFll ? bytes : 0xFFFFFFFFll),
      0x00020000);  // untyped, 32-bit data format, no stride
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)dst, 16, voff, soff, 0, 0);
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
  // K slice ks: chunks [ks*T/ksplit, (ks+1)*T/ksplit) of the T = K/64 (the
  // slices differ by at most one chunk when ksplit does not divide T)
  const int T = a.K / SK_KCH;
  const int cbeg = ks * T / a.ksplit;
  const int kbeg = cbeg * SK_KCH;
  const int nchunk = (ks + 1) * T / a.ksplit - cbeg;

  // Loader: 16 + NR/8 pieces of 1 KB per stage (A hi 8, A lo 8, B NR/8),
  // piece p at stage offset 512*p; wave w issues pieces w, w + NW, ...
  // Piece p covers rows 8*(p%8) .. +7 of A hi (p < 8) or A lo (p < 16), else
  // rows 8*(p-16) .. +7 of B; lane L -> row 8*(piece row) + L/8, physical
  // chunk L%8 holding logical chunk (L%8) ^ ((row >> 1) & 7).  Rows past M or
  // past the weight read a clamped valid row: they only feed outputs that are
  // never stored.
  static_assert((16 + NR / 8) % NW == 0, "pieces spread evenly over the waves");
  constexpr int NP = (16 + NR / 8) / NW;
  // The loads are raw buffer loads: a piece's matrix (uniform: an 8-row piece
  // never straddles two weight matrices, whose boundaries are multiples of
  // 32 rows) is its resource, a lane's 32-bit offset its row and chunk, and
  // the chunk's k position goes in the scalar offset.
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int lr = lane >> 3, lq = lane & 7;
  const u16 *pbase[NP];
  int64_t pbytes[NP];
  uint32_t poff[NP];
  bool pon[NP];  // pieces the MFMAs read
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int p = wv + NW * i;
    const int mat = p < 16 ? (p >> 3) : 2;  // 0: A hi, 1: A lo, 2: B
    const int row = mat < 2 ? (p & 7) * 8 + lr : (p - 16) * 8 + lr;  // row of its matrix
    const int c = lq ^ ((row >> 1) & 7);
    // activation rows from MB*16 on are never read by the MFMAs (few rows:
    // the prefill LM head, small decode batches), nor is the lo plane of a
    // one-plane activation: their pieces are skipped
    pon[i] = !(mat < 2 && ((p & 7) * 8 >= MB * 16 || (mat == 1 && !a.use_lo)));
    if (mat < 2) {
      pbase[i] = a.A;
      pbytes[i] = ((int64_t)(a.use_lo ? a.a_plane : 0) + (int64_t)a.M * a.lda) * 2;
      poff[i] = (uint32_t)(((mat == 1 && a.use_lo ? a.a_plane : 0) + (int64_t)min(row, a.M - 1) * a.lda + kbeg) * 2 +
                           c * 16);
    } else {
      const int prow = (p - 16) * 8;  // the piece's first tile row
      int wr, sel, nrows;
      if (EPI == SK_SWIGLU_HILO) {
        // tile rows: [gate 0-15 | up 0-15 | gate 16-31 | up 16-31] of this block's 32 output columns
        const int F = a.N / 2;
        wr = min(nblk0 * (NR / 2) + (row >> 5) * 16 + (row & 15), F - 1);
        sel = (prow >> 4) & 1;
        nrows = F;
      } else {
        const int n = min(nblk0 * NR + row, a.N - 1);
        const int np = min(nblk0 * NR + prow, a.N - 1);
        if (a.nq > 0) {
          sel = np < a.nq ? 0 : (np < a.nq + a.nk ? 1 : 2);
          wr = n < a.nq ? n : (n < a.nq + a.nk ? n - a.nq : n - a.nq - a.nk);
          nrows = sel == 0 ? a.nq : (sel == 1 ? a.nk : a.N - a.nq - a.nk);
        } else {
          sel = 0;
          wr = n;
          nrows = a.N;
        }
      }
      // the matrix as an offset from B0 in arithmetic (a select between the
      // pointer fields would load the argument block at a computed offset)
      const int64_t d1 = a.B1 - a.B0, d2 = a.B2 - a.B0;
      pbase[i] = a.B0 + (sel == 1 ? d1 : 0) + (sel == 2 ? d2 : 0);
      pbytes[i] = (int64_t)nrows * a.K * 2;
      poff[i] = (uint32_t)(((int64_t)wr * a.K + kbeg) * 2 + c * 16);
    }
  }
  auto issue = [&](int stage, int chunk) {
    u16 *st = sm + stage * ST_ELEMS;
#pragma unroll
    for (int i = 0; i < NP; ++i)
      if (pon[i]) sk_load_lds(pbase[i], pbytes[i], st + (wv + NW * i) * 8 * SK_KCH, poff[i], (uint32_t)chunk * (SK_KCH * 2));
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
  for (int i = 0; i < NP; ++i) nper += pon[i];
  // NS stages: chunks ch+1 .. ch+NS-1 are in flight while chunk ch is computed
  auto stage = [&](int ch) {
    // after the barrier every wave's pieces of chunk ch have landed (each
    // waited for its own before it), and every wave is done reading the
    // stage refilled next
    asm volatile("s_barrier" ::: "memory");
    if (ch + NS - 1 < nchunk) issue((ch + NS - 1) % NS, ch + NS - 1);
    const u16 *st = sm + (ch % NS) * ST_ELEMS;
    // this wave's 32-k half of the stage, rows rg*RW + 16 j of B (the row
    // swizzle is the same for every 16-row block)
    const int co = ((4 * khalf + (lane >> 4)) ^ sw) * 8;
    // all fragment reads of the stage first, so their latencies overlap
    bf16x8 bb[NB], ah[MB], al[MB];
#pragma unroll
    for (int j = 0; j < NB; ++j)
      bb[j] = *reinterpret_cast<const bf16x8 *>(st + 2 * 64 * SK_KCH + (rg * RW + j * 16 + frow) * SK_KCH + co);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) ah[mb] = *reinterpret_cast<const bf16x8 *>(st + (mb * 16 + frow) * SK_KCH + co);
    if (a.use_lo) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        al[mb] = *reinterpret_cast<const bf16x8 *>(st + (64 + mb * 16 + frow) * SK_KCH + co);
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int j = 0; j < NB; ++j) acc[mb][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[mb], bb[j], acc[mb][j], 0, 0, 0);
    if (a.use_lo) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int j = 0; j < NB; ++j)
          acc[mb][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[mb], bb[j], acc[mb][j], 0, 0, 0);
    }
  };
#pragma unroll
  for (int c = 0; c < NS - 1; ++c)
    if (c < nchunk) issue(c, c);
  // Before chunk ch, this wave waits for its own loads of chunk ch (loads
  // complete in order; those of the min(NS - 2, nchunk - 1 - ch) later
  // chunks may stay in flight).  With every piece on (the batched decode) and
  // at least NS - 2 chunks, every count is a constant: NS - 2 later chunks
  // until the last NS - 2 chunks, then one fewer each.
  if (nper == NP && nchunk >= NS - 2) {
    int ch = 0;
    for (; ch + NS - 2 < nchunk; ++ch) {
      __builtin_amdgcn_s_waitcnt(0x0F70 | ((NP * (NS - 2)) & 15) | (((NP * (NS - 2)) >> 4) << 14));
      stage(ch);
    }
    static_assert(NS <= 5, "tail of at most three chunks");
    auto tail = [&](auto later) {
      constexpr int n = NP * decltype(later)::value;
      __builtin_amdgcn_s_waitcnt(0x0F70 | (n & 15) | ((n >> 4) << 14));
      stage(ch);
      ++ch;
    };
    if constexpr (NS - 3 >= 2) tail(std::integral_constant<int, 2>{});
    if constexpr (NS - 3 >= 1) tail(std::integral_constant<int, 1>{});
    if constexpr (NS - 3 >= 0) tail(std::integral_constant<int, 0>{});
  } else {
    for (int ch = 0; ch < nchunk; ++ch) {
      wait_vmcnt(nper * max(0, min(NS - 2, nchunk - 1 - ch)));
      stage(ch);
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
// compute unit, as does the LM head (1002 blocks).  The K split of a
// one-round plan is the largest that keeps the blocks within 256 and every
// slice at 256 k or more, whether or not it divides K (the QKV product's 48
// row blocks take 5 slices, 240 blocks, instead of 4).
struct Plan {
  int nr, rw, ns, ks;
};

Plan skinny_plan(int N, int K, int epi) {
  if (epi == SK_LOGITS) return {128, 16, 2, 1};
  if (epi == SK_SWIGLU_HILO) return {128, 32, 4, 1};
  const int nb = (N + 127) / 128;
  int ks = 1;
  while (nb * (ks + 1) <= 256 && K / SK_KCH / (ks + 1) >= 4) ++ks;
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
  // the loads take 32-bit byte offsets: weights and activation planes below 4 GiB
  if ((int64_t)a.N * a.K * 2 > 0xFFFFFFFFll ||
      ((int64_t)(a.use_lo ? a.a_plane : 0) + (int64_t)a.M * a.lda) * 2 > 0xFFFFFFFFll)
    return hipErrorInvalidValue;
  const Plan p = skinny_plan(a.N, a.K, epi);
  if (epi == SK_PARTIAL && a.ksplit != p.ks) return hipErrorInvalidValue;  // partial planes sized for p.ks
  const dim3 grid(skinny_nblk(a.N, a.K, epi), a.ksplit);
  if (p.nr == 128 && p.rw == 32 && p.ns == 4) return launch_nr<128, 32, 4>(epi, a, grid, s);
  if (p.nr == 128) return launch_nr<128, 16, 2>(epi, a, grid, s);
  return launch_nr<64, 16, 2>(epi, a, grid, s);
}

}  // namespace llk
