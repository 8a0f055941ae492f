// Causal grouped-query attention [P1 6.11-8; P2 3.3-3.4; P4 GQA]:
//   for query head h of KV group g = h / n_rep, at absolute position p,
//   O_h = sum_{j <= p} softmax_j(q_h . k_g[j] / sqrt(hd)) v_g[j]
// Keys are stored after RoPE; masked keys get exactly zero weight.
//
// attn_fwd_bf16   prefill, bf16 MFMA (v_mfma_f32_32x32x16_bf16), online
//                 softmax in fp32.  One block holds 128 query rows: the n_rep
//                 heads of one KV group times 128/n_rep positions, so every
//                 K/V tile staged in LDS serves the whole group.  Scores are
//                 computed transposed, S^T = K Q^T, so a lane owns one query
//                 and its softmax statistics; the output is accumulated as
//                 O^T = V^T P^T, which consumes P^T straight from the score
//                 registers (V is staged transposed in LDS).
// attn_fwd_f32    prefill for the fp32 configuration (fp32 FMA, 32 queries of
//                 one head per block, 64-key tiles in LDS).
// attn_decode     one query per sequence over the KV cache, split into key
//                 chunks (partial max / sum / output), then combined.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace llk {

namespace {
constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------------------
// Prefill, bf16, MFMA
// ---------------------------------------------------------------------------
template <int HD>
__global__ __launch_bounds__(256) void attn_fwd_bf16(AttnArgs a) {
  constexpr int KT = 64;          // keys per tile
  constexpr int KLD = HD + 8;     // K tile row stride (bf16)
  constexpr int VLD = KT + 8;     // V^T row stride (bf16)
  constexpr int NT = HD / 16;     // MFMA k-steps over head_dim
  constexpr int NO = HD / 32;     // output blocks over head_dim
  __shared__ __align__(16) u16 Ks[KT * KLD];
  __shared__ __align__(16) u16 Vt[HD * VLD];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n_rep = a.H / a.G;
  const int QB = 128 / n_rep;  // positions per block
  const int qblk = gridDim.x - 1 - blockIdx.x;  // longest blocks first
  const int g = blockIdx.y, b = blockIdx.z;

  // this lane's query row (B operand column / output column)
  const int rho = wave * 32 + (lane & 31);
  const int r_head = rho / QB;
  const int s = qblk * QB + rho % QB;
  const bool valid = s < a.S;
  const int h = g * n_rep + r_head;
  const int qp = a.start_pos + (valid ? s : a.S - 1);
  const int qlo = a.kv_lo ? min(max(a.kv_lo[(int64_t)b * a.S + (valid ? s : a.S - 1)], 0), qp) : 0;
  const int gk = lane >> 5;

  const u16 *Q = static_cast<const u16 *>(a.q);
  const u16 *qrow = Q + (int64_t)(b * a.S + (valid ? s : a.S - 1)) * a.q_stride + h * HD;
  bf16x8 qf[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) qf[t] = *reinterpret_cast<const bf16x8 *>(qrow + t * 16 + gk * 8);

  f32x16 o[NO];
#pragma unroll
  for (int i = 0; i < NO; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[i][r] = 0.f;
  float m = -INFINITY, l = 0.f;
  const float c = a.scale * kLog2e;

  const int last_s = min(a.S, (qblk + 1) * QB) - 1;
  const int kv_end = a.start_pos + last_s + 1;  // keys [0, kv_end)
  const int ntiles = (kv_end + KT - 1) / KT;
  const u16 *Kg = static_cast<const u16 *>(a.k) + ((int64_t)b * a.kcap * a.G + g) * HD;
  const u16 *Vg = static_cast<const u16 *>(a.v) + ((int64_t)b * a.kcap * a.G + g) * HD;
  const int64_t kstride = (int64_t)a.G * HD;

  for (int kt = 0; kt < ntiles; ++kt) {
    const int k0 = kt * KT;
    // stage K (row-major) and V (transposed) for keys k0 .. k0+63
    for (int cidx = tid; cidx < KT * HD / 8; cidx += 256) {
      const int key = cidx / (HD / 8), c8 = (cidx % (HD / 8)) * 8;
      uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
      if (k0 + key < kv_end) {
        kv = *reinterpret_cast<const uint4 *>(Kg + (k0 + key) * kstride + c8);
        vv = *reinterpret_cast<const uint4 *>(Vg + (k0 + key) * kstride + c8);
      }
      *reinterpret_cast<uint4 *>(Ks + key * KLD + c8) = kv;
      const u16 *ve = reinterpret_cast<const u16 *>(&vv);
#pragma unroll
      for (int e = 0; e < 8; ++e) Vt[(c8 + e) * VLD + key] = ve[e];
    }
    __syncthreads();

    // S^T = K Q^T for two 32-key blocks
    f32x16 sc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[kb][r] = 0.f;
      const u16 *kr = Ks + (kb * 32 + (lane & 31)) * KLD + gk * 8;
#pragma unroll
      for (int t = 0; t < NT; ++t)
        sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8 *>(kr + t * 16), qf[t], sc[kb],
                                                         0, 0, 0);
    }
    // mask, scale, tile max
    float tmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = k0 + kb * 32 + 8 * (r / 4) + 4 * gk + (r % 4);
        float v = sc[kb][r] * c;
        v = (key <= qp && key >= qlo) ? v : -INFINITY;
        sc[kb][r] = v;
        tmax = fmaxf(tmax, v);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave));
    const float m_new = fmaxf(m, tmax);
    // m_new stays -inf while every key so far is masked (keys before the
    // query's document); 0 stands in for it so that those weights are 0
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = exp2f(m - m_use);  // m == -inf before the first visible key: alpha = 0
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = exp2f(sc[kb][r] - m_use);
        sc[kb][r] = p;
        rs += p;
      }
    rs += __shfl_xor(rs, 32, kWave);
    l = l * alpha + rs;
    m = m_new;
#pragma unroll
    for (int i = 0; i < NO; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[i][r] *= alpha;

    // P^T fragments (bf16) for the four 16-key steps
    bf16x8 pf[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int e = 0; e < 8; ++e) pf[kb][t][e] = (__bf16)sc[kb][t * 8 + e];

    // O^T += V^T P^T
#pragma unroll
    for (int ob = 0; ob < NO; ++ob) {
      const u16 *vr = Vt + (ob * 32 + (lane & 31)) * VLD + 4 * gk;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int kofs = kb * 32 + t * 16;
          uint4 av;
          const uint2 lo = *reinterpret_cast<const uint2 *>(vr + kofs);
          const uint2 hi = *reinterpret_cast<const uint2 *>(vr + kofs + 8);
          av.x = lo.x; av.y = lo.y; av.z = hi.x; av.w = hi.y;
          o[ob] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<bf16x8 *>(&av), pf[kb][t], o[ob], 0, 0, 0);
        }
    }
    __syncthreads();
  }

  if (valid) {
    const float inv = 1.0f / l;
    u16 *orow = static_cast<u16 *>(a.o) + (int64_t)(b * a.S + s) * a.q_stride + h * HD;
#pragma unroll
    for (int ob = 0; ob < NO; ++ob)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d = ob * 32 + 8 * q4 + 4 * gk;
        uint2 pk;
        pk.x = (uint32_t)f2bf(o[ob][q4 * 4 + 0] * inv) | ((uint32_t)f2bf(o[ob][q4 * 4 + 1] * inv) << 16);
        pk.y = (uint32_t)f2bf(o[ob][q4 * 4 + 2] * inv) | ((uint32_t)f2bf(o[ob][q4 * 4 + 3] * inv) << 16);
        *reinterpret_cast<uint2 *>(orow + d) = pk;
      }
  }
}

// ---------------------------------------------------------------------------
// Prefill, bf16, head_dim 128: K/V tiles double-buffered through LDS
//
// A block covers 256 query rows of one KV group g: the group's n_rep heads
// times 256/n_rep positions, so each K/V tile in LDS serves every head of
// the group [P2 3.4 repeat_kv; P1 8].  Each of the eight waves owns 32 query
// rows with its Q fragments in registers.  Per 64-key tile:
//   S^T = K Q^T      v_mfma_f32_32x32x16_bf16; A = K rows from LDS, B = Q
//                    fragments kept in registers.  Lane l holds the scores of
//                    query l%32 for keys 8*(r/4) + 4*(l/32) + r%4.
//   online softmax   in fp32, log2 units, per query in its own lane.
//   O^T += V^T P^T   A = V^T read from row-major V with ds_read_b64_tr_b16,
//                    B = P^T taken from the score registers as bf16.
// Two waves share each SIMD, so one wave's softmax (vector ALU, exp) runs
// while the other's MFMAs do, and each fills the other's gaps between
// dependent MFMAs (S^T has only two accumulator blocks per wave).
// K and V arrive with global_load_lds_dwordx4 (no VGPR round trip) while the
// previous tile is being computed.  Rows are 256 bytes; K and Q keep 16-byte
// chunk c of row r at c ^ (r & 15), so the 32 rows a fragment read touches
// fall in distinct banks; V uses the swizzle its transposed reads need.
// Block order: consecutive block ids cycle through the KV groups, so the
// blocks one XCD receives (ids congruent mod 8) share a group's K/V in L2;
// within a group the longest causal ranges start first.
// ---------------------------------------------------------------------------
// DOC: queries also have a lowest visible key (document mask); the block
// starts at the tile of its lowest bound and each wave classifies tiles by
// its own bounds.
template <bool DOC>
__global__ __launch_bounds__(512) void attn_fwd_w8(AttnArgs a) {
  constexpr int HD = 128;
  constexpr int KT = 64;            // keys per tile
  constexpr int TILE = KT * HD;     // elements per K or V tile
  constexpr int NT = HD / 16;       // S^T k-steps over head_dim
  constexpr int NO = HD / 32;       // O^T row blocks over head_dim
  // one LDS object per stage: the compiler can then tell the stage being
  // read from the one being filled and keeps the prefetch in flight
  __shared__ __align__(16) u16 Ks0[TILE], Ks1[TILE];
  __shared__ __align__(16) u16 Vs0[TILE], Vs1[TILE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;  // 8 waves
  const int n_rep = a.H / a.G;
  const int QB = 256 / n_rep;  // positions per block
  const int nq = (a.S + QB - 1) / QB;
  const int L = blockIdx.x;
  const int g = L % a.G;
  const int rest = L / a.G;
  const int b = rest % a.B;
  const int qblk = nq - 1 - rest / a.B;

  const int hf = lane >> 5;  // half of the wave
  const int rho = wave * 32 + (lane & 31);
  const int hq = g * n_rep + rho / QB;
  const int sq = qblk * QB + rho % QB;
  const bool valid = sq < a.S;
  const int srow = valid ? sq : a.S - 1;
  const int qpos = a.start_pos + srow;
  const int wmax = (int)wave_max((float)qpos);
  const int wmin = -(int)wave_max((float)-qpos);
  int qlo = 0, wlo_min = 0, wlo_max = 0, kt_first = 0;
  if (DOC) {
    __shared__ int blo[8];
    qlo = min(max(a.kv_lo[(int64_t)b * a.S + srow], 0), qpos);
    wlo_max = (int)wave_max((float)qlo);
    wlo_min = -(int)wave_max((float)-qlo);
    if (lane == 0) blo[wave] = wlo_min;
    __syncthreads();
    int mn = blo[0];
#pragma unroll
    for (int w = 1; w < 8; ++w) mn = min(mn, blo[w]);
    kt_first = mn / 64;
  }

  // Q fragments (B operand of S^T = K Q^T): row rho, head-dim 16t + 8*hf .. +7
  bf16x8 qf[NT];
  {
    const u16 *qrow = static_cast<const u16 *>(a.q) + (int64_t)(b * a.S + srow) * a.q_stride + hq * HD + 8 * hf;
#pragma unroll
    for (int t = 0; t < NT; ++t) qf[t] = *reinterpret_cast<const bf16x8 *>(qrow + 16 * t);
  }

  const int last_s = min(a.S, (qblk + 1) * QB) - 1;
  const int kv_end = a.start_pos + last_s + 1;  // keys [0, kv_end)
  const int ntiles = (kv_end + KT - 1) / KT;
  const int64_t kstride = (int64_t)a.G * HD;
  const u16 *Kg = static_cast<const u16 *>(a.k) + ((int64_t)b * a.kcap * a.G + g) * HD;
  const u16 *Vg = static_cast<const u16 *>(a.v) + ((int64_t)b * a.kcap * a.G + g) * HD;

  // loader: piece p = wave + 8i (i < 2) covers tile rows 4p .. 4p+3; lane L
  // -> row 4p + L/16, physical chunk L%16.  K keeps logical chunk
  // (L%16) ^ (row & 15) there, V (L%16) ^ vswz(row), vswz(r) =
  // ((r & 3) << 2) | ((r >> 2) & 3), matched to its transposed reads.
  int lrow[2], lcol[2], lcolv[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int p = wave + 8 * i;
    lrow[i] = 4 * p + (lane >> 4);
    lcol[i] = ((lane & 15) ^ (lrow[i] & 15)) * 8;
    lcolv[i] = ((lane & 15) ^ (((lrow[i] & 3) << 2) | ((lrow[i] >> 2) & 3))) * 8;
  }
  auto issue = [&](int kt, auto buf_c) {
    constexpr int BUF = decltype(buf_c)::value;
    u16 *kd = BUF ? Ks1 : Ks0;
    u16 *vd = BUF ? Vs1 : Vs0;
    const int k0 = kt * KT;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int key = min(k0 + lrow[i], kv_end - 1);  // rows past the end are masked
      const int p = __builtin_amdgcn_readfirstlane(wave + 8 * i);
      __builtin_amdgcn_global_load_lds((const void *)(Kg + (int64_t)key * kstride + lcol[i]),
                                       (__attribute__((address_space(3))) void *)(kd + p * 4 * HD), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void *)(Vg + (int64_t)key * kstride + lcolv[i]),
                                       (__attribute__((address_space(3))) void *)(vd + p * 4 * HD), 16, 0, 0);
    }
  };

  f32x16 o[NO];
#pragma unroll
  for (int i = 0; i < NO; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[i][r] = 0.f;
  float m = -INFINITY, l = 0.f;
  const float c = a.scale * kLog2e;

  // V^T fragments (tr16 reads): 16-lane group G reads rows 4*hf + j/4 (+8)
  // of a 16-key step at columns 32*ob + 16*(G&1) + 4*(j&3); lane j then
  // holds V[4 keys][d], d = 32*ob + lane%32
  const int jj = lane & 15, dg = (lane >> 4) & 1;
  const int vr0 = 4 * hf + (jj >> 2);
  const int vq = 2 * dg + ((jj & 3) >> 1), vhalf = (jj & 1) * 4;
  // per-lane LDS element offsets, the same for both stages.  K: row lane%32,
  // chunk (2t + hf) ^ (lane & 15) of head-dim step t (+32 rows for the second
  // key block).  V^T: rows vr0 + 8*h2 (+16 per key step; the swizzle depends
  // only on the row modulo 16) at output columns 32*ob + ...
  int kofs[NT], vofs[NO][2];
#pragma unroll
  for (int t = 0; t < NT; ++t) kofs[t] = (lane & 31) * HD + (((2 * t + hf) ^ (lane & 15)) * 8);
#pragma unroll
  for (int ob = 0; ob < NO; ++ob)
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const int r = vr0 + 8 * h2;
      const int vsw = ((r & 3) << 2) | ((r >> 2) & 3);
      vofs[ob][h2] = r * HD + (((4 * ob + vq) ^ vsw) * 8) + vhalf;
    }

  auto tile = [&](int kt, auto mask_c, auto buf_c) {
    constexpr bool MASK = decltype(mask_c)::value;
    constexpr int BUF = decltype(buf_c)::value;
    const int k0 = kt * KT;
    // z is 0, opaque to the compiler: addresses are formed here from the
    // shared offsets instead of being kept per stage across the loop
    int z = 0;
    asm volatile("" : "+v"(z));
    const u16 *ks = (BUF ? Ks1 : Ks0) + z;
    const u16 *vs = (BUF ? Vs1 : Vs0) + z;
    // S^T = K Q^T: two 32-key blocks; K rows kb*32 + lane%32
    f32x16 sc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[kb][r] = 0.f;
    bf16x8 kf[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) kf[0][kb] = *reinterpret_cast<const bf16x8 *>(ks + kofs[0] + kb * 32 * HD);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int cb = t & 1;
      if (t + 1 < NT) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          kf[cb ^ 1][kb] = *reinterpret_cast<const bf16x8 *>(ks + kofs[t + 1] + kb * 32 * HD);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[cb][kb], qf[t], sc[kb], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    typedef short v4s __attribute__((ext_vector_type(4)));
    typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
    // V^T fragments of the first 16-key step, read before the softmax so the
    // first P.V products need not wait for them (non-document kernel)
    u32x2 wv0[NO][2];
    if constexpr (!DOC) {
#pragma unroll
      for (int ob = 0; ob < NO; ++ob)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const v4s w = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) v4s *)(const __attribute__((address_space(3))) u16 *)(vs + vofs[ob][h2]));
          wv0[ob][h2] = __builtin_bit_cast(u32x2, w);
        }
      __builtin_amdgcn_sched_barrier(0);
    }
    // online softmax of this lane's query, log2 units, lazy rescale (the
    // running maximum moves only when a tile exceeds it by more than 8)
    if (MASK) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
          if (key > qpos || (DOC && key < qlo)) sc[kb][r] = -INFINITY;
        }
    }
    float rs = 0.f;
    float pw[2][16];
    auto weights = [&]() {
      rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float p = __builtin_amdgcn_exp2f(fmaf(sc[kb][r], c, -m));
          // a lane with no visible key yet has m = -inf: its masked scores weigh 0
          if (DOC && MASK && sc[kb][r] == -INFINITY) p = 0.f;
          pw[kb][r] = p;
          rs += p;
        }
    };
    bool need_max = true;
    if constexpr (!DOC) {
      // Weights against the running maximum first.  While every lane's
      // partial row sum stays below 2^7, no weight reaches 2^7, so no score
      // exceeds the running maximum by 7 and the rescale test below could
      // not fire: these are the weights the maximum-first order gives.  A
      // larger sum, inf or NaN (the first tile, where m is still -inf, gives
      // those) sends the wave through the maximum-first order.
      weights();
      need_max = __builtin_amdgcn_ballot_w64(!(rs < 128.f)) != 0;
    }
    if (need_max) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[kb][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, kWave)) * c;
      if (__builtin_amdgcn_ballot_w64(mx > m + 8.f) != 0) {
        // finite where the lane has a visible key so far (always without
        // documents: key 0 is visible to every query)
        const float m_new = fmaxf(m, mx);
        float alpha = __builtin_amdgcn_exp2f(m - m_new);
        // a lane still without a visible key keeps m = -inf (and l = o = 0)
        if (DOC && m_new == -INFINITY) alpha = 1.f;
        l *= alpha;
        m = m_new;
#pragma unroll
        for (int i = 0; i < NO; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[i][r] *= alpha;
      }
      weights();
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[kb][r] = pw[kb][r];
    l += rs + __shfl_xor(rs, 32, kWave);
    // O^T += V^T P^T over four 16-key steps
#pragma unroll
    for (int ksp = 0; ksp < 4; ++ksp) {
      const int kb = ksp >> 1, t = ksp & 1;
      bf16x8 pf;
#pragma unroll
      for (int e = 0; e < 8; ++e) pf[e] = (__bf16)sc[kb][8 * t + e];
#pragma unroll
      for (int ob = 0; ob < NO; ++ob) {
        u32x2 wv[2];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          if (!DOC && ksp == 0) {
            wv[h2] = wv0[ob][h2];
            continue;
          }
          const u16 *src = vs + vofs[ob][h2] + 16 * ksp * HD;
          const v4s w = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) v4s *)(const __attribute__((address_space(3))) u16 *)src);
          wv[h2] = __builtin_bit_cast(u32x2, w);
        }
        const bf16x8 vf = __builtin_bit_cast(bf16x8, make_uint4(wv[0].x, wv[0].y, wv[1].x, wv[1].y));
        o[ob] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, o[ob], 0, 0, 0);
      }
    }
  };

  // tiles [0, nfull) are visible to every query of this wave; the rest are
  // masked, and tiles past the wave's last query are skipped.  Every wave
  // passes the same ntiles barriers.
  const int nfull = min(ntiles, (wmin + 1) / KT);
  using Plain = std::integral_constant<bool, false>;
  using Masked = std::integral_constant<bool, true>;
  auto step = [&](int kt, auto buf_c) {
    constexpr int BUF = decltype(buf_c)::value;
    // the only loads in flight are this wave's pieces of tile kt: wait for
    // them, then the barrier makes the whole tile visible (and every wave is
    // done with tile kt-1, whose stage the prefetch below overwrites).  A
    // wave that skips tiles must still wait here for its pieces.
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    if (kt + 1 < ntiles) issue(kt + 1, std::integral_constant<int, 1 - BUF>());
    const int k0 = kt * KT;
    if (DOC) {
      // skip tiles wholly below the wave's lowest bound or past its last query
      if (k0 + KT - 1 < wlo_min || k0 > wmax) return;
      if (k0 >= wlo_max && kt < nfull)
        tile(kt, Plain(), buf_c);
      else
        tile(kt, Masked(), buf_c);
    } else if (kt < nfull) {
      tile(kt, Plain(), buf_c);
    } else if (k0 <= wmax) {
      tile(kt, Masked(), buf_c);
    }
  };
  // tile kt lives in stage kt & 1; the loop runs two tiles per pass so that
  // both stages are compile-time constants
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  int kt = kt_first;
  if (kt & 1) {
    issue(kt, S1());
    step(kt, S1());
    ++kt;
  } else {
    issue(kt, S0());
  }
  for (; kt < ntiles; kt += 2) {
    step(kt, S0());
    if (kt + 1 < ntiles) step(kt + 1, S1());
  }

  // lane holds O^T[d = 32*ob + 8*(r/4) + 4*hf + r%4][query lane%32]
  if (valid) {
    const float inv = 1.0f / l;
    u16 *orow = static_cast<u16 *>(a.o) + (int64_t)(b * a.S + srow) * a.q_stride + hq * HD;
#pragma unroll
    for (int ob = 0; ob < NO; ++ob)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d = ob * 32 + 8 * q4 + 4 * hf;
        uint2 pk;
        pk.x = (uint32_t)f2bf(o[ob][q4 * 4 + 0] * inv) | ((uint32_t)f2bf(o[ob][q4 * 4 + 1] * inv) << 16);
        pk.y = (uint32_t)f2bf(o[ob][q4 * 4 + 2] * inv) | ((uint32_t)f2bf(o[ob][q4 * 4 + 3] * inv) << 16);
        *reinterpret_cast<uint2 *>(orow + d) = pk;
      }
  }
}

// ---------------------------------------------------------------------------
// Prefill, fp32 (one wave per block, one query per lane)
// ---------------------------------------------------------------------------
template <int HD>
__global__ __launch_bounds__(256) void attn_fwd_f32(AttnArgs a) {
  // A block owns 32 query positions of one head; 64-key tiles of K and V go
  // through LDS.  Thread (tr, tc) = (t / 16, t % 16) scores rows 2tr, 2tr+1
  // against keys tc + 16j (j < 4) and accumulates output columns tc + 16c.
  // Row statistics (max, sum) are reduced over the 16 lanes of a row group.
  constexpr int QT = 32, KT = 64, NC = HD / 16;
  __shared__ float Qs[QT][HD + 1];
  __shared__ float Ks[KT][HD + 1];
  __shared__ __align__(16) float Vs[KT][HD];
  __shared__ float Ps[QT][KT + 1];
  const int tid = threadIdx.x, tr = tid >> 4, tc = tid & 15;
  const int qblk = gridDim.x - 1 - blockIdx.x;  // longest causal ranges first
  const int h = blockIdx.y, b = blockIdx.z;
  const int g = h / (a.H / a.G);
  const float *Q = static_cast<const float *>(a.q);
  for (int i = tid; i < QT * HD; i += 256) {
    const int r = i / HD, d = i % HD;
    const int s = min(qblk * QT + r, a.S - 1);
    Qs[r][d] = Q[(int64_t)(b * a.S + s) * a.q_stride + h * HD + d];
  }
  int qp[2], qlo[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int s = min(qblk * QT + 2 * tr + i, a.S - 1);
    qp[i] = a.start_pos + s;
    qlo[i] = a.kv_lo ? min(max(a.kv_lo[(int64_t)b * a.S + s], 0), qp[i]) : 0;
  }
  float o[2][NC], m[2], l[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    m[i] = -INFINITY;
    l[i] = 0.f;
#pragma unroll
    for (int c = 0; c < NC; ++c) o[i][c] = 0.f;
  }
  const int kv_end = a.start_pos + min(a.S, (qblk + 1) * QT);  // keys [0, kv_end)
  const float *Kg = static_cast<const float *>(a.k) + ((int64_t)b * a.kcap * a.G + g) * HD;
  const float *Vg = static_cast<const float *>(a.v) + ((int64_t)b * a.kcap * a.G + g) * HD;
  const int64_t kstride = (int64_t)a.G * HD;
  for (int k0 = 0; k0 < kv_end; k0 += KT) {
    __syncthreads();  // the previous tile's K, V and P are no longer read
    for (int i = tid; i < KT * HD / 4; i += 256) {
      const int key = i / (HD / 4), d = (i % (HD / 4)) * 4;
      const int kk = min(k0 + key, kv_end - 1);  // rows past the end are masked
      const float4 kv = *reinterpret_cast<const float4 *>(Kg + (int64_t)kk * kstride + d);
      const float4 vv = *reinterpret_cast<const float4 *>(Vg + (int64_t)kk * kstride + d);
      Ks[key][d] = kv.x; Ks[key][d + 1] = kv.y; Ks[key][d + 2] = kv.z; Ks[key][d + 3] = kv.w;
      *reinterpret_cast<float4 *>(&Vs[key][d]) = vv;
    }
    __syncthreads();
    float sc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) sc[i][j] = 0.f;
#pragma unroll 8
    for (int d = 0; d < HD; ++d) {
      const float q0 = Qs[2 * tr][d], q1 = Qs[2 * tr + 1][d];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float kv = Ks[tc + 16 * j][d];
        sc[0][j] = fmaf(q0, kv, sc[0][j]);
        sc[1][j] = fmaf(q1, kv, sc[1][j]);
      }
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      float tmax = -INFINITY;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int key = k0 + tc + 16 * j;
        const bool vis = key <= qp[i] && key >= qlo[i] && key < kv_end;
        sc[i][j] = vis ? sc[i][j] * a.scale : -INFINITY;
        tmax = fmaxf(tmax, sc[i][j]);
      }
#pragma unroll
      for (int x = 8; x >= 1; x >>= 1) tmax = fmaxf(tmax, __shfl_xor(tmax, x, kWave));
      const float m_new = fmaxf(m[i], tmax);
      // m_new stays -inf while every key so far is masked; 0 stands in for it
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = expf(m[i] - m_use);
      float rs = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float p = expf(sc[i][j] - m_use);
        Ps[2 * tr + i][tc + 16 * j] = p;
        rs += p;
      }
#pragma unroll
      for (int x = 8; x >= 1; x >>= 1) rs += __shfl_xor(rs, x, kWave);
      l[i] = l[i] * alpha + rs;
      m[i] = m_new;
#pragma unroll
      for (int c = 0; c < NC; ++c) o[i][c] *= alpha;
    }
    __syncthreads();
#pragma unroll 4
    for (int k = 0; k < KT; ++k) {
      const float p0 = Ps[2 * tr][k], p1 = Ps[2 * tr + 1][k];
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const float v = Vs[k][tc + 16 * c];
        o[0][c] = fmaf(p0, v, o[0][c]);
        o[1][c] = fmaf(p1, v, o[1][c]);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int s = qblk * QT + 2 * tr + i;
    if (s >= a.S) continue;
    float *orow = static_cast<float *>(a.o) + (int64_t)(b * a.S + s) * a.q_stride + h * HD;
    const float inv = 1.0f / l[i];
#pragma unroll
    for (int c = 0; c < NC; ++c) orow[tc + 16 * c] = o[i][c] * inv;
  }
}

// ---------------------------------------------------------------------------
// Decode: one query per sequence, split over key chunks
// ---------------------------------------------------------------------------
template <typename TC, int HD>
__global__ __launch_bounds__(256) void attn_decode_kernel(DecodeAttnArgs a) {
  constexpr int MAXREP = 16;
  constexpr int CH = 256;  // keys per chunk (a.chunk == CH)
  __shared__ float qs[MAXREP][HD];
  __shared__ float sc[MAXREP][CH];
  __shared__ float ml[MAXREP][2];
  const int tid = threadIdx.x;
  const int ci = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int n_rep = a.H / a.G;
  int pb = a.pos[b];
  pb = pb < 0 ? 0 : (pb > a.cap - 1 ? a.cap - 1 : pb);
  const int kstart = a.kv_lo ? min(max(a.kv_lo[b], 0), pb) : 0;  // lowest visible key (document)
  const int c0 = max(ci * CH, kstart);
  const int kend = min(ci * CH + CH, a.knew ? pb : pb + 1);  // own position added by the combine when knew is set
  const int64_t pidx = ((int64_t)b * a.H + g * n_rep) * a.nchunk + ci;  // + r * nchunk per head
  if (c0 >= kend) {
    for (int i = tid; i < n_rep * HD; i += 256) {
      const int r = i / HD, d = i % HD;
      a.po[(pidx + (int64_t)r * a.nchunk) * HD + d] = 0.f;
    }
    if (tid < n_rep) {
      a.pm[pidx + (int64_t)tid * a.nchunk] = -INFINITY;
      a.pl[pidx + (int64_t)tid * a.nchunk] = 0.f;
    }
    return;
  }
  const int nk = kend - c0;
  for (int i = tid; i < n_rep * HD; i += 256) {
    const int r = i / HD, d = i % HD;
    qs[r][d] = a.q[((int64_t)b * a.H + g * n_rep + r) * HD + d];
  }
  __syncthreads();
  const TC *Kg = static_cast<const TC *>(a.k) + ((int64_t)b * a.cap * a.G + g) * HD;
  const TC *Vg = static_cast<const TC *>(a.v) + ((int64_t)b * a.cap * a.G + g) * HD;
  const int64_t kstride = (int64_t)a.G * HD;
  if (tid < nk) {
    const TC *kr = Kg + (int64_t)(c0 + tid) * kstride;
    float dot[MAXREP];
    for (int r = 0; r < n_rep; ++r) dot[r] = 0.f;
    for (int d = 0; d < HD; ++d) {
      const float kv = Elem<TC>::load(kr + d);
      for (int r = 0; r < n_rep; ++r) dot[r] = fmaf(qs[r][d], kv, dot[r]);
    }
    for (int r = 0; r < n_rep; ++r) sc[r][tid] = dot[r] * a.scale * kLog2e;
  }
  __syncthreads();
  const int wave = tid >> 6, lane = tid & 63;
  for (int r = wave; r < n_rep; r += 4) {
    float mx = -INFINITY;
    for (int j = lane; j < nk; j += 64) mx = fmaxf(mx, sc[r][j]);
    mx = wave_max(mx);
    float sum = 0.f;
    for (int j = lane; j < nk; j += 64) {
      const float p = exp2f(sc[r][j] - mx);
      sc[r][j] = p;
      sum += p;
    }
    sum = wave_sum(sum);
    if (lane == 0) { ml[r][0] = mx; ml[r][1] = sum; }
  }
  __syncthreads();
  for (int i = tid; i < n_rep * HD; i += 256) {
    const int r = i / HD, d = i % HD;
    float acc = 0.f;
    for (int j = 0; j < nk; ++j) acc = fmaf(sc[r][j], Elem<TC>::load(Vg + (int64_t)(c0 + j) * kstride + d), acc);
    a.po[(pidx + (int64_t)r * a.nchunk) * HD + d] = acc;
  }
  if (tid < n_rep) {
    a.pm[pidx + (int64_t)tid * a.nchunk] = ml[tid][0];
    a.pl[pidx + (int64_t)tid * a.nchunk] = ml[tid][1];
  }
}

// ---------------------------------------------------------------------------
// Decode, bf16 cache, MFMA for the scores.  A block takes 256 keys of one
// (sequence, KV group); each wave takes 64 of them.
//   S^T = K Q^T on v_mfma_f32_16x16x32_bf16: the K rows are the A operand,
//   read straight from the cache (16 keys x 64 contiguous bytes per load);
//   the group's n_rep query heads are the B columns, each fp32 query split
//   into hi + lo bf16 (two MFMAs) so the scores keep ~16 significant bits.
//   P V runs on the vector ALUs in fp32: lane (kq, dc) streams 16-byte
//   pieces of the V rows of keys 4i + kq, reads the probabilities of that
//   key from LDS and accumulates 8 output columns for every head.
// The four waves are merged through LDS into one (max, sum, output) partial
// per head and key chunk; maxima are in log2 units.
// ---------------------------------------------------------------------------
template <int HD, int NR>
__global__ __launch_bounds__(256) void attn_decode_mfma(DecodeAttnArgs a) {
  constexpr int CH = 256;
  constexpr int KW = 64;
  constexpr int NS = HD / 32;
  constexpr int NDC = HD / 8;
  __shared__ __align__(16) float Ps[4][KW][NR];
  __shared__ float red_m[4][NR], red_l[4][NR];
  __shared__ __align__(16) float red_o[4][NR][HD];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ci = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int n_rep = a.H / a.G;
  int pb = a.pos[b];
  pb = pb < 0 ? 0 : (pb > a.cap - 1 ? a.cap - 1 : pb);
  const int c0 = ci * CH;
  const int kend = min(c0 + CH, a.knew ? pb : pb + 1);  // own position added by the combine when knew is set
  const int kstart = a.kv_lo ? min(max(a.kv_lo[b], 0), pb) : 0;  // lowest visible key (document)
  const int64_t pidx = ((int64_t)b * a.H + g * n_rep) * a.nchunk + ci;
  if (c0 >= kend || c0 + CH <= kstart) {
    for (int i = tid; i < n_rep * HD; i += 256) a.po[(pidx + (int64_t)(i / HD) * a.nchunk) * HD + i % HD] = 0.f;
    if (tid < n_rep) {
      a.pm[pidx + (int64_t)tid * a.nchunk] = -INFINITY;
      a.pl[pidx + (int64_t)tid * a.nchunk] = 0.f;
    }
    return;
  }
  const int j = lane & 15, grp = lane >> 4;
  const int64_t kstride = (int64_t)a.G * HD;
  const u16 *Kb = static_cast<const u16 *>(a.k) + ((int64_t)b * a.cap * a.G + g) * HD;
  const u16 *Vb = static_cast<const u16 *>(a.v) + ((int64_t)b * a.cap * a.G + g) * HD;
  const int kw0 = c0 + wave * KW;

  // issue every load of this wave first: K fragments and V pieces.  Keys past
  // the end read the last visible row (their scores are masked, their
  // weights are 0) and lanes past the head dimension read its last piece
  // (never stored), so no load waits on a select of its data.
  const int kmax = kend - 1;
  uint4 kf[4][NS];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const u16 *src = Kb + (int64_t)min(kw0 + kb * 16 + j, kmax) * kstride + grp * 8;
#pragma unroll
    for (int t = 0; t < NS; ++t) kf[kb][t] = *reinterpret_cast<const uint4 *>(src + t * 32);
  }
  uint4 vf[16];
  const int jc = min(j, NDC - 1);
#pragma unroll
  for (int i = 0; i < 16; ++i)
    vf[i] = *reinterpret_cast<const uint4 *>(Vb + (int64_t)min(kw0 + i * 4 + grp, kmax) * kstride + jc * 8);

  // query fragments (B operand): column j = head of the group, k = head_dim
  const float c = a.scale * kLog2e;
  bf16x8 qh[NS], ql[NS];
  // every lane loads (columns past the group's heads from head 0) and zeroes
  // afterwards, so the loads are issued together rather than one per branch
  float4 qv[NS][2];
  {
    const float *qrow = a.q + ((int64_t)b * a.H + g * n_rep + (j < n_rep ? j : 0)) * HD + grp * 8;
#pragma unroll
    for (int t = 0; t < NS; ++t) {
      qv[t][0] = *reinterpret_cast<const float4 *>(qrow + t * 32);
      qv[t][1] = *reinterpret_cast<const float4 *>(qrow + t * 32 + 4);
    }
  }
#pragma unroll
  for (int t = 0; t < NS; ++t) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float4 q4 = qv[t][e >> 2];
      const float qe = (e & 3) == 0 ? q4.x : (e & 3) == 1 ? q4.y : (e & 3) == 2 ? q4.z : q4.w;
      const float v = j < n_rep ? qe * c : 0.f;
      u16 hi, lo;
      split_hilo(v, hi, lo);
      qh[t][e] = __builtin_bit_cast(__bf16, hi);
      ql[t][e] = __builtin_bit_cast(__bf16, lo);
    }
  }

  // scores (log2 units), masked beyond the sequence's position
  f32x4 sc[4];
  float mx = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    sc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < NS; ++t) {
      const bf16x8 kv = __builtin_bit_cast(bf16x8, kf[kb][t]);
      sc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, qh[t], sc[kb], 0, 0, 0);
      sc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, ql[t], sc[kb], 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = kw0 + kb * 16 + 4 * grp + r;
      if (key >= kend || key < kstart) sc[kb][r] = -INFINITY;
      mx = fmaxf(mx, sc[kb][r]);
    }
  }
  mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
  mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
  float ls = 0.f;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float p = mx == -INFINITY ? 0.f : exp2f(sc[kb][r] - mx);
      ls += p;
      if (j < NR) Ps[wave][kb * 16 + 4 * grp + r][j] = p;
    }
  ls += __shfl_xor(ls, 16, kWave);
  ls += __shfl_xor(ls, 32, kWave);
  if (grp == 0 && j < NR) {
    red_m[wave][j] = mx;
    red_l[wave][j] = ls;
  }
  __syncthreads();

  // P V in fp32: lane (grp, j) handles keys 4i + grp and columns 8j .. 8j+7
  float acc[NR][8];
#pragma unroll
  for (int h = 0; h < NR; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int kl = i * 4 + grp;
    float v[8];
    const u16 *vp = reinterpret_cast<const u16 *>(&vf[i]);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = bf2f(vp[e]);
#pragma unroll
    for (int h4 = 0; h4 < NR; h4 += 4) {
      const float4 p4 = *reinterpret_cast<const float4 *>(&Ps[wave][kl][h4]);
      const float pp[4] = {p4.x, p4.y, p4.z, p4.w};
#pragma unroll
      for (int hh = 0; hh < 4; ++hh)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h4 + hh][e] = fmaf(pp[hh], v[e], acc[h4 + hh][e]);
    }
  }
#pragma unroll
  for (int h = 0; h < NR; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float t = acc[h][e];
      t += __shfl_xor(t, 16, kWave);
      t += __shfl_xor(t, 32, kWave);
      acc[h][e] = t;
    }
  if (grp == 0 && j < NDC) {
#pragma unroll
    for (int h = 0; h < NR; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) red_o[wave][h][j * 8 + e] = acc[h][e];
  }
  __syncthreads();

  // merge the four waves into this chunk's partial
  for (int i = tid; i < n_rep * HD; i += 256) {
    const int h = i / HD, d = i % HD;
    float M = red_m[0][h];
#pragma unroll
    for (int w = 1; w < 4; ++w) M = fmaxf(M, red_m[w][h]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float wt = red_m[w][h] == -INFINITY ? 0.f : exp2f(red_m[w][h] - M);
      L += wt * red_l[w][h];
      O += wt * red_o[w][h][d];
    }
    a.po[(pidx + (int64_t)h * a.nchunk) * HD + d] = O;
    if (d == 0) {
      a.pm[pidx + (int64_t)h * a.nchunk] = M;
      a.pl[pidx + (int64_t)h * a.nchunk] = L;
    }
  }
}

// ---------------------------------------------------------------------------
// Decode, bf16 cache, head_dim 128: scores and P V both on MFMA
// (v_mfma_f32_16x16x32_bf16).  A block takes 256 keys of one (sequence, KV
// group), each wave 64 of them.
//   * K rows are loaded straight into registers as the A operand of
//     S^T = K Q^T (16 keys x 64 contiguous bytes per load); the query heads
//     of the group are the B columns, pre-split into hi + lo bf16 and
//     pre-scaled by log2(e)/sqrt(hd) by the RoPE kernel.
//   * V rows go HBM -> LDS with global_load_lds_dwordx4 (1 KB = 4 rows per
//     wave instruction, 16-byte chunk c of row r stored at chunk c ^ (r & 15)).
//   * P stays in registers: the score accumulator layout (lane = head column,
//     four keys per register group) is already the A-operand layout of
//     O = P V.  P is split into hi + lo bf16 (two MFMAs against the same V
//     fragment, ~16 significant bits) and V's B operand is read with
//     ds_read_b64_tr_b16, which hands lane i of each 16-lane group column i
//     of the four 32-byte row pieces its group addresses.
// The four waves merge into one (max, sum, output) partial per head and key
// chunk; maxima are in log2 units.
// ---------------------------------------------------------------------------
template <int NR>
__global__ __launch_bounds__(256) void attn_decode_mfma2(DecodeAttnArgs a) {
  constexpr int HD = 128;
  constexpr int CH = 256;
  constexpr int KW = 64;
  constexpr int NS = HD / 32;  // score k-steps
  constexpr int NB = HD / 16;  // output column blocks
  __shared__ __align__(16) u16 Vs[4][KW * HD];  // 16 KB per wave
  __shared__ float red_m[4][NR], red_l[4][NR];
  __shared__ __align__(16) float red_o[4][NR][HD];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ci = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int n_rep = a.H / a.G;
  int pb = a.pos[b];
  pb = pb < 0 ? 0 : (pb > a.cap - 1 ? a.cap - 1 : pb);
  const int c0 = ci * CH;
  const int kend = min(c0 + CH, a.knew ? pb : pb + 1);  // own position added by the combine when knew is set
  const int kstart = a.kv_lo ? min(max(a.kv_lo[b], 0), pb) : 0;  // lowest visible key (document)
  const int64_t pidx = ((int64_t)b * a.H + g * n_rep) * a.nchunk + ci;
  if (c0 >= kend || c0 + CH <= kstart) {
    for (int i = tid; i < n_rep * HD; i += 256) a.po[(pidx + (int64_t)(i / HD) * a.nchunk) * HD + i % HD] = 0.f;
    if (tid < n_rep) {
      a.pm[pidx + (int64_t)tid * a.nchunk] = -INFINITY;
      a.pl[pidx + (int64_t)tid * a.nchunk] = 0.f;
    }
    return;
  }
  const int j = lane & 15, grp = lane >> 4;
  const int64_t kstride = (int64_t)a.G * HD;
  const u16 *Kb = static_cast<const u16 *>(a.k) + ((int64_t)b * a.cap * a.G + g) * HD;
  const u16 *Vb = static_cast<const u16 *>(a.v) + ((int64_t)b * a.cap * a.G + g) * HD;
  const int kw0 = c0 + wave * KW;
  const int kmax = kend - 1;  // keys past the end read a valid row; their scores are masked

  // query fragments (B operand): column j = head of the group
  bf16x8 qh[NS], ql[NS];
  {
    const int hq = j < n_rep ? j : 0;
    const int64_t qo = ((int64_t)b * a.H + g * n_rep + hq) * HD + grp * 8;
    const int64_t plane = (int64_t)a.B * a.H * HD;
#pragma unroll
    for (int t = 0; t < NS; ++t) {
      qh[t] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(a.qhl + qo + t * 32));
      ql[t] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(a.qhl + plane + qo + t * 32));
    }
  }

  // K fragments (A operand): key kw0 + 16kb + j, head_dim slice 32t + 8grp;
  // raw buffer loads over the sequence's rows of the group (32-bit offsets:
  // the cache block of one sequence is below 4 GiB, checked at launch)
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<u16 *>(Kb), (short)0, (int)(uint32_t)(((int64_t)a.cap * a.G - g) * HD * 2), 0x00020000);
  u32x4 kf[4][NS];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const uint32_t key = (uint32_t)min(kw0 + kb * 16 + j, kmax);
    const uint32_t vo = key * (uint32_t)(kstride * 2) + (uint32_t)(grp * 16);
#pragma unroll
    for (int t = 0; t < NS; ++t) kf[kb][t] = __builtin_amdgcn_raw_buffer_load_b128(rk, vo, t * 64, 0);
  }
  // V: 16 direct-to-LDS instructions, 4 rows each; lane L -> row 4i + L/16, chunk L%16.
  // Issued after q and K, so the score products can start while V is in flight.
  u16 *vs = Vs[wave];
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<u16 *>(Vb), (short)0, (int)(uint32_t)(((int64_t)a.cap * a.G - g) * HD * 2), 0x00020000);
#pragma unroll
  for (int i = 0; i < KW / 4; ++i) {
    const int r = 4 * i + (lane >> 4);
    const int c = (lane & 15) ^ (r & 15);
    const uint32_t key = (uint32_t)min(kw0 + r, kmax);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (__attribute__((address_space(3))) void *)(vs + i * 4 * HD), 16,
                                             key * (uint32_t)(kstride * 2) + (uint32_t)(c * 16), 0, 0, 0);
  }
  __builtin_amdgcn_sched_barrier(0);  // every load is issued before the first product waits for K
  if (j >= n_rep) {  // columns past the group's heads (a select on loaded data placed earlier would wait for it)
#pragma unroll
    for (int t = 0; t < NS; ++t) {
      qh[t] = __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
      ql[t] = qh[t];
    }
  }
  // S^T (log2 units), masked past the sequence's position
  f32x4 sc[4];
  float mx = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    sc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < NS; ++t) {
      const bf16x8 kv = __builtin_bit_cast(bf16x8, kf[kb][t]);
      sc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, qh[t], sc[kb], 0, 0, 0);
      sc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, ql[t], sc[kb], 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = kw0 + kb * 16 + 4 * grp + r;
      if (key >= kend || key < kstart) sc[kb][r] = -INFINITY;
      mx = fmaxf(mx, sc[kb][r]);
    }
  }
  mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
  mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
  float ls = 0.f;
  bf16x8 pf[2], pl[2];  // A operands (hi, lo) of P V for the two 32-key steps
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float p = mx == -INFINITY ? 0.f : exp2f(sc[kb][r] - mx);
      ls += p;
      const __bf16 ph = (__bf16)p;
      pf[kb >> 1][(kb & 1) * 4 + r] = ph;
      pl[kb >> 1][(kb & 1) * 4 + r] = (__bf16)(p - (float)ph);
    }
  ls += __shfl_xor(ls, 16, kWave);
  ls += __shfl_xor(ls, 32, kWave);
  if (grp == 0 && j < NR) {
    red_m[wave][j] = mx;
    red_l[wave][j] = ls;
  }

  // O = P V: B operand via transposed LDS reads.  For step t, half h, lane
  // (grp, j) addresses row 32t + 16h + 4grp + j/4, columns 16nb + 4(j%4) .. +3.
  __builtin_amdgcn_s_waitcnt(0);  // this wave's V rows have landed
  __builtin_amdgcn_wave_barrier();
  f32x4 o[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) o[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int e = j >> 2, q = j & 3;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      // whole 32-bit words are moved: element-wise bit casts of the read
      // results are not kept apart by this compiler
      typedef short v4s __attribute__((ext_vector_type(4)));
      typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
      u32x2 wv[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int r = 32 * t + 16 * h + 4 * grp + e;
        const int c = (2 * nb + (q >> 1)) ^ (r & 15);
        const int off = (r * HD + c * 8 + (q & 1) * 4) * (int)sizeof(u16);
        const v4s w = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) v4s *)((__attribute__((address_space(3))) char *)vs + off));
        wv[h] = __builtin_bit_cast(u32x2, w);
      }
      const uint4 vw = make_uint4(wv[0].x, wv[0].y, wv[1].x, wv[1].y);
      const bf16x8 vb = __builtin_bit_cast(bf16x8, vw);
      o[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pf[t], vb, o[nb], 0, 0, 0);
      o[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl[t], vb, o[nb], 0, 0, 0);
    }
  }
  // lane (grp, j) holds O[head 4grp + r][16nb + j]
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = 4 * grp + r;
      if (h < NR) red_o[wave][h][nb * 16 + j] = o[nb][r];
    }
  __syncthreads();

  for (int i = tid; i < n_rep * HD; i += 256) {
    const int h = i / HD, d = i % HD;
    float M = red_m[0][h];
#pragma unroll
    for (int w = 1; w < 4; ++w) M = fmaxf(M, red_m[w][h]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float wt = red_m[w][h] == -INFINITY ? 0.f : exp2f(red_m[w][h] - M);
      L += wt * red_l[w][h];
      O += wt * red_o[w][h][d];
    }
    a.po[(pidx + (int64_t)h * a.nchunk) * HD + d] = O;
    if (d == 0) {
      a.pm[pidx + (int64_t)h * a.nchunk] = M;
      a.pl[pidx + (int64_t)h * a.nchunk] = L;
    }
  }
}

// Combine the chunk partials of one (sequence, head); maxima are in log2
// units: O = sum_c 2^{m_c - M} o_c / sum_c 2^{m_c - M} l_c, M = max_c m_c.
// With knew/vnew the query's own key and value join as one more partial
// (m = q.k_new * scale * log2 e, l = 1, o = v_new), all in fp32.
template <int HD>
__global__ __launch_bounds__(((HD + 63) / 64) * 64) void attn_combine_kernel(DecodeAttnArgs a) {
  constexpr int NW = (HD + 63) / 64;  // whole waves; lanes d >= HD only join the reduction
  __shared__ float red[NW];
  const int h = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
  const bool on = t < HD;
  const int d = on ? t : HD - 1;
  const int64_t base = ((int64_t)b * a.H + h) * a.nchunk;
  // Only chunks that hold visible keys are merged: keys 0..pos-1 when the
  // own term is added here, 0..pos otherwise (the chunk kernels leave the
  // others empty).  They are merged 16 at a time: each group's loads
  // (clamped to a valid chunk; the extra ones are skipped) are issued
  // together, and the running maximum M rescales what earlier groups summed.
  // The first group's loads go out before the own term's dot product.
  int pb = a.pos[b];
  pb = pb < 0 ? 0 : (pb > a.cap - 1 ? a.cap - 1 : pb);
  const int nkeys = a.knew ? pb : pb + 1;
  const int nc = min(a.nchunk, (nkeys + a.chunk - 1) / a.chunk);
  constexpr int CG = 16;
  float pm[CG], pl[CG], po[CG];
  auto load_group = [&](int c0) {
#pragma unroll
    for (int u = 0; u < CG; ++u) {
      const int64_t c = base + max(0, min(c0 + u, nc - 1));
      pm[u] = a.pm[c];
      pl[u] = a.pl[c];
      po[u] = a.po[c * HD + d];
    }
  };
  load_group(0);
  float ms = -INFINITY, vself = 0.f;
  if (a.knew) {
    const int g = h / (a.H / a.G);
    const int64_t kv = ((int64_t)b * a.G + g) * HD + d;
    float qk = on ? a.q[((int64_t)b * a.H + h) * HD + d] * a.knew[kv] : 0.f;
    qk = wave_sum(qk);
    if ((t & 63) == 0) red[t >> 6] = qk;
    __syncthreads();
    float dot = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) dot += red[w];
    ms = dot * a.scale * kLog2e;
    vself = a.vnew[kv];
  }
  float M = ms, L = 0.f, acc = 0.f;
  if (a.knew) {
    L = 1.f;
    acc = vself;
  }
  for (int c0 = 0; c0 < nc; c0 += CG) {
    if (c0 > 0) load_group(c0);
    float Mg = M;
#pragma unroll
    for (int u = 0; u < CG; ++u)
      if (c0 + u < nc) Mg = fmaxf(Mg, pm[u]);
    if (Mg == -INFINITY) continue;  // nothing visible yet
    const float r = exp2f(M - Mg);  // 0 when M is -inf
    L *= r;
    acc *= r;
    M = Mg;
#pragma unroll
    for (int u = 0; u < CG; ++u) {
      if (c0 + u >= nc || pm[u] == -INFINITY) continue;
      const float w = exp2f(pm[u] - M);
      L += w * pl[u];
      acc += w * po[u];
    }
  }
  if (!on) return;
  const float v = acc / L;
  const int64_t o = (int64_t)b * a.H * HD + h * HD + d;
  if (a.out_mode == 0) {
    static_cast<float *>(a.out)[o] = v;
  } else {
    u16 hi, lo;
    split_hilo(v, hi, lo);
    static_cast<u16 *>(a.out)[o] = hi;
    static_cast<u16 *>(a.out)[a.out_plane + o] = lo;
  }
}

template <int HD>
hipError_t prefill_hd(int dtype, const AttnArgs &a, hipStream_t s) {
  if (dtype == 1 && HD == 128) {
    const int QB = 256 / (a.H / a.G);
    const int nblk = ((a.S + QB - 1) / QB) * a.G * a.B;
    if (a.kv_lo)
      hipLaunchKernelGGL(attn_fwd_w8<true>, dim3(nblk), dim3(512), 0, s, a);
    else
      hipLaunchKernelGGL(attn_fwd_w8<false>, dim3(nblk), dim3(512), 0, s, a);
  } else if (dtype == 1) {
    const int QB = 128 / (a.H / a.G);
    dim3 grid((a.S + QB - 1) / QB, a.G, a.B);
    hipLaunchKernelGGL(attn_fwd_bf16<HD>, grid, dim3(256), 0, s, a);
  } else {
    dim3 grid((a.S + 31) / 32, a.H, a.B);
    hipLaunchKernelGGL(attn_fwd_f32<HD>, grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

template <int HD>
hipError_t decode_hd(int dtype, const DecodeAttnArgs &a, hipStream_t s) {
  dim3 grid(a.nchunk, a.G, a.B);
  const int n_rep = a.H / a.G;
  // attn_decode_mfma2 addresses one sequence's cache block with 32-bit offsets
  const bool below4g = (int64_t)a.cap * a.G * HD * 2 <= 0xFFFFFFFFll;
  if (dtype == 1 && HD == 128 && a.qhl && below4g && n_rep <= 4)
    hipLaunchKernelGGL((attn_decode_mfma2<4>), grid, dim3(256), 0, s, a);
  else if (dtype == 1 && HD == 128 && a.qhl && below4g && n_rep <= 16)
    hipLaunchKernelGGL((attn_decode_mfma2<16>), grid, dim3(256), 0, s, a);
  else if (dtype == 1 && n_rep <= 4)
    hipLaunchKernelGGL((attn_decode_mfma<HD, 4>), grid, dim3(256), 0, s, a);
  else if (dtype == 1 && n_rep <= 8)
    hipLaunchKernelGGL((attn_decode_mfma<HD, 8>), grid, dim3(256), 0, s, a);
  else if (dtype == 1)
    hipLaunchKernelGGL((attn_decode_kernel<u16, HD>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((attn_decode_kernel<float, HD>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_attn_prefill(int dtype, const AttnArgs &a, hipStream_t s) {
  switch (a.hd) {
    case 64: return prefill_hd<64>(dtype, a, s);
    case 96: return prefill_hd<96>(dtype, a, s);
    case 128: return prefill_hd<128>(dtype, a, s);
  }
  return hipErrorInvalidValue;
}

// Document starts: an inclusive max-scan of the run-start positions
// (p where doc[p] != doc[p-1], and 0).  One block per sequence.
__global__ __launch_bounds__(1024) void doc_starts_kernel(const int32_t *__restrict__ doc, int start_pos, int S,
                                                          int32_t *__restrict__ kv_lo) {
  const int b = blockIdx.x;
  const int n = start_pos + S;
  const int32_t *d = doc + (int64_t)b * n;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __shared__ int wm[16];
  __shared__ int carry;
  if (threadIdx.x == 0) carry = 0;
  __syncthreads();
  for (int base = 0; base < n; base += 1024) {
    const int p = base + threadIdx.x;
    int v = 0;
    if (p < n) v = (p == 0 || d[p] != d[p - 1]) ? p : 0;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(v, o, kWave);
      if (lane >= o) v = max(v, t);
    }
    if (lane == 63) wm[wave] = v;
    __syncthreads();
    int pre = carry;
    for (int w = 0; w < wave; ++w) pre = max(pre, wm[w]);
    v = max(v, pre);
    if (p >= start_pos && p < n) kv_lo[(int64_t)b * S + (p - start_pos)] = v;
    __syncthreads();
    if (threadIdx.x == 1023) carry = v;
    __syncthreads();
  }
}

hipError_t launch_doc_starts(const int32_t *doc, int B, int start_pos, int S, int32_t *kv_lo, hipStream_t s) {
  hipLaunchKernelGGL(doc_starts_kernel, dim3(B), dim3(1024), 0, s, doc, start_pos, S, kv_lo);
  return hipGetLastError();
}

hipError_t launch_attn_combine(const DecodeAttnArgs &a, hipStream_t s) {
  switch (a.hd) {
    case 64: hipLaunchKernelGGL(attn_combine_kernel<64>, dim3(a.H, a.B), dim3(64), 0, s, a); break;
    case 96: hipLaunchKernelGGL(attn_combine_kernel<96>, dim3(a.H, a.B), dim3(128), 0, s, a); break;
    case 128: hipLaunchKernelGGL(attn_combine_kernel<128>, dim3(a.H, a.B), dim3(128), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attn_decode(int dtype, const DecodeAttnArgs &a, hipStream_t s) {
  switch (a.hd) {
    case 64: return decode_hd<64>(dtype, a, s);
    case 96: return decode_hd<96>(dtype, a, s);
    case 128: return decode_hd<128>(dtype, a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace llk
