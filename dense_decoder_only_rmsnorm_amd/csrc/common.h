// Shared device helpers for the gfx950 kernels: bf16 storage conversions,
// vector types for MFMA operands, wavefront reductions.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace llk {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint16_t u16;

constexpr int kWave = 64;

// bf16 <-> fp32.  Storage is raw uint16 bit patterns; widening is exact,
// narrowing rounds to nearest even (the hardware conversion, one instruction
// on gfx950; inputs are finite).
__device__ __forceinline__ float bf2f(u16 b) { return __uint_as_float(((uint32_t)b) << 16); }
__device__ __forceinline__ u16 f2bf(float f) { return __builtin_bit_cast(u16, (__bf16)f); }
// Split v into hi + lo, both bf16, with hi = bf16(v) and lo = bf16(v - hi):
// hi + lo carries about 16 significant bits of v.
__device__ __forceinline__ void split_hilo(float v, u16 &hi, u16 &lo) {
  hi = f2bf(v);
  lo = f2bf(v - bf2f(hi));
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float load(const float *p) { return *p; }
  static __device__ __forceinline__ void store(float *p, float v) { *p = v; }
};
template <> struct Elem<u16> {
  static __device__ __forceinline__ float load(const u16 *p) { return bf2f(*p); }
  static __device__ __forceinline__ void store(u16 *p, float v) { *p = f2bf(v); }
};

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// silu(x) = x / (1 + e^-x), the quotient through the hardware reciprocal
// (about 1 ulp; the result is rounded to bf16 or compared at fp32 tolerance)
__device__ __forceinline__ float silu(float x) { return x * __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }

// (a + i b) * (c + i s): the rotation of one RoPE pair by an angle with
// cosine c and sine s.
__device__ __forceinline__ float2 rotate_pair(float a, float b, float c, float s) {
  return make_float2(a * c - b * s, a * s + b * c);
}

}  // namespace llk
