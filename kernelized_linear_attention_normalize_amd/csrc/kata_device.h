// Device-side helpers shared by the KATA kernels (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8_t __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4_t __attribute__((ext_vector_type(4)));

namespace kata {

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// fp32 -> bf16 bits, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(uint16_t, b);
}

// Load element i of an fp32 or bf16 array as fp32.
template <bool BF16>
__device__ __forceinline__ float load_as_f32(const void* base, int64_t i) {
  if constexpr (BF16) return bf16_bits_to_f32(static_cast<const uint16_t*>(base)[i]);
  else return static_cast<const float*>(base)[i];
}

// Store fp32 value x as element i of an fp32 or bf16 array.
template <bool BF16>
__device__ __forceinline__ void store_from_f32(void* base, int64_t i, float x) {
  if constexpr (BF16) static_cast<uint16_t*>(base)[i] = f32_to_bf16_bits(x);
  else static_cast<float*>(base)[i] = x;
}

// 1/||u|| for a row with squared norm ss; 0 for a zero row (the lift of 0 is 0).
__device__ __forceinline__ float inv_norm(float ss) { return ss > 0.f ? 1.0f / sqrtf(ss) : 0.f; }

// Packed coordinate f of the row-major upper triangle (incl. diagonal) -> (i, j).
// start(i) = i*p - i*(i-1)/2 is the packed index of (i, i).
__device__ __forceinline__ void packed_ij(int f, int p, int& i, int& j) {
  float b = 2.0f * p + 1.0f;
  int ii = (int)((b - sqrtf(b * b - 8.0f * f)) * 0.5f);
  ii = ii < 0 ? 0 : (ii > p - 1 ? p - 1 : ii);
  // exact integer correction of the float estimate
  while (ii > 0 && ii * p - (ii * (ii - 1)) / 2 > f) --ii;
  while (ii + 1 < p && (ii + 1) * p - ((ii + 1) * ii) / 2 <= f) ++ii;
  i = ii;
  j = ii + (f - (ii * p - (ii * (ii - 1)) / 2));
}

__device__ __forceinline__ float sqrt2f() { return 1.41421356237309515f; }

// Sum over the 64 lanes of a wave.
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

}  // namespace kata
