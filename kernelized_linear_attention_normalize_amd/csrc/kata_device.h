// Device-side helpers shared by the KATA kernels (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kata_launch.h"

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8_t __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

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
// fast reciprocal square root (about 1 ulp; results feed bf16 MFMA operands)
__device__ __forceinline__ float inv_norm_fast(float ss) { return ss > 0.f ? __builtin_amdgcn_rsqf(ss) : 0.f; }

// two fp32 -> packed bf16 pair (one v_cvt_pk_bf16_f32, round to nearest even)
__device__ __forceinline__ uint32_t pk2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// raw buffer resource over [base, base + bytes): loads past the end return 0 and stores
// past the end are dropped by the hardware range check, so ragged tails need no branches
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// ---- V^T staging shared by the MFMA kernels. Keys come in pairs (2 rows of V, 8 columns
// per piece); V^T is bf16 [DV][pitch] in LDS.
// Key position: key 32a + 16s + 4g + j is stored at 32a + 8g + 4s + j, so MFMA lane group g
// reads its 8 k-slots (keys 32a + 4g + j and 32a + 16 + 4g + j: the row order of 16x16
// score accumulators) with one 16-byte read.
__device__ __forceinline__ int vt_pos(int k) { return (k & ~31) + 8 * ((k >> 2) & 3) + 4 * ((k >> 4) & 1) + (k & 3); }
// Physical LDS row of V^T column d: the low 2 bits are XOR-swizzled by (d / 8) & 3 so the
// transposed writes of 4 column groups land in distinct banks.
__device__ __forceinline__ int vt_row(int d) { return d ^ ((d >> 3) & 3); }
// Piece pc -> (key pair vp, column group vd): each 32-lane half loads 8 key pairs x 4
// column groups (64 contiguous bytes per row) whose transposed 4-byte LDS writes hit 32
// distinct banks (key-pair positions distinct mod 8, rows swizzled by vd & 3) when the
// pitch in floats is 8 modulo 32. Needs a multiple of 16 key pairs.
template <int DV>
__device__ __forceinline__ void vt_piece(int pc, int& vp, int& vd) {
  constexpr int NVD = DV / 8, VL = NVD < 4 ? NVD : 4, VH = NVD / VL;
  const int qd = pc / (8 * VL), r = pc % (8 * VL);
  const int vl = r / VL, sg = qd / VH;
  vd = r % VL + VL * (qd % VH);
  vp = 16 * (sg >> 1) + 4 * (sg & 1) + (vl & 3) + 8 * (vl >> 2);
}

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

// x of the lane that DPP control CTRL selects inside this lane's 16-lane row
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xf, 0xf, true));
}
// x + x of lane ^ 16 (gfx950 permlane16 swap: odd rows trade with even rows)
__device__ __forceinline__ float xor16_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// x + x of lane ^ 32 (gfx950 permlane32 swap: the wave halves trade)
__device__ __forceinline__ float xor32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// Sum over aligned groups of G adjacent lanes (G = 1, 2, 4, ..., 64) without LDS traffic:
// DPP inside 16-lane rows, permlane swaps across rows. Every step adds a symmetric pair,
// so all lanes of a group end with the bitwise same sum.
template <int G>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (G >= 2) x += dpp_f<0xB1>(x);   // quad_perm [1,0,3,2]: lane ^ 1
  if constexpr (G >= 4) x += dpp_f<0x4E>(x);   // quad_perm [2,3,0,1]: lane ^ 2
  if constexpr (G >= 8) x += dpp_f<0x141>(x);  // row_half_mirror: the other quad of the 8
  if constexpr (G >= 16) x += dpp_f<0x140>(x); // row_mirror: the other half of the row
  if constexpr (G >= 32) x = xor16_sum(x);
  if constexpr (G >= 64) x = xor32_sum(x);
  return x;
}

// Sum over the 64 lanes of a wave.
__device__ __forceinline__ float wave_sum(float x) { return group_sum<64>(x); }

// First row, row step (in rows) and rows in use of sequence bh = (b, h) of a chunked
// forward (see SeqLayout). Lengths clamp to [0, T] and packed offsets to [0, total], so every
// row a kernel touches lies inside the tensors whatever the device arrays hold.
__device__ __forceinline__ void seq_rows_of(const SeqLayout& L, int64_t bh, int H, int T, int64_t& row0,
                                            int& step, int& len) {
  const int64_t b = bh / H, h = bh % H;
  if (L.cu != nullptr) {
    int s = L.cu[b], e = L.cu[b + 1];
    s = s < 0 ? 0 : (s > L.total ? L.total : s);
    e = e < s ? s : (e > L.total ? L.total : e);
    row0 = (int64_t)s * H + h;
    step = H;
    len = e - s < T ? e - s : T;
  } else {
    row0 = bh * (int64_t)T;
    step = 1;
    len = L.lens == nullptr ? T : min(max(L.lens[b], 0), T);
  }
}

}  // namespace kata
