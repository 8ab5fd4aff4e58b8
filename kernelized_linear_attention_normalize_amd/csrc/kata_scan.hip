// Inclusive scan, in place, of per-segment state summaries across the segments of each
// (b,h): slot s ends up holding the sum of slots 0..s, i.e. the exclusive prefix of
// segment s+1. "Kernelized Linear Attention: Breaking the Capacity Wall with Symmetric
// Cones" (arXiv 2607.17419), arXiv HTML page, chunked-forward paragraph: the state prefix
// over chunks is an associative cumulative sum and admits a parallel scan of depth
// ceil(log2 N); the feature slices are independent.
//
// Layout: lane = slot inside a segment of SEG lanes (SEG = 16, 32 or 64 >= nslots), and
// every lane carries 4 consecutive state elements (one 16-byte load and store). A wave
// holds 64 / SEG column groups, so for the usual <= 16 slots all 64 lanes work. Rounds
// d = 1, 2, 4, .. < SEG add the value d slots up: inside 16-lane rows a DPP row shift
// (rows past the segment start read 0), across rows a wave shuffle.
#include "kata_device.h"
#include "kata_launch.h"

namespace kata {

constexpr int SCAN_ITER = 4;  // column groups per thread

typedef float scan_f4 __attribute__((ext_vector_type(4)));

// value of the lane d slots up in this lane's segment, 0 for slots < d
template <int SEG>
__device__ __forceinline__ float scan_up(float x, int d, int slot) {
  if (SEG == 16) {
    switch (d) {  // row_shr:d, bound_ctrl: lanes shifted in from outside the row read 0
      case 1: return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x111, 0xf, 0xf, true));
      case 2: return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x112, 0xf, 0xf, true));
      case 4: return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x114, 0xf, 0xf, true));
      default: return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x118, 0xf, 0xf, true));
    }
  }
  const float y = __shfl_up(x, d, SEG);
  return slot >= d ? y : 0.f;
}

template <int SEG>
__global__ __launch_bounds__(256) void segment_scan_kernel(float* __restrict__ ws, int nslots, int64_t E) {
  constexpr int G = 64 / SEG;                  // column groups per wave
  constexpr int COLS = 4 * G * 4 * SCAN_ITER;  // elements per workgroup
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int slot = lane % SEG, grp = lane / SEG;
  const int64_t ncolblk = (E + COLS - 1) / COLS;
  const int64_t bh = blockIdx.x / ncolblk;
  float* base = ws + bh * nslots * E + (int64_t)slot * E;
#pragma unroll
  for (int it = 0; it < SCAN_ITER; ++it) {
    const int64_t e = (blockIdx.x % ncolblk) * COLS + ((it * 4 + wave) * G + grp) * 4;
    const bool ok = slot < nslots && e < E;  // E is a multiple of 4
    scan_f4 x = {0.f, 0.f, 0.f, 0.f};
    if (ok) x = *reinterpret_cast<const scan_f4*>(base + e);
#pragma unroll
    for (int d = 1; d < SEG; d <<= 1)
#pragma unroll
      for (int j = 0; j < 4; ++j) x[j] += scan_up<SEG>(x[j], d, slot);
    if (ok) *reinterpret_cast<scan_f4*>(base + e) = x;
  }
}

hipError_t launch_scan(float* ws, int BH, int nslots, int64_t E, hipStream_t st) {
  if (nslots <= 1) return hipSuccess;  // one summary: already its own inclusive prefix
  if (nslots > 64 || E % 4 != 0) return hipErrorInvalidValue;
  auto grid = [&](int seg) {
    const int64_t cols = 4 * (64 / seg) * 4 * SCAN_ITER;
    return dim3((unsigned)(((E + cols - 1) / cols) * BH));
  };
  if (nslots <= 16)
    segment_scan_kernel<16><<<grid(16), dim3(256), 0, st>>>(ws, nslots, E);
  else if (nslots <= 32)
    segment_scan_kernel<32><<<grid(32), dim3(256), 0, st>>>(ws, nslots, E);
  else
    segment_scan_kernel<64><<<grid(64), dim3(256), 0, st>>>(ws, nslots, E);
  return hipGetLastError();
}

}  // namespace kata
