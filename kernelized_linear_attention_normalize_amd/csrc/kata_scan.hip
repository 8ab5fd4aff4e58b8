// Inclusive scan, in place, of per-segment state summaries across the segments of each
// (b,h): slot s ends up holding the sum of slots 0..s, i.e. the exclusive prefix of
// segment s+1. "Kernelized Linear Attention: Breaking the Capacity Wall with Symmetric
// Cones" (arXiv 2607.17419), arXiv HTML page, chunked-forward paragraph: the state prefix
// over chunks is an associative cumulative sum and admits a parallel scan of depth
// ceil(log2 N); the feature slices are independent. Here each wave scans one state
// element across all slots with a Hillis-Steele scan over lanes (lane = slot), and a
// workgroup moves 64 consecutive elements x all slots through LDS so that every HBM
// access is a coalesced 256-byte row.
#include "kata_device.h"
#include "kata_launch.h"

namespace kata {

constexpr int SCAN_COLS = 64;
constexpr int SCAN_MAXSLOTS = 64;

__global__ __launch_bounds__(256) void segment_scan_kernel(float* __restrict__ ws, int nslots,
                                                           int64_t E) {
  __shared__ float tile[SCAN_MAXSLOTS][SCAN_COLS + 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t ncolblk = (E + SCAN_COLS - 1) / SCAN_COLS;
  const int64_t e0 = ((int64_t)blockIdx.x % ncolblk) * SCAN_COLS;
  float* base = ws + ((int64_t)blockIdx.x / ncolblk) * nslots * E;
  for (int idx = tid; idx < nslots * SCAN_COLS; idx += 256) {
    const int s = idx / SCAN_COLS, e = idx % SCAN_COLS;
    tile[s][e] = e0 + e < E ? base[s * E + e0 + e] : 0.f;
  }
  __syncthreads();
  for (int col = wave; col < SCAN_COLS; col += 4) {
    float x = lane < nslots ? tile[lane][col] : 0.f;
    for (int d = 1; d < nslots; d <<= 1) {  // ceil(log2 nslots) rounds
      const float y = __shfl_up(x, d, 64);
      if (lane >= d) x += y;
    }
    if (lane < nslots) tile[lane][col] = x;
  }
  __syncthreads();
  for (int idx = tid; idx < nslots * SCAN_COLS; idx += 256) {
    const int s = idx / SCAN_COLS, e = idx % SCAN_COLS;
    if (e0 + e < E) base[s * E + e0 + e] = tile[s][e];
  }
}

hipError_t launch_scan(float* ws, int BH, int nslots, int64_t E, hipStream_t st) {
  if (nslots <= 1) return hipSuccess;  // one summary: already its own inclusive prefix
  dim3 grid((unsigned)(((E + SCAN_COLS - 1) / SCAN_COLS) * BH)), block(256);
  segment_scan_kernel<<<grid, block, 0, st>>>(ws, nslots, E);
  return hipGetLastError();
}

}  // namespace kata
