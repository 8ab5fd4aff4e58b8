// Row-wise kernels: the packed rank-one lift and the recurrent decode step.
//
// Lift: "Kernelized Linear Attention: Breaking the Capacity Wall with Symmetric Cones"
// (arXiv 2607.17419), arXiv HTML page, rank-one lift display after Eq. (8) and Eq. (8)
// (n = p(p+1)/2 packed coordinates). Decode: constant-time recurrent inference (abstract)
// with the feature-value state S_t = Psi(K_{1:t})^T V_{1:t} (state display) and the
// normalized readout psi(q)^T S / psi(q)^T Z (normalized-readout paragraph).
#include "kata_device.h"
#include "kata_launch.h"

namespace kata {

// ---------------------------------------------------------------------------- lift
// One workgroup lifts LIFT_ROWS rows. The packed (i, j) table is built once per
// workgroup in LDS, then every thread writes consecutive packed coordinates of a row,
// so the [rows, n] output is written with fully coalesced stores.
constexpr int LIFT_ROWS = 16;
constexpr int LIFT_MAXP = 128;

template <bool IN_BF16, bool OUT_BF16>
__global__ __launch_bounds__(256) void lift_kernel(const void* __restrict__ u, int64_t rows, int p,
                                                   void* __restrict__ psi) {
  __shared__ float uh[LIFT_ROWS][LIFT_MAXP];
  __shared__ uint16_t pairs[LIFT_MAXP * (LIFT_MAXP + 1) / 2];
  const int tid = threadIdx.x;
  const int n = p * (p + 1) / 2;
  const int64_t r0 = (int64_t)blockIdx.x * LIFT_ROWS;

  for (int f = tid; f < n; f += 256) {
    int i, j;
    packed_ij(f, p, i, j);
    pairs[f] = (uint16_t)((i << 8) | j);
  }
  // 16 threads per row: load, sum of squares, normalise
  {
    const int rr = tid >> 4, l16 = tid & 15;
    const int64_t row = r0 + rr;
    float ss = 0.f;
    for (int c = l16; c < p; c += 16) {
      float x = row < rows ? load_as_f32<IN_BF16>(u, row * p + c) : 0.f;
      uh[rr][c] = x;
      ss += x * x;
    }
    ss = group_sum<16>(ss);
    const float inv = inv_norm(ss);
    for (int c = l16; c < p; c += 16) uh[rr][c] *= inv;
  }
  __syncthreads();
  const int nrows = (int)min<int64_t>(LIFT_ROWS, rows - r0);
  for (int rr = 0; rr < nrows; ++rr) {
    const int64_t obase = (r0 + rr) * (int64_t)n;
    for (int f = tid; f < n; f += 256) {
      const int i = pairs[f] >> 8, j = pairs[f] & 255;
      float val = uh[rr][i] * uh[rr][j];
      if (i != j) val *= sqrt2f();
      store_from_f32<OUT_BF16>(psi, obase + f, val);
    }
  }
}

hipError_t launch_lift(const void* u, bool u_bf16, int64_t rows, int p, void* psi, bool psi_bf16,
                       hipStream_t st) {
  const int64_t nblk = (rows + LIFT_ROWS - 1) / LIFT_ROWS;
  dim3 grid((unsigned)nblk), block(256);
  if (u_bf16 && psi_bf16) lift_kernel<true, true><<<grid, block, 0, st>>>(u, rows, p, psi);
  else if (u_bf16) lift_kernel<true, false><<<grid, block, 0, st>>>(u, rows, p, psi);
  else if (psi_bf16) lift_kernel<false, true><<<grid, block, 0, st>>>(u, rows, p, psi);
  else lift_kernel<false, false><<<grid, block, 0, st>>>(u, rows, p, psi);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------- decode
// One workgroup per (sequence, head). The state row S[f, :] (dv fp32) is streamed once
// from HBM: read, add psi_f(k) v, write back, and accumulate psi_f(q) * S_new[f, :].
// Bytes per head-step: 2 n dv 4 (S) + 2 n 4 (Z) + q, k, v, o. Threads are laid out so
// that consecutive threads touch consecutive 16-byte pieces of consecutive rows.
// The state loads do not depend on the lifts, so each thread issues its first DEC_PF
// pieces before normalising and lifting q and k (every workgroup of the grid starts at
// once, and HBM would otherwise idle through that prologue), and then keeps DEC_PF loads
// in flight: once pass it is updated and stored, its registers are refilled with pass
// it + DEC_PF. The shape (p = 32, dv = 64) is compiled with fixed sizes, so its 33 passes
// unroll and the compiler waits for exactly the load a pass needs.
constexpr int DEC_MAXP = 64;
constexpr int DEC_MAXN = DEC_MAXP * (DEC_MAXP + 1) / 2;
constexpr int DEC_PF = 8;  // state pieces in flight per thread

// PT, DVT > 0 fix p and dv at compile time (the pass loop then unrolls into straight-line
// code whose load waits the compiler counts exactly); 0 takes them from the arguments
template <bool IN_BF16, bool OUT_BF16, int PT = 0, int DVT = 0>
__global__ __launch_bounds__(256) void decode_kernel(const void* __restrict__ q,
                                                     const void* __restrict__ k,
                                                     const void* __restrict__ v,
                                                     float* __restrict__ S, float* __restrict__ Z,
                                                     void* __restrict__ o, int p_arg, int dv_arg) {
  const int p = PT > 0 ? PT : p_arg, dv = DVT > 0 ? DVT : dv_arg;
  __shared__ float qh[DEC_MAXP], kh[DEC_MAXP], vv[DEC_MAXP];
  __shared__ float psq[DEC_MAXN], psk[DEC_MAXN];
  __shared__ f32x4_t red[256];
  __shared__ float dred[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t bh = blockIdx.x;
  const int n = p * (p + 1) / 2;

  const int D4 = dv >> 2;                 // float4 pieces per state row
  const int RPP = 256 / D4;               // rows per pass
  const bool active = tid < RPP * D4;
  const int d4 = tid % D4, rr = tid / D4;
  const int npass = (n + RPP - 1) / RPP;  // passes over the rows (row rr + RPP it)
  // this head's state through a buffer resource: pieces past row n - 1 load as zero and
  // their stores are dropped, so the loads need no bounds test
  const __amdgpu_buffer_rsrc_t rs = buf_rsrc(S + bh * (int64_t)n * dv, (uint32_t)(n * dv * 4));
  const uint32_t off0 = (uint32_t)(rr * dv * 4 + d4 * 16), stp = (uint32_t)(RPP * dv * 4);
  u32x4_t pre[DEC_PF];
#pragma unroll
  for (int u = 0; u < DEC_PF; ++u)
    pre[u] = active ? __builtin_amdgcn_raw_buffer_load_b128(rs, off0 + u * stp, 0, 0) : u32x4_t{0u, 0u, 0u, 0u};

  if (wave < 2) {  // wave 0 normalises q, wave 1 normalises k (p <= 64)
    const void* src = wave == 0 ? q : k;
    float x = lane < p ? load_as_f32<IN_BF16>(src, bh * p + lane) : 0.f;
    const float inv = inv_norm(wave_sum(x * x));
    if (lane < p) (wave == 0 ? qh : kh)[lane] = x * inv;
  } else if (wave == 2 && lane < dv) {
    vv[lane] = load_as_f32<IN_BF16>(v, bh * dv + lane);
  }
  __syncthreads();
  for (int f = tid; f < n; f += 256) {
    int i, j;
    packed_ij(f, p, i, j);
    const float c = i == j ? 1.f : sqrt2f();
    psq[f] = c * qh[i] * qh[j];
    psk[f] = c * kh[i] * kh[j];
  }
  __syncthreads();

  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  if (active) {
    const f32x4_t v4 = {vv[4 * d4], vv[4 * d4 + 1], vv[4 * d4 + 2], vv[4 * d4 + 3]};
#pragma unroll
    for (int it = 0; it < npass; it += DEC_PF) {
      const uint32_t offc = off0 + (uint32_t)it * stp;
#pragma unroll
      for (int u = 0; u < DEC_PF; ++u) {
        // slot u: update pass it + u, then refill the slot's registers with pass it + u + DEC_PF
        // (in that order, so the refill lands in the registers the loop carries and needs no
        // copy, which would wait for the load)
        const int f = rr + (it + u) * RPP;
        if (f < n) {
          const f32x4_t s = __builtin_bit_cast(f32x4_t, pre[u]) + psk[f] * v4;
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, s), rs, offc + u * stp, 0, 0);
          acc += psq[f] * s;
        }
        __builtin_amdgcn_sched_barrier(0);
        pre[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, offc + (DEC_PF + u) * stp, 0, 0);
      }
    }
  }
  red[tid] = acc;
  float dacc = 0.f;
  float* Zb = Z + bh * (int64_t)n;
  for (int f = tid; f < n; f += 256) {
    const float z = Zb[f] + psk[f];
    Zb[f] = z;
    dacc += psq[f] * z;
  }
  dacc = wave_sum(dacc);
  if (lane == 0) dred[wave] = dacc;
  __syncthreads();
  if (tid < dv) {
    const int dd4 = tid >> 2, c = tid & 3;
    float num = 0.f;
    for (int r = 0; r < RPP; ++r) num += red[r * D4 + dd4][c];
    const float den = dred[0] + dred[1] + dred[2] + dred[3];
    store_from_f32<OUT_BF16>(o, bh * dv + tid, den > 0.f ? num / den : 0.f);
  }
}

hipError_t launch_decode(const void* q, const void* k, const void* v, bool in_bf16, float* S,
                         float* Z, void* o, bool o_bf16, int N, int H, int p, int dv,
                         hipStream_t st) {
  dim3 grid((unsigned)((int64_t)N * H)), block(256);
  if (in_bf16 && o_bf16 && p == 32 && dv == 64) decode_kernel<true, true, 32, 64><<<grid, block, 0, st>>>(q, k, v, S, Z, o, p, dv);
  else if (in_bf16 && o_bf16) decode_kernel<true, true><<<grid, block, 0, st>>>(q, k, v, S, Z, o, p, dv);
  else if (in_bf16) decode_kernel<true, false><<<grid, block, 0, st>>>(q, k, v, S, Z, o, p, dv);
  else if (o_bf16) decode_kernel<false, true><<<grid, block, 0, st>>>(q, k, v, S, Z, o, p, dv);
  else decode_kernel<false, false><<<grid, block, 0, st>>>(q, k, v, S, Z, o, p, dv);
  return hipGetLastError();
}

// ---- zero fill (the state of empty sequences)
__global__ __launch_bounds__(256) void fill_zero_kernel(float* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0.f;
}

hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096;
  fill_zero_kernel<<<dim3((unsigned)blocks), dim3(256), 0, st>>>(p, n);
  return hipGetLastError();
}

}  // namespace kata
