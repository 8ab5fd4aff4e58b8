// The reduced PSD feature families KATA-Sigma g and KATA-M g on plain VALU kernels:
// packed lift, recurrent decode step, chunked-state forward (sequential or associative
// prefix) and the flash-style quadratic form, for fp32 or bf16 inputs.
//
// Source: "Kernelized Linear Attention: Breaking the Capacity Wall with Symmetric Cones"
// (arXiv 2607.17419), arXiv HTML page, reduced PSD families paragraph: the unit-normalised
// projection u is split into g blocks of m = p / g components;
//   Sigma g: psi(u) = sum_a u_a u_a^T (m x m, m(m+1)/2 packed coordinates), weight
//            <psi(q), psi(k)> = sum_{a,b} (q_a . k_b)^2;
//   M g:     psi(u) = (u_1 u_1^T, ..., u_g u_g^T) (g m(m+1)/2 coordinates, block 1 first),
//            weight sum_a (q_a . k_a)^2.
// Packing inside an m x m block is the full map's (row-major upper triangle, sqrt(2) off the
// diagonal). The readout, the state and the chunk algebra are those of the full map
// (normalized-readout paragraph, feature-value state display, chunked-forward paragraph).
#include "kata_device.h"
#include "kata_launch.h"

namespace kata {

namespace {

struct Feat {
  int sigma;  // 1: Sigma g, 0: M g
  int g, m, nb, n;  // blocks, block width, packed coordinates per block, total coordinates
  int order;  // r of the weight's even power (q . k)^(2r) per block pair; 1 for the families
};

// (i, j) of packed coordinate f of an m x m block (f < m(m+1)/2), as a 16:16 table entry
__device__ __forceinline__ uint32_t pair_entry(const Feat& F, int f) {
  const int a = F.sigma ? 0 : f / F.nb, fl = F.sigma ? f : f % F.nb;
  int i, j;
  packed_ij(fl, F.m, i, j);
  return (uint32_t)((a * F.m + i) << 16) | (uint32_t)(a * F.m + j);
}

// psi_f of a normalised row u from its table entry
__device__ __forceinline__ float feat_val(const Feat& F, uint32_t e, const float* u) {
  const int i = (int)(e >> 16), j = (int)(e & 0xffffu);
  const float c = i == j ? 1.f : sqrt2f();
  if (!F.sigma) return c * u[i] * u[j];
  float s = 0.f;
  for (int a = 0; a < F.g; ++a) s += u[a * F.m + i] * u[a * F.m + j];
  return c * s;
}

// weight <psi(q), psi(k)> of two normalised rows from block dot products
__device__ __forceinline__ float feat_weight(const Feat& F, const float* q, const float* k) {
  float w = 0.f;
  for (int a = 0; a < F.g; ++a)
    for (int b = 0; b < F.g; ++b) {
      if (!F.sigma && b != a) continue;
      float d = 0.f;
      for (int i = 0; i < F.m; ++i) d += q[a * F.m + i] * k[b * F.m + i];
      const float d2 = d * d;
      float x = d2;
      for (int o = 1; o < F.order; ++o) x *= d2;
      w += x;
    }
  return w;
}

// normalise row r of a [rows, p] input into dst (fp32); rows past `rows` are zero
template <bool IN_BF16>
__device__ __forceinline__ void load_norm_row(const void* src, int64_t row, bool valid, int p, float* dst) {
  float ss = 0.f;
  for (int i = 0; i < p; ++i) {
    const float x = valid ? load_as_f32<IN_BF16>(src, row * p + i) : 0.f;
    dst[i] = x;
    ss += x * x;
  }
  const float inv = inv_norm(ss);
  for (int i = 0; i < p; ++i) dst[i] *= inv;
}

Feat make_feat(int p, int fam, int g) {
  Feat F;
  F.sigma = fam == 1 ? 1 : 0;
  F.g = g;
  F.m = p / g;
  F.nb = F.m * (F.m + 1) / 2;
  F.n = F.sigma ? F.nb : g * F.nb;
  F.order = 1;
  return F;
}

// the full map with weights (q_hat . k_hat)^(2r): one block, no lift (weight form only)
Feat make_order(int p, int r) {
  Feat F = make_feat(p, 2, 1);
  F.order = r;
  return F;
}

}  // namespace

int64_t family_state_floats(int p, int dv, int fam, int g) {
  const Feat F = make_feat(p, fam, g);
  return ((int64_t)F.n * dv + F.n + 3) / 4 * 4;  // padded to 16 bytes (the scan's unit)
}

size_t family_chunked_lds_bytes(int p, int dv, int C, int fam, int g) {
  const Feat F = make_feat(p, fam, g);
  return 4 * ((size_t)F.n * dv + F.n + 2 * (size_t)C * p + (size_t)C * dv + C + F.n);
}

// ---------------------------------------------------------------------------- lift
constexpr int FL_ROWS = 16, FL_MAXP = 128, FL_MAXN = FL_MAXP * (FL_MAXP + 1) / 2;

template <bool IN_BF16, bool OUT_BF16>
__global__ __launch_bounds__(256) void family_lift_kernel(const void* __restrict__ u, int64_t rows, int p,
                                                          Feat F, void* __restrict__ psi) {
  __shared__ float uh[FL_ROWS][FL_MAXP];
  __shared__ uint32_t tab[FL_MAXN];
  const int tid = threadIdx.x;
  const int64_t r0 = (int64_t)blockIdx.x * FL_ROWS;
  for (int f = tid; f < F.n; f += 256) tab[f] = pair_entry(F, f);
  if (tid < FL_ROWS) load_norm_row<IN_BF16>(u, r0 + tid, r0 + tid < rows, p, uh[tid]);
  __syncthreads();
  const int nrows = (int)min<int64_t>(FL_ROWS, rows - r0);
  for (int rr = 0; rr < nrows; ++rr)
    for (int f = tid; f < F.n; f += 256)
      store_from_f32<OUT_BF16>(psi, (r0 + rr) * (int64_t)F.n + f, feat_val(F, tab[f], uh[rr]));
}

hipError_t launch_family_lift(const void* u, bool u_bf16, int64_t rows, int p, int fam, int g, void* psi,
                              bool psi_bf16, hipStream_t st) {
  const Feat F = make_feat(p, fam, g);
  dim3 grid((unsigned)((rows + FL_ROWS - 1) / FL_ROWS)), block(256);
  if (u_bf16 && psi_bf16) family_lift_kernel<true, true><<<grid, block, 0, st>>>(u, rows, p, F, psi);
  else if (u_bf16) family_lift_kernel<true, false><<<grid, block, 0, st>>>(u, rows, p, F, psi);
  else if (psi_bf16) family_lift_kernel<false, true><<<grid, block, 0, st>>>(u, rows, p, F, psi);
  else family_lift_kernel<false, false><<<grid, block, 0, st>>>(u, rows, p, F, psi);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------- psi_2r lift
// Coordinate f <-> the f-th multiset i_1 <= ... <= i_2r of range(p) in lexicographic order,
// value sqrt((2r)! / prod mult!) prod u_hat_i (arXiv HTML page, psi_2r display: the packed
// inner product is (u . v)^(2r)).

// number of multisets of size len over {lo, ..., p-1}: binom(p - lo + len - 1, len)
__device__ __forceinline__ double n_multisets(int p, int lo, int len) {
  const int nn = p - lo;
  if (len == 0) return 1.0;
  if (nn <= 0) return 0.0;
  double c = 1.0;
  for (int i = 1; i <= len; ++i) c = c * (nn + len - i) / i;
  return c;
}

template <bool IN_BF16, bool OUT_BF16>
__global__ __launch_bounds__(256) void order_lift_kernel(const void* __restrict__ u, int64_t rows, int p, int r,
                                                         int64_t n, void* __restrict__ psi) {
  __shared__ float uh[FL_ROWS][FL_MAXP];
  const int tid = threadIdx.x;
  const int64_t r0 = (int64_t)blockIdx.y * FL_ROWS;
  if (tid < FL_ROWS) load_norm_row<IN_BF16>(u, r0 + tid, r0 + tid < rows, p, uh[tid]);
  __syncthreads();
  const int64_t f = (int64_t)blockIdx.x * 256 + tid;
  if (f >= n) return;
  // unrank f: choose each element as the smallest value whose block of multisets holds f
  int idx[8];
  double rank = (double)f;
  int lo = 0;
  for (int pos = 0; pos < 2 * r; ++pos) {
    int i = lo;
    for (;; ++i) {
      const double cnt = n_multisets(p, i, 2 * r - pos - 1);
      if (rank < cnt || i == p - 1) break;
      rank -= cnt;
    }
    idx[pos] = i;
    lo = i;
  }
  double coef = 1.0;  // (2r)! / prod mult!
  for (int i = 2; i <= 2 * r; ++i) coef *= i;
  int run = 1;
  for (int pos = 1; pos <= 2 * r; ++pos) {
    if (pos < 2 * r && idx[pos] == idx[pos - 1]) {
      ++run;
    } else {
      for (int i = 2; i <= run; ++i) coef /= i;
      run = 1;
    }
  }
  const float c = (float)sqrt(coef);
  const int nrows = (int)min<int64_t>(FL_ROWS, rows - r0);
  for (int rr = 0; rr < nrows; ++rr) {
    float val = c;
    for (int pos = 0; pos < 2 * r; ++pos) val *= uh[rr][idx[pos]];
    store_from_f32<OUT_BF16>(psi, (r0 + rr) * n + f, val);
  }
}

hipError_t launch_order_lift(const void* u, bool u_bf16, int64_t rows, int p, int r, int64_t n, void* psi,
                             bool psi_bf16, hipStream_t st) {
  dim3 grid((unsigned)((n + 255) / 256), (unsigned)((rows + FL_ROWS - 1) / FL_ROWS)), block(256);
  if (u_bf16 && psi_bf16) order_lift_kernel<true, true><<<grid, block, 0, st>>>(u, rows, p, r, n, psi);
  else if (u_bf16) order_lift_kernel<true, false><<<grid, block, 0, st>>>(u, rows, p, r, n, psi);
  else if (psi_bf16) order_lift_kernel<false, true><<<grid, block, 0, st>>>(u, rows, p, r, n, psi);
  else order_lift_kernel<false, false><<<grid, block, 0, st>>>(u, rows, p, r, n, psi);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------- decode
// One workgroup per (sequence, head): update then read out, streaming S once.
constexpr int FD_MAXP = 64, FD_MAXN = FD_MAXP * (FD_MAXP + 1) / 2;

template <bool IN_BF16, bool OUT_BF16>
__global__ __launch_bounds__(256) void family_decode_kernel(const void* __restrict__ q, const void* __restrict__ k,
                                                            const void* __restrict__ v, float* __restrict__ S,
                                                            float* __restrict__ Z, void* __restrict__ o, int p,
                                                            int dv, Feat F) {
  __shared__ float qh[FD_MAXP], kh[FD_MAXP], vv[FD_MAXP];
  __shared__ float psq[FD_MAXN], psk[FD_MAXN];
  __shared__ float red[256];
  const int tid = threadIdx.x;
  const int64_t bh = blockIdx.x;
  if (tid == 0) load_norm_row<IN_BF16>(q, bh, true, p, qh);
  if (tid == 64) load_norm_row<IN_BF16>(k, bh, true, p, kh);
  if (tid >= 128 && tid < 128 + dv) vv[tid - 128] = load_as_f32<IN_BF16>(v, bh * dv + (tid - 128));
  __syncthreads();
  for (int f = tid; f < F.n; f += 256) {
    const uint32_t e = pair_entry(F, f);
    psq[f] = feat_val(F, e, qh);
    psk[f] = feat_val(F, e, kh);
  }
  __syncthreads();
  // S rows: thread (f0, d) walks rows f0, f0 + R, ... for column d
  const int R = 256 / dv, d = tid % dv, f0 = tid / dv;
  float num = 0.f;
  float* Sb = S + bh * (int64_t)F.n * dv;
  if (f0 < R)
    for (int f = f0; f < F.n; f += R) {
      const float s = Sb[(int64_t)f * dv + d] + psk[f] * vv[d];
      Sb[(int64_t)f * dv + d] = s;
      num += psq[f] * s;
    }
  float den = 0.f;
  float* Zb = Z + bh * (int64_t)F.n;
  for (int f = tid; f < F.n; f += 256) {
    const float z = Zb[f] + psk[f];
    Zb[f] = z;
    den += psq[f] * z;
  }
  red[tid] = den;
  __syncthreads();
  if (tid == 0) {
    float t = 0.f;
    for (int i = 0; i < 256; ++i) t += red[i];
    red[0] = t;
  }
  __syncthreads();
  const float dsum = red[0];
  __syncthreads();
  red[tid] = f0 < R ? num : 0.f;
  __syncthreads();
  if (tid < dv) {
    float t = 0.f;
    for (int r = 0; r < R; ++r) t += red[r * dv + tid];
    store_from_f32<OUT_BF16>(o, bh * dv + tid, dsum > 0.f ? t / dsum : 0.f);
  }
}

hipError_t launch_family_decode(const void* q, const void* k, const void* v, bool in_bf16, float* S, float* Z,
                                void* o, bool o_bf16, int N, int H, int p, int dv, int fam, int g,
                                hipStream_t st) {
  const Feat F = make_feat(p, fam, g);
  dim3 grid((unsigned)((int64_t)N * H)), block(256);
  if (in_bf16 && o_bf16) family_decode_kernel<true, true><<<grid, block, 0, st>>>(q, k, v, S, Z, o, p, dv, F);
  else if (in_bf16) family_decode_kernel<true, false><<<grid, block, 0, st>>>(q, k, v, S, Z, o, p, dv, F);
  else if (o_bf16) family_decode_kernel<false, true><<<grid, block, 0, st>>>(q, k, v, S, Z, o, p, dv, F);
  else family_decode_kernel<false, false><<<grid, block, 0, st>>>(q, k, v, S, Z, o, p, dv, F);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------- chunked
// One workgroup per (b*h, segment), state [S | Z] in LDS in packed order.
// MODE 0: forward of one segment from its prefix (the last segment of a sequence also
// writes the final state to s_out / z_out when given); MODE 1: the segment's summary.
// LDS: S[n*dv] Z[n] qh[C*p] kh[C*p] vv[C*dv] den[C] tab[n]
template <bool IN_BF16, bool OUT_BF16, int MODE>
__global__ __launch_bounds__(256) void family_chunked_kernel(const void* __restrict__ q, const void* __restrict__ k,
                                                             const void* __restrict__ v, void* __restrict__ o,
                                                             int T, int p, int dv, int C, Feat F, int nseg,
                                                             int cps, int nblk_per_bh, float* __restrict__ ws,
                                                             int64_t state_floats, float* __restrict__ s_out,
                                                             float* __restrict__ z_out, SeqLayout lay, int H) {
  extern __shared__ float sm[];
  const int n = F.n;
  float* Ss = sm;
  float* Zs = Ss + n * dv;
  float* qh = Zs + n;
  float* kh = qh + C * p;
  float* vv = kh + C * p;
  float* den = vv + C * dv;
  uint32_t* tab = reinterpret_cast<uint32_t*>(den + C);
  const int tid = threadIdx.x;
  const int64_t bh = blockIdx.x / nblk_per_bh;
  const int seg = blockIdx.x % nblk_per_bh;
  int64_t row0;
  int rstep, Tb;  // first row, row step, this sequence's rows
  seq_rows_of(lay, bh, H, T, row0, rstep, Tb);
  const int nchunks = (Tb + C - 1) / C;
  const int c0 = seg * cps, c1 = min(nchunks, c0 + cps);

  for (int f = tid; f < n; f += 256) tab[f] = pair_entry(F, f);
  if (MODE == 0 && seg > 0) {  // exclusive prefix of this segment (inclusive scan slot seg - 1)
    const float* src = ws + (bh * (nseg - 1) + (seg - 1)) * state_floats;
    for (int e = tid; e < n * dv + n; e += 256) Ss[e] = src[e];
  } else {
    for (int e = tid; e < n * dv + n; e += 256) Ss[e] = 0.f;
  }
  for (int c = c0; c < c1; ++c) {
    const int t0 = c * C;
    const int L = min(C, Tb - t0);
    __syncthreads();
    for (int r = tid; r < 2 * C; r += 256) {  // rows r < C: queries, C <= r < 2C: keys
      const bool isq = r < C;
      const int t = isq ? r : r - C;
      if (MODE == 1 && isq) continue;
      load_norm_row<IN_BF16>(isq ? q : k, row0 + (int64_t)(t0 + t) * rstep, t < L, p, (isq ? qh : kh) + t * p);
    }
    for (int e = tid; e < C * dv; e += 256)
      vv[e] = e / dv < L ? load_as_f32<IN_BF16>(v, (row0 + (int64_t)(t0 + e / dv) * rstep) * dv + e % dv) : 0.f;
    __syncthreads();
    if (MODE == 0) {
      for (int t = tid; t < L; t += 256) {  // denominator: psi(q_t) . Z + intra weights
        const float* qt = qh + t * p;
        float d = 0.f;
        for (int f = 0; f < n; ++f) d += feat_val(F, tab[f], qt) * Zs[f];
        for (int s = 0; s <= t; ++s) d += feat_weight(F, qt, kh + s * p);
        den[t] = d;
      }
      __syncthreads();
      for (int e = tid; e < L * dv; e += 256) {
        const int t = e / dv, dd = e % dv;
        const float* qt = qh + t * p;
        float num = 0.f;
        for (int f = 0; f < n; ++f) num += feat_val(F, tab[f], qt) * Ss[f * dv + dd];
        for (int s = 0; s <= t; ++s) num += feat_weight(F, qt, kh + s * p) * vv[s * dv + dd];
        const float dn = den[t];
        store_from_f32<OUT_BF16>(o, (row0 + (int64_t)(t0 + t) * rstep) * dv + dd, dn > 0.f ? num / dn : 0.f);
      }
      __syncthreads();
    }
    for (int e = tid; e < n * dv + n; e += 256) {  // S += psi(K_c)^T V_c, Z += psi(K_c)^T 1
      const bool isz = e >= n * dv;
      const int f = isz ? e - n * dv : e / dv, dd = isz ? 0 : e % dv;
      float acc = 0.f;
      for (int t = 0; t < L; ++t) {
        const float ps = feat_val(F, tab[f], kh + t * p);
        acc += isz ? ps : ps * vv[t * dv + dd];
      }
      Ss[e] += acc;
    }
  }
  __syncthreads();
  if (MODE == 1) {
    float* dst = ws + (bh * (nseg - 1) + seg) * state_floats;
    for (int e = tid; e < n * dv + n; e += 256) dst[e] = Ss[e];
  }
  if (MODE == 0 && s_out != nullptr && seg == nblk_per_bh - 1) {
    for (int e = tid; e < n * dv; e += 256) s_out[bh * n * dv + e] = Ss[e];
    for (int f = tid; f < n; f += 256) z_out[bh * n + f] = Zs[f];
  }
}

hipError_t launch_scan(float* ws, int BH, int nslots, int64_t E, hipStream_t st);

template <bool IN_BF16>
static hipError_t launch_family_chunked_t(const void* q, const void* k, const void* v, void* o, bool o_bf16,
                                          int B, int H, int T, int p, int dv, int C, int fam, int g,
                                          const SegPlan& plan, float* ws, float* s_out, float* z_out,
                                          SeqLayout lay, hipStream_t st) {
  const Feat F = make_feat(p, fam, g);
  const int BH = B * H;
  const size_t lds = family_chunked_lds_bytes(p, dv, C, fam, g);
  const int64_t sf = family_state_floats(p, dv, fam, g);
  hipError_t e;
  if (plan.nseg > 1) {
    auto ks = family_chunked_kernel<IN_BF16, false, 1>;
    if ((e = hipFuncSetAttribute((const void*)ks, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds)) != hipSuccess)
      return e;
    ks<<<dim3((unsigned)(BH * (plan.nseg - 1))), dim3(256), lds, st>>>(q, k, v, nullptr, T, p, dv, C, F, plan.nseg,
                                                                       plan.cps, plan.nseg - 1, ws, sf, nullptr,
                                                                       nullptr, lay, H);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = launch_scan(ws, BH, plan.nseg - 1, sf, st)) != hipSuccess) return e;
  }
  auto kf = o_bf16 ? family_chunked_kernel<IN_BF16, true, 0> : family_chunked_kernel<IN_BF16, false, 0>;
  if ((e = hipFuncSetAttribute((const void*)kf, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds)) != hipSuccess)
    return e;
  kf<<<dim3((unsigned)(BH * plan.nseg)), dim3(256), lds, st>>>(q, k, v, o, T, p, dv, C, F, plan.nseg, plan.cps,
                                                              plan.nseg, ws, sf, s_out, z_out, lay, H);
  return hipGetLastError();
}

hipError_t launch_family_chunked(const void* q, const void* k, const void* v, bool in_bf16, void* o,
                                 bool o_bf16, int B, int H, int T, int p, int dv, int C, int fam, int g,
                                 const SegPlan& plan, float* ws, float* s_out, float* z_out, SeqLayout lay,
                                 hipStream_t st) {
  if (in_bf16)
    return launch_family_chunked_t<true>(q, k, v, o, o_bf16, B, H, T, p, dv, C, fam, g, plan, ws, s_out, z_out,
                                         lay, st);
  return launch_family_chunked_t<false>(q, k, v, o, o_bf16, B, H, T, p, dv, C, fam, g, plan, ws, s_out, z_out,
                                        lay, st);
}

// ---------------------------------------------------------------------------- quadratic
// One workgroup per (query block of 32, b*h), key blocks of 32 staged in LDS, longest
// query blocks first over all sequences.
constexpr int FQ_BQ = 32, FQ_BK = 32;

template <bool IN_BF16, bool OUT_BF16>
__global__ __launch_bounds__(256) void family_quadratic_kernel(const void* __restrict__ q, const void* __restrict__ k,
                                                               const void* __restrict__ v, void* __restrict__ o,
                                                               int T, int p, int dv, Feat F, SeqLayout lay, int H) {
  extern __shared__ float sm[];
  float* qh = sm;                  // [BQ][p]
  float* kh = qh + FQ_BQ * p;      // [BK][p]
  float* vv = kh + FQ_BK * p;      // [BK][dv]
  float* w = vv + FQ_BK * dv;      // [BQ][BK + 1]
  const int tid = threadIdx.x;
  const int nqb = (T + FQ_BQ - 1) / FQ_BQ;
  const int nbh = (int)(gridDim.x / nqb);
  const int64_t bh = blockIdx.x % nbh;
  const int tq0 = (nqb - 1 - (int)(blockIdx.x / nbh)) * FQ_BQ;
  // rows of this sequence: row0 + t * stp for t < len (padded: bh T + t, len = T)
  int64_t row0;
  int stp, len;
  seq_rows_of(lay, bh, H, T, row0, stp, len);
  if (tq0 >= len) return;  // the whole workgroup: no query of this block exists
  auto row = [&](int t) { return row0 + (int64_t)t * stp; };
  for (int r = tid; r < FQ_BQ; r += 256) load_norm_row<IN_BF16>(q, row(tq0 + r), tq0 + r < len, p, qh + r * p);
  const int qi = tid >> 3, dsub = tid & 7;  // thread owns query qi, columns dsub + 8u
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float dacc = 0.f;
  for (int kb0 = 0; kb0 <= tq0; kb0 += FQ_BK) {
    __syncthreads();
    for (int r = tid; r < FQ_BK; r += 256) load_norm_row<IN_BF16>(k, row(kb0 + r), kb0 + r < len, p, kh + r * p);
    for (int e = tid; e < FQ_BK * dv; e += 256)
      vv[e] = kb0 + e / dv < len ? load_as_f32<IN_BF16>(v, row(kb0 + e / dv) * dv + e % dv) : 0.f;
    __syncthreads();
    for (int e = tid; e < FQ_BQ * FQ_BK; e += 256) {
      const int i = e / FQ_BK, j = e % FQ_BK;
      w[i * (FQ_BK + 1) + j] = (kb0 + j <= tq0 + i) ? feat_weight(F, qh + i * p, kh + j * p) : 0.f;
    }
    __syncthreads();
    for (int j = 0; j < FQ_BK; ++j) {
      const float wij = w[qi * (FQ_BK + 1) + j];
      dacc += wij;
      for (int u = 0; u < 8; ++u) {
        const int dd = dsub + 8 * u;
        if (dd < dv) acc[u] += wij * vv[j * dv + dd];
      }
    }
  }
  const int t = tq0 + qi;
  if (t < len)
    for (int u = 0; u < 8; ++u) {
      const int dd = dsub + 8 * u;
      if (dd < dv) store_from_f32<OUT_BF16>(o, row(t) * dv + dd, dacc > 0.f ? acc[u] / dacc : 0.f);
    }
}

hipError_t launch_family_quadratic(const void* q, const void* k, const void* v, bool in_bf16, void* o, bool o_bf16,
                                   int B, int H, int T, int p, int dv, int fam, int g, hipStream_t st,
                                   SeqLayout lay) {
  // fam 3: the full map with weights (q_hat . k_hat)^(2g) (order r = g)
  const Feat F = fam == 3 ? make_order(p, g) : make_feat(p, fam, g);
  const size_t lds = 4 * ((size_t)FQ_BQ * p + (size_t)FQ_BK * p + (size_t)FQ_BK * dv + FQ_BQ * (FQ_BK + 1));
  dim3 grid((unsigned)((int64_t)((T + FQ_BQ - 1) / FQ_BQ) * B * H)), block(256);
  if (in_bf16 && o_bf16) family_quadratic_kernel<true, true><<<grid, block, lds, st>>>(q, k, v, o, T, p, dv, F, lay, H);
  else if (in_bf16) family_quadratic_kernel<true, false><<<grid, block, lds, st>>>(q, k, v, o, T, p, dv, F, lay, H);
  else if (o_bf16) family_quadratic_kernel<false, true><<<grid, block, lds, st>>>(q, k, v, o, T, p, dv, F, lay, H);
  else family_quadratic_kernel<false, false><<<grid, block, lds, st>>>(q, k, v, o, T, p, dv, F, lay, H);
  return hipGetLastError();
}

}  // namespace kata
