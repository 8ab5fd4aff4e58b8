// Gradients of the causal KATA forward in the flash-style (quadratic) form, for the full map
// and the reduced PSD families, on VALU kernels (fp32 arithmetic; fp32 or bf16 inputs).
//
// The pages describe no backward pass; this is the calculus of the forward they define
// ("Kernelized Linear Attention: Breaking the Capacity Wall with Symmetric Cones", arXiv
// 2607.17419, arXiv HTML page: normalized-readout paragraph, rank-one lift display, reduced
// PSD families paragraph). With a_ts,ab = q_hat_t,a . k_hat_s,b over the family's block pairs,
// w_ts = sum a^2 (s <= t), D_t = sum_s w_ts, o_t = sum_s w_ts v_s / D_t, g_t = dL/do_t and
// delta_t = g_t . o_t:
//   dv_s = sum_{t>=s} (w_ts / D_t) g_t,    dw_ts = (g_t . v_s - delta_t) / D_t,
//   dq_hat_t,a = sum_s sum_b 2 dw_ts a_ts,ab k_hat_s,b,   dk_hat_s,b = sum_t sum_a 2 dw_ts a_ts,ab q_hat_t,a,
//   du = (du_hat - u_hat (u_hat . du_hat)) / |u|   (zero rows get zero gradients).
// Kernel 1 (query blocks) recomputes o_t, stores D_t and delta_t, and accumulates dq; kernel 2
// (key blocks) reads them back and accumulates dk and dv. O(T^2) work: a parity-grade
// reference for training, not a tuned kernel.
#include "kata_device.h"
#include "kata_launch.h"

namespace kata {

namespace {

constexpr int BW_B = 32;        // rows per block (queries or keys)
constexpr int BW_MAXPR = 16;    // block pairs held in LDS

struct BwFeat {
  int npr, m;             // block pairs, block width
  int8_t pa[BW_MAXPR];    // query block of pair r
  int8_t pb[BW_MAXPR];    // key block of pair r
};

BwFeat make_bw(int p, int fam, int g) {
  BwFeat F{};
  F.m = p / g;
  F.npr = 0;
  for (int a = 0; a < g; ++a)
    for (int b = 0; b < g; ++b)
      if (fam == 1 || a == b) {  // Sigma g: all pairs; M g and the full map: a = b
        F.pa[F.npr] = (int8_t)a;
        F.pb[F.npr] = (int8_t)b;
        ++F.npr;
      }
  return F;
}

// normalise a row into dst; returns |u| (0 for a zero row, whose dst is zero)
template <bool IN_BF16>
__device__ float bw_load_row(const void* src, int64_t row, bool valid, int p, float* dst) {
  float ss = 0.f;
  for (int i = 0; i < p; ++i) {
    const float x = valid ? load_as_f32<IN_BF16>(src, row * p + i) : 0.f;
    dst[i] = x;
    ss += x * x;
  }
  const float inv = inv_norm(ss);
  for (int i = 0; i < p; ++i) dst[i] *= inv;
  return ss > 0.f ? sqrtf(ss) : 0.f;
}

// dots[r][i][j] = q_hat_i,a_r . k_hat_j,b_r and w[i][j] = sum_r dots^2 (0 where masked)
__device__ void bw_dots(const BwFeat& F, const float* qh, const float* kh, int p, float* dots, float* w,
                        int tq0, int tk0, int T) {
  for (int e = threadIdx.x; e < BW_B * BW_B; e += 256) {
    const int i = e / BW_B, j = e % BW_B;
    const bool ok = tk0 + j <= tq0 + i && tq0 + i < T && tk0 + j < T;
    float ws = 0.f;
    for (int r = 0; r < F.npr; ++r) {
      float d = 0.f;
      const float* qa = qh + i * p + F.pa[r] * F.m;
      const float* kb = kh + j * p + F.pb[r] * F.m;
      for (int c = 0; c < F.m; ++c) d += qa[c] * kb[c];
      d = ok ? d : 0.f;
      dots[(r * BW_B + i) * (BW_B + 1) + j] = d;
      ws += d * d;
    }
    w[i * (BW_B + 1) + j] = ws;
  }
}

}  // namespace

// ---------------------------------------------------------------------------- kernel 1
// LDS: qh[B][p] gq[B][dv] kh[B][p] vv[B][dv] dots[npr][B][B+1] w[B][B+1] D[B] delta[B] qn[B]
template <bool IN_BF16>
__global__ __launch_bounds__(256) void bwd_query_kernel(const void* __restrict__ q, const void* __restrict__ k,
                                                        const void* __restrict__ v, const void* __restrict__ go,
                                                        int T, int p, int dv, BwFeat F, float* __restrict__ ws,
                                                        float* __restrict__ dq, SeqLayout lay, int H) {
  extern __shared__ float sm[];
  float* qh = sm;
  float* gq = qh + BW_B * p;
  float* kh = gq + BW_B * dv;
  float* vv = kh + BW_B * p;
  float* dots = vv + BW_B * dv;
  float* w = dots + F.npr * BW_B * (BW_B + 1);
  float* Ds = w + BW_B * (BW_B + 1);
  float* dl = Ds + BW_B;
  float* qn = dl + BW_B;
  const int tid = threadIdx.x;
  const int nqb = (T + BW_B - 1) / BW_B;
  const int64_t bh = blockIdx.x / nqb;
  const int tq0 = (blockIdx.x % nqb) * BW_B;
  // rows of this sequence: row0 + t * stp for t < len (padded: bh T + t, len = T)
  int64_t row0;
  int stp, len;
  seq_rows_of(lay, bh, H, T, row0, stp, len);
  if (tq0 >= len) return;  // the whole workgroup: no query of this block exists
  auto row = [&](int t) { return row0 + (int64_t)t * stp; };
  const int qi = tid >> 3, sub = tid & 7;  // thread: query qi, columns / components sub + 8u
  if (tid < BW_B) qn[tid] = bw_load_row<IN_BF16>(q, row(tq0 + tid), tq0 + tid < len, p, qh + tid * p);
  for (int e = tid; e < BW_B * dv; e += 256)
    gq[e] = tq0 + e / dv < len ? load_as_f32<IN_BF16>(go, row(tq0 + e / dv) * dv + e % dv) : 0.f;
  // ---- forward recompute: N_t, D_t
  float num[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  for (int tk0 = 0; tk0 <= tq0; tk0 += BW_B) {
    __syncthreads();
    if (tid < BW_B) bw_load_row<IN_BF16>(k, row(tk0 + tid), tk0 + tid < len, p, kh + tid * p);
    for (int e = tid; e < BW_B * dv; e += 256)
      vv[e] = tk0 + e / dv < len ? load_as_f32<IN_BF16>(v, row(tk0 + e / dv) * dv + e % dv) : 0.f;
    __syncthreads();
    bw_dots(F, qh, kh, p, dots, w, tq0, tk0, len);
    __syncthreads();
    for (int j = 0; j < BW_B; ++j) {
      const float wij = w[qi * (BW_B + 1) + j];
      den += wij;
      for (int u = 0; u < 8; ++u)
        if (sub + 8 * u < dv) num[u] += wij * vv[j * dv + sub + 8 * u];
    }
  }
  // delta_t = g_t . o_t: the 8 threads of a query hold disjoint columns
  const float inv = den > 0.f ? 1.f / den : 0.f;
  float part = 0.f;
  for (int u = 0; u < 8; ++u)
    if (sub + 8 * u < dv) part += gq[qi * dv + sub + 8 * u] * num[u] * inv;
  part = group_sum<8>(part);
  __syncthreads();
  if (sub == 0) {
    Ds[qi] = den;
    dl[qi] = part;
    if (tq0 + qi < len) {
      ws[row(tq0 + qi) * 2] = den;
      ws[row(tq0 + qi) * 2 + 1] = part;
    }
  }
  // ---- gradient pass: dq_hat
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};  // components sub + 8u
  for (int tk0 = 0; tk0 <= tq0; tk0 += BW_B) {
    __syncthreads();
    if (tid < BW_B) bw_load_row<IN_BF16>(k, row(tk0 + tid), tk0 + tid < len, p, kh + tid * p);
    for (int e = tid; e < BW_B * dv; e += 256)
      vv[e] = tk0 + e / dv < len ? load_as_f32<IN_BF16>(v, row(tk0 + e / dv) * dv + e % dv) : 0.f;
    __syncthreads();
    bw_dots(F, qh, kh, p, dots, w, tq0, tk0, len);
    __syncthreads();
    for (int e = tid; e < BW_B * BW_B; e += 256) {  // w <- dw
      const int i = e / BW_B, j = e % BW_B;
      float gv = 0.f;
      for (int d = 0; d < dv; ++d) gv += gq[i * dv + d] * vv[j * dv + d];
      const float D = Ds[i];
      const bool ok = tk0 + j <= tq0 + i;
      w[i * (BW_B + 1) + j] = ok && D > 0.f ? (gv - dl[i]) / D : 0.f;
    }
    __syncthreads();
    for (int u = 0; u < 8; ++u) {
      const int c = sub + 8 * u;
      if (c >= p) break;
      const int a = c / F.m, ci = c % F.m;
      float s = 0.f;
      for (int r = 0; r < F.npr; ++r) {
        if (F.pa[r] != a) continue;
        const float* dr = dots + (r * BW_B + qi) * (BW_B + 1);
        const int kc = F.pb[r] * F.m + ci;
        for (int j = 0; j < BW_B; ++j) s += 2.f * w[qi * (BW_B + 1) + j] * dr[j] * kh[j * p + kc];
      }
      acc[u] += s;
    }
  }
  // dq = (dq_hat - q_hat (q_hat . dq_hat)) / |q|
  float pr = 0.f;
  for (int u = 0; u < 8; ++u)
    if (sub + 8 * u < p) pr += acc[u] * qh[qi * p + sub + 8 * u];
  pr = group_sum<8>(pr);
  const float nq = qn[qi];
  if (tq0 + qi < len)
    for (int u = 0; u < 8; ++u) {
      const int c = sub + 8 * u;
      if (c < p) dq[row(tq0 + qi) * p + c] = nq > 0.f ? (acc[u] - qh[qi * p + c] * pr) / nq : 0.f;
    }
}

// ---------------------------------------------------------------------------- kernel 2
// LDS: kh[B][p] vv[B][dv] qh[B][p] gq[B][dv] dots[npr][B][B+1] w[B][B+1] P[B][B+1] D[B] delta[B] kn[B]
template <bool IN_BF16>
__global__ __launch_bounds__(256) void bwd_key_kernel(const void* __restrict__ q, const void* __restrict__ k,
                                                      const void* __restrict__ v, const void* __restrict__ go, int T,
                                                      int p, int dv, BwFeat F, const float* __restrict__ ws,
                                                      float* __restrict__ dk, float* __restrict__ dvo, SeqLayout lay,
                                                      int H) {
  extern __shared__ float sm[];
  float* kh = sm;
  float* vv = kh + BW_B * p;
  float* qh = vv + BW_B * dv;
  float* gq = qh + BW_B * p;
  float* dots = gq + BW_B * dv;
  float* w = dots + F.npr * BW_B * (BW_B + 1);
  float* P = w + BW_B * (BW_B + 1);
  float* Ds = P + BW_B * (BW_B + 1);
  float* dl = Ds + BW_B;
  float* kn = dl + BW_B;
  const int tid = threadIdx.x;
  const int nkb = (T + BW_B - 1) / BW_B;
  const int64_t bh = blockIdx.x / nkb;
  const int tk0 = (blockIdx.x % nkb) * BW_B;
  int64_t row0;
  int stp, len;
  seq_rows_of(lay, bh, H, T, row0, stp, len);
  if (tk0 >= len) return;  // the whole workgroup: no key of this block exists
  auto row = [&](int t) { return row0 + (int64_t)t * stp; };
  const int sj = tid >> 3, sub = tid & 7;  // thread: key sj, columns / components sub + 8u
  if (tid < BW_B) kn[tid] = bw_load_row<IN_BF16>(k, row(tk0 + tid), tk0 + tid < len, p, kh + tid * p);
  for (int e = tid; e < BW_B * dv; e += 256)
    vv[e] = tk0 + e / dv < len ? load_as_f32<IN_BF16>(v, row(tk0 + e / dv) * dv + e % dv) : 0.f;
  float gvs[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};  // dv_s, columns sub + 8u
  float gks[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};  // dk_hat_s, components sub + 8u
  for (int tq0 = tk0; tq0 < len; tq0 += BW_B) {
    __syncthreads();
    if (tid < BW_B) {
      const bool ok = tq0 + tid < len;
      bw_load_row<IN_BF16>(q, row(tq0 + tid), ok, p, qh + tid * p);
      Ds[tid] = ok ? ws[row(tq0 + tid) * 2] : 0.f;
      dl[tid] = ok ? ws[row(tq0 + tid) * 2 + 1] : 0.f;
    }
    for (int e = tid; e < BW_B * dv; e += 256)
      gq[e] = tq0 + e / dv < len ? load_as_f32<IN_BF16>(go, row(tq0 + e / dv) * dv + e % dv) : 0.f;
    __syncthreads();
    bw_dots(F, qh, kh, p, dots, w, tq0, tk0, len);  // dots[r][t][s], w[t][s]
    __syncthreads();
    for (int e = tid; e < BW_B * BW_B; e += 256) {
      const int i = e / BW_B, j = e % BW_B;  // query i, key j
      float gv = 0.f;
      for (int d = 0; d < dv; ++d) gv += gq[i * dv + d] * vv[j * dv + d];
      const float D = Ds[i];
      const float inv = D > 0.f ? 1.f / D : 0.f;
      P[i * (BW_B + 1) + j] = w[i * (BW_B + 1) + j] * inv;
      w[i * (BW_B + 1) + j] = tk0 + j <= tq0 + i ? (gv - dl[i]) * inv : 0.f;  // dw
    }
    __syncthreads();
    for (int u = 0; u < 8; ++u) {
      const int d = sub + 8 * u;
      if (d < dv)
        for (int i = 0; i < BW_B; ++i) gvs[u] += P[i * (BW_B + 1) + sj] * gq[i * dv + d];
    }
    for (int u = 0; u < 8; ++u) {
      const int c = sub + 8 * u;
      if (c >= p) break;
      const int b = c / F.m, ci = c % F.m;
      float s = 0.f;
      for (int r = 0; r < F.npr; ++r) {
        if (F.pb[r] != b) continue;
        const int qc = F.pa[r] * F.m + ci;
        for (int i = 0; i < BW_B; ++i)
          s += 2.f * w[i * (BW_B + 1) + sj] * dots[(r * BW_B + i) * (BW_B + 1) + sj] * qh[i * p + qc];
      }
      gks[u] += s;
    }
  }
  float pr = 0.f;
  for (int u = 0; u < 8; ++u)
    if (sub + 8 * u < p) pr += gks[u] * kh[sj * p + sub + 8 * u];
  pr = group_sum<8>(pr);
  const float nk = kn[sj];
  if (tk0 + sj < len) {
    for (int u = 0; u < 8; ++u) {
      const int c = sub + 8 * u;
      if (c < p) dk[row(tk0 + sj) * p + c] = nk > 0.f ? (gks[u] - kh[sj * p + c] * pr) / nk : 0.f;
      const int d = sub + 8 * u;
      if (d < dv) dvo[row(tk0 + sj) * dv + d] = gvs[u];
    }
  }
}

int bwd_pairs(int p, int fam, int g) { return make_bw(p, fam, g).npr; }

hipError_t launch_quadratic_bwd(const void* q, const void* k, const void* v, const void* go, bool in_bf16, int B,
                                int H, int T, int p, int dv, int fam, int g, float* ws, float* dq, float* dk,
                                float* dvo, hipStream_t st, SeqLayout lay) {
  const BwFeat F = make_bw(p, fam, g);
  const int64_t BH = (int64_t)B * H;
  const int nb = (T + BW_B - 1) / BW_B;
  const size_t ldsq =
      4 * ((size_t)BW_B * (2 * p + 2 * dv) + (size_t)(F.npr + 1) * BW_B * (BW_B + 1) + 3 * BW_B);
  const size_t ldsk =
      4 * ((size_t)BW_B * (2 * p + 2 * dv) + (size_t)(F.npr + 2) * BW_B * (BW_B + 1) + 3 * BW_B);
  hipError_t e;
  auto k1 = in_bf16 ? bwd_query_kernel<true> : bwd_query_kernel<false>;
  auto k2 = in_bf16 ? bwd_key_kernel<true> : bwd_key_kernel<false>;
  if ((e = hipFuncSetAttribute((const void*)k1, hipFuncAttributeMaxDynamicSharedMemorySize, (int)ldsq)) != hipSuccess)
    return e;
  if ((e = hipFuncSetAttribute((const void*)k2, hipFuncAttributeMaxDynamicSharedMemorySize, (int)ldsk)) != hipSuccess)
    return e;
  k1<<<dim3((unsigned)(BH * nb)), dim3(256), ldsq, st>>>(q, k, v, go, T, p, dv, F, ws, dq, lay, H);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  k2<<<dim3((unsigned)(BH * nb)), dim3(256), ldsk, st>>>(q, k, v, go, T, p, dv, F, ws, dk, dvo, lay, H);
  return hipGetLastError();
}

}  // namespace kata
