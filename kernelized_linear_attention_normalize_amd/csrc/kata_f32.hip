// fp32-input kernels: chunked-state forward, segment scan, and the quadratic form, all
// evaluated in fp32 on the vector ALUs (fp32 accuracy; these serve fp32 inputs, the bf16
// inputs run the MFMA kernels).
//
// Source: "Kernelized Linear Attention: Breaking the Capacity Wall with Symmetric Cones"
// (arXiv 2607.17419), arXiv HTML page: chunked-forward paragraph (per-chunk state, the
// inter-chunk prefix as an associative cumulative sum, the local C x C causal block),
// rank-one lift display (psi(u) = u u^T, <psi(a), psi(b)> = (a.b)^2), normalized-readout
// paragraph (explicit denominator), feature-value state display.
#include "kata_device.h"
#include "kata_launch.h"

namespace kata {

int64_t f32_state_floats(int p, int dv) {
  const int64_t n = (int64_t)p * (p + 1) / 2;
  return n * dv + n;
}

// LDS: S[n*dv] Z[n] qh[C*p] kh[C*p] vv[C*dv] den[C] pairs[n] (ints)
size_t f32_chunked_lds_bytes(int p, int dv, int C) {
  const size_t n = (size_t)p * (p + 1) / 2;
  return 4 * (n * dv + n + 2 * (size_t)C * p + (size_t)C * dv + C + n);
}

// Value-column parts of the fp32 chunked forward: 1 when the whole state fits in LDS, 2 when
// only half of the value columns do (each output column is its own ratio with the same
// denominator, so the columns split exactly), 0 when neither fits.
int f32_chunked_parts(int p, int dv, int C) {
  if (f32_chunked_lds_bytes(p, dv, C) <= 160 * 1024) return 1;
  if (dv % 2 == 0 && f32_chunked_lds_bytes(p, dv / 2, C) <= 160 * 1024) return 2;
  return 0;
}

// workspace floats per (sequence-head, segment summary) over all parts
int64_t f32_chunked_state_floats(int p, int dv, int C) {
  const int parts = f32_chunked_parts(p, dv, C);
  return parts > 0 ? parts * f32_state_floats(p, dv / parts) : 0;
}

// MODE 0: forward of one segment starting from its prefix state (or zero); the last
//         segment of a sequence also writes the final state to s_out / z_out if given;
// MODE 1: state summary of one segment (psi(K)^T [V | 1]) written to the workspace.
// The kernel handles value columns col0 .. col0 + dv - 1 of rows ldv wide (v, o and the
// final state S); a part of the columns when the whole state does not fit in LDS.
template <bool OUT_BF16, int MODE>
__global__ __launch_bounds__(256) void chunked_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    void* __restrict__ o, int T, int p, int dv, int C, int nseg, int cps, int nblk_per_bh,
    float* __restrict__ ws, float* __restrict__ s_out, float* __restrict__ z_out,
    SeqLayout lay, int H, int ldv, int col0) {
  extern __shared__ float sm[];
  const int n = p * (p + 1) / 2;
  float* Ss = sm;
  float* Zs = Ss + n * dv;
  float* qh = Zs + n;
  float* kh = qh + C * p;
  float* vv = kh + C * p;
  float* den = vv + C * dv;
  int* pairs = reinterpret_cast<int*>(den + C);
  const int tid = threadIdx.x;
  const int64_t bh = blockIdx.x / nblk_per_bh;
  const int seg = blockIdx.x % nblk_per_bh;
  int64_t row0;
  int rstep, Tb;  // first row, row step, this sequence's rows
  seq_rows_of(lay, bh, H, T, row0, rstep, Tb);
  const int nchunks = (Tb + C - 1) / C;
  const int c0 = seg * cps, c1 = min(nchunks, c0 + cps);
  const int64_t state_floats = (int64_t)n * dv + n;

  for (int f = tid; f < n; f += 256) {
    int i, j;
    packed_ij(f, p, i, j);
    pairs[f] = (i << 16) | j;
  }
  if (MODE == 0 && seg > 0) {  // exclusive prefix of this segment (inclusive scan slot seg-1)
    const float* src = ws + (bh * (nseg - 1) + (seg - 1)) * state_floats;
    for (int e = tid; e < n * dv + n; e += 256) Ss[e] = src[e];
  } else {
    for (int e = tid; e < n * dv + n; e += 256) Ss[e] = 0.f;
  }
  const float* qb = q + row0 * p;
  const float* kb = k + row0 * p;
  const float* vb = v + row0 * ldv + col0;

  for (int c = c0; c < c1; ++c) {
    const int t0 = c * C;
    const int L = min(C, Tb - t0);
    __syncthreads();
    // load + normalise rows: thread r < C handles q row r, C <= r < 2C handles k row r-C
    for (int r = tid; r < 2 * C; r += 256) {
      const bool isq = r < C;
      const int t = isq ? r : r - C;
      if (MODE == 1 && isq) continue;
      float* dst = (isq ? qh : kh) + t * p;
      const float* src = (isq ? qb : kb) + (int64_t)(t0 + t) * rstep * p;
      float ss = 0.f;
      for (int i = 0; i < p; ++i) {
        const float x = t < L ? src[i] : 0.f;
        dst[i] = x;
        ss += x * x;
      }
      const float inv = inv_norm(ss);
      for (int i = 0; i < p; ++i) dst[i] *= inv;
    }
    for (int e = tid; e < C * dv; e += 256) {
      const int t = e / dv;
      vv[e] = t < L ? vb[(int64_t)(t0 + t) * rstep * ldv + e % dv] : 0.f;
    }
    __syncthreads();
    if (MODE == 0) {
      // denominator: psi(q_t)^T Z (state before this chunk) + sum_{s<=t} (q_t . k_s)^2
      for (int t = tid; t < L; t += 256) {
        const float* qt = qh + t * p;
        float d = 0.f;
        for (int f = 0; f < n; ++f) {
          const int i = pairs[f] >> 16, j = pairs[f] & 0xffff;
          d += (i == j ? 1.f : sqrt2f()) * qt[i] * qt[j] * Zs[f];
        }
        for (int s = 0; s <= t; ++s) {
          float a = 0.f;
          for (int i = 0; i < p; ++i) a += qt[i] * kh[s * p + i];
          d += a * a;
        }
        den[t] = d;
      }
      __syncthreads();
      for (int e = tid; e < L * dv; e += 256) {
        const int t = e / dv, dd = e % dv;
        const float* qt = qh + t * p;
        float num = 0.f;
        for (int f = 0; f < n; ++f) {
          const int i = pairs[f] >> 16, j = pairs[f] & 0xffff;
          num += (i == j ? 1.f : sqrt2f()) * qt[i] * qt[j] * Ss[f * dv + dd];
        }
        for (int s = 0; s <= t; ++s) {
          float a = 0.f;
          for (int i = 0; i < p; ++i) a += qt[i] * kh[s * p + i];
          num += a * a * vv[s * dv + dd];
        }
        const float dn = den[t];
        store_from_f32<OUT_BF16>(o, (row0 + (int64_t)(t0 + t) * rstep) * ldv + col0 + dd, dn > 0.f ? num / dn : 0.f);
      }
      __syncthreads();
    }
    // state update: S += psi(K_c)^T V_c, Z += psi(K_c)^T 1
    for (int e = tid; e < n * dv + n; e += 256) {
      const bool isz = e >= n * dv;
      const int f = isz ? e - n * dv : e / dv, dd = isz ? 0 : e % dv;
      const int i = pairs[f] >> 16, j = pairs[f] & 0xffff;
      const float cf = i == j ? 1.f : sqrt2f();
      float acc = 0.f;
      for (int t = 0; t < L; ++t) {
        const float ps = cf * kh[t * p + i] * kh[t * p + j];
        acc += isz ? ps : ps * vv[t * dv + dd];
      }
      Ss[e] += acc;
    }
  }
  if (MODE == 1) {
    __syncthreads();
    float* dst = ws + (bh * (nseg - 1) + seg) * state_floats;
    for (int e = tid; e < n * dv + n; e += 256) dst[e] = Ss[e];
  }
  if (MODE == 0 && s_out != nullptr && seg == nblk_per_bh - 1) {  // S then Z: the decode layout
    __syncthreads();
    for (int e = tid; e < n * dv; e += 256) s_out[(bh * n + e / dv) * ldv + col0 + e % dv] = Ss[e];
    for (int f = tid; f < n; f += 256) z_out[bh * n + f] = Zs[f];
  }
}

hipError_t launch_scan(float* ws, int BH, int nslots, int64_t E, hipStream_t st);

hipError_t launch_chunked_f32(const float* q, const float* k, const float* v, void* o, bool o_bf16,
                              int B, int H, int T, int p, int dv, int C, const SegPlan& plan,
                              float* ws, float* s_out, float* z_out, SeqLayout lay, int passes,
                              hipStream_t st) {
  const int BH = B * H;
  const int parts = f32_chunked_parts(p, dv, C);
  if (parts == 0) return hipErrorInvalidValue;
  const int dvp = dv / parts;
  const size_t lds = f32_chunked_lds_bytes(p, dvp, C);
  const int64_t part_ws = plan.nseg > 1 ? (int64_t)BH * (plan.nseg - 1) * f32_state_floats(p, dvp) : 0;
  hipError_t e;
  if (plan.nseg > 1 && (passes & PASS_SUMMARIES)) {
    auto kfn = chunked_f32_kernel<false, 1>;
    if ((e = hipFuncSetAttribute((const void*)kfn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds)) != hipSuccess)
      return e;
    for (int part = 0; part < parts; ++part) {
      kfn<<<dim3((unsigned)(BH * (plan.nseg - 1))), dim3(256), lds, st>>>(
          q, k, v, nullptr, T, p, dvp, C, plan.nseg, plan.cps, plan.nseg - 1, ws + part * part_ws, nullptr, nullptr,
          lay, H, dv, part * dvp);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
  }
  if (plan.nseg > 1 && (passes & PASS_SCAN))
    for (int part = 0; part < parts; ++part)
      if ((e = launch_scan(ws + part * part_ws, BH, plan.nseg - 1, f32_state_floats(p, dvp), st)) != hipSuccess)
        return e;
  if (!(passes & PASS_SEGMENTS)) return hipSuccess;
  auto kfn = o_bf16 ? chunked_f32_kernel<true, 0> : chunked_f32_kernel<false, 0>;
  if ((e = hipFuncSetAttribute((const void*)kfn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds)) != hipSuccess)
    return e;
  for (int part = 0; part < parts; ++part) {
    kfn<<<dim3((unsigned)(BH * plan.nseg)), dim3(256), lds, st>>>(q, k, v, o, T, p, dvp, C, plan.nseg, plan.cps,
                                                                plan.nseg, ws + part * part_ws, s_out, z_out, lay,
                                                                H, dv, part * dvp);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

// ---------------------------------------------------------------------------- quadratic
// Flash-style causal form in fp32: one workgroup per (query block of 32, b*h); key
// blocks of 32 are staged in LDS; the output accumulates sum_s w_ts [v_s | 1] and is
// divided once at the end. No running maximum is needed: w = (q_hat . k_hat)^2 is in [0, 1].
constexpr int QF_BQ = 32, QF_BK = 32;

template <bool OUT_BF16>
__global__ __launch_bounds__(256) void quadratic_f32_kernel(const float* __restrict__ q,
                                                            const float* __restrict__ k,
                                                            const float* __restrict__ v,
                                                            void* __restrict__ o, int T, int p,
                                                            int dv, SeqLayout lay, int H) {
  extern __shared__ float sm[];
  float* qh = sm;                   // [BQ][p]
  float* kh = qh + QF_BQ * p;       // [BK][p]
  float* vv = kh + QF_BK * p;       // [BK][dv]
  float* w = vv + QF_BK * dv;       // [BQ][BK+1]
  const int tid = threadIdx.x;
  const int nqb = (T + QF_BQ - 1) / QF_BQ;
  const int64_t bh = blockIdx.x / nqb;
  const int qblk = nqb - 1 - (int)(blockIdx.x % nqb);  // longest rows first
  const int tq0 = qblk * QF_BQ;
  // rows of this sequence: row0 + t * stp for t < len (padded: bh T + t, len = T)
  int64_t row0;
  int stp, len;
  seq_rows_of(lay, bh, H, T, row0, stp, len);
  if (tq0 >= len) return;  // the whole workgroup: no query of this block exists
  auto row = [&](int t) { return row0 + (int64_t)t * stp; };
  for (int r = tid; r < QF_BQ; r += 256) {
    float ss = 0.f;
    for (int i = 0; i < p; ++i) {
      const float x = tq0 + r < len ? q[row(tq0 + r) * p + i] : 0.f;
      qh[r * p + i] = x;
      ss += x * x;
    }
    const float inv = inv_norm(ss);
    for (int i = 0; i < p; ++i) qh[r * p + i] *= inv;
  }
  const int qi = tid >> 3, dsub = tid & 7;  // thread owns query qi, columns dsub + 8u
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float dacc = 0.f;
  for (int kb0 = 0; kb0 <= tq0; kb0 += QF_BK) {
    __syncthreads();
    for (int r = tid; r < QF_BK; r += 256) {
      float ss = 0.f;
      for (int i = 0; i < p; ++i) {
        const float x = kb0 + r < len ? k[row(kb0 + r) * p + i] : 0.f;
        kh[r * p + i] = x;
        ss += x * x;
      }
      const float inv = inv_norm(ss);
      for (int i = 0; i < p; ++i) kh[r * p + i] *= inv;
    }
    for (int e = tid; e < QF_BK * dv; e += 256)
      vv[e] = kb0 + e / dv < len ? v[row(kb0 + e / dv) * dv + e % dv] : 0.f;
    __syncthreads();
    for (int e = tid; e < QF_BQ * QF_BK; e += 256) {
      const int i = e / QF_BK, j = e % QF_BK;
      float a = 0.f;
      for (int c = 0; c < p; ++c) a += qh[i * p + c] * kh[j * p + c];
      w[i * (QF_BK + 1) + j] = (kb0 + j <= tq0 + i) ? a * a : 0.f;
    }
    __syncthreads();
    for (int j = 0; j < QF_BK; ++j) {
      const float wij = w[qi * (QF_BK + 1) + j];
      dacc += wij;
      for (int u = 0; u < 8; ++u) {
        const int dd = dsub + 8 * u;
        if (dd < dv) acc[u] += wij * vv[j * dv + dd];
      }
    }
  }
  const int t = tq0 + qi;
  if (t < len) {
    for (int u = 0; u < 8; ++u) {
      const int dd = dsub + 8 * u;
      if (dd < dv) store_from_f32<OUT_BF16>(o, row(t) * dv + dd, dacc > 0.f ? acc[u] / dacc : 0.f);
    }
  }
}

hipError_t launch_quadratic_f32(const float* q, const float* k, const float* v, void* o,
                                bool o_bf16, int B, int H, int T, int p, int dv, hipStream_t st, SeqLayout lay) {
  const size_t lds = 4 * ((size_t)QF_BQ * p + (size_t)QF_BK * p + (size_t)QF_BK * dv + QF_BQ * (QF_BK + 1));
  dim3 grid((unsigned)((int64_t)((T + QF_BQ - 1) / QF_BQ) * B * H)), block(256);
  if (o_bf16) quadratic_f32_kernel<true><<<grid, block, lds, st>>>(q, k, v, o, T, p, dv, lay, H);
  else quadratic_f32_kernel<false><<<grid, block, lds, st>>>(q, k, v, o, T, p, dv, lay, H);
  return hipGetLastError();
}

}  // namespace kata
