// O(T) chunked-state gradients of the causal full-map forward (fp32 VALU kernels).
//
// Source: the forward of "Kernelized Linear Attention: Breaking the Capacity Wall with
// Symmetric Cones" (arXiv 2607.17419), HTML page: feature-value state display (S_t, Z_t),
// normalized-readout paragraph (o_t = psi(q_t)^T S_t / psi(q_t)^T Z_t), chunked-forward
// paragraph (additive chunk states, prefix by an associative scan). The pages give no
// backward pass; this is its calculus in the state form. With q_hat, k_hat the unit rows,
// D_t = psi(q_hat_t)^T Z_t, delta_t = g_t . o_t, a_t = g_t / D_t, b_t = -delta_t / D_t:
//   dpsi(q_hat_t) = S_t a_t + Z_t b_t                         (forward-time state, s <= t)
//   R_s = sum_{t>=s} psi(q_hat_t) a_t^T,  r_s = sum_{t>=s} psi(q_hat_t) b_t   (reverse time)
//   dpsi(k_hat_s) = R_s v_s + r_s,   dv_s = R_s^T psi(k_hat_s),
// and through the lift, J^T x for u: (2 x_ii u_i + sqrt(2) sum_{j != i} x_ij u_j)_i, then the
// projection onto the tangent of the unit sphere, du = (du_hat - u_hat (u_hat . du_hat)) / |u|.
// Inside a chunk the pairs use the weight identity: the contribution of key s to query t is
// e_ts = (v_s . a_t + b_t) 2 (q_hat_t . k_hat_s) times k_hat_s (to dq_hat_t) or q_hat_t (to
// dk_hat_s), and w_ts a_t to dv_s. Across chunks the states carry the rest:
//   mode FSUM: [S | Z] summary of a segment          (segments 0 .. nseg - 2)
//   mode FDQ : forward-time pass from the exclusive prefix: D_t and delta_t to stats, dq
//   mode RSUM: [R | r] summary of a segment           (segments 1 .. nseg - 1)
//   mode RDK : reverse-time pass from the exclusive suffix: dk, dv
// Summaries are scanned in place like the forward's (reverse summaries in reversed slot
// order, so the inclusive scan yields suffixes). One workgroup of 256 threads per
// (b, h, segment), the state in LDS in packed order.
#include "kata_device.h"
#include "kata_launch.h"

namespace kata {

enum : int { CB_FSUM = 0, CB_FDQ = 1, CB_RSUM = 2, CB_RDK = 3 };

// LDS floats: state n (dv + 1), pairs n, q_hat / k_hat / dq_hat C p each, v / g / a C dv each,
// b / D / |q| / |k| C each, w / e C^2 each
size_t chunked_bwd_lds_bytes(int p, int dv, int C) {
  const size_t n = (size_t)p * (p + 1) / 2;
  return 4 * (n * (dv + 1) + n + 3 * (size_t)C * p + 3 * (size_t)C * dv + 4 * (size_t)C + 2 * (size_t)C * C);
}
int64_t chunked_bwd_state_floats(int p, int dv) {
  const int64_t n = (int64_t)p * (p + 1) / 2;
  return (n * dv + n + 3) / 4 * 4;
}

template <bool IN_BF16, int MODE>
__global__ __launch_bounds__(256) void chunked_bwd_kernel(const void* __restrict__ q, const void* __restrict__ k,
                                                          const void* __restrict__ v, const void* __restrict__ go,
                                                          int T, int p, int dv, int C, int nseg, int cps,
                                                          int nblk_per_bh, float* __restrict__ fsum,
                                                          float* __restrict__ rsum, int64_t sf,
                                                          float* __restrict__ stats, float* __restrict__ dq,
                                                          float* __restrict__ dk, float* __restrict__ dvo,
                                                          SeqLayout lay, int H) {
  extern __shared__ float sm[];
  const int n = p * (p + 1) / 2;
  float* St = sm;                 // [n][dv] then [n]: S | Z or R | r
  float* Zt = St + n * dv;
  int* pairs = reinterpret_cast<int*>(Zt + n);
  float* qh = reinterpret_cast<float*>(pairs + n);
  float* kh = qh + C * p;
  float* dh = kh + C * p;         // dq_hat or dk_hat of the chunk
  float* vv = dh + C * p;
  float* gg = vv + C * dv;
  float* aa = gg + C * dv;        // a_t (and, first, g_t o_t in FDQ)
  float* bb = aa + C * dv;
  float* dd = bb + C;             // D_t
  float* qn = dd + C;             // |q_t|
  float* kn = qn + C;             // |k_s|
  float* W = kn + C;              // w_ts
  float* E = W + C * C;           // e_ts
  const int tid = threadIdx.x;
  const int64_t bh = blockIdx.x / nblk_per_bh;
  const int seg = (int)(blockIdx.x % nblk_per_bh) + (MODE == CB_RSUM ? 1 : 0);
  // rows of this sequence: row0 + t * stp for t < Tb (padded: bh T + t, Tb = T); the plan is
  // that of T, so the segments past a shorter sequence's end are empty (zero summaries)
  int64_t row0;
  int stp, Tb;
  seq_rows_of(lay, bh, H, T, row0, stp, Tb);
  auto row = [&](int t) { return row0 + (int64_t)t * stp; };
  const int nchunks = (Tb + C - 1) / C;
  const int c0 = seg * cps, c1 = min(nchunks, c0 + cps);
  const float r2 = 1.41421356237309515f;

  for (int f = tid; f < n; f += 256) {
    int i, j;
    packed_ij(f, p, i, j);
    pairs[f] = (i << 16) | j;
  }
  const float* init = nullptr;  // exclusive prefix (FDQ) or suffix (RDK) of this segment
  if (MODE == CB_FDQ && seg > 0) init = fsum + (bh * (nseg - 1) + (seg - 1)) * sf;
  if (MODE == CB_RDK && seg < nseg - 1) init = rsum + (bh * (nseg - 1) + (nseg - 2 - seg)) * sf;
  for (int e = tid; e < n * dv + n; e += 256) St[e] = init ? init[e] : 0.f;

  const bool fwd_order = MODE == CB_FSUM || MODE == CB_FDQ;
  for (int ci = 0; ci < c1 - c0; ++ci) {
    const int c = fwd_order ? c0 + ci : c1 - 1 - ci;
    const int t0 = c * C;
    const int L = min(C, Tb - t0);
    __syncthreads();
    // rows of the chunk: normalised q and k with their norms, v, g; rows >= L are zero
    const bool need_q = MODE != CB_FSUM, need_k = MODE != CB_RSUM, need_v = MODE != CB_RSUM;
    for (int r = tid; r < 2 * C; r += 256) {
      const bool isq = r < C;
      const int t = isq ? r : r - C;
      if ((isq && !need_q) || (!isq && !need_k)) continue;
      float* dst = (isq ? qh : kh) + t * p;
      float ss = 0.f;
      for (int i = 0; i < p; ++i) {
        const float x = t < L ? load_as_f32<IN_BF16>(isq ? q : k, row(t0 + t) * p + i) : 0.f;
        dst[i] = x;
        ss += x * x;
      }
      const float inv = inv_norm(ss);
      for (int i = 0; i < p; ++i) dst[i] *= inv;
      (isq ? qn : kn)[t] = ss > 0.f ? sqrtf(ss) : 0.f;
    }
    for (int e = tid; e < C * dv; e += 256) {
      const int t = e / dv;
      const int64_t gi = row(t0 + t) * dv + e % dv;
      if (need_v) vv[e] = t < L ? load_as_f32<IN_BF16>(v, gi) : 0.f;
      if (MODE != CB_FSUM) gg[e] = t < L ? load_as_f32<IN_BF16>(go, gi) : 0.f;
    }
    if (MODE == CB_RSUM || MODE == CB_RDK) {  // D_t and delta_t from the forward-time pass
      for (int t = tid; t < C; t += 256) {
        float D = 0.f, dl = 0.f;
        if (t < L) {
          D = stats[row(t0 + t) * 2];
          dl = stats[row(t0 + t) * 2 + 1];
        }
        const float inv = D > 0.f ? 1.f / D : 0.f;
        dd[t] = inv;  // here: 1 / D_t
        bb[t] = -dl * inv;
      }
    }
    __syncthreads();
    if (MODE == CB_RSUM || MODE == CB_RDK) {
      for (int e = tid; e < C * dv; e += 256) aa[e] = gg[e] * dd[e / dv];
      __syncthreads();
    }

    if (MODE == CB_FDQ) {
      // D_t = psi(q_t)^T Z + sum_{s<=t} w_ts; w_ts of the chunk
      for (int e = tid; e < C * C; e += 256) {
        const int t = e / C, s = e % C;
        float a = 0.f;
        if (t < L && s <= t)
          for (int i = 0; i < p; ++i) a += qh[t * p + i] * kh[s * p + i];
        W[e] = a * a;
        E[e] = a;  // the dot, for e_ts below
      }
      __syncthreads();
      for (int t = tid; t < C; t += 256) {
        float d = 0.f;
        if (t < L) {
          const float* qt = qh + t * p;
          for (int f = 0; f < n; ++f) {
            const int i = pairs[f] >> 16, j = pairs[f] & 0xffff;
            d += (i == j ? 1.f : r2) * qt[i] * qt[j] * Zt[f];
          }
          for (int s = 0; s <= t; ++s) d += W[t * C + s];
        }
        dd[t] = d;
      }
      __syncthreads();
      // o_t = N_t / D_t, then g_t o_t (into aa), delta_t, a_t, b_t
      for (int e = tid; e < C * dv; e += 256) {
        const int t = e / dv, d = e % dv;
        float num = 0.f;
        if (t < L) {
          const float* qt = qh + t * p;
          for (int f = 0; f < n; ++f) {
            const int i = pairs[f] >> 16, j = pairs[f] & 0xffff;
            num += (i == j ? 1.f : r2) * qt[i] * qt[j] * St[f * dv + d];
          }
          for (int s = 0; s <= t; ++s) num += W[t * C + s] * vv[s * dv + d];
        }
        aa[e] = dd[t] > 0.f ? gg[e] * num / dd[t] : 0.f;
      }
      __syncthreads();
      for (int t = tid; t < C; t += 256) {
        float dl = 0.f;
        for (int d = 0; d < dv; ++d) dl += aa[t * dv + d];
        const float D = dd[t], inv = D > 0.f ? 1.f / D : 0.f;
        if (t < L) *reinterpret_cast<float2*>(stats + row(t0 + t) * 2) = make_float2(D, dl);
        bb[t] = -dl * inv;
        dd[t] = inv;
      }
      __syncthreads();
      for (int e = tid; e < C * dv; e += 256) aa[e] = gg[e] * dd[e / dv];
      __syncthreads();
      // e_ts = (v_s . a_t + b_t) 2 (q_hat_t . k_hat_s), s <= t
      for (int e = tid; e < C * C; e += 256) {
        const int t = e / C, s = e % C;
        float x = 0.f;
        if (t < L && s <= t) {
          for (int d = 0; d < dv; ++d) x += vv[s * dv + d] * aa[t * dv + d];
          x = (x + bb[t]) * 2.f * E[e];
        }
        E[e] = x;
      }
      __syncthreads();
      // dq_hat_t,i: J^T (S a_t + Z b_t) over the pairs of i, plus sum_s e_ts k_hat_s,i
      for (int e = tid; e < C * p; e += 256) {
        const int t = e / p, i = e % p;
        float acc = 0.f;
        if (t < L) {
          const float* qt = qh + t * p;
          for (int j = 0; j < p; ++j) {
            const int a = min(i, j), b = max(i, j);
            const int f = a * p - a * (a - 1) / 2 + (b - a);
            float x = Zt[f] * bb[t];
            for (int d = 0; d < dv; ++d) x += St[f * dv + d] * aa[t * dv + d];
            acc += (i == j ? 2.f : r2) * x * qt[j];
          }
          for (int s = 0; s <= t; ++s) acc += E[t * C + s] * kh[s * p + i];
        }
        dh[e] = acc;
      }
      __syncthreads();
      for (int e = tid; e < C * p; e += 256) {  // projection onto the sphere's tangent, / |q|
        const int t = e / p;
        if (t >= L) continue;
        float pr = 0.f;
        for (int i = 0; i < p; ++i) pr += qh[t * p + i] * dh[t * p + i];
        dq[row(t0 + t) * p + e % p] = qn[t] > 0.f ? (dh[e] - qh[e] * pr) / qn[t] : 0.f;
      }
    }

    if (MODE == CB_RDK) {
      // w_ts and e_ts for t >= s (row t, column s)
      for (int e = tid; e < C * C; e += 256) {
        const int t = e / C, s = e % C;
        float w = 0.f, x = 0.f;
        if (t < L && s <= t) {
          float a = 0.f;
          for (int i = 0; i < p; ++i) a += qh[t * p + i] * kh[s * p + i];
          w = a * a;
          for (int d = 0; d < dv; ++d) x += vv[s * dv + d] * aa[t * dv + d];
          x = (x + bb[t]) * 2.f * a;
        }
        W[e] = w;
        E[e] = x;
      }
      __syncthreads();
      // dk_hat_s,i: J^T (R v_s + r) plus sum_{t>=s} e_ts q_hat_t,i
      for (int e = tid; e < C * p; e += 256) {
        const int s = e / p, i = e % p;
        float acc = 0.f;
        if (s < L) {
          const float* ks = kh + s * p;
          for (int j = 0; j < p; ++j) {
            const int a = min(i, j), b = max(i, j);
            const int f = a * p - a * (a - 1) / 2 + (b - a);
            float y = Zt[f];
            for (int d = 0; d < dv; ++d) y += St[f * dv + d] * vv[s * dv + d];
            acc += (i == j ? 2.f : r2) * y * ks[j];
          }
          for (int t = s; t < L; ++t) acc += E[t * C + s] * qh[t * p + i];
        }
        dh[e] = acc;
      }
      // dv_s = R^T psi(k_hat_s) + sum_{t>=s} w_ts a_t
      for (int e = tid; e < C * dv; e += 256) {
        const int s = e / dv, d = e % dv;
        if (s >= L) continue;
        const float* ks = kh + s * p;
        float acc = 0.f;
        for (int f = 0; f < n; ++f) {
          const int i = pairs[f] >> 16, j = pairs[f] & 0xffff;
          acc += (i == j ? 1.f : r2) * ks[i] * ks[j] * St[f * dv + d];
        }
        for (int t = s; t < L; ++t) acc += W[t * C + s] * aa[t * dv + d];
        dvo[row(t0 + s) * dv + d] = acc;
      }
      __syncthreads();
      for (int e = tid; e < C * p; e += 256) {
        const int s = e / p;
        if (s >= L) continue;
        float pr = 0.f;
        for (int i = 0; i < p; ++i) pr += kh[s * p + i] * dh[s * p + i];
        dk[row(t0 + s) * p + e % p] = kn[s] > 0.f ? (dh[e] - kh[e] * pr) / kn[s] : 0.f;
      }
    }
    __syncthreads();
    // state update: forward time S += psi(K)^T V, Z += psi(K)^T 1; reverse time
    // R += psi(Q)^T A, r += psi(Q)^T b
    for (int e = tid; e < n * dv + n; e += 256) {
      const bool isz = e >= n * dv;
      const int f = isz ? e - n * dv : e / dv, d = isz ? 0 : e % dv;
      const int i = pairs[f] >> 16, j = pairs[f] & 0xffff;
      const float cf = i == j ? 1.f : r2;
      const float* U = fwd_order ? kh : qh;
      float acc = 0.f;
      for (int t = 0; t < L; ++t) {
        const float ps = cf * U[t * p + i] * U[t * p + j];
        acc += ps * (fwd_order ? (isz ? 1.f : vv[t * dv + d]) : (isz ? bb[t] : aa[t * dv + d]));
      }
      St[e] += acc;
    }
  }
  __syncthreads();
  if (MODE == CB_FSUM || MODE == CB_RSUM) {
    const int slot = MODE == CB_FSUM ? seg : nseg - 1 - seg;
    float* dst = (MODE == CB_FSUM ? fsum : rsum) + (bh * (nseg - 1) + slot) * sf;
    for (int e = tid; e < n * dv + n; e += 256) dst[e] = St[e];
  }
}

hipError_t launch_scan(float* ws, int BH, int nslots, int64_t E, hipStream_t st);

template <bool IN_BF16>
static hipError_t launch_cb(const void* q, const void* k, const void* v, const void* go, int B, int H, int T, int p,
                            int dv, int C, const SegPlan& plan, float* stats, float* fsum, float* rsum, float* dq,
                            float* dk, float* dvo, hipStream_t st, SeqLayout lay) {
  const int BH = B * H;
  const size_t lds = chunked_bwd_lds_bytes(p, dv, C);
  const int64_t sf = chunked_bwd_state_floats(p, dv);
  hipError_t e;
  auto run = [&](auto kern, unsigned nblk_per_bh) -> hipError_t {
    hipError_t r = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (r != hipSuccess) return r;
    kern<<<dim3(nblk_per_bh * (unsigned)BH), dim3(256), lds, st>>>(q, k, v, go, T, p, dv, C, plan.nseg, plan.cps,
                                                                  (int)nblk_per_bh, fsum, rsum, sf, stats, dq, dk,
                                                                  dvo, lay, H);
    return hipGetLastError();
  };
  const bool segs = plan.nseg > 1;
  if (segs) {
    if ((e = run(chunked_bwd_kernel<IN_BF16, CB_FSUM>, plan.nseg - 1)) != hipSuccess) return e;
    if ((e = launch_scan(fsum, BH, plan.nseg - 1, sf, st)) != hipSuccess) return e;
  }
  if ((e = run(chunked_bwd_kernel<IN_BF16, CB_FDQ>, plan.nseg)) != hipSuccess) return e;
  if (segs) {
    if ((e = run(chunked_bwd_kernel<IN_BF16, CB_RSUM>, plan.nseg - 1)) != hipSuccess) return e;
    if ((e = launch_scan(rsum, BH, plan.nseg - 1, sf, st)) != hipSuccess) return e;
  }
  return run(chunked_bwd_kernel<IN_BF16, CB_RDK>, plan.nseg);
}

hipError_t launch_chunked_bwd(const void* q, const void* k, const void* v, const void* go, bool in_bf16, int B, int H,
                              int T, int p, int dv, int C, const SegPlan& plan, float* stats, float* fsum,
                              float* rsum, float* dq, float* dk, float* dvo, hipStream_t st, SeqLayout lay) {
  if (in_bf16)
    return launch_cb<true>(q, k, v, go, B, H, T, p, dv, C, plan, stats, fsum, rsum, dq, dk, dvo, st, lay);
  return launch_cb<false>(q, k, v, go, B, H, T, p, dv, C, plan, stats, fsum, rsum, dq, dk, dvo, st, lay);
}

}  // namespace kata
