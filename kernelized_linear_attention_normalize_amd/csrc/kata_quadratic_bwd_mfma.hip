// Gradients of the causal full-map forward on bf16 MFMA (gfx950), flash style: no state and
// no T x T matrix is materialised.
//
// Source: the forward of "Kernelized Linear Attention: Breaking the Capacity Wall with
// Symmetric Cones" (arXiv 2607.17419), HTML page: normalized-readout paragraph (o_t =
// sum_s w_ts v_s / sum_s w_ts), rank-one lift display after Eq. (8) (w_ts = (q_hat . k_hat)^2).
// The pages give no backward pass; this is its calculus. As in the forward kernels the query
// is used raw: with w_ts = (q_t . k_hat_s)^2 = |q_t|^2 (q_hat_t . k_hat_s)^2, D_t = sum_s w_ts
// and the output is unchanged, and differentiating this raw form gives the exact gradient
// (the output does not depend on |q_t|). With g_t = dL/do_t and delta_t = g_t . o_t:
//   dW_ts = (g_t . v_s - delta_t) / D_t,  S_ts = q_t . k_s (raw),  ik_s = 1 / |k_s|,
//   dv_s = sum_t (w_ts / D_t) g_t, with w_ts rounded to bf16 exactly as the forward rounds it
//          before summing D_t (so one token gives dv = g exactly),
//   dq_t = 2 sum_s dW_ts S_ts ik_s^2 k_s,
//   dk_s = 2 ik_s^2 (sum_t c_ts q_t - ik_s^2 k_s sum_t c_ts S_ts),  c_ts = dW_ts S_ts.
// D_t and delta_t come from the forward kernel's statistics epilogue (kata_quadratic.hip).
//
// bwd_keys_kernel: one workgroup of 8 waves per 256 keys, 32 keys per wave; query blocks of
//   64 (q rows, g rows and their transposes in the shared permuted layout) are staged in LDS,
//   double-buffered, from the workgroup's first key to the end. S = Q K^T and dP = G V^T
//   (queries as rows: the accumulator rows are the k-slots of the next products) give the
//   per-pair weights; dV += P G and dK += C Q with the lane's keys as rows.
// bwd_queries_kernel: one workgroup of 8 waves per 512 queries, 64 queries per wave (the
//   forward's layout); key blocks of 64 (k rows, v rows, k transposed, ik^2) staged in LDS
//   from the start to the wave's last query. S^T = K Q^T and dP^T = V G^T (keys as rows),
//   dQ^T += K^T C^T.
// PK: packed token-major sequences (row0 + t * stp for t < len from cu_seqlens, T = max_len);
//   workgroups past a sequence's length return at once, rows past it read as zero.
#include <type_traits>

#include "kata_device.h"
#include "kata_launch.h"

namespace kata {
namespace qbwd {
constexpr int NW = 8, NTHR = 64 * NW;
constexpr int BQ = 64;    // staged block (queries for the key kernel, keys for the query kernel)
constexpr int VTP = 80;   // bf16 pitch of the transposed, permuted rows of a 64-row block
constexpr int KW = 32;    // keys per wave in the key kernel
constexpr int KB = KW * NW;
constexpr int QW = 64;    // queries per wave in the query kernel
constexpr int QB = QW * NW;
template <int W> constexpr int row_pitch() { return W == 64 ? 80 : 48; }  // bf16, 8 * odd floats
}  // namespace qbwd

__device__ __forceinline__ f32x4_t mfma_b(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8_t pack8f(const float (&x)[8]) {
  return __builtin_bit_cast(bf16x8_t, u32x4_t{pk2(x[0], x[1]), pk2(x[2], x[3]), pk2(x[4], x[5]), pk2(x[6], x[7])});
}

// Staging of one 64-row block of a sequence's rows of a bf16 tensor of width W (rows r0..): raw
// rows at pitch row_pitch<W>() and, when TR, the transposed rows in the permuted key layout of
// the forward (column c at vt_row(c), row r of the block at vt_pos(r)). Rows past the
// sequence's length lie outside the buffer resource and read as zero.
template <int W, bool TR>
struct BlockStager {
  static constexpr int RP = qbwd::row_pitch<W>();
  static constexpr int RPIECES = qbwd::BQ * W / 8;        // 16-byte row pieces
  static constexpr int RI = (RPIECES + qbwd::NTHR - 1) / qbwd::NTHR;
  static constexpr int TPIECES = (qbwd::BQ / 2) * (W / 8);  // (row pair, 8 columns) pieces
  u32x4_t rr[RI];
  u32x4_t tr[2];
  int vp = 0, vd = 0;
  // tfirst: the first thread of this tensor's transposed pieces (two tensors share the threads);
  // rs: elements from one row to the next (W padded, H W packed)
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rsrc, int r0, int tfirst, int rs) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < RI; ++i) {
      const int pc = tid + qbwd::NTHR * i;
      if (pc < RPIECES)
        rr[i] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, (uint32_t)((r0 + pc / (W / 8)) * rs + 8 * (pc % (W / 8))) * 2, 0, 0);
    }
    if constexpr (TR) {
      const int pc = tid - tfirst;
      if (pc >= 0 && pc < TPIECES) {
        vt_piece<W>(pc, vp, vd);
        const uint32_t off = (uint32_t)((r0 + 2 * vp) * rs + 8 * vd) * 2;
        tr[0] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, off, 0, 0);
        tr[1] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, off + (uint32_t)rs * 2, 0, 0);
      }
    }
  }
  __device__ __forceinline__ void store(uint16_t* rows, uint16_t* trows, int tfirst) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < RI; ++i) {
      const int pc = tid + qbwd::NTHR * i;
      if (pc < RPIECES) *reinterpret_cast<u32x4_t*>(rows + (pc / (W / 8)) * RP + 8 * (pc % (W / 8))) = rr[i];
    }
    if constexpr (TR) {
      const int pc = tid - tfirst;
      if (pc >= 0 && pc < TPIECES) {
        char* base = reinterpret_cast<char*>(trows) + ((8 * vd) * qbwd::VTP + vt_pos(2 * vp)) * 2;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t a = (tr[0][e >> 1] >> (16 * (e & 1))) & 0xffffu;
          const uint32_t b = (tr[1][e >> 1] >> (16 * (e & 1))) & 0xffffu;
          *reinterpret_cast<uint32_t*>(base + ((e & 4) + ((e & 3) ^ (vd & 3))) * qbwd::VTP * 2) = a | (b << 16);
        }
      }
    }
  }
};

// 1 / |row| of the row whose P components are spread as 8-component pieces over the four lane
// groups (lg) and KS k-steps of fragments f[ks]
template <int KS>
__device__ __forceinline__ float frag_inv_norm(const bf16x8_t (&f)[KS]) {
  float ss = 0.f;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const u32x4_t u = __builtin_bit_cast(u32x4_t, f[ks]);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float lo = bf16_bits_to_f32(u[e] & 0xffffu), hi = __uint_as_float(u[e] & 0xffff0000u);
      ss += lo * lo + hi * hi;
    }
  }
  return inv_norm_fast(xor32_sum(xor16_sum(ss)));
}

// ---------------------------------------------------------------- dK, dV (keys own the wave)
template <int P, int DV, bool PK>
__global__ __launch_bounds__(qbwd::NTHR, 1) void bwd_keys_kernel(const uint16_t* __restrict__ q,
                                                                 const uint16_t* __restrict__ k,
                                                                 const uint16_t* __restrict__ v,
                                                                 const uint16_t* __restrict__ gout,
                                                                 const float* __restrict__ stats,
                                                                 float* __restrict__ dk, float* __restrict__ dvo,
                                                                 int T, int nkb, SeqLayout lay, int H) {
  using namespace qbwd;
  constexpr int KS = P / 32, DS = DV / 32, NKT = KW / 16;
  constexpr int QP = row_pitch<P>(), GP = row_pitch<DV>();
  __shared__ __align__(16) uint16_t sQ[2][BQ * QP];
  __shared__ __align__(16) uint16_t sG[2][BQ * GP];
  __shared__ __align__(16) uint16_t sQt[2][P * VTP];
  __shared__ __align__(16) uint16_t sGt[2][DV * VTP];
  __shared__ __align__(16) float sDinv[2][BQ];  // 1 / D_t (0 where D_t = 0 or t >= T)
  __shared__ __align__(16) float sNd[2][BQ];    // -delta_t / D_t
  __shared__ __align__(16) float sIK2[KB];      // ik_s^2 of this workgroup's keys
  __shared__ __align__(16) float sBK[KB];       // sum_t c_ts S_ts per key

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ln = lane & 15, lg = lane >> 4;
  // key blocks with more queries after them go first: workgroup x takes key block x / BH
  const int nbh = (int)(gridDim.x / nkb);
  const int64_t bh = blockIdx.x % nbh;
  const int K0 = (int)(blockIdx.x / nbh) * KB;
  const int kw0 = K0 + wave * KW;
  // Rows of this sequence: row0 + t * stp for t < len (padded: bh T + t; packed token-major
  // (PK): H rows apart, the length from cu_seqlens, T = max_len)
  int64_t row0 = bh * (int64_t)T;
  int stp = 1, len = T;
  if constexpr (PK) {
    seq_rows_of(lay, bh, H, T, row0, stp, len);
    if (K0 >= len) return;  // uniform over the workgroup: no key of this block exists
  }
  const int RQ = PK ? stp * P : P, RV = PK ? stp * DV : DV;  // elements from one row to the next
  const __amdgpu_buffer_rsrc_t rq = buf_rsrc(q + row0 * P, (uint32_t)len * RQ * 2);
  const __amdgpu_buffer_rsrc_t rk = buf_rsrc(k + row0 * P, (uint32_t)len * RQ * 2);
  const __amdgpu_buffer_rsrc_t rv = buf_rsrc(v + row0 * DV, (uint32_t)len * RV * 2);
  const __amdgpu_buffer_rsrc_t rg = buf_rsrc(gout + row0 * DV, (uint32_t)len * RV * 2);

  // this wave's keys as B operands: key kw0 + 16 kt + ln, components / columns 32 ks + 8 lg ..
  bf16x8_t kf[NKT][KS], vf[NKT][DS];
  float ik1[NKT], ik2[NKT];
#pragma unroll
  for (int kt = 0; kt < NKT; ++kt) {
    const int key = kw0 + 16 * kt + ln;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      kf[kt][ks] = __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(rk, (uint32_t)(key * RQ + 32 * ks + 8 * lg) * 2, 0, 0));
#pragma unroll
    for (int ds = 0; ds < DS; ++ds)
      vf[kt][ds] = __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(rv, (uint32_t)(key * RV + 32 * ds + 8 * lg) * 2, 0, 0));
    const float ik = frag_inv_norm<KS>(kf[kt]);
    ik1[kt] = ik;
    ik2[kt] = ik * ik;
    if (lg == 0) sIK2[wave * KW + 16 * kt + ln] = ik2[kt];
  }

  BlockStager<P, true> stq;
  BlockStager<DV, true> stg;
  float dstat[2] = {0.f, 0.f};
  constexpr int QT_FIRST = 0, GT_FIRST = (BQ / 2) * (P / 8);  // transposed pieces: q first, then g
  static_assert(GT_FIRST + (BQ / 2) * (DV / 8) <= NTHR, "staging layout");
  auto prefetch = [&](int qb0) {
    stq.load(rq, qb0, QT_FIRST, RQ);
    stg.load(rg, qb0, GT_FIRST, RV);
    if (tid < BQ) {
      const int t = qb0 + tid;
      dstat[0] = dstat[1] = 0.f;
      if (t < len) {
        const u32x2_t s2 = *reinterpret_cast<const u32x2_t*>(stats + (row0 + (int64_t)t * stp) * 2);
        dstat[0] = __uint_as_float(s2[0]);
        dstat[1] = __uint_as_float(s2[1]);
      }
    }
  };
  auto stage = [&](int buf) {
    stq.store(sQ[buf], sQt[buf], QT_FIRST);
    stg.store(sG[buf], sGt[buf], GT_FIRST);
    if (tid < BQ) {
      const float inv = dstat[0] > 0.f ? __builtin_amdgcn_rcpf(dstat[0]) : 0.f;
      sDinv[buf][tid] = inv;
      sNd[buf][tid] = -dstat[1] * inv;
    }
  };

  f32x4_t dVa[NKT][DV / 16], dKa[NKT][P / 16];
  float bk[NKT];
#pragma unroll
  for (int kt = 0; kt < NKT; ++kt) {
    bk[kt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DV / 16; ++dt) dVa[kt][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int pt = 0; pt < P / 16; ++pt) dKa[kt][pt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  const int qb_first = K0 / BQ, nqb = (len + BQ - 1) / BQ;
  if (qb_first < nqb) {
    prefetch(qb_first * BQ);
    stage(0);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the key fragments are complete
  __syncthreads();
  for (int qb = qb_first; qb < nqb; ++qb) {
    const int buf = (qb - qb_first) & 1;
    const int qb0 = qb * BQ;
    if (qb + 1 < nqb) prefetch(qb0 + BQ);
    // queries t >= key s: a block wholly before this wave's first key contributes nothing
    auto block = [&](auto diag_c) {
      constexpr bool DIAG = decltype(diag_c)::value;
#pragma unroll
      for (int qp = 0; qp < BQ / 32; ++qp) {
        // statistics of the lane's 8 queries 32 qp + 16 h + 4 lg + r (the k-slot order)
        const f32x4_t di0 = *reinterpret_cast<const f32x4_t*>(&sDinv[buf][32 * qp + 4 * lg]);
        const f32x4_t di1 = *reinterpret_cast<const f32x4_t*>(&sDinv[buf][32 * qp + 16 + 4 * lg]);
        const f32x4_t nd0 = *reinterpret_cast<const f32x4_t*>(&sNd[buf][32 * qp + 4 * lg]);
        const f32x4_t nd1 = *reinterpret_cast<const f32x4_t*>(&sNd[buf][32 * qp + 16 + 4 * lg]);
        bf16x8_t gt[DV / 16], qt[P / 16];
#pragma unroll
        for (int dt = 0; dt < DV / 16; ++dt)
          gt[dt] = *reinterpret_cast<const bf16x8_t*>(&sGt[buf][vt_row(16 * dt + ln) * VTP + 32 * qp + 8 * lg]);
#pragma unroll
        for (int pt = 0; pt < P / 16; ++pt)
          qt[pt] = *reinterpret_cast<const bf16x8_t*>(&sQt[buf][vt_row(16 * pt + ln) * VTP + 32 * qp + 8 * lg]);
        bf16x8_t qa[2][KS], ga[2][DS];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
            qa[h][ks] = *reinterpret_cast<const bf16x8_t*>(&sQ[buf][(32 * qp + 16 * h + ln) * QP + 32 * ks + 8 * lg]);
#pragma unroll
          for (int ds = 0; ds < DS; ++ds)
            ga[h][ds] = *reinterpret_cast<const bf16x8_t*>(&sG[buf][(32 * qp + 16 * h + ln) * GP + 32 * ds + 8 * lg]);
        }
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) {
          const int key = kw0 + 16 * kt + ln;
          float pv[8], cv[8];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            f32x4_t S = {0.f, 0.f, 0.f, 0.f}, dP = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) S = mfma_b(qa[h][ks], kf[kt][ks], S);
#pragma unroll
            for (int ds = 0; ds < DS; ++ds) dP = mfma_b(ga[h][ds], vf[kt][ds], dP);
            const f32x4_t di = h ? di1 : di0, nd = h ? nd1 : nd0;
            float w[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              float s = S[r];
              if (DIAG && qb0 + 32 * qp + 16 * h + 4 * lg + r < key) s = 0.f;
              const float dw = dP[r] * di[r] + nd[r];
              const float c = dw * s;
              const float sk = s * ik1[kt];
              w[r] = sk * sk;
              cv[4 * h + r] = c;
              bk[kt] += c * s;
            }
            // the forward's weights: rounded to bf16 before they are summed into D_t
            const uint32_t w01 = pk2(w[0], w[1]), w23 = pk2(w[2], w[3]);
            pv[4 * h + 0] = bf16_bits_to_f32(w01 & 0xffffu) * di[0];
            pv[4 * h + 1] = __uint_as_float(w01 & 0xffff0000u) * di[1];
            pv[4 * h + 2] = bf16_bits_to_f32(w23 & 0xffffu) * di[2];
            pv[4 * h + 3] = __uint_as_float(w23 & 0xffff0000u) * di[3];
          }
          const bf16x8_t pa = pack8f(pv), ca = pack8f(cv);
#pragma unroll
          for (int dt = 0; dt < DV / 16; ++dt) dVa[kt][dt] = mfma_b(pa, gt[dt], dVa[kt][dt]);
#pragma unroll
          for (int pt = 0; pt < P / 16; ++pt) dKa[kt][pt] = mfma_b(ca, qt[pt], dKa[kt][pt]);
        }
      }
    };
    if (qb0 + BQ - 1 >= kw0 && kw0 < len) {
      if (qb0 < kw0 + KW - 1) block(std::true_type{});
      else block(std::false_type{});
    }
    if (qb + 1 < nqb) stage(buf ^ 1);  // buffer of block qb - 1: every wave is past it
    __syncthreads();
  }

  // ---- epilogue: per-key sums, then dv and dk; lane holds columns 16 t + ln of keys
  // kw0 + 16 kt + 4 lg + r
#pragma unroll
  for (int kt = 0; kt < NKT; ++kt) {
    const float tot = xor32_sum(xor16_sum(bk[kt]));
    if (lg == 0) sBK[wave * KW + 16 * kt + ln] = tot;
  }
  __syncthreads();
#pragma unroll
  for (int kt = 0; kt < NKT; ++kt) {
    const f32x4_t i2 = *reinterpret_cast<const f32x4_t*>(&sIK2[wave * KW + 16 * kt + 4 * lg]);
    const f32x4_t bs = *reinterpret_cast<const f32x4_t*>(&sBK[wave * KW + 16 * kt + 4 * lg]);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = kw0 + 16 * kt + 4 * lg + r;
      if (key >= len) continue;
      const int64_t row = row0 + (int64_t)key * stp;
#pragma unroll
      for (int dt = 0; dt < DV / 16; ++dt) dvo[row * DV + 16 * dt + ln] = dVa[kt][dt][r];
#pragma unroll
      for (int pt = 0; pt < P / 16; ++pt) {
        const float kc = bf16_bits_to_f32(k[row * P + 16 * pt + ln]);
        dk[row * P + 16 * pt + ln] = 2.f * i2[r] * (dKa[kt][pt][r] - i2[r] * kc * bs[r]);
      }
    }
  }
}

// ---------------------------------------------------------------- dQ (queries own the wave)
template <int P, int DV, bool PK>
__global__ __launch_bounds__(qbwd::NTHR, 1) void bwd_queries_kernel(const uint16_t* __restrict__ q,
                                                                    const uint16_t* __restrict__ k,
                                                                    const uint16_t* __restrict__ v,
                                                                    const uint16_t* __restrict__ gout,
                                                                    const float* __restrict__ stats,
                                                                    float* __restrict__ dq, int T, int nqb,
                                                                    SeqLayout lay, int H) {
  using namespace qbwd;
  constexpr int KS = P / 32, DS = DV / 32, NQT = QW / 16;
  constexpr int KP = row_pitch<P>(), VP = row_pitch<DV>();
  __shared__ __align__(16) uint16_t sK[2][BQ * KP];
  __shared__ __align__(16) uint16_t sV[2][BQ * VP];
  __shared__ __align__(16) uint16_t sKt[2][P * VTP];
  __shared__ __align__(16) float sIK2[2][BQ];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ln = lane & 15, lg = lane >> 4;
  // the forward's order: the longest query blocks first over all sequences
  const int nbh = (int)(gridDim.x / nqb);
  const int64_t bh = blockIdx.x % nbh;
  const int qb0 = (nqb - 1 - (int)(blockIdx.x / nbh)) * QB;
  const int qw0 = qb0 + wave * QW;
  int64_t row0 = bh * (int64_t)T;  // rows of this sequence, as in bwd_keys_kernel
  int stp = 1, len = T;
  if constexpr (PK) {
    seq_rows_of(lay, bh, H, T, row0, stp, len);
    if (qb0 >= len) return;  // uniform over the workgroup: no query of this block exists
  }
  const int RQ = PK ? stp * P : P, RV = PK ? stp * DV : DV;
  const __amdgpu_buffer_rsrc_t rq = buf_rsrc(q + row0 * P, (uint32_t)len * RQ * 2);
  const __amdgpu_buffer_rsrc_t rk = buf_rsrc(k + row0 * P, (uint32_t)len * RQ * 2);
  const __amdgpu_buffer_rsrc_t rv = buf_rsrc(v + row0 * DV, (uint32_t)len * RV * 2);
  const __amdgpu_buffer_rsrc_t rg = buf_rsrc(gout + row0 * DV, (uint32_t)len * RV * 2);

  // this wave's queries as B operands: query qw0 + 16 qt + ln, components / columns 32 ks + 8 lg ..
  bf16x8_t qf[NQT][KS], gf[NQT][DS];
  float dinv[NQT], nd[NQT];
#pragma unroll
  for (int qt = 0; qt < NQT; ++qt) {
    const int query = qw0 + 16 * qt + ln;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[qt][ks] = __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(rq, (uint32_t)(query * RQ + 32 * ks + 8 * lg) * 2, 0, 0));
#pragma unroll
    for (int ds = 0; ds < DS; ++ds)
      gf[qt][ds] = __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(rg, (uint32_t)(query * RV + 32 * ds + 8 * lg) * 2, 0, 0));
    dinv[qt] = nd[qt] = 0.f;
    if (query < len) {
      const u32x2_t s2 = *reinterpret_cast<const u32x2_t*>(stats + (row0 + (int64_t)query * stp) * 2);
      const float D = __uint_as_float(s2[0]);
      dinv[qt] = D > 0.f ? __builtin_amdgcn_rcpf(D) : 0.f;
      nd[qt] = -__uint_as_float(s2[1]) * dinv[qt];
    }
  }

  BlockStager<P, true> stk;
  BlockStager<DV, false> stv;
  static_assert(BlockStager<P, true>::RI == 1, "one key-row piece per thread");
  auto prefetch = [&](int kb0) {
    stk.load(rk, kb0, 0, RQ);
    stv.load(rv, kb0, 0, RV);
  };
  // rows to LDS, and ik^2 per key from the row pieces: the P / 8 pieces of a row sit on
  // adjacent lanes (whole waves take part or none)
  auto stage = [&](int buf) {
    stk.store(sK[buf], sKt[buf], 0);
    stv.store(sV[buf], nullptr, 0);
    if (tid < BlockStager<P, true>::RPIECES) {
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t u = stk.rr[0][e];
        const float lo = bf16_bits_to_f32(u & 0xffffu), hi = __uint_as_float(u & 0xffff0000u);
        ss += lo * lo + hi * hi;
      }
      ss = group_sum<P / 8>(ss);
      const float ik = inv_norm_fast(ss);
      if (tid % (P / 8) == 0) sIK2[buf][tid / (P / 8)] = ik * ik;
    }
  };

  f32x4_t dQa[NQT][P / 16];
#pragma unroll
  for (int qt = 0; qt < NQT; ++qt)
#pragma unroll
    for (int pt = 0; pt < P / 16; ++pt) dQa[qt][pt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int kend = min(len, qb0 + QB);
  const int nkb = (kend + BQ - 1) / BQ;
  prefetch(0);
  stage(0);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the query fragments are complete
  __syncthreads();
  for (int kb = 0; kb < nkb; ++kb) {
    const int buf = kb & 1;
    const int kb0 = kb * BQ;
    if (kb + 1 < nkb) prefetch(kb0 + BQ);
    auto block = [&](auto diag_c) {
      constexpr bool DIAG = decltype(diag_c)::value;
#pragma unroll
      for (int kp = 0; kp < BQ / 32; ++kp) {
        // keys 32 kp + 16 h + 4 lg + r: ik^2 and the transposed keys (A of dQ^T)
        const f32x4_t i20 = *reinterpret_cast<const f32x4_t*>(&sIK2[buf][32 * kp + 4 * lg]);
        const f32x4_t i21 = *reinterpret_cast<const f32x4_t*>(&sIK2[buf][32 * kp + 16 + 4 * lg]);
        bf16x8_t kt_[P / 16];
#pragma unroll
        for (int pt = 0; pt < P / 16; ++pt)
          kt_[pt] = *reinterpret_cast<const bf16x8_t*>(&sKt[buf][vt_row(16 * pt + ln) * VTP + 32 * kp + 8 * lg]);
        bf16x8_t ka[2][KS], va[2][DS];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
            ka[h][ks] = *reinterpret_cast<const bf16x8_t*>(&sK[buf][(32 * kp + 16 * h + ln) * KP + 32 * ks + 8 * lg]);
#pragma unroll
          for (int ds = 0; ds < DS; ++ds)
            va[h][ds] = *reinterpret_cast<const bf16x8_t*>(&sV[buf][(32 * kp + 16 * h + ln) * VP + 32 * ds + 8 * lg]);
        }
#pragma unroll
        for (int qt = 0; qt < NQT; ++qt) {
          const int query = qw0 + 16 * qt + ln;
          float cv[8];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            f32x4_t St = {0.f, 0.f, 0.f, 0.f}, dPt = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) St = mfma_b(ka[h][ks], qf[qt][ks], St);
#pragma unroll
            for (int ds = 0; ds < DS; ++ds) dPt = mfma_b(va[h][ds], gf[qt][ds], dPt);
            const f32x4_t i2 = h ? i21 : i20;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              float s = St[r];
              if (DIAG && kb0 + 32 * kp + 16 * h + 4 * lg + r > query) s = 0.f;
              const float dw = dPt[r] * dinv[qt] + nd[qt];
              cv[4 * h + r] = dw * s * i2[r];
            }
          }
          const bf16x8_t ca = pack8f(cv);
#pragma unroll
          for (int pt = 0; pt < P / 16; ++pt) dQa[qt][pt] = mfma_b(kt_[pt], ca, dQa[qt][pt]);
        }
      }
    };
    if (kb0 <= qw0 + QW - 1 && qw0 < len) {
      if (kb0 + BQ - 1 > qw0) block(std::true_type{});
      else block(std::false_type{});
    }
    if (kb + 1 < nkb) stage(buf ^ 1);  // buffer of block kb - 1: every wave is past it
    __syncthreads();
  }

  // ---- epilogue: lane holds components 16 pt + 4 lg + r of query qw0 + 16 qt + ln
#pragma unroll
  for (int qt = 0; qt < NQT; ++qt) {
    const int query = qw0 + 16 * qt + ln;
    if (query >= len) continue;
#pragma unroll
    for (int pt = 0; pt < P / 16; ++pt)
      *reinterpret_cast<f32x4_t*>(dq + (row0 + (int64_t)query * stp) * P + 16 * pt + 4 * lg) = dQa[qt][pt] * 2.f;
  }
}

hipError_t launch_quadratic_bf16_stats(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* gout,
                                       float* stats, int B, int H, int T, int p, int dv, hipStream_t st);
hipError_t launch_quadratic_bf16_stats_varlen(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                              const uint16_t* gout, float* stats, int B, int H, int max_len, int p,
                                              int dv, SeqLayout lay, hipStream_t st);

bool quadratic_bwd_mfma_supported(int p, int dv) { return (p == 32 || p == 64) && (dv == 32 || dv == 64); }

template <int P, int DV, bool PK>
static hipError_t launch_bwd_pd(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* gout,
                                float* stats, float* dq, float* dk, float* dvo, int BH, int H, int T, SeqLayout lay,
                                hipStream_t st) {
  const int nkb = (T + qbwd::KB - 1) / qbwd::KB;
  bwd_keys_kernel<P, DV, PK><<<dim3((unsigned)((int64_t)nkb * BH)), dim3(qbwd::NTHR), 0, st>>>(
      q, k, v, gout, stats, dk, dvo, T, nkb, lay, H);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nqb = (T + qbwd::QB - 1) / qbwd::QB;
  bwd_queries_kernel<P, DV, PK><<<dim3((unsigned)((int64_t)nqb * BH)), dim3(qbwd::NTHR), 0, st>>>(
      q, k, v, gout, stats, dq, T, nqb, lay, H);
  return hipGetLastError();
}

hipError_t launch_quadratic_bwd_mfma(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* gout,
                                     int B, int H, int T, int p, int dv, float* stats, float* dq, float* dk,
                                     float* dvo, hipStream_t st) {
  hipError_t e = launch_quadratic_bf16_stats(q, k, v, gout, stats, B, H, T, p, dv, st);
  if (e != hipSuccess) return e;
  const int BH = B * H;
#define KATA_BCASE(PP, DD) \
  if (p == PP && dv == DD) return launch_bwd_pd<PP, DD, false>(q, k, v, gout, stats, dq, dk, dvo, BH, H, T, SeqLayout{}, st);
  KATA_BCASE(32, 32) KATA_BCASE(32, 64) KATA_BCASE(64, 32) KATA_BCASE(64, 64)
#undef KATA_BCASE
  return hipErrorInvalidValue;
}

hipError_t launch_quadratic_bwd_mfma_varlen(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                            const uint16_t* gout, int B, int H, int max_len, int p, int dv,
                                            SeqLayout lay, float* stats, float* dq, float* dk, float* dvo,
                                            hipStream_t st) {
  hipError_t e = launch_quadratic_bf16_stats_varlen(q, k, v, gout, stats, B, H, max_len, p, dv, lay, st);
  if (e != hipSuccess) return e;
  const int BH = B * H;
#define KATA_BCASE(PP, DD) \
  if (p == PP && dv == DD) return launch_bwd_pd<PP, DD, true>(q, k, v, gout, stats, dq, dk, dvo, BH, H, max_len, lay, st);
  KATA_BCASE(32, 32) KATA_BCASE(32, 64) KATA_BCASE(64, 32) KATA_BCASE(64, 64)
#undef KATA_BCASE
  return hipErrorInvalidValue;
}

}  // namespace kata
