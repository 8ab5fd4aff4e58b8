// Flash-attention-style KATA forward on bf16 MFMA (gfx950): no state is materialised.
//
// Source: "Kernelized Linear Attention: Breaking the Capacity Wall with Symmetric Cones"
// (arXiv 2607.17419): the abstract's flash-attention-style operating point; the weight
// identity <psi(q), psi(k)> = (q_hat . k_hat)^2 of the rank-one lift display (after
// Eq. (8)); the normalized readout with explicit denominator (normalized-readout
// paragraph); inclusive causality of the state S_t (feature-value state display).
//
// Per workgroup: 128 queries of one (b,h), 4 waves x 32 queries. Key blocks of 64 are
// normalised once per workgroup into LDS (bf16 K_hat, K_hat transposed-free; V stored
// transposed so the W.V operand is two 8-byte reads), double-buffered with the next
// block's global loads issued before the current block's MFMAs.
//   S^T = K_hat Q_hat^T   (16x16x32 bf16 MFMA, keys as M so the accumulator is already
//                          the A operand layout of the next product)
//   W   = (S^T)^2, causal mask on the diagonal blocks, rounded to bf16
//   [O | den] += W [V | 1] (the ones column gives the denominator from the same weights)
// Weights lie in [0, 1] and the denominator is a plain sum, so unlike softmax there is no
// running maximum and no rescaling. For the first 128 queries, where a denominator is a
// sum of only a few weights, the scores use a split-bf16 product (hi*hi + lo*hi + hi*lo).
#include "kata_device.h"
#include "kata_launch.h"

namespace kata {

namespace quad {
constexpr int BM = 128, BN = 64, QW = 32, NQT = QW / 16, NKT = BN / 16, NKP = BN / 32;
}

__device__ __forceinline__ bf16x8_t as_bf16x8(u16x8_t x) { return __builtin_bit_cast(bf16x8_t, x); }

__device__ __forceinline__ f32x4_t mfma16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <int P, int DV, bool OUT_BF16>
__global__ __launch_bounds__(256, 2) void quadratic_bf16_kernel(const uint16_t* __restrict__ q,
                                                                const uint16_t* __restrict__ k,
                                                                const uint16_t* __restrict__ v,
                                                                void* __restrict__ o, int T,
                                                                int nqb) {
  using namespace quad;
  constexpr int KS = (P + 31) / 32;    // 32-wide k-steps over the components
  constexpr int KPITCH = P + 8;        // bf16 row pitch of K_hat in LDS
  constexpr int VPITCH = BN + 8;       // bf16 row pitch of V^T in LDS
  constexpr int NT = DV / 16;          // 16-wide output column tiles
  constexpr int KQ = P / 4;            // components per staging thread (4 threads per key row)
  constexpr int KBUF = BN * KPITCH, VBUF = DV * VPITCH;
  __shared__ __align__(16) uint16_t sKh[2][KBUF];
  __shared__ __align__(16) uint16_t sKl[2][KBUF];
  __shared__ __align__(16) uint16_t sVt[2][VBUF];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ln = lane & 15, lg = lane >> 4;
  const int64_t bh = blockIdx.x / nqb;
  const int qb0 = (nqb - 1 - (int)(blockIdx.x % nqb)) * BM;  // longest rows first
  const int qw0 = qb0 + wave * QW;
  const bool split = qb0 == 0;
  const uint16_t* qbase = q + bh * (int64_t)T * P;
  const uint16_t* kbase = k + bh * (int64_t)T * P;
  const uint16_t* vbase = v + bh * (int64_t)T * DV;

  // ---- this lane's query fragments (B operand of S^T): query 16*qt + ln, comps 32*ks + 8*lg..+7
  bf16x8_t qh[NQT][KS], ql[NQT][KS];
#pragma unroll
  for (int qt = 0; qt < NQT; ++qt) {
    const int t = qw0 + 16 * qt + ln;
    float x[KS][8];
    float ss = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int c0 = 32 * ks + 8 * lg;
      u16x8_t raw = {0, 0, 0, 0, 0, 0, 0, 0};
      if (t < T && c0 < P) raw = *reinterpret_cast<const u16x8_t*>(qbase + (int64_t)t * P + c0);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        x[ks][j] = bf16_bits_to_f32(raw[j]);
        ss += x[ks][j] * x[ks][j];
      }
    }
    ss += __shfl_xor(ss, 16, 64);
    ss += __shfl_xor(ss, 32, 64);
    const float inv = inv_norm(ss);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u16x8_t h, l;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float y = x[ks][j] * inv;
        h[j] = f32_to_bf16_bits(y);
        l[j] = f32_to_bf16_bits(y - bf16_bits_to_f32(h[j]));
      }
      qh[qt][ks] = as_bf16x8(h);
      ql[qt][ks] = as_bf16x8(l);
    }
  }

  // ---- key-block staging: 4 threads per key row normalise and write bf16 hi/lo;
  //      V is written transposed, one (key pair, 8 columns) piece per thread.
  const int krow = tid >> 2, kq = tid & 3;
  constexpr int VPIECES = (BN / 2) * (DV / 8);
  const int vpair = tid / (DV / 8), vdg = tid % (DV / 8);
  uint16_t kreg[KQ];
  u16x8_t vreg0, vreg1;
  auto prefetch = [&](int kb0) {
    const int key = kb0 + krow;
#pragma unroll
    for (int i = 0; i < KQ; ++i) kreg[i] = 0;
    if (key < T) {
      const uint16_t* src = kbase + (int64_t)key * P + kq * KQ;
      if constexpr (KQ == 16) {
        *reinterpret_cast<u16x8_t*>(&kreg[0]) = *reinterpret_cast<const u16x8_t*>(src);
        *reinterpret_cast<u16x8_t*>(&kreg[8]) = *reinterpret_cast<const u16x8_t*>(src + 8);
      } else if constexpr (KQ == 8) {
        *reinterpret_cast<u16x8_t*>(&kreg[0]) = *reinterpret_cast<const u16x8_t*>(src);
      } else {
        *reinterpret_cast<u16x4_t*>(&kreg[0]) = *reinterpret_cast<const u16x4_t*>(src);
      }
    }
    vreg0 = u16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
    vreg1 = vreg0;
    if (tid < VPIECES) {
      const int key0 = kb0 + 2 * vpair;
      if (key0 < T) vreg0 = *reinterpret_cast<const u16x8_t*>(vbase + (int64_t)key0 * DV + 8 * vdg);
      if (key0 + 1 < T) vreg1 = *reinterpret_cast<const u16x8_t*>(vbase + (int64_t)(key0 + 1) * DV + 8 * vdg);
    }
  };
  auto stage = [&](int buf) {
    float x[KQ];
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < KQ; ++i) {
      x[i] = bf16_bits_to_f32(kreg[i]);
      ss += x[i] * x[i];
    }
    ss += __shfl_xor(ss, 1, 64);
    ss += __shfl_xor(ss, 2, 64);
    const float inv = inv_norm(ss);
    uint16_t* dh = &sKh[buf][krow * KPITCH + kq * KQ];
    uint16_t* dl = &sKl[buf][krow * KPITCH + kq * KQ];
#pragma unroll
    for (int i = 0; i < KQ; ++i) {
      const float y = x[i] * inv;
      const uint16_t h = f32_to_bf16_bits(y);
      dh[i] = h;
      dl[i] = f32_to_bf16_bits(y - bf16_bits_to_f32(h));
    }
    if (tid < VPIECES) {
      uint32_t* vt = reinterpret_cast<uint32_t*>(&sVt[buf][0]);
#pragma unroll
      for (int i = 0; i < 8; ++i)
        vt[((8 * vdg + i) * VPITCH + 2 * vpair) >> 1] = (uint32_t)vreg0[i] | ((uint32_t)vreg1[i] << 16);
    }
  };

  f32x4_t O[NQT][NT], D[NQT];
#pragma unroll
  for (int qt = 0; qt < NQT; ++qt) {
    D[qt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) O[qt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  u16x8_t ones_u;
#pragma unroll
  for (int j = 0; j < 8; ++j) ones_u[j] = 0x3F80;  // bf16 1.0
  const bf16x8_t ones = as_bf16x8(ones_u);

  const int kend = min(T, qb0 + BM);
  const int nkb = (kend + BN - 1) / BN;
  prefetch(0);
  stage(0);
  __syncthreads();
  for (int kb = 0; kb < nkb; ++kb) {
    const int buf = kb & 1;
    const int kb0 = kb * BN;
    if (kb + 1 < nkb) prefetch(kb0 + BN);
    if (kb0 <= qw0 + QW - 1 && qw0 < T) {
      const bool diag = kb0 + BN - 1 > qw0;  // some (key > query) pairs in this block
      // S^T tiles: keys 16*kt + row, queries 16*qt + col
      f32x4_t St[NKT][NQT];
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) {
#pragma unroll
        for (int qt = 0; qt < NQT; ++qt) St[kt][qt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          u16x8_t ah = {0, 0, 0, 0, 0, 0, 0, 0}, al = ah;
          if (P >= 32 || lg < 2) {
            ah = *reinterpret_cast<const u16x8_t*>(&sKh[buf][(16 * kt + ln) * KPITCH + 32 * ks + 8 * lg]);
            if (split) al = *reinterpret_cast<const u16x8_t*>(&sKl[buf][(16 * kt + ln) * KPITCH + 32 * ks + 8 * lg]);
          }
#pragma unroll
          for (int qt = 0; qt < NQT; ++qt) {
            St[kt][qt] = mfma16(as_bf16x8(ah), qh[qt][ks], St[kt][qt]);
            if (split) {
              St[kt][qt] = mfma16(as_bf16x8(al), qh[qt][ks], St[kt][qt]);
              St[kt][qt] = mfma16(as_bf16x8(ah), ql[qt][ks], St[kt][qt]);
            }
          }
        }
      }
      // W = S^2 (masked on the diagonal), packed as the A operand of W.[V|1]
#pragma unroll
      for (int kp = 0; kp < NKP; ++kp) {
        // V^T operand for this key pair: keys 32kp + 4lg + j and 32kp + 16 + 4lg + j
        bf16x8_t vb[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const uint16_t* row = &sVt[buf][(16 * nt + ln) * VPITCH + 32 * kp + 4 * lg];
          const u16x4_t a = *reinterpret_cast<const u16x4_t*>(row);
          const u16x4_t b = *reinterpret_cast<const u16x4_t*>(row + 16);
          vb[nt] = as_bf16x8(u16x8_t{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]});
        }
#pragma unroll
        for (int qt = 0; qt < NQT; ++qt) {
          const int query = qw0 + 16 * qt + ln;
          u16x8_t w;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int kt = 2 * kp + (j >> 2), r = j & 3;
            const float s = St[kt][qt][r];
            float ww = s * s;
            if (diag) {
              const int key = kb0 + 16 * kt + 4 * lg + r;
              ww = key <= query ? ww : 0.f;
            }
            w[j] = f32_to_bf16_bits(ww);
          }
          const bf16x8_t wa = as_bf16x8(w);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) O[qt][nt] = mfma16(wa, vb[nt], O[qt][nt]);
          D[qt] = mfma16(wa, ones, D[qt]);
        }
      }
    }
    if (kb + 1 < nkb) {
      __syncthreads();  // every wave is done with buffer buf^1 (used two blocks ago)
      stage(buf ^ 1);
      __syncthreads();
    }
  }

  // ---- epilogue: o[query, d] = O / den; lane holds queries 16qt + 4lg + r, column 16nt + ln
#pragma unroll
  for (int qt = 0; qt < NQT; ++qt) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int query = qw0 + 16 * qt + 4 * lg + r;
      if (query >= T) continue;
      const float den = D[qt][r];
      const float inv = den > 0.f ? 1.0f / den : 0.f;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        store_from_f32<OUT_BF16>(o, (bh * T + query) * (int64_t)DV + 16 * nt + ln, O[qt][nt][r] * inv);
    }
  }
}

template <int P, int DV>
static hipError_t launch_quad_pd(const uint16_t* q, const uint16_t* k, const uint16_t* v, void* o,
                                 bool o_bf16, int BH, int T, hipStream_t st) {
  const int nqb = (T + quad::BM - 1) / quad::BM;
  dim3 grid((unsigned)((int64_t)nqb * BH)), block(256);
  if (o_bf16) quadratic_bf16_kernel<P, DV, true><<<grid, block, 0, st>>>(q, k, v, o, T, nqb);
  else quadratic_bf16_kernel<P, DV, false><<<grid, block, 0, st>>>(q, k, v, o, T, nqb);
  return hipGetLastError();
}

hipError_t launch_quadratic_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v, void* o,
                                 bool o_bf16, int B, int H, int T, int p, int dv, hipStream_t st) {
  const int BH = B * H;
#define KATA_QCASE(PP, DD) \
  if (p == PP && dv == DD) return launch_quad_pd<PP, DD>(q, k, v, o, o_bf16, BH, T, st);
  KATA_QCASE(16, 16) KATA_QCASE(16, 32) KATA_QCASE(16, 64)
  KATA_QCASE(32, 16) KATA_QCASE(32, 32) KATA_QCASE(32, 64)
  KATA_QCASE(64, 16) KATA_QCASE(64, 32) KATA_QCASE(64, 64)
#undef KATA_QCASE
  return hipErrorInvalidValue;
}

}  // namespace kata
