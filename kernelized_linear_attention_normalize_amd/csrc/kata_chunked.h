// Exact O(T) chunked-state KATA forward on bf16 MFMA (gfx950).
//
// Source: "Kernelized Linear Attention: Breaking the Capacity Wall with Symmetric Cones"
// (arXiv 2607.17419), arXiv HTML page:
//   * chunked-forward paragraph: per-chunk state psi(K_c)^T [V_c | 1], the inter-chunk
//     prefix as an associative cumulative sum, the local C x C causal block, and the
//     remark that writing per-chunk states to HBM is the real bottleneck;
//   * rank-one lift display after Eq. (8): psi(u) = u u^T on the unit sphere,
//     <psi(a), psi(b)> = (a.b)^2;  Eq. (8): n = p(p+1)/2 packed coordinates;
//   * normalized-readout paragraph: o_t = psi(q_t)^T S_t / psi(q_t)^T Z_t;
//   * the remark on the fused rank-two forward: the per-token psi tensor is never
//     written to HBM.
//
// Design (one workgroup = 4 waves per (b,h,segment); the state never leaves the chip):
//   * The n = p(p+1)/2 packed features are ordered internally as tiles of 16 features.
//     In tile tau, row m (0..15) holds a pair (i, j) in which one index is m (or 16+m)
//     and the other is m rotated by a tile constant inside its 16-lane row. Hence a
//     lane that holds the natural components k_hat[t][m], k_hat[t][16+m] builds its
//     A-operand row with ONE v_mul_f32 whose second operand is a DPP row rotation:
//     the lift costs one multiply per feature and never touches LDS or HBM.
//     p = 32 gives 33 tiles = 528 features exactly; p = 16 gives 9 tiles (136 + 8 pad).
//   * The state S (fp32) lives in MFMA accumulators, split by feature tiles over the 4
//     waves. The accumulator layout of a 16x16 tile (rows 4g..4g+3 in lane group g) is
//     used directly as the B operand of the readout psi(Q) S (k-slots permuted the same
//     way on the A side), so S needs no LDS round trip: one cvt_pk_bf16 per 2 entries.
//   * Off-diagonal coordinates carry sqrt(2) in psi; their product c_ij^2 = 2 is folded
//     into the state build (the key side is scaled by 2), so the readout side uses raw
//     products q_i q_j.
//   * The denominator psi(q)^T Z = q_hat^T M q_hat with the Gram matrix
//     M = sum_s k_hat_s k_hat_s^T (p x p): M is updated and applied with split-bf16
//     MFMAs (hi*hi + hi*lo + lo*hi), so the normaliser is fp32-accurate.
//   * Intra-chunk block: S^T = K_hat Q_hat^T (keys as M), W = (S^T)^2 masked, rounded to
//     bf16, O += W V. Global chunk 0, where denominators are sums of few weights, uses
//     split-bf16 scores.
//   * Each wave's readout covers its own features for every token of the chunk; the 4
//     partial outputs are summed through LDS, divided by the denominator and stored.
//   * SEQUENTIAL: one workgroup per (b,h) walks all chunks. ASSOCIATIVE: a summary pass
//     writes each segment's [S | M] (fp32, in this tile layout), an in-place scan forms
//     exclusive prefixes, and every segment runs its chunks from its prefix.
#pragma once
#include <utility>

#include "kata_device.h"
#include "kata_launch.h"

namespace kata {

hipError_t launch_scan(float* ws, int BH, int nslots, int64_t E, hipStream_t st);

namespace chk {

constexpr int NW = 4;
enum : int { K_DIAG = 0, K_WITHIN = 1, K_WITHIN8 = 2, K_CROSS = 3 };

template <int P> constexpr int ntiles() { return P == 32 ? 33 : 9; }
// tile -> (kind, half, delta); see the header comment for the feature of row m
template <int P> constexpr int tile_kind(int t) {
  if (P == 16) return t == 0 ? K_DIAG : (t < 8 ? K_WITHIN : K_WITHIN8);
  return t < 2 ? K_DIAG : (t < 16 ? K_WITHIN : (t == 16 ? K_WITHIN8 : K_CROSS));
}
template <int P> constexpr int tile_half(int t) {
  if (P == 16) return 0;
  return t < 2 ? t : (t < 16 ? (t - 2) / 7 : 0);
}
template <int P> constexpr int tile_delta(int t) {
  if (P == 16) return t == 0 ? 0 : (t < 8 ? t : 8);
  return t < 2 ? 0 : (t < 16 ? (t - 2) % 7 + 1 : (t == 16 ? 8 : t - 17));
}
// contiguous tile ranges per wave: p=32 -> 9,8,8,8; p=16 -> 3,2,2,2
template <int P> constexpr int wave_t0(int w) { return P == 32 ? (w == 0 ? 0 : 1 + 8 * w) : (w == 0 ? 0 : 1 + 2 * w); }
template <int P> constexpr int wave_nt(int w) { return P == 32 ? (w == 0 ? 9 : 8) : (w == 0 ? 3 : 2); }

// lane m of each 16-lane row receives x from lane (m + D) & 15 (DPP row_ror by 16 - D)
template <int D>
__device__ __forceinline__ float rot(float x) {
  if constexpr ((D & 15) == 0) return x;
  else
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                                  0x120 + (16 - (D & 15)), 0xf, 0xf, false));
}

__device__ __forceinline__ f32x4_t mfma(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t zero4() { return f32x4_t{0.f, 0.f, 0.f, 0.f}; }
__device__ __forceinline__ bf16x8_t zero_bf8() {
  return __builtin_bit_cast(bf16x8_t, u16x8_t{0, 0, 0, 0, 0, 0, 0, 0});
}

// A operand of the state build for tile TAU: row m = this lane's feature, 8 tokens.
// N[h][j] = k_hat[token j][16h + m]; N2 = 2 N (folds c_ij^2 = 2 of off-diagonal entries).
template <int P, int TAU>
__device__ __forceinline__ bf16x8_t build_frag(const float (&N)[P / 16][8], const float (&N2)[P / 16][8],
                                               bool mlow) {
  constexpr int kind = tile_kind<P>(TAU), h = tile_half<P>(TAU), d = tile_delta<P>(TAU);
  bf16x8_t r;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float x;
    if constexpr (kind == K_DIAG) {
      x = N[h][j] * N[h][j];
    } else if constexpr (kind == K_WITHIN) {
      x = N2[h][j] * rot<d>(N[h][j]);
    } else if constexpr (kind == K_WITHIN8) {
      if constexpr (P == 32) {
        const float a = mlow ? N2[0][j] : N2[1][j];
        const float b = mlow ? N[1][j] : N[0][j];
        x = a * rot<8>(b);
      } else {
        const float a = mlow ? N2[0][j] : 0.f;
        x = a * rot<8>(N[0][j]);
      }
    } else {
      x = N2[0][j] * rot<d>(N[P / 16 - 1][j]);
    }
    r[j] = (__bf16)x;
  }
  return r;
}

// readout-side feature of row 4g + JJ of tile TAU for this lane's token, from
// Y[x] = q_hat[(x & ~15) | ((x + 4g) & 15)] (raw product; c^2 sits in the state)
template <int P, int TAU, int JJ>
__device__ __forceinline__ float ro_feat(const float (&Y)[P], bool glow) {
  constexpr int kind = tile_kind<P>(TAU), h = tile_half<P>(TAU), d = tile_delta<P>(TAU);
  if constexpr (kind == K_DIAG) {
    return Y[16 * h + JJ] * Y[16 * h + JJ];
  } else if constexpr (kind == K_WITHIN) {
    return Y[16 * h + JJ] * Y[16 * h + ((JJ + d) & 15)];
  } else if constexpr (kind == K_WITHIN8) {
    if constexpr (P == 32) {
      const float a = glow ? Y[JJ] : Y[16 + JJ];
      const float b = glow ? Y[(JJ + 8) & 15] : Y[16 + ((JJ + 8) & 15)];
      return a * b;
    } else {
      return glow ? Y[JJ] * Y[(JJ + 8) & 15] : 0.f;
    }
  } else {
    return Y[JJ] * Y[16 + ((JJ + d) & 15)];
  }
}

template <int P, int T1, int T2, bool HAS2>
__device__ __forceinline__ bf16x8_t readout_frag(const float (&Y)[P], bool glow) {
  bf16x8_t r;
  r[0] = (__bf16)ro_feat<P, T1, 0>(Y, glow);
  r[1] = (__bf16)ro_feat<P, T1, 1>(Y, glow);
  r[2] = (__bf16)ro_feat<P, T1, 2>(Y, glow);
  r[3] = (__bf16)ro_feat<P, T1, 3>(Y, glow);
  if constexpr (HAS2) {
    r[4] = (__bf16)ro_feat<P, T2, 0>(Y, glow);
    r[5] = (__bf16)ro_feat<P, T2, 1>(Y, glow);
    r[6] = (__bf16)ro_feat<P, T2, 2>(Y, glow);
    r[7] = (__bf16)ro_feat<P, T2, 3>(Y, glow);
  } else {
    r[4] = r[5] = r[6] = r[7] = (__bf16)0.f;
  }
  return r;
}

// split x (8 fp32) into bf16 hi and lo = bf16(x - hi)
__device__ __forceinline__ void split8(const float (&x)[8], bf16x8_t& hi, bf16x8_t& lo) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const __bf16 h = (__bf16)x[j];
    hi[j] = h;
    lo[j] = (__bf16)(x[j] - (float)h);
  }
}

template <int P, int DV, int C>
struct Cfg {
  static constexpr int NT = DV / 16;          // output column tiles
  static constexpr int NH = P / 16;           // 16-component halves
  static constexpr int NMT = C / 16;          // token tiles per chunk
  static constexpr int GMT = NMT < 4 ? NMT : 4;  // token tiles per readout group
  static constexpr int NG = NMT / GMT;        // readout groups per chunk
  static constexpr int KSTEP = C / 32;        // 32-token k-steps of the build
  static constexpr int QP = P + 4;            // fp32 pitch of q_hat / k_hat rows
  static constexpr int KTP = C + 4;           // fp32 pitch of k_hat^T rows
  static constexpr int VTP = C + 8;           // bf16 pitch of V^T rows
  static constexpr int MP = P + 8;            // bf16 pitch of the Gram matrix rows
  static constexpr int PP = DV + 4;           // fp32 pitch of the partial outputs
  static constexpr int NTL = ntiles<P>();
  static constexpr int64_t STATE_FLOATS = (int64_t)NTL * NT * 256 + NH * NH * 256;
  // LDS layout (bytes)
  static constexpr int OFF_QH = 0;
  static constexpr int OFF_KH = OFF_QH + C * QP * 4;
  static constexpr int OFF_KT = OFF_KH + C * QP * 4;
  static constexpr int OFF_VT = OFF_KT + P * KTP * 4;
  static constexpr int OFF_M = OFF_VT + DV * VTP * 2;           // [2 buf][hi,lo][P][MP] bf16
  static constexpr int OFF_DEN = OFF_M + 2 * 2 * P * MP * 2;
  static constexpr int OFF_PP = OFF_DEN + C * 4;
  static constexpr int LDS = OFF_PP + NW * GMT * 16 * PP * 4;
  static_assert(LDS <= 160 * 1024, "LDS budget");
  // global-load work per thread
  static constexpr int ROWS_PT = (C + 63) / 64;                // q/k rows per thread
  static constexpr int KQ = P / 4;                             // components per thread
  static constexpr int VPIECES = (C / 2) * (DV / 8);           // (key pair, 8 columns) pieces
  static constexpr int VPT = (VPIECES + 255) / 256;
};

struct Args {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  void* o;
  float* ws;
  int T, nseg, cps, nblk_per_bh;
  int o_f32;  // output dtype: 1 = fp32, 0 = bf16
};

// store CPL consecutive outputs of one row
template <int CPL>
__device__ __forceinline__ void store_row(const Args& a, int64_t off, const float (&s)[CPL], float inv) {
  if (a.o_f32) {
    float* ob = static_cast<float*>(a.o) + off;
#pragma unroll
    for (int e = 0; e < CPL; e += 4)
      *reinterpret_cast<f32x4_t*>(ob + e) = f32x4_t{s[e] * inv, s[e + 1] * inv, s[e + 2] * inv, s[e + 3] * inv};
  } else {
    uint16_t* ob = static_cast<uint16_t*>(a.o) + off;
#pragma unroll
    for (int e = 0; e < CPL; e += 4)
      *reinterpret_cast<u16x4_t*>(ob + e) = u16x4_t{f32_to_bf16_bits(s[e] * inv), f32_to_bf16_bits(s[e + 1] * inv),
                                                    f32_to_bf16_bits(s[e + 2] * inv), f32_to_bf16_bits(s[e + 3] * inv)};
  }
}

// ---- chunk staging: global bf16 -> registers (prefetch) -> normalised LDS (stage)
template <int P, int DV, int C, bool WITH_Q>
struct Stager {
  using CF = Cfg<P, DV, C>;
  uint16_t qr[CF::ROWS_PT][CF::KQ];
  uint16_t kr[CF::ROWS_PT][CF::KQ];
  u16x8_t vr[CF::VPT][2];

  __device__ __forceinline__ void load_row(uint16_t (&dst)[CF::KQ], const uint16_t* src) {
    if constexpr (CF::KQ == 8) *reinterpret_cast<u16x8_t*>(&dst[0]) = *reinterpret_cast<const u16x8_t*>(src);
    else *reinterpret_cast<u16x4_t*>(&dst[0]) = *reinterpret_cast<const u16x4_t*>(src);
  }

  __device__ __forceinline__ void prefetch(const Args& a, int64_t bh, int t0) {
    const int tid = threadIdx.x;
    const int kq = tid & 3;
#pragma unroll
    for (int i = 0; i < CF::ROWS_PT; ++i) {
      const int row = (tid >> 2) + 64 * i;
      const int t = t0 + row;
#pragma unroll
      for (int e = 0; e < CF::KQ; ++e) qr[i][e] = kr[i][e] = 0;
      if (row < C && t < a.T) {
        const int64_t off = (bh * a.T + t) * P + kq * CF::KQ;
        if (WITH_Q) load_row(qr[i], a.q + off);
        load_row(kr[i], a.k + off);
      }
    }
#pragma unroll
    for (int i = 0; i < CF::VPT; ++i) {
      const int pc = tid + 256 * i;
      vr[i][0] = vr[i][1] = u16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
      if (pc < CF::VPIECES) {
        const int vp = pc / (DV / 8), vd = pc % (DV / 8);
        const int t = t0 + 2 * vp;
        const uint16_t* src = a.v + (bh * a.T + t) * DV + 8 * vd;
        if (t < a.T) vr[i][0] = *reinterpret_cast<const u16x8_t*>(src);
        if (t + 1 < a.T) vr[i][1] = *reinterpret_cast<const u16x8_t*>(src + DV);
      }
    }
  }

  __device__ __forceinline__ void stage(char* lds) {
    const int tid = threadIdx.x;
    const int kq = tid & 3;
    float* qh = reinterpret_cast<float*>(lds + CF::OFF_QH);
    float* kh = reinterpret_cast<float*>(lds + CF::OFF_KH);
    float* kt = reinterpret_cast<float*>(lds + CF::OFF_KT);
    uint32_t* vt = reinterpret_cast<uint32_t*>(lds + CF::OFF_VT);
#pragma unroll
    for (int i = 0; i < CF::ROWS_PT; ++i) {
      const int row = (tid >> 2) + 64 * i;
#pragma unroll
      for (int isq = 0; isq < (WITH_Q ? 2 : 1); ++isq) {
        const uint16_t(&src)[CF::KQ] = (WITH_Q && isq == 0) ? qr[i] : kr[i];
        float x[CF::KQ];
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < CF::KQ; ++e) {
          x[e] = bf16_bits_to_f32(src[e]);
          ss += x[e] * x[e];
        }
        ss += __shfl_xor(ss, 1, 64);
        ss += __shfl_xor(ss, 2, 64);
        const float inv = inv_norm(ss);
        if (row < C) {
          float* dst = ((WITH_Q && isq == 0) ? qh : kh) + row * CF::QP + kq * CF::KQ;
#pragma unroll
          for (int e = 0; e < CF::KQ; ++e) {
            x[e] *= inv;
            dst[e] = x[e];
          }
          if (!(WITH_Q && isq == 0)) {
#pragma unroll
            for (int e = 0; e < CF::KQ; ++e) kt[(kq * CF::KQ + e) * CF::KTP + row] = x[e];
          }
        }
      }
    }
#pragma unroll
    for (int i = 0; i < CF::VPT; ++i) {
      const int pc = tid + 256 * i;
      if (pc < CF::VPIECES) {
        const int vp = pc / (DV / 8), vd = pc % (DV / 8);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          vt[((8 * vd + e) * CF::VTP + 2 * vp) >> 1] = (uint32_t)vr[i][0][e] | ((uint32_t)vr[i][1][e] << 16);
      }
    }
  }
};

// ---- per-wave body; W (wave index) is a template parameter so every tile index is a
// compile-time constant and the lift indexes registers directly.
template <int P, int DV, int C, bool FWD, int W>
__device__ __forceinline__ void run_wave(const Args& a, char* lds) {
  using CF = Cfg<P, DV, C>;
  constexpr int NT = CF::NT, NH = CF::NH, NTW = wave_nt<P>(W), T0 = wave_t0<P>(W);
  constexpr int NPAIR = (NTW + 1) / 2;
  constexpr bool OWN_M = W < NH * NH;
  constexpr int MRT = W / NH, MCT = W % NH;  // Gram tile owned (when OWN_M)
  const int lane = threadIdx.x & 63, ln = lane & 15, lg = lane >> 4;
  const bool mlow = ln < 8, glow = lg < 2;

  float* qh = reinterpret_cast<float*>(lds + CF::OFF_QH);
  float* kh = reinterpret_cast<float*>(lds + CF::OFF_KH);
  float* khT = reinterpret_cast<float*>(lds + CF::OFF_KT);
  uint16_t* vt = reinterpret_cast<uint16_t*>(lds + CF::OFF_VT);
  uint16_t* mlds = reinterpret_cast<uint16_t*>(lds + CF::OFF_M);
  float* den = reinterpret_cast<float*>(lds + CF::OFF_DEN);
  float* pp = reinterpret_cast<float*>(lds + CF::OFF_PP);

  const int64_t bh = blockIdx.x / a.nblk_per_bh;
  const int seg = blockIdx.x % a.nblk_per_bh;
  const int nchunks = (a.T + C - 1) / C;
  const int c0 = seg * a.cps;
  const int c1 = min(nchunks, c0 + a.cps);

  // ---- initial state
  f32x4_t S[NTW][NT];
  f32x4_t Mt = zero4();
  const bool from_ws = FWD && seg > 0;
  {
    const float* src = from_ws ? a.ws + (bh * (a.nseg - 1) + (seg - 1)) * CF::STATE_FLOATS : nullptr;
#pragma unroll
    for (int i = 0; i < NTW; ++i)
#pragma unroll
      for (int dt = 0; dt < NT; ++dt)
        S[i][dt] = from_ws ? *reinterpret_cast<const f32x4_t*>(src + (((T0 + i) * NT + dt) * 64 + lane) * 4) : zero4();
    if constexpr (OWN_M)
      if (from_ws) Mt = *reinterpret_cast<const f32x4_t*>(src + (int64_t)CF::NTL * NT * 256 + (W * 64 + lane) * 4);
  }
  auto write_m = [&](int buf) {  // Gram tile -> LDS as bf16 hi / lo
    if constexpr (OWN_M) {
      uint16_t* mh = mlds + (buf * 2 + 0) * P * CF::MP;
      uint16_t* ml = mlds + (buf * 2 + 1) * P * CF::MP;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * MRT + 4 * lg + r, col = 16 * MCT + ln;
        const uint16_t h = f32_to_bf16_bits(Mt[r]);
        mh[row * CF::MP + col] = h;
        ml[row * CF::MP + col] = f32_to_bf16_bits(Mt[r] - bf16_bits_to_f32(h));
      }
    }
  };
  bf16x8_t Sb[NPAIR][NT];
  auto convert_state = [&]() {
#pragma unroll
    for (int pi = 0; pi < NPAIR; ++pi)
#pragma unroll
      for (int dt = 0; dt < NT; ++dt) {
        bf16x8_t b;
#pragma unroll
        for (int r = 0; r < 4; ++r) b[r] = (__bf16)S[2 * pi][dt][r];
#pragma unroll
        for (int r = 0; r < 4; ++r) b[4 + r] = (2 * pi + 1 < NTW) ? (__bf16)S[2 * pi + 1 < NTW ? 2 * pi + 1 : 0][dt][r] : (__bf16)0.f;
        Sb[pi][dt] = b;
      }
  };
  if constexpr (FWD) convert_state();
  write_m(c0 & 1);

  Stager<P, DV, C, FWD> stg;
  stg.prefetch(a, bh, c0 * C);
  stg.stage(lds);
  __syncthreads();

  for (int c = c0; c < c1; ++c) {
    const int t0 = c * C;
    const int cur = c & 1;
    if (c + 1 < c1) stg.prefetch(a, bh, t0 + C);

    if constexpr (FWD) {
      const bool split = c == 0;
      // ---- intra-chunk block and denominator for the token tiles this wave owns
      f32x4_t Oi[(CF::NMT + 3) / 4][NT];
#pragma unroll
      for (int oi = 0; oi < (CF::NMT + 3) / 4; ++oi) {
        const int mt = W + 4 * oi;
#pragma unroll
        for (int dt = 0; dt < NT; ++dt) Oi[oi][dt] = zero4();
        if (mt >= CF::NMT) continue;
        // query operand (B of S^T and of X^T): q_hat[16mt + ln][8lg..8lg+7]
        bf16x8_t qbh = zero_bf8(), qbl = zero_bf8();
        if (P == 32 || lg < 2) {
          const float* src = qh + (16 * mt + ln) * CF::QP + 8 * lg;
          const f32x4_t x0 = *reinterpret_cast<const f32x4_t*>(src);
          const f32x4_t x1 = *reinterpret_cast<const f32x4_t*>(src + 4);
          const float xs[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
          split8(xs, qbh, qbl);
        }
        // den_inter partial: X^T = M Q_hat^T (rows: components), then q_hat . X
        float dpart = 0.f;
#pragma unroll
        for (int rt = 0; rt < NH; ++rt) {
          bf16x8_t mh = zero_bf8(), ml = zero_bf8();
          if (P == 32 || lg < 2) {
            const uint16_t* mrow = mlds + (cur * 2) * P * CF::MP + (16 * rt + ln) * CF::MP + 8 * lg;
            mh = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u16x8_t*>(mrow));
            ml = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u16x8_t*>(mrow + P * CF::MP));
          }
          f32x4_t X = zero4();
          X = mfma(mh, qbh, X);
          X = mfma(ml, qbh, X);
          X = mfma(mh, qbl, X);
          const f32x4_t qv = *reinterpret_cast<const f32x4_t*>(qh + (16 * mt + ln) * CF::QP + 16 * rt + 4 * lg);
          dpart += X[0] * qv[0] + X[1] * qv[1] + X[2] * qv[2] + X[3] * qv[3];
        }
        // S^T = K_hat Q_hat^T over key tiles kt <= mt; W = (S^T)^2; O += W V
#pragma unroll
        for (int kp = 0; kp < (CF::NMT + 1) / 2; ++kp) {
          if (2 * kp > mt) continue;
          float wv[8];
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const int kt = 2 * kp + half;
            f32x4_t St = zero4();
            if (kt <= mt) {
              bf16x8_t kbh = zero_bf8(), kbl = zero_bf8();
              if (P == 32 || lg < 2) {
                const float* src = kh + (16 * kt + ln) * CF::QP + 8 * lg;
                const f32x4_t x0 = *reinterpret_cast<const f32x4_t*>(src);
                const f32x4_t x1 = *reinterpret_cast<const f32x4_t*>(src + 4);
                const float xs[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
                split8(xs, kbh, kbl);
              }
              St = mfma(kbh, qbh, St);
              if (split) {
                St = mfma(kbl, qbh, St);
                St = mfma(kbh, qbl, St);
              }
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              float w = St[r] * St[r];
              if (kt == mt && 4 * lg + r > ln) w = 0.f;  // causal: key <= query
              if (kt > mt) w = 0.f;
              const __bf16 wb = (__bf16)w;
              wv[4 * half + r] = (float)wb;
              dpart += (float)wb;
            }
          }
          bf16x8_t wa;
#pragma unroll
          for (int j = 0; j < 8; ++j) wa[j] = (__bf16)wv[j];
#pragma unroll
          for (int dt = 0; dt < NT; ++dt) {
            const uint16_t* row = vt + (16 * dt + ln) * CF::VTP + 32 * kp + 4 * lg;
            const u16x4_t x0 = *reinterpret_cast<const u16x4_t*>(row);
            const u16x4_t x1 = *reinterpret_cast<const u16x4_t*>(row + 16);
            const bf16x8_t vb = __builtin_bit_cast(bf16x8_t, u16x8_t{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]});
            Oi[oi][dt] = mfma(wa, vb, Oi[oi][dt]);
          }
        }
        dpart += __shfl_xor(dpart, 16, 64);
        dpart += __shfl_xor(dpart, 32, 64);
        if (lg == 0) den[16 * mt + ln] = dpart;
      }

      // ---- readout psi(Q) S over this wave's features, per token group
#pragma unroll
      for (int g = 0; g < CF::NG; ++g) {
#pragma unroll
        for (int ml = 0; ml < CF::GMT; ++ml) {
          const int mt = g * CF::GMT + ml;
          f32x4_t acc[NT];
#pragma unroll
          for (int dt = 0; dt < NT; ++dt) acc[dt] = (mt % 4 == W) ? Oi[mt / 4][dt] : zero4();
          float Y[P];
          {
            const float* src = qh + (16 * mt + ln) * CF::QP;
#pragma unroll
            for (int h = 0; h < NH; ++h)
#pragma unroll
              for (int u = 0; u < 4; ++u) {
                const f32x4_t x = *reinterpret_cast<const f32x4_t*>(src + 16 * h + ((4 * u + 4 * lg) & 15));
#pragma unroll
                for (int e = 0; e < 4; ++e) Y[16 * h + 4 * u + e] = x[e];
              }
          }
          [&]<int... PI>(std::integer_sequence<int, PI...>) {
            (([&] {
               constexpr int t1 = T0 + 2 * PI, t2 = T0 + 2 * PI + 1;
               constexpr bool has2 = 2 * PI + 1 < NTW;
               const bf16x8_t af = readout_frag<P, t1, has2 ? t2 : t1, has2>(Y, glow);
#pragma unroll
               for (int dt = 0; dt < NT; ++dt) acc[dt] = mfma(af, Sb[PI][dt], acc[dt]);
             }()),
             ...);
          }(std::make_integer_sequence<int, NPAIR>{});
          float* dst = pp + (W * CF::GMT + ml) * 16 * CF::PP;
#pragma unroll
          for (int dt = 0; dt < NT; ++dt)
#pragma unroll
            for (int r = 0; r < 4; ++r) dst[(4 * lg + r) * CF::PP + 16 * dt + ln] = acc[dt][r];
        }
        if (g + 1 < CF::NG) {
          __syncthreads();
          if (W < CF::GMT) {
            // reduce (same code as after the build, for an earlier token group)
            const int mt = g * CF::GMT + W;
            constexpr int CPL = DV / 4;
            const int row = lane >> 2, col0 = (lane & 3) * CPL;
            const int t = t0 + 16 * mt + row;
            float s[CPL];
#pragma unroll
            for (int e = 0; e < CPL; ++e) s[e] = 0.f;
#pragma unroll
            for (int w2 = 0; w2 < NW; ++w2) {
              const float* src = pp + ((w2 * CF::GMT + W) * 16 + row) * CF::PP + col0;
#pragma unroll
              for (int e = 0; e < CPL; e += 4) {
                const f32x4_t x = *reinterpret_cast<const f32x4_t*>(src + e);
                s[e] += x[0]; s[e + 1] += x[1]; s[e + 2] += x[2]; s[e + 3] += x[3];
              }
            }
            const float dn = den[16 * mt + row];
            const float inv = dn > 0.f ? 1.0f / dn : 0.f;
            if (t < a.T) store_row<CPL>(a, (bh * a.T + t) * DV + col0, s, inv);
          }
          __syncthreads();
        }
      }
    }

    // ---- state build: S += psi(K_c)^T V_c over this wave's tiles; Gram tile update
#pragma unroll
    for (int ks = 0; ks < CF::KSTEP; ++ks) {
      float N[NH][8], N2[NH][8];
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        const float* src = khT + (16 * h + ln) * CF::KTP + 32 * ks + 8 * lg;
        const f32x4_t x0 = *reinterpret_cast<const f32x4_t*>(src);
        const f32x4_t x1 = *reinterpret_cast<const f32x4_t*>(src + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          N[h][e] = x0[e];
          N[h][4 + e] = x1[e];
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) N2[h][e] = 2.f * N[h][e];
      }
      bf16x8_t vb[NT];
#pragma unroll
      for (int dt = 0; dt < NT; ++dt)
        vb[dt] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u16x8_t*>(vt + (16 * dt + ln) * CF::VTP + 32 * ks + 8 * lg));
      [&]<int... TI>(std::integer_sequence<int, TI...>) {
        (([&] {
           const bf16x8_t af = build_frag<P, T0 + TI>(N, N2, mlow);
#pragma unroll
           for (int dt = 0; dt < NT; ++dt) S[TI][dt] = mfma(af, vb[dt], S[TI][dt]);
         }()),
         ...);
      }(std::make_integer_sequence<int, NTW>{});
      if constexpr (OWN_M) {
        bf16x8_t ah, al, bh_, bl;
        split8(N[MRT], ah, al);
        split8(N[MCT], bh_, bl);
        Mt = mfma(ah, bh_, Mt);
        Mt = mfma(al, bh_, Mt);
        Mt = mfma(ah, bl, Mt);
      }
    }
    write_m(cur ^ 1);
    if constexpr (FWD) convert_state();
    __syncthreads();

    if constexpr (FWD) {
      // ---- combine the 4 partial outputs of the last token group, normalise, store
      if (W < CF::GMT) {
        const int mt = (CF::NG - 1) * CF::GMT + W;
        constexpr int CPL = DV / 4;
        const int row = lane >> 2, col0 = (lane & 3) * CPL;
        const int t = t0 + 16 * mt + row;
        float s[CPL];
#pragma unroll
        for (int e = 0; e < CPL; ++e) s[e] = 0.f;
#pragma unroll
        for (int w2 = 0; w2 < NW; ++w2) {
          const float* src = pp + ((w2 * CF::GMT + W) * 16 + row) * CF::PP + col0;
#pragma unroll
          for (int e = 0; e < CPL; e += 4) {
            const f32x4_t x = *reinterpret_cast<const f32x4_t*>(src + e);
            s[e] += x[0]; s[e + 1] += x[1]; s[e + 2] += x[2]; s[e + 3] += x[3];
          }
        }
        const float dn = den[16 * mt + row];
        const float inv = dn > 0.f ? 1.0f / dn : 0.f;
        if (t < a.T) store_row<CPL>(a, (bh * a.T + t) * DV + col0, s, inv);
      }
    }
    if (c + 1 < c1) stg.stage(lds);
    __syncthreads();
  }

  if constexpr (!FWD) {  // segment summary -> workspace slot seg
    float* dst = a.ws + (bh * (a.nseg - 1) + seg) * CF::STATE_FLOATS;
#pragma unroll
    for (int i = 0; i < NTW; ++i)
#pragma unroll
      for (int dt = 0; dt < NT; ++dt)
        *reinterpret_cast<f32x4_t*>(dst + (((T0 + i) * NT + dt) * 64 + lane) * 4) = S[i][dt];
    if constexpr (OWN_M)
      *reinterpret_cast<f32x4_t*>(dst + (int64_t)CF::NTL * NT * 256 + (W * 64 + lane) * 4) = Mt;
  }
}

template <int P, int DV, int C, bool FWD>
__global__ __launch_bounds__(256, 1) void chunked_bf16_kernel(Args a) {
  __shared__ __align__(16) char lds[Cfg<P, DV, C>::LDS];
  switch (threadIdx.x >> 6) {
    case 0: run_wave<P, DV, C, FWD, 0>(a, lds); break;
    case 1: run_wave<P, DV, C, FWD, 1>(a, lds); break;
    case 2: run_wave<P, DV, C, FWD, 2>(a, lds); break;
    default: run_wave<P, DV, C, FWD, 3>(a, lds); break;
  }
}

template <int P, int DV, int C>
hipError_t launch_pdc(const uint16_t* q, const uint16_t* k, const uint16_t* v, void* o, bool o_bf16,
                      int B, int H, int T, const SegPlan& plan, float* ws, hipStream_t st) {
  const int BH = B * H;
  Args a{q, k, v, o, ws, T, plan.nseg, plan.cps, 0, o_bf16 ? 0 : 1};
  hipError_t e;
  if (plan.nseg > 1) {
    a.nblk_per_bh = plan.nseg - 1;
    chunked_bf16_kernel<P, DV, C, false><<<dim3((unsigned)(BH * (plan.nseg - 1))), dim3(256), 0, st>>>(a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = launch_scan(ws, BH, plan.nseg - 1, Cfg<P, DV, C>::STATE_FLOATS, st)) != hipSuccess) return e;
  }
  a.nblk_per_bh = plan.nseg;
  chunked_bf16_kernel<P, DV, C, true><<<dim3((unsigned)(BH * plan.nseg)), dim3(256), 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace chk

}  // namespace kata
