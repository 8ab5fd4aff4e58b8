// O(T) gradients of the causal full-map forward on bf16 MFMA (bf16 q, k, v, grad_o;
// p in {16, 32}, dv in {32, 64}).
//
// Source: "Kernelized Linear Attention: Breaking the Capacity Wall with Symmetric Cones"
// (arXiv 2607.17419), HTML page: feature-value state display (S_t, Z_t), normalized-readout
// paragraph, chunked-forward paragraph (additive chunk states, associative prefix). The pages
// give no backward pass; the calculus is that of the fp32 state-form kernels. With q_hat,
// k_hat the unit rows, D_t = psi(q_hat_t)^T Z_t, delta_t = g_t . o_t, a_t = g_t / D_t and
// b_t = -delta_t / D_t:
//   dpsi(q_hat_t) = S_t a_t + Z_t b_t,   R_s = sum_{t>=s} psi(q_hat_t) a_t^T (r_s with b_t),
//   dpsi(k_hat_s) = R_s v_s + r_s,       dv_s = R_s^T psi(k_hat_s),
// then the lift's transpose and the projection onto the unit sphere's tangent. The Z and r
// parts reduce to Gram matrices: J^T (Z b_t) = 2 b_t M q_hat_t with M = sum k_hat k_hat^T,
// J^T r_s = 2 N k_hat_s with N = sum_{t>=s} b_t q_hat_t q_hat_t^T. Pairs inside a chunk use
// the weight identity: key s adds (v_s . a_t + b_t) 2 (q_hat_t . k_hat_s) k_hat_s to
// dq_hat_t, the same times q_hat_t to dk_hat_s, and w_ts a_t to dv_s.
//
// Pipeline on one stream: the segment summaries [S | 2M] of the bf16 chunked forward,
// scanned into prefixes, then
//   fdq  : forward time over 32-token chunks from each segment's prefix: D_t, delta_t
//          (stats) and dq. delta_t D_t = psi(q_hat_t)^T S g_t + sum_s w_ts v_s . g_t is formed
//          from the same state and weights as the gradient (not from a forward output), so
//          the difference v_s . g_t - delta_t that every pair term carries is exact where it
//          must vanish (at t = 0, o_0 = v_0 whatever q_0 is);
//   rsum : [R | 2N] of every segment but the first, scanned in reversed slot order so that a
//          slot holds the suffix of the segments after one;
//   rdk  : reverse time from each segment's suffix, two kernels that each rebuild R: dk (R v_s
//          through the lift's transpose) and dv (R^T psi(k_hat_s), a quarter of the feature
//          pairs of one key tile per wave, summed through LDS).
//
// Layouts. States use the feature tiles of the forward (33 tiles of 16 rows at p = 32, each
// row a pair (i, j) of components; see kata_chunked.h). fdq and the dk kernel build them with
// the forward build's MFMA operands swapped, S^T = V^T psi(K): lane (m, g) of a 16 x 16
// accumulator tile holds feature row m at value columns 16 dt + 4 g + r. Two column tiles of a
// feature tile are then directly an MFMA operand whose k-slots are 32 value columns, so S g_t
// and R v_s run from registers (g_t and v_s exact in bf16; 1 / D_t is applied to the summed
// result). Their result X^T (feature rows 4 g + r, one token per lane) goes through the lift's
// transpose inside the lane: the token's row is held rotated,
// Y[x] = u[(x & ~15) | ((x + 4 g) & 15)] as in the forward readout, every feature row of a tile
// is a product Y_a Y_b of two compile-time registers, and its gradient adds x Y_b to G[a] and
// x Y_a to G[b] of an equally rotated accumulator (the state carries c_f^2 like the forward's,
// so the lift's constants cancel). The lanes' G are summed in registers (lane groups g and
// g + 2, whose rotations differ by 8) and then across waves through per-wave LDS partials.
// R = sum_t psi(q_hat_t / sqrt(D_t)) g_t^T, which is A^T psi(Q) with the exact g_t as values.
// The dv kernel reads R only through the forward readout's fragments, so it builds R in the
// forward's orientation.
#include "kata_chunked.h"

namespace kata {
namespace cbm {
using namespace chk;

constexpr int CB = 32;   // tokens per chunk

template <int P, int DV>
struct Lay {
  static constexpr int NT = DV / 16, NH = P / 16, KQ = P / 4, NKS = DV / 32, NV8 = DV / 8;
  static constexpr int NTL = ntiles<P>(), NPAIR = (NTL + 1) / 2;
  // fp32 row pitch: 16 lanes reading 16 rows at one column with 16-byte reads then start at
  // 16 distinct 4-bank groups (at P + 8 = 40 floats only 8, a 2-way conflict; P + 4 measured
  // 3.6% faster over the whole backward, bitwise equal)
  static constexpr int QP = P + 4;
  static constexpr int TP = 80;      // transposed fp32 rows: token t of component c at c TP + 8 (c / KQ) + t
  static constexpr int VTP = 80;     // transposed bf16 rows, token t at vt_pos(t)
  static constexpr int RP = DV + 8;  // bf16 row pitch
  static constexpr int MP = P + 8;   // bf16 pitch of the Gram halves
  static constexpr int64_t STATE = (int64_t)NTL * NT * 256 + NH * NH * 256;
  static_assert(CB * (DV / 8) <= 256, "value pieces fit waves 4..7");
};

// ---- lift transpose: feature row 4 lg + JJ of tile TAU (see ro_feat) with X^T value x
template <int P, int TAU, int JJ>
__device__ __forceinline__ void tr_feat(float (&G)[P], const float (&Y)[P], float x, bool glow) {
  constexpr int kind = tile_kind<P>(TAU), h = tile_half<P>(TAU), d = tile_delta<P>(TAU);
  if constexpr (kind == K_DIAG) {
    constexpr int a = 16 * h + JJ;
    G[a] += 2.f * x * Y[a];
  } else if constexpr (kind == K_WITHIN) {
    constexpr int a = 16 * h + JJ, b = 16 * h + ((JJ + d) & 15);
    G[a] += x * Y[b];
    G[b] += x * Y[a];
  } else if constexpr (kind == K_WITHIN8) {
    constexpr int a0 = JJ, b0 = (JJ + 8) & 15;
    const float xl = glow ? x : 0.f;
    G[a0] += xl * Y[b0];
    G[b0] += xl * Y[a0];
    if constexpr (P == 32) {
      constexpr int a1 = 16 + JJ, b1 = 16 + ((JJ + 8) & 15);
      const float xh = glow ? 0.f : x;
      G[a1] += xh * Y[b1];
      G[b1] += xh * Y[a1];
    }
  } else {
    constexpr int a = JJ, b = 16 + ((JJ + d) & 15);
    G[a] += x * Y[b];
    G[b] += x * Y[a];
  }
}
template <int P, int TAU>
__device__ __forceinline__ void tr_tile(float (&G)[P], const float (&Y)[P], const f32x4_t& X, bool glow) {
  tr_feat<P, TAU, 0>(G, Y, X[0], glow);
  tr_feat<P, TAU, 1>(G, Y, X[1], glow);
  tr_feat<P, TAU, 2>(G, Y, X[2], glow);
  tr_feat<P, TAU, 3>(G, Y, X[3], glow);
}

// A operand over value columns 32 ks + 4 lg + j, 32 ks + 16 + 4 lg + j from two swapped
// accumulator tiles
template <int NT>
__device__ __forceinline__ bf16x8_t sfrag(const f32x4_t (&Sd)[NT], int ks) {
  const f32x4_t& x = Sd[2 * ks];
  const f32x4_t& y = Sd[2 * ks + 1];
  return __builtin_bit_cast(bf16x8_t, u32x4_t{pk2(x[0], x[1]), pk2(x[2], x[3]), pk2(y[0], y[1]), pk2(y[2], y[3])});
}
// the same k-slots of a bf16 row (columns 32 ks + 4 lg .. + 3 and 32 ks + 16 + 4 lg .. + 3)
__device__ __forceinline__ bf16x8_t row_frag(const uint16_t* row, int ks, int lg) {
  const u32x2_t lo = *reinterpret_cast<const u32x2_t*>(row + 32 * ks + 4 * lg);
  const u32x2_t hi = *reinterpret_cast<const u32x2_t*>(row + 32 * ks + 16 + 4 * lg);
  return __builtin_bit_cast(bf16x8_t, u32x4_t{lo[0], lo[1], hi[0], hi[1]});
}
// components 4 lg .. + 3 and 16 + 4 lg .. + 3 of an fp32 row
template <int P>
__device__ __forceinline__ void comp8(const float* row, int lg, float (&x)[8]) {
  const f32x4_t x0 = *reinterpret_cast<const f32x4_t*>(row + 4 * lg);
  const f32x4_t x1 = P == 32 ? *reinterpret_cast<const f32x4_t*>(row + 16 + 4 * lg) : f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[e] = x0[e];
    x[4 + e] = x1[e];
  }
}
// the row rotated per lane group: Y[x] = u[(x & ~15) | ((x + 4 lg) & 15)]
template <int P>
__device__ __forceinline__ void rot_row(const float* row, int lg, float (&Y)[P]) {
#pragma unroll
  for (int h = 0; h < P / 16; ++h)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const f32x4_t x = *reinterpret_cast<const f32x4_t*>(row + 16 * h + ((4 * u + 4 * lg) & 15));
#pragma unroll
      for (int e = 0; e < 4; ++e) Y[16 * h + 4 * u + e] = x[e];
    }
}
// sqrt(2)-scaled transposed rows (components 16 h + ln, token slots 4 lg + j and 16 + 4 lg + j)
template <int P>
__device__ __forceinline__ void tr_rows(const float* tp, int ln, int lg, float (&N)[P / 16][8]) {
  constexpr int TP = 80, KQ = P / 4;
#pragma unroll
  for (int h = 0; h < P / 16; ++h) {
    const float* src = tp + (16 * h + ln) * TP + 8 * ((16 * h + ln) / KQ) + 4 * lg;
    const f32x4_t x0 = *reinterpret_cast<const f32x4_t*>(src);
    const f32x4_t x1 = *reinterpret_cast<const f32x4_t*>(src + 16);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      N[h][e] = x0[e];
      N[h][4 + e] = x1[e];
    }
  }
}
// Gram halves (bf16 hi, lo) of m at [2][P][MP] from a Gram tile holding 2 m
template <int P, int MT>
__device__ __forceinline__ void write_gram(uint16_t* mm, const f32x4_t& Mt, int ln, int lg) {
  constexpr int NH = P / 16, MP = P + 8;
  if constexpr (MT >= 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 16 * (MT / NH) + 4 * lg + r, col = 16 * (MT % NH) + ln;
      const float m = 0.5f * Mt[r];
      const uint16_t h = f32_to_bf16_bits(m);
      mm[row * MP + col] = h;
      mm[P * MP + row * MP + col] = f32_to_bf16_bits(m - bf16_bits_to_f32(h));
    }
  }
}
// X^T = m u for the token of this lane (u exact in bf16 as the B operand), rows 16 rt + 4 lg + r
template <int P>
__device__ __forceinline__ void gram_apply(const uint16_t* mm, bf16x8_t ub, int ln, int lg, f32x4_t (&X)[P / 16]) {
  constexpr int MP = P + 8;
#pragma unroll
  for (int rt = 0; rt < P / 16; ++rt) {
    const uint16_t* mrow = mm + (16 * rt + ln) * MP + 4 * lg;
    const u32x2_t h0 = *reinterpret_cast<const u32x2_t*>(mrow);
    const u32x2_t l0 = *reinterpret_cast<const u32x2_t*>(mrow + P * MP);
    const u32x2_t h1 = P == 32 ? *reinterpret_cast<const u32x2_t*>(mrow + 16) : u32x2_t{0, 0};
    const u32x2_t l1 = P == 32 ? *reinterpret_cast<const u32x2_t*>(mrow + P * MP + 16) : u32x2_t{0, 0};
    X[rt] = mfma(__builtin_bit_cast(bf16x8_t, u32x4_t{h0[0], h0[1], h1[0], h1[1]}), ub, zero4());
    X[rt] = mfma(__builtin_bit_cast(bf16x8_t, u32x4_t{l0[0], l0[1], l1[0], l1[1]}), ub, X[rt]);
  }
}
// Lanes 0..31 end with the sum of this lane's G and that of lane + 32 (lane group lg + 2,
// whose rotation differs by 8: its element x ^ 8 is this lane's element x); the upper half's
// G is left as it was.
template <int P>
__device__ __forceinline__ void pair_sum_lo(float (&G)[P]) {
  float H[P];
#pragma unroll
  for (int x = 0; x < P; ++x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(G[x ^ 8]), __float_as_uint(G[x]), false, false);
    H[x] = __uint_as_float(r[1]);  // lanes 0..31: G[x ^ 8] of lane + 32
  }
#pragma unroll
  for (int x = 0; x < P; ++x) G[x] += H[x];
}
// rotated G of lane group lg (< 2) stored un-rotated as row t of a [rows][P + 4] fp32 slot
template <int P>
__device__ __forceinline__ void store_rotated(float* slot, const float (&G)[P], int t, int lg) {
#pragma unroll
  for (int h = 0; h < P / 16; ++h)
#pragma unroll
    for (int u = 0; u < 4; ++u)
      *reinterpret_cast<f32x4_t*>(slot + t * (P + 4) + 16 * h + ((4 * u + 4 * lg) & 15)) =
          f32x4_t{G[16 * h + 4 * u], G[16 * h + 4 * u + 1], G[16 * h + 4 * u + 2], G[16 * h + 4 * u + 3]};
}

// ---- per-thread staging of one chunk: waves 0-1 q pieces, 2-3 k pieces (4 threads per row),
// waves 4-7 value-row pieces (8 columns each)
template <int P, int DV, int W>
struct Piece {
  using LY = Lay<P, DV>;
  static constexpr int KQ = LY::KQ, NV8 = LY::NV8;
  static constexpr bool ISQ = W < 2, ISK = W >= 2 && W < 4;
  static constexpr bool ISV = W >= 4 && 64 * (W - 4) < CB * NV8;
  typedef uint16_t row_t __attribute__((ext_vector_type(KQ)));
  __device__ static __forceinline__ int pc() { return 64 * (W & (W < 4 ? 1 : 3)) + (threadIdx.x & 63); }
  __device__ static __forceinline__ int row() { return ISV ? pc() / NV8 : pc() >> 2; }
  __device__ static __forceinline__ int sub() { return ISV ? pc() % NV8 : pc() & 3; }
  __device__ static __forceinline__ row_t load_qk(const uint16_t* base, int64_t r, bool ok) {
    row_t x;
    if (ok) x = *reinterpret_cast<const row_t*>(base + r * P + sub() * KQ);
    else
      for (int e = 0; e < KQ; ++e) x[e] = 0;
    return x;
  }
  // the piece as fp32 and its row's inverse norm (4 lanes per row)
  __device__ static __forceinline__ float unpack(const row_t& x, float (&f)[KQ]) {
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < KQ; ++e) {
      f[e] = bf16_bits_to_f32(x[e]);
      ss += f[e] * f[e];
    }
    return inv_norm(group_sum<4>(ss));
  }
};

// ============================================================ forward time: stats and dq
struct FArgs {
  const uint16_t *q, *k, *v, *g;
  const float* fws;   // forward segment prefixes (forward tile layout), slot s after segment s
  float* stats;       // [rows][2]: D_t, delta_t
  float* dq;          // [rows][P]
  int T, nseg, seg_chunks;
  SeqLayout lay;      // row layout (padded [B, H, T] or packed token-major) and lengths
  int H;
};

template <int P, int DV>
struct FL {
  using LY = Lay<P, DV>;
  static constexpr int QR = 0;                                 // raw q rows fp32 [CB][QP]
  static constexpr int QH = QR + CB * LY::QP * 4;              // q_hat rows fp32 [2][CB][QP]
  static constexpr int KH = QH + 2 * CB * LY::QP * 4;          // k_hat rows fp32 [CB][QP]
  static constexpr int KT = KH + CB * LY::QP * 4;              // sqrt2 k_hat^T fp32 [P][TP]
  static constexpr int VT = KT + P * LY::TP * 4;               // V^T bf16 [DV][VTP]
  static constexpr int VR = VT + DV * LY::VTP * 2;             // v rows bf16 [CB][RP]
  static constexpr int GR = VR + CB * LY::RP * 2;              // g rows bf16
  static constexpr int MM = GR + CB * LY::RP * 2;              // Gram halves bf16 [2][P][MP]
  static constexpr int GP = MM + 2 * P * LY::MP * 2;           // dq_hat partials fp32 [8 waves x 2][CB][P + 4]
  static constexpr int G2 = GP + 16 * CB * (P + 4) * 4;        // the owners' part of dq_hat [CB][P + 4]
  static constexpr int IQ = G2 + CB * (P + 4) * 4;             // 1 / |q| [2][CB]
  static constexpr int DL = IQ + 2 * CB * 4;                   // psi(q_hat)^T S g partials [8 waves][CB]
  static constexpr int ID = DL + 8 * CB * 4;                   // 1 / D [CB]
  static constexpr int BYTES = ID + CB * 4;
  static_assert(BYTES <= 160 * 1024, "LDS budget");
};

template <int P, int DV, int W>
struct FStage : Piece<P, DV, W> {
  using B = Piece<P, DV, W>;
  using LY = Lay<P, DV>;
  using FLY = FL<P, DV>;
  typename B::row_t x;
  u16x8_t vv, gg;
  // rows t0 .. of the sequence at row0 + t step (rows at or past len read as zero)
  __device__ __forceinline__ void load(const FArgs& a, int64_t row0, int step, int len, int t0) {
    const int t = t0 + B::row();
    const bool ok = t >= 0 && t < len;
    const int64_t row = row0 + (int64_t)t * step;
    if constexpr (B::ISQ) x = B::load_qk(a.q, row, ok);
    if constexpr (B::ISK) x = B::load_qk(a.k, row, ok);
    if constexpr (B::ISV) {
      if (ok) {
        const int64_t off = row * DV + 8 * B::sub();
        vv = *reinterpret_cast<const u16x8_t*>(a.v + off);
        gg = *reinterpret_cast<const u16x8_t*>(a.g + off);
      } else {
        for (int e = 0; e < 8; ++e) vv[e] = gg[e] = 0;
      }
    }
  }
  __device__ __forceinline__ void stage(char* lds, int buf) {
    const int r = B::row(), s = B::sub();
    if constexpr (B::ISQ || B::ISK) {
      float f[B::KQ];
      const float inv = B::unpack(x, f);
      if constexpr (B::ISQ) {
        float* qr = reinterpret_cast<float*>(lds + FLY::QR) + r * LY::QP + s * B::KQ;
        float* qh = reinterpret_cast<float*>(lds + FLY::QH) + (buf * CB + r) * LY::QP + s * B::KQ;
#pragma unroll
        for (int e = 0; e < B::KQ; ++e) {
          qr[e] = f[e];
          qh[e] = f[e] * inv;
        }
        if (s == 0) reinterpret_cast<float*>(lds + FLY::IQ)[buf * CB + r] = inv;
      } else {
        float* kh = reinterpret_cast<float*>(lds + FLY::KH) + r * LY::QP + s * B::KQ;
        float* kt = reinterpret_cast<float*>(lds + FLY::KT) + (s * B::KQ) * LY::TP + 8 * s + r;
#pragma unroll
        for (int e = 0; e < B::KQ; ++e) {
          kh[e] = f[e] * inv;
          kt[e * LY::TP] = f[e] * inv * 1.41421356237309515f;
        }
      }
    }
    if constexpr (B::ISV) {
      *reinterpret_cast<u16x8_t*>(lds + FLY::VR + (r * LY::RP + 8 * s) * 2) = vv;
      *reinterpret_cast<u16x8_t*>(lds + FLY::GR + (r * LY::RP + 8 * s) * 2) = gg;
      uint16_t* vt = reinterpret_cast<uint16_t*>(lds + FLY::VT);
      const int pos = vt_pos(r);
#pragma unroll
      for (int e = 0; e < 8; ++e) vt[vt_row(8 * s + e) * LY::VTP + pos] = vv[e];
    }
  }
};

template <int P, int DV, int W>
__device__ __forceinline__ void run_fdq(const FArgs& a, char* lds) {
  using LY = Lay<P, DV>;
  using FLY = FL<P, DV>;
  constexpr int NT = LY::NT, NH = LY::NH, NKS = LY::NKS, NTW = wave_nt<P>(W), MT = m_tile<P>(W);
  constexpr bool OWN = W >= 6;  // waves 6, 7: denominators and the intra block of token tile W - 6
  constexpr int TT = OWN ? W - 6 : 0;
  const int lane = threadIdx.x & 63, ln = lane & 15, lg = lane >> 4;
  const bool glow = lg < 2, mlow = ln < 8;
  const int64_t bh = blockIdx.x / a.nseg;
  const int seg = blockIdx.x % a.nseg;
  int64_t row0;
  int rstep, Tb;  // first row, row step, this sequence's length
  seq_rows_of(a.lay, bh, a.H, a.T, row0, rstep, Tb);
  const int nch = (Tb + CB - 1) / CB;
  const int c0 = seg * a.seg_chunks, c1 = min(nch, c0 + a.seg_chunks);

  const float* qr = reinterpret_cast<const float*>(lds + FLY::QR);
  const float* kh = reinterpret_cast<const float*>(lds + FLY::KH);
  const float* kt = reinterpret_cast<const float*>(lds + FLY::KT);
  const uint16_t* vt = reinterpret_cast<const uint16_t*>(lds + FLY::VT);
  const uint16_t* vr = reinterpret_cast<const uint16_t*>(lds + FLY::VR);
  const uint16_t* gr = reinterpret_cast<const uint16_t*>(lds + FLY::GR);
  uint16_t* mm = reinterpret_cast<uint16_t*>(lds + FLY::MM);
  float* gp = reinterpret_cast<float*>(lds + FLY::GP);
  float* g2s = reinterpret_cast<float*>(lds + FLY::G2);
  const float* iq = reinterpret_cast<const float*>(lds + FLY::IQ);
  float* dla = reinterpret_cast<float*>(lds + FLY::DL);
  float* idl = reinterpret_cast<float*>(lds + FLY::ID);

  // ---- state before the segment: the forward's prefix, transposed into the swapped layout
  f32x4_t S[wave_na<P>(W)][NT];
  f32x4_t Mt = zero4();
#pragma unroll
  for (int i = 0; i < NTW; ++i)
#pragma unroll
    for (int dt = 0; dt < NT; ++dt) S[i][dt] = zero4();
  if (seg > 0) {
    const float* src = a.fws + (bh * (a.nseg - 1) + (seg - 1)) * LY::STATE;
#pragma unroll
    for (int i = 0; i < NTW; ++i)
#pragma unroll
      for (int dt = 0; dt < NT; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int sl = ((ln >> 2) << 4) | (4 * lg + r);
          S[i][dt][r] = src[((wave_tile<P>(W, i) * NT + dt) * 64 + sl) * 4 + (ln & 3)];
        }
    if constexpr (MT >= 0) Mt = *reinterpret_cast<const f32x4_t*>(src + LY::NTL * NT * 256 + (MT * 64 + lane) * 4);
  }

  FStage<P, DV, W> stg;
  stg.load(a, row0, rstep, Tb, c0 * CB);
  stg.stage(lds, c0 & 1);
  write_gram<P, MT>(mm, Mt, ln, lg);
  __syncthreads();

  for (int c = c0; c < c1; ++c) {
    const int t0 = c * CB, buf = c & 1;
    const float* qh = reinterpret_cast<const float*>(lds + FLY::QH) + buf * CB * LY::QP;
    if (c + 1 < c1) stg.load(a, row0, rstep, Tb, t0 + CB);
    // ================= phase 1 (owners): D_t; scores and v_s . g_t kept for phase 2
    f32x4_t Sc[2], Ev[2], Xm[NH];
    float invq = 0.f, invD = 0.f, dintra = 0.f, Dt = 0.f;
    if constexpr (OWN) {
      const int t = 16 * TT + ln;
      float xs[8];
      comp8<P>(qr + t * LY::QP, lg, xs);
      const bf16x8_t qb = pack8(xs);  // the raw query: exact in bf16
      invq = iq[buf * CB + t];
      gram_apply<P>(mm, qb, ln, lg, Xm);  // X^T = M q
      float dpart = 0.f;
#pragma unroll
      for (int rt = 0; rt < NH; ++rt) {
        const f32x4_t qv = *reinterpret_cast<const f32x4_t*>(qr + t * LY::QP + 16 * rt + 4 * lg);
        dpart += Xm[rt][0] * qv[0] + Xm[rt][1] * qv[1] + Xm[rt][2] * qv[2] + Xm[rt][3] * qv[3];
      }
      dpart *= invq * invq;
      bf16x8_t gf[NKS];  // g_t, exact in bf16
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) gf[ks] = row_frag(gr + t * LY::RP, ks, lg);
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        Sc[k2] = zero4();
        Ev[k2] = zero4();
        if (k2 <= TT) {  // scores q_hat . k_hat with k_hat as bf16 hi + lo; v_s . g_t exact
          float ks8[8];
          comp8<P>(kh + (16 * k2 + ln) * LY::QP, lg, ks8);
          bf16x8_t khi, klo;
          split8(ks8, khi, klo);
          Sc[k2] = mfma(klo, qb, mfma(khi, qb, zero4()));
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) Ev[k2] = mfma(row_frag(vr + (16 * k2 + ln) * LY::RP, ks, lg), gf[ks], Ev[k2]);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float s = Sc[k2][r] * invq;
            if (k2 == TT && 4 * lg + r > ln) s = 0.f;  // causal: key <= query
            Sc[k2][r] = s;
            dpart += s * s;
            dintra += s * s * Ev[k2][r];
          }
        }
      }
      Dt = xor32_sum(xor16_sum(dpart));
      dintra = xor32_sum(xor16_sum(dintra));
      invD = Dt > 0.f ? 1.f / Dt : 0.f;
      if (lg == 0) idl[t] = invD;
    }
    // ================= phase 1, all waves: D_t-free parts of dq_hat (1 / D_t is applied to their
    // sum), then the build
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int t = 16 * tt + ln;
      bf16x8_t af[NKS];  // g_t, exact in bf16
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) af[ks] = row_frag(gr + t * LY::RP, ks, lg);
      float Y[P], G[P];
      rot_row<P>(qh + t * LY::QP, lg, Y);
#pragma unroll
      for (int x = 0; x < P; ++x) G[x] = 0.f;
      // x = S g_t over this wave's feature tiles, through the lift's transpose
      [&]<int... TI>(std::integer_sequence<int, TI...>) {
        (([&] {
           constexpr int tau = wave_tile<P>(W, TI);
           f32x4_t X = zero4();
#pragma unroll
           for (int ks = 0; ks < NKS; ++ks) X = mfma(sfrag<NT>(S[TI], ks), af[ks], X);
           tr_tile<P, tau>(G, Y, X, glow);
         }()),
         ...);
      }(std::make_integer_sequence<int, NTW>{});
      {
        // psi(q_hat_t)^T (S g_t) = (1/2) sum_x Y[x] G[x] (psi is homogeneous of degree 2),
        // summed over this wave's feature rows
        float ds = 0.f;
#pragma unroll
        for (int x = 0; x < P; ++x) ds += Y[x] * G[x];
        ds = xor32_sum(xor16_sum(ds));
        if (lg == 0) dla[W * CB + t] = 0.5f * ds;
      }
      pair_sum_lo<P>(G);
      if (lg < 2) store_rotated<P>(gp + (2 * W + lg) * CB * (P + 4), G, t, lg);
    }
    {  // build: S^T += V^T psi(K), 2 M += (sqrt2 K)^T (sqrt2 K)
      float N[NH][8];
      tr_rows<P>(kt, ln, lg, N);
      bf16x8_t vbf[NT];
#pragma unroll
      for (int dt = 0; dt < NT; ++dt)
        vbf[dt] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u16x8_t*>(vt + vt_row(16 * dt + ln) * LY::VTP + 8 * lg));
      [&]<int... TI>(std::integer_sequence<int, TI...>) {
        (([&] {
           const bf16x8_t bfr = build_frag<P, wave_tile<P>(W, TI)>(N, mlow);
#pragma unroll
           for (int dt = 0; dt < NT; ++dt) S[TI][dt] = mfma(vbf[dt], bfr, S[TI][dt]);
         }()),
         ...);
      }(std::make_integer_sequence<int, NTW>{});
      if constexpr (MT >= 0) Mt = mfma(pack8(N[MT / NH]), pack8(N[MT % NH]), Mt);
    }
    __syncthreads();
    // ================= phase 2 (owners): delta_t, then the parts of dq_hat that carry it:
    // b_t J^T Z = -delta_t / D_t 2 M q_hat_t, and the intra block
    // (v_s . g_t - delta_t) / D_t 2 (q_hat_t . k_hat_s) k_hat_s over keys s <= t
    if constexpr (OWN) {
      const int t = 16 * TT + ln;
      float sd = dintra;
#pragma unroll
      for (int w = 0; w < 8; ++w) sd += dla[w * CB + t];
      const float delta = sd * invD;
      const float bt = -delta * invD;
      float G2[NH][4];
#pragma unroll
      for (int rt = 0; rt < NH; ++rt)
#pragma unroll
        for (int r = 0; r < 4; ++r) G2[rt][r] = 2.f * bt * invq * Xm[rt][r];
      float pw[8];
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
        for (int r = 0; r < 4; ++r) pw[4 * k2 + r] = (Ev[k2][r] - delta) * invD * Sc[k2][r] * 1.41421356237309515f;
      const bf16x8_t pb = pack8(pw);
      float N[NH][8];
      tr_rows<P>(kt, ln, lg, N);  // sqrt(2) k_hat^T: the product carries the factor 2
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        const f32x4_t out = mfma(pack8(N[h]), pb, zero4());
#pragma unroll
        for (int r = 0; r < 4; ++r) G2[h][r] += out[r];
      }
      // components 16 h + 4 lg + r of token t: one lane each
#pragma unroll
      for (int h = 0; h < NH; ++h)
        *reinterpret_cast<f32x4_t*>(g2s + t * (P + 4) + 16 * h + 4 * lg) = f32x4_t{G2[h][0], G2[h][1], G2[h][2], G2[h][3]};
      if (lg == 0 && t0 + t < Tb)
        *reinterpret_cast<f32x2_t*>(a.stats + (row0 + (int64_t)(t0 + t) * rstep) * 2) = f32x2_t{Dt, delta};
    }
    __syncthreads();
    // ================= phase 3: dq of the chunk (waves 4-7), staging of chunk c + 1, M after c
    if constexpr (W >= 4) {
      constexpr int TPR = P / 4;
      const int u = threadIdx.x - 256;
      if (u < CB * TPR) {
        const int r = u / TPR, c4 = (u % TPR) * 4;
        f32x4_t dsum = zero4();
#pragma unroll
        for (int j = 0; j < 16; ++j) dsum += *reinterpret_cast<const f32x4_t*>(gp + (j * CB + r) * (P + 4) + c4);
        dsum = dsum * idl[r] + *reinterpret_cast<const f32x4_t*>(g2s + r * (P + 4) + c4);
        const float d[4] = {dsum[0], dsum[1], dsum[2], dsum[3]};
        const f32x4_t qv = *reinterpret_cast<const f32x4_t*>(qh + r * LY::QP + c4);
        const float pr = group_sum<TPR>(qv[0] * d[0] + qv[1] * d[1] + qv[2] * d[2] + qv[3] * d[3]);
        const float s = iq[buf * CB + r];
        if (t0 + r < Tb)
          *reinterpret_cast<f32x4_t*>(a.dq + (row0 + (int64_t)(t0 + r) * rstep) * P + c4) =
              f32x4_t{(d[0] - qv[0] * pr) * s, (d[1] - qv[1] * pr) * s, (d[2] - qv[2] * pr) * s, (d[3] - qv[3] * pr) * s};
      }
    }
    if (c + 1 < c1) stg.stage(lds, buf ^ 1);
    write_gram<P, MT>(mm, Mt, ln, lg);
    __syncthreads();
  }
}

// ============================================================ reverse time: summaries, dk, dv
struct RArgs {
  const uint16_t *q, *k, *v, *g;
  const float* stats;  // [rows][2]: D_t, delta_t
  float* rsum;         // reverse summaries [bh][nseg - 1] (slot nseg - 1 - s holds segment s)
  float* dk;           // [rows][P]
  float* dv;           // [rows][DV]
  int T, nseg, seg_chunks;
  SeqLayout lay;
  int H;
};

// reverse-time kernels: segment summaries [R | 2N], dk, dv (each rebuilds R over its chunks)
enum : int { RM_SUM = 0, RM_DK = 1, RM_DV = 2 };

template <int P, int DV, int MODE>
struct RL {
  using LY = Lay<P, DV>;
  static constexpr bool DK = MODE == RM_DK, DVM = MODE == RM_DV, SCORES = MODE != RM_SUM;
  static constexpr int SB_BYTES = DVM ? LY::NPAIR * LY::NT * 64 * 16 : 0;
  static constexpr int QD = 0;                                        // sqrt2 q_hat^T / sqrt(D) fp32 [P][TP]
  static constexpr int GT = QD + P * LY::TP * 4;                      // G^T bf16 [DV][VTP]
  static constexpr int QH = GT + DV * LY::VTP * 2;                    // q_hat rows fp32 [CB][QP]
  static constexpr int KR = QH + (SCORES ? CB * LY::QP * 4 : 0);      // raw k rows fp32 [CB][QP]
  static constexpr int KH = KR + (SCORES ? CB * LY::QP * 4 : 0);      // k_hat rows fp32 [2][CB][QP]
  static constexpr int QT = KH + (SCORES ? 2 * CB * LY::QP * 4 : 0);  // sqrt2 q_hat^T fp32 [P][TP]
  static constexpr int GR = QT + (DK ? P * LY::TP * 4 : 0);           // g rows bf16 [CB][RP]
  static constexpr int VR = GR + (DK ? CB * LY::RP * 2 : 0);          // v rows bf16 [CB][RP]
  static constexpr int NN = VR + (DK ? CB * LY::RP * 2 : 0);          // weighted Gram halves bf16 [2][P][MP]
  static constexpr int GP = NN + (DK ? 2 * P * LY::MP * 2 : 0);       // dk_hat partials [8 waves x 2][CB][P + 4]
  static constexpr int SB = GP + (DK ? 16 * CB * (P + 4) * 4 : 0);    // R, readout fragment order
  static constexpr int VP = SB + SB_BYTES;                            // dv partials [4 pair ranges][CB][DV + 4]
  static constexpr int IK = VP + (DVM ? 4 * CB * (DV + 4) * 4 : 0);   // 1 / |k| [2][CB]
  static constexpr int DL = IK + 2 * CB * 4;                          // delta [CB]
  static constexpr int ID = DL + CB * 4;                              // 1 / D [CB]
  static constexpr int BYTES = ID + CB * 4;
  static_assert(BYTES <= 160 * 1024, "LDS budget");
};

template <int P, int DV, int W, int MODE>
struct RStage : Piece<P, DV, W> {
  using B = Piece<P, DV, W>;
  using LY = Lay<P, DV>;
  using RLY = RL<P, DV, MODE>;
  static constexpr bool SCORES = MODE != RM_SUM, DK = MODE == RM_DK;
  typename B::row_t x;
  u16x8_t vv, gg;
  f32x2_t st;  // D_t, delta_t of the piece's row
  // rows t0 .. of the sequence at row0 + t step (rows at or past len read as zero)
  __device__ __forceinline__ void load(const RArgs& a, int64_t row0, int step, int len, int t0) {
    const int t = t0 + B::row();
    const bool ok = t >= 0 && t < len;
    const int64_t row = row0 + (int64_t)t * step;
    if constexpr (B::ISQ || B::ISV) st = ok ? *reinterpret_cast<const f32x2_t*>(a.stats + row * 2) : f32x2_t{0.f, 0.f};
    if constexpr (B::ISQ) x = B::load_qk(a.q, row, ok);
    if constexpr (B::ISK && SCORES) x = B::load_qk(a.k, row, ok);
    if constexpr (B::ISV) {
      if (ok) {
        const int64_t off = row * DV + 8 * B::sub();
        if constexpr (DK) vv = *reinterpret_cast<const u16x8_t*>(a.v + off);
        gg = *reinterpret_cast<const u16x8_t*>(a.g + off);
      } else {
        for (int e = 0; e < 8; ++e) vv[e] = gg[e] = 0;
      }
    }
  }
  __device__ __forceinline__ void stage(char* lds, int buf) {
    const int r = B::row(), s = B::sub();
    if constexpr (B::ISQ) {
      float f[B::KQ];
      const float inv = B::unpack(x, f);
      // psi(q_hat_t) / D_t = psi(q_hat_t / sqrt(D_t)): the build's operand carries a_t's 1 / D_t
      const float isd = st[0] > 0.f ? 1.f / sqrtf(st[0]) : 0.f;
      float* qh = reinterpret_cast<float*>(lds + RLY::QH) + r * LY::QP + s * B::KQ;
      float* qt = reinterpret_cast<float*>(lds + RLY::QT) + (s * B::KQ) * LY::TP + 8 * s + r;
      float* qd = reinterpret_cast<float*>(lds + RLY::QD) + (s * B::KQ) * LY::TP + 8 * s + r;
#pragma unroll
      for (int e = 0; e < B::KQ; ++e) {
        const float u = f[e] * inv * 1.41421356237309515f;
        if constexpr (SCORES) qh[e] = f[e] * inv;
        if constexpr (DK) qt[e * LY::TP] = u;
        qd[e * LY::TP] = u * isd;
      }
    }
    if constexpr (B::ISK && SCORES) {
      float f[B::KQ];
      const float inv = B::unpack(x, f);
      float* kr = reinterpret_cast<float*>(lds + RLY::KR) + r * LY::QP + s * B::KQ;
      float* kh = reinterpret_cast<float*>(lds + RLY::KH) + (buf * CB + r) * LY::QP + s * B::KQ;
#pragma unroll
      for (int e = 0; e < B::KQ; ++e) {
        kr[e] = f[e];
        kh[e] = f[e] * inv;
      }
      if (s == 0) reinterpret_cast<float*>(lds + RLY::IK)[buf * CB + r] = inv;
    }
    if constexpr (B::ISV) {
      if constexpr (DK) {
        *reinterpret_cast<u16x8_t*>(lds + RLY::VR + (r * LY::RP + 8 * s) * 2) = vv;
        *reinterpret_cast<u16x8_t*>(lds + RLY::GR + (r * LY::RP + 8 * s) * 2) = gg;
      }
      uint16_t* gt = reinterpret_cast<uint16_t*>(lds + RLY::GT);
      const int pos = vt_pos(r);
#pragma unroll
      for (int e = 0; e < 8; ++e) gt[vt_row(8 * s + e) * LY::VTP + pos] = gg[e];
      if (s == 0) {
        reinterpret_cast<float*>(lds + RLY::DL)[r] = st[1];
        reinterpret_cast<float*>(lds + RLY::ID)[r] = st[0] > 0.f ? 1.f / st[0] : 0.f;
      }
    }
  }
};

// R built in the forward's orientation (lane (d, g) holds feature rows 4 g + r at value column
// 16 dt + d) into the readout's fragment order: contiguous 16-byte fragments of tile pairs
template <int P, int DV, int W>
__device__ __forceinline__ void write_pairs(uint16_t* sb, const f32x4_t (&R)[wave_na<P>(W)][DV / 16], int lane) {
  constexpr int NT = DV / 16, NTW = wave_nt<P>(W);
#pragma unroll
  for (int i = 0; i < NTW; i += 2) {
    const int pair = wave_tile<P>(W, i) >> 1;
#pragma unroll
    for (int dt = 0; dt < NT; ++dt) {
      const f32x4_t& x = R[i][dt];
      const f32x4_t& y = R[i + 1 < NTW ? i + 1 : i][dt];
      const bool two = i + 1 < NTW;  // the odd last tile of a wave has no partner
      *reinterpret_cast<u32x4_t*>(sb + ((pair * NT + dt) * 64 + lane) * 8) =
          u32x4_t{pk2(x[0], x[1]), pk2(x[2], x[3]), two ? pk2(y[0], y[1]) : 0u, two ? pk2(y[2], y[3]) : 0u};
    }
  }
}

// scores q_hat_t . k_hat_s of the query tile q2 against key s of this lane (q_hat as bf16
// hi + lo, the raw key exact), masked to t >= s: lane (s, lg) holds queries 16 q2 + 4 lg + r
template <int P>
__device__ __forceinline__ f32x4_t rev_scores(const float* qhr, bf16x8_t kb, float invk, int q2, int kt, int ln, int lg) {
  constexpr int QP = P + 4;  // Lay::QP
  f32x4_t Sc = zero4();
  if (q2 >= kt) {
    float qs[8];
    comp8<P>(qhr + (16 * q2 + ln) * QP, lg, qs);
    bf16x8_t qhi, qlo;
    split8(qs, qhi, qlo);
    Sc = mfma(qlo, kb, mfma(qhi, kb, zero4()));
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    Sc[r] *= invk;
    if (q2 < kt || (q2 == kt && 4 * lg + r < ln)) Sc[r] = 0.f;  // causal: query >= key
  }
  return Sc;
}

template <int P, int DV, int W, int MODE>
__device__ __forceinline__ void run_rev(const RArgs& a, char* lds) {
  using LY = Lay<P, DV>;
  using RLY = RL<P, DV, MODE>;
  constexpr bool SUM = MODE == RM_SUM, DK = MODE == RM_DK, DVM = MODE == RM_DV;
  constexpr int NT = LY::NT, NH = LY::NH, NKS = LY::NKS, NTW = wave_nt<P>(W), MT = m_tile<P>(W);
  constexpr bool OWN = DK && W >= 6;  // dk: waves 6, 7 take the r part and intra block of key tile W - 6
  constexpr int KO = OWN ? W - 6 : 0;
  // dv: key tile KV, readout pairs [VPB, VPE) over all value columns; the intra term on the
  // waves of the last pair range
  constexpr int KV = W & 1, FV = W >> 1;
  constexpr int VPB = FV * LY::NPAIR / 4, VPE = (FV + 1) * LY::NPAIR / 4;
  const int lane = threadIdx.x & 63, ln = lane & 15, lg = lane >> 4;
  const bool glow = lg < 2, mlow = ln < 8;
  const int nblk = SUM ? a.nseg - 1 : a.nseg;
  const int64_t bh = blockIdx.x / nblk;
  const int seg = (int)(blockIdx.x % nblk) + (SUM ? 1 : 0);
  int64_t row0;
  int rstep, Tb;  // first row, row step, this sequence's length
  seq_rows_of(a.lay, bh, a.H, a.T, row0, rstep, Tb);
  const int nch = (Tb + CB - 1) / CB;
  const int c0 = seg * a.seg_chunks, c1 = min(nch, c0 + a.seg_chunks);

  const float* qd = reinterpret_cast<const float*>(lds + RLY::QD);
  const uint16_t* gt = reinterpret_cast<const uint16_t*>(lds + RLY::GT);
  const float* qhr = reinterpret_cast<const float*>(lds + RLY::QH);
  const float* kr = reinterpret_cast<const float*>(lds + RLY::KR);
  const float* qt = reinterpret_cast<const float*>(lds + RLY::QT);
  const uint16_t* gr = reinterpret_cast<const uint16_t*>(lds + RLY::GR);
  const uint16_t* vr = reinterpret_cast<const uint16_t*>(lds + RLY::VR);
  uint16_t* nn = reinterpret_cast<uint16_t*>(lds + RLY::NN);
  float* gp = reinterpret_cast<float*>(lds + RLY::GP);
  uint16_t* sb = reinterpret_cast<uint16_t*>(lds + RLY::SB);
  float* vp = reinterpret_cast<float*>(lds + RLY::VP);
  const float* ik = reinterpret_cast<const float*>(lds + RLY::IK);
  const float* dl = reinterpret_cast<const float*>(lds + RLY::DL);
  const float* idl = reinterpret_cast<const float*>(lds + RLY::ID);

  // ---- suffix state of the segments after this one (the scanned reverse summaries)
  f32x4_t R[wave_na<P>(W)][NT];
  f32x4_t Nt = zero4();  // weighted Gram tile: 2 N
#pragma unroll
  for (int i = 0; i < NTW; ++i)
#pragma unroll
    for (int dt = 0; dt < NT; ++dt) R[i][dt] = zero4();
  if (!SUM && seg < a.nseg - 1) {
    const float* src = a.rsum + (bh * (a.nseg - 1) + (a.nseg - 2 - seg)) * LY::STATE;
#pragma unroll
    for (int i = 0; i < NTW; ++i)
#pragma unroll
      for (int dt = 0; dt < NT; ++dt) {
        if constexpr (DVM) {  // dv builds R in the forward's orientation: transposed load
#pragma unroll
          for (int r = 0; r < 4; ++r)
            R[i][dt][r] = src[((wave_tile<P>(W, i) * NT + dt) * 64 + (((ln >> 2) << 4) | (4 * lg + r))) * 4 + (ln & 3)];
        } else {
          R[i][dt] = *reinterpret_cast<const f32x4_t*>(src + ((wave_tile<P>(W, i) * NT + dt) * 64 + lane) * 4);
        }
      }
    if constexpr (MT >= 0) Nt = *reinterpret_cast<const f32x4_t*>(src + LY::NTL * NT * 256 + (MT * 64 + lane) * 4);
  }

  RStage<P, DV, W, MODE> stg;
  const int cl = c1 - 1;  // chunks run from the last to the first (none past the sequence's end)
  if (c0 <= cl) {
    stg.load(a, row0, rstep, Tb, cl * CB);
    stg.stage(lds, cl & 1);
  }
  if constexpr (DK) write_gram<P, MT>(nn, Nt, ln, lg);
  if constexpr (DVM) write_pairs<P, DV, W>(sb, R, lane);
  __syncthreads();

  for (int c = cl; c >= c0; --c) {
    const int t0 = c * CB, buf = c & 1;
    if (c - 1 >= c0) stg.load(a, row0, rstep, Tb, t0 - CB);
    const float* kh = reinterpret_cast<const float*>(lds + RLY::KH) + buf * CB * LY::QP;
    // ================= phase A
    if constexpr (DK) {  // dk_hat of the chunk's keys
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        const int s = 16 * k2 + ln;
        bf16x8_t vf[NKS];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) vf[ks] = row_frag(vr + s * LY::RP, ks, lg);
        float Y[P], G[P];
        rot_row<P>(kh + s * LY::QP, lg, Y);
#pragma unroll
        for (int x = 0; x < P; ++x) G[x] = 0.f;
        // R v_s over this wave's feature tiles, through the lift's transpose
        [&]<int... TI>(std::integer_sequence<int, TI...>) {
          (([&] {
             constexpr int tau = wave_tile<P>(W, TI);
             f32x4_t X = zero4();
#pragma unroll
             for (int ks = 0; ks < NKS; ++ks) X = mfma(sfrag<NT>(R[TI], ks), vf[ks], X);
             tr_tile<P, tau>(G, Y, X, glow);
           }()),
           ...);
        }(std::make_integer_sequence<int, NTW>{});
        if constexpr (OWN) {
          if (k2 == KO) {
            float xs[8];
            comp8<P>(kr + s * LY::QP, lg, xs);
            const bf16x8_t kb = pack8(xs);  // the raw key: exact in bf16
            const float invk = ik[buf * CB + s];
            // r part: 2 N k_hat_s (components 16 rt + 4 lg + r are G[16 rt + r])
            f32x4_t Xn[NH];
            gram_apply<P>(nn, kb, ln, lg, Xn);
#pragma unroll
            for (int rt = 0; rt < NH; ++rt)
#pragma unroll
              for (int r = 0; r < 4; ++r) G[16 * rt + r] += 2.f * invk * Xn[rt][r];
            // intra block over queries t >= s: e_ts = (v_s . g_t - delta_t) / D_t 2 (q_hat_t . k_hat_s)
            // (v_s . g_t exact), times q_hat_t
            float pw[8];
#pragma unroll
            for (int q2 = 0; q2 < 2; ++q2) {
              const f32x4_t Sc = rev_scores<P>(qhr, kb, invk, q2, KO, ln, lg);
              f32x4_t E = zero4();
              if (q2 >= KO) {
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) E = mfma(row_frag(gr + (16 * q2 + ln) * LY::RP, ks, lg), vf[ks], E);
              }
              const f32x4_t dq4 = *reinterpret_cast<const f32x4_t*>(dl + 16 * q2 + 4 * lg);
              const f32x4_t id4 = *reinterpret_cast<const f32x4_t*>(idl + 16 * q2 + 4 * lg);
#pragma unroll
              for (int r = 0; r < 4; ++r) pw[4 * q2 + r] = (E[r] - dq4[r]) * id4[r] * Sc[r] * 1.41421356237309515f;
            }
            const bf16x8_t pb = pack8(pw);
            float Nq[NH][8];
            tr_rows<P>(qt, ln, lg, Nq);  // sqrt(2) q_hat^T
#pragma unroll
            for (int h = 0; h < NH; ++h) {
              const f32x4_t out = mfma(pack8(Nq[h]), pb, zero4());
#pragma unroll
              for (int r = 0; r < 4; ++r) G[16 * h + r] += out[r];
            }
          }
        }
        pair_sum_lo<P>(G);
        if (lg < 2) store_rotated<P>(gp + (2 * W + lg) * CB * (P + 4), G, s, lg);
      }
    }
    if constexpr (DVM) {  // dv of key tile KV over pairs [VPB, VPE): R^T psi(k_hat_s) (+ sum_t (w_ts / D_t) g_t)
      const int s = 16 * KV + ln;
      float Y[P];
      rot_row<P>(kh + s * LY::QP, lg, Y);
      f32x4_t O[NT];
#pragma unroll
      for (int dt = 0; dt < NT; ++dt) O[dt] = zero4();
      [&]<int... PI>(std::integer_sequence<int, PI...>) {
        (([&] {
           constexpr int t1 = 2 * (VPB + PI), t2 = t1 + 1;
           constexpr bool has2 = t2 < LY::NTL;
           const bf16x8_t af = readout_frag<P, t1, has2 ? t2 : t1, has2>(Y, glow);
#pragma unroll
           for (int dt = 0; dt < NT; ++dt)
             O[dt] = mfma(*reinterpret_cast<const bf16x8_t*>(sb + (((VPB + PI) * NT + dt) * 64 + lane) * 8), af, O[dt]);
         }()),
         ...);
      }(std::make_integer_sequence<int, VPE - VPB>{});
      if constexpr (FV == 3) {
        float xs[8];
        comp8<P>(kr + s * LY::QP, lg, xs);
        const bf16x8_t kb = pack8(xs);
        const float invk = ik[buf * CB + s];
        float wv[8];
#pragma unroll
        for (int q2 = 0; q2 < 2; ++q2) {
          const f32x4_t Sc = rev_scores<P>(qhr, kb, invk, q2, KV, ln, lg);
          const f32x4_t id4 = *reinterpret_cast<const f32x4_t*>(idl + 16 * q2 + 4 * lg);
#pragma unroll
          for (int r = 0; r < 4; ++r) wv[4 * q2 + r] = Sc[r] * Sc[r] * id4[r];
        }
        const bf16x8_t wb = pack8(wv);
#pragma unroll
        for (int dt = 0; dt < NT; ++dt)
          O[dt] = mfma(__builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u16x8_t*>(gt + vt_row(16 * dt + ln) * LY::VTP + 8 * lg)),
                       wb, O[dt]);
      }
      // lane (s, lg) holds columns 16 dt + 4 lg .. + 3
#pragma unroll
      for (int dt = 0; dt < NT; ++dt)
        *reinterpret_cast<f32x4_t*>(vp + (FV * CB + s) * (DV + 4) + 16 * dt + 4 * lg) = O[dt];
    }
    {  // build: R^T += G^T psi(Q / sqrt(D)) (= A^T psi(Q)), 2 N += (-delta sqrt2 Q')^T (sqrt2 Q'), Q' = Q / sqrt(D)
      float Nq[NH][8];
      tr_rows<P>(qd, ln, lg, Nq);
      bf16x8_t abf[NT];
#pragma unroll
      for (int dt = 0; dt < NT; ++dt)
        abf[dt] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u16x8_t*>(gt + vt_row(16 * dt + ln) * LY::VTP + 8 * lg));
      [&]<int... TI>(std::integer_sequence<int, TI...>) {
        (([&] {
           const bf16x8_t bfr = build_frag<P, wave_tile<P>(W, TI)>(Nq, mlow);
#pragma unroll
           for (int dt = 0; dt < NT; ++dt) R[TI][dt] = DVM ? mfma(bfr, abf[dt], R[TI][dt]) : mfma(abf[dt], bfr, R[TI][dt]);
         }()),
         ...);
      }(std::make_integer_sequence<int, NTW>{});
      if constexpr (MT >= 0 && !DVM) {
        const f32x4_t b0 = *reinterpret_cast<const f32x4_t*>(dl + 4 * lg);
        const f32x4_t b1 = *reinterpret_cast<const f32x4_t*>(dl + 16 + 4 * lg);
        float nw[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          nw[e] = -Nq[MT / NH][e] * b0[e];
          nw[4 + e] = -Nq[MT / NH][4 + e] * b1[e];
        }
        Nt = mfma(pack8(nw), pack8(Nq[MT % NH]), Nt);
      }
    }
    __syncthreads();
    // ================= phase B: dk or dv of the chunk (waves 4-7), staging of chunk c - 1, state after c
    if constexpr (DK && W >= 4) {
      constexpr int TPR = P / 4;
      const int u = threadIdx.x - 256;
      if (u < CB * TPR) {
        const int r = u / TPR, c4 = (u % TPR) * 4;
        f32x4_t dsum = zero4();
#pragma unroll
        for (int j = 0; j < 16; ++j) dsum += *reinterpret_cast<const f32x4_t*>(gp + (j * CB + r) * (P + 4) + c4);
        const f32x4_t kv = *reinterpret_cast<const f32x4_t*>(kh + r * LY::QP + c4);
        const float pr = group_sum<TPR>(kv[0] * dsum[0] + kv[1] * dsum[1] + kv[2] * dsum[2] + kv[3] * dsum[3]);
        const float s = ik[buf * CB + r];
        if (t0 + r < Tb)
          *reinterpret_cast<f32x4_t*>(a.dk + (row0 + (int64_t)(t0 + r) * rstep) * P + c4) = (dsum - kv * pr) * s;
      }
    }
    if constexpr (DVM && W >= 4) {  // dv of the chunk: the four pair ranges' sums
      const int u = threadIdx.x - 256;
      if (u < CB * LY::NV8) {
        const int r = u / LY::NV8, c8 = (u % LY::NV8) * 8;
        f32x4_t d0 = zero4(), d1 = zero4();
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          d0 += *reinterpret_cast<const f32x4_t*>(vp + (f * CB + r) * (DV + 4) + c8);
          d1 += *reinterpret_cast<const f32x4_t*>(vp + (f * CB + r) * (DV + 4) + c8 + 4);
        }
        if (t0 + r < Tb) {
          float* dst = a.dv + (row0 + (int64_t)(t0 + r) * rstep) * DV + c8;
          *reinterpret_cast<f32x4_t*>(dst) = d0;
          *reinterpret_cast<f32x4_t*>(dst + 4) = d1;
        }
      }
    }
    if (c - 1 >= c0) stg.stage(lds, buf ^ 1);
    if constexpr (DK) write_gram<P, MT>(nn, Nt, ln, lg);
    if constexpr (DVM) write_pairs<P, DV, W>(sb, R, lane);
    __syncthreads();
  }
  if constexpr (SUM) {  // segment summary to slot nseg - 1 - seg (reversed, so the scan gives suffixes)
    float* dst = a.rsum + (bh * (a.nseg - 1) + (a.nseg - 1 - seg)) * LY::STATE;
#pragma unroll
    for (int i = 0; i < NTW; ++i)
#pragma unroll
      for (int dt = 0; dt < NT; ++dt)
        *reinterpret_cast<f32x4_t*>(dst + ((wave_tile<P>(W, i) * NT + dt) * 64 + lane) * 4) = R[i][dt];
    if constexpr (MT >= 0) *reinterpret_cast<f32x4_t*>(dst + LY::NTL * NT * 256 + (MT * 64 + lane) * 4) = Nt;
  }
}

#define KATA_CBM_SWITCH(CALL)      \
  switch (threadIdx.x >> 6) {      \
    case 0: CALL(0); break;        \
    case 1: CALL(1); break;        \
    case 2: CALL(2); break;        \
    case 3: CALL(3); break;        \
    case 4: CALL(4); break;        \
    case 5: CALL(5); break;        \
    case 6: CALL(6); break;        \
    default: CALL(7); break;       \
  }

template <int P, int DV>
__global__ __launch_bounds__(512, 1) void fdq_kernel(FArgs a) {
  extern __shared__ __align__(16) char lds[];
#define KATA_FDQ(WW) run_fdq<P, DV, WW>(a, lds)
  KATA_CBM_SWITCH(KATA_FDQ)
#undef KATA_FDQ
}
template <int P, int DV, int MODE>
__global__ __launch_bounds__(512, 1) void rev_kernel(RArgs a) {
  extern __shared__ __align__(16) char lds[];
#define KATA_REV(WW) run_rev<P, DV, WW, MODE>(a, lds)
  KATA_CBM_SWITCH(KATA_REV)
#undef KATA_REV
}
#undef KATA_CBM_SWITCH

template <int P, int DV>
hipError_t launch(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* go, int B, int H, int T,
                  int scan, SeqLayout lay, int64_t rows, float* ws, float* dq, float* dk, float* dvo, hipStream_t st) {
  using LY = Lay<P, DV>;
  const SegPlan plan = seg_plan(B, H, T, CHUNKED_BWD_FWD_C, scan);
  const int64_t BH = (int64_t)B * H;
  const int64_t sums = plan.nseg > 1 ? BH * (plan.nseg - 1) * LY::STATE : 0;
  float* stats = ws;
  float* fws = stats + ((rows * 2 + 3) & ~(int64_t)3);
  float* rsum = fws + sums;
  hipError_t e;
  // the forward's segment summaries [S | 2M], scanned into prefixes
  if (plan.nseg > 1 &&
      (e = launch_chunked_bf16(q, k, v, nullptr, false, B, H, T, P, DV, CHUNKED_BWD_FWD_C, plan, fws, nullptr,
                               nullptr, lay, PASS_SUMMARIES | PASS_SCAN, st)) != hipSuccess)
    return e;
  const int seg_chunks = plan.cps * (CHUNKED_BWD_FWD_C / CB);
  FArgs fa{q, k, v, go, fws, stats, dq, T, plan.nseg, seg_chunks, lay, H};
  auto kf = fdq_kernel<P, DV>;
  if ((e = hipFuncSetAttribute((const void*)kf, hipFuncAttributeMaxDynamicSharedMemorySize, FL<P, DV>::BYTES)) != hipSuccess)
    return e;
  kf<<<dim3((unsigned)(BH * plan.nseg)), dim3(512), FL<P, DV>::BYTES, st>>>(fa);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  RArgs ra{q, k, v, go, stats, rsum, dk, dvo, T, plan.nseg, seg_chunks, lay, H};
  auto rev = [&](auto kern, int lds, int nblk) -> hipError_t {
    hipError_t r = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (r != hipSuccess) return r;
    kern<<<dim3((unsigned)(BH * nblk)), dim3(512), lds, st>>>(ra);
    return hipGetLastError();
  };
  if (plan.nseg > 1) {
    if ((e = rev(rev_kernel<P, DV, RM_SUM>, RL<P, DV, RM_SUM>::BYTES, plan.nseg - 1)) != hipSuccess) return e;
    if ((e = launch_scan(rsum, (int)BH, plan.nseg - 1, LY::STATE, st)) != hipSuccess) return e;
  }
  if ((e = rev(rev_kernel<P, DV, RM_DK>, RL<P, DV, RM_DK>::BYTES, plan.nseg)) != hipSuccess) return e;
  return rev(rev_kernel<P, DV, RM_DV>, RL<P, DV, RM_DV>::BYTES, plan.nseg);
}

}  // namespace cbm

bool chunked_bwd_mfma_supported(int p, int dv) { return (p == 16 || p == 32) && (dv == 32 || dv == 64); }

size_t chunked_bwd_mfma_workspace_floats(int B, int H, int T, int p, int dv, int scan, int64_t rows) {
  const SegPlan plan = seg_plan(B, H, T, CHUNKED_BWD_FWD_C, scan);
  const size_t BH = (size_t)B * H;
  const size_t sums = plan.nseg > 1 ? BH * (plan.nseg - 1) * (size_t)mfma_state_floats(p, dv) : 0;
  return ((rows * 2 + 3) & ~(size_t)3) + 2 * sums;
}

hipError_t launch_chunked_bwd_mfma(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* go,
                                   int B, int H, int T, int p, int dv, int scan, SeqLayout lay, int64_t rows,
                                   float* ws, float* dq, float* dk, float* dvo, hipStream_t st) {
#define KATA_CBM_CASE(PP, DD) \
  if (p == PP && dv == DD) return cbm::launch<PP, DD>(q, k, v, go, B, H, T, scan, lay, rows, ws, dq, dk, dvo, st);
  KATA_CBM_CASE(16, 32) KATA_CBM_CASE(16, 64) KATA_CBM_CASE(32, 32) KATA_CBM_CASE(32, 64)
#undef KATA_CBM_CASE
  return hipErrorInvalidValue;
}

}  // namespace kata
