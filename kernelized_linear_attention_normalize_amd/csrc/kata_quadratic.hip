// Flash-attention-style KATA forward on bf16 MFMA (gfx950): no state is materialised.
//
// Source: "Kernelized Linear Attention: Breaking the Capacity Wall with Symmetric Cones"
// (arXiv 2607.17419): the abstract's flash-attention-style operating point; the weight
// identity <psi(q), psi(k)> = (q_hat . k_hat)^2 of the rank-one lift display (after
// Eq. (8)); the normalized readout with explicit denominator (normalized-readout
// paragraph); inclusive causality of the state S_t (feature-value state display).
//
// Per workgroup: 512 queries of one (b,h), 8 waves x 64 queries; key blocks of 128 (64 for the
// reduced families),
// double-buffered in LDS with one barrier per block (the next block's global loads are in
// flight during the current block's MFMAs).
//   * Scores s = q_hat . k_hat on fp16 MFMA operands: every query is normalised once in
//     registers and every key when its block is staged; unit-norm components lie in [-1, 1],
//     where fp16 resolves 2^-11 (8x finer than bf16), and the weight is one square s^2 per
//     pair with no norm left to apply. The backward's statistics variant keeps the raw query
//     (its D_t is in raw-query units): scores from the raw bf16 inputs (exact products), with
//     a per-key reciprocal norm staged next to the raw K rows, s = (q . k) / ||k||.
//   * S^T = K Q^T (16x16x32 MFMA, keys as M: the accumulator rows are the k-slots of the next
//     product), W = s^2 masked on the diagonal blocks, rounded to bf16.
//   * O^T += V^T W^T and den += 1^T W^T (operands swapped, so a lane ends with 4 consecutive
//     output columns of one query, stored with one 8-byte write, and its own denominator).
// Weights lie in [0, ||q||^2] and the denominator is a plain sum, so unlike softmax there is
// no running maximum and no rescaling.
#include <type_traits>

#include "kata_device.h"
#include "kata_launch.h"

namespace kata {

// Tile shape (compile-time overridable): KATA_QBM queries per workgroup in waves of KATA_QW
// queries; KATA_QOCC workgroups per CU for the register budget.
#ifndef KATA_QW
#define KATA_QW 64
#endif
#ifndef KATA_QOCC
#define KATA_QOCC 1
#endif
#ifndef KATA_QBM
#define KATA_QBM 512
#endif
namespace quad {
constexpr int BM = KATA_QBM, QW = KATA_QW, NQT = QW / 16;
constexpr int NTHR = 64 * (BM / QW);  // threads per workgroup
// keys per block: 128 for the full map (half the barriers and block bookkeeping of 64), 64 for
// the reduced families, whose block products need more registers
constexpr int bn(int fam) { return fam == 0 ? 128 : 64; }
}

__device__ __forceinline__ f32x4_t mfma16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
typedef _Float16 qh8_t __attribute__((ext_vector_type(8)));
typedef float qf2_t __attribute__((ext_vector_type(2)));
typedef _Float16 qh2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ f32x4_t mfma16(qh8_t a, qh8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
// 8 bf16 values (16 bytes) times s, as fp16
__device__ __forceinline__ u32x4_t bf16x8_scaled_f16(const u32x4_t x, float s) {
  u32x4_t r;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const qh2_t h = __builtin_convertvector(qf2_t{bf16_bits_to_f32(x[e] & 0xffffu) * s, __uint_as_float(x[e] & 0xffff0000u) * s}, qh2_t);
    r[e] = __builtin_bit_cast(uint32_t, h);
  }
  return r;
}

// FAM: 0 the full map; 1 KATA-Sigma G, 2 KATA-M G (reduced PSD families paragraph) with
// blocks of P / G components, a whole number of 32-wide k-steps each: the block dot products
// q_a . k_b come from pairing the k-steps of block b of the keys with those of block a of the
// queries, and the weight is the sum of their squares (all pairs for Sigma, a = b for M).
// R (full map only): weights (q_hat . k_hat)^(2R), the inner product of the higher even-order
// lift psi_2R (psi_2r display of the HTML page); R = 1 is the rank-one map.
// STATS (backward, full map): no output; instead row t's denominator D_t = sum_s w_ts (with
// the raw query, as everywhere here) and delta_t = gout_t . o_t go to stats[2 r], [2 r + 1],
// r the tensor row of query t (bh T + t padded, its packed row under PK).
template <int P, int DV, bool OUT_BF16, int FAM = 0, int G = 1, int R = 1, bool STATS = false, bool PK = false>
__global__ __launch_bounds__(quad::NTHR, KATA_QOCC) void quadratic_bf16_kernel(const uint16_t* __restrict__ q,
                                                                const uint16_t* __restrict__ k,
                                                                const uint16_t* __restrict__ v,
                                                                void* __restrict__ o, int T,
                                                                int nqb, const uint16_t* __restrict__ gout,
                                                                float* __restrict__ stats,
                                                                SeqLayout lay = SeqLayout{}, int H = 0) {
  using namespace quad;
  constexpr int BN = bn(FAM), NKP = BN / 32;
  // bf16 pitch of V^T rows: BN + 16 (a float pitch of 8 mod 32: the transposed writes and the
  // 16-byte reads are conflict-free)
  constexpr int VTP = BN + 16;
  static_assert((VTP / 2) % 32 == 8, "V^T pitch");
  constexpr bool NRM = !STATS;  // normalised fp16 scores (else raw bf16 scores with 1/||k||)
  using qop_t = std::conditional_t<NRM, qh8_t, bf16x8_t>;
  constexpr int KS = (P + 31) / 32;                        // 32-wide k-steps over components
  constexpr int KP = P == 64 ? 80 : (P == 32 ? 48 : 16);   // bf16 pitch of K rows (8 * odd floats)
  constexpr int NT = DV / 16;                              // 16-wide output column tiles
  constexpr int KPC = P / 8;                               // 16-byte pieces per key row
  constexpr int KPIECES = BN * KPC;
  // Staging runs on the first half of the waves only. Of the two waves sharing a SIMD, the
  // older one gets the matrix core first and finishes its block's MFMAs well ahead of the
  // other (oldest-first arbitration), so it loads and stages the next block while the
  // younger one is still computing, instead of both staging after their MFMAs. The loads are
  // issued after the block's MFMAs, so no staging registers are live across them.
  // (the statistics variant, which needs more registers for its raw-query scores, stages on
  // every wave)
  constexpr int SW = STATS ? NTHR : NTHR / 2;  // staging threads
  constexpr int KI = (KPIECES + SW - 1) / SW;
  constexpr int VPIECES = (BN / 2) * (DV / 8);
  constexpr int VI = (VPIECES + SW - 1) / SW;
  static_assert(KPIECES % 64 == 0 && SW % 64 == 0, "staging layout");
  constexpr int KM = KS / G;  // k-steps per feature block
  static_assert(FAM == 0 ? G == 1 : (P % (32 * G) == 0), "feature blocks are whole k-steps");
  __shared__ __align__(16) uint16_t sK[2][BN * KP];
  __shared__ __align__(16) float sInvK[2][BN];
  __shared__ __align__(16) uint16_t sVt[2][DV * VTP];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ln = lane & 15, lg = lane >> 4;
  // The work of a query block grows with its index, so workgroups go out longest first over
  // all sequences: workgroup x takes query block nqb - 1 - x / BH of sequence x % BH.
  const int nbh = (int)(gridDim.x / nqb);
  const int64_t bh = blockIdx.x % nbh;
  const int qb0 = (nqb - 1 - (int)(blockIdx.x / nbh)) * BM;
  const int qw0 = qb0 + wave * QW;
  // Rows of this sequence: row0 + t * stp for t < len. Padded [B, H, T]: contiguous, all T
  // rows. Packed token-major (PK): H rows apart, the length from cu_seqlens (T = max_len).
  int64_t row0 = bh * (int64_t)T;
  int stp = 1, len = T;
  if constexpr (PK) {
    seq_rows_of(lay, bh, H, T, row0, stp, len);
    if (qb0 >= len) return;  // uniform over the workgroup: no query of this block exists
  }
  const int RQ = PK ? stp * P : P, RV = PK ? stp * DV : DV;  // elements from one row to the next
  // rows at or past len lie outside the resources and read as zero
  const __amdgpu_buffer_rsrc_t rq = buf_rsrc(q + row0 * P, (uint32_t)len * RQ * 2);
  const __amdgpu_buffer_rsrc_t rk = buf_rsrc(k + row0 * P, (uint32_t)len * RQ * 2);
  const __amdgpu_buffer_rsrc_t rv = buf_rsrc(v + row0 * DV, (uint32_t)len * RV * 2);

  // ---- query fragments (B operand of S^T): query qw0 + 16 qt + ln, comps 32 ks + 8 lg..;
  //      normalised to fp16 (NRM) over the query's four lane groups, else the raw bf16
  qop_t qf[NQT][KS];
#pragma unroll
  for (int qt = 0; qt < NQT; ++qt) {
    u32x4_t raw[KS];
    float ss = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      raw[ks] = u32x4_t{0u, 0u, 0u, 0u};
      if (P >= 32 || lg < 2)  // rows past T read as zero
        raw[ks] = __builtin_amdgcn_raw_buffer_load_b128(rq, (uint32_t)((qw0 + 16 * qt + ln) * RQ + 32 * ks + 8 * lg) * 2, 0, 0);
      if constexpr (NRM) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float lo = bf16_bits_to_f32(raw[ks][e] & 0xffffu), hi = __uint_as_float(raw[ks][e] & 0xffff0000u);
          ss += lo * lo + hi * hi;
        }
      }
    }
    if constexpr (NRM) {
      const float inv = inv_norm_fast(xor32_sum(xor16_sum(ss)));  // lanes ln + 16 lg hold the query
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qf[qt][ks] = __builtin_bit_cast(qh8_t, bf16x8_scaled_f16(raw[ks], inv));
    } else {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qf[qt][ks] = __builtin_bit_cast(bf16x8_t, raw[ks]);
    }
  }

  // ---- key-block staging: raw K rows (16-byte pieces) + 1/||k|| per key; V^T with the
  //      shared permuted / swizzled layout, one (key pair, 8 columns) piece per thread
  const bool stager = tid < SW;  // whole waves
  u32x4_t kreg[KI];
  u32x4_t vreg[VI][2];
  // V piece tid + SW i is piece tid shifted by SW / 8 key pairs (vt_piece: 8 pieces per key
  // pair; the shift keeps the column group), and vt_pos moves whole 32-key blocks, so piece i
  // writes at the same addresses plus a constant
  static_assert(VI == 1 || (SW % 256 == 0 && (SW / 4) % 32 == 0), "V piece shift");
  int vp = 0, vd = 0;
  if (stager) vt_piece<DV>(tid, vp, vd);
  auto prefetch = [&](int kb0) {
    if (!stager) return;
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      const int pc = tid + SW * i;
      if (pc < KPIECES)
        kreg[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, (uint32_t)((kb0 + pc / KPC) * RQ + 8 * (pc % KPC)) * 2, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < VI; ++i) {
      if (tid + SW * i < VPIECES) {
        const uint32_t off = (uint32_t)((kb0 + 2 * vp + (SW / 4) * i) * RV + 8 * vd) * 2;
        vreg[i][0] = __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, 0);
        vreg[i][1] = __builtin_amdgcn_raw_buffer_load_b128(rv, off + RV * 2, 0, 0);
      }
    }
  };
  auto stage = [&](int buf) {
    if (!stager) return;
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      const int pc = tid + SW * i;
      if (pc < KPIECES) {  // whole waves
        const int row = pc / KPC, col = pc % KPC;
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float lo = bf16_bits_to_f32(kreg[i][e] & 0xffffu), hi = __uint_as_float(kreg[i][e] & 0xffff0000u);
          ss += lo * lo + hi * hi;
        }
        ss = group_sum<KPC>(ss);  // the row's pieces are adjacent lanes
        if constexpr (NRM) {  // k_hat in fp16
          *reinterpret_cast<u32x4_t*>(&sK[buf][row * KP + 8 * col]) = bf16x8_scaled_f16(kreg[i], inv_norm_fast(ss));
        } else {
          *reinterpret_cast<u32x4_t*>(&sK[buf][row * KP + 8 * col]) = kreg[i];
          if (col == 0) sInvK[buf][row] = inv_norm_fast(ss);
        }
      }
    }
    char* vbase = reinterpret_cast<char*>(&sVt[buf][0]) + ((8 * vd) * VTP + vt_pos(2 * vp)) * 2;
#pragma unroll
    for (int i = 0; i < VI; ++i) {
      if (tid + SW * i < VPIECES) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t a = (vreg[i][0][e >> 1] >> (16 * (e & 1))) & 0xffffu;
          const uint32_t b = (vreg[i][1][e >> 1] >> (16 * (e & 1))) & 0xffffu;
          *reinterpret_cast<uint32_t*>(vbase + (((e & 4) + ((e & 3) ^ (vd & 3))) * VTP + (SW / 4) * i) * 2) = a | (b << 16);
        }
      }
    }
  };

  f32x4_t O[NQT][NT], D[NQT];
#pragma unroll
  for (int qt = 0; qt < NQT; ++qt) {
    D[qt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) O[qt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  const bf16x8_t ones = __builtin_bit_cast(bf16x8_t, u32x4_t{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});

  const int kend = min(len, qb0 + BM);
  const int nkb = (kend + BN - 1) / BN;
  prefetch(0);
  stage(0);
  // The query fragments are complete here; without this wait the counter bookkeeping
  // (which sees the staging waits only on some paths) keeps them pending into the loop
  // and waits for the next block's prefetch before the first MFMA of every block.
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();
  for (int kb = 0; kb < nkb; ++kb) {
    const int buf = kb & 1;
    const int kb0 = kb * BN;
    // one key block against this wave's queries; DIAG: some (key > query) pairs to mask
    auto block = [&](auto diag_c) {
      constexpr bool DIAG = decltype(diag_c)::value;
      if constexpr (FAM != 0) {  // reduced family: block dot products, squared and summed
#pragma unroll
        for (int kp = 0; kp < NKP; ++kp) {
          u32x4_t a[2][KS];
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
              a[h][ks] = *reinterpret_cast<const u32x4_t*>(&sK[buf][(16 * (2 * kp + h) + ln) * KP + 32 * ks + 8 * lg]);
          f32x4_t ik2[2] = {f32x4_t{1.f, 1.f, 1.f, 1.f}, f32x4_t{1.f, 1.f, 1.f, 1.f}};
          if constexpr (!NRM) {
            const f32x4_t ik0 = *reinterpret_cast<const f32x4_t*>(&sInvK[buf][32 * kp + 4 * lg]);
            const f32x4_t ik1 = *reinterpret_cast<const f32x4_t*>(&sInvK[buf][32 * kp + 16 + 4 * lg]);
            ik2[0] = ik0 * ik0;
            ik2[1] = ik1 * ik1;
          }
          bf16x8_t vb[NT];
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
            vb[nt] = *reinterpret_cast<const bf16x8_t*>(&sVt[buf][vt_row(16 * nt + ln) * VTP + 32 * kp + 8 * lg]);
#pragma unroll
          for (int qt = 0; qt < NQT; ++qt) {
            const int query = qw0 + 16 * qt + ln;
            float w[8];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              f32x4_t sq = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
              for (int qa = 0; qa < G; ++qa)
#pragma unroll
                for (int kb = 0; kb < G; ++kb) {
                  if (FAM == 2 && kb != qa) continue;
                  f32x4_t St = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                  for (int i = 0; i < KM; ++i)
                    St = mfma16(__builtin_bit_cast(qop_t, a[h][kb * KM + i]), qf[qt][qa * KM + i], St);
                  sq += St * St;
                }
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                w[4 * h + r] = NRM ? sq[r] : sq[r] * ik2[h][r];
                if (DIAG && kb0 + 32 * kp + 16 * h + 4 * lg + r > query) w[4 * h + r] = 0.f;
              }
            }
            const bf16x8_t wa = __builtin_bit_cast(bf16x8_t, u32x4_t{pk2(w[0], w[1]), pk2(w[2], w[3]), pk2(w[4], w[5]), pk2(w[6], w[7])});
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) O[qt][nt] = mfma16(vb[nt], wa, O[qt][nt]);
            D[qt] = mfma16(ones, wa, D[qt]);
          }
        }
        return;
      }
#pragma unroll
      for (int kp = 0; kp < NKP; ++kp) {
        // S^T tiles of key pair kp: keys 32 kp + 16 h + 4 lg + r (rows), queries 16 qt + ln
        f32x4_t St[2][NQT];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int kt = 2 * kp + h;
#pragma unroll
          for (int qt = 0; qt < NQT; ++qt) St[h][qt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            u32x4_t a = {0u, 0u, 0u, 0u};
            if (P >= 32 || lg < 2) a = *reinterpret_cast<const u32x4_t*>(&sK[buf][(16 * kt + ln) * KP + 32 * ks + 8 * lg]);
#pragma unroll
            for (int qt = 0; qt < NQT; ++qt) St[h][qt] = mfma16(__builtin_bit_cast(qop_t, a), qf[qt][ks], St[h][qt]);
          }
        }
        f32x4_t ik0 = f32x4_t{1.f, 1.f, 1.f, 1.f}, ik1 = ik0;
        if constexpr (!NRM) {
          ik0 = *reinterpret_cast<const f32x4_t*>(&sInvK[buf][32 * kp + 4 * lg]);
          ik1 = *reinterpret_cast<const f32x4_t*>(&sInvK[buf][32 * kp + 16 + 4 * lg]);
        }
        // V^T operand: keys 32kp + 4lg + j and 32kp + 16 + 4lg + j, one 16-byte read
        bf16x8_t vb[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          vb[nt] = *reinterpret_cast<const bf16x8_t*>(&sVt[buf][vt_row(16 * nt + ln) * VTP + 32 * kp + 8 * lg]);
#pragma unroll
        for (int qt = 0; qt < NQT; ++qt) {
          const int query = qw0 + 16 * qt + ln;
          float w[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int h = j >> 2, r = j & 3;
            const float s = NRM ? St[h][qt][r] : St[h][qt][r] * (h ? ik1[r] : ik0[r]);
            const float s2 = s * s;
            float ww = s2;
#pragma unroll
            for (int o = 1; o < R; ++o) ww *= s2;
            w[j] = ww;
            if (DIAG && kb0 + 32 * kp + 16 * h + 4 * lg + r > query) w[j] = 0.f;
          }
          const bf16x8_t wa = __builtin_bit_cast(bf16x8_t, u32x4_t{pk2(w[0], w[1]), pk2(w[2], w[3]), pk2(w[4], w[5]), pk2(w[6], w[7])});
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) O[qt][nt] = mfma16(vb[nt], wa, O[qt][nt]);  // O^T += V^T W^T
          D[qt] = mfma16(ones, wa, D[qt]);
        }
      }
    };
    if (kb0 <= qw0 + QW - 1 && qw0 < len) {
      if (kb0 + BN - 1 > qw0) block(std::true_type{});
      else block(std::false_type{});
    }
    if (kb + 1 < nkb) {  // into the buffer of block kb - 1: every wave is past it
      prefetch(kb0 + BN);
      stage(buf ^ 1);
    }
    __syncthreads();
  }

  // ---- epilogue: lane holds columns 16 nt + 4 lg + r of query qw0 + 16 qt + ln
  if constexpr (STATS) {
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt) {
      const int query = qw0 + 16 * qt + ln;
      const float den = D[qt][0];
      const float inv = den > 0.f ? __builtin_amdgcn_rcpf(den) : 0.f;
      float part = 0.f;  // this lane's columns of gout . o
      const int64_t row = row0 + (int64_t)query * stp;
      if (query < len) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const u32x2_t gw = *reinterpret_cast<const u32x2_t*>(gout + row * DV + 16 * nt + 4 * lg);
          const f32x4_t x = O[qt][nt] * inv;
          part += x[0] * bf16_bits_to_f32(gw[0] & 0xffffu) + x[1] * __uint_as_float(gw[0] & 0xffff0000u) +
                  x[2] * bf16_bits_to_f32(gw[1] & 0xffffu) + x[3] * __uint_as_float(gw[1] & 0xffff0000u);
        }
      }
      part = xor32_sum(xor16_sum(part));  // over the four lane groups (all lanes take part)
      if (query < len && lg == 0)
        *reinterpret_cast<u32x2_t*>(stats + row * 2) = u32x2_t{__float_as_uint(den), __float_as_uint(part)};
    }
    return;
  }
#pragma unroll
  for (int qt = 0; qt < NQT; ++qt) {
    const int query = qw0 + 16 * qt + ln;
    if (query >= len) continue;
    const float den = D[qt][0];
    const float inv = den > 0.f ? __builtin_amdgcn_rcpf(den) : 0.f;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const f32x4_t x = O[qt][nt] * inv;
      const int64_t idx = (row0 + (int64_t)query * stp) * DV + 16 * nt + 4 * lg;
      if constexpr (OUT_BF16)
        *reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(o) + idx) = u32x2_t{pk2(x[0], x[1]), pk2(x[2], x[3])};
      else
        *reinterpret_cast<f32x4_t*>(static_cast<float*>(o) + idx) = x;
    }
  }
}

template <int P, int DV>
static hipError_t launch_quad_pd(const uint16_t* q, const uint16_t* k, const uint16_t* v, void* o,
                                 bool o_bf16, int BH, int T, hipStream_t st) {
  const int nqb = (T + quad::BM - 1) / quad::BM;
  dim3 grid((unsigned)((int64_t)nqb * BH)), block(quad::NTHR);
  if (o_bf16) quadratic_bf16_kernel<P, DV, true><<<grid, block, 0, st>>>(q, k, v, o, T, nqb, nullptr, nullptr);
  else quadratic_bf16_kernel<P, DV, false><<<grid, block, 0, st>>>(q, k, v, o, T, nqb, nullptr, nullptr);
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

// packed token-major sequences (SeqLayout with cu set): grid of the padded call with
// T = max_len; query blocks past a sequence's length return at once
template <int P, int DV, int FAM = 0, int G = 1>
static hipError_t launch_quad_packed(const uint16_t* q, const uint16_t* k, const uint16_t* v, void* o, bool o_bf16,
                                     int BH, int H, int max_len, SeqLayout lay, hipStream_t st) {
  const int nqb = (max_len + quad::BM - 1) / quad::BM;
  dim3 grid((unsigned)((int64_t)nqb * BH)), block(quad::NTHR);
  if (o_bf16)
    quadratic_bf16_kernel<P, DV, true, FAM, G, 1, false, true>
        <<<grid, block, 0, st>>>(q, k, v, o, max_len, nqb, nullptr, nullptr, lay, H);
  else
    quadratic_bf16_kernel<P, DV, false, FAM, G, 1, false, true>
        <<<grid, block, 0, st>>>(q, k, v, o, max_len, nqb, nullptr, nullptr, lay, H);
  return hipGetLastError();
}

hipError_t launch_quadratic_bf16_varlen(const uint16_t* q, const uint16_t* k, const uint16_t* v, void* o,
                                        bool o_bf16, int B, int H, int max_len, int p, int dv, int fam, int g,
                                        SeqLayout lay, hipStream_t st) {
  const int BH = B * H;
  if (fam != 0) {  // the reduced families with 32-component blocks (p = 64, g = 2)
    if (!quadratic_bf16_family_supported(p, dv, fam, g)) return hipErrorInvalidValue;
#define KATA_QVFCASE(DD, FF) \
  if (dv == DD && fam == FF) return launch_quad_packed<64, DD, FF, 2>(q, k, v, o, o_bf16, BH, H, max_len, lay, st);
    KATA_QVFCASE(16, 1) KATA_QVFCASE(32, 1) KATA_QVFCASE(64, 1)
    KATA_QVFCASE(16, 2) KATA_QVFCASE(32, 2) KATA_QVFCASE(64, 2)
#undef KATA_QVFCASE
    return hipErrorInvalidValue;
  }
#define KATA_QVCASE(PP, DD) \
  if (p == PP && dv == DD) return launch_quad_packed<PP, DD>(q, k, v, o, o_bf16, BH, H, max_len, lay, st);
  KATA_QVCASE(16, 16) KATA_QVCASE(16, 32) KATA_QVCASE(16, 64)
  KATA_QVCASE(32, 16) KATA_QVCASE(32, 32) KATA_QVCASE(32, 64)
  KATA_QVCASE(64, 16) KATA_QVCASE(64, 32) KATA_QVCASE(64, 64)
#undef KATA_QVCASE
  return hipErrorInvalidValue;
}

template <int P, int DV, int R>
static hipError_t launch_quad_order(const uint16_t* q, const uint16_t* k, const uint16_t* v, void* o, bool o_bf16,
                                    int BH, int T, hipStream_t st) {
  const int nqb = (T + quad::BM - 1) / quad::BM;
  dim3 grid((unsigned)((int64_t)nqb * BH)), block(quad::NTHR);
  if (o_bf16) quadratic_bf16_kernel<P, DV, true, 0, 1, R><<<grid, block, 0, st>>>(q, k, v, o, T, nqb, nullptr, nullptr);
  else quadratic_bf16_kernel<P, DV, false, 0, 1, R><<<grid, block, 0, st>>>(q, k, v, o, T, nqb, nullptr, nullptr);
  return hipGetLastError();
}

// weights (q_hat . k_hat)^4 (r = 2) on the MFMA kernel for the full map's (p, dv) set
hipError_t launch_quadratic_bf16_order2(const uint16_t* q, const uint16_t* k, const uint16_t* v, void* o,
                                        bool o_bf16, int B, int H, int T, int p, int dv, hipStream_t st) {
  const int BH = B * H;
#define KATA_QOCASE(PP, DD) \
  if (p == PP && dv == DD) return launch_quad_order<PP, DD, 2>(q, k, v, o, o_bf16, BH, T, st);
  KATA_QOCASE(16, 16) KATA_QOCASE(16, 32) KATA_QOCASE(16, 64)
  KATA_QOCASE(32, 16) KATA_QOCASE(32, 32) KATA_QOCASE(32, 64)
  KATA_QOCASE(64, 16) KATA_QOCASE(64, 32) KATA_QOCASE(64, 64)
#undef KATA_QOCASE
  return hipErrorInvalidValue;
}

// reduced families with 32-component blocks (p = 64, g = 2); false if not covered here
bool quadratic_bf16_family_supported(int p, int dv, int fam, int g) {
  return p == 64 && g == 2 && (fam == 1 || fam == 2) && (dv == 16 || dv == 32 || dv == 64);
}

template <int DV, int FAM>
static hipError_t launch_quad_fam(const uint16_t* q, const uint16_t* k, const uint16_t* v, void* o, bool o_bf16,
                                  int BH, int T, hipStream_t st) {
  const int nqb = (T + quad::BM - 1) / quad::BM;
  dim3 grid((unsigned)((int64_t)nqb * BH)), block(quad::NTHR);
  if (o_bf16) quadratic_bf16_kernel<64, DV, true, FAM, 2><<<grid, block, 0, st>>>(q, k, v, o, T, nqb, nullptr, nullptr);
  else quadratic_bf16_kernel<64, DV, false, FAM, 2><<<grid, block, 0, st>>>(q, k, v, o, T, nqb, nullptr, nullptr);
  return hipGetLastError();
}

hipError_t launch_quadratic_bf16_family(const uint16_t* q, const uint16_t* k, const uint16_t* v, void* o,
                                        bool o_bf16, int B, int H, int T, int p, int dv, int fam, int g,
                                        hipStream_t st) {
  if (!quadratic_bf16_family_supported(p, dv, fam, g)) return hipErrorInvalidValue;
  const int BH = B * H;
  if (fam == 1) {
    if (dv == 16) return launch_quad_fam<16, 1>(q, k, v, o, o_bf16, BH, T, st);
    if (dv == 32) return launch_quad_fam<32, 1>(q, k, v, o, o_bf16, BH, T, st);
    return launch_quad_fam<64, 1>(q, k, v, o, o_bf16, BH, T, st);
  }
  if (dv == 16) return launch_quad_fam<16, 2>(q, k, v, o, o_bf16, BH, T, st);
  if (dv == 32) return launch_quad_fam<32, 2>(q, k, v, o, o_bf16, BH, T, st);
  return launch_quad_fam<64, 2>(q, k, v, o, o_bf16, BH, T, st);
}

// backward statistics of the full map over packed sequences (T = max_len; stats per row of
// the packed layout)
hipError_t launch_quadratic_bf16_stats_varlen(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                              const uint16_t* gout, float* stats, int B, int H, int max_len, int p,
                                              int dv, SeqLayout lay, hipStream_t st) {
  const int BH = B * H;
  const int nqb = (max_len + quad::BM - 1) / quad::BM;
  dim3 grid((unsigned)((int64_t)nqb * BH)), block(quad::NTHR);
#define KATA_SCASE(PP, DD)                                                                                   \
  if (p == PP && dv == DD) {                                                                                 \
    quadratic_bf16_kernel<PP, DD, false, 0, 1, 1, true, true>                                                \
        <<<grid, block, 0, st>>>(q, k, v, nullptr, max_len, nqb, gout, stats, lay, H);                       \
    return hipGetLastError();                                                                                \
  }
  KATA_SCASE(32, 32) KATA_SCASE(32, 64) KATA_SCASE(64, 32) KATA_SCASE(64, 64)
#undef KATA_SCASE
  return hipErrorInvalidValue;
}

// backward statistics of the full map (STATS above) for bf16 q, k, v, gout
hipError_t launch_quadratic_bf16_stats(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* gout,
                                       float* stats, int B, int H, int T, int p, int dv, hipStream_t st) {
  const int BH = B * H;
  const int nqb = (T + quad::BM - 1) / quad::BM;
  dim3 grid((unsigned)((int64_t)nqb * BH)), block(quad::NTHR);
#define KATA_SCASE(PP, DD)                                                                                        \
  if (p == PP && dv == DD) {                                                                                      \
    quadratic_bf16_kernel<PP, DD, false, 0, 1, 1, true><<<grid, block, 0, st>>>(q, k, v, nullptr, T, nqb, gout,  \
                                                                               stats);                           \
    return hipGetLastError();                                                                                     \
  }
  KATA_SCASE(32, 32) KATA_SCASE(32, 64) KATA_SCASE(64, 32) KATA_SCASE(64, 64)
#undef KATA_SCASE
  return hipErrorInvalidValue;
}

}  // namespace kata
