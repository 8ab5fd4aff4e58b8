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
// Design (one workgroup = 8 waves per (b,h,segment); the state never leaves the chip):
//   * The n = p(p+1)/2 packed features are ordered internally as tiles of 16 features.
//     In tile tau, row m (0..15) holds a pair (i, j) in which one index is m (or 16+m)
//     and the other is m rotated by a tile constant inside its 16-lane row. Hence a
//     lane that holds the natural components k_hat[t][m], k_hat[t][16+m] builds its
//     A-operand row of psi(K)^T with ONE v_mul_f32 whose first operand is a DPP row
//     rotation: the lift costs one multiply per feature and never touches LDS or HBM.
//     p = 32 gives 33 tiles = 528 features exactly; p = 16 gives 9 tiles (136 + 8 pad).
//   * The state S (fp32) lives in MFMA accumulators, split by feature tiles over the 8
//     waves in whole readout pairs (two tiles = one 32-feature k-step). After each
//     chunk's build every wave writes its pairs once to LDS as bf16 B fragments
//     (accumulator rows 4g..4g+3 of the two tiles become the k-slots of lane group g;
//     the readout side permutes its k-slots the same way).
//   * Readout: wave w serves token tile w mod (C/16) over a range of the feature pairs;
//     the splits of a token tile exchange partial sums through LDS. Operands are swapped
//     (O^T = S^T psi(Q)^T): each lane ends with 4 consecutive output columns of one query.
//     psi(q) comes from a per-lane-group rotated copy of q (raw products q_i q_j).
//   * Queries are used as given, not normalised: psi(q) = ||q||^2 psi(q_hat) scales the
//     numerator and the denominator of o_t alike. The raw bf16 q is exact as an MFMA
//     operand, so the denominator and the intra scores need no split query.
//   * Off-diagonal coordinates carry sqrt(2) in psi; their product c_ij^2 = 2 is folded
//     into the state build: k_hat^T is staged as sqrt(2) k_hat, so an off-diagonal product
//     is 2 k_i k_j, a diagonal one is halved, and the Gram tile (2 M) is halved when
//     applied. The readout uses raw products q_i q_j.
//   * The denominator psi(q)^T Z = q^T M q with the Gram matrix M = sum_s k_hat_s k_hat_s^T
//     (p x p), applied as bf16 hi + lo of M against the exact q (2 MFMAs per tile), so the
//     normaliser is fp32-accurate.
//   * Intra-chunk block: S^T = K_hat Q^T (keys as M), W = (S^T)^2 masked, rounded to
//     bf16, O^T += V^T W^T. Global chunk 0, where denominators are sums of few weights,
//     uses split-bf16 keys.
//   * Per chunk: phase 1 = readout from the state before the chunk + the chunk's build
//     into the registers (both read only the state before it) | barrier | phase 2 =
//     output, staging of the next chunk, state back to LDS | barrier.
//   * LDS layouts follow measured gfx950 bank behaviour: 4-byte writes go in 32-lane
//     passes over 32 banks; 16-byte reads by lanes (row, group) at row * pitch + 4 group
//     floats are conflict-free for pitch = 8 * odd (mod 128 floats).
//   * SEQUENTIAL: one workgroup per (b,h) walks all chunks. ASSOCIATIVE: a summary pass
//     writes each segment's [S | M] (fp32, in this tile layout), an in-place scan forms
//     the prefixes, and every segment runs its chunks from its prefix.
#pragma once
#include <utility>

#include "kata_device.h"
#include "kata_launch.h"

namespace kata {

hipError_t launch_scan(float* ws, int BH, int nslots, int64_t E, hipStream_t st);

namespace chk {

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
// lane m of each 16-lane row receives x from lane (m + D) & 15 (DPP row_ror by 16 - D)
template <int D>
__device__ __forceinline__ float rot(float x) {
  if constexpr ((D & 15) == 0) return x;
  else
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x),
                                                               0x120 + (16 - (D & 15)), 0xf, 0xf, true));
}

__device__ __forceinline__ f32x4_t mfma(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t zero4() { return f32x4_t{0.f, 0.f, 0.f, 0.f}; }
__device__ __forceinline__ bf16x8_t zero_bf8() {
  return __builtin_bit_cast(bf16x8_t, u16x8_t{0, 0, 0, 0, 0, 0, 0, 0});
}

__device__ __forceinline__ bf16x8_t pack8(const float (&x)[8]) {
  return __builtin_bit_cast(bf16x8_t, u32x4_t{pk2(x[0], x[1]), pk2(x[2], x[3]), pk2(x[4], x[5]), pk2(x[6], x[7])});
}
// low / high bf16 of a packed pair as fp32
__device__ __forceinline__ float lo_f32(uint32_t p) { return __uint_as_float(p << 16); }
__device__ __forceinline__ float hi_f32(uint32_t p) { return __uint_as_float(p & 0xffff0000u); }

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
  float x[8];
  x[0] = ro_feat<P, T1, 0>(Y, glow);
  x[1] = ro_feat<P, T1, 1>(Y, glow);
  x[2] = ro_feat<P, T1, 2>(Y, glow);
  x[3] = ro_feat<P, T1, 3>(Y, glow);
  if constexpr (HAS2) {
    x[4] = ro_feat<P, T2, 0>(Y, glow);
    x[5] = ro_feat<P, T2, 1>(Y, glow);
    x[6] = ro_feat<P, T2, 2>(Y, glow);
    x[7] = ro_feat<P, T2, 3>(Y, glow);
  } else {
    x[4] = x[5] = x[6] = x[7] = 0.f;
  }
  return pack8(x);
}

// split x (8 fp32) into bf16 hi and lo = bf16(x - hi)
__device__ __forceinline__ void split8(const float (&x)[8], bf16x8_t& hi, bf16x8_t& lo) {
  u32x4_t h, l;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    h[j] = pk2(x[2 * j], x[2 * j + 1]);
    l[j] = pk2(x[2 * j] - lo_f32(h[j]), x[2 * j + 1] - hi_f32(h[j]));
  }
  hi = __builtin_bit_cast(bf16x8_t, h);
  lo = __builtin_bit_cast(bf16x8_t, l);
}

// ---- work split over the 8 waves of a workgroup
constexpr int NW = 8;
// state-build tiles per wave, aligned to readout pairs (2 tiles) so every wave writes whole
// 16-byte state fragments. p=32: wave 0 has tiles 0..3 and the odd tile 32, wave w > 0 has
// 4w..4w+3; p=16: waves 0..3 have 2w, 2w+1, wave 4 tile 8, waves 5..7 none. Low waves get
// the extra build work: the high waves of a token tile carry its intra block.
template <int P> constexpr int wave_nt(int w) { return P == 32 ? (w == 0 ? 5 : 4) : (w < 4 ? 2 : (w == 4 ? 1 : 0)); }
template <int P> constexpr int wave_tile(int w, int i) {
  return P == 32 ? (w == 0 ? (i < 4 ? i : 32) : 4 * w + i) : (w < 4 ? 2 * w + i : 8);
}
// register array extent (at least 1; a wave without tiles keeps one unused)
template <int P> constexpr int wave_na(int w) { return wave_nt<P>(w) > 0 ? wave_nt<P>(w) : 1; }
// Gram-matrix tile owned by wave w (-1: none; p=32 has 4 tiles, on waves 1..4, p=16 one)
template <int P> constexpr int m_tile(int w) { return P == 32 ? (w >= 1 && w <= 4 ? w - 1 : -1) : (w == 5 ? 0 : -1); }

// Build-work maps: state tiles, Gram tile and (pass 1 only) one column tile of the odd
// state tile 32 per wave. Map8: the forward's 8 waves, as above.
struct Map8 {
  template <int P> static constexpr int nt(int w) { return wave_nt<P>(w); }
  template <int P> static constexpr int tile(int w, int i) { return wave_tile<P>(w, i); }
  template <int P> static constexpr int mtile(int w) { return m_tile<P>(w); }
  template <int P> static constexpr int xdt(int, int) { return -1; }
};
// Map16: pass 1 (segment summaries) on 16 waves, 4 per SIMD. p=32: wave w builds tiles
// 2w, 2w+1; tile 32 is split by output column tile over waves 8..8+NT-1 and the Gram tiles
// sit on waves 12..15 (waves 0-7 also normalise the chunk's keys, 8-15 only write V^T).
// p=16: wave w < 9 builds tile w; the Gram tile is on wave 9.
struct Map16 {
  template <int P> static constexpr int nt(int w) { return P == 32 ? 2 : (w < 9 ? 1 : 0); }
  template <int P> static constexpr int tile(int w, int i) { return P == 32 ? 2 * w + i : (w < 9 ? w : 0); }
  template <int P> static constexpr int mtile(int w) { return P == 32 ? (w >= 12 ? w - 12 : -1) : (w == 9 ? 0 : -1); }
  template <int P> static constexpr int xdt(int w, int nt) { return P == 32 && w >= 8 && w < 8 + nt ? w - 8 : -1; }
};
template <class MAP, int P> constexpr int map_na(int w) { return MAP::template nt<P>(w) > 0 ? MAP::template nt<P>(w) : 1; }

// A operand of the state build for tile TAU: row m = this lane's feature, 8 tokens.
// N[h][j] = sqrt(2) k_hat[token j][16h + m] (staged that way): an off-diagonal product
// N_i N_j = 2 k_i k_j already carries c_ij^2 = 2, a diagonal one is halved. Both operands
// come straight from LDS, so the compiler folds the DPP row rotation into the multiply.
template <int P, int TAU>
__device__ __forceinline__ bf16x8_t build_frag(const float (&N)[P / 16][8], bool mlow) {
  constexpr int kind = tile_kind<P>(TAU), h = tile_half<P>(TAU), d = tile_delta<P>(TAU);
  float x[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if constexpr (kind == K_DIAG) {
      x[j] = (N[h][j] * N[h][j]) * 0.5f;
    } else if constexpr (kind == K_WITHIN) {
      x[j] = N[h][j] * rot<d>(N[h][j]);
    } else if constexpr (kind == K_WITHIN8) {
      if constexpr (P == 32) {
        const float a = mlow ? N[0][j] : N[1][j];
        const float b = mlow ? N[1][j] : N[0][j];
        x[j] = a * rot<8>(b);
      } else {
        const float a = mlow ? N[0][j] : 0.f;
        x[j] = a * rot<8>(N[0][j]);
      }
    } else {
      x[j] = N[0][j] * rot<d>(N[P / 16 - 1][j]);
    }
  }
  return pack8(x);
}


template <int P, int DV, int C>
struct Cfg {
  static constexpr int NT = DV / 16;            // output column tiles
  static constexpr int NH = P / 16;             // 16-component halves
  static constexpr int NMT = C / 16;            // token tiles per chunk
  static constexpr int FS = NW / NMT;           // waves sharing one token tile's readout
  static constexpr int KSTEP = C / 32;          // 32-token k-steps of the build
  static constexpr int NTL = ntiles<P>();       // 16-feature tiles
  static constexpr int NPAIR = (NTL + 1) / 2;   // 32-feature readout k-steps
  // LDS pitches: 16-byte reads by lanes (row ln, group lg) at ln * pitch + 4 lg floats are
  // conflict-free when the pitch is 8 * odd floats modulo 128 (measured on gfx950)
  static constexpr int QP = P + 8;              // fp32 pitch of q_hat / k_hat rows
  // k_hat^T: component row r at r * KTP + 8 (r / KQ) (skew per staging quarter), token
  // planes HP apart; with KTP = 16 (mod 32) both its transposed 4-byte writes and the
  // build's 16-byte reads are conflict-free
  static constexpr int HP = C / 2;
  static constexpr int KTP = 16 + 32 * ((C + 8 + 31) / 32);
  static constexpr int VTP = 80 + 128 * ((C - 80 + 127) / 128);  // bf16 pitch of V^T rows
  static constexpr int MP = C == 128 ? P : P + 8;  // bf16 pitch of the Gram matrix rows (unpadded where LDS is short)
  static constexpr int SB_BYTES = NPAIR * NT * 64 * 16;            // bf16 state, B-fragment order
  static constexpr int PART_BYTES = NMT * (FS - 1) * NT * 64 * 16;  // partial outputs (fp32 acc layout)
  static constexpr int PD_BYTES = FS > 1 ? NMT * 64 * 4 : 0;        // denominators handed to the other splits
  static constexpr int OFF_SB = 0;
  static constexpr int OFF_QH = OFF_SB + SB_BYTES;
  static constexpr int OFF_KH = OFF_QH + C * QP * 4;
  static constexpr int OFF_VT = OFF_KH + C * QP * 4;  // V^T, read by the intra block and the build
  static constexpr int OFF_KT = OFF_VT + DV * VTP * 2;
  static constexpr int OFF_M = OFF_KT + P * KTP * 4;                // bf16 [hi,lo][P][MP]
  static constexpr int OFF_PART = OFF_M + 2 * P * MP * 2;
  static constexpr int OFF_PD = OFF_PART + PART_BYTES;
  static constexpr int LDS = OFF_PD + PD_BYTES;
  static_assert(LDS <= 160 * 1024, "LDS budget");
  // summary pass: build operands only, double-buffered
  static constexpr int SUM_BUF = DV * VTP * 2 + P * KTP * 4;
  static constexpr int SUM_LDS = 2 * SUM_BUF;
  static constexpr int64_t STATE_FLOATS = (int64_t)NTL * NT * 256 + NH * NH * 256;
  // staging work per thread: 4 threads per q/k row (KQ components), one (key pair,
  // 8 columns) V piece
  static constexpr int KQ = P / 4;
  static constexpr int QK_PIECES = 2 * 4 * C;                  // q and k row pieces
  static_assert(VTP >= C && KTP >= 24 + 2 * HP, "pitches");
  static constexpr int QKI = (QK_PIECES + 511) / 512;
  static constexpr int VPIECES = (C / 2) * (DV / 8);
  static constexpr int VI = (VPIECES + 511) / 512;
  __device__ static __forceinline__ void vpiece(int pc, int& vp, int& vd) { vt_piece<DV>(pc, vp, vd); }
  // readout pair ranges of token tile tt: split fs covers pairs [pr(fs, tt), pr(fs + 1, tt)).
  // The last split also runs the intra block and the denominator (more work for larger tt),
  // so it takes fewer pairs; the others share the rest evenly.
  static constexpr int owner_pairs(int tt) {
    const int even = NPAIR / FS, less = 3 + tt / 2;
    return FS == 1 ? NPAIR : (even - less >= 1 ? even - less : 1);
  }
  static constexpr int pr(int fs, int tt) {
    return fs >= FS ? NPAIR : (FS == 1 ? 0 : (fs * (NPAIR - owner_pairs(tt))) / (FS - 1));
  }
  // the FS splits of a token tile share its output: split out_owner(dt) normalises and
  // stores output column tile dt, after adding the other splits' partial sums
  static constexpr int out_owner(int dt) { return NT >= FS ? dt * FS / NT : dt; }
  static constexpr bool owns_any(int f) { return NT >= FS || f < NT; }
  // LDS slot of split f's partial sum of column tile dt of token tile tt (f != out_owner(dt))
  static constexpr int part_slot(int tt, int dt, int f) {
    return (tt * NT + dt) * (FS - 1) + (f < out_owner(dt) ? f : f - 1);
  }
};

struct Args {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  void* o;
  float* ws;
  int T, nseg, cps, nblk_per_bh;
  int o_f32;  // output dtype: 1 = fp32, 0 = bf16
  float* s_out;  // final state S [B,H,n,DV] in the decode layout, or null
  float* z_out;  // final state Z [B,H,n], or null
  SeqLayout lay;     // row layout and per-sequence lengths (S2: padded layout only)
  int H;
};

// first q/k row, row step and rows in use of sequence bh. Under S2 a.T counts virtual rows
// (two per token) of the padded layout and a length counts tokens.
template <bool S2>
__device__ __forceinline__ void seq_view(const Args& a, int64_t bh, int64_t& row0, int& step, int& len) {
  if constexpr (S2) {
    row0 = bh * (int64_t)a.T;
    step = 1;
    if (a.lay.lens == nullptr) {
      len = a.T;
    } else {
      const int L = a.lay.lens[bh / a.H];
      const int64_t r = (int64_t)(L < 0 ? 0 : L) * 2;
      len = r < a.T ? (int)r : a.T;
    }
  } else {
    seq_rows_of(a.lay, bh, a.H, a.T, row0, step, len);
  }
}



// ---- chunk staging: global bf16 -> registers (load) -> normalised LDS layouts.
// S2 (KATA-Sigma 2 on 2P-wide inputs): a token's two P-component blocks are consecutive
// "virtual" rows of the same memory read as [2T][P] (a.T counts virtual rows); a key is
// normalised over both blocks, and both virtual rows carry the token's value row.
template <int P, int DV, int C, bool WITH_Q, bool S2 = false>
struct Stager {
  using CF = Cfg<P, DV, C>;
  typedef uint16_t row_t __attribute__((ext_vector_type(P / 4)));
  // WITH_Q (forward, 512 threads): q then k row pieces on tid + 512 i, V pieces on
  // tid + 512 i. Otherwise (pass 1, 1024 threads): k pieces on threads 0..4C-1 and V pieces
  // on the threads after them, one of either per thread.
  static constexpr int NQK = WITH_Q ? CF::QKI : 1, NV = WITH_Q ? CF::VI : 1;
  static_assert(WITH_Q || 4 * C + CF::VPIECES <= 1024, "pass-1 staging layout");
  row_t qk[NQK];          // piece i: q (first 4C pieces) or k row piece
  float kx[NQK][CF::KQ];  // normalised k pieces of the rows staged last (forward only)
  u16x8_t vr[NV][2];
  // q/k piece index of slot i (k pieces are numbered from 4C), -1 for none
  __device__ static __forceinline__ int qk_piece(int i) {
    const int tid = threadIdx.x;
    if constexpr (WITH_Q) return tid + 512 * i;
    return tid < 4 * C ? 4 * C + tid : -1;
  }
  // V piece index of slot i (may be out of [0, VPIECES))
  __device__ static __forceinline__ int v_piece(int i) {
    const int tid = threadIdx.x;
    if constexpr (WITH_Q) return tid + 512 * i;
    return tid - 4 * C;
  }
  const uint16_t *qb, *kb, *vb;
  int T;           // rows in use
  uint32_t rsp, rsv;  // elements between consecutive q / k rows and v rows

  __device__ __forceinline__ void init(const Args& a, int64_t bh) {
    int64_t row0;
    int rs;
    seq_view<S2>(a, bh, row0, rs, T);  // rows past the sequence's length read as zero
    rsp = (uint32_t)rs * P;
    rsv = (uint32_t)rs * DV;
    qb = a.q + row0 * P;
    kb = a.k + row0 * P;
    vb = a.v + (S2 ? bh * (int64_t)(a.T / 2) : row0) * DV;
  }

  __device__ __forceinline__ row_t load_piece(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    if constexpr (P == 32)
      return __builtin_bit_cast(row_t, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
    else
      return __builtin_bit_cast(row_t, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
  }

  // the chunk's rows t0.. as buffers: rows past T read as zero
  __device__ __forceinline__ void load(int t0) {
    const int tid = threadIdx.x;
    const uint32_t left = (uint32_t)(t0 < T ? T - t0 : 0);  // a chunk past the end reads zeros
    // byte ranges end with the last row in use (rows are rs rows apart)
    const uint32_t qk_bytes = left ? ((left - 1) * rsp + P) * 2 : 0;
    const uint32_t v_bytes = left ? ((left - 1) * rsv + DV) * 2 : 0;
    const __amdgpu_buffer_rsrc_t rq = buf_rsrc(qb + (int64_t)t0 * rsp, qk_bytes);
    const __amdgpu_buffer_rsrc_t rk = buf_rsrc(kb + (int64_t)t0 * rsp, qk_bytes);
    const __amdgpu_buffer_rsrc_t rv = S2 ? buf_rsrc(vb + (int64_t)(t0 / 2) * DV, (left / 2) * DV * 2)
                                         : buf_rsrc(vb + (int64_t)t0 * rsv, v_bytes);
#pragma unroll
    for (int i = 0; i < NQK; ++i) {
      const int pc = qk_piece(i);
      if (pc < 0) continue;  // whole waves
      // q or k is uniform across a wave (4C is a multiple of 64)
      const int isq = __builtin_amdgcn_readfirstlane(pc < 4 * C ? 1 : 0);
      const int row = (isq ? pc : pc - 4 * C) >> 2, kq = pc & 3;
      const uint32_t voff = (row * rsp + kq * CF::KQ) * 2;
      if (pc < CF::QK_PIECES && (WITH_Q || !isq)) qk[i] = load_piece(isq ? rq : rk, voff, 0);
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int pc = v_piece(i);
      if (pc >= 0 && pc < CF::VPIECES) {
        int vp, vd;
        CF::vpiece(pc, vp, vd);
        if constexpr (S2) {  // key pair vp = the two blocks of token vp: one value row
          const uint32_t voff = (uint32_t)(vp * DV + 8 * vd) * 2;
          vr[i][0] = __builtin_bit_cast(u16x8_t, __builtin_amdgcn_raw_buffer_load_b128(rv, voff, 0, 0));
          vr[i][1] = vr[i][0];
        } else {
          const uint32_t voff = (2 * vp * rsv + 8 * vd) * 2;
          vr[i][0] = __builtin_bit_cast(u16x8_t, __builtin_amdgcn_raw_buffer_load_b128(rv, voff, 0, 0));
          vr[i][1] = __builtin_bit_cast(u16x8_t, __builtin_amdgcn_raw_buffer_load_b128(rv, voff + rsv * 2, 0, 0));
        }
      }
    }
  }

  // normalised row piece (4 consecutive lanes share a row, 8 a token under S2; the norm is
  // combined over them)
  __device__ __forceinline__ void normalise(const row_t& src, float (&x)[CF::KQ], float scale = 1.f) {
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < CF::KQ; ++e) {
      x[e] = bf16_bits_to_f32(src[e]);
      ss += x[e] * x[e];
    }
    ss = group_sum<S2 ? 8 : 4>(ss);
    const float inv = inv_norm_fast(ss) * scale;
#pragma unroll
    for (int e = 0; e < CF::KQ; ++e) x[e] *= inv;
  }

  // V^T (bf16 [DV][VTP]); key 32a + 16s + 4g + j is stored at 32a + 8g + 4s + j, so lane
  // group g reads its 8 k-slots (keys 32a + 4g + j, 32a + 16 + 4g + j: the row order of the
  // score fragments and of the k_hat^T planes) with one 16-byte read
  __device__ __forceinline__ void write_vt(char* vt_bytes) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int pc = v_piece(i);
      if (pc >= 0 && pc < CF::VPIECES) {
        int vp, vd;
        CF::vpiece(pc, vp, vd);
        const int pos = vt_pos(2 * vp);
        // column 8 vd + e lives in row 8 vd + (e ^ (vd & 3)) (see vt_row)
        char* base = vt_bytes + ((8 * vd) * CF::VTP + pos) * 2;
        char* rb[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) rb[j] = base + (j ^ (vd & 3)) * CF::VTP * 2;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          *reinterpret_cast<uint32_t*>(rb[e & 3] + (e & 4) * CF::VTP * 2) =
              (uint32_t)vr[i][0][e] | ((uint32_t)vr[i][1][e] << 16);
      }
    }
  }

  // row-major q_hat, k_hat (fp32) and V^T for the readout / intra block
  __device__ __forceinline__ void stage_rows(char* lds) {
    static_assert(WITH_Q, "forward staging");
#pragma unroll
    for (int i = 0; i < NQK; ++i) {
      const int pc = qk_piece(i);
      if (CF::QK_PIECES % 512 != 0 && pc >= CF::QK_PIECES) continue;  // whole waves
      const bool isq = pc < 4 * C;
      if (!WITH_Q && isq) continue;
      const int row = (isq ? pc : pc - 4 * C) >> 2, kq = pc & 3;
      float(&x)[CF::KQ] = kx[i];  // k: kept for stage_kt of the same chunk
      if (isq) {  // queries are used unnormalised: the scale of q cancels in the output
#pragma unroll
        for (int e = 0; e < CF::KQ; ++e) x[e] = bf16_bits_to_f32(qk[i][e]);
      } else {
        normalise(qk[i], x);
      }
      float* dst = reinterpret_cast<float*>(lds + (isq ? CF::OFF_QH : CF::OFF_KH)) + row * CF::QP + kq * CF::KQ;
#pragma unroll
      for (int e = 0; e < CF::KQ; e += 4)
        *reinterpret_cast<f32x4_t*>(dst + e) = f32x4_t{x[e], x[e + 1], x[e + 2], x[e + 3]};
    }
  }

  // k_hat^T (fp32) for the state build at byte offset off_kt; ROWS_STAGED: stage_rows already
  // normalised this chunk's k pieces
  template <bool ROWS_STAGED>
  __device__ __forceinline__ void stage_kt(char* lds, int off_kt) {
#pragma unroll
    for (int i = 0; i < NQK; ++i) {
      const int pc = qk_piece(i);
      if (pc < 0 || (CF::QK_PIECES % 512 != 0 && pc >= CF::QK_PIECES)) continue;
      if (pc < 4 * C) continue;  // q pieces
      const int row = (pc - 4 * C) >> 2, kq = pc & 3;
      float x[CF::KQ];  // sqrt(2) k_hat (see build_frag)
      if constexpr (ROWS_STAGED) {
#pragma unroll
        for (int e = 0; e < CF::KQ; ++e) x[e] = kx[i][e] * 1.41421356237309515f;
      } else {
        normalise(qk[i], x, 1.41421356237309515f);
      }
      // component row r starts at r * KTP + 8 (r / KQ); token t sits in plane (t / 16) & 1
      // at (t / 32) * 16 + t % 16 of it
      float* kt = reinterpret_cast<float*>(lds + off_kt) + (kq * CF::KQ) * CF::KTP + 8 * kq +
                  ((row >> 4) & 1) * CF::HP + (row >> 5) * 16 + (row & 15);
#pragma unroll
      for (int e = 0; e < CF::KQ; ++e) kt[e * CF::KTP] = x[e];
    }
  }
};

// ---- state build over this wave's tiles for one chunk
template <int P, int DV, int C, class MAP, int W>
__device__ __forceinline__ void build_chunk(f32x4_t (&S)[(map_na<MAP, P>(W))][DV / 16], f32x4_t& Sx,
                                            f32x4_t& Mt, const float* khT, const uint16_t* vb_lds) {
  using CF = Cfg<P, DV, C>;
  constexpr int NT = CF::NT, NH = CF::NH, NTW = MAP::template nt<P>(W);
  constexpr int MT = MAP::template mtile<P>(W), MRT = MT / NH, MCT = MT % NH;
  constexpr int XDT = MAP::template xdt<P>(W, NT);
  const int lane = threadIdx.x & 63, ln = lane & 15, lg = lane >> 4;
  const bool mlow = ln < 8;
#pragma unroll
  for (int ks = 0; ks < CF::KSTEP; ++ks) {
    float N[NH][8];
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      // k-slot (lg, j) is token 32ks + 16 (j / 4) + 4lg + j % 4: plane 0, then plane 1
      const float* src = khT + (16 * h + ln) * CF::KTP + 8 * ((16 * h + ln) / CF::KQ) + 16 * ks + 4 * lg;
      const f32x4_t x0 = *reinterpret_cast<const f32x4_t*>(src);
      const f32x4_t x1 = *reinterpret_cast<const f32x4_t*>(src + CF::HP);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        N[h][e] = x0[e];
        N[h][4 + e] = x1[e];
      }
    }
    bf16x8_t vbf[NT];
#pragma unroll
    for (int dt = 0; dt < NT; ++dt)
      vbf[dt] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u16x8_t*>(vb_lds + vt_row(16 * dt + ln) * CF::VTP + 32 * ks + 8 * lg));
    [&]<int... TI>(std::integer_sequence<int, TI...>) {
      (([&] {
         const bf16x8_t af = build_frag<P, MAP::template tile<P>(W, TI)>(N, mlow);
#pragma unroll
         for (int dt = 0; dt < NT; ++dt) S[TI][dt] = mfma(af, vbf[dt], S[TI][dt]);
       }()),
       ...);
    }(std::make_integer_sequence<int, NTW>{});
    if constexpr (XDT >= 0) Sx = mfma(build_frag<P, ntiles<P>() - 1>(N, mlow), vbf[XDT], Sx);
    if constexpr (MT >= 0) {  // Gram tile of 2 M = sum 2 k k^T over these 32 tokens (halved when applied)
      Mt = mfma(pack8(N[MRT]), pack8(N[MCT]), Mt);
    }
  }
}

// Packed pair (a, b) of row m of state tile tau (the build side's feature; see build_frag);
// false for the padding rows of the p = 16 half tile.
template <int P>
__device__ __forceinline__ bool feat_pair(int tau, int m, int& a, int& b) {
  const int kind = tile_kind<P>(tau), h = tile_half<P>(tau), d = tile_delta<P>(tau);
  if (kind == K_DIAG) {
    a = b = 16 * h + m;
  } else if (kind == K_WITHIN) {
    a = 16 * h + m;
    b = 16 * h + ((m + d) & 15);
  } else if (kind == K_WITHIN8) {
    if (P == 16) {
      if (m >= 8) return false;
      a = m;
      b = m + 8;
    } else {  // component m (m < 8) or 16 + m, times the rotated partner of the other half
      const int src = (m + 8) & 15;
      a = m < 8 ? m : 16 + m;
      b = src < 8 ? 16 + src : src;
    }
  } else {
    a = m;
    b = 16 + ((m + d) & 15);
  }
  return true;
}

// The recurrent state after a sequence's last token, in the decode layout (feature-value
// state display): S[f][d] = sum_s psi_f(k_hat_s) v_s[d], Z[f] = sum_s psi_f(k_hat_s), with f
// the packed row-major upper-triangle index. The registers hold off-diagonal features with
// c^2 = 2 folded in (divide by sqrt(2) for psi_f) and the Gram tile as 2 M (Z_f = c_f M_ab).
template <int P, int DV, int W>
__device__ __forceinline__ void write_final_state(const Args& a, int64_t bh,
                                                  const f32x4_t (&S)[wave_na<P>(W)][DV / 16],
                                                  const f32x4_t& Mt) {
  constexpr int n = P * (P + 1) / 2, NT = DV / 16, NH = P / 16;
  constexpr int MT = m_tile<P>(W);
  const int lane = threadIdx.x & 63, ln = lane & 15, lg = lane >> 4;
  float* so = a.s_out + bh * (int64_t)n * DV;
#pragma unroll
  for (int i = 0; i < wave_nt<P>(W); ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      int fa, fb;
      if (!feat_pair<P>(wave_tile<P>(W, i), 4 * lg + r, fa, fb)) continue;
      const int i0 = fa < fb ? fa : fb, j0 = fa < fb ? fb : fa;
      const int f = i0 * P - i0 * (i0 - 1) / 2 + (j0 - i0);
      const float sc = i0 == j0 ? 1.f : 0.70710678118654752f;
#pragma unroll
      for (int dt = 0; dt < NT; ++dt) so[(int64_t)f * DV + 16 * dt + ln] = S[i][dt][r] * sc;
    }
  if constexpr (MT >= 0) {
    float* zo = a.z_out + bh * (int64_t)n;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 16 * (MT / NH) + 4 * lg + r, col = 16 * (MT % NH) + ln;
      if (row > col) continue;  // the upper triangle (M is symmetric)
      const int f = row * P - row * (row - 1) / 2 + (col - row);
      zo[f] = 0.5f * Mt[r] * (row == col ? 1.f : 1.41421356237309515f);
    }
  }
}

// ---- forward of one segment; W (wave index) is a template parameter so every tile and
// pair index is a compile-time constant and the lift indexes registers directly.
// S2: KATA-Sigma 2 over virtual rows (see Stager): psi(q)^T S and the denominator of a token
// are the sums over its two virtual query rows (adjacent lanes), the causal mask compares
// tokens, and output row t is token t.
template <int P, int DV, int C, int W, bool S2 = false>
__device__ __forceinline__ void run_fwd(const Args& a, char* lds) {
  using CF = Cfg<P, DV, C>;
  constexpr int NT = CF::NT, NH = CF::NH, NTW = wave_nt<P>(W);
  constexpr int MT = m_tile<P>(W), MRT = MT / NH, MCT = MT % NH;
  constexpr int TT = W % CF::NMT, FSI = W / CF::NMT;   // token tile, feature split
  constexpr bool OWNER = FSI == CF::FS - 1;            // intra block, denominator, output
  constexpr int PB = CF::pr(FSI, TT), PE = CF::pr(FSI + 1, TT);
  const int lane = threadIdx.x & 63, ln = lane & 15, lg = lane >> 4;
  const bool glow = lg < 2;

  const float* qh = reinterpret_cast<const float*>(lds + CF::OFF_QH);
  const float* kh = reinterpret_cast<const float*>(lds + CF::OFF_KH);
  const float* khT = reinterpret_cast<const float*>(lds + CF::OFF_KT);
  const uint16_t* vt = reinterpret_cast<const uint16_t*>(lds + CF::OFF_VT);
  uint16_t* mlds = reinterpret_cast<uint16_t*>(lds + CF::OFF_M);
  char* sb = lds + CF::OFF_SB;
  char* part = lds + CF::OFF_PART;
  float* pd = reinterpret_cast<float*>(lds + CF::OFF_PD);

  const int64_t bh = blockIdx.x / a.nblk_per_bh;
  const int seg = blockIdx.x % a.nblk_per_bh;
  int64_t row0;
  int rstep, Tb;  // first row, row step, this sequence's rows
  seq_view<S2>(a, bh, row0, rstep, Tb);
  const uint32_t orsv = (uint32_t)rstep * DV;  // elements between consecutive output rows
  const int nchunks = (Tb + C - 1) / C;
  const int c0 = seg * a.cps;
  const int c1 = min(nchunks, c0 + a.cps);
  const int osz = a.o_f32 ? 4 : 2;
  char* obase = static_cast<char*>(a.o) + (S2 ? bh * (int64_t)(a.T / 2) : row0) * DV * osz;

  // ---- initial state (exclusive prefix of this segment, or zero)
  f32x4_t S[wave_na<P>(W)][NT];
  f32x4_t Mt = zero4();
#pragma unroll
  for (int i = 0; i < NTW; ++i)
#pragma unroll
    for (int dt = 0; dt < NT; ++dt) S[i][dt] = zero4();
  if (seg > 0) {
    const float* src = a.ws + (bh * (a.nseg - 1) + (seg - 1)) * CF::STATE_FLOATS;
#pragma unroll
    for (int i = 0; i < NTW; ++i)
#pragma unroll
      for (int dt = 0; dt < NT; ++dt)
        S[i][dt] = *reinterpret_cast<const f32x4_t*>(src + ((wave_tile<P>(W, i) * NT + dt) * 64 + lane) * 4);
    if constexpr (MT >= 0)
      Mt = *reinterpret_cast<const f32x4_t*>(src + (int64_t)CF::NTL * NT * 256 + (MT * 64 + lane) * 4);
  }
  auto write_m = [&]() {  // Gram tile -> LDS as bf16 hi / lo
    if constexpr (MT >= 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * MRT + 4 * lg + r, col = 16 * MCT + ln;
        const float m = 0.5f * Mt[r];  // the tile holds 2 M (built from sqrt(2) k_hat)
        const uint16_t h = f32_to_bf16_bits(m);
        mlds[row * CF::MP + col] = h;
        mlds[P * CF::MP + row * CF::MP + col] = f32_to_bf16_bits(m - bf16_bits_to_f32(h));
      }
    }
  };
  auto write_state = [&]() {  // tiles 2i, 2i+1 of this wave form readout pair wave_tile(2i) / 2
#pragma unroll
    for (int i = 0; i < NTW; i += 2) {
      const int pair = wave_tile<P>(W, i) >> 1;
#pragma unroll
      for (int dt = 0; dt < NT; ++dt) {
        u32x4_t u;
        u[0] = pk2(S[i][dt][0], S[i][dt][1]);
        u[1] = pk2(S[i][dt][2], S[i][dt][3]);
        if (i + 1 < NTW) {
          u[2] = pk2(S[i + 1 < NTW ? i + 1 : i][dt][0], S[i + 1 < NTW ? i + 1 : i][dt][1]);
          u[3] = pk2(S[i + 1 < NTW ? i + 1 : i][dt][2], S[i + 1 < NTW ? i + 1 : i][dt][3]);
        } else {
          u[2] = u[3] = 0;  // the odd last tile has no partner
        }
        *reinterpret_cast<u32x4_t*>(sb + ((pair * NT + dt) * 64 + lane) * 16) = u;
      }
    }
  };

  Stager<P, DV, C, true, S2> stg;
  stg.init(a, bh);
  stg.load(c0 * C);
  stg.stage_rows(lds);
  stg.template stage_kt<true>(lds, CF::OFF_KT);
  stg.write_vt(lds + CF::OFF_VT);
  write_state();
  write_m();
  __syncthreads();

  // Per chunk c, two phases: (1) readout of chunk c from the state before it (LDS) and the
  // build of chunk c into the registers; (2) output, staging of chunk c + 1, and the state
  // after chunk c into LDS. Both readout and build read only the state before chunk c.
  for (int c = c0; c < c1; ++c) {
    const int t0 = c * C;
    if (c + 1 < c1) stg.load(t0 + C);  // rows of the next chunk, staged in phase 2
    // ================= phase 1: readout =================
    const int qrow = 16 * TT + ln;
    f32x4_t O[NT];
#pragma unroll
    for (int dt = 0; dt < NT; ++dt) O[dt] = zero4();
    float dpart = 0.f;
    if constexpr (OWNER) {
      // query operand (B of S^T and of X^T): the raw query row is exact in bf16.
      // Component k-slots of lane group lg: 4lg..4lg+3 and 16+4lg..16+4lg+3 (16-byte steps)
      bf16x8_t qbh;
      {
        const float* src = qh + qrow * CF::QP + 4 * lg;
        const f32x4_t x0 = *reinterpret_cast<const f32x4_t*>(src);
        const f32x4_t x1 = P == 32 ? *reinterpret_cast<const f32x4_t*>(src + 16) : zero4();
        const float xs[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
        qbh = pack8(xs);
      }
      // denominator, inter-chunk part: X^T = M Q^T (rows: components; M as bf16 hi + lo),
      // then q . X
#pragma unroll
      for (int rt = 0; rt < NH; ++rt) {
        const uint16_t* mrow = mlds + (16 * rt + ln) * CF::MP + 4 * lg;
        const u32x2_t h0 = *reinterpret_cast<const u32x2_t*>(mrow);
        const u32x2_t l0 = *reinterpret_cast<const u32x2_t*>(mrow + P * CF::MP);
        const u32x2_t h1 = P == 32 ? *reinterpret_cast<const u32x2_t*>(mrow + 16) : u32x2_t{0, 0};
        const u32x2_t l1 = P == 32 ? *reinterpret_cast<const u32x2_t*>(mrow + P * CF::MP + 16) : u32x2_t{0, 0};
        const bf16x8_t mh = __builtin_bit_cast(bf16x8_t, u32x4_t{h0[0], h0[1], h1[0], h1[1]});
        const bf16x8_t ml = __builtin_bit_cast(bf16x8_t, u32x4_t{l0[0], l0[1], l1[0], l1[1]});
        f32x4_t X = zero4();
        X = mfma(mh, qbh, X);
        X = mfma(ml, qbh, X);
        const f32x4_t qv = *reinterpret_cast<const f32x4_t*>(qh + qrow * CF::QP + 16 * rt + 4 * lg);
        dpart += X[0] * qv[0] + X[1] * qv[1] + X[2] * qv[2] + X[3] * qv[3];
      }
      // intra block: S^T = K_hat Q^T over key tiles kt <= TT; W = (S^T)^2; O += W V.
      // Global chunk 0 (denominators of few weights) uses split-bf16 scores; the two
      // variants are separate code so the common one carries no split work.
      auto intra = [&]<bool SPLIT>() {
#pragma unroll
      for (int kp = 0; kp <= TT / 2; ++kp) {
        float wv[8];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int kt = 2 * kp + half;
          f32x4_t St = zero4();
          if (kt <= TT) {
            bf16x8_t kbh, kbl;
            const float* src = kh + (16 * kt + ln) * CF::QP + 4 * lg;
            const f32x4_t x0 = *reinterpret_cast<const f32x4_t*>(src);
            const f32x4_t x1 = P == 32 ? *reinterpret_cast<const f32x4_t*>(src + 16) : zero4();
            float xs[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
            if constexpr (SPLIT) {
              split8(xs, kbh, kbl);
              St = mfma(kbh, qbh, St);
              St = mfma(kbl, qbh, St);
            } else {
              St = mfma(pack8(xs), qbh, St);
            }
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float w = St[r] * St[r];
            // causal: key <= query on the diagonal tile (token indices under S2)
            if (kt == TT && (S2 ? ((4 * lg + r) >> 1) > (ln >> 1) : 4 * lg + r > ln)) w = 0.f;
            wv[4 * half + r] = w;
            dpart += w;
          }
        }
        const bf16x8_t wa = pack8(wv);
#pragma unroll
        for (int dt = 0; dt < NT; ++dt) {
          // keys 32kp + 4lg + j and 32kp + 16 + 4lg + j, stored adjacent (permuted V^T)
          const bf16x8_t vbf = *reinterpret_cast<const bf16x8_t*>(vt + vt_row(16 * dt + ln) * CF::VTP + 32 * kp + 8 * lg);
          O[dt] = mfma(vbf, wa, O[dt]);  // O^T += V^T W^T
        }
      }
      };
      if (c == 0)
        intra.template operator()<true>();
      else
        intra.template operator()<false>();
      dpart = xor32_sum(xor16_sum(dpart));  // denominator of query qrow, in every lane group
    }
    // readout psi(Q) S over pairs [PB, PE): Y[x] = q_hat[qrow][(x & ~15) | ((x + 4 lg) & 15)]
    {
      float Y[P];
      const float* src = qh + qrow * CF::QP;
#pragma unroll
      for (int h = 0; h < NH; ++h)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const f32x4_t x = *reinterpret_cast<const f32x4_t*>(src + 16 * h + ((4 * u + 4 * lg) & 15));
#pragma unroll
          for (int e = 0; e < 4; ++e) Y[16 * h + 4 * u + e] = x[e];
        }
      // state fragments of the next pair are read while this pair's features are built
      bf16x8_t fr[2][NT];
      auto load_pair = [&](int pair, bf16x8_t(&dst)[NT]) {
#pragma unroll
        for (int dt = 0; dt < NT; ++dt)
          dst[dt] = *reinterpret_cast<const bf16x8_t*>(sb + ((pair * NT + dt) * 64 + lane) * 16);
      };
      if constexpr (PE > PB) load_pair(PB, fr[0]);
      [&]<int... PI>(std::integer_sequence<int, PI...>) {
        (([&] {
           constexpr int t1 = 2 * (PB + PI), t2 = t1 + 1;
           constexpr bool has2 = t2 < CF::NTL;
           if constexpr (PB + PI + 1 < PE) load_pair(PB + PI + 1, fr[(PI + 1) & 1]);
           // keep the next pair's reads ahead of this pair's work: under register pressure the
           // scheduler otherwise sinks each read to its MFMA and waits out the LDS latency
           __builtin_amdgcn_sched_barrier(0);
           const bf16x8_t af = readout_frag<P, t1, has2 ? t2 : t1, has2>(Y, glow);
#pragma unroll
           for (int dt = 0; dt < NT; ++dt) O[dt] = mfma(fr[PI & 1][dt], af, O[dt]);  // O^T += S^T psi(Q)^T
         }()),
         ...);
      }(std::make_integer_sequence<int, PE - PB>{});
    }
    // ================= phase 1: build =================
    build_chunk<P, DV, C, Map8, W>(S, Mt, Mt, khT, vt);  // no odd-tile slice in the forward
    // O holds O^T: lane (ln, lg) has columns 16 dt + 4 lg + r of query 16 TT + ln
    if constexpr (CF::FS > 1) {
#pragma unroll
      for (int dt = 0; dt < NT; ++dt)
        if (CF::out_owner(dt) != FSI)
          *reinterpret_cast<f32x4_t*>(part + (CF::part_slot(TT, dt, FSI) * 64 + lane) * 16) = O[dt];
      if constexpr (OWNER) pd[TT * 64 + lane] = dpart;
    }
    __syncthreads();
    // ================= phase 2 =================
    if constexpr (CF::owns_any(FSI)) {  // add the other splits' sums, normalise, store
      float den = dpart;
      if constexpr (!OWNER) den = pd[TT * 64 + lane];
      if constexpr (S2) den += dpp_f<0xB1>(den);  // the token's other virtual query row (lane ^ 1)
      const float inv = den > 0.f ? __builtin_amdgcn_rcpf(den) : 0.f;
      const int orow0 = S2 ? t0 / 2 : t0, orows = S2 ? (Tb - t0) / 2 : Tb - t0;
      const __amdgpu_buffer_rsrc_t ro =
          buf_rsrc(obase + (int64_t)orow0 * orsv * osz, ((uint32_t)(orows - 1) * orsv + DV) * osz);
      // rows past the length are dropped; under S2 the even lane of a token stores it
      const uint32_t ob = (uint32_t)(S2 ? (16 * TT + ln) >> 1 : 16 * TT + ln) * orsv + 4 * lg;
      const bool store = !S2 || (ln & 1) == 0;
#pragma unroll
      for (int dt = 0; dt < NT; ++dt) {
        if (CF::out_owner(dt) != FSI) continue;
        f32x4_t o = O[dt];
#pragma unroll
        for (int f = 0; f < CF::FS; ++f)
          if (f != FSI) o += *reinterpret_cast<const f32x4_t*>(part + (CF::part_slot(TT, dt, f) * 64 + lane) * 16);
        if constexpr (S2) {
#pragma unroll
          for (int r = 0; r < 4; ++r) o[r] += dpp_f<0xB1>(o[r]);
        }
        o *= inv;
        if (store) {
          if (a.o_f32)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, o), ro, (ob + 16 * dt) * 4, 0, 0);
          else
            __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{pk2(o[0], o[1]), pk2(o[2], o[3])}, ro, (ob + 16 * dt) * 2, 0, 0);
        }
      }
    }
    if (c + 1 < c1) {
      stg.stage_rows(lds);
      stg.template stage_kt<true>(lds, CF::OFF_KT);
      stg.write_vt(lds + CF::OFF_VT);
    }
    write_state();  // last: waits for the build's MFMAs
    write_m();
    __syncthreads();
  }
  // the last segment of a sequence ends with the state after its last token
  if (a.s_out != nullptr && seg == a.nblk_per_bh - 1) write_final_state<P, DV, W>(a, bh, S, Mt);
}

// ---- pass 1: summary [S | M] of one segment after its chunks, to workspace slot seg
template <int P, int DV, int C, int W, bool S2 = false>
__device__ __forceinline__ void run_sum16(const Args& a, char* lds) {
  using CF = Cfg<P, DV, C>;
  constexpr int NT = CF::NT, NTW = Map16::nt<P>(W), MT = Map16::mtile<P>(W);
  constexpr int XDT = Map16::xdt<P>(W, NT);
  constexpr int OKT = 0, OVB = P * CF::KTP * 4;
  const int lane = threadIdx.x & 63;
  const int64_t bh = blockIdx.x / a.nblk_per_bh;
  const int seg = blockIdx.x % a.nblk_per_bh;
  int64_t row0;
  int rstep, Tb;  // this sequence's rows
  seq_view<S2>(a, bh, row0, rstep, Tb);
  const int nchunks = (Tb + C - 1) / C;
  const int c0 = seg * a.cps;
  const int c1 = min(nchunks, c0 + a.cps);

  f32x4_t S[(map_na<Map16, P>(W))][NT];
  f32x4_t Sx = zero4(), Mt = zero4();
#pragma unroll
  for (int i = 0; i < NTW; ++i)
#pragma unroll
    for (int dt = 0; dt < NT; ++dt) S[i][dt] = zero4();

  Stager<P, DV, C, false, S2> stg;
  stg.init(a, bh);
  stg.load(c0 * C);
  stg.template stage_kt<false>(lds, OKT);
  stg.write_vt(lds + OVB);
  if (c0 + 1 < c1) stg.load((c0 + 1) * C);
  __syncthreads();
  for (int c = c0; c < c1; ++c) {  // k_hat^T / V^T double-buffered: one barrier per chunk
    const int buf = (c - c0) & 1;
    char* base = lds + buf * CF::SUM_BUF;
    build_chunk<P, DV, C, Map16, W>(S, Sx, Mt, reinterpret_cast<const float*>(base + OKT),
                                    reinterpret_cast<const uint16_t*>(base + OVB));
    if (c + 1 < c1) {
      stg.template stage_kt<false>(lds + (buf ^ 1) * CF::SUM_BUF, OKT);
      stg.write_vt(lds + (buf ^ 1) * CF::SUM_BUF + OVB);
      if (c + 2 < c1) stg.load((c + 2) * C);
    }
    __syncthreads();
  }
  float* dst = a.ws + (bh * (a.nseg - 1) + seg) * CF::STATE_FLOATS;
#pragma unroll
  for (int i = 0; i < NTW; ++i)
#pragma unroll
    for (int dt = 0; dt < NT; ++dt)
      *reinterpret_cast<f32x4_t*>(dst + ((Map16::tile<P>(W, i) * NT + dt) * 64 + lane) * 4) = S[i][dt];
  if constexpr (XDT >= 0)
    *reinterpret_cast<f32x4_t*>(dst + (((ntiles<P>() - 1) * NT + XDT) * 64 + lane) * 4) = Sx;
  if constexpr (MT >= 0)
    *reinterpret_cast<f32x4_t*>(dst + (int64_t)CF::NTL * NT * 256 + (MT * 64 + lane) * 4) = Mt;
}

// forward of the segments (8 waves)
template <int P, int DV, int C, bool S2 = false>
__global__ __launch_bounds__(512, 1) void chunked_bf16_kernel(Args a) {
  extern __shared__ __align__(16) char lds[];
  switch (threadIdx.x >> 6) {
    case 0: run_fwd<P, DV, C, 0, S2>(a, lds); break;
    case 1: run_fwd<P, DV, C, 1, S2>(a, lds); break;
    case 2: run_fwd<P, DV, C, 2, S2>(a, lds); break;
    case 3: run_fwd<P, DV, C, 3, S2>(a, lds); break;
    case 4: run_fwd<P, DV, C, 4, S2>(a, lds); break;
    case 5: run_fwd<P, DV, C, 5, S2>(a, lds); break;
    case 6: run_fwd<P, DV, C, 6, S2>(a, lds); break;
    default: run_fwd<P, DV, C, 7, S2>(a, lds); break;
  }
}

// segment summaries (16 waves)
template <int P, int DV, int C, bool S2 = false>
__global__ __launch_bounds__(1024, 1) void summary_bf16_kernel(Args a) {
  extern __shared__ __align__(16) char lds[];
  switch (threadIdx.x >> 6) {
    case 0: run_sum16<P, DV, C, 0, S2>(a, lds); break;
    case 1: run_sum16<P, DV, C, 1, S2>(a, lds); break;
    case 2: run_sum16<P, DV, C, 2, S2>(a, lds); break;
    case 3: run_sum16<P, DV, C, 3, S2>(a, lds); break;
    case 4: run_sum16<P, DV, C, 4, S2>(a, lds); break;
    case 5: run_sum16<P, DV, C, 5, S2>(a, lds); break;
    case 6: run_sum16<P, DV, C, 6, S2>(a, lds); break;
    case 7: run_sum16<P, DV, C, 7, S2>(a, lds); break;
    case 8: run_sum16<P, DV, C, 8, S2>(a, lds); break;
    case 9: run_sum16<P, DV, C, 9, S2>(a, lds); break;
    case 10: run_sum16<P, DV, C, 10, S2>(a, lds); break;
    case 11: run_sum16<P, DV, C, 11, S2>(a, lds); break;
    case 12: run_sum16<P, DV, C, 12, S2>(a, lds); break;
    case 13: run_sum16<P, DV, C, 13, S2>(a, lds); break;
    case 14: run_sum16<P, DV, C, 14, S2>(a, lds); break;
    default: run_sum16<P, DV, C, 15, S2>(a, lds); break;
  }
}

// pass 1 on nblk workgroups (a.nblk_per_bh set by the caller). A template of its own so a
// translation unit can instantiate it with other code-generation options than the forward.
template <int P, int DV, int C, bool S2 = false>
hipError_t launch_summary(const Args& a, unsigned nblk, hipStream_t st) {
  using CF = Cfg<P, DV, C>;
  auto ks = summary_bf16_kernel<P, DV, C, S2>;
  hipError_t e = hipFuncSetAttribute((const void*)ks, hipFuncAttributeMaxDynamicSharedMemorySize, CF::SUM_LDS);
  if (e != hipSuccess) return e;
  ks<<<dim3(nblk), dim3(1024), CF::SUM_LDS, st>>>(a);
  return hipGetLastError();
}

// T: rows of q / k (virtual rows, 2x the tokens, under S2)
template <int P, int DV, int C, bool S2 = false>
hipError_t launch_pdc(const uint16_t* q, const uint16_t* k, const uint16_t* v, void* o, bool o_bf16,
                      int B, int H, int T, const SegPlan& plan, float* ws, float* s_out, float* z_out,
                      SeqLayout lay, int passes, hipStream_t st) {
  using CF = Cfg<P, DV, C>;
  const int BH = B * H;
  Args a{q, k, v, o, ws, T, plan.nseg, plan.cps, 0, o_bf16 ? 0 : 1, s_out, z_out, lay, H};
  hipError_t e;
  if (plan.nseg > 1 && (passes & PASS_SUMMARIES)) {
    a.nblk_per_bh = plan.nseg - 1;
    if ((e = launch_summary<P, DV, C, S2>(a, (unsigned)(BH * (plan.nseg - 1)), st)) != hipSuccess) return e;
  }
  if (plan.nseg > 1 && (passes & PASS_SCAN))
    if ((e = launch_scan(ws, BH, plan.nseg - 1, CF::STATE_FLOATS, st)) != hipSuccess) return e;
  if (!(passes & PASS_SEGMENTS)) return hipSuccess;
  auto kf = chunked_bf16_kernel<P, DV, C, S2>;
  if ((e = hipFuncSetAttribute((const void*)kf, hipFuncAttributeMaxDynamicSharedMemorySize, CF::LDS)) != hipSuccess) return e;
  a.nblk_per_bh = plan.nseg;
  kf<<<dim3((unsigned)(BH * plan.nseg)), dim3(512), CF::LDS, st>>>(a);
  return hipGetLastError();
}

}  // namespace chk

}  // namespace kata
