// Exact O(T) chunked-state KATA forward with fp16 MFMA operands (gfx950), p = 32.
//
// Source: "Kernelized Linear Attention: Breaking the Capacity Wall with Symmetric Cones"
// (arXiv 2607.17419), arXiv HTML page:
//   * chunked-forward paragraph: per-chunk state psi(K_c)^T [V_c | 1], the inter-chunk
//     prefix as an associative cumulative sum, the local C x C causal block;
//   * rank-one lift display after Eq. (8): psi(u) = u u^T on the unit sphere,
//     <psi(a), psi(b)> = (a.b)^2;  Eq. (8): n = p(p+1)/2 packed coordinates;
//   * normalized-readout paragraph: o_t = psi(q_t)^T S_t / psi(q_t)^T Z_t.
//
// Why fp16 operands. The lift is the kernel's VALU cost: every lifted coordinate feeds only
// 2 dv MFMA flops. With fp16 operands one v_pk_mul_f16 produces two coordinates already in
// MFMA operand format (0.5 instruction per coordinate, against 1.5 for an fp32 product
// rounded to bf16). Unit-norm components and their products lie in [-1, 1], where fp16 is
// 8x finer than bf16. The ranges that fp16 cannot hold are handled by exact power-of-two
// scales:
//   * queries are staged as lambda q_hat with lambda = 2^7, so lifted queries and the
//     intra-chunk weights are 2^14 (q_hat . k_hat)^2: tiny weights stay normal numbers. The
//     factor cancels between numerator and denominator.
//   * values are staged as sigma v, sigma = 2^e a per-workgroup scale chosen from a running
//     bound beta >= max |S| (the prefix's max plus C max|v| per chunk), so that sigma S and
//     sigma v stay below 2^13. sigma only ever decreases; the register state is rescaled by
//     the exact power of two when it does. The output divides by sigma once.
//   * the Gram matrix M = sum k_hat k_hat^T of the denominator (entries up to the token
//     count) is applied as fp16 hi + lo of M 2^-ceil(log2 tokens).
// The first chunk of a sequence, where a denominator is a sum of few weights, computes its
// scores from hi + lo splits of both q_hat and k_hat.
//
// Feature tiles. The 528 packed features are carried as 576 slots in 18 tiles of 32 rows.
// Row m = 4a + c of a tile holds own component 4a + c times partner component
// 4B + (c XOR r) (blocks of 4 components; a = the row's quad). Tiles 0-3 pair a block with
// itself (XOR r = tile): tile 0 is the diagonal, tiles 1-3 hold each within-block pair
// twice. Tiles 4-15 pair block a with a + d (d = 1..3, XOR r), tiles 16-17 block a with
// a + 4. Every unordered pair of different blocks appears exactly once per XOR, so each
// off-diagonal coordinate appears once, with c^2 = 2 folded into the build (partner copies
// are staged at 2 k_hat), and the within-block pairs twice at weight 1 (tiles 1-3 are built
// at 2x and halved when the state is handed to the readout).
//   * Build (ψ(K)^T V on 32x32x16 MFMA): lane = (row, 8 tokens). The staged key rows come
//     in five copies (own; partner x2 with XOR 0..3 inside each 4-component block), so that
//     ds_read_b64_tr_b16 transposed reads give every lane its own and its partner component
//     for 4 tokens at a time: 4 consecutive lanes read 4 consecutive components, which is
//     exactly a quad's (4a + c, 4B + (c XOR r)).
//   * Readout (O^T = S^T psi(Q)^T): lane = (token, lane half). A lane holds its token's 32
//     components as 16 packed fp16 pairs, rotated by one block in the upper lane half, so
//     one instruction stream serves quads 4s, 4s+2 (lower half) and 4s+1, 4s+3 (upper);
//     each pair of slots is one v_pk_mul_f16 with op_sel choosing the partner's halves.
//   * The readout's state fragment of k-step s is the build accumulator's registers
//     8s..8s+7 of the same lane: the build lane converts and writes 16 bytes, the readout
//     lane reads them back.
//   * Denominator psi(q)^T Z = q^T M q (Gram matrix, fp32-accurate as hi + lo); the
//     intra-chunk block computes (q_hat . k_hat)^2 from the components (weight identity of
//     the lift display) and sums the same fp16 weights that multiply V.
//
// Waves: 0-3 read out (token group of 32, or a share of the tiles of one), 4-7 build
// (tiles 0-4, 5-9, 10-13 with the Gram tile, 14-17); wave w and w + 4 share a SIMD. Per
// chunk: phase 1 = readout of chunk c from the state before it and build of chunk c |
// barrier | phase 2 = output, staging of chunk c + 1, state after chunk c to LDS | barrier.
// ASSOCIATIVE runs a summary pass (build only, 8 waves), the segment scan and the segments;
// SEQUENTIAL runs one segment per sequence.
#pragma once
#include <utility>

#include "kata_device.h"
#include "kata_launch.h"

namespace kata {

hipError_t launch_scan(float* ws, int BH, int nslots, int64_t E, hipStream_t st);

namespace c16 {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h4_t __attribute__((ext_vector_type(4)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float acc_t __attribute__((ext_vector_type(16)));
typedef short s4_t __attribute__((ext_vector_type(4)));
typedef float f32x2v_t __attribute__((ext_vector_type(2)));

constexpr int P = 32;     // projected width
constexpr int NTL = 18;   // 32-slot feature tiles
constexpr float LAMBDA = 128.f;  // query staging scale (2^7)

// ---- feature tiles (see the header comment)
constexpr int tile_partner(int t, int a) {
  return t < 4 ? a : (t < 16 ? (a + 1 + (t - 4) / 4) & 7 : (a + 4) & 7);
}
constexpr int tile_xor(int t, int a) {
  return t < 4 ? t : (t < 16 ? (t - 4) % 4 : (t - 16) + (a < 4 ? 0 : 2));
}
// key copy read for the partner: 0 = own (unscaled), 1 + r = doubled with XOR r
constexpr int tile_copy(int t, int a) { return t == 0 ? 0 : 1 + tile_xor(t, a); }
// tiles whose slots are built at twice their weight (halved for the readout)
constexpr bool tile_doubled(int t) { return t >= 1 && t < 4; }

// Every packed coordinate (i <= j) is covered with total weight c_ij^2 (1 on the
// diagonal, 2 off it): checked at compile time.
constexpr bool tiles_cover_exactly() {
  int w[P][P] = {};
  for (int t = 0; t < NTL; ++t)
    for (int m = 0; m < 32; ++m) {
      const int a = m / 4, c = m % 4;
      const int i = 4 * a + c, j = 4 * tile_partner(t, a) + (c ^ tile_xor(t, a));
      const int wt = t == 0 ? 1 : (tile_doubled(t) ? 1 : 2);  // doubled tiles are halved
      const int lo = i < j ? i : j, hi = i < j ? j : i;
      w[lo][hi] += wt;
    }
  for (int i = 0; i < P; ++i)
    for (int j = i; j < P; ++j)
      if (w[i][j] != (i == j ? 1 : 2)) return false;
  return true;
}
static_assert(tiles_cover_exactly(), "feature tiles must cover each packed coordinate once");

__device__ __forceinline__ acc_t mfma(h8_t a, h8_t b, acc_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ acc_t zero_acc() {
  acc_t z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// fp16 vectors are assembled and split with shuffles only: this compiler mis-lowers a
// bit cast of an element extracted from a 32-bit vector into a packed-half vector
__device__ __forceinline__ h4_t cat2(h2_t a, h2_t b) { return __builtin_shufflevector(a, b, 0, 1, 2, 3); }
__device__ __forceinline__ h8_t cat44(h4_t a, h4_t b) { return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7); }
__device__ __forceinline__ h8_t cat4(h2_t a, h2_t b, h2_t c, h2_t d) { return cat44(cat2(a, b), cat2(c, d)); }
__device__ __forceinline__ h2_t lo2(h4_t x) { return __builtin_shufflevector(x, x, 0, 1); }
__device__ __forceinline__ h2_t hi2(h4_t x) { return __builtin_shufflevector(x, x, 2, 3); }
__device__ __forceinline__ h2_t swp(h2_t x) { return __builtin_shufflevector(x, x, 1, 0); }
__device__ __forceinline__ h2_t cvt2(float a, float b) { return __builtin_convertvector(f32x2v_t{a, b}, h2_t); }
__device__ __forceinline__ h4_t ld4(const char* p) { return *reinterpret_cast<const h4_t*>(p); }
__device__ __forceinline__ h8_t ld8(const char* p) { return *reinterpret_cast<const h8_t*>(p); }
__device__ __forceinline__ void st4(char* p, h4_t x) { *reinterpret_cast<h4_t*>(p) = x; }
__device__ __forceinline__ void st8(char* p, h8_t x) { *reinterpret_cast<h8_t*>(p) = x; }

// transposed LDS read: lane i of each 16-lane group gets element i % 4 of the 8-byte
// chunks addressed by lanes i / 4 + 4 j, j = 0..3 (ds_read_b64_tr_b16)
__device__ __forceinline__ h4_t tr16(const char* lds, uint32_t off) {
  const s4_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4_t*)(lds + off));
  return __builtin_bit_cast(h4_t, r);
}
__device__ __forceinline__ h8_t tr16x2(const char* lds, uint32_t off0, uint32_t off1) {
  return cat44(tr16(lds, off0), tr16(lds, off1));
}

// ---- LDS layout and work split
template <int DV, int C>
struct Lay {
  static constexpr int NDT = DV / 32;          // 32-column value tiles
  static constexpr int NG = C / 32;            // 32-token groups per chunk
  static constexpr int FS = 4 / NG;            // readout waves per token group
  static constexpr int NSTEP = C / 16;         // 16-token build steps
  static constexpr int QPB = 72;               // q_hat row pitch, bytes (8-byte block reads conflict-free)
  static constexpr int KPB = 64;               // key row pitch per copy, bytes
  static constexpr int VPB = 2 * DV + 16;      // value row pitch, bytes
  static constexpr int MPB = 80;               // Gram row pitch, bytes
  static constexpr int ST = NTL * 2 * NDT * 1024;  // state fragments (fp16)
  static constexpr int OFF_Q = ST;
  static constexpr int OFF_K = OFF_Q + C * QPB;
  static constexpr int KCOPY = C * KPB;
  static constexpr int OFF_V = OFF_K + 5 * KCOPY;
  static constexpr int OFF_M = OFF_V + C * VPB;  // hi, lo
  static constexpr int OFF_PART = OFF_M + 2 * 32 * MPB;
  static constexpr int PART = FS > 1 ? NG * (FS - 1) * NDT * 64 * 64 : 0;
  static constexpr int OFF_RED = OFF_PART + PART;  // 8 reduction slots (uint32)
  static constexpr int LDS = OFF_RED + 64;
  // first-chunk split operands alias the state area (there is no readout at chunk 0)
  static constexpr int OFF_QLO = 0;
  static constexpr int OFF_KLO = C * QPB;
  static_assert(OFF_KLO + C * KPB <= ST, "split operands fit the state area");
  static_assert(LDS <= 160 * 1024, "LDS budget");
  // summary pass: key copies and values, double-buffered
  static constexpr int SUM_BUF = 5 * KCOPY + C * VPB;
  static constexpr int SUM_RED = 2 * SUM_BUF;
  static constexpr int SUM_LDS = SUM_RED + 64;
  static_assert(SUM_LDS <= 160 * 1024, "LDS budget (summaries)");
  // workspace summary: state tiles in accumulator layout, then the Gram tile
  static constexpr int64_t STATE_FLOATS = (int64_t)NTL * NDT * 1024 + 1024;
  // readout tile range of split f (the last split also runs the intra block and the
  // denominator, so it takes fewer tiles)
  static constexpr int rb(int f) {
    return FS == 1 ? (f == 0 ? 0 : NTL) : (FS == 2 ? (f == 0 ? 0 : (f == 1 ? 10 : NTL)) : (f <= 2 ? 5 * f : (f == 3 ? 14 : NTL)));
  }
};

// build tiles of wave j: forward (4 build waves) and summary pass (8 build waves)
struct Fwd4 {
  static constexpr int NW = 4;
  static constexpr int tb(int j) { return j == 0 ? 0 : (j == 1 ? 5 : (j == 2 ? 10 : (j == 3 ? 14 : 18))); }
  static constexpr bool gram(int j) { return j == 2; }
};
struct Sum8 {
  static constexpr int NW = 8;
  static constexpr int tb(int j) { return j == 0 ? 0 : (j == 8 ? 18 : (j < 8 ? 1 + 2 * j : 18)); }
  static constexpr bool gram(int j) { return j == 2; }
};

struct Args {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  void* o;
  float* ws;
  int T, nseg, cps, nblk_per_bh;
  int o_f32;
  float* s_out;
  float* z_out;
  SeqLayout lay;
  int H;
};

// ---- value scale sigma = 2^e from the running bound beta (see the header comment)
__device__ __forceinline__ int scale_exp(float beta, int e_cur) {
  if (!(beta > 0.f)) return e_cur;
  int e = 13 - __builtin_amdgcn_frexp_expf(beta);
  e = e < -100 ? -100 : (e > 100 ? 100 : e);
  return e < e_cur ? e : e_cur;
}
__device__ __forceinline__ float pow2f(int e) { return __builtin_amdgcn_ldexpf(1.f, e); }
// exponent of the Gram scale 2^-g with M 2^-g <= 1 for `tokens` tokens
__device__ __forceinline__ int gram_exp(int tokens) { return tokens <= 1 ? 0 : 32 - __builtin_clz((unsigned)tokens - 1u); }

// max over a wave of nonnegative floats (as ordered bit patterns)
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t y = (uint32_t)__shfl_xor((int)x, d);
    x = x > y ? x : y;
  }
  return x;
}

// ---- staging of a chunk (global bf16 -> registers -> scaled fp16 LDS layouts)
template <int DV, int C, int NTHR>
struct KVStage {  // keys (five copies) and values, staged by NTHR threads (tid 0..NTHR-1)
  using L = Lay<DV, C>;
  static constexpr int KP = (4 * C + NTHR - 1) / NTHR;       // key pieces (8 components) per thread
  static constexpr int VP = (C * DV / 8 + NTHR - 1) / NTHR;  // value pieces (8 columns) per thread
  u32x4_t kr[KP];
  u32x4_t vr[VP];
  const uint16_t *kb, *vb;
  int len;
  uint32_t rsp, rsv;
  __device__ __forceinline__ void init(const uint16_t* k, const uint16_t* v, int64_t row0, int step, int n) {
    kb = k + row0 * P;
    vb = v + row0 * DV;
    len = n;
    rsp = (uint32_t)step * P;
    rsv = (uint32_t)step * DV;
  }
  __device__ __forceinline__ void load(int t0, int tid) {
    const uint32_t left = (uint32_t)(t0 < len ? len - t0 : 0);
    const uint32_t kbytes = left ? ((left - 1) * rsp + P) * 2 : 0;
    const uint32_t vbytes = left ? ((left - 1) * rsv + DV) * 2 : 0;
    const __amdgpu_buffer_rsrc_t rk = buf_rsrc(kb + (int64_t)t0 * rsp, kbytes);
    const __amdgpu_buffer_rsrc_t rv = buf_rsrc(vb + (int64_t)t0 * rsv, vbytes);
#pragma unroll
    for (int i = 0; i < KP; ++i) {
      const int pc = tid + NTHR * i;
      if (pc < 4 * C)
        kr[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rk, ((pc >> 2) * rsp + 8 * (pc & 3)) * 2, 0, 0));
    }
#pragma unroll
    for (int i = 0; i < VP; ++i) {
      const int pc = tid + NTHR * i;
      constexpr int VPR = DV / 8;
      if (pc < C * VPR)
        vr[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rv, ((pc / VPR) * rsv + 8 * (pc % VPR)) * 2, 0, 0));
    }
  }
  // max |v| of the loaded values as bf16 magnitude bits (ordered like the values)
  __device__ __forceinline__ uint32_t vmax_bits(int tid) const {
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < VP; ++i) {
      const int pc = tid + NTHR * i;
      if (pc < C * (DV / 8)) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t x = vr[i][e] & 0x7fff7fffu;
          const uint32_t lo = x & 0xffffu, hi = x >> 16;
          m = m > lo ? m : lo;
          m = m > hi ? m : hi;
        }
      }
    }
    return m;
  }
  // LDS writes: own copy (unscaled k_hat), four doubled XOR copies, sigma v; the optional
  // lo part of the own copy (first chunk of a sequence)
  template <bool LO>
  __device__ __forceinline__ void store(char* lds, int off_k, int off_v, float sig, int tid, int off_klo) const {
#pragma unroll
    for (int i = 0; i < KP; ++i) {
      const int pc = tid + NTHR * i;
      if (pc >= 4 * C) continue;
      const int row = pc >> 2, e4 = pc & 3;
      float x[8];
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[2 * e] = __uint_as_float(kr[i][e] << 16);
        x[2 * e + 1] = __uint_as_float(kr[i][e] & 0xffff0000u);
        ss += x[2 * e] * x[2 * e] + x[2 * e + 1] * x[2 * e + 1];
      }
      ss = group_sum<4>(ss);
      const float inv = inv_norm_fast(ss);
      h2_t own[4], dbl[4], sw[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        own[e] = cvt2(x[2 * e] * inv, x[2 * e + 1] * inv);
        dbl[e] = own[e] * h2_t{(_Float16)2.f, (_Float16)2.f};
        sw[e] = swp(dbl[e]);
      }
      char* base = lds + off_k + row * L::KPB + 16 * e4;
      st8(base, cat4(own[0], own[1], own[2], own[3]));
      // XOR r inside each 4-component block (two registers): r=1 swaps halves, r=2 swaps
      // registers, r=3 both
      st8(base + 1 * L::KCOPY, cat4(dbl[0], dbl[1], dbl[2], dbl[3]));
      st8(base + 2 * L::KCOPY, cat4(sw[0], sw[1], sw[2], sw[3]));
      st8(base + 3 * L::KCOPY, cat4(dbl[1], dbl[0], dbl[3], dbl[2]));
      st8(base + 4 * L::KCOPY, cat4(sw[1], sw[0], sw[3], sw[2]));
      if constexpr (LO) {
        h2_t lo[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          lo[e] = cvt2(x[2 * e] * inv - (float)own[e][0], x[2 * e + 1] * inv - (float)own[e][1]);
        st8(lds + off_klo + row * L::KPB + 16 * e4, cat4(lo[0], lo[1], lo[2], lo[3]));
      }
    }
#pragma unroll
    for (int i = 0; i < VP; ++i) {
      const int pc = tid + NTHR * i;
      constexpr int VPR = DV / 8;
      if (pc >= C * VPR) continue;
      h2_t y[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        y[e] = cvt2(__uint_as_float(vr[i][e] << 16) * sig, __uint_as_float(vr[i][e] & 0xffff0000u) * sig);
      st8(lds + off_v + (pc / VPR) * L::VPB + 16 * (pc % VPR), cat4(y[0], y[1], y[2], y[3]));
    }
  }
};

// queries of one token group: NTHR threads stage rows [r0, r0 + 32) as lambda q_hat
template <int DV, int C, int NTHR>
struct QStage {
  using L = Lay<DV, C>;
  static constexpr int QP = (128 + NTHR - 1) / NTHR;
  u32x4_t qr[QP];
  const uint16_t* qb;
  int len;
  uint32_t rsp;
  __device__ __forceinline__ void init(const uint16_t* q, int64_t row0, int step, int n) {
    qb = q + row0 * P;
    len = n;
    rsp = (uint32_t)step * P;
  }
  __device__ __forceinline__ void load(int t0, int r0, int tid) {
    const int first = t0 + r0;
    const uint32_t left = (uint32_t)(first < len ? len - first : 0);
    const uint32_t bytes = left ? ((left - 1) * rsp + P) * 2 : 0;
    const __amdgpu_buffer_rsrc_t rq = buf_rsrc(qb + (int64_t)first * rsp, bytes);
#pragma unroll
    for (int i = 0; i < QP; ++i) {
      const int pc = tid + NTHR * i;
      if (pc < 128)
        qr[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rq, ((pc >> 2) * rsp + 8 * (pc & 3)) * 2, 0, 0));
    }
  }
  template <bool LO>
  __device__ __forceinline__ void store(char* lds, int r0, int tid) const {
#pragma unroll
    for (int i = 0; i < QP; ++i) {
      const int pc = tid + NTHR * i;
      if (pc >= 128) continue;
      const int row = r0 + (pc >> 2), e4 = pc & 3;
      float x[8];
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[2 * e] = __uint_as_float(qr[i][e] << 16);
        x[2 * e + 1] = __uint_as_float(qr[i][e] & 0xffff0000u);
        ss += x[2 * e] * x[2 * e] + x[2 * e + 1] * x[2 * e + 1];
      }
      ss = group_sum<4>(ss);
      const float inv = inv_norm_fast(ss) * LAMBDA;
      h2_t hv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) hv[e] = cvt2(x[2 * e] * inv, x[2 * e + 1] * inv);
      char* dst = lds + L::OFF_Q + row * L::QPB + 16 * e4;
      st4(dst, cat2(hv[0], hv[1]));
      st4(dst + 8, cat2(hv[2], hv[3]));
      if constexpr (LO) {
        h2_t lv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) lv[e] = cvt2(x[2 * e] * inv - (float)hv[e][0], x[2 * e + 1] * inv - (float)hv[e][1]);
        char* dl = lds + L::OFF_QLO + row * L::QPB + 16 * e4;
        st4(dl, cat2(lv[0], lv[1]));
        st4(dl + 8, cat2(lv[2], lv[3]));
      }
    }
  }
};

// ---- build: S[tile][dt] += psi(K_tile)^T (sigma V) over one chunk; Gram M += K^T K
template <int DV, int C, int NTW, int TB, bool GRAM>
__device__ __forceinline__ void build_chunk(acc_t (&S)[NTW > 0 ? NTW : 1][DV / 32], acc_t& Mt, const char* lds,
                                            int off_k, int off_v) {
  using L = Lay<DV, C>;
  constexpr int NDT = L::NDT;
  const int lane = threadIdx.x & 63, g = lane >> 4, i = lane & 15;
  const int qs = 4 * (g & 1) + (i & 3);             // quad of the row this lane addresses
  const int tok = 8 * (g >> 1) + (i >> 2);          // token this lane addresses (+ 4 for the second read)
  const uint32_t own = (uint32_t)(off_k + tok * L::KPB + 8 * qs);
  const uint32_t vl = (uint32_t)(off_v + tok * L::VPB + 2 * (16 * (g & 1) + 4 * (i & 3)));
  uint32_t part[NTW > 0 ? NTW : 1];
  [&]<int... TI>(std::integer_sequence<int, TI...>) {
    ((part[TI] = (uint32_t)(off_k + tile_copy(TB + TI, qs) * L::KCOPY + tok * L::KPB + 8 * tile_partner(TB + TI, qs))), ...);
  }(std::make_integer_sequence<int, NTW>{});
#pragma unroll
  for (int st = 0; st < L::NSTEP; ++st) {
    const uint32_t k0 = 16 * st * L::KPB, k1 = k0 + 4 * L::KPB;
    const h8_t ko = tr16x2(lds, own + k0, own + k1);
    h8_t vf[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
      vf[dt] = tr16x2(lds, vl + 16 * st * L::VPB + 64 * dt, vl + (16 * st + 4) * L::VPB + 64 * dt);
#pragma unroll
    for (int t = 0; t < NTW; ++t) {
      const h8_t kp = tr16x2(lds, part[t] + k0, part[t] + k1);
      const h8_t psi = ko * kp;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) S[t][dt] = mfma(psi, vf[dt], S[t][dt]);
    }
    if constexpr (GRAM) Mt = mfma(ko, ko, Mt);
  }
}

// state fragments of this wave's tiles (sigma S, fp16) for the readout
template <int DV, int C, int NTW, int TB>
__device__ __forceinline__ void write_state(const acc_t (&S)[NTW > 0 ? NTW : 1][DV / 32], char* lds) {
  using L = Lay<DV, C>;
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int t = 0; t < NTW; ++t)
#pragma unroll
    for (int dt = 0; dt < L::NDT; ++dt)
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        h2_t y[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          y[e] = cvt2(S[t][dt][8 * s + 2 * e], S[t][dt][8 * s + 2 * e + 1]);
          if (tile_doubled(TB + t)) y[e] = y[e] * h2_t{(_Float16)0.5f, (_Float16)0.5f};
        }
        st8(lds + (((TB + t) * 2 + s) * L::NDT + dt) * 1024 + lane * 16, cat4(y[0], y[1], y[2], y[3]));
      }
}

// Gram matrix to LDS as fp16 hi + lo of M 2^-ge, columns permuted so that the denominator's
// operand reads its k-slots (components 16s + 8(e/4) + 4h + e%4) as 16 bytes
template <int DV, int C>
__device__ __forceinline__ void write_gram(const acc_t& Mt, char* lds, int ge) {
  using L = Lay<DV, C>;
  const int lane = threadIdx.x & 63, n = lane & 31, h = lane >> 5;
  const float sc = pow2f(-ge);
#pragma unroll
  for (int half = 0; half < 2; ++half) {  // accumulator rows 8i + 4h + j, i = 2 half, 2 half + 1
    h2_t hi[4], lo[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float a = Mt[8 * half + 2 * e] * sc, b = Mt[8 * half + 2 * e + 1] * sc;
      hi[e] = cvt2(a, b);
      lo[e] = cvt2(a - (float)hi[e][0], b - (float)hi[e][1]);
    }
    char* row = lds + L::OFF_M + n * L::MPB + 2 * (16 * half + 8 * h);
    st8(row, cat4(hi[0], hi[1], hi[2], hi[3]));
    st8(row + 32 * L::MPB, cat4(lo[0], lo[1], lo[2], lo[3]));
  }
}

// final state in the decode layout: S[f][d] = sum_s psi_f(k_hat_s) v_s[d] (packed order,
// sqrt(2) off the diagonal), Z[f] = sum_s psi_f(k_hat_s), from registers holding sigma S
template <int DV, int NTW, int TB, bool GRAM>
__device__ __forceinline__ void write_final_state(const Args& a, int64_t bh, const acc_t (&S)[NTW > 0 ? NTW : 1][DV / 32],
                                                  const acc_t& Mt, float inv_sig) {
  constexpr int n = P * (P + 1) / 2;
  const int lane = threadIdx.x & 63, col = lane & 31, h = lane >> 5;
  float* so = a.s_out + bh * (int64_t)n * DV;
#pragma unroll
  for (int t = 0; t < NTW; ++t) {
#pragma unroll
    for (int ii = 0; ii < 4; ++ii)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int m = 8 * ii + 4 * h + j, qa = m >> 2, c = m & 3;
        const int tt = TB + t;
        const int r = tile_xor(tt, qa);
        const int fa = 4 * qa + c, fb = 4 * tile_partner(tt, qa) + (c ^ r);
        if (tile_doubled(tt) && c > (c ^ r)) continue;  // the other copy of this pair
        const int i0 = fa < fb ? fa : fb, j0 = fa < fb ? fb : fa;
        const int f = i0 * P - i0 * (i0 - 1) / 2 + (j0 - i0);
        const float sc = (tt == 0 ? 1.f : 0.70710678118654752f) * inv_sig;
#pragma unroll
        for (int dt = 0; dt < DV / 32; ++dt) so[(int64_t)f * DV + 32 * dt + col] = S[t][dt][4 * ii + j] * sc;
      }
  }
  if constexpr (GRAM) {
    float* zo = a.z_out + bh * (int64_t)n;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = 8 * ii + 4 * h + j;
        if (row > col) continue;
        const int f = row * P - row * (row - 1) / 2 + (col - row);
        zo[f] = Mt[4 * ii + j] * (row == col ? 1.f : 1.41421356237309515f);
      }
  }
}

// ---- readout wave: token group G, tiles [TB, TE); OWNER also runs the intra block, the
// denominator and the output
template <int DV, int C, int W>
struct Reader {
  using L = Lay<DV, C>;
  static constexpr int NDT = L::NDT;
  static constexpr int G = W / L::FS, F = W % L::FS;
  static constexpr int TB = L::rb(F), TE = L::rb(F + 1);
  static constexpr bool OWNER = F == L::FS - 1;

  // psi'(q) slots of quad a (lower-half view) for tile T: (c0, c1) and (c2, c3)
  template <int T, int A>
  __device__ static __forceinline__ void quad_slots(const h2_t (&R)[16], h2_t& p01, h2_t& p23) {
    constexpr int B = tile_partner(T, A), r = tile_xor(T, A);
    const h2_t x01 = R[2 * B + (r >> 1)], x23 = R[2 * B + 1 - (r >> 1)];
    p01 = R[2 * A] * ((r & 1) ? swp(x01) : x01);
    p23 = R[2 * A + 1] * ((r & 1) ? swp(x23) : x23);
  }

  __device__ static __forceinline__ void run(const Args& a, char* lds) {
    const int lane = threadIdx.x & 63, t = lane & 31, h = lane >> 5;
    const int64_t bh = blockIdx.x / a.nblk_per_bh;
    const int seg = blockIdx.x % a.nblk_per_bh;
    int64_t row0;
    int rstep, Tb;
    seq_rows_of(a.lay, bh, a.H, a.T, row0, rstep, Tb);
    const int nchunks = (Tb + C - 1) / C;
    const int c0 = seg * a.cps, c1 = min(nchunks, c0 + a.cps);
    const int osz = a.o_f32 ? 4 : 2;
    char* obase = static_cast<char*>(a.o) + row0 * DV * osz;
    const uint32_t orsv = (uint32_t)rstep * DV;
    uint32_t* red = reinterpret_cast<uint32_t*>(lds + L::OFF_RED);

    QStage<DV, C, 64 * L::FS> qs;
    qs.init(a.q, row0, rstep, Tb);
    const int qtid = F * 64 + lane;
    if (c0 < c1) qs.load(c0 * C, 32 * G, qtid);
    __syncthreads();  // prologue 1: prefix maxima and the first chunk's value maximum published
    // every wave follows the same bound and scale: beta >= max |S| over the state so far
    float beta;
    int e_sig;
    {
      const float pm = __uint_as_float(max(max(red[0], red[1]), max(red[2], red[3])));
      const uint32_t vb = max(max(red[4], red[5]), max(red[6], red[7]));
      beta = pm + (float)C * __uint_as_float(vb << 16);
      e_sig = scale_exp(beta, 100);
    }
    if (c0 < c1) {
      if (c0 == 0) qs.template store<true>(lds, 32 * G, qtid);
      else qs.template store<false>(lds, 32 * G, qtid);
    }
    __syncthreads();  // prologue 2: chunk c0 staged, state before it in LDS

    for (int c = c0; c < c1; ++c) {
      const int t0 = c * C;
      if (c + 1 < c1) qs.load(t0 + C, 32 * G, qtid);
      // ---- phase 1: readout of chunk c
      h2_t R[16];
      {
        const char* qrow = lds + L::OFF_Q + (32 * G + t) * L::QPB;
#pragma unroll
        for (int b = 0; b < 8; ++b) {
          const h4_t x = ld4(qrow + 8 * ((b + h) & 7));
          R[2 * b] = lo2(x);
          R[2 * b + 1] = hi2(x);
        }
      }
      acc_t O[NDT];
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) O[dt] = zero_acc();
      if (c > 0) {
        [&]<int... TI>(std::integer_sequence<int, TI...>) {
          (([&] {
             constexpr int T = TB + TI / 2, s = TI % 2;
             h2_t p0, p1, p2, p3;
             quad_slots<T, 4 * s>(R, p0, p1);
             quad_slots<T, 4 * s + 2>(R, p2, p3);
             const h8_t psi = cat4(p0, p1, p2, p3);
#pragma unroll
             for (int dt = 0; dt < NDT; ++dt) {
               const h8_t sf = ld8(lds + ((T * 2 + s) * NDT + dt) * 1024 + lane * 16);
               O[dt] = mfma(sf, psi, O[dt]);
             }
           }()),
           ...);
        }(std::make_integer_sequence<int, 2 * (TE - TB)>{});
      }
      float den = 0.f;
      if constexpr (OWNER) {
        // query operand of the component contractions: k-slots 16s + 8(e/4) + 4h + e%4
        const h8_t qop[2] = {cat4(R[0], R[1], R[4], R[5]), cat4(R[8], R[9], R[12], R[13])};
        if (c > 0) {  // denominator, inter-chunk part: X = (M 2^-ge) Q^T, then q . X
          acc_t X = zero_acc();
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            const char* mrow = lds + L::OFF_M + t * L::MPB + 2 * (16 * s + 8 * h);
            X = mfma(ld8(mrow), qop[s], X);
            X = mfma(ld8(mrow + 32 * L::MPB), qop[s], X);
          }
          float dx = 0.f;
#pragma unroll
          for (int ii = 0; ii < 4; ++ii)
#pragma unroll
            for (int j = 0; j < 4; ++j) dx += X[4 * ii + j] * (float)R[4 * ii + j / 2][j & 1];
          den = dx * pow2f(gram_exp(t0));
        }
        // intra-chunk block over key groups 0..G
        auto intra = [&]<bool SPLIT>() {
          h8_t qlo[2];
          if constexpr (SPLIT) {
            const char* lrow = lds + L::OFF_QLO + (32 * G + t) * L::QPB;
#pragma unroll
            for (int s = 0; s < 2; ++s) qlo[s] = cat44(ld4(lrow + 8 * (4 * s + h)), ld4(lrow + 8 * (4 * s + 2 + h)));
          }
          const int lg = lane >> 4, li = lane & 15;
          const uint32_t vrow = (uint32_t)(L::OFF_V + (4 * (lg >> 1) + (li >> 2)) * L::VPB + 2 * (16 * (lg & 1) + 4 * (li & 3)));
#pragma unroll
          for (int kg = 0; kg <= G; ++kg) {
            acc_t Sc = zero_acc();
            const char* krow = lds + L::OFF_K + (32 * kg + t) * L::KPB;
#pragma unroll
            for (int s = 0; s < 2; ++s) {
              const h8_t kop = cat44(ld4(krow + 8 * (4 * s + h)), ld4(krow + 8 * (4 * s + 2 + h)));
              Sc = mfma(kop, qop[s], Sc);
              if constexpr (SPLIT) {
                const char* lrow = lds + L::OFF_KLO + (32 * kg + t) * L::KPB;
                Sc = mfma(cat44(ld4(lrow + 8 * (4 * s + h)), ld4(lrow + 8 * (4 * s + 2 + h))), qop[s], Sc);
                Sc = mfma(kop, qlo[s], Sc);
              }
            }
            // weights: keys 8ii + 4h + j of group kg for query t; causal on the diagonal group
            h2_t wv[8];
#pragma unroll
            for (int ii = 0; ii < 4; ++ii)
#pragma unroll
              for (int j = 0; j < 4; j += 2) {
                float w0 = Sc[4 * ii + j] * Sc[4 * ii + j];
                float w1 = Sc[4 * ii + j + 1] * Sc[4 * ii + j + 1];
                if (kg == G) {
                  if (8 * ii + 4 * h + j > t) w0 = 0.f;
                  if (8 * ii + 4 * h + j + 1 > t) w1 = 0.f;
                }
                const h2_t wp = cvt2(w0, w1);
                wv[2 * ii + j / 2] = wp;
                den += (float)wp[0];
                den += (float)wp[1];
              }
#pragma unroll
            for (int s = 0; s < 2; ++s) {
              const h8_t wop = cat4(wv[4 * s], wv[4 * s + 1], wv[4 * s + 2], wv[4 * s + 3]);
#pragma unroll
              for (int dt = 0; dt < NDT; ++dt) {
                const uint32_t o0 = vrow + (32 * kg + 16 * s) * L::VPB + 64 * dt;
                const h8_t vfr = tr16x2(lds, o0, o0 + 8 * L::VPB);
                O[dt] = mfma(vfr, wop, O[dt]);
              }
            }
          }
        };
        if (c == 0) intra.template operator()<true>();
        else intra.template operator()<false>();
        den = xor32_sum(den);
      }
      if constexpr (!OWNER) {  // hand the partial readout to the owner of this group
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          char* dst = lds + L::OFF_PART + ((G * (L::FS - 1) + F) * NDT + dt) * 4096 + lane * 64;
#pragma unroll
          for (int u = 0; u < 4; ++u)
            *reinterpret_cast<f32x4_t*>(dst + 16 * u) = f32x4_t{O[dt][4 * u], O[dt][4 * u + 1], O[dt][4 * u + 2], O[dt][4 * u + 3]};
        }
      }
      __syncthreads();
      // ---- phase 2: output of chunk c (with this chunk's sigma), staging of chunk c + 1
      if constexpr (OWNER) {
#pragma unroll
        for (int f = 0; f < L::FS - 1; ++f)
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) {
            const char* src = lds + L::OFF_PART + ((G * (L::FS - 1) + f) * NDT + dt) * 4096 + lane * 64;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const f32x4_t x = *reinterpret_cast<const f32x4_t*>(src + 16 * u);
#pragma unroll
              for (int e = 0; e < 4; ++e) O[dt][4 * u + e] += x[e];
            }
          }
        const float inv = den > 0.f ? pow2f(-e_sig) * __builtin_amdgcn_rcpf(den) : 0.f;
        const int orow = t0 + 32 * G;
        const int orows = Tb - orow;
        if (orows > 0) {
          const __amdgpu_buffer_rsrc_t ro = buf_rsrc(obase + (int64_t)orow * orsv * osz, ((uint32_t)(orows - 1) * orsv + DV) * osz);
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
              const uint32_t ob = (uint32_t)t * orsv + 32 * dt + 8 * ii + 4 * h;
              const float o0 = O[dt][4 * ii] * inv, o1 = O[dt][4 * ii + 1] * inv;
              const float o2 = O[dt][4 * ii + 2] * inv, o3 = O[dt][4 * ii + 3] * inv;
              if (a.o_f32)
                __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{__float_as_uint(o0), __float_as_uint(o1), __float_as_uint(o2), __float_as_uint(o3)},
                                                       ro, ob * 4, 0, 0);
              else
                __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{pk2(o0, o1), pk2(o2, o3)}, ro, ob * 2, 0, 0);
            }
        }
      }
      if (c + 1 < c1) {
        // the bound grows by at most C max|v| per chunk (|psi_f| <= 1 with c^2 folded in)
        const uint32_t vb = max(max(red[4], red[5]), max(red[6], red[7]));
        beta += (float)C * __uint_as_float(vb << 16);
        e_sig = scale_exp(beta, e_sig);
        qs.template store<false>(lds, 32 * G, qtid);
      }
      __syncthreads();
    }
  }
};

// ---- build wave j of the forward (tiles Fwd4::tb(j) .. tb(j+1))
template <int DV, int C, int J>
struct Builder {
  using L = Lay<DV, C>;
  static constexpr int NDT = L::NDT;
  static constexpr int TB = Fwd4::tb(J), NTW = Fwd4::tb(J + 1) - Fwd4::tb(J);
  static constexpr bool GRAM = Fwd4::gram(J);

  __device__ static __forceinline__ void run(const Args& a, char* lds) {
    const int lane = threadIdx.x & 63;
    const int btid = J * 64 + lane;  // 0..255 over the build waves
    const int64_t bh = blockIdx.x / a.nblk_per_bh;
    const int seg = blockIdx.x % a.nblk_per_bh;
    int64_t row0;
    int rstep, Tb;
    seq_rows_of(a.lay, bh, a.H, a.T, row0, rstep, Tb);
    const int nchunks = (Tb + C - 1) / C;
    const int c0 = seg * a.cps, c1 = min(nchunks, c0 + a.cps);
    uint32_t* red = reinterpret_cast<uint32_t*>(lds + L::OFF_RED);

    acc_t S[NTW > 0 ? NTW : 1][NDT];
    acc_t Mt = zero_acc();
#pragma unroll
    for (int i = 0; i < NTW; ++i)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) S[i][dt] = zero_acc();
    float pmax = 0.f;
    if (seg > 0) {  // exclusive prefix of this segment (true units)
      const float* src = a.ws + (bh * (a.nseg - 1) + (seg - 1)) * L::STATE_FLOATS;
#pragma unroll
      for (int i = 0; i < NTW; ++i)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const float* p = src + ((TB + i) * NDT + dt) * 1024 + lane * 16;
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const f32x4_t x = *reinterpret_cast<const f32x4_t*>(p + 4 * u);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              S[i][dt][4 * u + e] = x[e];
              pmax = fmaxf(pmax, fabsf(x[e]));
            }
          }
        }
      if constexpr (GRAM) {
        const float* p = src + (int64_t)NTL * NDT * 1024 + lane * 16;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const f32x4_t x = *reinterpret_cast<const f32x4_t*>(p + 4 * u);
#pragma unroll
          for (int e = 0; e < 4; ++e) Mt[4 * u + e] = x[e];
        }
      }
    }
    KVStage<DV, C, 256> kv;
    kv.init(a.k, a.v, row0, rstep, Tb);
    if (c0 < c1) kv.load(c0 * C, btid);
    {
      const uint32_t pm = wave_max_u32(__float_as_uint(pmax));
      const uint32_t vm = wave_max_u32(c0 < c1 ? kv.vmax_bits(btid) : 0u);
      if (lane == 0) {
        red[J] = pm;
        red[4 + J] = vm;
      }
    }
    __syncthreads();  // prologue 1
    float beta;
    int e_sig;
    {
      const float pm = __uint_as_float(max(max(red[0], red[1]), max(red[2], red[3])));
      const uint32_t vb = max(max(red[4], red[5]), max(red[6], red[7]));
      beta = pm + (float)C * __uint_as_float(vb << 16);
      e_sig = scale_exp(beta, 100);
    }
    if (seg > 0) {
      const float sg = pow2f(e_sig);
#pragma unroll
      for (int i = 0; i < NTW; ++i)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) S[i][dt] *= sg;
    }
    if (c0 < c1) {
      if (c0 == 0) {
        kv.template store<true>(lds, L::OFF_K, L::OFF_V, pow2f(e_sig), btid, L::OFF_KLO);
      } else {
        kv.template store<false>(lds, L::OFF_K, L::OFF_V, pow2f(e_sig), btid, 0);
        write_state<DV, C, NTW, TB>(S, lds);
        if constexpr (GRAM) write_gram<DV, C>(Mt, lds, gram_exp(c0 * C));
      }
    }
    __syncthreads();  // prologue 2

    for (int c = c0; c < c1; ++c) {
      const int t0 = c * C;
      if (c + 1 < c1) kv.load(t0 + C, btid);
      // ---- phase 1: build of chunk c
      build_chunk<DV, C, NTW, TB, GRAM>(S, Mt, lds, L::OFF_K, L::OFF_V);
      if (c + 1 < c1) {
        const uint32_t vm = wave_max_u32(kv.vmax_bits(btid));
        if (lane == 0) red[4 + J] = vm;
      }
      __syncthreads();
      // ---- phase 2: state after chunk c (scaled for chunk c + 1), staging of chunk c + 1
      if (c + 1 < c1) {
        const uint32_t vb = max(max(red[4], red[5]), max(red[6], red[7]));
        beta += (float)C * __uint_as_float(vb << 16);
        const int e_new = scale_exp(beta, e_sig);
        if (e_new != e_sig) {
          const float f = pow2f(e_new - e_sig);
#pragma unroll
          for (int i = 0; i < NTW; ++i)
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) S[i][dt] *= f;
          e_sig = e_new;
        }
        kv.template store<false>(lds, L::OFF_K, L::OFF_V, pow2f(e_sig), btid, 0);
        write_state<DV, C, NTW, TB>(S, lds);
        if constexpr (GRAM) write_gram<DV, C>(Mt, lds, gram_exp(t0 + C));
      }
      __syncthreads();
    }
    if (a.s_out != nullptr && seg == a.nblk_per_bh - 1)
      write_final_state<DV, NTW, TB, GRAM>(a, bh, S, Mt, pow2f(-e_sig));
  }
};

// ---- summary pass: [S | M] of one segment after its chunks (8 build waves, key and value
// staging double-buffered, one barrier per chunk), written in true units
template <int DV, int C, int J>
__device__ __forceinline__ void run_summary(const Args& a, char* lds) {
  using L = Lay<DV, C>;
  constexpr int NDT = L::NDT;
  constexpr int TB = Sum8::tb(J), NTW = Sum8::tb(J + 1) - Sum8::tb(J);
  constexpr bool GRAM = Sum8::gram(J);
  const int lane = threadIdx.x & 63, tid = threadIdx.x;
  const int64_t bh = blockIdx.x / a.nblk_per_bh;
  const int seg = blockIdx.x % a.nblk_per_bh;
  int64_t row0;
  int rstep, Tb;
  seq_rows_of(a.lay, bh, a.H, a.T, row0, rstep, Tb);
  const int nchunks = (Tb + C - 1) / C;
  const int c0 = seg * a.cps, c1 = min(nchunks, c0 + a.cps);
  uint32_t* red = reinterpret_cast<uint32_t*>(lds + L::SUM_RED);  // [2 parities][8 waves]

  acc_t S[NTW > 0 ? NTW : 1][NDT];
  acc_t Mt = zero_acc();
#pragma unroll
  for (int i = 0; i < NTW; ++i)
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) S[i][dt] = zero_acc();
  KVStage<DV, C, 512> kv;
  kv.init(a.k, a.v, row0, rstep, Tb);
  auto publish = [&](int chunk) {  // max |v| of the loaded chunk into slot set chunk & 1
    const uint32_t vm = wave_max_u32(kv.vmax_bits(tid));
    if (lane == 0) red[8 * (chunk & 1) + J] = vm;
  };
  auto vmax_of = [&](int chunk) {
    const uint32_t* r = red + 8 * (chunk & 1);
    uint32_t m = 0;
#pragma unroll
    for (int w = 0; w < 8; ++w) m = max(m, r[w]);
    return __uint_as_float(m << 16);
  };
  float beta = 0.f;
  int e_sig = 100;
  if (c0 < c1) {
    kv.load(c0 * C, tid);
    publish(c0);
  }
  __syncthreads();
  if (c0 < c1) {
    beta = (float)C * vmax_of(c0);
    e_sig = scale_exp(beta, e_sig);
    kv.template store<false>(lds, 0, 5 * L::KCOPY, pow2f(e_sig), tid, 0);
    if (c0 + 1 < c1) {
      kv.load((c0 + 1) * C, tid);
      publish(c0 + 1);
    }
  }
  __syncthreads();
  for (int c = c0; c < c1; ++c) {
    const int buf = (c - c0) & 1;
    build_chunk<DV, C, NTW, TB, GRAM>(S, Mt, lds, buf * L::SUM_BUF, buf * L::SUM_BUF + 5 * L::KCOPY);
    if (c + 1 < c1) {
      beta += (float)C * vmax_of(c + 1);
      const int e_new = scale_exp(beta, e_sig);
      if (e_new != e_sig) {
        const float f = pow2f(e_new - e_sig);
#pragma unroll
        for (int i = 0; i < NTW; ++i)
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) S[i][dt] *= f;
        e_sig = e_new;
      }
      const int nb = (buf ^ 1) * L::SUM_BUF;
      kv.template store<false>(lds, nb, nb + 5 * L::KCOPY, pow2f(e_sig), tid, 0);
      if (c + 2 < c1) {
        kv.load((c + 2) * C, tid);
        publish(c + 2);
      }
    }
    __syncthreads();
  }
  float* dst = a.ws + (bh * (a.nseg - 1) + seg) * L::STATE_FLOATS;
  const float inv = pow2f(-e_sig);
#pragma unroll
  for (int i = 0; i < NTW; ++i)
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      float* p = dst + ((TB + i) * NDT + dt) * 1024 + lane * 16;
#pragma unroll
      for (int u = 0; u < 4; ++u)
        *reinterpret_cast<f32x4_t*>(p + 4 * u) =
            f32x4_t{S[i][dt][4 * u] * inv, S[i][dt][4 * u + 1] * inv, S[i][dt][4 * u + 2] * inv, S[i][dt][4 * u + 3] * inv};
    }
  if constexpr (GRAM) {
    float* p = dst + (int64_t)NTL * NDT * 1024 + lane * 16;
#pragma unroll
    for (int u = 0; u < 4; ++u)
      *reinterpret_cast<f32x4_t*>(p + 4 * u) = f32x4_t{Mt[4 * u], Mt[4 * u + 1], Mt[4 * u + 2], Mt[4 * u + 3]};
  }
}

template <int DV, int C>
__global__ __launch_bounds__(512, 1) void summary_f16_kernel(Args a) {
  extern __shared__ __align__(16) char lds[];
  switch (threadIdx.x >> 6) {
    case 0: run_summary<DV, C, 0>(a, lds); break;
    case 1: run_summary<DV, C, 1>(a, lds); break;
    case 2: run_summary<DV, C, 2>(a, lds); break;
    case 3: run_summary<DV, C, 3>(a, lds); break;
    case 4: run_summary<DV, C, 4>(a, lds); break;
    case 5: run_summary<DV, C, 5>(a, lds); break;
    case 6: run_summary<DV, C, 6>(a, lds); break;
    default: run_summary<DV, C, 7>(a, lds); break;
  }
}

template <int DV, int C>
__global__ __launch_bounds__(512, 1) void chunked_f16_kernel(Args a) {
  extern __shared__ __align__(16) char lds[];
  switch (threadIdx.x >> 6) {
    case 0: Reader<DV, C, 0>::run(a, lds); break;
    case 1: Reader<DV, C, 1>::run(a, lds); break;
    case 2: Reader<DV, C, 2>::run(a, lds); break;
    case 3: Reader<DV, C, 3>::run(a, lds); break;
    case 4: Builder<DV, C, 0>::run(a, lds); break;
    case 5: Builder<DV, C, 1>::run(a, lds); break;
    case 6: Builder<DV, C, 2>::run(a, lds); break;
    default: Builder<DV, C, 3>::run(a, lds); break;
  }
}

}  // namespace c16
}  // namespace kata

namespace kata {
namespace c16 {

template <int DV, int C>
hipError_t launch(const uint16_t* q, const uint16_t* k, const uint16_t* v, void* o, bool o_bf16, int B, int H, int T,
                  const SegPlan& plan, float* ws, float* s_out, float* z_out, SeqLayout lay, int passes,
                  hipStream_t st) {
  using L = Lay<DV, C>;
  const int BH = B * H;
  Args a{q, k, v, o, ws, T, plan.nseg, plan.cps, 0, o_bf16 ? 0 : 1, s_out, z_out, lay, H};
  hipError_t e;
  if (plan.nseg > 1 && (passes & PASS_SUMMARIES)) {
    a.nblk_per_bh = plan.nseg - 1;
    auto ks = summary_f16_kernel<DV, C>;
    if ((e = hipFuncSetAttribute((const void*)ks, hipFuncAttributeMaxDynamicSharedMemorySize, L::SUM_LDS)) != hipSuccess)
      return e;
    ks<<<dim3((unsigned)(BH * (plan.nseg - 1))), dim3(512), L::SUM_LDS, st>>>(a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (plan.nseg > 1 && (passes & PASS_SCAN))
    if ((e = launch_scan(ws, BH, plan.nseg - 1, L::STATE_FLOATS, st)) != hipSuccess) return e;
  if (!(passes & PASS_SEGMENTS)) return hipSuccess;
  auto kf = chunked_f16_kernel<DV, C>;
  if ((e = hipFuncSetAttribute((const void*)kf, hipFuncAttributeMaxDynamicSharedMemorySize, L::LDS)) != hipSuccess) return e;
  a.nblk_per_bh = plan.nseg;
  kf<<<dim3((unsigned)(BH * plan.nseg)), dim3(512), L::LDS, st>>>(a);
  return hipGetLastError();
}

}  // namespace c16
}  // namespace kata
