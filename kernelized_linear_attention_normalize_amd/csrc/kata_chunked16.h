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
// off-diagonal coordinate appears once, with c^2 = 2 folded into the build (the segment pass
// doubles the own operand of tiles 1-17; the summary pass doubles its result), and the
// within-block pairs twice at weight 1 (tiles 1-3 are built at 2x and halved when the state
// is handed to the readout).
//   * Build (psi(K)^T V on 16x16x32 MFMA, 16-row tiles u = 2 t + half): lane = (row,
//     8 tokens). Keys and values are staged transposed (component-major k_hat^T and
//     sigma V^T), so each operand of a 32-token step is one 16-byte LDS read: own component,
//     partner component, value column. The row and piece placement (the
//     tpos comment) keeps those reads free of bank conflicts for ds_read_b128's lane groups.
//   * Readout (O^T = S^T psi(Q)^T): lane = (token, lane half). A lane holds its token's 32
//     components as 16 packed fp16 pairs, rotated by one block in the upper lane half, so
//     one instruction stream serves quads 4s, 4s+2 (lower half) and 4s+1, 4s+3 (upper);
//     each pair of slots is one v_pk_mul_f16 with op_sel choosing the partner's halves.
//   * State fragments: build lane (value column, quad g) of tile u converts its 4
//     accumulators to fp16 and writes 8 bytes, placed so that readout lane (value row, half h)
//     reads quads h and h + 2 of the tile as one 16-byte piece.
//   * Denominator psi(q)^T Z = q^T M q (Gram matrix, fp32-accurate as hi + lo); the
//     intra-chunk block computes (q_hat . k_hat)^2 from the components (weight identity of
//     the lift display); the denominator sums the fp32 weights, whose fp16 copies multiply V
//     (each within 2^-11 of it).
//
// Segment pass waves: 0-3 read out (token group of 32, or a share of the tiles of one) and
// stage the queries, 4-11 build (nine 16-row tiles per SIMD, waves w and w + 4 share one) and
// stage the keys and values. The chunk operands are double-buffered. Per chunk: phase 1 =
// staging of chunk c + 1 into the other buffers (its loads were issued during chunk c - 1),
// readout of chunk c from the state before it, build of chunk c, loads of chunk c + 2 |
// barrier | phase 2 = output, state after chunk c to LDS | barrier. ASSOCIATIVE runs a
// summary pass (8 build waves and 4 staging waves over a double buffer, one barrier per
// chunk), the segment scan and the segments; SEQUENTIAL runs one segment per sequence.
//
// S2 (KATA-Sigma 2, reduced PSD families paragraph of the HTML page: psi(u) = u_1 u_1^T +
// u_2 u_2^T over two 32-component blocks of a 64-component row, normalised as a whole): the
// same tiles, state and scales, with every lifted coordinate the sum of both blocks'
// products, intra-chunk weights sum_{a,b} (q_a . k_b)^2 and the Gram matrix summed over the
// blocks. Its operands take twice the rows, so the chunk operands are single-buffered and
// the next chunk is staged in phase 2.
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
// LDS byte address of a pointer into the kernel's dynamic LDS, and a 16-byte read at such an
// address. These kernels declare no static LDS, so the dynamic block starts at address 0 and
// a base folded into an address keeps bits 0-7 of the offset (step reads XOR bits 6-7).
__device__ __forceinline__ uint32_t lds_addr(const char* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}
__device__ __forceinline__ h8_t ld8a(uint32_t a) {
  return *(const __attribute__((address_space(3))) h8_t*)(uintptr_t)a;
}

// ---- LDS layout and work split
// 12 waves: 0-3 read out, 4-11 build; wave w runs on SIMD w % 4, so every SIMD hosts one
// readout wave and two build waves.
constexpr int NU = 2 * NTL;  // 16-row build tiles: u = 2 t + half holds quads 4 half .. 4 half + 3 of tile t

template <int DV, int C, bool S2 = false>
struct Lay {
  // S2: KATA-Sigma 2 on 64-component rows (two 32-component blocks whose lifts are summed);
  // its operands take twice the rows, so the chunk operands are single-buffered to fit LDS
  static constexpr int PC = S2 ? 64 : 32;      // components per query and key row
  static constexpr int NBUF = S2 ? 1 : 2;      // chunk operand buffers
  static constexpr int NDT = DV / 32;          // 32-column value tiles of the readout
  static constexpr int NDV = DV / 16;          // 16-column value tiles of the build
  static constexpr int NG = C / 32;            // 32-token groups per chunk
  static constexpr int FS = 4 / NG;            // readout waves per token group
  static constexpr int NS = C / 32;            // 32-token build steps
  static constexpr int QPB = 2 * PC + 8;       // q_hat row pitch, bytes (8-byte block reads conflict-free)
  static constexpr int KPB = 64;               // row-major key rows (unscaled k_hat) of one 32-component block, bytes
  // Byte offset of 4-component block b (8 bytes) of key row r. A read of 8 bytes serves 32
  // lanes per cycle; the intra-chunk product's lanes read rows 32 kg + t (t = lane % 32) at
  // a common block, and at a 64-byte pitch rows t and t + 4 would share banks. Block b of
  // row r therefore sits at block b ^ (r / 4) % 8: the 32 lanes cover all 64 banks. S2 keeps
  // each 32-component block of the keys in a region of its own (block b / 8 of the row), so
  // the second block's reads are the first block's at a constant offset.
  __device__ static __forceinline__ int krpos(int r, int b) {
    return S2 ? (b >> 3) * (C * KPB) + r * KPB + 8 * ((b & 7) ^ ((r >> 2) & 7)) : r * KPB + 8 * (b ^ ((r >> 2) & 7));
  }
  static constexpr int RPB = 256;              // transposed rows (one component or value column), bytes
  static constexpr int MPB = 80;               // Gram row pitch, bytes
  static constexpr int ST = NU * NDV * 64 * 8;  // state fragments: [u][value tile][lane half][column] x 8 fp16
  // chunk operands, two buffers each (chunk c + 1 is staged while chunk c is used)
  static constexpr int QB = C * QPB, KRB = C * KPB * (PC / 32), KTB = PC * RPB, VTB = DV * RPB;
  static constexpr int OFF_Q = ST;                      // lambda q_hat rows
  static constexpr int OFF_KR = OFF_Q + NBUF * QB;      // k_hat rows (intra-chunk scores)
  static constexpr int OFF_KT = OFF_KR + NBUF * KRB;    // k_hat^T (build operands, Gram)
  static constexpr int OFF_VT = OFF_KT + NBUF * KTB;    // sigma V^T
  static constexpr int OFF_M = OFF_VT + NBUF * VTB;     // Gram hi, lo
  static constexpr int KOFF = 32 * RPB;                 // k_hat^T rows of the second block (S2)
  static constexpr int OFF_PART = OFF_M + 2 * 32 * MPB;
  static constexpr int PART = FS > 1 ? NG * (FS - 1) * NDT * 64 * 64 : 0;
  // [8 prefix maxima][2 chunk parities][8 value maxima] (uint32)
  static constexpr int OFF_RED = OFF_PART + PART;
  static constexpr int LDS = OFF_RED + 128;
  __device__ static __forceinline__ int offq(int b) { return OFF_Q + (NBUF == 2 ? b : 0) * QB; }
  __device__ static __forceinline__ int offkr(int b) { return OFF_KR + (NBUF == 2 ? b : 0) * KRB; }
  __device__ static __forceinline__ int offkt(int b) { return OFF_KT + (NBUF == 2 ? b : 0) * KTB; }
  __device__ static __forceinline__ int offvt(int b) { return OFF_VT + (NBUF == 2 ? b : 0) * VTB; }
  // first-chunk split operands alias the state area (there is no readout at chunk 0)
  static constexpr int OFF_QLO = 0;
  static constexpr int OFF_KLO = C * QPB;
  static_assert(OFF_KLO + KRB <= ST, "split operands fit the state area");
  static_assert(LDS <= 160 * 1024, "LDS budget");
  static_assert(C <= 128, "four 64-byte blocks per transposed row");
  static_assert(OFF_KT % 256 == 0 && KTB % 256 == 0 && OFF_VT % 256 == 0 && VTB % 256 == 0, "step reads XOR the address");
    // summary pass: [k_hat^T | sigma V^T], double-buffered (partners read k_hat^T and the
  // factor 2 of tiles 1-17 is applied to the summary); value maxima [2 parities][4 staging
  // waves]
  static constexpr int SUM_BUF = (PC + DV) * RPB;
  static constexpr int SUM_RED = 2 * SUM_BUF;
  static constexpr int SUM_LDS = SUM_RED + 128;
  static_assert(SUM_LDS <= 160 * 1024, "LDS budget (summaries)");
  // workspace summary: build tiles in accumulator layout, then the four Gram blocks
  static constexpr int64_t STATE_FLOATS = (int64_t)NU * NDV * 256 + 1024;
  // readout tile range of split f (the last split also runs the intra block and the
  // denominator, so it takes fewer tiles)
  static constexpr int rb(int f) {
    return FS == 1 ? (f == 0 ? 0 : NTL) : (FS == 2 ? (f == 0 ? 0 : (f == 1 ? 10 : NTL)) : (f <= 2 ? 5 * f : (f == 3 ? 14 : NTL)));
  }
  // Byte offset of (row, token position) in a transposed buffer (rows of 256 bytes, buffers
  // 256-byte aligned). Tokens sit at position pi(t) (bits 2 and 3 of t swapped), so that the
  // intra-chunk product finds its k-slots, keys 16s + 4h + j and 16s + 8 + 4h + j, at 8
  // consecutive positions. The 64-byte block of positions 32b .. 32b + 31 is stored at block
  // b ^ (row / 4) % 4 of the row and its 16-byte piece g at piece g ^ row % 4: a 16-byte
  // MFMA operand read serves 16 lanes per cycle, lanes {0-3, 12-15, 20-27} together and
  // {4-11, 16-19, 28-31} together (and both + 32), and with this placement every such lane
  // set meets 16 distinct piece slots of the 256-byte bank window, for own, partner and value
  // rows alike, while the staging writes of one row stay contiguous. Step b of a read adds
  // nothing but XOR 64 b to the address of step 0.
  __device__ static __forceinline__ int tpos(int row, int pos) {
    return row * RPB + 64 * (((pos >> 5) ^ (row >> 2)) & 3) + 16 * (((pos >> 3) & 3) ^ (row & 3)) + 2 * (pos & 7);
  }
  __device__ static __forceinline__ int pi(int t) { return (t & ~12) | ((t >> 1) & 4) | ((t << 1) & 8); }
};

// Build tiles of build wave j: u = first(j) + 2 i, i < count(j), all of one parity (one own
// operand per step). Forward: 8 build waves, even tiles on waves 0-3 (5, 4, 5, 4), odd tiles
// on waves 4-7 (4, 5, 4, 5), 9 tiles per SIMD (waves j and j + 4 share a SIMD). The summary
// pass uses the same map.
struct Fwd8 {
  static constexpr int cnt(int j) { return (j < 4 ? (j % 2 == 0) : (j % 2 == 1)) ? 5 : 4; }
  static constexpr int first(int j) {
    int idx = 0;
    for (int w = (j < 4 ? 0 : 4); w < j; ++w) idx += cnt(w);
    return 2 * idx + (j < 4 ? 0 : 1);
  }
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

typedef float acc4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ acc4_t mfma16(h8_t a, h8_t b, acc4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ acc4_t zero4a() { return acc4_t{0.f, 0.f, 0.f, 0.f}; }

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
// (DPP inside 16-lane rows, permlane swaps across rows: no LDS round trips, unlike
// __shfl_xor, whose ds_bpermute waits would sit on the path to the barrier)
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  auto mx = [](uint32_t a, uint32_t b) { return a > b ? a : b; };
  x = mx(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xf, 0xf, true));   // lane ^ 1
  x = mx(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xf, 0xf, true));   // lane ^ 2
  x = mx(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x141, 0xf, 0xf, true));  // other quad of 8
  x = mx(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x140, 0xf, 0xf, true));  // other half row
  {
    const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    x = mx(r[0], r[1]);
  }
  {
    const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    x = mx(r[0], r[1]);
  }
  return x;
}

// ---- staging of a chunk (global bf16 -> registers -> scaled fp16 LDS layouts)
// LDS targets of the key/value staging (byte offsets; kr < 0: no row-major key copy, kt2 < 0:
// no doubled copy)
struct KVTarget {
  int kr, kt, kt2, vt, klo;
};

template <int DV, int C, int NTHR, bool S2 = false>
struct KVStage {  // keys and values of a chunk, staged by NTHR threads (tid 0..NTHR-1)
  using L = Lay<DV, C, S2>;
  static constexpr int PC = L::PC, KQ = PC / 4;
  // key item = (token pair p, component quarter cq): the KQ items of a pair are adjacent lanes
  static constexpr int KI = KQ * (C / 2);
  static constexpr int KP = (KI + NTHR - 1) / NTHR;
  // value item = (8-column group dg, token pair p), pairs fastest (row writes of whole lanes)
  static constexpr int VI = (C / 2) * (DV / 8);
  static constexpr int VP = (VI + NTHR - 1) / NTHR;
  u32x2_t kr[KP][2];
  u32x4_t vr[VP][2];
  const uint16_t *kb, *vb;
  int len;
  uint32_t rsp, rsv;
  __device__ __forceinline__ void init(const uint16_t* k, const uint16_t* v, int64_t row0, int step, int n) {
    kb = k + row0 * PC;
    vb = v + row0 * DV;
    len = n;
    rsp = (uint32_t)step * PC;
    rsv = (uint32_t)step * DV;
  }
  __device__ __forceinline__ void load(int t0, int tid) {
    const uint32_t left = (uint32_t)(t0 < len ? len - t0 : 0);
    const uint32_t kbytes = left ? ((left - 1) * rsp + PC) * 2 : 0;
    const uint32_t vbytes = left ? ((left - 1) * rsv + DV) * 2 : 0;
    const __amdgpu_buffer_rsrc_t rk = buf_rsrc(kb + (int64_t)t0 * rsp, kbytes);
    const __amdgpu_buffer_rsrc_t rv = buf_rsrc(vb + (int64_t)t0 * rsv, vbytes);
#pragma unroll
    for (int i = 0; i < KP; ++i) {
      const int pc = tid + NTHR * i;
      if (pc < KI) {
        const int p = pc >> (S2 ? 4 : 3), cq = pc & (KQ - 1);
#pragma unroll
        for (int u = 0; u < 2; ++u)
          kr[i][u] = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(rk, ((2 * p + u) * rsp + 4 * cq) * 2, 0, 0));
      }
    }
#pragma unroll
    for (int i = 0; i < VP; ++i) {
      const int pc = tid + NTHR * i;
      if (pc < VI) {
        const int dg = pc / (C / 2), p = pc % (C / 2);
#pragma unroll
        for (int u = 0; u < 2; ++u)
          vr[i][u] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rv, ((2 * p + u) * rsv + 8 * dg) * 2, 0, 0));
      }
    }
  }
  // max |v| of the loaded values as bf16 magnitude bits (ordered like the values)
  __device__ __forceinline__ uint32_t vmax_bits(int tid) const {
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < VP; ++i) {
      const int pc = tid + NTHR * i;
      if (pc < VI) {
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t x = vr[i][u][e] & 0x7fff7fffu;
            const uint32_t lo = x & 0xffffu, hi = x >> 16;
            m = m > lo ? m : lo;
            m = m > hi ? m : hi;
          }
      }
    }
    return m;
  }
  // LDS writes: k_hat rows (if tg.kr >= 0) and their lo parts (LO), k_hat^T, 2 k_hat^T,
  // sigma V^T
  template <bool LO>
  __device__ __forceinline__ void store(char* lds, const KVTarget& tg, float sig, int tid) const {
#pragma unroll
    for (int i = 0; i < KP; ++i) {
      const int pc = tid + NTHR * i;
      if (pc >= KI) continue;
      const int p = pc >> (S2 ? 4 : 3), cq = pc & (KQ - 1);
      float x[2][4], inv[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          x[u][2 * e] = __uint_as_float(kr[i][u][e] << 16);
          x[u][2 * e + 1] = __uint_as_float(kr[i][u][e] & 0xffff0000u);
          ss += x[u][2 * e] * x[u][2 * e] + x[u][2 * e + 1] * x[u][2 * e + 1];
        }
        inv[u] = inv_norm_fast(group_sum<KQ>(ss));
#pragma unroll
        for (int e = 0; e < 4; ++e) x[u][e] *= inv[u];
      }
      if (tg.kr >= 0) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const h2_t a = cvt2(x[u][0], x[u][1]), b = cvt2(x[u][2], x[u][3]);
          st4(lds + tg.kr + L::krpos(2 * p + u, cq), cat2(a, b));
          if constexpr (LO)
            st4(lds + tg.klo + L::krpos(2 * p + u, cq),
                cat2(cvt2(x[u][0] - (float)a[0], x[u][1] - (float)a[1]), cvt2(x[u][2] - (float)b[0], x[u][3] - (float)b[1])));
        }
      }
      const int pos = L::pi(2 * p);  // tokens 2p, 2p + 1 share a 4-byte word
      // lanes cq >= 4 write their components in the order 2, 3, 0, 1: rows 4 cq + c and
      // 4 (cq + 4) + c share bank slots (S2: quarters cq and cq + 8 still meet, 2-way)
      const bool sw = S2 ? (cq & 4) != 0 : cq >= 4;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = i ^ (sw ? 2 : 0);
        const h2_t y = sw ? cvt2(x[0][i ^ 2], x[1][i ^ 2]) : cvt2(x[0][i], x[1][i]);
        const int off = L::tpos(4 * cq + c, pos);
        *reinterpret_cast<h2_t*>(lds + tg.kt + off) = y;
        if (tg.kt2 >= 0) *reinterpret_cast<h2_t*>(lds + tg.kt2 + off) = y * h2_t{(_Float16)2.f, (_Float16)2.f};
      }
    }
#pragma unroll
    for (int i = 0; i < VP; ++i) {
      const int pc = tid + NTHR * i;
      if (pc >= VI) continue;
      const int dg = pc / (C / 2), p = pc % (C / 2);
      const int pos = L::pi(2 * p);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const h2_t ya = cvt2(__uint_as_float(vr[i][0][e] << 16) * sig, __uint_as_float(vr[i][1][e] << 16) * sig);
        const h2_t yb = cvt2(__uint_as_float(vr[i][0][e] & 0xffff0000u) * sig, __uint_as_float(vr[i][1][e] & 0xffff0000u) * sig);
        *reinterpret_cast<h2_t*>(lds + tg.vt + L::tpos(8 * dg + 2 * e, pos)) = ya;
        *reinterpret_cast<h2_t*>(lds + tg.vt + L::tpos(8 * dg + 2 * e + 1, pos)) = yb;
      }
    }
  }
};

// queries of one token group: NTHR threads stage rows [r0, r0 + 32) as lambda q_hat
template <int DV, int C, int NTHR, bool S2 = false>
struct QStage {
  using L = Lay<DV, C, S2>;
  static constexpr int PC = L::PC, QE = PC / 8;  // 8-component pieces per row
  static constexpr int QI = 32 * QE;             // pieces of a 32-row token group
  static constexpr int QP = (QI + NTHR - 1) / NTHR;
  u32x4_t qr[QP];
  const uint16_t* qb;
  int len;
  uint32_t rsp;
  __device__ __forceinline__ void init(const uint16_t* q, int64_t row0, int step, int n) {
    qb = q + row0 * PC;
    len = n;
    rsp = (uint32_t)step * PC;
  }
  __device__ __forceinline__ void load(int t0, int r0, int tid) {
    const int first = t0 + r0;
    const uint32_t left = (uint32_t)(first < len ? len - first : 0);
    const uint32_t bytes = left ? ((left - 1) * rsp + PC) * 2 : 0;
    const __amdgpu_buffer_rsrc_t rq = buf_rsrc(qb + (int64_t)first * rsp, bytes);
#pragma unroll
    for (int i = 0; i < QP; ++i) {
      const int pc = tid + NTHR * i;
      if (pc < QI)
        qr[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rq, ((pc >> (S2 ? 3 : 2)) * rsp + 8 * (pc & (QE - 1))) * 2, 0, 0));
    }
  }
  template <bool LO>
  __device__ __forceinline__ void store(char* lds, int off_q, int r0, int tid) const {
#pragma unroll
    for (int i = 0; i < QP; ++i) {
      const int pc = tid + NTHR * i;
      if (pc >= QI) continue;
      const int row = r0 + (pc >> (S2 ? 3 : 2)), e4 = pc & (QE - 1);
      float x[8];
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[2 * e] = __uint_as_float(qr[i][e] << 16);
        x[2 * e + 1] = __uint_as_float(qr[i][e] & 0xffff0000u);
        ss += x[2 * e] * x[2 * e] + x[2 * e + 1] * x[2 * e + 1];
      }
      ss = group_sum<QE>(ss);
      const float inv = inv_norm_fast(ss) * LAMBDA;
      h2_t hv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) hv[e] = cvt2(x[2 * e] * inv, x[2 * e + 1] * inv);
      char* dst = lds + off_q + row * L::QPB + 16 * e4;
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

// ---- build (16x16x32 MFMA, 32-token steps): S[u][dv] += psi(K_u)^T (sigma V) for the
// wave's tiles u = UB, UB + 2, .. (quads 4 HALF .. 4 HALF + 3). A operand lane = (tile row m,
// 8 token positions of group g): own component 16 HALF + m times the row's partner component,
// both from k_hat^T, one 16-byte read each; B operand lane = (value column, the same 8
// positions) from sigma V^T. Accumulator lane (column n, group g) holds quad g of the tile.
// DBL: tiles 1-17 take the own operand doubled (one packed add per step, shared by the
// wave's tiles), which folds c^2 = 2 of the off-diagonal coordinates into the build; without
// it the caller applies the factor to the result.
// S2: the lift is summed over the two 32-component blocks of a key: psi = own_1 partner_1 +
// own_2 partner_2, the second block's rows 32 rows (a constant offset) further on.
template <int DV, int C, int NU_W, int UB, bool DBL, bool S2 = false>
__device__ __forceinline__ void build_chunk(acc4_t (&S)[NU_W][DV / 16], const char* lds, int off_kt, int off_vt) {
  using L = Lay<DV, C, S2>;
  constexpr uint32_t KO = L::KOFF;
  constexpr int NDV = L::NDV, HALF = UB % 2;
  const int lane = threadIdx.x & 63, g = lane >> 4, m = lane & 15;
  const uint32_t base = lds_addr(lds);
  const uint32_t own = base + (uint32_t)(off_kt + L::tpos(16 * HALF + m, 8 * g));
  uint32_t vl[NDV];
#pragma unroll
  for (int dv = 0; dv < NDV; ++dv) vl[dv] = base + (uint32_t)(off_vt + L::tpos(16 * dv + m, 8 * g));
  uint32_t part[NU_W];
  [&]<int... UI>(std::integer_sequence<int, UI...>) {
    ((part[UI] = base + (uint32_t)(off_kt + ((UB + 2 * UI) / 2 == 0
                                                 ? L::tpos(16 * HALF + m, 8 * g)
                                                 : L::tpos(4 * tile_partner((UB + 2 * UI) / 2, 4 * HALF + (m >> 2)) +
                                                                           ((m & 3) ^ tile_xor((UB + 2 * UI) / 2, 4 * HALF + (m >> 2))),
                                                                       8 * g)))),
     ...);
  }(std::make_integer_sequence<int, NU_W>{});
  // steps stay a loop: unrolled, the scheduler hoists every step's operand reads and the
  // live ranges exceed the register budget of three waves per SIMD
#pragma unroll 1
  for (int st = 0; st < L::NS; ++st) {
    const uint32_t so = 64 * st;
    // Left to itself, the scheduler issues each partner read after the previous tile's
    // MFMAs and waits for it at once. The summary pass (more registers free) issues all of a
    // step's reads before its first product; the segment pass keeps one partner read ahead.
    if constexpr (!DBL && !S2) {
      const h8_t ko = ld8a(own ^ so);
      h8_t pt[NU_W], vf[NDV];
#pragma unroll
      for (int u = 0; u < NU_W; ++u) pt[u] = ld8a(part[u] ^ so);
#pragma unroll
      for (int dv = 0; dv < NDV; ++dv) vf[dv] = ld8a(vl[dv] ^ so);
      __builtin_amdgcn_sched_barrier(0);
      // every tile's lifted operand first, each in its partner's registers, then the products
      // back to back (a lift into the registers of the previous tile's operand, in flight in
      // its MFMAs, measured 1.3% slower)
#pragma unroll
      for (int u = 0; u < NU_W; ++u) pt[u] = ko * pt[u];
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < NU_W; ++u) {
#pragma unroll
        for (int dv = 0; dv < NDV; ++dv) S[u][dv] = mfma16(pt[u], vf[dv], S[u][dv]);
      }
    } else if constexpr (!S2) {
      const h8_t ko = ld8a(own ^ so);
      h8_t vf[NDV];
#pragma unroll
      for (int dv = 0; dv < NDV; ++dv) vf[dv] = ld8a(vl[dv] ^ so);
      h8_t pn = ld8a(part[0] ^ so);
      __builtin_amdgcn_sched_barrier(0);
      const h8_t ko2 = ko + ko;
#pragma unroll
      for (int u = 0; u < NU_W; ++u) {
        const h8_t psi = ((UB + 2 * u) / 2 == 0 ? ko : ko2) * pn;
        if (u + 1 < NU_W) pn = ld8a(part[u + 1] ^ so);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int dv = 0; dv < NDV; ++dv) S[u][dv] = mfma16(psi, vf[dv], S[u][dv]);
      }
    } else {  // S2, one partner pair read ahead in both passes
      const h8_t ka = ld8a(own ^ so), kb = ld8a((own ^ so) + KO);
      h8_t vf[NDV];
#pragma unroll
      for (int dv = 0; dv < NDV; ++dv) vf[dv] = ld8a(vl[dv] ^ so);
      h8_t pa = ld8a(part[0] ^ so), pb = ld8a((part[0] ^ so) + KO);
      __builtin_amdgcn_sched_barrier(0);
      const h8_t ka2 = DBL ? ka + ka : ka, kb2 = DBL ? kb + kb : kb;
#pragma unroll
      for (int u = 0; u < NU_W; ++u) {
        const bool diag = (UB + 2 * u) / 2 == 0;
        const h8_t psi = (diag ? ka : ka2) * pa + (diag ? kb : kb2) * pb;
        if (u + 1 < NU_W) {
          pa = ld8a(part[u + 1] ^ so);
          pb = ld8a((part[u + 1] ^ so) + KO);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int dv = 0; dv < NDV; ++dv) S[u][dv] = mfma16(psi, vf[dv], S[u][dv]);
      }
    }
  }
}

// Gram blocks M_ab = K_a^T K_b (components 16a.., 16b..) of one chunk, a, b in {0, 1}
// (S2: summed over the two 32-component blocks of the keys)
template <int DV, int C, bool S2 = false>
__device__ __forceinline__ void gram_chunk(acc4_t (&Mg)[4], const char* lds, int off_kt) {
  using L = Lay<DV, C, S2>;
  const int lane = threadIdx.x & 63, g = lane >> 4, m = lane & 15;
  const uint32_t base = lds_addr(lds);
  const uint32_t o0 = base + (uint32_t)(off_kt + L::tpos(m, 8 * g));
  const uint32_t o1 = base + (uint32_t)(off_kt + L::tpos(16 + m, 8 * g));
#pragma unroll 1
  for (int st = 0; st < L::NS; ++st) {
    const uint32_t so = 64 * st;
#pragma unroll
    for (int blk = 0; blk < (S2 ? 2 : 1); ++blk) {
      const h8_t olo = ld8a((o0 ^ so) + blk * L::KOFF), ohi = ld8a((o1 ^ so) + blk * L::KOFF);
      Mg[0] = mfma16(olo, olo, Mg[0]);
      Mg[1] = mfma16(olo, ohi, Mg[1]);
      Mg[2] = mfma16(ohi, olo, Mg[2]);
      Mg[3] = mfma16(ohi, ohi, Mg[3]);
    }
  }
}

// state fragments of this wave's tiles (sigma S, fp16) for the readout: build lane (column
// n, group g) writes 8 bytes at [u][value tile][g % 2][n] + 8 (g / 2), so readout lane
// (value row, half h) reads quads h and h + 2 of tile u as one 16-byte piece
template <int DV, int C, int NU_W, int UB>
__device__ __forceinline__ void write_state(const acc4_t (&S)[NU_W][DV / 16], char* lds) {
  using L = Lay<DV, C>;
  const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
  const int lo = (g & 1) * 256 + n * 16 + (g >> 1) * 8;
#pragma unroll
  for (int u = 0; u < NU_W; ++u)
#pragma unroll
    for (int dv = 0; dv < L::NDV; ++dv) {
      h2_t y0 = cvt2(S[u][dv][0], S[u][dv][1]), y1 = cvt2(S[u][dv][2], S[u][dv][3]);
      if (tile_doubled((UB + 2 * u) / 2)) {
        y0 = y0 * h2_t{(_Float16)0.5f, (_Float16)0.5f};
        y1 = y1 * h2_t{(_Float16)0.5f, (_Float16)0.5f};
      }
      st4(lds + ((UB + 2 * u) * L::NDV + dv) * 512 + lo, cat2(y0, y1));
    }
}

// Gram matrix to LDS as fp16 hi + lo of M 2^-ge. Row r holds the denominator operand's
// k-slots (components 16s + 8(e/4) + 4h + e%4 at position 16s + 8h + e: bits 2 and 3 of
// the column swapped); by symmetry block (a, b) writes rows 16b + n, columns 16a + 4g + j.
template <int DV, int C, bool S2 = false>
__device__ __forceinline__ void write_gram(const acc4_t (&Mg)[4], char* lds, int ge) {
  using L = Lay<DV, C, S2>;
  const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
  const int gs = ((g & 1) << 1) | (g >> 1);
  const float sc = pow2f(-ge);
#pragma unroll
  for (int ab = 0; ab < 4; ++ab) {
    const int a = ab >> 1, b = ab & 1;
    const float x0 = Mg[ab][0] * sc, x1 = Mg[ab][1] * sc, x2 = Mg[ab][2] * sc, x3 = Mg[ab][3] * sc;
    const h2_t h0 = cvt2(x0, x1), h1 = cvt2(x2, x3);
    const h2_t l0 = cvt2(x0 - (float)h0[0], x1 - (float)h0[1]), l1 = cvt2(x2 - (float)h1[0], x3 - (float)h1[1]);
    char* row = lds + L::OFF_M + (16 * b + n) * L::MPB + 2 * (16 * a + 4 * gs);
    st4(row, cat2(h0, h1));
    st4(row + 32 * L::MPB, cat2(l0, l1));
  }
}

// final state in the decode layout: S[f][d] = sum_s psi_f(k_hat_s) v_s[d] (packed order,
// sqrt(2) off the diagonal) from registers holding sigma S; Z[f] = sum_s psi_f(k_hat_s) from
// the Gram blocks
template <int DV, int NU_W, int UB>
__device__ __forceinline__ void write_final_s(const Args& a, int64_t bh, const acc4_t (&S)[NU_W][DV / 16], float inv_sig) {
  constexpr int n = P * (P + 1) / 2;
  const int lane = threadIdx.x & 63, col = lane & 15, g = lane >> 4;
  float* so = a.s_out + bh * (int64_t)n * DV;
#pragma unroll
  for (int u = 0; u < NU_W; ++u)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int tt = (UB + 2 * u) / 2, qa = 4 * (UB % 2) + g, c = j;
      const int r = tile_xor(tt, qa);
      const int fa = 4 * qa + c, fb = 4 * tile_partner(tt, qa) + (c ^ r);
      if (tile_doubled(tt) && c > (c ^ r)) continue;  // the other copy of this pair
      const int i0 = fa < fb ? fa : fb, j0 = fa < fb ? fb : fa;
      const int f = i0 * P - i0 * (i0 - 1) / 2 + (j0 - i0);
      const float sc = (tt == 0 ? 1.f : 0.70710678118654752f) * inv_sig;
#pragma unroll
      for (int dv = 0; dv < DV / 16; ++dv) so[(int64_t)f * DV + 16 * dv + col] = S[u][dv][j] * sc;
    }
}
__device__ __forceinline__ void write_final_z(const Args& a, int64_t bh, const acc4_t (&Mg)[4]) {
  constexpr int n = P * (P + 1) / 2;
  const int lane = threadIdx.x & 63, col16 = lane & 15, g = lane >> 4;
  float* zo = a.z_out + bh * (int64_t)n;
#pragma unroll
  for (int ab = 0; ab < 4; ++ab)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = 16 * (ab >> 1) + 4 * g + j, col = 16 * (ab & 1) + col16;
      if (row > col) continue;
      const int f = row * P - row * (row - 1) / 2 + (col - row);
      zo[f] = Mg[ab][j] * (row == col ? 1.f : 1.41421356237309515f);
    }
}

// ---- readout wave: token group G, tiles [TB, TE); OWNER also runs the intra block, the
// denominator and the output; wave 0 also accumulates the Gram blocks of the denominator
template <int DV, int C, int W, bool S2 = false>
struct Reader {
  using L = Lay<DV, C, S2>;
  static constexpr int NDT = L::NDT;
  static constexpr int G = W / L::FS, F = W % L::FS;
  static constexpr int TB = L::rb(F), TE = L::rb(F + 1);
  static constexpr bool OWNER = F == L::FS - 1;
  static constexpr bool GRAM = W == 0;

  // psi'(q) slots of quad a (lower-half view) for tile T: (c0, c1) and (c2, c3); S2: the
  // sum of both blocks' products (second block in R[16..31])
  template <int T, int A>
  __device__ static __forceinline__ void quad_slots(const h2_t (&R)[S2 ? 32 : 16], h2_t& p01, h2_t& p23) {
    constexpr int B = tile_partner(T, A), r = tile_xor(T, A);
    const h2_t x01 = R[2 * B + (r >> 1)], x23 = R[2 * B + 1 - (r >> 1)];
    p01 = R[2 * A] * ((r & 1) ? swp(x01) : x01);
    p23 = R[2 * A + 1] * ((r & 1) ? swp(x23) : x23);
    if constexpr (S2) {
      const h2_t y01 = R[16 + 2 * B + (r >> 1)], y23 = R[16 + 2 * B + 1 - (r >> 1)];
      p01 = R[16 + 2 * A] * ((r & 1) ? swp(y01) : y01) + p01;
      p23 = R[16 + 2 * A + 1] * ((r & 1) ? swp(y23) : y23) + p23;
    }
  }

  __device__ static __forceinline__ void run(const Args& a, char* lds) {
    const int lane = threadIdx.x & 63, t_lane = lane & 31, h_lane = lane >> 5;
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
    const uint32_t* red = reinterpret_cast<const uint32_t*>(lds + L::OFF_RED);

    acc4_t Mg[4] = {zero4a(), zero4a(), zero4a(), zero4a()};
    if constexpr (GRAM) {
      if (seg > 0) {
        const float* p = a.ws + (bh * (a.nseg - 1) + (seg - 1)) * L::STATE_FLOATS + (int64_t)NU * L::NDV * 256 + lane * 4;
#pragma unroll
        for (int ab = 0; ab < 4; ++ab) {
          const f32x4_t x = *reinterpret_cast<const f32x4_t*>(p + ab * 256);
          Mg[ab] = acc4_t{x[0], x[1], x[2], x[3]};
        }
      }
    }
    QStage<DV, C, 64 * L::FS, S2> qs;
    qs.init(a.q, row0, rstep, Tb);
    const int qtid = F * 64 + lane;
    if (c0 < c1) qs.load(c0 * C, 32 * G, qtid);
    __syncthreads();  // prologue 1: prefix maxima and the first chunk's value maximum published
    // every wave follows the same bound and scale: beta >= max |S| over the state so far
    float beta;
    int e_sig;
    {
      uint32_t pm = 0, vb = 0;
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        pm = max(pm, red[w]);
        vb = max(vb, red[8 + 8 * (c0 & 1) + w]);
      }
      beta = __uint_as_float(pm) + (float)C * __uint_as_float(vb << 16);
      e_sig = scale_exp(beta, 100);
    }
    if (c0 < c1) {
      if (c0 == 0) qs.template store<true>(lds, L::offq(0), 32 * G, qtid);
      else qs.template store<false>(lds, L::offq(0), 32 * G, qtid);
      if constexpr (L::NBUF == 2)
        if (c0 + 1 < c1) qs.load((c0 + 1) * C, 32 * G, qtid);
      if constexpr (GRAM)
        if (c0 > 0) write_gram<DV, C, S2>(Mg, lds, gram_exp(c0 * C));
    }
    __syncthreads();  // prologue 2: chunk c0 staged, state before it in LDS

    for (int c = c0; c < c1; ++c) {
      const int t0 = c * C, buf = (c - c0) & 1;
      // token row t of the group and lane half h (S2: opaque per chunk, so that the many
      // operand addresses derived from them are formed in the chunk, not held across it)
      int t = t_lane, h = h_lane;
      if constexpr (S2) asm volatile("" : "+v"(t), "+v"(h));
      // this lane's state fragment: readout lane (value row t, half h) reads quads h and h + 2
      // of build tile u, value tile 2 dt + t / 16, as one 16-byte piece
      const uint32_t fbase = (uint32_t)((t >> 4) * 512 + h * 256 + (t & 15) * 16);
      // ---- phase 1: queries of chunk c + 1 into the other buffer (loaded during the previous
      // chunk), readout of chunk c, loads of chunk c + 2 (single buffer: both in phase 2)
      if constexpr (L::NBUF == 2)
        if (c + 1 < c1) qs.template store<false>(lds, L::offq(buf ^ 1), 32 * G, qtid);
      h2_t R[S2 ? 32 : 16];
      {
        const char* qrow = lds + L::offq(buf) + (32 * G + t) * L::QPB;
#pragma unroll
        for (int blk = 0; blk < (S2 ? 2 : 1); ++blk)
#pragma unroll
          for (int b = 0; b < 8; ++b) {
            const h4_t x = ld4(qrow + 64 * blk + 8 * ((b + h) & 7));
            R[16 * blk + 2 * b] = lo2(x);
            R[16 * blk + 2 * b + 1] = hi2(x);
          }
      }
      acc_t O[NDT];
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) O[dt] = zero_acc();
      if (c > 0) {
        constexpr int NP = 2 * (TE - TB);
        auto frag = [&](int T, int s, int dt) -> h8_t {
          return ld8(lds + fbase + (uint32_t)(((2 * T + s) * L::NDV + 2 * dt) * 512));
        };
        h8_t fr[2][NDT];
        if constexpr (NP > 0) {
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) fr[0][dt] = frag(TB, 0, dt);
        }
        [&]<int... PI>(std::integer_sequence<int, PI...>) {
          (([&] {
             constexpr int T = TB + PI / 2, s = PI % 2;
             if constexpr (PI + 1 < NP) {
#pragma unroll
               for (int dt = 0; dt < NDT; ++dt) fr[(PI + 1) & 1][dt] = frag(TB + (PI + 1) / 2, (PI + 1) % 2, dt);
             }
             // keep the next fragments' reads ahead of this step's work
             __builtin_amdgcn_sched_barrier(0);
             h2_t p0, p1, p2, p3;
             quad_slots<T, 4 * s>(R, p0, p1);
             quad_slots<T, 4 * s + 2>(R, p2, p3);
             const h8_t psi = cat4(p0, p1, p2, p3);
#pragma unroll
             for (int dt = 0; dt < NDT; ++dt) O[dt] = mfma(fr[PI & 1][dt], psi, O[dt]);
           }()),
           ...);
        }(std::make_integer_sequence<int, NP>{});
      }
      if constexpr (GRAM) gram_chunk<DV, C, S2>(Mg, lds, L::offkt(buf));
      float den = 0.f;
      if constexpr (OWNER) {
        // query operand of the component contractions: k-slots 16s + 8(e/4) + 4h + e%4 of
        // block blk (S2: two blocks)
        constexpr int NB = S2 ? 2 : 1;
        h8_t qop[NB][2];
        if constexpr (S2) {  // read again from the query rows: R is not kept past the readout
          const char* qrow = lds + L::offq(buf) + (32 * G + t) * L::QPB;
#pragma unroll
          for (int blk = 0; blk < NB; ++blk)
#pragma unroll
            for (int s = 0; s < 2; ++s)
              qop[blk][s] = cat44(ld4(qrow + 64 * blk + 8 * (4 * s + h)), ld4(qrow + 64 * blk + 8 * (4 * s + 2 + h)));
        } else {
          qop[0][0] = cat4(R[0], R[1], R[4], R[5]);
          qop[0][1] = cat4(R[8], R[9], R[12], R[13]);
        }
        if (c > 0) {  // denominator, inter-chunk part: X = (M 2^-ge) Q^T, then q . X (per block)
          float dx = 0.f;
#pragma unroll
          for (int blk = 0; blk < NB; ++blk) {
            acc_t X = zero_acc();
#pragma unroll
            for (int s = 0; s < 2; ++s) {
              const char* mrow = lds + L::OFF_M + t * L::MPB + 2 * (16 * s + 8 * h);
              X = mfma(ld8(mrow), qop[blk][s], X);
              X = mfma(ld8(mrow + 32 * L::MPB), qop[blk][s], X);
            }
#pragma unroll
            for (int ii = 0; ii < 4; ++ii)
#pragma unroll
              for (int j = 0; j < 4; ++j)
                dx += X[4 * ii + j] * (S2 ? (float)qop[blk][ii >> 1][4 * (ii & 1) + j] : (float)R[16 * blk + 4 * ii + j / 2][j & 1]);
          }
          den = dx * pow2f(gram_exp(t0));
        }
        // intra-chunk block over key groups 0..G
        auto intra = [&]<bool SPLIT>() {
          h8_t qlo[NB][2];
          if constexpr (SPLIT) {
            const char* lrow = lds + L::OFF_QLO + (32 * G + t) * L::QPB;
#pragma unroll
            for (int blk = 0; blk < NB; ++blk)
#pragma unroll
              for (int s = 0; s < 2; ++s)
                qlo[blk][s] = cat44(ld4(lrow + 64 * blk + 8 * (4 * s + h)), ld4(lrow + 64 * blk + 8 * (4 * s + 2 + h)));
          }
#pragma unroll
          for (int kg = 0; kg <= G; ++kg) {
            const char* krow = lds + L::offkr(buf);
            const int kr = 32 * kg + t;
            // scores of the block pairs (query block qa, key block kb); S2: the weight sums
            // the squares of all four (sq)
            auto score = [&](int qa, int kb) {
              // S2: one block pair's operand reads at a time (hoisted over all pairs and key
              // groups they would not fit the registers)
              if constexpr (S2) __builtin_amdgcn_sched_barrier(0);
              acc_t Sc = zero_acc();
#pragma unroll
              for (int s = 0; s < 2; ++s) {
                const h8_t kop = cat44(ld4(krow + L::krpos(kr, 8 * kb + 4 * s + h)), ld4(krow + L::krpos(kr, 8 * kb + 4 * s + 2 + h)));
                Sc = mfma(kop, qop[qa][s], Sc);
                if constexpr (SPLIT) {
                  const char* lrow = lds + L::OFF_KLO;
                  Sc = mfma(cat44(ld4(lrow + L::krpos(kr, 8 * kb + 4 * s + h)), ld4(lrow + L::krpos(kr, 8 * kb + 4 * s + 2 + h))),
                            qop[qa][s], Sc);
                  Sc = mfma(kop, qlo[qa][s], Sc);
                }
              }
              return Sc;
            };
            const acc_t Sc = score(0, 0);
            float sq[S2 ? 16 : 1];
            if constexpr (S2) {
#pragma unroll
              for (int e = 0; e < 16; ++e) sq[e] = Sc[e] * Sc[e];
#pragma unroll
              for (int pr = 1; pr < 4; ++pr) {
                const acc_t Sp = score(pr >> 1, pr & 1);
#pragma unroll
                for (int e = 0; e < 16; ++e) sq[e] += Sp[e] * Sp[e];
              }
            }
            // weights: keys 8ii + 4h + j of group kg for query t; causal on the diagonal group
            h2_t wv[8];
#pragma unroll
            for (int ii = 0; ii < 4; ++ii)
#pragma unroll
              for (int j = 0; j < 4; j += 2) {
                float w0 = S2 ? sq[(4 * ii + j) % (S2 ? 16 : 1)] : Sc[4 * ii + j] * Sc[4 * ii + j];
                float w1 = S2 ? sq[(4 * ii + j + 1) % (S2 ? 16 : 1)] : Sc[4 * ii + j + 1] * Sc[4 * ii + j + 1];
                if (kg == G) {
                  if (8 * ii + 4 * h + j > t) w0 = 0.f;
                  if (8 * ii + 4 * h + j + 1 > t) w1 = 0.f;
                }
                wv[2 * ii + j / 2] = cvt2(w0, w1);
                den += w0 + w1;
              }
#pragma unroll
            for (int s = 0; s < 2; ++s) {
              const h8_t wop = cat4(wv[4 * s], wv[4 * s + 1], wv[4 * s + 2], wv[4 * s + 3]);
#pragma unroll
              for (int dt = 0; dt < NDT; ++dt) {
                // keys 16s + 4h + j, 16s + 8 + 4h + j sit at positions 16s + 8h .. + 7
                const h8_t vfr = ld8(lds + L::offvt(buf) + L::tpos(32 * dt + t, 32 * kg + 16 * s + 8 * h));
                O[dt] = mfma(vfr, wop, O[dt]);
              }
            }
          }
        };
        if (c == 0) intra.template operator()<true>();
        else intra.template operator()<false>();
        den = xor32_sum(den);
      }
      if constexpr (L::NBUF == 2) {
        if (c + 2 < c1) qs.load(t0 + 2 * C, 32 * G, qtid);
      } else {  // single buffer: chunk c + 1's queries, staged after the barrier
        if (c + 1 < c1) qs.load(t0 + C, 32 * G, qtid);
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
        uint32_t vb = 0;
#pragma unroll
        for (int w = 0; w < 8; ++w) vb = max(vb, red[8 + 8 * ((c + 1) & 1) + w]);
        beta += (float)C * __uint_as_float(vb << 16);
        e_sig = scale_exp(beta, e_sig);
        if constexpr (GRAM) write_gram<DV, C, S2>(Mg, lds, gram_exp(t0 + C));
      }
      if constexpr (L::NBUF == 1)  // queries of chunk c + 1 (every wave is past chunk c's)
        if (c + 1 < c1) qs.template store<false>(lds, L::offq(0), 32 * G, qtid);
      __syncthreads();
    }
    if constexpr (GRAM)
      if (a.z_out != nullptr && seg == a.nblk_per_bh - 1) write_final_z(a, bh, Mg);
  }
};

// ---- build wave j of the forward (tiles Fwd8::ub(j) .. ub(j + 1)), which also stages the
// keys and values of the next chunk
template <int DV, int C, int J, bool S2 = false>
struct Builder {
  using L = Lay<DV, C, S2>;
  static constexpr int NDV = L::NDV;
  static constexpr int UB = Fwd8::first(J), NU_W = Fwd8::cnt(J);

  __device__ static __forceinline__ void run(const Args& a, char* lds) {
    const int lane = threadIdx.x & 63;
    const int btid = J * 64 + lane;  // 0..511 over the build waves
    const int64_t bh = blockIdx.x / a.nblk_per_bh;
    const int seg = blockIdx.x % a.nblk_per_bh;
    int64_t row0;
    int rstep, Tb;
    seq_rows_of(a.lay, bh, a.H, a.T, row0, rstep, Tb);
    const int nchunks = (Tb + C - 1) / C;
    const int c0 = seg * a.cps, c1 = min(nchunks, c0 + a.cps);
    uint32_t* red = reinterpret_cast<uint32_t*>(lds + L::OFF_RED);

    acc4_t S[NU_W][NDV];
#pragma unroll
    for (int u = 0; u < NU_W; ++u)
#pragma unroll
      for (int dv = 0; dv < NDV; ++dv) S[u][dv] = zero4a();
    float pmax = 0.f;
    if (seg > 0) {  // exclusive prefix of this segment (true units)
      const float* src = a.ws + (bh * (a.nseg - 1) + (seg - 1)) * L::STATE_FLOATS;
#pragma unroll
      for (int u = 0; u < NU_W; ++u)
#pragma unroll
        for (int dv = 0; dv < NDV; ++dv) {
          const f32x4_t x = *reinterpret_cast<const f32x4_t*>(src + (((UB + 2 * u) * NDV + dv) * 64 + lane) * 4);
          S[u][dv] = acc4_t{x[0], x[1], x[2], x[3]};
#pragma unroll
          for (int e = 0; e < 4; ++e) pmax = fmaxf(pmax, fabsf(x[e]));
        }
    }
    KVStage<DV, C, 512, S2> kv;
    kv.init(a.k, a.v, row0, rstep, Tb);
    if (c0 < c1) kv.load(c0 * C, btid);
    auto publish = [&](int chunk) {  // max |v| of the loaded chunk, slot set chunk & 1
      const uint32_t vm = wave_max_u32(kv.vmax_bits(btid));
      if (lane == 0) red[8 + 8 * (chunk & 1) + J] = vm;
    };
    auto target = [&](int b, int klo) { return KVTarget{L::offkr(b), L::offkt(b), -1, L::offvt(b), klo}; };
    {
      const uint32_t pm = wave_max_u32(__float_as_uint(pmax));
      const uint32_t vm = wave_max_u32(c0 < c1 ? kv.vmax_bits(btid) : 0u);
      if (lane == 0) {
        red[J] = pm;
        red[8 + 8 * (c0 & 1) + J] = vm;
      }
    }
    __syncthreads();  // prologue 1
    float beta;
    int e_sig;
    {
      uint32_t pm = 0, vb = 0;
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        pm = max(pm, red[w]);
        vb = max(vb, red[8 + 8 * (c0 & 1) + w]);
      }
      beta = __uint_as_float(pm) + (float)C * __uint_as_float(vb << 16);
      e_sig = scale_exp(beta, 100);
    }
    if (seg > 0) {
      const float sg = pow2f(e_sig);
#pragma unroll
      for (int u = 0; u < NU_W; ++u)
#pragma unroll
        for (int dv = 0; dv < NDV; ++dv) S[u][dv] *= sg;
    }
    if (c0 < c1) {
      if (c0 == 0) {
        kv.template store<true>(lds, target(0, L::OFF_KLO), pow2f(e_sig), btid);
      } else {
        kv.template store<false>(lds, target(0, 0), pow2f(e_sig), btid);
        write_state<DV, C, NU_W, UB>(S, lds);
      }
      if (c0 + 1 < c1) {
        kv.load((c0 + 1) * C, btid);
        publish(c0 + 1);
      }
    }
    __syncthreads();  // prologue 2

    if constexpr (L::NBUF == 1) {
      // single buffer: phase 1 = value maximum of chunk c + 1 (in registers since phase 2 of
      // chunk c - 1; chunk c0 + 1's went out in the prologue), build of chunk c | barrier |
      // phase 2 = state after chunk c (scaled for c + 1), keys and values of c + 1, loads of
      // c + 2 | barrier
      for (int c = c0; c < c1; ++c) {
        if (c > c0 && c + 1 < c1) publish(c + 1);
        build_chunk<DV, C, NU_W, UB, true, S2>(S, lds, L::offkt(0), L::offvt(0));
        __syncthreads();
        if (c + 1 < c1) {
          uint32_t vb = 0;
#pragma unroll
          for (int w = 0; w < 8; ++w) vb = max(vb, red[8 + 8 * ((c + 1) & 1) + w]);
          beta += (float)C * __uint_as_float(vb << 16);
          const int e_next = scale_exp(beta, e_sig);
          if (e_next != e_sig) {
            const float f = pow2f(e_next - e_sig);
#pragma unroll
            for (int u = 0; u < NU_W; ++u)
#pragma unroll
              for (int dv = 0; dv < NDV; ++dv) S[u][dv] *= f;
            e_sig = e_next;
          }
          write_state<DV, C, NU_W, UB>(S, lds);
          kv.template store<false>(lds, target(0, 0), pow2f(e_sig), btid);
          if (c + 2 < c1) kv.load((c + 2) * C, btid);
        }
        __syncthreads();
      }
    } else
    for (int c = c0; c < c1; ++c) {
      const int buf = (c - c0) & 1;
      // ---- phase 1: keys and values of chunk c + 1 into the other buffers (scaled for chunk
      // c + 1; loaded during the previous chunk), build of chunk c, loads of chunk c + 2
      int e_next = e_sig;
      if (c + 1 < c1) {
        uint32_t vb = 0;
#pragma unroll
        for (int w = 0; w < 8; ++w) vb = max(vb, red[8 + 8 * ((c + 1) & 1) + w]);
        beta += (float)C * __uint_as_float(vb << 16);
        e_next = scale_exp(beta, e_sig);
        kv.template store<false>(lds, target(buf ^ 1, 0), pow2f(e_next), btid);
      }
      build_chunk<DV, C, NU_W, UB, true>(S, lds, L::offkt(buf), L::offvt(buf));
      if (c + 2 < c1) kv.load((c + 2) * C, btid);
      __syncthreads();
      // ---- phase 2: state after chunk c, scaled for chunk c + 1, to LDS; value maximum of
      // chunk c + 2 (read by every wave after the next barrier)
      if (c + 2 < c1) publish(c + 2);
      if (c + 1 < c1) {
        if (e_next != e_sig) {
          const float f = pow2f(e_next - e_sig);
#pragma unroll
          for (int u = 0; u < NU_W; ++u)
#pragma unroll
            for (int dv = 0; dv < NDV; ++dv) S[u][dv] *= f;
          e_sig = e_next;
        }
        write_state<DV, C, NU_W, UB>(S, lds);
      }
      __syncthreads();
    }
    if (a.s_out != nullptr && seg == a.nblk_per_bh - 1) write_final_s<DV, NU_W, UB>(a, bh, S, pow2f(-e_sig));
  }
};

// ---- summary pass: [S | M] of one segment after its chunks, written in true units. Waves
// 0-3, one per SIMD, load and stage the keys and values of the next chunk into the other half
// of a double buffer, so their conversion work runs beside the build MFMAs; they are the
// oldest waves of their SIMDs, whose instructions win the issue arbitration, so the staging
// is not left waiting behind the builds. Waves 4-11 build (tiles of Fwd8, one build pair per
// SIMD) and wave 4 also forms the Gram matrix. One barrier per chunk.
template <int DV, int C, int J, bool S2 = false>
__device__ __forceinline__ void run_summary(const Args& a, char* lds) {
  using L = Lay<DV, C, S2>;
  constexpr int NDV = L::NDV;
  constexpr bool STAGER = J < 4;
  constexpr int JB = STAGER ? 0 : J - 4;
  constexpr int UB = Fwd8::first(JB), NU_W = STAGER ? 1 : Fwd8::cnt(JB);
  constexpr bool GRAM = J == 4;
  const int lane = threadIdx.x & 63;
  const int stid = J * 64 + lane;  // 0..255 over the staging waves
  const int64_t bh = blockIdx.x / a.nblk_per_bh;
  const int seg = blockIdx.x % a.nblk_per_bh;
  int64_t row0;
  int rstep, Tb;
  seq_rows_of(a.lay, bh, a.H, a.T, row0, rstep, Tb);
  const int nchunks = (Tb + C - 1) / C;
  const int c0 = seg * a.cps, c1 = min(nchunks, c0 + a.cps);
  uint32_t* red = reinterpret_cast<uint32_t*>(lds + L::SUM_RED);  // [2 parities][4 staging waves]

  KVStage<DV, C, 256, S2> kv;
  auto publish = [&](int chunk) {  // max |v| of the loaded chunk into slot set chunk & 1
    const uint32_t vm = wave_max_u32(kv.vmax_bits(stid));
    if (lane == 0) red[4 * (chunk & 1) + J] = vm;
  };
  auto vmax_of = [&](int chunk) {
    const uint32_t* r = red + 4 * (chunk & 1);
    const uint32_t m = max(max(r[0], r[1]), max(r[2], r[3]));
    return __uint_as_float(m << 16);
  };
  auto target = [&](int buf) {
    const int b = buf * L::SUM_BUF;
    return KVTarget{-1, b, -1, b + L::PC * L::RPB, 0};
  };
  if constexpr (STAGER) {
    kv.init(a.k, a.v, row0, rstep, Tb);
    if (c0 < c1) {
      kv.load(c0 * C, stid);
      publish(c0);
    }
  }
  __syncthreads();
  float beta = 0.f;
  int e_sig = 100;
  if (c0 < c1) {
    beta = (float)C * vmax_of(c0);
    e_sig = scale_exp(beta, e_sig);
    if constexpr (STAGER) {
      kv.template store<false>(lds, target(0), pow2f(e_sig), stid);
      if (c0 + 1 < c1) {
        kv.load((c0 + 1) * C, stid);
        publish(c0 + 1);
      }
    }
  }
  __syncthreads();
  if constexpr (STAGER) {
    for (int c = c0; c < c1; ++c) {
      if (c + 1 < c1) {
        beta += (float)C * vmax_of(c + 1);
        e_sig = scale_exp(beta, e_sig);
        kv.template store<false>(lds, target((c - c0 + 1) & 1), pow2f(e_sig), stid);
        if (c + 2 < c1) {
          kv.load((c + 2) * C, stid);
          publish(c + 2);
        }
      }
      __syncthreads();
    }
  } else {
    acc4_t S[NU_W][NDV];
#pragma unroll
    for (int u = 0; u < NU_W; ++u)
#pragma unroll
      for (int dv = 0; dv < NDV; ++dv) S[u][dv] = zero4a();
    acc4_t Mg[4] = {zero4a(), zero4a(), zero4a(), zero4a()};
    for (int c = c0; c < c1; ++c) {
      const KVTarget tg = target((c - c0) & 1);
      build_chunk<DV, C, NU_W, UB, false, S2>(S, lds, tg.kt, tg.vt);
      if constexpr (GRAM) gram_chunk<DV, C, S2>(Mg, lds, tg.kt);
      if (c + 1 < c1) {
        beta += (float)C * vmax_of(c + 1);
        const int e_new = scale_exp(beta, e_sig);
        if (e_new != e_sig) {
          const float f = pow2f(e_new - e_sig);
#pragma unroll
          for (int u = 0; u < NU_W; ++u)
#pragma unroll
            for (int dv = 0; dv < NDV; ++dv) S[u][dv] *= f;
          e_sig = e_new;
        }
      }
      __syncthreads();
    }
    float* dst = a.ws + (bh * (a.nseg - 1) + seg) * L::STATE_FLOATS;
    // summaries are in the forward's accumulator units: tiles 1-17 carry the factor 2 that
    // the forward's doubled partner copy supplies
    const float inv = pow2f(-e_sig);
#pragma unroll
    for (int u = 0; u < NU_W; ++u) {
      const float f = (UB + 2 * u) / 2 == 0 ? inv : 2.f * inv;
#pragma unroll
      for (int dv = 0; dv < NDV; ++dv)
        *reinterpret_cast<f32x4_t*>(dst + (((UB + 2 * u) * NDV + dv) * 64 + lane) * 4) =
            f32x4_t{S[u][dv][0] * f, S[u][dv][1] * f, S[u][dv][2] * f, S[u][dv][3] * f};
    }
    if constexpr (GRAM) {
      float* p = dst + (int64_t)NU * NDV * 256 + lane * 4;
#pragma unroll
      for (int ab = 0; ab < 4; ++ab)
        *reinterpret_cast<f32x4_t*>(p + ab * 256) = f32x4_t{Mg[ab][0], Mg[ab][1], Mg[ab][2], Mg[ab][3]};
    }
  }
}

template <int DV, int C, bool S2 = false>
__global__ __launch_bounds__(768, 1) void summary_f16_kernel(Args a) {
  extern __shared__ __align__(16) char lds[];
  switch (threadIdx.x >> 6) {
    case 0: run_summary<DV, C, 0, S2>(a, lds); break;
    case 1: run_summary<DV, C, 1, S2>(a, lds); break;
    case 2: run_summary<DV, C, 2, S2>(a, lds); break;
    case 3: run_summary<DV, C, 3, S2>(a, lds); break;
    case 4: run_summary<DV, C, 4, S2>(a, lds); break;
    case 5: run_summary<DV, C, 5, S2>(a, lds); break;
    case 6: run_summary<DV, C, 6, S2>(a, lds); break;
    case 7: run_summary<DV, C, 7, S2>(a, lds); break;
    case 8: run_summary<DV, C, 8, S2>(a, lds); break;
    case 9: run_summary<DV, C, 9, S2>(a, lds); break;
    case 10: run_summary<DV, C, 10, S2>(a, lds); break;
    default: run_summary<DV, C, 11, S2>(a, lds); break;
  }
}

template <int DV, int C, bool S2 = false>
__global__ __launch_bounds__(768, 1) void chunked_f16_kernel(Args a) {
  extern __shared__ __align__(16) char lds[];
  switch (threadIdx.x >> 6) {
    case 0: Reader<DV, C, 0, S2>::run(a, lds); break;
    case 1: Reader<DV, C, 1, S2>::run(a, lds); break;
    case 2: Reader<DV, C, 2, S2>::run(a, lds); break;
    case 3: Reader<DV, C, 3, S2>::run(a, lds); break;
    case 4: Builder<DV, C, 0, S2>::run(a, lds); break;
    case 5: Builder<DV, C, 1, S2>::run(a, lds); break;
    case 6: Builder<DV, C, 2, S2>::run(a, lds); break;
    case 7: Builder<DV, C, 3, S2>::run(a, lds); break;
    case 8: Builder<DV, C, 4, S2>::run(a, lds); break;
    case 9: Builder<DV, C, 5, S2>::run(a, lds); break;
    case 10: Builder<DV, C, 6, S2>::run(a, lds); break;
    default: Builder<DV, C, 7, S2>::run(a, lds); break;
  }
}

}  // namespace c16

namespace c16 {

template <int DV, int C, bool S2 = false>
hipError_t launch(const uint16_t* q, const uint16_t* k, const uint16_t* v, void* o, bool o_bf16, int B, int H, int T,
                  const SegPlan& plan, float* ws, float* s_out, float* z_out, SeqLayout lay, int passes,
                  hipStream_t st) {
  using L = Lay<DV, C, S2>;
  const int BH = B * H;
  Args a{q, k, v, o, ws, T, plan.nseg, plan.cps, 0, o_bf16 ? 0 : 1, s_out, z_out, lay, H};
  hipError_t e;
  if (plan.nseg > 1 && (passes & PASS_SUMMARIES)) {
    a.nblk_per_bh = plan.nseg - 1;
    auto ks = summary_f16_kernel<DV, C, S2>;
    if ((e = hipFuncSetAttribute((const void*)ks, hipFuncAttributeMaxDynamicSharedMemorySize, L::SUM_LDS)) != hipSuccess)
      return e;
    ks<<<dim3((unsigned)(BH * (plan.nseg - 1))), dim3(768), L::SUM_LDS, st>>>(a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (plan.nseg > 1 && (passes & PASS_SCAN))
    if ((e = launch_scan(ws, BH, plan.nseg - 1, L::STATE_FLOATS, st)) != hipSuccess) return e;
  if (!(passes & PASS_SEGMENTS)) return hipSuccess;
  auto kf = chunked_f16_kernel<DV, C, S2>;
  if ((e = hipFuncSetAttribute((const void*)kf, hipFuncAttributeMaxDynamicSharedMemorySize, L::LDS)) != hipSuccess) return e;
  a.nblk_per_bh = plan.nseg;
  kf<<<dim3((unsigned)(BH * plan.nseg)), dim3(768), L::LDS, st>>>(a);
  return hipGetLastError();
}

}  // namespace c16
}  // namespace kata
