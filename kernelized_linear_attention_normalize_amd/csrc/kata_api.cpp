// C ABI of the KATA library: argument validation (host only, before any HIP call),
// dtype/shape dispatch, workspace sizing and kernel launches on the caller's stream.
// The entry points are declared, with their contracts, in include/kata.h.
#include "kata.h"

#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>
#include <utility>

#include "kata_launch.h"

namespace {

constexpr int64_t kMaxGrid = INT32_MAX;

bool valid_dt(kata_dtype_t d) { return d == KATA_DTYPE_F32 || d == KATA_DTYPE_BF16; }
size_t dt_size(kata_dtype_t d) { return d == KATA_DTYPE_F32 ? 4 : 2; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// [a, a+na) and [b, b+nb) share a byte
bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

bool in_set(int x, std::initializer_list<int> s) {
  for (int y : s)
    if (x == y) return true;
  return false;
}

// element count a*b*c*d without signed overflow, or -1
int64_t mul4(int64_t a, int64_t b, int64_t c, int64_t d) {
  const int64_t lim = INT64_MAX / 8;
  int64_t r = 1;
  for (int64_t x : {a, b, c, d}) {
    if (x != 0 && r > lim / x) return -1;
    r *= x;
  }
  return r;
}

kata_status_t hip_status(hipError_t e) { return e == hipSuccess ? KATA_OK : KATA_ERR_HIP; }

// (fam, g) valid for width p: KATA_OK or KATA_ERR_FEATURE
kata_status_t check_feature(int p, kata_feature_t fam, int g) {
  return kata_feature_dim(p, fam, g) > 0 ? KATA_OK : KATA_ERR_FEATURE;
}

}  // namespace

namespace kata {

SegPlan seg_plan(int B, int H, int T, int C, int scan) {
  SegPlan s;
  s.nchunks = (T + C - 1) / C;
  if (scan == KATA_SCAN_SEQUENTIAL || s.nchunks <= 1) {
    s.nseg = 1;
    s.cps = s.nchunks;
    return s;
  }
  // aim for about one workgroup per compute unit of a 256-CU part; at most 64 segments
  const int64_t BH = (int64_t)B * H;
  int64_t want = (256 + BH - 1) / BH;
  if (want > 64) want = 64;
  if (want > s.nchunks) want = s.nchunks;
  if (want < 1) want = 1;
  s.cps = (int)((s.nchunks + want - 1) / want);
  s.nseg = (s.nchunks + s.cps - 1) / s.cps;
  return s;
}

}  // namespace kata

extern "C" {

int64_t kata_packed_dim(int p) { return p < 1 ? -1 : (int64_t)p * (p + 1) / 2; }

int64_t kata_feature_dim(int p, kata_feature_t fam, int g) {
  if (p < 1 || g < 1 || p % g != 0) return -1;
  if (fam == KATA_FEAT_FULL) return g == 1 ? kata_packed_dim(p) : -1;
  if (fam != KATA_FEAT_SIGMA && fam != KATA_FEAT_BLOCK) return -1;
  const int64_t m = p / g, nb = m * (m + 1) / 2;
  return fam == KATA_FEAT_SIGMA ? nb : g * nb;
}

const char* kata_status_string(kata_status_t s) {
  switch (s) {
    case KATA_OK: return "KATA_OK";
    case KATA_ERR_NULL: return "KATA_ERR_NULL: a required pointer is NULL";
    case KATA_ERR_SHAPE: return "KATA_ERR_SHAPE: invalid or too large size";
    case KATA_ERR_DTYPE: return "KATA_ERR_DTYPE: invalid dtype";
    case KATA_ERR_UNSUPPORTED: return "KATA_ERR_UNSUPPORTED: unsupported p / dv / C combination";
    case KATA_ERR_ALIGN: return "KATA_ERR_ALIGN: pointer not 16-byte aligned";
    case KATA_ERR_ALIAS: return "KATA_ERR_ALIAS: output overlaps another buffer";
    case KATA_ERR_WORKSPACE: return "KATA_ERR_WORKSPACE: workspace missing or too small";
    case KATA_ERR_HIP: return "KATA_ERR_HIP: kernel launch failed";
    case KATA_ERR_SCAN: return "KATA_ERR_SCAN: invalid scan mode";
    case KATA_ERR_PASS: return "KATA_ERR_PASS: invalid pass mask";
    case KATA_ERR_FEATURE: return "KATA_ERR_FEATURE: invalid feature family or block count";
    case KATA_ERR_SCRATCH:
      return "KATA_ERR_SCRATCH: the call needs more workspace than the fixed no-allocation scratch holds";
  }
  return "KATA_ERR_UNKNOWN";
}

static kata_status_t lift_impl(const void* u, kata_dtype_t u_dt, int64_t rows, int p,
                               kata_feature_t fam, int g, void* psi, kata_dtype_t psi_dt,
                               kata_stream_t stream) {
  if (!valid_dt(u_dt) || !valid_dt(psi_dt)) return KATA_ERR_DTYPE;
  if (rows < 0 || p < 1) return KATA_ERR_SHAPE;
  kata_status_t s = check_feature(p, fam, g);
  if (s != KATA_OK) return s;
  if (p > 128) return KATA_ERR_UNSUPPORTED;
  if (rows == 0) return KATA_OK;
  const int64_t n = kata_feature_dim(p, fam, g);
  if (mul4(rows, n, 1, 1) < 0 || (rows + 15) / 16 > kMaxGrid) return KATA_ERR_SHAPE;
  if (!u || !psi) return KATA_ERR_NULL;
  if (!aligned16(u) || !aligned16(psi)) return KATA_ERR_ALIGN;
  if (overlap(u, rows * p * dt_size(u_dt), psi, rows * n * dt_size(psi_dt))) return KATA_ERR_ALIAS;
  if (fam != KATA_FEAT_FULL)
    return hip_status(kata::launch_family_lift(u, u_dt == KATA_DTYPE_BF16, rows, p, (int)fam, g, psi,
                                               psi_dt == KATA_DTYPE_BF16, (hipStream_t)stream));
  return hip_status(kata::launch_lift(u, u_dt == KATA_DTYPE_BF16, rows, p, psi,
                                      psi_dt == KATA_DTYPE_BF16, (hipStream_t)stream));
}

kata_status_t kata_lift(const void* u, kata_dtype_t u_dt, int64_t rows, int p, void* psi,
                        kata_dtype_t psi_dt, kata_stream_t stream) {
  return lift_impl(u, u_dt, rows, p, KATA_FEAT_FULL, 1, psi, psi_dt, stream);
}

kata_status_t kata_lift_family(const void* u, kata_dtype_t u_dt, int64_t rows, int p,
                               kata_feature_t fam, int g, void* psi, kata_dtype_t psi_dt,
                               kata_stream_t stream) {
  return lift_impl(u, u_dt, rows, p, fam, g, psi, psi_dt, stream);
}

// shared checks of the [B,H,T,*] forward entry points; returns KATA_OK to continue,
// or a status to return (zero_size set when the call is a no-op)
static kata_status_t check_fwd(const void* q, const void* k, const void* v, kata_dtype_t in_dt,
                               const void* o, kata_dtype_t o_dt, int B, int H, int T, int p,
                               int dv, bool& zero_size) {
  zero_size = false;
  if (!valid_dt(in_dt) || !valid_dt(o_dt)) return KATA_ERR_DTYPE;
  if (B < 0 || H < 0 || T < 0 || p < 1 || dv < 1) return KATA_ERR_SHAPE;
  if ((int64_t)B * H * T == 0) {
    zero_size = true;
    return KATA_OK;
  }
  if (mul4(B, H, T, p > dv ? p : dv) < 0) return KATA_ERR_SHAPE;
  // the kernels address one sequence with 32-bit byte offsets (4-byte elements at most)
  if ((int64_t)T * (p > dv ? p : dv) * 4 >= INT32_MAX) return KATA_ERR_SHAPE;
  if (!q || !k || !v || !o) return KATA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return KATA_ERR_ALIGN;
  return KATA_OK;
}

// rows: rows of q / k / v / o (B*H*T in the padded layout, total*H in the packed one)
static kata_status_t check_fwd_alias(const void* q, const void* k, const void* v,
                                     kata_dtype_t in_dt, const void* o, kata_dtype_t o_dt, size_t rows,
                                     int p, int dv) {
  const size_t qb = rows * p * dt_size(in_dt), vb = rows * dv * dt_size(in_dt);
  const size_t ob = rows * dv * dt_size(o_dt);
  if (overlap(o, ob, q, qb) || overlap(o, ob, k, qb) || overlap(o, ob, v, vb)) return KATA_ERR_ALIAS;
  return KATA_OK;
}

size_t kata_chunked_workspace_bytes(int B, int H, int T, int p, int dv, int C, kata_scan_t scan,
                                    kata_dtype_t in_dt) {
  if (!valid_dt(in_dt) || (scan != KATA_SCAN_SEQUENTIAL && scan != KATA_SCAN_ASSOCIATIVE)) return 0;
  if (B <= 0 || H <= 0 || T <= 0 || p < 1 || dv < 1 || C < 1) return 0;
  if (!in_set(p, {16, 32}) || !in_set(dv, {16, 32, 64}) || !in_set(C, {32, 64, 128})) return 0;
  const kata::SegPlan plan = kata::seg_plan(B, H, T, C, scan);
  if (plan.nseg <= 1) return 0;
  if (in_dt != KATA_DTYPE_BF16 && kata::f32_chunked_parts(p, dv, C) == 0) return 0;
  const int64_t sf = in_dt != KATA_DTYPE_BF16            ? kata::f32_chunked_state_floats(p, dv, C)
                     : kata::chunked_f16_supported(p, dv, C) ? kata::f16_state_floats(dv)
                                                             : kata::mfma_state_floats(p, dv);
  return (size_t)B * H * (plan.nseg - 1) * sf * sizeof(float);
}

// kata_chunked_fwd_passes, plus the final state when S and Z are given (want_state)
// KATA-Sigma 2 at p = 64 with bf16 inputs runs on MFMA kernels: the fp16-operand kernels with
// the two-block lift at dv = 64 (sigma2_f16), else the bf16 kernels over 2T virtual rows
static bool sigma2_mfma(int p, int dv, int C, kata_dtype_t in_dt, kata_feature_t fam, int g) {
  return fam == KATA_FEAT_SIGMA && g == 2 && p == 64 && in_dt == KATA_DTYPE_BF16 && in_set(dv, {32, 64}) &&
         in_set(C, {64, 128});
}
static bool sigma2_f16(int p, int dv, int C, kata_dtype_t in_dt, kata_feature_t fam, int g) {
  return sigma2_mfma(p, dv, C, in_dt, fam, g) && kata::chunked_f16_s2_supported(dv, C);
}

// the chunked forward's supported (p, dv, C) for a family and input dtype
// (packed: the packed token-major layout, which the Sigma 2 virtual-row kernels do not take)
static bool chunked_supported(int p, int dv, int C, kata_dtype_t in_dt, kata_feature_t fam, int g,
                              bool packed = false) {
  if (!in_set(C, {32, 64, 128})) return false;
  if (sigma2_f16(p, dv, C, in_dt, fam, g)) return true;  // padded, ragged or packed
  if (!packed && sigma2_mfma(p, dv, C, in_dt, fam, g)) return true;
  if (fam == KATA_FEAT_FULL) {
    if (!in_set(p, {16, 32}) || !in_set(dv, {16, 32, 64})) return false;
    return in_dt == KATA_DTYPE_BF16 || kata::f32_chunked_parts(p, dv, C) > 0;
  }
  return p <= 64 && dv <= 64 && kata::family_chunked_lds_bytes(p, dv, C, (int)fam, g) <= 160 * 1024;
}

// kata_chunked_fwd_passes for any family, plus the final state when S and Z are given
// (want_state)
static kata_status_t chunked_impl(const void* q, const void* k, const void* v, kata_dtype_t in_dt,
                                  void* o, kata_dtype_t o_dt, int B, int H, int T, int p, int dv,
                                  int C, kata_scan_t scan, kata_feature_t fam, int g,
                                  void* workspace, size_t workspace_bytes, int passes,
                                  bool want_state, float* S, float* Z, const int32_t* lens,
                                  const int32_t* cu, int total, kata_stream_t stream,
                                  bool use_scratch = false) {
  if (scan != KATA_SCAN_SEQUENTIAL && scan != KATA_SCAN_ASSOCIATIVE) return KATA_ERR_SCAN;
  if (passes < 1 || passes > KATA_PASS_ALL) return KATA_ERR_PASS;
  if (C < 1) return KATA_ERR_SHAPE;
  bool zero = false;
  kata_status_t s = check_fwd(q, k, v, in_dt, o, o_dt, B, H, T, p, dv, zero);
  if (s != KATA_OK) return s;
  if ((s = check_feature(p, fam, g)) != KATA_OK) return s;
  if (fam != KATA_FEAT_FULL && passes != KATA_PASS_ALL) return KATA_ERR_PASS;
  const bool packed = cu != nullptr;
  // rows of q / k / v / o
  const size_t rows = packed ? (size_t)total * H : (size_t)B * H * T;
  if (packed && !zero && total == 0) zero = true;
  if (want_state) {
    if ((int64_t)B * H == 0) return KATA_OK;
    if (!chunked_supported(p, dv, C, in_dt, fam, g, packed)) return KATA_ERR_UNSUPPORTED;
    if (!S || !Z) return KATA_ERR_NULL;
    if (!aligned16(S) || !aligned16(Z)) return KATA_ERR_ALIGN;
    const int64_t n = kata_feature_dim(p, fam, g);
    if (mul4(B, H, n, dv) < 0) return KATA_ERR_SHAPE;
    const size_t Sb = (size_t)B * H * n * dv * 4, Zb = (size_t)B * H * n * 4;
    if (overlap(S, Sb, Z, Zb)) return KATA_ERR_ALIAS;
    if (T == 0 || rows == 0) {  // empty sequences: the zero state
      hipStream_t st = (hipStream_t)stream;
      hipError_t e = kata::launch_fill_zero(S, (int64_t)B * H * n * dv, st);
      if (e == hipSuccess) e = kata::launch_fill_zero(Z, (int64_t)B * H * n, st);
      return hip_status(e);
    }
    const size_t qb = rows * p * dt_size(in_dt), vb = rows * dv * dt_size(in_dt);
    const size_t ob = rows * dv * dt_size(o_dt);
    for (const auto& [ptr, bytes] : {std::pair<const void*, size_t>{S, Sb}, {Z, Zb}})
      if (overlap(ptr, bytes, q, qb) || overlap(ptr, bytes, k, qb) || overlap(ptr, bytes, v, vb) ||
          overlap(ptr, bytes, o, ob))
        return KATA_ERR_ALIAS;
  }
  if (zero) return KATA_OK;
  if (!chunked_supported(p, dv, C, in_dt, fam, g, packed)) return KATA_ERR_UNSUPPORTED;
  // the kernels address one sequence's rows (H rows apart when packed) with 32-bit byte offsets
  if (packed && (int64_t)T * H * (p > dv ? p : dv) * 4 >= INT32_MAX) return KATA_ERR_SHAPE;
  if ((s = check_fwd_alias(q, k, v, in_dt, o, o_dt, rows, p, dv)) != KATA_OK) return s;
  const bool s2f = sigma2_f16(p, dv, C, in_dt, fam, g);
  const bool s2 = cu == nullptr && !s2f && sigma2_mfma(p, dv, C, in_dt, fam, g);  // virtual rows
  if (s2 && (int64_t)T * 2 > INT32_MAX) return KATA_ERR_SHAPE;
  const kata::SegPlan plan = kata::seg_plan(B, H, s2 ? 2 * T : T, C, scan);
  if ((int64_t)B * H * plan.nseg > kMaxGrid) return KATA_ERR_SHAPE;
  const size_t need = kata_chunked_workspace_bytes_family(B, H, T, p, dv, C, scan, in_dt, fam, g);
  if (need > 0 && use_scratch) {
    // the library's own scratch array: cannot overlap caller buffers; resolved only after
    // every argument has been validated
    if (need > KATA_NOALLOC_SCRATCH_BYTES) return KATA_ERR_SCRATCH;
    if (kata::noalloc_scratch(&workspace) != hipSuccess) return KATA_ERR_HIP;
    workspace_bytes = need;
  } else if (need > 0) {
    if (!workspace || workspace_bytes < need) return KATA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return KATA_ERR_ALIGN;
    const size_t ob = rows * dv * dt_size(o_dt);
    if (overlap(o, ob, workspace, need)) return KATA_ERR_ALIAS;
    if (want_state) {
      const int64_t n = kata_feature_dim(p, fam, g);
      if (overlap(S, (size_t)B * H * n * dv * 4, workspace, need) ||
          overlap(Z, (size_t)B * H * n * 4, workspace, need))
        return KATA_ERR_ALIAS;
    }
  }
  float* ws = need > 0 ? static_cast<float*>(workspace) : nullptr;
  float* so = want_state ? S : nullptr;
  float* zo = want_state ? Z : nullptr;
  const bool ob16 = o_dt == KATA_DTYPE_BF16;
  hipStream_t st = (hipStream_t)stream;
  if (s2f)
    return hip_status(kata::launch_chunked_f16_s2(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                                                  static_cast<const uint16_t*>(v), o, ob16, B, H, T, dv, C, plan, ws,
                                                  so, zo, kata::SeqLayout{lens, cu, total}, st));
  if (s2)
    return hip_status(kata::launch_chunked_bf16_sigma2(static_cast<const uint16_t*>(q),
                                                       static_cast<const uint16_t*>(k),
                                                       static_cast<const uint16_t*>(v), o, ob16, B, H, T, dv,
                                                       C, plan, ws, so, zo, lens, st));
  const kata::SeqLayout lay{lens, cu, total};
  if (fam != KATA_FEAT_FULL)
    return hip_status(kata::launch_family_chunked(q, k, v, in_dt == KATA_DTYPE_BF16, o, ob16, B, H, T, p,
                                                  dv, C, (int)fam, g, plan, ws, so, zo, lay, st));
  if (in_dt == KATA_DTYPE_BF16 && kata::chunked_f16_supported(p, dv, C))
    return hip_status(kata::launch_chunked_f16(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                                               static_cast<const uint16_t*>(v), o, ob16, B, H, T, p, dv, C, plan, ws,
                                               so, zo, lay, passes, st));
  if (in_dt == KATA_DTYPE_BF16)
    return hip_status(kata::launch_chunked_bf16(static_cast<const uint16_t*>(q),
                                                static_cast<const uint16_t*>(k),
                                                static_cast<const uint16_t*>(v), o, ob16, B, H, T,
                                                p, dv, C, plan, ws, so, zo, lay, passes, st));
  return hip_status(kata::launch_chunked_f32(static_cast<const float*>(q),
                                             static_cast<const float*>(k),
                                             static_cast<const float*>(v), o, ob16, B, H, T, p, dv,
                                             C, plan, ws, so, zo, lay, passes, st));
}

size_t kata_chunked_workspace_bytes_family(int B, int H, int T, int p, int dv, int C,
                                           kata_scan_t scan, kata_dtype_t in_dt,
                                           kata_feature_t fam, int g) {
  if (kata_feature_dim(p, fam, g) <= 0) return 0;
  if (fam == KATA_FEAT_FULL) return kata_chunked_workspace_bytes(B, H, T, p, dv, C, scan, in_dt);
  if (!valid_dt(in_dt) || (scan != KATA_SCAN_SEQUENTIAL && scan != KATA_SCAN_ASSOCIATIVE)) return 0;
  if (B <= 0 || H <= 0 || T <= 0 || dv < 1 || C < 1) return 0;
  if (!chunked_supported(p, dv, C, in_dt, fam, g)) return 0;
  const bool s2f = sigma2_f16(p, dv, C, in_dt, fam, g);
  const bool s2 = !s2f && sigma2_mfma(p, dv, C, in_dt, fam, g);  // virtual rows
  if (s2 && (int64_t)T * 2 > INT32_MAX) return 0;
  const kata::SegPlan plan = kata::seg_plan(B, H, s2 ? 2 * T : T, C, scan);
  if (plan.nseg <= 1) return 0;
  const int64_t sf = s2f  ? kata::f16_state_floats(dv)
                     : s2 ? kata::mfma_state_floats(32, dv)
                          : kata::family_state_floats(p, dv, (int)fam, g);
  return (size_t)B * H * (plan.nseg - 1) * sf * sizeof(float);
}

kata_status_t kata_chunked_fwd_passes(const void* q, const void* k, const void* v,
                                      kata_dtype_t in_dt, void* o, kata_dtype_t o_dt, int B, int H,
                                      int T, int p, int dv, int C, kata_scan_t scan,
                                      void* workspace, size_t workspace_bytes, int passes,
                                      kata_stream_t stream) {
  return chunked_impl(q, k, v, in_dt, o, o_dt, B, H, T, p, dv, C, scan, KATA_FEAT_FULL, 1, workspace,
                      workspace_bytes, passes, false, nullptr, nullptr, nullptr, nullptr, 0, stream);
}

kata_status_t kata_chunked_fwd_state(const void* q, const void* k, const void* v,
                                     kata_dtype_t in_dt, void* o, kata_dtype_t o_dt, int B, int H,
                                     int T, int p, int dv, int C, kata_scan_t scan,
                                     void* workspace, size_t workspace_bytes, float* S, float* Z,
                                     kata_stream_t stream) {
  return chunked_impl(q, k, v, in_dt, o, o_dt, B, H, T, p, dv, C, scan, KATA_FEAT_FULL, 1, workspace,
                      workspace_bytes, KATA_PASS_ALL, true, S, Z, nullptr, nullptr, 0, stream);
}

kata_status_t kata_chunked_fwd_family(const void* q, const void* k, const void* v,
                                      kata_dtype_t in_dt, void* o, kata_dtype_t o_dt, int B,
                                      int H, int T, int p, int dv, int C, kata_scan_t scan,
                                      kata_feature_t fam, int g, void* workspace,
                                      size_t workspace_bytes, float* S, float* Z,
                                      kata_stream_t stream) {
  if ((S == nullptr) != (Z == nullptr)) return KATA_ERR_NULL;
  return chunked_impl(q, k, v, in_dt, o, o_dt, B, H, T, p, dv, C, scan, fam, g, workspace,
                      workspace_bytes, KATA_PASS_ALL, S != nullptr, S, Z, nullptr, nullptr, 0, stream);
}

kata_status_t kata_chunked_fwd_ragged(const void* q, const void* k, const void* v,
                                      kata_dtype_t in_dt, void* o, kata_dtype_t o_dt, int B,
                                      int H, int T, int p, int dv, int C, kata_scan_t scan,
                                      kata_feature_t fam, int g, const int32_t* lens,
                                      void* workspace, size_t workspace_bytes, float* S, float* Z,
                                      kata_stream_t stream) {
  if ((S == nullptr) != (Z == nullptr)) return KATA_ERR_NULL;
  if ((int64_t)B * H > 0 && T > 0) {
    if (lens == nullptr) return KATA_ERR_NULL;
    if (!aligned16(lens)) return KATA_ERR_ALIGN;
  }
  return chunked_impl(q, k, v, in_dt, o, o_dt, B, H, T, p, dv, C, scan, fam, g, workspace,
                      workspace_bytes, KATA_PASS_ALL, S != nullptr, S, Z, lens, nullptr, 0, stream);
}

kata_status_t kata_chunked_fwd_varlen(const void* q, const void* k, const void* v,
                                      kata_dtype_t in_dt, void* o, kata_dtype_t o_dt, int B,
                                      int H, int total, int max_len, int p, int dv, int C,
                                      kata_scan_t scan, kata_feature_t fam, int g,
                                      const int32_t* cu_seqlens, void* workspace,
                                      size_t workspace_bytes, float* S, float* Z,
                                      kata_stream_t stream) {
  if ((S == nullptr) != (Z == nullptr)) return KATA_ERR_NULL;
  if (total < 0 || max_len < 0) return KATA_ERR_SHAPE;
  if ((int64_t)B * H > 0) {
    if (cu_seqlens == nullptr) return KATA_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(cu_seqlens) % 4 != 0) return KATA_ERR_ALIGN;
  }
  if ((int64_t)total * H * (p > dv ? p : dv) < 0 || mul4(total, H, p > dv ? p : dv, 1) < 0) return KATA_ERR_SHAPE;
  return chunked_impl(q, k, v, in_dt, o, o_dt, B, H, max_len, p, dv, C, scan, fam, g, workspace,
                      workspace_bytes, KATA_PASS_ALL, S != nullptr, S, Z, nullptr, cu_seqlens, total, stream);
}

kata_status_t kata_chunked_fwd_noalloc(const void* q, const void* k, const void* v, kata_dtype_t in_dt,
                                       void* o, kata_dtype_t o_dt, int B, int H, int T, int p, int dv,
                                       int C, kata_scan_t scan, kata_stream_t stream) {
  return chunked_impl(q, k, v, in_dt, o, o_dt, B, H, T, p, dv, C, scan, KATA_FEAT_FULL, 1, nullptr, 0,
                      KATA_PASS_ALL, false, nullptr, nullptr, nullptr, nullptr, 0, stream, true);
}

kata_status_t kata_chunked_fwd(const void* q, const void* k, const void* v, kata_dtype_t in_dt,
                               void* o, kata_dtype_t o_dt, int B, int H, int T, int p, int dv,
                               int C, kata_scan_t scan, void* workspace, size_t workspace_bytes,
                               kata_stream_t stream) {
  return kata_chunked_fwd_passes(q, k, v, in_dt, o, o_dt, B, H, T, p, dv, C, scan, workspace,
                                 workspace_bytes, KATA_PASS_ALL, stream);
}

static kata_status_t quadratic_impl(const void* q, const void* k, const void* v, kata_dtype_t in_dt,
                                    void* o, kata_dtype_t o_dt, int B, int H, int T, int p, int dv,
                                    kata_feature_t fam, int g, kata_stream_t stream) {
  bool zero = false;
  kata_status_t s = check_fwd(q, k, v, in_dt, o, o_dt, B, H, T, p, dv, zero);
  if (s != KATA_OK) return s;
  if ((s = check_feature(p, fam, g)) != KATA_OK || zero) return s;
  if (fam == KATA_FEAT_FULL ? (!in_set(p, {16, 32, 64}) || !in_set(dv, {16, 32, 64})) : (p > 64 || dv > 64))
    return KATA_ERR_UNSUPPORTED;
  if ((s = check_fwd_alias(q, k, v, in_dt, o, o_dt, (size_t)B * H * T, p, dv)) != KATA_OK) return s;
  if ((int64_t)B * H * ((T + 31) / 32) > kMaxGrid) return KATA_ERR_SHAPE;
  const bool ob16 = o_dt == KATA_DTYPE_BF16;
  hipStream_t st = (hipStream_t)stream;
  if (fam != KATA_FEAT_FULL) {
    if (in_dt == KATA_DTYPE_BF16 && kata::quadratic_bf16_family_supported(p, dv, (int)fam, g))
      return hip_status(kata::launch_quadratic_bf16_family(static_cast<const uint16_t*>(q),
                                                           static_cast<const uint16_t*>(k),
                                                           static_cast<const uint16_t*>(v), o, ob16, B, H,
                                                           T, p, dv, (int)fam, g, st));
    return hip_status(kata::launch_family_quadratic(q, k, v, in_dt == KATA_DTYPE_BF16, o, ob16, B, H, T, p,
                                                    dv, (int)fam, g, st));
  }
  if (in_dt == KATA_DTYPE_BF16)
    return hip_status(kata::launch_quadratic_bf16(static_cast<const uint16_t*>(q),
                                                  static_cast<const uint16_t*>(k),
                                                  static_cast<const uint16_t*>(v), o, ob16, B, H,
                                                  T, p, dv, st));
  return hip_status(kata::launch_quadratic_f32(static_cast<const float*>(q),
                                               static_cast<const float*>(k),
                                               static_cast<const float*>(v), o, ob16, B, H, T, p,
                                               dv, st));
}

kata_status_t kata_quadratic_fwd(const void* q, const void* k, const void* v, kata_dtype_t in_dt,
                                 void* o, kata_dtype_t o_dt, int B, int H, int T, int p, int dv,
                                 kata_stream_t stream) {
  return quadratic_impl(q, k, v, in_dt, o, o_dt, B, H, T, p, dv, KATA_FEAT_FULL, 1, stream);
}

kata_status_t kata_quadratic_fwd_varlen(const void* q, const void* k, const void* v, kata_dtype_t in_dt,
                                        void* o, kata_dtype_t o_dt, int B, int H, int total, int max_len, int p,
                                        int dv, kata_feature_t fam, int g, const int32_t* cu_seqlens,
                                        kata_stream_t stream) {
  if (!valid_dt(in_dt) || !valid_dt(o_dt)) return KATA_ERR_DTYPE;
  if (B < 0 || H < 0 || total < 0 || max_len < 0 || p < 1 || dv < 1) return KATA_ERR_SHAPE;
  kata_status_t s = check_feature(p, fam, g);
  if (s != KATA_OK) return s;
  // the shapes of kata_quadratic_fwd_family: bf16 MFMA kernels where they exist, else the
  // fp32 VALU kernel (full map) or the VALU family kernel, all with the packed layout
  const bool full = fam == KATA_FEAT_FULL, bf16 = in_dt == KATA_DTYPE_BF16;
  const bool mfma = bf16 && in_set(dv, {16, 32, 64}) &&
                    (full ? in_set(p, {16, 32, 64}) : kata::quadratic_bf16_family_supported(p, dv, (int)fam, g));
  if (full ? (!in_set(p, {16, 32, 64}) || !in_set(dv, {16, 32, 64})) : (p > 64 || dv > 64))
    return KATA_ERR_UNSUPPORTED;
  if ((int64_t)B * H == 0 || total == 0 || max_len == 0) return KATA_OK;
  if (cu_seqlens == nullptr) return KATA_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(cu_seqlens) % 4 != 0) return KATA_ERR_ALIGN;
  // one sequence's rows (H apart) are addressed with 32-bit byte offsets, up to a query
  // block of 512 rows past its end
  const int w = p > dv ? p : dv;
  if (mul4(total, H, w, 1) < 0 || ((int64_t)max_len + 512) * H * w * 4 >= INT32_MAX) return KATA_ERR_SHAPE;
  if ((int64_t)B * H * ((max_len + 31) / 32) > kMaxGrid) return KATA_ERR_SHAPE;
  if (!q || !k || !v || !o) return KATA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return KATA_ERR_ALIGN;
  if ((s = check_fwd_alias(q, k, v, in_dt, o, o_dt, (size_t)total * H, p, dv)) != KATA_OK) return s;
  kata::SeqLayout lay;
  lay.cu = cu_seqlens;
  lay.total = total;
  const hipStream_t st = (hipStream_t)stream;
  if (!mfma && full)
    return hip_status(kata::launch_quadratic_f32(static_cast<const float*>(q), static_cast<const float*>(k),
                                                 static_cast<const float*>(v), o, o_dt == KATA_DTYPE_BF16, B, H,
                                                 max_len, p, dv, st, lay));
  if (!mfma)
    return hip_status(kata::launch_family_quadratic(q, k, v, bf16, o, o_dt == KATA_DTYPE_BF16, B, H, max_len, p, dv,
                                                    (int)fam, g, st, lay));
  return hip_status(kata::launch_quadratic_bf16_varlen(static_cast<const uint16_t*>(q),
                                                       static_cast<const uint16_t*>(k),
                                                       static_cast<const uint16_t*>(v), o,
                                                       o_dt == KATA_DTYPE_BF16, B, H, max_len, p, dv, (int)fam,
                                                       g, lay, (hipStream_t)stream));
}

kata_status_t kata_quadratic_fwd_family(const void* q, const void* k, const void* v,
                                        kata_dtype_t in_dt, void* o, kata_dtype_t o_dt, int B,
                                        int H, int T, int p, int dv, kata_feature_t fam, int g,
                                        kata_stream_t stream) {
  return quadratic_impl(q, k, v, in_dt, o, o_dt, B, H, T, p, dv, fam, g, stream);
}

static kata_status_t decode_impl(const void* q, const void* k, const void* v, kata_dtype_t in_dt,
                                 kata_feature_t fam, int g, float* S, float* Z, void* o,
                                 kata_dtype_t o_dt, int N, int H, int p, int dv,
                                 kata_stream_t stream) {
  if (!valid_dt(in_dt) || !valid_dt(o_dt)) return KATA_ERR_DTYPE;
  if (N < 0 || H < 0 || p < 1 || dv < 1) return KATA_ERR_SHAPE;
  kata_status_t s = check_feature(p, fam, g);
  if (s != KATA_OK) return s;
  if (p > 64 || dv > 64 || (fam == KATA_FEAT_FULL && dv % 4 != 0)) return KATA_ERR_UNSUPPORTED;
  const int64_t NH = (int64_t)N * H;
  if (NH == 0) return KATA_OK;
  if (NH > kMaxGrid) return KATA_ERR_SHAPE;
  if (!q || !k || !v || !S || !Z || !o) return KATA_ERR_NULL;
  for (const void* ptr : {q, k, v, (const void*)S, (const void*)Z, (const void*)o})
    if (!aligned16(ptr)) return KATA_ERR_ALIGN;
  const int64_t n = kata_feature_dim(p, fam, g);
  const size_t qb = NH * p * dt_size(in_dt), vb = NH * dv * dt_size(in_dt);
  const size_t ob = NH * dv * dt_size(o_dt), Sb = NH * n * dv * 4, Zb = NH * n * 4;
  const void* outs[3] = {o, S, Z};
  const size_t outb[3] = {ob, Sb, Zb};
  for (int i = 0; i < 3; ++i) {
    if (overlap(outs[i], outb[i], q, qb) || overlap(outs[i], outb[i], k, qb) ||
        overlap(outs[i], outb[i], v, vb))
      return KATA_ERR_ALIAS;
    for (int j = i + 1; j < 3; ++j)
      if (overlap(outs[i], outb[i], outs[j], outb[j])) return KATA_ERR_ALIAS;
  }
  if (fam != KATA_FEAT_FULL)
    return hip_status(kata::launch_family_decode(q, k, v, in_dt == KATA_DTYPE_BF16, S, Z, o,
                                                 o_dt == KATA_DTYPE_BF16, N, H, p, dv, (int)fam, g,
                                                 (hipStream_t)stream));
  return hip_status(kata::launch_decode(q, k, v, in_dt == KATA_DTYPE_BF16, S, Z, o,
                                        o_dt == KATA_DTYPE_BF16, N, H, p, dv,
                                        (hipStream_t)stream));
}

kata_status_t kata_decode_step(const void* q, const void* k, const void* v, kata_dtype_t in_dt,
                               float* S, float* Z, void* o, kata_dtype_t o_dt, int N, int H, int p,
                               int dv, kata_stream_t stream) {
  return decode_impl(q, k, v, in_dt, KATA_FEAT_FULL, 1, S, Z, o, o_dt, N, H, p, dv, stream);
}

kata_status_t kata_decode_step_family(const void* q, const void* k, const void* v,
                                      kata_dtype_t in_dt, kata_feature_t fam, int g, float* S,
                                      float* Z, void* o, kata_dtype_t o_dt, int N, int H, int p,
                                      int dv, kata_stream_t stream) {
  return decode_impl(q, k, v, in_dt, fam, g, S, Z, o, o_dt, N, H, p, dv, stream);
}

size_t kata_quadratic_bwd_workspace_bytes(int B, int H, int T) {
  if (B <= 0 || H <= 0 || T <= 0) return 0;
  return (size_t)B * H * T * 2 * sizeof(float);
}

kata_status_t kata_quadratic_bwd(const void* q, const void* k, const void* v, const void* grad_o,
                                 kata_dtype_t in_dt, int B, int H, int T, int p, int dv,
                                 kata_feature_t fam, int g, float* dq, float* dk, float* dv_out,
                                 void* workspace, size_t workspace_bytes, kata_stream_t stream) {
  if (!valid_dt(in_dt)) return KATA_ERR_DTYPE;
  if (B < 0 || H < 0 || T < 0 || p < 1 || dv < 1) return KATA_ERR_SHAPE;
  kata_status_t s = check_feature(p, fam, g);
  if (s != KATA_OK) return s;
  if (p > 64 || dv > 64 || kata::bwd_pairs(p, (int)fam, g) > 16) return KATA_ERR_UNSUPPORTED;
  if ((int64_t)B * H * T == 0) return KATA_OK;
  if (mul4(B, H, T, p > dv ? p : dv) < 0 || (int64_t)B * H * ((T + 31) / 32) > kMaxGrid) return KATA_ERR_SHAPE;
  if (!q || !k || !v || !grad_o || !dq || !dk || !dv_out) return KATA_ERR_NULL;
  for (const void* ptr : {q, k, v, grad_o, (const void*)dq, (const void*)dk, (const void*)dv_out})
    if (!aligned16(ptr)) return KATA_ERR_ALIGN;
  const size_t need = kata_quadratic_bwd_workspace_bytes(B, H, T);
  if (!workspace || workspace_bytes < need) return KATA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return KATA_ERR_ALIGN;
  const size_t rows = (size_t)B * H * T;
  const size_t qb = rows * p * dt_size(in_dt), vb = rows * dv * dt_size(in_dt);
  const void* outs[4] = {dq, dk, dv_out, workspace};
  const size_t outb[4] = {rows * p * 4, rows * p * 4, rows * dv * 4, need};
  for (int i = 0; i < 4; ++i) {
    if (overlap(outs[i], outb[i], q, qb) || overlap(outs[i], outb[i], k, qb) || overlap(outs[i], outb[i], v, vb) ||
        overlap(outs[i], outb[i], grad_o, vb))
      return KATA_ERR_ALIAS;
    for (int j = i + 1; j < 4; ++j)
      if (overlap(outs[i], outb[i], outs[j], outb[j])) return KATA_ERR_ALIAS;
  }
  if (in_dt == KATA_DTYPE_BF16 && fam == KATA_FEAT_FULL && kata::quadratic_bwd_mfma_supported(p, dv))
    return hip_status(kata::launch_quadratic_bwd_mfma(
        static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
        static_cast<const uint16_t*>(grad_o), B, H, T, p, dv, static_cast<float*>(workspace), dq, dk, dv_out,
        (hipStream_t)stream));
  return hip_status(kata::launch_quadratic_bwd(q, k, v, grad_o, in_dt == KATA_DTYPE_BF16, B, H, T, p, dv,
                                               (int)fam, g, static_cast<float*>(workspace), dq, dk, dv_out,
                                               (hipStream_t)stream));
}

size_t kata_quadratic_bwd_varlen_workspace_bytes(int B, int H, int total) {
  if (B <= 0 || H <= 0 || total <= 0) return 0;
  return (size_t)total * H * 2 * sizeof(float);
}

kata_status_t kata_quadratic_bwd_varlen(const void* q, const void* k, const void* v, const void* grad_o,
                                        kata_dtype_t in_dt, int B, int H, int total, int max_len, int p, int dv,
                                        const int32_t* cu_seqlens, float* dq, float* dk, float* dv_out,
                                        void* workspace, size_t workspace_bytes, kata_stream_t stream) {
  if (!valid_dt(in_dt)) return KATA_ERR_DTYPE;
  if (B < 0 || H < 0 || total < 0 || max_len < 0 || p < 1 || dv < 1) return KATA_ERR_SHAPE;
  // bf16 MFMA kernels for their shapes, else the VALU kernels (p, dv <= 64), packed layout
  const bool mfma = in_dt == KATA_DTYPE_BF16 && kata::quadratic_bwd_mfma_supported(p, dv);
  if (p > 64 || dv > 64) return KATA_ERR_UNSUPPORTED;
  if ((int64_t)B * H == 0 || total == 0 || max_len == 0) return KATA_OK;
  if (cu_seqlens == nullptr) return KATA_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(cu_seqlens) % 4 != 0) return KATA_ERR_ALIGN;
  // one sequence's rows (H apart) are addressed with 32-bit byte offsets, up to a block of
  // 512 rows past its end (MFMA kernels; the same bound for both paths)
  const int w = p > dv ? p : dv;
  if (mul4(total, H, w, 1) < 0 || ((int64_t)max_len + 512) * H * w * 4 >= INT32_MAX) return KATA_ERR_SHAPE;
  if ((int64_t)B * H * ((max_len + 31) / 32) > kMaxGrid) return KATA_ERR_SHAPE;
  if (!q || !k || !v || !grad_o || !dq || !dk || !dv_out) return KATA_ERR_NULL;
  for (const void* ptr : {q, k, v, grad_o, (const void*)dq, (const void*)dk, (const void*)dv_out})
    if (!aligned16(ptr)) return KATA_ERR_ALIGN;
  const size_t need = kata_quadratic_bwd_varlen_workspace_bytes(B, H, total);
  if (!workspace || workspace_bytes < need) return KATA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return KATA_ERR_ALIGN;
  const size_t rows = (size_t)total * H;
  const size_t qb = rows * p * dt_size(in_dt), vb = rows * dv * dt_size(in_dt);
  const void* outs[4] = {dq, dk, dv_out, workspace};
  const size_t outb[4] = {rows * p * 4, rows * p * 4, rows * dv * 4, need};
  for (int i = 0; i < 4; ++i) {
    if (overlap(outs[i], outb[i], q, qb) || overlap(outs[i], outb[i], k, qb) || overlap(outs[i], outb[i], v, vb) ||
        overlap(outs[i], outb[i], grad_o, vb))
      return KATA_ERR_ALIAS;
    for (int j = i + 1; j < 4; ++j)
      if (overlap(outs[i], outb[i], outs[j], outb[j])) return KATA_ERR_ALIAS;
  }
  kata::SeqLayout lay;
  lay.cu = cu_seqlens;
  lay.total = total;
  if (!mfma)
    return hip_status(kata::launch_quadratic_bwd(q, k, v, grad_o, in_dt == KATA_DTYPE_BF16, B, H, max_len, p, dv,
                                                 (int)KATA_FEAT_FULL, 1, static_cast<float*>(workspace), dq, dk,
                                                 dv_out, (hipStream_t)stream, lay));
  return hip_status(kata::launch_quadratic_bwd_mfma_varlen(
      static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
      static_cast<const uint16_t*>(grad_o), B, H, max_len, p, dv, lay, static_cast<float*>(workspace), dq, dk,
      dv_out, (hipStream_t)stream));
}

// fp32 VALU state-form kernels: the chunk's rows and the fp32 state within LDS
static bool chunked_bwd_valu_supported(int p, int dv, int C) {
  return p >= 1 && p <= 64 && dv >= 1 && dv <= 64 && in_set(C, {16, 32, 64}) &&
         kata::chunked_bwd_lds_bytes(p, dv, C) <= 160 * 1024;
}
// a shape one of the two paths runs (the bf16 MFMA kernels choose their own chunking)
static bool chunked_bwd_supported(int p, int dv, int C) {
  return in_set(C, {16, 32, 64}) && (chunked_bwd_valu_supported(p, dv, C) || kata::chunked_bwd_mfma_supported(p, dv));
}

// chunk of the VALU kernels when the caller gives none (packed sequences): the largest that fits
static int chunked_bwd_valu_chunk(int p, int dv) {
  for (int C : {64, 32, 16})
    if (chunked_bwd_valu_supported(p, dv, C)) return C;
  return 0;
}

size_t kata_chunked_bwd_workspace_bytes(int B, int H, int T, int p, int dv, int C, kata_scan_t scan) {
  if (B <= 0 || H <= 0 || T <= 0 || (scan != KATA_SCAN_SEQUENTIAL && scan != KATA_SCAN_ASSOCIATIVE)) return 0;
  if (!chunked_bwd_supported(p, dv, C)) return 0;
  size_t need = 0;
  if (chunked_bwd_valu_supported(p, dv, C)) {
    const kata::SegPlan plan = kata::seg_plan(B, H, T, C, scan);
    const size_t rows = (size_t)B * H * T;
    const size_t sums = plan.nseg > 1 ? (size_t)B * H * (plan.nseg - 1) * kata::chunked_bwd_state_floats(p, dv) : 0;
    need = (rows * 2 + 2 * sums) * sizeof(float);
  }
  if (kata::chunked_bwd_mfma_supported(p, dv)) {  // the size does not depend on the input dtype
    const size_t m = kata::chunked_bwd_mfma_workspace_floats(B, H, T, p, dv, scan, (int64_t)B * H * T) * sizeof(float);
    need = m > need ? m : need;
  }
  return need;
}

kata_status_t kata_chunked_bwd(const void* q, const void* k, const void* v, const void* grad_o, kata_dtype_t in_dt,
                               int B, int H, int T, int p, int dv, int C, kata_scan_t scan, float* dq, float* dk,
                               float* dv_out, void* workspace, size_t workspace_bytes, kata_stream_t stream) {
  if (!valid_dt(in_dt)) return KATA_ERR_DTYPE;
  if (scan != KATA_SCAN_SEQUENTIAL && scan != KATA_SCAN_ASSOCIATIVE) return KATA_ERR_SCAN;
  if (B < 0 || H < 0 || T < 0 || p < 1 || dv < 1 || C < 1) return KATA_ERR_SHAPE;
  if (!chunked_bwd_supported(p, dv, C)) return KATA_ERR_UNSUPPORTED;
  const bool mfma = in_dt == KATA_DTYPE_BF16 && kata::chunked_bwd_mfma_supported(p, dv);
  if (!mfma && !chunked_bwd_valu_supported(p, dv, C)) return KATA_ERR_UNSUPPORTED;
  if ((int64_t)B * H * T == 0) return KATA_OK;
  const kata::SegPlan plan = kata::seg_plan(B, H, T, mfma ? kata::CHUNKED_BWD_FWD_C : C, scan);
  if (mul4(B, H, T, p > dv ? p : dv) < 0 || (int64_t)B * H * plan.nseg > kMaxGrid) return KATA_ERR_SHAPE;
  // the forward that the MFMA path runs first addresses a sequence with 32-bit byte offsets
  if (mfma && (int64_t)T * (p > dv ? p : dv) * 4 >= INT32_MAX) return KATA_ERR_SHAPE;
  if (!q || !k || !v || !grad_o || !dq || !dk || !dv_out) return KATA_ERR_NULL;
  for (const void* ptr : {q, k, v, grad_o, (const void*)dq, (const void*)dk, (const void*)dv_out})
    if (!aligned16(ptr)) return KATA_ERR_ALIGN;
  const size_t need = kata_chunked_bwd_workspace_bytes(B, H, T, p, dv, C, scan);
  if (!workspace || workspace_bytes < need) return KATA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return KATA_ERR_ALIGN;
  const size_t rows = (size_t)B * H * T;
  const size_t qb = rows * p * dt_size(in_dt), vb = rows * dv * dt_size(in_dt);
  const void* outs[4] = {dq, dk, dv_out, workspace};
  const size_t outb[4] = {rows * p * 4, rows * p * 4, rows * dv * 4, need};
  for (int i = 0; i < 4; ++i) {
    if (overlap(outs[i], outb[i], q, qb) || overlap(outs[i], outb[i], k, qb) || overlap(outs[i], outb[i], v, vb) ||
        overlap(outs[i], outb[i], grad_o, vb))
      return KATA_ERR_ALIAS;
    for (int j = i + 1; j < 4; ++j)
      if (overlap(outs[i], outb[i], outs[j], outb[j])) return KATA_ERR_ALIAS;
  }
  if (mfma)
    return hip_status(kata::launch_chunked_bwd_mfma(
        static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
        static_cast<const uint16_t*>(grad_o), B, H, T, p, dv, (int)scan, kata::SeqLayout{}, (int64_t)B * H * T,
        static_cast<float*>(workspace), dq, dk, dv_out, (hipStream_t)stream));
  float* stats = static_cast<float*>(workspace);
  const size_t sums = plan.nseg > 1 ? (size_t)B * H * (plan.nseg - 1) * kata::chunked_bwd_state_floats(p, dv) : 0;
  float* fsum = stats + rows * 2;
  float* rsum = fsum + sums;
  return hip_status(kata::launch_chunked_bwd(q, k, v, grad_o, in_dt == KATA_DTYPE_BF16, B, H, T, p, dv, C, plan,
                                             stats, fsum, rsum, dq, dk, dv_out, (hipStream_t)stream));
}

size_t kata_chunked_bwd_varlen_workspace_bytes(int B, int H, int total, int max_len, int p, int dv, kata_scan_t scan) {
  if (B <= 0 || H <= 0 || total < 0 || max_len <= 0 || (scan != KATA_SCAN_SEQUENTIAL && scan != KATA_SCAN_ASSOCIATIVE))
    return 0;
  // the larger of the two paths' needs (the size does not depend on the input dtype)
  size_t need = 0;
  if (const int C = chunked_bwd_valu_chunk(p, dv)) {
    const kata::SegPlan plan = kata::seg_plan(B, H, max_len, C, scan);
    const size_t rows = (size_t)total * H;
    const size_t sums = plan.nseg > 1 ? (size_t)B * H * (plan.nseg - 1) * kata::chunked_bwd_state_floats(p, dv) : 0;
    need = (rows * 2 + 2 * sums) * sizeof(float);
  }
  if (kata::chunked_bwd_mfma_supported(p, dv)) {
    const size_t m =
        kata::chunked_bwd_mfma_workspace_floats(B, H, max_len, p, dv, scan, (int64_t)total * H) * sizeof(float);
    need = m > need ? m : need;
  }
  return need;
}

kata_status_t kata_chunked_bwd_varlen(const void* q, const void* k, const void* v, const void* grad_o,
                                      kata_dtype_t in_dt, int B, int H, int total, int max_len, int p, int dv,
                                      kata_scan_t scan, const int32_t* cu_seqlens, float* dq, float* dk,
                                      float* dv_out, void* workspace, size_t workspace_bytes, kata_stream_t stream) {
  if (!valid_dt(in_dt)) return KATA_ERR_DTYPE;
  if (scan != KATA_SCAN_SEQUENTIAL && scan != KATA_SCAN_ASSOCIATIVE) return KATA_ERR_SCAN;
  if (B < 0 || H < 0 || total < 0 || max_len < 0 || p < 1 || dv < 1) return KATA_ERR_SHAPE;
  // bf16 MFMA kernels for their shapes, else the fp32 VALU kernels at the largest chunk that fits
  const bool mfma = in_dt == KATA_DTYPE_BF16 && kata::chunked_bwd_mfma_supported(p, dv);
  const int Cv = mfma ? 0 : chunked_bwd_valu_chunk(p, dv);
  if (!mfma && Cv == 0) return KATA_ERR_UNSUPPORTED;
  if ((int64_t)B * H == 0 || total == 0 || max_len == 0) return KATA_OK;
  if (cu_seqlens == nullptr) return KATA_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(cu_seqlens) % 4 != 0) return KATA_ERR_ALIGN;
  const int w = p > dv ? p : dv;
  if (mul4(total, H, w, 1) < 0 || (int64_t)max_len * H * w * 4 >= INT32_MAX) return KATA_ERR_SHAPE;
  const kata::SegPlan plan = kata::seg_plan(B, H, max_len, mfma ? kata::CHUNKED_BWD_FWD_C : Cv, scan);
  if ((int64_t)B * H * plan.nseg > kMaxGrid) return KATA_ERR_SHAPE;
  if (!q || !k || !v || !grad_o || !dq || !dk || !dv_out) return KATA_ERR_NULL;
  for (const void* ptr : {q, k, v, grad_o, (const void*)dq, (const void*)dk, (const void*)dv_out})
    if (!aligned16(ptr)) return KATA_ERR_ALIGN;
  const size_t need = kata_chunked_bwd_varlen_workspace_bytes(B, H, total, max_len, p, dv, scan);
  if (!workspace || workspace_bytes < need) return KATA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return KATA_ERR_ALIGN;
  const size_t rows = (size_t)total * H;
  const size_t qb = rows * p * dt_size(in_dt), vb = rows * dv * dt_size(in_dt);
  const void* outs[4] = {dq, dk, dv_out, workspace};
  const size_t outb[4] = {rows * p * 4, rows * p * 4, rows * dv * 4, need};
  for (int i = 0; i < 4; ++i) {
    if (overlap(outs[i], outb[i], q, qb) || overlap(outs[i], outb[i], k, qb) || overlap(outs[i], outb[i], v, vb) ||
        overlap(outs[i], outb[i], grad_o, vb))
      return KATA_ERR_ALIAS;
    for (int j = i + 1; j < 4; ++j)
      if (overlap(outs[i], outb[i], outs[j], outb[j])) return KATA_ERR_ALIAS;
  }
  kata::SeqLayout lay;
  lay.cu = cu_seqlens;
  lay.total = total;
  if (!mfma) {
    float* stats = static_cast<float*>(workspace);
    const size_t sums = plan.nseg > 1 ? (size_t)B * H * (plan.nseg - 1) * kata::chunked_bwd_state_floats(p, dv) : 0;
    float* fsum = stats + rows * 2;
    float* rsum = fsum + sums;
    return hip_status(kata::launch_chunked_bwd(q, k, v, grad_o, in_dt == KATA_DTYPE_BF16, B, H, max_len, p, dv, Cv,
                                               plan, stats, fsum, rsum, dq, dk, dv_out, (hipStream_t)stream, lay));
  }
  return hip_status(kata::launch_chunked_bwd_mfma(
      static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
      static_cast<const uint16_t*>(grad_o), B, H, max_len, p, dv, (int)scan, lay, (int64_t)rows,
      static_cast<float*>(workspace), dq, dk, dv_out, (hipStream_t)stream));
}

int64_t kata_order_dim(int p, int r) {
  if (p < 1 || r < 1 || r > 4) return -1;
  double c = 1.0;  // binom(p + 2r - 1, 2r)
  for (int i = 1; i <= 2 * r; ++i) c = c * (p + 2 * r - i) / i;
  if (c > 9.0e15) return -1;
  return (int64_t)(c + 0.5);
}

kata_status_t kata_lift_order(const void* u, kata_dtype_t u_dt, int64_t rows, int p, int r, void* psi,
                              kata_dtype_t psi_dt, kata_stream_t stream) {
  if (!valid_dt(u_dt) || !valid_dt(psi_dt)) return KATA_ERR_DTYPE;
  if (rows < 0 || p < 1) return KATA_ERR_SHAPE;
  if (r < 1 || r > 4) return KATA_ERR_FEATURE;
  if (r == 1) return kata_lift(u, u_dt, rows, p, psi, psi_dt, stream);
  if (p > 128) return KATA_ERR_UNSUPPORTED;
  if (rows == 0) return KATA_OK;
  const int64_t n = kata_order_dim(p, r);
  if (n < 0 || n > (int64_t)256 * 65535 || mul4(rows, n, 1, 1) < 0 || (rows + 15) / 16 > 65535)
    return KATA_ERR_SHAPE;
  if (!u || !psi) return KATA_ERR_NULL;
  if (!aligned16(u) || !aligned16(psi)) return KATA_ERR_ALIGN;
  if (overlap(u, rows * p * dt_size(u_dt), psi, rows * n * dt_size(psi_dt))) return KATA_ERR_ALIAS;
  return hip_status(kata::launch_order_lift(u, u_dt == KATA_DTYPE_BF16, rows, p, r, n, psi,
                                            psi_dt == KATA_DTYPE_BF16, (hipStream_t)stream));
}

kata_status_t kata_quadratic_fwd_order(const void* q, const void* k, const void* v, kata_dtype_t in_dt,
                                       void* o, kata_dtype_t o_dt, int B, int H, int T, int p, int dv, int r,
                                       kata_stream_t stream) {
  if (r == 1) return kata_quadratic_fwd(q, k, v, in_dt, o, o_dt, B, H, T, p, dv, stream);
  bool zero = false;
  kata_status_t s = check_fwd(q, k, v, in_dt, o, o_dt, B, H, T, p, dv, zero);
  if (s != KATA_OK) return s;
  if (r < 1 || r > 4) return KATA_ERR_FEATURE;
  if (zero) return KATA_OK;
  if (p > 64 || dv > 64) return KATA_ERR_UNSUPPORTED;
  if ((s = check_fwd_alias(q, k, v, in_dt, o, o_dt, (size_t)B * H * T, p, dv)) != KATA_OK) return s;
  if ((int64_t)B * H * ((T + 31) / 32) > kMaxGrid) return KATA_ERR_SHAPE;
  const bool ob16 = o_dt == KATA_DTYPE_BF16;
  hipStream_t st = (hipStream_t)stream;
  if (in_dt == KATA_DTYPE_BF16 && r == 2 && in_set(p, {16, 32, 64}) && in_set(dv, {16, 32, 64}))
    return hip_status(kata::launch_quadratic_bf16_order2(static_cast<const uint16_t*>(q),
                                                         static_cast<const uint16_t*>(k),
                                                         static_cast<const uint16_t*>(v), o, ob16, B, H, T, p,
                                                         dv, st));
  return hip_status(kata::launch_family_quadratic(q, k, v, in_dt == KATA_DTYPE_BF16, o, ob16, B, H, T, p, dv, 3, r,
                                                  st));
}

}  // extern "C"
