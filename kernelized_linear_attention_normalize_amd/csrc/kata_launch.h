// Internal host-side launchers (one per kernel family). Arguments are already validated.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kata {

// segment plan of the chunked forward (shared by the workspace query and the launch)
struct SegPlan {
  int nchunks;       // ceil(T / C)
  int nseg;          // number of segments per (b,h)
  int cps;           // chunks per segment (last segment may have fewer)
};
SegPlan seg_plan(int B, int H, int T, int C, int scan);

// device address of the library's fixed scratch array on the current device (resolved once
// per device; see kata_chunked_fwd_noalloc)
hipError_t noalloc_scratch(void** out);

// Where the rows of sequence bh = (b, h) of a chunked forward live. Padded layout
// [B, H, T, *] (cu null): rows bh * T + t, cut at lens[b] when lens (device, [B]) is given.
// Packed token-major layout [total, H, *] (cu: device cu_seqlens[B + 1]): rows
// (cu[b] + t) * H + h for t < cu[b + 1] - cu[b]. T bounds every length (the segment plan is
// that of T).
struct SeqLayout {
  const int* lens = nullptr;
  const int* cu = nullptr;
  int total = 0;  // rows per head of the packed layout
};

// passes of the chunked forward (the values of kata_pass_t)
enum : int { PASS_SUMMARIES = 1, PASS_SCAN = 2, PASS_SEGMENTS = 4 };

// floats of one segment summary in the bf16 MFMA kernel's tile layout
int64_t mfma_state_floats(int p, int dv);
// floats of one segment summary in the fp32 kernel's layout (S then Z, packed order)
int64_t f32_state_floats(int p, int dv);
// dynamic LDS bytes of the fp32 chunked kernel (0 if it cannot run)
size_t f32_chunked_lds_bytes(int p, int dv, int C);
// value-column parts of the fp32 chunked forward (0: unsupported) and its workspace floats per
// segment summary over all parts
int f32_chunked_parts(int p, int dv, int C);
int64_t f32_chunked_state_floats(int p, int dv, int C);

hipError_t launch_lift(const void* u, bool u_bf16, int64_t rows, int p, void* psi, bool psi_bf16,
                       hipStream_t st);
hipError_t launch_decode(const void* q, const void* k, const void* v, bool in_bf16, float* S,
                         float* Z, void* o, bool o_bf16, int N, int H, int p, int dv,
                         hipStream_t st);
// s_out / z_out (may be null): the state after the last token of every sequence, in the
// decode layout (S [B,H,n,dv], Z [B,H,n], fp32, packed order), written by pass 3.
// lay: the row layout (SeqLayout); rows past a sequence's length are not used and their
// outputs are not written.
hipError_t launch_chunked_f32(const float* q, const float* k, const float* v, void* o, bool o_bf16,
                              int B, int H, int T, int p, int dv, int C, const SegPlan& plan,
                              float* ws, float* s_out, float* z_out, SeqLayout lay, int passes,
                              hipStream_t st);
hipError_t launch_quadratic_f32(const float* q, const float* k, const float* v, void* o,
                                bool o_bf16, int B, int H, int T, int p, int dv, hipStream_t st,
                                SeqLayout lay = SeqLayout{});
// fp16-operand chunked forward (kata_chunked16.h): p = 32, dv = 64, C in {64, 128}
bool chunked_f16_supported(int p, int dv, int C);
int64_t f16_state_floats(int dv);
hipError_t launch_chunked_f16(const uint16_t* q, const uint16_t* k, const uint16_t* v, void* o, bool o_bf16, int B,
                              int H, int T, int p, int dv, int C, const SegPlan& plan, float* ws, float* s_out,
                              float* z_out, SeqLayout lay, int passes, hipStream_t st);
// the same kernels for KATA-Sigma 2 at p = 64 (dv = 64, C in {64, 128}); segment summaries of
// f16_state_floats(dv) floats, plan over T
bool chunked_f16_s2_supported(int dv, int C);
hipError_t launch_chunked_f16_s2(const uint16_t* q, const uint16_t* k, const uint16_t* v, void* o, bool o_bf16, int B,
                                 int H, int T, int dv, int C, const SegPlan& plan, float* ws, float* s_out,
                                 float* z_out, SeqLayout lay, hipStream_t st);
hipError_t launch_chunked_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v, void* o,
                               bool o_bf16, int B, int H, int T, int p, int dv, int C,
                               const SegPlan& plan, float* ws, float* s_out, float* z_out,
                               SeqLayout lay, int passes, hipStream_t st);
// n float zeros at p (a fill kernel, so the call is safe under graph capture)
hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t st);

// ---- reduced PSD families (fam 1: Sigma g, 2: M g; m = p / g), VALU kernels
// floats of one segment summary (n*dv + n, padded to a multiple of 4)
int64_t family_state_floats(int p, int dv, int fam, int g);
// dynamic LDS bytes of the family chunked kernel
size_t family_chunked_lds_bytes(int p, int dv, int C, int fam, int g);
hipError_t launch_family_lift(const void* u, bool u_bf16, int64_t rows, int p, int fam, int g, void* psi,
                              bool psi_bf16, hipStream_t st);
hipError_t launch_family_decode(const void* q, const void* k, const void* v, bool in_bf16, float* S, float* Z,
                                void* o, bool o_bf16, int N, int H, int p, int dv, int fam, int g,
                                hipStream_t st);
hipError_t launch_family_chunked(const void* q, const void* k, const void* v, bool in_bf16, void* o,
                                 bool o_bf16, int B, int H, int T, int p, int dv, int C, int fam, int g,
                                 const SegPlan& plan, float* ws, float* s_out, float* z_out, SeqLayout lay,
                                 hipStream_t st);
// bf16 MFMA chunked forward of KATA-Sigma 2 at p = 64 (dv in {32, 64}, C in {64, 128}); plan
// over the 2T virtual rows (two 32-component blocks per token)
hipError_t launch_chunked_bf16_sigma2(const uint16_t* q, const uint16_t* k, const uint16_t* v, void* o,
                                      bool o_bf16, int B, int H, int T, int dv, int C, const SegPlan& plan,
                                      float* ws, float* s_out, float* z_out, const int* lens, hipStream_t st);
// gradients of the quadratic form (VALU): ws holds 2 floats (D_t, g_t . o_t) per row
int bwd_pairs(int p, int fam, int g);
// O(T) chunked backward of the full map (fp32 VALU): LDS bytes, summary floats, launch
size_t chunked_bwd_lds_bytes(int p, int dv, int C);
int64_t chunked_bwd_state_floats(int p, int dv);
hipError_t launch_chunked_bwd(const void* q, const void* k, const void* v, const void* go, bool in_bf16, int B, int H,
                              int T, int p, int dv, int C, const SegPlan& plan, float* stats, float* fsum,
                              float* rsum, float* dq, float* dk, float* dvo, hipStream_t st,
                              SeqLayout lay = SeqLayout{});
// O(T) chunked backward of the full map on bf16 MFMA (p in {16, 32}, dv in {32, 64}); the
// forward it runs first (for o and the segment prefixes) uses chunks of CHUNKED_BWD_FWD_C
constexpr int CHUNKED_BWD_FWD_C = 128;
bool chunked_bwd_mfma_supported(int p, int dv);
// workspace floats: D_t, delta_t for `rows` rows (B H T padded, total H packed) and the two
// sets of segment summaries of the plan of T
size_t chunked_bwd_mfma_workspace_floats(int B, int H, int T, int p, int dv, int scan, int64_t rows);
hipError_t launch_chunked_bwd_mfma(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* go,
                                   int B, int H, int T, int p, int dv, int scan, SeqLayout lay, int64_t rows,
                                   float* ws, float* dq, float* dk, float* dvo, hipStream_t st);
// full map, bf16 q, k, v, gout: MFMA backward (p, dv in {32, 64}); stats: 2 floats per row
bool quadratic_bwd_mfma_supported(int p, int dv);
hipError_t launch_quadratic_bwd_mfma(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* gout,
                                     int B, int H, int T, int p, int dv, float* stats, float* dq, float* dk,
                                     float* dvo, hipStream_t st);
// the same over packed sequences (lay.cu, lay.total; T = max_len; stats per packed row)
hipError_t launch_quadratic_bwd_mfma_varlen(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                            const uint16_t* gout, int B, int H, int max_len, int p, int dv,
                                            SeqLayout lay, float* stats, float* dq, float* dk, float* dvo,
                                            hipStream_t st);
hipError_t launch_quadratic_bwd(const void* q, const void* k, const void* v, const void* go, bool in_bf16, int B,
                                int H, int T, int p, int dv, int fam, int g, float* ws, float* dq, float* dk,
                                float* dvo, hipStream_t st, SeqLayout lay = SeqLayout{});
// bf16 MFMA quadratic form with weights (q_hat . k_hat)^4 (psi_4), full map's (p, dv) set
hipError_t launch_quadratic_bf16_order2(const uint16_t* q, const uint16_t* k, const uint16_t* v, void* o,
                                        bool o_bf16, int B, int H, int T, int p, int dv, hipStream_t st);
// bf16 MFMA quadratic form for the reduced families with 32-component blocks
bool quadratic_bf16_family_supported(int p, int dv, int fam, int g);
hipError_t launch_quadratic_bf16_family(const uint16_t* q, const uint16_t* k, const uint16_t* v, void* o,
                                        bool o_bf16, int B, int H, int T, int p, int dv, int fam, int g,
                                        hipStream_t st);
// packed psi_2r lift (n = binom(p + 2r - 1, 2r) coordinates per row, VALU)
hipError_t launch_order_lift(const void* u, bool u_bf16, int64_t rows, int p, int r, int64_t n, void* psi,
                             bool psi_bf16, hipStream_t st);
// fam 3 selects the full map with weights (q_hat . k_hat)^(2g)
hipError_t launch_family_quadratic(const void* q, const void* k, const void* v, bool in_bf16, void* o, bool o_bf16,
                                   int B, int H, int T, int p, int dv, int fam, int g, hipStream_t st,
                                   SeqLayout lay = SeqLayout{});
hipError_t launch_quadratic_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v, void* o,
                                 bool o_bf16, int B, int H, int T, int p, int dv, hipStream_t st);
// the same over packed token-major sequences (lay.cu set; T = max_len): the full map (fam 0)
// or a reduced family that quadratic_bf16_family_supported covers
hipError_t launch_quadratic_bf16_varlen(const uint16_t* q, const uint16_t* k, const uint16_t* v, void* o,
                                        bool o_bf16, int B, int H, int max_len, int p, int dv, int fam, int g,
                                        SeqLayout lay, hipStream_t st);

}  // namespace kata
