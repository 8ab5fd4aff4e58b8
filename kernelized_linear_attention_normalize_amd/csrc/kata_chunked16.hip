// Dispatch of the fp16-operand chunked forward (kata_chunked16.h): the full map at p = 32 and
// KATA-Sigma 2 at p = 64 (two 32-component blocks).
#include "kata_chunked16.h"

namespace kata {

bool chunked_f16_supported(int p, int dv, int C) { return p == 32 && dv == 64 && (C == 64 || C == 128); }

int64_t f16_state_floats(int dv) { return dv == 64 ? c16::Lay<64, 128>::STATE_FLOATS : 0; }

hipError_t launch_chunked_f16(const uint16_t* q, const uint16_t* k, const uint16_t* v, void* o, bool o_bf16, int B,
                              int H, int T, int p, int dv, int C, const SegPlan& plan, float* ws, float* s_out,
                              float* z_out, SeqLayout lay, int passes, hipStream_t st) {
  if (p == 32 && dv == 64 && C == 128)
    return c16::launch<64, 128>(q, k, v, o, o_bf16, B, H, T, plan, ws, s_out, z_out, lay, passes, st);
  if (p == 32 && dv == 64 && C == 64)
    return c16::launch<64, 64>(q, k, v, o, o_bf16, B, H, T, plan, ws, s_out, z_out, lay, passes, st);
  return hipErrorInvalidValue;
}

bool chunked_f16_s2_supported(int dv, int C) { return dv == 64 && (C == 64 || C == 128); }

hipError_t launch_chunked_f16_s2(const uint16_t* q, const uint16_t* k, const uint16_t* v, void* o, bool o_bf16, int B,
                                 int H, int T, int dv, int C, const SegPlan& plan, float* ws, float* s_out,
                                 float* z_out, SeqLayout lay, hipStream_t st) {
  constexpr int ALL = PASS_SUMMARIES | PASS_SCAN | PASS_SEGMENTS;
  if (dv == 64 && C == 128)
    return c16::launch<64, 128, true>(q, k, v, o, o_bf16, B, H, T, plan, ws, s_out, z_out, lay, ALL, st);
  if (dv == 64 && C == 64)
    return c16::launch<64, 64, true>(q, k, v, o, o_bf16, B, H, T, plan, ws, s_out, z_out, lay, ALL, st);
  return hipErrorInvalidValue;
}

}  // namespace kata
