// Dispatch of the fp16-operand chunked forward (kata_chunked16.h) for p = 32.
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

}  // namespace kata
