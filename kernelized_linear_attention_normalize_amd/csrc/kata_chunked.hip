// Dispatch of the bf16 chunked forward to its (p, dv, C) instantiations; the kernels are
// in kata_chunked.h and are instantiated per (p, dv) in kata_chunked_p*_dv*.hip so that
// they compile in parallel.
#include "kata_device.h"
#include "kata_launch.h"

namespace kata {
namespace chk {
template <int P, int DV, int C, bool S2>
hipError_t launch_pdc(const uint16_t* q, const uint16_t* k, const uint16_t* v, void* o, bool o_bf16,
                      int B, int H, int T, const SegPlan& plan, float* ws, float* s_out, float* z_out,
                      SeqLayout lay, int passes, hipStream_t st);
}  // namespace chk

int64_t mfma_state_floats(int p, int dv) {
  const int nt = p == 32 ? 33 : 9;
  return (int64_t)nt * (dv / 16) * 256 + (p / 16) * (p / 16) * 256;
}

hipError_t launch_chunked_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v, void* o,
                               bool o_bf16, int B, int H, int T, int p, int dv, int C,
                               const SegPlan& plan, float* ws, float* s_out, float* z_out,
                               SeqLayout lay, int passes, hipStream_t st) {
#define KATA_CCASE(PP, DD, CC) \
  if (p == PP && dv == DD && C == CC) return chk::launch_pdc<PP, DD, CC, false>(q, k, v, o, o_bf16, B, H, T, plan, ws, s_out, z_out, lay, passes, st);
#define KATA_CCASE3(PP, DD) KATA_CCASE(PP, DD, 32) KATA_CCASE(PP, DD, 64) KATA_CCASE(PP, DD, 128)
  KATA_CCASE3(16, 16) KATA_CCASE3(16, 32) KATA_CCASE3(16, 64)
  KATA_CCASE3(32, 16) KATA_CCASE3(32, 32) KATA_CCASE3(32, 64)
#undef KATA_CCASE3
#undef KATA_CCASE
  return hipErrorInvalidValue;
}

}  // namespace kata
