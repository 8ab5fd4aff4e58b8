// Instantiations of the bf16 chunked forward for p = 16, dv = 16 (see kata_chunked.h).
#include "kata_chunked.h"

namespace kata {
namespace chk {
template hipError_t launch_pdc<16, 16, 32>(const uint16_t*, const uint16_t*, const uint16_t*, void*, bool, int,
                                         int, int, const SegPlan&, float*, float*, float*, SeqLayout, int, hipStream_t);
template hipError_t launch_pdc<16, 16, 64>(const uint16_t*, const uint16_t*, const uint16_t*, void*, bool, int,
                                         int, int, const SegPlan&, float*, float*, float*, SeqLayout, int, hipStream_t);
template hipError_t launch_pdc<16, 16, 128>(const uint16_t*, const uint16_t*, const uint16_t*, void*, bool, int,
                                          int, int, const SegPlan&, float*, float*, float*, SeqLayout, int, hipStream_t);
}  // namespace chk
}  // namespace kata
