// Instantiations of the bf16 chunked forward for p = 32, dv = 64 (see kata_chunked.h).
#include "kata_chunked.h"

namespace kata {
namespace chk {
// pass 1 of this shape is compiled in kata_summary_p32_dv64.hip
extern template hipError_t launch_summary<32, 64, 32>(const Args&, unsigned, hipStream_t);
extern template hipError_t launch_summary<32, 64, 64>(const Args&, unsigned, hipStream_t);
extern template hipError_t launch_summary<32, 64, 128>(const Args&, unsigned, hipStream_t);
template hipError_t launch_pdc<32, 64, 32>(const uint16_t*, const uint16_t*, const uint16_t*, void*, bool, int,
                                         int, int, const SegPlan&, float*, float*, float*, SeqLayout, int, hipStream_t);
template hipError_t launch_pdc<32, 64, 64>(const uint16_t*, const uint16_t*, const uint16_t*, void*, bool, int,
                                         int, int, const SegPlan&, float*, float*, float*, SeqLayout, int, hipStream_t);
template hipError_t launch_pdc<32, 64, 128>(const uint16_t*, const uint16_t*, const uint16_t*, void*, bool, int,
                                          int, int, const SegPlan&, float*, float*, float*, SeqLayout, int, hipStream_t);
}  // namespace chk
}  // namespace kata
