// Pass 1 (segment summaries) of the bf16 chunked forward for p = 32, dv = 64, in a
// translation unit of its own: the build compiles it with the LLVM AMDGPU max-ILP
// scheduling strategy, which measured 6% faster for this kernel (and slower for the
// forward kernel, which keeps the default).
#include "kata_chunked.h"

namespace kata {
namespace chk {
template hipError_t launch_summary<32, 64, 32>(const Args&, unsigned, hipStream_t);
template hipError_t launch_summary<32, 64, 64>(const Args&, unsigned, hipStream_t);
template hipError_t launch_summary<32, 64, 128>(const Args&, unsigned, hipStream_t);
}  // namespace chk
}  // namespace kata
