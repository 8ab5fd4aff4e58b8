// bf16 MFMA chunked forward for KATA-Sigma 2 on 64-component queries and keys (reduced PSD
// families paragraph of the HTML page: psi(u) = u_1 u_1^T + u_2 u_2^T with 32-component
// blocks, weight sum_{a,b} (q_a . k_b)^2). The two blocks of a token are two consecutive
// 32-component rows of the same memory, so the full-map kernels for p = 32 run it over 2T
// "virtual" rows: the state sum_t sum_b psi_32(k_hat_{t,b}) v_t^T is exactly the Sigma 2
// state (528 x dv), and a token's readout and denominator are the sums over its two
// virtual query rows (kata_chunked.h, S2).
#include "kata_chunked.h"

namespace kata {

hipError_t launch_chunked_bf16_sigma2(const uint16_t* q, const uint16_t* k, const uint16_t* v, void* o,
                                      bool o_bf16, int B, int H, int T, int dv, int C, const SegPlan& plan,
                                      float* ws, float* s_out, float* z_out, const int* lens, hipStream_t st) {
#define KATA_S2CASE(DD, CC)                                                                        \
  if (dv == DD && C == CC)                                                                         \
    return chk::launch_pdc<32, DD, CC, true>(q, k, v, o, o_bf16, B, H, 2 * T, plan, ws, s_out, z_out,       \
                                             SeqLayout{lens, nullptr, 0}, PASS_SUMMARIES | PASS_SCAN | PASS_SEGMENTS, st);
  KATA_S2CASE(32, 64) KATA_S2CASE(32, 128) KATA_S2CASE(64, 64) KATA_S2CASE(64, 128)
#undef KATA_S2CASE
  return hipErrorInvalidValue;
}

}  // namespace kata
