// The persistent matrix-core decode over an OCP e5m2 pool: the codes are converted exactly to
// bf16 (v_cvt_scalef32_pk_bf16_bf8) where the e4m3fn kernels convert theirs; everything else is
// the e4m3fn path (per-KV-head or per-page scales, bf16 or fp8 q, rotate-half RoPE).
#include "decode_persist.hpp"

namespace pdk {

template <int D, int PS, int GP, bool ROPE>
hipError_t launch_persist_e5m2(const DecodeParams& p, long long max_jobs, hipStream_t st) {
  return launch_persist_k<kFP8E5M2, D, PS, GP, ROPE, false>(p, max_jobs, st);
}

#define PDK_E5M2_GP(D, PS, ROPE)                                                                 \
  template hipError_t launch_persist_e5m2<D, PS, 1, ROPE>(const DecodeParams&, long long,        \
                                                          hipStream_t);                          \
  template hipError_t launch_persist_e5m2<D, PS, 2, ROPE>(const DecodeParams&, long long,        \
                                                          hipStream_t);                          \
  template hipError_t launch_persist_e5m2<D, PS, 4, ROPE>(const DecodeParams&, long long,        \
                                                          hipStream_t);                          \
  template hipError_t launch_persist_e5m2<D, PS, 8, ROPE>(const DecodeParams&, long long,        \
                                                          hipStream_t);
#define PDK_E5M2_SHAPES(ROPE) \
  PDK_E5M2_GP(64, 16, ROPE)   \
  PDK_E5M2_GP(64, 32, ROPE)   \
  PDK_E5M2_GP(128, 16, ROPE)  \
  PDK_E5M2_GP(128, 32, ROPE)

PDK_E5M2_SHAPES(false)
PDK_E5M2_SHAPES(true)

}  // namespace pdk
