// Decode with several query tokens per sequence (pdecode_attention_multi): the MT instantiations
// of the persistent matrix-core decode kernel (decode_persist.hpp), built apart from
// decode_mfma.hip. The G q heads of a KV head times the T tokens fill up to 16 columns of the MFMA
// B operand (group bound GP 2, 4, 8 or 16). With RoPE (rotate-half or interleaved), token t of a
// sequence is rotated t positions after the sequence's first query position.
#include "decode_persist.hpp"

namespace pdk {

template <int KVT, int D, int PS, int GP, bool ROPE>
hipError_t launch_persist_multi(const DecodeParams& p, long long max_jobs, hipStream_t st) {
  if constexpr (GP < 2) return hipErrorInvalidValue;
  else if constexpr (ROPE) {
    if (p.rotary == 2)  // interleaved pairs
      return launch_persist_k<KVT, D, PS, GP, true, false, true, true>(p, max_jobs, st);
    return launch_persist_k<KVT, D, PS, GP, true, false, true>(p, max_jobs, st);
  } else {
    return launch_persist_k<KVT, D, PS, GP, false, false, true>(p, max_jobs, st);
  }
}

#define PDK_MULTI(KVT, D, PS, GP, ROPE)                                                           \
  template hipError_t launch_persist_multi<KVT, D, PS, GP, ROPE>(const DecodeParams&, long long, \
                                                                 hipStream_t);
#define PDK_MULTI_GP(KVT, D, PS, ROPE) \
  PDK_MULTI(KVT, D, PS, 1, ROPE)       \
  PDK_MULTI(KVT, D, PS, 2, ROPE)       \
  PDK_MULTI(KVT, D, PS, 4, ROPE)       \
  PDK_MULTI(KVT, D, PS, 8, ROPE)       \
  PDK_MULTI(KVT, D, PS, 16, ROPE)
#define PDK_MULTI_SHAPES(KVT, ROPE)  \
  PDK_MULTI_GP(KVT, 64, 16, ROPE)    \
  PDK_MULTI_GP(KVT, 64, 32, ROPE)    \
  PDK_MULTI_GP(KVT, 128, 16, ROPE)   \
  PDK_MULTI_GP(KVT, 128, 32, ROPE)

PDK_MULTI_SHAPES(kBF16, false)
PDK_MULTI_SHAPES(kBF16, true)
PDK_MULTI_SHAPES(kFP8, false)
PDK_MULTI_SHAPES(kFP8, true)

}  // namespace pdk
