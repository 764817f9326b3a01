// Attention with the fused KV append (pdecode_append_attention): the FUSED instantiations of the
// persistent matrix-core decode kernel (decode_persist.hpp), built apart from decode_mfma.hip.
#include "decode_persist.hpp"

namespace pdk {

template <int KVT, int D, int PS, int GP, bool ROPE>
hipError_t launch_persist_fused(const DecodeParams& p, long long max_jobs, hipStream_t st) {
  return launch_persist_k<KVT, D, PS, GP, ROPE, true>(p, max_jobs, st);
}

// Every (KV dtype, head dim, page size, group bound, RoPE) the persistent schedule launches; RoPE
// included for bf16 and fp8 KV.
#define PDK_FUSED_GP(KVT, D, PS, ROPE)                                                            \
  template hipError_t launch_persist_fused<KVT, D, PS, 1, ROPE>(const DecodeParams&, long long,  \
                                                                hipStream_t);                    \
  template hipError_t launch_persist_fused<KVT, D, PS, 2, ROPE>(const DecodeParams&, long long,  \
                                                                hipStream_t);                    \
  template hipError_t launch_persist_fused<KVT, D, PS, 4, ROPE>(const DecodeParams&, long long,  \
                                                                hipStream_t);                    \
  template hipError_t launch_persist_fused<KVT, D, PS, 8, ROPE>(const DecodeParams&, long long,  \
                                                                hipStream_t);
#define PDK_FUSED_SHAPES(KVT, ROPE)  \
  PDK_FUSED_GP(KVT, 64, 16, ROPE)    \
  PDK_FUSED_GP(KVT, 64, 32, ROPE)    \
  PDK_FUSED_GP(KVT, 128, 16, ROPE)   \
  PDK_FUSED_GP(KVT, 128, 32, ROPE)

PDK_FUSED_SHAPES(kBF16, false)
PDK_FUSED_SHAPES(kBF16, true)
PDK_FUSED_SHAPES(kFP8, false)
PDK_FUSED_SHAPES(kFP8, true)

}  // namespace pdk
