// Decode with interleaved RoPE (rotary_mode 2, pairs (2i, 2i + 1)): the ILV instantiations of the
// persistent matrix-core decode kernel (decode_persist.hpp), plain and with the fused append,
// built apart from decode_mfma.hip.
#include "decode_persist.hpp"

namespace pdk {

template <int KVT, int D, int PS, int GP>
hipError_t launch_persist_ilv(const DecodeParams& p, long long max_jobs, hipStream_t st) {
  // with the fused append: the new row is substituted in its raw form, before the rotation
  if (p.new_k != nullptr)
    return launch_persist_k<KVT, D, PS, GP, true, true, false, true>(p, max_jobs, st);
  return launch_persist_k<KVT, D, PS, GP, true, false, false, true>(p, max_jobs, st);
}

#define PDK_ILV(KVT, D, PS, GP)                                                                    \
  template hipError_t launch_persist_ilv<KVT, D, PS, GP>(const DecodeParams&, long long,           \
                                                         hipStream_t);
#define PDK_ILV_GP(KVT, D, PS) \
  PDK_ILV(KVT, D, PS, 1)       \
  PDK_ILV(KVT, D, PS, 2)       \
  PDK_ILV(KVT, D, PS, 4)       \
  PDK_ILV(KVT, D, PS, 8)
#define PDK_ILV_SHAPES(KVT)  \
  PDK_ILV_GP(KVT, 64, 16)    \
  PDK_ILV_GP(KVT, 64, 32)    \
  PDK_ILV_GP(KVT, 128, 16)   \
  PDK_ILV_GP(KVT, 128, 32)

PDK_ILV_SHAPES(kBF16)
PDK_ILV_SHAPES(kFP8)

}  // namespace pdk
