// KV append (vLLM nki_flash_attn page, reshape_and_cache): token t's K and V rows go to
// pages[slot / page_size, 0|1, h, slot % page_size, :] for every KV head; a negative slot (or one
// past the pool) is skipped. fp8 pools store x / scale[h] (fp32 division) rounded to e4m3fn.
// One workgroup per token; each thread moves one element.
#include "device.hpp"
#include "launch.hpp"

namespace pdk {

template <int IT, int KVT>
__global__ __launch_bounds__(256) void append_kernel(AppendParams p) {
  const int t = blockIdx.x;
  const int slot = p.slots[t];
  if (slot < 0 || slot / p.PS >= p.max_num_pages) return;
  const size_t page = static_cast<size_t>(slot / p.PS);
  const int off = slot % p.PS;
  const int per_kv = p.H_kv * p.D;
  for (int idx = threadIdx.x; idx < 2 * per_kv; idx += blockDim.x) {
    const int kv = idx / per_kv;
    const int h = (idx - kv * per_kv) / p.D;
    const int d = idx - kv * per_kv - h * p.D;
    const size_t src = (size_t(t) * p.H_kv + h) * p.D + d;
    const size_t dst = (((page * 2 + kv) * p.H_kv + h) * p.PS + off) * p.D + d;
    const void* in = kv ? p.new_v : p.new_k;
    if constexpr (KVT == kF32) {
      static_cast<float*>(p.pages)[dst] = static_cast<const float*>(in)[src];
    } else if constexpr (KVT == kBF16) {
      static_cast<uint16_t*>(p.pages)[dst] = static_cast<const uint16_t*>(in)[src];
    } else {
      const float x = load_q<IT>(in, src);
      const float sc = kv ? p.v_scale[h] : p.k_scale[h];
      static_cast<uint8_t*>(p.pages)[dst] = f32_to_fp8(__fdiv_rn(x, sc));
    }
  }
}

hipError_t launch_append(const AppendParams& p, int in_dtype, int kv_dtype, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(p.T)), block(256);
  if (in_dtype == kF32 && kv_dtype == kF32) hipLaunchKernelGGL((append_kernel<kF32, kF32>), grid, block, 0, st, p);
  else if (in_dtype == kBF16 && kv_dtype == kBF16) hipLaunchKernelGGL((append_kernel<kBF16, kBF16>), grid, block, 0, st, p);
  else if (in_dtype == kBF16 && kv_dtype == kFP8) hipLaunchKernelGGL((append_kernel<kBF16, kFP8>), grid, block, 0, st, p);
  else if (in_dtype == kF32 && kv_dtype == kFP8) hipLaunchKernelGGL((append_kernel<kF32, kFP8>), grid, block, 0, st, p);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pdk
