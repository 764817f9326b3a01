// KV append (vLLM nki_flash_attn page, reshape_and_cache): token t's K and V rows go to
// pages[slot / page_size, 0|1, h, slot % page_size, :] for every KV head; a negative slot (or one
// past the pool) is skipped. fp8 pools store x / scale (fp32 division) rounded to the pool's
// format (e4m3fn, IEEE-style e4m3 or e5m2, nearest even, saturating).
// Vector form: a thread writes 16 bytes of one destination row (8 bf16, 4 fp32 or 16 fp8
// elements), threads in (token, K|V, head, vector) order, so the reads of the new rows are
// contiguous and each destination row is written whole. Rows that are not whole 16-byte vectors,
// or unaligned pointers, take the element form: one workgroup per token, one element per thread.
#include "device.hpp"
#include "launch.hpp"

#include <climits>

namespace pdk {

// Page and row of token t's slot; false for a skipped slot.
__device__ __forceinline__ bool append_slot(const AppendParams& p, int t, size_t& page, int& off) {
  const int slot = p.slots[t];
  if (slot < 0 || slot / p.PS >= p.max_num_pages) return false;
  page = static_cast<size_t>(slot / p.PS);
  off = slot % p.PS;
  return true;
}

// x (already divided by its scale) -> the code of fp8 pool type KVT
template <int KVT> __device__ __forceinline__ uint8_t encode_fp8(float x) {
  if constexpr (KVT == kFP8E4M3) return f32_to_fp8_e4m3(x);
  else if constexpr (KVT == kFP8E5M2) return f32_to_fp8_e5m2(x);
  else return f32_to_fp8(x);
}

template <int IT, int KVT>
__global__ __launch_bounds__(256) void append_vec_kernel(AppendParams p, int vpr, long long total) {
  constexpr int EPV = KVT == kF32 ? 4 : KVT == kBF16 ? 8 : 16;  // elements per 16-byte output
  const long long i = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int v = static_cast<int>(i % vpr);
  const long long r = i / vpr;            // (t, kv, h) row
  const int h = static_cast<int>(r % p.H_kv);
  const int kv = static_cast<int>((r / p.H_kv) % 2);
  const int t = static_cast<int>(r / (2 * p.H_kv));
  size_t page;
  int off;
  if (!append_slot(p, t, page, off)) return;
  const size_t src = (size_t(t) * p.H_kv + h) * p.D + size_t(v) * EPV;  // element index
  const size_t dst_row = ((page * 2 + kv) * p.H_kv + h) * p.PS + off;
  const void* in = kv ? p.new_v : p.new_k;
  uint4 o;
  if constexpr (KVT == kF32 || KVT == kBF16) {
    static_assert(IT == KVT, "same element type in and out");
    o = *reinterpret_cast<const uint4*>(static_cast<const char*>(in) + src * (KVT == kF32 ? 4 : 2));
  } else {
    const float sc = append_scale(p, kv, page, h);
    float x[16];
    if constexpr (IT == kF32) {
      const uint4* s4 = reinterpret_cast<const uint4*>(static_cast<const float*>(in) + src);
#pragma unroll
      for (int q = 0; q < 4; ++q) Kv<kF32>::unpack(s4[q], x + 4 * q);
    } else {
      const uint4* s4 = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(in) + src);
#pragma unroll
      for (int q = 0; q < 2; ++q) Kv<kBF16>::unpack(s4[q], x + 8 * q);
    }
    auto enc = [](float v) { return encode_fp8<KVT>(v); };
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      w[q] = uint32_t(enc(__fdiv_rn(x[4 * q], sc))) |
             uint32_t(enc(__fdiv_rn(x[4 * q + 1], sc))) << 8 |
             uint32_t(enc(__fdiv_rn(x[4 * q + 2], sc))) << 16 |
             uint32_t(enc(__fdiv_rn(x[4 * q + 3], sc))) << 24;
    o = make_uint4(w[0], w[1], w[2], w[3]);
  }
  reinterpret_cast<uint4*>(p.pages)[dst_row * vpr + v] = o;
}

template <int IT, int KVT>
__global__ __launch_bounds__(256) void append_kernel(AppendParams p) {
  const int t = blockIdx.x;
  size_t page;
  int off;
  if (!append_slot(p, t, page, off)) return;
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
      const float sc = append_scale(p, kv, page, h);
      const float y = __fdiv_rn(x, sc);
      static_cast<uint8_t*>(p.pages)[dst] = encode_fp8<KVT>(y);
    }
  }
}

template <int IT, int KVT>
static hipError_t launch_it(const AppendParams& p, hipStream_t st) {
  constexpr int OB = KVT == kF32 ? 4 : KVT == kBF16 ? 2 : 1;  // output bytes per element
  constexpr int IB = IT == kF32 ? 4 : 2;                      // input bytes per element
  const int row_bytes = p.D * OB;
  const uintptr_t a = reinterpret_cast<uintptr_t>(p.new_k) | reinterpret_cast<uintptr_t>(p.new_v) |
                      reinterpret_cast<uintptr_t>(p.pages);
  const long long total = static_cast<long long>(p.T) * 2 * p.H_kv * (row_bytes / 16);
  if (row_bytes % 16 == 0 && (p.D * IB) % 16 == 0 && a % 16 == 0 && (total + 255) / 256 <= INT_MAX) {
    const int vpr = row_bytes / 16;
    hipLaunchKernelGGL((append_vec_kernel<IT, KVT>), dim3(static_cast<unsigned>((total + 255) / 256)),
                       dim3(256), 0, st, p, vpr, total);
  } else {
    hipLaunchKernelGGL((append_kernel<IT, KVT>), dim3(static_cast<unsigned>(p.T)), dim3(256), 0, st, p);
  }
  return hipGetLastError();
}

hipError_t launch_append(const AppendParams& p, int in_dtype, int kv_dtype, hipStream_t st) {
  if (in_dtype == kF32 && kv_dtype == kF32) return launch_it<kF32, kF32>(p, st);
  if (in_dtype == kBF16 && kv_dtype == kBF16) return launch_it<kBF16, kBF16>(p, st);
  if (in_dtype == kBF16 && kv_dtype == kFP8) return launch_it<kBF16, kFP8>(p, st);
  if (in_dtype == kF32 && kv_dtype == kFP8) return launch_it<kF32, kFP8>(p, st);
  if (in_dtype == kBF16 && kv_dtype == kFP8E4M3) return launch_it<kBF16, kFP8E4M3>(p, st);
  if (in_dtype == kF32 && kv_dtype == kFP8E4M3) return launch_it<kF32, kFP8E4M3>(p, st);
  if (in_dtype == kBF16 && kv_dtype == kFP8E5M2) return launch_it<kBF16, kFP8E5M2>(p, st);
  if (in_dtype == kF32 && kv_dtype == kFP8E5M2) return launch_it<kF32, kFP8E5M2>(p, st);
  return hipErrorInvalidValue;
}

}  // namespace pdk
