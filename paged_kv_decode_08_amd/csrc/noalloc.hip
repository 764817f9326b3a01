// pdecode_attention_noalloc: pdecode_attention for callers that cannot allocate (code under HIP
// graph capture, tight serving loops, harnesses that forbid hipMalloc). The split counters, the
// job-queue counters and the split partial states live in a file-scope device array instead of a
// caller workspace; each GPU holds its own copy of the array until the process ends.
//
// Layout of the array: a counter region (kScratchCounterBytes) at offset 0, then the partial-state
// region (kScratchPartialBytes). The counters sit at the same place in every call, so the zero
// state that every call leaves behind (the loader zero-fills the array, and the first call on a
// device clears the region once more) is never overwritten by partial states.
#include <hip/hip_runtime.h>

#include <mutex>

#include "api_internal.hpp"
#include "pdecode.h"

namespace {
constexpr size_t kScratchCounterBytes = size_t(64) << 10;  // 16384 int32: B * H_kv + 2 counters
constexpr size_t kScratchPartialBytes = size_t(32) << 20;  // split partial states (O and lse)
constexpr int kMaxDevices = 64;
}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchCounterBytes + kScratchPartialBytes];

namespace {

__global__ void clear_counters_kernel(int* counters, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x)
    counters[i] = 0;
}

std::mutex g_mu;
unsigned char* g_ptr[kMaxDevices];  // device address of `scratch` on each device (null: not yet)

// The device address of `scratch` on device `dev` (current), taken once per device; the first
// call also clears the counter region on `st`. Returns null on a HIP error.
unsigned char* scratch_on(int dev, hipStream_t st) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_ptr[dev]) return g_ptr[dev];
  void* ptr = nullptr;
  if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
    return nullptr;
  const int n = static_cast<int>(kScratchCounterBytes / sizeof(int));
  hipLaunchKernelGGL(clear_counters_kernel, dim3(16), dim3(256), 0, st, static_cast<int*>(ptr), n);
  if (hipGetLastError() != hipSuccess) return nullptr;
  g_ptr[dev] = static_cast<unsigned char*>(ptr);
  return g_ptr[dev];
}

}  // namespace

extern "C" pdecode_status pdecode_attention_noalloc(const pdecode_desc* d, const void* q,
                                                    const void* pages,
                                                    const int32_t* page_indptr,
                                                    const int32_t* page_values,
                                                    const int32_t* length_info,
                                                    const pdecode_rope* rope, float sm_scale,
                                                    void* out, float* lse, void* stream) {
  // every host-side check first (arguments, plan against the scratch regions): nothing touches
  // the device for a call that is refused
  const pdk::FixedScratch sizes{nullptr, kScratchCounterBytes, nullptr, kScratchPartialBytes};
  pdecode_status st = pdk::attention_fixed_scratch(d, q, pages, page_indptr, page_values,
                                                   length_info, rope, sm_scale, out, lse, &sizes,
                                                   stream, /*check_only=*/true);
  if (st != PDECODE_OK || d->batch == 0) return st;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PDECODE_ERR_HIP;
  hipStream_t s = static_cast<hipStream_t>(stream);
  unsigned char* base = scratch_on(dev, s);
  if (!base) return PDECODE_ERR_HIP;
  const pdk::FixedScratch fs{reinterpret_cast<int*>(base), kScratchCounterBytes,
                             reinterpret_cast<float*>(base + kScratchCounterBytes),
                             kScratchPartialBytes};
  return pdk::attention_fixed_scratch(d, q, pages, page_indptr, page_values, length_info, rope,
                                      sm_scale, out, lse, &fs, stream, /*check_only=*/false);
}
