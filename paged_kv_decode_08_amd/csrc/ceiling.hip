// Streaming-read ceiling of the device: a plain coalesced read of a large buffer, for comparing a
// decode's KV bytes per second with what the memory system delivers to a kernel that does nothing
// but read. Not part of the decode path.
//
// Thread t of a grid of N threads reads the 16-byte vectors t, t + N, t + 2N, ... in rounds of U
// loads (all U issued before any is used). Adjacent lanes read adjacent vectors, so every load
// instruction of a wave covers 1 KiB of contiguous memory. The words read are folded with XOR into
// one 32-bit value per thread, written to `sink`, so no load can be dropped.
#include "pdecode_bench.h"

#include <hip/hip_runtime.h>

namespace {

constexpr int kThreads = 256;
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

template <int U, bool NT>
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const uint4* __restrict__ buf,
                                                               int64_t n_vec, uint32_t* sink) {
  const int64_t nthreads = int64_t(gridDim.x) * kThreads;
  const int64_t tid = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  uint32_t acc = 0;
  int64_t i = tid;
  for (; i + (U - 1) * nthreads < n_vec; i += U * nthreads) {
    uint4 x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if constexpr (NT) {
        const u32x4_t v =
            __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(buf + i + u * nthreads));
        x[u] = make_uint4(v[0], v[1], v[2], v[3]);
      } else {
        x[u] = buf[i + u * nthreads];
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= x[u].x ^ x[u].y ^ x[u].z ^ x[u].w;
  }
  for (; i < n_vec; i += nthreads) {
    const uint4 x = buf[i];
    acc ^= x.x ^ x.y ^ x.z ^ x.w;
  }
  sink[tid] = acc;
}

template <int U>
hipError_t launch_u(const uint4* buf, int64_t n_vec, bool nt, unsigned wgs, uint32_t* sink,
                    hipStream_t st) {
  if (nt)
    hipLaunchKernelGGL((stream_read_kernel<U, true>), dim3(wgs), dim3(kThreads), 0, st, buf,
                       n_vec, sink);
  else
    hipLaunchKernelGGL((stream_read_kernel<U, false>), dim3(wgs), dim3(kThreads), 0, st, buf,
                       n_vec, sink);
  return hipGetLastError();
}

}  // namespace

extern "C" pdecode_status pdecode_bench_stream_read(const void* buf, size_t bytes,
                                                    int32_t loads_per_lane, int32_t nontemporal,
                                                    int32_t workgroups, uint32_t* sink,
                                                    void* stream) {
  if (!buf || !sink || workgroups <= 0 || bytes < 16 || bytes % 16 != 0 ||
      reinterpret_cast<uintptr_t>(buf) % 16 != 0)
    return PDECODE_ERR_INVALID_ARG;
  const uint4* b = static_cast<const uint4*>(buf);
  const int64_t n_vec = static_cast<int64_t>(bytes / 16);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const unsigned wgs = static_cast<unsigned>(workgroups);
  const bool nt = nontemporal != 0;
  hipError_t e;
  switch (loads_per_lane) {
    case 1: e = launch_u<1>(b, n_vec, nt, wgs, sink, st); break;
    case 2: e = launch_u<2>(b, n_vec, nt, wgs, sink, st); break;
    case 4: e = launch_u<4>(b, n_vec, nt, wgs, sink, st); break;
    case 8: e = launch_u<8>(b, n_vec, nt, wgs, sink, st); break;
    case 16: e = launch_u<16>(b, n_vec, nt, wgs, sink, st); break;
    default: return PDECODE_ERR_UNSUPPORTED;
  }
  return e == hipSuccess ? PDECODE_OK : PDECODE_ERR_HIP;
}
