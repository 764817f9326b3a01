// Pairwise attention-state merge in place (TVM relax decode-kernels page, _merge_state_inplace):
// s_max = max(s, s'); a = 2^(s - s_max); b = 2^(s' - s_max);
// v = v a / (a + b) + v' b / (a + b); s = log2(a + b) + s_max.
// Vector form: a lane moves 16 bytes (8 bf16 or 4 fp32 elements) of a (n, head) row, a wave holds
// 64 / VPR whole rows (VPR = 16-byte vectors per row), so a row's s is read by all its lanes before
// one of them writes it back, in one wave. Rows whose bytes are not whole 16-byte vectors, or
// unaligned pointers, take the element form: one wave per row, one element per lane per step.
#include "device.hpp"
#include "launch.hpp"

namespace pdk {

__device__ __forceinline__ void merge_weights(float s, float so, float& wa, float& wb, float& s_new) {
  const float s_max = fmaxf(s, so);
  const float a = exp2f(s - s_max), bw = exp2f(so - s_max);
  wa = a / (a + bw);
  wb = bw / (a + bw);
  s_new = log2f(a + bw) + s_max;
}

template <int VT>
__global__ __launch_bounds__(256) void merge_state_vec_kernel(MergeParams p, int vpr, int rows_per_wave) {
  constexpr int EPV = VT == kF32 ? 4 : 8;  // elements per 16-byte vector
  const int wave = blockIdx.x * 4 + threadIdx.x / 64;
  const int lane = threadIdx.x % 64;
  const int r_in = lane / vpr, v = lane - r_in * vpr;
  const int row = wave * rows_per_wave + r_in;
  if (r_in >= rows_per_wave || row >= p.rows) return;
  float wa, wb, s_new;
  merge_weights(p.s[row], p.s_other[row], wa, wb, s_new);
  const size_t off = size_t(row) * vpr + v;
  uint4* dst = static_cast<uint4*>(p.v) + off;
  const uint4 x = *dst;
  const uint4 y = static_cast<const uint4*>(p.v_other)[off];
  float fx[EPV], fy[EPV];
  Kv<VT>::unpack(x, fx);
  Kv<VT>::unpack(y, fy);
  uint4 o;
  if constexpr (VT == kF32) {
    o = make_uint4(__float_as_uint(fx[0] * wa + fy[0] * wb), __float_as_uint(fx[1] * wa + fy[1] * wb),
                   __float_as_uint(fx[2] * wa + fy[2] * wb), __float_as_uint(fx[3] * wa + fy[3] * wb));
  } else {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = uint32_t(f32_to_bf16(fx[2 * i] * wa + fy[2 * i] * wb)) |
             uint32_t(f32_to_bf16(fx[2 * i + 1] * wa + fy[2 * i + 1] * wb)) << 16;
    o = make_uint4(w[0], w[1], w[2], w[3]);
  }
  *dst = o;
  if (v == 0) p.s[row] = s_new;
}

template <int VT>
__global__ __launch_bounds__(256) void merge_state_kernel(MergeParams p) {
  const int row = blockIdx.x * 4 + threadIdx.x / 64;
  const int lane = threadIdx.x % 64;
  if (row >= p.rows) return;
  float wa, wb, s_new;
  merge_weights(p.s[row], p.s_other[row], wa, wb, s_new);
  const size_t base = size_t(row) * p.D;
  for (int d = lane; d < p.D; d += 64) {
    float x, y;
    if constexpr (VT == kF32) {
      x = static_cast<const float*>(p.v)[base + d];
      y = static_cast<const float*>(p.v_other)[base + d];
    } else {
      x = bf16_to_f32(static_cast<const uint16_t*>(p.v)[base + d]);
      y = bf16_to_f32(static_cast<const uint16_t*>(p.v_other)[base + d]);
    }
    store_out<VT>(p.v, base + d, x * wa + y * wb);
  }
  if (lane == 0) p.s[row] = s_new;
}

template <int VT>
static hipError_t launch_vt(const MergeParams& p, hipStream_t st) {
  const int eb = VT == kF32 ? 4 : 2;
  const int row_bytes = p.D * eb;
  const bool aligned = (reinterpret_cast<uintptr_t>(p.v) | reinterpret_cast<uintptr_t>(p.v_other)) % 16 == 0;
  if (aligned && row_bytes % 16 == 0 && row_bytes / 16 <= 64) {
    const int vpr = row_bytes / 16;
    const int rpw = 64 / vpr;
    const long long waves = (static_cast<long long>(p.rows) + rpw - 1) / rpw;
    hipLaunchKernelGGL(merge_state_vec_kernel<VT>, dim3(static_cast<unsigned>((waves + 3) / 4)),
                       dim3(256), 0, st, p, vpr, rpw);
  } else {
    const unsigned grid = (static_cast<unsigned>(p.rows) + 3) / 4;
    hipLaunchKernelGGL(merge_state_kernel<VT>, dim3(grid), dim3(256), 0, st, p);
  }
  return hipGetLastError();
}

hipError_t launch_merge_state(const MergeParams& p, int v_dtype, hipStream_t st) {
  if (v_dtype == kF32) return launch_vt<kF32>(p, st);
  if (v_dtype == kBF16) return launch_vt<kBF16>(p, st);
  return hipErrorInvalidValue;
}

}  // namespace pdk
