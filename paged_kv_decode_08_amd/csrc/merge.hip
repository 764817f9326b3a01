// Pairwise attention-state merge in place (TVM relax decode-kernels page, _merge_state_inplace):
// s_max = max(s, s'); a = 2^(s - s_max); b = 2^(s' - s_max);
// v = v a / (a + b) + v' b / (a + b); s = log2(a + b) + s_max.
// One wavefront per (n, head) row; each lane handles head_dim / 64 (rounded up) elements.
#include "device.hpp"
#include "launch.hpp"

namespace pdk {

template <int VT>
__global__ __launch_bounds__(256) void merge_state_kernel(MergeParams p) {
  const int row = blockIdx.x * 4 + threadIdx.x / 64;
  const int lane = threadIdx.x % 64;
  if (row >= p.rows) return;
  const float s = p.s[row], so = p.s_other[row];
  const float s_max = fmaxf(s, so);
  const float a = exp2f(s - s_max), bw = exp2f(so - s_max);
  const float wa = a / (a + bw), wb = bw / (a + bw);
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
  if (lane == 0) p.s[row] = log2f(a + bw) + s_max;
}

hipError_t launch_merge_state(const MergeParams& p, int v_dtype, hipStream_t st) {
  const unsigned grid = (static_cast<unsigned>(p.rows) + 3) / 4;
  if (v_dtype == kF32) hipLaunchKernelGGL(merge_state_kernel<kF32>, dim3(grid), dim3(256), 0, st, p);
  else if (v_dtype == kBF16) hipLaunchKernelGGL(merge_state_kernel<kBF16>, dim3(grid), dim3(256), 0, st, p);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pdk
