// Split-KV merge: combines the normalised partial states that the decode kernels write for a
// sequence split into several chunks (TVM relax decode-kernels page, _merge_state_inplace, applied
// over all chunks at once).
#include "device.hpp"
#include "launch.hpp"

namespace pdk {

// Combines the normalised partial states of every split sequence by log-sum-exp:
// M = max_c lse_c, w_c = 2^(lse_c - M), out = sum_c w_c O_c / sum_c w_c, lse = M + log2(sum w_c).
// Sequences that used a single chunk were finalised by the decode kernel and are skipped.
template <int QT, int D, int PS>
__global__ __launch_bounds__(64) void split_merge_kernel(DecodeParams p) {
  const int lane = threadIdx.x;
  const int b = blockIdx.x / p.H_qo;
  const int hq = blockIdx.x - b * p.H_qo;
  const SeqGeom sg = seq_geom(p.indptr, p.length_info, p.B, b, PS, p.sliding);
  const int nch = chunks_used(sg.n_slots, p.chunk_slots, p.num_chunks);
  if (nch <= 1) return;
  const size_t row0 = (size_t(b) * p.H_qo + hq) * p.num_chunks;
  float M = -INFINITY;
  for (int c = lane; c < nch; c += 64) M = fmaxf(M, p.part_lse[row0 + c]);
#pragma unroll
  for (int msk = 1; msk < 64; msk <<= 1) M = fmaxf(M, __shfl_xor(M, msk, 64));
  constexpr int PER = D / 64;
  float acc[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) acc[k] = 0.f;
  float W = 0.f;
  for (int c0 = 0; c0 < nch; c0 += 64) {
    // weights of 64 chunks at once, one per lane, then broadcast one by one
    const int cl = c0 + lane;
    const float wl = cl < nch ? exp2f(p.part_lse[row0 + cl] - M) : 0.f;
    W += wl;
    const int cnt = min(64, nch - c0);
    const float* po = p.part_o + (row0 + c0) * D + lane;
#pragma unroll 8
    for (int k = 0; k < cnt; ++k) {
      const float wk = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wl), k));
#pragma unroll
      for (int kk = 0; kk < PER; ++kk) acc[kk] = fmaf(wk, po[size_t(k) * D + 64 * kk], acc[kk]);
    }
  }
#pragma unroll
  for (int msk = 1; msk < 64; msk <<= 1) W += __shfl_xor(W, msk, 64);
  const float inv = 1.0f / W;
  const size_t ob = (size_t(b) * p.H_qo + hq) * D;
#pragma unroll
  for (int k = 0; k < PER; ++k) store_out<QT>(p.out, ob + lane + 64 * k, acc[k] * inv);
  if (lane == 0) p.lse[size_t(b) * p.H_qo + hq] = M + log2f(W);
}

template <int QT, int D>
static hipError_t launch_merge_ps(const DecodeParams& p, int PS, unsigned grid, hipStream_t st) {
  if (PS == 16) hipLaunchKernelGGL((split_merge_kernel<QT, D, 16>), dim3(grid), dim3(64), 0, st, p);
  else if (PS == 32) hipLaunchKernelGGL((split_merge_kernel<QT, D, 32>), dim3(grid), dim3(64), 0, st, p);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_split_merge(const DecodeParams& p, int q_dtype, int D, int PS, hipStream_t st) {
  const unsigned grid = static_cast<unsigned>(p.B) * p.H_qo;
  if (q_dtype == kF32 && D == 64) return launch_merge_ps<kF32, 64>(p, PS, grid, st);
  if (q_dtype == kF32 && D == 128) return launch_merge_ps<kF32, 128>(p, PS, grid, st);
  if (q_dtype == kBF16 && D == 64) return launch_merge_ps<kBF16, 64>(p, PS, grid, st);
  if (q_dtype == kBF16 && D == 128) return launch_merge_ps<kBF16, 128>(p, PS, grid, st);
  return hipErrorInvalidValue;
}

}  // namespace pdk
