// Split-KV completion inside the decode kernels. Every workgroup of a split (sequence, KV head)
// stores its normalised partial state (O_c, lse_c) for the G query heads with store_agent(),
// waits for those stores to complete, then takes a ticket from an agent-scope counter; the
// workgroup holding the last ticket merges all chunks by log-sum-exp (TVM relax decode-kernels page, _merge_state_inplace, applied over all chunks):
//   M = max_c lse_c, w_c = 2^(lse_c - M), out = sum_c w_c O_c / sum_c w_c, lse = M + log2(sum_c w_c)
// and puts the counter back to zero, so the workspace counters are zero between calls.
#pragma once

#include "device.hpp"

namespace pdk {

// Raw v_exp_f32: 2^x, results below the smallest normal flush to zero (softmax weights only).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Partial states cross workgroups (and XCDs): relaxed agent-scope atomic stores and loads.
__device__ __forceinline__ void store_agent(float* ptr, float v) {
  __hip_atomic_store(ptr, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_agent(const float* ptr) {
  return __hip_atomic_load(ptr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Merges the nch chunk states of (sequence b, KV head h), all stored and complete, into out and lse.
// Every thread of the workgroup takes part.
template <int QT, int D, int GP, int NT>
__device__ void merge_chunks(const DecodeParams& p, int b, int h, int nch) {
  __shared__ float s_mx[GP];
  __shared__ float s_w[GP][64];
  const int tid = threadIdx.x;
  const int G = p.G;
  const size_t row0 = (size_t(b) * p.H_qo + h * G) * p.num_chunks;  // head g: row0 + g * num_chunks
  // per-head maximum of the chunk lse values
  for (int g = tid / 64; g < G; g += NT / 64) {
    const int lane = tid & 63;
    float mx = -INFINITY;
    for (int c = lane; c < nch; c += 64) mx = fmaxf(mx, load_agent(&p.part_lse[row0 + size_t(g) * p.num_chunks + c]));
#pragma unroll
    for (int msk = 1; msk < 64; msk <<= 1) mx = fmaxf(mx, __shfl_xor(mx, msk, 64));
    if (lane == 0) s_mx[g] = mx;
  }
  constexpr int PER = (GP * D + NT - 1) / NT;
  float acc[PER], wsum[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) acc[k] = wsum[k] = 0.f;
  for (int c0 = 0; c0 < nch; c0 += 64) {
    __syncthreads();
    for (int idx = tid; idx < G * 64; idx += NT) {
      const int g = idx / 64, cc = idx % 64;
      const int cidx = c0 + cc;
      s_w[g][cc] = cidx < nch
          ? fast_exp2(load_agent(&p.part_lse[row0 + size_t(g) * p.num_chunks + cidx]) - s_mx[g]) : 0.f;
    }
    __syncthreads();
    const int cnt = min(64, nch - c0);
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int idx = tid + k * NT;
      if (idx >= G * D) break;
      const int g = idx / D, d = idx % D;
      const float* po = p.part_o + (row0 + size_t(g) * p.num_chunks + c0) * D + d;
      float a = acc[k], ws = wsum[k];
      // 8 chunks' loads issued together (one round trip per 8 chunks, not one per chunk)
      for (int cc = 0; cc < cnt; cc += 8) {
        float x[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) x[u] = cc + u < cnt ? load_agent(&po[size_t(cc + u) * D]) : 0.f;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          if (cc + u < cnt) {
            const float wc = s_w[g][cc + u];
            a = fmaf(wc, x[u], a);
            ws += wc;
          }
        }
      }
      acc[k] = a;
      wsum[k] = ws;
    }
  }
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int idx = tid + k * NT;
    if (idx >= G * D) break;
    const int g = idx / D, d = idx % D;
    const int hq = h * G + g;
    store_out<QT>(p.out, (size_t(b) * p.H_qo + hq) * D + d, acc[k] / wsum[k]);
    if (d == 0) p.lse[size_t(b) * p.H_qo + hq] = s_mx[g] + log2f(wsum[k]);
  }
}

template <int QT, int D, int GP, int NT>
__device__ void split_finish(const DecodeParams& p, int b, int h, int nch) {
  __shared__ int s_last;
  const int tid = threadIdx.x;
  // The partial states were stored as agent-scope atomics (coherent across the XCDs' L2s without
  // cache write-back). Drain them, then take the ticket.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (tid == 0) {
    int* cnt = &p.counters[b * p.H_kv + h];
    const int ticket = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = ticket == nch - 1;
    if (ticket == nch - 1) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (!s_last) return;
  merge_chunks<QT, D, GP, NT>(p, b, h, nch);
}

}  // namespace pdk
