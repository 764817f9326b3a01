// Paged-KV decode attention for bf16 KV on gfx950: q.K on the matrix cores, softmax and P.V on
// the vector ALUs. One workgroup of WAVES wavefronts per (sequence, KV head, chunk of page
// slots); wave w takes slots w, w + WAVES, ... of the chunk and the waves' states are merged at
// the end.
//
// Computation (TVM relax decode-kernels page, _attention_decode): score s = sm_scale * q . k kept
// in log2 units, online softmax with running max m and denominator d, output O / d and
// lse = m + log2(d); the waves' partial states are merged like the page's per-thread-group merge.
//
// Per page slot and wave (bf16, 16 rows x D):
//  * q.K: the G query heads of the KV head form the 16 columns of a v_mfma_f32_16x16x32_bf16 B
//    operand (unused columns zero). The K tile of 16 rows is the A operand straight from the
//    16-byte global loads: lane l holds row l % 16, elements [8 (4j + l/16), +8) for k-step j,
//    i.e. each load instruction reads 16 rows x 64 contiguous bytes. The accumulator gives lane l
//    the scores of rows 4 (l/16) + {0..3} for head l % 16.
//  * softmax: the tile max per head needs two cross-row exchanges; exp2 per score.
//  * P.V: P goes through LDS (transposed, [head][row]) to the V layout, where lane l holds 8
//    consecutive dims of NI consecutive rows (each V load instruction reads whole 256-byte rows);
//    O[g][dims] accumulates in fp32 FMAs.
// The next DEPTH slots' K and V are in flight while the current one is computed. A split sequence
// is finished by the last of its workgroups to arrive (split.hpp).
#include "device.hpp"
#include "launch.hpp"
#include "split.hpp"

#ifndef PDK_MFMA_WAVES
#define PDK_MFMA_WAVES 4  // wavefronts per workgroup (each takes every WAVES-th slot of the chunk)
#endif
#ifndef PDK_MFMA_DEPTH
#define PDK_MFMA_DEPTH 1  // slots in flight per wave besides the one being computed
#endif

namespace pdk {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma_16x16x32_bf16(const uint4& a, const uint4& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ float xmax(float v, int mask) {
  return fmaxf(v, __shfl_xor(v, mask, 64));
}

// Keeps the compiler from moving LDS accesses across this point; the LDS unit executes one
// wave's instructions in order, so this orders one wave's writes and reads of its own buffer.
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int D, int PS, int GP, int WAVES, int DEPTH>
__global__ __launch_bounds__(64 * WAVES) void decode_mfma_bf16_kernel(DecodeParams p) {
  constexpr int RB = PS / 16;          // 16-row blocks per page
  constexpr int KS = D / 32;           // MFMA k-steps over the head dim
  constexpr int NK = RB * KS;          // K loads (16 B) per lane per page
  constexpr int VPR = D / 8;           // 16-byte vectors per V row
  constexpr int RPI = 64 / VPR;        // V rows per load instruction
  constexpr int NI = PS / RPI;         // V loads per lane per page (consecutive rows)
  constexpr int BLOCK = PS * D * 2;    // bytes of one (page, K|V, head) block
  constexpr int ROW = D * 2;
  static_assert(GP <= 16 && (NI == 2 || NI % 4 == 0), "unsupported shape");

  __shared__ __attribute__((aligned(16))) float s_pt[WAVES][16][PS];  // P^T [head][row] per wave
  __shared__ float s_alpha[WAVES][16];
  __shared__ float s_m[WAVES][GP];
  __shared__ float s_d[WAVES][GP];
  __shared__ float s_o[WAVES][GP][D];

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int l = tid & 63;
  const int n = l & 15;                // MFMA layout: head column
  const int qg = l >> 4;               //              k-group / row quad
  const int cv = l % VPR;              // V layout: 16-byte column
  const int rg = l / VPR;              //           row group (rows NI*rg .. NI*rg + NI - 1)

  const int units = p.B * p.H_kv;
  const int c = blockIdx.x / units;
  const int u = blockIdx.x - c * units;
  const int b = u / p.H_kv;
  const int h = u - b * p.H_kv;
  const int G = p.G;

  const SeqGeom sg = seq_geom(p.indptr, p.length_info, p.B, b, PS, p.sliding);
  const int nch = chunks_used(sg.n_slots, p.chunk_slots, p.num_chunks);
  if (nch == 0) {
    if (c != 0) return;
    for (int idx = tid; idx < G * D; idx += 64 * WAVES)
      store_out<kBF16>(p.out, (size_t(b) * p.H_qo + h * G) * D + idx, 0.f);
    if (tid < G) p.lse[size_t(b) * p.H_qo + h * G + tid] = kEmptyLse;
    return;
  }
  if (c >= nch) return;
  const int s_begin = c * p.chunk_slots;
  const int s_end = (c == nch - 1) ? sg.n_slots : s_begin + p.chunk_slots;
  const int s_w = s_begin + w;                                       // this wave's first slot
  const int nw = s_w < s_end ? (s_end - s_w + WAVES - 1) / WAVES : 0;  // slots of this wave

  // q as the MFMA B operand: head n, elements [32 j + 8 qg, +8).
  uint4 qop[KS];
  {
    const int nq = n < G ? n : 0;  // columns past the group are zero; never address past q
    const uint16_t* qb = static_cast<const uint16_t*>(p.q) + (size_t(b) * p.H_qo + h * G + nq) * D;
#pragma unroll
    for (int j = 0; j < KS; ++j)
      qop[j] = n < G ? *reinterpret_cast<const uint4*>(qb + 32 * j + 8 * qg) : make_uint4(0, 0, 0, 0);
  }

  float m = -INFINITY;   // running max of head n (MFMA layout, identical across qg)
  float dl = 0.f;        // partial denominator over this lane's rows
  float O[GP][8];
#pragma unroll
  for (int g = 0; g < GP; ++g)
#pragma unroll
    for (int e = 0; e < 8; ++e) O[g][e] = 0.f;

  // Page ids of this wave's slots, 64 per coalesced load, two batches kept.
  auto slot_of = [&](int k) { return s_w + k * WAVES; };
  auto page_in_seq = [&](int s) { return s < sg.n0 ? s : sg.first1 + (s - sg.n0); };
  auto fetch_id = [&](int k) {
    int id = 0;
    if (k < nw) id = p.values[sg.beg + min(page_in_seq(slot_of(k)), sg.np - 1)];
    return min(max(id, 0), p.max_num_pages - 1);
  };
  int id_base = 0;
  int ids0 = fetch_id(l), ids1 = fetch_id(64 + l);
  auto page_of = [&](int k) {
    const int r = k - id_base;
    return r < 64 ? __builtin_amdgcn_readlane(ids0, r) : __builtin_amdgcn_readlane(ids1, r - 64);
  };

  const char* pool = static_cast<const char*>(p.pages);
  auto issue = [&](uint4 (&kr)[NK], uint4 (&vr)[NI], int page) {
    const char* kb = pool + (size_t(page) * 2 * p.H_kv + h) * BLOCK;
    const char* vb = kb + size_t(p.H_kv) * BLOCK;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int j = 0; j < KS; ++j)
        kr[rb * KS + j] = *reinterpret_cast<const uint4*>(kb + (rb * 16 + n) * ROW + (4 * j + qg) * 16);
#pragma unroll
    for (int i = 0; i < NI; ++i)
      vr[i] = *reinterpret_cast<const uint4*>(vb + (NI * rg + i) * ROW + cv * 16);
  };

  const float scale = p.score_scale;
  auto process = [&](const uint4 (&kr)[NK], const uint4 (&vr)[NI], int k) {
    const int s = slot_of(k);
    const int j = page_in_seq(s);
    int lo, hi;
    if (s < sg.n0) {
      lo = 0;
      hi = min(PS, sg.sink - j * PS);
    } else {
      lo = max(0, sg.win_off - j * PS);
      hi = min(PS, sg.total - j * PS);
    }
    // scores S^T[row][head] on the matrix cores
    f32x4_t acc[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      acc[rb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int jj = 0; jj < KS; ++jj) acc[rb] = mfma_16x16x32_bf16(kr[rb * KS + jj], qop[jj], acc[rb]);
    }
    float sv[RB][4];
    float tmax = -INFINITY;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = rb * 16 + 4 * qg + v;
        float x = acc[rb][v] * scale;
        x = (row >= lo && row < hi) ? x : -INFINITY;
        sv[rb][v] = x;
        tmax = fmaxf(tmax, x);
      }
    tmax = xmax(xmax(tmax, 16), 32);
    const float mn = fmaxf(m, tmax);
    const float alpha = fast_exp2(m - mn);
    m = mn;
    float psum = 0.f;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        sv[rb][v] = fast_exp2(sv[rb][v] - mn);
        psum += sv[rb][v];
      }
    dl = dl * alpha + psum;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
      *reinterpret_cast<float4*>(&s_pt[w][n][rb * 16 + 4 * qg]) =
          make_float4(sv[rb][0], sv[rb][1], sv[rb][2], sv[rb][3]);
    if (qg == 0) s_alpha[w][n] = alpha;
    const bool rescale = __ballot(alpha != 1.0f) != 0;
    wave_lds_fence();
    if (rescale) {
#pragma unroll
      for (int g = 0; g < GP; ++g) {
        const float a = s_alpha[w][g];
#pragma unroll
        for (int e = 0; e < 8; ++e) O[g][e] *= a;
      }
    }
    float pv[GP][NI];
#pragma unroll
    for (int g = 0; g < GP; ++g) {
      const float* src = &s_pt[w][g][NI * rg];
      if constexpr (NI == 2) {
        const float2 t = *reinterpret_cast<const float2*>(src);
        pv[g][0] = t.x; pv[g][1] = t.y;
      } else {
#pragma unroll
        for (int i4 = 0; i4 < NI; i4 += 4) {
          const float4 t = *reinterpret_cast<const float4*>(src + i4);
          pv[g][i4] = t.x; pv[g][i4 + 1] = t.y; pv[g][i4 + 2] = t.z; pv[g][i4 + 3] = t.w;
        }
      }
    }
    wave_lds_fence();
    const bool partial = lo > 0 || hi < PS;  // rows outside [lo, hi) may hold anything, even NaN
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      float vf[8];
      Kv<kBF16>::unpack(vr[i], vf);
      if (partial) {
        const bool ok = NI * rg + i >= lo && NI * rg + i < hi;
#pragma unroll
        for (int e = 0; e < 8; ++e) vf[e] = ok ? vf[e] : 0.f;
      }
#pragma unroll
      for (int g = 0; g < GP; ++g)
#pragma unroll
        for (int e = 0; e < 8; ++e) O[g][e] = fmaf(pv[g][i], vf[e], O[g][e]);
    }
  };

  if (nw > 0) {
    // Ring of DEPTH + 1 register buffers: slot k is computed while slots k+1 .. k+DEPTH load.
    uint4 kbuf[DEPTH + 1][NK], vbuf[DEPTH + 1][NI];
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) issue(kbuf[d], vbuf[d], page_of(min(d, nw - 1)));
    for (int k = 0; k < nw; k += DEPTH + 1) {
      if (k - id_base >= 64) {  // keep the ids of slots k .. k + 2 DEPTH at hand
        id_base += 64;
        ids0 = ids1;
        ids1 = fetch_id(id_base + 64 + l);
      }
#pragma unroll
      for (int r = 0; r <= DEPTH; ++r) {
        if (k + r >= nw) break;
        // unconditional, so the compiler's wait counts are static; past the end it re-reads the
        // last slot's blocks (cache hits)
        issue(kbuf[(r + DEPTH) % (DEPTH + 1)], vbuf[(r + DEPTH) % (DEPTH + 1)],
              page_of(min(k + r + DEPTH, nw - 1)));
        process(kbuf[r], vbuf[r], k + r);
      }
    }
  }

  // ---- per-wave totals: d over the row quads, O over the row groups
  dl += __shfl_xor(dl, 16, 64);
  dl += __shfl_xor(dl, 32, 64);
#pragma unroll
  for (int msk = VPR; msk < 64; msk <<= 1)
#pragma unroll
    for (int g = 0; g < GP; ++g)
#pragma unroll
      for (int e = 0; e < 8; ++e) O[g][e] += __shfl_xor(O[g][e], msk, 64);
  if (qg == 0 && n < GP) {
    s_m[w][n] = m;
    s_d[w][n] = dl;
  }
  if (rg == 0) {
#pragma unroll
    for (int g = 0; g < GP; ++g)
#pragma unroll
      for (int e = 0; e < 8; ++e) s_o[w][g][cv * 8 + e] = O[g][e];
  }
  __syncthreads();

  // ---- merge the waves' states and store (final output, or this chunk's partial state)
  for (int idx = tid; idx < G * D; idx += 64 * WAVES) {
    const int g = idx / D;
    const int d = idx - g * D;
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < WAVES; ++ww) M = fmaxf(M, s_m[ww][g]);
    float wsum = 0.f, o = 0.f;
#pragma unroll
    for (int ww = 0; ww < WAVES; ++ww) {
      const float f = fast_exp2(s_m[ww][g] - M);  // 0 for a wave without slots (m = -inf)
      wsum = fmaf(f, s_d[ww][g], wsum);
      o = fmaf(f, s_o[ww][g][d], o);
    }
    const int hq = h * G + g;
    const float val = o / wsum;
    const float l2 = M + log2f(wsum);
    if (nch == 1) {
      store_out<kBF16>(p.out, (size_t(b) * p.H_qo + hq) * D + d, val);
      if (d == 0) p.lse[size_t(b) * p.H_qo + hq] = l2;
    } else {
      const size_t row = (size_t(b) * p.H_qo + hq) * p.num_chunks + c;
      store_agent(&p.part_o[row * D + d], val);
      if (d == 0) store_agent(&p.part_lse[row], l2);
    }
  }
  if (nch > 1) split_finish<kBF16, D, GP, 64 * WAVES>(p, b, h, nch);
}

template <int D, int PS, int GP>
static hipError_t launch_w(const DecodeParams& p, unsigned grid, hipStream_t st) {
  constexpr int WAVES = PDK_MFMA_WAVES;
  constexpr int DEPTH = PDK_MFMA_DEPTH;
  hipLaunchKernelGGL((decode_mfma_bf16_kernel<D, PS, GP, WAVES, DEPTH>), dim3(grid),
                     dim3(64 * WAVES), 0, st, p);
  return hipGetLastError();
}

template <int D, int PS>
static hipError_t launch_g(const DecodeParams& p, int gp, unsigned grid, hipStream_t st) {
  switch (gp) {
    case 1: return launch_w<D, PS, 1>(p, grid, st);
    case 2: return launch_w<D, PS, 2>(p, grid, st);
    case 4: return launch_w<D, PS, 4>(p, grid, st);
    case 8: return launch_w<D, PS, 8>(p, grid, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode_mfma_bf16(const DecodeParams& p, int D, int PS, int gp, unsigned grid,
                                   hipStream_t st) {
  if (D == 64 && PS == 16) return launch_g<64, 16>(p, gp, grid, st);
  if (D == 64 && PS == 32) return launch_g<64, 32>(p, gp, grid, st);
  if (D == 128 && PS == 16) return launch_g<128, 16>(p, gp, grid, st);
  if (D == 128 && PS == 32) return launch_g<128, 32>(p, gp, grid, st);
  return hipErrorInvalidValue;
}

}  // namespace pdk
