// Paged-KV decode attention for bf16 or fp8-e4m3fn KV (bf16 q) on gfx950: q.K on the matrix cores,
// softmax and P.V on the vector ALUs. One workgroup of WAVES wavefronts per (sequence, KV head,
// chunk of page slots); wave w takes slots w, w + WAVES, ... of the chunk and the waves' states
// are merged at the end.
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
//    consecutive dims of NI consecutive rows (each V load instruction reads whole rows);
//    O[g][dims] accumulates in fp32 FMAs (bf16 V) or in v_dot2_f32_bf16 over row pairs (fp8 V:
//    two rows' bytes interleaved with v_perm, converted exactly to bf16, P rounded to bf16).
//  * fp8 K: each lane loads 16 codes of a row and converts them exactly to bf16 operands
//    (v_cvt_scalef32_pk_bf16_fp8, scale 1); k_scale multiplies the scores, v_scale the output.
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

template <int KVT> struct VVec;
template <> struct VVec<kBF16> { using type = uint4; };   // 8 bf16
template <> struct VVec<kFP8> { using type = uint2; };    // 8 e4m3fn codes

// Two packed e4m3fn codes (bytes 0,1 or 2,3 of w) -> two packed bf16 (exact).
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<int>(w), 1.0f, HI));
}
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};  // round to nearest even
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

template <int KVT, int D, int PS, int GP, int WAVES, int DEPTH>
__global__ __launch_bounds__(64 * WAVES) void decode_mfma_kernel(DecodeParams p) {
  constexpr bool FP8 = KVT == kFP8;
  constexpr int EB = FP8 ? 1 : 2;      // bytes per element
  constexpr int ROW = D * EB;          // bytes per row
  constexpr int BLOCK = PS * ROW;      // bytes of one (page, K|V, head) block
  constexpr int RB = PS / 16;          // 16-row blocks per page
  constexpr int KS = D / 32;           // MFMA k-steps over the head dim
  constexpr int KL = FP8 ? D / 64 : KS;  // 16-byte K loads per lane per 16-row block
  constexpr int NK = RB * KL;          // K loads per lane per page
  constexpr int VPR = D / 8;           // 8-element V vectors per row
  constexpr int RPI = 64 / VPR;        // V rows per load instruction
  constexpr int NI = PS / RPI;         // V loads per lane per page (consecutive rows)
  using VT = typename VVec<KVT>::type;
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
  const int cv = l % VPR;              // V layout: 8-element column
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
      store_out<kBF16>(p.out, (size_t(b) * p.H_qo + h * G) * D + idx, 0.f);  // out is bf16
    if (tid < G) p.lse[size_t(b) * p.H_qo + h * G + tid] = kEmptyLse;
    return;
  }
  if (c >= nch) return;
  const int s_begin = c * p.chunk_slots;
  const int s_end = (c == nch - 1) ? sg.n_slots : s_begin + p.chunk_slots;
  const int s_w = s_begin + w;                                       // this wave's first slot
  const int nw = s_w < s_end ? (s_end - s_w + WAVES - 1) / WAVES : 0;  // slots of this wave

  // q as the MFMA B operand: head n, for k-step j the 8 dims the K operand of k-group qg holds:
  // bf16 [32 j + 8 qg, +8); fp8 [64 (j/2) + 16 qg + 8 (j%2), +8).
  uint4 qop[KS];
  {
    const int nq = n < G ? n : 0;  // columns past the group are zero; never address past q
    const uint16_t* qb = static_cast<const uint16_t*>(p.q) + (size_t(b) * p.H_qo + h * G + nq) * D;
#pragma unroll
    for (int j = 0; j < KS; ++j) {
      const int d0 = FP8 ? 64 * (j / 2) + 16 * qg + 8 * (j % 2) : 32 * j + 8 * qg;
      qop[j] = n < G ? *reinterpret_cast<const uint4*>(qb + d0) : make_uint4(0, 0, 0, 0);
    }
  }
  const float kscale = FP8 ? p.k_scale[h] : 1.0f;
  const float vscale = FP8 ? p.v_scale[h] : 1.0f;

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
  auto issue = [&](uint4 (&kr)[NK], VT (&vr)[NI], int page) {
    const char* kb = pool + (size_t(page) * 2 * p.H_kv + h) * BLOCK;
    const char* vb = kb + size_t(p.H_kv) * BLOCK;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int j = 0; j < KL; ++j) {
        // bf16: 16 B = k-step j; fp8: 16 codes = k-steps 2j and 2j + 1
        const int off = FP8 ? 64 * j + 16 * qg : (4 * j + qg) * 16;
        kr[rb * KL + j] = *reinterpret_cast<const uint4*>(kb + (rb * 16 + n) * ROW + off);
      }
#pragma unroll
    for (int i = 0; i < NI; ++i)
      vr[i] = *reinterpret_cast<const VT*>(vb + (NI * rg + i) * ROW + cv * 8 * EB);
  };

  const float scale = p.score_scale * kscale;
  auto process = [&](const uint4 (&kr)[NK], const VT (&vr)[NI], int k) {
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
      for (int jj = 0; jj < KS; ++jj) {
        uint4 a;
        if constexpr (FP8) {
          const uint4 raw = kr[rb * KL + jj / 2];
          const uint32_t w0 = (jj % 2) ? raw.z : raw.x, w1 = (jj % 2) ? raw.w : raw.y;
          a = make_uint4(fp8x2_to_bf16x2<false>(w0), fp8x2_to_bf16x2<true>(w0),
                         fp8x2_to_bf16x2<false>(w1), fp8x2_to_bf16x2<true>(w1));
        } else {
          a = kr[rb * KS + jj];
        }
        acc[rb] = mfma_16x16x32_bf16(a, qop[jj], acc[rb]);
      }
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
    // this lane's rows of P, per head: fp32 (bf16 V) or bf16 row pairs (fp8 V)
    float pv[FP8 ? 1 : GP][NI];
    uint32_t pp[FP8 ? GP : 1][NI / 2];
#pragma unroll
    for (int g = 0; g < GP; ++g) {
      const float* src = &s_pt[w][g][NI * rg];
      float t[NI];
      if constexpr (NI == 2) {
        const float2 v2 = *reinterpret_cast<const float2*>(src);
        t[0] = v2.x; t[1] = v2.y;
      } else {
#pragma unroll
        for (int i4 = 0; i4 < NI; i4 += 4) {
          const float4 v4 = *reinterpret_cast<const float4*>(src + i4);
          t[i4] = v4.x; t[i4 + 1] = v4.y; t[i4 + 2] = v4.z; t[i4 + 3] = v4.w;
        }
      }
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        if constexpr (FP8) {
          if (i % 2) pp[g][i / 2] = pack_bf16x2(t[i - 1], t[i]);
        } else {
          pv[g][i] = t[i];
        }
      }
    }
    wave_lds_fence();
    const bool partial = lo > 0 || hi < PS;  // rows outside [lo, hi) may hold anything, even NaN
    if constexpr (FP8) {
      VT vv[NI];
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        vv[i] = vr[i];
        if (partial && !(NI * rg + i >= lo && NI * rg + i < hi)) vv[i] = make_uint2(0, 0);
      }
#pragma unroll
      for (int ip = 0; ip < NI / 2; ++ip) {
        // rows (2 ip, 2 ip + 1): P as a bf16 pair per head, V as a bf16 pair per dim
        const uint32_t a[2] = {vv[2 * ip].x, vv[2 * ip].y}, bb[2] = {vv[2 * ip + 1].x, vv[2 * ip + 1].y};
#pragma unroll
        for (int wi = 0; wi < 2; ++wi) {
          const uint32_t lo4 = __builtin_amdgcn_perm(bb[wi], a[wi], 0x05010400u);  // a0 b0 a1 b1
          const uint32_t hi4 = __builtin_amdgcn_perm(bb[wi], a[wi], 0x07030602u);  // a2 b2 a3 b3
          const uint32_t vp[4] = {fp8x2_to_bf16x2<false>(lo4), fp8x2_to_bf16x2<true>(lo4),
                                  fp8x2_to_bf16x2<false>(hi4), fp8x2_to_bf16x2<true>(hi4)};
#pragma unroll
          for (int g = 0; g < GP; ++g)
#pragma unroll
            for (int e = 0; e < 4; ++e) O[g][4 * wi + e] = dot2_bf16(pp[g][ip], vp[e], O[g][4 * wi + e]);
        }
      }
    } else {
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
    }
  };

  if (nw > 0) {
    // Ring of DEPTH + 1 register buffers: slot k is computed while slots k+1 .. k+DEPTH load.
    uint4 kbuf[DEPTH + 1][NK];
    VT vbuf[DEPTH + 1][NI];
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
    const float val = o / wsum * vscale;
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

template <int KVT, int D, int PS, int GP>
static hipError_t launch_w(const DecodeParams& p, unsigned grid, hipStream_t st) {
  constexpr int WAVES = PDK_MFMA_WAVES;
  constexpr int DEPTH = PDK_MFMA_DEPTH;
  hipLaunchKernelGGL((decode_mfma_kernel<KVT, D, PS, GP, WAVES, DEPTH>), dim3(grid),
                     dim3(64 * WAVES), 0, st, p);
  return hipGetLastError();
}

template <int KVT, int D, int PS>
static hipError_t launch_g(const DecodeParams& p, int gp, unsigned grid, hipStream_t st) {
  switch (gp) {
    case 1: return launch_w<KVT, D, PS, 1>(p, grid, st);
    case 2: return launch_w<KVT, D, PS, 2>(p, grid, st);
    case 4: return launch_w<KVT, D, PS, 4>(p, grid, st);
    case 8: return launch_w<KVT, D, PS, 8>(p, grid, st);
  }
  return hipErrorInvalidValue;
}

template <int KVT>
static hipError_t launch_kv(const DecodeParams& p, int D, int PS, int gp, unsigned grid,
                            hipStream_t st) {
  if (D == 64 && PS == 16) return launch_g<KVT, 64, 16>(p, gp, grid, st);
  if (D == 64 && PS == 32) return launch_g<KVT, 64, 32>(p, gp, grid, st);
  if (D == 128 && PS == 16) return launch_g<KVT, 128, 16>(p, gp, grid, st);
  if (D == 128 && PS == 32) return launch_g<KVT, 128, 32>(p, gp, grid, st);
  return hipErrorInvalidValue;
}

hipError_t launch_decode_mfma(const DecodeParams& p, int kv_dtype, int D, int PS, int gp,
                              unsigned grid, hipStream_t st) {
  if (kv_dtype == kBF16) return launch_kv<kBF16>(p, D, PS, gp, grid, st);
  if (kv_dtype == kFP8) return launch_kv<kFP8>(p, D, PS, gp, grid, st);
  return hipErrorInvalidValue;
}

}  // namespace pdk
