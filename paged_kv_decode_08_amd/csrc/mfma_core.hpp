// Per-wave building blocks of the matrix-core decode kernels (bf16 or fp8-e4m3fn KV, bf16 q).
//
// Computation (TVM relax decode-kernels page, _attention_decode): score s = sm_scale * q . k kept in
// log2 units, online softmax with running max m and denominator d, output O / d and
// lse = m + log2(d).
//
// One wave handles one page slot of one (sequence, KV head) at a time:
//  * q.K: the G query heads of the KV head form the 16 columns of a v_mfma_f32_16x16x32_bf16 B
//    operand (unused columns zero). The K tile of 16 rows is the A operand straight from the
//    16-byte global loads: lane l holds row l % 16; bf16: elements [8 (4j + l/16), +8) for k-step
//    j; fp8: 16 codes [64 j' + 16 (l/16), +16) converted exactly to bf16 for k-steps 2j', 2j'+1.
//    The accumulator gives lane l the scores of rows 4 (l/16) + {0..3} for head l % 16.
//  * softmax: the tile max per head needs two cross-row exchanges; one exp2 per score.
//  * P.V: P goes through LDS (transposed, [head][row]) to the V layout, where lane l holds 8
//    consecutive dims of NI consecutive rows (each V load instruction reads whole rows);
//    O[g][dims] accumulates in fp32 FMAs (bf16 V, up to 4 heads) or in v_dot2_f32_bf16 over row
//    pairs with P rounded to bf16 (fp8 V: two rows' bytes interleaved with v_perm, converted
//    exactly to bf16; bf16 V with 8 heads: two rows' elements regrouped with v_perm).
//  * fp8: k_scale multiplies the scores, v_scale the output.
//  * RoPE (ROPE = true): rotate-half pairs dims i and i + D/2, and the MFMA layout puts both in
//    the same lane (k-steps j and j + KS/2; fp8 codes are converted exactly to fp32 first), except
//    for fp8 at D = 64, where the partner is in lane l ^ 32 and is fetched with a lane exchange
//    (XLANE); so q (once per job) and each K row (per item)
//    are rotated in registers in fp32 (angles: rope_cs_hw). The rotated values no longer
//    fit bf16, so each is split into a bf16 high part and a bf16 remainder, and the scores take
//    three products: q_hi.k_hi + q_hi.k_lo + q_lo.k_hi (the dropped q_lo.k_lo is below 2^-16 of
//    the score).
//  * rows outside the attended range [lo, hi) of a page are masked out of the scores and their V
//    entries zeroed before use (an unused slot may hold anything, NaN included).
#pragma once

#include "device.hpp"

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


// Raw v_exp_f32: 2^x, results below the smallest normal flush to zero (softmax weights only).
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

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
  return __builtin_bit_cast(uint32_t,
                            __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<int>(w), 1.0f, HI));
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

// Splits x into a bf16 high part and a bf16 remainder (x - hi), both rounded to nearest even.
__device__ __forceinline__ void split_bf16(float x, float y, uint32_t& hi, uint32_t& lo) {
  hi = pack_bf16x2(x, y);
  lo = pack_bf16x2(x - bf16_lo(hi), y - bf16_hi(hi));
}

// ILV (with ROPE): the interleaved RoPE layout, pairs (2i, 2i + 1), both in the 8 consecutive
// dims a lane holds per k-step.
template <int KVT, int D, int PS, int GP, bool ROPE = false, bool ILV = false>
struct MfmaCore {
  static constexpr bool FP8 = KVT == kFP8;
  static constexpr int EB = FP8 ? 1 : 2;        // bytes per element
  static constexpr int ROW = D * EB;            // bytes per row
  static constexpr int BLOCK = PS * ROW;        // bytes of one (page, K|V, head) block
  static constexpr int RB = PS / 16;            // 16-row blocks per page
  static constexpr int KS = D / 32;             // MFMA k-steps over the head dim
  static constexpr int KL = FP8 ? D / 64 : KS;  // 16-byte K loads per lane per 16-row block
  static constexpr int NK = RB * KL;            // K loads per lane per page
  static constexpr int VPR = D / 8;             // 8-element V vectors per row
  static constexpr int RPI = 64 / VPR;          // V rows per load instruction
  static constexpr int NI = PS / RPI;           // V loads per lane per page (consecutive rows)
  static constexpr int NLOADS = NK + NI;        // vector-memory instructions per page
  static constexpr int PT_STRIDE = PS + 4;      // P^T row stride in floats (bank-conflict-free)
  using VT = typename VVec<KVT>::type;
  static_assert(GP <= 16 && (NI == 2 || NI % 4 == 0), "unsupported shape");
  static_assert(!ROPE || RB == 1, "RoPE on the matrix cores: 16-row items");
  static constexpr int KH = KS / 2;             // k-steps of the lower half of the head dim
  // Rotate-half RoPE finds dims i and i + D/2 in one lane for bf16, and for fp8 at D = 128; fp8 at
  // D = 64 holds dims [16 qg, +16) per lane, so each dim's partner sits in lane l ^ 32.
  static constexpr bool XLANE = ROPE && !ILV && FP8 && D == 64;
  // P.V with P rounded to bf16 and row pairs through v_dot2_f32_bf16: fp8 V always, bf16 V with 8
  // heads (fp32 P for 8 heads would take the kernel past 256 VGPRs, one wave per SIMD)
  static constexpr bool PBF16 = FP8 || GP >= 8;

  struct Buf {
    uint4 k[NK];
    VT v[NI];
  };

  int l, n, qg, cv, rg;  // lane coordinates: MFMA layout (n, qg), V layout (cv, rg)
  uint4 qop[KS];         // q as the MFMA B operand (with RoPE: the bf16 high part)
  uint4 qlo[ROPE ? KS : 1];  // with RoPE: the bf16 remainder of the rotated q
  float m;               // running max of head n (MFMA layout, identical across qg)
  float dl;              // partial denominator over this lane's rows
  float O[GP][8];

  __device__ __forceinline__ void init_lane(int lane) {
    l = lane;
    n = l & 15;
    qg = l >> 4;
    cv = l % VPR;
    rg = l / VPR;
  }

  __device__ __forceinline__ void reset() {
    m = -INFINITY;
    dl = 0.f;
#pragma unroll
    for (int g = 0; g < GP; ++g)
#pragma unroll
      for (int e = 0; e < 8; ++e) O[g][e] = 0.f;
  }

  // Element offset, within one q row, of the 8 dims that k-step j of k-group qg holds:
  // bf16 [32 j + 8 qg, +8); fp8 [64 (j/2) + 16 qg + 8 (j%2), +8).
  __device__ __forceinline__ int q_dim0(int j) const {
    return FP8 ? 64 * (j / 2) + 16 * qg + 8 * (j % 2) : 32 * j + 8 * qg;
  }

  // q rows of the G heads from a contiguous [G][D] bf16 block (global or LDS); columns past G
  // are zero and never addressed.
  __device__ __forceinline__ void load_q(const uint16_t* rows, int G) {
    const uint16_t* qr = rows + (n < G ? n : 0) * D;
#pragma unroll
    for (int j = 0; j < KS; ++j)
      qop[j] = n < G ? *reinterpret_cast<const uint4*>(qr + q_dim0(j)) : make_uint4(0, 0, 0, 0);
  }

  // The 8 fp8 codes of k-step jj (even: words x, y; odd: z, w) of a 16-code load, in fp32.
  __device__ __forceinline__ static void fp8_kstep(const uint4& raw, int jj, float (&x)[8]) {
    const uint32_t w0 = (jj % 2) ? raw.z : raw.x, w1 = (jj % 2) ? raw.w : raw.y;
    fp8x2_to_f32<false>(w0, x[0], x[1]);
    fp8x2_to_f32<true>(w0, x[2], x[3]);
    fp8x2_to_f32<false>(w1, x[4], x[5]);
    fp8x2_to_f32<true>(w1, x[6], x[7]);
  }

  // The 8 K elements of k-step jj of this lane's row, in fp32 (fp8 codes convert exactly).
  __device__ __forceinline__ void kstep_f32(const Buf& bf, int jj, float (&x)[8]) const {
    if constexpr (FP8) fp8_kstep(bf.k[jj / 2], jj, x);
    else Kv<kBF16>::unpack(bf.k[jj], x);
  }

  // The same words of lane l ^ 32 (the other half of the wave).
  __device__ __forceinline__ static uint4 other_half(const uint4& v) {
    return make_uint4(uint32_t(__shfl_xor(int(v.x), 32)), uint32_t(__shfl_xor(int(v.y), 32)),
                      uint32_t(__shfl_xor(int(v.z), 32)), uint32_t(__shfl_xor(int(v.w), 32)));
  }

  // XLANE rotate-half at position pos: x holds this lane's 8 dims of k-step j, xp the same
  // k-step of lane l ^ 32, i.e. the dims D/2 away. Lanes of the lower half (qg < 2) compute
  // x c - xp s, the upper half x c + xp s; the result is split into bf16 high parts and
  // remainders.
  __device__ __forceinline__ void rope_xlane(const float (&x)[8], const float (&xp)[8], int j,
                                             int pos, const float2* s_freq, uint4& hi,
                                             uint4& lo) const {
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float2 f = s_freq[(q_dim0(j) + e) % (D / 2)];
      float c, sn;
      rope_cs_hw(pos, f.x, f.y, c, sn);
      y[e] = qg < 2 ? x[e] * c - xp[e] * sn : x[e] * c + xp[e] * sn;
    }
    uint32_t h[4], l4[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) split_bf16(y[2 * e], y[2 * e + 1], h[e], l4[e]);
    hi = make_uint4(h[0], h[1], h[2], h[3]);
    lo = make_uint4(l4[0], l4[1], l4[2], l4[3]);
  }

  // Rotates the q operand to position qpos (RoPE) and splits it into qop (high) and qlo.
  // s_freq[i] = (fhi, flo) of frequency i (rope_freq).
  __device__ __forceinline__ void rope_q(int qpos, const float2* s_freq) {
    if constexpr (ROPE && ILV) {
#pragma unroll
      for (int j = 0; j < KS; ++j) {
        float x[8], y[8];
        Kv<kBF16>::unpack(qop[j], x);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float2 f = s_freq[q_dim0(j) / 2 + e];
          float c, sn;
          rope_cs_hw(qpos, f.x, f.y, c, sn);
          y[2 * e] = x[2 * e] * c - x[2 * e + 1] * sn;
          y[2 * e + 1] = x[2 * e + 1] * c + x[2 * e] * sn;
        }
        uint32_t h[4], lo[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) split_bf16(y[2 * e], y[2 * e + 1], h[e], lo[e]);
        qop[j] = make_uint4(h[0], h[1], h[2], h[3]);
        qlo[j] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
      }
    } else if constexpr (XLANE) {
#pragma unroll
      for (int j = 0; j < KS; ++j) {
        float x[8], xp[8];
        Kv<kBF16>::unpack(qop[j], x);
        Kv<kBF16>::unpack(other_half(qop[j]), xp);
        rope_xlane(x, xp, j, qpos, s_freq, qop[j], qlo[j]);
      }
    } else if constexpr (ROPE) {
#pragma unroll
      for (int j = 0; j < KH; ++j) {
        float x1[8], x2[8];
        Kv<kBF16>::unpack(qop[j], x1);
        Kv<kBF16>::unpack(qop[j + KH], x2);
        float y1[8], y2[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float2 f = s_freq[q_dim0(j) + e];
          float c, sn;
          rope_cs_hw(qpos, f.x, f.y, c, sn);
          y1[e] = x1[e] * c - x2[e] * sn;
          y2[e] = x2[e] * c + x1[e] * sn;
        }
        uint32_t h1[4], l1[4], h2[4], l2[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          split_bf16(y1[2 * e], y1[2 * e + 1], h1[e], l1[e]);
          split_bf16(y2[2 * e], y2[2 * e + 1], h2[e], l2[e]);
        }
        qop[j] = make_uint4(h1[0], h1[1], h1[2], h1[3]);
        qlo[j] = make_uint4(l1[0], l1[1], l1[2], l1[3]);
        qop[j + KH] = make_uint4(h2[0], h2[1], h2[2], h2[3]);
        qlo[j + KH] = make_uint4(l2[0], l2[1], l2[2], l2[3]);
      }
    }
  }

  // Issues the K and V loads of one (page, head) block pair.
  __device__ __forceinline__ void issue(Buf& bf, const char* kb, size_t kv_stride) const {
    const char* vb = kb + kv_stride;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int j = 0; j < KL; ++j) {
        // bf16: 16 B = k-step j; fp8: 16 codes = k-steps 2j and 2j + 1
        const int off = FP8 ? 64 * j + 16 * qg : (4 * j + qg) * 16;
        bf.k[rb * KL + j] = kv_load(reinterpret_cast<const uint4*>(kb + (rb * 16 + n) * ROW + off));
      }
#pragma unroll
    for (int i = 0; i < NI; ++i)
      bf.v[i] = kv_load(reinterpret_cast<const VT*>(vb + (NI * rg + i) * ROW + cv * 8 * EB));
  }

  // Fused append: row rn of the item (loaded from the pool, whatever it held) is replaced by the
  // staged new row `row` (K then V, ROW bytes each, in the pool's element type), in the registers
  // that issue() loads it into.
  __device__ __forceinline__ void substitute(Buf& bf, int rn, const uint32_t* row) const {
    static_assert(RB == 1, "16-row items");
    const uint4* nk = reinterpret_cast<const uint4*>(row);
    const char* nv = reinterpret_cast<const char*>(row) + ROW;
    if (n == rn) {
#pragma unroll
      for (int j = 0; j < KL; ++j) bf.k[j] = nk[4 * j + qg];  // bytes 16 (4 j + qg), as issue()
    }
#pragma unroll
    for (int i = 0; i < NI; ++i)
      if (NI * rg + i == rn) bf.v[i] = *reinterpret_cast<const VT*>(nv + cv * 8 * EB);
  }

  // Online-softmax update with one page whose attended rows are [lo, hi) (lo < hi).
  // s_pt: this wave's [16][PT_STRIDE] P^T tile; s_alpha: this wave's 16 rescale factors.
  // RoPE: row r of the item is at position pos0 + r; s_freq as in rope_q.
  // COLCAP (several query tokens): this lane's column also masks the rows above `cap`, so a
  // column may have no row left in the item, or in the whole job so far (m = -inf).
  template <bool COLCAP = false>
  __device__ __forceinline__ void process(const Buf& bf, int lo, int hi, float scale,
                                          float (*s_pt)[PT_STRIDE], float* s_alpha, int pos0 = 0,
                                          const float2* s_freq = nullptr, int cap = 15) {
    // scores S^T[row][head] on the matrix cores
    f32x4_t acc[RB];
    if constexpr (ROPE) {
      // this lane's K row (n) rotated to its position, split into high parts and remainders
      uint4 khi[KS], klo[KS];
      if constexpr (ILV) {
#pragma unroll
        for (int j = 0; j < KS; ++j) {
          float x[8], y[8];
          kstep_f32(bf, j, x);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float2 f = s_freq[q_dim0(j) / 2 + e];
            float c, sn;
            rope_cs_hw(pos0 + n, f.x, f.y, c, sn);
            y[2 * e] = x[2 * e] * c - x[2 * e + 1] * sn;
            y[2 * e + 1] = x[2 * e + 1] * c + x[2 * e] * sn;
          }
          uint32_t h[4], lo[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) split_bf16(y[2 * e], y[2 * e + 1], h[e], lo[e]);
          khi[j] = make_uint4(h[0], h[1], h[2], h[3]);
          klo[j] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
        }
      } else if constexpr (XLANE) {
        const uint4 oth = other_half(bf.k[0]);  // one 16-code load per row at D = 64
#pragma unroll
        for (int j = 0; j < KS; ++j) {
          float x[8], xp[8];
          fp8_kstep(bf.k[0], j, x);
          fp8_kstep(oth, j, xp);
          rope_xlane(x, xp, j, pos0 + n, s_freq, khi[j], klo[j]);
        }
      } else {
#pragma unroll
      for (int j = 0; j < KH; ++j) {
        float x1[8], x2[8];
        kstep_f32(bf, j, x1);
        kstep_f32(bf, j + KH, x2);
        float y1[8], y2[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float2 f = s_freq[q_dim0(j) + e];
          float c, sn;
          rope_cs_hw(pos0 + n, f.x, f.y, c, sn);
          y1[e] = x1[e] * c - x2[e] * sn;
          y2[e] = x2[e] * c + x1[e] * sn;
        }
        uint32_t h1[4], l1[4], h2[4], l2[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          split_bf16(y1[2 * e], y1[2 * e + 1], h1[e], l1[e]);
          split_bf16(y2[2 * e], y2[2 * e + 1], h2[e], l2[e]);
        }
        khi[j] = make_uint4(h1[0], h1[1], h1[2], h1[3]);
        klo[j] = make_uint4(l1[0], l1[1], l1[2], l1[3]);
        khi[j + KH] = make_uint4(h2[0], h2[1], h2[2], h2[3]);
        klo[j + KH] = make_uint4(l2[0], l2[1], l2[2], l2[3]);
        if constexpr (COLCAP) {
          // several tokens: each rotated k-step pair goes to the matrix cores at once, so the
          // rotated K pieces are not all live together (the 8-column kernel is at 256 VGPRs)
          if (j == 0) acc[0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int jj = j; jj < KS; jj += KH) {
            acc[0] = mfma_16x16x32_bf16(khi[jj], qop[jj], acc[0]);
            acc[0] = mfma_16x16x32_bf16(klo[jj], qop[jj], acc[0]);
            acc[0] = mfma_16x16x32_bf16(khi[jj], qlo[jj], acc[0]);
          }
        }
      }
      }
      if constexpr (!COLCAP || ILV || XLANE) {
        acc[0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int jj = 0; jj < KS; ++jj) {
          acc[0] = mfma_16x16x32_bf16(khi[jj], qop[jj], acc[0]);
          acc[0] = mfma_16x16x32_bf16(klo[jj], qop[jj], acc[0]);
          acc[0] = mfma_16x16x32_bf16(khi[jj], qlo[jj], acc[0]);
        }
      }
    } else {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        acc[rb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int jj = 0; jj < KS; ++jj) {
          uint4 a;
          if constexpr (FP8) {
            const uint4 raw = bf.k[rb * KL + jj / 2];
            const uint32_t w0 = (jj % 2) ? raw.z : raw.x, w1 = (jj % 2) ? raw.w : raw.y;
            a = make_uint4(fp8x2_to_bf16x2<false>(w0), fp8x2_to_bf16x2<true>(w0),
                           fp8x2_to_bf16x2<false>(w1), fp8x2_to_bf16x2<true>(w1));
          } else {
            a = bf.k[rb * KS + jj];
          }
          acc[rb] = mfma_16x16x32_bf16(a, qop[jj], acc[rb]);
        }
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
        x = (row >= lo && row < hi && (!COLCAP || row <= cap)) ? x : -INFINITY;
        sv[rb][v] = x;
        tmax = fmaxf(tmax, x);
      }
    tmax = xmax(xmax(tmax, 16), 32);
    const float mn = fmaxf(m, tmax);  // finite unless COLCAP: the page has an attended row
    // a column with no row yet keeps m = -inf, O = 0, d = 0 (reference 0: every weight is 0)
    const float mref = COLCAP && mn == -INFINITY ? 0.f : mn;
    const float alpha = exp2_fast(m - mref);
    m = mn;
    float psum = 0.f;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        sv[rb][v] = exp2_fast(sv[rb][v] - mref);
        psum += sv[rb][v];
      }
    dl = dl * alpha + psum;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
      *reinterpret_cast<float4*>(&s_pt[n][rb * 16 + 4 * qg]) =
          make_float4(sv[rb][0], sv[rb][1], sv[rb][2], sv[rb][3]);
    if (qg == 0) s_alpha[n] = alpha;
    const bool rescale = __ballot(alpha != 1.0f) != 0;
    wave_lds_fence();
    if (rescale) {
#pragma unroll
      for (int g = 0; g < GP; ++g) {
        const float a = s_alpha[g];
#pragma unroll
        for (int e = 0; e < 8; ++e) O[g][e] *= a;
      }
    }
    // this lane's rows of P, per head: fp32 (bf16 V) or bf16 row pairs (fp8 V)
    float pv[PBF16 ? 1 : GP][NI];
    uint32_t pp[PBF16 ? GP : 1][NI / 2];
#pragma unroll
    for (int g = 0; g < GP; ++g) {
      const float* src = &s_pt[g][NI * rg];
      float t[NI];
      if constexpr (NI == 2) {
        const float2 v2 = *reinterpret_cast<const float2*>(src);
        t[0] = v2.x;
        t[1] = v2.y;
      } else {
#pragma unroll
        for (int i4 = 0; i4 < NI; i4 += 4) {
          const float4 v4 = *reinterpret_cast<const float4*>(src + i4);
          t[i4] = v4.x;
          t[i4 + 1] = v4.y;
          t[i4 + 2] = v4.z;
          t[i4 + 3] = v4.w;
        }
      }
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        if constexpr (PBF16) {
          if (i % 2) pp[g][i / 2] = pack_bf16x2(t[i - 1], t[i]);
        } else {
          pv[g][i] = t[i];
        }
      }
    }
    wave_lds_fence();
    const bool partial = lo > 0 || hi < PS;
    if constexpr (FP8) {
      VT vv[NI];
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        vv[i] = bf.v[i];
        if (partial && !(NI * rg + i >= lo && NI * rg + i < hi)) vv[i] = make_uint2(0, 0);
      }
#pragma unroll
      for (int ip = 0; ip < NI / 2; ++ip) {
        // rows (2 ip, 2 ip + 1): P as a bf16 pair per head, V as a bf16 pair per dim
        const uint32_t a[2] = {vv[2 * ip].x, vv[2 * ip].y};
        const uint32_t bb[2] = {vv[2 * ip + 1].x, vv[2 * ip + 1].y};
#pragma unroll
        for (int wi = 0; wi < 2; ++wi) {
          const uint32_t lo4 = __builtin_amdgcn_perm(bb[wi], a[wi], 0x05010400u);  // a0 b0 a1 b1
          const uint32_t hi4 = __builtin_amdgcn_perm(bb[wi], a[wi], 0x07030602u);  // a2 b2 a3 b3
          const uint32_t vp[4] = {fp8x2_to_bf16x2<false>(lo4), fp8x2_to_bf16x2<true>(lo4),
                                  fp8x2_to_bf16x2<false>(hi4), fp8x2_to_bf16x2<true>(hi4)};
#pragma unroll
          for (int g = 0; g < GP; ++g)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              O[g][4 * wi + e] = dot2_bf16(pp[g][ip], vp[e], O[g][4 * wi + e]);
        }
      }
    } else if constexpr (PBF16) {
      VT vv[NI];
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        vv[i] = bf.v[i];
        if (partial && !(NI * rg + i >= lo && NI * rg + i < hi)) vv[i] = make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int ip = 0; ip < NI / 2; ++ip) {
        // rows (2 ip, 2 ip + 1): P as a bf16 pair per head; V dims (2w, 2w + 1) of both rows
        // regrouped into one bf16 pair per dim
        const uint32_t a[4] = {vv[2 * ip].x, vv[2 * ip].y, vv[2 * ip].z, vv[2 * ip].w};
        const uint32_t bb[4] = {vv[2 * ip + 1].x, vv[2 * ip + 1].y, vv[2 * ip + 1].z,
                                vv[2 * ip + 1].w};
#pragma unroll
        for (int wi = 0; wi < 4; ++wi) {
          const uint32_t d0 = __builtin_amdgcn_perm(bb[wi], a[wi], 0x05040100u);  // a.lo b.lo
          const uint32_t d1 = __builtin_amdgcn_perm(bb[wi], a[wi], 0x07060302u);  // a.hi b.hi
#pragma unroll
          for (int g = 0; g < GP; ++g) {
            O[g][2 * wi] = dot2_bf16(pp[g][ip], d0, O[g][2 * wi]);
            O[g][2 * wi + 1] = dot2_bf16(pp[g][ip], d1, O[g][2 * wi + 1]);
          }
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        float vf[8];
        Kv<kBF16>::unpack(bf.v[i], vf);
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
  }

  // Reduces this wave's state over its lanes (d over the row quads, O over the row groups) and
  // writes it to the wave's slots of the workgroup merge buffers.
  __device__ __forceinline__ void to_lds(float* s_m, float* s_d, float (*s_o)[D]) {
    float d = dl;
    d += __shfl_xor(d, 16, 64);
    d += __shfl_xor(d, 32, 64);
#pragma unroll
    for (int msk = VPR; msk < 64; msk <<= 1)
#pragma unroll
      for (int g = 0; g < GP; ++g)
#pragma unroll
        for (int e = 0; e < 8; ++e) O[g][e] += __shfl_xor(O[g][e], msk, 64);
    if (qg == 0 && n < GP) {
      s_m[n] = m;
      s_d[n] = d;
    }
    if (rg == 0) {
#pragma unroll
      for (int g = 0; g < GP; ++g) {
        *reinterpret_cast<float4*>(&s_o[g][cv * 8]) = make_float4(O[g][0], O[g][1], O[g][2], O[g][3]);
        *reinterpret_cast<float4*>(&s_o[g][cv * 8 + 4]) =
            make_float4(O[g][4], O[g][5], O[g][6], O[g][7]);
      }
    }
  }
};

// Attended rows [lo, hi) of page slot s of a sequence (slots [0, n0) are the sink pages, the rest
// cover positions [win_off, total)), and the index j of that page in the sequence's page list.
// (Value selects, no branches: keeps the geometry in registers.)
__device__ __forceinline__ void slot_rows(const SeqGeom& g, int s, int PS, int& j, int& lo, int& hi) {
  const bool sink_slot = s < g.n0;
  const int sink = g.sink, total = g.total, win_off = g.win_off, first1 = g.first1, n0 = g.n0;
  j = sink_slot ? s : first1 + (s - n0);
  lo = sink_slot ? 0 : max(0, win_off - j * PS);
  hi = min(PS, (sink_slot ? sink : total) - j * PS);
}

}  // namespace pdk
