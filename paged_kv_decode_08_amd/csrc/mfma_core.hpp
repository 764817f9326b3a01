// Per-wave building blocks of the matrix-core decode kernels (bf16, fp8-e4m3fn or fp8-e5m2 KV,
// bf16 q).
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
//  * softmax: the tile max per head needs two cross-row exchanges (v_permlane16/32_swap); one
//    exp2 per score.
//  * P.V on the matrix cores too: O^T[dims][heads] += V^T P, one v_mfma_f32_16x16x16_bf16 per 16
//    dims. P is the B operand as it stands in the score accumulator (lane l: rows 4 (l/16) + {0..3}
//    of head l % 16), rounded to bf16. V (lane l loads 8 consecutive dims of NI consecutive rows,
//    so each load instruction reads whole rows; fp8 codes are converted exactly to bf16) goes to
//    a per-wave LDS tile and is read back transposed with ds_read_b64_tr_b16 as the A operand.
//    The accumulators hold the 16 columns' outputs whatever the number of heads, and the rescale
//    of a column's output by its softmax correction is lane-local.
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

typedef short i16x4_t __attribute__((ext_vector_type(4)));
// v_mfma_f32_16x16x16_bf16: A lane l = A[m = l % 16][k = 4 (l / 16) .. + 4], B lane l =
// B[k = 4 (l / 16) .. + 4][n = l % 16], accumulator lane l = D[m = 4 (l / 16) + v][n = l % 16].
__device__ __forceinline__ f32x4_t mfma_16x16x16_bf16(const i16x4_t& a, const uint2& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, __builtin_bit_cast(i16x4_t, b), c, 0, 0, 0);
}

// ds_read_b64_tr_b16: within each group of 16 lanes, lane i receives element i % 4 of the 8-byte
// chunks that lanes 4e + i / 4 address, for e = 0..3 (measured on gfx950).
__device__ __forceinline__ i16x4_t lds_read_tr16(const unsigned char* p) {
  typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
}



// max / sum of v over lanes l and l ^ 16 (ROWS = 16) or l ^ 32 (ROWS = 32), on the VALU:
// v_permlane16_swap / v_permlane32_swap with v in both operands return the lane's own value and
// its partner's (in an order that depends on the lane: the max and the sum do not care).
template <int ROWS>
__device__ __forceinline__ float xmax(float v) {
  const uint32_t u = __float_as_uint(v);
  const auto p = ROWS == 16 ? __builtin_amdgcn_permlane16_swap(u, u, false, false)
                            : __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
template <int ROWS>
__device__ __forceinline__ float xsum(float v) {
  const uint32_t u = __float_as_uint(v);
  const auto p = ROWS == 16 ? __builtin_amdgcn_permlane16_swap(u, u, false, false)
                            : __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
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
template <> struct VVec<kFP8E5M2> { using type = uint2; };  // 8 e5m2 codes

// Two packed e4m3fn codes (E5M2: e5m2 codes) (bytes 0,1 or 2,3 of w) -> two packed bf16 (exact:
// bf16 has the exponent range and mantissa bits of both formats, subnormals included).
template <bool HI, bool E5M2 = false>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  if constexpr (E5M2)
    return __builtin_bit_cast(uint32_t,
                              __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(static_cast<int>(w), 1.0f, HI));
  else
    return __builtin_bit_cast(uint32_t,
                              __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<int>(w), 1.0f, HI));
}
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};  // round to nearest even
  return __builtin_bit_cast(uint32_t, v);
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
  static constexpr bool E5M2 = KVT == kFP8E5M2;  // fp8 codes are e5m2, else e4m3fn
  static constexpr bool FP8 = KVT == kFP8 || E5M2;
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
  // P.V on the matrix cores: V goes through a per-wave LDS tile [16 rows][VSTRIDE bytes] of
  // bf16 (rows padded by 32 bytes against bank conflicts of the transposed reads) and comes back
  // transposed as the A operand; P stays in registers.
  static constexpr int VSTRIDE = D * 2 + 32;
  static constexpr int TILE_BYTES = 16 * VSTRIDE;  // this wave's V tile
  static constexpr int NB = D / 16;             // 16-dim blocks of the output
  using VT = typename VVec<KVT>::type;
  static_assert(GP <= 16 && (NI == 2 || NI % 4 == 0), "unsupported shape");
  static_assert(RB == 1, "16-row items");
  static constexpr int KH = KS / 2;             // k-steps of the lower half of the head dim
  // Rotate-half RoPE finds dims i and i + D/2 in one lane for bf16, and for fp8 at D = 128; fp8 at
  // D = 64 holds dims [16 qg, +16) per lane, so each dim's partner sits in lane l ^ 32.
  static constexpr bool XLANE = ROPE && !ILV && FP8 && D == 64;

  struct Buf {
    uint4 k[NK];
    VT v[NI];
    float ks, vs;  // fp8 pools with per-page scales: the item's (page, KV head) K and V scales
  };

  int l, n, qg, cv, rg;  // lane coordinates: MFMA layout (n, qg), V layout (cv, rg)
  uint4 qop[KS];         // q as the MFMA B operand (with RoPE: the bf16 high part)
  uint4 qlo[ROPE ? KS : 1];  // with RoPE: the bf16 remainder of the rotated q
  float m;               // running max of head n (MFMA layout, identical across qg)
  float dl;              // partial denominator over this lane's rows
  f32x4_t OT[NB];         // O^T of head (column) n: dims 16 b + 4 qg + v of block b

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
    for (int b = 0; b < NB; ++b) OT[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
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
    fp8x2_to_f32<false, E5M2>(w0, x[0], x[1]);
    fp8x2_to_f32<true, E5M2>(w0, x[2], x[3]);
    fp8x2_to_f32<false, E5M2>(w1, x[4], x[5]);
    fp8x2_to_f32<true, E5M2>(w1, x[6], x[7]);
  }

  // The 8 K elements of k-step jj of this lane's row, in fp32 (fp8 codes convert exactly).
  __device__ __forceinline__ void kstep_f32(const Buf& bf, int jj, float (&x)[8]) const {
    if constexpr (FP8) fp8_kstep(bf.k[jj / 2], jj, x);
    else Kv<kBF16>::unpack(bf.k[jj], x);
  }

  // The same words of lane l ^ 32 (the other half of the wave).
  // (v_permlane32_swap with v in both operands returns (own, partner) in the lower half of the
  // wave and (partner, own) in the upper half)
  __device__ __forceinline__ uint4 other_half(const uint4& v) const {
    const bool lo = l < 32;
    auto part = [lo](uint32_t x) {
      const auto p = __builtin_amdgcn_permlane32_swap(x, x, false, false);
      return lo ? p[1] : p[0];
    };
    return make_uint4(part(v.x), part(v.y), part(v.z), part(v.w));
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
  // tile: this wave's LDS V tile (TILE_BYTES, 16-byte aligned).
  // RoPE: row r of the item is at position pos0 + r; s_freq as in rope_q.
  // COLCAP (several query tokens): this lane's column also masks the rows above `cap`, so a
  // column may have no row left in the item, or in the whole job so far (m = -inf).
  template <bool COLCAP = false>
  // vf: a factor on this item's V rows (an fp8 pool's per-page V scale), applied to P.
  __device__ __forceinline__ void process(const Buf& bf, int lo, int hi, float scale,
                                          unsigned char* tile, int pos0 = 0,
                                          const float2* s_freq = nullptr, int cap = 15,
                                          float vf = 1.f) {
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
            a = make_uint4(fp8x2_to_bf16x2<false, E5M2>(w0), fp8x2_to_bf16x2<true, E5M2>(w0),
                           fp8x2_to_bf16x2<false, E5M2>(w1), fp8x2_to_bf16x2<true, E5M2>(w1));
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
    tmax = xmax<32>(xmax<16>(tmax));
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
    // O^T[dims][head n] += V^T . P on the matrix cores. P (this lane: rows 4 qg .. + 4 of head n,
    // where the QK accumulator left them) is the B operand as bf16; V goes to this wave's LDS tile
    // (rows outside [lo, hi) as zeros: 0 x NaN would poison O) and comes back transposed, 16 dims
    // per read, as the A operand.
    const float pf = FP8 ? vf : 1.f;  // the denominator dl above takes P without it
    const uint2 pb = make_uint2(pack_bf16x2(sv[0][0] * pf, sv[0][1] * pf),
                                pack_bf16x2(sv[0][2] * pf, sv[0][3] * pf));
    if (__ballot(alpha != 1.0f) != 0) {
#pragma unroll
      for (int b = 0; b < NB; ++b) OT[b] *= alpha;
    }
    const bool partial = lo > 0 || hi < PS;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int row = NI * rg + i;
      uint4 x;
      if constexpr (FP8) {
        const uint2 c8 = bf.v[i];
        x = make_uint4(fp8x2_to_bf16x2<false, E5M2>(c8.x), fp8x2_to_bf16x2<true, E5M2>(c8.x),
                       fp8x2_to_bf16x2<false, E5M2>(c8.y), fp8x2_to_bf16x2<true, E5M2>(c8.y));
      } else {
        x = bf.v[i];
      }
      if (partial && !(row >= lo && row < hi)) x = make_uint4(0, 0, 0, 0);
      *reinterpret_cast<uint4*>(tile + row * VSTRIDE + cv * 16) = x;
    }
    wave_lds_fence();
    const unsigned char* src = tile + (4 * qg + n / 4) * VSTRIDE + 8 * (n % 4);
#pragma unroll
    for (int b = 0; b < NB; ++b) OT[b] = mfma_16x16x16_bf16(lds_read_tr16(src + 32 * b), pb, OT[b]);
    wave_lds_fence();  // the tile is free for the next item
  }

  // Reduces this wave's state over its lanes (d over the row quads, O over the row groups) and
  // writes it to the wave's slots of the workgroup merge buffers.
  __device__ __forceinline__ void to_lds(float* s_m, float* s_d, float (*s_o)[D]) {
    const float d = xsum<32>(xsum<16>(dl));
    if (qg == 0 && n < GP) {
      s_m[n] = m;
      s_d[n] = d;
    }
    if (n < GP) {
#pragma unroll
      for (int b = 0; b < NB; ++b)
        *reinterpret_cast<float4*>(&s_o[n][16 * b + 4 * qg]) =
            make_float4(OT[b][0], OT[b][1], OT[b][2], OT[b][3]);
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
