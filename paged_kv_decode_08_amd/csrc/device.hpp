// Device-side helpers and kernel parameter blocks shared by the libpdecode kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pdk {

// kFP8: OCP e4m3fn; kFP8E4M3: the IEEE-style e4m3 (max 240), written only by the append kernel
// (its finite codes decode as e4m3fn codes do, so the decode kernels read it as kFP8);
// kFP8E5M2: OCP e5m2 (bias 15, max 57344), a type of its own in the decode kernels too
enum Dtype : int { kF32 = 0, kBF16 = 1, kFP8 = 2, kFP8E4M3 = 3, kFP8E5M2 = 4 };

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kEmptyLse = -5e4f;  // lse of a sequence with no attended rows

// ---------------------------------------------------------------------------------------------
// Parameter blocks (passed by value to the kernels).
struct DecodeParams {
  const void* q;
  const void* pages;
  const int32_t* indptr;
  const int32_t* values;
  const int32_t* length_info;
  const int32_t* q_pos;      // RoPE: query positions [B]
  const int32_t* k_off;      // RoPE: position of attended row 0 [B]
  const float* k_scale;      // fp8 KV: per-KV-head scales
  const float* v_scale;
  const float* k_scale_page; // fp8 KV: per-(page, KV head) scales [max_num_pages, H_kv], or
  const float* v_scale_page; // null; they replace k_scale / v_scale (persistent schedule only)
  const float* q_scale;      // non-null: q holds e4m3fn codes, q = code * q_scale[h_qo]
                             // (persistent schedule only)
  void* out;
  float* lse;
  float* part_o;             // split-KV partial outputs [B, T, H_qo, num_chunks, D] (normalised)
  float* part_lse;           // split-KV partial lse [B, T, H_qo, num_chunks]
  int* counters;             // split-KV arrival counters [B, H_kv]; zero between calls
  int* queue;                // persistent schedule: [0] next job ticket, [1] workgroups done;
                             // zero between calls
  int* plan_word;            // automatic persistent plan: the call's chunk size, written by the
                             // decode kernel's workgroup 0 for the split merge kernel (the word
                             // after the partial lse; need not be zero)
  const void* new_k;         // fused append: the step's K and V rows [B, H_kv, D] (bf16), written
  const void* new_v;         // to each sequence's last position; null: attention only
  void* pages_w;             // fused append: the pool (the same memory as pages)
  const float* sink;         // learned sink logit per q head [H_qo] (natural-log units), or null
  int32_t B, H_qo, H_kv, G;
  int32_t T;                 // query tokens per sequence in this launch (1: single-token decode)
  int32_t T_all, tok0;       // query tokens of the call, and this launch's first one: q, out and
                             // lse are [B, T_all, H_qo, ...]; the launch's token t is the call's
                             // token tok0 + t, which sees positions <= total - T_all + tok0 + t
                             // (a call of more than 16 q columns per KV head runs as launches of
                             // at most 16); single token: T = T_all = 1, tok0 = 0
  int32_t max_num_pages;     // page ids are clamped into the pool before any KV address is formed
  int32_t sliding, rotary;
  float rope_scale, rope_theta;
  float score_scale;         // sm_scale * log2(e): scores are kept in log2 units
  int32_t chunk_slots;       // page slots per chunk (automatic persistent plan: the least chunk)
  int32_t num_chunks;        // chunks in the grid; the last one takes every remaining slot
  int32_t auto_chunk;        // persistent schedule: 1 = the chunk size is chosen on the device
                             // from the call's lengths
};

// Learned attention sink of one q head (logit sink2 in log2 units) folded into a finished state
// (M, wsum = sum_r 2^(x_r - M)): the denominator gains 2^sink2 and no value row is added. Updates
// M and wsum; returns the factor of the unnormalised output sum_r 2^(x_r - M) v_r.
__device__ __forceinline__ float fold_sink(float sink2, float& M, float& wsum) {
  const float Mn = fmaxf(M, sink2);
  const float a = __builtin_amdgcn_exp2f(M - Mn);
  wsum = wsum * a + __builtin_amdgcn_exp2f(sink2 - Mn);
  M = Mn;
  return a;
}

struct AppendParams {
  const void* new_k;
  const void* new_v;
  const int32_t* slots;
  void* pages;
  const float* k_scale;
  const float* v_scale;
  int32_t T, H_kv, D, PS, max_num_pages;
  const float* k_scale_page;  // fp8 pool: per-(page, KV head) scales [max_num_pages, H_kv], or
  const float* v_scale_page;  // null (then k_scale / v_scale)
};

// The scale an fp8 element of (page, KV head h) is stored with: its block's, or its head's.
__device__ __forceinline__ float append_scale(const AppendParams& p, int kv, size_t page, int h) {
  const float* tab = kv ? p.v_scale_page : p.k_scale_page;
  return tab ? tab[page * p.H_kv + h] : (kv ? p.v_scale[h] : p.k_scale[h]);
}

struct MergeParams {
  void* v;
  float* s;
  const void* v_other;
  const float* s_other;
  int32_t rows;              // n * num_heads
  int32_t D;
};

// ---------------------------------------------------------------------------------------------
// K/V rows are read once per call: the loads carry the nontemporal hint (the `nt` cache policy),
// which measured 6 % faster on the Llama-3-8B-shaped call (67.7 -> 63.7 us) and 7 % on the
// long-context one (131 -> 121.5 us), with bit-identical results.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 kv_load(const uint4* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ uint2 kv_load(const uint2* p) {
  const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
  return make_uint2(v[0], v[1]);
}

// ---------------------------------------------------------------------------------------------
// Element codecs.
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// fp32 -> bf16, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Two OCP e4m3fn codes (E5M2: e5m2 codes) (bytes 0,1 or 2,3 of `w`) -> two floats, with the
// gfx950 converters (exact: every fp8 value is an fp32 value).
template <bool HI, bool E5M2 = false>
__device__ __forceinline__ void fp8x2_to_f32(uint32_t w, float& a, float& b) {
  if constexpr (E5M2) {
    auto r = __builtin_amdgcn_cvt_pk_f32_bf8(static_cast<int>(w), HI);
    a = r[0];
    b = r[1];
  } else {
    auto r = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), HI);
    a = r[0];
    b = r[1];
  }
}

// fp32 -> OCP e4m3fn code, round to nearest even, saturating to +-448 (NaN -> 0x7F). Bit-level,
// so fp8 subnormals (down to 2^-9) are produced exactly.
__device__ __forceinline__ uint8_t f32_to_fp8(float x) {
  const uint32_t bits = __float_as_uint(x);
  const uint32_t sign = (bits >> 24) & 0x80u;
  const uint32_t u = bits & 0x7fffffffu;
  if (u > 0x7f800000u) return 0x7f;                   // NaN
  if (u >= 0x43e00000u) return sign | 0x7eu;          // |x| >= 448 (and inf): saturate
  if (u >= 0x3c800000u) {                             // |x| >= 2^-6: normal fp8
    const uint32_t r = (u + 0x7ffffu + ((u >> 20) & 1u)) >> 20;  // 3 mantissa bits, RNE
    return static_cast<uint8_t>(sign | (r - (120u << 3)));      // rebias exponent 127 -> 7
  }
  // subnormal: value = m * 2^-9; |x| * 512 is exact, rintf rounds to nearest even (m = 8 is the
  // smallest normal, code 0x08)
  const uint32_t m = static_cast<uint32_t>(rintf(__uint_as_float(u) * 512.0f));
  return static_cast<uint8_t>(sign | m);
}

// IEEE-style e4m3 (bias 7, exponent 15 reserved for infinity and NaN, max 240), round to nearest
// even with saturation to +-240: below 248 in magnitude the e4m3fn code is the e4m3 code; from 248
// up e4m3fn rounds to 256 or more (exponent 15), which saturates to 240. NaN stays NaN (0x7F).
__device__ __forceinline__ uint8_t f32_to_fp8_e4m3(float x) {
  const uint8_t c = f32_to_fp8(x);
  return ((c & 0x78) == 0x78 && (c & 0x7F) != 0x7F) ? static_cast<uint8_t>((c & 0x80) | 0x77) : c;
}

// fp32 -> OCP e5m2 code (bias 15, 2 mantissa bits), round to nearest even, saturating to +-57344
// (infinity included; NaN -> 0x7F). Bit-level, so e5m2 subnormals (down to 2^-16) are exact.
__device__ __forceinline__ uint8_t f32_to_fp8_e5m2(float x) {
  const uint32_t bits = __float_as_uint(x);
  const uint32_t sign = (bits >> 24) & 0x80u;
  const uint32_t u = bits & 0x7fffffffu;
  if (u > 0x7f800000u) return 0x7f;                   // NaN
  if (u >= 0x47600000u) return sign | 0x7bu;          // |x| >= 57344 (and inf): saturate
  if (u >= 0x38800000u) {                             // |x| >= 2^-14: normal e5m2
    // 2 mantissa bits, RNE; below 57344 the rounding never reaches the infinity code
    const uint32_t r = (u + 0xfffffu + ((u >> 21) & 1u)) >> 21;
    return static_cast<uint8_t>(sign | (r - (112u << 2)));      // rebias exponent 127 -> 15
  }
  // subnormal: value = m * 2^-16; |x| * 65536 is exact, rintf rounds to nearest even (m = 4 is
  // the smallest normal, code 0x04)
  const uint32_t m = static_cast<uint32_t>(rintf(__uint_as_float(u) * 65536.0f));
  return static_cast<uint8_t>(sign | m);
}

// A 16-byte vector of KV elements decoded to fp32.
template <int KVT> struct Kv;
template <> struct Kv<kF32> {
  static constexpr int EB = 4, EPV = 4;
  __device__ static void unpack(const uint4& v, float* f) {
    f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
  }
};
template <> struct Kv<kBF16> {
  static constexpr int EB = 2, EPV = 8;
  __device__ static void unpack(const uint4& v, float* f) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) { f[2 * i] = bf16_lo(w[i]); f[2 * i + 1] = bf16_hi(w[i]); }
  }
};
template <> struct Kv<kFP8> {
  static constexpr int EB = 1, EPV = 16;
  __device__ static void unpack(const uint4& v, float* f) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      fp8x2_to_f32<false>(w[i], f[4 * i], f[4 * i + 1]);
      fp8x2_to_f32<true>(w[i], f[4 * i + 2], f[4 * i + 3]);
    }
  }
};

template <int QT> __device__ __forceinline__ float load_q(const void* base, size_t idx) {
  if constexpr (QT == kF32) return static_cast<const float*>(base)[idx];
  else return bf16_to_f32(static_cast<const uint16_t*>(base)[idx]);
}
template <int QT> __device__ __forceinline__ void store_out(void* base, size_t idx, float v) {
  if constexpr (QT == kF32) static_cast<float*>(base)[idx] = v;
  else static_cast<uint16_t*>(base)[idx] = f32_to_bf16(v);
}

// ---------------------------------------------------------------------------------------------
// Sequence geometry: which page slots a sequence attends and which rows of each page count.
// Slots [0, n0) are the sink pages (positions [0, sink)); slots [n0, n_slots) are the pages from
// first1 on that cover positions [win_off, total). Without a window sink = win_off = 0.
struct SeqGeom {
  int32_t beg, np, total, sink, win_off, n0, first1, n_slots;
};

__device__ __forceinline__ SeqGeom seq_geom(const int32_t* indptr, const int32_t* li, int B,
                                            int b, int ps, int sliding) {
  // every load is issued before any is used (one memory round trip); all are in bounds whatever
  // the page count
  const int32_t i0 = indptr[b], i1 = indptr[b + 1];
  const int32_t last = li[b];
  const int32_t woff = sliding ? li[B + b] : 0;
  const int32_t snk = sliding ? li[2 * B + b] : 0;
  SeqGeom g;
  g.beg = i0;
  g.np = i1 - i0;
  const bool any = g.np > 0;
  g.total = any ? (g.np - 1) * ps + last : 0;
  g.win_off = any ? woff : 0;
  g.sink = any ? snk : 0;
  g.n0 = (g.sink + ps - 1) / ps;
  g.first1 = g.win_off / ps;
  const int n1 = g.win_off < g.total ? g.np - g.first1 : 0;
  g.n_slots = any ? g.n0 + n1 : 0;
  return g;
}

// ---------------------------------------------------------------------------------------------
// RoPE angles. Frequency index i in [0, D/2) (dims i and i + D/2 rotate together): angle =
// pos * rope_scale * theta^(-2i/D). The frequency is kept in revolutions, f = angle / (2 pi pos), as
// a float pair fhi + flo (about 48 bits), so that frac(pos * f) and the angle stay accurate to a
// few 1e-7 rad at positions in the millions.
__device__ __forceinline__ void rope_freq(int i, int D, float rope_scale, float rope_theta,
                                          float& fhi, float& flo) {
  const double f = static_cast<double>(rope_scale) *
                   exp2(-(2.0 * i / D) * log2(static_cast<double>(rope_theta))) /
                   (2.0 * 3.14159265358979323846);
  fhi = static_cast<float>(f);
  flo = static_cast<float>(f - static_cast<double>(fhi));
}

// cos and sin of 2*pi*frac(pos * f) with f = fhi + flo: the product is split exactly (fma) so the
// whole revolutions drop out before the angle is formed.
__device__ __forceinline__ void rope_cs(int pos, float fhi, float flo, float& c, float& s) {
  // No contraction here: fused into fma(pf, fhi, -rint(prod)), the subtraction below would hold
  // the exact product and the residual err would be counted twice (an angle error of up to half
  // an ulp of prod, ~3e-3 rad at position 1.2e5).
#pragma clang fp contract(off)
  const float pf = static_cast<float>(pos);
  const float prod = pf * fhi;
  const float err = fmaf(pf, fhi, -prod);
  const float rev = (prod - rintf(prod)) + fmaf(pf, flo, err);
  sincospif(2.0f * rev, &s, &c);
}

// The same angle with the hardware sine and cosine, which take revolutions (v_sin_f32 /
// v_cos_f32: sin(2 pi x), cos(2 pi x); |x| <= 0.5 here, far inside their domain). About 12
// instructions instead of ~70 for sincospif; used per K row on the matrix-core path.
__device__ __forceinline__ void rope_cs_hw(int pos, float fhi, float flo, float& c, float& s) {
#pragma clang fp contract(off)  // as in rope_cs
  const float pf = static_cast<float>(pos);
  const float prod = pf * fhi;
  const float err = fmaf(pf, fhi, -prod);
  const float rev = (prod - rintf(prod)) + fmaf(pf, flo, err);
  s = __builtin_amdgcn_sinf(rev);
  c = __builtin_amdgcn_cosf(rev);
}

// Chunks a sequence with n_slots page slots occupies.
__device__ __forceinline__ int chunks_used(int n_slots, int chunk_slots, int num_chunks) {
  if (n_slots <= 0) return 0;
  int n = (n_slots + chunk_slots - 1) / chunk_slots;
  return n < num_chunks ? n : num_chunks;
}

// Slots [begin, end) of chunk c when a sequence's n_slots are split evenly over nch chunks: with
// q = n_slots / nch and rem = n_slots % nch, the first rem chunks take q + 1 slots, the others q
// (none exceeds chunk_slots unless the sequence is longer than chunk_slots * num_chunks).
__device__ __forceinline__ void chunk_bounds_q(int q, int rem, int c, int& begin, int& end) {
  begin = c * q + (c < rem ? c : rem);
  end = begin + q + (c < rem ? 1 : 0);
}
__device__ __forceinline__ void chunk_bounds(int n_slots, int nch, int c, int& begin, int& end) {
  const int q = n_slots / nch;
  chunk_bounds_q(q, n_slots - q * nch, c, begin, end);
}

}  // namespace pdk
