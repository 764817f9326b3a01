// Oracle for single-token paged-KV decode attention: TEST INFRASTRUCTURE ONLY.
//
// A plain, slow, scalar CPU implementation with fp64 arithmetic. Only the tests, the smoke check
// and the CPU-baseline leg of the benchmark may load it. It shares no code, header or constant
// table with the GPU library.
//
// What it follows (pages as printed by their sources):
//   * Decode: TVM relax "_decode_kernels.py", function _attention_decode_cpu (the scalar
//     batch_decode_paged_kv_cpu prim_func). Per sequence, the number of attended rows comes from
//     the CSR page table and length_info; every row is gathered through the page table; the score
//     is sm_scale * q.k; the result is the softmax-weighted sum of V rows and a base-2 log-sum-exp
//     (the page keeps scores in log2 units and stores m + log2(d)).
//     That algorithm reaches exactly (up to rounding order) the plain two-pass definition
//         out = sum_r e^{s_r - M} v_r / sum_r e^{s_r - M},   lse = log2 sum_r e^{s_r},
//     which is what this file writes out, in fp64.
//   * No attended rows (no pages, or an empty window with no sink): the same function initialises
//     m = -5e4, d = 1, O = 0 and loops over zero rows, so it emits out = 0 and
//     lse = -5e4 + log2(1) = -5e4.
//   * length_info: the comment block of the same function ([B] = last_page_len, or [3, B] =
//     last_page_len, sliding-window start offset, attention-sink length).
//   * Merge: TVM "_decode_kernels.py", _merge_state_inplace_cpu (pairwise merge in base 2).
//   * Append: vLLM "nki_flash_attn.py", reshape_and_cache (slot // block_size, slot % block_size),
//     re-expressed for the pages[page, K|V, head, offset, dim] layout; a negative slot is skipped
//     (the AWS Neuron attention_block_tkg docs, parameter kv_cache_update_idx, mark a skipped
//     write with the all-ones uint32 value, which reads as -1 in int32).
//   * fp8: OCP float8 e4m3fn (bias 7, no infinities, S.1111.111 = NaN, max 448), the OCP variant
//     named in the attention_block_tkg docs (dtype_mode). Encode = round to nearest, ties to even,
//     saturating to +-448. The same docs' default NON_OCP mode takes float8_e4m3 with max 240:
//     read as the IEEE-style e4m3 (bias 7, exponent 15 = infinity / NaN), encoded the same way
//     with saturation to +-240.
//   * fp8 e5m2 pool (the e5m2 entry of the survey's fp8 extras; the pages name no e5m2 format):
//     read as OCP float8 e5m2 (bias 15, exponent 31 = infinity / NaN, max 1.75 * 2^15 = 57344),
//     encoded the same way, saturating to +-57344.
//
// Readings where the pages are silent (the helper bodies _get_kv_chunk_len, _get_seq_offset and
// _rope are imported but not shown):
//   * Window: attended positions are [0, sink) followed by [win_off, total); row r maps to
//     position r when r < sink, else r - sink + win_off.
//   * RoPE: rotate-half, pairing element i with i + D/2 (the attention_block_tkg docs, parameter
//     rope_contiguous_layout, offer this split-in-halves layout besides an interleaved one),
//     frequency theta^(-2i/D), angle = position * rope_scale * frequency; applied iff
//     rotary_mode == 1; rotary_mode == 2 takes that interleaved layout instead, pairing elements
//     2i and 2i + 1 with the same frequency i; the K position is k_rope_pos_offset[b] + r
//     (compacted row index r, as the page passes row_idx). Pinned to transformers' Llama
//     rotate_half (default inverse frequencies) and GPT-J's rotate_every_two by the CPU tests;
//     PARITY UNPINNED against the pages themselves, which do not show the helper.
//   * fp8 scales multiply the decoded payload, per KV head.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>

namespace {

// DT_FP8: OCP e4m3fn (max 448); DT_FP8_E4M3: the IEEE-style e4m3 of the attention_block_tkg
// page's default NON_OCP dtype mode (max 240: exponent 15 holds infinities and NaN).
// DT_FP8_E5M2: OCP e5m2 (max 57344).
enum { DT_F32 = 0, DT_BF16 = 1, DT_FP8 = 2, DT_FP8_E4M3 = 3, DT_FP8_E5M2 = 4 };
bool is_fp8(int dt) { return dt == DT_FP8 || dt == DT_FP8_E4M3 || dt == DT_FP8_E5M2; }

int elem_bytes(int dt) { return dt == DT_F32 ? 4 : dt == DT_BF16 ? 2 : is_fp8(dt) ? 1 : 0; }

// bfloat16 is the upper 16 bits of an IEEE binary32.
double bf16_value(uint16_t h) {
  uint32_t u = static_cast<uint32_t>(h) << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

// OCP e4m3fn: sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent 0 is subnormal;
// exponent 15 with mantissa 7 is NaN; there is no infinity.
double fp8_value(uint8_t c) {
  int s = (c >> 7) & 1, e = (c >> 3) & 15, m = c & 7;
  double mag;
  if (e == 15 && m == 7) return std::nan("");
  if (e == 0) mag = std::ldexp(m / 8.0, -6);
  else mag = std::ldexp(1.0 + m / 8.0, e - 7);
  return s ? -mag : mag;
}

// IEEE-style e4m3: sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent 0 is subnormal;
// exponent 15 is infinity (mantissa 0) or NaN; the largest finite value is 1.75 * 2^7 = 240.
double fp8_e4m3_value(uint8_t c) {
  int s = (c >> 7) & 1, e = (c >> 3) & 15, m = c & 7;
  double mag;
  if (e == 15) {
    if (m != 0) return std::nan("");
    mag = HUGE_VAL;
  } else if (e == 0) {
    mag = std::ldexp(m / 8.0, -6);
  } else {
    mag = std::ldexp(1.0 + m / 8.0, e - 7);
  }
  return s ? -mag : mag;
}

// OCP e5m2: sign, 5 exponent bits (bias 15), 2 mantissa bits; exponent 0 is subnormal;
// exponent 31 is infinity (mantissa 0) or NaN; the largest finite value is 1.75 * 2^15 = 57344.
double fp8_e5m2_value(uint8_t c) {
  int s = (c >> 7) & 1, e = (c >> 2) & 31, m = c & 3;
  double mag;
  if (e == 31) {
    if (m != 0) return std::nan("");
    mag = HUGE_VAL;
  } else if (e == 0) {
    mag = std::ldexp(m / 4.0, -14);
  } else {
    mag = std::ldexp(1.0 + m / 4.0, e - 15);
  }
  return s ? -mag : mag;
}

double load_value(const void* base, int dt, size_t idx) {
  if (dt == DT_F32) return static_cast<const float*>(base)[idx];
  if (dt == DT_BF16) return bf16_value(static_cast<const uint16_t*>(base)[idx]);
  if (dt == DT_FP8_E4M3) return fp8_e4m3_value(static_cast<const uint8_t*>(base)[idx]);
  if (dt == DT_FP8_E5M2) return fp8_e5m2_value(static_cast<const uint8_t*>(base)[idx]);
  return fp8_value(static_cast<const uint8_t*>(base)[idx]);
}

// Nearest e4m3fn code to a float, ties to the even code, saturating to +-448.
// Brute force over the 127 non-negative finite codes: obviously correct, not fast.
uint8_t fp8_encode(float x) {
  if (std::isnan(x)) return 0x7F;
  uint8_t sign = std::signbit(x) ? 0x80 : 0x00;
  double a = std::fabs(static_cast<double>(x));
  if (a >= 448.0) return sign | 0x7E;
  int best = 0;
  double best_err = a;  // code 0 is +0
  for (int c = 1; c <= 0x7E; ++c) {
    double err = std::fabs(a - fp8_value(static_cast<uint8_t>(c)));
    if (err < best_err || (err == best_err && (c & 1) == 0 && (best & 1) == 1)) {
      best = c;
      best_err = err;
    }
  }
  return sign | static_cast<uint8_t>(best);
}

// Nearest IEEE-style e4m3 code to a float, ties to the even code, saturating to +-240 (finite
// codes only). Brute force over the 120 non-negative finite codes.
uint8_t fp8_e4m3_encode(float x) {
  if (std::isnan(x)) return 0x7F;
  uint8_t sign = std::signbit(x) ? 0x80 : 0x00;
  double a = std::fabs(static_cast<double>(x));
  if (a >= 240.0) return sign | 0x77;
  int best = 0;
  double best_err = a;
  for (int c = 1; c <= 0x77; ++c) {
    double err = std::fabs(a - fp8_e4m3_value(static_cast<uint8_t>(c)));
    if (err < best_err || (err == best_err && (c & 1) == 0 && (best & 1) == 1)) {
      best = c;
      best_err = err;
    }
  }
  return sign | static_cast<uint8_t>(best);
}

// Nearest e5m2 code to a float, ties to the even code, saturating to +-57344 (finite codes only).
// Brute force over the 123 non-negative finite codes.
uint8_t fp8_e5m2_encode(float x) {
  if (std::isnan(x)) return 0x7F;
  uint8_t sign = std::signbit(x) ? 0x80 : 0x00;
  double a = std::fabs(static_cast<double>(x));
  if (a >= 57344.0) return sign | 0x7B;
  int best = 0;
  double best_err = a;
  for (int c = 1; c <= 0x7B; ++c) {
    double err = std::fabs(a - fp8_e5m2_value(static_cast<uint8_t>(c)));
    if (err < best_err || (err == best_err && (c & 1) == 0 && (best & 1) == 1)) {
      best = c;
      best_err = err;
    }
  }
  return sign | static_cast<uint8_t>(best);
}

// RoPE on a D-vector in place (reading of the absent _rope helper, see header): pair i is
// (i, i + D/2) (rotate-half) or, interleaved, (2i, 2i + 1).
void rope_rotate(double* x, int D, double pos, double rope_scale, double rope_theta,
                 bool interleaved = false) {
  int half = D / 2;
  for (int i = 0; i < half; ++i) {
    double freq = std::pow(rope_theta, -2.0 * i / D);
    double ang = pos * rope_scale * freq;
    double c = std::cos(ang), s = std::sin(ang);
    const int i0 = interleaved ? 2 * i : i, i1 = interleaved ? 2 * i + 1 : i + half;
    double a = x[i0], b = x[i1];
    x[i0] = a * c - b * s;
    x[i1] = b * c + a * s;
  }
}

struct DecodeArgs {
  int32_t B, H_qo, H_kv, D, ps, max_num_pages, q_dtype, kv_dtype;
  const void* q;
  const void* pages;
  const int32_t* indptr;
  const int32_t* values;
  int32_t nnz;
  const int32_t* length_info;
  int32_t sliding_window;
  int32_t rotary_mode;
  float rope_scale, rope_theta;
  const int32_t* q_rope_position;
  const int32_t* k_rope_pos_offset;
  float sm_scale;
  const float* k_scale;
  const float* v_scale;
  const float* k_scale_page;  // [max_num_pages, H_kv] or null: per (page, KV head) scales
  const float* v_scale_page;
  const float* q_scale;       // [H_qo], fp8 q only: q = code * q_scale[h_qo]
};

// Index of element (page, kv, head, off, dim) in the pages[P, 2, H_kv, ps, D] pool.
size_t pool_index(const DecodeArgs& a, int64_t page, int kv, int h, int off, int d) {
  return ((((static_cast<size_t>(page) * 2 + kv) * a.H_kv + h) * a.ps + off) * a.D) + d;
}

// Computes out[D] and lse for one (b, h_qo). Returns 0, or a nonzero code for a malformed table.
int decode_one(const DecodeArgs& a, int b, int h_qo, double* out, double* lse) {
  const int G = a.H_qo / a.H_kv;
  const int h = h_qo / G;
  const int D = a.D;
  const int64_t beg = a.indptr[b], end = a.indptr[b + 1];
  const int64_t np = end - beg;
  if (np < 0 || beg < 0 || end > a.nnz) return 1;
  if (np == 0) {
    for (int d = 0; d < D; ++d) out[d] = 0.0;
    *lse = -5e4;
    return 0;
  }
  const int64_t last = a.length_info[b];
  const int64_t total = (np - 1) * a.ps + last;
  int64_t sink = 0, win_off = 0;
  if (a.sliding_window) {
    win_off = a.length_info[a.B + b];
    sink = a.length_info[2 * a.B + b];
  }
  const int64_t L = total - win_off + sink;
  if (last < 1 || last > a.ps || sink < 0 || win_off < sink || win_off > total) return 3;
  if (L == 0) {  // pages but no attended row (empty window, no sink): the same initial state
    for (int d = 0; d < D; ++d) out[d] = 0.0;
    *lse = -5e4;
    return 0;
  }

  std::vector<double> qv(D), kv(D), vv(D), acc(D, 0.0), scores(L);
  // fp8 q: a stored value is code * the q head's scale, as for the pool
  const double qscale = is_fp8(a.q_dtype) ? static_cast<double>(a.q_scale[h_qo]) : 1.0;
  for (int d = 0; d < D; ++d)
    qv[d] = load_value(a.q, a.q_dtype, (static_cast<size_t>(b) * a.H_qo + h_qo) * D + d) * qscale;
  const bool rope = a.rotary_mode == 1 || a.rotary_mode == 2;
  const bool ilv = a.rotary_mode == 2;
  if (rope) rope_rotate(qv.data(), D, a.q_rope_position[b], a.rope_scale, a.rope_theta, ilv);
  // fp8 pool: a stored value is code * scale, the scale of the row's KV head, or of its
  // (page, KV head) block when per-page scales are given (they replace the per-head ones)
  const bool per_page = is_fp8(a.kv_dtype) && a.k_scale_page != nullptr;
  auto scale_of = [&](const float* per_head, const float* per_page_tab, int64_t page) -> double {
    if (!is_fp8(a.kv_dtype)) return 1.0;
    if (per_page) return static_cast<double>(per_page_tab[page * a.H_kv + h]);
    return static_cast<double>(per_head[h]);
  };

  auto locate = [&](int64_t r, int64_t* page, int* off) -> int {
    int64_t pos = (r < sink) ? r : r - sink + win_off;
    int64_t slot = beg + pos / a.ps;
    if (slot < beg || slot >= end) return 2;
    *page = a.values[slot];
    if (*page < 0 || *page >= a.max_num_pages) return 2;
    *off = static_cast<int>(pos % a.ps);
    return 0;
  };

  // Pass 1: scores s_r = sm_scale * q . k_r.
  double M = -INFINITY;
  for (int64_t r = 0; r < L; ++r) {
    int64_t page;
    int off;
    if (int rc = locate(r, &page, &off)) return rc;
    const double kscale = scale_of(a.k_scale, a.k_scale_page, page);
    for (int d = 0; d < D; ++d)
      kv[d] = load_value(a.pages, a.kv_dtype, pool_index(a, page, 0, h, off, d)) * kscale;
    if (rope) rope_rotate(kv.data(), D, static_cast<double>(a.k_rope_pos_offset[b]) + r,
                          a.rope_scale, a.rope_theta, ilv);
    double s = 0.0;
    for (int d = 0; d < D; ++d) s += qv[d] * kv[d];
    s *= static_cast<double>(a.sm_scale);
    scores[r] = s;
    M = std::max(M, s);
  }
  // Pass 2: softmax weights and the weighted sum of V rows.
  double Z = 0.0;
  for (int64_t r = 0; r < L; ++r) {
    int64_t page;
    int off;
    if (int rc = locate(r, &page, &off)) return rc;
    double w = std::exp(scores[r] - M);
    Z += w;
    const double vscale = scale_of(a.v_scale, a.v_scale_page, page);
    for (int d = 0; d < D; ++d)
      acc[d] += w * load_value(a.pages, a.kv_dtype, pool_index(a, page, 1, h, off, d)) * vscale;
  }
  for (int d = 0; d < D; ++d) out[d] = acc[d] / Z;
  *lse = (M + std::log(Z)) / std::log(2.0);
  return 0;
}

}  // namespace

extern "C" {

double oracle_fp8_e4m3fn_value(uint8_t code) { return fp8_value(code); }
uint8_t oracle_fp8_e4m3fn_encode(float x) { return fp8_encode(x); }
double oracle_fp8_e4m3_value(uint8_t code) { return fp8_e4m3_value(code); }
uint8_t oracle_fp8_e4m3_encode(float x) { return fp8_e4m3_encode(x); }
double oracle_fp8_e5m2_value(uint8_t code) { return fp8_e5m2_value(code); }
uint8_t oracle_fp8_e5m2_encode(float x) { return fp8_e5m2_encode(x); }
double oracle_bf16_value(uint16_t bits) { return bf16_value(bits); }

// Applies the RoPE reading to x[D] in place at position pos (exposed for the invariant pins).
void oracle_rope_rotate(double* x, int32_t D, double pos, float rope_scale, float rope_theta,
                        int32_t interleaved) {
  rope_rotate(x, D, pos, rope_scale, rope_theta, interleaved != 0);
}

// Decode attention for the selected (b, h_qo) pairs (sel = [n_sel, 2]; n_sel == 0 means every
// pair, in (b, h_qo) row-major order). out is [n, D] fp64, lse is [n] fp64, n = number of pairs.
// Returns 0 on success, 1 bad indptr, 2 page index out of range, 3 bad length_info, 4 bad args.
int32_t oracle_decode(int32_t B, int32_t H_qo, int32_t H_kv, int32_t D, int32_t ps,
                      int32_t max_num_pages, int32_t q_dtype, int32_t kv_dtype, const void* q,
                      const void* pages, const int32_t* indptr, const int32_t* values, int32_t nnz,
                      const int32_t* length_info, int32_t sliding_window, int32_t rotary_mode,
                      float rope_scale, float rope_theta, const int32_t* q_rope_position,
                      const int32_t* k_rope_pos_offset, float sm_scale, const float* k_scale,
                      const float* v_scale, const float* k_scale_page, const float* v_scale_page,
                      const float* q_scale, int32_t n_sel, const int32_t* sel, double* out,
                      double* lse, int32_t nthreads) {
  if (B < 0 || H_kv <= 0 || H_qo <= 0 || H_qo % H_kv != 0 || D <= 0 || D % 2 != 0 || ps <= 0)
    return 4;
  if (elem_bytes(q_dtype) == 0 || elem_bytes(kv_dtype) == 0) return 4;
  if ((k_scale_page == nullptr) != (v_scale_page == nullptr)) return 4;
  if (is_fp8(kv_dtype) && k_scale_page == nullptr && (k_scale == nullptr || v_scale == nullptr))
    return 4;
  if (is_fp8(q_dtype) && q_scale == nullptr) return 4;
  DecodeArgs a{B, H_qo, H_kv, D, ps, max_num_pages, q_dtype, kv_dtype, q, pages, indptr, values,
               nnz, length_info, sliding_window, rotary_mode, rope_scale, rope_theta,
               q_rope_position, k_rope_pos_offset, sm_scale, k_scale, v_scale, k_scale_page,
               v_scale_page, q_scale};
  const int64_t n = n_sel > 0 ? n_sel : static_cast<int64_t>(B) * H_qo;
  std::atomic<int64_t> next{0};
  std::atomic<int32_t> status{0};
  auto worker = [&]() {
    for (;;) {
      int64_t i = next.fetch_add(1);
      if (i >= n) return;
      int b = n_sel > 0 ? sel[2 * i] : static_cast<int>(i / H_qo);
      int hq = n_sel > 0 ? sel[2 * i + 1] : static_cast<int>(i % H_qo);
      if (b < 0 || b >= B || hq < 0 || hq >= H_qo) { status.store(4); return; }
      int rc = decode_one(a, b, hq, out + i * D, lse + i);
      if (rc) { status.store(rc); return; }
    }
  };
  int nt = nthreads > 0 ? nthreads : static_cast<int>(std::thread::hardware_concurrency());
  nt = std::max(1, static_cast<int>(std::min<int64_t>(nt, std::max<int64_t>(n, 1))));
  std::vector<std::thread> pool;
  for (int t = 1; t < nt; ++t) pool.emplace_back(worker);
  worker();
  for (auto& t : pool) t.join();
  return status.load();
}

// Pairwise merge of two attention states in place, base 2, as in _merge_state_inplace_cpu:
// s_max = max(s, s'); a = 2^(s - s_max); b = 2^(s' - s_max);
// v = v * a/(a+b) + v' * b/(a+b); s = log2(a+b) + s_max.   v: [N, H, D], s: [N, H] (fp64).
void oracle_merge_state(int32_t N, int32_t H, int32_t D, double* v, double* s,
                        const double* v_other, const double* s_other) {
  for (int64_t i = 0; i < static_cast<int64_t>(N) * H; ++i) {
    double s_max = std::max(s[i], s_other[i]);
    double wa = std::exp2(s[i] - s_max), wb = std::exp2(s_other[i] - s_max);
    for (int d = 0; d < D; ++d)
      v[i * D + d] = v[i * D + d] * (wa / (wa + wb)) + v_other[i * D + d] * (wb / (wa + wb));
    s[i] = std::log2(wa + wb) + s_max;
  }
}

// KV append: for token t with slot s >= 0, page = s / ps, off = s % ps, and every head h:
// pages[page, 0, h, off, :] = k[t, h, :], pages[page, 1, h, off, :] = v[t, h, :].
// Same dtype: the bits are copied. fp8 pool: the element is divided by its head's scale (or its
// (page, head) block's scale when per-page scales are given) in fp32 and encoded to e4m3fn
// (nearest, ties to even, saturating). Returns 0, or 2 for a slot whose page is out of range, 4
// for bad arguments.
int32_t oracle_append_kv(int32_t T, int32_t H_kv, int32_t D, int32_t ps, int32_t max_num_pages,
                         int32_t in_dtype, int32_t kv_dtype, const void* new_k, const void* new_v,
                         const int32_t* slots, const float* k_scale, const float* v_scale,
                         const float* k_scale_page, const float* v_scale_page, void* pages) {
  if (T < 0 || H_kv <= 0 || D <= 0 || ps <= 0) return 4;
  const int ib = elem_bytes(in_dtype), kb = elem_bytes(kv_dtype);
  if (ib == 0 || kb == 0) return 4;
  if (!is_fp8(kv_dtype) && in_dtype != kv_dtype) return 4;
  if ((k_scale_page == nullptr) != (v_scale_page == nullptr)) return 4;
  if (is_fp8(kv_dtype) && (is_fp8(in_dtype) || (!k_scale_page && (!k_scale || !v_scale))))
    return 4;
  for (int t = 0; t < T; ++t) {
    int64_t s = slots[t];
    if (s < 0) continue;
    int64_t page = s / ps, off = s % ps;
    if (page >= max_num_pages) return 2;
    for (int kv = 0; kv < 2; ++kv) {
      const void* src = kv == 0 ? new_k : new_v;
      for (int h = 0; h < H_kv; ++h) {
        for (int d = 0; d < D; ++d) {
          size_t si = (static_cast<size_t>(t) * H_kv + h) * D + d;
          size_t di = ((((static_cast<size_t>(page) * 2 + kv) * H_kv + h) * ps + off) * D) + d;
          if (is_fp8(kv_dtype)) {
            float x = static_cast<float>(load_value(src, in_dtype, si));
            const float* tab = kv == 0 ? k_scale_page : v_scale_page;
            float sc = tab ? tab[page * H_kv + h] : (kv == 0 ? k_scale[h] : v_scale[h]);
            static_cast<uint8_t*>(pages)[di] =
                kv_dtype == DT_FP8        ? fp8_encode(x / sc)
                : kv_dtype == DT_FP8_E5M2 ? fp8_e5m2_encode(x / sc)
                                          : fp8_e4m3_encode(x / sc);
          } else {
            std::memcpy(static_cast<uint8_t*>(pages) + di * kb,
                        static_cast<const uint8_t*>(src) + si * ib, kb);
          }
        }
      }
    }
  }
  return 0;
}

// Checks the device-side preconditions of a page table on host copies.
// 0 ok; 1 indptr not monotone or outside [0, nnz]; 2 page id outside [0, max_num_pages);
// 3 last_page_len outside [1, ps] for a non-empty sequence; 4 window bounds violated
// (need 0 <= sink <= win_off <= total).
int32_t oracle_validate_page_table(int32_t B, int32_t ps, int32_t max_num_pages, int32_t nnz,
                                   const int32_t* indptr, const int32_t* values,
                                   const int32_t* length_info, int32_t sliding_window) {
  if (indptr[0] < 0) return 1;
  for (int b = 0; b < B; ++b)
    if (indptr[b + 1] < indptr[b] || indptr[b + 1] > nnz) return 1;
  for (int64_t i = indptr[0]; i < indptr[B]; ++i)
    if (values[i] < 0 || values[i] >= max_num_pages) return 2;
  for (int b = 0; b < B; ++b) {
    int64_t np = indptr[b + 1] - indptr[b];
    if (np == 0) continue;
    int64_t last = length_info[b];
    if (last < 1 || last > ps) return 3;
    if (sliding_window) {
      int64_t total = (np - 1) * ps + last;
      int64_t off = length_info[B + b], sink = length_info[2 * B + b];
      if (sink < 0 || sink > off || off > total) return 4;
    }
  }
  return 0;
}

}  // extern "C"
