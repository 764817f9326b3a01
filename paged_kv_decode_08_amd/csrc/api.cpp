// C ABI of libpdecode: host-side argument checks, split-KV planning and kernel launches.
// Declarations and the contract of every entry point are in include/pdecode.h.
#include "pdecode.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdio>
#include <cstdlib>

#include "api_internal.hpp"
#include "launch.hpp"

namespace {

constexpr int kTargetWorkgroups = 2048;  // workgroups of the one-workgroup-per-chunk kernels
constexpr int kMinChunkRows = 256;
// The persistent schedule (decode_persist.hpp): its LDS job table holds kPersistMaxBatch
// sequences and it runs at most kPersistMaxGrid workgroups, so its automatic plan never wants
// more than 2 kPersistMaxGrid jobs (kAutoJobRoom); the 8-column instantiations merge split
// sequences themselves up to kInMergeChunks chunks each.
constexpr int kPersistMaxBatch = 1024;
constexpr int kPersistMaxGrid = 1024;
constexpr int64_t kAutoJobRoom = 4 * kPersistMaxGrid;
constexpr int kInMergeChunks = 8;

struct Plan {
  int32_t chunk_slots = 1;
  int32_t num_chunks = 1;
  bool auto_chunk = false;  // persistent schedule: the chunk size is chosen on the device
  int64_t max_jobs = 1;     // jobs of the call at most (the one-workgroup-per-chunk grid)
  size_t part_o_bytes = 0;
  size_t part_lse_bytes = 0;
  size_t counter_bytes = 0;
  bool persistent = false;  // matrix-core kernel on the persistent schedule
  size_t workspace_bytes() const { return part_o_bytes + part_lse_bytes + counter_bytes; }
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

bool is_fp8(int kv) {
  return kv == PDECODE_FP8_E4M3FN || kv == PDECODE_FP8_E4M3 || kv == PDECODE_FP8_E5M2;
}

bool supported_pair(int q, int kv) {
  return (q == PDECODE_F32 && kv == PDECODE_F32) || (q == PDECODE_BF16 && kv == PDECODE_BF16) ||
         (q == PDECODE_BF16 && is_fp8(kv)) ||
         (q == PDECODE_FP8_E4M3FN && (kv == PDECODE_BF16 || is_fp8(kv)));
}

pdecode_status check_desc(const pdecode_desc* d) {
  if (!d) return PDECODE_ERR_INVALID_ARG;
  if (d->batch < 0 || d->num_qo_heads <= 0 || d->num_kv_heads <= 0 || d->head_dim <= 0 ||
      d->page_size <= 0 || d->max_num_pages <= 0 || d->max_kv_len < 0 || d->num_kv_splits < 0)
    return PDECODE_ERR_INVALID_ARG;
  if (d->num_qo_heads % d->num_kv_heads != 0) return PDECODE_ERR_INVALID_ARG;
  if (d->sliding_window != 0 && d->sliding_window != 1) return PDECODE_ERR_INVALID_ARG;
  if (d->q_dtype < 0 || d->q_dtype > 2 || d->kv_dtype < 0 || d->kv_dtype > 4)
    return PDECODE_ERR_INVALID_ARG;
  // fp8 scales: per KV head, or per (page, KV head) (both tables or neither; fp8 pools only)
  const bool page_scales = d->k_scale_page != nullptr || d->v_scale_page != nullptr;
  if (page_scales && (!d->k_scale_page || !d->v_scale_page || !is_fp8(d->kv_dtype)))
    return PDECODE_ERR_INVALID_ARG;
  if (is_fp8(d->kv_dtype) && !page_scales && (!d->k_scale || !d->v_scale))
    return PDECODE_ERR_INVALID_ARG;
  if (!supported_pair(d->q_dtype, d->kv_dtype)) return PDECODE_ERR_UNSUPPORTED;
  // fp8 q: its per-q-head scales, and only then
  if ((d->q_dtype == PDECODE_FP8_E4M3FN) != (d->q_scale != nullptr)) return PDECODE_ERR_INVALID_ARG;
  return PDECODE_OK;
}

pdecode_status check_attention_shape(const pdecode_desc* d) {
  const int G = d->num_qo_heads / d->num_kv_heads;
  if (G > 8) return PDECODE_ERR_UNSUPPORTED;
  if (d->head_dim != 64 && d->head_dim != 128) return PDECODE_ERR_UNSUPPORTED;
  if (d->page_size != 16 && d->page_size != 32) return PDECODE_ERR_UNSUPPORTED;
  return PDECODE_OK;
}

// Chunking of each sequence's page slots. A sequence with n slots uses ceil(n / chunk_slots)
// chunks, capped at num_chunks (the last chunk then takes every remaining slot), so any length
// is computed exactly; max_kv_len only sizes the grid.
// The persistent schedule's automatic plan (num_kv_splits 0) is made on the device at each call,
// from the call's lengths (auto_chunk_slots in decode_persist.hpp); the host only sizes its
// partial states, and max_kv_len plays no part.
// The plan does not depend on RoPE: calls with and without it run the same kernel family.
Plan make_plan(const pdecode_desc* d, int qo_len = 1) {
  Plan pl;
  const int64_t ps = d->page_size;
  const int64_t max_len = d->max_kv_len > 0 ? d->max_kv_len : int64_t(d->max_num_pages) * ps;
  const int64_t max_slots = (max_len + ps - 1) / ps + (d->sliding_window ? 2 : 0);
  const int64_t units = int64_t(d->batch) * d->num_kv_heads;
  const int64_t min_chunk = (kMinChunkRows + ps - 1) / ps;
  const size_t cols = size_t(qo_len) * (d->num_qo_heads / d->num_kv_heads);

  const bool persistent = (d->kv_dtype == PDECODE_BF16 || is_fp8(d->kv_dtype)) &&
                          d->batch <= kPersistMaxBatch;
  pl.persistent = persistent;
  if (persistent && d->num_kv_splits == 0) {
    // chunks per sequence at most: room for kAutoJobRoom jobs over the (sequence, KV head)
    // pairs, at least 2 (the device plan's fallback halves the longest sequence); the 8-column
    // single-token kernels keep to kInMergeChunks (and merge in the kernel) when that still leaves
    // room for 2 kPersistMaxGrid jobs
    int64_t cap = (kAutoJobRoom + units - 1) / (units > 0 ? units : 1);
    if (cap < 2) cap = 2;
    const bool eight_cols = qo_len == 1 && d->num_qo_heads / d->num_kv_heads > 4;
    if (eight_cols && cap > kInMergeChunks && units * kInMergeChunks >= 2 * kPersistMaxGrid)
      cap = kInMergeChunks;
    pl.auto_chunk = true;
    pl.chunk_slots = static_cast<int32_t>(min_chunk);
    pl.num_chunks = static_cast<int32_t>(cap);
    pl.max_jobs = units * cap;
  } else {
    int64_t chunk;
    if (d->num_kv_splits == 1) {
      chunk = max_slots;
    } else if (d->num_kv_splits > 1) {
      chunk = (max_slots + d->num_kv_splits - 1) / d->num_kv_splits;
    } else {
      // about kTargetWorkgroups workgroups
      chunk = (units * max_slots + kTargetWorkgroups - 1) / kTargetWorkgroups;
      if (chunk < min_chunk) chunk = min_chunk;
    }
    if (chunk < 1) chunk = 1;
    int64_t n = (max_slots + chunk - 1) / chunk;
    if (n < 1) n = 1;
    if (n > INT_MAX / 2) n = INT_MAX / 2;
    pl.chunk_slots = static_cast<int32_t>(chunk > INT_MAX ? INT_MAX : chunk);
    pl.num_chunks = static_cast<int32_t>(n);
    pl.max_jobs = units * n;
  }
  // split partial states [B, T, H_qo, num_chunks, D]
  if (pl.num_chunks > 1) {
    const size_t rows = size_t(pl.max_jobs) * cols;
    pl.part_o_bytes = align256(rows * d->head_dim * sizeof(float));
    pl.part_lse_bytes = align256((rows + 1) * sizeof(float));  // + the plan word
  }
  // split arrival counters [B * H_kv], then the two job-queue counters of the persistent schedule.
  // They lead the workspace, at the same offset and size in every plan of a description (any
  // query-token count), so a workspace alternating between those plans keeps its counters apart
  // from the partial states.
  if (pl.num_chunks > 1 || pl.persistent)
    pl.counter_bytes = align256((size_t(d->batch) * d->num_kv_heads + 2) * sizeof(int32_t));
  return pl;
}

pdecode_status hip_status(hipError_t e) { return e == hipSuccess ? PDECODE_OK : PDECODE_ERR_HIP; }

// PDECODE_DEBUG set (to anything) in the environment: every attention call prints its plan to
// stderr. Read once.
bool debug_enabled() {
  static const bool on = std::getenv("PDECODE_DEBUG") != nullptr;
  return on;
}

}  // namespace

extern "C" {

const char* pdecode_status_string(pdecode_status s) {
  switch (s) {
    case PDECODE_OK: return "PDECODE_OK";
    case PDECODE_ERR_INVALID_ARG: return "PDECODE_ERR_INVALID_ARG";
    case PDECODE_ERR_UNSUPPORTED: return "PDECODE_ERR_UNSUPPORTED";
    case PDECODE_ERR_WORKSPACE_TOO_SMALL: return "PDECODE_ERR_WORKSPACE_TOO_SMALL";
    case PDECODE_ERR_HIP: return "PDECODE_ERR_HIP";
  }
  return "PDECODE_UNKNOWN_STATUS";
}

size_t pdecode_workspace_bytes(const pdecode_desc* d) {
  if (check_desc(d) != PDECODE_OK || check_attention_shape(d) != PDECODE_OK) return 0;
  return make_plan(d).workspace_bytes();
}

pdecode_status pdecode_workspace_layout(const pdecode_desc* d, int32_t qo_len,
                                        size_t* part_o_offset, size_t* part_lse_offset,
                                        size_t* plan_word_offset, int32_t* num_chunks) {
  pdecode_status st = check_desc(d);
  if (st != PDECODE_OK) return st;
  if ((st = check_attention_shape(d)) != PDECODE_OK) return st;
  if (qo_len < 1 || !part_o_offset || !part_lse_offset || !plan_word_offset || !num_chunks)
    return PDECODE_ERR_INVALID_ARG;
  const Plan pl = make_plan(d, qo_len);
  *num_chunks = pl.num_chunks;
  if (pl.part_o_bytes == 0) {
    *part_o_offset = *part_lse_offset = *plan_word_offset = 0;
    return PDECODE_OK;
  }
  *part_o_offset = pl.counter_bytes;
  *part_lse_offset = pl.counter_bytes + pl.part_o_bytes;
  *plan_word_offset = pl.counter_bytes + pl.part_o_bytes +
                      size_t(pl.max_jobs) * qo_len * (d->num_qo_heads / d->num_kv_heads) * 4;
  return PDECODE_OK;
}

pdecode_status pdecode_plan(const pdecode_desc* d, int32_t* chunk_pages, int32_t* num_chunks) {
  pdecode_status st = check_desc(d);
  if (st != PDECODE_OK) return st;
  if ((st = check_attention_shape(d)) != PDECODE_OK) return st;
  if (!chunk_pages || !num_chunks) return PDECODE_ERR_INVALID_ARG;
  const Plan pl = make_plan(d);
  *chunk_pages = pl.auto_chunk ? 0 : pl.chunk_slots;
  *num_chunks = pl.num_chunks;
  return PDECODE_OK;
}

}  // extern "C"

namespace {

// pdecode_attention, and with new_k / new_v set the fused append of pdecode_append_attention
// (the persistent matrix-core schedule only).
// qo_len > 1: several query tokens per sequence (pdecode_attention_multi; no window).
// fixed: the caller's scratch split into a counter region and a partial-state region at fixed
// places (pdecode_attention_noalloc) instead of one workspace laid out by the plan.
pdecode_status attention_impl(const pdecode_desc* d, const void* new_k, const void* new_v,
                              const void* q, const void* pages, const int32_t* page_indptr,
                              const int32_t* page_values, const int32_t* length_info,
                              const pdecode_rope* rope, float sm_scale, void* out, float* lse,
                              void* workspace, size_t workspace_bytes, void* stream,
                              int qo_len = 1, const pdk::FixedScratch* fixed = nullptr,
                              bool check_only = false) {
  const bool fused = new_k != nullptr;
  pdecode_status st = check_desc(d);
  if (st != PDECODE_OK) return st;
  if ((st = check_attention_shape(d)) != PDECODE_OK) return st;
  if (!std::isfinite(sm_scale)) return PDECODE_ERR_INVALID_ARG;
  // rotary_mode 1: rotate-half; 2: interleaved pairs; anything else: no RoPE
  const bool rotary = rope && (rope->rotary_mode == 1 || rope->rotary_mode == 2);
  if (rotary && (!rope->q_rope_position || !rope->k_rope_pos_offset ||
                 !(rope->rope_theta > 0.f) || !std::isfinite(rope->rope_theta) ||
                 !std::isfinite(rope->rope_scale)))
    return PDECODE_ERR_INVALID_ARG;
  if (d->batch == 0) return PDECODE_OK;
  if (!q || !pages || !page_indptr || !page_values || !length_info || !out || !lse)
    return PDECODE_ERR_INVALID_ARG;
  const Plan pl = make_plan(d, qo_len);
  if ((fused || qo_len > 1 || d->sink_logits) && !pl.persistent) return PDECODE_ERR_UNSUPPORTED;
  // the fused append writes e4m3fn codes only, with per-KV-head scales
  if (fused && d->kv_dtype == PDECODE_FP8_E4M3) return PDECODE_ERR_UNSUPPORTED;
  // per-page fp8 scales and fp8 q: the persistent schedule, attention without the fused append
  if ((d->k_scale_page || d->q_scale) && (!pl.persistent || fused)) return PDECODE_ERR_UNSUPPORTED;
  // e5m2 pool: the persistent single-token kernels, without the fused append or interleaved RoPE
  if (d->kv_dtype == PDECODE_FP8_E5M2 &&
      (!pl.persistent || fused || qo_len > 1 || (rotary && rope->rotary_mode == 2)))
    return PDECODE_ERR_UNSUPPORTED;
  // interleaved RoPE: the persistent matrix-core kernels only
  if (rotary && rope->rotary_mode == 2 && !pl.persistent)
    return PDECODE_ERR_UNSUPPORTED;
  const int64_t grid = pl.max_jobs;  // persistent schedule: a bound on its workgroups
  if (grid > INT_MAX) return PDECODE_ERR_UNSUPPORTED;
  if (fixed) {
    if (pl.counter_bytes > fixed->counter_bytes ||
        pl.part_o_bytes + pl.part_lse_bytes > fixed->partial_bytes)
      return PDECODE_ERR_WORKSPACE_TOO_SMALL;
  } else if (pl.workspace_bytes() > 0) {
    if (!workspace || workspace_bytes < pl.workspace_bytes()) return PDECODE_ERR_WORKSPACE_TOO_SMALL;
    if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return PDECODE_ERR_INVALID_ARG;
  }
  if (check_only) return PDECODE_OK;

  pdk::DecodeParams p{};
  p.q = q;
  p.pages = pages;
  p.indptr = page_indptr;
  p.values = page_values;
  p.length_info = length_info;
  p.q_pos = rotary ? rope->q_rope_position : nullptr;
  p.k_off = rotary ? rope->k_rope_pos_offset : nullptr;
  p.k_scale = d->k_scale;
  p.v_scale = d->v_scale;
  p.k_scale_page = d->k_scale_page;
  p.v_scale_page = d->v_scale_page;
  p.q_scale = d->q_scale;
  p.new_k = new_k;
  p.new_v = new_v;
  p.pages_w = fused ? const_cast<void*>(pages) : nullptr;
  p.sink = d->sink_logits;
  p.out = out;
  p.lse = lse;
  const bool ws = pl.workspace_bytes() > 0;
  if (fixed) {
    p.counters = ws ? fixed->counters : nullptr;
    p.part_o = ws ? fixed->partials : nullptr;
    p.part_lse = ws ? reinterpret_cast<float*>(reinterpret_cast<char*>(fixed->partials) +
                                               pl.part_o_bytes)
                    : nullptr;
  } else {
    char* wsb = static_cast<char*>(workspace);
    p.counters = ws ? reinterpret_cast<int*>(wsb) : nullptr;
    p.part_o = ws ? reinterpret_cast<float*>(wsb + pl.counter_bytes) : nullptr;
    p.part_lse = ws ? reinterpret_cast<float*>(wsb + pl.counter_bytes + pl.part_o_bytes) : nullptr;
  }
  p.queue = ws ? p.counters + size_t(d->batch) * d->num_kv_heads : nullptr;
  // the word after the partial lse rows [B, T, H_qo, num_chunks]
  p.plan_word = pl.part_lse_bytes > 0 ? reinterpret_cast<int32_t*>(
                    p.part_lse + size_t(pl.max_jobs) * qo_len * (d->num_qo_heads / d->num_kv_heads))
                                      : nullptr;
  p.B = d->batch;
  p.H_qo = d->num_qo_heads;
  p.H_kv = d->num_kv_heads;
  p.G = d->num_qo_heads / d->num_kv_heads;
  p.T = qo_len;
  p.T_all = qo_len;
  p.tok0 = 0;
  p.max_num_pages = d->max_num_pages;
  p.sliding = d->sliding_window;
  p.rotary = rotary ? rope->rotary_mode : 0;
  p.rope_scale = rotary ? rope->rope_scale : 1.f;
  p.rope_theta = rotary ? rope->rope_theta : 1.f;
  p.score_scale = sm_scale * pdk::kLog2e;
  p.chunk_slots = pl.chunk_slots;
  p.num_chunks = pl.num_chunks;
  p.auto_chunk = pl.auto_chunk ? 1 : 0;
  if (debug_enabled())
    std::fprintf(stderr,
                 "pdecode: B=%d H_qo=%d H_kv=%d D=%d page=%d T=%d q=%d kv=%d %s plan: %s chunks of "
                 "%d slots, at most %d per sequence; workspace %zu bytes%s\n",
                 d->batch, d->num_qo_heads, d->num_kv_heads, d->head_dim, d->page_size, qo_len,
                 d->q_dtype, d->kv_dtype, fused ? "fused append," : "",
                 pl.persistent ? "persistent," : "one workgroup per chunk,",
                 pl.auto_chunk ? 0 : pl.chunk_slots, pl.num_chunks, pl.workspace_bytes(),
                 pl.auto_chunk ? " (chunk size chosen on the device; see the plan word)" : "");
  hipStream_t s = static_cast<hipStream_t>(stream);
  // bf16 / fp8 KV: q.K on the matrix cores (4-wave workgroups, persistent over a job queue up to
  // kPersistMaxBatch sequences, else one per chunk), RoPE included; fp32 KV: the vector-ALU kernel
  // (one wave per chunk; RoPE rotates K in fp32).
  // An IEEE-style e4m3 pool holds finite codes only (a precondition; the append saturates to
  // +-240), and every finite code has its e4m3fn value: the decode kernels read it as e4m3fn.
  const int kv_read = d->kv_dtype == PDECODE_FP8_E4M3 ? PDECODE_FP8_E4M3FN : d->kv_dtype;
  const bool mfma = kv_read == PDECODE_BF16 || is_fp8(kv_read);
  // Several tokens: the matrix-core B operand holds 16 q columns, G per token, so a call of more
  // than 16 / G tokens runs as launches of 16 / G tokens each (the last takes the rest), one
  // after the other on the stream; each reads the KV cache once and writes its tokens' rows (its
  // split partial states are rows of the same [B, qo_len, H_qo, C, D] layout).
  const int per = qo_len > 1 ? std::max(1, 16 / p.G) : 1;
  for (int t0 = 0; t0 < qo_len; t0 += per) {
    p.tok0 = t0;
    p.T = std::min(per, qo_len - t0);
    const int cols = p.G * p.T;  // q columns of the matrix-core B operand
    const int gp = cols <= 1 ? 1 : cols <= 2 ? 2 : cols <= 4 ? 4 : cols <= 8 ? 8 : 16;
    if (mfma)
      st = hip_status(pdk::launch_decode_mfma(p, kv_read, d->head_dim, d->page_size, gp,
                                              pl.persistent, rotary, grid, s));
    else
      st = hip_status(pdk::launch_decode_valu(p, kv_read, d->head_dim, d->page_size, gp,
                                              static_cast<unsigned>(grid), s));
    if (st != PDECODE_OK) break;
  }
  return st;
}

}  // namespace

namespace pdk {

pdecode_status attention_fixed_scratch(const pdecode_desc* d, const void* q, const void* pages,
                                       const int32_t* page_indptr, const int32_t* page_values,
                                       const int32_t* length_info, const pdecode_rope* rope,
                                       float sm_scale, void* out, float* lse,
                                       const FixedScratch* fixed, void* stream, bool check_only) {
  return attention_impl(d, nullptr, nullptr, q, pages, page_indptr, page_values, length_info,
                        rope, sm_scale, out, lse, nullptr, 0, stream, 1, fixed, check_only);
}

}  // namespace pdk

extern "C" {

pdecode_status pdecode_attention(const pdecode_desc* d, const void* q, const void* pages,
                                 const int32_t* page_indptr, const int32_t* page_values,
                                 const int32_t* length_info, const pdecode_rope* rope,
                                 float sm_scale, void* out, float* lse, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  return attention_impl(d, nullptr, nullptr, q, pages, page_indptr, page_values, length_info,
                        rope, sm_scale, out, lse, workspace, workspace_bytes, stream);
}

size_t pdecode_workspace_bytes_multi(const pdecode_desc* d, int32_t qo_len) {
  if (qo_len < 1) return 0;
  if (check_desc(d) != PDECODE_OK || check_attention_shape(d) != PDECODE_OK) return 0;
  return make_plan(d, qo_len).workspace_bytes();
}

pdecode_status pdecode_attention_multi(const pdecode_desc* d, int32_t qo_len, const void* q,
                                       const void* pages, const int32_t* page_indptr,
                                       const int32_t* page_values, const int32_t* length_info,
                                       const pdecode_rope* rope, float sm_scale, void* out,
                                       float* lse, void* workspace, size_t workspace_bytes,
                                       void* stream) {
  pdecode_status st = check_desc(d);
  if (st != PDECODE_OK) return st;
  if (qo_len < 1) return PDECODE_ERR_INVALID_ARG;
  if (qo_len == 1)
    return attention_impl(d, nullptr, nullptr, q, pages, page_indptr, page_values, length_info,
                          rope, sm_scale, out, lse, workspace, workspace_bytes, stream);
  if (int64_t(d->batch) * qo_len * d->num_qo_heads > INT_MAX) return PDECODE_ERR_UNSUPPORTED;
  return attention_impl(d, nullptr, nullptr, q, pages, page_indptr, page_values, length_info,
                        rope, sm_scale, out, lse, workspace, workspace_bytes, stream, qo_len);
}

pdecode_status pdecode_append_attention(const pdecode_desc* d, const void* new_k,
                                        const void* new_v, const void* q, void* pages,
                                        const int32_t* page_indptr, const int32_t* page_values,
                                        const int32_t* length_info, const pdecode_rope* rope,
                                        float sm_scale, void* out, float* lse, void* workspace,
                                        size_t workspace_bytes, void* stream) {
  if (d && d->batch > 0 && (!new_k || !new_v)) return PDECODE_ERR_INVALID_ARG;
  if (d && d->batch > 0 &&
      !(d->kv_dtype == PDECODE_BF16 || is_fp8(d->kv_dtype)))
    return check_desc(d) != PDECODE_OK ? check_desc(d) : PDECODE_ERR_UNSUPPORTED;
  return attention_impl(d, new_k, new_v, q, pages, page_indptr, page_values, length_info, rope,
                        sm_scale, out, lse, workspace, workspace_bytes, stream);
}

pdecode_status pdecode_merge_state_inplace(int32_t n, int32_t num_heads, int32_t head_dim,
                                           int32_t v_dtype, void* v, float* s,
                                           const void* v_other, const float* s_other,
                                           void* stream) {
  if (n < 0 || num_heads <= 0 || head_dim <= 0) return PDECODE_ERR_INVALID_ARG;
  if (v_dtype != PDECODE_F32 && v_dtype != PDECODE_BF16) return PDECODE_ERR_UNSUPPORTED;
  if (n == 0) return PDECODE_OK;
  if (!v || !s || !v_other || !s_other || v == v_other) return PDECODE_ERR_INVALID_ARG;
  if (int64_t(n) * num_heads > INT_MAX) return PDECODE_ERR_UNSUPPORTED;
  pdk::MergeParams p{v, s, v_other, s_other, n * num_heads, head_dim};
  return hip_status(pdk::launch_merge_state(p, v_dtype, static_cast<hipStream_t>(stream)));
}

pdecode_status pdecode_append_kv(const pdecode_desc* d, const void* new_k, const void* new_v,
                                 const int32_t* slot_ids, int32_t num_tokens, void* pages,
                                 void* stream) {
  pdecode_status st = check_desc(d);
  // Append also quantises fp32 rows into an fp8 pool.
  if (st == PDECODE_ERR_UNSUPPORTED && d->q_dtype == PDECODE_F32 && is_fp8(d->kv_dtype))
    st = PDECODE_OK;
  if (st != PDECODE_OK) return st;
  if (d->q_dtype == PDECODE_FP8_E4M3FN) return PDECODE_ERR_UNSUPPORTED;  // rows come as f32 / bf16
  if (num_tokens < 0) return PDECODE_ERR_INVALID_ARG;
  if (num_tokens == 0) return PDECODE_OK;
  if (!new_k || !new_v || !slot_ids || !pages) return PDECODE_ERR_INVALID_ARG;
  pdk::AppendParams p{new_k, new_v, slot_ids, pages, d->k_scale, d->v_scale, num_tokens,
                      d->num_kv_heads, d->head_dim, d->page_size, d->max_num_pages,
                      d->k_scale_page, d->v_scale_page};
  return hip_status(pdk::launch_append(p, d->q_dtype, d->kv_dtype, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
