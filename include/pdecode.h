/* libpdecode: single-token paged-KV decode attention for AMD Instinct MI355X (gfx950).
 *
 * Operations (each cites the page that defines it):
 *   pdecode_attention            TVM relax decode-kernels page, _attention_decode_cpu /
 *                                _attention_decode (batch_decode_paged_kv): one query token per
 *                                sequence, K/V gathered through a CSR page table, grouped-query
 *                                heads, online softmax, output plus base-2 log-sum-exp, optional
 *                                RoPE on Q and K, optional sliding window with attention sink.
 *   pdecode_merge_state_inplace  Same page, _merge_state_inplace: combine two attention states
 *                                (V, lse) in place.
 *   pdecode_attention_multi      Several query tokens per sequence, causal over the new tokens
 *                                (the same page's decode per token, over its visible prefix).
 *   pdecode_append_attention     pdecode_append_kv of each sequence's newest token fused into
 *                                pdecode_attention (one launch).
 *   pdecode_append_kv            vLLM nki_flash_attn page, reshape_and_cache: write new K/V rows
 *                                into their cache slots. The fp8 KV cache with k_scale / v_scale
 *                                follows the AWS Neuron attention_block_tkg page (OCP e4m3fn);
 *                                here the scales are per KV head and a stored value is
 *                                code * scale (read) and x / scale rounded to e4m3fn (write).
 *
 * Conventions for every call:
 *   - Tensor pointers are DEVICE pointers owned by the caller; host structs are read during the
 *     call only. The library allocates nothing, never synchronises and keeps no per-call state
 *     (it is reentrant). Its only state is a thread-safe cache of how many workgroups of each
 *     kernel fit on a device (keyed by kernel, device and LDS size), and, for
 *     pdecode_attention_noalloc only, each device's scratch array and its address. Work is enqueued on `stream` (a hipStream_t; NULL = the default
 *     stream) and runs asynchronously.
 *   - Arguments are checked on the host before anything is launched; on error nothing is
 *     launched and the call returns a status other than PDECODE_OK. Device-resident data
 *     (page tables, lengths, slots) are preconditions, not checked on the device (see below).
 *   - Layouts are row-major:
 *       q, out        [batch, num_qo_heads, head_dim]       (dtype q_dtype)
 *       pages         [max_num_pages, 2, num_kv_heads, page_size, head_dim]; index 1: 0 = K, 1 = V
 *       page_indptr   int32 [batch + 1]; page_values int32 [page_indptr[batch]]
 *       length_info   int32 [batch] = last_page_len, or, with sliding_window, int32 [3, batch] =
 *                     (last_page_len, window start offset, sink length)
 *       lse           fp32 [batch, num_qo_heads], base 2: lse = log2(sum_r exp(s_r))
 *   - Sequence b owns pages page_values[page_indptr[b] .. page_indptr[b+1]); with np of them its
 *     length is total = (np - 1) * page_size + last_page_len. Without a window it attends rows
 *     0..total-1. With a window it attends positions [0, sink) and then [win_off, total), and the
 *     K RoPE position of attended row r (0-based over the attended rows) is
 *     k_rope_pos_offset[b] + r. A sequence with no pages yields out = 0 and lse = -5e4.
 *   - Score of row r for q head h_qo: s_r = sm_scale * q[h_qo] . k_r, with k_r read from KV head
 *     h_qo / (num_qo_heads / num_kv_heads).
 *   - Device preconditions: page_indptr non-decreasing from 0; page ids in [0, max_num_pages);
 *     1 <= last_page_len <= page_size for non-empty sequences; 0 <= sink <= win_off <= total.
 */
#ifndef PDECODE_H
#define PDECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pdecode_status {
  PDECODE_OK = 0,
  PDECODE_ERR_INVALID_ARG = 1,          /* null pointer, non-positive size, inconsistent heads   */
  PDECODE_ERR_UNSUPPORTED = 2,          /* valid but outside the supported set (see below)       */
  PDECODE_ERR_WORKSPACE_TOO_SMALL = 3,  /* workspace missing or smaller than required            */
  PDECODE_ERR_HIP = 4                   /* a HIP launch failed                                   */
} pdecode_status;

typedef enum pdecode_dtype {
  PDECODE_F32 = 0,
  PDECODE_BF16 = 1,
  PDECODE_FP8_E4M3FN = 2,               /* OCP e4m3fn: bias 7, no infinities, max 448            */
  PDECODE_FP8_E4M3 = 3,                 /* IEEE-style e4m3: bias 7, exponent 15 = inf / NaN, max
                                           240 (the AWS attention_block_tkg page's default
                                           NON_OCP float8_e4m3). As a pool: the append writes it
                                           (round to nearest even, saturating to +-240); a pool
                                           read by the decode must hold finite codes, which have
                                           their e4m3fn values. Not with pdecode_append_attention. */
  PDECODE_FP8_E5M2 = 4                  /* OCP e5m2: bias 15, exponent 31 = inf / NaN, max 57344
                                           (the e5m2 of the fp8 extras; the pages name no e5m2).
                                           As a pool only: the append writes it (round to nearest
                                           even, saturating to +-57344); the decode reads finite
                                           codes exactly, with per-KV-head or per-page scales, on
                                           the persistent schedule (batch <= 1024), one query
                                           token, no RoPE or rotate-half RoPE; not with
                                           pdecode_append_attention or pdecode_attention_multi. */
} pdecode_dtype;

/* Problem description shared by pdecode_attention and pdecode_append_kv.
 * Supported set: head_dim in {64, 128}; page_size in {16, 32}; group size
 * num_qo_heads / num_kv_heads in 1..8; (q_dtype, kv_dtype) in {(F32, F32), (BF16, BF16),
 * (BF16, FP8_E4M3FN), (BF16, FP8_E4M3), (BF16, FP8_E5M2), (FP8_E4M3FN, BF16 or any FP8)}
 * (FP8_E5M2 pools within the limits given at PDECODE_FP8_E5M2). The output dtype equals
 * q_dtype, except BF16 for an FP8 q. */
typedef struct pdecode_desc {
  int32_t batch;          /* B >= 0                                                            */
  int32_t num_qo_heads;   /* H_qo > 0, a multiple of num_kv_heads                              */
  int32_t num_kv_heads;   /* H_kv > 0                                                          */
  int32_t head_dim;       /* D                                                                 */
  int32_t page_size;      /* rows per page                                                     */
  int32_t max_num_pages;  /* pages in the pool (first dimension of `pages`)                    */
  int32_t q_dtype;        /* pdecode_dtype of q and out (and of new_k / new_v for append)      */
  int32_t kv_dtype;       /* pdecode_dtype of the pool                                         */
  int32_t sliding_window; /* 0: length_info is [B]; 1: length_info is [3, B]                   */
  int32_t max_kv_len;     /* host-side upper bound on attended rows per sequence, used only to
                             plan the split-KV grid of the fixed-split and fp32 / large-batch
                             plans; 0 = take max_num_pages * page_size. The automatic plan of the
                             bf16 / fp8 kernels (batch <= 1024) ignores it. A sequence longer than
                             the bound is still computed exactly.                               */
  int32_t num_kv_splits;  /* 0 = automatic: for bf16 / fp8 KV and batch <= 1024 the chunk size is
                             chosen on the device at each call from the lengths (about one or two
                             jobs per resident workgroup where sequences must be split to fill
                             the chip; whole sequences where (sequence, KV head) pairs outnumber
                             the resident workgroups and none exceeds a workgroup's share);
                             1 = never split a sequence; n > 1 = split each sequence's pages
                             into at most n chunks merged by log-sum-exp                        */
  const float *k_scale;   /* device fp32 [H_kv]; required iff kv_dtype is an FP8: K = code * scale */
  const float *v_scale;   /* device fp32 [H_kv]; required iff kv_dtype is an FP8: V = code * scale */
  const float *sink_logits; /* device fp32 [H_qo] or NULL: learned attention sink per q head (the
                             AWS attention_block_tkg page's `sink`, one value per q head). Read as
                             a logit in the units of the scaled score: a sequence with attended
                             rows gets out = sum_r e^{s_r} v_r / (e^{sink} + sum_r e^{s_r}) and
                             lse = log2(e^{sink} + sum_r e^{s_r}); one without keeps out = 0,
                             lse = -5e4. Attention calls on the persistent matrix-core schedule
                             only (BF16 / FP8 pool, batch <= 1024); otherwise UNSUPPORTED.       */
  const float *k_scale_page; /* device fp32 [max_num_pages, H_kv] or NULL, FP8 pools only: a scale
                             per (page, KV head) block, K = code * k_scale_page[page][h]; with
                             v_scale_page (set both or neither, else INVALID_ARG) it replaces
                             k_scale / v_scale, which may then be NULL. An extension of the
                             pages' single K and V scale (AWS attention_block_tkg page, k_scale /
                             v_scale) to one scale per page block. pdecode_append_kv stores a
                             row as x / (its page's scale). Attention calls on the persistent
                             matrix-core schedule (batch <= 1024), not pdecode_append_attention;
                             otherwise UNSUPPORTED.                                             */
  const float *v_scale_page; /* device fp32 [max_num_pages, H_kv] or NULL: V's, as k_scale_page    */
  const float *q_scale;   /* device fp32 [H_qo]; required iff q_dtype is FP8_E4M3FN: q = code *
                             q_scale[h_qo] (the pool's reading of a scaled code, applied to q).
                             fp8 q pairs with a BF16 or FP8 pool, writes a BF16 out, and runs on
                             the persistent matrix-core schedule (batch <= 1024; attention calls,
                             single- or multi-token, not pdecode_append_attention); otherwise
                             UNSUPPORTED. pdecode_append_kv does not take fp8 rows.             */
} pdecode_desc;

/* Rotary embedding on Q and K inside the kernel; a NULL pointer to this struct means none.
 * rotary_mode == 1: rotate-half over the two contiguous halves of the head dimension: for
 * i < D/2, angle = position * rope_scale * rope_theta^(-2i/D), x'[i] = x[i] cos - x[i + D/2] sin,
 * x'[i + D/2] = x[i + D/2] cos + x[i] sin. rotary_mode == 2: the interleaved layout (the AWS
 * attention_block_tkg page's rope_contiguous_layout = False), the same rotation on the pairs
 * (2i, 2i + 1); supported on the persistent matrix-core schedule (BF16 or FP8 pool, batch
 * <= 1024), including pdecode_append_attention and pdecode_attention_multi; otherwise
 * UNSUPPORTED. Any other value: no RoPE. The rotated q and k stay in fp32 (or a bf16 pair that holds them to 2^-16). */
typedef struct pdecode_rope {
  int32_t rotary_mode;
  float rope_scale;
  float rope_theta;                   /* > 0                                                   */
  const int32_t *q_rope_position;     /* device int32 [B]: position of the query token        */
  const int32_t *k_rope_pos_offset;   /* device int32 [B]: position of attended row 0         */
} pdecode_rope;

/* Bytes of device workspace pdecode_attention needs for this description: the split partial
 * states and counters (for the persistent bf16 / fp8 schedule also its job-queue counters), 0 when
 * the planned launch needs none of them. Depends only on host fields of `d`. Returns 0 for an
 * invalid description. */
size_t pdecode_workspace_bytes(const pdecode_desc *d);

/* The split plan for `d` (with or without RoPE): rows are processed in chunks of *chunk_pages page
 * slots and a sequence uses at most *num_chunks chunks. *chunk_pages = 0: the chunk size is chosen
 * on the device at each call (automatic plan of the bf16 / fp8 kernels), within *num_chunks
 * chunks per sequence. Returns PDECODE_OK or an argument error. */
pdecode_status pdecode_plan(const pdecode_desc *d, int32_t *chunk_pages, int32_t *num_chunks);

/* Inspection of a split plan (debugging; the survey's per-split partial dump): where a call on a
 * workspace of pdecode_workspace_bytes(_multi)(d[, qo_len]) bytes leaves its split partial states.
 * Byte offsets into the workspace of part_o [B, qo_len, H_qo, C, D] fp32 (normalised partial
 * outputs) and part_lse [B, qo_len, H_qo, C] fp32 (base-2 log-sum-exp), C = *num_chunks, and of
 * the int32 chunk size in page slots that the persistent schedule's automatic plan chose (valid
 * once the call has run). Chunk c of a split sequence holds the state of the decode over that
 * chunk's rows alone; rows of sequences that did not split, and chunks past a sequence's count,
 * hold whatever an earlier call left. All offsets are 0 when the plan has no partial states.
 * Returns PDECODE_OK or an argument error. Setting PDECODE_DEBUG in the environment makes every
 * attention call print its plan to stderr. */
pdecode_status pdecode_workspace_layout(const pdecode_desc *d, int32_t qo_len,
                                        size_t *part_o_offset, size_t *part_lse_offset,
                                        size_t *plan_word_offset, int32_t *num_chunks);

/* Decode attention (see the header comment for the computation and layouts).
 * q, pages, page_indptr, page_values, length_info, out, lse: device pointers as above.
 * rope: NULL or a host struct. sm_scale: the score scale (typically 1/sqrt(head_dim)).
 * workspace: device memory of at least pdecode_workspace_bytes(d) bytes, 256-byte aligned
 * (may be NULL when that is 0). It starts with the arrival counters of the split (sequence, KV
 * head) pairs and the job-queue counters of the persistent schedule, followed by the split partial
 * states. Zero-fill it once before its first use; every call leaves the counters zero again, so
 * a later call whose batch x KV-head count is no larger than the previous call's can reuse it as
 * it is (with or without RoPE, any hint or split count that fits). Before a call with a larger
 * count, zero its first pdecode_workspace_bytes(new description) bytes again. Calls that may run
 * at the same time need separate workspaces.
 * out and lse are fully written. Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE_TOO_SMALL (nothing
 * launched), HIP (launch failure). */
pdecode_status pdecode_attention(const pdecode_desc *d, const void *q, const void *pages,
                                 const int32_t *page_indptr, const int32_t *page_values,
                                 const int32_t *length_info, const pdecode_rope *rope,
                                 float sm_scale, void *out, float *lse, void *workspace,
                                 size_t workspace_bytes, void *stream);

/* For callers that cannot allocate (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): pdecode_attention without a workspace. The split and job-queue counters
 * and the split partial states live in a device array inside the library, one per GPU, held from
 * the first call on that GPU until the process ends: a counter region of 64 KiB (room for
 * batch * num_kv_heads <= 16382) and a partial-state region of 32 MiB. The arguments, results and
 * supported set are those of pdecode_attention; the array is used on the device current at the
 * call, which must be the device of `stream`, q and the other buffers. Nothing is allocated (no
 * hipMalloc, no allocating library call): the first call on a device takes the array's device
 * address and clears its counters once (a kernel on `stream`); every call leaves the counters at
 * zero. All calls on one GPU share the array and it keeps the last call's partial states, so calls
 * that may run at the same time on one GPU (other streams, other threads) race: serialise them.
 * Errors: those of pdecode_attention; PDECODE_ERR_WORKSPACE_TOO_SMALL (nothing launched) when the
 * plan needs more counters or partial state than the array holds (use pdecode_attention with a
 * workspace then); PDECODE_ERR_HIP when the array's address cannot be taken. */
pdecode_status pdecode_attention_noalloc(const pdecode_desc *d, const void *q, const void *pages,
                                         const int32_t *page_indptr, const int32_t *page_values,
                                         const int32_t *length_info, const pdecode_rope *rope,
                                         float sm_scale, void *out, float *lse, void *stream);

/* Decode with qo_len query tokens per sequence, causal over the new tokens (speculative
 * verification, chunked decode): the sequence's last qo_len positions hold the new tokens, already
 * in the pool, and token t (0-based) attends the positions 0 .. total_b - qo_len + t. Each token's
 * result is that of pdecode_attention over that prefix of the sequence (TVM relax decode-kernels
 * page, _attention_decode); a token whose prefix is empty (total_b < qo_len - t) gets out = 0 and
 * lse = -5e4, as a sequence without pages does.
 * q, out: device [batch, qo_len, num_qo_heads, head_dim] (q_dtype); lse: fp32 [batch, qo_len,
 * num_qo_heads]. The other arguments are those of pdecode_attention; the workspace is sized by
 * pdecode_workspace_bytes_multi(d, qo_len), with the same reuse rules. With RoPE (either
 * rotary_mode), token t's query sits at position q_rope_position[b] + t; the keys are placed as in
 * pdecode_attention.
 * With a sliding window (length_info [3, B]) the sequence's window start and sink apply to all
 * its new tokens: token t attends the sink rows and the window rows at positions up to
 * total_b - qo_len + t (a reading: the pages define no per-token window).
 * qo_len == 1 is pdecode_attention. Supported for qo_len > 1: the persistent
 * matrix-core schedule (BF16, FP8_E4M3FN or FP8_E4M3 pool, batch <= 1024) and
 * batch * qo_len * num_qo_heads <= INT_MAX; otherwise UNSUPPORTED. The kernel takes 16 q columns
 * (G = num_qo_heads / num_kv_heads per token): more than 16 / G tokens run as consecutive launches
 * of 16 / G tokens each on the stream, each reading the KV cache once. Errors: as
 * pdecode_attention, and INVALID_ARG for qo_len < 1. */
size_t pdecode_workspace_bytes_multi(const pdecode_desc *d, int32_t qo_len);
pdecode_status pdecode_attention_multi(const pdecode_desc *d, int32_t qo_len, const void *q,
                                       const void *pages, const int32_t *page_indptr,
                                       const int32_t *page_values, const int32_t *length_info,
                                       const pdecode_rope *rope, float sm_scale, void *out,
                                       float *lse, void *workspace, size_t workspace_bytes,
                                       void *stream);

/* One decode step with its KV append fused into the attention launch: for every sequence b with
 * pages and every KV head h, new_k[b, h, :] and new_v[b, h, :] are written to the sequence's row
 * of position total_b - 1 (page page_values[page_indptr[b+1] - 1], row last_page_len[b] - 1)
 * exactly as pdecode_append_kv writes a token to that slot (vLLM nki_flash_attn page,
 * reshape_and_cache), and out / lse are those of pdecode_attention over the updated pool (TVM
 * relax decode-kernels page, _attention_decode). The AWS Neuron attention_block_tkg page fuses
 * its cache update with the attention in the same way. The row is read from the staged new
 * values, never from the pool, so the result does not depend on what the row held before.
 * new_k, new_v: device [batch, num_kv_heads, head_dim] of q_dtype (BF16); pages is written; the
 * other arguments, the workspace rules and the results are those of pdecode_attention.
 * Supported: the calls pdecode_attention runs on its persistent matrix-core schedule (BF16 or
 * FP8_E4M3FN pool, batch <= 1024); otherwise UNSUPPORTED. Errors: as pdecode_attention, and INVALID_ARG for a null new_k / new_v. */
pdecode_status pdecode_append_attention(const pdecode_desc *d, const void *new_k,
                                        const void *new_v, const void *q, void *pages,
                                        const int32_t *page_indptr, const int32_t *page_values,
                                        const int32_t *length_info, const pdecode_rope *rope,
                                        float sm_scale, void *out, float *lse, void *workspace,
                                        size_t workspace_bytes, void *stream);

/* Merges the attention state (v_other, s_other) into (v, s) in place, base 2:
 *   s_max = max(s, s'); a = 2^(s - s_max); b = 2^(s' - s_max);
 *   v = v * a / (a + b) + v' * b / (a + b);  s = log2(a + b) + s_max.
 * v, v_other: device [n, num_heads, head_dim] of v_dtype (F32 or BF16); s, s_other: device fp32
 * [n, num_heads]. Arithmetic in fp32; bf16 results are rounded to nearest even. v must not
 * alias v_other. n == 0 is a no-op. Errors: INVALID_ARG (null pointer, negative size),
 * UNSUPPORTED (v_dtype), HIP. */
pdecode_status pdecode_merge_state_inplace(int32_t n, int32_t num_heads, int32_t head_dim,
                                           int32_t v_dtype, void *v, float *s,
                                           const void *v_other, const float *s_other,
                                           void *stream);

/* Writes token t's K and V rows into slot slot_ids[t] of the pool, for every KV head:
 *   pages[slot / page_size, 0, h, slot % page_size, :] = new_k[t, h, :]   (V at index 1).
 * new_k, new_v: device [num_tokens, num_kv_heads, head_dim] of d->q_dtype; slot_ids: device
 * int32 [num_tokens]. A negative slot skips its token; so does a slot at or beyond
 * max_num_pages * page_size. Slots >= 0 must be distinct. Same dtype: bits are copied. FP8 pool:
 * each element is divided by its head's scale in fp32 and rounded to the nearest e4m3fn value,
 * ties to even, saturating to +-448. Uses d's head, size and dtype fields only; besides the
 * attention pairs it also accepts fp32 rows into an FP8 pool.
 * Errors: INVALID_ARG, UNSUPPORTED, HIP. */
pdecode_status pdecode_append_kv(const pdecode_desc *d, const void *new_k, const void *new_v,
                                 const int32_t *slot_ids, int32_t num_tokens, void *pages,
                                 void *stream);

/* Static string naming a status. */
const char *pdecode_status_string(pdecode_status s);

#ifdef __cplusplus
}
#endif

#endif /* PDECODE_H */
