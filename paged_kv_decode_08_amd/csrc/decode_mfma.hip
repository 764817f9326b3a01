// Paged-KV decode attention for bf16 or fp8-e4m3fn KV (bf16 q) on gfx950: q.K on the matrix cores,
// softmax and P.V on the vector ALUs, optional RoPE on q and K in registers (per-item steps:
// mfma_core.hpp).
//
// Work unit ("job"): one chunk of page slots of one (sequence, KV head), done by one workgroup of
// 4 wavefronts (kWaves, kPWaves); wave w takes slots w, w + 4, ... of the chunk and the waves' states are
// merged through LDS at the end of the job, as the TVM relax decode-kernels page
// (_attention_decode) merges its thread groups. A sequence split over several chunks leaves one
// normalised partial state (O_c, lse_c) per chunk, combined by log-sum-exp (the same page,
// _merge_state_inplace, applied over all chunks).
//
// Two schedules:
//  * persistent (decode_mfma_persist_kernel): as many workgroups as fit on
//    the chip at once; each takes jobs from an atomic queue over a compact job list built in LDS
//    from the page table. The job after the current one is fetched, decoded and its page ids and q
//    loaded while the current one streams, and its first page is in flight before the current
//    job's last page is computed, so a workgroup's load stream does not stop at job boundaries.
//    When the call has at most kInMergeChunks chunks per sequence, the workgroup whose waves
//    complete a split sequence's count of arrivals merges it at the end of its next job (each wave
//    arrives once its own partial stores are known complete, one job late, so no wait falls on the
//    load stream); with more chunks a second, row-parallel kernel (split_merge_kernel) merges them.
//  * one workgroup per job (decode_mfma_kernel), for batches too large for the LDS job table: the
//    last workgroup of a split sequence to finish merges it (split.hpp).
#include "device.hpp"
#include "launch.hpp"
#include "mfma_core.hpp"
#include "split.hpp"

#include <mutex>

namespace pdk {

constexpr int kWaves = 4;             // wavefronts per workgroup
constexpr int kPWaves = 4;            // wavefronts per workgroup of the persistent schedule
constexpr int kPersistMaxBatch = 1024;  // sequences the persistent schedule's LDS table holds

// ------------------------------------------------------------------------------------------------
// One workgroup per job.
template <int KVT, int D, int PS, int GP, bool ROPE>
__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(2)))
void decode_mfma_kernel(DecodeParams p) {
  // items of 16 rows: a 32-row page is two items (half the registers per item in flight)
  using C = MfmaCore<KVT, D, 16, GP, ROPE>;
  constexpr int SUB = PS / 16;
  constexpr int BLOCK = PS * C::ROW;  // bytes of one (page, K|V, head) block
  using Buf = typename C::Buf;
  constexpr int NT = 64 * kWaves;
  __shared__ __attribute__((aligned(16))) float s_pt[kWaves][16][C::PT_STRIDE];
  __shared__ float s_alpha[kWaves][16];
  __shared__ float s_m[kWaves][GP];
  __shared__ float s_d[kWaves][GP];
  __shared__ __attribute__((aligned(16))) float s_o[kWaves][GP][D];
  __shared__ float2 s_freq[ROPE ? D / 2 : 1];  // RoPE: frequencies (rope_freq) of dims i, i + D/2

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index (wave-uniform)
  C core;
  core.init_lane(tid & 63);
  const int l = core.l;
  if constexpr (ROPE) {
    if (tid < D / 2) {
      float fhi, flo;
      rope_freq(tid, D, p.rope_scale, p.rope_theta, fhi, flo);
      s_freq[tid] = make_float2(fhi, flo);
    }
    __syncthreads();
  }

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
    for (int idx = tid; idx < G * D; idx += NT)
      store_out<kBF16>(p.out, (size_t(b) * p.H_qo + h * G) * D + idx, 0.f);
    if (tid < G) p.lse[size_t(b) * p.H_qo + h * G + tid] = kEmptyLse;
    return;
  }
  if (c >= nch) return;
  int s_begin, s_end;
  chunk_bounds(sg.n_slots, nch, c, s_begin, s_end);
  const int s_w = s_begin + w;                                           // this wave's first slot
  const int nw = s_w < s_end ? (s_end - s_w + kWaves - 1) / kWaves : 0;  // slots of this wave

  core.load_q(static_cast<const uint16_t*>(p.q) + (size_t(b) * p.H_qo + h * G) * D, G);
  const int kro = ROPE ? p.k_off[b] : 0;
  if constexpr (ROPE) core.rope_q(p.q_pos[b], s_freq);
  const float scale = p.score_scale * (C::FP8 ? p.k_scale[h] : 1.0f);
  const float vscale = C::FP8 ? p.v_scale[h] : 1.0f;
  core.reset();

  // Page ids of this wave's slots, 64 per coalesced load, two batches kept.
  auto slot_of = [&](int k) { return s_w + k * kWaves; };
  auto fetch_id = [&](int k) {
    int id = 0;
    if (k < nw) {
      const int s = slot_of(k);
      const int j = s < sg.n0 ? s : sg.first1 + (s - sg.n0);
      id = p.values[sg.beg + min(j, sg.np - 1)];
    }
    return min(max(id, 0), p.max_num_pages - 1);
  };
  int id_base = 0;
  int ids0 = fetch_id(l), ids1 = fetch_id(64 + l);
  auto page_of = [&](int k) {
    const int r = k - id_base;
    return r < 64 ? __builtin_amdgcn_readlane(ids0, r) : __builtin_amdgcn_readlane(ids1, r - 64);
  };
  const char* pool = static_cast<const char*>(p.pages);
  const size_t kv_stride = size_t(p.H_kv) * BLOCK;
  // item i: rows 16 (i % SUB) .. + 16 of the wave's slot i / SUB
  auto item_block = [&](int i) {
    return pool + (size_t(page_of(i / SUB)) * 2 * p.H_kv + h) * BLOCK + (i % SUB) * 16 * C::ROW;
  };
  const int nitems = nw * SUB;

  if (nw > 0) {
    // two register buffers: item k is computed while item k + 1 loads
    Buf buf[2];
    core.issue(buf[0], item_block(0), kv_stride);
    for (int k = 0; k < nitems; k += 2) {
      if (k / SUB - id_base >= 64) {  // keep the ids of the slots of items k .. k + 2 at hand
        id_base += 64;
        ids0 = ids1;
        ids1 = fetch_id(id_base + 64 + l);
      }
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        if (k + r >= nitems) break;
        // unconditional, so the compiler's wait counts are static; past the end it re-reads the
        // last item's rows (cache hits)
        core.issue(buf[r ^ 1], item_block(min(k + r + 1, nitems - 1)), kv_stride);
        int j, lo, hi;
        slot_rows(sg, slot_of((k + r) / SUB), PS, j, lo, hi);
        const int r0 = 16 * ((k + r) % SUB);
        lo = max(lo - r0, 0);
        hi = min(hi - r0, 16);
        // RoPE position of the item's row 0 (attended rows numbered from the sequence's first)
        const int pos0 = kro + j * PS + r0 +
                         (slot_of((k + r) / SUB) < sg.n0 ? 0 : sg.sink - sg.win_off);
        if (lo < hi) core.process(buf[r], lo, hi, scale, s_pt[w], s_alpha[w], pos0, s_freq);
      }
    }
  }
  core.to_lds(s_m[w], s_d[w], s_o[w]);
  __syncthreads();

  // merge the waves' states and store (final output, or this chunk's partial state)
  for (int idx = tid; idx < G * D; idx += NT) {
    const int g = idx / D;
    const int d = idx - g * D;
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, s_m[ww][g]);
    float wsum = 0.f, o = 0.f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
      const float f = exp2_fast(s_m[ww][g] - M);  // 0 for a wave without slots (m = -inf)
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
  if (nch > 1) split_finish<kBF16, D, GP, NT>(p, b, h, nch);
}

// ------------------------------------------------------------------------------------------------
// Persistent workgroups over a job queue.

// Per-sequence table in LDS. Sequences are ranked by the size of their chunks, largest first (four
// size classes, stable within a class), and jobs are numbered in that order: the queue hands out
// long jobs first and ends with short ones, which shortens the tail of the call. Jobs of one
// sequence are ordered chunk-major, KV head minor. What a job needs is stored by rank, so decoding
// a job number takes two ballots and one round of LDS reads.
struct SeqTable {
  int4* geo;    // [B] by sequence: beg, np, total, win_off (multi-wave build only)
  int4* rgeo;   // [B] by rank: the same
  int4* rsb;    // [B] by rank: sink, sequence, chunks, slots per chunk (rounded down)
  int* pre;     // [B + 1] by rank: first job of each rank (exclusive prefix); pre[B] = all jobs
  int* njobs;   // [B] by sequence: chunks x H_kv
  int* rnj;     // [B] by rank: the same
  int* sink;    // [B] by sequence (multi-wave build only)
  int2* rpos;   // [B] by rank, RoPE only: q position, position of attended row 0
};

__host__ __device__ inline size_t seq_table_bytes(int B) {
  const size_t pre = size_t((B + 4) & ~3);
  const size_t rest = size_t((B + 3) & ~3);
  return size_t(B) * (16 + 16 + 16) + (pre + 3 * rest) * 4 + size_t(B) * 8;
}

__device__ inline SeqTable seq_table(int* base, int B) {
  const int pre = (B + 4) & ~3;
  const int rest = (B + 3) & ~3;
  SeqTable t;
  t.geo = reinterpret_cast<int4*>(base);
  t.rgeo = t.geo + B;
  t.rsb = t.rgeo + B;
  t.pre = reinterpret_cast<int*>(t.rsb + B);
  t.njobs = t.pre + pre;
  t.rnj = t.njobs + rest;
  t.sink = t.rnj + rest;
  t.rpos = reinterpret_cast<int2*>(t.sink + rest);
  return t;
}

// A job as one wave sees it (wave-uniform values).
struct Job {
  int valid;
  int b, h, c, nch;
  SeqGeom g;
  int s_w;      // this wave's first slot
  int nw;       // slots of this wave (may be 0)
  int nitems;   // nw * SUB rounded up to even, at least 2: items past that are unused (re-reads)
  int s_first;  // first slot of the chunk (its page serves the item of a wave without slots)
  int qpos, kro;  // RoPE: position of q and of the sequence's attended row 0
};

__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

// s_waitcnt immediate (gfx9 encoding) that waits until at most n vector-memory operations are
// outstanding, and not for the export or LDS/scalar counters.
constexpr int vmcnt_imm(int n) { return (n & 0xf) | ((n >> 4) & 3) << 14 | 0x7 << 4 | 0xf << 8; }

// ceil(2^32 / d) for d >= 2: __umulhi(r, it) is r / d or r / d + 1 for every 32-bit r.
__device__ __forceinline__ uint32_t div_reciprocal(uint32_t d) { return 0xffffffffu / d + 1u; }

// SUB: items per page slot (a 32-row page is walked as two 16-row items).
template <int PS, int SUB, bool ROPE>
__device__ __forceinline__ Job decode_job(const DecodeParams& p, const SeqTable& t, int total_jobs,
                                          uint32_t hinv, int j, int w, int l) {
  Job J;
  J.valid = j < total_jobs;
  J.b = J.h = J.c = J.nch = J.s_w = J.nw = J.s_first = J.qpos = J.kro = 0;
  J.nitems = 2;
  J.g = SeqGeom{0, 0, 0, 0, 0, 0, 0, 0};
  if (!J.valid) return J;
  // rank = the largest r with pre[r] <= j (pre is non-decreasing from pre[0] = 0; sequences
  // without jobs repeat a value): a ballot over every S-th entry, then one over the S - 1 entries
  // after the last one found
  static_assert(kPersistMaxBatch <= 64 * 16, "two ballots cover the table");
  const int S = (p.B + 63) >> 6;
  int idx = l * S;
  int rank = (__popcll(__ballot(idx < p.B && t.pre[idx] <= j)) - 1) * S;
  if (S > 1) {
    idx = rank + l;
    rank += __popcll(__ballot(l >= 1 && l < S && idx < p.B && t.pre[idx] <= j));
  }
  rank = uni(rank);
  const int4 gg = t.rgeo[rank];
  const int4 sk_b = t.rsb[rank];
  const int p0 = uni(t.pre[rank]);
  const int b = uni(sk_b.y);
  SeqGeom g;
  g.beg = uni(gg.x);
  g.np = uni(gg.y);
  g.total = uni(gg.z);
  g.win_off = uni(gg.w);
  g.sink = uni(sk_b.x);
  g.n0 = (g.sink + PS - 1) / PS;
  g.first1 = g.win_off / PS;
  g.n_slots = g.n0 + (g.win_off < g.total ? g.np - g.first1 : 0);
  // job r of the sequence is chunk r / H_kv, KV head r % H_kv (hinv = div_reciprocal(H_kv))
  const uint32_t r = uint32_t(j - p0);
  uint32_t c = p.H_kv == 1 ? r : __umulhi(r, hinv);
  c -= c * uint32_t(p.H_kv) > r ? 1u : 0u;
  J.nch = uni(sk_b.z);
  J.c = int(c);
  J.h = int(r - c * uint32_t(p.H_kv));
  J.b = b;
  J.g = g;
  if constexpr (ROPE) {
    const int2 rp = t.rpos[rank];
    J.qpos = uni(rp.x);
    J.kro = uni(rp.y);
  }
  int sb, se;
  const int q = uni(sk_b.w);
  chunk_bounds_q(q, g.n_slots - q * J.nch, J.c, sb, se);
  J.s_first = sb;
  J.s_w = sb + w;
  J.nw = J.s_w < se ? (se - J.s_w + kPWaves - 1) / kPWaves : 0;
  J.nitems = max(2, (J.nw * SUB + 1) & ~1);
  return J;
}

// Raw page-table entry of item k of a job for this wave. The load is unconditional (an invalid job
// reads indptr[0] instead) and nothing consumes the value here, so the wait for it falls where the
// id is used; clamp_page() clamps it into the pool there.
__device__ __forceinline__ int load_id(const DecodeParams& p, const Job& J, int k) {
  const int s = J.nw > 0 ? J.s_w + kPWaves * min(k, J.nw - 1) : J.s_first;
  const int j = s < J.g.n0 ? s : J.g.first1 + (s - J.g.n0);
  const int32_t* src = J.valid ? p.values + J.g.beg + min(j, J.g.np - 1) : p.indptr;
  return *src;
}
__device__ __forceinline__ int clamp_page(const DecodeParams& p, int id) {
  return min(max(id, 0), p.max_num_pages - 1);
}

// Split sequences of calls with at most this many chunks are merged inside the persistent kernel.
constexpr int kInMergeChunks = 8;

// Merges the nch (2 .. kInMergeChunks) chunk states of (sequence b, KV head h), stored with
// store_agent() and complete, into out and lse: M = max_c lse_c, w_c = 2^(lse_c - M),
// out = sum_c w_c O_c / sum_c w_c, lse = M + log2(sum_c w_c). Thread t produces 4 dims of one q
// head; every load is issued before any is used (one memory round trip). All threads take part.
template <int D, int GP, int NT>
__device__ void merge_split(const DecodeParams& p, int b, int h, int nch) {
  constexpr int V = D / 4;
  static_assert(GP * V <= NT, "one float4 of output per thread");
  __shared__ float s_l[GP][kInMergeChunks];
  const int tid = threadIdx.x;
  const int G = p.G;
  const size_t row0 = (size_t(b) * p.H_qo + size_t(h) * G) * p.num_chunks;
  if (tid < G * nch) {
    const int g = tid / nch;
    s_l[g][tid - g * nch] = load_agent(&p.part_lse[row0 + size_t(g) * p.num_chunks + (tid - g * nch)]);
  }
  const int g = min(tid / V, G - 1);
  const int v = tid % V;
  const float* src = p.part_o + (row0 + size_t(g) * p.num_chunks) * D + 4 * v;
  float o[kInMergeChunks][4];
#pragma unroll
  for (int c = 0; c < kInMergeChunks; ++c) {
    if (c < nch) {
#pragma unroll
      for (int k = 0; k < 4; ++k) o[c][k] = load_agent(src + size_t(c) * D + k);
    }
  }
  __syncthreads();
  float M = -INFINITY;
#pragma unroll
  for (int c = 0; c < kInMergeChunks; ++c)
    if (c < nch) M = fmaxf(M, s_l[g][c]);
  float ws = 0.f, a[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < kInMergeChunks; ++c) {
    if (c < nch) {
      const float wc = exp2_fast(s_l[g][c] - M);
      ws += wc;
#pragma unroll
      for (int k = 0; k < 4; ++k) a[k] = fmaf(wc, o[c][k], a[k]);
    }
  }
  if (tid < G * V) {
    const float inv = 1.f / ws;
    const size_t orow = size_t(b) * p.H_qo + size_t(h) * G + g;
    uint16_t* dst = static_cast<uint16_t*>(p.out) + orow * D + 4 * v;
    *reinterpret_cast<uint2*>(dst) = make_uint2(
        uint32_t(f32_to_bf16(a[0] * inv)) | uint32_t(f32_to_bf16(a[1] * inv)) << 16,
        uint32_t(f32_to_bf16(a[2] * inv)) | uint32_t(f32_to_bf16(a[3] * inv)) << 16);
    if (v == 0) p.lse[orow] = M + log2f(ws);
  }
  __syncthreads();  // s_l is free again
}

template <int KVT, int D, int PS, int GP, bool ROPE>
__global__ __launch_bounds__(64 * kPWaves) __attribute__((amdgpu_waves_per_eu(2)))
void decode_mfma_persist_kernel(DecodeParams p) {
  // items of 16 rows: a 32-row page is two items (half the registers per item in flight)
  using C = MfmaCore<KVT, D, 16, GP, ROPE>;
  constexpr int SUB = PS / 16;
  constexpr int BLOCK = PS * C::ROW;  // bytes of one (page, K|V, head) block
  using Buf = typename C::Buf;
  constexpr int NT = 64 * kPWaves;
  // q of the next job, staged in LDS by all threads: QW 32-bit words per thread
  constexpr int QWORDS = GP * D / 2;
  constexpr int QW = (QWORDS + NT - 1) / NT;
  extern __shared__ __attribute__((aligned(16))) int s_dyn[];
  __shared__ __attribute__((aligned(16))) float s_pt[kPWaves][16][C::PT_STRIDE];
  __shared__ float s_alpha[kPWaves][16];
  __shared__ float s_m[kPWaves][GP];
  __shared__ float s_d[kPWaves][GP];
  __shared__ __attribute__((aligned(16))) float s_o[kPWaves][GP][D];
  __shared__ __attribute__((aligned(16))) uint32_t s_q[2][QW * NT];
  __shared__ int s_ids[2][kPWaves][64];  // page-table entries of each wave's first 64 items
  __shared__ int s_scan[kPWaves];
  __shared__ unsigned long long s_scan64[kPWaves];
  __shared__ int s_ticket;
  __shared__ int s_mrg[kPWaves];  // wave w's arrival completed the previous job's split sequence
  __shared__ float2 s_freq[ROPE ? D / 2 : 1];  // RoPE: frequencies (rope_freq) of dims i, i + D/2

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index (wave-uniform)
  const int l = tid & 63;
  const int B = p.B;
  const int G = p.G;
  C core;
  core.init_lane(l);
  if constexpr (ROPE) {
    if (tid < D / 2) {
      float fhi, flo;
      rope_freq(tid, D, p.rope_scale, p.rope_theta, fhi, flo);
      s_freq[tid] = make_float2(fhi, flo);
    }
  }

  // ---- job table: sequences ranked by chunk size (largest first), exclusive prefix of their
  // jobs (chunks x H_kv) in rank order
  const SeqTable tab = seq_table(s_dyn, B);
  {
    // size class of a sequence: 0 for chunks above 7/8 of chunk_slots, .. 3 for 5/8 and below
    auto size_class = [&](int n_slots, int nch) {
      const int sz = nch > 0 ? (n_slots + nch - 1) / nch : 0;
      return 8 * sz > 7 * p.chunk_slots ? 0 : 8 * sz > 6 * p.chunk_slots ? 1
             : 8 * sz > 5 * p.chunk_slots ? 2 : 3;
    };
    if (B <= 64) {
      // One wave, lane b for sequence b: the rank counts the sequences of lower classes (ballots)
      // and those of the same class before b (mbcnt); the job prefix is a wave scan.
      if (w == 0) {
        const bool ok = l < B;
        const SeqGeom g = seq_geom(p.indptr, p.length_info, B, ok ? l : B - 1, PS, p.sliding);
        const int nch = chunks_used(g.n_slots, p.chunk_slots, p.num_chunks);
        const int nj = nch * p.H_kv;
        const int c = ok ? size_class(g.n_slots, nch) : 4;
        int rank = 0;
        unsigned long long same = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const unsigned long long m = __ballot(c == k);
          if (k < c) rank += __popcll(m);
          if (k == c) same = m;
        }
        rank += __builtin_amdgcn_mbcnt_hi(uint32_t(same >> 32),
                                          __builtin_amdgcn_mbcnt_lo(uint32_t(same), 0u));
        if (ok) {
          tab.njobs[l] = nj;
          tab.rgeo[rank] = make_int4(g.beg, g.np, g.total, g.win_off);
          tab.rsb[rank] = make_int4(g.sink, l, nch, nch > 0 ? g.n_slots / nch : 0);
          tab.rnj[rank] = nj;
          if constexpr (ROPE) tab.rpos[rank] = make_int2(p.q_pos[l], p.k_off[l]);
        }
        wave_lds_fence();
        int x = ok ? tab.rnj[l] : 0;  // jobs of rank l, then the inclusive prefix
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const int y = __shfl_up(x, o, 64);
          if (l >= o) x += y;
        }
        if (ok) tab.pre[l + 1] = x;
        if (l == 0) tab.pre[0] = 0;
      }
      __syncthreads();
    } else {
      // Every thread takes `per` consecutive sequences; class counts and the job prefix are
      // scanned over the workgroup.
      const int per = (B + NT - 1) / NT;
      const int b0 = min(B, tid * per), b1 = min(B, b0 + per);
      unsigned long long cnt = 0;  // this thread's sequences per class, 16 bits each
      for (int b = b0; b < b1; ++b) {
        const SeqGeom g = seq_geom(p.indptr, p.length_info, B, b, PS, p.sliding);
        tab.geo[b] = make_int4(g.beg, g.np, g.total, g.win_off);
        tab.sink[b] = g.sink;
        const int nch = chunks_used(g.n_slots, p.chunk_slots, p.num_chunks);
        tab.njobs[b] = nch * p.H_kv;
        cnt += 1ull << (16 * size_class(g.n_slots, nch));
      }
      unsigned long long x = cnt;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const unsigned long long y = __shfl_up(x, o, 64);
        if (l >= o) x += y;
      }
      if (l == 63) s_scan64[w] = x;
      __syncthreads();
      unsigned long long off = x - cnt, total = 0;
#pragma unroll
      for (int ww = 0; ww < kPWaves; ++ww) {
        if (ww < w) off += s_scan64[ww];
        total += s_scan64[ww];
      }
      int cls_start[4];
      int acc = 0;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        cls_start[c] = acc + int((off >> (16 * c)) & 0xffff);
        acc += int((total >> (16 * c)) & 0xffff);
      }
      for (int b = b0; b < b1; ++b) {
        const int4 gg = tab.geo[b];
        const int sk = tab.sink[b];
        const int n0 = (sk + PS - 1) / PS;
        const int n_slots = gg.y > 0 ? n0 + (gg.w < gg.z ? gg.y - gg.w / PS : 0) : 0;
        const int nch = tab.njobs[b] / p.H_kv;
        const int rank = cls_start[size_class(n_slots, nch)]++;
        tab.rgeo[rank] = gg;
        tab.rsb[rank] = make_int4(sk, b, nch, nch > 0 ? n_slots / nch : 0);
        tab.rnj[rank] = tab.njobs[b];
        if constexpr (ROPE) tab.rpos[rank] = make_int2(p.q_pos[b], p.k_off[b]);
      }
      __syncthreads();
      int run = 0;
      for (int r = b0; r < b1; ++r) {
        run += tab.rnj[r];
        tab.pre[r + 1] = run;
      }
      int y = run;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int z = __shfl_up(y, o, 64);
        if (l >= o) y += z;
      }
      if (l == 63) s_scan[w] = y;
      __syncthreads();
      int off2 = y - run;
      for (int ww = 0; ww < w; ++ww) off2 += s_scan[ww];
      for (int r = b0; r < b1; ++r) tab.pre[r + 1] += off2;
      if (tid == 0) tab.pre[0] = 0;
      __syncthreads();
    }
  }
  const int total_jobs = tab.pre[B];
  const uint32_t hinv = div_reciprocal(uint32_t(max(p.H_kv, 2)));

  // ---- sequences without attended rows: out = 0, lse = -5e4
  for (int b = blockIdx.x; b < B; b += gridDim.x) {
    if (tab.njobs[b] != 0) continue;
    for (int idx = tid; idx < p.H_qo * D; idx += NT)
      store_out<kBF16>(p.out, size_t(b) * p.H_qo * D + idx, 0.f);
    for (int hq = tid; hq < p.H_qo; hq += NT) p.lse[size_t(b) * p.H_qo + hq] = kEmptyLse;
  }

  const char* pool = static_cast<const char*>(p.pages);
  const size_t kv_stride = size_t(p.H_kv) * BLOCK;
  auto block_of = [&](int page, int h) {
    return pool + (size_t(page) * 2 * p.H_kv + h) * BLOCK;
  };
  const uint32_t* qsrc = static_cast<const uint32_t*>(p.q);
  // This thread's share of J's q rows (words past the G rows repeat the last one; an invalid job
  // reads sequence 0's). Unconditional loads, consumed only when staged into LDS.
  auto q_words = [&](const Job& J, uint32_t (&qs)[QW]) {
    const size_t base = (size_t(J.b) * p.H_qo + size_t(J.h) * G) * (D / 2);
#pragma unroll
    for (int i = 0; i < QW; ++i) qs[i] = qsrc[base + min(tid + i * NT, G * D / 2 - 1)];
  };

  // ---- the first two jobs are static, later ones come from the queue.
  // The next job's page ids and q words, and the ticket of the job after it, are loaded at the top
  // of the current job's first item and staged into LDS right after that item is computed (the
  // wait for the item covers them); nothing loaded lives across items in registers, which keeps
  // the compiler's memory-wait counts exact in the item loop.
  int* queue = p.queue;
  Job J = decode_job<PS, SUB, ROPE>(p, tab, total_jobs, hinv, blockIdx.x, w, l);
  int par = 0;  // s_q[par] / s_ids[par] hold J's data, [par ^ 1] receive J1's
  // J's page ids and q words are loaded first; J1 is decoded while they are in flight. (Issuing
  // J's first item before the barrier, from each wave's own ids, keeps its registers live across
  // the prologue and costs 12 VGPRs at the peak.)
  const int ids0 = load_id(p, J, l);
  uint32_t q0[QW];
  q_words(J, q0);
  Job J1 = decode_job<PS, SUB, ROPE>(p, tab, total_jobs, hinv, blockIdx.x + gridDim.x, w, l);
#pragma unroll
  for (int i = 0; i < QW; ++i) s_q[0][tid + i * NT] = q0[i];
  s_ids[0][w][l] = ids0;
  __syncthreads();

  if (J.valid) {
    core.load_q(reinterpret_cast<const uint16_t*>(s_q[0]), G);
    core.rope_q(J.qpos, s_freq);
    float scale = p.score_scale * (C::FP8 ? p.k_scale[J.h] : 1.0f);
    float vscale = C::FP8 ? p.v_scale[J.h] : 1.0f;
    core.reset();
    Buf buf0, buf1;
    core.issue(buf0, block_of(clamp_page(p, uni(s_ids[0][w][0])), J.h), kv_stride);

    // Page id of item k of the current job (slot k / SUB of the wave; refilled per 64 slots from
    // the page table).
    auto item_id = [&](int k) __attribute__((always_inline)) {
      const int si = k / SUB;
      if ((si & 63) == 0 && si > 0 && k % SUB == 0) {  // chunks of more than 64 slots per wave only
        const int id = load_id(p, J, si + l);
        wave_lds_fence();
        s_ids[par][w][l] = id;
        wave_lds_fence();
      }
      return s_ids[par][w][si & 63];
    };
    // Computes item k from `cur` (rows 16 (k % SUB) .. + 16 of slot k / SUB; items past the
    // wave's slots are unused), then retires `cur`: only the loads just issued stay in flight.
    auto compute = [&](const Buf& cur, int k) __attribute__((always_inline)) {
      const int si = k / SUB;
      if (si < J.nw) {
        int j, lo, hi;
        slot_rows(J.g, J.s_w + kPWaves * si, PS, j, lo, hi);
        const int r0 = 16 * (k % SUB);
        lo = max(lo - r0, 0);
        hi = min(hi - r0, 16);
        // RoPE position of the item's row 0: attended rows are numbered from the sequence's
        // first one, so window pages shift by the rows the window skips (sink - win_off)
        const int pos0 = J.kro + j * PS + r0 +
                         (J.s_w + kPWaves * si < J.g.n0 ? 0 : J.g.sink - J.g.win_off);
        if (lo < hi) core.process(cur, lo, hi, scale, s_pt[w], s_alpha[w], pos0, s_freq);
      }
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(C::NLOADS));
    };
    // Issues the loads of item `k`'s 16 rows (k % SUB selects the rows in the page).
    auto issue_id = [&](Buf& nxt, int raw, int hh, int k) __attribute__((always_inline)) {
      core.issue(nxt, block_of(clamp_page(p, uni(raw)), uni(hh)) + (k % SUB) * 16 * C::ROW,
                 kv_stride);
    };

    // Split sequences are merged here when the call has few chunks. Each wave arrives at its
    // sequence's counter once its own partial stores are known complete (in the next job's first
    // pair, where they are older than the loads waited for); the workgroup whose wave brings the
    // count to chunks x waves merges the sequence at the end of that next job. pb < 0: no
    // arrival pending.
    const bool in_merge = p.num_chunks <= kInMergeChunks;
    int pb = -1, ph = 0, pnch = 0;

    // Every job has an even number of items per wave, item k in buf0 for even k, so the next
    // job's first item is always in flight in buf0 when a job ends: every path into the loops has
    // the same loads in flight and the compiler's wait counts stay exact.
    for (;;) {
      // ---- items 0 and 1, with the loads for the next job (its page ids and q words, staged into
      // LDS once item 1 is computed). The ticket of the job after the next one is taken in the
      // last pair of items, so a workgroup holds at most one job beyond the current one.
      {
        const bool last = J.nitems == 2;
        const int ids_n = load_id(p, J1, l);
        uint32_t qs[QW];
        q_words(J1, qs);
        int ticket_raw = 0;
        if (last && J1.valid && tid == 0) ticket_raw = atomicAdd(queue, 1);
        issue_id(buf1, item_id(1), J.h, 1);
        compute(buf0, 0);
        // the previous job's partial stores are older than the loads just waited for
        int arrival = 0;
        if (pb >= 0 && l == 0)
          arrival = __hip_atomic_fetch_add(&p.counters[pb * p.H_kv + ph], 1, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
        if (!last) issue_id(buf0, item_id(2), J.h, 2);
        else if (J1.valid) issue_id(buf0, __builtin_amdgcn_readlane(ids_n, 0), J1.h, 0);
        else issue_id(buf0, item_id(1), J.h, 1);
        compute(buf1, 1);
#pragma unroll
        for (int i = 0; i < QW; ++i) s_q[par ^ 1][tid + i * NT] = qs[i];
        s_ids[par ^ 1][w][l] = ids_n;
        if (last && tid == 0) s_ticket = 2 * int(gridDim.x) + ticket_raw;
        if (l == 0) s_mrg[w] = pb >= 0 && arrival == pnch * kPWaves - 1;
      }
      // ---- items 2 .. nitems - 3
      for (int k = 2; k + 2 < J.nitems; k += 2) {
        issue_id(buf1, item_id(k + 1), J.h, k + 1);
        compute(buf0, k);
        issue_id(buf0, item_id(k + 2), J.h, k + 2);
        compute(buf1, k + 1);
      }
      // ---- the last pair takes the ticket and issues the next job's first item
      if (J.nitems > 2) {
        const int k = J.nitems - 2;
        int ticket_raw = 0;
        if (J1.valid && tid == 0) ticket_raw = atomicAdd(queue, 1);
        issue_id(buf1, item_id(k + 1), J.h, k + 1);
        compute(buf0, k);
        if (J1.valid) issue_id(buf0, s_ids[par ^ 1][w][0], J1.h, 0);
        else issue_id(buf0, item_id(k + 1), J.h, k + 1);
        compute(buf1, k + 1);
        if (tid == 0) s_ticket = 2 * int(gridDim.x) + ticket_raw;
      }

      // ---- end of job J: merge the waves, store
      core.to_lds(s_m[w], s_d[w], s_o[w]);
      __syncthreads();
      const int next_ticket = s_ticket;
      int merge_prev = 0;  // s_mrg: written in this job's first pair, rewritten after the next barrier
#pragma unroll
      for (int ww = 0; ww < kPWaves; ++ww) merge_prev |= s_mrg[ww];
#pragma unroll
      for (int it = 0; it < (GP * D + NT - 1) / NT; ++it) {
        const int idx = tid + it * NT;
        if (idx < G * D) {
          const int g = idx / D;
          const int d = idx - g * D;
          float M = -INFINITY;
#pragma unroll
          for (int ww = 0; ww < kPWaves; ++ww) M = fmaxf(M, s_m[ww][g]);
          float wsum = 0.f, o = 0.f;
#pragma unroll
          for (int ww = 0; ww < kPWaves; ++ww) {
            const float f = exp2_fast(s_m[ww][g] - M);  // 0 for a wave without slots
            wsum = fmaf(f, s_d[ww][g], wsum);
            o = fmaf(f, s_o[ww][g][d], o);
          }
          const int hq = J.h * G + g;
          const float val = o / wsum * vscale;
          const float l2 = M + log2f(wsum);
          if (J.nch == 1) {
            store_out<kBF16>(p.out, (size_t(J.b) * p.H_qo + hq) * D + d, val);
            if (d == 0) p.lse[size_t(J.b) * p.H_qo + hq] = l2;
          } else {
            const size_t row = (size_t(J.b) * p.H_qo + hq) * p.num_chunks + J.c;
            if (in_merge) {
              store_agent(&p.part_o[row * D + d], val);
              if (d == 0) store_agent(&p.part_lse[row], l2);
            } else {
              p.part_o[row * D + d] = val;
              if (d == 0) p.part_lse[row] = l2;
            }
          }
        }
      }
      __syncthreads();  // s_m / s_d / s_o / s_ticket are free again
      if (merge_prev) {
        merge_split<D, GP, NT>(p, pb, ph, pnch);
        if (tid == 0)
          __hip_atomic_store(&p.counters[pb * p.H_kv + ph], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      pb = in_merge && J.nch > 1 ? J.b : -1;
      ph = J.h;
      pnch = J.nch;
      if (!J1.valid) {
        // no next job to hide the arrival behind: drain the stores, arrive, merge if last
        if (pb >= 0) {
          __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
          __syncthreads();  // every wave's partial stores are complete
          if (tid == 0) {
            const int t = __hip_atomic_fetch_add(&p.counters[pb * p.H_kv + ph], kPWaves,
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            s_ticket = t == (pnch - 1) * kPWaves;
          }
          __syncthreads();
          if (s_ticket) {
            merge_split<D, GP, NT>(p, pb, ph, pnch);
            if (tid == 0)
              __hip_atomic_store(&p.counters[pb * p.H_kv + ph], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
        }
        break;
      }
      // ---- move on: J1 becomes current; decode the job after it
      J = J1;
      par ^= 1;
      core.load_q(reinterpret_cast<const uint16_t*>(s_q[par]), G);
      core.rope_q(J.qpos, s_freq);
      if (C::FP8) {
        scale = p.score_scale * p.k_scale[J.h];
        vscale = p.v_scale[J.h];
      }
      core.reset();
      J1 = decode_job<PS, SUB, ROPE>(p, tab, total_jobs, hinv, next_ticket, w, l);
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  }

  // ---- the last workgroup out puts the queue back to zero for the next call
  if (tid == 0 && atomicAdd(queue + 1, 1) == int(gridDim.x) - 1) {
    __hip_atomic_store(queue, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(queue + 1, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Combines the chunks of every split sequence: M = max_c lse_c, w_c = 2^(lse_c - M),
// out = sum_c w_c O_c / sum_c w_c, lse = M + log2(sum_c w_c).
// One wavefront per output row (sequence, q head), kMergeRows rows per workgroup. A lane holds one
// float4 of one chunk's row, so a wave-wide load covers CPW chunks. The row's first 64 lse values,
// its first CB partial rows and its sequence's page-table bounds are all loaded before any is
// used: a row with at most CB chunks costs one memory round trip. Chunk indexes are clamped into
// the row's num_chunks slots; values of chunks past the sequence's count are never used.
constexpr int kMergeRows = 4;

template <int D, int PS>
__global__ __launch_bounds__(64 * kMergeRows) void split_merge_kernel(DecodeParams p) {
  constexpr int V = D / 4;      // float4 per partial row
  constexpr int CPW = 64 / V;   // chunks per wave-wide load
  constexpr int NB = 8;         // float4 loads per lane per batch
  constexpr int CB = NB * CPW;  // chunks per batch
  static_assert(64 % CB == 0 || CB % 64 == 0, "batches and lse words line up");
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kMergeRows + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (row >= p.B * p.H_qo) return;
  const int b = row / p.H_qo;
  const int nc = p.num_chunks;
  const float* lse_c = p.part_lse + size_t(row) * nc;
  const float* o_c = p.part_o + size_t(row) * nc * D;
  const int v = lane % V, ph = lane / V;
  float4 x[NB];
  auto load_batch = [&](int c0) {
#pragma unroll
    for (int i = 0; i < NB; ++i)
      x[i] = *reinterpret_cast<const float4*>(o_c + size_t(min(c0 + i * CPW + ph, nc - 1)) * D + 4 * v);
  };
  const float lse_l = lse_c[min(lane, nc - 1)];
  load_batch(0);
  const SeqGeom sg = seq_geom(p.indptr, p.length_info, p.B, b, PS, p.sliding);
  const int nch = chunks_used(sg.n_slots, p.chunk_slots, nc);

  float mx = lane < nch ? lse_l : -INFINITY;
  for (int c = 64 + lane; c < nch; c += 64) mx = fmaxf(mx, lse_c[c]);
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
  const float M = mx;
  const float w_l = lane < nch ? exp2_fast(lse_l - M) : 0.f;  // weight of chunk `lane`
  float ws = w_l;
  for (int c = 64 + lane; c < nch; c += 64) ws += exp2_fast(lse_c[c] - M);
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) ws += __shfl_xor(ws, o, 64);

  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int c0 = 0; c0 < nch; c0 += CB) {
    if (c0 > 0) load_batch(c0);
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int c = c0 + i * CPW + ph;
      const float wc = c < 64 ? __shfl(w_l, c & 63, 64) : exp2_fast(lse_c[min(c, nc - 1)] - M);
      if (c < nch) {  // select, not a product: a stale partial past nch may hold any bits
        acc.x = fmaf(wc, x[i].x, acc.x);
        acc.y = fmaf(wc, x[i].y, acc.y);
        acc.z = fmaf(wc, x[i].z, acc.z);
        acc.w = fmaf(wc, x[i].w, acc.w);
      }
    }
  }
  // add the CPW chunk phases (lanes v, v + V, ...)
#pragma unroll
  for (int o = V; o < 64; o <<= 1) {
    acc.x += __shfl_xor(acc.x, o, 64);
    acc.y += __shfl_xor(acc.y, o, 64);
    acc.z += __shfl_xor(acc.z, o, 64);
    acc.w += __shfl_xor(acc.w, o, 64);
  }
  if (nch <= 1) return;  // unsplit (or empty) sequence: the decode kernel wrote its row
  if (lane < V) {
    const float inv = 1.f / ws;
    uint16_t* dst = static_cast<uint16_t*>(p.out) + size_t(row) * D + 4 * lane;
    const uint2 packed = make_uint2(
        uint32_t(f32_to_bf16(acc.x * inv)) | uint32_t(f32_to_bf16(acc.y * inv)) << 16,
        uint32_t(f32_to_bf16(acc.z * inv)) | uint32_t(f32_to_bf16(acc.w * inv)) << 16);
    *reinterpret_cast<uint2*>(dst) = packed;
  }
  if (lane == 0) p.lse[row] = M + log2f(ws);
}

// ------------------------------------------------------------------------------------------------
// Launchers.

template <int KVT, int D, int PS, int GP, bool ROPE>
static hipError_t launch_chunked(const DecodeParams& p, unsigned grid, hipStream_t st) {
  hipLaunchKernelGGL((decode_mfma_kernel<KVT, D, PS, GP, ROPE>), dim3(grid), dim3(64 * kWaves), 0,
                     st, p);
  return hipGetLastError();
}

// Workgroups of a kernel that fit on the current device at once (cached per kernel, device and
// dynamic LDS size).
static int resident_workgroups(const void* kernel, size_t lds) {
  struct Entry {
    const void* k;
    int dev;
    size_t lds;
    int n;
  };
  static std::mutex mu;
  static Entry cache[64];
  static int ncache = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  {
    std::lock_guard<std::mutex> lock(mu);
    for (int i = 0; i < ncache; ++i)
      if (cache[i].k == kernel && cache[i].dev == dev && cache[i].lds == lds) return cache[i].n;
  }
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 64 * kPWaves, lds) != hipSuccess)
    return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  const int n = per_cu * cus;
  std::lock_guard<std::mutex> lock(mu);
  if (ncache < 64) cache[ncache++] = Entry{kernel, dev, lds, n};
  return n;
}

template <int KVT, int D, int PS, int GP, bool ROPE>
static hipError_t launch_persist(const DecodeParams& p, long long max_jobs, hipStream_t st) {
  const void* k = reinterpret_cast<const void*>(&decode_mfma_persist_kernel<KVT, D, PS, GP, ROPE>);
  const size_t lds = seq_table_bytes(p.B);
  const int resident = resident_workgroups(k, lds);
  if (resident <= 0) return hipErrorInvalidConfiguration;
  const unsigned grid = static_cast<unsigned>((max_jobs < resident ? (max_jobs > 0 ? max_jobs : 1) : resident));
  hipLaunchKernelGGL((decode_mfma_persist_kernel<KVT, D, PS, GP, ROPE>), dim3(grid),
                     dim3(64 * kPWaves), lds, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.num_chunks <= 1 || p.num_chunks <= kInMergeChunks) return e;
  const unsigned rows = static_cast<unsigned>(p.B) * p.H_qo;
  hipLaunchKernelGGL((split_merge_kernel<D, PS>), dim3((rows + kMergeRows - 1) / kMergeRows),
                     dim3(64 * kMergeRows), 0, st, p);
  return hipGetLastError();
}

// RoPE on the matrix cores: bf16 KV, or fp8 KV at D = 128.
template <int KVT, int D, int PS, int GP>
static hipError_t launch_sched(const DecodeParams& p, bool persistent, bool rope, long long grid,
                               hipStream_t st) {
  if (rope) {
    if constexpr (KVT == kBF16 || D == 128) {
      return persistent ? launch_persist<KVT, D, PS, GP, true>(p, grid, st)
                        : launch_chunked<KVT, D, PS, GP, true>(p, static_cast<unsigned>(grid), st);
    }
    return hipErrorInvalidValue;
  }
  return persistent ? launch_persist<KVT, D, PS, GP, false>(p, grid, st)
                    : launch_chunked<KVT, D, PS, GP, false>(p, static_cast<unsigned>(grid), st);
}

template <int KVT, int D, int PS>
static hipError_t launch_g(const DecodeParams& p, int gp, bool persistent, bool rope,
                           long long grid, hipStream_t st) {
  switch (gp) {
    case 1: return launch_sched<KVT, D, PS, 1>(p, persistent, rope, grid, st);
    case 2: return launch_sched<KVT, D, PS, 2>(p, persistent, rope, grid, st);
    case 4: return launch_sched<KVT, D, PS, 4>(p, persistent, rope, grid, st);
    case 8: return launch_sched<KVT, D, PS, 8>(p, persistent, rope, grid, st);
  }
  return hipErrorInvalidValue;
}

template <int KVT>
static hipError_t launch_kv(const DecodeParams& p, int D, int PS, int gp, bool persistent,
                            bool rope, long long grid, hipStream_t st) {
  if (D == 64 && PS == 16) return launch_g<KVT, 64, 16>(p, gp, persistent, rope, grid, st);
  if (D == 64 && PS == 32) return launch_g<KVT, 64, 32>(p, gp, persistent, rope, grid, st);
  if (D == 128 && PS == 16) return launch_g<KVT, 128, 16>(p, gp, persistent, rope, grid, st);
  if (D == 128 && PS == 32) return launch_g<KVT, 128, 32>(p, gp, persistent, rope, grid, st);
  return hipErrorInvalidValue;
}

hipError_t launch_decode_mfma(const DecodeParams& p, int kv_dtype, int D, int PS, int gp,
                              bool persistent, bool rope, long long grid, hipStream_t st) {
  if (kv_dtype == kBF16) return launch_kv<kBF16>(p, D, PS, gp, persistent, rope, grid, st);
  if (kv_dtype == kFP8) return launch_kv<kFP8>(p, D, PS, gp, persistent, rope, grid, st);
  return hipErrorInvalidValue;
}

}  // namespace pdk
