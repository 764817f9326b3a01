// Paged-KV decode attention for bf16 or fp8-e4m3fn KV (bf16 q) on gfx950: q.K on the matrix cores,
// softmax and P.V on the vector ALUs (per-page steps: mfma_core.hpp).
//
// Work unit ("job"): one chunk of page slots of one (sequence, KV head), done by one workgroup of
// kWaves wavefronts; wave w takes slots w, w + kWaves, ... of the chunk and the waves' states are
// merged through LDS at the end of the job, as the TVM relax decode-kernels page
// (_attention_decode) merges its thread groups. A sequence split over several chunks leaves one
// normalised partial state (O_c, lse_c) per chunk, combined by log-sum-exp (the same page,
// _merge_state_inplace, applied over all chunks).
//
// Two schedules:
//  * persistent (decode_mfma_persist_kernel + split_merge_kernel): as many workgroups as fit on
//    the chip at once; each takes jobs from an atomic queue over a compact job list built in LDS
//    from the page table. The job after the current one is fetched, decoded and its page ids and q
//    loaded while the current one streams, and its first page is in flight before the current
//    job's last page is computed, so a workgroup's load stream does not stop at job boundaries.
//    Partial states go to the workspace without waiting; a second, small kernel merges the split
//    sequences.
//  * one workgroup per job (decode_mfma_kernel), for batches too large for the LDS job table: the
//    last workgroup of a split sequence to finish merges it (split.hpp).
#include "device.hpp"
#include "launch.hpp"
#include "mfma_core.hpp"
#include "split.hpp"

#include <mutex>

namespace pdk {

constexpr int kWaves = 4;             // wavefronts per workgroup
constexpr int kPersistMaxBatch = 1024;  // sequences the persistent schedule's LDS table holds

// ------------------------------------------------------------------------------------------------
// One workgroup per job.
template <int KVT, int D, int PS, int GP>
__global__ __launch_bounds__(64 * kWaves) void decode_mfma_kernel(DecodeParams p) {
  using C = MfmaCore<KVT, D, PS, GP>;
  using Buf = typename C::Buf;
  constexpr int NT = 64 * kWaves;
  __shared__ __attribute__((aligned(16))) float s_pt[kWaves][16][C::PT_STRIDE];
  __shared__ float s_alpha[kWaves][16];
  __shared__ float s_m[kWaves][GP];
  __shared__ float s_d[kWaves][GP];
  __shared__ __attribute__((aligned(16))) float s_o[kWaves][GP][D];

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index (wave-uniform)
  C core;
  core.init_lane(tid & 63);
  const int l = core.l;

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
  const size_t kv_stride = size_t(p.H_kv) * C::BLOCK;
  auto block_of = [&](int page) { return pool + (size_t(page) * 2 * p.H_kv + h) * C::BLOCK; };

  if (nw > 0) {
    // two register buffers: slot k is computed while slot k + 1 loads
    Buf buf[2];
    core.issue(buf[0], block_of(page_of(0)), kv_stride);
    for (int k = 0; k < nw; k += 2) {
      if (k - id_base >= 64) {  // keep the ids of slots k .. k + 2 at hand
        id_base += 64;
        ids0 = ids1;
        ids1 = fetch_id(id_base + 64 + l);
      }
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        if (k + r >= nw) break;
        // unconditional, so the compiler's wait counts are static; past the end it re-reads the
        // last slot's blocks (cache hits)
        core.issue(buf[r ^ 1], block_of(page_of(min(k + r + 1, nw - 1))), kv_stride);
        int j, lo, hi;
        slot_rows(sg, slot_of(k + r), PS, j, lo, hi);
        core.process(buf[r], lo, hi, scale, s_pt[w], s_alpha[w]);
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
// sequence are ordered chunk-major, KV head minor.
struct SeqTable {
  int* pre;     // [B + 1]: first job of the sequence of each rank (exclusive prefix)
  int* seq;     // [B]: sequence of each rank
  int* njobs;   // [B]: jobs of each sequence
  int4* geo;    // [B]: beg, np, total, win_off
  int* sink;    // [B]
};

__host__ __device__ inline size_t seq_table_bytes(int B) {
  const size_t pre = size_t((B + 4) & ~3);
  const size_t rest = size_t((B + 3) & ~3);
  return (pre + 2 * rest) * 4 + size_t(B) * 16 + rest * 4;
}

__device__ inline SeqTable seq_table(int* base, int B) {
  const int pre = (B + 4) & ~3;
  const int rest = (B + 3) & ~3;
  SeqTable t;
  t.pre = base;
  t.seq = base + pre;
  t.njobs = t.seq + rest;
  t.geo = reinterpret_cast<int4*>(t.njobs + rest);
  t.sink = reinterpret_cast<int*>(t.geo + B);
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
};

__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

// s_waitcnt immediate (gfx9 encoding) that waits until at most n vector-memory operations are
// outstanding, and not for the export or LDS/scalar counters.
constexpr int vmcnt_imm(int n) { return (n & 0xf) | ((n >> 4) & 3) << 14 | 0x7 << 4 | 0xf << 8; }

// SUB: items per page slot (a 32-row page is walked as two 16-row items).
template <int PS, int SUB>
__device__ __forceinline__ Job decode_job(const DecodeParams& p, const SeqTable& t, int total_jobs,
                                          int j, int w) {
  Job J;
  J.valid = j < total_jobs;
  J.b = J.h = J.c = J.nch = J.s_w = J.nw = J.s_first = 0;
  J.nitems = 2;
  J.g = SeqGeom{0, 0, 0, 0, 0, 0, 0, 0};
  if (!J.valid) return J;
  // largest b with pre[b] <= j (sequences without jobs repeat the prefix value); a fixed number of
  // halving steps (B <= kPersistMaxBatch), no loop
  static_assert(kPersistMaxBatch <= 1024, "search depth");
  int lo = 0;
#pragma unroll
  for (int s = 512; s >= 1; s >>= 1) {
    const int c = lo + s;
    if (c < p.B && t.pre[c] <= j) lo = c;
  }
  const int rank = uni(lo);
  const int b = uni(t.seq[rank]);
  const int4 gg = t.geo[b];
  SeqGeom g;
  g.beg = uni(gg.x);
  g.np = uni(gg.y);
  g.total = uni(gg.z);
  g.win_off = uni(gg.w);
  g.sink = uni(t.sink[b]);
  g.n0 = (g.sink + PS - 1) / PS;
  g.first1 = g.win_off / PS;
  g.n_slots = g.n0 + (g.win_off < g.total ? g.np - g.first1 : 0);
  const int p0 = uni(t.pre[rank]);
  const int r = j - p0;
  J.nch = (uni(t.pre[rank + 1]) - p0) / p.H_kv;
  J.c = r / p.H_kv;
  J.h = r - J.c * p.H_kv;
  J.b = b;
  J.g = g;
  int sb, se;
  chunk_bounds(g.n_slots, J.nch, J.c, sb, se);
  J.s_first = sb;
  J.s_w = sb + w;
  J.nw = J.s_w < se ? (se - J.s_w + kWaves - 1) / kWaves : 0;
  J.nitems = max(2, (J.nw * SUB + 1) & ~1);
  return J;
}

// Raw page-table entry of item k of a job for this wave. The load is unconditional (an invalid job
// reads indptr[0] instead) and nothing consumes the value here, so the wait for it falls where the
// id is used; clamp_page() clamps it into the pool there.
__device__ __forceinline__ int load_id(const DecodeParams& p, const Job& J, int k) {
  const int s = J.nw > 0 ? J.s_w + kWaves * min(k, J.nw - 1) : J.s_first;
  const int j = s < J.g.n0 ? s : J.g.first1 + (s - J.g.n0);
  const int32_t* src = J.valid ? p.values + J.g.beg + min(j, J.g.np - 1) : p.indptr;
  return *src;
}
__device__ __forceinline__ int clamp_page(const DecodeParams& p, int id) {
  return min(max(id, 0), p.max_num_pages - 1);
}

template <int KVT, int D, int PS, int GP>
__global__ __launch_bounds__(64 * kWaves) void decode_mfma_persist_kernel(DecodeParams p) {
  // items of 16 rows: a 32-row page is two items (half the registers per item in flight)
  using C = MfmaCore<KVT, D, 16, GP>;
  constexpr int SUB = PS / 16;
  constexpr int BLOCK = PS * C::ROW;  // bytes of one (page, K|V, head) block
  using Buf = typename C::Buf;
  constexpr int NT = 64 * kWaves;
  // q of the next job, staged in LDS by all threads: QW 32-bit words per thread
  constexpr int QWORDS = GP * D / 2;
  constexpr int QW = (QWORDS + NT - 1) / NT;
  extern __shared__ __attribute__((aligned(16))) int s_dyn[];
  __shared__ __attribute__((aligned(16))) float s_pt[kWaves][16][C::PT_STRIDE];
  __shared__ float s_alpha[kWaves][16];
  __shared__ float s_m[kWaves][GP];
  __shared__ float s_d[kWaves][GP];
  __shared__ __attribute__((aligned(16))) float s_o[kWaves][GP][D];
  __shared__ __attribute__((aligned(16))) uint32_t s_q[2][QW * NT];
  __shared__ int s_ids[2][kWaves][64];  // page-table entries of each wave's first 64 items
  __shared__ int s_scan[kWaves];
  __shared__ unsigned long long s_scan64[kWaves];
  __shared__ int s_ticket;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index (wave-uniform)
  const int l = tid & 63;
  const int B = p.B;
  const int G = p.G;
  C core;
  core.init_lane(l);

  // ---- job table: sequences ranked by chunk size (largest first), exclusive prefix of their
  // jobs (chunks x H_kv) in rank order
  const SeqTable tab = seq_table(s_dyn, B);
  {
    const int per = (B + NT - 1) / NT;
    const int b0 = min(B, tid * per), b1 = min(B, b0 + per);
    // size class of a sequence: 0 for chunks above 7/8 of chunk_slots, .. 3 for 5/8 and below
    auto size_class = [&](int n_slots, int nch) {
      const int sz = nch > 0 ? (n_slots + nch - 1) / nch : 0;
      return 8 * sz > 7 * p.chunk_slots ? 0 : 8 * sz > 6 * p.chunk_slots ? 1
             : 8 * sz > 5 * p.chunk_slots ? 2 : 3;
    };
    unsigned long long cnt = 0;  // this thread's sequences per class, 16 bits each
    for (int b = b0; b < b1; ++b) {
      const SeqGeom g = seq_geom(p.indptr, p.length_info, B, b, PS, p.sliding);
      tab.geo[b] = make_int4(g.beg, g.np, g.total, g.win_off);
      tab.sink[b] = g.sink;
      const int nch = chunks_used(g.n_slots, p.chunk_slots, p.num_chunks);
      tab.njobs[b] = nch * p.H_kv;
      cnt += 1ull << (16 * size_class(g.n_slots, nch));
    }
    // exclusive scan of the packed class counts over the workgroup
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
    for (int ww = 0; ww < kWaves; ++ww) {
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
      SeqGeom g;
      g.np = gg.y;
      g.total = gg.z;
      g.win_off = gg.w;
      g.sink = tab.sink[b];
      const int n0 = (g.sink + PS - 1) / PS;
      const int n_slots = g.np > 0 ? n0 + (g.win_off < g.total ? g.np - g.win_off / PS : 0) : 0;
      const int c = size_class(n_slots, tab.njobs[b] / p.H_kv);
      tab.seq[cls_start[c]++] = b;
    }
    __syncthreads();
    // prefix of the jobs in rank order
    int run = 0;
    for (int r = b0; r < b1; ++r) {
      run += tab.njobs[tab.seq[r]];
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
  const int total_jobs = tab.pre[B];

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
  Job J = decode_job<PS, SUB>(p, tab, total_jobs, blockIdx.x, w);
  Job J1 = decode_job<PS, SUB>(p, tab, total_jobs, blockIdx.x + gridDim.x, w);
  int par = 0;  // s_q[par] / s_ids[par] hold J's data, [par ^ 1] receive J1's
  {
    uint32_t q0[QW];
    q_words(J, q0);
#pragma unroll
    for (int i = 0; i < QW; ++i) s_q[0][tid + i * NT] = q0[i];
    s_ids[0][w][l] = load_id(p, J, l);
  }
  __syncthreads();

  if (J.valid) {
    core.load_q(reinterpret_cast<const uint16_t*>(s_q[0]), G);
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
        slot_rows(J.g, J.s_w + kWaves * si, PS, j, lo, hi);
        const int r0 = 16 * (k % SUB);
        lo = max(lo - r0, 0);
        hi = min(hi - r0, 16);
        if (lo < hi) core.process(cur, lo, hi, scale, s_pt[w], s_alpha[w]);
      }
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(C::NLOADS));
    };
    // Issues the loads of item `k`'s 16 rows (k % SUB selects the rows in the page).
    auto issue_id = [&](Buf& nxt, int raw, int hh, int k) __attribute__((always_inline)) {
      core.issue(nxt, block_of(clamp_page(p, uni(raw)), uni(hh)) + (k % SUB) * 16 * C::ROW,
                 kv_stride);
    };

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
        if (!last) issue_id(buf0, item_id(2), J.h, 2);
        else if (J1.valid) issue_id(buf0, __builtin_amdgcn_readlane(ids_n, 0), J1.h, 0);
        else issue_id(buf0, item_id(1), J.h, 1);
        compute(buf1, 1);
#pragma unroll
        for (int i = 0; i < QW; ++i) s_q[par ^ 1][tid + i * NT] = qs[i];
        s_ids[par ^ 1][w][l] = ids_n;
        if (last && tid == 0) s_ticket = 2 * int(gridDim.x) + ticket_raw;
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
#pragma unroll
      for (int it = 0; it < (GP * D + NT - 1) / NT; ++it) {
        const int idx = tid + it * NT;
        if (idx < G * D) {
          const int g = idx / D;
          const int d = idx - g * D;
          float M = -INFINITY;
#pragma unroll
          for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, s_m[ww][g]);
          float wsum = 0.f, o = 0.f;
#pragma unroll
          for (int ww = 0; ww < kWaves; ++ww) {
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
            p.part_o[row * D + d] = val;
            if (d == 0) p.part_lse[row] = l2;
          }
        }
      }
      __syncthreads();  // s_m / s_d / s_o / s_ticket are free again
      if (!J1.valid) break;
      // ---- move on: J1 becomes current; decode the job after it
      J = J1;
      par ^= 1;
      core.load_q(reinterpret_cast<const uint16_t*>(s_q[par]), G);
      if (C::FP8) {
        scale = p.score_scale * p.k_scale[J.h];
        vscale = p.v_scale[J.h];
      }
      core.reset();
      J1 = decode_job<PS, SUB>(p, tab, total_jobs, next_ticket, w);
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
// out = sum_c w_c O_c / sum_c w_c, lse = M + log2(sum_c w_c). One workgroup per output row
// (sequence, q head); thread t sums 4 dims of every CG-th chunk (16-byte loads, a chunk's row read
// by D/4 consecutive threads), and the CG partial sums are added through LDS.
template <int D, int PS>
__global__ __launch_bounds__(256) void split_merge_kernel(DecodeParams p) {
  constexpr int NT = 256;
  constexpr int V = D / 4;     // float4 per row
  constexpr int CG = NT / V;   // chunk groups
  __shared__ float s_w[NT];
  __shared__ float s_red[2][NT / 64];
  __shared__ float4 s_acc[CG][V];
  const int tid = threadIdx.x;
  const int row = blockIdx.x;  // b * H_qo + hq
  const int b = row / p.H_qo;
  const SeqGeom sg = seq_geom(p.indptr, p.length_info, p.B, b, PS, p.sliding);
  const int nch = chunks_used(sg.n_slots, p.chunk_slots, p.num_chunks);
  if (nch <= 1) return;
  const float* lse_c = p.part_lse + size_t(row) * p.num_chunks;
  const float* o_c = p.part_o + size_t(row) * p.num_chunks * D;

  // M = max_c lse_c and sum_c 2^(lse_c - M) over the workgroup
  float mx = -INFINITY;
  for (int c = tid; c < nch; c += NT) mx = fmaxf(mx, lse_c[c]);
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
  if ((tid & 63) == 0) s_red[0][tid >> 6] = mx;
  __syncthreads();
  float M = s_red[0][0];
#pragma unroll
  for (int i = 1; i < NT / 64; ++i) M = fmaxf(M, s_red[0][i]);
  float ws = 0.f;
  for (int c = tid; c < nch; c += NT) ws += exp2_fast(lse_c[c] - M);
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) ws += __shfl_xor(ws, o, 64);
  if ((tid & 63) == 0) s_red[1][tid >> 6] = ws;

  const int v = tid % V;
  const int cg = tid / V;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int c0 = 0; c0 < nch; c0 += NT) {
    __syncthreads();
    s_w[tid] = c0 + tid < nch ? exp2_fast(lse_c[c0 + tid] - M) : 0.f;
    __syncthreads();
    const int cn = min(NT, nch - c0);
#pragma unroll 4
    for (int cc = cg; cc < cn; cc += CG) {
      const float wc = s_w[cc];
      const float4 x = *reinterpret_cast<const float4*>(o_c + size_t(c0 + cc) * D + 4 * v);
      acc.x = fmaf(wc, x.x, acc.x);
      acc.y = fmaf(wc, x.y, acc.y);
      acc.z = fmaf(wc, x.z, acc.z);
      acc.w = fmaf(wc, x.w, acc.w);
    }
  }
  s_acc[cg][v] = acc;
  __syncthreads();
  float wsum = 0.f;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) wsum += s_red[1][i];
  if (tid < V) {
    float4 t = s_acc[0][tid];
#pragma unroll
    for (int i = 1; i < CG; ++i) {
      const float4 u = s_acc[i][tid];
      t.x += u.x;
      t.y += u.y;
      t.z += u.z;
      t.w += u.w;
    }
    const float inv = 1.f / wsum;
    uint16_t* dst = static_cast<uint16_t*>(p.out) + size_t(row) * D + 4 * tid;
    const uint2 packed = make_uint2(uint32_t(f32_to_bf16(t.x * inv)) | uint32_t(f32_to_bf16(t.y * inv)) << 16,
                                    uint32_t(f32_to_bf16(t.z * inv)) | uint32_t(f32_to_bf16(t.w * inv)) << 16);
    *reinterpret_cast<uint2*>(dst) = packed;
  }
  if (tid == 0) p.lse[row] = M + log2f(wsum);
}

// ------------------------------------------------------------------------------------------------
// Launchers.

template <int KVT, int D, int PS, int GP>
static hipError_t launch_chunked(const DecodeParams& p, unsigned grid, hipStream_t st) {
  hipLaunchKernelGGL((decode_mfma_kernel<KVT, D, PS, GP>), dim3(grid), dim3(64 * kWaves), 0, st, p);
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
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 64 * kWaves, lds) != hipSuccess)
    return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  const int n = per_cu * cus;
  std::lock_guard<std::mutex> lock(mu);
  if (ncache < 64) cache[ncache++] = Entry{kernel, dev, lds, n};
  return n;
}

template <int KVT, int D, int PS, int GP>
static hipError_t launch_persist(const DecodeParams& p, long long max_jobs, hipStream_t st) {
  const void* k = reinterpret_cast<const void*>(&decode_mfma_persist_kernel<KVT, D, PS, GP>);
  const size_t lds = seq_table_bytes(p.B);
  const int resident = resident_workgroups(k, lds);
  if (resident <= 0) return hipErrorInvalidConfiguration;
  const unsigned grid = static_cast<unsigned>((max_jobs < resident ? (max_jobs > 0 ? max_jobs : 1) : resident));
  hipLaunchKernelGGL((decode_mfma_persist_kernel<KVT, D, PS, GP>), dim3(grid), dim3(64 * kWaves),
                     lds, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.num_chunks <= 1) return e;
  hipLaunchKernelGGL((split_merge_kernel<D, PS>), dim3(p.B * p.H_qo), dim3(256), 0, st, p);
  return hipGetLastError();
}

template <int KVT, int D, int PS, int GP>
static hipError_t launch_sched(const DecodeParams& p, bool persistent, long long grid,
                               hipStream_t st) {
  return persistent ? launch_persist<KVT, D, PS, GP>(p, grid, st)
                    : launch_chunked<KVT, D, PS, GP>(p, static_cast<unsigned>(grid), st);
}

template <int KVT, int D, int PS>
static hipError_t launch_g(const DecodeParams& p, int gp, bool persistent, long long grid,
                           hipStream_t st) {
  switch (gp) {
    case 1: return launch_sched<KVT, D, PS, 1>(p, persistent, grid, st);
    case 2: return launch_sched<KVT, D, PS, 2>(p, persistent, grid, st);
    case 4: return launch_sched<KVT, D, PS, 4>(p, persistent, grid, st);
    case 8: return launch_sched<KVT, D, PS, 8>(p, persistent, grid, st);
  }
  return hipErrorInvalidValue;
}

template <int KVT>
static hipError_t launch_kv(const DecodeParams& p, int D, int PS, int gp, bool persistent,
                            long long grid, hipStream_t st) {
  if (D == 64 && PS == 16) return launch_g<KVT, 64, 16>(p, gp, persistent, grid, st);
  if (D == 64 && PS == 32) return launch_g<KVT, 64, 32>(p, gp, persistent, grid, st);
  if (D == 128 && PS == 16) return launch_g<KVT, 128, 16>(p, gp, persistent, grid, st);
  if (D == 128 && PS == 32) return launch_g<KVT, 128, 32>(p, gp, persistent, grid, st);
  return hipErrorInvalidValue;
}

hipError_t launch_decode_mfma(const DecodeParams& p, int kv_dtype, int D, int PS, int gp,
                              bool persistent, long long grid, hipStream_t st) {
  if (kv_dtype == kBF16) return launch_kv<kBF16>(p, D, PS, gp, persistent, grid, st);
  if (kv_dtype == kFP8) return launch_kv<kFP8>(p, D, PS, gp, persistent, grid, st);
  return hipErrorInvalidValue;
}

}  // namespace pdk
