// Persistent matrix-core decode (bf16 or fp8-e4m3fn KV, bf16 q): workgroups resident for the
// whole call take (sequence, KV head, chunk) jobs from an atomic queue (TVM relax decode-kernels
// page, _attention_decode, for the computation; the schedule is this library's). Included by
// decode_mfma.hip (attention) and decode_fused.hip (attention with the fused KV append), which
// instantiate it separately so the two compile in parallel.
#pragma once

#include <mutex>

#include "device.hpp"
#include "mfma_core.hpp"
#include "split.hpp"

namespace pdk {

constexpr int kPWaves = 4;              // wavefronts per workgroup of the persistent schedule

// Call timeline, compiled in only with -DPDECODE_TIMELINE (the separate library that
// `python -m paged_kv_decode_08_amd.build --timeline` builds; `bench.py --timeline` reads it).
// Thread 0 of a workgroup stores (s_memrealtime, tag, value) into row blockIdx.x of a static
// device array at fixed points: 1 entry, 2 job table built, 3 first K/V loads issued, 4 job start
// (value: wave 0's slots in the job), 5 job end (value: 1 if the workgroup merged a split sequence
// there), 6 exit; the split merge kernel's workgroups use rows 2048 + blockIdx.x (7 start, 8 end).
// Each translation unit has its own array; the reader (decode_mfma.hip) sees the plain persistent
// instantiations and the split merge kernel. Marks past the array's bounds are dropped.
constexpr int kTimelineRows = 4096, kTimelineMarks = 64;
#ifdef PDECODE_TIMELINE
static __device__ unsigned long long g_timeline[kTimelineRows][kTimelineMarks];
__device__ __forceinline__ void timeline_mark(int row, int& k, int tag, int val) {
  if (threadIdx.x == 0 && row < kTimelineRows && k < kTimelineMarks)
    g_timeline[row][k] = ((__builtin_amdgcn_s_memrealtime() & 0xFFFFFFFFFFull) << 24) |
                         (uint64_t(tag) << 20) | uint64_t(val & 0xfffff);
  ++k;
}
#define PDK_MARK_DECL int pdk_mark_k = 0
#define PDK_MARK(row, tag, val) timeline_mark(row, pdk_mark_k, tag, val)
#else
#define PDK_MARK_DECL static_cast<void>(0)
#define PDK_MARK(row, tag, val) static_cast<void>(0)
#endif
constexpr int kPersistMaxBatch = 1024;  // sequences the persistent schedule's LDS table holds
constexpr int kPersistMaxGrid = 1024;   // workgroups of the persistent schedule, at most
// Size classes of the job order, a quarter octave of chunk size each
constexpr int kSizeClasses = 16;

// ------------------------------------------------------------------------------------------------
// Persistent workgroups over a job queue.

// Per-sequence table in LDS. Sequences are ranked by the size of their chunks, largest first (16
// size classes a quarter octave wide, stable within a class), and jobs are numbered in that
// order: the queue hands out long jobs first and ends with short ones, which shortens the tail of
// the call. Jobs of one
// sequence are ordered chunk-major, KV head minor. What a job needs is stored by rank, so decoding
// a job number takes two ballots and one round of LDS reads.
struct SeqTable {
  int4* geo;    // [B] by sequence: beg, np, total, win_off (multi-wave build only)
  int4* rgeo;   // [B] by rank: the same
  int4* rsb;    // [B] by rank: sink, sequence, chunks, slot units per chunk (rounded down)
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

// Chunk shape of the persistent schedule. A chunk's page slots are dealt to the four waves in
// turn, so a chunk of A = 8 / SUB slots (eight 16-row items) gives each wave the same, even number
// of items: no wave idles at the job's closing barrier and none pads its item pairs with a re-read.
// Chunks are whole multiples of A slots (the u = n / A units are dealt evenly), and the last chunk
// also takes the n mod A leftover slots. A sequence never has more chunks than units.
template <int PS>
constexpr int slot_unit() { return PS == 16 ? 8 : 4; }

template <int PS>
__host__ __device__ inline int persist_chunks(int n_slots, int chunk_slots, int num_chunks) {
  if (n_slots <= 0) return 0;
  int nch = (n_slots + chunk_slots - 1) / chunk_slots;
  if (nch > num_chunks) nch = num_chunks;
  const int u = n_slots / slot_unit<PS>();
  return nch > 1 && nch > u ? (u > 1 ? u : 1) : nch;
}

// Slots [begin, end) of chunk c of nch, uq = (n_slots / A) / nch units per chunk (the first
// units % nch chunks take one unit more).
template <int PS>
__device__ __forceinline__ void persist_bounds(int n_slots, int nch, int uq, int c, int& begin,
                                               int& end) {
  constexpr int A = slot_unit<PS>();
  const int u = n_slots / A;
  const int urem = u - uq * nch;
  begin = A * (c * uq + min(c, urem));
  end = c == nch - 1 ? n_slots : begin + A * (uq + (c < urem ? 1 : 0));
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

__device__ __forceinline__ long long wave_sum64(long long x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}
// Wave reductions and the inclusive scan of the job-table build on the DPP lane network (gfx9
// row operations: quad permutes, the half-row and row mirrors, row shifts and the row-15 / row-31
// broadcasts), a few cycles a step instead of an LDS round trip (ds_bpermute) a step; the
// reductions end with the four rows' values read into scalars, so every lane gets the result.
// Lanes without a source (or in rows outside the mask) read 0.
template <int CTRL, int ROWMASK = 0xf>
__device__ __forceinline__ int dpp0(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROWMASK, 0xf, false);
}
template <int CTRL>
__device__ __forceinline__ int dpp_same(int v) {  // every lane has a source here
  return __builtin_amdgcn_update_dpp(v, v, CTRL, 0xf, 0xf, false);
}
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;
__device__ __forceinline__ float wave_sum_f(float x) {
  int v = __float_as_int(x);
  v = __float_as_int(__int_as_float(v) + __int_as_float(dpp_same<kDppXor1>(v)));
  v = __float_as_int(__int_as_float(v) + __int_as_float(dpp_same<kDppXor2>(v)));
  v = __float_as_int(__int_as_float(v) + __int_as_float(dpp_same<kDppHalfMirror>(v)));
  v = __float_as_int(__int_as_float(v) + __int_as_float(dpp_same<kDppMirror>(v)));
  return (__int_as_float(__builtin_amdgcn_readlane(v, 0)) +
          __int_as_float(__builtin_amdgcn_readlane(v, 16))) +
         (__int_as_float(__builtin_amdgcn_readlane(v, 32)) +
          __int_as_float(__builtin_amdgcn_readlane(v, 48)));
}
__device__ __forceinline__ int wave_sum_i(int v) {
  v += dpp_same<kDppXor1>(v);
  v += dpp_same<kDppXor2>(v);
  v += dpp_same<kDppHalfMirror>(v);
  v += dpp_same<kDppMirror>(v);
  return __builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16) +
         __builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48);
}
__device__ __forceinline__ int wave_max(int v) {
  v = max(v, dpp_same<kDppXor1>(v));
  v = max(v, dpp_same<kDppXor2>(v));
  v = max(v, dpp_same<kDppHalfMirror>(v));
  v = max(v, dpp_same<kDppMirror>(v));
  return max(max(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
             max(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}
__device__ __forceinline__ float wave_max_f(float x) {
  int v = __float_as_int(x);
  v = __float_as_int(fmaxf(__int_as_float(v), __int_as_float(dpp_same<kDppXor1>(v))));
  v = __float_as_int(fmaxf(__int_as_float(v), __int_as_float(dpp_same<kDppXor2>(v))));
  v = __float_as_int(fmaxf(__int_as_float(v), __int_as_float(dpp_same<kDppHalfMirror>(v))));
  v = __float_as_int(fmaxf(__int_as_float(v), __int_as_float(dpp_same<kDppMirror>(v))));
  return fmaxf(fmaxf(__int_as_float(__builtin_amdgcn_readlane(v, 0)),
                     __int_as_float(__builtin_amdgcn_readlane(v, 16))),
               fmaxf(__int_as_float(__builtin_amdgcn_readlane(v, 32)),
                     __int_as_float(__builtin_amdgcn_readlane(v, 48))));
}
// Inclusive prefix sum over the wave's 64 lanes: shifts by 1, 2, 4 and 8 within each row of 16,
// then row 0's and row 2's last lanes into rows 1 and 3, and lane 31 into rows 2 and 3.
__device__ __forceinline__ int wave_scan_i(int v) {
  v += dpp0<0x111>(v);       // row_shr:1
  v += dpp0<0x112>(v);       // row_shr:2
  v += dpp0<0x114>(v);       // row_shr:4
  v += dpp0<0x118>(v);       // row_shr:8
  v += dpp0<0x142, 0xa>(v);  // row_bcast:15
  v += dpp0<0x143, 0xc>(v);  // row_bcast:31
  return v;
}

// A plan of one job per workgroup is taken when no job is above this many times the mean work of
// a workgroup (the workgroups that finish early leave the chip to the larger jobs, which then
// stream faster). Where split sequences are merged in the kernel, a second round of jobs also
// carries the first round's merges, and one round pays off at larger jobs. Measured at the
// Llama-3-8B lengths: 8 q heads merged in the kernel, one job per workgroup (97-slot chunks, the
// largest job 1.4x the mean) 60.0 against 62.7 us for two rounds of 64-slot chunks; merged by the
// split merge kernel, 4 q heads (109-slot chunks, 1.44x) 64.1 against 60.6 us, and 2 or 4 query
// tokens 65.2 and 68.2 against 61.8 and 66.4 us.
constexpr float one_job_bound(bool merges_in_kernel) { return merges_in_kernel ? 1.5f : 1.25f; }

// With more (sequence, KV head) pairs than workgroups, sequences stay whole when the longest is at
// most this many times the mean work of a workgroup. Measured: fp8 GQA-8 shape (2048 pairs) 200.4
// against 210.3 us with the longest sequence halved; 1024 and 512 sequences of 64-1023 rows (8
// KV heads) 403.5 and 191.1 against 466.4 and 222.4 us.
constexpr float kWholeSeqBound = 1.0f;

// Chunk size in page slots of the automatic plan, chosen from the call's own lengths: N attended
// slots over the n_seq sequences that have any, at most n_max in one; H KV heads (a job is one
// chunk of one KV head); P workgroups; at least min_chunk slots and at most max_chunks chunks per
// sequence (the partial states have room for that many). jobs(c) is the call's job count with
// chunks of c slots (non-increasing in c); every thread that calls this calls it with the same
// values.
// * One job per workgroup, if no job is then above one_job (one_job_bound) times the mean work of
//   a workgroup (few sequences of similar length: long contexts, sliding windows; with split
//   sequences merged in the kernel also mixed lengths); measured 7 us (6 %) faster than two per
//   workgroup on the long-context shape.
// * Otherwise about max(2 P, 2 pairs) chunks of the longest sequence's size over the
//   (sequence, KV head) pairs: what the host plans from a tight length hint, whose chunk size was
//   tuned on the Llama-3-8B shape (64 slots there; 61 and 44 slots measured 2.4 and 2.8 us
//   slower). With more pairs than workgroups: whole sequences if none is above kWholeSeqBound
//   times the mean work of a workgroup, else the longest sequence halved.
template <typename Jobs>
__device__ int auto_chunk_slots(float N, int n_seq, int n_max, int H, int P, int min_chunk,
                                int max_chunks, float one_job, Jobs jobs) {
  // Every workgroup runs this in its prologue, so it decides from single-precision estimates
  // (the same on every workgroup) and counts jobs at most four times: 64-bit divisions and a
  // search here measured 2.3 us per call on the Llama-3-8B shape.
  if (n_max <= 0) return max(min_chunk, 1);
  min_chunk = max(min_chunk, (n_max + max_chunks - 1) / max_chunks);
  auto up = [](float x) { return int(fminf(ceilf(x), 1073741824.f)); };
  const float NH = N * float(H);
  const float pairs = float(n_seq) * float(H);
  if (pairs <= float(P)) {
    const float lim = one_job * NH / float(P);  // the largest job a one-per-workgroup plan may have
    // about the smallest chunk giving P jobs, a sequence's last chunk taken as half full, grown by
    // the excess until the plan has at most P jobs; whole sequences (n_max) give pairs <= P jobs
    int c = max(min_chunk, up(NH / (float(P) - 0.5f * pairs)));
    bool fits = false;
    for (int it = 0; it < 4 && c < n_max && float(c) <= lim; ++it) {
      const long long J = jobs(c);
      if (J <= P) {
        fits = true;
        break;
      }
      c = max(c + 1, up(float(c) * float(J) / float(P)));
    }
    if (!fits) c = n_max;
    if (float(c) <= lim) return c;
  }
  // more pairs than workgroups: whole sequences while the longest is no more than the mean work
  // of a workgroup (the queue, largest first, then balances them); else halve the longest
  if (pairs > float(P) && float(n_max) <= kWholeSeqBound * NH / float(P)) return max(min_chunk, n_max);
  const float target = fmaxf(2.f * float(P), 2.f * pairs);
  return max(min_chunk, up(pairs * float(n_max) / target));
}

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
  persist_bounds<PS>(g.n_slots, J.nch, uni(sk_b.w), J.c, sb, se);
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

// Fused append for a sequence that no job covers (no attended rows): every KV head's new K and V
// rows go to the row of position total - 1 when the sequence has pages (the append kernel's
// element arithmetic). All threads take part; one element per thread and step.
template <int KVT, int D, int PS, int NT>
__device__ void append_last_row(const DecodeParams& p, int b) {
  const SeqGeom g = seq_geom(p.indptr, p.length_info, p.B, b, PS, p.sliding);
  if (g.np == 0) return;
  const size_t page = size_t(clamp_page(p, p.values[g.beg + g.np - 1]));
  const int row = g.total - (g.np - 1) * PS - 1;
  for (int idx = threadIdx.x; idx < 2 * p.H_kv * D; idx += NT) {
    const int kv = idx / (p.H_kv * D);
    const int h = (idx - kv * p.H_kv * D) / D;
    const int d = idx % D;
    const uint16_t x = static_cast<const uint16_t*>(kv ? p.new_v : p.new_k)[(size_t(b) * p.H_kv + h) * D + d];
    const size_t dst = (((page * 2 + kv) * p.H_kv + h) * PS + row) * D + d;
    if constexpr (KVT == kFP8) {
      const float sc = (kv ? p.v_scale : p.k_scale)[h];
      static_cast<uint8_t*>(p.pages_w)[dst] = f32_to_fp8(__fdiv_rn(bf16_to_f32(x), sc));
    } else {
      static_cast<uint16_t*>(p.pages_w)[dst] = x;
    }
  }
}

// Split sequences of calls with at most this many chunks per sequence (the plan's cap) are merged
// inside the persistent kernel by its single-token instantiations; with a larger cap, and with
// several query tokens, every split sequence goes to split_merge_kernel. Measured on the same box:
// where sequences do split, the separate kernel was faster for 4 q columns (Llama-3-8B shape with
// the cap forced to 8: 61.8 against 63.4 us) and the in-kernel merge for 8 (0.6-4 us on the bf16
// and fp8 8-head shapes), and so it was with 4 q heads x 2 tokens (75.1 against 78.6 us). Where
// the automatic plan splits nothing (one job per workgroup) the second launch alone costs about
// 4 us (RoPE + window shape: 165.4 against 169.0 us), so a cap of at most 8 merges in the kernel
// at any width.
constexpr int kInMergeChunks = 8;
template <int GP>
constexpr bool merges_in_kernel(int num_chunks, bool several_tokens) {
  return GP <= 8 && !several_tokens && num_chunks <= kInMergeChunks;
}

// Output row of q column c of (sequence b, KV head h): columns are token-major (the launch's
// token c / G, i.e. the call's token tok0 + c / G; q head h G + c % G); with one token, c is the
// q head's index in the group.
template <bool MT>
__device__ __forceinline__ size_t out_row(const DecodeParams& p, int b, int h, int c) {
  if constexpr (MT)
    return (size_t(b) * p.T_all + p.tok0 + c / p.G) * p.H_qo + size_t(h) * p.G + c % p.G;
  else
    return size_t(b) * p.H_qo + size_t(h) * p.G + c;
}

// Merges the nch (2 .. kInMergeChunks) chunk states of (sequence b, KV head h), stored with
// store_agent() and complete, into out and lse (TVM relax decode-kernels page,
// _merge_state_inplace, applied over all chunks): M = max_c lse_c, w_c = 2^(lse_c - M),
// out = sum_c w_c O_c / sum_c w_c, lse = M + log2(sum_c w_c). Thread t produces 4 dims of one q
// column and loads the chunks present, 8 at a time, before using any (one memory round trip per
// 8 chunks; the state is rescaled as the running maximum grows). All threads take part.
// MT: several query tokens (p.T in the launch): G T columns, and a column whose token sees no
// row of the sequence (all chunk lse -inf) gives out = 0, lse = -5e4.
template <int D, int GP, int NT, bool MT = false>
__device__ void merge_split(const DecodeParams& p, int b, int h, int nch) {
  constexpr int V = D / 4;
  constexpr int CB = 8;  // chunks per batch of loads
  const int GC = MT ? p.G * p.T : p.G;  // columns
  for (int it = threadIdx.x; it < GC * V; it += NT) {
    const int g = it / V;
    const int v = it - g * V;
    float M = -INFINITY, ws = 0.f, a[4] = {0.f, 0.f, 0.f, 0.f};
    for (int c0 = 0; c0 < nch; c0 += CB) {
      float l[CB], o[CB][4];
#pragma unroll
      for (int u = 0; u < CB; ++u) {
        l[u] = -INFINITY;
        o[u][0] = o[u][1] = o[u][2] = o[u][3] = 0.f;
        if (c0 + u < nch) {  // uniform over the workgroup
          const size_t row = out_row<MT>(p, b, h, g) * p.num_chunks + c0 + u;
          l[u] = load_agent(&p.part_lse[row]);
#pragma unroll
          for (int k = 0; k < 4; ++k) o[u][k] = load_agent(&p.part_o[row * D + 4 * v + k]);
        }
      }
      float Mn = M;
#pragma unroll
      for (int u = 0; u < CB; ++u)
        if (c0 + u < nch) Mn = fmaxf(Mn, l[u]);
      // MT: every chunk so far may be -inf (the column's token sees none of their rows)
      const float Ms = Mn == -INFINITY ? 0.f : Mn;
      const float r = exp2_fast(M - Ms);  // 0 while M is -inf
      ws *= r;
#pragma unroll
      for (int k = 0; k < 4; ++k) a[k] *= r;
#pragma unroll
      for (int u = 0; u < CB; ++u) {
        if (c0 + u < nch) {
          const float wc = exp2_fast(l[u] - Ms);
          ws += wc;
#pragma unroll
          for (int k = 0; k < 4; ++k) a[k] = fmaf(wc, o[u][k], a[k]);
        }
      }
      M = Mn;
    }
    const bool none = MT && M == -INFINITY;
    if (none) M = 0.f;
    const size_t orow = out_row<MT>(p, b, h, g);
    float fo = 1.f;  // learned sink: folded into the denominator once, here
    if (p.sink != nullptr && !none) fo = fold_sink(p.sink[h * p.G + g % p.G] * kLog2e, M, ws);
    const float inv = none ? 0.f : fo / ws;
    uint16_t* dst = static_cast<uint16_t*>(p.out) + orow * D + 4 * v;
    *reinterpret_cast<uint2*>(dst) = make_uint2(
        uint32_t(f32_to_bf16(a[0] * inv)) | uint32_t(f32_to_bf16(a[1] * inv)) << 16,
        uint32_t(f32_to_bf16(a[2] * inv)) | uint32_t(f32_to_bf16(a[3] * inv)) << 16);
    if (v == 0) p.lse[orow] = none ? kEmptyLse : M + log2f(ws);
  }
}

// FUSED: the call also appends each sequence's new K/V row (p.new_k, p.new_v).
// MT: several query tokens per sequence (p.T_all > 1; a sliding window holds for all of them):
// the G T columns of the MFMA B operand are token-major and each is causally capped.
// ILV (with ROPE): the interleaved RoPE layout (rotary_mode 2).
template <int KVT, int D, int PS, int GP, bool ROPE, bool FUSED, bool MT = false, bool ILV = false>
__global__ __launch_bounds__(64 * kPWaves) __attribute__((amdgpu_waves_per_eu(2)))
void decode_mfma_persist_kernel(DecodeParams p) {
  // items of 16 rows: a 32-row page is two items (half the registers per item in flight)
  using C = MfmaCore<KVT, D, 16, GP, ROPE, ILV>;
  constexpr int SUB = PS / 16;
  constexpr int BLOCK = PS * C::ROW;  // bytes of one (page, K|V, head) block
  using Buf = typename C::Buf;
  constexpr int NT = 64 * kPWaves;
  // q of the next job, staged in LDS by all threads: QW 32-bit words per thread
  constexpr int QWORDS = GP * D / 2;
  constexpr int QW = (QWORDS + NT - 1) / NT;
  extern __shared__ __attribute__((aligned(16))) int s_dyn[];
  __shared__ __attribute__((aligned(16))) unsigned char s_tile[kPWaves][C::TILE_BYTES];  // V tiles
  __shared__ float s_m[kPWaves][GP];
  __shared__ float s_d[kPWaves][GP];
  __shared__ __attribute__((aligned(16))) float s_o[kPWaves][GP][D];
  __shared__ __attribute__((aligned(16))) uint32_t s_q[2][QW * NT];
  // fused append: the new K and V rows of the current and the next job, in the pool's element type
  __shared__ __attribute__((aligned(16))) uint32_t s_new[FUSED ? 2 : 1][FUSED ? 2 * C::ROW / 4 : 1];
  __shared__ int s_ids[2][kPWaves][64];  // page-table entries of each wave's first 64 items
  __shared__ float s_qsc[2][16];         // fp8 q: each MFMA column's q-head scale (1 otherwise)
  __shared__ int s_scan[kPWaves];
  __shared__ unsigned long long s_scan64[kPWaves];
  __shared__ uint32_t s_cls[kPWaves][kSizeClasses / 2];  // class counts per wave (B > 64)
  __shared__ int s_ticket;
  __shared__ int s_mrg[kPWaves];  // wave w's arrival completed the previous job's split sequence
  __shared__ float2 s_freq[ROPE ? D / 2 : 1];  // RoPE: frequencies (rope_freq) of dims i, i + D/2

  const int tid = threadIdx.x;
  PDK_MARK_DECL;
  PDK_MARK(blockIdx.x, 1, 0);
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index (wave-uniform)
  const int l = tid & 63;
  const int B = p.B;
  const int G = p.G;
  const int T = MT ? p.T : 1;
  const int GC = G * T;  // q columns of the MFMA B operand
  C core;
  core.init_lane(l);
  const int tok = MT ? core.n / G : 0;  // query token of this lane's MFMA column (in the launch)
  // several tokens: that token's RoPE offset from the call's first token, and the rows it cannot
  // see at the end of the sequence (those of the call's later tokens)
  const int qtok = MT ? p.tok0 + tok : 0;
  const int tlate = MT ? p.T_all - p.tok0 - tok : 1;
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
    constexpr int kUnit = slot_unit<PS>();
    // size class of a sequence, on a quarter-octave scale of its chunk size sz against the chunk
    // target cs: class k holds cs 2^(-(k+1)/4) < sz <= cs 2^(-k/4) (class 0 also everything
    // larger; the last class everything smaller, and sequences without chunks)
    auto size_class = [&](int n_slots, int nch, int cs) {
      if (nch <= 0) return kSizeClasses - 1;
      const float r = float((n_slots + nch - 1) / nch) / float(cs);
      // the same instructions on the same values in every workgroup: the same class
      return int(fminf(fmaxf(-4.f * __log2f(r), 0.f), float(kSizeClasses - 1)));
    };
    const int P = int(gridDim.x);
    const float one_job = one_job_bound(merges_in_kernel<GP>(p.num_chunks, MT));
    if (B <= 64) {
      // One wave, lane b for sequence b: the rank counts the sequences of lower classes (ballots)
      // and those of the same class before b (mbcnt); the job prefix is a wave scan.
      if (w == 0) {
        const bool ok = l < B;
        const SeqGeom g = seq_geom(p.indptr, p.length_info, B, ok ? l : B - 1, PS, p.sliding);
        const int n = ok ? g.n_slots : 0;
        int cs = p.chunk_slots;
        if (p.auto_chunk)
          cs = auto_chunk_slots(wave_sum_f(float(n)), __popcll(__ballot(n > 0)), wave_max(n), p.H_kv, P,
                                p.chunk_slots, p.num_chunks, one_job, [&](int cc) {
                                  // at most 64 x num_chunks: a 32-bit DPP sum
                                  return static_cast<long long>(p.H_kv) *
                                         wave_sum_i(persist_chunks<PS>(n, cc, p.num_chunks));
                                });
        // the split merge kernel reads the chunk size after the job counters
        if (p.auto_chunk && blockIdx.x == 0 && l == 0 && p.plan_word) *p.plan_word = cs;
        const int nch = persist_chunks<PS>(n, cs, p.num_chunks);
        const int nj = nch * p.H_kv;
        const int c = ok ? size_class(n, nch, cs) : kSizeClasses;
        int rank = 0;
        unsigned long long same = 0;
#pragma unroll
        for (int k = 0; k < kSizeClasses; ++k) {
          const unsigned long long m = __ballot(c == k);
          if (k < c) rank += __popcll(m);
          if (k == c) same = m;
        }
        rank += __builtin_amdgcn_mbcnt_hi(uint32_t(same >> 32),
                                          __builtin_amdgcn_mbcnt_lo(uint32_t(same), 0u));
        if (ok) {
          tab.njobs[l] = nj;
          tab.rgeo[rank] = make_int4(g.beg, g.np, g.total, g.win_off);
          tab.rsb[rank] = make_int4(g.sink, l, nch, nch > 0 ? g.n_slots / kUnit / nch : 0);
          tab.rnj[rank] = nj;
          if constexpr (ROPE) tab.rpos[rank] = make_int2(p.q_pos[l], p.k_off[l]);
        }
        wave_lds_fence();
        const int x = wave_scan_i(ok ? tab.rnj[l] : 0);  // jobs of rank l, inclusive prefix
        if (ok) tab.pre[l + 1] = x;
        if (l == 0) tab.pre[0] = 0;
      }
      __syncthreads();
    } else {
      // Every thread takes `per` consecutive sequences; class counts and the job prefix are
      // scanned over the workgroup.
      const int per = (B + NT - 1) / NT;
      static_assert(kPersistMaxBatch <= 8 * NT, "a thread's classes fit 4 bits each in an int");
      const int b0 = min(B, tid * per), b1 = min(B, b0 + per);
      // Sums over the workgroup (every thread calls them alike; s_scan64 is free again after).
      auto block_sum = [&](long long x) {
        x = wave_sum64(x);
        if (l == 0) s_scan64[w] = static_cast<unsigned long long>(x);
        __syncthreads();
        long long t = 0;
#pragma unroll
        for (int ww = 0; ww < kPWaves; ++ww) t += static_cast<long long>(s_scan64[ww]);
        __syncthreads();
        return t;
      };
      long long n_sum = 0;
      int n_seq = 0, n_max = 0;
      for (int b = b0; b < b1; ++b) {
        const SeqGeom g = seq_geom(p.indptr, p.length_info, B, b, PS, p.sliding);
        tab.geo[b] = make_int4(g.beg, g.np, g.total, g.win_off);
        tab.sink[b] = g.sink;
        tab.njobs[b] = g.n_slots;  // replaced by the job count below
        n_sum += g.n_slots;
        n_seq += g.n_slots > 0;
        n_max = max(n_max, g.n_slots);
      }
      int cs = p.chunk_slots;
      if (p.auto_chunk) {
        // totals over the workgroup in one barrier: per-wave fp32 sum and sequence count in
        // s_scan64, maximum in s_scan
        const float wsum = wave_sum_f(float(n_sum));
        const int wcnt = wave_sum_i(n_seq);
        const int wmax = wave_max(n_max);
        if (l == 0) {
          s_scan64[w] = (static_cast<unsigned long long>(static_cast<uint32_t>(wcnt)) << 32) |
                        __float_as_uint(wsum);
          s_scan[w] = wmax;
        }
        __syncthreads();
        float tot = 0.f;
        int bmax = 0, nseq = 0;
#pragma unroll
        for (int ww = 0; ww < kPWaves; ++ww) {
          tot += __uint_as_float(static_cast<uint32_t>(s_scan64[ww]));
          nseq += static_cast<int>(s_scan64[ww] >> 32);
          bmax = max(bmax, s_scan[ww]);
        }
        __syncthreads();  // s_scan64 is free again (block_sum below)
        cs = auto_chunk_slots(tot, nseq, bmax, p.H_kv, P, p.chunk_slots, p.num_chunks, one_job,
                              [&](int cc) {
          long long x = 0;
          for (int b = b0; b < b1; ++b) x += persist_chunks<PS>(tab.njobs[b], cc, p.num_chunks);
          return p.H_kv * block_sum(x);
        });
        if (blockIdx.x == 0 && tid == 0 && p.plan_word) *p.plan_word = cs;  // for split_merge_kernel
      }
      // this thread's sequences per class, 16 bits each, two classes per 32-bit word
      constexpr int kWords = kSizeClasses / 2;
      int cls_list = 0;  // classes of this thread's sequences, 4 bits each (computed once)
      uint32_t cnt[kWords];
#pragma unroll
      for (int i = 0; i < kWords; ++i) cnt[i] = 0;
      for (int b = b0; b < b1; ++b) {
        const int n = tab.njobs[b];
        const int nch = persist_chunks<PS>(n, cs, p.num_chunks);
        tab.njobs[b] = nch * p.H_kv;
        const int c = size_class(n, nch, cs);
        cls_list |= c << (4 * (b - b0));
#pragma unroll
        for (int i = 0; i < kWords; ++i) cnt[i] += c / 2 == i ? 1u << (16 * (c & 1)) : 0u;
      }
      // the 16-bit class fields hold at most 4 x 64 sequences of a wave and 1024 of the
      // workgroup: the words scan independently
      uint32_t off[kWords], total[kWords];
#pragma unroll
      for (int i = 0; i < kWords; ++i) {
        const uint32_t x = static_cast<uint32_t>(wave_scan_i(static_cast<int>(cnt[i])));
        if (l == 63) s_cls[w][i] = x;
        off[i] = x - cnt[i];
        total[i] = 0;
      }
      __syncthreads();
#pragma unroll
      for (int ww = 0; ww < kPWaves; ++ww) {
#pragma unroll
        for (int i = 0; i < kWords; ++i) {
          if (ww < w) off[i] += s_cls[ww][i];
          total[i] += s_cls[ww][i];
        }
      }
      // class c's field of a packed word array (selects, no indexed registers)
      auto field = [](const uint32_t (&a)[kWords], int c) {
        uint32_t v = 0;
#pragma unroll
        for (int i = 0; i < kWords; ++i) v = i == c / 2 ? a[i] : v;
        return int((v >> (16 * (c & 1))) & 0xffffu);
      };
      // first rank of each class (the same in every thread), computed once
      int base[kSizeClasses];
      base[0] = 0;
#pragma unroll
      for (int k = 1; k < kSizeClasses; ++k)
        base[k] = base[k - 1] + int((total[(k - 1) / 2] >> (16 * ((k - 1) & 1))) & 0xffffu);
      for (int b = b0; b < b1; ++b) {
        const int4 gg = tab.geo[b];
        const int sk = tab.sink[b];
        const int n0 = (sk + PS - 1) / PS;
        const int n_slots = gg.y > 0 ? n0 + (gg.w < gg.z ? gg.y - gg.w / PS : 0) : 0;
        const int nch = tab.njobs[b] / p.H_kv;
        const int c = (cls_list >> (4 * (b - b0))) & 15;
        // sequences of lower classes, then those of class c in lower threads and before b here
        int rank = field(off, c);
#pragma unroll
        for (int k = 1; k < kSizeClasses; ++k) rank += k == c ? base[k] : 0;
        for (int i = 0; i < b - b0; ++i) rank += ((cls_list >> (4 * i)) & 15) == c ? 1 : 0;
        tab.rgeo[rank] = gg;
        tab.rsb[rank] = make_int4(sk, b, nch, nch > 0 ? n_slots / kUnit / nch : 0);
        tab.rnj[rank] = tab.njobs[b];
        if constexpr (ROPE) tab.rpos[rank] = make_int2(p.q_pos[b], p.k_off[b]);
      }
      __syncthreads();
      int run = 0;
      for (int r = b0; r < b1; ++r) {
        run += tab.rnj[r];
        tab.pre[r + 1] = run;
      }
      const int y = wave_scan_i(run);
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
  PDK_MARK(blockIdx.x, 2, total_jobs);
  const uint32_t hinv = div_reciprocal(uint32_t(max(p.H_kv, 2)));

  // ---- sequences without attended rows: out = 0, lse = -5e4 (fused append: a sequence with pages
  // still gets its new row, written by append_last_row)
  for (int b = blockIdx.x; b < B; b += gridDim.x) {
    if (tab.njobs[b] != 0) continue;
    // this launch's tokens of sequence b: rows (b T_all + tok0 + t) H_qo + q head, t < T
    const size_t r0 = (size_t(b) * (MT ? p.T_all : 1) + (MT ? p.tok0 : 0)) * p.H_qo;
    for (int idx = tid; idx < T * p.H_qo * D; idx += NT)
      store_out<kBF16>(p.out, r0 * D + idx, 0.f);
    for (int hq = tid; hq < T * p.H_qo; hq += NT) p.lse[r0 + hq] = kEmptyLse;
    if constexpr (FUSED) append_last_row<KVT, D, PS, NT>(p, b);
  }

  const char* pool = static_cast<const char*>(p.pages);
  const size_t kv_stride = size_t(p.H_kv) * BLOCK;
  auto block_of = [&](int page, int h) {
    return pool + (size_t(page) * 2 * p.H_kv + h) * BLOCK;
  };
  const uint32_t* qsrc = static_cast<const uint32_t*>(p.q);
  // This thread's share of J's q rows (words past the G rows repeat the last one; an invalid job
  // reads sequence 0's). Unconditional loads, consumed only when staged into LDS.
  // MT: column c's row is q[b, c / G, h G + c % G, :] (token-major columns); the part of this
  // thread's word offsets that does not depend on the job, (t H_qo + g) D / 2 + word, is fixed
  int qoff[MT ? QW : 1];
  if constexpr (MT) {
#pragma unroll
    for (int i = 0; i < QW; ++i) {
      const int wd = min(tid + i * NT, GC * D / 2 - 1);
      const int c = wd / (D / 2);
      qoff[i] = ((c / G) * p.H_qo + c % G) * (D / 2) + (wd - c * (D / 2));
    }
  }
  // fp8 q (p.q_scale set): the same element pairs from 16-bit code pairs, converted exactly to
  // bf16 pairs; the q head's scale multiplies its column's scores (q_col_scale)
  const bool q8 = p.q_scale != nullptr;
  const uint16_t* q8src = static_cast<const uint16_t*>(p.q);
  auto q_word = [&](size_t i) __attribute__((always_inline)) {
    return q8 ? fp8x2_to_bf16x2<false>(uint32_t(q8src[i])) : qsrc[i];
  };
  auto q_words = [&](const Job& J, uint32_t (&qs)[QW]) {
    if constexpr (MT) {
      const size_t base = ((size_t(J.b) * p.T_all + p.tok0) * p.H_qo + size_t(J.h) * G) * (D / 2);
#pragma unroll
      for (int i = 0; i < QW; ++i) qs[i] = q_word(base + qoff[i]);
    } else {
      const size_t base = (size_t(J.b) * p.H_qo + size_t(J.h) * G) * (D / 2);
#pragma unroll
      for (int i = 0; i < QW; ++i) qs[i] = q_word(base + min(tid + i * NT, G * D / 2 - 1));
    }
  };
  // per-column score factor of fp8 q: thread c < GC loads column c's q-head scale with J's q
  // words, and it is staged into s_qsc with them
  auto q_scale_of = [&](const Job& J) __attribute__((always_inline)) {
    return q8 && tid < 16 ? p.q_scale[J.h * G + min(tid, GC - 1) % G] : 1.f;
  };

  // ---- fused append (p.new_k set): thread t < 2 * D / 8 takes 8 elements of J's new K (t < D / 8)
  // or V row: loads them with J's q words (new_words), then, once the loads are waited for,
  // encodes them into the pool's element type (fp8: x / scale rounded to e4m3fn, as the append
  // kernel), stages them in LDS for the item holding the row, and, in the sequence's last chunk,
  // stores them to the row of position total - 1 (stage_new). Every thread of an invalid job reads
  // sequence 0's rows and page-table entry 0, and nothing is staged or stored.
  constexpr bool fused = FUSED;
  constexpr int NV = D / 8;
  struct NewWords {
    uint4 x;    // 8 bf16 elements
    int pid;    // page id of the sequence's last page
    float sc;   // fp8: the row's scale
  };
  auto new_words = [&](const Job& J, NewWords& nw) __attribute__((always_inline)) {
    const int t = min(tid, 2 * NV - 1);
    const int kv = t >= NV;
    const uint16_t* src = static_cast<const uint16_t*>(kv ? p.new_v : p.new_k) +
                          (size_t(J.b) * p.H_kv + J.h) * D + 8 * (t - kv * NV);
    nw.x = *reinterpret_cast<const uint4*>(src);
    nw.pid = *(J.valid ? p.values + J.g.beg + J.g.np - 1 : p.indptr);
    nw.sc = C::FP8 ? (kv ? p.v_scale : p.k_scale)[J.h] : 1.f;
  };
  auto stage_new = [&](const Job& J, const NewWords& nw, uint32_t* dst) __attribute__((always_inline)) {
    if (!J.valid || tid >= 2 * NV) return;
    const int kv = tid >= NV;
    const int v = tid - kv * NV;
    const int row = J.g.total - (J.g.np - 1) * PS - 1;  // last_page_len - 1
    char* prow = static_cast<char*>(p.pages_w) +
                 (size_t(clamp_page(p, nw.pid)) * 2 * p.H_kv + kv * p.H_kv + J.h) * BLOCK +
                 row * C::ROW;
    const bool store = J.c == J.nch - 1;
    if constexpr (C::FP8) {
      float f[8];
      Kv<kBF16>::unpack(nw.x, f);
      uint32_t w2[2];
#pragma unroll
      for (int q = 0; q < 2; ++q)
        w2[q] = uint32_t(f32_to_fp8(__fdiv_rn(f[4 * q], nw.sc))) |
                uint32_t(f32_to_fp8(__fdiv_rn(f[4 * q + 1], nw.sc))) << 8 |
                uint32_t(f32_to_fp8(__fdiv_rn(f[4 * q + 2], nw.sc))) << 16 |
                uint32_t(f32_to_fp8(__fdiv_rn(f[4 * q + 3], nw.sc))) << 24;
      const uint2 o = make_uint2(w2[0], w2[1]);
      *reinterpret_cast<uint2*>(dst + kv * (C::ROW / 4) + 2 * v) = o;
      if (store) *reinterpret_cast<uint2*>(prow + 8 * v) = o;
    } else {
      *reinterpret_cast<uint4*>(dst + kv * (C::ROW / 4) + 4 * v) = nw.x;
      if (store) *reinterpret_cast<uint4*>(prow + 16 * v) = nw.x;
    }
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
  const float qsc0 = q_scale_of(J);
  NewWords nw0;
  if constexpr (FUSED) new_words(J, nw0);
  Job J1 = decode_job<PS, SUB, ROPE>(p, tab, total_jobs, hinv, blockIdx.x + gridDim.x, w, l);
#pragma unroll
  for (int i = 0; i < QW; ++i) s_q[0][tid + i * NT] = q0[i];
  s_ids[0][w][l] = ids0;
  if (tid < 16) s_qsc[0][tid] = qsc0;
  if constexpr (FUSED) stage_new(J, nw0, s_new[0]);
  __syncthreads();

  if (J.valid) {
    core.load_q(reinterpret_cast<const uint16_t*>(s_q[0]), GC);
    core.rope_q(J.qpos + qtok, s_freq);  // several tokens: the call's token t sits t positions later
    // fp8: the KV head's scales, or 1 with per-page scales (applied per item)
    const bool page_scales = C::FP8 && p.k_scale_page != nullptr;
    float scale = p.score_scale * (C::FP8 && !page_scales ? p.k_scale[J.h] : 1.0f);
    float qcs = s_qsc[0][core.n];  // this lane's column: its q head's scale (fp8 q), else 1
    float vscale = C::FP8 && !page_scales ? p.v_scale[J.h] : 1.0f;
    core.reset();
    Buf buf0, buf1;
    {
      const int page0 = clamp_page(p, uni(s_ids[0][w][0]));
      core.issue(buf0, block_of(page0, J.h), kv_stride);
      PDK_MARK(blockIdx.x, 3, 0);
      if constexpr (C::FP8) {
        if (page_scales) {
          buf0.ks = p.k_scale_page[size_t(page0) * p.H_kv + J.h];
          buf0.vs = p.v_scale_page[size_t(page0) * p.H_kv + J.h];
        }
      }
    }

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
    // wave's slots are unused).
    auto process_item = [&](Buf& cur, int k) __attribute__((always_inline)) {
      const int si = k / SUB;
      if (si < J.nw) {
        int j, lo, hi;
        slot_rows(J.g, J.s_w + kPWaves * si, PS, j, lo, hi);
        const int r0 = 16 * (k % SUB);
        if constexpr (FUSED) {
          if (j == J.g.np - 1) {
            // the sequence's last page: its row at position total - 1 is the appended one
            const int rn = J.g.total - (J.g.np - 1) * PS - 1 - r0;
            if (rn >= 0 && rn < 16) core.substitute(cur, rn, s_new[par]);
          }
        }
        lo = max(lo - r0, 0);
        hi = min(hi - r0, 16);
        // RoPE position of the item's row 0: attended rows are numbered from the sequence's
        // first one, so window pages shift by the rows the window skips (sink - win_off)
        const int pos0 = J.kro + j * PS + r0 +
                         (J.s_w + kPWaves * si < J.g.n0 ? 0 : J.g.sink - J.g.win_off);
        // fp8 pool with per-page scales: this item's block scales (the job's are 1); fp8 q: this
        // lane's column scale
        float isc = scale * qcs, ivf = 1.f;
        if constexpr (C::FP8) {
          if (page_scales) {
            isc = p.score_scale * cur.ks * qcs;
            ivf = cur.vs;
          }
        }
        if constexpr (MT) {
          // this lane's column (the call's token tok0 + n / G) sees positions
          // <= total - T_all + tok0 + n / G
          const int cap = J.g.total - tlate - (j * PS + r0);
          if (lo < hi)
            core.template process<true>(cur, lo, hi, isc, s_tile[w], pos0, s_freq, cap, ivf);
        } else {
          if (lo < hi) core.process(cur, lo, hi, isc, s_tile[w], pos0, s_freq, 15, ivf);
        }
      }
    };
    // Issue priority from the items this wave has left in its job: of two waves sharing a SIMD,
    // the one further from its job's end goes first. Without it the older wave wins the
    // arbitration whatever its remaining work: on the Llama-3-8B shape the first workgroup
    // dispatched to each CU drew 16.1 GB/s and the second, which shares the CU with it, 10.4 GB/s,
    // and the second ones' first jobs became the tail of the call. Measured 0.5-1.5 us faster per
    // call on that shape, 2-3 us on the fp8 GQA-8 one and 8 us on RoPE + window. The levels
    // start at 24, 12 and 6 items left: against 12, 8 and 4, 3.5 us faster on RoPE + window and
    // 0.2-0.4 us on the Llama-3-8B, GQA-8 bf16 and long-context shapes (fp8 GQA-8 unchanged);
    // counting the next job's items too was slower on the Llama-3-8B and GQA-8 bf16 shapes.
    auto set_prio = [&](int k) __attribute__((always_inline)) {
      const int rem = J.nitems - k;
      if (rem > 24) __builtin_amdgcn_s_setprio(3);
      else if (rem > 12) __builtin_amdgcn_s_setprio(2);
      else if (rem > 6) __builtin_amdgcn_s_setprio(1);
      else __builtin_amdgcn_s_setprio(0);
    };
    // process_item, then retires `cur`: only the loads just issued stay in flight.
    auto compute = [&](Buf& cur, int k) __attribute__((always_inline)) {
      set_prio(k);
      process_item(cur, k);
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(C::NLOADS));
    };
    // Issues the loads of item `k`'s 16 rows (k % SUB selects the rows in the page).
    // Items are computed in pairs, so a wave with an odd number of items in a job loads one more
    // that it does not compute, and after its last job a wave loads one item that no job uses.
    // Those padding items read a fixed block (page 0, KV head 0), which stays in L2, instead of
    // re-reading a page of the job: with non-temporal K/V loads that page has usually left L2 by
    // then, and the re-read went to HBM (about 12 MB per call on the Llama-3-8B shape: 0.9 us). A
    // wave without slots keeps reading the chunk's first page, which wave 0 loads at the same
    // time (on the fp8 GQA-8 shape, where most short chunks leave three waves idle, the fixed block
    // there was about 1 us slower).
    auto pad_item = [&](const Job& JJ, int k) __attribute__((always_inline)) {
      return JJ.nw > 0 && k / SUB >= JJ.nw;
    };
    auto issue_id = [&](Buf& nxt, int raw, int hh, int k, bool pad = false) __attribute__((always_inline)) {
      if (pad) raw = hh = 0;
      const int page = clamp_page(p, uni(raw));
      core.issue(nxt, block_of(page, uni(hh)) + (k % SUB) * 16 * C::ROW, kv_stride);
      if constexpr (C::FP8) {
        if (page_scales) {  // the item's block scales, loaded with its rows
          const size_t e = size_t(page) * p.H_kv + uni(hh);
          nxt.ks = p.k_scale_page[e];
          nxt.vs = p.v_scale_page[e];
        }
      }
    };

    // Split sequences are merged here when the call has few chunks. Each wave arrives at its
    // sequence's counter once its own partial stores are known complete (in the next job's first
    // pair, where they are older than the loads waited for); the workgroup whose wave brings the
    // count to chunks x waves merges the sequence at the end of that next job. pb < 0: no
    // arrival pending.
    const bool in_merge = merges_in_kernel<GP>(p.num_chunks, MT);
    int pb = -1, ph = 0, pnch = 0;

    // Every job has an even number of items per wave, item k in buf0 for even k, so the next
    // job's first item is always in flight in buf0 when a job ends: every path into the loops has
    // the same loads in flight and the compiler's wait counts stay exact. (Also issuing the next
    // job's second item before the job-end merge, keeping two items in flight through it, measured
    // 1-2 us slower per call on the Llama-3-8B, long-context and RoPE + window shapes.)
    for (;;) {
      PDK_MARK(blockIdx.x, 4, J.nw);
      int arrival = 0;  // this wave's arrival for the previous job's split sequence
      // ---- items 0 and 1, with the loads for the next job (its page ids and q words, staged into
      // LDS once item 1 is computed). The ticket of the job after the next one is taken in the
      // last pair of items, so a workgroup holds at most one job beyond the current one.
      {
        const bool last = J.nitems == 2;
        const int ids_n = load_id(p, J1, l);
        uint32_t qs[QW];
        q_words(J1, qs);
        const float qsc_n = q_scale_of(J1);
        NewWords nw1;
        if constexpr (FUSED) new_words(J1, nw1);
        int ticket_raw = 0;
        if (last && J1.valid && tid == 0) ticket_raw = atomicAdd(queue, 1);
        issue_id(buf1, item_id(1), J.h, 1, pad_item(J, 1));
        // no wait after item 0: the next job's ids and q words were issued with item 1, and
        // waiting for them here would leave only item 1 in flight while they arrive
        process_item(buf0, 0);
        if (!last) issue_id(buf0, item_id(2), J.h, 2, pad_item(J, 2));
        else if (J1.valid) issue_id(buf0, __builtin_amdgcn_readlane(ids_n, 0), J1.h, 0);
        else issue_id(buf0, item_id(1), J.h, 1, true);
        compute(buf1, 1);
        // the previous job's partial stores are older than the loads just waited for; the
        // arrival's result is read at the end of this job
        if (pb >= 0 && l == 0)
          arrival = __hip_atomic_fetch_add(&p.counters[pb * p.H_kv + ph], 1, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
        for (int i = 0; i < QW; ++i) s_q[par ^ 1][tid + i * NT] = qs[i];
        s_ids[par ^ 1][w][l] = ids_n;
        if (tid < 16) s_qsc[par ^ 1][tid] = qsc_n;
        if constexpr (FUSED) stage_new(J1, nw1, s_new[par ^ 1]);
        if (last && tid == 0) s_ticket = 2 * int(gridDim.x) + ticket_raw;
      }
      // ---- items 2 .. nitems - 3
      for (int k = 2; k + 2 < J.nitems; k += 2) {
        issue_id(buf1, item_id(k + 1), J.h, k + 1, pad_item(J, k + 1));
        compute(buf0, k);
        issue_id(buf0, item_id(k + 2), J.h, k + 2, pad_item(J, k + 2));
        compute(buf1, k + 1);
      }
      // ---- the last pair takes the ticket and issues the next job's first item
      if (J.nitems > 2) {
        const int k = J.nitems - 2;
        int ticket_raw = 0;
        if (J1.valid && tid == 0) ticket_raw = atomicAdd(queue, 1);
        issue_id(buf1, item_id(k + 1), J.h, k + 1, pad_item(J, k + 1));
        compute(buf0, k);
        if (J1.valid) issue_id(buf0, s_ids[par ^ 1][w][0], J1.h, 0);
        else issue_id(buf0, item_id(k + 1), J.h, k + 1, true);
        compute(buf1, k + 1);
        if (tid == 0) s_ticket = 2 * int(gridDim.x) + ticket_raw;
      }

      // ---- end of job J: merge the waves, store
      if (l == 0) s_mrg[w] = pb >= 0 && arrival == pnch * kPWaves - 1;
      core.to_lds(s_m[w], s_d[w], s_o[w]);
      __syncthreads();
      const int next_ticket = s_ticket;
      int merge_prev = 0;  // s_mrg: written before the barrier above, rewritten after the next one
#pragma unroll
      for (int ww = 0; ww < kPWaves; ++ww) merge_prev |= s_mrg[ww];
#pragma unroll
      for (int it = 0; it < (GP * D + NT - 1) / NT; ++it) {
        const int idx = tid + it * NT;
        if (idx < GC * D) {
          const int g = idx / D;
          const int d = idx - g * D;
          float M = -INFINITY;
#pragma unroll
          for (int ww = 0; ww < kPWaves; ++ww) M = fmaxf(M, s_m[ww][g]);
          // MT: a column whose token sees no row of this job (M = -inf) leaves out 0 and lse
          // -5e4, or a partial of weight 0
          const bool none = MT && M == -INFINITY;
          if (MT && none) M = 0.f;
          float wsum = 0.f, o = 0.f;
#pragma unroll
          for (int ww = 0; ww < kPWaves; ++ww) {
            const float f = exp2_fast(s_m[ww][g] - M);  // 0 for a wave without slots
            wsum = fmaf(f, s_d[ww][g], wsum);
            o = fmaf(f, s_o[ww][g][d], o);
          }
          const size_t orow = out_row<MT>(p, J.b, J.h, g);
          // learned sink: folded into a finished row only (a split one gets it when merged)
          if (p.sink != nullptr && J.nch == 1 && !none)
            o *= fold_sink(p.sink[J.h * G + g % G] * kLog2e, M, wsum);
          const float val = none ? 0.f : o / wsum * vscale;
          const float l2 = none ? (J.nch == 1 ? kEmptyLse : -INFINITY) : M + log2f(wsum);
          if (J.nch == 1) {
            store_out<kBF16>(p.out, orow * D + d, val);
            if (d == 0) p.lse[orow] = l2;
          } else {
            const size_t row = orow * p.num_chunks + J.c;
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
      PDK_MARK(blockIdx.x, 5, merge_prev);
      if constexpr (!MT) {  // several tokens never merge in the kernel (merges_in_kernel)
        if (merge_prev) {
          merge_split<D, GP, NT, MT>(p, pb, ph, pnch);
          if (tid == 0)
            __hip_atomic_store(&p.counters[pb * p.H_kv + ph], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
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
          if constexpr (!MT) {
            if (s_ticket) {
              merge_split<D, GP, NT, MT>(p, pb, ph, pnch);
              if (tid == 0)
                __hip_atomic_store(&p.counters[pb * p.H_kv + ph], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
          }
        }
        break;
      }
      // ---- move on: J1 becomes current; decode the job after it
      J = J1;
      par ^= 1;
      core.load_q(reinterpret_cast<const uint16_t*>(s_q[par]), GC);
      qcs = s_qsc[par][core.n];
      core.rope_q(J.qpos + qtok, s_freq);  // several tokens: the call's token t sits t positions later
      if (C::FP8 && !page_scales) {
        scale = p.score_scale * p.k_scale[J.h];
        vscale = p.v_scale[J.h];
      }
      core.reset();
      J1 = decode_job<PS, SUB, ROPE>(p, tab, total_jobs, hinv, next_ticket, w, l);
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  }

  PDK_MARK(blockIdx.x, 6, 0);
  // ---- the last workgroup out puts the queue back to zero for the next call
  if (tid == 0 && atomicAdd(queue + 1, 1) == int(gridDim.x) - 1) {
    __hip_atomic_store(queue, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(queue + 1, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Workgroups of a kernel that fit on the current device at once (cached per kernel, device and
// dynamic LDS size).
inline int resident_workgroups(const void* kernel, size_t lds) {
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

template <int KVT, int D, int PS, int GP, bool ROPE, bool FUSED, bool MT = false, bool ILV = false>
hipError_t launch_persist_k(const DecodeParams& p, long long max_jobs, hipStream_t st) {
  const void* k = reinterpret_cast<const void*>(
      &decode_mfma_persist_kernel<KVT, D, PS, GP, ROPE, FUSED, MT, ILV>);
  const size_t lds = seq_table_bytes(p.B);
  const int resident = resident_workgroups(k, lds);
  if (resident <= 0) return hipErrorInvalidConfiguration;
  long long g = resident < kPersistMaxGrid ? resident : kPersistMaxGrid;
  if (max_jobs < g) g = max_jobs > 0 ? max_jobs : 1;
  const unsigned grid = static_cast<unsigned>(g);
  hipLaunchKernelGGL((decode_mfma_persist_kernel<KVT, D, PS, GP, ROPE, FUSED, MT, ILV>), dim3(grid),
                     dim3(64 * kPWaves), lds, st, p);
  return hipGetLastError();
}

// The fused-append instantiations of launch_persist_k (decode_fused.hip).
template <int KVT, int D, int PS, int GP, bool ROPE>
hipError_t launch_persist_fused(const DecodeParams& p, long long max_jobs, hipStream_t st);

// The several-query-token instantiations of launch_persist_k (decode_multi.hip): without and with
// RoPE in either layout; no fused append.
template <int KVT, int D, int PS, int GP, bool ROPE>
hipError_t launch_persist_multi(const DecodeParams& p, long long max_jobs, hipStream_t st);

// The interleaved-RoPE instantiations of launch_persist_k (decode_rope_ilv.hip): bf16 and fp8 KV,
// plain and fused.
template <int KVT, int D, int PS, int GP>
hipError_t launch_persist_ilv(const DecodeParams& p, long long max_jobs, hipStream_t st);

// The e5m2-pool instantiations of launch_persist_k (decode_e5m2.hip): one query token, no fused
// append, without RoPE or with rotate-half RoPE.
template <int D, int PS, int GP, bool ROPE>
hipError_t launch_persist_e5m2(const DecodeParams& p, long long max_jobs, hipStream_t st);

}  // namespace pdk
