// Paged-KV decode attention for bf16 or fp8-e4m3fn KV (bf16 q) on gfx950: q.K and P.V on the
// matrix cores, the softmax on the vector ALUs, optional RoPE on q and K in registers (per-item
// steps: mfma_core.hpp).
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
//    In the single-token instantiations, when the call has at most kInMergeChunks chunks per
//    sequence, the workgroup whose waves complete a split sequence's count of arrivals merges
//    it at the end of its next job (each wave arrives once its own partial stores are known
//    complete, a pair of items into the next job, so no wait falls on the load stream); otherwise
//    a second, row-parallel kernel (split_merge_kernel) merges them (merges_in_kernel). The chunk
//    size is chosen on the device from the call's lengths (auto_chunk_slots) unless the caller
//    fixed the split count.
//  * one workgroup per job (decode_mfma_kernel), for batches too large for the LDS job table: the
//    last workgroup of a split sequence to finish merges it (split.hpp).
#include "decode_persist.hpp"
#include "launch.hpp"

namespace pdk {

constexpr int kWaves = 4;             // wavefronts per workgroup

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
  __shared__ __attribute__((aligned(16))) unsigned char s_tile[kWaves][C::TILE_BYTES];  // V tiles
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
        if (lo < hi) core.process(buf[r], lo, hi, scale, s_tile[w], pos0, s_freq);
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
  constexpr int NB = 4;         // float4 loads per lane per batch
  constexpr int CB = NB * CPW;  // chunks per batch
  static_assert(64 % CB == 0 || CB % 64 == 0, "batches and lse words line up");
  const int lane = threadIdx.x & 63;
  PDK_MARK_DECL;
  PDK_MARK(2048 + blockIdx.x, 7, 0);
  // this launch's rows [B, T, H_qo], i.e. rows (b T_all + tok0 + t) H_qo + q head of the call
  const int lrow = blockIdx.x * kMergeRows + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (lrow >= p.B * p.T * p.H_qo) return;
  const int b = lrow / (p.T * p.H_qo);
  const int row = (b * p.T_all + p.tok0) * p.H_qo + (lrow - b * p.T * p.H_qo);
  const int nc = p.num_chunks;
  const float* lse_c = p.part_lse + size_t(row) * nc;
  const float* o_c = p.part_o + size_t(row) * nc * D;
  const int v = lane % V, ph = lane / V;
  // the first batch is loaded before the row's chunk count is known (indexes clamped into the
  // plan's slots); later ones once it is, clamped to the row's own chunks (no stale rows read),
  // two batches in flight
  float4 x[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i)
    x[i] = *reinterpret_cast<const float4*>(o_c + size_t(min(i * CPW + ph, nc - 1)) * D + 4 * v);
  const float lse_l = lse_c[min(lane, nc - 1)];
  // automatic plan: the chunk size the decode kernel chose (its workgroup 0 stored it after the
  // partial lse); loaded with the rest, used only once everything has arrived
  const int cs = p.auto_chunk ? *p.plan_word : p.chunk_slots;
  const SeqGeom sg = seq_geom(p.indptr, p.length_info, p.B, b, PS, p.sliding);
  const int nch = persist_chunks<PS>(sg.n_slots, cs, nc);

  float mx = lane < nch ? lse_l : -INFINITY;
  for (int c = 64 + lane; c < nch; c += 64) mx = fmaxf(mx, lse_c[c]);
  mx = wave_max_f(mx);
  // several query tokens: a token that sees no row of the sequence has every chunk lse -inf
  const bool none = mx == -INFINITY;
  const float M = none ? 0.f : mx;
  const float w_l = lane < nch ? exp2_fast(lse_l - M) : 0.f;  // weight of chunk `lane`
  float ws = w_l;
  for (int c = 64 + lane; c < nch; c += 64) ws += exp2_fast(lse_c[c] - M);
  ws = wave_sum_f(ws);

  constexpr int NB2 = NB;          // float4 loads per lane in a later batch
  constexpr int CB2 = NB2 * CPW;   // chunks per later batch
  float4 y[NB2], z[NB2];
  auto load_later = [&](float4 (&buf)[NB2], int c0) {
#pragma unroll
    for (int i = 0; i < NB2; ++i)
      buf[i] = *reinterpret_cast<const float4*>(o_c + size_t(min(c0 + i * CPW + ph, nch - 1)) * D + 4 * v);
  };
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  auto accumulate = [&](const auto& buf, int c0) __attribute__((always_inline)) {
    constexpr int nb = sizeof(buf) / sizeof(float4);
#pragma unroll
    for (int i = 0; i < nb; ++i) {
      const int c = c0 + i * CPW + ph;
      const float wc = c < 64 ? __shfl(w_l, c & 63, 64) : exp2_fast(lse_c[min(c, nc - 1)] - M);
      if (c < nch) {  // select, not a product: a stale partial past nch may hold any bits
        acc.x = fmaf(wc, buf[i].x, acc.x);
        acc.y = fmaf(wc, buf[i].y, acc.y);
        acc.z = fmaf(wc, buf[i].z, acc.z);
        acc.w = fmaf(wc, buf[i].w, acc.w);
      }
    }
  };
  if (CB < nch) load_later(y, CB);
  if (CB + CB2 < nch) load_later(z, CB + CB2);
  accumulate(x, 0);
  for (int c0 = CB; c0 < nch; c0 += 2 * CB2) {
    accumulate(y, c0);
    if (c0 + 2 * CB2 < nch) load_later(y, c0 + 2 * CB2);
    if (c0 + CB2 < nch) {
      accumulate(z, c0 + CB2);
      if (c0 + 3 * CB2 < nch) load_later(z, c0 + 3 * CB2);
    }
  }
  // add the CPW chunk phases (lanes v, v + V, ...): over l ^ 32, and for V = 16 over l ^ 16 first
  static_assert(V == 16 || V == 32, "two or four chunk phases");
  if constexpr (V == 16) {
    acc.x = xsum<16>(acc.x);
    acc.y = xsum<16>(acc.y);
    acc.z = xsum<16>(acc.z);
    acc.w = xsum<16>(acc.w);
  }
  acc.x = xsum<32>(acc.x);
  acc.y = xsum<32>(acc.y);
  acc.z = xsum<32>(acc.z);
  acc.w = xsum<32>(acc.w);
  if (nch <= 1) return;  // unsplit (or empty) sequence: the decode kernel wrote its row
  float Mf = M;
  float fo = 1.f;  // learned sink of the row's q head, folded once
  if (p.sink != nullptr && !none) fo = fold_sink(p.sink[row % p.H_qo] * kLog2e, Mf, ws);
  if (lane < V) {
    const float inv = none ? 0.f : fo / ws;
    uint16_t* dst = static_cast<uint16_t*>(p.out) + size_t(row) * D + 4 * lane;
    const uint2 packed = make_uint2(
        uint32_t(f32_to_bf16(acc.x * inv)) | uint32_t(f32_to_bf16(acc.y * inv)) << 16,
        uint32_t(f32_to_bf16(acc.z * inv)) | uint32_t(f32_to_bf16(acc.w * inv)) << 16);
    *reinterpret_cast<uint2*>(dst) = packed;
  }
  if (lane == 0) p.lse[row] = none ? kEmptyLse : Mf + log2f(ws);
  PDK_MARK(2048 + blockIdx.x, 8, 0);
}

// ------------------------------------------------------------------------------------------------
// Launchers.

template <int KVT, int D, int PS, int GP, bool ROPE>
static hipError_t launch_chunked(const DecodeParams& p, unsigned grid, hipStream_t st) {
  hipLaunchKernelGGL((decode_mfma_kernel<KVT, D, PS, GP, ROPE>), dim3(grid), dim3(64 * kWaves), 0,
                     st, p);
  return hipGetLastError();
}

// After a persistent decode: the split merge kernel, where split sequences were left to it.
template <int D, int PS, int GP>
static hipError_t merge_splits(const DecodeParams& p, hipStream_t st) {
  if (p.num_chunks <= 1 || merges_in_kernel<GP>(p.num_chunks, p.T_all > 1)) return hipSuccess;
  const unsigned rows = static_cast<unsigned>(p.B) * p.T * p.H_qo;
  hipLaunchKernelGGL((split_merge_kernel<D, PS>), dim3((rows + kMergeRows - 1) / kMergeRows),
                     dim3(64 * kMergeRows), 0, st, p);
  return hipGetLastError();
}

template <int KVT, int D, int PS, int GP, bool ROPE>
static hipError_t launch_persist(const DecodeParams& p, long long max_jobs, hipStream_t st) {
  hipError_t e;
  if constexpr (GP == 16) {  // 16 q columns: several query tokens only
    if (p.T_all <= 1) return hipErrorInvalidValue;
    e = launch_persist_multi<KVT, D, PS, GP, ROPE>(p, max_jobs, st);
  } else if (p.T_all > 1) {  // several tokens, also a launch of one of them
    e = launch_persist_multi<KVT, D, PS, GP, ROPE>(p, max_jobs, st);  // either RoPE layout
  } else if (ROPE && p.rotary == 2) {
    e = launch_persist_ilv<KVT, D, PS, GP>(p, max_jobs, st);  // interleaved RoPE, plain or fused
  } else {
    e = p.new_k != nullptr ? launch_persist_fused<KVT, D, PS, GP, ROPE>(p, max_jobs, st)
                           : launch_persist_k<KVT, D, PS, GP, ROPE, false>(p, max_jobs, st);
  }
  return e != hipSuccess ? e : merge_splits<D, PS, GP>(p, st);
}

// e5m2 pool: the persistent schedule, one query token, no fused append, no RoPE or rotate-half
// RoPE (the host refuses the rest).
template <int D, int PS, int GP>
static hipError_t launch_e5m2_g(const DecodeParams& p, bool rope, long long grid, hipStream_t st) {
  if (p.T_all != 1 || p.new_k != nullptr || (rope && p.rotary != 1)) return hipErrorInvalidValue;
  const hipError_t e = rope ? launch_persist_e5m2<D, PS, GP, true>(p, grid, st)
                            : launch_persist_e5m2<D, PS, GP, false>(p, grid, st);
  return e != hipSuccess ? e : merge_splits<D, PS, GP>(p, st);
}

template <int D, int PS>
static hipError_t launch_e5m2_shape(const DecodeParams& p, int gp, bool rope, long long grid,
                                    hipStream_t st) {
  switch (gp) {
    case 1: return launch_e5m2_g<D, PS, 1>(p, rope, grid, st);
    case 2: return launch_e5m2_g<D, PS, 2>(p, rope, grid, st);
    case 4: return launch_e5m2_g<D, PS, 4>(p, rope, grid, st);
    case 8: return launch_e5m2_g<D, PS, 8>(p, rope, grid, st);
  }
  return hipErrorInvalidValue;
}

static hipError_t launch_e5m2(const DecodeParams& p, int D, int PS, int gp, bool persistent,
                              bool rope, long long grid, hipStream_t st) {
  if (!persistent) return hipErrorInvalidValue;
  if (D == 64 && PS == 16) return launch_e5m2_shape<64, 16>(p, gp, rope, grid, st);
  if (D == 64 && PS == 32) return launch_e5m2_shape<64, 32>(p, gp, rope, grid, st);
  if (D == 128 && PS == 16) return launch_e5m2_shape<128, 16>(p, gp, rope, grid, st);
  if (D == 128 && PS == 32) return launch_e5m2_shape<128, 32>(p, gp, rope, grid, st);
  return hipErrorInvalidValue;
}

// RoPE on the matrix cores: bf16 or fp8 KV, every head dim.
template <int KVT, int D, int PS, int GP>
static hipError_t launch_sched(const DecodeParams& p, bool persistent, bool rope, long long grid,
                               hipStream_t st) {
  if constexpr (GP == 16) {  // several query tokens on the persistent schedule only
    if (!persistent) return hipErrorInvalidValue;
    return rope ? launch_persist<KVT, D, PS, GP, true>(p, grid, st)
                : launch_persist<KVT, D, PS, GP, false>(p, grid, st);
  }
  if (rope)
    return persistent ? launch_persist<KVT, D, PS, GP, true>(p, grid, st)
                      : launch_chunked<KVT, D, PS, GP, true>(p, static_cast<unsigned>(grid), st);
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
    case 16: return launch_sched<KVT, D, PS, 16>(p, persistent, rope, grid, st);
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
  if (kv_dtype == kFP8E5M2) return launch_e5m2(p, D, PS, gp, persistent, rope, grid, st);
  return hipErrorInvalidValue;
}

}  // namespace pdk

#ifdef PDECODE_TIMELINE
// Timeline build only: copy the marks out / clear them (synchronous; host buffer of
// kTimelineRows x kTimelineMarks uint64).
extern "C" int pdk_timeline_read(void* host) {
  return hipMemcpyFromSymbol(host, HIP_SYMBOL(pdk::g_timeline), sizeof(pdk::g_timeline)) ==
                 hipSuccess ? 0 : 1;
}
extern "C" int pdk_timeline_clear() {
  static unsigned long long zero[pdk::kTimelineRows][pdk::kTimelineMarks];
  return hipMemcpyToSymbol(HIP_SYMBOL(pdk::g_timeline), zero, sizeof(zero)) == hipSuccess ? 0 : 1;
}
#endif
