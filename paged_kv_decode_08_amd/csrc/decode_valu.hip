// Paged-KV single-token decode attention, gfx950 (wave64). One wavefront per
// (sequence, KV head, chunk of page slots).
//
// Computation (TVM relax decode-kernels page, _attention_decode_cpu / _attention_decode): scores
// s = sm_scale * q . k in log2 units, online softmax with a running max m and denominator d, output
// O / d and lse = m + log2(d). Split-KV chunks write normalised partial states that are combined
// by log-sum-exp (the page's merge-state formula applied over all chunks).
//
// Data path per page slot: the (page, K|V, head) block of page_size rows is contiguous
// (page_size * head_dim * elem_bytes bytes, 1-16 KiB). The wave reads it with 16-byte loads,
// lane l taking bytes [16 l, 16 l + 16) of every 1 KiB, so each load instruction is one
// contiguous KiB. A lane therefore holds EPV consecutive elements (column vector cv = l % VPR) of
// rows i * RPI + l / VPR. q . k is a per-lane partial dot over its EPV elements followed by a
// butterfly sum over the VPR lanes of the row; every lane then holds the full scores of its
// rows, which are exactly the rows of the V elements it holds, so P.V needs no data exchange.
// Each row group keeps partial (d, O) under a wave-uniform running max; they are summed across
// row groups once at the end. The next slot's K/V is loaded while the current one is computed;
// page ids come from one coalesced load per 64 slots. A split sequence is finished by the last of
// its workgroups to arrive (split.hpp).
#include "device.hpp"
#include "launch.hpp"
#include "split.hpp"

namespace pdk {

__device__ __forceinline__ float shfl_xor_f(float v, int mask) { return __shfl_xor(v, mask, 64); }

constexpr int kRopeAnchor = 8;  // page slots between exact RoPE angles (the rest by recurrence)

template <int KVT, int QT, int D, int PS, int GP>
__global__ __launch_bounds__(64) void decode_valu_kernel(DecodeParams p) {
  using KV = Kv<KVT>;
  constexpr int EPV = KV::EPV;           // elements per 16-byte vector
  constexpr int VPR = D / EPV;           // vectors per row
  constexpr int RPI = 64 / VPR;          // rows per load instruction
  constexpr int NI = PS / RPI;           // load instructions per (page, K|V, head) block
  constexpr int BLOCK_BYTES = PS * D * KV::EB;
  static_assert(VPR >= 1 && VPR <= 64 && PS % RPI == 0, "unsupported shape");

  const int lane = threadIdx.x;
  const int cv = lane % VPR;
  const int rg = lane / VPR;
  const int units = p.B * p.H_kv;
  const int c = blockIdx.x / units;
  const int u = blockIdx.x - c * units;
  const int b = u / p.H_kv;
  const int h = u - b * p.H_kv;
  const int G = p.G;

  const SeqGeom sg = seq_geom(p.indptr, p.length_info, p.B, b, PS, p.sliding);
  const int nch = chunks_used(sg.n_slots, p.chunk_slots, p.num_chunks);
  if (nch == 0) {
    // No attended rows: out = 0 and lse = -5e4, written by chunk 0 only.
    if (c != 0) return;
    for (int g = 0; g < G; ++g) {
      const int hq = h * G + g;
      for (int d = lane; d < D; d += 64) store_out<QT>(p.out, (size_t(b) * p.H_qo + hq) * D + d, 0.f);
      if (lane == 0) p.lse[size_t(b) * p.H_qo + hq] = kEmptyLse;
    }
    return;
  }
  if (c >= nch) return;
  int s_begin, s_end;
  chunk_bounds(sg.n_slots, nch, c, s_begin, s_end);

  // ---- q (fp32, pre-scaled to log2 units; fp8 folds k_scale in), optionally rotated.
  const float kscale = (KVT == kFP8) ? p.k_scale[h] : 1.0f;
  const float qscale = p.score_scale * kscale;
  const bool rotary = p.rotary != 0;
  const int d0 = cv * EPV;                       // first dim this lane holds
  const bool lower = d0 < D / 2;
  float fhi[EPV], flo[EPV];                      // RoPE frequencies / 2pi of the lane's dims
  // RoPE angle of the lane's current K row (cos, sin per dim), advanced row by row by the
  // rotation of RPI positions (stc, sts); re-anchored exactly every kRopeAnchor slots and where
  // the compacted positions jump (first window slot after the sink pages)
  float rc[EPV] = {}, rsn[EPV] = {}, stc[EPV] = {}, sts[EPV] = {};
  float qo[GP][EPV];
#pragma unroll
  for (int g = 0; g < GP; ++g) {
    const bool live = g < G;
    const size_t qb = (size_t(b) * p.H_qo + h * G + (live ? g : 0)) * D;
#pragma unroll
    for (int e = 0; e < EPV; ++e) qo[g][e] = live ? load_q<QT>(p.q, qb + d0 + e) : 0.f;
  }
  if (rotary) {
    const int qpos = p.q_pos[b];
    const int pd0 = lower ? d0 + D / 2 : d0 - D / 2;   // partner dims
#pragma unroll
    for (int e = 0; e < EPV; ++e) {
      rope_freq((d0 + e) % (D / 2), D, p.rope_scale, p.rope_theta, fhi[e], flo[e]);
      rope_cs(RPI, fhi[e], flo[e], stc[e], sts[e]);
      float cs, sn;
      rope_cs(qpos, fhi[e], flo[e], cs, sn);
#pragma unroll
      for (int g = 0; g < GP; ++g) {
        const bool live = g < G;
        const size_t qb = (size_t(b) * p.H_qo + h * G + (live ? g : 0)) * D;
        const float partner = live ? load_q<QT>(p.q, qb + pd0 + e) : 0.f;
        qo[g][e] = lower ? qo[g][e] * cs - partner * sn : qo[g][e] * cs + partner * sn;
      }
    }
  }
#pragma unroll
  for (int g = 0; g < GP; ++g)
#pragma unroll
    for (int e = 0; e < EPV; ++e) qo[g][e] *= qscale;

  // ---- running state: m is wave-uniform per head; d and O are per row group.
  float m[GP], dsum[GP], O[GP][EPV];
#pragma unroll
  for (int g = 0; g < GP; ++g) {
    m[g] = -INFINITY;
    dsum[g] = 0.f;
#pragma unroll
    for (int e = 0; e < EPV; ++e) O[g][e] = 0.f;
  }

  const char* pool = static_cast<const char*>(p.pages);
  const int kro = rotary ? p.k_off[b] : 0;
  auto slot_page = [&](int s) { return s < sg.n0 ? s : sg.first1 + (s - sg.n0); };
  int ids = 0;
  auto load_ids = [&](int base) {
    const int s = base + lane;
    int id = 0;
    if (s < s_end) id = p.values[sg.beg + min(slot_page(s), sg.np - 1)];
    ids = min(max(id, 0), p.max_num_pages - 1);
  };
  auto issue = [&](uint4 (&kr)[NI], uint4 (&vr)[NI], int page) {
    const char* kb = pool + (size_t(page) * 2 * p.H_kv + h) * BLOCK_BYTES + lane * 16;
    const char* vb = kb + size_t(p.H_kv) * BLOCK_BYTES;
#pragma unroll
    for (int i = 0; i < NI; ++i) kr[i] = kv_load(reinterpret_cast<const uint4*>(kb + i * 1024));
#pragma unroll
    for (int i = 0; i < NI; ++i) vr[i] = kv_load(reinterpret_cast<const uint4*>(vb + i * 1024));
  };

  uint4 kc[NI], vc[NI], kn[NI], vn[NI];
  load_ids(s_begin);
  int pg = __builtin_amdgcn_readfirstlane(ids);
  issue(kc, vc, pg);
  for (int s = s_begin; s < s_end; ++s) {
    const int sn = s + 1;
    int pgn = pg;
    if (sn < s_end) {
      if (((sn - s_begin) & 63) == 0) load_ids(sn);
      pgn = __builtin_amdgcn_readlane(ids, (sn - s_begin) & 63);
    }
    issue(kn, vn, pgn);  // past the end this re-reads the current block (a cache hit)

    // Rows of this slot's page that are attended, and the compacted-row offset for RoPE.
    const int j = slot_page(s);
    int lo, hi, roff;
    if (s < sg.n0) {
      lo = 0;
      hi = min(PS, sg.sink - j * PS);
      roff = 0;
    } else {
      lo = max(0, sg.win_off - j * PS);
      hi = min(PS, sg.total - j * PS);
      roff = sg.sink - sg.win_off;
    }

    // ---- scores
    if (rotary && (s == s_begin || s == sg.n0 || (s - s_begin) % kRopeAnchor == 0)) {
      const int pos0 = kro + j * PS + rg + roff;  // the lane's first row in this page
#pragma unroll
      for (int e = 0; e < EPV; ++e) rope_cs(pos0, fhi[e], flo[e], rc[e], rsn[e]);
    }
    float sc[NI][GP];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      float kf[EPV];
      KV::unpack(kc[i], kf);
      if (rotary) {
        float kp[EPV];
#pragma unroll
        for (int e = 0; e < EPV; ++e) kp[e] = shfl_xor_f(kf[e], VPR / 2);
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
          kf[e] = lower ? kf[e] * rc[e] - kp[e] * rsn[e] : kf[e] * rc[e] + kp[e] * rsn[e];
          const float c2 = rc[e] * stc[e] - rsn[e] * sts[e];  // next row: RPI positions on
          rsn[e] = rsn[e] * stc[e] + rc[e] * sts[e];
          rc[e] = c2;
        }
      }
#pragma unroll
      for (int g = 0; g < GP; ++g) {
        float a = 0.f;
#pragma unroll
        for (int e = 0; e < EPV; ++e) a = fmaf(qo[g][e], kf[e], a);
        sc[i][g] = a;
      }
    }
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int g = 0; g < GP; ++g)
#pragma unroll
        for (int msk = 1; msk < VPR; msk <<= 1) sc[i][g] += shfl_xor_f(sc[i][g], msk);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int row = i * RPI + rg;
      if (row < lo || row >= hi) {
#pragma unroll
        for (int g = 0; g < GP; ++g) sc[i][g] = -INFINITY;
      }
    }

    // ---- online softmax (base 2)
#pragma unroll
    for (int g = 0; g < GP; ++g) {
      float tm = sc[0][g];
#pragma unroll
      for (int i = 1; i < NI; ++i) tm = fmaxf(tm, sc[i][g]);
#pragma unroll
      for (int msk = VPR; msk < 64; msk <<= 1) tm = fmaxf(tm, shfl_xor_f(tm, msk));
      const float mn = fmaxf(m[g], tm);
      const float alpha = exp2f(m[g] - mn);
      m[g] = mn;
      dsum[g] *= alpha;
#pragma unroll
      for (int e = 0; e < EPV; ++e) O[g][e] *= alpha;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const float pr = exp2f(sc[i][g] - mn);
        sc[i][g] = pr;
        dsum[g] += pr;
      }
    }

    // ---- P.V
    const bool partial = lo > 0 || hi < PS;  // rows outside [lo, hi) may hold anything, even NaN
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      float vf[EPV];
      KV::unpack(vc[i], vf);
      if (partial) {
        const bool ok = i * RPI + rg >= lo && i * RPI + rg < hi;
#pragma unroll
        for (int e = 0; e < EPV; ++e) vf[e] = ok ? vf[e] : 0.f;
      }
#pragma unroll
      for (int g = 0; g < GP; ++g)
#pragma unroll
        for (int e = 0; e < EPV; ++e) O[g][e] = fmaf(sc[i][g], vf[e], O[g][e]);
    }

#pragma unroll
    for (int i = 0; i < NI; ++i) { kc[i] = kn[i]; vc[i] = vn[i]; }
    pg = pgn;
  }

  // ---- sum the row groups, normalise, store
#pragma unroll
  for (int g = 0; g < GP; ++g) {
#pragma unroll
    for (int msk = VPR; msk < 64; msk <<= 1) {
      dsum[g] += shfl_xor_f(dsum[g], msk);
#pragma unroll
      for (int e = 0; e < EPV; ++e) O[g][e] += shfl_xor_f(O[g][e], msk);
    }
  }
  const float vscale = (KVT == kFP8) ? p.v_scale[h] : 1.0f;
  if (rg == 0) {
#pragma unroll
    for (int g = 0; g < GP; ++g) {
      if (g >= G) break;
      const int hq = h * G + g;
      const float inv = vscale / dsum[g];
      const float l = m[g] + log2f(dsum[g]);
      if (nch == 1) {
        const size_t ob = (size_t(b) * p.H_qo + hq) * D + d0;
#pragma unroll
        for (int e = 0; e < EPV; ++e) store_out<QT>(p.out, ob + e, O[g][e] * inv);
        if (cv == 0) p.lse[size_t(b) * p.H_qo + hq] = l;
      } else {
        const size_t row = (size_t(b) * p.H_qo + hq) * p.num_chunks + c;
        float* po = p.part_o + row * D + d0;
#pragma unroll
        for (int e = 0; e < EPV; ++e) store_agent(&po[e], O[g][e] * inv);
        if (cv == 0) store_agent(&p.part_lse[row], l);
      }
    }
  }
  if (nch > 1) split_finish<QT, D, GP, 64>(p, b, h, nch);
}

// ---------------------------------------------------------------------------------------------
// Host-side dispatch over the compiled shapes.
template <int KVT, int QT, int D, int PS>
static hipError_t launch_gp(const DecodeParams& p, int gp, unsigned grid, hipStream_t st) {
  switch (gp) {
    case 1: hipLaunchKernelGGL((decode_valu_kernel<KVT, QT, D, PS, 1>), dim3(grid), dim3(64), 0, st, p); break;
    case 2: hipLaunchKernelGGL((decode_valu_kernel<KVT, QT, D, PS, 2>), dim3(grid), dim3(64), 0, st, p); break;
    case 4: hipLaunchKernelGGL((decode_valu_kernel<KVT, QT, D, PS, 4>), dim3(grid), dim3(64), 0, st, p); break;
    case 8: hipLaunchKernelGGL((decode_valu_kernel<KVT, QT, D, PS, 8>), dim3(grid), dim3(64), 0, st, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int KVT, int QT>
static hipError_t launch_shape(const DecodeParams& p, int D, int PS, int gp, unsigned grid,
                               hipStream_t st) {
  if (D == 64 && PS == 16) return launch_gp<KVT, QT, 64, 16>(p, gp, grid, st);
  if (D == 64 && PS == 32) return launch_gp<KVT, QT, 64, 32>(p, gp, grid, st);
  if (D == 128 && PS == 16) return launch_gp<KVT, QT, 128, 16>(p, gp, grid, st);
  if (D == 128 && PS == 32) return launch_gp<KVT, QT, 128, 32>(p, gp, grid, st);
  return hipErrorInvalidValue;
}

hipError_t launch_decode_valu(const DecodeParams& p, int kv_dtype, int D, int PS, int gp,
                         unsigned grid, hipStream_t st) {
  if (kv_dtype == kF32) return launch_shape<kF32, kF32>(p, D, PS, gp, grid, st);
  if (kv_dtype == kBF16) return launch_shape<kBF16, kBF16>(p, D, PS, gp, grid, st);
  if (kv_dtype == kFP8) return launch_shape<kFP8, kBF16>(p, D, PS, gp, grid, st);
  return hipErrorInvalidValue;
}

}  // namespace pdk
