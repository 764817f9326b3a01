"""Seeded synthetic inputs for paged-KV decode attention.

This module only draws and lays out inputs; it holds none of the method's arithmetic (no scores,
softmax, merge or fp8 encoder of its own). Casts of the drawn fp32 values to bf16 and fp8-e4m3fn
use torch's own conversions (round to nearest even), so both the GPU library and the oracle see the
same stored bits.

Layouts (row-major), as in the TVM decode page (batch_decode_paged_kv buffers):
  q            [B, H_qo, D]
  pages        [max_num_pages, 2, H_kv, page_size, D]   (index 1: 0 = K, 1 = V)
  page_indptr  int32 [B + 1],  page_values int32 [nnz]
  length_info  int32 [B] (last_page_len) or [3, B] (last_page_len, window start, sink length)

Unused pool pages, and the unused slots past the end of each sequence's last page, are poisoned
with NaN (fp32 NaN, bf16 0x7FC0, fp8 0x7F) so a stray gather or an unmasked row shows.
Storage dtypes: fp32 -> np.float32, bf16 -> np.uint16 bits, fp8 -> np.uint8 codes.
"""
from __future__ import annotations

import concurrent.futures
import dataclasses
import math

import numpy as np
import torch

# "fp8": OCP e4m3fn codes; "fp8e4m3": IEEE-style e4m3 codes (max 240), drawn within +-240 where
# both formats give the same code to every value; "fp8e5m2": OCP e5m2 codes
DTYPE_CODE = {"f32": 0, "bf16": 1, "fp8": 2, "fp8e4m3": 3, "fp8e5m2": 4}
FP8_POOLS = ("fp8", "fp8e4m3", "fp8e5m2")
Q_PAYLOAD_SIGMA = 112.0  # fp8 q: spread of the codes, a quarter of e4m3fn's range
STORAGE = {"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8, "fp8e4m3": np.uint8,
           "fp8e5m2": np.uint8}
ELEM_BYTES = {"f32": 4, "bf16": 2, "fp8": 1, "fp8e4m3": 1, "fp8e5m2": 1}
POISON = {"f32": np.float32(np.nan).view(np.uint32), "bf16": 0x7FC0, "fp8": 0x7F,
          "fp8e4m3": 0x7F, "fp8e5m2": 0x7F}


def _rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream])))


def cast_f32(x: np.ndarray, dtype: str) -> np.ndarray:
    """fp32 values -> storage bits of `dtype` with torch's round-to-nearest-even conversions."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f32":
        return x
    t = torch.from_numpy(x)
    if dtype == "bf16":
        return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    if dtype == "fp8":
        return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    if dtype == "fp8e4m3":  # within +-240 the e4m3fn code is the e4m3 code
        return torch.clamp(t, -240.0, 240.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    if dtype == "fp8e5m2":
        return torch.clamp(t, -57344.0, 57344.0).to(torch.float8_e5m2).view(torch.uint8).numpy()
    raise ValueError(dtype)


def poisoned_pool(max_num_pages, H_kv, page_size, D, dtype):
    shape = (max_num_pages, 2, H_kv, page_size, D)
    if dtype == "f32":
        return np.full(shape, np.nan, np.float32)
    return np.full(shape, POISON[dtype], STORAGE[dtype])


@dataclasses.dataclass
class Workload:
    name: str
    B: int
    H_qo: int
    H_kv: int
    D: int
    page_size: int
    max_num_pages: int
    q_dtype: str
    kv_dtype: str
    seq_lens: np.ndarray          # int32 [B] total tokens per sequence
    attended: np.ndarray          # int32 [B] rows attended (window + sink applied)
    q: np.ndarray
    pages: np.ndarray
    page_indptr: np.ndarray
    page_values: np.ndarray
    length_info: np.ndarray
    sliding_window: bool
    rotary_mode: int
    rope_scale: float
    rope_theta: float
    q_rope_position: np.ndarray
    k_rope_pos_offset: np.ndarray
    sm_scale: float
    k_scale: np.ndarray | None
    v_scale: np.ndarray | None
    used_pages: np.ndarray        # int32 ids of pages holding data
    # fp8 pools with per-(page, KV head) scales [max_num_pages, H_kv] (replace k_scale / v_scale)
    k_scale_page: np.ndarray | None = None
    v_scale_page: np.ndarray | None = None
    # fp8 q: a scale per q head [H_qo] (q = code * scale)
    q_scale: np.ndarray | None = None

    @property
    def kv_bytes(self) -> int:
        """KV bytes of attended rows: sum_b attended_b * H_kv * 2 * D * elem_bytes."""
        return int(self.attended.astype(np.int64).sum()) * self.H_kv * 2 * self.D * ELEM_BYTES[self.kv_dtype]

    def oracle_kwargs(self):
        return dict(B=self.B, H_qo=self.H_qo, H_kv=self.H_kv, D=self.D, ps=self.page_size,
                    max_num_pages=self.max_num_pages, q_dtype=DTYPE_CODE[self.q_dtype],
                    kv_dtype=DTYPE_CODE[self.kv_dtype], q=self.q, pages=self.pages,
                    indptr=self.page_indptr, values=self.page_values,
                    length_info=self.length_info, sliding_window=self.sliding_window,
                    rotary_mode=self.rotary_mode, rope_scale=self.rope_scale,
                    rope_theta=self.rope_theta, q_rope_position=self.q_rope_position,
                    k_rope_pos_offset=self.k_rope_pos_offset, sm_scale=self.sm_scale,
                    k_scale=self.k_scale, v_scale=self.v_scale, k_scale_page=self.k_scale_page,
                    v_scale_page=self.v_scale_page, q_scale=self.q_scale)


def make_workload(*, name="custom", B, H_qo, H_kv, D, page_size, seq_lens, max_num_pages=None,
                  q_dtype="bf16", kv_dtype="bf16", seed=0, sm_scale=None, window=None, sink=0,
                  rotary_mode=0, rope_theta=1e4, rope_scale=1.0, q_rope_position=None,
                  k_rope_pos_offset=None, page_order="shuffled", kv_sigma=1.0,
                  fp8_payload_sigma=112.0, scale_range=(0.5 / 448, 2.0 / 448),
                  page_scales=False) -> Workload:
    """Draws a workload. seq_lens: total tokens per sequence (0 = empty sequence).
    window: None (length_info [B]) or W (length_info [3, B]: last_page_len, max(sink', L - W),
    sink') with sink' = min(sink, L).
    page_order: 'shuffled' (a seeded permutation of the pool, consecutive slices per sequence) or
    'identity' (pages 0, 1, 2, ... in order). fp8 KV: payload codes are fp8(clip(N(0,1) *
    fp8_payload_sigma, +-448)); per-KV-head scales ~ U[scale_range], and with page_scales a scale
    per (page, KV head) ~ U[scale_range] as well (for every page of the pool)."""
    seq_lens = np.asarray(seq_lens, np.int64)
    assert seq_lens.shape == (B,)
    ps = page_size
    npages = (seq_lens + ps - 1) // ps
    nnz = int(npages.sum())
    if max_num_pages is None:
        max_num_pages = max(nnz, 1)
    assert nnz <= max_num_pages, "pool too small"
    rng_tab = _rng(seed, 1)
    if page_order == "shuffled":
        ids = rng_tab.permutation(max_num_pages)[:nnz].astype(np.int32)
    else:
        ids = np.arange(nnz, dtype=np.int32)
    indptr = np.zeros(B + 1, np.int32)
    indptr[1:] = np.cumsum(npages)
    last = np.where(npages > 0, seq_lens - (npages - 1) * ps, 0).astype(np.int32)
    if window is None:
        length_info = last
        attended = seq_lens.astype(np.int32)
    else:
        sinks = np.where(npages > 0, np.minimum(sink, seq_lens), 0).astype(np.int32)
        win_off = np.where(npages > 0, np.maximum(sinks, seq_lens - window), 0).astype(np.int32)
        length_info = np.stack([last, win_off, sinks]).astype(np.int32)
        attended = np.where(npages > 0, seq_lens - win_off + sinks, 0).astype(np.int32)

    # Data for the used pages only; the rest of the pool is NaN-poisoned. Blocks of pages draw
    # from independent streams (seed, 1000 + block) so they can be filled in parallel threads.
    pool = poisoned_pool(max_num_pages, H_kv, ps, D, kv_dtype)
    order = np.sort(ids)
    k_scale = v_scale = None
    if kv_dtype in FP8_POOLS:
        rng_sc = _rng(seed, 4)
        k_scale = rng_sc.uniform(*scale_range, size=H_kv).astype(np.float32)
        v_scale = rng_sc.uniform(*scale_range, size=H_kv).astype(np.float32)
    k_scale_page = v_scale_page = None
    if page_scales:
        assert kv_dtype in FP8_POOLS, "per-page scales are for fp8 pools"
        rng_ps = _rng(seed, 5)
        k_scale_page = rng_ps.uniform(*scale_range, size=(max_num_pages, H_kv)).astype(np.float32)
        v_scale_page = rng_ps.uniform(*scale_range, size=(max_num_pages, H_kv)).astype(np.float32)
    CH = 512

    def fill(i):
        blk = order[i * CH:(i + 1) * CH]
        x = _rng(seed, 1000 + i).standard_normal((blk.size, 2, H_kv, ps, D), dtype=np.float32)
        if kv_dtype in FP8_POOLS:
            x *= np.float32(fp8_payload_sigma)
            np.clip(x, -448.0, 448.0, out=x)
        elif kv_sigma != 1.0:
            x *= np.float32(kv_sigma)
        pool[blk] = cast_f32(x, kv_dtype)

    nblk = (order.size + CH - 1) // CH
    if nblk > 1:
        with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, nblk)) as ex:
            list(ex.map(fill, range(nblk)))
    elif nblk == 1:
        fill(0)
    # Slots past the end of each sequence's last page are unused: poison them too.
    for b in range(B):
        if npages[b] > 0 and last[b] < ps:
            pool[ids[indptr[b + 1] - 1], :, :, last[b]:, :] = poisoned_pool(1, 1, 1, 1, kv_dtype)[0, 0, 0, 0, 0]
    rng_q = _rng(seed, 3)
    q_scale = None
    if q_dtype == "fp8":
        # codes of N(0, 1) * Q_PAYLOAD_SIGMA, and per-q-head scales ~ U[0.5, 2] / Q_PAYLOAD_SIGMA
        q = cast_f32(np.clip(rng_q.standard_normal((B, H_qo, D), dtype=np.float32) *
                             np.float32(Q_PAYLOAD_SIGMA), -448, 448), "fp8")
        q_scale = _rng(seed, 7).uniform(0.5, 2.0, size=H_qo).astype(np.float32) / np.float32(
            Q_PAYLOAD_SIGMA)
    else:
        q = cast_f32(rng_q.standard_normal((B, H_qo, D), dtype=np.float32), q_dtype)
    if sm_scale is None:
        sm_scale = float(np.float32(1.0 / math.sqrt(D)))
    if q_rope_position is None:
        q_rope_position = np.maximum(seq_lens - 1, 0).astype(np.int32)
    if k_rope_pos_offset is None:
        k_rope_pos_offset = np.zeros(B, np.int32)
    return Workload(name=name, B=B, H_qo=H_qo, H_kv=H_kv, D=D, page_size=ps,
                    max_num_pages=max_num_pages, q_dtype=q_dtype, kv_dtype=kv_dtype,
                    seq_lens=seq_lens.astype(np.int32), attended=attended, q=q, pages=pool,
                    page_indptr=indptr, page_values=ids, length_info=length_info,
                    sliding_window=window is not None, rotary_mode=rotary_mode,
                    rope_scale=float(rope_scale), rope_theta=float(rope_theta),
                    q_rope_position=np.asarray(q_rope_position, np.int32),
                    k_rope_pos_offset=np.asarray(k_rope_pos_offset, np.int32),
                    sm_scale=float(sm_scale), k_scale=k_scale, v_scale=v_scale, used_pages=order,
                    k_scale_page=k_scale_page, v_scale_page=v_scale_page, q_scale=q_scale)


# The five benchmark workloads. Their sizes follow the decode settings the pages describe
# (Llama-3-8B-shaped GQA heads, page size 16, long-context split, RoPE + sliding window + sink,
# fp8 KV with per-KV-head scales); every value is synthetic.
def tiny_fp32(seed=1001, lens=None):
    return make_workload(name="tiny_fp32", B=4, H_qo=4, H_kv=4, D=64, page_size=16,
                         seq_lens=[1, 17, 33, 50] if lens is None else lens, max_num_pages=16,
                         q_dtype="f32",
                         kv_dtype="f32", seed=seed, sm_scale=1.0 / 8.0)


def llama3_8b_bf16(seed=1002, B=32, lens=None):
    if lens is None:
        lens = _rng(seed, 0).integers(512, 4096, size=B, endpoint=True)
    return make_workload(name="llama3_8b_decode_bf16", B=B, H_qo=32, H_kv=8, D=128,
                         page_size=16, seq_lens=lens, max_num_pages=16384, seed=seed)


def long_ctx_bf16(seed=1003, lens=None):
    return make_workload(name="long_ctx_split_bf16", B=2, H_qo=32, H_kv=8, D=128, page_size=16,
                         seq_lens=[32768, 131072] if lens is None else lens,
                         max_num_pages=16384, seed=seed)


def rope_swa_bf16(seed=1004, B=64, lens=None):
    if lens is None:
        lens = _rng(seed, 0).integers(1024, 16384, size=B, endpoint=True)
    return make_workload(name="rope_swa_bf16", B=B, H_qo=32, H_kv=8, D=128, page_size=16,
                         seq_lens=lens, max_num_pages=65536, seed=seed, window=4096, sink=4,
                         rotary_mode=1, rope_theta=500000.0, rope_scale=1.0)


def fp8_gqa8(seed=1005, B=256, lens=None, sigma=0.5):
    if lens is None:
        z = _rng(seed, 0).standard_normal(B)
        lens = np.minimum(8192, np.maximum(1, np.rint(2048.0 * np.exp(sigma * z)))).astype(np.int64)
    return make_workload(name="fp8_kv_gqa8", B=B, H_qo=64, H_kv=8, D=128, page_size=32,
                         seq_lens=lens, max_num_pages=65536, q_dtype="bf16", kv_dtype="fp8",
                         seed=seed)


def gqa8_bf16(seed=1006, B=32, lens=None):
    """Llama-3-70B-shaped attention layer (64 q / 8 KV heads, GQA 8) at the Llama-3-8B lengths."""
    if lens is None:
        lens = _rng(seed, 0).integers(512, 4096, size=B, endpoint=True)
    return make_workload(name="gqa8_decode_bf16", B=B, H_qo=64, H_kv=8, D=128, page_size=16,
                         seq_lens=lens, max_num_pages=16384, seed=seed)


CONFIGS = {
    "tiny_fp32": tiny_fp32,
    "llama3_8b_bf16": llama3_8b_bf16,
    "long_ctx_bf16": long_ctx_bf16,
    "rope_swa_bf16": rope_swa_bf16,
    "fp8_gqa8": fp8_gqa8,
    "gqa8_bf16": gqa8_bf16,
}


def multi_query(w, T, seed):
    """q for T query tokens per sequence of workload w: [B, T, H_qo, D] in w.q_dtype storage,
    N(0, 1) from its own seeded stream (fp8 q: codes of N(0, 1) * Q_PAYLOAD_SIGMA, read with the
    workload's q_scale)."""
    rng = _rng(seed, 6)
    x = rng.standard_normal((w.B, T, w.H_qo, w.D), dtype=np.float32)
    if w.q_dtype == "fp8":
        x = np.clip(x * np.float32(Q_PAYLOAD_SIGMA), -448, 448)
    return cast_f32(x, w.q_dtype)


def append_inputs(*, T, H_kv, D, page_size, max_num_pages, in_dtype, seed, skip_every=0,
                  slots=None):
    """New K/V rows [T, H_kv, D] in `in_dtype` storage and int32 slot ids: distinct slots drawn
    from the pool (slot = page * page_size + offset); every `skip_every`-th slot is -1 (skip)."""
    rng = _rng(seed, 5)
    if slots is None:
        slots = rng.choice(max_num_pages * page_size, size=T, replace=False).astype(np.int32)
        if skip_every:
            slots[::skip_every] = -1
    k = cast_f32(rng.standard_normal((T, H_kv, D), dtype=np.float32), in_dtype)
    v = cast_f32(rng.standard_normal((T, H_kv, D), dtype=np.float32), in_dtype)
    return k, v, np.asarray(slots, np.int32)
