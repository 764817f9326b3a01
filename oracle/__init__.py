"""Oracle for single-token paged-KV decode attention: TEST INFRASTRUCTURE ONLY.

A plain scalar C++ implementation in fp64 (``oracle.cpp``), loaded through ctypes. Only the
tests, the smoke check and the benchmark's CPU-baseline leg may import this package; the GPU
library never does, and the two share no code.

Every function takes and returns host NumPy arrays. Floating-point results are fp64.
dtype codes: 0 = fp32, 1 = bf16 (raw uint16 bits), 2 = fp8 e4m3fn, 3 = IEEE-style e4m3 (max 240),
4 = fp8 e5m2 (the fp8 codes as raw uint8 bits).

What each function follows is cited in ``oracle.cpp``. Parity against the pages is pinned by the
``-m "not gpu"`` tests. The RoPE convention, whose helper body the pages do not show, is pinned
to transformers' Llama rotate_half and GPT-J rotate_every_two instead: parity unpinned against
the pages themselves.
"""
import ctypes
import os

import numpy as np

from .build import LIB, build

F32, BF16, FP8 = 0, 1, 2
FP8_E4M3, FP8_E5M2 = 3, 4

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        L = ctypes.CDLL(LIB)
        P = ctypes.c_void_p
        i32 = ctypes.c_int32
        f32 = ctypes.c_float
        L.oracle_decode.restype = i32
        L.oracle_decode.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32, P, P, P, P, i32, P,
                                    i32, i32, f32, f32, P, P, f32, P, P, P, P, P, i32, P, P, P,
                                    i32]
        L.oracle_merge_state.restype = None
        L.oracle_merge_state.argtypes = [i32, i32, i32, P, P, P, P]
        L.oracle_append_kv.restype = i32
        L.oracle_append_kv.argtypes = [i32, i32, i32, i32, i32, i32, i32, P, P, P, P, P, P, P,
                                       P]
        L.oracle_validate_page_table.restype = i32
        L.oracle_validate_page_table.argtypes = [i32, i32, i32, i32, P, P, P, i32]
        L.oracle_fp8_e4m3fn_value.restype = ctypes.c_double
        L.oracle_fp8_e4m3fn_value.argtypes = [ctypes.c_uint8]
        L.oracle_fp8_e4m3fn_encode.restype = ctypes.c_uint8
        L.oracle_fp8_e4m3fn_encode.argtypes = [f32]
        L.oracle_fp8_e4m3_value.restype = ctypes.c_double
        L.oracle_fp8_e4m3_value.argtypes = [ctypes.c_uint8]
        L.oracle_fp8_e4m3_encode.restype = ctypes.c_uint8
        L.oracle_fp8_e4m3_encode.argtypes = [f32]
        L.oracle_fp8_e5m2_value.restype = ctypes.c_double
        L.oracle_fp8_e5m2_value.argtypes = [ctypes.c_uint8]
        L.oracle_fp8_e5m2_encode.restype = ctypes.c_uint8
        L.oracle_fp8_e5m2_encode.argtypes = [f32]
        L.oracle_bf16_value.restype = ctypes.c_double
        L.oracle_bf16_value.argtypes = [ctypes.c_uint16]
        L.oracle_rope_rotate.restype = None
        L.oracle_rope_rotate.argtypes = [P, i32, ctypes.c_double, f32, f32, i32]
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


LOG2E = 1.0 / np.log(2.0)


class OracleError(RuntimeError):
    pass


def decode(*, B, H_qo, H_kv, D, ps, max_num_pages, q_dtype, kv_dtype, q, pages, indptr, values,
           length_info, sliding_window=False, rotary_mode=0, rope_scale=1.0, rope_theta=1e4,
           q_rope_position=None, k_rope_pos_offset=None, sm_scale, k_scale=None, v_scale=None,
           k_scale_page=None, v_scale_page=None, q_scale=None, select=None, nthreads=0):
    """Decode attention. q/pages are raw arrays in their storage dtype (fp32, uint16 bf16 bits,
    uint8 fp8 codes). fp8 pools: per-KV-head scales k_scale/v_scale [H_kv], or per (page, KV
    head) scales k_scale_page/v_scale_page [max_num_pages, H_kv], which replace them. fp8 q: a
    scale per q head q_scale [H_qo] (q = code * scale).
    Returns (out[n, D] fp64, lse[n] fp64) for the selected (b, h_qo) pairs
    (select = int array [n, 2]) or for all pairs in (b, h_qo) order reshaped to [B, H_qo, ...]."""
    indptr = _c(indptr, np.int32)
    values = _c(values, np.int32)
    length_info = _c(length_info, np.int32)
    if values.size == 0:
        values = np.zeros(1, np.int32)
    qrp = _c(q_rope_position, np.int32) if q_rope_position is not None else np.zeros(max(B, 1), np.int32)
    kro = _c(k_rope_pos_offset, np.int32) if k_rope_pos_offset is not None else np.zeros(max(B, 1), np.int32)
    ks = _c(k_scale, np.float32)
    vs = _c(v_scale, np.float32)
    ksp = _c(k_scale_page, np.float32)
    vsp = _c(v_scale_page, np.float32)
    qs = _c(q_scale, np.float32)
    sel = None if select is None else _c(select, np.int32).reshape(-1, 2)
    n = sel.shape[0] if sel is not None else B * H_qo
    out = np.zeros((max(n, 1), D), np.float64)
    lse = np.zeros(max(n, 1), np.float64)
    q = np.ascontiguousarray(q)
    pages = np.ascontiguousarray(pages)
    nnz = int(indptr[-1]) if indptr.size else 0
    rc = lib().oracle_decode(B, H_qo, H_kv, D, ps, max_num_pages, q_dtype, kv_dtype, _ptr(q),
                             _ptr(pages), _ptr(indptr), _ptr(values), max(nnz, values.size),
                             _ptr(length_info), int(bool(sliding_window)), int(rotary_mode),
                             float(rope_scale), float(rope_theta), _ptr(qrp), _ptr(kro),
                             float(sm_scale), _ptr(ks), _ptr(vs), _ptr(ksp), _ptr(vsp),
                             _ptr(qs), 0 if sel is None else n,
                             _ptr(sel), _ptr(out), _ptr(lse), int(nthreads))
    if rc != 0:
        raise OracleError(f"oracle_decode failed with code {rc}")
    out, lse = out[:n], lse[:n]
    if sel is None:
        return out.reshape(B, H_qo, D), lse.reshape(B, H_qo)
    return out, lse


def merge_state(v, s, v_other, s_other):
    """Pairwise base-2 merge; returns new (v, s) arrays (fp64). v: [N, H, D], s: [N, H]."""
    v = np.array(v, dtype=np.float64, order="C")
    s = np.array(s, dtype=np.float64, order="C")
    vo = _c(v_other, np.float64)
    so = _c(s_other, np.float64)
    N, H, D = v.shape
    lib().oracle_merge_state(N, H, D, _ptr(v), _ptr(s), _ptr(vo), _ptr(so))
    return v, s


def append_kv(*, pages, new_k, new_v, slots, H_kv, D, ps, in_dtype, kv_dtype, k_scale=None,
              v_scale=None, k_scale_page=None, v_scale_page=None):
    """KV append on a host copy of the pool (modified in place and returned)."""
    assert pages.flags["C_CONTIGUOUS"]
    new_k = np.ascontiguousarray(new_k)
    new_v = np.ascontiguousarray(new_v)
    slots = _c(slots, np.int32)
    ks = _c(k_scale, np.float32)
    vs = _c(v_scale, np.float32)
    ksp = _c(k_scale_page, np.float32)
    vsp = _c(v_scale_page, np.float32)
    max_num_pages = pages.shape[0]
    rc = lib().oracle_append_kv(slots.size, H_kv, D, ps, max_num_pages, in_dtype, kv_dtype,
                                _ptr(new_k), _ptr(new_v), _ptr(slots), _ptr(ks), _ptr(vs),
                                _ptr(ksp), _ptr(vsp), _ptr(pages))
    if rc != 0:
        raise OracleError(f"oracle_append_kv failed with code {rc}")
    return pages


def apply_sink(out, lse, sink_logits):
    """Folds a learned attention sink per q head (a logit in the units of the scaled score, with
    no value row) into finished decode states (out [..., H_qo, D], lse [..., H_qo], base 2): the
    softmax denominator gains e^sink, so lse' = log2(2^lse + 2^(sink log2 e)) and
    out' = out 2^(lse - lse'). Rows with the empty convention (lse = -5e4, out = 0) are kept."""
    out = np.array(out, np.float64)
    lse = np.array(lse, np.float64)
    s2 = np.asarray(sink_logits, np.float64) * LOG2E
    s2 = np.broadcast_to(s2, lse.shape)
    empty = lse == -5e4
    m = np.maximum(lse, s2)
    new = m + np.log2(np.exp2(lse - m) + np.exp2(s2 - m))
    f = np.exp2(lse - new)
    out = np.where(empty[..., None], out, out * f[..., None])
    return out, np.where(empty, lse, new)


def decode_multi(*, qo_len, q, select=None, **kw):
    """Decode with qo_len query tokens per sequence (q [B, qo_len, H_qo, D]), causal over the new
    tokens: the last qo_len positions of each sequence are the new tokens, and token t attends
    positions 0 .. total - qo_len + t, i.e. it is the TVM page's single-token decode over that
    prefix of the sequence (its first ceil(len / ps) pages, the last one holding len - (np - 1) ps
    rows). An empty prefix gives the empty convention. With a sliding window (length_info [3, B])
    the call's window applies to all its tokens (reading: one window start and sink per
    sequence, as length_info gives them): token t's prefix of n rows keeps the sink rows below n
    and the window rows from the window start up to n, i.e. the decode over that prefix with
    window start min(win_off, n) and sink min(sink, n); the keys' RoPE positions are the
    sequence's compacted row indices, as for one token. With RoPE (rotary_mode 1, rotate-half, or
    2, interleaved), token t's query is at position q_rope_position[b] + t (the new tokens are
    consecutive) and the keys keep the sequence's k_rope_pos_offset[b]. Returns (out
    [B, T, H_qo, D], lse [B, T, H_qo]), or, for select = int array [n, 3] of (b, t, h_qo),
    (out [n, D], lse [n])."""
    B, T, ps = kw["B"], int(qo_len), kw["ps"]
    sliding = bool(kw.get("sliding_window"))
    indptr = np.asarray(kw["indptr"], np.int64)
    values = np.asarray(kw["values"], np.int64)
    li = np.asarray(kw["length_info"], np.int64).reshape(-1)
    last = li[:B]
    win = li[B:2 * B] if sliding else np.zeros(B, np.int64)
    snk = li[2 * B:3 * B] if sliding else np.zeros(B, np.int64)
    ip2, val2, last2, win2, snk2 = [0], [], [], [], []
    for b in range(B):
        npg = int(indptr[b + 1] - indptr[b])
        total = (npg - 1) * ps + int(last[b]) if npg else 0
        for t in range(T):
            n = total - T + t + 1  # rows token t sees
            if n <= 0:
                ip2.append(ip2[-1])
                last2.append(0)
                win2.append(0)
                snk2.append(0)
                continue
            k = (n + ps - 1) // ps
            val2.extend(values[indptr[b]:indptr[b] + k].tolist())
            ip2.append(ip2[-1] + k)
            last2.append(n - (k - 1) * ps)
            win2.append(min(int(win[b]), n))
            snk2.append(min(int(snk[b]), n))
    kw = dict(kw)
    li2 = np.array(last2 + win2 + snk2 if sliding else last2, np.int32)
    kw.update(B=B * T, indptr=np.array(ip2, np.int32), values=np.array(val2, np.int32),
              length_info=li2, q=np.ascontiguousarray(q).reshape(B * T, kw["H_qo"], kw["D"]))
    if kw.get("rotary_mode", 0) in (1, 2):
        qrp = np.asarray(kw["q_rope_position"], np.int64).reshape(-1)[:B]
        kro = np.asarray(kw["k_rope_pos_offset"], np.int64).reshape(-1)[:B]
        kw["q_rope_position"] = (qrp[:, None] + np.arange(T)[None, :]).reshape(-1).astype(np.int32)
        kw["k_rope_pos_offset"] = np.repeat(kro, T).astype(np.int32)
    else:
        for key in ("q_rope_position", "k_rope_pos_offset", "rotary_mode"):
            kw.pop(key, None)
    if select is not None:
        sel = np.asarray(select, np.int64).reshape(-1, 3)
        return decode(select=np.stack([sel[:, 0] * T + sel[:, 1], sel[:, 2]], 1), **kw)
    out, lse = decode(**kw)
    return out.reshape(B, T, kw["H_qo"], kw["D"]), lse.reshape(B, T, kw["H_qo"])


def last_position_slots(*, B, ps, indptr, values, length_info):
    """Pool slot (page * ps + row) of each sequence's position total - 1, the row a decode step's
    new token occupies: its last page page_values[indptr[b+1] - 1], row last_page_len[b] - 1 (the
    TVM relax decode-kernels page's length of a paged sequence). -1 for a sequence without pages,
    which has no such row. length_info: [B] or [3, B] (row 0 is last_page_len)."""
    indptr = np.asarray(indptr, np.int64)
    values = np.asarray(values, np.int64)
    last = np.asarray(length_info, np.int64).reshape(-1, B)[0] if B else np.zeros(0, np.int64)
    slots = np.full(B, -1, np.int64)
    for b in range(B):
        if indptr[b + 1] > indptr[b]:
            slots[b] = values[indptr[b + 1] - 1] * ps + last[b] - 1
    return slots.astype(np.int32)


def append_then_decode(*, new_k, new_v, **kw):
    """The fused decode step: append_kv of token b's new K/V rows (new_k/new_v [B, H_kv, D]) to
    sequence b's last position (last_position_slots; skipped without pages), on a copy of the
    pool, then decode over the updated pool. Returns (out, lse, updated pool)."""
    pages = np.array(kw.pop("pages"), copy=True, order="C")
    slots = last_position_slots(B=kw["B"], ps=kw["ps"], indptr=kw["indptr"], values=kw["values"],
                                length_info=kw["length_info"])
    append_kv(pages=pages, new_k=new_k, new_v=new_v, slots=slots, H_kv=kw["H_kv"], D=kw["D"],
              ps=kw["ps"], in_dtype=kw["q_dtype"], kv_dtype=kw["kv_dtype"],
              k_scale=kw.get("k_scale"), v_scale=kw.get("v_scale"))
    out, lse = decode(pages=pages, **kw)
    return out, lse, pages


def validate_page_table(*, B, ps, max_num_pages, indptr, values, length_info, sliding_window=False):
    indptr = _c(indptr, np.int32)
    values = _c(values, np.int32)
    if values.size == 0:
        values = np.zeros(1, np.int32)
    length_info = _c(length_info, np.int32)
    return int(lib().oracle_validate_page_table(B, ps, max_num_pages, int(values.size),
                                                _ptr(indptr), _ptr(values), _ptr(length_info),
                                                int(bool(sliding_window))))


def fp8_value(code: int) -> float:
    return float(lib().oracle_fp8_e4m3fn_value(code))


def fp8_encode(x: float) -> int:
    return int(lib().oracle_fp8_e4m3fn_encode(x))


def fp8_encode_array(x):
    x = np.asarray(x, np.float32).ravel()
    f = lib().oracle_fp8_e4m3fn_encode
    return np.array([f(float(v)) for v in x], np.uint8)


def fp8_e4m3_value(code: int) -> float:
    """IEEE-style e4m3 (the NON_OCP float8_e4m3, max 240): value of a code."""
    return float(lib().oracle_fp8_e4m3_value(code))


def fp8_e4m3_encode(x: float) -> int:
    return int(lib().oracle_fp8_e4m3_encode(x))


def fp8_e5m2_value(code: int) -> float:
    """OCP e5m2 (bias 15, max 57344): value of a code."""
    return float(lib().oracle_fp8_e5m2_value(code))


def fp8_e5m2_encode(x: float) -> int:
    return int(lib().oracle_fp8_e5m2_encode(x))


def bf16_value(bits: int) -> float:
    return float(lib().oracle_bf16_value(bits))


def rope_rotate(x, pos, rope_scale, rope_theta, interleaved=False):
    x = np.array(x, dtype=np.float64, order="C")
    lib().oracle_rope_rotate(_ptr(x), x.size, float(pos), float(rope_scale), float(rope_theta),
                             int(bool(interleaved)))
    return x
