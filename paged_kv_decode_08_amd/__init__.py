"""Python binding of libpdecode (single-token paged-KV decode attention on MI355X / gfx950).

Argument marshalling only: every step of the computation runs in the library's HIP kernels. The
functions take torch tensors that live on the GPU and pass their device pointers, with the current
HIP stream, to the C ABI declared in include/pdecode.h. There is no CPU fallback: if the shared
library is missing the import of any entry point raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpdecode.so")

F32, BF16, FP8_E4M3FN, FP8_E4M3, FP8_E5M2 = 0, 1, 2, 3, 4
STATUS = {0: "PDECODE_OK", 1: "PDECODE_ERR_INVALID_ARG", 2: "PDECODE_ERR_UNSUPPORTED",
          3: "PDECODE_ERR_WORKSPACE_TOO_SMALL", 4: "PDECODE_ERR_HIP"}
_DTYPE_CODE = {"f32": F32, "bf16": BF16, "fp8": FP8_E4M3FN, "fp8e4m3": FP8_E4M3,
               "fp8e5m2": FP8_E5M2}
_ELEM_BYTES = {F32: 4, BF16: 2, FP8_E4M3FN: 1, FP8_E4M3: 1, FP8_E5M2: 1}

_c_i32 = ctypes.c_int32
_c_ptr = ctypes.c_void_p


class Desc(ctypes.Structure):
    _fields_ = [("batch", _c_i32), ("num_qo_heads", _c_i32), ("num_kv_heads", _c_i32),
                ("head_dim", _c_i32), ("page_size", _c_i32), ("max_num_pages", _c_i32),
                ("q_dtype", _c_i32), ("kv_dtype", _c_i32), ("sliding_window", _c_i32),
                ("max_kv_len", _c_i32), ("num_kv_splits", _c_i32), ("k_scale", _c_ptr),
                ("v_scale", _c_ptr), ("sink_logits", _c_ptr), ("k_scale_page", _c_ptr),
                ("v_scale_page", _c_ptr), ("q_scale", _c_ptr)]


class Rope(ctypes.Structure):
    _fields_ = [("rotary_mode", _c_i32), ("rope_scale", ctypes.c_float),
                ("rope_theta", ctypes.c_float), ("q_rope_position", _c_ptr),
                ("k_rope_pos_offset", _c_ptr)]


class PdecodeError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {STATUS.get(status, status)}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libpdecode.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        P = _c_ptr
        L.pdecode_workspace_bytes.restype = ctypes.c_size_t
        L.pdecode_workspace_bytes.argtypes = [ctypes.POINTER(Desc)]
        L.pdecode_plan.restype = _c_i32
        L.pdecode_plan.argtypes = [ctypes.POINTER(Desc), ctypes.POINTER(_c_i32),
                                   ctypes.POINTER(_c_i32)]
        sz = ctypes.POINTER(ctypes.c_size_t)
        L.pdecode_workspace_layout.restype = _c_i32
        L.pdecode_workspace_layout.argtypes = [ctypes.POINTER(Desc), _c_i32, sz, sz, sz,
                                               ctypes.POINTER(_c_i32)]
        L.pdecode_attention.restype = _c_i32
        L.pdecode_attention.argtypes = [ctypes.POINTER(Desc), P, P, P, P, P,
                                        ctypes.POINTER(Rope), ctypes.c_float, P, P, P,
                                        ctypes.c_size_t, P]
        L.pdecode_workspace_bytes_multi.restype = ctypes.c_size_t
        L.pdecode_workspace_bytes_multi.argtypes = [ctypes.POINTER(Desc), _c_i32]
        L.pdecode_attention_multi.restype = _c_i32
        L.pdecode_attention_multi.argtypes = [ctypes.POINTER(Desc), _c_i32, P, P, P, P, P,
                                              ctypes.POINTER(Rope), ctypes.c_float, P, P, P,
                                              ctypes.c_size_t, P]
        L.pdecode_append_attention.restype = _c_i32
        L.pdecode_append_attention.argtypes = [ctypes.POINTER(Desc), P, P, P, P, P, P, P,
                                               ctypes.POINTER(Rope), ctypes.c_float, P, P, P,
                                               ctypes.c_size_t, P]
        L.pdecode_merge_state_inplace.restype = _c_i32
        L.pdecode_merge_state_inplace.argtypes = [_c_i32, _c_i32, _c_i32, _c_i32, P, P, P, P, P]
        L.pdecode_append_kv.restype = _c_i32
        L.pdecode_append_kv.argtypes = [ctypes.POINTER(Desc), P, P, P, _c_i32, P, P]
        L.pdecode_attention_noalloc.restype = _c_i32
        L.pdecode_attention_noalloc.argtypes = [ctypes.POINTER(Desc), P, P, P, P, P,
                                                ctypes.POINTER(Rope), ctypes.c_float, P, P, P]
        L.pdecode_bench_stream_read.restype = _c_i32
        L.pdecode_bench_stream_read.argtypes = [P, ctypes.c_size_t, _c_i32, _c_i32, _c_i32, P, P]
        L.pdecode_status_string.restype = ctypes.c_char_p
        L.pdecode_status_string.argtypes = [_c_i32]
        _lib = L
    return _lib


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def dtype_code(dt) -> int:
    return _DTYPE_CODE[dt] if isinstance(dt, str) else int(dt)


def make_desc(*, batch, num_qo_heads, num_kv_heads, head_dim, page_size, max_num_pages,
              q_dtype, kv_dtype, sliding_window=False, max_kv_len=0, num_kv_splits=0,
              k_scale=None, v_scale=None, sink_logits=None, k_scale_page=None,
              v_scale_page=None, q_scale=None) -> Desc:
    d = Desc(batch, num_qo_heads, num_kv_heads, head_dim, page_size, max_num_pages,
             dtype_code(q_dtype), dtype_code(kv_dtype), int(bool(sliding_window)),
             int(max_kv_len), int(num_kv_splits), None, None, None, None, None, None)
    d.k_scale = _ptr(k_scale)
    d.v_scale = _ptr(v_scale)
    d.sink_logits = _ptr(sink_logits)
    d.k_scale_page = _ptr(k_scale_page)
    d.v_scale_page = _ptr(v_scale_page)
    d.q_scale = _ptr(q_scale)
    # keep the tensors alive with the struct
    d._keep = (k_scale, v_scale, sink_logits, k_scale_page, v_scale_page, q_scale)
    return d


def make_rope(*, rotary_mode=1, rope_scale=1.0, rope_theta=1e4, q_rope_position,
              k_rope_pos_offset) -> Rope:
    r = Rope(int(rotary_mode), float(rope_scale), float(rope_theta), _ptr(q_rope_position),
             _ptr(k_rope_pos_offset))
    r._keep = (q_rope_position, k_rope_pos_offset)
    return r


def status_string(status: int) -> str:
    return lib().pdecode_status_string(status).decode()


def workspace_bytes(desc: Desc) -> int:
    return int(lib().pdecode_workspace_bytes(ctypes.byref(desc)))


def workspace_bytes_multi(desc: Desc, qo_len: int) -> int:
    return int(lib().pdecode_workspace_bytes_multi(ctypes.byref(desc), int(qo_len)))


def plan(desc: Desc):
    """(chunk_pages, num_chunks) the library plans for this description; (0, 0) when the
    chunk size is chosen on the device at each call (the persistent schedule's automatic plan)."""
    cp, nc = _c_i32(0), _c_i32(0)
    st = lib().pdecode_plan(ctypes.byref(desc), ctypes.byref(cp), ctypes.byref(nc))
    if st:
        raise PdecodeError(st, "pdecode_plan")
    return cp.value, nc.value


def workspace_layout(desc: Desc, qo_len: int = 1) -> dict:
    """pdecode_workspace_layout: byte offsets of the split partial states (part_o, part_lse)
    and of the automatic plan's chunk-size word in a workspace, and the chunk cap."""
    o, l, w = ctypes.c_size_t(0), ctypes.c_size_t(0), ctypes.c_size_t(0)
    nc = _c_i32(0)
    st = lib().pdecode_workspace_layout(ctypes.byref(desc), int(qo_len), ctypes.byref(o),
                                        ctypes.byref(l), ctypes.byref(w), ctypes.byref(nc))
    if st:
        raise PdecodeError(st, "pdecode_workspace_layout")
    return {"part_o": o.value, "part_lse": l.value, "plan_word": w.value, "num_chunks": nc.value}


def alloc_workspace(desc: Desc, device="cuda") -> torch.Tensor | None:
    """A zero-filled workspace of pdecode_workspace_bytes(desc) bytes (the library keeps its
    split counters zero between calls), or None when none is needed."""
    n = workspace_bytes(desc)
    return torch.zeros(n, dtype=torch.uint8, device=device) if n else None


def attention(desc: Desc, q, pages, page_indptr, page_values, length_info, out, lse, sm_scale,
              rope: Rope | None = None, workspace=None, stream=None) -> None:
    """pdecode_attention: writes out [B, H_qo, D] and lse [B, H_qo] (fp32, base 2)."""
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().pdecode_attention(ctypes.byref(desc), _ptr(q), _ptr(pages), _ptr(page_indptr),
                                 _ptr(page_values), _ptr(length_info),
                                 None if rope is None else ctypes.byref(rope),
                                 float(sm_scale), _ptr(out), _ptr(lse), _ptr(workspace),
                                 ws_bytes, _stream(stream))
    if st:
        raise PdecodeError(st, "pdecode_attention")


def attention_noalloc(desc: Desc, q, pages, page_indptr, page_values, length_info, out, lse,
                      sm_scale, rope: Rope | None = None, stream=None) -> None:
    """pdecode_attention_noalloc: pdecode_attention with the library's own per-GPU scratch (no
    workspace, nothing allocated); calls that may overlap on one GPU race."""
    st = lib().pdecode_attention_noalloc(ctypes.byref(desc), _ptr(q), _ptr(pages),
                                         _ptr(page_indptr), _ptr(page_values), _ptr(length_info),
                                         None if rope is None else ctypes.byref(rope),
                                         float(sm_scale), _ptr(out), _ptr(lse), _stream(stream))
    if st:
        raise PdecodeError(st, "pdecode_attention_noalloc")


def alloc_workspace_multi(desc: Desc, qo_len: int, device="cuda") -> torch.Tensor | None:
    """A zero-filled workspace of pdecode_workspace_bytes_multi(desc, qo_len) bytes, or None."""
    n = workspace_bytes_multi(desc, qo_len)
    return torch.zeros(n, dtype=torch.uint8, device=device) if n else None


def attention_multi(desc: Desc, qo_len: int, q, pages, page_indptr, page_values, length_info,
                    out, lse, sm_scale, rope: Rope | None = None, workspace=None,
                    stream=None) -> None:
    """pdecode_attention_multi: q/out [B, qo_len, H_qo, D], lse [B, qo_len, H_qo]; token t of a
    sequence attends its positions up to total - qo_len + t (with RoPE, its query sits at
    q_rope_position[b] + t)."""
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().pdecode_attention_multi(ctypes.byref(desc), int(qo_len), _ptr(q), _ptr(pages),
                                       _ptr(page_indptr), _ptr(page_values), _ptr(length_info),
                                       None if rope is None else ctypes.byref(rope),
                                       float(sm_scale), _ptr(out), _ptr(lse), _ptr(workspace),
                                       ws_bytes, _stream(stream))
    if st:
        raise PdecodeError(st, "pdecode_attention_multi")


def append_attention(desc: Desc, new_k, new_v, q, pages, page_indptr, page_values, length_info,
                     out, lse, sm_scale, rope: Rope | None = None, workspace=None,
                     stream=None) -> None:
    """pdecode_append_attention: writes new_k/new_v [B, H_kv, D] (bf16) to each sequence's row of
    position total - 1 in `pages`, then writes out [B, H_qo, D] and lse [B, H_qo] as attention()."""
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().pdecode_append_attention(ctypes.byref(desc), _ptr(new_k), _ptr(new_v), _ptr(q),
                                        _ptr(pages), _ptr(page_indptr), _ptr(page_values),
                                        _ptr(length_info),
                                        None if rope is None else ctypes.byref(rope),
                                        float(sm_scale), _ptr(out), _ptr(lse), _ptr(workspace),
                                        ws_bytes, _stream(stream))
    if st:
        raise PdecodeError(st, "pdecode_append_attention")


def merge_state_inplace(v, s, v_other, s_other, stream=None) -> None:
    """pdecode_merge_state_inplace on v [n, H, D] (fp32 or bf16) and s [n, H] (fp32)."""
    if v.dtype == torch.float32:
        vd = F32
    elif v.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        vd = BF16
    else:
        raise ValueError("v must be fp32 or bf16")
    n, H, D = v.shape
    if tuple(v_other.shape) != (n, H, D) or tuple(s.shape) != (n, H) or tuple(s_other.shape) != (n, H):
        raise ValueError("shape mismatch")
    st = lib().pdecode_merge_state_inplace(n, H, D, vd, _ptr(v), _ptr(s), _ptr(v_other),
                                           _ptr(s_other), _stream(stream))
    if st:
        raise PdecodeError(st, "pdecode_merge_state_inplace")


def append_kv(desc: Desc, new_k, new_v, slot_ids, pages, stream=None) -> None:
    """pdecode_append_kv: new_k/new_v [T, H_kv, D] in desc.q_dtype, slot_ids int32 [T]."""
    st = lib().pdecode_append_kv(ctypes.byref(desc), _ptr(new_k), _ptr(new_v), _ptr(slot_ids),
                                 int(slot_ids.numel()), _ptr(pages), _stream(stream))
    if st:
        raise PdecodeError(st, "pdecode_append_kv")


def bench_stream_read(buf, loads_per_lane, nontemporal, workgroups, sink, stream=None) -> None:
    """pdecode_bench_stream_read (include/pdecode_bench.h): one streaming read of the whole of
    `buf` (a contiguous GPU tensor whose byte size is a multiple of 16); sink: uint32 or int32
    [workgroups * 256] on the GPU."""
    nbytes = buf.numel() * buf.element_size()
    if sink.numel() * sink.element_size() < 4 * 256 * int(workgroups):
        raise ValueError("sink must hold workgroups * 256 uint32 values")
    st = lib().pdecode_bench_stream_read(_ptr(buf), nbytes, int(loads_per_lane),
                                         int(bool(nontemporal)), int(workgroups), _ptr(sink),
                                         _stream(stream))
    if st:
        raise PdecodeError(st, "pdecode_bench_stream_read")
