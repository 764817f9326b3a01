"""GPU-side helpers for the parity tests: upload a synthetic workload and run the library."""
import numpy as np
import torch

import paged_kv_decode_08_amd as pk

TORCH_STORAGE = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8,
                 "fp8e4m3": torch.uint8, "fp8e5m2": torch.uint8}


def to_device_storage(x: np.ndarray, dtype: str, device="cuda"):
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype == "bf16":
        t = t.view(torch.int16).view(torch.bfloat16)
    return t.to(device)


def upload(w, device="cuda"):
    d = dict(
        q=to_device_storage(w.q, w.q_dtype, device),
        pages=to_device_storage(w.pages, w.kv_dtype, device),
        indptr=torch.from_numpy(w.page_indptr).to(device),
        values=torch.from_numpy(w.page_values if w.page_values.size else np.zeros(1, np.int32)).to(device),
        length_info=torch.from_numpy(np.ascontiguousarray(w.length_info)).to(device),
        q_pos=torch.from_numpy(w.q_rope_position).to(device),
        k_off=torch.from_numpy(w.k_rope_pos_offset).to(device),
        k_scale=None if w.k_scale is None else torch.from_numpy(w.k_scale).to(device),
        v_scale=None if w.v_scale is None else torch.from_numpy(w.v_scale).to(device),
        k_scale_page=(None if getattr(w, "k_scale_page", None) is None
                      else torch.from_numpy(w.k_scale_page).to(device)),
        v_scale_page=(None if getattr(w, "v_scale_page", None) is None
                      else torch.from_numpy(w.v_scale_page).to(device)),
        q_scale=(None if getattr(w, "q_scale", None) is None
                 else torch.from_numpy(w.q_scale).to(device)),
    )
    return d


def desc_for(w, dev, num_kv_splits=0, max_kv_len=None, sink_logits=None):
    if max_kv_len is None:
        max_kv_len = int(w.attended.max()) if w.B else 0
    return pk.make_desc(batch=w.B, num_qo_heads=w.H_qo, num_kv_heads=w.H_kv, head_dim=w.D,
                        page_size=w.page_size, max_num_pages=w.max_num_pages,
                        q_dtype=w.q_dtype, kv_dtype=w.kv_dtype,
                        sliding_window=w.sliding_window, max_kv_len=max_kv_len,
                        num_kv_splits=num_kv_splits, k_scale=dev["k_scale"],
                        v_scale=dev["v_scale"], sink_logits=sink_logits,
                        k_scale_page=dev.get("k_scale_page"), v_scale_page=dev.get("v_scale_page"),
                        q_scale=dev.get("q_scale"))


def run_attention(w, dev, num_kv_splits=0, max_kv_len=None, out=None, lse=None, stream=None):
    desc = desc_for(w, dev, num_kv_splits, max_kv_len)
    if out is None:
        odt = "bf16" if w.q_dtype == "fp8" else w.q_dtype  # fp8 q writes a bf16 out
        out = torch.empty((w.B, w.H_qo, w.D), dtype=TORCH_STORAGE[odt], device="cuda")
        if odt == "bf16":
            out.view(torch.int16).fill_(0x7FC0)   # NaN: any element not written shows
        else:
            out.fill_(float("nan"))
    if lse is None:
        lse = torch.full((w.B, w.H_qo), float("nan"), dtype=torch.float32, device="cuda")
    rope = None
    if w.rotary_mode:
        rope = pk.make_rope(rotary_mode=w.rotary_mode, rope_scale=w.rope_scale,
                            rope_theta=w.rope_theta, q_rope_position=dev["q_pos"],
                            k_rope_pos_offset=dev["k_off"])
    ws = pk.alloc_workspace(desc)
    pk.attention(desc, dev["q"], dev["pages"], dev["indptr"], dev["values"], dev["length_info"],
                 out, lse, w.sm_scale, rope=rope, workspace=ws, stream=stream)
    return out, lse


def to_np64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


TOL = {"f32": (1e-5, 1e-5), "bf16": (2e-2, 1e-3), "fp8": (2e-2, 1e-3), "fp8e4m3": (2e-2, 1e-3),
       "fp8e5m2": (2e-2, 1e-3)}


def tolerance(w):
    """(|d out| bound, |d lse| bound) stated for this path: fp32 1e-5 / 1e-5; bf16 and fp8 KV
    (after dequantisation) 2e-2 absolute / 1e-3."""
    return TOL["f32"] if w.kv_dtype == "f32" else TOL[w.kv_dtype]


# A second bound for bf16 and fp8 KV, per output row (one (sequence, q head) or (sequence, token,
# q head)): |d out| <= REL_ROW * max|out_ref over the row| + REL_FLOOR. The 2e-2 absolute bound
# alone is loose where outputs are small (averages of many random V rows are ~1e-2 at the
# workloads' lengths). The arithmetic bounds the error well inside it: the bf16 output rounding
# moves a value by at most 2^-9 (0.2 %) of itself, q.K is exact per product with fp32 sums, and P
# rounded to bf16 in P.V (fp8 KV, 8-head groups) moves the weighted mean by at most 2^-9 of
# max|v| in the worst case and by ~2^-9 |v| / sqrt(rows) for spread-out weights.
REL_ROW, REL_FLOOR = 1e-2, 1e-4


def row_error(w, out_ref, out_gpu):
    """(max |d out|, worst ratio |d out| / (REL_ROW max|ref row| + REL_FLOOR)) over the rows of
    [..., D] outputs; the ratio must stay <= 1 for bf16 / fp8 KV."""
    ref = np.asarray(out_ref, np.float64)
    err = np.abs(np.asarray(out_gpu, np.float64) - ref)
    bound = REL_ROW * np.abs(ref).max(axis=-1, keepdims=True) + REL_FLOOR
    return float(err.max(initial=0)), float((err / bound).max(initial=0))
