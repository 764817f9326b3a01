"""Helpers for the oracle pins: dense (contiguous-cache) brute force in NumPy fp64.

Written independently of the oracle: the contiguous cache of a sequence is taken by flattening its
pages in page-table order, and attention is the textbook softmax(q K^T * scale) V.
"""
import numpy as np
import torch

LOG2E = 1.0 / np.log(2.0)


def to_f64(x, dtype):
    """Storage bits -> fp64 values, through torch's own dtype views (a library decode)."""
    x = np.ascontiguousarray(x)
    if dtype == "f32":
        return x.astype(np.float64)
    if dtype == "bf16":
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    if dtype == "fp8":
        return torch.from_numpy(x).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    if dtype == "fp8e4m3":
        # finite IEEE-style e4m3 codes (exponent below 15) have their e4m3fn values
        assert not np.any(((x & 0x78) == 0x78) & ((x & 0x7F) != 0x7F)), "non-finite e4m3 code"
        return torch.from_numpy(x).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    if dtype == "fp8e5m2":
        return torch.from_numpy(x).view(torch.float8_e5m2).to(torch.float64).numpy()
    raise ValueError(dtype)


def contiguous_kv(w, b, h):
    """K, V rows [total, D] (fp64, scales applied) of sequence b, kv head h."""
    pages = w.page_values[w.page_indptr[b]:w.page_indptr[b + 1]]
    total = int(w.seq_lens[b])
    blk = to_f64(w.pages[pages], w.kv_dtype)  # [np, 2, H_kv, ps, D]
    K = blk[:, 0, h].reshape(-1, w.D)[:total]
    V = blk[:, 1, h].reshape(-1, w.D)[:total]
    if w.kv_dtype in ("fp8", "fp8e4m3", "fp8e5m2"):
        if getattr(w, "k_scale_page", None) is not None:
            # row r of the flattened cache sits on page r // ps of the sequence
            ks = np.repeat(w.k_scale_page[pages, h].astype(np.float64), w.page_size)[:total]
            vs = np.repeat(w.v_scale_page[pages, h].astype(np.float64), w.page_size)[:total]
            K = K * ks[:, None]
            V = V * vs[:, None]
        else:
            K = K * float(w.k_scale[h])
            V = V * float(w.v_scale[h])
    return K, V


def dense_attention(q, K, V, sm_scale):
    """Textbook attention of one query over rows K, V (fp64). Returns out[D], lse (base 2)."""
    s = (K @ q) * sm_scale
    m = s.max()
    e = np.exp(s - m)
    out = (e[:, None] * V).sum(0) / e.sum()
    lse = (m + np.log(e.sum())) * LOG2E
    return out, lse
