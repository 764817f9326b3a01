"""Pins the oracle to what the pages and the mathematics fix (CPU only).

Each test checks the oracle against something other than itself: brute force on a contiguous cache,
closed forms, invariants, the pages' own online recurrences run in fp64, and library routines
(torch's fp8 / bf16 conversions).
"""
import os

import numpy as np
import pytest

import oracle
import synth
from tests.dense_ref import LOG2E, contiguous_kv, dense_attention, to_f64


def run_oracle(w, **over):
    kw = w.oracle_kwargs()
    kw.update(over)
    return oracle.decode(**kw)


def small(**kw):
    base = dict(B=3, H_qo=4, H_kv=2, D=16, page_size=4, seq_lens=[7, 1, 13], q_dtype="f32",
                kv_dtype="f32", seed=11, max_num_pages=12)
    base.update(kw)
    return synth.make_workload(**base)


@pytest.mark.parametrize("kv_dtype,q_dtype", [("f32", "f32"), ("bf16", "bf16"), ("fp8", "bf16")])
@pytest.mark.parametrize("order", ["identity", "shuffled"])
def test_matches_dense_bruteforce(kv_dtype, q_dtype, order):
    """Paged oracle == textbook softmax(q K^T s) V on the flattened contiguous cache."""
    w = small(kv_dtype=kv_dtype, q_dtype=q_dtype, page_order=order, seq_lens=[7, 1, 13])
    out, lse = run_oracle(w)
    G = w.H_qo // w.H_kv
    q64 = to_f64(w.q, w.q_dtype)
    for b in range(w.B):
        for hq in range(w.H_qo):
            K, V = contiguous_kv(w, b, hq // G)
            o, l = dense_attention(q64[b, hq], K, V, w.sm_scale)
            np.testing.assert_allclose(out[b, hq], o, rtol=0, atol=1e-12)
            assert abs(lse[b, hq] - l) < 1e-12


def test_single_row_closed_form():
    """L = 1: out = v_0 exactly and lse = s_0 * log2(e)."""
    w = small(seq_lens=[1, 1, 1])
    out, lse = run_oracle(w)
    q64 = to_f64(w.q, "f32")
    for b in range(w.B):
        page = w.page_values[w.page_indptr[b]]
        for hq in range(w.H_qo):
            h = hq // 2
            k = w.pages[page, 0, h, 0].astype(np.float64)
            v = w.pages[page, 1, h, 0].astype(np.float64)
            assert np.array_equal(out[b, hq], v)
            assert abs(lse[b, hq] - w.sm_scale * float(q64[b, hq] @ k) * LOG2E) < 1e-13


def test_zero_query_is_mean():
    """q = 0: every score is 0, so out = mean of V rows and lse = log2(L)."""
    w = small(seq_lens=[7, 4, 13])
    w.q[:] = 0
    out, lse = run_oracle(w)
    for b in range(w.B):
        for hq in range(w.H_qo):
            _, V = contiguous_kv(w, b, hq // 2)
            np.testing.assert_allclose(out[b, hq], V.mean(0), rtol=0, atol=1e-14)
            assert abs(lse[b, hq] - np.log2(w.seq_lens[b])) < 1e-13


def test_uniform_v_gives_v():
    """Every V row equal to u: out = u whatever the scores."""
    w = small(seq_lens=[9, 3, 16])
    u = np.linspace(-1, 1, w.D).astype(np.float32)
    for p in w.used_pages:
        w.pages[p, 1] = u
    out, _ = run_oracle(w)
    np.testing.assert_allclose(out, np.broadcast_to(u, out.shape), rtol=0, atol=1e-14)


def test_empty_sequence_convention():
    """A sequence with no pages: out = 0, lse = -5e4 (the CPU variant's initial state, no rows)."""
    w = small(seq_lens=[5, 0, 9])
    out, lse = run_oracle(w)
    assert np.all(out[1] == 0.0) and np.all(lse[1] == -5e4)
    assert np.all(np.isfinite(out[[0, 2]]))


def test_empty_window_convention():
    """Pages but zero attended rows (window start at the end, no sink): out = 0, lse = -5e4."""
    w = small(seq_lens=[5, 6, 9])
    li = np.stack([w.length_info, w.seq_lens, np.zeros(w.B, np.int32)]).astype(np.int32)
    out, lse = run_oracle(w, length_info=li, sliding_window=True)
    assert np.all(out == 0.0) and np.all(lse == -5e4)


def test_lse_matches_natural_log_recurrence():
    """The NKI flash kernel (vLLM nki_flash_attn page, _flash_attention_core) keeps the LSE in
    natural log, tile by tile: first tile l = max + log(sum), later l = m + log(exp(l_prev - m) +
    sum) with m the running max. Run that recurrence in fp64; lse_2 must equal lse_e * log2(e)."""
    w = small(seq_lens=[13, 6, 16])
    _, lse = run_oracle(w)
    q64 = to_f64(w.q, "f32")
    tile = 3
    for b in range(w.B):
        for hq in range(w.H_qo):
            K, _ = contiguous_kv(w, b, hq // 2)
            s = (K @ q64[b, hq]) * w.sm_scale
            l = None
            m = -np.inf
            for t0 in range(0, s.size, tile):
                st = s[t0:t0 + tile]
                m = max(m, st.max())
                ps = np.exp(st - m).sum()
                l = m + np.log(ps) if l is None else m + np.log(np.exp(l - m) + ps)
            assert abs(lse[b, hq] - l * LOG2E) < 1e-12


def test_pages_online_recurrence_matches_two_pass():
    """The TVM CPU decode's own algorithm (m = -5e4, d = 1, O = 0; scores in log2 units; per row
    new_m = max(m, s), d = d 2^(m - new_m) + 2^(s - new_m), O rescaled then += 2^(s - m) V;
    out = O / d, lse = m + log2 d), run in fp64, equals the oracle's two-pass definition."""
    w = small(seq_lens=[13, 2, 16])
    out, lse = run_oracle(w)
    q64 = to_f64(w.q, "f32")
    for b in range(w.B):
        for hq in range(w.H_qo):
            K, V = contiguous_kv(w, b, hq // 2)
            m, d, O = -5e4, 1.0, np.zeros(w.D)
            for r in range(K.shape[0]):
                s = float(q64[b, hq] @ K[r]) * w.sm_scale * LOG2E
                new_m = max(m, s)
                d = d * 2.0 ** (m - new_m) + 2.0 ** (s - new_m)
                O = O * 2.0 ** (m - new_m)
                m = new_m
                O = O + V[r] * 2.0 ** (s - m)
            np.testing.assert_allclose(out[b, hq], O / d, rtol=0, atol=1e-12)
            assert abs(lse[b, hq] - (m + np.log2(d))) < 1e-12


def test_gqa_equals_mha_with_repeated_heads():
    """GQA (q head h_qo reads kv head h_qo // G) == MHA whose kv heads are repeated G times."""
    w = small(H_qo=8, H_kv=2, seq_lens=[7, 12, 5])
    out_g, lse_g = run_oracle(w)
    pages_mha = np.repeat(w.pages, 4, axis=2)
    out_m, lse_m = run_oracle(w, H_kv=8, pages=pages_mha)
    assert np.array_equal(out_g, out_m) and np.array_equal(lse_g, lse_m)


def test_page_permutation_invariance():
    """Relabel physical pages by a permutation and move the data: outputs are bit-identical."""
    w = small(seq_lens=[7, 12, 5])
    out0, lse0 = run_oracle(w)
    perm = np.random.default_rng(5).permutation(w.max_num_pages).astype(np.int32)
    pool = np.empty_like(w.pages)
    pool[perm] = w.pages
    out1, lse1 = run_oracle(w, pages=pool, values=perm[w.page_values])
    assert np.array_equal(out0, out1) and np.array_equal(lse0, lse1)


def _prefix_and_suffix(w, b, k):
    """Page tables of rows [0, k) (truncated list + last_page_len) and rows [k, L) (window with
    sink 0 starting at k) for one sequence b of w, as separate single-sequence problems."""
    ps = w.page_size
    pages = w.page_values[w.page_indptr[b]:w.page_indptr[b + 1]]
    L = int(w.seq_lens[b])
    np_pre = (k + ps - 1) // ps
    pre = dict(B=1, indptr=np.array([0, np_pre], np.int32), values=pages[:np_pre],
               length_info=np.array([k - (np_pre - 1) * ps], np.int32), sliding_window=False)
    suf = dict(B=1, indptr=np.array([0, pages.size], np.int32), values=pages,
               length_info=np.array([[L - (pages.size - 1) * ps], [k], [0]], np.int32),
               sliding_window=True)
    return pre, suf


@pytest.mark.parametrize("k", [4, 8, 5, 11])  # page boundaries (ps = 4) and mid-page
def test_merge_of_two_halves_equals_whole(k):
    w = small(seq_lens=[13, 13, 13], B=3)
    out, lse = run_oracle(w)
    b = 2
    pre, suf = _prefix_and_suffix(w, b, k)
    q1 = w.q[b:b + 1]
    o1, l1 = run_oracle(w, q=q1, **pre)
    o2, l2 = run_oracle(w, q=q1, **suf)
    om, lm = oracle.merge_state(o1, l1, o2, l2)
    np.testing.assert_allclose(om[0], out[b], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lm[0], lse[b], rtol=0, atol=1e-12)


def test_nway_merge_is_order_independent_and_exact():
    """Three partitions merged in two different orders both equal the whole (associativity)."""
    w = small(seq_lens=[16, 16, 16])
    out, lse = run_oracle(w)
    b = 0
    ps = w.page_size
    pages = w.page_values[w.page_indptr[b]:w.page_indptr[b + 1]]
    q1 = w.q[b:b + 1]
    cuts = [0, 5, 11, 16]
    states = []
    for lo, hi in zip(cuts[:-1], cuts[1:]):
        npg = (hi + ps - 1) // ps
        li = np.array([[hi - (npg - 1) * ps], [lo], [0]], np.int32)
        states.append(run_oracle(w, q=q1, B=1, indptr=np.array([0, npg], np.int32),
                                 values=pages[:npg], length_info=li, sliding_window=True))
    a = oracle.merge_state(*oracle.merge_state(*states[0], *states[1]), *states[2])
    c = oracle.merge_state(*states[0], *oracle.merge_state(*states[1], *states[2]))
    for o, l in (a, c):
        np.testing.assert_allclose(o[0], out[b], rtol=0, atol=1e-12)
        np.testing.assert_allclose(l[0], lse[b], rtol=0, atol=1e-12)


def test_merge_closed_forms():
    """Merging a state with itself keeps V and adds exactly 1 to the base-2 lse; merging with a
    state 2^-60 times lighter leaves V unchanged to fp64 rounding."""
    rng = np.random.default_rng(3)
    v = rng.standard_normal((2, 3, 8))
    s = rng.standard_normal((2, 3)) * 10
    vm, sm = oracle.merge_state(v, s, v, s)
    np.testing.assert_allclose(vm, v, rtol=0, atol=1e-15)
    np.testing.assert_allclose(sm, s + 1.0, rtol=0, atol=1e-13)
    vm, sm = oracle.merge_state(v, s, rng.standard_normal((2, 3, 8)), s - 60)
    np.testing.assert_allclose(vm, v, rtol=0, atol=1e-17 * 1e2)


@pytest.mark.parametrize("sink,window", [(2, 6), (0, 5), (3, 100)])
def test_window_and_sink_bruteforce(sink, window):
    """Window reading: attended rows are the first `sink` positions then positions
    [win_off, total) with win_off = max(sink, total - window)."""
    w = small(seq_lens=[13, 3, 16], window=window, sink=sink)
    out, lse = run_oracle(w)
    q64 = to_f64(w.q, "f32")
    for b in range(w.B):
        L = int(w.seq_lens[b])
        off = max(sink, L - window)
        rows = list(range(min(sink, L))) + list(range(off, L))
        for hq in range(w.H_qo):
            K, V = contiguous_kv(w, b, hq // 2)
            o, l = dense_attention(q64[b, hq], K[rows], V[rows], w.sm_scale)
            np.testing.assert_allclose(out[b, hq], o, rtol=0, atol=1e-12)
            assert abs(lse[b, hq] - l) < 1e-12


def test_window_zero_reduces_to_plain():
    """sink = 0 and win_off = 0 is the no-window path."""
    w = small(seq_lens=[13, 3, 16])
    out0, lse0 = run_oracle(w)
    li = np.stack([w.length_info, np.zeros(w.B, np.int32), np.zeros(w.B, np.int32)])
    out1, lse1 = run_oracle(w, length_info=li, sliding_window=True)
    assert np.array_equal(out0, out1) and np.array_equal(lse0, lse1)


# ---------------------------------------------------------------- RoPE invariants
def test_rope_position_zero_is_identity():
    rng = np.random.default_rng(2)
    x = rng.standard_normal(128)
    assert np.array_equal(oracle.rope_rotate(x, 0, 1.0, 5e5), x)


def test_rope_decode_uses_compacted_row_positions():
    """With rope on, the K row r sits at position k_rope_pos_offset + r: rotating the contiguous
    K rows by their row index and q by its position reproduces the oracle through brute force."""
    w = small(seq_lens=[13, 3, 16], rotary_mode=1, rope_theta=1e4)
    qp = np.array([12, 2, 15], np.int32)
    ko = np.array([0, 5, 100], np.int32)
    out, lse = run_oracle(w, q_rope_position=qp, k_rope_pos_offset=ko)
    q64 = to_f64(w.q, "f32")
    for b in range(w.B):
        for hq in range(w.H_qo):
            K, V = contiguous_kv(w, b, hq // 2)
            Kr = np.stack([oracle.rope_rotate(K[r], ko[b] + r, 1.0, 1e4) for r in range(K.shape[0])])
            qr = oracle.rope_rotate(q64[b, hq], qp[b], 1.0, 1e4)
            o, l = dense_attention(qr, Kr, V, w.sm_scale)
            np.testing.assert_allclose(out[b, hq], o, rtol=0, atol=1e-12)
            assert abs(lse[b, hq] - l) < 1e-12


def test_rope_only_modes_one_and_two_apply():
    """rotary_mode 1 (rotate-half) and 2 (interleaved) apply RoPE; any other value applies none."""
    w = small(seq_lens=[13, 3, 16])
    out0, lse0 = run_oracle(w)
    pos = np.array([100, 7, 3], np.int32)
    for mode in (1, 2):
        out1, _ = run_oracle(w, rotary_mode=mode, q_rope_position=pos, k_rope_pos_offset=pos)
        assert np.abs(out1 - out0).max() > 1e-3
    for mode in (0, 3, -1):
        out1, lse1 = run_oracle(w, rotary_mode=mode, q_rope_position=pos, k_rope_pos_offset=pos)
        assert np.array_equal(out0, out1) and np.array_equal(lse0, lse1)


@pytest.mark.parametrize("mode", [1, 2])
def test_rope_relative_position_invariance(mode):
    """Shifting the q position and the k offset by the same amount leaves every score unchanged
    (both layouts)."""
    w = small(seq_lens=[13, 3, 16], rotary_mode=mode, rope_theta=500000.0)
    qp = np.array([12, 2, 15], np.int32)
    ko = np.zeros(3, np.int32)
    out0, lse0 = run_oracle(w, q_rope_position=qp, k_rope_pos_offset=ko)
    out1, lse1 = run_oracle(w, q_rope_position=qp + 9000, k_rope_pos_offset=ko + 9000)
    np.testing.assert_allclose(out1, out0, rtol=0, atol=1e-9)
    np.testing.assert_allclose(lse1, lse0, rtol=0, atol=1e-9)
    out2, _ = run_oracle(w, q_rope_position=qp + 5, k_rope_pos_offset=ko)
    assert np.abs(out2 - out0).max() > 1e-3  # and a relative shift does change the result


def test_rope_is_a_rotation():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(64)
    for pos in (1, 37, 4099):
        y = oracle.rope_rotate(x, pos, 1.0, 1e4)
        assert abs(np.linalg.norm(y) - np.linalg.norm(x)) < 1e-12
        # pairs (i, i + D/2) keep their norms
        np.testing.assert_allclose(y[:32] ** 2 + y[32:] ** 2, x[:32] ** 2 + x[32:] ** 2, atol=1e-12)
    a = oracle.rope_rotate(oracle.rope_rotate(x, 123, 1.0, 5e5), 456, 1.0, 5e5)
    np.testing.assert_allclose(a, oracle.rope_rotate(x, 579, 1.0, 5e5), atol=1e-11)
    np.testing.assert_allclose(oracle.rope_rotate(oracle.rope_rotate(x, 77, 1.0, 1e4), -77, 1.0, 1e4),
                               x, atol=1e-12)
    # position scaling: R_scale(p) == R_1(p * scale)
    np.testing.assert_allclose(oracle.rope_rotate(x, 10, 0.25, 1e4), oracle.rope_rotate(x, 2.5, 1.0, 1e4),
                               atol=1e-13)


def test_rope_two_dims_is_plane_rotation():
    """D = 2: a single pair at frequency theta^0 = 1, i.e. the textbook plane rotation by p."""
    for p in (0.0, 1.0, 2.5, 100.0):
        y = oracle.rope_rotate(np.array([1.0, 0.0]), p, 1.0, 1e4)
        np.testing.assert_allclose(y, [np.cos(p), np.sin(p)], atol=1e-15)


# ---------------------------------------------------------------- RoPE against common implementations
# The pages import the rotation helper without showing it, so its convention (which dims pair up,
# the frequency schedule, the sign of the rotation) is pinned here against the two layouts that the
# attention_block_tkg page names, as the transformers library implements them: Llama's rotate-half
# (contiguous halves) and GPT-J's rotate-every-two (interleaved pairs), with their own frequency
# schedules. Positions reach 131 071, so a wrong schedule (theta^(-i/D), theta^(-2i/(D-2)), ...),
# a swapped pairing or a flipped sign fails by O(1).
RPOS = np.array([0, 1, 2, 17, 100, 4095, 4096, 65537, 131071], np.int64)


def _llama_inv_freq64(D, theta, rope_type="default", factor=None):
    """transformers' Llama inverse frequencies, evaluated with the library's own formula in
    float64 (its arange dtype, torch.float, patched to float64 for the call)."""
    import torch
    from unittest import mock
    from transformers import LlamaConfig
    from transformers.modeling_rope_utils import ROPE_INIT_FUNCTIONS
    from transformers.models.llama import modeling_llama as ml
    params = {"rope_type": rope_type, "rope_theta": float(theta)}
    if factor is not None:
        params["factor"] = float(factor)
    cfg = LlamaConfig(hidden_size=D, num_attention_heads=1, head_dim=D, rope_parameters=params)
    fn = (ml.LlamaRotaryEmbedding.compute_default_rope_parameters if rope_type == "default"
          else ROPE_INIT_FUNCTIONS[rope_type])
    with mock.patch.object(torch, "float", torch.float64):
        inv, _ = fn(cfg, None)
    assert inv.dtype == torch.float64 and inv.shape == (D // 2,)
    return inv


def _oracle_rows(x, pos, scale, theta, interleaved=False):
    return np.stack([oracle.rope_rotate(x[i], float(pos[i]), scale, theta, interleaved=interleaved)
                     for i in range(len(pos))])


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("theta", [1e4, 5e5])
def test_rope_rotate_half_matches_transformers_llama(D, theta):
    """Rotate-half against transformers' Llama rotate_half / apply_rotary_pos_emb with its
    default inverse frequencies (float64), at positions up to 131 071."""
    torch = pytest.importorskip("torch")
    ml = pytest.importorskip("transformers.models.llama.modeling_llama")
    rng = np.random.default_rng(int(D + theta) % 1000)
    x = rng.standard_normal((len(RPOS), D))
    inv = _llama_inv_freq64(D, theta)
    freqs = torch.from_numpy(RPOS.astype(np.float64))[:, None] * inv[None, :]
    emb = torch.cat((freqs, freqs), dim=-1)[None]  # [1, n, D], as the library's forward builds it
    xt = torch.from_numpy(x)[None, None]  # [1, 1, n, D]
    ref, _ = ml.apply_rotary_pos_emb(xt, xt, emb.cos(), emb.sin(), unsqueeze_dim=1)
    got = _oracle_rows(x, RPOS, 1.0, theta)
    np.testing.assert_allclose(got, ref[0, 0].numpy(), rtol=0, atol=1e-9)


@pytest.mark.parametrize("D", [64, 128])
def test_rope_rotate_half_matches_transformers_llama_fp32_pipeline(D):
    """The same against the library's whole float32 path (LlamaRotaryEmbedding.forward, then
    apply_rotary_pos_emb) at positions where float32 angles stay within 2e-3 rad."""
    torch = pytest.importorskip("torch")
    ml = pytest.importorskip("transformers.models.llama.modeling_llama")
    from transformers import LlamaConfig
    pos = np.array([0, 1, 3, 50, 511, 2047], np.int64)
    cfg = LlamaConfig(hidden_size=D, num_attention_heads=1, head_dim=D,
                      rope_parameters={"rope_type": "default", "rope_theta": 500000.0})
    rot = ml.LlamaRotaryEmbedding(cfg)
    x = np.random.default_rng(5).standard_normal((len(pos), D)).astype(np.float32)
    xt = torch.from_numpy(x)[None, None]
    cos, sin = rot(xt, torch.from_numpy(pos)[None])
    ref, _ = ml.apply_rotary_pos_emb(xt, xt, cos, sin, unsqueeze_dim=1)
    got = _oracle_rows(x.astype(np.float64), pos, 1.0, 500000.0)
    np.testing.assert_allclose(got, ref[0, 0].double().numpy(), rtol=0, atol=5e-3)


def test_rope_scale_matches_transformers_linear_scaling():
    """rope_scale multiplies the position: transformers' 'linear' RoPE with factor 4 divides every
    frequency by 4, which is rope_scale = 0.25."""
    torch = pytest.importorskip("torch")
    ml = pytest.importorskip("transformers.models.llama.modeling_llama")
    D, theta = 128, 1e4
    inv = _llama_inv_freq64(D, theta, rope_type="linear", factor=4.0)
    x = np.random.default_rng(9).standard_normal((len(RPOS), D))
    freqs = torch.from_numpy(RPOS.astype(np.float64))[:, None] * inv[None, :]
    emb = torch.cat((freqs, freqs), dim=-1)[None]
    xt = torch.from_numpy(x)[None, None]
    ref, _ = ml.apply_rotary_pos_emb(xt, xt, emb.cos(), emb.sin(), unsqueeze_dim=1)
    got = _oracle_rows(x, RPOS, 0.25, theta)
    np.testing.assert_allclose(got, ref[0, 0].numpy(), rtol=0, atol=1e-9)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("theta", [1e4, 5e5])
def test_rope_interleaved_matches_transformers_gptj(D, theta):
    """Interleaved pairs against transformers' GPT-J rotate_every_two / apply_rotary_pos_emb
    (sin and cos repeated per pair), float64, with the inverse frequencies of the Llama schedule,
    which GPT-J's own table uses (pinned at base 1e4 by the float32 test below)."""
    torch = pytest.importorskip("torch")
    mg = pytest.importorskip("transformers.models.gptj.modeling_gptj")
    inv = _llama_inv_freq64(D, theta)
    x = np.random.default_rng(int(theta) % 997 + D).standard_normal((len(RPOS), D))
    ang = torch.from_numpy(RPOS.astype(np.float64))[:, None] * inv[None, :]  # [n, D/2]
    xt = torch.from_numpy(x)[None, :, None, :]  # [batch, seq, heads, D]
    ref = mg.apply_rotary_pos_emb(xt, ang.sin()[None], ang.cos()[None])
    got = _oracle_rows(x, RPOS, 1.0, theta, interleaved=True)
    np.testing.assert_allclose(got, ref[0, :, 0].numpy(), rtol=0, atol=1e-9)


@pytest.mark.parametrize("D", [64, 128])
def test_rope_interleaved_matches_gptj_sinusoid_table(D):
    """Interleaved pairs against GPT-J's whole float32 path: its sinusoid table
    (create_sinusoidal_positions, base 1e4), split into sin and cos, then apply_rotary_pos_emb."""
    torch = pytest.importorskip("torch")
    mg = pytest.importorskip("transformers.models.gptj.modeling_gptj")
    pos = np.array([0, 1, 3, 50, 511, 2047], np.int64)
    table = mg.create_sinusoidal_positions(2048, D)  # [pos, D] = (sin | cos)
    sincos = table[torch.from_numpy(pos)][None]
    sin, cos = torch.split(sincos, D // 2, dim=-1)
    x = np.random.default_rng(6).standard_normal((len(pos), D)).astype(np.float32)
    ref = mg.apply_rotary_pos_emb(torch.from_numpy(x)[None, :, None, :], sin, cos)
    got = _oracle_rows(x.astype(np.float64), pos, 1.0, 1e4, interleaved=True)
    np.testing.assert_allclose(got, ref[0, :, 0].double().numpy(), rtol=0, atol=5e-3)


def test_rope_wrong_schedules_fail_the_pin():
    """The pins above separate the schedule from plausible mistakes: at the positions they use,
    theta^(-i/D) and theta^(-2i/(D-2)) move some element by far more than their tolerances."""
    D, theta = 128, 5e5
    i = np.arange(D // 2)
    right = theta ** (-2.0 * i / D)
    for wrong in (theta ** (-1.0 * i / D), theta ** (-2.0 * i / (D - 2))):
        dphi = np.abs(np.outer(RPOS, wrong - right))
        assert np.abs(np.sin(dphi / 2)).max() > 0.1


# ---------------------------------------------------------------- fp8 e4m3fn and bf16 codecs
def test_fp8_reference_values():
    """Values fixed by the OCP FP8 e4m3fn definition (see tests/golden/fp8_e4m3fn_values.txt)."""
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "fp8_e4m3fn_values.txt")
    n = 0
    for line in open(path):
        line = line.split("#")[0].strip()
        if not line:
            continue
        code, val = line.split()
        code = int(code, 16)
        if val == "nan":
            assert np.isnan(oracle.fp8_value(code))
        else:
            v = float.fromhex(val) if "p" in val else float(val)
            got = oracle.fp8_value(code)
            assert got == v and np.signbit(got) == np.signbit(v), (hex(code), got, v)
        n += 1
    assert n >= 12


def test_fp8_table_shape():
    """Codes 0x00..0x7E increase strictly; within each binade the step is constant; 254 finite
    codes; the negative half mirrors the positive half."""
    vals = np.array([oracle.fp8_value(c) for c in range(256)])
    pos = vals[:0x7F]
    assert np.all(np.diff(pos) > 0)
    assert np.sum(np.isfinite(vals)) == 254
    np.testing.assert_array_equal(vals[0x80:0xFF], -pos)
    for e in range(1, 15):
        binade = pos[8 * e:8 * e + 8]
        steps = np.diff(binade)
        assert np.all(steps == steps[0])


def test_fp8_decode_matches_library():
    import torch
    codes = torch.arange(256, dtype=torch.uint8)
    lib = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = np.array([oracle.fp8_value(c) for c in range(256)])
    same = (lib == ours) | (np.isnan(lib) & np.isnan(ours))
    assert same.all()


def test_fp8_encode_roundtrip_ties_and_saturation():
    vals = [oracle.fp8_value(c) for c in range(256)]
    for c in range(256):
        if np.isfinite(vals[c]):
            assert oracle.fp8_encode(vals[c]) == c
    # midpoints between neighbours go to the even code
    for c in range(0, 0x7E):
        mid = (vals[c] + vals[c + 1]) / 2
        if np.float32(mid) == mid:
            got = oracle.fp8_encode(mid)
            assert got == (c if c % 2 == 0 else c + 1), hex(c)
    assert oracle.fp8_encode(1e6) == 0x7E and oracle.fp8_encode(-1e6) == 0xFE
    assert oracle.fp8_encode(float("inf")) == 0x7E and oracle.fp8_encode(float("-inf")) == 0xFE
    assert oracle.fp8_encode(464.0) == 0x7E and oracle.fp8_encode(449.0) == 0x7E
    assert oracle.fp8_encode(float("nan")) & 0x7F == 0x7F


def test_fp8_encode_is_nearest_bruteforce_and_library():
    import torch
    rng = np.random.default_rng(9)
    x = np.concatenate([rng.standard_normal(3000) * 100, rng.standard_normal(1000) * 0.01,
                        rng.uniform(-448, 448, 1000)]).astype(np.float32)
    codes = oracle.fp8_encode_array(x)
    table = np.array([oracle.fp8_value(c) for c in range(0x7F)])
    for xi, c in zip(x, codes):
        err = abs(abs(float(xi)) - table)
        assert abs(abs(float(xi)) - table[c & 0x7F]) == err.min()
    lib = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(lib, codes)


def test_bf16_value_matches_library():
    import torch
    bits = np.arange(0, 65536, 7, dtype=np.uint16)
    lib = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    ours = np.array([oracle.bf16_value(int(b)) for b in bits])
    same = (lib == ours) | (np.isnan(lib) & np.isnan(ours))
    assert same.all()


# ---------------------------------------------------------------- append
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_append_bitexact_bruteforce(dtype):
    H_kv, D, ps, P = 3, 16, 4, 10
    pool = synth.poisoned_pool(P, H_kv, ps, D, dtype)
    before = pool.copy()
    k, v, slots = synth.append_inputs(T=9, H_kv=H_kv, D=D, page_size=ps, max_num_pages=P,
                                      in_dtype=dtype, seed=4, skip_every=4)
    oracle.append_kv(pages=pool, new_k=k, new_v=v, slots=slots, H_kv=H_kv, D=D, ps=ps,
                     in_dtype=synth.DTYPE_CODE[dtype], kv_dtype=synth.DTYPE_CODE[dtype])
    expect = before.copy()
    for t, s in enumerate(slots):
        if s >= 0:
            expect[s // ps, 0, :, s % ps, :] = k[t]
            expect[s // ps, 1, :, s % ps, :] = v[t]
    assert expect.tobytes() == pool.tobytes()
    assert (slots < 0).sum() == 3


def test_append_fp8_matches_library_quantization():
    import torch
    H_kv, D, ps, P = 2, 16, 8, 6
    pool = synth.poisoned_pool(P, H_kv, ps, D, "fp8")
    k, v, slots = synth.append_inputs(T=7, H_kv=H_kv, D=D, page_size=ps, max_num_pages=P,
                                      in_dtype="bf16", seed=8, skip_every=3)
    ks = np.array([0.5 / 448, 2.0 / 448], np.float32)
    vs = np.array([1.0 / 448, 0.75 / 448], np.float32)
    before = pool.copy()
    oracle.append_kv(pages=pool, new_k=k, new_v=v, slots=slots, H_kv=H_kv, D=D, ps=ps,
                     in_dtype=1, kv_dtype=2, k_scale=ks, v_scale=vs)
    kf = to_f64(k, "bf16").astype(np.float32)
    vf = to_f64(v, "bf16").astype(np.float32)
    expect = before.copy()
    for t, s in enumerate(slots):
        if s < 0:
            continue
        for kv, x, sc in ((0, kf, ks), (1, vf, vs)):
            y = np.clip(x[t] / sc[:, None], -448, 448)  # fp32 divide, then satfinite
            expect[s // ps, kv, :, s % ps, :] = (torch.from_numpy(np.ascontiguousarray(y))
                                                 .to(torch.float8_e4m3fn).view(torch.uint8).numpy())
    assert expect.tobytes() == pool.tobytes()


# ---------------------------------------------------------------- validator
def test_validator_codes():
    w = small(seq_lens=[7, 0, 13], window=6, sink=2)
    kw = dict(B=w.B, ps=w.page_size, max_num_pages=w.max_num_pages, indptr=w.page_indptr,
              values=w.page_values, length_info=w.length_info, sliding_window=True)
    assert oracle.validate_page_table(**kw) == 0
    bad = dict(kw, indptr=np.array([0, 3, 2, w.page_indptr[-1]], np.int32))
    assert oracle.validate_page_table(**bad) == 1
    vals = w.page_values.copy(); vals[0] = w.max_num_pages
    assert oracle.validate_page_table(**dict(kw, values=vals)) == 2
    li = w.length_info.copy(); li[0, 0] = 0
    assert oracle.validate_page_table(**dict(kw, length_info=li)) == 3
    li = w.length_info.copy(); li[2, 0] = li[1, 0] + 1
    assert oracle.validate_page_table(**dict(kw, length_info=li)) == 4


def test_oracle_rejects_out_of_range_page():
    w = small()
    vals = w.page_values.copy()
    vals[-1] = 99
    with pytest.raises(oracle.OracleError):
        run_oracle(w, values=vals)


# ---- fused decode step (append at each sequence's last position, then decode)

def test_last_position_slots_brute_force():
    """The slot of position total - 1, found by walking every position of every sequence through
    the page table (position p -> page values[beg + p // ps], row p % ps), for lengths at and
    around page boundaries, an empty sequence and shuffled page ids."""
    ps = 4
    lens = [0, 1, 3, 4, 5, 8, 9, 13]
    B = len(lens)
    npages = [(L + ps - 1) // ps for L in lens]
    indptr = np.concatenate([[0], np.cumsum(npages)]).astype(np.int32)
    values = np.random.default_rng(3).permutation(64)[: indptr[-1]].astype(np.int32)
    last = np.array([L - (n - 1) * ps if n else 0 for L, n in zip(lens, npages)], np.int32)
    got = oracle.last_position_slots(B=B, ps=ps, indptr=indptr, values=values, length_info=last)
    for b, L in enumerate(lens):
        want = -1
        for pos in range(L):
            want = int(values[indptr[b] + pos // ps]) * ps + pos % ps
        assert got[b] == want, (b, L)
    # with a window the row is the same: length_info row 0 is still last_page_len
    li3 = np.stack([last, np.zeros(B, np.int32), np.zeros(B, np.int32)])
    got3 = oracle.last_position_slots(B=B, ps=ps, indptr=indptr, values=values, length_info=li3)
    assert np.array_equal(got3, got)


def test_append_then_decode_single_row_is_the_new_row():
    """Sequences of one row: after the step that row is the new token, so out = new_v of the KV
    head and lse = sm_scale * (q . new_k) * log2 e (the L = 1 closed form), whatever the pool held
    there before (here NaN); a sequence without pages gets no row and the empty convention."""
    B, H_kv, G, D, ps = 3, 2, 2, 8, 4
    H_qo = H_kv * G
    rng = np.random.default_rng(11)
    q = rng.standard_normal((B, H_qo, D)).astype(np.float32)
    pages = np.full((6, 2, H_kv, ps, D), np.nan, np.float32)
    indptr = np.array([0, 1, 1, 2], np.int32)
    values = np.array([4, 1], np.int32)
    last = np.array([1, 0, 1], np.int32)
    nk = rng.standard_normal((B, H_kv, D)).astype(np.float32)
    nv = rng.standard_normal((B, H_kv, D)).astype(np.float32)
    sm = float(np.float32(0.3))  # the oracle takes sm_scale as the fp32 value the ABI receives
    out, lse, pool = oracle.append_then_decode(
        new_k=nk, new_v=nv, B=B, H_qo=H_qo, H_kv=H_kv, D=D, ps=ps, max_num_pages=6, q_dtype=0,
        kv_dtype=0, q=q, pages=pages, indptr=indptr, values=values, length_info=last,
        sm_scale=sm)
    for b in (0, 2):
        for h in range(H_qo):
            hk = h // G
            assert np.array_equal(out[b, h], nv[b, hk].astype(np.float64))
            s = sm * float(np.dot(q[b, h].astype(np.float64), nk[b, hk].astype(np.float64)))
            assert abs(lse[b, h] - s * LOG2E) < 1e-12
    assert np.all(out[1] == 0) and np.all(lse[1] == -5e4)
    assert np.array_equal(pool[4, 0, :, 0], nk[0]) and np.array_equal(pool[1, 1, :, 0], nv[2])
    assert np.isnan(pool[4, 0, :, 1:]).all()  # nothing else written


# ---- several query tokens per sequence (causal over the new tokens)

@pytest.mark.parametrize("kv_dtype,q_dtype", [("f32", "f32"), ("bf16", "bf16"), ("fp8", "bf16")])
@pytest.mark.parametrize("T", [2, 3])
def test_multi_token_matches_dense_causal_bruteforce(kv_dtype, q_dtype, T):
    """Token t of a sequence of total rows L = textbook softmax over the flattened cache's rows
    0 .. L - T + t; a token whose prefix is empty gets out = 0, lse = -5e4."""
    w = small(B=4, kv_dtype=kv_dtype, q_dtype=q_dtype, page_order="shuffled",
              seq_lens=[7, 1, 13, 0])
    qm = synth.multi_query(w, T, seed=5)
    out, lse = oracle.decode_multi(qo_len=T, q=qm, **{k: v for k, v in w.oracle_kwargs().items()
                                                     if k != "q"})
    G = w.H_qo // w.H_kv
    q64 = to_f64(qm, w.q_dtype)
    for b in range(w.B):
        L = int(w.seq_lens[b])
        for t in range(T):
            n = L - T + t + 1
            for hq in range(w.H_qo):
                if n <= 0:
                    assert np.all(out[b, t, hq] == 0) and lse[b, t, hq] == -5e4
                    continue
                K, V = contiguous_kv(w, b, hq // G)
                o, l = dense_attention(q64[b, t, hq], K[:n], V[:n], w.sm_scale)
                np.testing.assert_allclose(out[b, t, hq], o, rtol=0, atol=1e-12)
                assert abs(lse[b, t, hq] - l) < 1e-12


@pytest.mark.parametrize("mode", [1, 2])
@pytest.mark.parametrize("kv_dtype,q_dtype", [("f32", "f32"), ("bf16", "bf16")])
def test_multi_token_rope_matches_dense_causal_bruteforce(kv_dtype, q_dtype, mode):
    """RoPE (rotate-half or interleaved) with several tokens: token t's query rotated to
    q_rope_position + t, the flattened cache's row r to k_rope_pos_offset + r, then the causal
    brute force as above."""
    T = 3
    ilv = mode == 2
    w = small(B=4, kv_dtype=kv_dtype, q_dtype=q_dtype, page_order="shuffled",
              seq_lens=[7, 1, 13, 0], rotary_mode=mode, rope_theta=1e4)
    qm = synth.multi_query(w, T, seed=7)
    qp = np.array([40, 0, 12, 3], np.int32)
    ko = np.array([33, 5, 0, 0], np.int32)
    kw = {k: v for k, v in w.oracle_kwargs().items() if k != "q"}
    kw.update(q_rope_position=qp, k_rope_pos_offset=ko)
    out, lse = oracle.decode_multi(qo_len=T, q=qm, **kw)
    G = w.H_qo // w.H_kv
    q64 = to_f64(qm, w.q_dtype)
    for b in range(w.B):
        L = int(w.seq_lens[b])
        for t in range(T):
            n = L - T + t + 1
            for hq in range(w.H_qo):
                if n <= 0:
                    assert np.all(out[b, t, hq] == 0) and lse[b, t, hq] == -5e4
                    continue
                K, V = contiguous_kv(w, b, hq // G)
                Kr = np.stack([oracle.rope_rotate(K[r], ko[b] + r, 1.0, 1e4, interleaved=ilv)
                               for r in range(n)])
                qr = oracle.rope_rotate(q64[b, t, hq], qp[b] + t, 1.0, 1e4, interleaved=ilv)
                o, l = dense_attention(qr, Kr, V[:n], w.sm_scale)
                np.testing.assert_allclose(out[b, t, hq], o, rtol=0, atol=1e-12)
                assert abs(lse[b, t, hq] - l) < 1e-12
    # and the positions matter: without RoPE the result differs
    kw0 = {k: v for k, v in w.oracle_kwargs().items() if k != "q"}
    kw0["rotary_mode"] = 0
    out0, _ = oracle.decode_multi(qo_len=T, q=qm, **kw0)
    assert np.abs(out0 - out).max() > 1e-3


@pytest.mark.parametrize("rope", [0, 1])
def test_multi_token_window_matches_dense_causal_bruteforce(rope):
    """Several tokens with a sliding window and a sink (one window per sequence for all its
    tokens): token t sees the flattened cache's rows r <= L - T + t with r < sink or r >= win_off;
    with RoPE the keys sit at k_rope_pos_offset + their compacted index (r below the sink,
    sink + r - win_off in the window) and token t's query at q_rope_position + t."""
    T = 4
    w = small(B=5, kv_dtype="bf16", q_dtype="bf16", page_order="shuffled",
              seq_lens=[30, 3, 21, 0, 12], window=9, sink=2, rotary_mode=rope, rope_theta=1e4,
              max_num_pages=24)
    qm = synth.multi_query(w, T, seed=9)
    kw = {k: v for k, v in w.oracle_kwargs().items() if k != "q"}
    qp = np.array([50, 3, 20, 0, 9], np.int32)
    ko = np.array([5, 0, 11, 0, 2], np.int32)
    if rope:
        kw.update(q_rope_position=qp, k_rope_pos_offset=ko)
    out, lse = oracle.decode_multi(qo_len=T, q=qm, **kw)
    G = w.H_qo // w.H_kv
    q64 = to_f64(qm, w.q_dtype)
    seen_window = seen_sink_only = 0
    for b in range(w.B):
        L = int(w.seq_lens[b])
        off, sink = int(w.length_info[1, b]), int(w.length_info[2, b])
        for t in range(T):
            n = L - T + t + 1
            rows = [r for r in range(max(n, 0)) if r < sink or r >= off]
            seen_window += any(r >= off for r in rows) and any(r < off for r in range(max(n, 0)))
            seen_sink_only += bool(rows) and all(r < sink for r in rows) and n > sink
            for hq in range(w.H_qo):
                if not rows:
                    assert np.all(out[b, t, hq] == 0) and lse[b, t, hq] == -5e4
                    continue
                K, V = contiguous_kv(w, b, hq // G)
                K, V = K[rows], V[rows]
                q = q64[b, t, hq]
                if rope:
                    pos = [r if r < sink else sink + r - off for r in rows]
                    K = np.stack([oracle.rope_rotate(K[i], ko[b] + pos[i], 1.0, 1e4)
                                  for i in range(len(rows))])
                    q = oracle.rope_rotate(q, qp[b] + t, 1.0, 1e4)
                o, l = dense_attention(q, K, V, w.sm_scale)
                np.testing.assert_allclose(out[b, t, hq], o, rtol=0, atol=1e-12)
                assert abs(lse[b, t, hq] - l) < 1e-12
    assert seen_window > 0  # tokens whose prefix crosses the window start


def test_multi_token_one_token_is_decode():
    """qo_len = 1 is the single-token decode, bit for bit."""
    w = small(seq_lens=[7, 1, 13])
    out1, lse1 = oracle.decode_multi(qo_len=1, q=w.q[:, None], **{
        k: v for k, v in w.oracle_kwargs().items() if k != "q"})
    out, lse = run_oracle(w)
    assert np.array_equal(out1[:, 0], out) and np.array_equal(lse1[:, 0], lse)


# ---- learned attention sink per q head

@pytest.mark.parametrize("kv_dtype,q_dtype", [("f32", "f32"), ("bf16", "bf16"), ("fp8", "bf16")])
def test_sink_matches_dense_with_an_extra_logit(kv_dtype, q_dtype):
    """A sink logit is one more softmax entry with a zero value row: textbook attention over the
    scores plus the sink, on the flattened cache; the empty sequence keeps its convention."""
    w = small(B=4, kv_dtype=kv_dtype, q_dtype=q_dtype, page_order="shuffled",
              seq_lens=[7, 1, 13, 0])
    sinks = np.array([0.5, -3.0, 2.5, 40.0], np.float32)  # 40: the sink takes almost everything
    out0, lse0 = run_oracle(w)
    out, lse = oracle.apply_sink(out0, lse0, sinks)
    G = w.H_qo // w.H_kv
    q64 = to_f64(w.q, w.q_dtype)
    for b in range(w.B):
        for hq in range(w.H_qo):
            if w.seq_lens[b] == 0:
                assert np.all(out[b, hq] == 0) and lse[b, hq] == -5e4
                continue
            K, V = contiguous_kv(w, b, hq // G)
            s = np.concatenate([(K @ q64[b, hq]) * w.sm_scale, [float(sinks[hq])]])
            Vx = np.vstack([V, np.zeros((1, w.D))])
            m = s.max()
            e = np.exp(s - m)
            np.testing.assert_allclose(out[b, hq], (e[:, None] * Vx).sum(0) / e.sum(), rtol=0,
                                       atol=1e-12)
            assert abs(lse[b, hq] - (m + np.log(e.sum())) * LOG2E) < 1e-12


def test_interleaved_rope_is_rotate_half_of_the_deinterleaved_vector():
    """The interleaved layout pairs (2i, 2i + 1) with frequency i; moving element 2i to i and
    2i + 1 to i + D/2 turns it into rotate-half: R_ilv(x) = P^-1 R_half(P x) for every position,
    scale and base; R_ilv(0) = I and pairs (2i, 2i + 1) keep their norms."""
    rng = np.random.default_rng(2)
    D = 64
    x = rng.standard_normal(D)
    perm = np.concatenate([np.arange(0, D, 2), np.arange(1, D, 2)])  # P x = x[perm]
    for pos, scale, theta in ((0, 1.0, 1e4), (1, 1.0, 1e4), (37, 0.5, 5e5), (4099, 1.0, 1e4)):
        y = oracle.rope_rotate(x, pos, scale, theta, interleaved=True)
        z = np.empty(D)
        z[perm] = oracle.rope_rotate(x[perm], pos, scale, theta)
        np.testing.assert_allclose(y, z, rtol=0, atol=1e-12)
        np.testing.assert_allclose(y[0::2] ** 2 + y[1::2] ** 2, x[0::2] ** 2 + x[1::2] ** 2,
                                   atol=1e-12)
    assert np.array_equal(oracle.rope_rotate(x, 0, 1.0, 1e4, interleaved=True), x)


def test_multi_token_select_matches_full():
    """decode_multi on selected (b, t, h_qo) triples returns those rows of the full result."""
    w = small(B=4, seq_lens=[7, 1, 13, 0])
    qm = synth.multi_query(w, 3, seed=6)
    kw = {k: v for k, v in w.oracle_kwargs().items() if k != "q"}
    out, lse = oracle.decode_multi(qo_len=3, q=qm, **kw)
    sel = np.array([[0, 2, 1], [2, 0, 3], [1, 0, 0], [3, 1, 2]], np.int32)
    o, l = oracle.decode_multi(qo_len=3, q=qm, select=sel, **kw)
    assert np.array_equal(o, out[sel[:, 0], sel[:, 1], sel[:, 2]])
    assert np.array_equal(l, lse[sel[:, 0], sel[:, 1], sel[:, 2]])


# ---- IEEE-style e4m3 (the NON_OCP float8_e4m3, max 240)

def test_fp8_e4m3_values_and_relation_to_e4m3fn():
    """Every code: exponent below 15 has the e4m3fn value (pinned against torch); exponent 15 is
    infinity (mantissa 0) or NaN; the fixture's values (max 240) hold."""
    for c in range(256):
        e, m = (c >> 3) & 15, c & 7
        v = oracle.fp8_e4m3_value(c)
        if e < 15:
            assert v == oracle.fp8_value(c), c
        elif m == 0:
            assert np.isinf(v) and (v < 0) == bool(c & 0x80), c
        else:
            assert np.isnan(v), c
    path = os.path.join(os.path.dirname(__file__), "golden", "fp8_e4m3_values.txt")
    for line in open(path):
        if line.startswith("#") or not line.strip():
            continue
        code, val = line.split()
        got = oracle.fp8_e4m3_value(int(code, 16))
        want = float(val)
        assert (np.isnan(got) and np.isnan(want)) or got == want, (code, got, want)


def test_fp8_e4m3_encode_is_e4m3fn_rounding_saturated_at_240():
    """Below 248 in magnitude the nearest-even e4m3 code is torch's e4m3fn cast (the two formats
    share every code up to 240 and 248 is the midpoint to the next e4m3fn value); from 248 up the
    encode saturates to +-240; NaN stays NaN."""
    import torch
    table = np.array([oracle.fp8_e4m3_value(c) for c in range(0x78)])
    mids = (table[:-1] + table[1:]) / 2
    xs = np.concatenate([table, mids, -table, -mids, [240.5, 247.99, 1e-4, 3e-3, -7e-4]]).astype(np.float32)
    ref = torch.from_numpy(xs).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.fp8_e4m3_encode(float(x)) for x in xs], np.uint8)
    assert np.array_equal(got, ref)
    for x in (248.0, 250.0, 448.0, 1e4, np.inf):
        assert oracle.fp8_e4m3_encode(x) == 0x77 and oracle.fp8_e4m3_encode(-x) == 0xF7
    assert oracle.fp8_e4m3_encode(float("nan")) == 0x7F


def test_fp8_e4m3_pool_matches_dense_bruteforce():
    """Decode over an IEEE-style e4m3 pool against the textbook softmax on the flattened cache."""
    w = small(kv_dtype="fp8e4m3", q_dtype="bf16", page_order="shuffled", seq_lens=[7, 1, 13])
    out, lse = run_oracle(w)
    G = w.H_qo // w.H_kv
    q64 = to_f64(w.q, w.q_dtype)
    for b in range(w.B):
        for hq in range(w.H_qo):
            K, V = contiguous_kv(w, b, hq // G)
            o, l = dense_attention(q64[b, hq], K, V, w.sm_scale)
            np.testing.assert_allclose(out[b, hq], o, rtol=0, atol=1e-12)
            assert abs(lse[b, hq] - l) < 1e-12


# ---- OCP e5m2 (bias 15, max 57344)

def _golden(name):
    path = os.path.join(os.path.dirname(__file__), "golden", name)
    for line in open(path):
        line = line.split("#")[0].strip()
        if line:
            code, val = line.split()
            yield int(code, 16), (float.fromhex(val) if "p" in val else float(val))


def test_fp8_e5m2_values_definition_and_library():
    """The fixture's closed-form values, then every code against torch's float8_e5m2 view."""
    import torch
    n = 0
    for code, want in _golden("fp8_e5m2_values.txt"):
        got = oracle.fp8_e5m2_value(code)
        assert (np.isnan(got) and np.isnan(want)) or (got == want and
                                                    np.signbit(got) == np.signbit(want)), hex(code)
        n += 1
    assert n >= 12
    lib = torch.arange(256, dtype=torch.uint8).view(torch.float8_e5m2).to(torch.float64).numpy()
    ours = np.array([oracle.fp8_e5m2_value(c) for c in range(256)])
    assert ((lib == ours) | (np.isnan(lib) & np.isnan(ours))).all()
    # table shape: strictly increasing over the 124 non-negative finite codes, 4 codes a binade
    pos = ours[:0x7C]
    assert np.all(np.diff(pos) > 0) and np.sum(np.isfinite(ours)) == 248
    for e in range(1, 31):
        steps = np.diff(pos[4 * e:4 * e + 4])
        assert np.all(steps == steps[0])


def test_fp8_e5m2_encode_roundtrip_ties_saturation_and_library():
    """Every finite code round-trips; midpoints go to the even code; torch's nearest-even cast
    agrees inside the range; from 57344 up (infinity included) the encode saturates; NaN stays
    NaN."""
    import torch
    vals = [oracle.fp8_e5m2_value(c) for c in range(256)]
    for c in range(256):
        if np.isfinite(vals[c]):
            assert oracle.fp8_e5m2_encode(vals[c]) == c, hex(c)
    for c in range(0, 0x7B):
        mid = (vals[c] + vals[c + 1]) / 2
        if np.float32(mid) == mid:
            assert oracle.fp8_e5m2_encode(mid) == (c if c % 2 == 0 else c + 1), hex(c)
    rng = np.random.default_rng(15)
    x = np.concatenate([rng.standard_normal(3000) * 300, rng.standard_normal(1000) * 1e-4,
                        rng.uniform(-57344, 57344, 1000)]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e5m2).view(torch.uint8).numpy()
    got = np.array([oracle.fp8_e5m2_encode(float(v)) for v in x], np.uint8)
    assert np.array_equal(got, ref)
    for big in (57344.0, 60000.0, 61439.0, 1e6, np.inf):
        assert oracle.fp8_e5m2_encode(big) == 0x7B and oracle.fp8_e5m2_encode(-big) == 0xFB
    nan = oracle.fp8_e5m2_encode(float("nan"))
    assert (nan & 0x7C) == 0x7C and (nan & 3) != 0


@pytest.mark.parametrize("page_scales", [False, True])
@pytest.mark.parametrize("window", [None, 5])
def test_fp8_e5m2_pool_matches_dense_bruteforce(page_scales, window):
    """Decode over an e5m2 pool (per-KV-head or per-page scales, with and without a window)
    against the textbook softmax on the flattened cache, decoded through torch's e5m2 view."""
    w = small(kv_dtype="fp8e5m2", q_dtype="bf16", page_order="shuffled", seq_lens=[7, 1, 13],
              page_scales=page_scales, window=window, sink=2 if window else 0)
    out, lse = run_oracle(w)
    G = w.H_qo // w.H_kv
    q64 = to_f64(w.q, w.q_dtype)
    for b in range(w.B):
        for hq in range(w.H_qo):
            K, V = contiguous_kv(w, b, hq // G)
            if window:
                off, sink = int(w.length_info[1, b]), int(w.length_info[2, b])
                rows = np.r_[0:sink, off:int(w.seq_lens[b])]
                K, V = K[rows], V[rows]
            o, l = dense_attention(q64[b, hq], K, V, w.sm_scale)
            np.testing.assert_allclose(out[b, hq], o, rtol=0, atol=1e-12)
            assert abs(lse[b, hq] - l) < 1e-12


def test_append_e5m2_matches_library_quantization():
    """Append into an e5m2 pool: x / scale in fp32, saturated to +-57344, then torch's
    nearest-even e5m2 cast."""
    import torch
    H_kv, D, ps, P = 2, 16, 8, 6
    pool = synth.poisoned_pool(P, H_kv, ps, D, "fp8e5m2")
    k, v, slots = synth.append_inputs(T=7, H_kv=H_kv, D=D, page_size=ps, max_num_pages=P,
                                      in_dtype="bf16", seed=18, skip_every=3)
    ks = np.array([0.5 / 448, 1e-5], np.float32)  # the second drives values past 57344
    vs = np.array([1.0 / 448, 0.75 / 448], np.float32)
    before = pool.copy()
    oracle.append_kv(pages=pool, new_k=k, new_v=v, slots=slots, H_kv=H_kv, D=D, ps=ps,
                     in_dtype=1, kv_dtype=4, k_scale=ks, v_scale=vs)
    kf = to_f64(k, "bf16").astype(np.float32)
    vf = to_f64(v, "bf16").astype(np.float32)
    expect = before.copy()
    saturated = 0
    for t, s in enumerate(slots):
        if s < 0:
            continue
        for kv, x, sc in ((0, kf, ks), (1, vf, vs)):
            y = x[t] / sc[:, None]
            saturated += int((np.abs(y) >= 57344).sum())
            y = np.clip(y, -57344, 57344)
            expect[s // ps, kv, :, s % ps, :] = (torch.from_numpy(np.ascontiguousarray(y))
                                                 .to(torch.float8_e5m2).view(torch.uint8).numpy())
    assert saturated > 0
    assert expect.tobytes() == pool.tobytes()


# ---------------------------------------------------------------- fp8 pools with per-page scales
# A scale per (page, KV head) block, in place of one per KV head: a stored value is still code x
# scale, with the scale of the block that holds the row.
@pytest.mark.parametrize("kv_dtype", ["fp8", "fp8e4m3"])
@pytest.mark.parametrize("window", [None, 5])
def test_page_scales_match_dense_bruteforce(kv_dtype, window):
    """Paged oracle == textbook attention over the flattened cache, each row dequantised with its
    own page's scale (sequences span pages of different scales; with a window and a sink the
    attended rows skip pages)."""
    w = small(kv_dtype=kv_dtype, q_dtype="bf16", page_scales=True, seq_lens=[7, 1, 13],
              window=window, sink=2 if window else 0)
    out, lse = run_oracle(w)
    G = w.H_qo // w.H_kv
    q64 = to_f64(w.q, w.q_dtype)
    for b in range(w.B):
        for hq in range(w.H_qo):
            K, V = contiguous_kv(w, b, hq // G)
            if window:
                off, sink = int(w.length_info[1, b]), int(w.length_info[2, b])
                rows = np.r_[0:sink, off:int(w.seq_lens[b])]
                K, V = K[rows], V[rows]
            o, l = dense_attention(q64[b, hq], K, V, w.sm_scale)
            np.testing.assert_allclose(out[b, hq], o, rtol=0, atol=1e-12)
            assert abs(lse[b, hq] - l) < 1e-12


def test_page_scales_equal_to_head_scales_are_per_head():
    """Every page given its KV head's scale: exactly the per-head result; random page scales
    change it."""
    w = small(kv_dtype="fp8", q_dtype="bf16", page_scales=True, seq_lens=[9, 4, 13])
    ksp = np.ascontiguousarray(np.broadcast_to(w.k_scale, w.k_scale_page.shape))
    vsp = np.ascontiguousarray(np.broadcast_to(w.v_scale, w.v_scale_page.shape))
    o_e, l_e = run_oracle(w, k_scale_page=ksp, v_scale_page=vsp)
    o_h, l_h = run_oracle(w, k_scale_page=None, v_scale_page=None)
    assert np.array_equal(o_e, o_h) and np.array_equal(l_e, l_h)
    o_p, _ = run_oracle(w)
    assert np.abs(o_p - o_h).max() > 1e-3


def test_page_v_scales_doubled_double_out():
    """Every page's V scale times 2 (exact in fp32 and fp64): out doubles exactly, lse stays."""
    w = small(kv_dtype="fp8", q_dtype="bf16", page_scales=True, seq_lens=[9, 4, 13])
    o1, l1 = run_oracle(w)
    o2, l2 = run_oracle(w, v_scale_page=w.v_scale_page * np.float32(2))
    assert np.array_equal(o2, 2 * o1) and np.array_equal(l1, l2)


def test_append_with_page_scales_matches_library_quantization():
    """Append into an fp8 pool with per-page scales: each element is x / (its slot's page scale)
    in fp32, encoded by torch's e4m3fn conversion (inputs kept inside +-448)."""
    import torch
    H_kv, D, ps, P = 2, 16, 8, 6
    pool = synth.poisoned_pool(P, H_kv, ps, D, "fp8")
    k, v, slots = synth.append_inputs(T=11, H_kv=H_kv, D=D, page_size=ps, max_num_pages=P,
                                      in_dtype="bf16", seed=9, skip_every=4)
    rng = np.random.default_rng(90)
    ksp = rng.uniform(1.0 / 112, 2.0 / 112, size=(P, H_kv)).astype(np.float32)
    vsp = rng.uniform(1.0 / 112, 2.0 / 112, size=(P, H_kv)).astype(np.float32)
    before = pool.copy()
    oracle.append_kv(pages=pool, new_k=k, new_v=v, slots=slots, H_kv=H_kv, D=D, ps=ps,
                     in_dtype=1, kv_dtype=2, k_scale_page=ksp, v_scale_page=vsp)
    kf = to_f64(k, "bf16").astype(np.float32)
    vf = to_f64(v, "bf16").astype(np.float32)
    expect = before.copy()
    for t, s in enumerate(slots):
        if s < 0:
            continue
        page = s // ps
        for kv, x, sc in ((0, kf, ksp), (1, vf, vsp)):
            y = x[t] / sc[page][:, None]
            assert np.abs(y).max() <= 448
            expect[page, kv, :, s % ps, :] = (torch.from_numpy(np.ascontiguousarray(y))
                                              .to(torch.float8_e4m3fn).view(torch.uint8).numpy())
    assert expect.tobytes() == pool.tobytes()


# ---------------------------------------------------------------- fp8 q
# q stored as e4m3fn codes with a scale per q head: q = code x q_scale[h_qo], read as the pool's
# codes are.
@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_fp8_q_matches_dense_bruteforce(kv_dtype):
    """fp8 q (codes x per-q-head scales) == textbook attention with the dequantised q."""
    w = small(kv_dtype=kv_dtype, q_dtype="fp8", seq_lens=[7, 1, 13])
    out, lse = run_oracle(w)
    G = w.H_qo // w.H_kv
    q64 = to_f64(w.q, "fp8") * w.q_scale.astype(np.float64)[None, :, None]
    for b in range(w.B):
        for hq in range(w.H_qo):
            K, V = contiguous_kv(w, b, hq // G)
            o, l = dense_attention(q64[b, hq], K, V, w.sm_scale)
            np.testing.assert_allclose(out[b, hq], o, rtol=0, atol=1e-12)
            assert abs(lse[b, hq] - l) < 1e-12


def test_fp8_q_with_power_of_two_scales_is_the_bf16_query():
    """Scales that are powers of two make every dequantised q element a bf16 value: the fp8-q
    result then equals the bf16-q result on those values exactly."""
    w = small(kv_dtype="fp8", q_dtype="fp8", seq_lens=[9, 4, 13])
    qs = np.float32(2.0) ** np.arange(-8, -8 + w.H_qo, dtype=np.float32)
    o8, l8 = run_oracle(w, q_scale=qs)
    qv = to_f64(w.q, "fp8") * qs.astype(np.float64)[None, :, None]
    qb = synth.cast_f32(qv.astype(np.float32), "bf16")
    assert np.array_equal(to_f64(qb, "bf16"), qv)  # exact in bf16
    ob, lb = run_oracle(w, q_dtype=1, q=qb, q_scale=None)
    assert np.array_equal(o8, ob) and np.array_equal(l8, lb)
