"""GPU parity: libpdecode (HIP, through the C ABI) against the oracle on the same seeded inputs.

Tolerances (stated for this path): fp32 KV |d out| <= 1e-5 and |d lse| <= 1e-5; bf16 KV and fp8
KV after dequantisation |d out| <= 2e-2 absolute and |d lse| <= 1e-3. Page gathers and append
placement are bit-exact. Unused pool pages are NaN-poisoned, so a stray gather shows as NaN.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_decode_08_amd as pk
    pk.lib()
    yield


def check(w, out, lse, select=None, label=""):
    """Compares GPU out/lse with the oracle (all pairs, or the selected (b, h_qo) pairs): the
    stated bounds, and for bf16 / fp8 KV also the per-row relative bound of gpu_util.row_error."""
    tol_o, tol_l = gu.tolerance(w)
    o_gpu = gu.to_np64(out)
    l_gpu = gu.to_np64(lse)
    assert np.all(np.isfinite(o_gpu)) and np.all(np.isfinite(l_gpu)), f"{label}: non-finite output"
    if select is None:
        o_ref, l_ref = oracle.decode(**w.oracle_kwargs())
        og, lg = o_gpu, l_gpu
    else:
        o_ref, l_ref = oracle.decode(**w.oracle_kwargs(), select=select)
        og = o_gpu[select[:, 0], select[:, 1]]
        lg = l_gpu[select[:, 0], select[:, 1]]
    do, ratio = gu.row_error(w, o_ref, og)
    dl = np.abs(lg - l_ref).max(initial=0)
    print(f"{label}: max|dout|={do:.3g} max|dlse|={dl:.3g} worst row ratio={ratio:.3g}", flush=True)
    assert do <= tol_o, f"{label}: |dout| {do} > {tol_o}"
    assert dl <= tol_l, f"{label}: |dlse| {dl} > {tol_l}"
    if w.kv_dtype != "f32":
        assert ratio <= 1.0, f"{label}: per-row relative error ratio {ratio} > 1"


def assert_close(w, o_ref, l_ref, o_gpu, l_gpu, label):
    """The checks of check() on arrays already in hand (any [..., D] / [...] layout)."""
    tol_o, tol_l = gu.tolerance(w)
    assert np.all(np.isfinite(o_gpu)) and np.all(np.isfinite(l_gpu)), f"{label}: non-finite output"
    do, ratio = gu.row_error(w, o_ref, o_gpu)
    dl = np.abs(np.asarray(l_gpu) - np.asarray(l_ref)).max(initial=0)
    print(f"{label}: max|dout|={do:.3g} max|dlse|={dl:.3g} worst row ratio={ratio:.3g}", flush=True)
    assert do <= tol_o and dl <= tol_l, (label, do, dl)
    if w.kv_dtype != "f32":
        assert ratio <= 1.0, f"{label}: per-row relative error ratio {ratio} > 1"


def run_and_check(w, **kw):
    dev = gu.upload(w)
    out, lse = gu.run_attention(w, dev, **kw)
    torch.cuda.synchronize()
    check(w, out, lse, label=w.name)
    return dev, out, lse


# ------------------------------------------------------------------ small cases, all outputs
def test_tiny_fp32_config():
    """The tiny fp32 workload: B=4, 4/4 heads, D=64, page 16, lengths {1,17,33,50}, pool 16."""
    run_and_check(synth.tiny_fp32())


@pytest.mark.parametrize("G", [1, 2, 3, 4, 5, 8])
@pytest.mark.parametrize("kv", ["f32", "bf16", "fp8"])
def test_group_sizes_and_dtypes(G, kv):
    qd = "f32" if kv == "f32" else "bf16"
    lens = [1, 15, 16, 17, 100, 257, 0, 33]
    w = synth.make_workload(name=f"G{G}_{kv}", B=len(lens), H_qo=2 * G, H_kv=2, D=128,
                            page_size=16 if kv != "fp8" else 32, seq_lens=lens, q_dtype=qd,
                            kv_dtype=kv, seed=100 + G, max_num_pages=64)
    run_and_check(w)


@pytest.mark.parametrize("D,ps", [(64, 16), (64, 32), (128, 16), (128, 32)])
@pytest.mark.parametrize("kv", ["f32", "bf16", "fp8"])
def test_head_dims_and_page_sizes(D, ps, kv):
    qd = "f32" if kv == "f32" else "bf16"
    lens = [3, 64, 130, 31, 1]
    w = synth.make_workload(name=f"D{D}_ps{ps}_{kv}", B=5, H_qo=8, H_kv=2, D=D, page_size=ps,
                            seq_lens=lens, q_dtype=qd, kv_dtype=kv, seed=7 + D + ps,
                            max_num_pages=32)
    run_and_check(w)


@pytest.mark.parametrize("splits", [0, 1, 2, 3, 7, 8, 9, 64])
def test_forced_splits(splits):
    """Split-KV chunking (any chunk count, ragged last chunk, more chunks than pages)."""
    lens = [1000, 17, 0, 513, 2048, 1]
    w = synth.make_workload(name=f"splits{splits}", B=6, H_qo=16, H_kv=4, D=128, page_size=16,
                            seq_lens=lens, seed=31, max_num_pages=400)
    run_and_check(w, num_kv_splits=splits)


def test_max_len_hint_too_small_is_still_exact():
    """max_kv_len only sizes the grid: a hint far below the real lengths still gives exact
    results (the last chunk takes the rest)."""
    lens = [700, 1200, 64]
    w = synth.make_workload(name="hint_small", B=3, H_qo=8, H_kv=2, D=128, page_size=16,
                            seq_lens=lens, seed=32, max_num_pages=200)
    run_and_check(w, max_kv_len=100)
    run_and_check(w, max_kv_len=1)


@pytest.mark.parametrize("sink,window", [(4, 64), (0, 50), (3, 1000), (16, 40), (5, 5)])
def test_sliding_window_and_sink(sink, window):
    lens = [300, 70, 16, 5, 0, 129]
    w = synth.make_workload(name=f"swa_s{sink}_w{window}", B=6, H_qo=8, H_kv=2, D=128,
                            page_size=16, seq_lens=lens, seed=41, max_num_pages=64,
                            window=window, sink=sink)
    run_and_check(w)
    run_and_check(w, num_kv_splits=3)


def test_rope_small():
    lens = [300, 70, 16, 1, 129]
    w = synth.make_workload(name="rope", B=5, H_qo=8, H_kv=2, D=128, page_size=16,
                            seq_lens=lens, seed=51, max_num_pages=64, rotary_mode=1,
                            rope_theta=500000.0)
    run_and_check(w)


def test_rope_window_large_positions():
    """RoPE with sink + window at positions up to ~16k (the angle must be computed accurately)."""
    lens = [16384, 9000, 4200]
    w = synth.make_workload(name="rope_swa_pos", B=3, H_qo=8, H_kv=2, D=128, page_size=16,
                            seq_lens=lens, seed=52, max_num_pages=2048, rotary_mode=1,
                            rope_theta=500000.0, window=4096, sink=4)
    run_and_check(w)
    w2 = synth.make_workload(name="rope_scale", B=3, H_qo=4, H_kv=1, D=64, page_size=32,
                             seq_lens=lens, seed=53, max_num_pages=2048, rotary_mode=1,
                             rope_theta=10000.0, rope_scale=0.25, window=2048, sink=0)
    run_and_check(w2)


@pytest.mark.parametrize("D,ps", [(64, 16), (64, 32), (128, 16), (128, 32)])
@pytest.mark.parametrize("splits", [0, 7])
def test_rope_fp32_kv(D, ps, splits):
    """fp32 q and KV with rotate-half RoPE (the vector-ALU kernel, whose cos/sin advance along the
    rows by a recurrence and are recomputed exactly every few pages), base 5e5: a window of 4096
    with sink 4, and keys placed from position 120 000 so that positions reach ~131 000, plus a
    sequence without a window; the fp32 bounds (1e-5 / 1e-5)."""
    lens = np.array([11000, 5000, 300, 1, 9000])
    off = np.full(5, 120000, np.int32)
    for window in (4096, None):
        att = np.minimum(lens, 4100) if window else lens
        w = synth.make_workload(name=f"rope_f32_D{D}_ps{ps}_w{window}", B=5, H_qo=4, H_kv=2, D=D,
                                page_size=ps, seq_lens=lens, q_dtype="f32", kv_dtype="f32",
                                seed=60 + D + ps, max_num_pages=2200, rotary_mode=1,
                                rope_theta=500000.0, window=window, sink=4,
                                k_rope_pos_offset=off,
                                q_rope_position=(off + att - 1).astype(np.int32))
        run_and_check(w, num_kv_splits=splits)


@pytest.mark.parametrize("kv,rot", [("bf16", 1), ("bf16", 2), ("fp8", 1), ("fp8", 2)])
def test_rope_large_positions_matrix_cores(kv, rot):
    """RoPE on the matrix-core kernels at positions up to ~131 000 (keys from 120 000, window
    4096 + sink 4, base 5e5), both layouts: the angle of a large position keeps its accuracy."""
    lens = np.array([11000, 5000, 300, 1, 9000])
    off = np.full(5, 120000, np.int32)
    att = np.minimum(lens, 4100)
    ps = 16 if kv == "bf16" else 32
    w = synth.make_workload(name=f"rope_big_{kv}_{rot}", B=5, H_qo=8, H_kv=2, D=128,
                            page_size=ps, seq_lens=lens, kv_dtype=kv, seed=66 + rot,
                            max_num_pages=2200, rotary_mode=rot, rope_theta=500000.0,
                            window=4096, sink=4, k_rope_pos_offset=off,
                            q_rope_position=(off + att - 1).astype(np.int32))
    run_and_check(w)
    run_and_check(w, num_kv_splits=6)


def test_empty_window():
    """Pages but an empty window and no sink: out = 0, lse = -5e4."""
    w = synth.make_workload(name="empty_win", B=3, H_qo=4, H_kv=2, D=64, page_size=16,
                            seq_lens=[5, 40, 0], seed=3, max_num_pages=16, window=4, sink=0)
    w.length_info[1] = w.seq_lens  # window starts at the end
    w.attended[:] = 0
    dev, out, lse = run_and_check(w)
    assert np.all(gu.to_np64(out) == 0) and np.all(gu.to_np64(lse) == -5e4)


def test_all_empty_batch():
    w = synth.make_workload(name="all_empty", B=4, H_qo=4, H_kv=4, D=64, page_size=16,
                            seq_lens=[0, 0, 0, 0], seed=3, max_num_pages=4, q_dtype="f32",
                            kv_dtype="f32")
    dev, out, lse = run_and_check(w)
    assert np.all(gu.to_np64(lse) == -5e4)


# ------------------------------------------------------------------ properties on the GPU
def test_deterministic_and_permutation_invariant():
    """Two runs are bit-identical; relabelling the physical pages (moving the data) leaves the
    GPU output bit-identical (the gather follows the table exactly)."""
    w = synth.llama3_8b_bf16(B=4, lens=[600, 1000, 37, 2100])
    dev = gu.upload(w)
    o1, l1 = gu.run_attention(w, dev)
    o2, l2 = gu.run_attention(w, dev)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
    perm = np.random.default_rng(9).permutation(w.max_num_pages).astype(np.int32)
    pool = np.empty_like(w.pages)
    pool[perm] = w.pages
    w2 = synth.Workload(**{**w.__dict__, "pages": pool, "page_values": perm[w.page_values]})
    dev2 = gu.upload(w2)
    o3, l3 = gu.run_attention(w2, dev2)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o3.view(torch.int16)) and torch.equal(l1, l3)


def test_split_equals_unsplit_long():
    """Long context (a scaled-down long-context split case): auto split vs. no split agree
    within the bf16 tolerance, and both match the oracle."""
    w = synth.make_workload(name="long_small", B=2, H_qo=32, H_kv=8, D=128, page_size=16,
                            seq_lens=[8192, 20000], seed=1003, max_num_pages=2048)
    dev = gu.upload(w)
    oa, la = gu.run_attention(w, dev, num_kv_splits=0)
    o1, l1 = gu.run_attention(w, dev, num_kv_splits=1)
    torch.cuda.synchronize()
    check(w, oa, la, label="auto split")
    check(w, o1, l1, label="no split")
    assert np.abs(gu.to_np64(oa) - gu.to_np64(o1)).max() <= 2e-2
    assert np.abs(gu.to_np64(la) - gu.to_np64(l1)).max() <= 1e-3


# ------------------------------------------------------------------ merge and append
@pytest.mark.parametrize("vd", ["f32", "bf16"])
def test_merge_state_inplace(vd):
    import paged_kv_decode_08_amd as pk
    rng = np.random.default_rng(4)
    n, H, D = 7, 5, 96
    v = rng.standard_normal((n, H, D)).astype(np.float32)
    vo = rng.standard_normal((n, H, D)).astype(np.float32)
    s = (rng.standard_normal((n, H)) * 8).astype(np.float32)
    so = (rng.standard_normal((n, H)) * 8).astype(np.float32)
    s[0, 0] = so[0, 0] = -5e4  # two empty states
    if vd == "bf16":
        v = synth.cast_f32(v, "bf16")
        vo = synth.cast_f32(vo, "bf16")
    tv = gu.to_device_storage(v, vd)
    tvo = gu.to_device_storage(vo, vd)
    ts = torch.from_numpy(s).cuda()
    tso = torch.from_numpy(so).cuda()
    pk.merge_state_inplace(tv, ts, tvo, tso)
    torch.cuda.synchronize()
    from tests.dense_ref import to_f64
    ref_v, ref_s = oracle.merge_state(to_f64(v, vd), s, to_f64(vo, vd), so)
    tol = 1e-5 if vd == "f32" else 2e-2
    assert np.abs(gu.to_np64(tv) - ref_v).max() <= tol
    assert np.abs(gu.to_np64(ts) - ref_s).max() <= 1e-5 * max(1, np.abs(ref_s).max())


def test_merge_two_halves_equals_whole_on_gpu():
    """Attention over rows [0, k) and over [k, L) (a window with sink 0 starting at k), merged by
    pdecode_merge_state_inplace, equals attention over [0, L)."""
    import paged_kv_decode_08_amd as pk
    L, k = 1000, 421
    w = synth.make_workload(name="whole", B=1, H_qo=8, H_kv=2, D=128, page_size=16,
                            seq_lens=[L], seed=61, max_num_pages=128)
    dev = gu.upload(w)
    ow, lw = gu.run_attention(w, dev)
    np_pre = (k + 15) // 16
    pre = synth.Workload(**{**w.__dict__, "page_indptr": np.array([0, np_pre], np.int32),
                            "length_info": np.array([k - (np_pre - 1) * 16], np.int32),
                            "attended": np.array([k], np.int32)})
    suf = synth.Workload(**{**w.__dict__, "sliding_window": True,
                            "length_info": np.array([[w.length_info[0]], [k], [0]], np.int32),
                            "attended": np.array([L - k], np.int32)})
    o1, l1 = gu.run_attention(pre, gu.upload(pre))
    o2, l2 = gu.run_attention(suf, gu.upload(suf))
    pk.merge_state_inplace(o1, l1, o2, l2)
    torch.cuda.synchronize()
    assert np.abs(gu.to_np64(o1) - gu.to_np64(ow)).max() <= 2e-2
    assert np.abs(gu.to_np64(l1) - gu.to_np64(lw)).max() <= 1e-3
    check(w, o1, l1, label="merged halves")


@pytest.mark.parametrize("D", [128, 36])
@pytest.mark.parametrize("kv", ["f32", "bf16", "fp8"])
def test_append_bitexact(kv, D):
    """Placement and encoding are bit-exact. D = 128 takes the 16-byte vector form for every
    dtype; D = 36 (rows of 72 bf16 bytes, 36 fp8 bytes) the element form, fp32 still vectors."""
    import paged_kv_decode_08_amd as pk
    ind = "f32" if kv == "f32" else "bf16"
    H_kv, ps, P = 8, 16 if kv != "fp8" else 32, 64
    pool = synth.poisoned_pool(P, H_kv, ps, D, kv)
    k, v, slots = synth.append_inputs(T=40, H_kv=H_kv, D=D, page_size=ps, max_num_pages=P,
                                      in_dtype=ind, seed=12, skip_every=5)
    slots[1] = P * ps + 3  # past the pool: skipped
    ks = vs = None
    if kv == "fp8":
        ks = np.random.default_rng(1).uniform(0.5 / 448, 2 / 448, H_kv).astype(np.float32)
        vs = np.random.default_rng(2).uniform(0.5 / 448, 2 / 448, H_kv).astype(np.float32)
        k = synth.cast_f32(np.random.default_rng(3).standard_normal(k.shape).astype(np.float32) * 0.6, "bf16")
    tks = None if ks is None else torch.from_numpy(ks).cuda()
    tvs = None if vs is None else torch.from_numpy(vs).cuda()
    desc = pk.make_desc(batch=1, num_qo_heads=H_kv, num_kv_heads=H_kv, head_dim=D, page_size=ps,
                        max_num_pages=P, q_dtype=ind, kv_dtype=kv, k_scale=tks, v_scale=tvs)
    tpool = gu.to_device_storage(pool, kv)
    pk.append_kv(desc, gu.to_device_storage(k, ind), gu.to_device_storage(v, ind),
                 torch.from_numpy(slots).cuda(), tpool)
    torch.cuda.synchronize()
    slots_o = slots.copy()
    slots_o[1] = -1
    ref = oracle.append_kv(pages=pool.copy(), new_k=k, new_v=v, slots=slots_o, H_kv=H_kv, D=D,
                           ps=ps, in_dtype=synth.DTYPE_CODE[ind], kv_dtype=synth.DTYPE_CODE[kv],
                           k_scale=ks, v_scale=vs)
    got = tpool.cpu()
    got = got.view(torch.int16).numpy().view(np.uint16) if kv == "bf16" else got.numpy()
    assert got.tobytes() == ref.tobytes()


def test_append_fp8_rounding_exhaustive():
    """Every e4m3fn code's value, the midpoints between neighbours (ties to even), values beyond
    448 (saturation) and tiny values, quantised by the GPU append, match the oracle's encoder."""
    import paged_kv_decode_08_amd as pk
    table = np.array([oracle.fp8_value(c) for c in range(0x7F)])
    mids = (table[:-1] + table[1:]) / 2
    xs = np.concatenate([table, mids, -table, -mids, [500.0, 1e4, -1e4, 448.5, 463.9, 464.0,
                                                      1e-4, 2e-3, -3e-3]]).astype(np.float32)
    D, H_kv, ps = 64, 1, 16
    T = (xs.size + D - 1) // D
    x = np.zeros(T * D, np.float32)
    x[:xs.size] = xs
    x = x.reshape(T, 1, D)
    ks = np.array([1.0], np.float32)
    P = (T + ps - 1) // ps
    pool = synth.poisoned_pool(P, H_kv, ps, D, "fp8")
    slots = np.arange(T, dtype=np.int32)
    desc = pk.make_desc(batch=1, num_qo_heads=1, num_kv_heads=1, head_dim=D, page_size=ps,
                        max_num_pages=P, q_dtype="f32", kv_dtype="fp8",
                        k_scale=torch.from_numpy(ks).cuda(), v_scale=torch.from_numpy(ks).cuda())
    # The public supported set pairs fp8 KV with bf16 q; fp32 input is used here only to feed
    # exact fp32 values to the quantiser.
    tpool = torch.from_numpy(pool).cuda()
    # keep every device tensor referenced until the asynchronous kernel has run
    tx = torch.from_numpy(x).cuda()
    tslots = torch.from_numpy(slots).cuda()
    st = pk.lib().pdecode_append_kv(
        __import__("ctypes").byref(desc), pk._ptr(tx), pk._ptr(tx), pk._ptr(tslots), T,
        pk._ptr(tpool), pk._stream(None))
    if st == 2:
        pytest.skip("fp32 -> fp8 append outside the supported set")
    assert st == 0
    torch.cuda.synchronize()
    got = tpool.cpu().numpy()[:, 0, 0].reshape(-1)[:T * D].reshape(T, D)
    ref = oracle.append_kv(pages=pool.copy(), new_k=x, new_v=x, slots=slots, H_kv=1, D=D, ps=ps,
                           in_dtype=0, kv_dtype=2, k_scale=ks, v_scale=ks)
    assert got.tobytes() == ref[:, 0, 0].reshape(-1)[:T * D].reshape(T, D).tobytes()


def test_append_then_decode():
    """Append one token per sequence into its next slot, then decode: matches the oracle run on
    the oracle's own appended pool."""
    import paged_kv_decode_08_amd as pk
    w = synth.make_workload(name="append_decode", B=4, H_qo=8, H_kv=2, D=128, page_size=16,
                            seq_lens=[31, 32, 1, 100], seed=71, max_num_pages=64)
    # slot of the next token of each sequence: its last page when not full, else a fresh page
    free = sorted(set(range(w.max_num_pages)) - set(w.page_values.tolist()))
    slots, new_vals, new_indptr, new_last = [], [], [0], []
    for b in range(w.B):
        pages = list(w.page_values[w.page_indptr[b]:w.page_indptr[b + 1]])
        last = int(w.length_info[b])
        if last == 16:
            pages.append(free.pop(0))
            last = 0
        slots.append(pages[-1] * 16 + last)
        new_vals += pages
        new_indptr.append(len(new_vals))
        new_last.append(last + 1)
    slots = np.array(slots, np.int32)
    k, v, _ = synth.append_inputs(T=w.B, H_kv=w.H_kv, D=w.D, page_size=16,
                                  max_num_pages=w.max_num_pages, in_dtype="bf16", seed=72,
                                  slots=slots)
    dev = gu.upload(w)
    desc = gu.desc_for(w, dev)
    pk.append_kv(desc, gu.to_device_storage(k, "bf16"), gu.to_device_storage(v, "bf16"),
                 torch.from_numpy(slots).cuda(), dev["pages"])
    pool_ref = oracle.append_kv(pages=w.pages.copy(), new_k=k, new_v=v, slots=slots,
                                H_kv=w.H_kv, D=w.D, ps=16, in_dtype=1, kv_dtype=1)
    w2 = synth.Workload(**{**w.__dict__, "pages": pool_ref,
                           "page_values": np.array(new_vals, np.int32),
                           "page_indptr": np.array(new_indptr, np.int32),
                           "length_info": np.array(new_last, np.int32),
                           "seq_lens": w.seq_lens + 1, "attended": w.attended + 1})
    dev["values"] = torch.from_numpy(w2.page_values).cuda()
    dev["indptr"] = torch.from_numpy(w2.page_indptr).cuda()
    dev["length_info"] = torch.from_numpy(w2.length_info).cuda()
    out, lse = gu.run_attention(w2, dev)
    torch.cuda.synchronize()
    check(w2, out, lse, label="append+decode")


# ------------------------------------------------------------------ full-size workloads, every output
@pytest.mark.parametrize("name", ["tiny_fp32", "llama3_8b_bf16", "long_ctx_bf16", "rope_swa_bf16",
                                  "fp8_gqa8", "gqa8_bf16"])
def test_full_size_config(name):
    """The five workloads, and the bf16 GQA-8 layer at the Llama-3-8B lengths (one job per
    workgroup, split sequences merged in the kernel), at full size in the benchmark's launch
    configuration (automatic split plan): every output against the oracle, with the stated bounds
    and the per-row relative one; every output finite."""
    w = synth.CONFIGS[name]()
    print(f"{name}: B={w.B} kv_bytes={w.kv_bytes}", flush=True)
    dev = gu.upload(w)
    out, lse = gu.run_attention(w, dev)
    torch.cuda.synchronize()
    check(w, out, lse, label=name)
    if name == "long_ctx_bf16":
        o1, l1 = gu.run_attention(w, dev, num_kv_splits=1)
        torch.cuda.synchronize()
        assert np.abs(gu.to_np64(out) - gu.to_np64(o1)).max() <= 2e-2
        assert np.abs(gu.to_np64(lse) - gu.to_np64(l1)).max() <= 1e-3


@pytest.mark.parametrize("name", ["llama3_8b_bf16", "fp8_gqa8"])
def test_no_length_hint(name):
    """max_kv_len = 0 (no length hint): the persistent schedule sizes its chunks on the device from
    the call's lengths, so the call is bit-identical to the one with a tight hint (and as fast);
    every output against the oracle."""
    w = synth.CONFIGS[name]()
    dev = gu.upload(w)
    out0, lse0 = gu.run_attention(w, dev, max_kv_len=0)
    out1, lse1 = gu.run_attention(w, dev)
    torch.cuda.synchronize()
    assert torch.equal(out0.view(torch.uint8), out1.view(torch.uint8))
    assert torch.equal(lse0, lse1)
    if name == "llama3_8b_bf16":
        check(w, out0, lse0, label=name + " no hint")


def test_fp8_unit_sigma():
    """fp8 KV whose dequantised K and V have sigma near 1 (scales ~ U[0.9, 1.1] / 112 on payloads
    drawn as N(0, 1) * 112): outputs and scores of the size the bf16 workloads have, at the fp8
    GQA-8 shape (64 q / 8 KV heads, page 32, lognormal lengths), every output."""
    z = np.random.default_rng(77).standard_normal(48)
    lens = np.minimum(8192, np.maximum(1, np.rint(2048.0 * np.exp(0.5 * z)))).astype(np.int64)
    w = synth.make_workload(name="fp8_unit_sigma", B=48, H_qo=64, H_kv=8, D=128, page_size=32,
                            seq_lens=lens, max_num_pages=8192, kv_dtype="fp8", seed=78,
                            scale_range=(0.9 / 112, 1.1 / 112))
    run_and_check(w)
    run_and_check(w, num_kv_splits=5)


@pytest.mark.parametrize("D,ps,G,splits,window,rope", [
    (128, 32, 8, 0, False, 0),   # the fp8 GQA-8 shape
    (128, 16, 4, 0, False, 0),
    (64, 16, 2, 3, False, 0),
    (128, 32, 4, 12, False, 0),  # more chunks than the in-kernel merge takes: the merge kernel
    (128, 16, 4, 5, True, 0),    # sliding window + sink
    (128, 32, 8, 0, False, 1),   # rotate-half RoPE
    (64, 32, 4, 5, False, 2),    # interleaved RoPE, D = 64 (K rotated across lanes)
    (64, 16, 1, 0, True, 1),
])
def test_fp8_page_scales(D, ps, G, splits, window, rope):
    """fp8 pool with a scale per (page, KV head) in place of the per-head ones: every item takes
    its block's K scale in the score and its V scale on P; lengths around page boundaries, empty
    and one-row sequences, every output against the oracle."""
    lens = [1, ps - 1, ps, ps + 1, 5 * ps + 3, 1700, 0, 2 * ps]
    w = synth.make_workload(name=f"pgsc_D{D}_ps{ps}_G{G}_s{splits}_w{int(window)}_r{rope}",
                            B=len(lens), H_qo=2 * G, H_kv=2, D=D, page_size=ps, seq_lens=lens,
                            q_dtype="bf16", kv_dtype="fp8", seed=1100 + D + ps + G + splits + rope,
                            max_num_pages=512, page_scales=True, window=300 if window else None,
                            sink=4 if window else 0, rotary_mode=rope, rope_theta=5e5)
    run_and_check(w, num_kv_splits=splits)


def test_fp8_page_scales_full_size():
    """The fp8 GQA-8 workload's shape (B=256, 64 q / 8 KV heads, page 32, lognormal lengths) with
    per-page scales, automatic plan: every output against the oracle."""
    base = synth.fp8_gqa8()
    lens = base.seq_lens.astype(np.int64)
    w = synth.make_workload(name="fp8_gqa8_page_scales", B=base.B, H_qo=64, H_kv=8, D=128,
                            page_size=32, seq_lens=lens, max_num_pages=65536, kv_dtype="fp8",
                            seed=1005, page_scales=True)
    run_and_check(w)


@pytest.mark.parametrize("G,T,splits", [(4, 2, 0), (2, 4, 12), (8, 2, 3)])
def test_fp8_page_scales_multi(G, T, splits):
    """Several query tokens over an fp8 pool with per-page scales."""
    w = synth.make_workload(name=f"pgsc_multi_G{G}_T{T}_s{splits}", B=5, H_qo=2 * G, H_kv=2,
                            D=128, page_size=32, seq_lens=[3000, T - 1, 700, 33, 64],
                            kv_dtype="fp8", seed=1200 + G + T + splits, max_num_pages=512,
                            page_scales=True)
    _multi_case(w, T, seed=121, num_kv_splits=splits)


def test_append_page_scales_bitexact():
    """pdecode_append_kv into an fp8 pool with per-page scales: each row quantised with its slot's
    page scale, bit-exact against the oracle."""
    import paged_kv_decode_08_amd as pk
    H_kv, D, ps, P = 8, 128, 32, 64
    pool = synth.poisoned_pool(P, H_kv, ps, D, "fp8")
    k, v, slots = synth.append_inputs(T=40, H_kv=H_kv, D=D, page_size=ps, max_num_pages=P,
                                      in_dtype="bf16", seed=13, skip_every=5)
    rng = np.random.default_rng(14)
    ksp = rng.uniform(0.5 / 448, 2 / 448, (P, H_kv)).astype(np.float32)
    vsp = rng.uniform(0.5 / 448, 2 / 448, (P, H_kv)).astype(np.float32)
    tks, tvs = torch.from_numpy(ksp).cuda(), torch.from_numpy(vsp).cuda()
    desc = pk.make_desc(batch=1, num_qo_heads=H_kv, num_kv_heads=H_kv, head_dim=D, page_size=ps,
                        max_num_pages=P, q_dtype="bf16", kv_dtype="fp8", k_scale_page=tks,
                        v_scale_page=tvs)
    tpool = gu.to_device_storage(pool, "fp8")
    pk.append_kv(desc, gu.to_device_storage(k, "bf16"), gu.to_device_storage(v, "bf16"),
                 torch.from_numpy(slots).cuda(), tpool)
    torch.cuda.synchronize()
    ref = oracle.append_kv(pages=pool.copy(), new_k=k, new_v=v, slots=slots, H_kv=H_kv, D=D, ps=ps,
                           in_dtype=1, kv_dtype=2, k_scale_page=ksp, v_scale_page=vsp)
    assert tpool.cpu().numpy().tobytes() == ref.tobytes()


@pytest.mark.parametrize("kv,D,ps,G,splits,window,rope,page_scales", [
    ("bf16", 128, 16, 4, 0, False, 0, False),   # the Llama-3-8B group with an fp8 q
    ("fp8", 128, 32, 8, 0, False, 0, False),    # the fp8 GQA-8 shape
    ("fp8", 64, 16, 2, 3, True, 0, False),
    ("bf16", 128, 32, 1, 12, False, 0, False),  # the merge kernel
    ("fp8", 128, 16, 4, 5, False, 1, False),    # rotate-half RoPE
    ("bf16", 64, 32, 8, 0, False, 2, False),    # interleaved RoPE
    ("fp8", 128, 32, 4, 3, False, 0, True),     # with per-page K/V scales
    ("fp8e4m3", 128, 16, 2, 0, False, 0, False),
])
def test_fp8_q(kv, D, ps, G, splits, window, rope, page_scales):
    """q as e4m3fn codes with a scale per q head: converted exactly to bf16 in the kernel, the
    head's scale applied to its column's scores; out is bf16. Every output against the oracle."""
    lens = [1, ps - 1, ps + 1, 5 * ps + 3, 1700, 0, 2 * ps]
    w = synth.make_workload(name=f"q8_{kv}_D{D}_ps{ps}_G{G}_s{splits}_w{int(window)}_r{rope}",
                            B=len(lens), H_qo=2 * G, H_kv=2, D=D, page_size=ps, seq_lens=lens,
                            q_dtype="fp8", kv_dtype=kv, seed=1300 + D + ps + G + splits + rope,
                            max_num_pages=512, page_scales=page_scales,
                            window=300 if window else None, sink=4 if window else 0,
                            rotary_mode=rope, rope_theta=5e5)
    run_and_check(w, num_kv_splits=splits)


def test_fp8_q_full_size():
    """The Llama-3-8B workload's shape and lengths with an fp8 q, automatic plan."""
    base = synth.llama3_8b_bf16()
    w = synth.make_workload(name="llama_fp8_q", B=32, H_qo=32, H_kv=8, D=128, page_size=16,
                            seq_lens=base.seq_lens.astype(np.int64), max_num_pages=16384,
                            q_dtype="fp8", seed=1002)
    run_and_check(w)


@pytest.mark.parametrize("kv,G,T,splits", [("bf16", 4, 2, 0), ("fp8", 2, 4, 12), ("fp8", 8, 2, 3)])
def test_fp8_q_multi(kv, G, T, splits):
    """Several query tokens with an fp8 q."""
    w = synth.make_workload(name=f"q8_multi_{kv}_G{G}_T{T}_s{splits}", B=5, H_qo=2 * G, H_kv=2,
                            D=128, page_size=16 if kv == "bf16" else 32,
                            seq_lens=[3000, T - 1, 700, 33, 64], q_dtype="fp8", kv_dtype=kv,
                            seed=1400 + G + T + splits, max_num_pages=512)
    _multi_case(w, T, seed=141, num_kv_splits=splits)


def _persist_chunk_bounds(n, cs, cap, ps):
    """Page-slot bounds of the chunks the persistent schedule cuts a sequence of n slots into with
    chunk size cs and at most cap chunks: whole multiples of A = 8 16-row items, the last chunk
    taking the rest (the kernel's rule, restated)."""
    A = 8 if ps == 16 else 4
    if n <= 0:
        return []
    nch = min(-(-n // cs), cap)
    u = n // A
    if nch > 1 and nch > u:
        nch = max(u, 1)
    if nch == 1:
        return [(0, n)]
    uq, urem = u // nch, u % nch
    out = []
    for c in range(nch):
        sb = A * (c * uq + min(c, urem))
        se = n if c == nch - 1 else sb + A * (uq + (1 if c < urem else 0))
        out.append((sb, se))
    return out


@pytest.mark.parametrize("kv,splits", [("bf16", 0), ("bf16", 5), ("fp8", 0)])
def test_split_partials_match_oracle_per_chunk(kv, splits):
    """The split partial states a call leaves in its workspace (pdecode_workspace_layout, the
    debug view of a split plan): chunk c of every split (sequence, q head) holds the decode over
    that chunk's rows alone (out normalised, lse base 2), against the oracle run on just those
    rows. With the automatic plan the chunk size is the one the kernel wrote to the plan word."""
    import paged_kv_decode_08_amd as pk
    ps = 16 if kv == "bf16" else 32
    lens = [3000, 17, 1200, 641, 2500, 90, 4100]
    w = synth.make_workload(name=f"partials_{kv}_{splits}", B=len(lens), H_qo=8, H_kv=2, D=128,
                            page_size=ps, seq_lens=lens, kv_dtype=kv, seed=1500 + splits,
                            max_num_pages=2048)
    dev = gu.upload(w)
    desc = gu.desc_for(w, dev, num_kv_splits=splits)
    ws = pk.alloc_workspace(desc)
    out = torch.empty((w.B, w.H_qo, w.D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.B, w.H_qo), dtype=torch.float32, device="cuda")
    pk.attention(desc, dev["q"], dev["pages"], dev["indptr"], dev["values"], dev["length_info"],
                 out, lse, w.sm_scale, workspace=ws)
    torch.cuda.synchronize()
    lay = pk.workspace_layout(desc)
    cp, _ = pk.plan(desc)
    C = lay["num_chunks"]
    wsn = ws.cpu().numpy()
    cs = cp if cp else int(wsn[lay["plan_word"]:lay["plan_word"] + 4].view(np.int32)[0])
    assert cs >= 1
    rows = w.B * w.H_qo * C
    part_o = wsn[lay["part_o"]:lay["part_o"] + rows * w.D * 4].view(np.float32).reshape(
        w.B, w.H_qo, C, w.D)
    part_lse = wsn[lay["part_lse"]:lay["part_lse"] + rows * 4].view(np.float32).reshape(
        w.B, w.H_qo, C)
    checked = 0
    for b in range(w.B):
        beg, end = int(w.page_indptr[b]), int(w.page_indptr[b + 1])
        bounds = _persist_chunk_bounds(end - beg, cs, C, ps)
        if len(bounds) < 2:
            continue
        for c, (sb, se) in enumerate(bounds):
            r1 = min(se * ps, int(lens[b]))
            kw = w.oracle_kwargs()
            kw.update(B=1, q=w.q[b:b + 1], indptr=np.array([0, se - sb], np.int32),
                      values=w.page_values[beg + sb:beg + se].copy(),
                      length_info=np.array([r1 - (se - 1) * ps], np.int32),
                      q_rope_position=None, k_rope_pos_offset=None)
            o_ref, l_ref = oracle.decode(**kw)
            do, ratio = gu.row_error(w, o_ref[0], part_o[b, :, c].astype(np.float64))
            dl = float(np.abs(part_lse[b, :, c] - l_ref[0]).max())
            assert do <= 2e-2 and ratio <= 1.0 and dl <= 1e-3, (b, c, do, ratio, dl)
            checked += 1
    print(f"{w.name}: chunk size {cs}, {checked} chunk states checked", flush=True)
    assert checked >= 8


def test_fp8_decode_all_codes():
    """Every finite e4m3fn code, read through decode with one attended row and v_scale = 1: the
    bf16 output equals the code's value exactly (all e4m3fn values are bf16 values)."""
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    D, ps = 128, 32
    B = (codes.size + D - 1) // D
    w = synth.make_workload(name="fp8_codes", B=B, H_qo=1, H_kv=1, D=D, page_size=ps,
                            seq_lens=[1] * B, q_dtype="bf16", kv_dtype="fp8", seed=5,
                            max_num_pages=B)
    vals = np.zeros(B * D, np.uint8)
    vals[:codes.size] = codes
    w.k_scale[:] = 1.0
    w.v_scale[:] = 1.0
    for b in range(B):
        page = w.page_values[w.page_indptr[b]]
        w.pages[page, 1, 0, 0, :] = vals[b * D:(b + 1) * D]
    dev = gu.upload(w)
    out, lse = gu.run_attention(w, dev)
    torch.cuda.synchronize()
    got = gu.to_np64(out).reshape(-1)[:codes.size]
    expect = np.array([oracle.fp8_value(int(c)) for c in codes])
    assert np.array_equal(got, expect)


def test_many_short_sequences():
    """Many short (and empty) sequences in one call."""
    lens = np.random.default_rng(17).integers(0, 60, size=300)
    w = synth.make_workload(name="many_short", B=300, H_qo=16, H_kv=4, D=128, page_size=16,
                            seq_lens=lens, seed=18, max_num_pages=1400)
    run_and_check(w)


def test_single_long_sequence():
    """One long sequence: each (sequence, KV head) is split into many chunks."""
    w = synth.make_workload(name="one_long", B=1, H_qo=8, H_kv=2, D=128, page_size=16,
                            seq_lens=[50000], seed=19, max_num_pages=3200)
    run_and_check(w)


@pytest.mark.parametrize("D,ps", [(64, 16), (64, 32), (128, 32)])
def test_shapes_with_small_hint(D, ps):
    lens = [1, 2, 600, 33, 0, 1000, 17]
    w = synth.make_workload(name=f"bal_D{D}_ps{ps}", B=7, H_qo=16, H_kv=2, D=D, page_size=ps,
                            seq_lens=lens, seed=20 + D + ps, max_num_pages=128)
    run_and_check(w)
    run_and_check(w, max_kv_len=50)


@pytest.mark.parametrize("B", [63, 64, 65, 257, 1024, 1025])
def test_batch_sizes_around_schedule_limits(B):
    """Batches at the limits of the persistent schedule's job-table build (one wave up to 64
    sequences, the whole workgroup above; 1024 is the largest batch the table holds, 1025 takes
    the one-workgroup-per-chunk grid), with empty, short and split sequences mixed."""
    rng = np.random.default_rng(300 + B)
    lens = rng.integers(0, 200, size=B)
    lens[rng.integers(0, B, size=max(1, B // 16))] = 0
    lens[rng.integers(0, B, size=max(1, B // 20))] = 1500
    pages = int(np.sum((lens + 15) // 16)) + 8
    w = synth.make_workload(name=f"batch{B}", B=B, H_qo=8, H_kv=2, D=128, page_size=16,
                            seq_lens=lens, seed=400 + B, max_num_pages=pages)
    run_and_check(w)


@pytest.mark.parametrize("splits", [4, 8, 9])
def test_split_counters_reset_across_calls(splits):
    """Split sequences merged inside the persistent kernel (up to 8 chunks in one round trip,
    more in several): the arrival counters and the job queue are back at zero after every call, so
    repeated calls on one workspace give identical results, and a smaller batch reusing the
    workspace is exact too."""
    lens = np.random.default_rng(500 + splits).integers(300, 3000, size=12)
    w = synth.make_workload(name=f"reuse{splits}", B=12, H_qo=16, H_kv=4, D=128, page_size=16,
                            seq_lens=lens, seed=501 + splits, max_num_pages=2400)
    dev = gu.upload(w)
    desc = gu.desc_for(w, dev, num_kv_splits=splits)
    ws = pk_alloc(desc)
    outs = []
    for _ in range(3):
        out = torch.empty((w.B, w.H_qo, w.D), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((w.B, w.H_qo), dtype=torch.float32, device="cuda")
        gu.pk.attention(desc, dev["q"], dev["pages"], dev["indptr"], dev["values"],
                        dev["length_info"], out, lse, w.sm_scale, workspace=ws)
        torch.cuda.synchronize()
        outs.append((out.clone(), lse.clone()))
    check(w, *outs[0], label=w.name)
    for o, l in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0][0].view(torch.int16))
        assert torch.equal(l, outs[0][1])
    # a smaller batch on the same workspace
    w2 = synth.make_workload(name=f"reuse{splits}_small", B=5, H_qo=16, H_kv=4, D=128,
                             page_size=16, seq_lens=lens[:5], seed=502 + splits,
                             max_num_pages=2400)
    dev2 = gu.upload(w2)
    desc2 = gu.desc_for(w2, dev2, num_kv_splits=splits)
    assert gu.pk.workspace_bytes(desc2) <= ws.numel()
    out = torch.empty((w2.B, w2.H_qo, w2.D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w2.B, w2.H_qo), dtype=torch.float32, device="cuda")
    gu.pk.attention(desc2, dev2["q"], dev2["pages"], dev2["indptr"], dev2["values"],
                    dev2["length_info"], out, lse, w2.sm_scale, workspace=ws)
    torch.cuda.synchronize()
    check(w2, out, lse, label=w2.name)


def pk_alloc(desc):
    return gu.pk.alloc_workspace(desc)


def test_workspace_shared_by_rope_and_plain_calls():
    """One description and one workspace used by calls with RoPE (vector-ALU kernel, its own
    chunking) and without (persistent matrix-core kernel): each call finds its counters zero and
    its results exact, in any order."""
    lens = np.random.default_rng(600).integers(200, 4000, size=16)
    common = dict(B=16, H_qo=32, H_kv=8, D=128, page_size=16, seq_lens=lens, seed=601,
                  max_num_pages=4200)
    w_rope = synth.make_workload(name="ws_rope", rotary_mode=1, rope_theta=500000.0, **common)
    w_plain = synth.make_workload(name="ws_plain", **common)
    dev_r, dev_p = gu.upload(w_rope), gu.upload(w_plain)
    desc = gu.desc_for(w_plain, dev_p)
    ws = gu.pk.alloc_workspace(desc)
    rope = gu.pk.make_rope(rotary_mode=1, rope_scale=w_rope.rope_scale,
                           rope_theta=w_rope.rope_theta, q_rope_position=dev_r["q_pos"],
                           k_rope_pos_offset=dev_r["k_off"])
    for w, dev, r in [(w_plain, dev_p, None), (w_rope, dev_r, rope), (w_plain, dev_p, None),
                      (w_rope, dev_r, rope), (w_plain, dev_p, None)]:
        out = torch.empty((w.B, w.H_qo, w.D), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((w.B, w.H_qo), dtype=torch.float32, device="cuda")
        gu.pk.attention(desc, dev["q"], dev["pages"], dev["indptr"], dev["values"],
                        dev["length_info"], out, lse, w.sm_scale, rope=r, workspace=ws)
        torch.cuda.synchronize()
        check(w, out, lse, label=w.name)


@pytest.mark.parametrize("G,D,ps", [(1, 128, 16), (2, 64, 32), (8, 128, 16), (8, 64, 32), (5, 128, 32)])
def test_rope_group_sizes_and_shapes(G, D, ps):
    """RoPE on the matrix-core path across q-head groups (8 heads take P.V through bf16 row
    pairs), head dims and page sizes, with a window and sink, and split sequences."""
    lens = [3000, 17, 0, 1100, 64, 5000]
    w = synth.make_workload(name=f"rope_G{G}_D{D}_ps{ps}", B=len(lens), H_qo=2 * G, H_kv=2, D=D,
                            page_size=ps, seq_lens=lens, seed=700 + G + D + ps,
                            max_num_pages=900, rotary_mode=1, rope_theta=500000.0,
                            rope_scale=0.5, window=2048, sink=4)
    run_and_check(w)
    run_and_check(w, num_kv_splits=5)


@pytest.mark.parametrize("kv,G,ps", [("fp8", 8, 32), ("bf16", 2, 32), ("bf16", 8, 16)])
def test_large_batch_one_workgroup_per_chunk(kv, G, ps):
    """More sequences than the persistent job table holds: the one-workgroup-per-chunk kernel,
    on 16-row items of 16- and 32-row pages, with short, empty and split sequences."""
    B = 1100
    rng = np.random.default_rng(800 + G + ps)
    lens = rng.integers(0, 160, size=B)
    lens[rng.integers(0, B, size=40)] = 1200
    pages = int(np.sum((lens + ps - 1) // ps)) + 8
    w = synth.make_workload(name=f"bigB_{kv}_G{G}_ps{ps}", B=B, H_qo=2 * G, H_kv=2, D=128,
                            page_size=ps, seq_lens=lens, seed=810 + G + ps, max_num_pages=pages,
                            kv_dtype=kv)
    run_and_check(w)


@pytest.mark.parametrize("G,D,ps", [(8, 128, 32), (4, 128, 16), (1, 128, 32), (4, 64, 16),
                                    (8, 64, 32), (1, 64, 16), (2, 64, 32)])
def test_rope_fp8_kv(G, D, ps):
    """RoPE with fp8 KV on the matrix cores (codes converted exactly to fp32 before the rotation);
    at D = 64 each dim's rotation partner is fetched from the other half of the wave."""
    lens = [2500, 33, 0, 700, 4100]
    w = synth.make_workload(name=f"rope_fp8_G{G}_D{D}_ps{ps}", B=len(lens), H_qo=2 * G, H_kv=2,
                            D=D, page_size=ps, seq_lens=lens, seed=900 + G + D + ps,
                            max_num_pages=800, kv_dtype="fp8", rotary_mode=1,
                            rope_theta=500000.0, window=3000, sink=4)
    run_and_check(w)
    run_and_check(w, num_kv_splits=4)


@pytest.mark.parametrize("kv,G,ps,D", [("bf16", 4, 16, 128), ("fp8", 8, 32, 128),
                                        ("fp8", 4, 16, 64)])
def test_large_batch_rope(kv, G, ps, D):
    """RoPE with more sequences than the persistent job table holds: the one-workgroup-per-chunk
    matrix-core kernel rotates q and K in registers too (window + sink, split sequences; fp8 at
    head dim 64 through the lane exchange)."""
    B = 1100
    rng = np.random.default_rng(850 + G + ps)
    lens = rng.integers(0, 200, size=B)
    lens[rng.integers(0, B, size=30)] = 2500
    pages = int(np.sum((lens + ps - 1) // ps)) + 8
    w = synth.make_workload(name=f"bigB_rope_{kv}_G{G}_ps{ps}_D{D}", B=B, H_qo=2 * G, H_kv=2, D=D,
                            page_size=ps, seq_lens=lens, seed=860 + G + ps, max_num_pages=pages,
                            kv_dtype=kv, rotary_mode=1, rope_theta=500000.0, window=1500, sink=4)
    run_and_check(w)


# ---- fused decode step: pdecode_append_attention

def _poison_last_rows(w):
    """NaN in every sequence's row of position total - 1 (all heads, K and V): the fused call must
    take that row from the new values, never from the pool."""
    slots = oracle.last_position_slots(B=w.B, ps=w.page_size, indptr=w.page_indptr,
                                       values=w.page_values, length_info=w.length_info)
    nan = {"bf16": 0x7FC0, "fp8": 0x7F}[w.kv_dtype]
    for s in slots[slots >= 0]:
        w.pages[s // w.page_size, :, :, s % w.page_size, :] = nan


def _fused_case(w, seed, num_kv_splits=0):
    _poison_last_rows(w)
    nk, nv, _ = synth.append_inputs(T=w.B, H_kv=w.H_kv, D=w.D, page_size=w.page_size,
                                    max_num_pages=w.max_num_pages, in_dtype="bf16", seed=seed,
                                    slots=np.zeros(w.B, np.int32))
    o_ref, l_ref, pool_ref = oracle.append_then_decode(new_k=nk, new_v=nv, **w.oracle_kwargs())
    dev = gu.upload(w)
    desc = gu.desc_for(w, dev, num_kv_splits)
    out = torch.empty((w.B, w.H_qo, w.D), dtype=torch.bfloat16, device="cuda")
    out.view(torch.int16).fill_(0x7FC0)
    lse = torch.full((w.B, w.H_qo), float("nan"), dtype=torch.float32, device="cuda")
    rope = None
    if w.rotary_mode:
        rope = pk.make_rope(rotary_mode=w.rotary_mode, rope_scale=w.rope_scale,
                            rope_theta=w.rope_theta, q_rope_position=dev["q_pos"],
                            k_rope_pos_offset=dev["k_off"])
    ws = pk.alloc_workspace(desc)
    nk_d = gu.to_device_storage(nk, "bf16")
    nv_d = gu.to_device_storage(nv, "bf16")
    pk.append_attention(desc, nk_d, nv_d, dev["q"], dev["pages"], dev["indptr"], dev["values"],
                        dev["length_info"], out, lse, w.sm_scale, rope=rope, workspace=ws)
    torch.cuda.synchronize()
    # the pool: bit-exact against the oracle's append, every byte of it
    pool_gpu = dev["pages"].view(torch.uint8).cpu().numpy().reshape(-1)
    assert np.array_equal(pool_gpu, np.ascontiguousarray(pool_ref).view(np.uint8).reshape(-1)), \
        f"{w.name}: pool differs from the oracle's append"
    o_gpu, l_gpu = gu.to_np64(out), gu.to_np64(lse)
    assert_close(w, o_ref, l_ref, o_gpu, l_gpu, f"{w.name} fused")
    # the same as the two separate calls on the updated pool, bit for bit
    out2 = torch.empty_like(out)
    lse2 = torch.empty_like(lse)
    pk.attention(desc, dev["q"], dev["pages"], dev["indptr"], dev["values"], dev["length_info"],
                 out2, lse2, w.sm_scale, rope=rope, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16)), w.name
    assert torch.equal(lse, lse2), w.name


import paged_kv_decode_08_amd as pk  # noqa: E402  (the fixture above loads the library)


@pytest.mark.parametrize("kv,G,D,ps", [("bf16", 4, 128, 16), ("bf16", 1, 64, 32),
                                       ("bf16", 8, 128, 16), ("fp8", 8, 128, 32),
                                       ("fp8", 2, 64, 16)])
def test_append_attention(kv, G, D, ps):
    """Fused append + decode against the oracle (append_kv at each sequence's last position, then
    decode): lengths at and around page boundaries, a one-row sequence and one without pages."""
    lens = [1, ps, ps + 1, 3 * ps - 1, 700, 0, 2 * ps]
    w = synth.make_workload(name=f"fused_{kv}_G{G}_D{D}_ps{ps}", B=len(lens), H_qo=2 * G,
                            H_kv=2, D=D, page_size=ps, seq_lens=lens, q_dtype="bf16",
                            kv_dtype=kv, seed=700 + G + D + ps, max_num_pages=256)
    _fused_case(w, seed=71 + G)


@pytest.mark.parametrize("splits", [3, 12])
def test_append_attention_split(splits):
    """Forced splits (3 and 12 chunks), merged in the kernel."""
    w = synth.make_workload(name=f"fused_split{splits}", B=4, H_qo=16, H_kv=4, D=128,
                            page_size=16, seq_lens=[3000, 17, 1200, 640], seed=720 + splits,
                            max_num_pages=512)
    _fused_case(w, seed=73, num_kv_splits=splits)


def test_append_attention_rope_window():
    """RoPE and a sliding window with a sink: the new row is the window's last (RoPE rotates it
    like any K row); one sequence shorter than the window."""
    w = synth.make_workload(name="fused_rope_swa", B=4, H_qo=32, H_kv=8, D=128, page_size=16,
                            seq_lens=[5000, 300, 4100, 2049], seed=730, max_num_pages=1024,
                            window=1024, sink=4, rotary_mode=1, rope_theta=500000.0)
    _fused_case(w, seed=74)


@pytest.mark.parametrize("kv,D,ps,splits", [("bf16", 128, 16, 0), ("fp8", 64, 32, 5),
                                             ("bf16", 64, 16, 12)])
def test_append_attention_interleaved_rope(kv, D, ps, splits):
    """Fused append with interleaved RoPE: the new row is substituted in its raw form and rotated
    in pairs (2i, 2i + 1) like every other K row; a window and sink on the first case."""
    win = dict(window=1024, sink=4) if splits == 0 else {}
    w = synth.make_workload(name=f"fused_ilv_{kv}_D{D}_ps{ps}_s{splits}", B=4, H_qo=16, H_kv=4,
                            D=D, page_size=ps, seq_lens=[3000, 1, 700, 2 * ps + 1], seed=770 + D,
                            max_num_pages=512, q_dtype="bf16", kv_dtype=kv, rotary_mode=2,
                            rope_theta=500000.0, **win)
    _fused_case(w, seed=79, num_kv_splits=splits)


def test_append_attention_no_attended_rows():
    """An empty window without a sink: no row is attended (out = 0, lse = -5e4), yet every
    sequence with pages still gets its new row."""
    w = synth.make_workload(name="fused_empty_win", B=3, H_qo=8, H_kv=2, D=128, page_size=16,
                            seq_lens=[40, 0, 16], seed=740, max_num_pages=64, window=0, sink=0)
    _fused_case(w, seed=75)


# ---- several query tokens per sequence: pdecode_attention_multi

def _multi_case(w, T, seed, num_kv_splits=0):
    qm = synth.multi_query(w, T, seed)
    kw = {k: v for k, v in w.oracle_kwargs().items() if k != "q"}
    o_ref, l_ref = oracle.decode_multi(qo_len=T, q=qm, **kw)
    dev = gu.upload(w)
    desc = gu.desc_for(w, dev, num_kv_splits)
    qd = gu.to_device_storage(qm, w.q_dtype)
    out = torch.empty((w.B, T, w.H_qo, w.D), dtype=torch.bfloat16, device="cuda")
    out.view(torch.int16).fill_(0x7FC0)
    lse = torch.full((w.B, T, w.H_qo), float("nan"), dtype=torch.float32, device="cuda")
    ws = pk.alloc_workspace_multi(desc, T)
    rope = None
    if w.rotary_mode:
        rope = pk.make_rope(rotary_mode=w.rotary_mode, rope_scale=w.rope_scale,
                            rope_theta=w.rope_theta, q_rope_position=dev["q_pos"],
                            k_rope_pos_offset=dev["k_off"])
    pk.attention_multi(desc, T, qd, dev["pages"], dev["indptr"], dev["values"],
                       dev["length_info"], out, lse, w.sm_scale, rope=rope, workspace=ws)
    torch.cuda.synchronize()
    o_gpu, l_gpu = gu.to_np64(out), gu.to_np64(lse)
    assert_close(w, o_ref, l_ref, o_gpu, l_gpu, f"{w.name} T={T}")
    return qd, desc, dev, out, lse, ws


@pytest.mark.parametrize("kv,G,T,D,ps,splits,rot", [
    ("bf16", 8, 4, 128, 16, 0, 0),   # GQA-8 with 4 tokens: 2 launches of 16 columns
    ("fp8", 8, 3, 128, 32, 0, 0),    # 2 launches: 2 tokens, then 1 (the 8-column kernel)
    ("bf16", 4, 8, 128, 16, 0, 0),   # the Llama-3-8B group with 8 tokens: 2 launches
    ("bf16", 1, 40, 64, 16, 0, 0),   # one head, 40 tokens: launches of 16, 16 and 8
    ("fp8", 2, 9, 128, 32, 12, 1),   # launches of 8 and 1 tokens, forced splits, rotate-half RoPE
    ("bf16", 4, 5, 64, 32, 3, 2),    # launches of 4 and 1 tokens, interleaved RoPE
    ("fp8e4m3", 8, 6, 128, 16, 0, 0),
])
def test_attention_multi_token_groups(kv, G, T, D, ps, splits, rot):
    """More than 16 q columns per KV head (G x T > 16): the call runs the 16-column kernel once per
    group of 16 / G tokens, each group with its own causal caps, RoPE positions and output rows.
    Every output against the oracle; sequences shorter than T and an empty one included."""
    lens = [1, T - 1, T, ps + 1, 3 * ps - 1, 700, 0, 2 * ps + T, 1500]
    w = synth.make_workload(name=f"multi_grp_{kv}_G{G}_T{T}_D{D}_ps{ps}_s{splits}_r{rot}",
                            B=len(lens), H_qo=2 * G, H_kv=2, D=D, page_size=ps, seq_lens=lens,
                            q_dtype="bf16", kv_dtype=kv, seed=1500 + G + T + D + ps + rot,
                            max_num_pages=512, rotary_mode=rot, rope_theta=5e5)
    _multi_case(w, T, seed=151 + T, num_kv_splits=splits)


@pytest.mark.parametrize("kv,G,T,D,ps,splits,rot,win", [
    ("bf16", 4, 3, 128, 16, 0, 0, 300),
    ("fp8", 8, 2, 128, 32, 5, 1, 300),     # rotate-half RoPE: keys at their compacted positions
    ("bf16", 8, 4, 64, 16, 0, 2, 300),     # two launches of 16 columns, interleaved RoPE
    ("bf16", 2, 5, 128, 32, 12, 0, 300),   # forced splits
    ("bf16", 4, 4, 128, 16, 0, 1, 2),      # a window of 2 rows: the first tokens see only the sink
])
def test_attention_multi_window(kv, G, T, D, ps, splits, rot, win):
    """Several query tokens with a sliding window and a sink (one window per sequence for all its
    tokens, each token causal within it): every output against the oracle; prefixes that end
    before the window start (sink rows only) and empty ones included."""
    lens = [1, T - 1, 3, ps + 1, 700, 0, 2000, 5 * ps + 3]
    w = synth.make_workload(name=f"multi_win_{kv}_G{G}_T{T}_D{D}_ps{ps}_s{splits}_r{rot}_w{win}",
                            B=len(lens), H_qo=2 * G, H_kv=2, D=D, page_size=ps, seq_lens=lens,
                            q_dtype="bf16", kv_dtype=kv, seed=1600 + G + T + D + rot,
                            max_num_pages=512, window=win, sink=4, rotary_mode=rot,
                            rope_theta=5e5)
    _multi_case(w, T, seed=161 + T, num_kv_splits=splits)


def test_attention_multi_token_groups_full_size():
    """The fp8 GQA-8 workload's shape (B=256, 64 q / 8 KV heads, page 32, lognormal lengths) with
    4 query tokens per sequence (32 columns per KV head: two launches), automatic plan: every
    output against the oracle."""
    base = synth.fp8_gqa8()
    w = synth.make_workload(name="fp8_gqa8_T4", B=base.B, H_qo=64, H_kv=8, D=128, page_size=32,
                            seq_lens=base.seq_lens.astype(np.int64), max_num_pages=65536,
                            kv_dtype="fp8", seed=1007)
    _multi_case(w, 4, seed=157)


@pytest.mark.parametrize("kv,G,T,D,ps", [("bf16", 4, 2, 128, 16), ("bf16", 1, 8, 64, 32),
                                         ("bf16", 2, 3, 128, 16), ("fp8", 2, 4, 128, 32),
                                         ("fp8", 1, 2, 64, 16), ("bf16", 8, 1, 128, 16),
                                         ("bf16", 4, 4, 128, 16), ("bf16", 8, 2, 128, 16),
                                         ("fp8", 8, 2, 128, 32), ("bf16", 1, 16, 64, 16),
                                         ("fp8", 4, 3, 64, 32), ("bf16", 5, 3, 128, 32)])
def test_attention_multi(kv, G, T, D, ps):
    """T query tokens, causal over the new ones, against the oracle (each token = decode over its
    visible prefix): sequences shorter than T (tokens with no row), an empty one, lengths around
    page boundaries; T x G from 6 to 16 MFMA columns (Llama-3-8B group with 4 tokens, GQA 8 with
    2, one head with 16)."""
    lens = [1, T - 1, ps, ps + 1, 3 * ps - 1, 700, 0, 2 * ps + T]
    w = synth.make_workload(name=f"multi_{kv}_G{G}_D{D}_ps{ps}", B=len(lens), H_qo=2 * G,
                            H_kv=2, D=D, page_size=ps, seq_lens=lens, q_dtype="bf16",
                            kv_dtype=kv, seed=800 + G + T + D + ps, max_num_pages=256)
    _multi_case(w, T, seed=81 + T)


@pytest.mark.parametrize("splits", [3, 12])
def test_attention_multi_split(splits):
    """Forced splits with two tokens (3 and 12 chunks), merged in the kernel, including chunks
    where the first token sees no row."""
    w = synth.make_workload(name=f"multi_split{splits}", B=4, H_qo=16, H_kv=4, D=128,
                            page_size=16, seq_lens=[3000, 17, 1200, 641], seed=820 + splits,
                            max_num_pages=512)
    _multi_case(w, 2, seed=83, num_kv_splits=splits)


@pytest.mark.parametrize("splits", [0, 4, 13])
def test_attention_multi_sixteen_columns_split(splits):
    """Four tokens on the Llama-3-8B group (16 columns): automatic plan and forced splits, merged
    in the kernel."""
    w = synth.make_workload(name=f"multi16_split{splits}", B=5, H_qo=16, H_kv=4, D=128,
                            page_size=16, seq_lens=[3000, 3, 1200, 641, 4], seed=840 + splits,
                            max_num_pages=512)
    _multi_case(w, 4, seed=85, num_kv_splits=splits)


@pytest.mark.parametrize("kv,G,T,D,ps,splits,rot", [("bf16", 4, 2, 128, 16, 0, 1),
                                                    ("bf16", 2, 3, 64, 32, 0, 1),
                                                    ("fp8", 2, 4, 128, 16, 0, 1),
                                                    ("bf16", 4, 2, 128, 16, 12, 1),
                                                    ("fp8", 1, 8, 128, 32, 3, 1),
                                                    ("fp8", 2, 3, 64, 32, 0, 1),
                                                    ("fp8", 4, 2, 64, 16, 12, 1),
                                                    ("bf16", 4, 2, 128, 16, 0, 2),
                                                    ("bf16", 1, 8, 64, 32, 5, 2),
                                                    ("fp8", 2, 4, 64, 16, 12, 2),
                                                    ("fp8", 8, 1, 128, 32, 0, 2),
                                                    ("bf16", 4, 4, 128, 16, 0, 1),
                                                    ("bf16", 8, 2, 128, 16, 7, 2),
                                                    ("fp8", 8, 2, 128, 32, 12, 1),
                                                    ("fp8", 4, 4, 64, 16, 0, 2)])
def test_attention_multi_rope(kv, G, T, D, ps, splits, rot):
    """RoPE with several tokens (rotate-half, or interleaved for rot = 2): token t's query at
    q_rope_position + t (oracle reading), Llama-3 base; lengths around page boundaries, tokens
    with no row, split sequences."""
    lens = [1, T - 1, ps, ps + 1, 3 * ps - 1, 2500, 0, 2 * ps + T]
    w = synth.make_workload(name=f"multi_rope{rot}_{kv}_G{G}_T{T}_D{D}_ps{ps}_s{splits}",
                            B=len(lens), H_qo=2 * G, H_kv=2, D=D, page_size=ps, seq_lens=lens,
                            q_dtype="bf16", kv_dtype=kv, seed=860 + G + T + D + ps + splits + rot,
                            max_num_pages=512, rotary_mode=rot, rope_theta=500000.0)
    _multi_case(w, T, seed=86 + T, num_kv_splits=splits)


def test_attention_multi_one_token_is_attention():
    """qo_len = 1 through pdecode_attention_multi is pdecode_attention, bit for bit."""
    w = synth.make_workload(name="multi_T1", B=5, H_qo=32, H_kv=8, D=128, page_size=16,
                            seq_lens=[900, 1, 17, 4000, 33], seed=840, max_num_pages=512)
    qd, desc, dev, out, lse, ws = _multi_case(w, 1, seed=84)
    out1 = torch.empty((w.B, w.H_qo, w.D), dtype=torch.bfloat16, device="cuda")
    lse1 = torch.empty((w.B, w.H_qo), dtype=torch.float32, device="cuda")
    pk.attention(desc, qd.view(w.B, w.H_qo, w.D), dev["pages"], dev["indptr"], dev["values"],
                 dev["length_info"], out1, lse1, w.sm_scale, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(out.view(w.B, w.H_qo, w.D).view(torch.int16), out1.view(torch.int16))
    assert torch.equal(lse.view(w.B, w.H_qo), lse1)


# ---- learned attention sink per q head

def _sink_case(w, sinks, num_kv_splits=0, T=1):
    dev = gu.upload(w)
    sk = torch.from_numpy(np.asarray(sinks, np.float32)).cuda()
    desc = gu.desc_for(w, dev, num_kv_splits, sink_logits=sk)
    kw = {k: v for k, v in w.oracle_kwargs().items()}
    rope = None
    if w.rotary_mode:
        rope = pk.make_rope(rotary_mode=w.rotary_mode, rope_scale=w.rope_scale,
                            rope_theta=w.rope_theta, q_rope_position=dev["q_pos"],
                            k_rope_pos_offset=dev["k_off"])
    if T == 1:
        o0, l0 = oracle.decode(**kw)
        out = torch.empty((w.B, w.H_qo, w.D), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((w.B, w.H_qo), dtype=torch.float32, device="cuda")
        ws = pk.alloc_workspace(desc)
        pk.attention(desc, dev["q"], dev["pages"], dev["indptr"], dev["values"],
                     dev["length_info"], out, lse, w.sm_scale, rope=rope, workspace=ws)
    else:
        qm = synth.multi_query(w, T, seed=91)
        kw.pop("q")
        o0, l0 = oracle.decode_multi(qo_len=T, q=qm, **kw)
        out = torch.empty((w.B, T, w.H_qo, w.D), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((w.B, T, w.H_qo), dtype=torch.float32, device="cuda")
        ws = pk.alloc_workspace_multi(desc, T)
        pk.attention_multi(desc, T, gu.to_device_storage(qm, w.q_dtype), dev["pages"],
                           dev["indptr"], dev["values"], dev["length_info"], out, lse, w.sm_scale,
                           rope=rope, workspace=ws)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.apply_sink(o0, l0, sinks)
    o_gpu, l_gpu = gu.to_np64(out), gu.to_np64(lse)
    assert_close(w, o_ref, l_ref, o_gpu, l_gpu, f"{w.name} sink")


@pytest.mark.parametrize("kv,G,ps,splits", [("bf16", 4, 16, 0), ("bf16", 4, 16, 3),
                                            ("bf16", 4, 16, 12), ("fp8", 8, 32, 0),
                                            ("bf16", 1, 32, 2)])
def test_learned_sink(kv, G, ps, splits):
    """Per-q-head sink logits, including one that dwarfs the scores (out ~ 0) and one far below
    them (no effect), against the oracle's fold of the sink into the finished state; unsplit and
    split (3 and 12 chunks, the sink folded once at the merge); an empty sequence keeps
    out = 0, lse = -5e4."""
    lens = [1, 300, 2000, 0, 5 * ps + 3]
    w = synth.make_workload(name=f"sink_{kv}_G{G}_ps{ps}_s{splits}", B=len(lens), H_qo=2 * G,
                            H_kv=2, D=128, page_size=ps, seq_lens=lens, q_dtype="bf16",
                            kv_dtype=kv, seed=900 + G + ps + splits, max_num_pages=512)
    sinks = np.random.default_rng(92).normal(0.0, 2.0, w.H_qo).astype(np.float32)
    sinks[0], sinks[-1] = 60.0, -60.0
    _sink_case(w, sinks, splits)


@pytest.mark.parametrize("kv,D,rot,T,splits", [("bf16", 128, 1, 1, 3), ("fp8", 64, 2, 1, 12),
                                               ("bf16", 64, 2, 2, 0), ("fp8", 128, 1, 2, 5)])
def test_learned_sink_with_rope(kv, D, rot, T, splits):
    """Sinks with RoPE (rotate-half or interleaved), one or two query tokens, split or not: the
    sink is folded into the state of the rotated scores."""
    w = synth.make_workload(name=f"sink_rope{rot}_{kv}_D{D}_T{T}_s{splits}", B=4, H_qo=8, H_kv=2,
                            D=D, page_size=16, seq_lens=[1, 40, 1500, 700], seed=940 + D + rot,
                            max_num_pages=256, q_dtype="bf16", kv_dtype=kv, rotary_mode=rot,
                            rope_theta=500000.0)
    sinks = np.random.default_rng(94).normal(0.0, 2.0, w.H_qo).astype(np.float32)
    _sink_case(w, sinks, splits, T=T)


def test_learned_sink_multi_token():
    """Sinks with two query tokens per sequence (each token's state gets its q head's sink)."""
    w = synth.make_workload(name="sink_multi", B=4, H_qo=8, H_kv=2, D=128, page_size=16,
                            seq_lens=[1, 40, 1500, 700], seed=930, max_num_pages=256)
    sinks = np.random.default_rng(93).normal(0.0, 2.0, w.H_qo).astype(np.float32)
    _sink_case(w, sinks, 3, T=2)
    _sink_case(w, sinks, 0, T=2)


# ---- interleaved RoPE (rotary_mode 2)

@pytest.mark.parametrize("kv,G,D,ps", [("bf16", 4, 128, 16), ("bf16", 2, 64, 32),
                                       ("bf16", 8, 128, 16), ("fp8", 4, 128, 32),
                                       ("fp8", 8, 128, 16), ("fp8", 4, 64, 16),
                                       ("fp8", 2, 64, 32)])
def test_rope_interleaved(kv, G, D, ps):
    """Interleaved RoPE (pairs (2i, 2i + 1)) against the oracle, with a window and sink on half of
    the cases, and large positions."""
    lens = [1, 40, 5000, 2049, 3 * ps + 5]
    win = dict(window=1024, sink=4) if G in (4, 8) and ps == 16 else {}
    w = synth.make_workload(name=f"ilv_{kv}_G{G}_D{D}_ps{ps}", B=len(lens), H_qo=2 * G, H_kv=2,
                            D=D, page_size=ps, seq_lens=lens, q_dtype="bf16", kv_dtype=kv,
                            seed=950 + G + D + ps, max_num_pages=1024, rotary_mode=2,
                            rope_theta=500000.0, **win)
    dev = gu.upload(w)
    out, lse = gu.run_attention(w, dev)
    check(w, out, lse, label=w.name)
    out3, lse3 = gu.run_attention(w, dev, num_kv_splits=3)
    check(w, out3, lse3, label=w.name + " split3")


def test_rope_interleaved_unsupported_where_not_built():
    """Interleaved RoPE is refused (before any launch) on the fp32 pool's vector-ALU kernel."""
    import paged_kv_decode_08_amd as pk
    for kv, D in (("f32", 64),):
        w = synth.make_workload(name=f"ilv_unsup_{kv}", B=2, H_qo=4, H_kv=2, D=D, page_size=16,
                                seq_lens=[30, 7], q_dtype="f32" if kv == "f32" else "bf16",
                                kv_dtype=kv, seed=960, max_num_pages=16, rotary_mode=2)
        dev = gu.upload(w)
        with pytest.raises(pk.PdecodeError) as e:
            gu.run_attention(w, dev)
        assert e.value.status == 2


@pytest.mark.parametrize("kv,splits", [("bf16", 2), ("bf16", 5), ("bf16", 8), ("fp8", 3),
                                       ("fp8", 8), ("bf16", 9)])
def test_forced_splits_eight_heads(kv, splits):
    """8 q heads per KV head, forced splits: up to 8 chunks are merged in one round trip of loads,
    9 in two."""
    lens = [5000, 1, 700, 2100, 33, 4096]
    w = synth.make_workload(name=f"g8_splits{splits}_{kv}", B=len(lens), H_qo=16, H_kv=2, D=128,
                            page_size=16 if kv == "bf16" else 32, seq_lens=lens, q_dtype="bf16",
                            kv_dtype=kv, seed=970 + splits, max_num_pages=1024)
    dev = gu.upload(w)
    out, lse = gu.run_attention(w, dev, num_kv_splits=splits)
    check(w, out, lse, label=w.name)


# ---- the additions at the full Llama-3-8B-shaped size, every output

def test_full_size_fused_step():
    """pdecode_append_attention on the full Llama-3-8B-shaped workload (NaN in every target row
    beforehand): every appended row bit-exact, every output against the oracle's append then
    decode."""
    w = synth.CONFIGS["llama3_8b_bf16"]()
    _poison_last_rows(w)
    nk, nv, _ = synth.append_inputs(T=w.B, H_kv=w.H_kv, D=w.D, page_size=w.page_size,
                                    max_num_pages=w.max_num_pages, in_dtype="bf16", seed=77,
                                    slots=np.zeros(w.B, np.int32))
    o_ref, l_ref, pool_ref = oracle.append_then_decode(new_k=nk, new_v=nv, **w.oracle_kwargs())
    dev = gu.upload(w)
    desc = gu.desc_for(w, dev)
    out = torch.empty((w.B, w.H_qo, w.D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.B, w.H_qo), dtype=torch.float32, device="cuda")
    pk.append_attention(desc, gu.to_device_storage(nk, "bf16"), gu.to_device_storage(nv, "bf16"),
                        dev["q"], dev["pages"], dev["indptr"], dev["values"], dev["length_info"],
                        out, lse, w.sm_scale, workspace=pk.alloc_workspace(desc))
    torch.cuda.synchronize()
    slots = oracle.last_position_slots(B=w.B, ps=w.page_size, indptr=w.page_indptr,
                                       values=w.page_values, length_info=w.length_info)
    pages_gpu = dev["pages"].view(torch.int16)
    for s in slots:
        pg, r = int(s) // w.page_size, int(s) % w.page_size
        got = pages_gpu[pg, :, :, r, :].cpu().numpy()
        assert np.array_equal(got, pool_ref[pg, :, :, r, :].view(np.int16)), (pg, r)
    assert_close(w, o_ref, l_ref, gu.to_np64(out), gu.to_np64(lse), "full-size fused")


@pytest.mark.parametrize("T", [2, 4, 6])
def test_full_size_multi_token_and_sink(T):
    """pdecode_attention_multi (two tokens, four: 16 MFMA columns, and six: launches of 4 and 2
    tokens) with learned sinks on the full Llama-3-8B-shaped workload: every (sequence, token,
    head) output against the oracle."""
    w = synth.CONFIGS["llama3_8b_bf16"]()
    qm = synth.multi_query(w, T, seed=78)
    sinks = np.random.default_rng(79).normal(0.0, 2.0, w.H_qo).astype(np.float32)
    kw = {k: v for k, v in w.oracle_kwargs().items() if k != "q"}
    o0, l0 = oracle.decode_multi(qo_len=T, q=qm, **kw)
    o_ref, l_ref = oracle.apply_sink(o0, l0, sinks)
    dev = gu.upload(w)
    desc = gu.desc_for(w, dev, sink_logits=torch.from_numpy(sinks).cuda())
    out = torch.empty((w.B, T, w.H_qo, w.D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.B, T, w.H_qo), dtype=torch.float32, device="cuda")
    pk.attention_multi(desc, T, gu.to_device_storage(qm, "bf16"), dev["pages"], dev["indptr"],
                       dev["values"], dev["length_info"], out, lse, w.sm_scale,
                       workspace=pk.alloc_workspace_multi(desc, T))
    torch.cuda.synchronize()
    assert_close(w, o_ref, l_ref, gu.to_np64(out), gu.to_np64(lse), "full-size multi + sink")


def test_full_size_multi_token_rope():
    """pdecode_attention_multi (two tokens) with rotate-half RoPE (Llama-3 base, token t at
    L - 2 + t, keys from position 0) on the full Llama-3-8B-shaped workload: every
    (sequence, token, head) output against the oracle."""
    import dataclasses
    w0 = synth.CONFIGS["llama3_8b_bf16"]()
    T = 2
    w = dataclasses.replace(w0, rotary_mode=1, rope_theta=500000.0, rope_scale=1.0,
                            q_rope_position=np.maximum(w0.seq_lens - T, 0).astype(np.int32),
                            k_rope_pos_offset=np.zeros(w0.B, np.int32))
    qm = synth.multi_query(w, T, seed=87)
    kw = {k: v for k, v in w.oracle_kwargs().items() if k != "q"}
    o_ref, l_ref = oracle.decode_multi(qo_len=T, q=qm, **kw)
    dev = gu.upload(w)
    desc = gu.desc_for(w, dev)
    rope = pk.make_rope(rotary_mode=1, rope_scale=1.0, rope_theta=500000.0,
                        q_rope_position=dev["q_pos"], k_rope_pos_offset=dev["k_off"])
    out = torch.empty((w.B, T, w.H_qo, w.D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.B, T, w.H_qo), dtype=torch.float32, device="cuda")
    pk.attention_multi(desc, T, gu.to_device_storage(qm, "bf16"), dev["pages"], dev["indptr"],
                       dev["values"], dev["length_info"], out, lse, w.sm_scale, rope=rope,
                       workspace=pk.alloc_workspace_multi(desc, T))
    torch.cuda.synchronize()
    assert_close(w, o_ref, l_ref, gu.to_np64(out), gu.to_np64(lse), "full-size multi + RoPE")


# ---- IEEE-style e4m3 pool (PDECODE_FP8_E4M3, max 240)

@pytest.mark.parametrize("G,ps,splits,D,rot", [(4, 32, 0, 128, 0), (8, 16, 3, 128, 0),
                                               (2, 32, 12, 128, 0), (4, 16, 0, 128, 1),
                                               (8, 32, 3, 64, 1), (2, 16, 0, 64, 2)])
def test_fp8_e4m3_pool_decode(G, ps, splits, D, rot):
    """Decode over an IEEE-style e4m3 pool (finite codes within +-240) against the oracle, also
    with rotate-half and interleaved RoPE at head dims 128 and 64."""
    lens = [1, 300, 2000, 0, 5 * ps + 3]
    w = synth.make_workload(name=f"e4m3_G{G}_ps{ps}_s{splits}_D{D}_r{rot}", B=len(lens),
                            H_qo=2 * G, H_kv=2, D=D, page_size=ps, seq_lens=lens, q_dtype="bf16",
                            kv_dtype="fp8e4m3", seed=990 + G + ps + D + rot, max_num_pages=512,
                            rotary_mode=rot, rope_theta=500000.0)
    run_and_check(w, num_kv_splits=splits)


@pytest.mark.parametrize("G,T,D,rot", [(2, 4, 128, 0), (4, 2, 64, 1)])
def test_fp8_e4m3_pool_multi_token(G, T, D, rot):
    """Several query tokens over an IEEE-style e4m3 pool, without and with RoPE."""
    lens = [1, T - 1, 16, 700, 0, 2500]
    w = synth.make_workload(name=f"e4m3_multi_G{G}_T{T}_D{D}_r{rot}", B=len(lens), H_qo=2 * G,
                            H_kv=2, D=D, page_size=16, seq_lens=lens, q_dtype="bf16",
                            kv_dtype="fp8e4m3", seed=995 + G + T + D, max_num_pages=512,
                            rotary_mode=rot, rope_theta=500000.0)
    _multi_case(w, T, seed=99 + T)


@pytest.mark.parametrize("in_dtype", ["f32", "bf16"])
def test_append_fp8_e4m3_rounding_exhaustive(in_dtype):
    """Every finite e4m3 value, the midpoints between neighbours (ties to even), values at and
    beyond 240 (saturation from 248 up) and tiny values, quantised by the GPU append into an
    e4m3 pool, match the oracle's encoder bit for bit."""
    import ctypes
    import paged_kv_decode_08_amd as pk
    table = np.array([oracle.fp8_e4m3_value(c) for c in range(0x78)])
    mids = (table[:-1] + table[1:]) / 2
    xs = np.concatenate([table, mids, -table, -mids, [240.5, 247.99, 248.0, 250.0, 1e4, -1e4,
                                                      1e-4, 2e-3, -3e-3]]).astype(np.float32)
    D, ps = 64, 16
    T = (xs.size + D - 1) // D
    x = np.zeros(T * D, np.float32)
    x[:xs.size] = xs
    x = synth.cast_f32(x.reshape(T, 1, D), in_dtype)
    ks = np.array([1.0], np.float32)
    P = (T + ps - 1) // ps
    pool = synth.poisoned_pool(P, 1, ps, D, "fp8e4m3")
    slots = np.arange(T, dtype=np.int32)
    desc = pk.make_desc(batch=1, num_qo_heads=1, num_kv_heads=1, head_dim=D, page_size=ps,
                        max_num_pages=P, q_dtype=in_dtype, kv_dtype="fp8e4m3",
                        k_scale=torch.from_numpy(ks).cuda(), v_scale=torch.from_numpy(ks).cuda())
    tpool = torch.from_numpy(pool).cuda()
    tx = gu.to_device_storage(x, in_dtype)
    tslots = torch.from_numpy(slots).cuda()
    st = pk.lib().pdecode_append_kv(ctypes.byref(desc), pk._ptr(tx), pk._ptr(tx), pk._ptr(tslots),
                                    T, pk._ptr(tpool), pk._stream(None))
    assert st == 0
    torch.cuda.synchronize()
    got = tpool.cpu().numpy()
    ref = oracle.append_kv(pages=pool.copy(), new_k=x, new_v=x, slots=slots, H_kv=1, D=D, ps=ps,
                           in_dtype=synth.DTYPE_CODE[in_dtype], kv_dtype=3, k_scale=ks,
                           v_scale=ks)
    assert got.tobytes() == ref.tobytes()


# ---- OCP e5m2 pool (PDECODE_FP8_E5M2)

@pytest.mark.parametrize("G,ps,splits,D,rot,window,page_scales,qd", [
    (4, 16, 0, 128, 0, False, False, "bf16"),  # the Llama-3-8B group
    (8, 32, 0, 128, 0, False, False, "bf16"),  # the GQA-8 group: split sequences merged in-kernel
    (2, 32, 12, 128, 0, False, False, "bf16"),  # more chunks: the split merge kernel
    (4, 16, 5, 128, 1, True, False, "bf16"),   # rotate-half RoPE, sliding window + sink
    (8, 32, 3, 64, 1, False, True, "bf16"),    # D = 64 RoPE across lanes, per-page scales
    (1, 16, 0, 64, 0, True, True, "fp8"),      # fp8 q
    (2, 16, 3, 128, 0, False, False, "fp8"),
])
def test_fp8_e5m2_pool_decode(G, ps, splits, D, rot, window, page_scales, qd):
    """Decode over an OCP e5m2 pool (codes converted exactly to bf16 in the kernel) against the
    oracle: per-KV-head or per-page scales, RoPE, a window, forced splits, an fp8 q; lengths
    around page boundaries, empty and one-row sequences, every output."""
    lens = [1, ps - 1, ps + 1, 5 * ps + 3, 1700, 0, 2 * ps, 300]
    w = synth.make_workload(name=f"e5m2_G{G}_ps{ps}_s{splits}_D{D}_r{rot}_w{int(window)}"
                                 f"_p{int(page_scales)}_{qd}", B=len(lens), H_qo=2 * G, H_kv=2,
                            D=D, page_size=ps, seq_lens=lens, q_dtype=qd, kv_dtype="fp8e5m2",
                            seed=1400 + G + ps + D + rot + splits, max_num_pages=512,
                            page_scales=page_scales, window=300 if window else None,
                            sink=4 if window else 0, rotary_mode=rot, rope_theta=5e5)
    run_and_check(w, num_kv_splits=splits)


def test_fp8_e5m2_pool_full_size():
    """The fp8 GQA-8 workload's shape and lengths (B=256, 64 q / 8 KV heads, page 32) over an e5m2
    pool, automatic plan: every output against the oracle."""
    base = synth.fp8_gqa8()
    w = synth.make_workload(name="fp8_gqa8_e5m2", B=base.B, H_qo=64, H_kv=8, D=128,
                            page_size=32, seq_lens=base.seq_lens.astype(np.int64),
                            max_num_pages=65536, kv_dtype="fp8e5m2", seed=1006)
    run_and_check(w)


def test_fp8_e5m2_decode_all_codes():
    """Every finite e5m2 code, read through decode with one attended row and v_scale = 1: the bf16
    output equals the code's value exactly (every e5m2 value, subnormals included, is a bf16
    value)."""
    codes = np.array([c for c in range(256) if (c & 0x7C) != 0x7C], np.uint8)
    assert codes.size == 248
    D, ps = 128, 16
    B = (codes.size + D - 1) // D
    w = synth.make_workload(name="e5m2_codes", B=B, H_qo=1, H_kv=1, D=D, page_size=ps,
                            seq_lens=[1] * B, q_dtype="bf16", kv_dtype="fp8e5m2", seed=6,
                            max_num_pages=B)
    vals = np.zeros(B * D, np.uint8)
    vals[:codes.size] = codes
    w.k_scale[:] = 1.0
    w.v_scale[:] = 1.0
    for b in range(B):
        page = w.page_values[w.page_indptr[b]]
        w.pages[page, 1, 0, 0, :] = vals[b * D:(b + 1) * D]
    dev = gu.upload(w)
    out, lse = gu.run_attention(w, dev)
    torch.cuda.synchronize()
    got = gu.to_np64(out).reshape(-1)[:codes.size]
    expect = np.array([oracle.fp8_e5m2_value(int(c)) for c in codes])
    assert np.array_equal(got, expect)


@pytest.mark.parametrize("in_dtype", ["f32", "bf16"])
def test_append_fp8_e5m2_rounding_exhaustive(in_dtype):
    """Every finite e5m2 value, the midpoints between neighbours (ties to even), values at and
    beyond 57344 (saturation, infinity included) and tiny values around the subnormal steps,
    quantised by the GPU append into an e5m2 pool, match the oracle's encoder bit for bit."""
    import ctypes
    import paged_kv_decode_08_amd as pk
    table = np.array([oracle.fp8_e5m2_value(c) for c in range(0x7C)])
    mids = (table[:-1] + table[1:]) / 2
    xs = np.concatenate([table, mids, -table, -mids,
                         [57344.0, 61439.0, 61440.0, 65536.0, 1e6, -1e6, np.inf, -np.inf,
                          2.0 ** -17, 3 * 2.0 ** -17, 2.0 ** -18, 1e-7, -2e-5]]).astype(np.float32)
    D, ps = 64, 16
    T = (xs.size + D - 1) // D
    x = np.zeros(T * D, np.float32)
    x[:xs.size] = xs
    x = synth.cast_f32(x.reshape(T, 1, D), in_dtype)
    ks = np.array([1.0], np.float32)
    P = (T + ps - 1) // ps
    pool = synth.poisoned_pool(P, 1, ps, D, "fp8e5m2")
    slots = np.arange(T, dtype=np.int32)
    desc = pk.make_desc(batch=1, num_qo_heads=1, num_kv_heads=1, head_dim=D, page_size=ps,
                        max_num_pages=P, q_dtype=in_dtype, kv_dtype="fp8e5m2",
                        k_scale=torch.from_numpy(ks).cuda(), v_scale=torch.from_numpy(ks).cuda())
    tpool = torch.from_numpy(pool).cuda()
    tx = gu.to_device_storage(x, in_dtype)
    tslots = torch.from_numpy(slots).cuda()
    st = pk.lib().pdecode_append_kv(ctypes.byref(desc), pk._ptr(tx), pk._ptr(tx), pk._ptr(tslots),
                                    T, pk._ptr(tpool), pk._stream(None))
    assert st == 0
    torch.cuda.synchronize()
    got = tpool.cpu().numpy()
    ref = oracle.append_kv(pages=pool.copy(), new_k=x, new_v=x, slots=slots, H_kv=1, D=D, ps=ps,
                           in_dtype=synth.DTYPE_CODE[in_dtype], kv_dtype=4, k_scale=ks,
                           v_scale=ks)
    assert got.tobytes() == ref.tobytes()


@pytest.mark.parametrize("D,page_scales", [(128, False), (36, False), (128, True)])
def test_append_fp8_e5m2_bitexact(D, page_scales):
    """pdecode_append_kv into an e5m2 pool, bit-exact against the oracle: the 16-byte vector form
    (D = 128), the element form (D = 36), per-KV-head or per-page scales, skipped slots."""
    import paged_kv_decode_08_amd as pk
    H_kv, ps, P = 8, 32, 64
    pool = synth.poisoned_pool(P, H_kv, ps, D, "fp8e5m2")
    k, v, slots = synth.append_inputs(T=40, H_kv=H_kv, D=D, page_size=ps, max_num_pages=P,
                                      in_dtype="bf16", seed=15, skip_every=5)
    rng = np.random.default_rng(16)
    kw = {}
    ref_kw = {}
    if page_scales:
        ksp = rng.uniform(0.5 / 448, 2 / 448, (P, H_kv)).astype(np.float32)
        vsp = rng.uniform(0.5 / 448, 2 / 448, (P, H_kv)).astype(np.float32)
        kw = dict(k_scale_page=torch.from_numpy(ksp).cuda(), v_scale_page=torch.from_numpy(vsp).cuda())
        ref_kw = dict(k_scale_page=ksp, v_scale_page=vsp)
    else:
        ks = rng.uniform(0.5 / 448, 2 / 448, H_kv).astype(np.float32)
        vs = rng.uniform(0.5 / 448, 2 / 448, H_kv).astype(np.float32)
        kw = dict(k_scale=torch.from_numpy(ks).cuda(), v_scale=torch.from_numpy(vs).cuda())
        ref_kw = dict(k_scale=ks, v_scale=vs)
    desc = pk.make_desc(batch=1, num_qo_heads=H_kv, num_kv_heads=H_kv, head_dim=D, page_size=ps,
                        max_num_pages=P, q_dtype="bf16", kv_dtype="fp8e5m2", **kw)
    tpool = gu.to_device_storage(pool, "fp8e5m2")
    pk.append_kv(desc, gu.to_device_storage(k, "bf16"), gu.to_device_storage(v, "bf16"),
                 torch.from_numpy(slots).cuda(), tpool)
    torch.cuda.synchronize()
    ref = oracle.append_kv(pages=pool.copy(), new_k=k, new_v=v, slots=slots, H_kv=H_kv, D=D, ps=ps,
                           in_dtype=1, kv_dtype=4, **ref_kw)
    assert tpool.cpu().numpy().tobytes() == ref.tobytes()


def test_append_attention_fp8_rope_window():
    """Fused append into an fp8 pool with RoPE and a window: the substituted row holds the encoded
    codes, which are converted and rotated like every other K row."""
    w = synth.make_workload(name="fused_fp8_rope_swa", B=4, H_qo=16, H_kv=2, D=128, page_size=32,
                            seq_lens=[3000, 200, 4100, 1], seed=760, max_num_pages=512,
                            q_dtype="bf16", kv_dtype="fp8", window=1024, sink=4, rotary_mode=1,
                            rope_theta=500000.0)
    _fused_case(w, seed=76)
    w2 = synth.make_workload(name="fused_fp8_rope_split", B=3, H_qo=8, H_kv=2, D=128,
                             page_size=16, seq_lens=[2500, 33, 900], seed=761, max_num_pages=512,
                             q_dtype="bf16", kv_dtype="fp8", rotary_mode=1, rope_theta=10000.0)
    _fused_case(w2, seed=77, num_kv_splits=5)
    w3 = synth.make_workload(name="fused_fp8_rope_d64", B=4, H_qo=8, H_kv=2, D=64, page_size=16,
                             seq_lens=[2500, 1, 900, 17], seed=762, max_num_pages=512,
                             q_dtype="bf16", kv_dtype="fp8", rotary_mode=1, rope_theta=500000.0)
    _fused_case(w3, seed=78)
