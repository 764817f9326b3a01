"""CPU checks of the C ABI: the library builds, loads and exports every declared symbol, and the
host-side argument checks return the documented status without launching anything."""
import ctypes
import os
import re

import pytest

import paged_kv_decode_08_amd as pk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails its host checks


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(pk.LIB_PATH):
        from paged_kv_decode_08_amd import build
        build.build()
    return pk.lib()


def declared_functions():
    """Every pdecode_* function declared in a header under include/."""
    names = set()
    inc = os.path.join(ROOT, "include")
    for h in sorted(os.listdir(inc)):
        if h.endswith(".h"):
            text = re.sub(r"/\*.*?\*/", "", open(os.path.join(inc, h)).read(), flags=re.S)
            names |= set(re.findall(r"\b(pdecode_[a-z_]+)\s*\(", text))
    return sorted(names)


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert len(names) >= 10 and "pdecode_bench_stream_read" in names
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    for code, name in pk.STATUS.items():
        assert pk.status_string(code) == name


def desc(**over):
    base = dict(batch=4, num_qo_heads=32, num_kv_heads=8, head_dim=128, page_size=16,
                max_num_pages=100, q_dtype="bf16", kv_dtype="bf16", max_kv_len=4096)
    base.update(over)
    return pk.make_desc(**base)


def attention_status(L, d, workspace=None, ws_bytes=0, rope=None, sm_scale=0.1, ptrs=True):
    P = FAKE if ptrs else None
    return L.pdecode_attention(ctypes.byref(d) if d is not None else None, P, P, P, P, P,
                               None if rope is None else ctypes.byref(rope), sm_scale, P, P,
                               workspace, ws_bytes, None)


@pytest.mark.parametrize("over,code", [
    (dict(num_qo_heads=30), 1),            # not a multiple of num_kv_heads
    (dict(batch=-1), 1),
    (dict(head_dim=0), 1),
    (dict(max_num_pages=0), 1),
    (dict(num_kv_splits=-2), 1),
    (dict(head_dim=96), 2),                # unsupported head dim
    (dict(page_size=8), 2),
    (dict(num_qo_heads=72), 2),            # group size 9
    (dict(q_dtype="f32", kv_dtype="bf16"), 2),
    (dict(q_dtype="f32", kv_dtype="fp8"), 1),  # fp8 without scales is an argument error first
])
def test_attention_argument_errors(L, over, code):
    assert attention_status(L, desc(**over)) == code


def test_attention_null_desc_and_pointers(L):
    assert attention_status(L, None) == 1
    assert attention_status(L, desc(), ptrs=False) == 1
    assert attention_status(L, desc(), sm_scale=float("nan")) == 1


def test_attention_workspace_checks(L):
    d = desc()
    need = pk.workspace_bytes(d)
    assert need > 0
    assert attention_status(L, d) == 3
    assert attention_status(L, d, workspace=FAKE, ws_bytes=need - 1) == 3
    unaligned = ctypes.c_void_p(0x1001)
    assert attention_status(L, d, workspace=unaligned, ws_bytes=need) == 1


def test_rope_checks(L):
    d = desc(num_kv_splits=1, q_dtype="f32", kv_dtype="f32")
    assert pk.workspace_bytes(d) == 0
    r = pk.Rope(1, 1.0, 5e5, None, None)
    assert attention_status(L, d, rope=r) == 1
    r = pk.Rope(1, 1.0, -1.0, FAKE, FAKE)
    assert attention_status(L, d, rope=r) == 1


def test_batch_zero_is_a_noop(L):
    assert attention_status(L, desc(batch=0), ptrs=False) == 0


def test_plan_and_workspace(L):
    # unsplit fp32: no workspace; unsplit bf16 / fp8: the persistent schedule's job-queue counters
    d = desc(num_kv_splits=1, q_dtype="f32", kv_dtype="f32")
    assert pk.plan(d)[1] == 1 and pk.workspace_bytes(d) == 0
    d = desc(num_kv_splits=1)
    assert pk.plan(d)[1] == 1 and pk.workspace_bytes(d) == 256
    assert pk.workspace_bytes(desc(num_kv_splits=1, batch=2000)) == 0  # above the persistent limit
    d = desc(num_kv_splits=5)
    cp, nc = pk.plan(d)
    assert nc == 5 and cp * 5 >= 4096 // 16
    ws = pk.workspace_bytes(d)
    assert ws >= 4 * 32 * 5 * (128 + 1) * 4 and ws % 256 == 0
    # automatic plan of the persistent schedule: the chunk size is chosen on the device at each
    # call (reported as 0); a sequence takes at most ceil(4096 / (B H_kv)) chunks (at least 2; at
    # most 8 for 8 q heads per KV head when B H_kv >= 256), whatever the length hint, so
    # max_kv_len = 0 plans exactly as a tight hint does
    assert pk.plan(desc(batch=2, max_kv_len=131072)) == (0, 256)
    assert pk.plan(desc(batch=1, num_qo_heads=4, num_kv_heads=1, max_kv_len=64)) == (0, 4096)
    assert pk.plan(desc(batch=32)) == (0, 16)
    assert pk.plan(desc(batch=32, num_qo_heads=64)) == (0, 8)
    assert pk.plan(desc(batch=256, num_qo_heads=64)) == (0, 2)
    ws = pk.workspace_bytes(desc())
    assert ws >= 4 * 32 * 128 * (128 + 1) * 4 + (4 * 8 + 2) * 4 and ws % 256 == 0
    assert pk.workspace_bytes(desc(max_kv_len=0)) == ws == pk.workspace_bytes(desc(max_kv_len=64))
    assert pk.workspace_bytes_multi(desc(), 4) >= 4 * 4 * 32 * 128 * (128 + 1) * 4
    # fp32 / fp8 KV: chunks of at least 256 rows; long contexts split, tiny ones do not
    cp, nc = pk.plan(desc(q_dtype="f32", kv_dtype="f32", batch=2, max_kv_len=131072))
    assert nc > 1 and cp * 16 >= 256
    assert pk.plan(desc(q_dtype="f32", kv_dtype="f32", batch=4, num_qo_heads=4, num_kv_heads=4,
                        head_dim=64, max_kv_len=50))[1] == 1
    assert pk.workspace_bytes(desc(head_dim=96)) == 0


def test_merge_argument_errors(L):
    f = L.pdecode_merge_state_inplace
    assert f(-1, 4, 128, 1, FAKE, FAKE, FAKE, FAKE, None) == 1
    assert f(3, 0, 128, 1, FAKE, FAKE, FAKE, FAKE, None) == 1
    assert f(3, 4, 128, 2, FAKE, FAKE, FAKE, FAKE, None) == 2
    assert f(3, 4, 128, 1, FAKE, FAKE, FAKE, FAKE, None) == 1  # v aliases v_other
    assert f(3, 4, 128, 1, None, FAKE, ctypes.c_void_p(0x2000), FAKE, None) == 1
    assert f(0, 4, 128, 1, None, None, None, None, None) == 0


def test_append_argument_errors(L):
    f = L.pdecode_append_kv
    d = desc()
    assert f(ctypes.byref(d), FAKE, FAKE, FAKE, -1, FAKE, None) == 1
    assert f(ctypes.byref(d), None, FAKE, FAKE, 4, FAKE, None) == 1
    assert f(ctypes.byref(d), FAKE, FAKE, FAKE, 0, FAKE, None) == 0
    assert f(ctypes.byref(desc(q_dtype="f32")), FAKE, FAKE, FAKE, 4, FAKE, None) == 2
    assert f(ctypes.byref(desc(kv_dtype="fp8")), FAKE, FAKE, FAKE, 4, FAKE, None) == 1
    assert f(None, FAKE, FAKE, FAKE, 4, FAKE, None) == 1


def test_binding_refuses_host_tensors():
    import torch
    with pytest.raises(ValueError):
        pk._ptr(torch.zeros(3))


def test_append_attention_argument_errors(L):
    """pdecode_append_attention: null new rows, an fp32 pool and a batch beyond the persistent
    schedule are refused before anything is launched; batch 0 is a no-op."""
    f = L.pdecode_append_attention

    def call(d, nk=FAKE, nv=FAKE):
        return f(ctypes.byref(d), nk, nv, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0.1, FAKE, FAKE,
                 FAKE, 1 << 30, None)
    assert call(desc(), nk=None) == 1
    assert call(desc(), nv=None) == 1
    assert call(desc(q_dtype="f32", kv_dtype="f32")) == 2
    assert call(desc(batch=2000)) == 2
    assert call(desc(kv_dtype="fp8")) == 1  # fp8 pool without scales
    assert call(desc(batch=0), nk=None, nv=None) == 0
    assert f(None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0.1, FAKE, FAKE, FAKE, 0,
             None) == 1


def test_attention_multi_argument_errors(L):
    """pdecode_attention_multi: qo_len < 1, an fp32 pool, a batch beyond the
    persistent schedule, more rows than an int holds and an invalid RoPE base are refused before
    anything is launched; the workspace size grows with the tokens. (More than 16 MFMA columns,
    group size x tokens, run as several launches: the GPU tests.)"""
    f = L.pdecode_attention_multi

    def call(d, T, rope=None):
        return f(ctypes.byref(d), T, FAKE, FAKE, FAKE, FAKE, FAKE,
                 None if rope is None else ctypes.byref(rope), 0.1, FAKE, FAKE, FAKE, 1 << 30,
                 None)
    assert call(desc(), 0) == 1
    assert call(desc(), 2, pk.Rope(1, 1.0, -1.0, FAKE, FAKE)) == 1
    assert call(desc(batch=1024), (1 << 31) // (1024 * 32) + 1) == 2  # rows past INT_MAX
    assert call(desc(num_qo_heads=8, batch=2000), 4) == 2
    assert call(desc(num_qo_heads=8, q_dtype="f32", kv_dtype="f32"), 4) == 2
    wb = L.pdecode_workspace_bytes_multi
    assert wb(ctypes.byref(desc()), 0) == 0
    assert wb(ctypes.byref(desc()), 2) >= L.pdecode_workspace_bytes(ctypes.byref(desc()))


def test_sink_outside_the_persistent_schedule_is_unsupported(L):
    """Learned sinks: an fp32 pool (vector-ALU kernel) and a batch above the persistent schedule's
    bound are refused before anything is launched."""
    for d in (desc(q_dtype="f32", kv_dtype="f32"), desc(batch=2000)):
        d.sink_logits = FAKE
        assert attention_status(L, d, workspace=FAKE, ws_bytes=1 << 30) == 2


def test_fp8_e4m3_pool_checks(L):
    """The IEEE-style e4m3 pool needs its scales, and is refused by the fused append (which writes
    e4m3fn codes only) before anything is launched."""
    assert attention_status(L, desc(kv_dtype="fp8e4m3")) == 1
    f = L.pdecode_append_attention
    ks = FAKE
    d = desc(kv_dtype="fp8e4m3")
    d.k_scale = ks
    d.v_scale = ks
    assert f(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0.1, FAKE, FAKE,
             FAKE, 1 << 30, None) == 2


def test_fp8_e5m2_pool_checks(L):
    """The e5m2 pool needs its scales, plans like the other fp8 pools, and is refused before
    anything is launched outside its kernels: several query tokens, the fused append,
    interleaved RoPE and batches above the persistent schedule's bound. An unknown dtype code is
    an argument error."""
    assert attention_status(L, desc(kv_dtype="fp8e5m2")) == 1

    def scaled(**over):
        d = desc(kv_dtype="fp8e5m2", **over)
        d.k_scale = FAKE
        d.v_scale = FAKE
        return d

    cp, nc = ctypes.c_int32(-1), ctypes.c_int32(-1)
    assert L.pdecode_plan(ctypes.byref(scaled()), ctypes.byref(cp), ctypes.byref(nc)) == 0
    cp8, nc8 = ctypes.c_int32(-1), ctypes.c_int32(-1)
    d8 = desc(kv_dtype="fp8")
    d8.k_scale = d8.v_scale = FAKE
    assert L.pdecode_plan(ctypes.byref(d8), ctypes.byref(cp8), ctypes.byref(nc8)) == 0
    assert (cp.value, nc.value) == (cp8.value, nc8.value)
    assert L.pdecode_workspace_bytes(ctypes.byref(scaled())) == \
        L.pdecode_workspace_bytes(ctypes.byref(d8))
    ws = dict(workspace=FAKE, ws_bytes=1 << 30)
    # several query tokens
    m = L.pdecode_attention_multi
    assert m(ctypes.byref(scaled()), 2, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0.1, FAKE, FAKE, FAKE,
             1 << 30, None) == 2
    # the fused append
    f = L.pdecode_append_attention
    assert f(ctypes.byref(scaled()), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0.1, FAKE,
             FAKE, FAKE, 1 << 30, None) == 2
    # interleaved RoPE
    rope = pk.Rope(2, 1.0, 1e4, FAKE, FAKE)
    assert attention_status(L, scaled(), rope=rope, **ws) == 2
    # a batch beyond the persistent schedule
    assert attention_status(L, scaled(batch=2000), **ws) == 2
    d = desc()
    d.kv_dtype = 5
    assert attention_status(L, d) == 1


def test_stream_read_argument_errors(L):
    """The ceiling helper checks its arguments on the host before launching anything."""
    sink = FAKE
    assert L.pdecode_bench_stream_read(None, 1 << 20, 4, 0, 8, sink, None) == 1
    assert L.pdecode_bench_stream_read(FAKE, 1 << 20, 4, 0, 8, None, None) == 1
    assert L.pdecode_bench_stream_read(FAKE, 1 << 20, 4, 0, 0, sink, None) == 1
    assert L.pdecode_bench_stream_read(FAKE, 8, 4, 0, 8, sink, None) == 1      # < 16 bytes
    assert L.pdecode_bench_stream_read(FAKE, 1000, 4, 0, 8, sink, None) == 1   # not 16-multiple
    assert L.pdecode_bench_stream_read(ctypes.c_void_p(0x1008), 1 << 20, 4, 0, 8, sink,
                                       None) == 1                            # misaligned
    assert L.pdecode_bench_stream_read(FAKE, 1 << 20, 3, 0, 8, sink, None) == 2


def noalloc_status(L, d, ptrs=True):
    P = FAKE if ptrs else None
    return L.pdecode_attention_noalloc(ctypes.byref(d) if d is not None else None, P, P, P, P, P,
                                       None, 0.1, P, P, None)


def test_noalloc_refuses_plans_beyond_its_scratch(L):
    """pdecode_attention_noalloc checks its description and plan on the host first: a plan whose
    partial states exceed the 32 MiB region, or whose counters exceed the 64 KiB one, is refused
    with WORKSPACE_TOO_SMALL before the device is touched; bad arguments as pdecode_attention."""
    big = desc(batch=1024, num_qo_heads=64, num_kv_heads=8, max_num_pages=1 << 20,
               max_kv_len=65536)
    assert noalloc_status(L, big) == 3
    many = desc(batch=2100, num_qo_heads=8, num_kv_heads=8, max_num_pages=1 << 20,
                max_kv_len=64, num_kv_splits=2)  # 16802 counters, 4.3 MB of partial states
    assert noalloc_status(L, many) == 3
    assert noalloc_status(L, None) == 1
    assert noalloc_status(L, desc(num_qo_heads=30)) == 1
    assert noalloc_status(L, desc(), ptrs=False) == 1
    assert noalloc_status(L, desc(head_dim=96)) == 2


def test_page_scale_arguments(L):
    """Per-page fp8 scales: both tables or neither, fp8 pools only (INVALID_ARG); the per-head
    scales may then be NULL; only the persistent schedule without the fused append takes them
    (UNSUPPORTED) -- all refused on the host before any launch."""
    def with_pages(d, k=True, v=True):
        d.k_scale_page = FAKE.value if k else None
        d.v_scale_page = FAKE.value if v else None
        return d

    ok = with_pages(desc(kv_dtype="fp8"))
    assert pk.workspace_bytes(ok) > 0
    assert attention_status(L, with_pages(desc(kv_dtype="fp8"), v=False)) == 1
    assert attention_status(L, with_pages(desc(kv_dtype="bf16"))) == 1
    big = with_pages(desc(kv_dtype="fp8", batch=2000, max_num_pages=1 << 16))
    assert attention_status(L, big) == 2
    P = FAKE
    assert L.pdecode_append_attention(ctypes.byref(ok), P, P, P, P, P, P, P, None, 0.1, P, P, P,
                                      1 << 30, None) == 2


def test_fp8_q_arguments(L):
    """fp8 q: its per-q-head scales are required, and only with it (INVALID_ARG); it pairs with a
    BF16 or FP8 pool on the persistent schedule, not with the fused append or an fp32 pool, and
    the append takes no fp8 rows (UNSUPPORTED) -- refused on the host."""
    def fp8q(d, scale=True):
        d.q_scale = FAKE.value if scale else None
        return d

    assert attention_status(L, desc(q_dtype="fp8")) == 1                 # no q_scale
    assert attention_status(L, fp8q(desc())) == 1                        # q_scale with bf16 q
    assert attention_status(L, fp8q(desc(q_dtype="fp8", kv_dtype="f32"))) == 2
    assert attention_status(L, fp8q(desc(q_dtype="fp8", batch=2000, max_num_pages=1 << 16))) == 2
    ok = fp8q(desc(q_dtype="fp8", kv_dtype="bf16"))
    assert pk.workspace_bytes(ok) > 0
    P = FAKE
    assert L.pdecode_append_attention(ctypes.byref(ok), P, P, P, P, P, P, P, None, 0.1, P, P, P,
                                      1 << 30, None) == 2
    assert L.pdecode_append_kv(ctypes.byref(ok), P, P, P, 4, P, None) == 2


def test_workspace_layout(L):
    """pdecode_workspace_layout: partial states after the counters, the plan word after the lse
    rows, all inside the workspace; zeros without partial states."""
    d = desc(batch=4)
    lay = pk.workspace_layout(d)
    C = lay["num_chunks"]
    rows = 4 * 32 * C
    assert lay["part_o"] >= (4 * 8 + 2) * 4 and lay["part_o"] % 256 == 0
    assert lay["part_lse"] >= lay["part_o"] + rows * 128 * 4
    assert lay["plan_word"] == lay["part_lse"] + rows * 4
    assert lay["plan_word"] + 4 <= pk.workspace_bytes(d)
    lay1 = pk.workspace_layout(desc(num_kv_splits=1))
    assert lay1["num_chunks"] == 1 and lay1["part_o"] == lay1["part_lse"] == lay1["plan_word"] == 0


def test_debug_env_prints_the_plan(tmp_path):
    """PDECODE_DEBUG in the environment: an attention call prints its plan to stderr (checked in a
    child process on the CPU, where the launch itself then fails with PDECODE_ERR_HIP)."""
    import subprocess
    import sys
    code = (
        "import ctypes, sys\n"
        f"sys.path.insert(0, {os.path.dirname(os.path.dirname(os.path.abspath(__file__)))!r})\n"
        "import paged_kv_decode_08_amd as pk\n"
        "L = pk.lib()\n"
        "d = pk.make_desc(batch=4, num_qo_heads=32, num_kv_heads=8, head_dim=128, page_size=16,\n"
        "                 max_num_pages=100, q_dtype='bf16', kv_dtype='bf16', max_kv_len=4096)\n"
        "P = ctypes.c_void_p(0x1000)\n"
        "st = L.pdecode_attention(ctypes.byref(d), P, P, P, P, P, None, 0.1, P, P, P, 1 << 30, None)\n"
        "print('status', st)\n")
    env = dict(os.environ, PDECODE_DEBUG="1", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env,
                       timeout=120)
    assert "pdecode: B=4 H_qo=32 H_kv=8 D=128 page=16" in r.stderr, r.stderr
    assert "persistent" in r.stderr
