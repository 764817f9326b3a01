"""Benchmark: single-token paged-KV decode attention on one MI355X.

One step = one pdecode_attention call (every kernel of the path, split-KV merge included) over one
batch of a decode workload; by default the Llama-3-8B-shaped bf16 one: B=32, 32 q / 8 kv heads,
D=128, page size 16, context lengths uniform in [512, 4096], page ids a shuffled subset of a
16384-page pool (--workload selects the other synthetic workloads of the parity tests). Inputs are
synthetic and resident in HBM before timing starts. When a step reads less than 512 MB, steps cycle
through several independent input sets (disjoint pools, same lengths) so that no step finds its KV
in the 256 MB last-level cache left warm by the previous one.

Prints one JSON line. value = KV-read GB/s (bytes of attended K/V rows per step / step time);
ms_per_step is the wall time per step between synchronisations; `roofline` uses the average
pdecode_attention duration from HIP events on the launch stream; `cpu_baseline` times the oracle
on the host on a bounded sample of the same workload.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, 8 TB/s
CTX_DESC = {"llama3_8b_bf16": "uniform[512,4096]", "long_ctx_bf16": "{32768,131072}",
            "rope_swa_bf16": "uniform[1024,16384], window 4096 + sink 4, RoPE theta 5e5",
            "fp8_gqa8": "lognormal(median 2048, sigma 0.5) capped at 8192",
            "gqa8_bf16": "uniform[512,4096]",
            "tiny_fp32": "{1,17,33,50}"}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200,
                    help="untimed calls first (a cold GPU takes on the order of a hundred calls "
                         "of the larger workloads to reach its steady rate)")
    ap.add_argument("--sets", type=int, default=4, help="independent input sets cycled per step")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the oracle leg")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--splits", type=int, default=0, help="num_kv_splits (0 = automatic plan)")
    ap.add_argument("--no-hint", action="store_true",
                    help="max_kv_len = 0 in the description (no length hint)")
    ap.add_argument("--workload", default="llama3_8b_bf16",
                    choices=["llama3_8b_bf16", "long_ctx_bf16", "rope_swa_bf16", "fp8_gqa8",
                             "tiny_fp32", "gqa8_bf16"])
    ap.add_argument("--op", choices=["merge_state", "append_kv", "append_attention", "multi"],
                    default=None,
                    help="instead of the decode, time pdecode_merge_state_inplace or "
                         "pdecode_append_kv at a decode-step size and a bulk size, or a whole "
                         "decode step of --workload: pdecode_append_attention against "
                         "pdecode_append_kv followed by pdecode_attention, or --qo-len query "
                         "tokens per sequence of --workload: one pdecode_attention_multi call "
                         "against --qo-len pdecode_attention calls")
    ap.add_argument("--qo-len", type=int, default=2, help="query tokens per sequence (--op multi)")
    ap.add_argument("--multi-rope", action="store_true",
                    help="--op multi: rotate-half RoPE (base 5e5), token t at position L - T + t")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the streaming-read ceiling sweep (profiler runs)")
    ap.add_argument("--ceiling", action="store_true",
                    help="instead of the decode, print the streaming-read ceiling sweep (every "
                         "launch shape of pdecode_bench_stream_read over a 2 GiB buffer, and a "
                         "plain read of the workload's KV bytes per step) and exit")
    ap.add_argument("--timeline", action="store_true",
                    help="instead of the timed run, load the timeline build of the library "
                         "(python -m paged_kv_decode_08_amd.build --timeline), run --warmup "
                         "calls of --workload, then 3 runs of 8 back-to-back calls, and print "
                         "each run's last call: per-workgroup entry, job table, first K/V issue, "
                         "jobs and exit times, the KV rate over the call (from each job's slots "
                         "and duration) and the split merge kernel's times")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="instead of the decode, run a plain 512 MiB device-to-device copy "
                         "(the reference point for the HBM byte counters) and exit")
    return ap.parse_args()


# Sources of the decode kernels: the HBM-traffic figure recorded under profiles/ is used only while
# their hash matches the one it was measured with.
KERNEL_SOURCES = ["paged_kv_decode_08_amd/csrc/decode_mfma.hip",
                  "paged_kv_decode_08_amd/csrc/decode_persist.hpp",
                  "paged_kv_decode_08_amd/csrc/mfma_core.hpp",
                  "paged_kv_decode_08_amd/csrc/decode_valu.hip",
                  "paged_kv_decode_08_amd/csrc/device.hpp",
                  "paged_kv_decode_08_amd/csrc/split.hpp",
                  "paged_kv_decode_08_amd/csrc/api.cpp"]


def kernel_source_hash():
    """sha256 of the kernel sources with comments and blank lines removed (no string literal in
    them holds a comment marker), so that an edit of comments alone keeps the recorded counters."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
        for line in text.splitlines():
            code = line.split("//", 1)[0].rstrip()
            if code:
                h.update(code.encode() + b"\n")
    return h.hexdigest()


def recorded_traffic(workload):
    """HBM bytes per launch from the FETCH_SIZE / WRITE_SIZE summary under profiles/ for this
    workload, or None when there is none or the kernel sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"decode_{workload}_hbm_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    sha = re.search(r"^source_sha256:\s*([0-9a-f]{64})", text, re.M)
    val = re.search(r"^traffic_bytes_per_launch:\s*([0-9.eE+]+)", text, re.M)
    if not sha or not val or sha.group(1) != kernel_source_hash():
        return None
    return float(val.group(1))


CEILING_BYTES = 2 << 30  # well above the 256 MB last-level cache


def _time_launches(fn, reps, stream):
    """Mean duration of fn() over `reps` launches, from one HIP event pair on `stream`."""
    import torch
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for i in range(reps):
        fn(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) * 1e-3 / reps


def measure_ceiling(step_bytes=None, verbose=False):
    """Streaming-read ceiling of this device (pdecode_bench_stream_read): the best rate over a
    sweep of launch shapes (workgroups per CU, 16-byte loads per lane per round, nontemporal
    hint), each reading a 2 GiB buffer once per launch, 10 timed launches after 3 warm-up ones.
    With step_bytes, the best shape also reads exactly that many bytes per launch, cycling over 4
    buffers so that no launch finds its bytes in the last-level cache: the time one launch of a
    step's size needs at best, launch ramp and drain included."""
    import torch

    import paged_kv_decode_08_amd as pk
    stream = torch.cuda.current_stream()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    buf = torch.zeros(CEILING_BYTES, dtype=torch.uint8, device="cuda")
    sink = torch.empty(cus * 16 * 256, dtype=torch.int32, device="cuda")
    sweep = []
    for per_cu in (1, 2, 4, 8):
        for u in (2, 4, 8, 16):
            for nt in (0, 1):
                fn = lambda i: pk.bench_stream_read(buf, u, nt, cus * per_cu, sink, stream=stream)
                for i in range(3):
                    fn(i)
                dt = _time_launches(fn, 10, stream)
                sweep.append({"workgroups_per_cu": per_cu, "loads_per_lane": u, "nontemporal": nt,
                              "us": round(dt * 1e6, 2), "GBps": round(CEILING_BYTES / dt / 1e9, 1)})
    best = max(sweep, key=lambda r: r["GBps"])
    res = {"GBps": best["GBps"], "bytes_per_launch": CEILING_BYTES,
           "shape": {k: best[k] for k in ("workgroups_per_cu", "loads_per_lane", "nontemporal")}}
    if verbose:
        res["sweep"] = sweep
    del buf
    if step_bytes:
        n = (int(step_bytes) + 15) // 16 * 16
        bufs = [torch.zeros(n, dtype=torch.uint8, device="cuda") for _ in range(4)]
        fn = lambda i: pk.bench_stream_read(bufs[i % 4], best["loads_per_lane"],
                                            best["nontemporal"], cus * best["workgroups_per_cu"],
                                            sink, stream=stream)
        for i in range(8):
            fn(i)
        dt = _time_launches(fn, 100, stream)
        res["step_size_read"] = {"bytes": n, "us": round(dt * 1e6, 2),
                                 "GBps": round(n / dt / 1e9, 1)}
    return res


def copy_calibration(steps):
    """A plain device-to-device copy of known size, for scaling the HBM byte counters."""
    import torch
    n = 512 << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": steps,
                      "GBps_read_plus_write": round(2 * n / dt / 1e9, 1)}), flush=True)


def op_bench(op, steps, warmup):
    """Times the two small calls of the path: one launch per step, HIP events around the K steps.
    merge_state: bf16 v [n, 32, 128] and fp32 s merged in place with (v', s'); bytes = both states
    read + one written. append_kv: T new bf16 K and V rows of 8 KV heads x 128 into a bf16 pool;
    bytes = rows read + written (+ slot ids)."""
    import numpy as np
    import torch

    import paged_kv_decode_08_amd as pk
    import synth

    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    results = []
    for label, size in (("decode_step", 32), ("bulk", 4096)):
        if op == "merge_state":
            n, H, D = size, 32, 128
            rng = np.random.default_rng(7)
            mk = lambda: torch.from_numpy(synth.cast_f32(
                rng.standard_normal((n, H, D), dtype=np.float32), "bf16")).view(torch.int16).view(
                    torch.bfloat16).cuda()
            v, vo = mk(), mk()
            s = torch.from_numpy(rng.standard_normal((n, H)).astype(np.float32)).cuda()
            so = torch.from_numpy(rng.standard_normal((n, H)).astype(np.float32)).cuda()
            nbytes = 3 * (n * H * D * 2 + n * H * 4)
            call = lambda: pk.merge_state_inplace(v, s, vo, so, stream=stream)
            shape = {"n": n, "num_heads": H, "head_dim": D, "v_dtype": "bf16"}
        else:
            T, H_kv, D, ps, pool = size, 8, 128, 16, 16384
            k, vv, slots = synth.append_inputs(T=T, H_kv=H_kv, D=D, page_size=ps,
                                               max_num_pages=pool, in_dtype="bf16", seed=8)
            desc = pk.make_desc(batch=1, num_qo_heads=H_kv, num_kv_heads=H_kv, head_dim=D,
                                page_size=ps, max_num_pages=pool, q_dtype="bf16", kv_dtype="bf16")
            tk = torch.from_numpy(k).view(torch.int16).view(torch.bfloat16).cuda()
            tv = torch.from_numpy(vv).view(torch.int16).view(torch.bfloat16).cuda()
            ts = torch.from_numpy(slots).cuda()
            pages = torch.zeros((pool, 2, H_kv, ps, D), dtype=torch.bfloat16, device="cuda")
            nbytes = 2 * 2 * T * H_kv * D * 2 + T * 4
            call = lambda: pk.append_kv(desc, tk, tv, ts, pages, stream=stream)
            shape = {"tokens": T, "num_kv_heads": H_kv, "head_dim": D, "page_size": ps,
                     "kv_dtype": "bf16"}
        for _ in range(warmup):
            call()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev0.record(stream)
        for _ in range(steps):
            call()
        ev1.record(stream)
        torch.cuda.synchronize()
        wall_us = (time.perf_counter() - t0) * 1e6 / steps
        ev_us = ev0.elapsed_time(ev1) * 1e3 / steps
        results.append({"size": label, **shape, "bytes": nbytes, "us_per_call_events": round(ev_us, 3),
                        "us_per_call_wall": round(wall_us, 3),
                        "GBps_events": round(nbytes / (ev_us * 1e-6) / 1e9, 1)})
    print(json.dumps({"op": op, "n_gpus": 1, "steps": steps, "warmup": warmup,
                      "data": "synthetic", "results": results}), flush=True)


def multi_bench(workload, T, steps, warmup, nsets, rope=False):
    """T query tokens per sequence (causal over the new tokens): one pdecode_attention_multi call,
    which reads the KV once for all T tokens, against T pdecode_attention calls (one per token,
    each over the whole sequence: the upper bound of the per-token work). K steps each between
    synchronisations, input sets cycled as in the decode bench."""
    import numpy as np
    import torch

    import paged_kv_decode_08_amd as pk
    import synth
    from tests import gpu_util as gu

    torch.cuda.set_device(0)
    make = synth.CONFIGS[workload]
    base = make()
    nsets = nsets if base.kv_bytes < 512e6 else 1
    lens = base.seq_lens.astype(np.int64)
    sets = [base] + [make(seed=1002 + 100 * i, lens=lens) for i in range(1, nsets)]
    devs = [gu.upload(w) for w in sets]
    desc = gu.desc_for(base, devs[0])
    ws = pk.alloc_workspace_multi(desc, T)
    qm = gu.to_device_storage(synth.multi_query(base, T, seed=10), base.q_dtype)
    out = torch.empty((base.B, T, base.H_qo, base.D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((base.B, T, base.H_qo), dtype=torch.float32, device="cuda")
    qt = [qm[:, t].contiguous() for t in range(T)]
    outs = [torch.empty((base.B, base.H_qo, base.D), dtype=torch.bfloat16, device="cuda")
            for _ in range(T)]
    lses = [torch.empty((base.B, base.H_qo), dtype=torch.float32, device="cuda") for _ in range(T)]
    stream = torch.cuda.current_stream()
    ropes = [None] * T  # per-token calls: token t's query at L - T + t
    mrope = None
    if rope:
        qpos = [torch.from_numpy(np.maximum(lens - T + t, 0).astype(np.int32)).cuda()
                for t in range(T)]
        koff = torch.zeros(base.B, dtype=torch.int32, device="cuda")
        ropes = [pk.make_rope(rotary_mode=1, rope_scale=1.0, rope_theta=500000.0,
                              q_rope_position=qpos[t], k_rope_pos_offset=koff) for t in range(T)]
        mrope = ropes[0]

    def multi(i):
        d = devs[i % len(devs)]
        pk.attention_multi(desc, T, qm, d["pages"], d["indptr"], d["values"], d["length_info"],
                           out, lse, base.sm_scale, rope=mrope, workspace=ws, stream=stream)

    def per_token(i):
        d = devs[i % len(devs)]
        for t in range(T):
            pk.attention(desc, qt[t], d["pages"], d["indptr"], d["values"], d["length_info"],
                         outs[t], lses[t], base.sm_scale, rope=ropes[t], workspace=ws,
                         stream=stream)

    res = {}
    for name, fn in (("per_token_calls", per_token), ("multi", multi),
                     ("per_token_calls_again", per_token), ("multi_again", multi)):
        for i in range(warmup):
            fn(i)
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev0.record(stream)
        for i in range(steps):
            fn(i)
        ev1.record(stream)
        torch.cuda.synchronize()
        res[name] = {"us_per_step_wall": round((time.perf_counter() - t0) * 1e6 / steps, 2),
                     "us_per_step_events": round(ev0.elapsed_time(ev1) * 1e3 / steps, 2)}
    us = res["multi"]["us_per_step_events"]
    print(json.dumps({"op": "multi", "workload": base.name, "qo_len": T, "rope": bool(rope),
                      "n_gpus": 1,
                      "steps": steps, "warmup": warmup, "input_sets": len(sets),
                      "kv_bytes_per_step": base.kv_bytes,
                      "multi_kv_GBps_events": round(base.kv_bytes / (us * 1e-6) / 1e9, 1),
                      "data": "synthetic", **res}), flush=True)


def step_bench(workload, steps, warmup, nsets):
    """A whole decode step: the step's new K/V row of every (sequence, KV head) goes to the
    sequence's last position, then attention. Fused (one pdecode_append_attention launch) against
    separate (pdecode_append_kv, then pdecode_attention), K steps each between synchronisations,
    input sets cycled as in the decode bench."""
    import numpy as np
    import torch

    import paged_kv_decode_08_amd as pk
    import synth
    from tests import gpu_util as gu

    torch.cuda.set_device(0)
    make = synth.CONFIGS[workload]
    base = make()
    nsets = nsets if base.kv_bytes < 512e6 else 1
    lens = base.seq_lens.astype(np.int64)
    sets = [base] + [make(seed=1002 + 100 * i, lens=lens) for i in range(1, nsets)]
    devs = [gu.upload(w) for w in sets]
    desc = gu.desc_for(base, devs[0])
    ws = pk.alloc_workspace(desc)
    out = torch.empty((base.B, base.H_qo, base.D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((base.B, base.H_qo), dtype=torch.float32, device="cuda")
    rng = np.random.default_rng(9)
    new = [torch.from_numpy(synth.cast_f32(rng.standard_normal((base.B, base.H_kv, base.D),
                                                               dtype=np.float32), "bf16"))
           .view(torch.int16).view(torch.bfloat16).cuda() for _ in range(2)]
    slots = []
    for w in sets:  # each sequence's position total - 1 (its last page, row last_page_len - 1)
        last = np.asarray(w.length_info).reshape(-1, w.B)[0].astype(np.int64)
        ids = w.page_values[w.page_indptr[1:] - 1].astype(np.int64)
        slots.append(torch.from_numpy((ids * w.page_size + last - 1).astype(np.int32)).cuda())
    ropes = [None] * len(devs)
    if base.rotary_mode:
        ropes = [pk.make_rope(rotary_mode=base.rotary_mode, rope_scale=base.rope_scale,
                              rope_theta=base.rope_theta, q_rope_position=d["q_pos"],
                              k_rope_pos_offset=d["k_off"]) for d in devs]
    stream = torch.cuda.current_stream()

    def fused(i):
        d = devs[i % len(devs)]
        pk.append_attention(desc, new[0], new[1], d["q"], d["pages"], d["indptr"], d["values"],
                            d["length_info"], out, lse, base.sm_scale, rope=ropes[i % len(devs)],
                            workspace=ws, stream=stream)

    def separate(i):
        d = devs[i % len(devs)]
        pk.append_kv(desc, new[0], new[1], slots[i % len(devs)], d["pages"], stream=stream)
        pk.attention(desc, d["q"], d["pages"], d["indptr"], d["values"], d["length_info"], out,
                     lse, base.sm_scale, rope=ropes[i % len(devs)], workspace=ws, stream=stream)

    res = {}
    for name, fn in (("separate", separate), ("fused", fused), ("separate_again", separate),
                     ("fused_again", fused)):
        for i in range(warmup):
            fn(i)
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev0.record(stream)
        for i in range(steps):
            fn(i)
        ev1.record(stream)
        torch.cuda.synchronize()
        res[name] = {"us_per_step_wall": round((time.perf_counter() - t0) * 1e6 / steps, 2),
                     "us_per_step_events": round(ev0.elapsed_time(ev1) * 1e3 / steps, 2)}
    print(json.dumps({"op": "append_attention", "workload": base.name, "n_gpus": 1,
                      "steps": steps, "warmup": warmup, "input_sets": len(sets),
                      "kv_bytes_per_step": base.kv_bytes, "data": "synthetic", **res}), flush=True)


def kernel_desc(kv_dtype, num_chunks):
    """What one timed pdecode_attention call launches for a plan of at most num_chunks chunks per
    sequence (the time covers all of it)."""
    if kv_dtype == "f32":
        return ("pdecode_attention: the vector-ALU decode kernel, one wave per chunk; the last "
                "chunk of a split sequence to finish merges it (one launch)")
    if num_chunks <= 1:
        return "pdecode_attention: the persistent matrix-core decode kernel (one launch, no splits)"
    if num_chunks <= 8:
        return ("pdecode_attention: the persistent matrix-core decode kernel, which merges split "
                "sequences itself (one launch)")
    return ("pdecode_attention: the persistent matrix-core decode kernel, then the split merge "
            "kernel (two launches)")


def _timeline_summary(marks, item_bytes):
    """One call's marks ([4096, 64] uint64: time << 24 | tag << 20 | value; time in 10 ns ticks of
    s_memrealtime) -> text lines and a dict of the key times (us from the first workgroup entry)."""
    import numpy as np
    dec = marks[:2048]
    used = np.nonzero(dec[:, 0])[0]
    t = (dec[used] >> np.uint64(24)).astype(np.float64) * 0.01
    tag = ((dec[used] >> np.uint64(20)) & np.uint64(0xF)).astype(int)
    val = (dec[used] & np.uint64(0xFFFFF)).astype(int)
    valid = dec[used] != 0
    t0 = t[:, 0].min()
    t = t - t0
    nwg = len(used)

    def first(i, k):
        sel = valid[i] & (tag[i] == k)
        return t[i][sel][0] if sel.any() else np.nan

    entry = t[:, 0]
    table = np.array([first(i, 2) for i in range(nwg)])
    issue = np.array([first(i, 3) for i in range(nwg)])
    exits = np.array([first(i, 6) for i in range(nwg)])
    pct = lambda x: [round(float(v), 2) for v in np.nanpercentile(x, [0, 10, 50, 90, 100])]
    jobs = []
    for i in range(nwg):
        st = t[i][valid[i] & (tag[i] == 4)]
        en = t[i][valid[i] & (tag[i] == 5)]
        nw = val[i][valid[i] & (tag[i] == 4)]
        for k in range(min(len(st), len(en))):
            jobs.append((st[k], en[k], nw[k]))
    jobs = np.array(jobs)
    nj = np.bincount(np.array([int((valid[i] & (tag[i] == 4)).sum()) for i in range(nwg)]))
    T = int(np.nanmax(exits)) + 2
    rate = np.zeros(T)
    active = np.zeros(T)
    for s_, e_, nw_ in jobs:  # a job's bytes spread evenly over its duration
        b = nw_ * 4 * item_bytes
        for u in range(int(s_), int(e_) + 1):
            lo, hi = max(s_, u), min(e_, u + 1)
            if hi > lo:
                rate[u] += b * (hi - lo) / (e_ - s_)
                active[u] += hi - lo
    lines = [f"  workgroups {nwg}; jobs per workgroup: " +
             ", ".join(f"{k}: {int(c)}" for k, c in enumerate(nj) if c),
             "  percentiles p0 p10 p50 p90 p100, us from the first workgroup's entry:",
             f"  entry           {pct(entry)}",
             f"  job table built {pct(table)}",
             f"  first K/V issue {pct(issue)}",
             f"  exit            {pct(exits)}",
             "  us: KV GB/s (job averages) / workgroups in a job"]
    cells = [f"{u:3d}: {rate[u] / 1e3:5.0f}/{active[u]:4.0f}" for u in range(T)]
    lines += ["   " + "  ".join(cells[k:k + 6]) for k in range(0, len(cells), 6)]
    res = {"entry_p100": pct(entry)[4], "table_p50": pct(table)[2], "first_issue_p50": pct(issue)[2],
           "first_issue_p90": pct(issue)[3], "exit_p10": pct(exits)[1], "exit_p50": pct(exits)[2],
           "exit_p100": pct(exits)[4], "peak_GBps": round(float(rate.max()) / 1e3, 0)}
    mk = marks[2048:]
    mu = np.nonzero(mk[:, 0])[0]
    if len(mu):
        ms = (mk[mu, 0] >> np.uint64(24)).astype(np.float64) * 0.01 - t0
        ends = mk[mu, 1]
        me = (ends[ends != 0] >> np.uint64(24)).astype(np.float64) * 0.01 - t0
        lines.append(f"  split merge kernel: {len(mu)} workgroups, start {pct(ms)}, end {pct(me)}")
        res.update(merge_start_p0=round(float(ms.min()), 2), merge_end_p100=round(float(me.max()), 2))
    return lines, res


def timeline(args):
    import ctypes

    import numpy as np
    import torch

    import paged_kv_decode_08_amd as pk
    from paged_kv_decode_08_amd import build as pbuild
    import synth
    from tests import gpu_util as gu

    if not os.path.exists(pbuild.LIB_TIMELINE):
        sys.exit("bench.py --timeline: build the timeline library first: "
                 "python -m paged_kv_decode_08_amd.build --timeline")
    pk.LIB_PATH = pbuild.LIB_TIMELINE
    pk._lib = None
    L = pk.lib()
    L.pdk_timeline_read.argtypes = [ctypes.c_void_p]
    torch.cuda.set_device(0)
    make = synth.CONFIGS[args.workload]
    base = make()
    nsets = args.sets if base.kv_bytes < 512e6 else 1
    lens = base.seq_lens.astype(np.int64)
    sets = [base] + [make(seed=1002 + 100 * i, lens=lens) for i in range(1, nsets)]
    devs = [gu.upload(w) for w in sets]
    desc = gu.desc_for(base, devs[0], num_kv_splits=args.splits,
                       max_kv_len=0 if args.no_hint else None)
    ws = pk.alloc_workspace(desc)
    out = torch.empty((base.B, base.H_qo, base.D), dtype=gu.TORCH_STORAGE[base.q_dtype],
                      device="cuda")
    lse = torch.empty((base.B, base.H_qo), dtype=torch.float32, device="cuda")
    ropes = [None] * len(devs)
    if base.rotary_mode:
        ropes = [pk.make_rope(rotary_mode=base.rotary_mode, rope_scale=base.rope_scale,
                              rope_theta=base.rope_theta, q_rope_position=d["q_pos"],
                              k_rope_pos_offset=d["k_off"]) for d in devs]
    stream = torch.cuda.current_stream()

    def step(i):
        d = devs[i % len(devs)]
        pk.attention(desc, d["q"], d["pages"], d["indptr"], d["values"], d["length_info"], out,
                     lse, base.sm_scale, rope=ropes[i % len(devs)], workspace=ws, stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # one item: 16 rows of K and of V of one KV head
    item_bytes = 2 * 16 * base.D * synth.ELEM_BYTES[base.kv_dtype]
    marks = np.zeros((4096, 64), np.uint64)
    runs = []
    print(f"timeline of {args.workload}: plan {pk.plan(desc)}, the last of 8 back-to-back calls",
          flush=True)
    for r in range(3):
        L.pdk_timeline_clear()
        torch.cuda.synchronize()
        for i in range(8):
            step(i + r)
        torch.cuda.synchronize()
        if L.pdk_timeline_read(marks.ctypes.data_as(ctypes.c_void_p)) != 0:
            sys.exit("bench.py --timeline: reading the marks failed")
        lines, res = _timeline_summary(marks, item_bytes)
        print(f"run {r}:")
        print("\n".join(lines), flush=True)
        runs.append(res)
    print(json.dumps({"timeline": args.workload, "runs": runs}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "the multi-GPU sharding of this path is a design note, not an implementation.",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(max(args.steps, 1))
        return
    if args.timeline:
        timeline(args)
        return
    if args.ceiling:
        import synth
        import torch
        torch.cuda.set_device(0)
        kvb = synth.CONFIGS[args.workload]().kv_bytes
        print(json.dumps({"ceiling": measure_ceiling(step_bytes=kvb, verbose=True),
                          "workload": args.workload}), flush=True)
        return
    if args.op == "multi":
        multi_bench(args.workload, args.qo_len, max(args.steps, 1), args.warmup, args.sets,
                    rope=args.multi_rope)
        return
    if args.op == "append_attention":
        step_bench(args.workload, max(args.steps, 1), args.warmup, args.sets)
        return
    if args.op:
        op_bench(args.op, max(args.steps, 1), args.warmup)
        return
    import numpy as np
    import torch

    import paged_kv_decode_08_amd as pk
    import synth
    from tests import gpu_util as gu

    torch.cuda.set_device(0)
    make = synth.CONFIGS[args.workload]
    base = make()
    nsets = args.sets if base.kv_bytes < 512e6 else 1
    lens = base.seq_lens.astype(np.int64)
    sets = [base] + [make(seed=1002 + 100 * i, lens=lens) for i in range(1, nsets)]
    devs = [gu.upload(w) for w in sets]
    kv_bytes = base.kv_bytes
    desc = gu.desc_for(base, devs[0], num_kv_splits=args.splits,
                       max_kv_len=0 if args.no_hint else None)
    ws = pk.alloc_workspace(desc)
    out = torch.empty((base.B, base.H_qo, base.D), dtype=gu.TORCH_STORAGE[base.q_dtype],
                      device="cuda")
    lse = torch.empty((base.B, base.H_qo), dtype=torch.float32, device="cuda")
    ropes = [None] * len(devs)
    if base.rotary_mode:
        ropes = [pk.make_rope(rotary_mode=base.rotary_mode, rope_scale=base.rope_scale,
                              rope_theta=base.rope_theta, q_rope_position=d["q_pos"],
                              k_rope_pos_offset=d["k_off"]) for d in devs]
    stream = torch.cuda.current_stream()

    def step(i):
        d = devs[i % len(devs)]
        pk.attention(desc, d["q"], d["pages"], d["indptr"], d["values"], d["length_info"], out,
                     lse, base.sm_scale, rope=ropes[i % len(devs)], workspace=ws, stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # Timed region: exactly `steps` steps between synchronisations, bracketed by one HIP event
    # pair on the launch stream for the mean per-call duration on the GPU. (An event pair around
    # every call would add the events' own GPU-side cost, several us, to every step.)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    avg_call_s = ev0.elapsed_time(ev1) * 1e-3 / args.steps

    # Spread of single calls, from a separate loop with an event pair around each call (these
    # durations carry the events' overhead; the timed region above does not).
    nspread = min(args.steps, 50)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(nspread)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(nspread)]
    for i in range(nspread):
        starts[i].record(stream)
        step(i)
        ends[i].record(stream)
    torch.cuda.synchronize()
    call_ms = np.array([s.elapsed_time(e) for s, e in zip(starts, ends)])
    value = kv_bytes / (ms_per_step * 1e-3) / 1e9
    achieved = kv_bytes / avg_call_s / 1e9
    cp, nc = pk.plan(desc)

    ceiling = None if args.no_ceiling else measure_ceiling(step_bytes=kv_bytes)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(base, args.cpu_seconds)

    line = {
        "metric": "decode-attn µs/step + KV-read GB/s (% of MI355X HBM peak), 1 GPU",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "us_per_step": round(ms_per_step * 1e3, 2),
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": base.kv_dtype if base.kv_dtype != "fp8" else "fp8-e4m3fn KV, bf16 q/out",
        "data": "synthetic",
        "config": {"workload": base.name, "batch": base.B,
                   "num_qo_heads": base.H_qo, "num_kv_heads": base.H_kv, "head_dim": base.D,
                   "page_size": base.page_size, "kv_dtype": base.kv_dtype,
                   "ctx_len": CTX_DESC.get(args.workload, ""),
                   "kv_bytes_per_step": kv_bytes, "input_sets": len(sets),
                   "split_plan": (f"chunks sized on the device from the call's lengths, at most "
                                  f"{nc} per sequence" if cp == 0 else
                                  f"chunks of {cp} page slots, at most {nc} per sequence"),
                   "max_kv_len_hint": int(desc.max_kv_len)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": recorded_traffic(args.workload),
                     "traffic_unit": "HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, copy-scaled)",
                     "algorithmic_bytes": kv_bytes,
                     "kernel": kernel_desc(base.kv_dtype, nc),
                     "avg_launch_us": round(avg_call_s * 1e6, 3),
                     "ceiling_GBps": ceiling["GBps"] if ceiling else None,
                     "frac_of_ceiling": round(achieved / ceiling["GBps"], 4) if ceiling else None,
                     "ceiling": ceiling,
                     "single_call_event_us_p10": round(float(np.percentile(call_ms, 10)) * 1e3, 3),
                     "single_call_event_us_p90": round(float(np.percentile(call_ms, 90)) * 1e3, 3)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


# Host threads for the oracle leg: every CPU this process may run on, up to the 16 that one GPU's
# share of the host is (the GPU hosts give each GPU 16 CPUs and set OMP_NUM_THREADS to match).
HOST_THREAD_SHARE = 16


def host_threads():
    cores = os.cpu_count() or 1
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        pass
    return max(1, min(cores, HOST_THREAD_SHARE))


def cpu_baseline(w, budget_s, threads=None):
    """The oracle on the host, on a bounded sample of (sequence, q head) outputs of the same
    workload; reported in KV GB/s over the KV bytes the sample reads. threads: host threads
    (default: host_threads()); a second, shorter run on one thread is reported beside it."""
    out = _cpu_baseline_run(w, budget_s, threads or host_threads())
    one = _cpu_baseline_run(w, max(2.0, budget_s / 3), 1)
    out["single_thread"] = {k: one[k] for k in ("value", "unit", "cores", "seconds",
                                                 "us_per_step", "sample")}
    return out


def _cpu_baseline_run(w, budget_s, cores):
    import numpy as np

    import oracle
    rng = np.random.default_rng(0)
    G = w.H_qo // w.H_kv
    groups = np.array([(b, h) for b in range(w.B) for h in range(w.H_kv)], np.int32)
    rng.shuffle(groups)

    def pairs_of(gs):
        return np.array([(b, h * G + g) for b, h in gs for g in range(G)], np.int32)

    # calibrate on a small slice, then size the sample of (sequence, KV head) groups to the budget
    n0 = min(len(groups), cores)
    t = time.perf_counter()
    oracle.decode(**w.oracle_kwargs(), select=pairs_of(groups[:n0]), nthreads=cores)
    dt = time.perf_counter() - t
    n = int(min(len(groups), max(n0, n0 * budget_s / max(dt, 1e-6))))
    sel = groups[:n]
    kw = w.oracle_kwargs()
    t = time.perf_counter()
    oracle.decode(**kw, select=pairs_of(sel), nthreads=cores)
    dt = time.perf_counter() - t
    # a sample that is the whole workload and finishes early is repeated up to the budget
    reps = 1
    if n == len(groups) and dt < budget_s / 2:
        reps = int(min(1000, budget_s / max(dt, 1e-6)))
        t = time.perf_counter()
        for _ in range(reps):
            oracle.decode(**kw, select=pairs_of(sel), nthreads=cores)
        dt = time.perf_counter() - t
    eb = synth_elem_bytes(w)
    bytes_read = reps * int(w.attended[sel[:, 0]].astype(np.int64).sum()) * 2 * w.D * eb
    return {"value": round(bytes_read / dt / 1e9, 4), "unit": "GB/s", "cores": cores,
            "kind": "oracle", "seconds": round(dt, 2),
            "us_per_step": round(dt / reps * 1e6 * len(groups) / n, 1),
            "sample": f"{n} of {len(groups)} (sequence, KV head) groups of the same workload "
                      f"(all {G} q heads each){f', {reps} passes' if reps > 1 else ''}, fp64 "
                      f"scalar C++ on {cores} host threads; GB/s over the K/V bytes the sample "
                      "reads"}


def synth_elem_bytes(w):
    import synth
    return synth.ELEM_BYTES[w.kv_dtype]


if __name__ == "__main__":
    main()
