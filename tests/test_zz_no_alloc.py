"""GPU: pdecode_attention_noalloc (the library's own per-GPU scratch, no workspace) against
pdecode_attention with a workspace, through the C ABI, on two calls in a row, the second with a
smaller input; both against the oracle's bounds."""
import numpy as np
import pytest
import torch

import paged_kv_decode_08_amd as pk
import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pk.lib()
    yield


def _both(w, splits=0):
    """(out, lse) of the workspace entry point and of the no-alloc one on the same inputs."""
    dev = gu.upload(w)
    ref_out, ref_lse = gu.run_attention(w, dev, num_kv_splits=splits)
    desc = gu.desc_for(w, dev, num_kv_splits=splits)
    out = torch.empty_like(ref_out)
    if w.q_dtype == "bf16":
        out.view(torch.int16).fill_(0x7FC0)
    else:
        out.fill_(float("nan"))
    lse = torch.full_like(ref_lse, float("nan"))
    rope = None
    if w.rotary_mode:
        rope = pk.make_rope(rotary_mode=w.rotary_mode, rope_scale=w.rope_scale,
                            rope_theta=w.rope_theta, q_rope_position=dev["q_pos"],
                            k_rope_pos_offset=dev["k_off"])
    pk.attention_noalloc(desc, dev["q"], dev["pages"], dev["indptr"], dev["values"],
                         dev["length_info"], out, lse, w.sm_scale, rope=rope)
    torch.cuda.synchronize()
    return ref_out, ref_lse, out, lse


def _check(w, splits=0):
    import oracle
    ref_out, ref_lse, out, lse = _both(w, splits)
    # the same kernels and plan: bit-identical to the workspace entry point
    assert torch.equal(out.view(torch.uint8) if out.dtype != torch.float32 else out.view(torch.int32),
                       ref_out.view(torch.uint8) if ref_out.dtype != torch.float32 else ref_out.view(torch.int32))
    assert torch.equal(lse.view(torch.int32), ref_lse.view(torch.int32))
    o_ref, l_ref = oracle.decode(**w.oracle_kwargs())
    tol_o, tol_l = gu.tolerance(w)
    do, ratio = gu.row_error(w, o_ref, gu.to_np64(out))
    dl = float(np.abs(gu.to_np64(lse) - l_ref).max(initial=0))
    print(f"{w.name} (no-alloc): max|dout|={do:.3g} max|dlse|={dl:.3g} row ratio={ratio:.3g}",
          flush=True)
    assert do <= tol_o and dl <= tol_l
    if w.kv_dtype != "f32":
        assert ratio <= 1.0


def test_noalloc_two_calls_second_smaller():
    """The Llama-3-8B-shaped workload (split sequences), then a smaller batch with
    more KV heads per q head and forced splits: the second call finds the first one's partial
    states in the scratch and must not be disturbed by them."""
    _check(synth.CONFIGS["llama3_8b_bf16"]())
    small = synth.make_workload(name="noalloc_small", B=5, H_qo=16, H_kv=2, D=128, page_size=16,
                                seq_lens=[3000, 17, 0, 900, 1], seed=81, max_num_pages=512)
    _check(small, splits=5)


def test_noalloc_other_paths():
    """fp8 with 8 heads per KV head (in-kernel merge), RoPE + window, and fp32 KV (vector-ALU
    kernel) through the no-alloc entry point, one after another."""
    _check(synth.make_workload(name="noalloc_fp8", B=40, H_qo=64, H_kv=8, D=128, page_size=32,
                               seq_lens=np.arange(40) * 97 + 5, kv_dtype="fp8", seed=82,
                               max_num_pages=4096), splits=3)
    _check(synth.make_workload(name="noalloc_rope", B=6, H_qo=32, H_kv=8, D=128, page_size=16,
                               seq_lens=[5000, 40, 900, 3, 4200, 16], seed=83, max_num_pages=1024,
                               window=1024, sink=4, rotary_mode=1, rope_theta=500000.0))
    _check(synth.tiny_fp32())


def test_noalloc_e5m2_page_scales_fp8_q():
    """An e5m2 pool with per-(page, KV head) scales and an fp8 q through the no-alloc entry point
    (the automatic plan with split sequences), bit-identical to the workspace entry point."""
    _check(synth.make_workload(name="noalloc_e5m2", B=12, H_qo=32, H_kv=8, D=128, page_size=16,
                               seq_lens=np.arange(12) * 331 + 7, kv_dtype="fp8e5m2", q_dtype="fp8",
                               page_scales=True, seed=84, max_num_pages=2048))
