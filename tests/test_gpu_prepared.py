"""The prepared decode call (arguments marshalled once) against the one-shot
entry point, on repeated calls with the query changing between calls."""
import pytest
import torch

import synth
from gpu_util import stage_spec

pytestmark = pytest.mark.gpu


def test_prepared_call_matches_one_shot_calls():
    import bit_quantized_kv_split_amd as fos
    spec = synth.SPECS["c2_paper_int2"].replace(batch=3, max_seq_len=4096)
    dev, q, lens = stage_spec(spec)
    layout = fos.layout_bits(spec.k_layout, spec.v_layout)
    args = (dev["q"], dev["packed_k"], dev["packed_v"], dev["k_scale"], dev["k_zero"], dev["v_scale"], dev["v_zero"],
            dev["seq_lens"], layout, spec.group)
    call = fos.prepare_decode(spec.bits, *args)
    for k in range(3):
        if k:
            dev["q"].copy_(torch.roll(dev["q"], 1, dims=1))  # new query contents, same storage
        out, lse = call()
        ref_out, ref_lse = fos.foscar_decode_int2(*args)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse), k


def test_dispatch_recorded_events_time_the_kernel():
    import bit_quantized_kv_split_amd as fos
    spec = synth.SPECS["c1_tiny_int2"]
    dev, q, lens = stage_spec(spec)
    layout = fos.layout_bits(spec.k_layout, spec.v_layout)
    call = fos.prepare_decode(spec.bits, dev["q"], dev["packed_k"], dev["packed_v"], dev["k_scale"], dev["k_zero"],
                              dev["v_scale"], dev["v_zero"], dev["seq_lens"], layout, spec.group)
    ref = [t.clone() for t in call()]
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    b.record()
    torch.cuda.synchronize()
    fos.foscar_record_next_launch(a, b)
    out, lse = call()
    torch.cuda.synchronize()
    assert torch.equal(out, ref[0]) and torch.equal(lse, ref[1])
    ms = a.elapsed_time(b)
    assert 0.0 < ms < 100.0, ms
