"""The prepared decode call (arguments marshalled once) against the one-shot
entry point, on repeated calls with the query changing between calls."""
import pytest
import torch

import synth
from gpu_util import assert_persistent, persistent_spec, stage_spec

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


@pytest.mark.parametrize("name", ["c2_paper_int2", "persistent"])
def test_graph_capture_replays_match_eager(name):
    """Decode steps captured in a HIP graph (after the workspace of the capture
    stream is reserved, a call allocates nothing and records no memset):
    every replay, with eager work and synchronisation between replays, equals
    the eager result bit for bit (the merge order is fixed, so the output is
    deterministic).  The ragged workload takes the persistent work order,
    whose counters the kernel itself resets for the next call."""
    import bit_quantized_kv_split_amd as fos
    if name == "persistent":
        spec = persistent_spec()
        assert_persistent(spec)
    else:
        spec = synth.SPECS[name].replace(batch=3, max_seq_len=4096)
    dev, q, lens = stage_spec(spec)
    layout = fos.layout_bits(spec.k_layout, spec.v_layout)
    args = (dev["q"], dev["packed_k"], dev["packed_v"], dev["k_scale"], dev["k_zero"], dev["v_scale"], dev["v_zero"],
            dev["seq_lens"], layout, spec.group)
    ref_out, ref_lse = fos.prepare_decode(spec.bits, *args)()
    torch.cuda.synchronize()
    ref_out, ref_lse = ref_out.clone(), ref_lse.clone()
    B, Hq, D = dev["q"].shape
    dims = fos.make_dims(B, Hq, dev["packed_k"].shape[1], D, dev["packed_k"].shape[2])
    side = torch.cuda.Stream()
    fos.foscar_workspace_reserve(dims, spec.bits, layout, spec.group, stream=side)
    out = torch.empty_like(ref_out)
    lse = torch.empty_like(ref_lse)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        call = fos.prepare_decode(spec.bits, *args, out=out, lse=lse, stream=side)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=side):
            for _ in range(3):
                call()
    for k in range(4):
        out.fill_(float("nan"))
        lse.fill_(0.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse), f"replay {k}"
        eager_out, eager_lse = fos.prepare_decode(spec.bits, *args)()  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(eager_out, ref_out) and torch.equal(eager_lse, ref_lse), f"eager after replay {k}"
