"""GPU parity of the decode at head dimensions other than 128 (a multiple of 32
up to 256: the head-dim-generic kernels) against the fp64 oracle, through the C
interface: the four fold cases at both bit widths, ragged and edge lengths with
NaN-poisoned padding, GQA ratios, forced range counts, the no-allocation entry
point, a larger shape and HIP-graph replay."""
import numpy as np
import pytest

import synth
from gpu_util import check, oracle_all, run, stage_spec

pytestmark = pytest.mark.gpu

TOK, CH = synth.TOKEN, synth.CHANNEL
EDGE_LENS = (0, 1, 2, 31, 63, 64, 65, 127, 129, 200, 255, 256)


def _groups(D, kl, vl):
    """Groups valid for this head dim: a token-wise side groups g channels of a token."""
    tokenwise = kl == TOK or vl == TOK
    return [g for g in (32, 64, 128) if not tokenwise or D % g == 0]


CASES = [(D, kl, vl, g) for D in (32, 64, 96, 256) for kl in (TOK, CH) for vl in (TOK, CH)
         for g in _groups(D, kl, vl)]


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("D,kl,vl,g", CASES)
def test_head_dim_edge_lengths_and_poisoned_padding(bits, D, kl, vl, g):
    spec = synth.Spec(f"hd{D}_{bits}_{kl}_{vl}_{g}", 21, bits, kl, vl, g, len(EDGE_LENS), 4, 1, D, 256,
                      lens=EDGE_LENS)
    dev, q, lens = stage_spec(spec, poison=True)
    out, lse = run(spec, dev)
    ro, rl = oracle_all(spec, q, lens, poison=True)
    check(out, lse, ro, rl, spec.name)
    assert np.all(out[0] == 0) and np.all(np.isneginf(lse[0]))


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("D,hq,hkv", [(64, 8, 2), (64, 16, 1), (256, 2, 2), (96, 12, 1)])
def test_head_dim_gqa_ratios(bits, D, hq, hkv):
    """G = 4, 16 (four work pairs per KV head), 1 and 12 (three pairs of four)."""
    g = 32
    spec = synth.Spec(f"hd{D}_gqa{hq}_{hkv}_{bits}", 22, bits, TOK, CH, g, 3, hq, hkv, D, 1024, ragged=True,
                      ragged_lo=100)
    dev, q, lens = stage_spec(spec)
    out, lse = run(spec, dev)
    ro, rl = oracle_all(spec, q, lens)
    check(out, lse, ro, rl, spec.name)


@pytest.mark.parametrize("splits", ["1", "3", "7", "16"])
@pytest.mark.parametrize("D,kl,vl,g", [(64, TOK, TOK, 64), (256, CH, CH, 32), (96, CH, TOK, 32)])
def test_head_dim_split_counts(monkeypatch, splits, D, kl, vl, g):
    """The result does not depend on how the cache is cut into ranges (every range a
    partial, merged by log-sum-exp in the second launch)."""
    monkeypatch.setenv("FOSCAR_SPLITS", splits)
    spec = synth.Spec(f"hd{D}_split{splits}", 23, 2, kl, vl, g, 2, 8, 2, D, 2048, lens=(2048, 1500))
    dev, q, lens = stage_spec(spec)
    out, lse = run(spec, dev)
    ro, rl = oracle_all(spec, q, lens)
    check(out, lse, ro, rl, spec.name)


@pytest.mark.parametrize("bits", [2, 4])
def test_head_dim_noalloc_matches_decode(bits):
    import torch
    import bit_quantized_kv_split_amd as fos
    spec = synth.Spec(f"hd64_noalloc_{bits}", 24, bits, CH, TOK, 64, 4, 8, 2, 64, 4096, ragged=True, ragged_lo=64)
    dev, q, lens = stage_spec(spec)
    out, lse = run(spec, dev)
    for n in (spec.batch, 2):  # a second, smaller call on the same static scratch
        o2 = torch.empty((n, spec.num_q_heads, 64), dtype=torch.bfloat16, device="cuda")
        l2 = torch.empty((n, spec.num_q_heads), dtype=torch.float32, device="cuda")
        args = {k: dev[k][:n] for k in ("q", "packed_k", "packed_v", "k_scale", "k_zero", "v_scale", "v_zero",
                                         "seq_lens")}
        call = fos.prepare_decode(bits, args["q"], args["packed_k"], args["packed_v"], args["k_scale"],
                                  args["k_zero"], args["v_scale"], args["v_zero"], args["seq_lens"],
                                  fos.layout_bits(spec.k_layout, spec.v_layout), spec.group, out=o2, lse=l2,
                                  sm_scale=spec.sm_scale, noalloc=True)
        call()
        torch.cuda.synchronize()
        assert np.array_equal(o2.float().cpu().numpy(), out[:n].astype(np.float32))
        assert np.array_equal(l2.cpu().numpy(), lse[:n].astype(np.float32))


@pytest.mark.parametrize("bits", [2, 4])
def test_head_dim_256_larger_shape(bits):
    """32 query heads over 8 KV heads, head dim 256, 8192-token capacity, ragged."""
    spec = synth.Spec(f"hd256_large_{bits}", 25, bits, TOK, TOK, 128, 2, 32, 8, 256, 8192, ragged=True,
                      ragged_lo=3000, k_outlier_frac=0.05)
    dev, q, lens = stage_spec(spec)
    out, lse = run(spec, dev)
    ro, rl = oracle_all(spec, q, lens)
    check(out, lse, ro, rl, spec.name)


@pytest.mark.parametrize("D,kl,vl,g", [(64, TOK, CH, 64), (256, CH, TOK, 32)])
def test_head_dim_graph_capture_replays_match_eager(D, kl, vl, g):
    """The two launches of a step captured in a HIP graph (workspace reserved on the capture
    stream first, so a call allocates nothing and records no memset): every replay, with eager
    work and synchronisation between replays, equals the eager result bit for bit."""
    import torch
    import bit_quantized_kv_split_amd as fos
    spec = synth.Spec(f"hd{D}_graph", 26, 2, kl, vl, g, 3, 8, 2, D, 2048, ragged=True, ragged_lo=100)
    dev, q, lens = stage_spec(spec)
    layout = fos.layout_bits(spec.k_layout, spec.v_layout)
    args = (dev["q"], dev["packed_k"], dev["packed_v"], dev["k_scale"], dev["k_zero"], dev["v_scale"], dev["v_zero"],
            dev["seq_lens"], layout, spec.group)
    ref_out, ref_lse = fos.prepare_decode(spec.bits, *args, sm_scale=spec.sm_scale)()
    torch.cuda.synchronize()
    ref_out, ref_lse = ref_out.clone(), ref_lse.clone()
    ro, rl = oracle_all(spec, q, lens)
    check(ref_out.float().cpu().numpy().astype(np.float64), ref_lse.cpu().numpy().astype(np.float64), ro, rl,
          spec.name)
    dims = fos.make_dims(spec.batch, spec.num_q_heads, spec.num_kv_heads, D, spec.max_seq_len)
    side = torch.cuda.Stream()
    fos.foscar_workspace_reserve(dims, spec.bits, layout, spec.group, stream=side)
    out = torch.empty_like(ref_out)
    lse = torch.empty_like(ref_lse)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        call = fos.prepare_decode(spec.bits, *args, out=out, lse=lse, sm_scale=spec.sm_scale, stream=side)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=side):
            for _ in range(2):
                call()
    for k in range(3):
        out.fill_(float("nan"))
        lse.fill_(0.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse), f"replay {k}"
        eager_out, eager_lse = fos.prepare_decode(spec.bits, *args, sm_scale=spec.sm_scale)()
        torch.cuda.synchronize()
        assert torch.equal(eager_out, ref_out) and torch.equal(eager_lse, ref_lse), f"eager after replay {k}"
