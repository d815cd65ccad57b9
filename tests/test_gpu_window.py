"""GPU parity of decode with a full-precision window of recent tokens
(foscar_decode_window_int2/int4, through the C interface) against the
oracle's attention over the union of dequantised cache tokens and window
tokens, with the decode bar of gpu_util: single-range and multi-range
sequences, the persistent work order, empty caches with a window, empty
windows, and nothing at all."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import assert_persistent, check, persistent_spec, stage_spec

pytestmark = pytest.mark.gpu


def _oracle(spec, q, lens, win):
    G = spec.num_q_heads // spec.num_kv_heads
    B, Hq, D = spec.batch, spec.num_q_heads, spec.head_dim
    out, lse = np.zeros((B, Hq, D)), np.zeros((B, Hq))
    for b in range(B):
        for h in range(spec.num_kv_heads):
            head = synth.make_head(spec, b, h, seq_len=int(lens[b]))
            w = {k: v[None, None] for k, v in head.items()}
            w["q"] = q[b:b + 1, h * G:(h + 1) * G]
            w["seq_lens"] = np.array([lens[b]], np.int32)
            wl = int(win["lens"][b])
            ws = {"k": win["k"][b:b + 1, h:h + 1], "v": win["v"][b:b + 1, h:h + 1], "lens": np.array([wl])}
            o, l = oracle.decode_window_rows(w, ws, [(0, i) for i in range(G)], k_layout=spec.k_layout,
                                             v_layout=spec.v_layout, group=spec.group, sm_scale=spec.sm_scale)
            out[b, h * G:(h + 1) * G], lse[b, h * G:(h + 1) * G] = o, l
    return out, lse


def _run(spec, dev, win):
    import torch
    import bit_quantized_kv_split_amd as fos
    wk = torch.from_numpy(win["k"]).to(torch.bfloat16).cuda()
    wv = torch.from_numpy(win["v"]).to(torch.bfloat16).cuda()
    wl = torch.from_numpy(win["lens"]).cuda()
    out, lse = fos.decode(dev["q"], dev["packed_k"], dev["packed_v"], dev["k_scale"], dev["k_zero"], dev["v_scale"],
                          dev["v_zero"], dev["seq_lens"], bits=spec.bits, k_layout=spec.k_layout,
                          v_layout=spec.v_layout, group=spec.group, window=(wk, wv, wl))
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


CASES = [(2, "token", "token", 128), (4, "token", "token", 64), (2, "channel", "channel", 32),
         (4, "channel", "channel", 128), (2, "token", "channel", 64), (4, "channel", "token", 32)]


@pytest.mark.parametrize("bits,kl,vl,g", CASES)
def test_window_matrix(bits, kl, vl, g):
    """Ragged cache lengths (one empty) and ragged windows (one empty, one on
    the empty cache, one sequence with neither)."""
    std = (0.1, 10.0) if "channel" in (kl, vl) else None
    spec = synth.Spec(f"win_{bits}_{kl}_{vl}_{g}", 12, bits, kl, vl, g, 5, 8, 2, 128, 768,
                      lens=(768, 517, 130, 0, 0), channel_std_logu=std)
    dev, q, lens = stage_spec(spec)
    win = synth.make_window(1, spec.batch, spec.num_kv_heads, 200, [200, 0, 37, 64, 0])
    out, lse = _run(spec, dev, win)
    ro, rl = _oracle(spec, q, lens, win)
    check(out, lse, ro, rl, spec.name)


@pytest.mark.parametrize("name,cap", [("c3_long_int2", 300), ("c3_long_int2", 512), ("c3_long_int2", 1024),
                                      ("c3_long_int2", 4096), ("persistent", 512), ("persistent", 4096)])
def test_window_multi_range_and_persistent(name, cap):
    """Many ranges per sequence (merge path) with the window attended inside the
    decode launch by 1-8 work-groups per pair, beside the ranges or ahead of
    the persistent round (ragged batch with empty sequences)."""
    if name == "persistent":
        spec = persistent_spec()
        assert_persistent(spec)
    else:
        spec = synth.SPECS[name].replace(batch=1, num_q_heads=4, num_kv_heads=1, max_seq_len=16384)
    dev, q, lens = stage_spec(spec)
    wl = [cap - 7 * b for b in range(spec.batch)]
    win = synth.make_window(2, spec.batch, spec.num_kv_heads, cap, wl)
    out, lse = _run(spec, dev, win)
    ro, rl = _oracle(spec, q, lens, win)
    check(out, lse, ro, rl, spec.name)


@pytest.mark.parametrize("G", [1, 3, 8])
def test_window_gqa_ratios_through_the_merge(G, monkeypatch):
    """G = 1, 3 and 8 query heads per KV head, 64 forced ranges and a window:
    window partials fold into the merge of every query row, including the
    pairs whose sequence has no cache token (G = 8: two groups of 4 query
    heads read each KV head's cache and window)."""
    spec = synth.Spec(f"win_gqa_{G}", 15, 2, "token", "token", 128, 3, 3 * G, 3, 128, 4096, lens=(4096, 2500, 0))
    monkeypatch.setenv("FOSCAR_SPLITS", "64")
    dev, q, lens = stage_spec(spec)
    win = synth.make_window(4, spec.batch, spec.num_kv_heads, 300, [300, 17, 150])
    out, lse = _run(spec, dev, win)
    ro, rl = _oracle(spec, q, lens, win)
    check(out, lse, ro, rl, spec.name)


def test_window_dominates_when_its_scores_are_larger():
    """A window whose keys align with the query takes almost all the weight:
    the output approaches the window's own attention output (a property of
    the merge, not only agreement with the oracle)."""
    spec = synth.SPECS["c1_tiny_int2"]
    dev, q, lens = stage_spec(spec)
    win = synth.make_window(3, 1, 1, 8, [8])
    win["k"][0, 0] = synth.bf16_round((q[0, 0] * 4.0).astype(np.float32))[None].repeat(8, 0)
    out, lse = _run(spec, dev, win)
    ro, rl = _oracle(spec, q, lens, win)
    check(out, lse, ro, rl, "dominant window")
    mean_v = win["v"][0, 0].astype(np.float64).mean(0)
    assert np.abs(out[0, 0] - mean_v).max() < 0.05
