"""foscar_decode_noalloc: the decode step whose split workspace is the
library's static scratch.  Called through the C interface, its output must
equal foscar_decode_int2/int4's on the same inputs (same kernels and plan) and
match the oracle; two calls in a row, the second on a smaller input, and no
device memory is taken by calls after the first."""
import numpy as np
import pytest

import synth
from gpu_util import check, oracle_all, stage_spec

pytestmark = pytest.mark.gpu


def _both(spec, dev):
    import torch
    import bit_quantized_kv_split_amd as fos
    layout = fos.layout_bits(spec.k_layout, spec.v_layout)
    args = (dev["q"], dev["packed_k"], dev["packed_v"], dev["k_scale"], dev["k_zero"], dev["v_scale"],
            dev["v_zero"], dev["seq_lens"], layout, spec.group)
    B, Hq, D = spec.batch, spec.num_q_heads, spec.head_dim
    out = torch.full((B, Hq, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device="cuda")
    fos.foscar_decode_noalloc(spec.bits, *args, out, lse, sm_scale=spec.sm_scale)
    torch.cuda.synchronize()
    ref = (fos.foscar_decode_int2 if spec.bits == 2 else fos.foscar_decode_int4)(*args, sm_scale=spec.sm_scale)
    torch.cuda.synchronize()
    return out, lse, ref[0], ref[1]


def _spec(bits, kl, vl, g, B, T, lens):
    return synth.Spec(f"noalloc_{bits}_{kl}_{vl}_{g}_{B}_{T}", 21, bits, kl, vl, g, B, 4 * 2, 2, 128, T, lens=lens)


@pytest.mark.parametrize("bits,kl,vl,g", [(2, "token", "token", 128), (4, "channel", "channel", 64),
                                          (2, "token", "channel", 32)])
def test_noalloc_matches_the_allocating_entry_point(bits, kl, vl, g):
    import torch
    first = _spec(bits, kl, vl, g, 3, 8192, (8192, 5000, 0))
    second = _spec(bits, kl, vl, g, 2, 1024, (700, 1024))  # smaller: fewer pairs, fewer ranges
    for n, spec in enumerate((first, second)):
        dev, q, lens = stage_spec(spec, poison=True)
        torch.cuda.synchronize()
        free0 = torch.cuda.mem_get_info()[0]
        out, lse, rout, rlse = _both(spec, dev)
        assert torch.equal(out.view(torch.int16), rout.view(torch.int16)), f"call {n}: out differs from the decode entry point"
        assert torch.equal(lse, rlse), f"call {n}: lse differs from the decode entry point"
        ro, rl = oracle_all(spec, q, lens, poison=True)
        check(out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), ro, rl,
              f"noalloc call {n}")
        if n:  # after the first call on the device nothing is allocated (the reference call's workspace exists)
            assert torch.cuda.mem_get_info()[0] == free0, "device memory changed across a no-allocation call"


def test_noalloc_rejects_what_the_scratch_cannot_hold():
    import torch
    import bit_quantized_kv_split_amd as fos
    # 8192 sequences x 4 KV heads: more range counters than the static scratch holds
    B, Hkv, G, T = 8192, 4, 1, 64
    q = torch.zeros((B, Hkv * G, 128), dtype=torch.bfloat16, device="cuda")
    pk = torch.zeros((B, Hkv, T, 8), dtype=torch.int32, device="cuda")
    pv = torch.zeros((B, Hkv, T // 16, 128), dtype=torch.int32, device="cuda")
    sc = torch.zeros((B, Hkv, T, 1), dtype=torch.float16, device="cuda")
    lens = torch.zeros(B, dtype=torch.int32, device="cuda")
    out = torch.zeros((B, Hkv * G, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((B, Hkv * G), dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError, match="static scratch"):
        fos.foscar_decode_noalloc(2, q, pk, pv, sc, sc, sc, sc, lens, 0, 128, out, lse)
