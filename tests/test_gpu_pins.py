"""GPU runs of the pages' worked receipt and closed forms, and bit-exact packing."""
import math

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

D = 128


def _stage_arrays(bits, q, k_codes, v_codes, ks, kz, vs, vz, lens, Tcap):
    import bit_quantized_kv_split_amd.staging as staging
    B, Hkv = k_codes.shape[:2]
    head = {"k_codes": k_codes, "v_codes": v_codes, "k_scale": ks, "k_zero": kz, "v_scale": vs, "v_zero": vz}
    shapes = {"k_scale": ks.shape, "k_zero": kz.shape, "v_scale": vs.shape, "v_zero": vz.shape}
    return staging.stage((B, q.shape[1], Hkv, Tcap, D), bits, q, np.array(lens, np.int32),
                         lambda b: {k: v[b] for k, v in head.items()}, shapes)


def _run(dev, bits, kl, vl, g):
    import bit_quantized_kv_split_amd as fos
    import torch
    out, lse = fos.decode(dev["q"], dev["packed_k"], dev["packed_v"], dev["k_scale"], dev["k_zero"], dev["v_scale"],
                          dev["v_zero"], dev["seq_lens"], bits=bits, k_layout=kl, v_layout=vl, group=g)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("bits", [2, 4])
def test_receipt_key_side(bits):
    """Explainer receipt: stickers (2,1,3) weighted by quantities (3,1,2) with
    rate 0.75 and fee -1.125 -> 0.75*13 - 1.125*6 = 3; one token, so
    lse = 3/sqrt(128) and the output is that token's value."""
    Tcap = 64
    q = np.zeros((1, 4, D), np.float32)
    q[0, :, :3] = [3, 1, 2]
    kc = np.zeros((1, 1, Tcap, D), np.uint8)
    kc[0, 0, 0, :3] = [2, 1, 3]
    vc = np.zeros((1, 1, Tcap, D), np.uint8)
    vc[0, 0, 0] = np.arange(D) % (1 << bits)
    ks = np.full((1, 1, Tcap, 1), 0.75, np.float16)
    kz = np.full((1, 1, Tcap, 1), -1.125, np.float16)
    vs = np.full((1, 1, Tcap, 1), 0.5, np.float16)
    vz = np.full((1, 1, Tcap, 1), -0.25, np.float16)
    dev = _stage_arrays(bits, q, kc, vc, ks, kz, vs, vz, [1], Tcap)
    out, lse = _run(dev, bits, "token", "token", 128)
    assert abs(lse[0, 0] - 3 / math.sqrt(128)) < 1e-6
    np.testing.assert_array_equal(out[0, 0], 0.5 * vc[0, 0, 0] - 0.25)


def test_receipt_key_side_own_rate_per_line():
    """Channel-wise K: every channel (line) has its own rate; operand-fold on Q."""
    Tcap = 128
    q = np.zeros((1, 4, D), np.float32)
    q[0, 0, :3] = [3, 1, 2]
    kc = np.zeros((1, 1, Tcap, D), np.uint8)
    kc[0, 0, 0, :3] = [2, 1, 3]
    ks = np.zeros((1, 1, 1, D), np.float16)
    ks[0, 0, 0, :3] = [0.5, 1.25, 2.0]
    kz = np.full((1, 1, 1, D), -0.375, np.float16)
    vc = np.zeros((1, 1, Tcap, D), np.uint8)
    vs = np.zeros((1, 1, 1, D), np.float16)
    vz = np.zeros((1, 1, 1, D), np.float16)
    dev = _stage_arrays(2, q, kc, vc, ks, kz, vs, vz, [1], Tcap)
    out, lse = _run(dev, 2, "channel", "channel", 128)
    score = 3 * 0.5 * 2 + 1 * 1.25 * 1 + 2 * 2.0 * 3 - 0.375 * 6
    assert abs(lse[0, 0] - score / math.sqrt(128)) < 1e-5


@pytest.mark.parametrize("vl", ["token", "channel"])
def test_receipt_value_side(vl):
    """Six equal keys give weights 1/6; value codes of channel 0 = (2,2,2,1,3,3)
    with s = 0.75, z = -1.125 -> out = (0.75*13 - 1.125*6)/6 = 0.5 exactly."""
    Tcap, T = 128, 6
    q = np.zeros((1, 4, D), np.float32)
    q[0, :, :4] = [0.5, -1.0, 2.0, 0.25]
    kc = np.ones((1, 1, Tcap, D), np.uint8)
    vc = np.zeros((1, 1, Tcap, D), np.uint8)
    vc[0, 0, :T, 0] = [2, 2, 2, 1, 3, 3]
    ks = np.ones((1, 1, Tcap, 1), np.float16)
    kz = np.zeros((1, 1, Tcap, 1), np.float16)
    if vl == "token":
        vs = np.full((1, 1, Tcap, 1), 0.75, np.float16)
        vz = np.full((1, 1, Tcap, 1), -1.125, np.float16)
    else:
        vs = np.full((1, 1, 1, D), 0.75, np.float16)
        vz = np.full((1, 1, 1, D), -1.125, np.float16)
    dev = _stage_arrays(2, q, kc, vc, ks, kz, vs, vz, [T], Tcap)
    out, lse = _run(dev, 2, "token", vl, 128)
    assert out[0, 0, 0] == 0.5
    score = (0.5 - 1.0 + 2.0 + 0.25) / math.sqrt(128)
    assert abs(lse[0, 0] - (math.log(6) + score)) < 1e-5


@pytest.mark.parametrize("vl", ["token", "channel"])
def test_constant_values_and_zero_query(vl):
    """s = 0, z = 0.75 everywhere: the output is 0.75 (softmax weights sum to 1);
    a zero query gives lse = ln T."""
    spec = synth.Spec("const", 14, 2, "token", vl, 128, 2, 8, 2, 128, 1024, lens=(1024, 333))
    from gpu_util import run, stage_spec
    dev, q, lens = stage_spec(spec)
    dev["v_scale"].zero_()
    dev["v_zero"].fill_(0.75)
    dev["q"].zero_()
    out, lse = run(spec, dev)
    np.testing.assert_array_equal(out, 0.75)
    np.testing.assert_allclose(lse[0], math.log(1024), atol=1e-5)
    np.testing.assert_allclose(lse[1], math.log(333), atol=1e-5)


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("pattern", ["random", "zeros", "max", "alternating", "high_bits"])
def test_pack_unpack_bit_exact(bits, pattern):
    import bit_quantized_kv_split_amd as fos
    import torch
    B, H, T = 2, 3, 256
    rng = np.random.default_rng(3)
    top = (1 << bits) - 1
    if pattern == "random":
        codes = rng.integers(0, top + 1, size=(B, H, T, D)).astype(np.uint8)
    elif pattern == "zeros":
        codes = np.zeros((B, H, T, D), np.uint8)
    elif pattern == "max":
        codes = np.full((B, H, T, D), top, np.uint8)
    elif pattern == "alternating":
        codes = ((np.indices((B, H, T, D)).sum(axis=0) % 2) * top).astype(np.uint8)
    else:  # bits above the code width are dropped by both packers
        codes = rng.integers(0, 256, size=(B, H, T, D)).astype(np.uint8)
    dc = torch.from_numpy(codes).cuda()
    for side, ref in ((fos.FOSCAR_SIDE_K, oracle.pack_k(codes, bits)), (fos.FOSCAR_SIDE_V, oracle.pack_v(codes, bits))):
        packed = fos.foscar_pack(bits, side, dc)
        torch.cuda.synchronize()
        got = packed.cpu().numpy().view(np.uint32)
        np.testing.assert_array_equal(got, ref)
        back = fos.foscar_unpack(bits, side, packed, codes.shape).cpu().numpy()
        np.testing.assert_array_equal(back, codes & top)


TARGETS = (0, 1, 2, 3, 4, 5, 7, 8, 15, 16, 17, 31, 33, 62, 63, 64, 65, 100, 127)


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("kl,vl,g", [("token", "token", 128), ("token", "token", 32), ("channel", "token", 128),
                                     ("token", "channel", 64), ("channel", "channel", 128)])
def test_one_hot_attention_selects_the_right_value_row(bits, kl, vl, g):
    """One token's score exceeds every other by about 34 nats, so softmax is
    one-hot to fp32 precision: the output must be that token's dequantised
    value row (s*q + z) and lse its score.  Run for targets at every position
    class of a 64-token tile; each sequence has its own target."""
    Tcap, T = 128, 128
    B = len(TARGETS)
    top = (1 << bits) - 1
    rng = np.random.default_rng(21)
    q = np.ones((B, 4, D), np.float32)
    kc = np.zeros((B, 1, Tcap, D), np.uint8)
    for b, t in enumerate(TARGETS):
        kc[b, 0, t, :] = top
    vc = rng.integers(0, top + 1, size=(B, 1, Tcap, D)).astype(np.uint8)
    if kl == "token":
        ks = np.full((B, 1, Tcap, D // g), 3.0 / top, np.float16)
        kz = np.zeros((B, 1, Tcap, D // g), np.float16)
    else:
        ks = np.full((B, 1, Tcap // g, D), 3.0 / top, np.float16)
        kz = np.zeros((B, 1, Tcap // g, D), np.float16)
    if vl == "token":
        vs = rng.uniform(0.1, 2.0, size=(B, 1, Tcap, D // g)).astype(np.float16)
        vz = rng.uniform(-3, 1, size=(B, 1, Tcap, D // g)).astype(np.float16)
    else:
        vs = rng.uniform(0.1, 2.0, size=(B, 1, Tcap // g, D)).astype(np.float16)
        vz = rng.uniform(-3, 1, size=(B, 1, Tcap // g, D)).astype(np.float16)
    dev = _stage_arrays(bits, q, kc, vc, ks, kz, vs, vz, [T] * B, Tcap)
    out, lse = _run(dev, bits, kl, vl, g)
    for b, t in enumerate(TARGETS):
        if vl == "token":
            s = np.repeat(vs[b, 0, t].astype(np.float64), g)
            z = np.repeat(vz[b, 0, t].astype(np.float64), g)
        else:
            s = vs[b, 0, t // g].astype(np.float64)
            z = vz[b, 0, t // g].astype(np.float64)
        expect = s * vc[b, 0, t] + z
        got = out[b, 0]
        bad = np.abs(got - expect) > 2e-3 + 2.0 ** -8 * np.abs(expect)
        assert not bad.any(), f"target token {t}: channels {np.nonzero(bad)[0][:8]} got {got[bad][:4]} want {expect[bad][:4]}"
        k_s = float(np.float16(3.0 / top))
        assert abs(lse[b, 0] - k_s * top * D / math.sqrt(D)) < 1e-3, f"target token {t}: lse {lse[b, 0]}"


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("kl,vl,g", [("token", "token", 128), ("token", "token", 32), ("token", "channel", 128),
                                     ("token", "channel", 32), ("channel", "channel", 64)])
def test_zero_query_gives_exact_mean_value(bits, kl, vl, g):
    """A zero query makes every score equal, so every softmax weight is
    exactly 1 before normalisation and the operand-folded weights P*s are the
    fp16 scales themselves (no rounding).  The output is the plain mean of the
    dequantised value rows and lse = ln T, to fp32 accumulation accuracy."""
    spec = synth.Spec(f"mean_{bits}_{kl}_{vl}_{g}", 15, bits, kl, vl, g, 3, 8, 2, 128, 2048, lens=(2048, 1500, 77),
                      channel_std_logu=(0.1, 10.0))
    from gpu_util import run, stage_spec
    dev, q, lens = stage_spec(spec)
    dev["q"].zero_()
    out, lse = run(spec, dev)
    for b in range(3):
        for h in range(2):
            head = synth.make_head(spec, b, h, seq_len=int(lens[b]))
            T = int(lens[b])
            vhat = oracle.dequantize(head["v_codes"][:T], head["v_scale"][:T] if vl == "token" else head["v_scale"][: -(-T // g)],
                                     head["v_zero"][:T] if vl == "token" else head["v_zero"][: -(-T // g)], vl, g)
            mean = vhat.mean(axis=0)
            for i in range(4 * h, 4 * h + 4):
                err = np.abs(out[b, i] - mean)
                scale = np.abs(vhat).mean(axis=0)
                assert np.all(err <= 1e-4 * scale + 2.0 ** -8 * np.abs(mean)), (
                    f"seq {b} head {i}: max err {err.max():.3e} at ch {np.argmax(err)}; mean {mean[np.argmax(err)]:.4f}")
            np.testing.assert_allclose(lse[b, 4 * h:4 * h + 4], math.log(T), atol=1e-5)


@pytest.mark.gpu
def test_occupancy_query_reports_resident_work_groups():
    """Every instantiation fits at least one work-group per CU; the INT2
    token-wise kernel of the long-context workload fits four."""
    import bit_quantized_kv_split_amd as fos
    for bits in (2, 4):
        for layout in range(4):
            for g in (32, 64, 128):
                assert fos.foscar_occupancy(bits, layout, g) >= 1
    print("INT2 token-wise g=128 work-groups per CU:", fos.foscar_occupancy(2, 0, 128))
