"""The seeded input generator: quantiser properties, shapes, reproducibility."""
import numpy as np
import pytest

import synth


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("axis", [0, 1])
def test_quantiser_range_and_error(bits, axis):
    rng = np.random.default_rng(0)
    x = rng.standard_normal((64, 32)).astype(np.float32) * 3
    q, s, z = synth.quantize_minmax(x, bits, axis=axis)
    assert q.dtype == np.uint8 and q.max() <= (1 << bits) - 1
    s64 = np.expand_dims(s.astype(np.float64), axis)
    z64 = np.expand_dims(z.astype(np.float64), axis)
    err = np.abs(x - (s64 * q + z64))
    # half a step, plus the fp16 rounding of s and z
    bound = s64 / 2 + np.abs(s64) * ((1 << bits) - 1) * 2 ** -10 + np.abs(z64) * 2 ** -10 + 1e-6
    assert np.all(err <= bound)
    # the group minimum maps to code 0 and the maximum to the top code (up to fp16 rounding)
    assert np.all(q.min(axis=axis) == 0)


def test_constant_group():
    x = np.full((4, 8), 1.25, np.float32)
    q, s, z = synth.quantize_minmax(x, 2, axis=1)
    assert np.all(q == 0) and np.all(s == 0) and np.all(z == np.float16(1.25))


def test_bf16_round():
    x = np.array([1.0, 1.00390625, 1.005859375, -3.14159, 0.0], np.float32)
    r = synth.bf16_round(x)
    assert r[0] == 1.0 and r[1] == 1.0          # tie to even
    assert r[2] == np.float32(1.0078125)        # rounds up
    assert np.all((r.view(np.uint32) & 0xFFFF) == 0)


def test_head_slices_are_reproducible_and_match_workload():
    spec = synth.SPECS["c5_ragged_int2_g64"].replace(batch=3, max_seq_len=256, ragged_lo=16)
    w = synth.make_workload(spec, threads=2)
    lens = spec.seq_lens()
    assert np.all((lens >= 16) & (lens <= 256))
    for b, h in [(0, 0), (2, 7)]:
        head = synth.make_head(spec, b, h)
        for k, v in head.items():
            np.testing.assert_array_equal(w[k][b, h], v)
        t = int(lens[b])
        assert np.all(w["k_codes"][b, h, t:] == 0)
        assert np.all(w["k_scale"][b, h, t:] == 0)


def test_poison_marks_only_padding():
    spec = synth.SPECS["c5_ragged_int4_g32"].replace(batch=2, max_seq_len=256, ragged_lo=16)
    clean = synth.make_head(spec, 1, 3)
    dirty = synth.make_head(spec, 1, 3, poison=True)
    t = int(spec.seq_lens()[1])
    np.testing.assert_array_equal(clean["k_codes"][:t], dirty["k_codes"][:t])
    np.testing.assert_array_equal(clean["v_scale"][: -(-t // 32)], dirty["v_scale"][: -(-t // 32)])
    if t < 256:
        assert np.all(np.isnan(dirty["k_scale"][t:]))


def test_outliers_and_channel_std():
    spec = synth.SPECS["c2_paper_int2"].replace(batch=1, max_seq_len=512)
    ch = synth._outlier_channels(spec, 0)
    assert len(ch) == 6 and len(set(ch.tolist())) == 6
    spec4 = synth.SPECS["c4_channel_int2"]
    std = synth._channel_std(spec4, 0, 0)
    assert std.min() >= 0.1 and std.max() <= 10.0


def test_append_case_and_window_generators_are_seeded_and_shaped():
    """The quantise-and-append and window inputs regenerate bit for bit from
    their seed, hold bf16 values, and have the interface's shapes."""
    a = synth.make_append_case(3, 2, 2, 256, 100, 2, [0, 64], [100, 10])
    b = synth.make_append_case(3, 2, 2, 256, 100, 2, [0, 64], [100, 10])
    for k in a:
        assert np.array_equal(a[k], b[k]), k
    assert a["k_src"].shape == (2, 2, 100, 128) and a["packed_k"].shape == (2, 2, 256, 8)
    assert a["packed_v"].shape == (2, 2, 16, 128) and a["k_scale_channel"].shape == (2, 2, 8, 128)
    assert np.array_equal(synth.bf16_round(a["k_src"]), a["k_src"])
    c = synth.make_append_case(4, 2, 2, 256, 100, 2, [0, 64], [100, 10])
    assert not np.array_equal(a["k_src"], c["k_src"])
    w1 = synth.make_window(5, 3, 2, 40, [40, 0, 7])
    w2 = synth.make_window(5, 3, 2, 40, [40, 0, 7])
    assert all(np.array_equal(w1[k], w2[k]) for k in w1)
    assert w1["k"].shape == (3, 2, 40, 128) and w1["lens"].dtype == np.int32
    assert np.array_equal(synth.bf16_round(w1["v"]), w1["v"])


def test_rotated_cache_holds_rotated_rows():
    """Spec.rotate: the stored rows dequantise to the drawn rows times the
    orthonormal Hadamard matrix (within the quantisation step), and the sides
    it does not name are the unrotated cache, code for code."""
    import oracle
    spec = synth.Spec("rot_gen", 40, 4, "token", "channel", 32, 1, 4, 1, 128, 256, channel_std_logu=(0.1, 10.0))
    plain = synth.make_head(spec, 0, 0)
    rot = synth.make_head(spec.replace(rotate="k"), 0, 0)
    for name in ("v_codes", "v_scale", "v_zero"):
        np.testing.assert_array_equal(rot[name], plain[name])
    H = oracle.hadamard(128)

    def deq(w):
        s = np.repeat(w["k_scale"].astype(np.float64), 32, axis=1)
        return s * w["k_codes"] + np.repeat(w["k_zero"].astype(np.float64), 32, axis=1)
    kp, kr = deq(plain), deq(rot)
    step = np.repeat(rot["k_scale"].astype(np.float64), 32, axis=1)
    # rotating the plain rows back and forth: kr H^T ~ kp, each side within its own quantisation step
    err = np.abs(kr @ H.T - kp)
    assert err.mean() < 0.5 * (step.mean() + np.repeat(plain["k_scale"].astype(np.float64), 32, axis=1).mean())
    assert np.abs(kr - kp).mean() > 10 * err.mean()  # and the stored rows did change
