"""Pins of the oracle's quantiser (oracle/quantize.py) to facts outside it.

* exact recovery: values that lie on a known grid z + s*k (s, z fp16-exact,
  k the codes, every group holding its lowest and highest code) come back as
  exactly those codes, scales and offsets -- value = s*q + z is the cache
  encoding of the FOSCAR explainer (encoding paragraph); different grids per
  group catch a group taken along the wrong axis;
* a constant group stores s = 0, q = 0 and the value itself as offset;
* ties round half to even;
* the rounding error bound of a min-max quantiser;
* an independent quantiser (the input generator's, fp64 quotient) agrees
  except where the two precisions round a quotient at a half differently;
* appending token by token (group by group) equals appending at once;
  writes outside the range, unaligned channel-wise starts and out-of-range
  starts leave the cache as it was.
"""
import math

import numpy as np
import pytest

import oracle
import oracle.quantize as oq
import synth


def _empty_cache(B, H, T, D, bits, k_layout, v_layout, g, rng):
    def sshape(layout):
        return (B, H, T, D // g) if layout == "token" else (B, H, T // g, D)
    c = {
        "k_codes": rng.integers(0, 1 << bits, (B, H, T, D), dtype=np.uint8),
        "v_codes": rng.integers(0, 1 << bits, (B, H, T, D), dtype=np.uint8),
    }
    for side, layout in (("k", k_layout), ("v", v_layout)):
        for part in ("scale", "zero"):
            c[f"{side}_{part}"] = rng.standard_normal(sshape(layout)).astype(np.float16)
    return c


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("k_layout,v_layout", [("token", "token"), ("channel", "channel"), ("token", "channel")])
@pytest.mark.parametrize("g", [4, 8])
def test_grid_values_recovered_exactly(bits, k_layout, v_layout, g):
    rng = np.random.default_rng(11)
    B, H, T, D = 2, 2, 32, 16
    L = (1 << bits) - 1
    cache = _empty_cache(B, H, T, D, bits, k_layout, v_layout, g, rng)
    srcs, want = {}, {}
    for side, layout in (("k", k_layout), ("v", v_layout)):
        k = rng.integers(0, L + 1, (B, H, T, D))
        if layout == "token":
            gs = (B, H, T, D // g)
            s = rng.integers(1, 256, gs) / 64.0
            z = rng.integers(-256, 256, gs) / 64.0
            kv = k.reshape(B, H, T, D // g, g)
            kv[..., 0], kv[..., 1] = 0, L                       # lowest and highest code in every group
            x = z[..., None] + s[..., None] * kv
            x = x.reshape(B, H, T, D)
        else:
            gs = (B, H, T // g, D)
            s = rng.integers(1, 256, gs) / 64.0
            z = rng.integers(-256, 256, gs) / 64.0
            kv = k.reshape(B, H, T // g, g, D)
            kv[:, :, :, 0, :], kv[:, :, :, 1, :] = 0, L
            x = z[:, :, :, None, :] + s[:, :, :, None, :] * kv
            x = x.reshape(B, H, T, D)
        srcs[side] = x.astype(np.float32)
        want[side] = (kv.reshape(B, H, T, D), s, z)
    out = oq.quantize_append(cache, srcs["k"], srcs["v"], np.zeros(B, int), np.full(B, T), bits=bits,
                             k_layout=k_layout, v_layout=v_layout, group=g)
    for side in ("k", "v"):
        k, s, z = want[side]
        assert np.array_equal(out[f"{side}_codes"], k)
        assert np.array_equal(out[f"{side}_scale"].astype(np.float64), s)
        assert np.array_equal(out[f"{side}_zero"].astype(np.float64), z)


@pytest.mark.parametrize("bits", [2, 4])
def test_constant_group(bits):
    q, s, z = oq.quantize_group(np.full(8, 0.3, np.float32), bits)
    assert s == 0 and z == np.float16(0.3) and not q.any()


def test_ties_round_half_to_even():
    q, s, z = oq.quantize_group(np.array([0, 3, 0.5, 1.5, 2.5], np.float32), 2)
    assert (s, z) == (1, 0) and q.tolist() == [0, 3, 0, 2, 2]
    q, s, z = oq.quantize_group(np.array([0, 15, 0.5, 1.5, 2.5, 7.5, 14.5], np.float32), 4)
    assert (s, z) == (1, 0) and q.tolist() == [0, 15, 0, 2, 2, 8, 14]


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("scale", [1.0, 10.0, 0.01])
def test_rounding_error_bound(bits, scale):
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((500, 64)) * scale).astype(np.float32)
    q, s16, z16 = oq.quantize_group(x, bits, axis=1)
    L = (1 << bits) - 1
    s = s16.astype(np.float64)[:, None]
    z = z16.astype(np.float64)[:, None]
    x64 = x.astype(np.float64)
    mn, mx = x64.min(1, keepdims=True), x64.max(1, keepdims=True)
    err = np.abs(x64 - (s * q + z))
    bound = 0.5 * s + L * np.abs((mx - mn) / L - s) + np.abs(mn - z) + 1e-6 * np.abs(x64).max()
    assert (err <= bound).all()
    assert q.min() == 0 and q.max() == L
    # codes 0 and L are reached by the group's own minimum and maximum
    assert (q[np.arange(len(x)), x.argmin(1)] == 0).all()


@pytest.mark.parametrize("bits", [2, 4])
def test_agrees_with_independent_quantiser(bits):
    rng = np.random.default_rng(5)
    x = synth.bf16_round(rng.standard_normal((2000, 128)).astype(np.float32))
    q, s, z = oq.quantize_group(x, bits, axis=1)
    q2, s2, z2 = synth.quantize_minmax(x, bits, axis=1)
    assert np.array_equal(s, s2) and np.array_equal(z, z2)
    diff = q != q2
    assert diff.mean() < 1e-4
    # where they differ, the exact quotient sits at a half: the two precisions round it differently
    quot = (x.astype(np.float64) - z.astype(np.float64)[:, None]) / s.astype(np.float64)[:, None]
    assert (np.abs(np.abs(quot - np.floor(quot)) - 0.5)[diff] < 1e-5).all()
    assert (np.abs(q.astype(int) - q2.astype(int)) <= 1).all()


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("k_layout,v_layout", [("token", "token"), ("channel", "channel"), ("token", "channel")])
def test_append_order_independent(bits, k_layout, v_layout):
    rng = np.random.default_rng(7)
    B, H, T, D, g = 2, 2, 64, 16, 8
    cache = _empty_cache(B, H, T, D, bits, k_layout, v_layout, g, rng)
    n = 45  # ends inside a channel-wise group
    ks = rng.standard_normal((B, H, n, D)).astype(np.float32)
    vs = rng.standard_normal((B, H, n, D)).astype(np.float32)
    kw = dict(bits=bits, k_layout=k_layout, v_layout=v_layout, group=g)
    once = oq.quantize_append(cache, ks, vs, np.zeros(B, int), np.full(B, n), **kw)
    step = 1 if "channel" not in (k_layout, v_layout) else g
    inc = cache
    for t0 in range(0, n, step):
        t1 = min(t0 + step, n)
        inc = oq.quantize_append(inc, ks[:, :, t0:t1], vs[:, :, t0:t1], np.full(B, t0), np.full(B, t1 - t0), **kw)
    for name in once:
        assert np.array_equal(once[name].view(np.uint8), inc[name].view(np.uint8)), name


def test_out_of_range_writes_nothing():
    rng = np.random.default_rng(9)
    B, H, T, D, g = 4, 1, 32, 8, 8
    cache = _empty_cache(B, H, T, D, 2, "channel", "token", g, rng)
    src = rng.standard_normal((B, H, 10, D)).astype(np.float32)
    # unaligned channel-wise start, start past Tcap, negative start, zero count
    out = oq.quantize_append(cache, src, src, np.array([3, T + 1, -8, 8]), np.array([5, 5, 5, 0]), bits=2,
                             k_layout="channel", v_layout="token", group=g)
    for name in cache:
        assert np.array_equal(out[name].view(np.uint8), cache[name].view(np.uint8)), name
    # count is clamped to the capacity: 10 requested at start 24 writes tokens 24..31 only
    cache = _empty_cache(B, H, T, D, 2, "token", "token", g, rng)
    out = oq.quantize_append(cache, src, src, np.array([24] * B), np.array([10] * B), bits=2,
                             k_layout="token", v_layout="token", group=g)
    assert np.array_equal(out["k_codes"][:, :, :24], cache["k_codes"][:, :, :24])
    assert not np.array_equal(out["k_scale"][:, :, 24:], cache["k_scale"][:, :, 24:])


# ---------------------------------------------------------------- rotated writer

def test_inv_sqrt_is_correctly_rounded():
    """1/sqrt(d) in fp64 within half an ulp of the exact value (50-digit decimal)."""
    from decimal import Decimal, getcontext
    getcontext().prec = 50
    for k in range(0, 12):
        d = 1 << k
        c = oq.inv_sqrt(d)
        exact = 1 / Decimal(d).sqrt()
        assert abs(Decimal(c) - exact) <= Decimal(math.ulp(c)) / 2, d


def test_rotate_rows_unit_vectors_and_fp64_product():
    """e_j H is row j of the +-1 matrix times 1/sqrt(D) (held in fp32);
    random bf16 rows agree with the fp64 product by the orthonormal matrix to
    fp32 rounding."""
    S = oracle.sylvester(128)
    c32 = np.float32(oq.inv_sqrt(128))
    for j in (0, 1, 77, 127):
        e = np.zeros(128)
        e[j] = 1.0
        np.testing.assert_array_equal(oq.rotate_rows(e), (S[j] * c32).astype(np.float32))
    rng = np.random.default_rng(81)
    x = synth.bf16_round(rng.standard_normal((64, 128)).astype(np.float32)).astype(np.float64)
    y = oq.rotate_rows(x).astype(np.float64)
    ref = x @ oracle.hadamard(128)
    assert np.abs(y - ref).max() <= 2.0 ** -23 * np.abs(ref).max()
    np.testing.assert_allclose(oq.rotate_rows(y) , x, atol=1e-5)  # H H = I up to the fp32 roundings


@pytest.mark.parametrize("rotate", ["k", "v", "kv"])
def test_rotated_append_quantises_rotated_rows(rotate):
    """quantize_append(rotate=...) equals quantize_append of rows rotated
    beforehand, side by side (the unnamed side untouched)."""
    rng = np.random.default_rng(82)
    B, H, T, N, g = 2, 1, 128, 70, 32
    cache = {"k_codes": np.zeros((B, H, T, 128), np.uint8), "v_codes": np.zeros((B, H, T, 128), np.uint8)}
    for n in ("k_scale", "k_zero"):
        cache[n] = np.zeros((B, H, T, 128 // g), np.float16)
    for n in ("v_scale", "v_zero"):
        cache[n] = np.zeros((B, H, T // g, 128), np.float16)
    ks = synth.bf16_round(rng.standard_normal((B, H, N, 128)).astype(np.float32))
    vs = synth.bf16_round(rng.standard_normal((B, H, N, 128)).astype(np.float32))
    kw = dict(bits=2, k_layout="token", v_layout="channel", group=g)
    got = oq.quantize_append(cache, ks, vs, [0, 32], [70, 50], rotate=rotate, **kw)
    want = oq.quantize_append(cache, oq.rotate_rows(ks) if "k" in rotate else ks,
                              oq.rotate_rows(vs) if "v" in rotate else vs, [0, 32], [70, 50], **kw)
    for name in got:
        np.testing.assert_array_equal(got[name], want[name])
    plain = oq.quantize_append(cache, ks, vs, [0, 32], [70, 50], **kw)
    for side in ("k", "v"):
        same = np.array_equal(got[side + "_codes"], plain[side + "_codes"])
        assert same == (side not in rotate)
