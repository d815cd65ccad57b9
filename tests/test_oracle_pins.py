"""Pins of the CPU oracle to facts outside itself.

* the worked receipt of the FOSCAR explainer (receipt paragraph), both the
  shared-rate form (acc-fold) and the own-rate-per-line form (operand-fold);
* exact fold-vs-unfold equality on tiny inputs, for the four fold cases of the
  explainer's fold-placement table, in rational arithmetic (the abstract
  states the fold preserves the dequantised output in exact arithmetic);
* closed forms (zero query, one token, constant values, empty sequence);
* invariants (token permutation, GQA replication, offset shift, softmax sums);
* a textbook special case (s = 1, z = 0) against a library attention routine
  and a brute-force loop;
* golden packed words derived by hand from the layout specification.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_receipt():
    vals = {}
    with open(os.path.join(GOLDEN, "receipt.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            k, *v = line.split()
            vals[k] = [int(x) for x in v]
    return vals


def _one_head(q_rows, k_codes, v_codes, ks, kz, vs, vz, seq_len=None):
    """Wrap single-head arrays into the oracle's batched dict (B = 1, Hkv = 1)."""
    q_rows = np.atleast_2d(np.asarray(q_rows, dtype=np.float64))
    T = k_codes.shape[0]
    return {
        "q": q_rows[None],
        "k_codes": np.asarray(k_codes)[None, None],
        "v_codes": np.asarray(v_codes)[None, None],
        "k_scale": np.asarray(ks, np.float16)[None, None],
        "k_zero": np.asarray(kz, np.float16)[None, None],
        "v_scale": np.asarray(vs, np.float16)[None, None],
        "v_zero": np.asarray(vz, np.float16)[None, None],
        "seq_lens": np.array([T if seq_len is None else seq_len], np.int32),
    }


# ---------------------------------------------------------------- receipt

@pytest.mark.parametrize("s,z", [(0.75, -1.125), (1.5, 0.25), (0.0625, 3.0), (2.0, -0.5)])
def test_receipt_key_side_shared_rate(s, z):
    """One token, three channels in one token-wise group: the score equals
    rate*13 + fee*6 (explainer, receipt paragraph)."""
    r = _read_receipt()
    qty, stk = r["quantities"], r["stickers"]
    assert sum(a * b for a, b in zip(qty, stk)) == r["weighted_subtotal"][0] == 13
    assert sum(qty) == r["total_quantity"][0] == 6
    D = 3
    k_codes = np.array([stk], np.uint8)
    w = _one_head([qty], k_codes, np.zeros((1, D), np.uint8), [[s]], [[z]], [[0.0]], [[0.0]])
    out, lse = oracle.decode(w, k_layout="token", v_layout="token", group=D, sm_scale=1.0)
    # T = 1: lse is the (scaled) score itself
    assert lse[0, 0] == s * 13 + z * 6


@pytest.mark.parametrize("rates", [(0.5, 1.25, 2.0), (3.0, 0.125, 0.75)])
def test_receipt_key_side_own_rate_per_line(rates):
    """Every line has its own rate: the quantities are pre-multiplied by their
    line's rate and the fee still multiplies the total quantity (explainer,
    receipt paragraph, last sentence) -- channel-wise K, one token."""
    r = _read_receipt()
    qty, stk = r["quantities"], r["stickers"]
    fee = -0.375
    k_codes = np.array([stk], np.uint8)
    ks = np.array([rates], np.float16)
    kz = np.full((1, 3), fee, np.float16)
    w = _one_head([qty], k_codes, np.zeros((1, 3), np.uint8), ks, kz, np.zeros((1, 3)), np.zeros((1, 3)))
    out, lse = oracle.decode(w, k_layout="channel", v_layout="channel", group=1, sm_scale=1.0)
    expect = sum((a * rt) * b for a, rt, b in zip(qty, rates, stk)) + fee * sum(qty)
    assert lse[0, 0] == expect


@pytest.mark.parametrize("v_layout", ["token", "channel"])
def test_receipt_value_side(v_layout):
    """Six tokens with equal keys give equal weights 1/6; value codes of
    channel 0 are the receipt's stickers repeated by quantity (2,2,2,1,3,3), so
    out[0] = (s*13 + z*6) / 6 (explainer receipt with the softmax weights as
    the quantities)."""
    r = _read_receipt()
    codes = sum(([st] * qt for qt, st in zip(r["quantities"], r["stickers"])), [])
    assert codes == [2, 2, 2, 1, 3, 3]
    T, D, s, z = 6, 4, 0.75, -1.125
    k_codes = np.ones((T, D), np.uint8)
    v_codes = np.zeros((T, D), np.uint8)
    v_codes[:, 0] = codes
    if v_layout == "token":
        vs, vz, g = np.full((T, 1), s), np.full((T, 1), z), D
    else:
        vs, vz, g = np.full((1, D), s), np.full((1, D), z), T
    w = _one_head([[0.5, -1.0, 2.0, 0.25]], k_codes, v_codes, np.ones((T, 1)), np.zeros((T, 1)), vs, vz)
    out, lse = oracle.decode(w, k_layout="token", v_layout=v_layout, group=g if v_layout == "channel" else D,
                             sm_scale=0.5) if v_layout == "channel" else \
        oracle.decode(w, k_layout="token", v_layout=v_layout, group=D, sm_scale=0.5)
    assert abs(out[0, 0, 0] - (s * 13 + z * 6) / 6) < 1e-15
    assert abs(out[0, 0, 0] - 0.5) < 1e-15
    score = 0.5 * (0.5 - 1.0 + 2.0 + 0.25)
    assert abs(lse[0, 0] - (math.log(6) + score)) < 1e-14


# ---------------------------------------------------- exact fold vs unfold

def _fold_scores(Q, kq, ks, kz, layout, g, sigma):
    """Pre-softmax scores by the fold rules of the explainer's table, in Fractions.

    token-wise K (acc-fold): sigma * sum_j [ s_tj * sum_{c in j} Q_c q_tc + z_tj * sum_{c in j} Q_c ]
    channel-wise K (operand-fold): sigma * [ sum_c (Q_c s_{tau,c}) q_tc + sum_c Q_c z_{tau,c} ]
    """
    T, D = kq.shape
    S = []
    for t in range(T):
        if layout == "token":
            tot = Fraction(0)
            for j in range(D // g):
                part = sum(Q[c] * int(kq[t, c]) for c in range(j * g, (j + 1) * g))
                qsum = sum(Q[c] for c in range(j * g, (j + 1) * g))
                tot += Fraction(float(ks[t, j])) * part + Fraction(float(kz[t, j])) * qsum
        else:
            tau = t // g
            tot = sum((Q[c] * Fraction(float(ks[tau, c]))) * int(kq[t, c]) for c in range(D)) \
                + sum(Q[c] * Fraction(float(kz[tau, c])) for c in range(D))
        S.append(sigma * tot)
    return S


def _fold_pv(P, vq, vs, vz, layout, g):
    """Unnormalised PV by the fold rules, in Fractions (P given as Fractions).

    token-wise V (operand-fold): sum_t (p_t s_{t,j(c)}) q_tc + sum_t p_t z_{t,j(c)}
    channel-wise V (acc-fold): sum_tau [ s_{tau,c} sum_{t in tau} p_t q_tc + z_{tau,c} sum_{t in tau} p_t ]
    """
    T, D = vq.shape
    out = []
    for c in range(D):
        if layout == "token":
            j = c // g
            acc = sum((P[t] * Fraction(float(vs[t, j]))) * int(vq[t, c]) for t in range(T)) \
                + sum(P[t] * Fraction(float(vz[t, j])) for t in range(T))
        else:
            acc = Fraction(0)
            for tau in range(-(-T // g)):
                ts = range(tau * g, min((tau + 1) * g, T))
                part = sum(P[t] * int(vq[t, c]) for t in ts)   # never crosses a group boundary
                psum = sum(P[t] for t in ts)
                acc += Fraction(float(vs[tau, c])) * part + Fraction(float(vz[tau, c])) * psum
        out.append(acc)
    return out


def _unfold_scores(Q, kq, ks, kz, layout, g, sigma):
    """Dequantise each value first, then dot -- in Fractions."""
    T, D = kq.shape
    S = []
    for t in range(T):
        tot = Fraction(0)
        for c in range(D):
            if layout == "token":
                s, z = ks[t, c // g], kz[t, c // g]
            else:
                s, z = ks[t // g, c], kz[t // g, c]
            tot += Q[c] * (Fraction(float(s)) * int(kq[t, c]) + Fraction(float(z)))
        S.append(sigma * tot)
    return S


def _dyadic_fp16(rng, shape, lo=-2.0, hi=2.0):
    return rng.uniform(lo, hi, size=shape).astype(np.float16)


FOLD_CASES = [
    # (k_layout, v_layout, bits, G, D, g, T, Tcap)
    ("token", "token", 2, 4, 8, 4, 7, 8),
    ("token", "channel", 2, 2, 8, 4, 11, 12),
    ("channel", "token", 4, 1, 8, 2, 5, 6),
    ("channel", "channel", 4, 4, 16, 8, 13, 16),
    ("token", "channel", 4, 2, 16, 8, 20, 24),
    ("channel", "channel", 2, 2, 8, 4, 9, 12),
]


@pytest.mark.parametrize("case", FOLD_CASES)
def test_fold_equals_unfold_exact_and_oracle(case):
    k_layout, v_layout, bits, G, D, g, T, Tcap = case
    rng = np.random.default_rng(sum(map(hash, map(str, case))) % (2 ** 32))
    Hkv = 2
    Hq = G * Hkv
    sigma = Fraction(1, 4)
    levels = (1 << bits) - 1
    kq = rng.integers(0, levels + 1, size=(Hkv, Tcap, D)).astype(np.uint8)
    vq = rng.integers(0, levels + 1, size=(Hkv, Tcap, D)).astype(np.uint8)

    def sz(layout):
        shp = (Hkv, Tcap, D // g) if layout == "token" else (Hkv, Tcap // g, D)
        return _dyadic_fp16(rng, shp, 0.05, 2.0), _dyadic_fp16(rng, shp)

    ks, kz = sz(k_layout)
    vs, vz = sz(v_layout)
    q = synth.bf16_round(rng.standard_normal((1, Hq, D)).astype(np.float32))
    w = {"q": q, "k_codes": kq[None], "v_codes": vq[None], "k_scale": ks[None], "k_zero": kz[None],
         "v_scale": vs[None], "v_zero": vz[None], "seq_lens": np.array([T], np.int32)}
    out, lse = oracle.decode(w, k_layout=k_layout, v_layout=v_layout, group=g, sm_scale=float(sigma))
    for i in range(Hq):
        h = i // G
        Q = [Fraction(float(x)) for x in q[0, i]]
        Sf = _fold_scores(Q, kq[h, :T], ks[h], kz[h], k_layout, g, sigma)
        Su = _unfold_scores(Q, kq[h, :T], ks[h], kz[h], k_layout, g, sigma)
        assert Sf == Su                                      # exact: folding changes nothing
        m = max(Sf)
        wts = [Fraction(math.exp(float(s - m))) for s in Sf]
        l = sum(wts)
        pv = _fold_pv(wts, vq[h, :T], vs[h], vz[h], v_layout, g)
        # unfolded PV in Fractions
        for c in range(D):
            unf = Fraction(0)
            for t in range(T):
                if v_layout == "token":
                    s_, z_ = vs[h, t, c // g], vz[h, t, c // g]
                else:
                    s_, z_ = vs[h, t // g, c], vz[h, t // g, c]
                unf += wts[t] * (Fraction(float(s_)) * int(vq[h, t, c]) + Fraction(float(z_)))
            assert unf == pv[c]                              # exact
        o_fold = np.array([float(x / l) for x in pv])
        lse_fold = float(m) + math.log(float(l))
        np.testing.assert_allclose(out[0, i], o_fold, rtol=1e-12, atol=1e-12)
        assert abs(lse[0, i] - lse_fold) <= 1e-12 * max(1.0, abs(lse_fold))


# ---------------------------------------------------------- closed forms

def _rand_case(rng, T=37, Tcap=40, D=16, g=8, k_layout="token", v_layout="channel", G=2, bits=2):
    Hkv = 1
    levels = (1 << bits) - 1
    kq = rng.integers(0, levels + 1, size=(1, Hkv, Tcap, D)).astype(np.uint8)
    vq = rng.integers(0, levels + 1, size=(1, Hkv, Tcap, D)).astype(np.uint8)

    def sz(layout):
        shp = (1, Hkv, Tcap, D // g) if layout == "token" else (1, Hkv, Tcap // g, D)
        return _dyadic_fp16(rng, shp, 0.05, 2.0), _dyadic_fp16(rng, shp)

    ks, kz = sz(k_layout)
    vs, vz = sz(v_layout)
    q = synth.bf16_round(rng.standard_normal((1, G * Hkv, D)).astype(np.float32))
    return {"q": q, "k_codes": kq, "v_codes": vq, "k_scale": ks, "k_zero": kz, "v_scale": vs,
            "v_zero": vz, "seq_lens": np.array([T], np.int32)}


@pytest.mark.parametrize("k_layout,v_layout", [("token", "token"), ("channel", "channel"), ("token", "channel")])
def test_zero_query_gives_mean_value(k_layout, v_layout):
    rng = np.random.default_rng(1)
    w = _rand_case(rng, k_layout=k_layout, v_layout=v_layout)
    w["q"][:] = 0
    out, lse = oracle.decode(w, k_layout=k_layout, v_layout=v_layout, group=8, sm_scale=0.3)
    T = int(w["seq_lens"][0])
    vq = w["v_codes"][0, 0, :T].astype(np.float64)
    if v_layout == "token":
        s = np.repeat(w["v_scale"][0, 0, :T].astype(np.float64), 8, axis=1)
        z = np.repeat(w["v_zero"][0, 0, :T].astype(np.float64), 8, axis=1)
    else:
        s = np.repeat(w["v_scale"][0, 0].astype(np.float64), 8, axis=0)[:T]
        z = np.repeat(w["v_zero"][0, 0].astype(np.float64), 8, axis=0)[:T]
    mean = np.mean(s * vq + z, axis=0)
    np.testing.assert_allclose(out[0, 0], mean, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(lse[0], math.log(T), rtol=1e-14)


def test_single_token_gives_its_value():
    rng = np.random.default_rng(2)
    w = _rand_case(rng, T=1, k_layout="token", v_layout="token")
    out, lse = oracle.decode(w, k_layout="token", v_layout="token", group=8, sm_scale=0.3)
    s = np.repeat(w["v_scale"][0, 0, 0].astype(np.float64), 8)
    z = np.repeat(w["v_zero"][0, 0, 0].astype(np.float64), 8)
    v0 = s * w["v_codes"][0, 0, 0] + z
    ks = np.repeat(w["k_scale"][0, 0, 0].astype(np.float64), 8)
    kz = np.repeat(w["k_zero"][0, 0, 0].astype(np.float64), 8)
    k0 = ks * w["k_codes"][0, 0, 0] + kz
    for i in range(2):
        np.testing.assert_array_equal(out[0, i], v0)
        assert abs(lse[0, i] - 0.3 * float(np.dot(w["q"][0, i].astype(np.float64), k0))) < 1e-13


@pytest.mark.parametrize("v_layout", ["token", "channel"])
def test_constant_values(v_layout):
    """s = 0 and z = c in every value group -> the output is c everywhere
    (softmax weights sum to one)."""
    rng = np.random.default_rng(3)
    w = _rand_case(rng, v_layout=v_layout)
    w["v_scale"][:] = 0
    w["v_zero"][:] = 0.75
    out, _ = oracle.decode(w, k_layout="token", v_layout=v_layout, group=8, sm_scale=0.3)
    np.testing.assert_allclose(out, 0.75, rtol=0, atol=1e-15)


def test_empty_sequence():
    rng = np.random.default_rng(4)
    w = _rand_case(rng)
    w["seq_lens"][:] = 0
    out, lse = oracle.decode(w, k_layout="token", v_layout="channel", group=8, sm_scale=0.3)
    assert np.all(out == 0)
    assert np.all(np.isneginf(lse))


def test_padding_past_length_is_ignored():
    rng = np.random.default_rng(5)
    w = _rand_case(rng, T=29)
    out1, lse1 = oracle.decode(w, k_layout="token", v_layout="channel", group=8, sm_scale=0.3)
    w["k_codes"][0, 0, 29:] = 3
    w["v_codes"][0, 0, 29:] = 3
    w["k_scale"][0, 0, 29:] = np.nan
    w["v_scale"][0, 0, 4:] = np.nan          # channel-wise groups starting at token 32
    out2, lse2 = oracle.decode(w, k_layout="token", v_layout="channel", group=8, sm_scale=0.3)
    np.testing.assert_array_equal(out1, out2)
    np.testing.assert_array_equal(lse1, lse2)


# ----------------------------------------------------------- invariants

def test_token_permutation_invariance():
    """Token-wise K and V: permuting tokens together with their (s, z) rows
    changes nothing (attention is a set operation over tokens)."""
    rng = np.random.default_rng(6)
    w = _rand_case(rng, T=40, k_layout="token", v_layout="token")
    out1, lse1 = oracle.decode(w, k_layout="token", v_layout="token", group=8, sm_scale=0.3)
    perm = rng.permutation(40)
    w2 = dict(w)
    for k in ("k_codes", "v_codes", "k_scale", "k_zero", "v_scale", "v_zero"):
        w2[k] = w[k][:, :, perm]
    out2, lse2 = oracle.decode(w2, k_layout="token", v_layout="token", group=8, sm_scale=0.3)
    np.testing.assert_allclose(out1, out2, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse1, lse2, rtol=1e-14)


def test_group_permutation_invariance_channel_wise():
    rng = np.random.default_rng(7)
    w = _rand_case(rng, T=40, k_layout="channel", v_layout="channel")
    out1, lse1 = oracle.decode(w, k_layout="channel", v_layout="channel", group=8, sm_scale=0.3)
    gperm = rng.permutation(5)
    tperm = np.concatenate([np.arange(8) + 8 * gg for gg in gperm])
    w2 = dict(w)
    for k in ("k_codes", "v_codes"):
        w2[k] = w[k][:, :, tperm]
    for k in ("k_scale", "k_zero", "v_scale", "v_zero"):
        w2[k] = w[k][:, :, gperm]
    out2, lse2 = oracle.decode(w2, k_layout="channel", v_layout="channel", group=8, sm_scale=0.3)
    np.testing.assert_allclose(out1, out2, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse1, lse2, rtol=1e-14)


def test_key_offset_shift():
    """Token-wise K with one group per token: adding d to every key offset adds
    sigma*d*sum(Q_i) to every score of query i, so the output is unchanged and
    lse moves by exactly that amount."""
    rng = np.random.default_rng(8)
    w = _rand_case(rng, T=33, D=16, g=16, k_layout="token", v_layout="token")
    # offsets on a 1/64 grid so that z + 0.5 stays exact in fp16
    w["k_zero"] = (np.round(w["k_zero"].astype(np.float64) * 64) / 64).astype(np.float16)
    out1, lse1 = oracle.decode(w, k_layout="token", v_layout="token", group=16, sm_scale=0.3)
    w2 = dict(w)
    w2["k_zero"] = (w["k_zero"].astype(np.float64) + 0.5).astype(np.float16)
    out2, lse2 = oracle.decode(w2, k_layout="token", v_layout="token", group=16, sm_scale=0.3)
    np.testing.assert_allclose(out1, out2, rtol=1e-12, atol=1e-13)
    for i in range(2):
        shift = 0.3 * 0.5 * float(np.sum(w["q"][0, i].astype(np.float64)))
        assert abs((lse2[0, i] - lse1[0, i]) - shift) < 1e-12


def test_gqa_replication():
    """G query heads on one KV head equal G separate KV heads holding copies."""
    rng = np.random.default_rng(9)
    w = _rand_case(rng, G=4)
    out1, lse1 = oracle.decode(w, k_layout="token", v_layout="channel", group=8, sm_scale=0.3)
    w2 = dict(w)
    for k in ("k_codes", "v_codes", "k_scale", "k_zero", "v_scale", "v_zero"):
        w2[k] = np.repeat(w[k], 4, axis=1)
    out2, lse2 = oracle.decode(w2, k_layout="token", v_layout="channel", group=8, sm_scale=0.3)
    np.testing.assert_array_equal(out1, out2)
    np.testing.assert_array_equal(lse1, lse2)


def test_heads_map_to_their_kv_head():
    """Query head i reads KV head i // G: changing KV head 1 changes only
    query heads G..2G-1."""
    rng = np.random.default_rng(10)
    w = _rand_case(rng, G=2)
    for k in ("k_codes", "v_codes", "k_scale", "k_zero", "v_scale", "v_zero"):
        w[k] = np.concatenate([w[k], w[k]], axis=1)
    w["q"] = np.concatenate([w["q"], w["q"]], axis=1)
    # offsets on a 1/64 grid so that z + 1 stays exact in fp16
    w["v_zero"] = (np.round(w["v_zero"].astype(np.float64) * 64) / 64).astype(np.float16)
    out1, _ = oracle.decode(w, k_layout="token", v_layout="channel", group=8, sm_scale=0.3)
    w["v_zero"] = w["v_zero"].copy()
    w["v_zero"][0, 1] += np.float16(1.0)
    out2, _ = oracle.decode(w, k_layout="token", v_layout="channel", group=8, sm_scale=0.3)
    np.testing.assert_array_equal(out1[0, :2], out2[0, :2])
    np.testing.assert_allclose(out2[0, 2:] - out1[0, 2:], 1.0, atol=1e-12)


# ------------------------------------------------- textbook special case

def test_textbook_attention_when_unit_scale():
    """s = 1, z = 0 makes the cache plain integers; the oracle must then equal
    softmax attention from a library routine and from a brute-force loop."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(11)
    T, D = 23, 16
    w = _rand_case(rng, T=T, Tcap=24, D=D, g=8, k_layout="token", v_layout="token", G=3)
    for k in ("k_scale", "v_scale"):
        w[k][:] = 1
    for k in ("k_zero", "v_zero"):
        w[k][:] = 0
    sigma = 0.37
    out, lse = oracle.decode(w, k_layout="token", v_layout="token", group=8, sm_scale=sigma)
    K = torch.tensor(w["k_codes"][0, 0, :T].astype(np.float64))
    V = torch.tensor(w["v_codes"][0, 0, :T].astype(np.float64))
    Q = torch.tensor(w["q"][0].astype(np.float64))
    ref = torch.nn.functional.scaled_dot_product_attention(Q[None], K[None], V[None], scale=sigma)[0]
    np.testing.assert_allclose(out[0], ref.numpy(), rtol=1e-12, atol=1e-12)
    # brute force with math.exp over Python floats
    for i in range(3):
        sc = [sigma * sum(float(w["q"][0, i, c]) * int(w["k_codes"][0, 0, t, c]) for c in range(D))
              for t in range(T)]
        den = sum(math.exp(s) for s in sc)
        assert abs(lse[0, i] - math.log(den)) < 1e-12
        for c in range(D):
            num = sum(math.exp(sc[t]) * int(w["v_codes"][0, 0, t, c]) for t in range(T))
            assert abs(out[0, i, c] - num / den) < 1e-11


# ------------------------------------------------------------- packing

def _golden_words():
    rows = []
    with open(os.path.join(GOLDEN, "packing.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            parts = line.split()
            bits = int(parts[0])
            codes = [int(x) for x in parts[1:-1]]
            rows.append((bits, codes, int(parts[-1], 16)))
    return rows


@pytest.mark.parametrize("row", _golden_words())
def test_pack_golden_words(row):
    bits, codes, word = row
    E = 32 // bits
    assert len(codes) == E
    # keys: the E codes are E consecutive channels of one token
    k = oracle.pack_k(np.array([codes], np.uint8), bits)
    assert k.shape == (1, 1) and int(k[0, 0]) == word
    # values: the E codes are E consecutive tokens of one channel
    v = oracle.pack_v(np.array(codes, np.uint8)[:, None], bits)
    assert v.shape == (1, 1) and int(v[0, 0]) == word


@pytest.mark.parametrize("bits", [2, 4])
def test_pack_roundtrip_and_positions(bits):
    rng = np.random.default_rng(12)
    codes = rng.integers(0, 1 << bits, size=(2, 3, 64, 128)).astype(np.uint8)
    pk = oracle.pack_k(codes, bits)
    pv = oracle.pack_v(codes, bits)
    assert pk.shape == (2, 3, 64, 128 * bits // 32)
    assert pv.shape == (2, 3, 64 * bits // 32, 128)
    np.testing.assert_array_equal(oracle.unpack_k(pk, bits, 128), codes)
    np.testing.assert_array_equal(oracle.unpack_v(pv, bits), codes)
    E = 32 // bits
    # spot-check positions against the specification, element by element
    for (b, h, t, c) in [(0, 0, 0, 0), (1, 2, 63, 127), (0, 1, 17, 45), (1, 0, 5, E - 1)]:
        sk = bits * ((c % E) // 2) + 16 * (c % 2)
        sv = bits * ((t % E) // 2) + 16 * (t % 2)
        assert (int(pk[b, h, t, c // E]) >> sk) & ((1 << bits) - 1) == codes[b, h, t, c]
        assert (int(pv[b, h, t // E, c]) >> sv) & ((1 << bits) - 1) == codes[b, h, t, c]


# ---------------------------------------------------------------- full-precision window

def _window_case(rng, T, W, wl, D=16, g=8):
    w = _one_head(rng.standard_normal((2, D)), rng.integers(0, 4, (T, D), dtype=np.uint8),
                  rng.integers(0, 4, (T, D), dtype=np.uint8), rng.integers(1, 64, (T, D // g)) / 32.0,
                  rng.integers(-64, 64, (T, D // g)) / 32.0, rng.integers(1, 64, (T, D // g)) / 32.0,
                  rng.integers(-64, 64, (T, D // g)) / 32.0)
    win = {"k": rng.standard_normal((1, 1, W, D)), "v": rng.standard_normal((1, 1, W, D)), "lens": np.array([wl])}
    return w, win


def test_window_only_is_plain_attention():
    """No cache token (T = 0): the window alone is textbook softmax attention."""
    rng = np.random.default_rng(21)
    w, win = _window_case(rng, 4, 12, 9)
    w["seq_lens"] = np.array([0], np.int32)
    out, lse = oracle.decode_window_rows(w, win, [(0, 0), (0, 1)], k_layout="token", v_layout="token", group=8,
                                         sm_scale=0.3)
    for n in range(2):
        q = w["q"][0, n]
        k, v = win["k"][0, 0, :9], win["v"][0, 0, :9]
        s = 0.3 * (k @ q)
        p = np.exp(s - s.max())
        assert np.allclose(out[n], (p / p.sum()) @ v, atol=1e-13)
        assert abs(lse[n] - (s.max() + np.log(p.sum()))) < 1e-13


def test_moving_tokens_between_cache_and_window_changes_nothing():
    """A window token whose value equals a cache token's dequantised value can
    move from the cache to the window (or back) without changing the output:
    attention is over the union of both token sets."""
    rng = np.random.default_rng(22)
    T, D, g = 10, 16, 8
    w, win = _window_case(rng, T, 6, 3, D, g)
    k_hat = oracle.dequantize(w["k_codes"][0, 0], w["k_scale"][0, 0], w["k_zero"][0, 0], "token", g)
    v_hat = oracle.dequantize(w["v_codes"][0, 0], w["v_scale"][0, 0], w["v_zero"][0, 0], "token", g)
    full, lse_full = oracle.decode_window_rows(w, win, [(0, 0)], k_layout="token", v_layout="token", group=g,
                                               sm_scale=0.25)
    # the last 4 cache tokens move into the window
    w2 = dict(w, seq_lens=np.array([T - 4], np.int32))
    win2 = {"k": np.concatenate([k_hat[None, None, T - 4:], win["k"][:, :, :3]], axis=2),
            "v": np.concatenate([v_hat[None, None, T - 4:], win["v"][:, :, :3]], axis=2), "lens": np.array([7])}
    moved, lse_moved = oracle.decode_window_rows(w2, win2, [(0, 0)], k_layout="token", v_layout="token", group=g,
                                                 sm_scale=0.25)
    assert np.allclose(full, moved, atol=1e-13) and abs(lse_full[0] - lse_moved[0]) < 1e-13
    # an empty window is the plain decode step
    none = dict(win, lens=np.array([0]))
    o1, l1 = oracle.decode_window_rows(w, none, [(0, 0)], k_layout="token", v_layout="token", group=g, sm_scale=0.25)
    o2, l2 = oracle.decode_rows(w, [(0, 0)], k_layout="token", v_layout="token", group=g, sm_scale=0.25)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    # nothing at all: out 0, lse -inf
    o3, l3 = oracle.decode_window_rows(dict(w, seq_lens=np.array([0], np.int32)), none, [(0, 0)], k_layout="token",
                                       v_layout="token", group=g, sm_scale=0.25)
    assert not o3.any() and l3[0] == -np.inf


# ---------------------------------------------------------------------------
# Paged cache: gather_paged puts a pool of blocks back in logical order.
# ---------------------------------------------------------------------------

def test_gather_paged_by_hand():
    """Three pool blocks of two tokens, one channel, one KV head; sequence 0
    uses blocks (2, 0), sequence 1 block 1 then an entry outside the pool (a
    block of zeros); values written out by hand."""
    codes = np.array([[[[10], [11]]], [[[20], [21]]], [[[30], [31]]]], np.uint8)  # [NB=3][H=1][P=2][D=1]
    scale = codes.astype(np.float16) / 8          # token-wise, one group of one channel
    pool = {"k_codes": codes, "v_codes": codes + 1, "k_scale": scale, "k_zero": -scale,
            "v_scale": scale, "v_zero": scale}
    table = np.array([[2, 0], [1, 7]], np.int32)
    w = oracle.gather_paged(pool, table, 2, k_layout="token", v_layout="token", group=1)
    assert w["k_codes"][:, 0, :, 0].tolist() == [[30, 31, 10, 11], [20, 21, 0, 0]]
    assert w["v_codes"][:, 0, :, 0].tolist() == [[31, 32, 11, 12], [21, 22, 0, 0]]
    assert w["k_zero"][0, 0, :, 0].tolist() == [-3.75, -3.875, -1.25, -1.375]
    assert w["v_scale"][1, 0, :, 0].tolist() == [2.5, 2.625, 0.0, 0.0]


def test_gather_paged_channel_wise_scale_rows():
    """Channel-wise groups of g tokens: each block of P tokens carries P/g scale
    rows, gathered with the block (P = 4, g = 2: two rows per block)."""
    nb, P, g = 3, 4, 2
    s = np.arange(nb * (P // g), dtype=np.float16).reshape(nb, 1, P // g, 1)
    codes = np.zeros((nb, 1, P, 1), np.uint8)
    pool = {"k_codes": codes, "v_codes": codes, "k_scale": s, "k_zero": s, "v_scale": s, "v_zero": s}
    w = oracle.gather_paged(pool, np.array([[1, 2, 0]]), P, k_layout="channel", v_layout="channel", group=g)
    assert w["k_scale"][0, 0, :, 0].tolist() == [2, 3, 4, 5, 0, 1]


@pytest.mark.parametrize("k_layout,v_layout,g,P", [("token", "token", 32, 64), ("token", "channel", 64, 128),
                                                   ("channel", "token", 32, 128), ("channel", "channel", 64, 64)])
def test_paged_decode_equals_contiguous_decode(k_layout, v_layout, g, P):
    """A seeded random block order (unused pool blocks poisoned with NaN scales)
    gives exactly the contiguous cache's result, ragged lengths with partial
    last blocks and an empty sequence included."""
    spec = synth.Spec("paged_pin", 22, 2, k_layout, v_layout, g, 3, 4, 2, 128, 256, lens=(256, 77, 0))
    table, nb = synth.make_block_table(5, spec.seq_lens(), 256 // P, P)
    pool = synth.make_pool(spec, table, nb, P)
    pool["q"] = synth.make_query(spec)
    pool["seq_lens"] = spec.seq_lens()
    rows = [(b, i) for b in range(3) for i in range(4)]
    kw = dict(k_layout=k_layout, v_layout=v_layout, group=g, sm_scale=spec.sm_scale)
    o_p, l_p = oracle.decode_paged_rows(pool, table, P, rows, **kw)
    w = synth.make_workload(spec)
    o_c, l_c = oracle.decode_rows(w, rows, **kw)
    assert np.array_equal(o_p, o_c) and np.array_equal(l_p, l_c)


# ---------------------------------------------------------------- rotated cache
# A cache of Hadamard-rotated rows (explainer, accuracy paragraph: "OSCAR's
# rotations"; related explainers: KVarN, Hadamard-rotated 2-bit KV).


@pytest.mark.parametrize("n", [1, 2, 4, 8, 16, 32, 64, 128])
def test_hadamard_is_scipys_normalised(n):
    """The Sylvester construction against scipy's own (a library routine)."""
    from scipy.linalg import hadamard as scipy_hadamard
    np.testing.assert_array_equal(oracle.hadamard(n), scipy_hadamard(n) / math.sqrt(n))


def test_hadamard_orthonormal_and_symmetric():
    H = oracle.hadamard(128)
    np.testing.assert_allclose(H @ H.T, np.eye(128), atol=1e-14)
    np.testing.assert_array_equal(H, H.T)
    # entry (i, j) = (-1)^popcount(i & j) / sqrt(128), brute force on a few entries
    for i, j in ((0, 0), (1, 1), (3, 5), (127, 127), (64, 63), (100, 37)):
        assert H[i, j] == (-1) ** bin(i & j).count("1") / math.sqrt(128)


def test_round_bf16_matches_torch():
    """Nearest-even bf16 rounding against torch's float32 -> bfloat16 cast, on
    fp32 values over many binades and on exact ties."""
    import torch
    rng = np.random.default_rng(71)
    x = (rng.standard_normal(4096) * np.exp2(rng.integers(-20, 20, 4096))).astype(np.float32)
    base = oracle.round_bf16(x.astype(np.float64))
    ties = (base + np.sign(base) * np.ldexp(1.0, np.frexp(base)[1] - 9)).astype(np.float32)  # + half an ulp
    assert (oracle.round_bf16(ties.astype(np.float64)) != ties).all()  # every one a tie
    for v in (x, ties):
        want = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
        np.testing.assert_array_equal(oracle.round_bf16(v.astype(np.float64)), want)


def test_round_bf16_closed_forms():
    assert oracle.round_bf16(1 / math.sqrt(128)) == 181 / 2048     # 1.41421356.. * 2^7 = 181.02
    assert oracle.round_bf16(1 + 2 ** -8) == 1.0                    # tie: to even
    assert oracle.round_bf16(1 + 3 * 2 ** -8) == 1 + 2 ** -6        # tie: to even
    assert oracle.round_bf16(-(1 + 3 * 2 ** -8)) == -(1 + 2 ** -6)


def _orthogonal(rng, n):
    """A random orthogonal matrix that is not symmetric (QR of a Gaussian)."""
    m, r = np.linalg.qr(rng.standard_normal((n, n)))
    m = m * np.sign(np.diag(r))
    assert np.abs(m - m.T).max() > 0.1
    return m


@pytest.mark.parametrize("rot_k,rot_v", [(True, True), (True, False), (False, True)])
def test_rotation_leaves_attention_unchanged(rot_k, rot_v):
    """R R^T = I: over a cache of K R / V R rows, the rotated query and the
    un-rotated output give plain attention over K, V exactly (up to fp64
    rounding).  R is a random non-symmetric orthogonal matrix, so a query
    rotated by R^T, an output taken back by R, or a dropped step fails."""
    rng = np.random.default_rng(72)
    D, T = 16, 23
    R = _orthogonal(rng, D)
    q, K, V = rng.standard_normal(D), rng.standard_normal((T, D)), rng.standard_normal((T, D))
    o_ref, l_ref = oracle.attend(q, K, V, 0.4)
    o, l = oracle.attend_rotated(q, K @ R if rot_k else K, V @ R if rot_v else V, 0.4, rot_k=rot_k, rot_v=rot_v,
                                 rot=R, round_query=False)
    np.testing.assert_allclose(o, o_ref, atol=1e-12)
    assert abs(l - l_ref) < 1e-12
    # the same cache read as unrotated differs: the pin can fail
    o_bad, _ = oracle.attend_rotated(q, K @ R if rot_k else K, V @ R if rot_v else V, 0.4, rot_k=False,
                                     rot_v=False, rot=R, round_query=False)
    assert np.abs(o_bad - o_ref).max() > 1e-3


def test_rotated_cache_with_unrotated_window():
    """Cache rows rotated, window rows in the model's basis: one softmax over
    both equals plain attention over the union."""
    rng = np.random.default_rng(73)
    D, T, W = 16, 11, 5
    R = _orthogonal(rng, D)
    q = rng.standard_normal(D)
    K, V = rng.standard_normal((T, D)), rng.standard_normal((T, D))
    Kw, Vw = rng.standard_normal((W, D)), rng.standard_normal((W, D))
    o_ref, l_ref = oracle.attend(q, np.concatenate([K, Kw]), np.concatenate([V, Vw]), 0.4)
    o, l = oracle.attend_rotated(q, K @ R, V @ R, 0.4, rot_k=True, rot_v=True, rot=R, round_query=False,
                                 win_k=Kw, win_v=Vw)
    np.testing.assert_allclose(o, o_ref, atol=1e-12)
    assert abs(l - l_ref) < 1e-12
    o, l = oracle.attend_rotated(q, np.zeros((0, D)), np.zeros((0, D)), 0.4, rot_k=True, rot_v=True,
                                 rot=R, win_k=Kw, win_v=Vw)  # window only: the query is not rotated
    o_ref, l_ref = oracle.attend(q, Kw, Vw, 0.4)
    np.testing.assert_allclose(o, o_ref, atol=1e-13)


def test_rotated_query_is_rounded_to_bf16():
    """q = c e_0: q H = c / sqrt(128) in every channel, held as bf16.  One
    token: lse = sm * bf16(c / sqrt(128)) * sum(k) and out = its value (the
    value side unrotated)."""
    rng = np.random.default_rng(74)
    D = 128
    k, v = rng.standard_normal((1, D)), rng.standard_normal((1, D))
    for c, qh in ((1.0, 181 / 2048), (2.0, 181 / 1024), (-0.5, -181 / 4096)):
        q = np.zeros(D)
        q[0] = c
        o, l = oracle.attend_rotated(q, k, v, 0.3, rot_k=True, rot_v=False)
        assert l == pytest.approx(0.3 * qh * k.sum(), rel=1e-14, abs=1e-14)
        np.testing.assert_array_equal(o, v[0])


@pytest.mark.parametrize("k_layout,v_layout", [("token", "token"), ("channel", "channel"), ("token", "channel")])
def test_decode_rotate_argument(k_layout, v_layout):
    """``rotate`` routes each side: "k" meets the stored keys with
    bf16(q H), "v" takes the output back by H (= H^T), "kv" both; lse only
    depends on the key side."""
    rng = np.random.default_rng(75)
    w = _rand_case(rng, k_layout=k_layout, v_layout=v_layout)
    H = oracle.hadamard(16)
    kw = dict(k_layout=k_layout, v_layout=v_layout, group=8, sm_scale=0.3)
    o0, l0 = oracle.decode(w, **kw)
    wq = dict(w, q=oracle.round_bf16(np.asarray(w["q"], np.float64) @ H))
    oq, lq = oracle.decode(wq, **kw)
    ok, lk = oracle.decode(w, rotate="k", **kw)
    ov, lv = oracle.decode(w, rotate="v", **kw)
    okv, lkv = oracle.decode(w, rotate="kv", **kw)
    np.testing.assert_allclose(ok, oq, atol=1e-13)
    np.testing.assert_allclose(lk, lq, atol=1e-13)
    np.testing.assert_allclose(ov, o0 @ H, atol=1e-13)
    np.testing.assert_allclose(lv, l0, atol=1e-13)
    np.testing.assert_allclose(okv, oq @ H, atol=1e-13)
    np.testing.assert_allclose(lkv, lq, atol=1e-13)
    assert np.abs(ok - o0).max() > 1e-3 and np.abs(ov - o0).max() > 1e-3
