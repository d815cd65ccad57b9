"""GPU parity of quantise-and-append (foscar_quantize_int2/int4, through the C
interface) against the oracle's quantiser (oracle/quantize.py): every packed
word, scale and offset bit-exact, on caches that already hold arbitrary
content, for every (bits, K layout, V layout, g) instance; ragged starts and
counts, unaligned channel-wise starts, out-of-range starts, single-token
appends over several calls, a full-size long-context prefill (sampled
slices), and quantise-then-decode against the decode oracle; the same for a
rotated cache (rows rotated by the Hadamard matrix before they are
quantised).
"""
import numpy as np
import pytest

import oracle
import oracle.quantize as oq
import synth
from gpu_util import check

pytestmark = pytest.mark.gpu

D = 128


def _fos():
    import bit_quantized_kv_split_amd as fos
    return fos


def _scales(case, side, layout, g, T):
    out = []
    for part in ("scale", "zero"):
        a = case[f"{side}_{part}_{layout}"]
        a = a[..., : D // g] if layout == "token" else a[:, :, : T // g]
        out.append(np.ascontiguousarray(a).view(np.float16))
    return out


def _expected(case, bits, kl, vl, g, T, rotate=""):
    ks, kz = _scales(case, "k", kl, g, T)
    vs, vz = _scales(case, "v", vl, g, T)
    cache = {"k_codes": oracle.unpack_k(case["packed_k"], bits, D), "v_codes": oracle.unpack_v(case["packed_v"], bits),
             "k_scale": ks, "k_zero": kz, "v_scale": vs, "v_zero": vz}
    out = oq.quantize_append(cache, case["k_src"], case["v_src"], case["start"], case["count"], bits=bits,
                             k_layout=kl, v_layout=vl, group=g, rotate=rotate)
    return {"packed_k": oracle.pack_k(out["k_codes"], bits), "packed_v": oracle.pack_v(out["v_codes"], bits),
            "k_scale": out["k_scale"], "k_zero": out["k_zero"], "v_scale": out["v_scale"], "v_zero": out["v_zero"]}


def _to_device(case, kl, vl, g, T):
    import torch
    dev = "cuda"
    ks, kz = _scales(case, "k", kl, g, T)
    vs, vz = _scales(case, "v", vl, g, T)
    return {
        "k_src": torch.from_numpy(case["k_src"]).to(torch.bfloat16).to(dev),
        "v_src": torch.from_numpy(case["v_src"]).to(torch.bfloat16).to(dev),
        "start": torch.from_numpy(case["start"]).to(dev), "count": torch.from_numpy(case["count"]).to(dev),
        "packed_k": torch.from_numpy(case["packed_k"].view(np.int32)).to(dev),
        "packed_v": torch.from_numpy(case["packed_v"].view(np.int32)).to(dev),
        "k_scale": torch.from_numpy(ks).to(dev), "k_zero": torch.from_numpy(kz).to(dev),
        "v_scale": torch.from_numpy(vs).to(dev), "v_zero": torch.from_numpy(vz).to(dev),
    }


def _quantize(d, bits, kl, vl, g, k_src=None, v_src=None, start=None, count=None, rotate=""):
    fos = _fos()
    fn = fos.foscar_quantize_int2 if bits == 2 else fos.foscar_quantize_int4
    fn(d["k_src"] if k_src is None else k_src, d["v_src"] if v_src is None else v_src,
       d["start"] if start is None else start, d["count"] if count is None else count,
       d["packed_k"], d["packed_v"], d["k_scale"], d["k_zero"], d["v_scale"], d["v_zero"],
       fos.layout_bits(kl, vl, rotate), g)


def _compare(d, exp, what):
    import torch
    torch.cuda.synchronize()
    for name in ("packed_k", "packed_v"):
        got = d[name].cpu().numpy().view(np.uint32)
        bad = np.argwhere(got != exp[name])
        assert bad.size == 0, f"{what}: {name} differs at {bad[:4].tolist()} ({len(bad)} words)"
    for name in ("k_scale", "k_zero", "v_scale", "v_zero"):
        got = d[name].cpu().numpy().view(np.uint16)
        bad = np.argwhere(got != exp[name].view(np.uint16))
        assert bad.size == 0, f"{what}: {name} differs at {bad[:4].tolist()} ({len(bad)} values)"


MATRIX = [(bits, kl, vl, g) for bits in (2, 4) for kl in ("token", "channel") for vl in ("token", "channel")
          for g in (32, 64, 128)]


@pytest.mark.parametrize("bits,kl,vl,g", MATRIX)
def test_layout_matrix_bit_exact(bits, kl, vl, g):
    """Ragged ranges over several 128-token blocks, with partial value words at
    both ends, a clamped count, a zero count and a start past the capacity;
    channel-wise layouts add an unaligned start (left untouched)."""
    T, N = 512, 300
    if "channel" in (kl, vl):
        starts, counts = [0, g, 2 * g + 1, 256, T + 64, 3 * g], [300, 45, 10, 1000, 5, 0]
    else:
        starts, counts = [0, 37, 200, 453, T + 1, 5], [300, 45, 1000, 1000, 5, 0]
    case = synth.make_append_case(1, len(starts), 2, T, N, bits, starts, counts)
    d = _to_device(case, kl, vl, g, T)
    _quantize(d, bits, kl, vl, g)
    _compare(d, _expected(case, bits, kl, vl, g, T), f"int{bits} {kl}/{vl} g{g}")


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("g", [32, 128])
def test_single_token_appends(bits, g):
    """Decode-time use: one token per sequence per call, 40 calls in a row
    (token-wise K and V), each call's ranges at different word offsets."""
    import torch
    T, B, H = 256, 3, 2
    case = synth.make_append_case(2, B, H, T, 40, bits, [0, 17, 215], [40, 40, 40])
    d = _to_device(case, "token", "token", g, T)
    count = torch.ones(B, dtype=torch.int32, device="cuda")
    for i in range(40):
        start = torch.from_numpy(case["start"] + np.int32(i)).cuda()
        _quantize(d, bits, "token", "token", g, k_src=d["k_src"][:, :, i:i + 1].contiguous(),
                  v_src=d["v_src"][:, :, i:i + 1].contiguous(), start=start, count=count)
    exp = _expected(case, bits, "token", "token", g, T)  # one call over all 40 tokens
    _compare(d, exp, f"int{bits} g{g} appends")


@pytest.mark.parametrize("bits", [2, 4])
def test_channel_group_completion(bits):
    """Channel-wise sides fed a partial group, then the whole group again once
    it is complete (the re-quantise the interface describes)."""
    import torch
    T, g, B, H = 256, 64, 2, 2
    case = synth.make_append_case(3, B, H, T, 2 * g, bits, [g, 0], [20, 2 * g])
    d = _to_device(case, "channel", "channel", g, T)
    _quantize(d, bits, "channel", "channel", g)
    full = torch.from_numpy(np.array([2 * g, 2 * g], np.int32)).cuda()
    _quantize(d, bits, "channel", "channel", g, count=full)
    exp = _expected(dict(case, count=np.array([2 * g, 2 * g], np.int32)), bits, "channel", "channel", g, T)
    _compare(d, exp, f"int{bits} group completion")


def test_full_size_long_context_sampled():
    """Prefill of the long-context shape (4 sequences x 8 KV heads x 131072
    tokens, INT2 token-wise g = 128) in one call; sampled (sequence, KV head)
    slices against the oracle, bit-exact."""
    import torch
    B, H, T, g, bits = 4, 8, 131072, 128, 2
    fos = _fos()
    k_src = synth.device_normal_bf16((B, H, T, D), 1234)
    v_src = synth.device_normal_bf16((B, H, T, D), 1235)
    pk = torch.zeros((B, H, T, D // 16), dtype=torch.int32, device="cuda")
    pv = torch.zeros((B, H, T // 16, D), dtype=torch.int32, device="cuda")
    sc = [torch.zeros((B, H, T, 1), dtype=torch.float16, device="cuda") for _ in range(4)]
    start = torch.zeros(B, dtype=torch.int32, device="cuda")
    count = torch.full((B,), T, dtype=torch.int32, device="cuda")
    fos.foscar_quantize_int2(k_src, v_src, start, count, pk, pv, *sc, fos.layout_bits("token", "token"), g)
    torch.cuda.synchronize()
    for b, h in ((0, 0), (3, 7), (2, 5)):
        ks_ = k_src[b:b + 1, h:h + 1].float().cpu().numpy()
        vs_ = v_src[b:b + 1, h:h + 1].float().cpu().numpy()
        cache = {"k_codes": np.zeros((1, 1, T, D), np.uint8), "v_codes": np.zeros((1, 1, T, D), np.uint8)}
        for name in ("k_scale", "k_zero", "v_scale", "v_zero"):
            cache[name] = np.zeros((1, 1, T, 1), np.float16)
        out = oq.quantize_append(cache, ks_, vs_, [0], [T], bits=bits, k_layout="token", v_layout="token", group=g)
        assert np.array_equal(pk[b, h].cpu().numpy().view(np.uint32), oracle.pack_k(out["k_codes"][0, 0], bits))
        assert np.array_equal(pv[b, h].cpu().numpy().view(np.uint32), oracle.pack_v(out["v_codes"][0, 0], bits))
        for name, t in zip(("k_scale", "k_zero", "v_scale", "v_zero"), sc):
            assert np.array_equal(t[b, h].cpu().numpy().view(np.uint16), out[name][0, 0].view(np.uint16)), name


@pytest.mark.parametrize("bits,kl,vl", [(2, "token", "token"), (4, "channel", "channel"), (2, "token", "channel")])
def test_quantize_then_decode(bits, kl, vl):
    """GPU-quantised cache decoded on the GPU against the decode oracle over
    the oracle-quantised cache (the same cache, bit for bit)."""
    import torch
    fos = _fos()
    T, N, g, B, H, Hq = 512, 448, 64, 2, 2, 8
    case = synth.make_append_case(4, B, H, T, N, bits, [0, 0], [N, 301])
    exp = _expected(case, bits, kl, vl, g, T)
    d = _to_device(case, kl, vl, g, T)
    _quantize(d, bits, kl, vl, g)
    _compare(d, exp, "quantised cache")
    lens = np.array([N, 301], np.int32)
    rng = np.random.default_rng(5)
    q = synth.bf16_round(rng.standard_normal((B, Hq, D)).astype(np.float32))
    out, lse = fos.decode(torch.from_numpy(q).to(torch.bfloat16).cuda(), d["packed_k"], d["packed_v"], d["k_scale"],
                          d["k_zero"], d["v_scale"], d["v_zero"], torch.from_numpy(lens).cuda(), bits=bits,
                          k_layout=kl, v_layout=vl, group=g)
    torch.cuda.synchronize()
    w = {"q": q, "k_codes": oracle.unpack_k(exp["packed_k"], bits, D), "v_codes": oracle.unpack_v(exp["packed_v"], bits),
         "k_scale": exp["k_scale"], "k_zero": exp["k_zero"], "v_scale": exp["v_scale"], "v_zero": exp["v_zero"],
         "seq_lens": lens}
    ro, rl = oracle.decode(w, k_layout=kl, v_layout=vl, group=g, sm_scale=1 / np.sqrt(D))
    check(out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), ro, rl,
          f"quantise+decode int{bits} {kl}/{vl}")


@pytest.mark.parametrize("bits,kl,vl,g", [(2, "token", "token", 32), (4, "token", "channel", 32),
                                        (2, "channel", "channel", 32)])
def test_capacity_a_multiple_of_32_write_then_decode(bits, kl, vl, g):
    """A 96-token capacity (32 mod 64): the writer's 128-token block ends at
    the capacity and the decode's last tile reaches past it."""
    import torch
    fos = _fos()
    T, N, B, H, Hq = 96, 96, 2, 2, 8
    case = synth.make_append_case(6, B, H, T, N, bits, [0, 0], [N, 61])
    exp = _expected(case, bits, kl, vl, g, T)
    d = _to_device(case, kl, vl, g, T)
    _quantize(d, bits, kl, vl, g)
    _compare(d, exp, "quantised cache, capacity 96")
    lens = np.array([N, 61], np.int32)
    rng = np.random.default_rng(7)
    q = synth.bf16_round(rng.standard_normal((B, Hq, D)).astype(np.float32))
    out, lse = fos.decode(torch.from_numpy(q).to(torch.bfloat16).cuda(), d["packed_k"], d["packed_v"], d["k_scale"],
                          d["k_zero"], d["v_scale"], d["v_zero"], torch.from_numpy(lens).cuda(), bits=bits,
                          k_layout=kl, v_layout=vl, group=g)
    torch.cuda.synchronize()
    w = {"q": q, "k_codes": oracle.unpack_k(exp["packed_k"], bits, D), "v_codes": oracle.unpack_v(exp["packed_v"], bits),
         "k_scale": exp["k_scale"], "k_zero": exp["k_zero"], "v_scale": exp["v_scale"], "v_zero": exp["v_zero"],
         "seq_lens": lens}
    ro, rl = oracle.decode(w, k_layout=kl, v_layout=vl, group=g, sm_scale=1 / np.sqrt(D))
    check(out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), ro, rl,
          f"capacity 96 int{bits} {kl}/{vl}")


@pytest.mark.parametrize("rotate", ["k", "v", "kv"])
@pytest.mark.parametrize("bits,kl,vl,g", [(2, "token", "token", 128), (4, "token", "channel", 32),
                                          (2, "channel", "token", 64), (4, "channel", "channel", 128)])
def test_rotated_writer_bit_exact(bits, kl, vl, g, rotate):
    """Rows rotated by the Hadamard matrix (fp64 butterflies, one rounding to
    fp32) before they are quantised: every word, scale and offset as the
    oracle's quantiser over its own rotation of the rows."""
    T, N = 512, 300
    if "channel" in (kl, vl):
        starts, counts = [0, g, 2 * g + 1, 256], [300, 45, 10, 1000]
    else:
        starts, counts = [0, 37, 200, 453], [300, 45, 1000, 1000]
    case = synth.make_append_case(6, len(starts), 2, T, N, bits, starts, counts)
    d = _to_device(case, kl, vl, g, T)
    _quantize(d, bits, kl, vl, g, rotate=rotate)
    _compare(d, _expected(case, bits, kl, vl, g, T, rotate=rotate), f"rotated {rotate} int{bits} {kl}/{vl} g{g}")


@pytest.mark.parametrize("bits,kl,vl", [(2, "token", "token"), (4, "channel", "token")])
def test_rotated_write_then_decode(bits, kl, vl):
    """A rotated cache written by the GPU quantiser and decoded with the
    rotation bits, against the decode oracle over the oracle's rotated cache."""
    import torch
    fos = _fos()
    T, N, g, B, H, Hq = 512, 448, 64, 2, 2, 8
    case = synth.make_append_case(7, B, H, T, N, bits, [0, 0], [N, 301])
    exp = _expected(case, bits, kl, vl, g, T, rotate="kv")
    d = _to_device(case, kl, vl, g, T)
    _quantize(d, bits, kl, vl, g, rotate="kv")
    _compare(d, exp, "rotated cache")
    lens = np.array([N, 301], np.int32)
    rng = np.random.default_rng(8)
    q = synth.bf16_round(rng.standard_normal((B, Hq, D)).astype(np.float32))
    out, lse = fos.decode(torch.from_numpy(q).to(torch.bfloat16).cuda(), d["packed_k"], d["packed_v"], d["k_scale"],
                          d["k_zero"], d["v_scale"], d["v_zero"], torch.from_numpy(lens).cuda(), bits=bits,
                          k_layout=kl, v_layout=vl, group=g, rotate="kv")
    torch.cuda.synchronize()
    w = {"q": q, "k_codes": oracle.unpack_k(exp["packed_k"], bits, D), "v_codes": oracle.unpack_v(exp["packed_v"], bits),
         "k_scale": exp["k_scale"], "k_zero": exp["k_zero"], "v_scale": exp["v_scale"], "v_zero": exp["v_zero"],
         "seq_lens": lens}
    ro, rl = oracle.decode(w, k_layout=kl, v_layout=vl, group=g, sm_scale=1 / np.sqrt(D), rotate="kv")
    got = out.float().cpu().numpy().astype(np.float64)
    check(got, lse.cpu().numpy().astype(np.float64), ro, rl, f"rotated write+decode int{bits} {kl}/{vl}")
