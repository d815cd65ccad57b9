"""The Python binding checks every tensor's full shape against include/foscar.h
before it calls the library: a cache of the other bit width, a head-dim-64
output or a short lengths array raise ValueError and launch nothing.  The
tensors here live on the CPU, so reaching a launch would fail differently."""
import os

import pytest

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def fos():
    from bit_quantized_kv_split_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("libfoscar.so not built")
    import bit_quantized_kv_split_amd as fos
    return fos


def _cache(bits, B=2, Hkv=2, T=256, D=128, kch=False, vch=False, g=128):
    E = 32 // bits
    i32, f16 = torch.int32, torch.float16
    sk = (B, Hkv, T // g, D) if kch else (B, Hkv, T, D // g)
    sv = (B, Hkv, T // g, D) if vch else (B, Hkv, T, D // g)
    return dict(packed_k=torch.zeros((B, Hkv, T, D // E), dtype=i32), packed_v=torch.zeros((B, Hkv, T // E, D), dtype=i32),
                k_scale=torch.zeros(sk, dtype=f16), k_zero=torch.zeros(sk, dtype=f16),
                v_scale=torch.zeros(sv, dtype=f16), v_zero=torch.zeros(sv, dtype=f16))


def _decode_args(bits=2, B=2, Hq=8, D=128, **kw):
    c = _cache(bits, B=B, D=D, **kw)
    return dict(q=torch.zeros((B, Hq, D), dtype=torch.bfloat16), seq_lens=torch.zeros(B, dtype=torch.int32), **c)


def _call_decode(fos, a, bits, layout=0, group=128, out=None, lse=None):
    return fos.prepare_decode(bits, a["q"], a["packed_k"], a["packed_v"], a["k_scale"], a["k_zero"], a["v_scale"],
                              a["v_zero"], a["seq_lens"], layout, group, out=out, lse=lse)


def test_two_bit_cache_passed_as_four_bit_is_rejected(fos):
    a = _decode_args(bits=2)
    with pytest.raises(ValueError, match="packed_k"):
        _call_decode(fos, a, 4)


def test_short_output_row_is_rejected(fos):
    a = _decode_args()
    with pytest.raises(ValueError, match="out"):
        _call_decode(fos, a, 2, out=torch.zeros((2, 8, 64), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="lse"):
        _call_decode(fos, a, 2, lse=torch.zeros((2, 4), dtype=torch.float32))


def test_lengths_and_values_are_checked(fos):
    a = _decode_args()
    a["seq_lens"] = torch.zeros(1, dtype=torch.int32)
    with pytest.raises(ValueError, match="seq_lens"):
        _call_decode(fos, a, 2)
    a = _decode_args()
    a["packed_v"] = torch.zeros((2, 2, 256 // 16, 64), dtype=torch.int32)
    with pytest.raises(ValueError, match="packed_v"):
        _call_decode(fos, a, 2)


@pytest.mark.parametrize("kch,vch,layout", [(False, False, 1), (True, False, 0), (False, True, 0), (True, True, 2)])
def test_scale_shapes_follow_the_layout(fos, kch, vch, layout):
    """Token-wise scales passed for a channel-wise side (and the reverse) fail."""
    a = _decode_args(kch=kch, vch=vch)
    with pytest.raises(ValueError, match="scale|zero"):
        _call_decode(fos, a, 2, layout=layout)


def test_group_must_divide_the_grouped_axis(fos):
    a = _decode_args(kch=True, vch=True, g=32)
    with pytest.raises(ValueError):
        _call_decode(fos, a, 2, layout=3, group=96)


def test_quantize_checks_the_cache_and_ranges(fos):
    c = _cache(2)
    src = torch.zeros((2, 2, 16, 128), dtype=torch.bfloat16)
    ok = dict(start=torch.zeros(2, dtype=torch.int32), count=torch.zeros(2, dtype=torch.int32))
    with pytest.raises(ValueError, match="packed_k"):  # 2-bit cache, 4-bit call
        fos.foscar_quantize_int4(src, src, ok["start"], ok["count"], c["packed_k"], c["packed_v"], c["k_scale"],
                                 c["k_zero"], c["v_scale"], c["v_zero"], 0, 128)
    with pytest.raises(ValueError, match="start"):
        fos.foscar_quantize_int2(src, src, torch.zeros(1, dtype=torch.int32), ok["count"], c["packed_k"],
                                 c["packed_v"], c["k_scale"], c["k_zero"], c["v_scale"], c["v_zero"], 0, 128)
    with pytest.raises(ValueError, match="scale|zero"):  # token-wise scales for a channel-wise key side
        fos.foscar_quantize_int2(src, src, ok["start"], ok["count"], c["packed_k"], c["packed_v"], c["k_scale"],
                                 c["k_zero"], c["v_scale"], c["v_zero"], 1, 128)
