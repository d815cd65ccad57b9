"""The C interface on the host: the library loads, exports every function that
include/foscar.h declares, and rejects invalid arguments with error codes
before touching the GPU (these calls run without a GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER_DIR = os.path.join(ROOT, "include")


def _declared_functions():
    names = []
    for fn in sorted(os.listdir(HEADER_DIR)):
        if not fn.endswith(".h"):
            continue
        text = open(os.path.join(HEADER_DIR, fn)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(foscar_[a-z0-9_]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    from bit_quantized_kv_split_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("libfoscar.so not built")
    return _lib.load()


def test_header_declares_the_expected_entry_points():
    names = _declared_functions()
    assert "foscar_decode_int2" in names and "foscar_decode_int4" in names
    from bit_quantized_kv_split_amd import _lib
    assert sorted(_lib.EXPORTS) == names


def test_every_declared_symbol_is_exported(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name


def _dims(**kw):
    import bit_quantized_kv_split_amd as fos
    d = dict(batch=1, num_q_heads=4, num_kv_heads=1, head_dim=128, max_seq_len=1024, sm_scale=0.0)
    d.update(kw)
    return fos.make_dims(**d)


def _decode(lib, dims, layout=0, group=128, ptr=1):
    p = ctypes.c_void_p(ptr) if ptr else None
    return lib.foscar_decode_int2(ctypes.byref(dims) if dims is not None else None, p, p, p, p, p, p, p, p,
                                  layout, group, p, p, None)


@pytest.mark.parametrize("kw,layout,group,code", [
    (dict(batch=1 << 20, num_q_heads=8, num_kv_heads=8), 0, 128, -2),
    (dict(max_seq_len=1 << 25), 0, 128, -2),
    (dict(head_dim=80), 0, 64, -2),                          # head dims: 128, or a multiple of 32 up to 256
    (dict(head_dim=288), 0, 32, -2),
    (dict(head_dim=64), 0, 128, -2),                         # a token-wise group of 128 channels in 64
    (dict(head_dim=64), 1, 128, -2),
    (dict(head_dim=64), 3 | 4, 64, -2),                      # rotated caches: head_dim 128 only
    (dict(num_q_heads=6, num_kv_heads=4), 0, 128, -1),
    (dict(num_q_heads=34, num_kv_heads=2), 0, 128, -2),     # 17 query heads per KV head
    (dict(batch=(1 << 20) + 1, num_q_heads=16, num_kv_heads=2), 0, 128, -2),  # over 2^22 work pairs (G = 8: two per KV head)
    (dict(max_seq_len=1000), 0, 128, -2),                    # not a multiple of 32
    (dict(max_seq_len=192), 2, 128, -2),                     # channel-wise group of 128 does not divide 192
    (dict(batch=-1), 0, 128, -1),
    (dict(), 16, 128, -1),                                   # bad layout bits (0-15: sides and rotation)
    (dict(), -1, 128, -1),
    (dict(max_seq_len=192), 2 | 4, 128, -2),                 # rotation bits keep the channel-wise check
    (dict(), 0, 48, -2),                                     # bad group
])
def test_invalid_arguments_return_codes_before_any_gpu_call(lib, kw, layout, group, code):
    assert _decode(lib, _dims(**kw), layout, group) == code


@pytest.mark.parametrize("D,layout,group", [(32, 0, 32), (64, 0, 64), (96, 2, 32), (192, 1, 64), (256, 0, 128),
                                             (64, 3, 128), (256, 3, 32)])
def test_other_head_dims_pass_the_shape_checks(lib, D, layout, group):
    """Head dims other than 128 (multiples of 32 up to 256) reach the plain decode: with null
    pointers the call fails on them, after every shape check, before any HIP call."""
    import bit_quantized_kv_split_amd as fos
    d = _dims(head_dim=D)
    assert _decode(lib, d, layout, group, ptr=0) == -1
    assert _noalloc(lib, d, layout=layout, group=group, ptr=0) == -1
    s, c = fos.foscar_split_plan(d, 2, layout, group)
    assert s * c >= d.max_seq_len and c % 64 == 0
    assert fos.foscar_packed_bytes(2, fos.FOSCAR_SIDE_K, d) == 1024 * D * 2 // 8
    assert _quantize(lib, d, layout, group) == -2                    # the quantiser: head_dim 128 only


def test_null_pointers_and_dims(lib):
    assert _decode(lib, None) == -1
    assert _decode(lib, _dims(), ptr=0) == -1
    assert _decode(lib, _dims(batch=0), ptr=0) == 0   # nothing to do


def test_sizes_and_strings(lib):
    import bit_quantized_kv_split_amd as fos
    d = _dims(batch=2, num_kv_heads=3, num_q_heads=6, max_seq_len=256)
    assert fos.foscar_packed_bytes(2, fos.FOSCAR_SIDE_K, d) == 2 * 3 * 256 * 128 * 2 // 8
    assert fos.foscar_packed_bytes(4, fos.FOSCAR_SIDE_V, d) == 2 * 3 * 256 * 128 * 4 // 8
    assert fos.foscar_packed_bytes(3, fos.FOSCAR_SIDE_V, d) == 0
    assert fos.foscar_scale_count(fos.FOSCAR_SIDE_K, fos.FOSCAR_K_TOKEN, 32, d) == 2 * 3 * 256 * 4
    assert fos.foscar_scale_count(fos.FOSCAR_SIDE_V, fos.FOSCAR_V_CHANNEL, 64, d) == 2 * 3 * 4 * 128
    assert fos.foscar_scale_count(fos.FOSCAR_SIDE_V, fos.FOSCAR_K_CHANNEL, 64, d) == 0
    assert fos.foscar_version() == 100
    for c, s in [(0, "ok"), (-1, "invalid argument"), (-2, "unsupported"), (-3, "HIP"), (-4, "memory")]:
        assert s in fos.foscar_strerror(c)
    with pytest.raises(ValueError):
        fos.foscar_split_plan(_dims(head_dim=80), 2, 0, 64)


def test_split_plan_covers_the_cache(lib, monkeypatch):
    import bit_quantized_kv_split_amd as fos
    monkeypatch.delenv("FOSCAR_SPLITS", raising=False)
    for kw, layout, g in [(dict(batch=4, num_q_heads=32, num_kv_heads=8, max_seq_len=131072), 0, 128),
                          (dict(batch=64, num_q_heads=32, num_kv_heads=8, max_seq_len=65536), 2, 32),
                          (dict(batch=8, num_q_heads=32, num_kv_heads=8, max_seq_len=32768), 3, 128),
                          (dict(max_seq_len=96), 0, 128), (dict(max_seq_len=160), 3, 32),
                          (dict(max_seq_len=4128), 0, 64), (dict(), 0, 128)]:
        d = _dims(**kw)
        s, c = fos.foscar_split_plan(d, 2, layout, g)
        unit = g if (layout and g > 64) else 64
        assert c % unit == 0 and s * c >= d.max_seq_len and (s - 1) * c < d.max_seq_len
    monkeypatch.setenv("FOSCAR_SPLITS", "3")
    s, c = fos.foscar_split_plan(_dims(), 2, 0, 128)
    assert s == 3 and c == 384


def test_occupancy_rejects_bad_arguments(lib):
    n = ctypes.c_int32(0)
    assert lib.foscar_occupancy(3, 0, 128, ctypes.byref(n)) == -2
    assert lib.foscar_occupancy(2, 0, 48, ctypes.byref(n)) == -2
    assert lib.foscar_occupancy(2, 16, 128, ctypes.byref(n)) == -1
    assert lib.foscar_occupancy(2, 0, 128, None) == -1


def test_split_plan_caps_the_range_count(lib, monkeypatch):
    import bit_quantized_kv_split_amd as fos
    monkeypatch.setenv("FOSCAR_SPLITS", "100000")
    s, c = fos.foscar_split_plan(_dims(max_seq_len=1 << 20), 2, 0, 128)
    assert s == 512 and c == 2048


def test_plan_and_reserve_reject_bad_bits(lib):
    import bit_quantized_kv_split_amd as fos
    with pytest.raises(ValueError):
        fos.foscar_split_plan(_dims(), 3, 0, 128)
    assert lib.foscar_workspace_reserve(ctypes.byref(_dims()), 8, 0, 128, None) == -1


def _quantize(lib, dims, layout=0, group=128, src_tokens=16, ptr=1, bits=2):
    p = ctypes.c_void_p(ptr) if ptr else None
    fn = lib.foscar_quantize_int2 if bits == 2 else lib.foscar_quantize_int4
    return fn(ctypes.byref(dims) if dims is not None else None, p, p, src_tokens, p, p, layout, group,
              p, p, p, p, p, p, None)


@pytest.mark.parametrize("kw,layout,group,src,code", [
    (dict(head_dim=64), 0, 128, 16, -2),
    (dict(max_seq_len=1000), 0, 128, 16, -2),                 # not a multiple of 32
    (dict(max_seq_len=192), 1, 128, 16, -2),                  # channel-wise group of 128 does not divide 192
    (dict(batch=70000), 0, 128, 16, -2),                      # grid z
    (dict(), 16, 128, 16, -1),                                # bad layout bits (0-15: sides and rotation)
    (dict(), 0, 16, 16, -2),                                  # bad group
    (dict(), 0, 128, -1, -1),                                 # negative source length
])
def test_quantize_rejects_bad_arguments_before_any_gpu_call(lib, kw, layout, group, src, code):
    assert _quantize(lib, _dims(**kw), layout, group, src) == code
    assert _quantize(lib, _dims(**kw), layout, group, src, bits=4) == code


def test_quantize_null_pointers_and_empty_calls(lib):
    assert _quantize(lib, None) == -1
    assert _quantize(lib, _dims(), ptr=0) == -1
    assert _quantize(lib, _dims(batch=0), ptr=0) == 0     # nothing to do
    assert _quantize(lib, _dims(), src_tokens=0, ptr=0) == 0


def _decode_window(lib, dims, win_cap=128, ptr=1, win_ptr=1, layout=0, group=128):
    p = ctypes.c_void_p(ptr) if ptr else None
    w = ctypes.c_void_p(win_ptr) if win_ptr else None
    return lib.foscar_decode_window_int2(ctypes.byref(dims) if dims is not None else None, p, p, p, p, p, p, p, p,
                                         layout, group, w, w, w, win_cap, p, p, None)


def test_decode_window_rejects_bad_arguments_before_any_gpu_call(lib):
    assert _decode_window(lib, _dims(), win_cap=-1) == -1
    assert _decode_window(lib, _dims(), win_cap=4097) == -2          # largest window: 4096 tokens
    assert _decode_window(lib, _dims(), win_ptr=0) == -1             # window pointers missing
    assert _decode_window(lib, _dims(head_dim=64)) == -2
    assert _decode_window(lib, _dims(head_dim=64), group=64) == -2   # other head dims: plain caches only
    assert _decode_window(lib, _dims(), layout=16) == -1
    assert _decode_window(lib, None) == -1
    assert _decode_window(lib, _dims(batch=0), ptr=0, win_ptr=0) == 0


def test_misaligned_pointers_are_rejected_before_any_gpu_call(lib):
    """16-byte loads and stores need 16-byte aligned packed arrays, scales and
    sources: a misaligned pointer is an argument error, never a launch.  The
    pointers are not real allocations, so this runs only where no GPU is
    visible (a broken check must not be able to launch on them)."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("host-only check: the pointers are fabricated")
    assert _decode(lib, _dims(), ptr=0x1008) == -1          # 8-byte aligned only
    assert _quantize(lib, _dims(), ptr=0x1004) == -1
    assert _decode_window(lib, _dims(), ptr=0x1000, win_ptr=0x1002) == -1


def _noalloc(lib, dims, bits=2, layout=0, group=128, ptr=1):
    p = ctypes.c_void_p(ptr) if ptr else None
    return lib.foscar_decode_noalloc(bits, ctypes.byref(dims) if dims is not None else None, p, p, p, p, p, p, p, p,
                                     layout, group, p, p, None)


def test_noalloc_rejects_before_any_gpu_call(lib):
    """The no-allocation decode validates like the decode entry points and
    rejects, before any HIP call, what its static scratch cannot hold."""
    assert _noalloc(lib, _dims(), bits=3) == -1
    assert _noalloc(lib, None) == -1
    assert _noalloc(lib, _dims(head_dim=80)) == -2
    assert _noalloc(lib, _dims(batch=0), ptr=0) == 0
    assert _noalloc(lib, _dims(batch=20000, num_q_heads=1, num_kv_heads=1)) == -5   # range counters
    assert _noalloc(lib, _dims(batch=1024, num_q_heads=32, num_kv_heads=8)) == -5   # partials of one range
    assert _noalloc(lib, _dims(), ptr=0) == -1
    assert "static scratch" in lib.foscar_strerror(-5).decode()
