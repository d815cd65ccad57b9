"""Python binding of libfoscar: decode attention over a 2-/4-bit KV cache on MI355X.

Thin marshalling over the C interface of include/foscar.h; every function of
that header is available here under the same name, taking torch tensors (used
only as device memory) instead of raw pointers, plus ``decode`` / ``pack`` /
``unpack`` conveniences.  All computation runs in the HIP kernels of
libfoscar.so; if the library is not built, importing the entry points raises.

Layout constants and shapes are those of the C header.
"""
import ctypes
import math

from . import _lib

FOSCAR_OK = 0
FOSCAR_EINVAL = -1
FOSCAR_EUNSUPPORTED = -2
FOSCAR_EHIP = -3
FOSCAR_ENOMEM = -4
FOSCAR_ESCRATCH = -5
FOSCAR_K_TOKEN = 0
FOSCAR_K_CHANNEL = 1
FOSCAR_V_TOKEN = 0
FOSCAR_V_CHANNEL = 2
FOSCAR_K_ROTATED = 4
FOSCAR_V_ROTATED = 8
FOSCAR_SIDE_K = 0
FOSCAR_SIDE_V = 1

FoscarDims = _lib.FoscarDims


class FoscarError(RuntimeError):
    def __init__(self, code, where):
        lib = _lib.load()
        msg = lib.foscar_strerror(code).decode()
        hip = lib.foscar_last_hip_error() if code == FOSCAR_EHIP else 0
        super().__init__(f"{where}: {msg} (code {code}{', hip error ' + str(hip) if hip else ''})")
        self.code = code


def _check(rc, where):
    if rc != FOSCAR_OK:
        if rc in (FOSCAR_EINVAL, FOSCAR_EUNSUPPORTED, FOSCAR_ESCRATCH):
            raise ValueError(f"{where}: {_lib.load().foscar_strerror(rc).decode()} (code {rc})")
        raise FoscarError(rc, where)


def layout_bits(k_layout: str, v_layout: str, rotate: str = "") -> int:
    """Layout word of the C interface; ``rotate`` ("", "k", "v", "kv") names the
    cache sides that hold Hadamard-rotated rows."""
    if rotate not in ("", "k", "v", "kv"):
        raise ValueError(f"rotate must be '', 'k', 'v' or 'kv', not {rotate!r}")
    return ((FOSCAR_K_CHANNEL if k_layout == "channel" else 0) | (FOSCAR_V_CHANNEL if v_layout == "channel" else 0)
            | (FOSCAR_K_ROTATED if "k" in rotate else 0) | (FOSCAR_V_ROTATED if "v" in rotate else 0))


def make_dims(batch, num_q_heads, num_kv_heads, head_dim, max_seq_len, sm_scale=0.0):
    return FoscarDims(int(batch), int(num_q_heads), int(num_kv_heads), int(head_dim), int(max_seq_len),
                      float(sm_scale))


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _require(t, name, dtype, device):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _shape(t, name, expect):
    if tuple(t.shape) != tuple(expect):
        raise ValueError(f"{name} must have shape {tuple(expect)}, got {tuple(t.shape)}")


def _scale_shape(side_channel, B, Hkv, Tcap, D, group):
    """Shape of one side's fp16 scales / offsets (include/foscar.h): token-wise
    [B][Hkv][Tcap][D/g], channel-wise [B][Hkv][Tcap/g][D].  None when the
    group does not divide the axis (the C interface rejects that call)."""
    if group <= 0:
        return None
    if side_channel:
        return (B, Hkv, Tcap // group, D) if Tcap % group == 0 else None
    return (B, Hkv, Tcap, D // group) if D % group == 0 else None


def _check_cache(bits, packed_k, packed_v, k_scale, k_zero, v_scale, v_zero, layout, group, B, D):
    """Every cache tensor against the header's shapes for (bits, layout, group),
    derived from packed_k's [B][Hkv][Tcap] and the head dimension D; a cache of
    another bit width or layout fails here, before any launch."""
    if packed_k.dim() != 4:
        raise ValueError("packed_k must be [B, Hkv, Tcap, D*bits/32]")
    Hkv, Tcap = int(packed_k.shape[1]), int(packed_k.shape[2])
    E = 32 // bits
    if D % E or Tcap % E:
        raise ValueError(f"head_dim {D} and max_seq_len {Tcap} must be multiples of {E} for {bits}-bit codes")
    _shape(packed_k, "packed_k", (B, Hkv, Tcap, D // E))
    _shape(packed_v, "packed_v", (B, Hkv, Tcap // E, D))
    for side_channel, names, ts in ((layout & FOSCAR_K_CHANNEL, ("k_scale", "k_zero"), (k_scale, k_zero)),
                                    (layout & FOSCAR_V_CHANNEL, ("v_scale", "v_zero"), (v_scale, v_zero))):
        expect = _scale_shape(bool(side_channel), B, Hkv, Tcap, D, int(group))
        if expect is None:
            raise ValueError(f"group {group} does not divide the grouped axis (max_seq_len {Tcap}, head_dim {D})")
        for n, t in zip(names, ts):
            _shape(t, n, expect)
    return Hkv, Tcap


class DecodeCall:
    """One decode step with its arguments checked and marshalled once.

    Calling the object launches the step again on the stream it was prepared
    for and returns (out, lse); the tensors it was built from must keep their
    storage (they are referenced, not copied), and their contents may change
    between calls.  This is the path for a serving loop: a call is one C call.
    """

    __slots__ = ("_fn", "_args", "_name", "_dev", "out", "lse", "_keep")

    def __call__(self):
        import torch
        if torch.cuda.current_device() != self._dev:
            with torch.cuda.device(self._dev):
                rc = self._fn(*self._args)
        else:
            rc = self._fn(*self._args)
        if rc != FOSCAR_OK:
            _check(rc, self._name)
        return self.out, self.lse


def prepare_decode(bits, q, packed_k, packed_v, k_scale, k_zero, v_scale, v_zero, seq_lens, layout, group,
                   out=None, lse=None, sm_scale=0.0, stream=None, window=None, noalloc=False, paged=None):
    """Check and marshal a decode step (arguments as foscar_decode_int2/4); returns a DecodeCall.
    ``window`` = (win_k, win_v, win_lens) marshals foscar_decode_window_int2/4 instead;
    ``noalloc`` marshals foscar_decode_noalloc (out and lse must then be given);
    ``paged`` = block_table int32 [B, blocks per sequence] marshals foscar_decode_paged_int2/4,
    with packed_k .. v_zero the block pools (include/foscar.h; block_size = packed_k.shape[2])."""
    import torch
    if bits not in (2, 4):
        raise ValueError(f"bits must be 2 or 4, got {bits}")
    if noalloc and (out is None or lse is None or window is not None):
        raise ValueError("foscar_decode_noalloc takes caller-provided out and lse, and no window")
    if paged is not None and (noalloc or window is not None):
        raise ValueError("the paged decode takes no window and allocates its workspace")
    lib = _lib.load()
    dev = q.device
    _require(q, "q", torch.bfloat16, dev)
    for name, t in (("packed_k", packed_k), ("packed_v", packed_v)):
        _require(t, name, torch.int32, dev)
    for name, t in (("k_scale", k_scale), ("k_zero", k_zero), ("v_scale", v_scale), ("v_zero", v_zero)):
        _require(t, name, torch.float16, dev)
    _require(seq_lens, "seq_lens", torch.int32, dev)
    if q.dim() != 3:
        raise ValueError("q must be [B, Hq, D]")
    B, Hq, D = (int(x) for x in q.shape)
    if paged is None:
        Hkv, Tcap = _check_cache(bits, packed_k, packed_v, k_scale, k_zero, v_scale, v_zero, int(layout), group, B, D)
    else:  # pools: the contiguous layout with (num_blocks, block_size) in place of (B, Tcap)
        block_table = paged
        _require(block_table, "block_table", torch.int32, dev)
        if packed_k.dim() != 4 or block_table.dim() != 2 or int(block_table.shape[0]) != B:
            raise ValueError("packed_k must be [num_blocks, Hkv, block_size, D*bits/32] and block_table [B, blocks]")
        num_blocks = int(packed_k.shape[0])
        Hkv, block_size = _check_cache(bits, packed_k, packed_v, k_scale, k_zero, v_scale, v_zero, int(layout), group,
                                       num_blocks, D)
        Tcap = int(block_table.shape[1]) * block_size
    _shape(seq_lens, "seq_lens", (B,))
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    _require(out, "out", torch.bfloat16, dev)
    _require(lse, "lse", torch.float32, dev)
    _shape(out, "out", (B, Hq, D))
    _shape(lse, "lse", (B, Hq))
    dims = make_dims(B, Hq, Hkv, D, Tcap, sm_scale)
    call = DecodeCall()
    call._fn = lib.foscar_decode_int2 if bits == 2 else lib.foscar_decode_int4
    with torch.cuda.device(dev):
        st = _stream(stream)
    call._args = (ctypes.byref(dims), _ptr(q), _ptr(packed_k), _ptr(packed_v), _ptr(k_scale), _ptr(k_zero),
                  _ptr(v_scale), _ptr(v_zero), _ptr(seq_lens), int(layout), int(group), _ptr(out), _ptr(lse), st)
    call._name = f"foscar_decode_int{bits}"
    if noalloc:
        call._fn = lib.foscar_decode_noalloc
        call._args = (int(bits),) + call._args
        call._name = "foscar_decode_noalloc"
    if paged is not None:
        call._fn = lib.foscar_decode_paged_int2 if bits == 2 else lib.foscar_decode_paged_int4
        call._args = call._args[:8] + (_ptr(block_table), int(block_size), int(num_blocks)) + call._args[8:]
        call._name = f"foscar_decode_paged_int{bits}"
    call._dev = dev.index if dev.index is not None else torch.cuda.current_device()
    call.out, call.lse = out, lse
    call._keep = (dims, q, packed_k, packed_v, k_scale, k_zero, v_scale, v_zero, seq_lens,
                  block_table if paged is not None else None)
    if window is not None:
        win_k, win_v, win_lens = window
        _require(win_k, "win_k", torch.bfloat16, dev)
        _require(win_v, "win_v", torch.bfloat16, dev)
        _require(win_lens, "win_lens", torch.int32, dev)
        if win_k.dim() != 4 or tuple(win_k.shape) != tuple(win_v.shape) or win_k.shape[0] != B \
                or win_k.shape[1] != Hkv or win_k.shape[3] != D or win_lens.numel() != B:
            raise ValueError("win_k / win_v must be [B, Hkv, W, D] and win_lens [B]")
        call._fn = lib.foscar_decode_window_int2 if bits == 2 else lib.foscar_decode_window_int4
        call._args = call._args[:11] + (_ptr(win_k), _ptr(win_v), _ptr(win_lens), int(win_k.shape[2])) + call._args[11:]
        call._name = f"foscar_decode_window_int{bits}"
        call._keep = call._keep + (win_k, win_v, win_lens)
    return call


def _decode(bits, q, packed_k, packed_v, k_scale, k_zero, v_scale, v_zero, seq_lens, layout, group,
            out=None, lse=None, sm_scale=0.0, stream=None):
    return prepare_decode(bits, q, packed_k, packed_v, k_scale, k_zero, v_scale, v_zero, seq_lens, layout, group,
                          out, lse, sm_scale, stream)()


def foscar_decode_int2(q, packed_k, packed_v, k_scale, k_zero, v_scale, v_zero, seq_lens, layout, group,
                       out=None, lse=None, sm_scale=0.0, stream=None):
    """2-bit decode step; tensors as in include/foscar.h (packed words as int32). Returns (out, lse)."""
    return _decode(2, q, packed_k, packed_v, k_scale, k_zero, v_scale, v_zero, seq_lens, layout, group,
                   out, lse, sm_scale, stream)


def foscar_decode_int4(q, packed_k, packed_v, k_scale, k_zero, v_scale, v_zero, seq_lens, layout, group,
                       out=None, lse=None, sm_scale=0.0, stream=None):
    """4-bit decode step; tensors as in include/foscar.h (packed words as int32). Returns (out, lse)."""
    return _decode(4, q, packed_k, packed_v, k_scale, k_zero, v_scale, v_zero, seq_lens, layout, group,
                   out, lse, sm_scale, stream)


def foscar_decode_noalloc(bits, q, packed_k, packed_v, k_scale, k_zero, v_scale, v_zero, seq_lens, layout, group,
                          out, lse, sm_scale=0.0, stream=None):
    """Decode step that allocates nothing (include/foscar.h): the split workspace is the
    library's static scratch; out [B, Hq, D] bf16 and lse [B, Hq] fp32 are the caller's."""
    return prepare_decode(bits, q, packed_k, packed_v, k_scale, k_zero, v_scale, v_zero, seq_lens, layout, group,
                          out, lse, sm_scale, stream, noalloc=True)()


def _decode_window(bits, q, packed_k, packed_v, k_scale, k_zero, v_scale, v_zero, seq_lens, layout, group, win_k,
                   win_v, win_lens, out=None, lse=None, sm_scale=0.0, stream=None):
    return prepare_decode(bits, q, packed_k, packed_v, k_scale, k_zero, v_scale, v_zero, seq_lens, layout, group, out,
                          lse, sm_scale, stream, window=(win_k, win_v, win_lens))()


def foscar_decode_window_int2(q, packed_k, packed_v, k_scale, k_zero, v_scale, v_zero, seq_lens, layout, group, win_k,
                              win_v, win_lens, out=None, lse=None, sm_scale=0.0, stream=None):
    """2-bit decode step plus a bf16 window of recent tokens [B, Hkv, W, D] (include/foscar.h)."""
    return _decode_window(2, q, packed_k, packed_v, k_scale, k_zero, v_scale, v_zero, seq_lens, layout, group, win_k,
                          win_v, win_lens, out, lse, sm_scale, stream)


def foscar_decode_window_int4(q, packed_k, packed_v, k_scale, k_zero, v_scale, v_zero, seq_lens, layout, group, win_k,
                              win_v, win_lens, out=None, lse=None, sm_scale=0.0, stream=None):
    """4-bit decode step plus a bf16 window of recent tokens [B, Hkv, W, D] (include/foscar.h)."""
    return _decode_window(4, q, packed_k, packed_v, k_scale, k_zero, v_scale, v_zero, seq_lens, layout, group, win_k,
                          win_v, win_lens, out, lse, sm_scale, stream)


def foscar_decode_paged_int2(q, k_pool, v_pool, k_scale, k_zero, v_scale, v_zero, block_table, seq_lens, layout,
                             group, out=None, lse=None, sm_scale=0.0, stream=None):
    """2-bit decode step over a paged cache: block pools [num_blocks, Hkv, block_size, ..] and
    block_table int32 [B, max_seq_len / block_size] (include/foscar.h). Returns (out, lse)."""
    return prepare_decode(2, q, k_pool, v_pool, k_scale, k_zero, v_scale, v_zero, seq_lens, layout, group, out, lse,
                          sm_scale, stream, paged=block_table)()


def foscar_decode_paged_int4(q, k_pool, v_pool, k_scale, k_zero, v_scale, v_zero, block_table, seq_lens, layout,
                             group, out=None, lse=None, sm_scale=0.0, stream=None):
    """4-bit decode step over a paged cache (see foscar_decode_paged_int2). Returns (out, lse)."""
    return prepare_decode(4, q, k_pool, v_pool, k_scale, k_zero, v_scale, v_zero, seq_lens, layout, group, out, lse,
                          sm_scale, stream, paged=block_table)()


def decode_paged(q, k_pool, v_pool, k_scale, k_zero, v_scale, v_zero, block_table, seq_lens, *, bits,
                 k_layout="token", v_layout="token", group=128, sm_scale=0.0, out=None, lse=None, stream=None,
                 rotate=""):
    """Decode step over a paged cache (pools and block table as foscar_decode_paged_int2)."""
    fn = foscar_decode_paged_int2 if bits == 2 else foscar_decode_paged_int4
    return fn(q, k_pool, v_pool, k_scale, k_zero, v_scale, v_zero, block_table, seq_lens,
              layout_bits(k_layout, v_layout, rotate), group, out, lse, sm_scale, stream)


def decode(q, packed_k, packed_v, k_scale, k_zero, v_scale, v_zero, seq_lens, *, bits, k_layout="token",
           v_layout="token", group=128, sm_scale=0.0, out=None, lse=None, stream=None, window=None, rotate=""):
    """Decode step; ``window`` = (win_k, win_v, win_lens) adds a bf16 window of recent tokens;
    ``rotate`` names the cache sides holding Hadamard-rotated rows ("k", "v", "kv")."""
    layout = layout_bits(k_layout, v_layout, rotate)
    if window is not None:
        return _decode_window(bits, q, packed_k, packed_v, k_scale, k_zero, v_scale, v_zero, seq_lens, layout, group,
                              *window, out, lse, sm_scale, stream)
    fn = foscar_decode_int2 if bits == 2 else foscar_decode_int4
    return fn(q, packed_k, packed_v, k_scale, k_zero, v_scale, v_zero, seq_lens, layout, group, out, lse, sm_scale,
              stream)


def _quantize(bits, k_src, v_src, start, count, packed_k, packed_v, k_scale, k_zero, v_scale, v_zero, layout, group,
              stream=None):
    import torch
    lib = _lib.load()
    dev = k_src.device
    _require(k_src, "k_src", torch.bfloat16, dev)
    _require(v_src, "v_src", torch.bfloat16, dev)
    if tuple(k_src.shape) != tuple(v_src.shape) or k_src.dim() != 4:
        raise ValueError("k_src and v_src must both be [B, Hkv, N, D]")
    for name, t in (("start", start), ("count", count)):
        _require(t, name, torch.int32, dev)
    for name, t in (("packed_k", packed_k), ("packed_v", packed_v)):
        _require(t, name, torch.int32, dev)
    for name, t in (("k_scale", k_scale), ("k_zero", k_zero), ("v_scale", v_scale), ("v_zero", v_zero)):
        _require(t, name, torch.float16, dev)
    B, Hkv, N, D = (int(x) for x in k_src.shape)
    if bits not in (2, 4):
        raise ValueError(f"bits must be 2 or 4, got {bits}")
    if packed_k.dim() != 4 or tuple(packed_k.shape[:2]) != (B, Hkv):
        raise ValueError("cache and sources disagree on [B, Hkv]")
    _, Tcap = _check_cache(bits, packed_k, packed_v, k_scale, k_zero, v_scale, v_zero, int(layout), group, B, D)
    _shape(start, "start", (B,))
    _shape(count, "count", (B,))
    dims = make_dims(B, Hkv, Hkv, D, Tcap)
    fn = lib.foscar_quantize_int2 if bits == 2 else lib.foscar_quantize_int4
    with torch.cuda.device(dev):
        rc = fn(ctypes.byref(dims), _ptr(k_src), _ptr(v_src), int(N), _ptr(start), _ptr(count), int(layout),
                int(group), _ptr(packed_k), _ptr(packed_v), _ptr(k_scale), _ptr(k_zero), _ptr(v_scale),
                _ptr(v_zero), _stream(stream))
    _check(rc, f"foscar_quantize_int{bits}")


def foscar_quantize_int2(k_src, v_src, start, count, packed_k, packed_v, k_scale, k_zero, v_scale, v_zero, layout,
                         group, stream=None):
    """Quantise bf16 keys / values [B, Hkv, N, D] into a 2-bit cache in place (include/foscar.h)."""
    _quantize(2, k_src, v_src, start, count, packed_k, packed_v, k_scale, k_zero, v_scale, v_zero, layout, group,
              stream)


def foscar_quantize_int4(k_src, v_src, start, count, packed_k, packed_v, k_scale, k_zero, v_scale, v_zero, layout,
                         group, stream=None):
    """Quantise bf16 keys / values [B, Hkv, N, D] into a 4-bit cache in place (include/foscar.h)."""
    _quantize(4, k_src, v_src, start, count, packed_k, packed_v, k_scale, k_zero, v_scale, v_zero, layout, group,
              stream)


def _pack_dims(codes_shape):
    B, Hkv, T, D = codes_shape
    return make_dims(B, Hkv, Hkv, D, T)


def packed_shape(bits, side, B, Hkv, T, D):
    E = 32 // bits
    return (B, Hkv, T, D // E) if side == FOSCAR_SIDE_K else (B, Hkv, T // E, D)


def foscar_pack(bits, side, codes, packed=None, stream=None):
    """codes uint8 [B, Hkv, Tcap, D] on the GPU -> packed int32 words (layout of include/foscar.h)."""
    import torch
    lib = _lib.load()
    _require(codes, "codes", torch.uint8, codes.device)
    dims = _pack_dims(codes.shape)
    if packed is None:
        packed = torch.empty(packed_shape(bits, side, *codes.shape), dtype=torch.int32, device=codes.device)
    _require(packed, "packed", torch.int32, codes.device)
    with torch.cuda.device(codes.device):
        rc = lib.foscar_pack(int(bits), int(side), ctypes.byref(dims), _ptr(codes), _ptr(packed), _stream(stream))
    _check(rc, "foscar_pack")
    return packed


def foscar_unpack(bits, side, packed, shape, codes=None, stream=None):
    """packed int32 words -> codes uint8 of ``shape`` = [B, Hkv, Tcap, D]."""
    import torch
    lib = _lib.load()
    _require(packed, "packed", torch.int32, packed.device)
    dims = _pack_dims(shape)
    if codes is None:
        codes = torch.empty(tuple(shape), dtype=torch.uint8, device=packed.device)
    _require(codes, "codes", torch.uint8, packed.device)
    with torch.cuda.device(packed.device):
        rc = lib.foscar_unpack(int(bits), int(side), ctypes.byref(dims), _ptr(packed), _ptr(codes), _stream(stream))
    _check(rc, "foscar_unpack")
    return codes


pack = foscar_pack
unpack = foscar_unpack


def foscar_packed_bytes(bits, side, dims):
    return int(_lib.load().foscar_packed_bytes(int(bits), int(side), ctypes.byref(dims)))


def foscar_scale_count(side, side_layout, group, dims):
    return int(_lib.load().foscar_scale_count(int(side), int(side_layout), int(group), ctypes.byref(dims)))


def foscar_workspace_reserve(dims, bits, layout, group, stream=None):
    _check(_lib.load().foscar_workspace_reserve(ctypes.byref(dims), int(bits), int(layout), int(group),
                                                _stream(stream)), "foscar_workspace_reserve")


def foscar_release():
    _lib.load().foscar_release()


def foscar_split_plan(dims, bits, layout, group):
    s, c = ctypes.c_int32(0), ctypes.c_int32(0)
    _check(_lib.load().foscar_split_plan(ctypes.byref(dims), int(bits), int(layout), int(group), ctypes.byref(s),
                                         ctypes.byref(c)), "foscar_split_plan")
    return s.value, c.value


def foscar_record_next_launch(start, stop):
    """Have the next decode call on this thread record `start`/`stop` with its
    kernel dispatch.  Events are torch.cuda.Event objects that have been
    recorded once (so that they exist) or raw hipEvent_t handles."""
    def handle(e):
        if e is None:
            return None
        return ctypes.c_void_p(e.cuda_event if hasattr(e, "cuda_event") else int(e))
    _lib.load().foscar_record_next_launch(handle(start), handle(stop))


def foscar_occupancy(bits, layout, group):
    """Work-groups of the decode kernel one compute unit holds at once."""
    n = ctypes.c_int32(0)
    _check(_lib.load().foscar_occupancy(int(bits), int(layout), int(group), ctypes.byref(n)), "foscar_occupancy")
    return int(n.value)


def foscar_strerror(code):
    return _lib.load().foscar_strerror(int(code)).decode()


def foscar_version():
    return int(_lib.load().foscar_version())


def foscar_last_hip_error():
    return int(_lib.load().foscar_last_hip_error())
