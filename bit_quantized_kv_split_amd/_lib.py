"""ctypes loader for libfoscar.so (the HIP library built from csrc/).

There is no fallback: if the shared library is missing this raises, so no
code path can silently compute elsewhere.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfoscar.so")

# Names declared in include/foscar.h, in order.
EXPORTS = [
    "foscar_decode_int2", "foscar_decode_int4", "foscar_decode_noalloc", "foscar_decode_window_int2",
    "foscar_decode_window_int4", "foscar_decode_paged_int2", "foscar_decode_paged_int4",
    "foscar_quantize_int2", "foscar_quantize_int4", "foscar_pack", "foscar_unpack", "foscar_packed_bytes",
    "foscar_scale_count", "foscar_workspace_reserve", "foscar_release", "foscar_split_plan", "foscar_occupancy",
    "foscar_record_next_launch",
    "foscar_strerror", "foscar_version", "foscar_last_hip_error",
]


class FoscarDims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("max_seq_len", ctypes.c_int32), ("sm_scale", ctypes.c_float)]


_lib = None


def load():
    """Load libfoscar.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m bit_quantized_kv_split_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    D = ctypes.POINTER(FoscarDims)
    for name in ("foscar_decode_int2", "foscar_decode_int4"):
        f = getattr(lib, name)
        f.argtypes = [D, P, P, P, P, P, P, P, P, I, I, P, P, P]
        f.restype = I
    lib.foscar_decode_noalloc.argtypes = [I, D, P, P, P, P, P, P, P, P, I, I, P, P, P]
    lib.foscar_decode_noalloc.restype = I
    for name in ("foscar_decode_window_int2", "foscar_decode_window_int4"):
        f = getattr(lib, name)
        f.argtypes = [D, P, P, P, P, P, P, P, P, I, I, P, P, P, ctypes.c_int32, P, P, P]
        f.restype = I
    for name in ("foscar_decode_paged_int2", "foscar_decode_paged_int4"):
        f = getattr(lib, name)
        f.argtypes = [D, P, P, P, P, P, P, P, P, ctypes.c_int32, ctypes.c_int32, P, I, I, P, P, P]
        f.restype = I
    for name in ("foscar_quantize_int2", "foscar_quantize_int4"):
        f = getattr(lib, name)
        f.argtypes = [D, P, P, ctypes.c_int32, P, P, I, I, P, P, P, P, P, P, P]
        f.restype = I
    lib.foscar_pack.argtypes = [I, I, D, P, P, P]
    lib.foscar_pack.restype = I
    lib.foscar_unpack.argtypes = [I, I, D, P, P, P]
    lib.foscar_unpack.restype = I
    lib.foscar_packed_bytes.argtypes = [I, I, D]
    lib.foscar_packed_bytes.restype = SZ
    lib.foscar_scale_count.argtypes = [I, I, I, D]
    lib.foscar_scale_count.restype = SZ
    lib.foscar_workspace_reserve.argtypes = [D, I, I, I, P]
    lib.foscar_workspace_reserve.restype = I
    lib.foscar_release.argtypes = []
    lib.foscar_release.restype = None
    lib.foscar_split_plan.argtypes = [D, I, I, I, ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32)]
    lib.foscar_split_plan.restype = I
    lib.foscar_occupancy.argtypes = [I, I, I, ctypes.POINTER(ctypes.c_int32)]
    lib.foscar_occupancy.restype = I
    lib.foscar_record_next_launch.argtypes = [P, P]
    lib.foscar_record_next_launch.restype = I
    lib.foscar_strerror.argtypes = [I]
    lib.foscar_strerror.restype = ctypes.c_char_p
    lib.foscar_version.argtypes = []
    lib.foscar_version.restype = I
    lib.foscar_last_hip_error.argtypes = []
    lib.foscar_last_hip_error.restype = I
    _lib = lib
    return lib
