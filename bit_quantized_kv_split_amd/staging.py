"""Put a host-side cache into device memory in the layout of the C interface.

Codes are uploaded one sequence at a time and packed on the GPU with
``foscar_pack`` into the packed tensors; scales, offsets, the query and the
lengths are copied as they are.  This is input staging, not part of a decode
step.
"""
import numpy as np
import torch

from . import FOSCAR_SIDE_K, FOSCAR_SIDE_V, foscar_pack, packed_shape


def stage(spec_shape, bits, q, seq_lens, head_fn, scale_shapes, device="cuda", sequences=None):
    """Build device tensors for one decode step.

    spec_shape: (B, Hq, Hkv, Tcap, D); q: fp32 array [B, Hq, D] holding bf16
    values; seq_lens: int32 [B]; head_fn(b) -> dict of per-KV-head lists
    (k_codes, v_codes uint8 [Hkv, Tcap, D], k_scale, k_zero, v_scale, v_zero);
    scale_shapes: dict name -> full fp16 shape.  Returns a dict of tensors with
    keys q, packed_k, packed_v, k_scale, k_zero, v_scale, v_zero, seq_lens.
    """
    B, Hq, Hkv, T, D = spec_shape
    dev = torch.device(device)
    out = {
        "q": torch.from_numpy(np.ascontiguousarray(q, np.float32)).to(torch.bfloat16).to(dev),
        "seq_lens": torch.from_numpy(np.ascontiguousarray(seq_lens, np.int32)).to(dev),
        "packed_k": torch.empty(packed_shape(bits, FOSCAR_SIDE_K, B, Hkv, T, D), dtype=torch.int32, device=dev),
        "packed_v": torch.empty(packed_shape(bits, FOSCAR_SIDE_V, B, Hkv, T, D), dtype=torch.int32, device=dev),
    }
    for name, shp in scale_shapes.items():
        out[name] = torch.empty(shp, dtype=torch.float16, device=dev)
    for b in range(B) if sequences is None else sequences:
        head = head_fn(b)
        for side, key in ((FOSCAR_SIDE_K, "k"), (FOSCAR_SIDE_V, "v")):
            codes = torch.from_numpy(np.ascontiguousarray(head[key + "_codes"], np.uint8))[None].to(dev)
            foscar_pack(bits, side, codes, packed=out["packed_" + key][b:b + 1])
            for part in ("scale", "zero"):
                out[f"{key}_{part}"][b].copy_(torch.from_numpy(np.ascontiguousarray(head[f"{key}_{part}"])))
        torch.cuda.synchronize(dev)
    return out


def stage_paged(bits, q, seq_lens, pool, block_table, device="cuda"):
    """Device tensors of a paged decode step: pools (codes packed on the GPU with
    ``foscar_pack``, one block standing for one sequence of block_size tokens)
    from ``pool`` (k_codes / v_codes uint8 [NB, Hkv, P, D], scales / offsets
    fp16), the block table int32 [B, blocks] and the query / lengths.  Keys:
    q, seq_lens, block_table, k_pool, v_pool, k_scale, k_zero, v_scale, v_zero."""
    dev = torch.device(device)
    NB, H, P, D = pool["k_codes"].shape
    out = {
        "q": torch.from_numpy(np.ascontiguousarray(q, np.float32)).to(torch.bfloat16).to(dev),
        "seq_lens": torch.from_numpy(np.ascontiguousarray(seq_lens, np.int32)).to(dev),
        "block_table": torch.from_numpy(np.ascontiguousarray(block_table, np.int32)).to(dev),
    }
    for side, key in ((FOSCAR_SIDE_K, "k"), (FOSCAR_SIDE_V, "v")):
        codes = torch.from_numpy(np.ascontiguousarray(pool[key + "_codes"], np.uint8)).to(dev)
        packed = torch.empty(packed_shape(bits, side, NB, H, P, D), dtype=torch.int32, device=dev)
        out[key + "_pool"] = foscar_pack(bits, side, codes, packed=packed)
        for part in ("scale", "zero"):
            out[f"{key}_{part}"] = torch.from_numpy(np.ascontiguousarray(pool[f"{key}_{part}"])).to(dev)
    torch.cuda.synchronize(dev)
    return out
