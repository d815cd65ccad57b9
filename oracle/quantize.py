"""CPU oracle for quantising new tokens into the low-bit cache -- TEST
INFRASTRUCTURE ONLY.

Only tests, the smoke check and the benchmark's CPU-baseline leg may import
this module.  The GPU library never calls it and shares no code with it.

What it computes (plain NumPy; the arithmetic that decides a code is fp32,
the precision the GPU quantiser decides codes in):

* ``quantize_group``: min-max asymmetric quantisation of one group of values
  to codes q in 0 .. 2**bits - 1 with one scale s and one offset z, so that
  the cache stores value = s*q + z (FOSCAR explainer, "FOSCAR speeds up 2-bit
  KV decode", encoding paragraph: a group of codes shares one scale and one
  offset).  The pages give no quantiser; the plainest one that matches the
  encoding is used: z = min, s = (max - min) / (2**bits - 1), q = the nearest
  code to (x - z) / s.  Readings: s is computed in fp32 and rounded to fp16,
  z = fp16(min), q = round-half-even((x - z16) / s16) in fp32, clamped to the
  code range; a group whose fp16 scale is 0 gets q = 0 (value = z).
* ``quantize_append``: writes tokens [start_b, start_b + count_b) of every
  sequence b into a cache held as logical codes plus (s, z) arrays.  Groups
  run token-wise (g consecutive channels of one token) or channel-wise (g
  consecutive tokens, from token 0, of one channel) -- explainer,
  fold-placement table.  Readings: a channel-wise side needs start_b to be a
  multiple of g (else the sequence is left untouched); a channel-wise group
  that the written range covers only in part is quantised over the tokens
  the range holds; codes and (s, z) of tokens outside the range are left as
  they were.

* ``rotate_rows``: a rotated cache (the accuracy recipe of the explainer's
  accuracy paragraph, "OSCAR's rotations"; its related explainer on a
  Hadamard-rotated 2-bit KV cache) stores the codes of x H instead of x, H
  the orthonormal Sylvester-Hadamard matrix.  Reading: the rotated rows are
  held in fp32, the precision the quantiser decides in, each the one fp32
  rounding of (the exact +-1 sum) times (1/sqrt(D) in fp64); ``quantize_append``
  rotates the sides ``rotate`` names before it quantises them.

Parity pins: ``tests/test_oracle_quant_pins.py`` (exact recovery of values
on a known grid, constant groups, round-half-even ties, the rounding error
bound, append order independence).
"""
from __future__ import annotations

import math

import numpy as np

from . import sylvester

TOKEN = "token"
CHANNEL = "channel"


def quantize_group(x, bits: int, axis: int = -1):
    """Quantise groups laid out along ``axis`` of ``x`` (values exactly
    representable in fp32).  Returns (codes uint8 like x, s fp16, z fp16)
    with ``axis`` reduced in s and z."""
    if bits not in (2, 4):
        raise ValueError("bits must be 2 or 4")
    levels = np.float32((1 << bits) - 1)
    xf = np.asarray(x, dtype=np.float32)
    mn = xf.min(axis=axis)
    mx = xf.max(axis=axis)
    s32 = (mx - mn).astype(np.float32) / levels          # fp32, rounded once
    s16 = s32.astype(np.float32).astype(np.float16)
    z16 = mn.astype(np.float16)
    s_b = np.expand_dims(s16.astype(np.float32), axis)
    z_b = np.expand_dims(z16.astype(np.float32), axis)
    zero = s_b == 0
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = (xf - z_b).astype(np.float32) / np.where(zero, np.float32(1), s_b)
    q = np.rint(ratio.astype(np.float32))
    q = np.clip(q, 0, levels)
    q = np.where(zero, 0, q)
    return q.astype(np.uint8), s16, z16


def inv_sqrt(d: int) -> float:
    """1/sqrt(d) for d a power of two, correctly rounded in fp64 (2^-k/2, or
    sqrt(2) 2^-(k+1)/2 with sqrt correctly rounded and the power exact)."""
    k = d.bit_length() - 1
    return math.ldexp(1.0, -k // 2) if k % 2 == 0 else math.ldexp(math.sqrt(2.0), -(k + 1) // 2)


def rotate_rows(x) -> np.ndarray:
    """Rows (last axis, D a power of two) of x -- bf16 values -- times the
    orthonormal Hadamard matrix, in fp32: the +-1 sums are exact in fp64 (for
    rows whose values span under 2^38 in magnitude), then scaled by
    fp64(1/sqrt(D)) and rounded once to fp32."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    return ((x @ sylvester(D)) * inv_sqrt(D)).astype(np.float32)


def quantize_append(cache: dict, k_src, v_src, start, count, *, bits: int, k_layout: str, v_layout: str,
                    group: int, rotate: str = "") -> dict:
    """Quantise new tokens into a copy of ``cache`` and return it.

    cache: k_codes, v_codes uint8 [B][Hkv][Tcap][D]; k_scale, k_zero,
    v_scale, v_zero fp16, token-wise [B][Hkv][Tcap][D/g] or channel-wise
    [B][Hkv][Tcap/g][D].
    k_src, v_src: [B][Hkv][N][D] values (fp32 arrays holding bf16 values);
    row r of sequence b is token start[b] + r.
    start, count: int [B].  Per sequence: start outside [0, Tcap] leaves it
    untouched; count is clamped to [0, min(N, Tcap - start)].
    rotate: "", "k", "v" or "kv" -- the sides whose rows are rotated
    (``rotate_rows``) before they are quantised.
    """
    if rotate not in ("", "k", "v", "kv"):
        raise ValueError(rotate)
    out = {k: np.array(v, copy=True) for k, v in cache.items()}
    B, Hkv, Tcap, D = out["k_codes"].shape
    N = np.asarray(k_src).shape[2]
    chan = CHANNEL in (k_layout, v_layout)
    for b in range(B):
        s0 = int(start[b])
        if s0 < 0 or s0 > Tcap:
            continue
        if chan and s0 % group != 0:
            continue
        n = int(min(max(int(count[b]), 0), N, Tcap - s0))
        if n == 0:
            continue
        for side, src, layout in (("k", k_src, k_layout), ("v", v_src, v_layout)):
            x = np.asarray(src, dtype=np.float32)[b, :, :n, :]          # [Hkv][n][D]
            if side in rotate:
                x = rotate_rows(x)
            codes = out[f"{side}_codes"][b]
            sc = out[f"{side}_scale"][b]
            zr = out[f"{side}_zero"][b]
            if layout == TOKEN:
                xg = x.reshape(Hkv, n, D // group, group)                   # groups along channels
                q, s16, z16 = quantize_group(xg, bits, axis=-1)
                codes[:, s0:s0 + n, :] = q.reshape(Hkv, n, D)
                sc[:, s0:s0 + n, :] = s16
                zr[:, s0:s0 + n, :] = z16
            elif layout == CHANNEL:
                for t0 in range(s0, s0 + n, group):                          # groups along tokens
                    t1 = min(t0 + group, s0 + n)
                    q, s16, z16 = quantize_group(x[:, t0 - s0:t1 - s0, :], bits, axis=1)
                    codes[:, t0:t1, :] = q
                    sc[:, t0 // group, :] = s16
                    zr[:, t0 // group, :] = z16
            else:
                raise ValueError(layout)
    return out
