"""Seeded synthetic decode-attention workloads (inputs only).

This module draws the query, the full-precision keys and values, and turns
the keys and values into a low-bit cache with one scale ``s`` and one
offset ``z`` per group (value = s*q + z).  It holds none of the attention
arithmetic: both the CPU oracle and the GPU path consume what it returns.

Sources (the FOSCAR pages):
  * explainer page "FOSCAR speeds up 2-bit KV decode -- Affine folding of
    KV dequantization", paragraph on the encoding: a 2- or 4-bit code q,
    a group of codes shares one scale and one offset, value = s*q + z;
  * the same page, fold-placement table: groups run token-wise (along the
    channels of one token) or channel-wise (along the tokens of one channel);
  * the same page, results paragraph: 32 query heads, 8 KV heads, head
    dimension 128, token-wise groups of 128.

Readings where the pages are silent (each one is listed in the design notes):
  * codes are unsigned, 0 .. 2**bits - 1;
  * min-max quantiser: s = (max - min) / (2**bits - 1) computed in fp32 and
    rounded to fp16, z = fp16(min), q = round-half-even((x - z16) / s16)
    clamped to the code range; a constant group gets s = 0 and q = 0;
  * a channel-wise group whose tokens run past the sequence length is
    quantised over its valid tokens only;
  * every random stream is ``numpy.random.default_rng([seed, workload id,
    tensor id, b, h])`` so any (sequence, KV head) slice can be regenerated
    on its own;
  * a rotated cache (``Spec.rotate``; the accuracy recipe the explainer's
    accuracy paragraph names, "OSCAR's rotations", and its related explainer
    on a Hadamard-rotated 2-bit KV cache) stores the quantised rows of x H,
    H = scipy.linalg.hadamard(D) / sqrt(D), where x are the drawn rows with
    their channel scales and outliers: the writer rotates, then quantises.
"""
from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np

TOKEN = "token"
CHANNEL = "channel"

# tensor ids for the random streams
_T_K, _T_V, _T_Q, _T_OUTLIER, _T_STD, _T_LENS, _T_POISON = range(7)


@dataclasses.dataclass(frozen=True)
class Spec:
    """Shape and value recipe of one synthetic workload."""

    name: str
    wid: int                  # workload id, part of every random stream key
    bits: int                 # 2 or 4
    k_layout: str             # TOKEN or CHANNEL
    v_layout: str
    group: int                # g: channels per group (token-wise) or tokens per group (channel-wise)
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    max_seq_len: int          # Tcap: allocated tokens per sequence
    ragged: bool = False      # lengths log-uniform in [ragged_lo, max_seq_len]
    ragged_lo: int = 1024
    seq_len: Optional[int] = None   # fixed length when not ragged (default Tcap)
    k_outlier_frac: float = 0.0     # fraction of K channels per KV head scaled by k_outlier_scale
    k_outlier_scale: float = 10.0
    channel_std_logu: Optional[tuple] = None  # (lo, hi) per-(head, channel) std, log-uniform
    seed: int = 0
    lens: Optional[tuple] = None    # explicit per-sequence lengths (edge-case tests)
    rotate: str = ""                # cache sides ("k", "v", "kv") stored as rows of x H (Hadamard-rotated)

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    def replace(self, **kw) -> "Spec":
        return dataclasses.replace(self, **kw)

    def seq_lens(self) -> np.ndarray:
        if self.lens is not None:
            return np.array(self.lens, dtype=np.int32)
        if self.ragged:
            rng = np.random.default_rng([self.seed, self.wid, _T_LENS])
            u = rng.uniform(math.log(self.ragged_lo), math.log(self.max_seq_len), size=self.batch)
            lens = np.floor(np.exp(u)).astype(np.int64)
            return np.clip(lens, self.ragged_lo, self.max_seq_len).astype(np.int32)
        t = self.max_seq_len if self.seq_len is None else self.seq_len
        return np.full(self.batch, t, dtype=np.int32)


def _base_specs():
    s = {}
    s["c1_tiny_int2"] = Spec("c1_tiny_int2", 1, 2, TOKEN, TOKEN, 128, 1, 4, 1, 128, 1024)
    for bits in (2, 4):
        s[f"c2_paper_int{bits}"] = Spec(f"c2_paper_int{bits}", 2, bits, TOKEN, TOKEN, 128, 16, 32, 8, 128, 8192,
                                        k_outlier_frac=0.05)
    s["c3_long_int2"] = Spec("c3_long_int2", 3, 2, TOKEN, TOKEN, 128, 4, 32, 8, 128, 131072)
    for bits in (2, 4):
        s[f"c4_channel_int{bits}"] = Spec(f"c4_channel_int{bits}", 4, bits, CHANNEL, CHANNEL, 128, 8, 32, 8, 128,
                                          32768, channel_std_logu=(0.1, 10.0))
    for bits in (2, 4):
        for g in (32, 64, 128):
            s[f"c5_ragged_int{bits}_g{g}"] = Spec(f"c5_ragged_int{bits}_g{g}", 5, bits, TOKEN, CHANNEL, g, 64, 32, 8,
                                                  128, 65536, ragged=True)
    return s


SPECS = _base_specs()


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even); returns fp32 holding bf16 values."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """The uint16 bit patterns of fp32 values that are already bf16-representable."""
    return (np.ascontiguousarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def quantize_minmax(x: np.ndarray, bits: int, axis: int, valid: Optional[np.ndarray] = None):
    """Min-max asymmetric quantisation of ``x`` along ``axis`` (the group axis).

    Returns (codes uint8, s fp16, z fp16); s and z have ``axis`` reduced.
    ``valid`` (bool, same shape as x) excludes entries from min/max; excluded
    entries get code 0.
    """
    levels = (1 << bits) - 1
    xf = np.asarray(x, dtype=np.float32)
    if valid is None:
        mn = xf.min(axis=axis)
        mx = xf.max(axis=axis)
    else:
        mn = np.where(valid, xf, np.inf).min(axis=axis)
        mx = np.where(valid, xf, -np.inf).max(axis=axis)
        empty = ~np.isfinite(mn)
        mn = np.where(empty, 0.0, mn).astype(np.float32)
        mx = np.where(empty, 0.0, mx).astype(np.float32)
    s16 = ((mx - mn) / np.float32(levels)).astype(np.float32).astype(np.float16)
    z16 = mn.astype(np.float16)
    s64 = np.expand_dims(s16.astype(np.float64), axis)
    z64 = np.expand_dims(z16.astype(np.float64), axis)
    q = xf.astype(np.float64)
    q -= z64
    q /= np.where(s64 == 0.0, 1.0, s64)      # a constant group (s = 0) keeps code 0 below
    np.rint(q, out=q)
    np.maximum(q, 0.0, out=q)
    np.minimum(q, float(levels), out=q)
    q = q.astype(np.uint8)
    q *= (s64 != 0.0).astype(np.uint8)
    if valid is not None:
        q *= valid.astype(np.uint8)
    return q, s16, z16


def _outlier_channels(spec: Spec, h: int) -> np.ndarray:
    n = int(round(spec.k_outlier_frac * spec.head_dim))
    rng = np.random.default_rng([spec.seed, spec.wid, _T_OUTLIER, h])
    return rng.choice(spec.head_dim, size=n, replace=False)


def _channel_std(spec: Spec, tensor: int, h: int) -> np.ndarray:
    lo, hi = spec.channel_std_logu
    rng = np.random.default_rng([spec.seed, spec.wid, _T_STD, tensor, h])
    return np.exp(rng.uniform(math.log(lo), math.log(hi), size=spec.head_dim)).astype(np.float32)


def _rotation(d: int) -> np.ndarray:
    from scipy.linalg import hadamard
    return hadamard(d) / math.sqrt(d)


_CHUNK = 65536  # tokens per generation step (a multiple of every group size)


def make_head(spec: Spec, b: int, h: int, seq_len: Optional[int] = None, poison: bool = False) -> dict:
    """Cache slice of one (sequence b, KV head h): codes and (s, z) for K and V.

    Values are drawn token by token from one stream per (b, h, tensor); only
    the valid tokens are drawn, in chunks (the same values as one draw).
    With ``poison`` the tokens past the sequence length get random codes and
    NaN scales/offsets, to show that nothing past the length reaches the result.
    """
    T, D, g = spec.max_seq_len, spec.head_dim, spec.group
    t_valid = int(spec.seq_lens()[b] if seq_len is None else seq_len)
    out = {}
    for tensor, name, layout in ((_T_K, "k", spec.k_layout), (_T_V, "v", spec.v_layout)):
        rng = np.random.default_rng([spec.seed, spec.wid, tensor, b, h])
        std = _channel_std(spec, tensor, h) if spec.channel_std_logu is not None else None
        outl = _outlier_channels(spec, h) if (tensor == _T_K and spec.k_outlier_frac > 0) else None
        q = np.zeros((T, D), np.uint8)
        sshape = (T, D // g) if layout == TOKEN else (T // g, D)
        s = np.zeros(sshape, np.float16)
        z = np.zeros(sshape, np.float16)
        for c0 in range(0, t_valid, _CHUNK):
            c1 = min(c0 + _CHUNK, t_valid)
            rows = -(-(c1 - c0) // g) * g if layout == CHANNEL else c1 - c0
            x = np.zeros((rows, D), np.float32)
            x[: c1 - c0] = rng.standard_normal((c1 - c0, D), dtype=np.float32)
            if std is not None:
                x *= std[None, :]
            if outl is not None:
                x[:, outl] *= np.float32(spec.k_outlier_scale)
            if name in spec.rotate:
                x = (x.astype(np.float64) @ _rotation(D)).astype(np.float32)
            if layout == TOKEN:
                qc, sc, zc = quantize_minmax(x.reshape(rows, D // g, g), spec.bits, axis=2)
                q[c0:c1] = qc.reshape(rows, D)
                s[c0:c1], z[c0:c1] = sc, zc
            else:
                valid = np.broadcast_to((np.arange(rows) < c1 - c0).reshape(rows // g, g, 1), (rows // g, g, D))
                qc, sc, zc = quantize_minmax(x.reshape(rows // g, g, D), spec.bits, axis=1, valid=valid)
                q[c0:c0 + rows] = qc.reshape(rows, D)
                s[c0 // g: (c0 + rows) // g], z[c0 // g: (c0 + rows) // g] = sc, zc
        if poison and t_valid < T:
            prng = np.random.default_rng([spec.seed, spec.wid, _T_POISON, tensor, b, h])
            q[t_valid:] = prng.integers(0, 1 << spec.bits, size=(T - t_valid, D), dtype=np.uint8)
            if layout == TOKEN:
                s[t_valid:] = np.float16(np.nan)
                z[t_valid:] = np.float16(np.nan)
            else:
                first_dead = -(-t_valid // g)
                s[first_dead:] = np.float16(np.nan)
                z[first_dead:] = np.float16(np.nan)
        out[name + "_codes"] = q
        out[name + "_scale"] = s
        out[name + "_zero"] = z
    return out


def make_query(spec: Spec) -> np.ndarray:
    """Query of the decode step: N(0,1) drawn in fp32, rounded to bf16; fp32 array [B, Hq, D]."""
    rng = np.random.default_rng([spec.seed, spec.wid, _T_Q])
    q = rng.standard_normal((spec.batch, spec.num_q_heads, spec.head_dim), dtype=np.float32)
    return bf16_round(q)


def scale_shape(spec: Spec, layout: str):
    T, D, g = spec.max_seq_len, spec.head_dim, spec.group
    return (T, D // g) if layout == TOKEN else (T // g, D)


def make_workload(spec: Spec, threads: Optional[int] = None, poison: bool = False) -> dict:
    """All inputs of one decode step, as numpy arrays in the boundary layouts.

    Keys: q (fp32 holding bf16 values, [B,Hq,D]), k_codes / v_codes (uint8
    [B,Hkv,Tcap,D]), k_scale / k_zero / v_scale / v_zero (fp16, token-wise
    [B,Hkv,Tcap,D/g], channel-wise [B,Hkv,Tcap/g,D]), seq_lens (int32 [B]).
    """
    B, H, T, D = spec.batch, spec.num_kv_heads, spec.max_seq_len, spec.head_dim
    lens = spec.seq_lens()
    w = {
        "q": make_query(spec),
        "seq_lens": lens,
        "k_codes": np.empty((B, H, T, D), np.uint8),
        "v_codes": np.empty((B, H, T, D), np.uint8),
        "k_scale": np.empty((B, H) + scale_shape(spec, spec.k_layout), np.float16),
        "k_zero": np.empty((B, H) + scale_shape(spec, spec.k_layout), np.float16),
        "v_scale": np.empty((B, H) + scale_shape(spec, spec.v_layout), np.float16),
        "v_zero": np.empty((B, H) + scale_shape(spec, spec.v_layout), np.float16),
    }

    def one(bh):
        b, h = bh
        head = make_head(spec, b, h, seq_len=int(lens[b]), poison=poison)
        for k, v in head.items():
            w[k][b, h] = v

    n = threads or min(16, os.cpu_count() or 1)
    jobs = [(b, h) for b in range(B) for h in range(H)]
    if n <= 1 or len(jobs) == 1:
        for j in jobs:
            one(j)
    else:
        with ThreadPoolExecutor(n) as ex:
            list(ex.map(one, jobs))
    return w


def algorithmic_bytes(spec: Spec, lens: Optional[np.ndarray] = None) -> int:
    """Bytes one decode step must move at least: packed K and V codes and their
    fp16 (s, z) for the valid tokens, the bf16 query, the bf16 output, the fp32
    lse and the int32 lengths."""
    if lens is None:
        lens = spec.seq_lens()
    D, H, g = spec.head_dim, spec.num_kv_heads, spec.group
    total = 0
    for t in lens.astype(np.int64):
        codes = 2 * t * D * spec.bits // 8
        sz = 0
        for layout in (spec.k_layout, spec.v_layout):
            if layout == TOKEN:
                sz += 2 * 2 * t * (D // g)
            else:
                sz += 2 * 2 * (-(-t // g)) * D
        total += H * (codes + sz)
    B, Hq = spec.batch, spec.num_q_heads
    total += 2 * B * Hq * D + 2 * B * Hq * D + 4 * B * Hq + 4 * B
    return int(total)


def make_sequence(spec: Spec, b: int, threads: Optional[int] = None, poison: bool = False) -> dict:
    """All KV heads of sequence b, stacked: codes [Hkv, Tcap, D], (s, z) [Hkv, ...]."""
    H = spec.num_kv_heads
    t = int(spec.seq_lens()[b])
    n = threads or min(16, os.cpu_count() or 1)
    if n > 1 and H > 1:
        with ThreadPoolExecutor(min(n, H)) as ex:
            heads = list(ex.map(lambda h: make_head(spec, b, h, seq_len=t, poison=poison), range(H)))
    else:
        heads = [make_head(spec, b, h, seq_len=t, poison=poison) for h in range(H)]
    return {k: np.stack([hd[k] for hd in heads]) for k in heads[0]}


def full_scale_shapes(spec: Spec) -> dict:
    B, H = spec.batch, spec.num_kv_heads
    ks = (B, H) + scale_shape(spec, spec.k_layout)
    vs = (B, H) + scale_shape(spec, spec.v_layout)
    return {"k_scale": ks, "k_zero": ks, "v_scale": vs, "v_zero": vs}


def make_append_case(seed: int, batch: int, num_kv_heads: int, max_seq_len: int, src_tokens: int, bits: int,
                     starts, counts, head_dim: int = 128, channel_std_logu=(0.1, 10.0)) -> dict:
    """Inputs of a quantise-and-append call (values only, no quantiser arithmetic).

    * k_src / v_src: fp32 arrays of bf16 values [B][Hkv][N][D], N(0,1) times a
      per-(head, channel) std drawn log-uniform in ``channel_std_logu``;
    * a cache that already holds arbitrary content: random packed words
      (uint32, the layouts of the C interface) and random fp16 bit patterns,
      NaN patterns included, for the scales and offsets of both layouts;
    * start / count: int32 [B] as given.
    """
    B, H, T, D, N = batch, num_kv_heads, max_seq_len, head_dim, src_tokens
    E = 32 // bits
    rng = np.random.default_rng([seed, 900, bits, B, H, T, N])
    lo, hi = channel_std_logu
    std = np.exp(rng.uniform(math.log(lo), math.log(hi), size=(2, 1, H, 1, D))).astype(np.float32)
    k = bf16_round(rng.standard_normal((B, H, N, D), dtype=np.float32) * std[0])
    v = bf16_round(rng.standard_normal((B, H, N, D), dtype=np.float32) * std[1])
    case = {
        "k_src": k, "v_src": v,
        "packed_k": rng.integers(0, 1 << 32, (B, H, T, D // E), dtype=np.uint64).astype(np.uint32),
        "packed_v": rng.integers(0, 1 << 32, (B, H, T // E, D), dtype=np.uint64).astype(np.uint32),
        "start": np.asarray(starts, np.int32), "count": np.asarray(counts, np.int32),
    }
    for side in ("k", "v"):
        for part in ("scale", "zero"):
            for layout in (TOKEN, CHANNEL):
                shp = (B, H, T, D // 32) if layout == TOKEN else (B, H, T // 32, D)  # sliced per g by the caller
                case[f"{side}_{part}_{layout}"] = rng.integers(0, 1 << 16, shp, dtype=np.uint32).astype(np.uint16)
    return case


def device_normal_bf16(shape, seed: int, device="cuda"):
    """N(0,1) values rounded to bf16, drawn on the device by a seeded torch
    generator (inputs too large to draw on the host in a test's time)."""
    import torch
    gen = torch.Generator(device=device).manual_seed(seed)
    return torch.randn(tuple(shape), generator=gen, device=device).to(torch.bfloat16)


def make_window(seed: int, batch: int, num_kv_heads: int, cap: int, lens, head_dim: int = 128, std: float = 1.0):
    """Full-precision window of recent tokens: keys and values N(0, std^2)
    rounded to bf16, fp32 arrays [B][Hkv][cap][D], and int32 lengths."""
    rng = np.random.default_rng([seed, 901, batch, num_kv_heads, cap])
    k = bf16_round((rng.standard_normal((batch, num_kv_heads, cap, head_dim)) * std).astype(np.float32))
    v = bf16_round((rng.standard_normal((batch, num_kv_heads, cap, head_dim)) * std).astype(np.float32))
    return {"k": k, "v": v, "lens": np.asarray(lens, np.int32)}


def make_block_table(seed: int, lens, blocks_per_seq: int, block_size: int, extra_blocks: int = 3):
    """A paged layout for sequences of the given lengths: each sequence's blocks
    below its length get distinct pool blocks in a seeded random order (the
    pool has ``extra_blocks`` blocks nobody uses); table entries at or past a
    sequence's length are -1.  Returns (table int32 [B, blocks_per_seq],
    num_blocks)."""
    lens = np.asarray(lens)
    used = [-(-int(t) // block_size) for t in lens]
    num_blocks = sum(used) + extra_blocks
    rng = np.random.default_rng([seed, 0x9A6E])
    perm = rng.permutation(num_blocks)
    table = np.full((len(lens), blocks_per_seq), -1, np.int32)
    k = 0
    for b, n in enumerate(used):
        table[b, :n] = perm[k:k + n]
        k += n
    return table, num_blocks


def make_pool(spec: Spec, table, num_blocks: int, block_size: int, poison: bool = True) -> dict:
    """Pools of a paged cache holding the spec's sequences: block table[b, j] of
    every array gets sequence b's tokens j*P .. j*P + P - 1 (P = block_size;
    scale rows P/g per block for a channel-wise side).  Blocks no sequence
    uses hold random codes and NaN scales/offsets (``poison``).  Keys as
    ``make_workload`` with num_blocks in place of B and P in place of Tcap."""
    P, H, D, g = block_size, spec.num_kv_heads, spec.head_dim, spec.group
    table = np.asarray(table)

    def rows(layout):
        return P if layout == TOKEN else P // g

    pool = {}
    for name, layout, cols in (("k", spec.k_layout, None), ("v", spec.v_layout, None)):
        pool[name + "_codes"] = np.zeros((num_blocks, H, P, D), np.uint8)
        sc = (num_blocks, H, rows(layout), D // g if layout == TOKEN else D)
        pool[name + "_scale"] = np.zeros(sc, np.float16)
        pool[name + "_zero"] = np.zeros(sc, np.float16)
    used = np.zeros(num_blocks, bool)
    for b in range(table.shape[0]):
        seq = make_sequence(spec, b)
        for j in range(table.shape[1]):
            blk = int(table[b, j])
            if blk < 0:
                continue
            used[blk] = True
            for name, layout in (("k", spec.k_layout), ("v", spec.v_layout)):
                pool[name + "_codes"][blk] = seq[name + "_codes"][:, j * P:(j + 1) * P]
                r = rows(layout)
                for part in ("_scale", "_zero"):
                    pool[name + part][blk] = seq[name + part][:, j * r:(j + 1) * r]
    if poison:
        rng = np.random.default_rng([spec.seed, spec.wid, _T_POISON, 0x9A6E])
        for blk in np.nonzero(~used)[0]:
            for name in ("k", "v"):
                pool[name + "_codes"][blk] = rng.integers(0, 1 << spec.bits, size=(H, P, D), dtype=np.uint8)
                pool[name + "_scale"][blk] = np.float16(np.nan)
                pool[name + "_zero"][blk] = np.float16(np.nan)
    return pool
