"""CPU oracle for low-bit KV decode attention -- TEST INFRASTRUCTURE ONLY.

Only tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The GPU library never calls it, and it shares no code with the
GPU library (the seeded input generator in ``synth`` is the only module both
sides use, and it holds none of the attention arithmetic).

What it computes (fp64 throughout):

* ``dequantize``: value = s*q + z with one (s, z) per group -- FOSCAR explainer
  ("FOSCAR speeds up 2-bit KV decode", learnaivisually), encoding paragraph;
  groups token-wise or channel-wise -- same page, fold-placement table.
* ``attend``: one query row against the dequantised keys and values with a
  two-pass softmax.  This is the "dequantized attention output" that the
  FOSCAR abstract (arXiv 2611.09722) says folding preserves in exact
  arithmetic; the oracle computes it directly, with no folding and no online
  softmax.
* ``decode`` / ``decode_rows``: every (sequence, query head) of a decode step;
  query head i reads KV head i // (Hq / Hkv) (GQA: "4 query heads per KV head",
  explainer, issue-budget paragraph).
* ``decode_window_rows``: the same decode step with a window of recent tokens
  kept in full precision beside the quantised cache (the accuracy recipe the
  explainer's accuracy paragraph names: "full-precision windows of recent
  tokens"); attention is over the union of the T_b dequantised cache tokens
  and the window's tokens, computed by ``attend`` on the concatenation.
* ``hadamard`` / ``round_bf16`` / ``attend_rotated`` and the ``rotate``
  argument of the decode functions: a rotated cache, the accuracy recipe the
  explainer's accuracy paragraph names ("OSCAR's rotations") and its related
  explainers list (KVarN, a Hadamard-rotated 2-bit KV cache).  The cache holds
  the quantised rows of K R and/or V R for an orthonormal R (the normalised
  Sylvester-Hadamard matrix of order D unless given); since R R^T = I the
  scores are (q R).(k R) and the output is (sum_t p_t v_t R) R^T.  Readings
  the pages leave open, taken here: the rotated query is held in bf16, the
  precision of the query itself (round to nearest even); a full-precision
  window holds the model's own, unrotated rows.
* ``gather_paged`` / ``decode_paged_rows``: a paged cache (pools of blocks of
  P tokens reached through a block table, the KV layout of the serving
  systems the explainer's integration paragraph names) is first put back in
  logical token order, then decoded as above: paging is an addressing
  indirection, not arithmetic.
* ``pack_k`` / ``pack_v`` / ``unpack_k`` / ``unpack_v``: the packed code layout
  of the C interface, written from its specification (keys packed along
  channels, values packed along tokens; even elements of a word in its low
  half-word, odd elements in its high half-word).

Parity pins: every function here is pinned by ``tests/test_oracle_pins.py``
(worked receipt, exact fold-vs-unfold, closed forms, invariants, a textbook
special case, golden packed words).
"""
from __future__ import annotations

import math

import numpy as np

TOKEN = "token"
CHANNEL = "channel"


def dequantize(codes, scale, zero, layout: str, group: int) -> np.ndarray:
    """Dequantised cache slice [T, D] in fp64: x = s*q + z.

    codes: [T, D] integer codes; scale, zero: fp16, [T, D/g] (token-wise:
    group = g consecutive channels of one token) or [T/g, D] (channel-wise:
    group = g consecutive tokens of one channel).  Every product is exact in
    fp64 (an 11-bit significand times a 4-bit integer plus an fp16 value).
    """
    q = np.asarray(codes, dtype=np.float64)
    s = np.asarray(scale, dtype=np.float64)
    z = np.asarray(zero, dtype=np.float64)
    T, D = q.shape
    if layout == TOKEN:
        s_full = np.repeat(s, group, axis=1)[:T, :D]
        z_full = np.repeat(z, group, axis=1)[:T, :D]
    elif layout == CHANNEL:
        s_full = np.repeat(s, group, axis=0)[:T, :D]
        z_full = np.repeat(z, group, axis=0)[:T, :D]
    else:
        raise ValueError(layout)
    return s_full * q + z_full


def attend(q_row, k_hat, v_hat, sm_scale: float):
    """Softmax attention of one query row over T dequantised tokens.

    Returns (o [D] fp64, lse fp64) with lse = ln sum_t exp(sm_scale * q.k_t).
    Two passes: the max first, then the exponentials.  T = 0 gives o = 0 and
    lse = -inf.
    """
    q = np.asarray(q_row, dtype=np.float64)
    T = k_hat.shape[0]
    if T == 0:
        return np.zeros(v_hat.shape[1]), -math.inf
    scores = sm_scale * (k_hat @ q)
    m = scores.max()
    w = np.exp(scores - m)
    l = w.sum()
    p = w / l
    assert abs(p.sum() - 1.0) < 1e-9
    o = p @ v_hat
    return o, m + math.log(l)


def sylvester(n: int) -> np.ndarray:
    """The +-1 Sylvester-Hadamard matrix of order n (a power of two):
    S_1 = [1], S_2m = [[S_m, S_m], [S_m, -S_m]]; entry (i, j) is
    (-1)^popcount(i & j)."""
    if n < 1 or n & (n - 1):
        raise ValueError("order must be a power of two")
    h = np.ones((1, 1))
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def hadamard(n: int) -> np.ndarray:
    """Orthonormal Sylvester-Hadamard matrix of order n: sylvester(n) /
    sqrt(n), symmetric and its own inverse."""
    return sylvester(n) / math.sqrt(n)


def round_bf16(x) -> np.ndarray:
    """Nearest bf16 value (8 significant bits), ties to even, for values in
    bf16's normal range (the query values this is applied to)."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)              # x = m 2^e with 1/2 <= |m| < 1
    return np.ldexp(np.round(m * 256.0), e - 8)  # np.round: half to even


def attend_rotated(q_row, k_hat, v_hat, sm_scale: float, *, rot_k: bool, rot_v: bool, rot=None,
                   round_query: bool = True, win_k=None, win_v=None):
    """Softmax attention of one query row over a rotated cache.

    k_hat / v_hat [T, D] are the dequantised cache rows as stored: k R when
    rot_k, v R when rot_v (R = ``rot``, default ``hadamard(D)``).  The query
    that meets the stored keys is q R (rounded to bf16 when round_query); the
    cache's weighted value sum is taken back to the model's basis by R^T.
    win_k / win_v [W, D] (optional) are full-precision window rows in the
    model's basis, met by q itself; one softmax runs over the T + W scores.
    Returns (o [D], lse) like ``attend``.
    """
    q = np.asarray(q_row, dtype=np.float64)
    D = q.shape[0]
    R = hadamard(D) if rot is None else np.asarray(rot, dtype=np.float64)
    qk = q @ R if rot_k else q
    if rot_k and round_query:
        qk = round_bf16(qk)
    k_hat = np.asarray(k_hat, dtype=np.float64)
    v_hat = np.asarray(v_hat, dtype=np.float64)
    wk = np.zeros((0, D)) if win_k is None else np.asarray(win_k, dtype=np.float64)
    wv = np.zeros((0, D)) if win_v is None else np.asarray(win_v, dtype=np.float64)
    T = k_hat.shape[0]
    scores = np.concatenate([sm_scale * (k_hat @ qk), sm_scale * (wk @ q)])
    if scores.size == 0:
        return np.zeros(D), -math.inf
    m = scores.max()
    w = np.exp(scores - m)
    l = w.sum()
    p = w / l
    oc = p[:T] @ v_hat
    if rot_v:
        oc = oc @ R.T
    return oc + p[T:] @ wv, m + math.log(l)


def _rot_flags(rotate: str):
    if rotate not in ("", "k", "v", "kv"):
        raise ValueError(rotate)
    return "k" in rotate, "v" in rotate


def _head(w: dict, b: int, h: int, t: int, k_layout: str, v_layout: str, group: int):
    k_hat = dequantize(w["k_codes"][b, h, :t], _scale_rows(w["k_scale"][b, h], k_layout, group, t),
                       _scale_rows(w["k_zero"][b, h], k_layout, group, t), k_layout, group)
    v_hat = dequantize(w["v_codes"][b, h, :t], _scale_rows(w["v_scale"][b, h], v_layout, group, t),
                       _scale_rows(w["v_zero"][b, h], v_layout, group, t), v_layout, group)
    return k_hat, v_hat


def _scale_rows(s, layout: str, group: int, t: int):
    """The (s, z) rows that cover the first t tokens."""
    if layout == TOKEN:
        return s[:t]
    return s[: -(-t // group)]


def decode(w: dict, *, k_layout: str, v_layout: str, group: int, sm_scale: float,
           num_kv_heads: int | None = None, rotate: str = ""):
    """Whole decode step.  ``w`` holds q [B,Hq,D], k_codes / v_codes
    [B,Hkv,Tcap,D], k_scale / k_zero / v_scale / v_zero in the layouts of
    ``dequantize`` (with leading [B,Hkv]) and seq_lens [B] (clamped to
    [0, Tcap]).  ``rotate`` ("", "k", "v" or "kv") names the sides whose
    cache holds Hadamard-rotated rows (``attend_rotated``).  Returns
    (out [B,Hq,D] fp64, lse [B,Hq] fp64)."""
    q = np.asarray(w["q"], dtype=np.float64)
    B, Hq, D = q.shape
    rows = [(b, i) for b in range(B) for i in range(Hq)]
    o, l = decode_rows(w, rows, k_layout=k_layout, v_layout=v_layout, group=group, sm_scale=sm_scale,
                       rotate=rotate)
    return o.reshape(B, Hq, D), l.reshape(B, Hq)


def decode_rows(w: dict, rows, *, k_layout: str, v_layout: str, group: int, sm_scale: float, rotate: str = ""):
    """Like ``decode`` for a list of (b, query head) pairs only."""
    rot_k, rot_v = _rot_flags(rotate)
    q = np.asarray(w["q"], dtype=np.float64)
    B, Hq, D = q.shape
    Hkv = w["k_codes"].shape[1]
    Tcap = w["k_codes"].shape[2]
    G = Hq // Hkv
    out = np.zeros((len(rows), D))
    lse = np.zeros(len(rows))
    cache = {}
    for n, (b, i) in enumerate(rows):
        h = i // G
        t = int(min(max(int(w["seq_lens"][b]), 0), Tcap))
        if (b, h) not in cache:
            cache = {(b, h): _head(w, b, h, t, k_layout, v_layout, group)}
        k_hat, v_hat = cache[(b, h)]
        if rot_k or rot_v:
            out[n], lse[n] = attend_rotated(q[b, i], k_hat, v_hat, sm_scale, rot_k=rot_k, rot_v=rot_v)
        else:
            out[n], lse[n] = attend(q[b, i], k_hat, v_hat, sm_scale)
    return out, lse


def decode_window_rows(w: dict, win: dict, rows, *, k_layout: str, v_layout: str, group: int, sm_scale: float,
                       rotate: str = ""):
    """``decode_rows`` over the quantised cache of ``w`` plus a full-precision
    window: win["k"], win["v"] [B][Hkv][W][D] (bf16 values, any float dtype),
    win["lens"] [B] (clamped to [0, W]).  Returns (out [n, D], lse [n]) in
    fp64; a row with no token at all gives out = 0, lse = -inf.  With
    ``rotate``, the cache sides it names hold rotated rows and the window the
    model's own (``attend_rotated``)."""
    rot_k, rot_v = _rot_flags(rotate)
    q = np.asarray(w["q"], dtype=np.float64)
    B, Hq, D = q.shape
    Hkv = w["k_codes"].shape[1]
    Tcap = w["k_codes"].shape[2]
    W = np.asarray(win["k"]).shape[2]
    G = Hq // Hkv
    out = np.zeros((len(rows), D))
    lse = np.zeros(len(rows))
    for n, (b, i) in enumerate(rows):
        h = i // G
        t = int(min(max(int(w["seq_lens"][b]), 0), Tcap))
        wl = int(min(max(int(win["lens"][b]), 0), W))
        k_hat, v_hat = _head(w, b, h, t, k_layout, v_layout, group)
        if rot_k or rot_v:
            out[n], lse[n] = attend_rotated(q[b, i], k_hat, v_hat, sm_scale, rot_k=rot_k, rot_v=rot_v,
                                            win_k=np.asarray(win["k"], np.float64)[b, h, :wl],
                                            win_v=np.asarray(win["v"], np.float64)[b, h, :wl])
            continue
        k_all = np.concatenate([k_hat, np.asarray(win["k"], np.float64)[b, h, :wl]], axis=0)
        v_all = np.concatenate([v_hat, np.asarray(win["v"], np.float64)[b, h, :wl]], axis=0)
        out[n], lse[n] = attend(q[b, i], k_all, v_all, sm_scale)
    return out, lse


def gather_paged(pool: dict, block_table, block_size: int, *, k_layout: str, v_layout: str, group: int) -> dict:
    """The contiguous cache of a paged one.

    ``pool`` holds k_codes / v_codes [NB, Hkv, P, D] and k_scale / k_zero /
    v_scale / v_zero with P in place of Tcap ([NB, Hkv, P, D/g] token-wise,
    [NB, Hkv, P/g, D] channel-wise); ``block_table`` [B, nb] maps logical block
    j of sequence b (tokens j*P .. j*P + P - 1) to pool block block_table[b, j].
    An entry outside [0, NB) stands for a block of zeros (codes, scales and
    offsets).  Returns the same keys laid out [B, Hkv, nb*P, ...] (the layout
    ``decode_rows`` reads), token t of sequence b at position t.
    """
    table = np.asarray(block_table)
    B, nb = table.shape
    P = int(block_size)
    out = {}
    for name in ("k_codes", "v_codes", "k_scale", "k_zero", "v_scale", "v_zero"):
        src = np.asarray(pool[name])
        NB, H = src.shape[0], src.shape[1]
        rows = src.shape[2]            # per block: P token rows, or P/g group rows
        dst = np.zeros((B, H, nb * rows) + src.shape[3:], src.dtype)
        for b in range(B):
            for j in range(nb):
                blk = int(table[b, j])
                if 0 <= blk < NB:
                    dst[b, :, j * rows:(j + 1) * rows] = src[blk]
        out[name] = dst
    return out


def decode_paged_rows(w_pool: dict, block_table, block_size: int, rows, *, k_layout: str, v_layout: str,
                      group: int, sm_scale: float, rotate: str = ""):
    """``decode_rows`` over a paged cache: w_pool holds q, seq_lens and the pools
    (see ``gather_paged``); only the blocks below each sequence's length are
    looked up (table entries past it may hold anything)."""
    table = np.array(block_table, dtype=np.int64)
    lens = np.asarray(w_pool["seq_lens"])
    for b in range(table.shape[0]):
        used = -(-int(max(lens[b], 0)) // block_size)
        table[b, used:] = -1
    w = gather_paged(w_pool, table, block_size, k_layout=k_layout, v_layout=v_layout, group=group)
    w["q"] = w_pool["q"]
    w["seq_lens"] = w_pool["seq_lens"]
    return decode_rows(w, rows, k_layout=k_layout, v_layout=v_layout, group=group, sm_scale=sm_scale,
                       rotate=rotate)


# ---------------------------------------------------------------------------
# Packed code layout of the C interface, written from its specification.
# E = 32 / bits codes per 32-bit word, packed along the axis the consuming
# product sums over:
#   keys:   word [t][c // E] holds channels E*(c // E) .. + E-1 of token t
#   values: word [t // E][c] holds tokens   E*(t // E) .. + E-1 of channel c
# Inside a word, element e (0 .. E-1) occupies bits
#   [bits*(e // 2) + 16*(e % 2), + bits)
# i.e. even elements fill the low half-word and odd elements the high
# half-word, each half in increasing order from bit 0 (resp. bit 16).
# ---------------------------------------------------------------------------

def _per_word(bits: int) -> int:
    if bits not in (2, 4):
        raise ValueError("bits must be 2 or 4")
    return 32 // bits


def element_shift(bits: int, e: int) -> int:
    """Bit offset of element e inside its word."""
    return bits * (e // 2) + 16 * (e % 2)


def pack_k(codes, bits: int) -> np.ndarray:
    """codes [..., T, D] -> uint32 [..., T, D*bits/32], packed along channels."""
    E = _per_word(bits)
    c = np.asarray(codes, dtype=np.uint32)
    *lead, T, D = c.shape
    c = c.reshape(*lead, T, D // E, E)
    word = np.zeros((*lead, T, D // E), dtype=np.uint32)
    for e in range(E):
        word |= (c[..., e] & ((1 << bits) - 1)) << np.uint32(element_shift(bits, e))
    return word


def unpack_k(words, bits: int, head_dim: int) -> np.ndarray:
    E = _per_word(bits)
    wv = np.asarray(words, dtype=np.uint32)
    *lead, T, W = wv.shape
    out = np.zeros((*lead, T, W, E), dtype=np.uint8)
    for e in range(E):
        out[..., e] = (wv >> np.uint32(element_shift(bits, e))) & ((1 << bits) - 1)
    return out.reshape(*lead, T, W * E)[..., :head_dim]


def pack_v(codes, bits: int) -> np.ndarray:
    """codes [..., T, D] -> uint32 [..., T/E, D], packed along tokens."""
    E = _per_word(bits)
    c = np.asarray(codes, dtype=np.uint32)
    *lead, T, D = c.shape
    c = c.reshape(*lead, T // E, E, D)
    word = np.zeros((*lead, T // E, D), dtype=np.uint32)
    for e in range(E):
        word |= (c[..., e, :] & ((1 << bits) - 1)) << np.uint32(element_shift(bits, e))
    return word


def unpack_v(words, bits: int) -> np.ndarray:
    E = _per_word(bits)
    wv = np.asarray(words, dtype=np.uint32)
    *lead, W, D = wv.shape
    out = np.zeros((*lead, W, E, D), dtype=np.uint8)
    for e in range(E):
        out[..., e, :] = (wv >> np.uint32(element_shift(bits, e))) & ((1 << bits) - 1)
    return out.reshape(*lead, W * E, D)
