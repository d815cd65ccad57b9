"""Per-work-group timeline of one decode launch (measurement tool).

    python -m bit_quantized_kv_split_amd.build --timeline      # once: libfoscar_timeline.so
    python -m bit_quantized_kv_split_amd.timeline c3_long_int2 [--splits S] [--save PATH]

Runs the named synthetic workload through libfoscar_timeline.so -- the same
kernels as libfoscar.so with the timeline marks compiled in -- for a few
launches over rotating cache copies, then reads the marks of the last launch
and prints, per phase of a work item, the percentiles over all work items:
query prologue (item start to the first tile's operands), tile loop, epilogue
and hand-off (to the arrival count), merge (last work-group of a pair only),
and the end times; then the same per XCD.  Times are from s_memrealtime
(100 MHz) relative to the earliest item start.  Only the contiguous,
unrotated kernels carry the marks.
"""
import argparse
import ctypes
import os
import sys

import numpy as np


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("workload")
    ap.add_argument("--splits", type=int, default=0, help="ranges per work pair (default: the library's plan)")
    ap.add_argument("--launches", type=int, default=12)
    ap.add_argument("--save", default="", help="write the raw marks [work-group][item][8] to this .npy")
    args = ap.parse_args(argv)
    if args.splits:
        os.environ["FOSCAR_SPLITS"] = str(args.splits)

    from . import _lib, build
    if not os.path.exists(build.LIB_TIMELINE):
        raise SystemExit(f"{build.LIB_TIMELINE} is missing: python -m bit_quantized_kv_split_amd.build --timeline")
    _lib.LIB_PATH = build.LIB_TIMELINE
    import torch

    import synth
    from . import staging
    import bit_quantized_kv_split_amd as fos

    spec = synth.SPECS[args.workload]
    q = synth.make_query(spec)
    lens = spec.seq_lens()
    base = staging.stage((spec.batch, spec.num_q_heads, spec.num_kv_heads, spec.max_seq_len, spec.head_dim),
                         spec.bits, q, lens, lambda b: synth.make_sequence(spec, b), synth.full_scale_shapes(spec))
    cache_bytes = sum(v.numel() * v.element_size() for v in base.values())
    n_copies = max(2, -(-(1 << 30) // cache_bytes))
    copies = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(n_copies - 1)]
    lib = _lib.load()
    lib.foscar_timeline_read.argtypes = [ctypes.c_void_p, ctypes.c_int]

    def step(d):
        fos.decode(d["q"], d["packed_k"], d["packed_v"], d["k_scale"], d["k_zero"], d["v_scale"], d["v_zero"],
                   d["seq_lens"], bits=spec.bits, k_layout=spec.k_layout, v_layout=spec.v_layout, group=spec.group)

    lib.foscar_timeline_clear.argtypes = [ctypes.c_void_p]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for i in range(args.launches - 1):
        step(copies[i % n_copies])
    # cleared on the same stream right before the recorded launch, with no host wait in between, so the
    # recorded launch follows the others back to back (stale marks of earlier launches cannot remain)
    if lib.foscar_timeline_clear(stream) != 0:
        raise SystemExit("timeline clear failed")
    step(copies[(args.launches - 1) % n_copies])
    torch.cuda.synchronize()
    wgs = 8192
    buf = np.zeros((wgs, 8, 8), np.uint64)
    if lib.foscar_timeline_read(buf.ctypes.data, wgs) != 0:
        raise SystemExit("timeline read failed")
    if args.save:
        np.save(args.save, buf)
    report(spec, buf)


def report(spec, buf):
    t = buf.astype(np.int64)
    valid = t[:, :, 0] > 0
    if not valid.any():
        raise SystemExit("no marks recorded (is this workload served by the contiguous, unrotated kernels?)")
    t0 = t[:, :, 0][valid].min()
    us = lambda x: (x - t0) * 0.01  # noqa: E731  (100 MHz counter)
    st, pro, loop, hand, end = (us(t[:, :, k]) for k in range(5))
    has = lambda k: valid & (t[:, :, k] > 0)  # noqa: E731
    merged = valid & (t[:, :, 6] == 1)
    pct = lambda v: " / ".join(f"{x:.2f}" for x in np.percentile(v, [0, 10, 50, 90, 100]))  # noqa: E731
    n_items = int(valid.sum())
    per_wg = valid.sum(axis=1)
    print(f"{spec.name}: {int((per_wg > 0).sum())} work-groups, {n_items} work items "
          f"(items per work-group: {np.bincount(per_wg[per_wg > 0]).tolist()})")
    print("phase (us; min / p10 / p50 / p90 / max over work items):")
    print(f"  start                 {pct(st[valid])}")
    print(f"  query prologue        {pct((pro - st)[has(1)])}")
    print(f"  tile loop             {pct((loop - pro)[has(2) & has(1)])}")
    if has(3).any():
        print(f"  epilogue + hand-off   {pct((hand - loop)[has(3) & has(2)])}")
    if merged.any():
        print(f"  merge (merging WGs)   {pct((end - hand)[merged & has(3)])}")
    print(f"  end                   {pct(end[has(4)])}")
    last = np.where(has(4), end, 0).max(axis=1)
    xcc = (t[:, 0, 7] >> 32) & 0xF
    print("per XCD: work-groups, items, tile loop p50, last end p50 / max (us)")
    for x in range(8):
        sel = (xcc == x) & (per_wg > 0)
        if sel.any():
            lp = (loop - pro)[sel][(has(2) & has(1))[sel]]
            print(f"  XCD {x}: {int(sel.sum())}, {int(per_wg[sel].sum())}, {np.median(lp):.2f}, "
                  f"{np.median(last[sel]):.2f} / {last[sel].max():.2f}")
    print(f"launch span: {us(t[:, :, 4][has(4)].max()):.2f} us")


if __name__ == "__main__":
    sys.exit(main())
