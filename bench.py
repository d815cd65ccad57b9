"""Benchmark: one decode step of the long-context INT2 workload on one MI355X.

Workload (default): batch 4, 32 query heads / 8 KV heads (GQA 4), head_dim
128, 131072 tokens per sequence, 2-bit codes, token-wise K and V groups of
128, K/V ~ N(0,1) min-max quantised, bf16 query -- one layer's decode step.

A step is one call of foscar_decode_int2 (one kernel launch: split-KV over
the whole chip plus the log-sum-exp merge).  Inputs are staged in HBM before
the timed region; steps rotate over --copies independent copies of the cache
so that every step streams its cache from HBM rather than from the 256 MB
Infinity Cache.

Prints one JSON line: metric/value (achieved HBM GB/s of algorithmic bytes per
step), ms_per_step, a roofline object for the decode kernel (HIP events on
the launch stream; rocprofv3 summaries of the same command are committed
under profiles/), the CPU oracle timed on a bounded sample, and (default run)
"int4": the paper-shaped INT4 step, timed the same way by a child run.
"""
import argparse
import hashlib
import json
import math
import os
import re
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "INT2/INT4 decode-attn achieved HBM GB/s (% of 8 TB/s) and µs/step"
# what the decode kernel computes in, by key layout
_ARITH = {
    "token": ("fp4/fp8 QK^T, f16 PV",
              "QK^T on the block-scaled matrix cores: key codes as fp4 (INT2) / fp8 (INT4) operands, the query as "
              "two exact e4m3 terms, fp32 accumulation; PV with value codes as fp16 matrix-core operands "
              "(magic-exponent AND-OR), fp32 accumulation; bf16 out"),
    "channel": ("f16",
                "codes -> fp16 matrix-core operands (magic-exponent AND-OR) for QK^T and PV, fp32 accumulation, "
                "bf16 out"),
}
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=200,
                    help="untimed steps first (default 200: about 13 ms of the long-context step, so that clocks "
                         "and power have settled under HBM load before the timed pass)")
    ap.add_argument("--workload", default="c3_long_int2")
    ap.add_argument("--copies", type=int, default=0,
                    help="cache copies rotated over the steps (default: enough for at least 1 GiB)")
    ap.add_argument("--sustain", type=int, default=2000,
                    help="steps of a second, sustained pass reported beside the timed one (0: none)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU time of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--dump-steps", action="store_true", help="print each step's kernel microseconds to stderr")
    ap.add_argument("--window", type=int, default=0,
                    help="decode with a bf16 window of this many recent tokens per sequence beside the cache")
    ap.add_argument("--no-int4", action="store_true",
                    help="skip the INT4 companion (the paper-shaped INT4 step) of the default run")
    ap.add_argument("--paged", type=int, default=0,
                    help="decode over pools of blocks of this many tokens through a shuffled block table")
    ap.add_argument("--rotate", default="", choices=["", "k", "v", "kv"],
                    help="decode with the rotated-cache layout bits (the query rotated per step, the output "
                         "taken back for a rotated value side); the same synthetic cache, for timing")
    ap.add_argument("--op", choices=["decode", "quantize"], default="decode",
                    help="decode: the decode step (default); quantize: quantise-and-append of the workload's cache")
    ap.add_argument("--gqa", type=int, default=0,
                    help="query heads per KV head (overrides the workload's; 1-16; the break-even sweep)")
    ap.add_argument("--group", type=int, default=0, help="group size g (overrides the workload's: 32, 64 or 128)")
    ap.add_argument("--head-dim", type=int, default=0,
                    help="head dimension (overrides the workload's 128: a multiple of 32 up to 256, the "
                         "head-dim-generic kernels)")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB before warm-up (counter calibration)")
    return ap.parse_args()


def kernel_sha():
    """Hash of the library sources (kernels, launch and split plan), with the
    comments and blank space taken out, so that only a change of code changes
    it (the sources hold no string with a comment marker)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "bit_quantized_kv_split_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        code = " ".join(text.split())
        h.update(name.encode() + b"\0" + code.encode())
    return h.hexdigest()[:16]


def int4_companion():
    """The paper-shaped INT4 step (c2_paper_int4: 16 sequences x 8192 tokens, 32 / 8 heads, INT4
    token-wise, g = 128), timed by a child run of this script; a summary of its JSON line."""
    cmd = [sys.executable, os.path.abspath(__file__), "--workload", "c2_paper_int4", "--steps", "50", "--warmup",
           "200", "--sustain", "1000", "--no-cpu-baseline", "--no-int4"]
    try:
        r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
        d = json.loads([x for x in r.stdout.splitlines() if x.startswith("{")][-1])
    except (subprocess.SubprocessError, IndexError, ValueError) as e:
        return {"workload": "c2_paper_int4", "error": f"{type(e).__name__}: {e}"}
    ro, su = d["roofline"], d.get("sustained", {})
    return {"workload": d["config"]["workload"], "value": d["value"], "unit": d["unit"],
            "us_per_step": d["us_per_step"], "pct_of_peak_hbm": d["pct_of_peak_hbm"],
            "kernel_us_avg": ro["kernel_us_avg"], "kernel_us_p50": ro["kernel_us_p50"], "frac": ro["frac"],
            "sustained_us_per_step": round(su["ms_per_step"] * 1e3, 2) if su else None,
            "sustained_kernel_us_avg": su.get("kernel_us_avg"), "cache": d["cache"],
            "algorithmic_bytes_per_step": d["config"]["algorithmic_bytes_per_step"],
            "kernel_source_sha": d["kernel_source_sha"]}


def to_pool(c, spec, P, seed):
    """The staged contiguous cache `c` as pools of P-token blocks (include/foscar.h: the
    contiguous layouts with [num_blocks] for B and P for Tcap), logical block j of sequence b at
    pool block perm[b * (Tcap / P) + j] for a seeded random permutation; returns (pools, block
    table int32 [B, Tcap / P]).  Plumbing on the GPU: reshapes and one scatter per array."""
    import torch
    nb = spec.max_seq_len // P
    perm = torch.randperm(spec.batch * nb, generator=torch.Generator().manual_seed(1000 + seed))
    out = dict(c)
    for name in ("packed_k", "packed_v", "k_scale", "k_zero", "v_scale", "v_zero"):
        t = c[name]
        B, H, R, W = t.shape  # R rows per sequence: tokens, value words or channel-wise group rows
        x = t.reshape(B, H, nb, R // nb, W).permute(0, 2, 1, 3, 4).reshape(B * nb, H, R // nb, W)
        pool = torch.empty_like(x)
        pool[perm.to(x.device)] = x
        out[name] = pool
    return out, perm.reshape(spec.batch, nb).to(torch.int32).to(c["q"].device)


def traffic_per_launch(workload):
    """HBM bytes per launch from the committed rocprofv3 counter runs, if they
    were taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"decode_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_sha") != kernel_sha():
        return None
    return t.get("bytes_per_launch")


def _cpu_info():
    """Host CPU model, logical CPUs, and the CPUs this process may run on."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count() or 1
    return model, os.cpu_count() or 1, usable


def _slice_bytes(spec, t, G):
    D = spec.head_dim
    sz = 0
    for layout in (spec.k_layout, spec.v_layout):
        sz += 2 * 2 * (t * (D // spec.group) if layout == "token" else -(-t // spec.group) * D)
    return 2 * t * D * spec.bits // 8 + sz + 2 * 2 * G * D + 4 * G


def _oracle_worker(args):
    """One worker: build its (sequence, KV head) slices (not timed), wait for
    every worker, then time the oracle over them; returns (start, end, bytes)."""
    spec_name, spec_kw, q, lens, slices = args
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle
    import synth

    spec = synth.SPECS[spec_name].replace(**spec_kw) if spec_kw else synth.SPECS[spec_name]
    G = spec.num_q_heads // spec.num_kv_heads
    work = []
    for b, h in slices:
        head = synth.make_head(spec, b, h, seq_len=int(lens[b]))
        w = {k: v[None, None] for k, v in head.items()}
        w["q"] = q[b:b + 1, h * G:(h + 1) * G]
        w["seq_lens"] = np.array([lens[b]], np.int32)
        work.append((w, _slice_bytes(spec, int(lens[b]), G)))
    _BARRIER[0].wait()
    with threadpool_limits(1):
        t0 = time.perf_counter()
        done = 0
        for w, nb in work:
            oracle.decode_rows(w, [(0, i) for i in range(G)], k_layout=spec.k_layout, v_layout=spec.v_layout,
                               group=spec.group, sm_scale=spec.sm_scale)
            done += nb
        t1 = time.perf_counter()
    return t0, t1, done


_BARRIER = [None]


def _init_worker(barrier):
    _BARRIER[0] = barrier


def cpu_baseline(spec, q, lens, target_s, max_workers=16, spec_kw=None):
    """The fp64 oracle (numpy, one BLAS thread per process) timed on the host
    cores: one worker process per core (at most the box's 16-CPU share of one
    GPU), the same workload's (sequence, KV head) slices dealt round-robin, all
    workers started together after building their inputs; wall clock from the
    first start to the last end.  The sample is the whole step when one core's
    estimated share fits target_s, otherwise the first slices that do."""
    import multiprocessing as mp

    model, logical, usable = _cpu_info()
    workers = max(1, min(max_workers, usable))
    G = spec.num_q_heads // spec.num_kv_heads
    pairs = [(b, h) for b in range(spec.batch) for h in range(spec.num_kv_heads) if int(lens[b]) > 0]
    # one core runs the fp64 oracle at about 80 MB of cache per second (the long-context step: 3.8 s for 302 MB)
    est = [_slice_bytes(spec, int(lens[b]), G) / 8e7 for b, h in pairs]
    budget, take = target_s * workers, []
    for p, e in zip(pairs, est):
        if take and sum(est[:len(take)]) + e > budget:
            break
        take.append(p)
    workers = min(workers, len(take))
    # fresh interpreters (spawn): the workers hold nothing of this process's GPU state
    ctx = mp.get_context("spawn")
    barrier = ctx.Barrier(workers, timeout=600)
    chunks = [take[i::workers] for i in range(workers)]
    with ctx.Pool(workers, initializer=_init_worker, initargs=(barrier,)) as pool:
        res = pool.map(_oracle_worker, [(spec.name, spec_kw, q, lens, c) for c in chunks], chunksize=1)
    t0 = min(r[0] for r in res)
    t1 = max(r[1] for r in res)
    done = sum(r[2] for r in res)
    wall = t1 - t0
    whole = len(take) == len(pairs)
    return {"value": round(done / wall / 1e9, 4), "unit": "GB/s", "cores": workers, "kind": "oracle",
            "sample": f"{len(take)} of {len(pairs)} (sequence, KV head) slices ({'the whole step' if whole else 'first slices'}), "
                      f"{len(take) * G} query heads, fp64 numpy, {workers} worker processes x 1 BLAS thread; "
                      f"wall {wall:.2f} s",
            "seconds_per_step": round(wall * len(pairs) / len(take), 3),
            "host": {"cpu_model": model, "logical_cpus": logical, "usable_cpus": usable}}


def quantize_bytes(spec, tokens_per_head):
    """Algorithmic bytes of quantising tokens_per_head tokens of every (sequence,
    KV head): bf16 keys and values read, codes and (s, z) of both sides
    written (token-wise groups), plus start/count."""
    D = spec.head_dim
    per_token = 2 * 2 * D + 2 * D * spec.bits // 8 + 2 * 2 * 2 * (D // spec.group)
    return spec.batch * spec.num_kv_heads * tokens_per_head * per_token + 8 * spec.batch


def bench_quantize(args, spec):
    """Quantise-and-append of the whole cache (a prefill: every token of every
    sequence in one call) and of one token per sequence (a decode-time append),
    timed with events on the launch stream."""
    import numpy as np
    import torch

    import bit_quantized_kv_split_amd as fos
    import synth

    if spec.k_layout != "token" or spec.v_layout != "token":
        raise SystemExit("--op quantize measures token-wise workloads")
    B, H, T, D, E = spec.batch, spec.num_kv_heads, spec.max_seq_len, spec.head_dim, 32 // spec.bits
    dev = "cuda"
    k_src = synth.device_normal_bf16((B, H, T, D), 1234)
    v_src = synth.device_normal_bf16((B, H, T, D), 1235)
    pk = torch.zeros((B, H, T, D // E), dtype=torch.int32, device=dev)
    pv = torch.zeros((B, H, T // E, D), dtype=torch.int32, device=dev)
    sc = [torch.zeros((B, H, T, D // spec.group), dtype=torch.float16, device=dev) for _ in range(4)]
    fn = fos.foscar_quantize_int2 if spec.bits == 2 else fos.foscar_quantize_int4
    layout = fos.layout_bits("token", "token")
    zero = torch.zeros(B, dtype=torch.int32, device=dev)
    full = torch.full((B,), T, dtype=torch.int32, device=dev)
    one = torch.ones(B, dtype=torch.int32, device=dev)
    k1, v1 = k_src[:, :, :1].contiguous(), v_src[:, :, :1].contiguous()
    at = torch.full((B,), T // 2 + 3, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    lines = []
    for name, call, toks in (("prefill", lambda: fn(k_src, v_src, zero, full, pk, pv, *sc, layout, spec.group), T),
                             ("append", lambda: fn(k1, v1, at, one, pk, pv, *sc, layout, spec.group), 1)):
        for _ in range(args.warmup):
            call()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        for a, b in ev:
            a.record(stream)
            call()
            b.record(stream)
        torch.cuda.synchronize()
        ms = [a.elapsed_time(b) for a, b in ev]
        avg = sum(ms) / len(ms)
        alg = quantize_bytes(spec, toks)
        lines.append({"op": f"quantize_{name}", "workload": spec.name, "tokens_per_head": toks,
                      "us_avg": round(avg * 1e3, 2), "us_median": round(sorted(ms)[len(ms) // 2] * 1e3, 2),
                      "us_min": round(min(ms) * 1e3, 2), "algorithmic_bytes": alg,
                      "roofline": {"bound": "hbm", "achieved": round(alg / (avg * 1e-3) / 1e9, 2),
                                   "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                   "frac": round(alg / (avg * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}})
    for line in lines:
        print(json.dumps(line), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    # the metric names INT2 and INT4: the default run also times the paper-shaped INT4 step, in a
    # child process started before this one touches the GPU, and reports it beside its own line
    int4 = None
    if (args.op == "decode" and args.workload == "c3_long_int2" and not args.no_int4 and not args.window
            and not args.paged and not args.rotate and not args.gqa and not args.group and not args.copies
            and not args.head_dim):
        int4 = int4_companion()
    import numpy as np
    import torch

    import bit_quantized_kv_split_amd as fos
    import bit_quantized_kv_split_amd.staging as staging
    import synth

    spec_kw = {}
    if args.gqa:
        spec_kw["num_q_heads"] = args.gqa * synth.SPECS[args.workload].num_kv_heads
    if args.group:
        spec_kw["group"] = args.group
    if args.head_dim:
        spec_kw["head_dim"] = args.head_dim
    spec = synth.SPECS[args.workload].replace(**spec_kw)
    if synth.TOKEN in (spec.k_layout, spec.v_layout) and spec.head_dim % spec.group:
        print(f"bench.py: a token-wise group of {spec.group} channels does not divide head_dim {spec.head_dim}; "
              "pass --group", file=sys.stderr)
        sys.exit(2)
    dev_name = "cuda:0"
    torch.cuda.set_device(0)
    if args.op == "quantize":
        return bench_quantize(args, spec)
    q = synth.make_query(spec)
    lens = spec.seq_lens()
    alg = synth.algorithmic_bytes(spec, lens) + 2 * 2 * spec.batch * spec.num_kv_heads * args.window * spec.head_dim
    t_stage = time.perf_counter()
    base = staging.stage((spec.batch, spec.num_q_heads, spec.num_kv_heads, spec.max_seq_len, spec.head_dim),
                         spec.bits, q, lens, lambda b: synth.make_sequence(spec, b), synth.full_scale_shapes(spec),
                         device=dev_name)
    # cold cache: the steps rotate over independent copies of the whole cache, at least 1 GiB of
    # them, so a copy was last touched at least 1 GiB of reads ago (the Infinity Cache holds 256 MB)
    cache_bytes = sum(v.numel() * v.element_size() for v in base.values())
    n_copies = args.copies if args.copies > 0 else max(2, -(-(1 << 30) // cache_bytes))
    copies = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(n_copies - 1)]
    tables = [None] * len(copies)
    if args.paged > 0:  # each copy regrouped on the GPU into a pool of blocks in a seeded random order
        copies, tables = (list(x) for x in zip(*[to_pool(c, spec, args.paged, i) for i, c in enumerate(copies)]))
    torch.cuda.synchronize()
    stage_s = time.perf_counter() - t_stage
    layout = fos.layout_bits(spec.k_layout, spec.v_layout)
    dims = fos.make_dims(spec.batch, spec.num_q_heads, spec.num_kv_heads, spec.head_dim, spec.max_seq_len)
    fos.foscar_workspace_reserve(dims, spec.bits, layout, spec.group)
    splits, chunk = fos.foscar_split_plan(dims, spec.bits, layout, spec.group)
    outs = [(torch.empty((spec.batch, spec.num_q_heads, spec.head_dim), dtype=torch.bfloat16, device=dev_name),
             torch.empty((spec.batch, spec.num_q_heads), dtype=torch.float32, device=dev_name)) for _ in copies]
    # one prepared call per cache copy: arguments checked and marshalled once, a step is one C call
    window = [None] * len(copies)
    if args.window > 0:  # decode beside a full-precision window: still one launch per step
        win = synth.make_window(0, spec.batch, spec.num_kv_heads, args.window, [args.window] * spec.batch,
                                spec.head_dim)
        window = [(torch.from_numpy(win["k"]).to(torch.bfloat16).to(dev_name),
                   torch.from_numpy(win["v"]).to(torch.bfloat16).to(dev_name),
                   torch.from_numpy(win["lens"]).to(dev_name)) for _ in copies]
    call_layout = fos.layout_bits(spec.k_layout, spec.v_layout, args.rotate)
    calls = [fos.prepare_decode(spec.bits, c["q"], c["packed_k"], c["packed_v"], c["k_scale"], c["k_zero"],
                                c["v_scale"], c["v_zero"], c["seq_lens"], call_layout, spec.group, out=o, lse=l,
                                window=w, paged=t)
             for c, (o, l), w, t in zip(copies, outs, window, tables)]

    if args.calibrate_copy_mib > 0:  # a plain copy of known size, for HBM byte counters
        n = args.calibrate_copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev_name).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def timed_pass(steps, first, every=5):
        """`steps` steps back to back.  Every `every`-th step's decode dispatch
        records its own start and stop events (hipExtLaunchKernel), the span
        rocprofv3's kernel trace reports; events on every step would add about
        5 us of queue work per step to the wall time.  The stride of 5 walks
        through the cache copies.  Returns (wall seconds between the two
        synchronisations, sampled kernel ms)."""
        picks = [k for k in range(steps) if k % every == every // 2] or [0]
        ev = {k: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for k in picks}
        stream = torch.cuda.current_stream()
        for a, b in ev.values():  # recorded once so that the events exist
            a.record(stream)
            b.record(stream)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(steps):
            if k in ev:
                fos.foscar_record_next_launch(ev[k][0], ev[k][1])
            calls[(first + k) % len(calls)]()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return wall, [a.elapsed_time(b) for a, b in ev.values()]

    def pct(xs, p):
        xs = sorted(xs)
        return xs[min(len(xs) - 1, max(0, int(round(p / 100 * (len(xs) - 1)))))]

    for k in range(args.warmup):
        calls[k % len(calls)]()
    torch.cuda.synchronize()
    # the reported pass: exactly `steps` steps; ms_per_step and the roofline both come from it
    wall, kernel_ms = timed_pass(args.steps, args.warmup)
    # a sustained pass right after it (clock and power settle under continuous HBM load)
    sus_wall, sus_ms = timed_pass(args.sustain, args.warmup + args.steps) if args.sustain > 0 else (None, None)
    if args.dump_steps:
        print("kernel us per step:", " ".join(f"{x * 1e3:.1f}" for x in kernel_ms), file=sys.stderr)
    ms_per_step = wall * 1e3 / args.steps
    value = alg / (ms_per_step * 1e-3) / 1e9
    k_avg = sum(kernel_ms) / len(kernel_ms)
    achieved = alg / (k_avg * 1e-3) / 1e9
    assert torch.isfinite(outs[0][0].float()).all(), "non-finite output"
    cold = n_copies * cache_bytes >= (1 << 30)

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "us_per_step": round(ms_per_step * 1e3, 2),
        "pct_of_peak_hbm": round(100 * value / PEAK_HBM_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": _ARITH[spec.k_layout][0],
        "arith": _ARITH[spec.k_layout][1],
        "data": "synthetic",
        "cache": ("cold: " if cold else "WARM (rotation under 1 GiB): ")
                 + f"{n_copies} copies x {cache_bytes / 1e6:.1f} MB rotated over the steps",
        "config": {"workload": f"{spec.name}: batch {spec.batch}, {spec.num_q_heads} query heads / "
                               f"{spec.num_kv_heads} KV heads, head_dim {spec.head_dim}, {spec.max_seq_len} tokens, "
                               f"INT{spec.bits}, K {spec.k_layout}-wise / V {spec.v_layout}-wise, group {spec.group}",
                   "global_batch": spec.batch, "seq_len": spec.max_seq_len, "bits": spec.bits,
                   "k_layout": spec.k_layout, "v_layout": spec.v_layout, "group": spec.group,
                   "splits": splits, "chunk": chunk, "cache_copies": n_copies, "window_tokens": args.window,
                   "paged_block_tokens": args.paged, "rotated_sides": args.rotate,
                   "algorithmic_bytes_per_step": alg},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": None if (spec_kw or args.paged or args.rotate or args.window)
                     else traffic_per_launch(spec.name),
                     "kernel": ("split_decode (one launch per step)" if spec.head_dim == 128 else
                                "gd_split + gd_merge (the head-dim-generic pair of launches per step)"),
                     "kernel_us_avg": round(k_avg * 1e3, 2),
                     "kernel_us_p10": round(pct(kernel_ms, 10) * 1e3, 2),
                     "kernel_us_p50": round(pct(kernel_ms, 50) * 1e3, 2),
                     "kernel_us_p90": round(pct(kernel_ms, 90) * 1e3, 2),
                     "kernel_us_min": round(min(kernel_ms) * 1e3, 2),
                     "kernel_launches_timed": len(kernel_ms),
                     "timing": "HIP events recorded by every 5th decode dispatch of the pass that gives ms_per_step"},
        "staging_s": round(stage_s, 1),
        "kernel_source_sha": kernel_sha(),
    }
    if sus_wall is not None:
        sus_ms_step = sus_wall * 1e3 / args.sustain
        line["sustained"] = {"steps": args.sustain, "ms_per_step": round(sus_ms_step, 5),
                             "kernel_launches_timed": len(sus_ms),
                             "value": round(alg / (sus_ms_step * 1e-3) / 1e9, 2),
                             "kernel_us_avg": round(sum(sus_ms) / len(sus_ms) * 1e3, 2),
                             "kernel_us_p10": round(pct(sus_ms, 10) * 1e3, 2),
                             "kernel_us_p50": round(pct(sus_ms, 50) * 1e3, 2),
                             "kernel_us_p90": round(pct(sus_ms, 90) * 1e3, 2),
                             "ratio_to_reported": round(sus_ms_step / ms_per_step, 4)}
    if int4 is not None:
        line["int4"] = int4
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(spec, q, lens, args.cpu_seconds, spec_kw=spec_kw or None)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
