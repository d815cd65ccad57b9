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
under profiles/), and the CPU oracle timed on a bounded sample.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "INT2/INT4 decode-attn achieved HBM GB/s (% of 8 TB/s) and µs/step"
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="c3_long_int2")
    ap.add_argument("--copies", type=int, default=2, help="independent cache copies rotated over the steps")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU time of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--dump-steps", action="store_true", help="print each step's kernel microseconds to stderr")
    ap.add_argument("--window", type=int, default=0,
                    help="decode with a bf16 window of this many recent tokens per sequence beside the cache")
    ap.add_argument("--op", choices=["decode", "quantize"], default="decode",
                    help="decode: the decode step (default); quantize: quantise-and-append of the workload's cache")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB before warm-up (counter calibration)")
    return ap.parse_args()


def kernel_sha():
    """Hash of the library sources (kernels, launch and split plan)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "bit_quantized_kv_split_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


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


def cpu_baseline(spec, q, lens, target_s):
    """The fp64 oracle (single-threaded numpy) on the first (sequence, KV head)
    slices of the same workload until about target_s seconds of CPU work."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle
    import synth

    G = spec.num_q_heads // spec.num_kv_heads
    done_bytes, spent, slices = 0, 0.0, 0
    D = spec.head_dim
    for b in range(spec.batch):
        for h in range(spec.num_kv_heads):
            head = synth.make_head(spec, b, h, seq_len=int(lens[b]))  # not timed
            w = {k: v[None, None] for k, v in head.items()}
            w["q"] = q[b:b + 1, h * G:(h + 1) * G]
            w["seq_lens"] = np.array([lens[b]], np.int32)
            with threadpool_limits(1):
                t0 = time.perf_counter()
                oracle.decode_rows(w, [(0, i) for i in range(G)], k_layout=spec.k_layout, v_layout=spec.v_layout,
                                   group=spec.group, sm_scale=spec.sm_scale)
                spent += time.perf_counter() - t0
            t = int(lens[b])
            sz = 0
            for layout in (spec.k_layout, spec.v_layout):
                sz += 2 * 2 * (t * (D // spec.group) if layout == "token" else -(-t // spec.group) * D)
            done_bytes += 2 * t * D * spec.bits // 8 + sz + 2 * 2 * G * D + 4 * G
            slices += 1
            if spent >= target_s:
                break
        if spent >= target_s:
            break
    return {"value": round(done_bytes / spent / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{slices} of {spec.batch * spec.num_kv_heads} (sequence, KV head) slices, "
                      f"{slices * G} query heads, fp64 numpy, BLAS limited to 1 thread; {spent:.1f} s",
            "seconds_per_step_extrapolated": round(spent / slices * spec.batch * spec.num_kv_heads, 2)}


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
    import numpy as np
    import torch

    import bit_quantized_kv_split_amd as fos
    import bit_quantized_kv_split_amd.staging as staging
    import synth

    spec = synth.SPECS[args.workload]
    dev_name = "cuda:0"
    torch.cuda.set_device(0)
    if args.op == "quantize":
        return bench_quantize(args, spec)
    q = synth.make_query(spec)
    lens = spec.seq_lens()
    t_stage = time.perf_counter()
    base = staging.stage((spec.batch, spec.num_q_heads, spec.num_kv_heads, spec.max_seq_len, spec.head_dim),
                         spec.bits, q, lens, lambda b: synth.make_sequence(spec, b), synth.full_scale_shapes(spec),
                         device=dev_name)
    copies = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(max(1, args.copies) - 1)]
    torch.cuda.synchronize()
    stage_s = time.perf_counter() - t_stage
    layout = fos.layout_bits(spec.k_layout, spec.v_layout)
    dims = fos.make_dims(spec.batch, spec.num_q_heads, spec.num_kv_heads, spec.head_dim, spec.max_seq_len)
    fos.foscar_workspace_reserve(dims, spec.bits, layout, spec.group)
    splits, chunk = fos.foscar_split_plan(dims, spec.bits, layout, spec.group)
    outs = [(torch.empty((spec.batch, spec.num_q_heads, spec.head_dim), dtype=torch.bfloat16, device=dev_name),
             torch.empty((spec.batch, spec.num_q_heads), dtype=torch.float32, device=dev_name)) for _ in copies]
    # one prepared call per cache copy: arguments checked and marshalled once, a step is one C call
    if args.window > 0:  # decode with a full-precision window: one call = window kernel + decode kernel
        win = synth.make_window(0, spec.batch, spec.num_kv_heads, args.window, [args.window] * spec.batch,
                                spec.head_dim)
        wins = [(torch.from_numpy(win["k"]).to(torch.bfloat16).to(dev_name),
                 torch.from_numpy(win["v"]).to(torch.bfloat16).to(dev_name),
                 torch.from_numpy(win["lens"]).to(dev_name)) for _ in copies]
        calls = [fos.prepare_decode(spec.bits, c["q"], c["packed_k"], c["packed_v"], c["k_scale"], c["k_zero"],
                                    c["v_scale"], c["v_zero"], c["seq_lens"], layout, spec.group, out=o, lse=l,
                                    window=w)
                 for c, (o, l), w in zip(copies, outs, wins)]
    else:
        calls = [fos.prepare_decode(spec.bits, c["q"], c["packed_k"], c["packed_v"], c["k_scale"], c["k_zero"],
                                    c["v_scale"], c["v_zero"], c["seq_lens"], layout, spec.group, out=o, lse=l)
                 for c, (o, l) in zip(copies, outs)]

    def step(k):
        calls[k % len(calls)]()

    if args.calibrate_copy_mib > 0:  # a plain copy of known size, for HBM byte counters
        n = args.calibrate_copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev_name).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    # whole-job throughput: exactly `steps` steps back to back, nothing else on the stream
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(k)
    enqueued = time.perf_counter() - t0
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # kernel durations, in a second pass of as many steps: events recorded by each decode
    # dispatch itself (hipExtLaunchKernel), the span rocprofv3's kernel trace reports;
    # recorded once first so that they exist
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for a, b in ev:
        a.record(stream)
        b.record(stream)
    torch.cuda.synchronize()
    for k in range(args.steps):
        if args.window > 0:  # two kernels per step: stream events around both
            ev[k][0].record(stream)
            step(k)
            ev[k][1].record(stream)
        else:
            fos.foscar_record_next_launch(ev[k][0], ev[k][1])
            step(k)
    torch.cuda.synchronize()
    kernel_ms = [a.elapsed_time(b) for a, b in ev]
    if args.dump_steps:
        print("kernel us per step:", " ".join(f"{x * 1e3:.1f}" for x in kernel_ms), file=sys.stderr)
    ms_per_step = wall * 1e3 / args.steps
    alg = synth.algorithmic_bytes(spec, lens) + 2 * 2 * spec.batch * spec.num_kv_heads * args.window * spec.head_dim
    value = alg / (ms_per_step * 1e-3) / 1e9
    k_avg = sum(kernel_ms) / len(kernel_ms)
    achieved = alg / (k_avg * 1e-3) / 1e9
    assert torch.isfinite(outs[0][0].float()).all(), "non-finite output"

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
        "dtype": "f16",
        "arith": "2-bit codes -> fp16 matrix-core operands (magic-exponent AND-OR), fp32 accumulation, bf16 out",
        "data": "synthetic",
        "config": {"workload": f"{spec.name}: batch {spec.batch}, {spec.num_q_heads} query heads / "
                               f"{spec.num_kv_heads} KV heads, head_dim {spec.head_dim}, {spec.max_seq_len} tokens, "
                               f"INT{spec.bits}, K {spec.k_layout}-wise / V {spec.v_layout}-wise, group {spec.group}",
                   "global_batch": spec.batch, "seq_len": spec.max_seq_len, "bits": spec.bits,
                   "k_layout": spec.k_layout, "v_layout": spec.v_layout, "group": spec.group,
                   "splits": splits, "chunk": chunk, "cache_copies": len(copies), "window_tokens": args.window,
                   "algorithmic_bytes_per_step": alg},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic_per_launch(spec.name),
                     "kernel": "split_decode (one launch per step)", "kernel_us_avg": round(k_avg * 1e3, 2),
                     "kernel_us_median": round(sorted(kernel_ms)[len(kernel_ms) // 2] * 1e3, 2),
                     "kernel_us_min": round(min(kernel_ms) * 1e3, 2),
                     "host_enqueue_us_per_step": round(enqueued * 1e6 / args.steps, 2)},
        "staging_s": round(stage_s, 1),
        "kernel_source_sha": kernel_sha(),
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(spec, q, lens, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
