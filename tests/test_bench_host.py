"""Host-side parts of bench.py that need no GPU: one-GPU refusal of --gpus N,
and the algorithmic-byte formulas the roofline figures divide by."""
import os
import subprocess
import sys

import numpy as np

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_algorithmic_bytes_of_the_long_context_step():
    spec = synth.SPECS["c3_long_int2"]
    # codes 64 B + (s, z) of both sides 8 B per token and KV head; q, out (bf16), lse, seq_lens
    expect = 4 * 8 * 131072 * (64 + 8) + 2 * 4 * 32 * 128 * 2 + 4 * 4 * 32 + 4 * 4
    assert synth.algorithmic_bytes(spec, spec.seq_lens()) == expect == 302055952


def test_quantize_bytes_per_token():
    sys.path.insert(0, ROOT)
    import bench
    spec = synth.SPECS["c3_long_int2"]
    # bf16 K and V read (512 B), INT2 codes written (64 B), fp16 (s, z) of both sides (8 B)
    assert bench.quantize_bytes(spec, 1) == 4 * 8 * 584 + 8 * 4
    assert bench.quantize_bytes(spec, 131072) == 2449473568
