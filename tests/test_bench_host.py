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


def test_pools_for_the_paged_timing_hold_every_block_once():
    """bench.py --paged regroups a staged contiguous cache into block pools; the
    oracle's gather through the block table gives the contiguous arrays back."""
    import torch
    import oracle
    sys.path.insert(0, ROOT)
    import bench
    spec = synth.SPECS["c1_tiny_int2"].replace(batch=3, max_seq_len=512, k_layout="channel", group=64)
    B, H, T, D, E, g = spec.batch, spec.num_kv_heads, spec.max_seq_len, spec.head_dim, 16, spec.group
    rng = np.random.default_rng(0)
    c = {"q": torch.zeros(1),
         "packed_k": torch.from_numpy(rng.integers(0, 1 << 31, (B, H, T, D // E), dtype=np.int64).astype(np.int32)),
         "packed_v": torch.from_numpy(rng.integers(0, 1 << 31, (B, H, T // E, D), dtype=np.int64).astype(np.int32)),
         "k_scale": torch.from_numpy(rng.standard_normal((B, H, T // g, D)).astype(np.float16)),
         "k_zero": torch.from_numpy(rng.standard_normal((B, H, T // g, D)).astype(np.float16)),
         "v_scale": torch.from_numpy(rng.standard_normal((B, H, T, D // g)).astype(np.float16)),
         "v_zero": torch.from_numpy(rng.standard_normal((B, H, T, D // g)).astype(np.float16))}
    P = 128
    pools, table = bench.to_pool(c, spec, P, 0)
    tab = table.numpy()
    assert sorted(tab.ravel().tolist()) == list(range(B * T // P))
    pool = {"k_codes": oracle.unpack_k(pools["packed_k"].numpy().view(np.uint32), spec.bits, D),
            "v_codes": oracle.unpack_v(pools["packed_v"].numpy().view(np.uint32), spec.bits)}
    for n in ("k_scale", "k_zero", "v_scale", "v_zero"):
        pool[n] = pools[n].numpy()
    got = oracle.gather_paged(pool, tab, P, k_layout="channel", v_layout="token", group=g)
    assert np.array_equal(got["k_codes"], oracle.unpack_k(c["packed_k"].numpy().view(np.uint32), spec.bits, D))
    assert np.array_equal(got["v_codes"], oracle.unpack_v(c["packed_v"].numpy().view(np.uint32), spec.bits))
    for n in ("k_scale", "k_zero", "v_scale", "v_zero"):
        assert np.array_equal(got[n], c[n].numpy()), n


def test_a_token_wise_group_that_does_not_divide_the_head_dim_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--head-dim", "64", "--group", "128",
                        "--no-cpu-baseline"], capture_output=True, text=True, timeout=300)
    assert r.returncode == 2 and "does not divide head_dim 64" in r.stderr
