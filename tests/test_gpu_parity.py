"""GPU parity: the HIP decode path (through the C interface) against the fp64
oracle, element by element, on seeded synthetic workloads.

Bar (written in gpu_util): |out - O| <= 2e-3 + 2^-8 |O| per element (bf16
output), |lse - lse_ref| <= 2e-3.
"""
import os

import numpy as np
import pytest

import synth
from gpu_util import assert_persistent, check, oracle_all, oracle_rows, persistent_spec, run, stage_spec

pytestmark = pytest.mark.gpu


def _spec(name, **kw):
    return synth.SPECS[name].replace(**kw)


def test_c1_tiny_full_size():
    spec = synth.SPECS["c1_tiny_int2"]
    dev, q, lens = stage_spec(spec)
    out, lse = run(spec, dev)
    ro, rl = oracle_all(spec, q, lens)
    check(out, lse, ro, rl, "c1")


MATRIX = [(bits, kl, vl, g) for bits in (2, 4) for kl in ("token", "channel") for vl in ("token", "channel")
          for g in (32, 64, 128)]


@pytest.mark.parametrize("bits,kl,vl,g", MATRIX)
def test_layout_matrix(bits, kl, vl, g):
    """Every kernel instance: 3 ragged sequences spanning several tiles with tails."""
    std = (0.1, 10.0) if "channel" in (kl, vl) else None
    spec = synth.Spec(f"matrix_{bits}_{kl}_{vl}_{g}", 11, bits, kl, vl, g, 3, 8, 2, 128, 768,
                      lens=(768, 517, 130), channel_std_logu=std)
    dev, q, lens = stage_spec(spec)
    out, lse = run(spec, dev)
    ro, rl = oracle_all(spec, q, lens)
    check(out, lse, ro, rl, spec.name)


SCALED = [
    _spec("c2_paper_int2", batch=2, num_q_heads=8, num_kv_heads=2, max_seq_len=2048),
    _spec("c2_paper_int4", batch=2, num_q_heads=8, num_kv_heads=2, max_seq_len=2048),
    _spec("c3_long_int2", batch=1, num_q_heads=4, num_kv_heads=1, max_seq_len=16384),
    _spec("c4_channel_int2", batch=2, num_q_heads=8, num_kv_heads=2, max_seq_len=2048),
    _spec("c4_channel_int4", batch=2, num_q_heads=8, num_kv_heads=2, max_seq_len=2048),
] + [_spec(f"c5_ragged_int{b}_g{g}", batch=6, num_q_heads=8, num_kv_heads=2, max_seq_len=4096, ragged_lo=64)
     for b in (2, 4) for g in (32, 64, 128)]


@pytest.mark.parametrize("spec", SCALED, ids=[s.name for s in SCALED])
def test_scaled_workloads(spec):
    """The five workloads' value recipes at sizes the oracle finishes in seconds."""
    dev, q, lens = stage_spec(spec)
    out, lse = run(spec, dev)
    ro, rl = oracle_all(spec, q, lens)
    check(out, lse, ro, rl, spec.name)


EDGE_LENS = (0, 1, 2, 63, 64, 65, 127, 128, 129, 255, 256)


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("kl,vl,g", [("token", "token", 128), ("channel", "channel", 128), ("token", "channel", 32),
                                     ("channel", "token", 64), ("channel", "token", 32), ("channel", "channel", 32),
                                     ("channel", "channel", 64)])
def test_edge_lengths_and_poisoned_padding(bits, kl, vl, g):
    """Empty, single-token, tile-boundary and group-boundary lengths; padding
    past each length holds random codes and NaN scales/offsets."""
    spec = synth.Spec(f"edge_{bits}_{kl}_{vl}_{g}", 12, bits, kl, vl, g, len(EDGE_LENS), 4, 1, 128, 256,
                      lens=EDGE_LENS)
    dev, q, lens = stage_spec(spec, poison=True)
    out, lse = run(spec, dev)
    ro, rl = oracle_all(spec, q, lens, poison=True)
    check(out, lse, ro, rl, spec.name)
    assert np.all(out[0] == 0) and np.all(np.isneginf(lse[0]))


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("kl,vl,g,tcap", [("token", "token", 128, 96), ("token", "channel", 32, 96),
                                          ("channel", "channel", 32, 160), ("channel", "token", 32, 96),
                                          ("token", "token", 64, 4128)])
def test_capacity_a_multiple_of_32(bits, kl, vl, g, tcap):
    """A cache capacity of 32 (mod 64) tokens: a wave's last tile reaches past
    the allocation, where its loads read zero and its tokens are masked.
    Lengths at the capacity, just under it, at tile and group boundaries and
    0; 4128 tokens take two ranges, the second ending past the capacity."""
    lens = (tcap, tcap - 1, tcap - 32, 65, 64, 33, 1, 0)
    spec = synth.Spec(f"tcap{tcap}_{bits}_{kl}_{vl}_{g}", 13, bits, kl, vl, g, len(lens), 4, 1, 128, tcap, lens=lens)
    dev, q, lens_np = stage_spec(spec, poison=True)
    out, lse = run(spec, dev)
    ro, rl = oracle_all(spec, q, lens_np, poison=True)
    check(out, lse, ro, rl, spec.name)


@pytest.mark.parametrize("G", [1, 2, 3, 4, 5, 6, 8, 12, 16])
def test_gqa_ratios(G):
    """G query heads per KV head; above 4 the library serves a KV head as
    groups of at most 4 query heads (5: five groups of 1, 6: two of 3, 8: two
    of 4, 12: three of 4, 16: four of 4), each reading the KV head."""
    spec = synth.Spec(f"gqa_{G}", 13, 2, "token", "channel", 64, 2, 3 * G, 3, 128, 512, lens=(512, 300))
    dev, q, lens = stage_spec(spec)
    out, lse = run(spec, dev)
    ro, rl = oracle_all(spec, q, lens)
    check(out, lse, ro, rl, spec.name)


@pytest.mark.parametrize("splits", ["1", "2", "7", "17", "32", "auto"])
def test_split_count_invariance(splits, monkeypatch):
    spec = _spec("c5_ragged_int2_g64", batch=4, num_q_heads=8, num_kv_heads=2, max_seq_len=2048, ragged_lo=100)
    if splits != "auto":
        monkeypatch.setenv("FOSCAR_SPLITS", splits)
    else:
        monkeypatch.delenv("FOSCAR_SPLITS", raising=False)
    dev, q, lens = stage_spec(spec)
    out, lse = run(spec, dev)
    ro, rl = oracle_all(spec, q, lens)
    check(out, lse, ro, rl, f"splits={splits}")


def test_many_ranges(monkeypatch):
    """More ranges than the merge handles in one batch of loads, up to the
    512-range cap (asking for 600 gives 512 ranges of 128 tokens)."""
    spec = _spec("c5_ragged_int2_g64", batch=2, num_q_heads=8, num_kv_heads=2, max_seq_len=65536, ragged_lo=20000)
    monkeypatch.setenv("FOSCAR_SPLITS", "600")
    dev, q, lens = stage_spec(spec)
    import bit_quantized_kv_split_amd as fos
    dims = fos.make_dims(spec.batch, spec.num_q_heads, spec.num_kv_heads, spec.head_dim, spec.max_seq_len)
    assert fos.foscar_split_plan(dims, spec.bits, fos.layout_bits(spec.k_layout, spec.v_layout), spec.group) == (512, 128)
    out, lse = run(spec, dev)
    ro, rl = oracle_all(spec, q, lens)
    check(out, lse, ro, rl, "512 ranges")


def test_workspace_reuse_across_shapes(monkeypatch):
    """A call with few (sequence, KV head) pairs and many ranges, then one with
    many pairs and few ranges on the same workspace: the second call's range
    counters must not land on the first call's partial results."""
    import bit_quantized_kv_split_amd as fos
    fos.foscar_release()
    first = _spec("c5_ragged_int2_g64", batch=1, num_q_heads=4, num_kv_heads=1, max_seq_len=16384, ragged_lo=16384)
    monkeypatch.setenv("FOSCAR_SPLITS", "256")
    dev, q, lens = stage_spec(first)
    out, lse = run(first, dev)
    ro, rl = oracle_all(first, q, lens)
    check(out, lse, ro, rl, "many ranges")
    second = _spec("c2_paper_int2", batch=16, num_q_heads=32, num_kv_heads=8, max_seq_len=512)
    monkeypatch.setenv("FOSCAR_SPLITS", "2")
    dev, q, lens = stage_spec(second)
    for _ in range(2):
        out, lse = run(second, dev)
        ro, rl = oracle_all(second, q, lens)
        check(out, lse, ro, rl, "many pairs after many ranges")


FULL = ["c2_paper_int2", "c2_paper_int4", "c3_long_int2", "c4_channel_int2", "c4_channel_int4",
        "c5_ragged_int2_g32", "c5_ragged_int4_g128"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled_rows(name):
    """Full workload size, default launch configuration; sampled rows against
    the oracle computed one (sequence, query head) at a time."""
    spec = synth.SPECS[name]
    dev, q, lens = stage_spec(spec)
    out, lse = run(spec, dev)
    rng = np.random.default_rng(7)
    rows = [(0, 0), (spec.batch - 1, spec.num_q_heads - 1)]
    rows += [(int(rng.integers(spec.batch)), int(rng.integers(spec.num_q_heads))) for _ in range(4)]
    ro, rl = oracle_rows(spec, rows, q, lens)
    for n, (b, i) in enumerate(rows):
        check(out[b, i][None], lse[b, i][None], ro[n][None], rl[n][None], f"{name} row {(b, i)}")
    assert np.all(np.isfinite(out))


def test_persistent_work_order_ragged_with_empty_sequences():
    """A batch whose plan needs more work-groups than one round runs the
    persistent, longest-first path: every row (including empty sequences and
    sequences of a few tokens) must match the oracle, on two calls in a row."""
    _check_persistent(persistent_spec(), "persistent ragged")


def test_persistent_work_order_capacity_a_multiple_of_32():
    """The persistent path over a 32800-token capacity (32 mod 64; value groups
    of 32 tokens, which divide it), with one sequence that fills it: its last
    range ends past the allocation."""
    base = persistent_spec()
    lens = (32800,) + tuple(base.lens[1:])
    _check_persistent(base.replace(max_seq_len=32800, group=32, lens=lens), "persistent capacity 32800")


def _check_persistent(spec, what):
    import oracle
    assert_persistent(spec)
    dev, q, lens_np = stage_spec(spec, poison=True)
    G = spec.num_q_heads // spec.num_kv_heads
    ro = np.zeros((spec.batch, spec.num_q_heads, spec.head_dim))
    rl = np.zeros((spec.batch, spec.num_q_heads))
    for b in range(spec.batch):
        for h in range(spec.num_kv_heads):
            head = synth.make_head(spec, b, h, seq_len=int(lens_np[b]), poison=True)
            w = {k: v[None, None] for k, v in head.items()}
            w["q"] = q[b:b + 1, h * G:(h + 1) * G]
            w["seq_lens"] = np.array([lens_np[b]], np.int32)
            o, l = oracle.decode_rows(w, [(0, i) for i in range(G)], k_layout=spec.k_layout, v_layout=spec.v_layout,
                                      group=spec.group, sm_scale=spec.sm_scale)
            ro[b, h * G:(h + 1) * G], rl[b, h * G:(h + 1) * G] = o, l
    for k in range(2):
        out, lse = run(spec, dev)
        check(out, lse, ro, rl, f"{what} call {k}")


@pytest.mark.parametrize("G", [1, 2, 3, 8, 16])
@pytest.mark.parametrize("splits", ["7", "64"])
def test_gqa_ratios_through_the_merge(G, splits, monkeypatch):
    """G = 1-3, 8 and 16 query heads per KV head with several ranges per
    sequence: the merge gives each query row of a group its own wave, and waves
    past the group's rows leave early.  64
    forced ranges give 4096 tokens two blocks of 32 ranges and 2500 tokens a
    block plus a masked remainder."""
    spec = synth.Spec(f"gqa_merge_{G}", 14, 2, "token", "channel", 64, 2, 3 * G, 3, 128, 4096, lens=(4096, 2500))
    monkeypatch.setenv("FOSCAR_SPLITS", splits)
    dev, q, lens = stage_spec(spec)
    out, lse = run(spec, dev)
    ro, rl = oracle_all(spec, q, lens)
    check(out, lse, ro, rl, f"{spec.name} splits={splits}")
