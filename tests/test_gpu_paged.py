"""GPU parity of the paged decode (foscar_decode_paged_int2/4 through the C
interface) against the oracle, which gathers the pool back into logical order
and decodes it by definition.  Pools hold the sequences' blocks in a seeded
random order plus unused blocks poisoned with random codes and NaN scales;
table entries past each sequence's length are -1.  Bar as test_gpu_parity."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import check

pytestmark = pytest.mark.gpu


def _run_paged(spec, P, seed=3, table_edit=None, splits=None, monkeypatch=None):
    import bit_quantized_kv_split_amd as fos
    import bit_quantized_kv_split_amd.staging as staging
    import torch
    lens = spec.seq_lens()
    table, nb = synth.make_block_table(seed, lens, spec.max_seq_len // P, P)
    pool = synth.make_pool(spec, table, nb, P)
    if table_edit is not None:
        table = table_edit(table.copy())
    q = synth.make_query(spec)
    dev = staging.stage_paged(spec.bits, q, lens, pool, table)
    if splits is not None:
        monkeypatch.setenv("FOSCAR_SPLITS", str(splits))
    out, lse = fos.decode_paged(dev["q"], dev["k_pool"], dev["v_pool"], dev["k_scale"], dev["k_zero"],
                                dev["v_scale"], dev["v_zero"], dev["block_table"], dev["seq_lens"], bits=spec.bits,
                                k_layout=spec.k_layout, v_layout=spec.v_layout, group=spec.group,
                                sm_scale=spec.sm_scale)
    torch.cuda.synchronize()
    pool["q"], pool["seq_lens"] = q, lens
    rows = [(b, i) for b in range(spec.batch) for i in range(spec.num_q_heads)]
    ro, rl = oracle.decode_paged_rows(pool, table, P, rows, k_layout=spec.k_layout, v_layout=spec.v_layout,
                                      group=spec.group, sm_scale=spec.sm_scale)
    B, Hq = spec.batch, spec.num_q_heads
    return (out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64),
            ro.reshape(B, Hq, -1), rl.reshape(B, Hq))


PAGED = [(2, "token", "token", 128, 64), (2, "token", "token", 128, 256), (4, "token", "token", 64, 128),
         (2, "token", "channel", 64, 64), (4, "token", "channel", 32, 128), (2, "channel", "token", 128, 128),
         (4, "channel", "token", 32, 64), (2, "channel", "channel", 64, 128), (4, "channel", "channel", 128, 256)]


@pytest.mark.parametrize("bits,kl,vl,g,P", PAGED)
def test_paged_layout_matrix(bits, kl, vl, g, P):
    """Every layout and bit width with blocks of 64-256 tokens: ragged lengths
    with partial last blocks, a one-token and an empty sequence."""
    std = (0.1, 10.0) if "channel" in (kl, vl) else None
    spec = synth.Spec(f"paged_{bits}_{kl}_{vl}_{g}_{P}", 23, bits, kl, vl, g, 4, 8, 2, 128, 1024,
                      lens=(1024, 517, 1, 0), channel_std_logu=std)
    out, lse, ro, rl = _run_paged(spec, P)
    check(out, lse, ro, rl, spec.name)


@pytest.mark.parametrize("splits", [1, 7, 64])
def test_paged_ranges_through_the_merge(splits, monkeypatch):
    """Forced range counts over blocks of 128 tokens: one range asked for still
    gets ranges of at most 63 blocks (16384 tokens: 3 ranges), 7 ranges start
    inside a block (ranges of 2368 tokens), 64 ranges take 2 blocks each."""
    spec = synth.Spec("paged_split", 24, 2, "token", "channel", 64, 2, 8, 2, 128, 16384, lens=(16384, 9001))
    out, lse, ro, rl = _run_paged(spec, 128, splits=splits, monkeypatch=monkeypatch)
    check(out, lse, ro, rl, f"paged splits={splits}")


@pytest.mark.parametrize("splits", [1, 2, None])
@pytest.mark.parametrize("bits", [2, 4])
def test_paged_block_of_one_unit_takes_64_blocks_per_range(bits, splits, monkeypatch):
    """Blocks of 64 tokens (the wave unit): every range starts on a block, so a
    range may hold 64 blocks (one per lane of the table row).  One range asked
    for over 8192 tokens gets two of 64 blocks; lengths at the range boundary,
    one block short of it and one token past it."""
    spec = synth.Spec(f"paged_unit_{bits}", 26, bits, "token", "token", 128, 4, 4, 1, 128, 8192,
                      lens=(8192, 4096, 4032, 4097))
    out, lse, ro, rl = _run_paged(spec, 64, splits=splits, monkeypatch=monkeypatch)
    check(out, lse, ro, rl, f"paged P=64 splits={splits}")


def test_paged_gqa_and_persistent_order():
    """16 query heads per KV head (four groups reading each block) on a ragged
    batch large enough for the persistent work order."""
    lens = tuple(int(x) for x in np.random.default_rng(9).integers(0, 8192, size=96))
    spec = synth.Spec("paged_persist", 25, 2, "token", "token", 128, 96, 32, 2, 128, 8192, lens=lens)
    out, lse, ro, rl = _run_paged(spec, 128)
    check(out, lse, ro, rl, "paged persistent G=16")


def test_paged_entry_outside_the_pool_reads_zeros():
    """A table entry outside the pool for a block below the length reads a block
    of zeros (codes, scales and offsets), as the oracle's gather does, and does
    not touch memory outside the pool."""
    spec = synth.Spec("paged_bad", 26, 4, "token", "token", 128, 2, 4, 1, 128, 512, lens=(512, 300))

    def edit(t):
        t[0, 1] = 10 ** 6
        t[1, 0] = -7
        return t
    out, lse, ro, rl = _run_paged(spec, 128, table_edit=edit)
    check(out, lse, ro, rl, "paged zero blocks")
