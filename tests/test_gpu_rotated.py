"""GPU parity of the rotated cache (layout bits FOSCAR_K_ROTATED /
FOSCAR_V_ROTATED through the C interface) against the oracle's
attend_rotated: the stored rows are those of K H and/or V H (H the
orthonormal Hadamard matrix of order 128), the kernel rotates the query in
its prologue and takes the output back after the merge.  The caches are
written as a rotating writer would: keys and values drawn in the model's
basis (with their channel scales), rotated, then quantised (synth's
``Spec.rotate``).  Every layout and
bit width, single-range sequences (the direct output path), the merge of
many ranges, the persistent work order, query-head groups of 1-16, a
full-precision window (unrotated) and a paged cache.  Bar as
test_gpu_parity."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import assert_persistent, check, oracle_all, persistent_spec, run, stage_spec

pytestmark = pytest.mark.gpu

LAYOUTS = [(2, "token", "token", 128), (4, "token", "token", 64), (2, "token", "channel", 64),
           (4, "token", "channel", 32), (2, "channel", "token", 128), (4, "channel", "token", 32),
           (2, "channel", "channel", 64), (4, "channel", "channel", 128)]


@pytest.mark.parametrize("rotate", ["k", "v", "kv"])
@pytest.mark.parametrize("bits,kl,vl,g", LAYOUTS)
def test_rotated_layout_matrix(bits, kl, vl, g, rotate):
    """Ragged lengths: full, partial, one short enough for a single range
    (direct output), one token and none."""
    std = (0.1, 10.0) if "channel" in (kl, vl) else None
    spec = synth.Spec(f"rot_{bits}_{kl}_{vl}_{g}_{rotate}", 31, bits, kl, vl, g, 5, 8, 2, 128, 1024,
                      lens=(1024, 517, 60, 1, 0), channel_std_logu=std, rotate=rotate)
    dev, q, lens = stage_spec(spec)
    out, lse = run(spec, dev, rotate=rotate)
    ro, rl = oracle_all(spec, q, lens, rotate=rotate)
    check(out, lse, ro, rl, spec.name)


@pytest.mark.parametrize("splits", [1, 64])
@pytest.mark.parametrize("rotate", ["v", "kv"])
def test_rotated_direct_and_merged_output(splits, rotate, monkeypatch):
    """One forced range per sequence: every row leaves through the direct
    output path and is taken back there; 64 ranges: through the merge."""
    spec = synth.Spec(f"rot_splits_{splits}", 32, 2, "token", "channel", 64, 3, 8, 2, 128, 4096,
                      lens=(4096, 3001, 64), channel_std_logu=(0.1, 10.0), rotate=rotate)
    monkeypatch.setenv("FOSCAR_SPLITS", str(splits))
    dev, q, lens = stage_spec(spec)
    out, lse = run(spec, dev, rotate=rotate)
    ro, rl = oracle_all(spec, q, lens, rotate=rotate)
    check(out, lse, ro, rl, spec.name)


@pytest.mark.parametrize("G", [1, 3, 8, 16])
def test_rotated_gqa(G):
    """Query rows of every group of <= 4 heads are rotated by their own work
    pair (G = 8, 16: two and four pairs read each KV head)."""
    spec = synth.Spec(f"rot_gqa_{G}", 33, 4, "token", "token", 128, 2, 2 * G, 2, 128, 2048, lens=(2048, 999),
                      rotate="kv")
    dev, q, lens = stage_spec(spec)
    out, lse = run(spec, dev, rotate="kv")
    ro, rl = oracle_all(spec, q, lens, rotate="kv")
    check(out, lse, ro, rl, spec.name)


def test_rotated_persistent_order():
    spec = persistent_spec().replace(rotate="kv")
    assert_persistent(spec)
    dev, q, lens = stage_spec(spec)
    out, lse = run(spec, dev, rotate="kv")
    ro, rl = oracle_all(spec, q, lens, rotate="kv")
    check(out, lse, ro, rl, "rotated persistent")


def test_rotation_relations_between_kernel_runs():
    """Relations that hold whatever the cache holds, checked kernel against
    kernel: the output of a cache read as rotated values, times H, is the
    output of the same cache read as unrotated (lse unchanged; compared in the
    cache's basis, where the unrotated run's errors stay elementwise); reading
    it as rotated keys gives the scores of an unrotated run on the query
    bf16(q H) rounded here from fp64, bit for bit (lse), and its output."""
    spec = synth.Spec("rot_rel", 34, 2, "token", "token", 128, 3, 8, 2, 128, 2048, lens=(2048, 700, 3))
    dev, q, lens = stage_spec(spec)
    o0, l0 = run(spec, dev)
    ov, lv = run(spec, dev, rotate="v")
    H = oracle.hadamard(128)
    np.testing.assert_allclose(ov @ H, o0, atol=4e-3, rtol=2 ** -7)  # H H = I; compared in the stored basis
    np.testing.assert_allclose(lv, l0, atol=1e-5)
    ok, lk = run(spec, dev, rotate="k")
    qr = oracle.round_bf16(q.astype(np.float64) @ H).astype(np.float32)
    dev_r, _, _ = stage_spec(spec, q=qr)
    oq, lq = run(spec, dev_r)
    # the scores, hence lse, are bit for bit those of the query bf16(q H); the outputs differ in
    # rounding only (the rotated variant centres the value codes)
    np.testing.assert_array_equal(lk, lq)
    np.testing.assert_allclose(ok, oq, atol=2e-3, rtol=2 ** -7)
    assert np.abs(ok - o0).max() > 1e-2 and np.abs(ov - o0).max() > 1e-2


def _window_oracle(spec, q, lens, win, rotate):
    G = spec.num_q_heads // spec.num_kv_heads
    B, Hq, D = spec.batch, spec.num_q_heads, spec.head_dim
    out, lse = np.zeros((B, Hq, D)), np.zeros((B, Hq))
    for b in range(B):
        for h in range(spec.num_kv_heads):
            head = synth.make_head(spec, b, h, seq_len=int(lens[b]))
            w = {k: v[None, None] for k, v in head.items()}
            w["q"] = q[b:b + 1, h * G:(h + 1) * G]
            w["seq_lens"] = np.array([lens[b]], np.int32)
            ws = {"k": win["k"][b:b + 1, h:h + 1], "v": win["v"][b:b + 1, h:h + 1],
                  "lens": np.array([int(win["lens"][b])])}
            o, l = oracle.decode_window_rows(w, ws, [(0, i) for i in range(G)], k_layout=spec.k_layout,
                                             v_layout=spec.v_layout, group=spec.group, sm_scale=spec.sm_scale,
                                             rotate=rotate)
            out[b, h * G:(h + 1) * G], lse[b, h * G:(h + 1) * G] = o, l
    return out, lse


@pytest.mark.parametrize("rotate", ["k", "kv"])
@pytest.mark.parametrize("max_len,splits", [(768, None), (8192, 16)])
def test_rotated_cache_with_window(rotate, max_len, splits, monkeypatch):
    """The window holds unrotated rows and meets the query itself; the cache's
    output is taken back before the window's partials join the merge.  Rows
    with no cache token are the window's alone."""
    import bit_quantized_kv_split_amd as fos
    import torch
    spec = synth.Spec(f"rot_win_{max_len}", 35, 2, "token", "channel", 64, 4, 8, 2, 128, max_len,
                      lens=(max_len, max_len // 3, 0, 0), rotate=rotate)
    if splits:
        monkeypatch.setenv("FOSCAR_SPLITS", str(splits))
    dev, q, lens = stage_spec(spec)
    win = synth.make_window(5, spec.batch, spec.num_kv_heads, 256, [256, 31, 100, 0])
    wk = torch.from_numpy(win["k"]).to(torch.bfloat16).cuda()
    wv = torch.from_numpy(win["v"]).to(torch.bfloat16).cuda()
    wl = torch.from_numpy(win["lens"]).cuda()
    out, lse = fos.decode(dev["q"], dev["packed_k"], dev["packed_v"], dev["k_scale"], dev["k_zero"], dev["v_scale"],
                          dev["v_zero"], dev["seq_lens"], bits=spec.bits, k_layout=spec.k_layout,
                          v_layout=spec.v_layout, group=spec.group, window=(wk, wv, wl), rotate=rotate)
    torch.cuda.synchronize()
    out = out.float().cpu().numpy().astype(np.float64)
    lse = lse.cpu().numpy().astype(np.float64)
    ro, rl = _window_oracle(spec, q, lens, win, rotate)
    check(out, lse, ro, rl, spec.name)


@pytest.mark.parametrize("bits,kl,vl,g,P", [(2, "token", "token", 128, 128), (4, "channel", "token", 64, 64)])
def test_rotated_paged(bits, kl, vl, g, P):
    import bit_quantized_kv_split_amd as fos
    import bit_quantized_kv_split_amd.staging as staging
    import torch
    std = (0.1, 10.0) if "channel" in (kl, vl) else None
    spec = synth.Spec(f"rot_paged_{bits}_{kl}", 36, bits, kl, vl, g, 3, 8, 2, 128, 2048, lens=(2048, 1000, 1),
                      channel_std_logu=std, rotate="kv")
    lens = spec.seq_lens()
    table, nb = synth.make_block_table(7, lens, spec.max_seq_len // P, P)
    pool = synth.make_pool(spec, table, nb, P)
    q = synth.make_query(spec)
    dev = staging.stage_paged(spec.bits, q, lens, pool, table)
    out, lse = fos.decode_paged(dev["q"], dev["k_pool"], dev["v_pool"], dev["k_scale"], dev["k_zero"],
                                dev["v_scale"], dev["v_zero"], dev["block_table"], dev["seq_lens"], bits=bits,
                                k_layout=kl, v_layout=vl, group=g, sm_scale=spec.sm_scale, rotate="kv")
    torch.cuda.synchronize()
    pool["q"], pool["seq_lens"] = q, lens
    rows = [(b, i) for b in range(spec.batch) for i in range(spec.num_q_heads)]
    ro, rl = oracle.decode_paged_rows(pool, table, P, rows, k_layout=kl, v_layout=vl, group=g,
                                      sm_scale=spec.sm_scale, rotate="kv")
    B, Hq = spec.batch, spec.num_q_heads
    check(out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64),
          ro.reshape(B, Hq, -1), rl.reshape(B, Hq), spec.name)
