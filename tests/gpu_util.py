"""Helpers shared by the GPU tests: stage a synthetic workload on the device,
run the HIP decode through the C interface, compute oracle rows, compare."""
import os

import numpy as np

import oracle
import synth

# Output bar, elementwise: |out - O| <= ATOL + RTOL_BF16 * |O|.  ATOL = 2e-3 is
# the target's absolute kernel error; RTOL_BF16 = 2^-8 covers the
# round-to-nearest of the bf16 output (half an ulp is at most 2^-9 relative)
# with a factor 2 margin, since a bf16 output cannot hold 2e-3 absolute once
# |O| > 0.5.
ATOL = 2e-3
RTOL_BF16 = 2.0 ** -8
LSE_ATOL = 2e-3


def stage_spec(spec, poison=False, q=None):
    import bit_quantized_kv_split_amd.staging as staging
    qh = synth.make_query(spec) if q is None else q
    lens = spec.seq_lens()
    dev = staging.stage((spec.batch, spec.num_q_heads, spec.num_kv_heads, spec.max_seq_len, spec.head_dim), spec.bits,
                        qh, lens, lambda b: synth.make_sequence(spec, b, poison=poison), synth.full_scale_shapes(spec))
    return dev, qh, lens


def run(spec, dev, sm_scale=0.0, rotate=""):
    import bit_quantized_kv_split_amd as fos
    import torch
    out, lse = fos.decode(dev["q"], dev["packed_k"], dev["packed_v"], dev["k_scale"], dev["k_zero"], dev["v_scale"],
                          dev["v_zero"], dev["seq_lens"], bits=spec.bits, k_layout=spec.k_layout,
                          v_layout=spec.v_layout, group=spec.group, sm_scale=sm_scale or spec.sm_scale,
                          rotate=rotate)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def oracle_rows(spec, rows, q, lens, poison=False, rotate=""):
    """Oracle output for (b, query head) rows, regenerating only the needed (b, KV head) slices."""
    G = spec.num_q_heads // spec.num_kv_heads
    outs, lses = [], []
    for (b, i) in rows:
        h = i // G
        head = synth.make_head(spec, b, h, seq_len=int(lens[b]), poison=poison)
        w = {k: v[None, None] for k, v in head.items()}
        w["q"] = q[b:b + 1, i:i + 1]
        w["seq_lens"] = np.array([lens[b]], np.int32)
        o, l = oracle.decode_rows(w, [(0, 0)], k_layout=spec.k_layout, v_layout=spec.v_layout, group=spec.group,
                                  sm_scale=spec.sm_scale, rotate=rotate)
        outs.append(o[0])
        lses.append(l[0])
    return np.array(outs), np.array(lses)


def oracle_all(spec, q, lens, poison=False, rotate=""):
    """(out, lse) for every row: out [B, Hq, D], lse [B, Hq]."""
    rows = [(b, i) for b in range(spec.batch) for i in range(spec.num_q_heads)]
    o, l = oracle_rows(spec, rows, q, lens, poison, rotate)
    B, Hq = spec.batch, spec.num_q_heads
    return o.reshape(B, Hq, -1), l.reshape(B, Hq)


def _log_parity(what, err, ref_out, bound, lse, ref_lse):
    """Append one JSON line per comparison to $FOSCAR_PARITY_LOG: max error,
    max |O| and max error/bound, so the suite's margin against the bar is on
    record."""
    log = os.environ.get("FOSCAR_PARITY_LOG")
    if not log:
        return
    import json
    fin = np.isfinite(ref_lse)
    lerr = float(np.abs(lse[fin] - ref_lse[fin]).max()) if fin.any() else 0.0
    rec = {"test": os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0], "what": what,
           "max_err": float(err.max()) if err.size else 0.0,
           "max_abs_out": float(np.abs(ref_out).max()) if ref_out.size else 0.0,
           "ratio": float((err / bound).max()) if err.size else 0.0,
           "lse_err": lerr}
    with open(log, "a") as f:
        f.write(json.dumps(rec) + "\n")


def check(out, lse, ref_out, ref_lse, what=""):
    err = np.abs(out - ref_out)
    bound = ATOL + RTOL_BF16 * np.abs(ref_out)
    worst = np.unravel_index(np.argmax(err - bound), err.shape)
    _log_parity(what, err, ref_out, bound, lse, ref_lse)
    assert np.all(np.isfinite(out)), f"{what}: non-finite output"
    assert np.all(err <= bound), (f"{what}: out error {err[worst]:.3e} > bound {bound[worst]:.3e} at {worst} "
                                  f"(got {out[worst]:.6f}, oracle {ref_out[worst]:.6f}); max err {err.max():.3e}")
    fin = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(lse), fin), f"{what}: lse finiteness differs"
    assert np.array_equal(np.isneginf(lse), np.isneginf(ref_lse)), f"{what}: lse -inf pattern differs"
    if fin.any():
        lerr = np.abs(lse[fin] - ref_lse[fin]).max()
        assert lerr <= LSE_ATOL, f"{what}: lse error {lerr:.3e}"
    return float(err.max())


# A ragged batch whose plan needs more work-groups than one round (the persistent,
# longest-first work order), with empty sequences and sequences of a few tokens.
PERSISTENT_LENS = (0, 3, 32768, 1, 20000, 0, 4096, 4097, 12000, 64, 65, 30000, 0, 8191, 100, 32767) * 4


def persistent_spec():
    return synth.SPECS["c5_ragged_int2_g64"].replace(batch=len(PERSISTENT_LENS), num_q_heads=8, num_kv_heads=2,
                                                     max_seq_len=32768, lens=PERSISTENT_LENS)


def assert_persistent(spec):
    """The plan of this spec needs more than one round of resident work-groups."""
    import bit_quantized_kv_split_amd as fos
    import torch
    dims = fos.make_dims(spec.batch, spec.num_q_heads, spec.num_kv_heads, spec.head_dim, spec.max_seq_len)
    layout = fos.layout_bits(spec.k_layout, spec.v_layout)
    s, c = fos.foscar_split_plan(dims, spec.bits, layout, spec.group)
    per_cu = fos.foscar_occupancy(spec.bits, layout, spec.group)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert s * spec.batch * spec.num_kv_heads > per_cu * cus, "the plan must need more than one round"
