"""Helpers shared by the GPU tests: stage a synthetic workload on the device,
run the HIP decode through the C interface, compute oracle rows, compare."""
import math
import os

import numpy as np

import oracle
import synth

# Output bar, elementwise: |out - O| <= ATOL * max(1, rms_c) + RTOL_BF16 * |O|.
# ATOL is the 2e-3 kernel-error scale for unit-scale values; rms_c is the RMS
# of the dequantised value channel c over the sequence, so the bar keeps the
# same relative meaning when channel scales reach 10 (a floating-point decode
# kernel's error is proportional to the magnitude of the values it averages).
# RTOL_BF16 = 2^-8 covers the round-to-nearest of the bf16 output (half an ulp
# is at most 2^-9 relative) with a factor 2 margin.
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


def run(spec, dev, sm_scale=0.0):
    import bit_quantized_kv_split_amd as fos
    import torch
    out, lse = fos.decode(dev["q"], dev["packed_k"], dev["packed_v"], dev["k_scale"], dev["k_zero"], dev["v_scale"],
                          dev["v_zero"], dev["seq_lens"], bits=spec.bits, k_layout=spec.k_layout,
                          v_layout=spec.v_layout, group=spec.group, sm_scale=sm_scale or spec.sm_scale)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def value_rms(spec, head, t):
    """RMS over the first t tokens of each dequantised value channel."""
    if t == 0:
        return np.zeros(spec.head_dim)
    if spec.v_layout == "token":
        s, z = head["v_scale"][:t], head["v_zero"][:t]
    else:
        s, z = head["v_scale"][: -(-t // spec.group)], head["v_zero"][: -(-t // spec.group)]
    v = oracle.dequantize(head["v_codes"][:t], s, z, spec.v_layout, spec.group)
    return np.sqrt(np.mean(v * v, axis=0))


def oracle_rows(spec, rows, q, lens, poison=False, with_scale=False):
    """Oracle output for (b, query head) rows, regenerating only the needed (b, KV head) slices."""
    G = spec.num_q_heads // spec.num_kv_heads
    outs, lses, scales = [], [], []
    for (b, i) in rows:
        h = i // G
        head = synth.make_head(spec, b, h, seq_len=int(lens[b]), poison=poison)
        w = {k: v[None, None] for k, v in head.items()}
        w["q"] = q[b:b + 1, i:i + 1]
        w["seq_lens"] = np.array([lens[b]], np.int32)
        o, l = oracle.decode_rows(w, [(0, 0)], k_layout=spec.k_layout, v_layout=spec.v_layout, group=spec.group,
                                  sm_scale=spec.sm_scale)
        outs.append(o[0])
        lses.append(l[0])
        scales.append(value_rms(spec, head, int(lens[b])))
    if with_scale:
        return np.array(outs), np.array(lses), np.array(scales)
    return np.array(outs), np.array(lses)


def oracle_all(spec, q, lens, poison=False):
    """(out, lse, value rms) for every row; out and rms are [B, Hq, D]."""
    rows = [(b, i) for b in range(spec.batch) for i in range(spec.num_q_heads)]
    o, l, sc = oracle_rows(spec, rows, q, lens, poison, with_scale=True)
    B, Hq = spec.batch, spec.num_q_heads
    return o.reshape(B, Hq, -1), l.reshape(B, Hq), sc.reshape(B, Hq, -1)


def check(out, lse, ref_out, ref_lse, what="", vscale=None):
    err = np.abs(out - ref_out)
    scale = 1.0 if vscale is None else np.maximum(1.0, vscale)
    bound = ATOL * scale + RTOL_BF16 * np.abs(ref_out)
    worst = np.unravel_index(np.argmax(err - bound), err.shape)
    log = os.environ.get("FOSCAR_PARITY_LOG")
    if log:
        with open(log, "a") as f:
            f.write(f"{what}: max|err| {err.max():.3e}  max err/bound {(err / bound).max():.3f}\n")
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
