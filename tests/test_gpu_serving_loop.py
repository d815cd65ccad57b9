"""The three entry points composed the way a serving loop uses them: every
step appends the new token's keys and values to the full-precision window and
decodes over cache plus window; whenever the window holds a whole group of g
tokens, those tokens are quantised into the cache (a channel-wise side needs
whole groups) and the window empties.  Each step is checked against the
oracle, whose cache is built by the oracle's own quantiser from the same
tokens (the GPU quantiser is bit-exact with it, so both sides attend the same
cache)."""
import numpy as np
import pytest

import oracle
import oracle.quantize as oq
import synth
from gpu_util import check

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("bits,kl,vl", [(2, "token", "channel"), (4, "channel", "channel"), (2, "token", "token")])
def test_append_window_quantise_decode_loop(bits, kl, vl):
    import torch
    import bit_quantized_kv_split_amd as fos
    B, H, G, D, g, Tcap, steps = 2, 2, 4, 128, 64, 512, 150
    Hq = H * G
    E = 32 // bits
    rng = np.random.default_rng(31)
    k_all = synth.bf16_round(rng.standard_normal((B, H, steps, D)).astype(np.float32))
    v_all = synth.bf16_round((rng.standard_normal((B, H, steps, D)) * 2.0).astype(np.float32))
    dev = "cuda"
    pk = torch.zeros((B, H, Tcap, D // E), dtype=torch.int32, device=dev)
    pv = torch.zeros((B, H, Tcap // E, D), dtype=torch.int32, device=dev)
    shp = lambda layout: (B, H, Tcap, D // g) if layout == "token" else (B, H, Tcap // g, D)
    ks, kz = (torch.zeros(shp(kl), dtype=torch.float16, device=dev) for _ in range(2))
    vs, vz = (torch.zeros(shp(vl), dtype=torch.float16, device=dev) for _ in range(2))
    win_k = torch.zeros((B, H, g, D), dtype=torch.bfloat16, device=dev)
    win_v = torch.zeros((B, H, g, D), dtype=torch.bfloat16, device=dev)
    cache = {"k_codes": np.zeros((B, H, Tcap, D), np.uint8), "v_codes": np.zeros((B, H, Tcap, D), np.uint8),
             "k_scale": np.zeros(shp(kl), np.float16), "k_zero": np.zeros(shp(kl), np.float16),
             "v_scale": np.zeros(shp(vl), np.float16), "v_zero": np.zeros(shp(vl), np.float16)}
    layout = fos.layout_bits(kl, vl)
    quant = fos.foscar_quantize_int2 if bits == 2 else fos.foscar_quantize_int4
    T, wl = 0, 0
    for t in range(steps):
        win_k[:, :, wl] = torch.from_numpy(k_all[:, :, t]).to(torch.bfloat16).to(dev)
        win_v[:, :, wl] = torch.from_numpy(v_all[:, :, t]).to(torch.bfloat16).to(dev)
        wl += 1
        q = synth.bf16_round(rng.standard_normal((B, Hq, D)).astype(np.float32))
        lens = np.full(B, T, np.int32)
        out, lse = fos.decode(torch.from_numpy(q).to(torch.bfloat16).to(dev), pk, pv, ks, kz, vs, vz,
                              torch.from_numpy(lens).to(dev), bits=bits, k_layout=kl, v_layout=vl, group=g,
                              window=(win_k, win_v, torch.full((B,), wl, dtype=torch.int32, device=dev)))
        torch.cuda.synchronize()
        w = dict(cache, q=q, seq_lens=lens)
        win = {"k": win_k.float().cpu().numpy(), "v": win_v.float().cpu().numpy(), "lens": np.full(B, wl)}
        rows = [(b, i) for b in range(B) for i in range(Hq)]
        ro, rl = oracle.decode_window_rows(w, win, rows, k_layout=kl, v_layout=vl, group=g, sm_scale=D ** -0.5)
        check(out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64),
              ro.reshape(B, Hq, D), rl.reshape(B, Hq), f"step {t} (cache {T}, window {wl})")
        if wl == g:  # the window holds a whole group: quantise it into the cache, empty the window
            start = torch.full((B,), T, dtype=torch.int32, device=dev)
            count = torch.full((B,), g, dtype=torch.int32, device=dev)
            quant(win_k, win_v, start, count, pk, pv, ks, kz, vs, vz, layout, g)
            cache = oq.quantize_append(cache, win["k"], win["v"], np.full(B, T), np.full(B, g), bits=bits,
                                       k_layout=kl, v_layout=vl, group=g)
            T, wl = T + g, 0
