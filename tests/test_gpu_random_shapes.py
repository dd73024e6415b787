"""Seeded random layer shapes through moe_forward against the oracle (GPU
required).

The fixed configurations exercise each kernel plan at the layer sizes the
pages discuss; these cases mix the sizes the plans switch on (tokens 1..1024,
experts 1..512, top-k 1..16, hidden and FFN widths down to one 64-wide block,
softmax or sigmoid with a Zipf-skewed bias, with or without renormalisation),
so the few-token router, the fused tiny-batch permutation, the streaming and
tiled GEMMs, ragged expert counts and the matrix-core router all meet
unusual combinations.  Bars, as in the forward parity test: routing
bit-exact outside the near-tie exemption, weights within 1e-5 relative, out
within the layer tolerance; and each batch's first rows alone give the same
bits as inside the batch.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from helpers import DEV, assert_out_close, bits, gpu, log, routing_compare, weights_close
from oracle import oracle as O
from serve_router_gemm_amd import inputs as I

pytestmark = gpu

if torch.cuda.is_available():
    from serve_router_gemm_amd import moe as M


def _cases(n=20, seed=20261203):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        E = int(rng.choice([1, 3, 8, 64, 129, 200, 512]))
        k = int(rng.choice([k for k in (1, 2, 4, 8, 16) if k <= E]))
        H = int(rng.choice([64, 128, 320, 1024, 2048]))
        F = int(rng.choice([64, 128, 192, 448]))
        T = int(rng.choice([1, 2, 3, 4, 5, 9, 33, 100, 300, 1024]))
        if T * k * H * F > 2.5e8:
            continue
        score = int(rng.integers(0, 2))
        renorm = bool(rng.integers(0, 2)) if score == I.SCORE_SIGMOID else True
        zipf = float(rng.choice([0.0, 1.2])) if score == I.SCORE_SIGMOID else 0.0
        out.append(I.LayerConfig(f"rand{len(out)}", H=H, E=E, k=k, F=F, score=score,
                                 renorm=renorm, w_std=0.02, T=T, seed=1000 + len(out),
                                 zipf_s=zipf))
    # one case on the matrix-core router plan (a block per chunk)
    out.append(I.LayerConfig("rand_mfma", H=2048, E=200, k=8, F=64, score=I.SCORE_SIGMOID,
                             renorm=True, w_std=0.02, T=1024, seed=1999, zipf_s=1.2))
    return out


@pytest.mark.parametrize("cfg", _cases(), ids=lambda c: f"{c.name}-T{c.T}-E{c.E}-k{c.k}-H{c.H}-F{c.F}")
def test_random_shape_forward_parity_and_invariance(cfg):
    L = I.make_layer(cfg, DEV)
    x = I.make_x(cfg, DEV)
    out, ids, w = M.forward(x, L["w_router"], L["w_gate"], L["w_up"], L["w_down"], cfg.k,
                            cfg.score, cfg.renorm, bias=L["bias"], return_routing=True)
    torch.cuda.synchronize()
    hb = {n: (bits(t) if t.dtype == torch.bfloat16 else t.cpu().numpy())
          for n, t in L.items() if t is not None}
    bias = L["bias"].cpu().numpy() if L["bias"] is not None else None
    rows = np.arange(cfg.T)
    out_r, ids_r, w_r, gap = O.forward_tokens(rows, bits(x), hb["w_router"], hb["w_gate"],
                                              hb["w_up"], hb["w_down"], cfg.k, cfg.score,
                                              cfg.renorm, bias=bias)
    ids_np = ids.cpu().numpy()
    n_ex, n_mis = routing_compare(ids_np, ids_r, gap)
    same = np.all(ids_np == ids_r, axis=1)
    weights_close(w.cpu().numpy()[same], w_r[same])
    stats = assert_out_close(bits(out)[same], out_r[same], what=f"{cfg.name} out")
    # the first rows alone: the same bits as inside the batch
    ob = bits(out)
    for n in sorted({1, min(3, cfg.T)}):
        o1 = M.forward(x[:n].contiguous(), L["w_router"], L["w_gate"], L["w_up"], L["w_down"],
                       cfg.k, cfg.score, cfg.renorm, bias=L["bias"])
        assert np.array_equal(bits(o1), ob[:n]), (cfg.name, n)
    log(f"[random] {I.describe(cfg)}: exempt={n_ex} exempt_mismatch={n_mis} {stats}")
